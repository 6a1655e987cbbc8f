"""Host checks of the full-state comparison used by the large GPU parity
tests (tests/full_state.py): on CPU tensors, a state the oracle itself
produced compares equal over several chunks and a ragged tail, and planted
differences in the compared state are counted or refused as the bars say."""
import numpy as np
import pytest
import torch

import oracle as o
from bf16_numerics_amd import workloads as W
from full_state import FullStateChecker, assert_counts, compare_bf16, compare_f32, parts


def _state(n, seed):
    rs = np.random.default_rng(seed)
    P = torch.from_numpy((rs.standard_normal(n) * 0.02).astype(np.float32)).to(torch.bfloat16)
    G = torch.from_numpy((rs.standard_normal(n) * 1e-3).astype(np.float32)).to(torch.bfloat16)
    m = torch.from_numpy((rs.standard_normal(n) * 1e-4).astype(np.float32))
    v = torch.from_numpy(rs.random(n).astype(np.float32) * 1e-7)
    return {"P": P, "M": P.to(torch.float32), "m": m, "v": v}, G


def _oracle_post(tbl, hp, pre, G, begin, scale, t, seed, master):
    h = {"P": pre["P"].view(torch.int16).numpy().view(np.uint16).copy(),
         "G": G.view(torch.int16).numpy().view(np.uint16).copy(),
         "M": pre["M"].numpy().copy() if master else None,
         "m": pre["m"].numpy().copy(), "v": pre["v"].numpy().copy()}
    o.adamw_step(tbl, begin, h["P"], h["G"], h["M"], h["m"], h["v"], hp, scale, t, seed)
    return {"P": torch.from_numpy(h["P"].view(np.int16)).view(torch.bfloat16),
            "M": torch.from_numpy(h["M"]) if master else None,
            "m": torch.from_numpy(h["m"]), "v": torch.from_numpy(h["v"])}


def test_parts_cover_and_align():
    for count, k in ((0, 4), (7, 4), (1000, 16), (12345, 3)):
        ps = parts(count, k)
        assert sum(b - a for a, b in ps) == count
        assert all(a % 8 == 0 for a, _ in ps)
        assert all(p[1] == q[0] for p, q in zip(ps, ps[1:]))


@pytest.mark.parametrize("master", [True, False])
def test_checker_equal_state_over_chunks(master):
    w = W.tiny()
    tbl = o.table(w.entries())
    hp = o.hparams(w.hparams.lr, w.hparams.beta1, w.hparams.beta2, w.hparams.eps, w.hparams.weight_decay)
    begin = 3000                                   # a window that starts mid-tensor
    n = 10_013
    pre, G = _state(n, 1)
    if not master:
        pre["M"] = None
    post = _oracle_post(tbl, hp, pre, G, begin, 0.5, 3, 77, master)
    chk = FullStateChecker(tbl, hp, 1.0, master, "cpu", chunk=1024, threads=3)
    counts, sumsq = chk.check_step(pre, post, G, begin, 0.5, 3, 77, o.ROUND_SR)
    assert all(c == 0 for c in counts.values()), counts
    assert sumsq == pytest.approx(o.grad_norm(G.view(torch.int16).numpy().view(np.uint16), 1.0)[0], rel=1e-12)
    rep = assert_counts(counts, n, "equal")
    assert rep["allowed_bf16"] == 0

    # one param one bf16 step off: counted, then refused by the allowance
    bad = dict(post)
    bad["P"] = post["P"].clone()
    bad["P"].view(torch.int16)[4321] += 1
    counts, _ = chk.check_step(pre, bad, G, begin, 0.5, 3, 77, o.ROUND_SR)
    assert counts["P"] == 1
    with pytest.raises(AssertionError):
        assert_counts(counts, n, "one step")
    assert assert_counts(counts, 2_000_000, "one step, large shard")["allowed_bf16"] == 2
    # two steps off: refused outright
    bad["P"].view(torch.int16)[4321] += 1
    with pytest.raises(AssertionError):
        chk.check_step(pre, bad, G, begin, 0.5, 3, 77, o.ROUND_SR)
    # a wrong seed moves many params: refused by the allowance
    counts, _ = chk.check_step(pre, post, G, begin, 0.5, 3, 78, o.ROUND_SR)
    assert counts["P"] > 100
    # fp32: within relative 1e-6 counted, beyond refused
    bad = dict(post)
    bad["m"] = post["m"].clone()
    bad["m"][9999] = float(np.nextafter(np.float32(post["m"][9999]), np.float32(np.inf)))
    counts, _ = chk.check_step(pre, bad, G, begin, 0.5, 3, 77, o.ROUND_SR)
    assert counts["m"] == 1
    bad["m"][10] = post["m"][10] * (1 + 1e-4)
    with pytest.raises(AssertionError):
        chk.check_step(pre, bad, G, begin, 0.5, 3, 77, o.ROUND_SR)
    chk.close()


def test_checker_host_reference_upload():
    w = W.tiny()
    tbl = o.table(w.entries())
    hp = o.hparams(w.hparams.lr, w.hparams.beta1, w.hparams.beta2, w.hparams.eps, w.hparams.weight_decay)
    n = w.n
    pre, G = _state(n, 2)
    chk = FullStateChecker(tbl, hp, 1.0, True, "cpu", chunk=4096, threads=4)
    h = {"P": pre["P"].view(torch.int16).numpy().view(np.uint16).copy(),
         "G": G.view(torch.int16).numpy().view(np.uint16).copy(),
         "M": pre["M"].numpy().copy(), "m": pre["m"].numpy().copy(), "v": pre["v"].numpy().copy()}
    chk.oracle_step_host(h, 0, 1.0, 1, 5, o.ROUND_SR)
    post = _oracle_post(tbl, hp, pre, G, 0, 1.0, 1, 5, True)   # one call over everything
    counts = chk.compare_host_to_device(post, h, "threaded oracle")
    assert all(c == 0 for c in counts.values()), counts
    chk.close()


def test_compare_nan_positions():
    a = torch.tensor([1.0, float("nan"), 2.0])
    b = torch.tensor([1.0, float("nan"), 2.0])
    assert compare_f32(a, b, "same") == 0
    with pytest.raises(AssertionError):
        compare_f32(a, torch.tensor([1.0, 3.0, 2.0]), "nan moved")
    x = torch.tensor([0x3F80, 0x7FC0, -0x4080], dtype=torch.int16)  # 1.0, NaN, -1.0 patterns
    assert compare_bf16(x, x.clone(), "same") == 0
    y = x.clone()
    y[2] = -0x4080 + 1                                             # one step, same sign
    assert compare_bf16(x, y, "one step") == 1
    z = x.clone()
    z[0] = 0x3F80 - 0x8000                                         # sign flipped
    with pytest.raises(AssertionError):
        compare_bf16(x, z, "sign")


def test_checker_segments_follow_a_per_tensor_shard():
    # A per-tensor shard (rank 1 of 2 of the d=32 model): shard elements map to
    # runs of global indices; the checker, told the runs, gives the oracle's
    # own mapped step over the whole shard, chunked across run boundaries.
    w = W.tiny()
    tbl = o.table(w.entries())
    hp = o.hparams(w.hparams.lr, w.hparams.beta1, w.hparams.beta2, w.hparams.eps, w.hparams.weight_decay)
    rc, gidx = o.shard_map_per_tensor(tbl, 2, 1)
    assert rc == o.OK
    S = gidx.size
    segs, lo = [], 0
    for j in range(1, S + 1):
        if j == S or gidx[j] != gidx[j - 1] + 1:
            segs.append((lo, j, int(gidx[lo])))
            lo = j
    pre, G = _state(S, 3)
    rs = np.random.default_rng(4)
    P_full = rs.integers(0, 1 << 16, w.n, dtype=np.uint64).astype(np.uint16)
    G_full = rs.integers(0, 1 << 16, w.n, dtype=np.uint64).astype(np.uint16) & 0x3FFF   # finite, small
    P_full[gidx] = pre["P"].view(torch.int16).numpy().view(np.uint16)
    G_full[gidx] = G.view(torch.int16).numpy().view(np.uint16)
    h = {"M": pre["M"].numpy().copy(), "m": pre["m"].numpy().copy(), "v": pre["v"].numpy().copy()}
    o.adamw_step_mapped(tbl, gidx, P_full, G_full, h["M"], h["m"], h["v"], hp, 0.7, 2, 99)
    post = {"P": torch.from_numpy(P_full[gidx].view(np.int16)).view(torch.bfloat16),
            "M": torch.from_numpy(h["M"]), "m": torch.from_numpy(h["m"]), "v": torch.from_numpy(h["v"])}
    chk = FullStateChecker(tbl, hp, 1.0, True, "cpu", chunk=1000, threads=3)
    counts, _ = chk.check_step(pre, post, G, 0, 0.7, 2, 99, o.ROUND_SR, segments=segs)
    assert all(c == 0 for c in counts.values()), counts
    # without the segments (as if the shard were contiguous from 0) the decay
    # flags and draws differ: refused
    with pytest.raises(AssertionError):
        chk.check_step(pre, post, G, 0, 0.7, 2, 99, o.ROUND_SR)
    chk.close()
