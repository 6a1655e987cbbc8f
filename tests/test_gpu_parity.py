"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Every case runs the library's kernels on cuda:0 and the oracle on the host
from the same seeded inputs.  Draws, shard offsets and decay masks must be
bit-exact; fp values must meet the bars in gpu_harness.
"""
import math

import numpy as np
import pytest
import torch

import oracle as o
from bf16_numerics_amd import workloads as W
from full_state import FullStateChecker, assert_counts, snapshot
from gpu_harness import (assert_bf16_parity, assert_f32_parity, assert_norm_parity,
                         assert_state_parity, dev_bf16, dev_f32, device_state, f32, host_copy,
                         oracle_hparams, oracle_step, step_seed, u16)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def bfo():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from bf16_numerics_amd import binding
    torch.cuda.set_device(0)
    return binding


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def ragged_workload(n_tiles=3, tail=13, seed=4):
    """Many small tensors (sizes 1..40 and a few large ones), alternating decay
    flags, n = n_tiles * 4096 + tail: crosses tiles, vectors and the ragged end."""
    rs = np.random.default_rng(seed)
    n = n_tiles * 4096 + tail
    tensors, off = [], 0
    while off < n:
        size = int(rs.integers(1, 41)) if rs.random() < 0.8 else int(rs.integers(500, 3000))
        size = min(size, n - off)
        shape = (size,) if rs.random() < 0.5 else (1, size)
        tensors.append((f"t{len(tensors)}", shape))
        off += size
    return W.Workload("ragged", tensors, grad_std=0.05, steps=3)


def windows(entries, b, e, half=40, n_random=24, seed=0):
    """Global [lo, hi) ranges around every tensor boundary inside [b, e), the
    shard ends, the powers of two from 2^31 where 32-bit element or byte
    offsets would wrap, and some random places; merged."""
    pts = {b, e} | {off for off, _, _ in entries if b < off < e}
    pts |= {1 << k for k in range(31, 36) if b < (1 << k) < e}
    rs = np.random.default_rng(seed)
    rng = [(max(b, p - half), min(e, p + half)) for p in pts]
    for x in rs.integers(b, max(b + 1, e - 64), n_random):
        rng.append((int(x), min(e, int(x) + 64)))
    rng.sort()
    merged = []
    for lo, hi in rng:
        if hi <= lo:
            continue
        if merged and lo <= merged[-1][1]:
            merged[-1] = (merged[-1][0], max(merged[-1][1], hi))
        else:
            merged.append((lo, hi))
    return merged


# --------------------------------------------------------------------- draws


@pytest.mark.parametrize("first,count,seed", [
    (0, 100_003, 0),
    (5, 4097, 0xDEADBEEF12345678),
    ((1 << 35) + 3, 10_001, 7),
    (6_738_415_616 - 4000, 4000, step_seed(20)),
    (2 ** 64 - 2000, 1990, 2 ** 64 - 1),
])
def test_rng_dump_bit_exact(bfo, first, count, seed):
    got = bfo.rng_dump(first, count, seed, DEV).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, o.rng16(first, count, seed))


# --------------------------------------------------------------------- decay masks


def test_decay_mask_tiny_all_shards(bfo):
    w = W.tiny()
    tbl = o.table(w.entries())
    for world in (1, 2, 4, 8):
        for r in range(world):
            T = bfo.Table(w.entries(), world, r)
            got = bfo.decay_mask_dump(T).cpu().numpy()
            assert np.array_equal(got, o.decay_mask(tbl, T.begin, T.size)), (world, r)


def test_decay_mask_ragged_full(bfo):
    w = ragged_workload(n_tiles=6, tail=5)
    T = bfo.Table(w.entries())
    got = bfo.decay_mask_dump(T).cpu().numpy()
    assert np.array_equal(got, o.decay_mask(o.table(w.entries()), 0, w.n))


@pytest.mark.parametrize("make", [W.gpt2_124m, W.gpt2_1p5b_shard, W.llama7b])
def test_decay_mask_windows_large(bfo, make):
    w = make()
    ents = w.entries()
    tbl = o.table(ents)
    for r in range(w.world):
        T = bfo.Table(ents, w.world, r)
        got = bfo.decay_mask_dump(T)
        for lo, hi in windows(ents, T.begin, T.end, seed=r):
            g = got[lo - T.begin:hi - T.begin].cpu().numpy()
            assert np.array_equal(g, o.decay_mask(tbl, lo, hi - lo)), (w.name, r, lo, hi)
        del got


# --------------------------------------------------------------------- norm


def _norm_case(bfo, bits):
    n = bits.size
    T = bfo.Table([(0, n, 1)] if n else [])
    G = dev_bf16(bits, DEV) if n else torch.empty(0, dtype=torch.bfloat16, device=DEV)
    res = bfo.new_norm_result(DEV)
    bfo.grad_global_norm(T, G, res, 1.0)
    got = bfo.read_norm_result(res)
    raw = res.cpu().numpy().tobytes()
    ref = o.grad_norm(np.ascontiguousarray(bits, np.uint16), 1.0)
    assert_norm_parity(got, ref)
    res.zero_()
    bfo.grad_global_norm(T, G, res, 1.0)
    assert res.cpu().numpy().tobytes() == raw        # bitwise repeatable
    return got


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 4096 * 3 + 5, 29_568, 2048 * 8 * 256 + 3, 5_000_011,
                               32_768 * 8192, 32_769 * 8192 + 5])
def test_norm_sizes(bfo, n):
    # the last two sizes sit on either side of the intermediate-reduction threshold
    rs = np.random.default_rng(n)
    x = rs.standard_normal(n, dtype=np.float32) * np.float32(1e-2)
    bits = W.bf16_bits_numpy(torch, torch.from_numpy(x).to(torch.bfloat16))
    got = _norm_case(bfo, bits)
    if n == 0:
        assert got == (0.0, 0.0, 1.0)


@pytest.mark.parametrize("make", [W.tiny, lambda: ragged_workload(9, 13), W.gpt2_124m])
def test_norm_flat_fast_path_equals_plan_path_bit_for_bit(bfo, make):
    # A flat table with 16-byte-aligned grads reads them directly; a
    # per-tensor table of one rank and a flat table given a 2-byte-aligned
    # copy go through the shard plan.  Same elements in the same order, same
    # partition: the three results must agree in every bit.
    w = make()
    ents = w.entries()
    G = torch.empty(w.n, dtype=torch.bfloat16, device=DEV)
    W.fill_grads(torch, w, G, 0, 1)
    buf = torch.zeros(w.n + 8, dtype=torch.bfloat16, device=DEV)
    buf[1:1 + w.n] = G
    Gmis = buf[1:1 + w.n]
    assert Gmis.data_ptr() % 16 != 0
    got = []
    for T, g in ((bfo.Table(ents), G), (bfo.Table(ents, 1, 0, layout=bfo.LAYOUT_PER_TENSOR), G),
                 (bfo.Table(ents), Gmis)):
        res = bfo.new_norm_result(DEV)
        bfo.grad_global_norm(T, g, res, w.hparams.max_norm)
        got.append(res.cpu().numpy().tobytes())
    assert got[0] == got[1] == got[2]
    assert_norm_parity(bfo.read_norm_result(res), o.grad_norm(u16(G), w.hparams.max_norm))
    # A per-tensor rank of four: tiles inside one run read at a fixed offset,
    # the others through the plan; a 2-byte-aligned copy takes the plan for
    # every tile.  Both must give the same bits, and the oracle's value.
    if all(numel % 4 == 0 for _, numel, _ in ents):
        T4 = bfo.Table(ents, 4, 1, layout=bfo.LAYOUT_PER_TENSOR)
        pair = []
        for g in (G, Gmis):
            res = bfo.new_norm_result(DEV)
            bfo.grad_global_norm(T4, g, res, w.hparams.max_norm)
            pair.append(res.cpu().numpy().tobytes())
        assert pair[0] == pair[1]
        gidx = T4.global_index().astype(np.int64)
        assert_norm_parity(bfo.read_norm_result(res), o.grad_norm(np.ascontiguousarray(u16(G)[gidx]),
                                                                  w.hparams.max_norm))


def test_norm_closed_form_and_extremes(bfo):
    assert _norm_case(bfo, np.full(1 << 24, 0x3A80, np.uint16)) == (16.0, 4.0, 0.25)
    assert _norm_case(bfo, np.zeros(1000, np.uint16)) == (0.0, 0.0, 1.0)
    big = _norm_case(bfo, np.array([0x7180] * 2 + [0] * 9, np.uint16))     # 2^100: beyond fp32 squares
    assert big[0] == 2.0 ** 201
    tiny = _norm_case(bfo, np.array([0x0380] * 4, np.uint16))              # 2^-120
    assert tiny[0] == 4 * 2.0 ** -240
    rs = np.random.default_rng(1)
    bits = rs.integers(0, 1 << 16, 100_000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    _norm_case(bfo, bits)                                                  # random patterns, norm overflows fp32


def test_norm_non_finite(bfo):
    bits = np.full(1000, 0x3C00, np.uint16)
    bits[17] = 0x7F80                                                      # +inf
    got = _norm_case(bfo, bits)
    assert math.isinf(got[1]) and got[2] == 0.0
    bits[500] = 0x7FC1                                                     # NaN
    got = _norm_case(bfo, bits)
    assert math.isnan(got[1]) and got[2] == 1.0


def test_norm_gpt2_124m_and_shards(bfo):
    w = W.gpt2_124m()
    G = torch.empty(w.n, dtype=torch.bfloat16, device=DEV)
    W.fill_grads(torch, w, G, 0, 1)
    T = bfo.Table(w.entries())
    res = bfo.new_norm_result(DEV)
    bfo.grad_global_norm(T, G, res, 1.0)
    got = bfo.read_norm_result(res)
    assert_norm_parity(got, o.grad_norm(u16(G), 1.0))
    assert got[1] > 1.0 and got[2] < 1.0                                   # clipping is active
    # ZeRO-1: shard sums add up to the global sum of squares
    parts = 0.0
    for r in range(4):
        Tr = bfo.Table(w.entries(), 4, r)
        bfo.grad_global_norm(Tr, G[Tr.begin:Tr.end], res, 1.0)
        parts += bfo.read_norm_result(res)[0]
    assert abs(parts - got[0]) <= 1e-12 * got[0]


def test_norm_workspace_size_and_two_streams(bfo):
    # The caller's workspace: its size follows the partition (none for shards
    # of at most 8 tiles, one binary64 per 8,192-element tile, one more per
    # 4,096 tiles above 32,768 tiles), and two norms of one table on two
    # streams with their own workspaces give the oracle's results, bit for bit
    # the same as one after the other.
    for S, want in ((1, 0), (8 * 8192, 0), (8 * 8192 + 1, 9 * 8), (32768 * 8192, 32768 * 8),
                    (32769 * 8192, (32769 + 9) * 8)):
        T = bfo.Table([(0, S, 0)])
        assert bfo.norm_workspace_bytes(T) == want, S
        T.close()
    n = 3 * (1 << 20) + 5
    T = bfo.Table([(0, n, 1)])
    grads = []
    for k in range(2):
        g = torch.empty(n, dtype=torch.bfloat16, device=DEV)
        W.fill_grads(torch, W.Workload("g", [("g", (n,))], grad_std=0.01 * (k + 1)), g, 0, k + 1)
        grads.append(g)
    ws = [bfo.new_norm_workspace(T) for _ in range(2)]
    serial = []
    for k in range(2):
        r = bfo.new_norm_result(DEV)
        bfo.grad_global_norm(T, grads[k], r, 1.0, workspace=ws[k])
        serial.append(r.cpu().numpy().tobytes())
    refs = [o.grad_norm(u16(g), 1.0) for g in grads]
    streams = [torch.cuda.Stream(device=DEV) for _ in range(2)]
    outs = [[bfo.new_norm_result(DEV) for _ in range(20)] for _ in range(2)]
    torch.cuda.synchronize()
    for i in range(20):                          # interleaved launches on the two streams
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                bfo.grad_global_norm(T, grads[k], outs[k][i], 1.0, workspace=ws[k])
    torch.cuda.synchronize()
    for k in range(2):
        for r in outs[k]:
            assert r.cpu().numpy().tobytes() == serial[k]
        assert_norm_parity(bfo.read_norm_result(outs[k][0]), refs[k])


def test_norm_max_norm_must_be_positive(bfo):
    n = 9 * 8192 + 1                                        # 10 tiles: the two-stage path
    T = bfo.Table([(0, n, 0)])
    G = torch.full((n,), 0.5, dtype=torch.bfloat16, device=DEV)
    res = bfo.new_norm_result(DEV)
    for bad in (0.0, -1.0, float("nan"), -float("inf")):
        with pytest.raises(bfo.BfoError) as e:
            bfo.grad_global_norm(T, G, res, bad)
        assert e.value.status == bfo.EINVAL, bad
    bfo.grad_global_norm(T, G, res, float("inf"))          # +inf: no clipping
    sumsq, norm, scale = bfo.read_norm_result(res)
    assert sumsq == 0.25 * n and scale == 1.0
    with pytest.raises(bfo.BfoError) as e:                  # workspace overlapping the grads
        bfo.grad_global_norm(T, G, res, 1.0, workspace=G.view(torch.uint8))
    assert e.value.status == bfo.EINVAL


# --------------------------------------------------------------------- update


def run_steps(bfo, w, T, tbl, st, h, steps, rounding=o.ROUND_SR, master=True, free_run=False,
              begin=0, check_each=True):
    res = bfo.new_norm_result(DEV)
    stats = []
    for t in range(1, steps + 1):
        W.fill_grads(torch, w, st["G"], begin, t)
        bfo.grad_global_norm(T, st["G"], res, w.hparams.max_norm)
        bfo.adamw_sr_step(T, st["P"], st["G"], st["M"] if master else None, st["m"], st["v"], w.hparams, t,
                          step_seed(t), scale=res, rounding=rounding)
        h["G"] = u16(st["G"])
        ref_norm = o.grad_norm(h["G"], w.hparams.max_norm)
        got_norm = bfo.read_norm_result(res)
        assert_norm_parity(got_norm, ref_norm)
        scale = ref_norm[2] if free_run else got_norm[2]
        oracle_step(tbl, begin, h, w.hparams, scale, t, step_seed(t), rounding)
        if check_each or t == steps:
            stats.append(assert_state_parity(host_copy(st), h, f"{w.name} t={t}"))
    return stats


def test_update_tiny_free_run_16_steps(bfo):
    w = W.tiny()
    T = bfo.Table(w.entries())
    st = device_state(w, 0, w.n, DEV)
    h = host_copy(st)
    stats = run_steps(bfo, w, T, o.table(w.entries()), st, h, w.steps, free_run=True)
    assert all(s == {"P": 0, "M": 0, "m": 0, "v": 0} for s in stats), stats
    # resume replay: the master alone rebuilds the bf16 weights bit for bit
    P2 = torch.empty_like(st["P"])
    bfo.master_to_bf16_sr(T, st["M"], P2, step_seed(w.steps))
    assert np.array_equal(u16(P2), u16(st["P"]))


@pytest.mark.parametrize("master,rounding", [(True, o.ROUND_SR), (True, o.ROUND_RNE),
                                             (False, o.ROUND_SR), (False, o.ROUND_RNE)])
@pytest.mark.parametrize("n_tiles,tail", [(3, 13), (1, 0), (0, 5), (5, 7)])
def test_update_ragged_modes(bfo, master, rounding, n_tiles, tail):
    w = ragged_workload(n_tiles, tail)
    T = bfo.Table(w.entries())
    st = device_state(w, 0, w.n, DEV, master=master)
    h = host_copy(st)
    run_steps(bfo, w, T, o.table(w.entries()), st, h, 3, rounding=rounding, master=master)


def test_update_gpt2_124m_all_ten_steps(bfo):
    # The whole 124M model, its 10 steps: the oracle carries its own copy of
    # the state from step to step on the host (fed the GPU's clip scale, the
    # norms being compared separately), and after every step each element of
    # P, M, m and v is compared with the GPU's.
    w = W.gpt2_124m()
    T = bfo.Table(w.entries())
    st = device_state(w, 0, w.n, DEV)
    h = host_copy(st)
    chk = FullStateChecker(o.table(w.entries()), oracle_hparams(w.hparams), w.hparams.max_norm, True, DEV)
    res = bfo.new_norm_result(DEV)
    for t in range(1, w.steps + 1):
        W.fill_grads(torch, w, st["G"], 0, t)
        bfo.grad_global_norm(T, st["G"], res, w.hparams.max_norm)
        bfo.adamw_sr_step(T, st["P"], st["G"], st["M"], st["m"], st["v"], w.hparams, t, step_seed(t), scale=res)
        h["G"] = u16(st["G"])
        got_norm = bfo.read_norm_result(res)
        assert_norm_parity(got_norm, o.grad_norm(h["G"], w.hparams.max_norm))
        chk.oracle_step_host(h, 0, got_norm[2], t, step_seed(t), o.ROUND_SR)
        counts = chk.compare_host_to_device(st, h, f"gpt2_124m t={t}")
        report(f"gpt2_124m t={t} (oracle state carried from t=1)", assert_counts(counts, w.n, f"gpt2_124m t={t}"))
    assert got_norm[2] < 1.0                           # the clip was active
    chk.close()


def _one_call_case(bfo, w, world, rank, layout, master, rounding, steps=3, nan_at=None):
    """The same steps through grad_global_norm + adamw_sr_step and through
    adamw_sr_step_with_norm, on copies of one state: identical bits."""
    T = bfo.Table(w.entries(), world, rank, layout=layout)
    n_pg = T.pg_size
    P0, _, _, _ = W.init_state(torch, w, 0, n_pg, DEV, master=False)
    a = {"P": P0, "M": (torch.randn(T.size, device=DEV) * 0.02) if master else None,
         "m": torch.zeros(T.size, device=DEV), "v": torch.zeros(T.size, device=DEV)}
    b = {k: (None if t is None else t.clone()) for k, t in a.items()}
    G = torch.empty(n_pg, dtype=torch.bfloat16, device=DEV)
    ra, rb = bfo.new_norm_result(DEV), bfo.new_norm_result(DEV)
    ws = bfo.new_norm_workspace(T)
    for t in range(1, steps + 1):
        W.fill_grads(torch, w, G, 0, t)
        if nan_at is not None and t == steps:
            G[nan_at] = float("nan")
        bfo.grad_global_norm(T, G, ra, w.hparams.max_norm)
        bfo.adamw_sr_step(T, a["P"], G, a["M"], a["m"], a["v"], w.hparams, t, step_seed(t), scale=ra,
                          rounding=rounding)
        bfo.adamw_sr_step_with_norm(T, b["P"], G, b["M"], b["m"], b["v"], w.hparams, t, step_seed(t), rb,
                                    w.hparams.max_norm, rounding=rounding, workspace=ws)
        assert ra.cpu().numpy().tobytes() == rb.cpu().numpy().tobytes(), ("norm", t)
    for k in ("P", "M", "m", "v"):
        if a[k] is not None:
            x, y = host_copy({k: a[k]})[k], host_copy({k: b[k]})[k]
            assert _same_bits(x, y), (k, w.name, world, rank, layout, master, rounding)
    return bfo.read_norm_result(rb)


@pytest.mark.parametrize("master,rounding", [(True, o.ROUND_SR), (False, o.ROUND_RNE)])
@pytest.mark.parametrize("case", ["tiny", "tiny_per_tensor", "tiny_misaligned", "ragged", "eight_tiles",
                                  "nine_tiles", "five"])
def test_one_call_step_equals_the_two_calls(bfo, case, master, rounding):
    # One launch for shards of at most 8 norm tiles (65,536 elements), the
    # two calls' launches above; every bit of the norm and the state equal.
    cases = {
        "tiny": (W.tiny(), 1, 0, bfo.LAYOUT_FLAT),
        "tiny_per_tensor": (W.tiny(), 2, 1, bfo.LAYOUT_PER_TENSOR),
        "tiny_misaligned": (padded_tiny(4), 4, 1, bfo.LAYOUT_FLAT),
        "ragged": (ragged_workload(3, 13), 1, 0, bfo.LAYOUT_FLAT),
        "eight_tiles": (W.Workload("e", [("a", (1000, 60)), ("b", (5536,))], grad_std=0.3), 1, 0,
                        bfo.LAYOUT_FLAT),
        "nine_tiles": (W.Workload("n", [("a", (1000, 60)), ("b", (5537,))], grad_std=0.3), 1, 0,
                       bfo.LAYOUT_FLAT),
        "five": (W.Workload("f", [("a", (5,))], grad_std=0.3), 1, 0, bfo.LAYOUT_FLAT),
    }
    w, world, rank, layout = cases[case]
    _one_call_case(bfo, w, world, rank, layout, master, rounding)


def test_one_call_step_skip_and_non_finite(bfo):
    w = W.tiny()
    got = _one_call_case(bfo, w, 1, 0, bfo.LAYOUT_FLAT, True, o.ROUND_SR, nan_at=77)
    assert math.isnan(got[1])
    T = bfo.Table(w.entries())
    st = device_state(w, 0, w.n, DEV)
    W.fill_grads(torch, w, st["G"], 0, 1)
    before = host_copy(st)
    res = bfo.new_norm_result(DEV)
    skip = torch.ones(1, dtype=torch.int32, device=DEV)
    bfo.adamw_sr_step_with_norm(T, st["P"], st["G"], st["M"], st["m"], st["v"], w.hparams, 1, step_seed(1), res,
                                skip=skip)
    after = host_copy(st)
    for k in ("P", "M", "m", "v"):
        assert _same_bits(before[k], after[k]), k
    assert_norm_parity(bfo.read_norm_result(res), o.grad_norm(before["G"], 1.0))      # the norm is still written
    with pytest.raises(bfo.BfoError) as e:                    # out inside m
        bfo.adamw_sr_step_with_norm(T, st["P"], st["G"], st["M"], st["m"], st["v"], w.hparams, 1, 1,
                                    st["m"][8:12].view(torch.float64))
    assert e.value.status == bfo.EINVAL


def test_update_is_deterministic(bfo):
    w = ragged_workload(40, 3)
    T = bfo.Table(w.entries())
    st = device_state(w, 0, w.n, DEV)
    W.fill_grads(torch, w, st["G"], 0, 1)
    snap = {k: v.clone() for k, v in st.items()}
    outs = []
    for _ in range(2):
        s2 = {k: v.clone() for k, v in snap.items()}
        res = bfo.new_norm_result(DEV)
        bfo.grad_global_norm(T, s2["G"], res)
        bfo.adamw_sr_step(T, s2["P"], s2["G"], s2["M"], s2["m"], s2["v"], w.hparams, 1, step_seed(1), scale=res)
        outs.append((res.cpu().numpy().tobytes(), host_copy(s2)))
    assert outs[0][0] == outs[1][0]
    for k in ("P", "M", "m", "v"):
        assert np.array_equal(outs[0][1][k].view(np.uint8), outs[1][1][k].view(np.uint8)), k


@pytest.mark.parametrize("rounding", [o.ROUND_SR, o.ROUND_RNE])
def test_master_path_never_reads_the_params(bfo, rounding):
    # With a master the update takes the old weight from the master and only
    # writes the bf16 params (which is why their stores may bypass the
    # caches): params holding NaN patterns before the step give the same
    # bits as the real params, on a whole buffer and on a rank whose params
    # and grads are views into full-length buffers starting mid-line.
    w = ragged_workload(40, 12)                        # n = 163,852: 4 shards of 40,963 (odd)
    for world, rank in ((1, 0), (4, 1)):
        T = bfo.Table(w.entries(), world, rank)
        b, e = T.begin, T.end
        st = device_state(w, b, e, DEV)
        W.fill_grads(torch, w, st["G"], b, 1)
        outs = []
        for poison in (False, True):
            P_full = torch.zeros(w.n, dtype=torch.bfloat16, device=DEV)
            G_full = torch.zeros(w.n, dtype=torch.bfloat16, device=DEV)
            P, G = P_full[b:e], G_full[b:e]
            P.copy_(st["P"])
            G.copy_(st["G"])
            if poison:
                P.view(torch.int16).fill_(0x7FC1)
            s2 = {"P": P, "G": G, "M": st["M"].clone(), "m": st["m"].clone(), "v": st["v"].clone()}
            res = bfo.new_norm_result(DEV)
            bfo.grad_global_norm(T, G, res)
            bfo.adamw_sr_step(T, P, G, s2["M"], s2["m"], s2["v"], w.hparams, 1, step_seed(1), scale=res,
                              rounding=rounding)
            outs.append(host_copy(s2))
        for k in ("P", "M", "m", "v"):
            assert np.array_equal(outs[0][k].view(np.uint8), outs[1][k].view(np.uint8)), (world, rank, k)


def test_shard_concatenation_bit_identical(bfo):
    # Running each 1/N shard separately rebuilds the unsharded result bit for
    # bit (the draws are keyed on the global index), with the global clip scale.
    w = W.tiny()
    base = device_state(w, 0, w.n, DEV)
    grads = []
    for t in range(1, 4):
        W.fill_grads(torch, w, base["G"], 0, t)
        grads.append(base["G"].clone())
    Tfull = bfo.Table(w.entries())

    def run(world):
        st = {k: v.clone() for k, v in base.items()}
        res = bfo.new_norm_result(DEV)
        tables = [bfo.Table(w.entries(), world, r) for r in range(world)]
        for t, G in enumerate(grads, 1):
            bfo.grad_global_norm(Tfull, G, res)             # the all-reduced norm
            for T in tables:
                sl = slice(T.begin, T.end)
                bfo.adamw_sr_step(T, st["P"][sl], G[sl], st["M"][sl], st["m"][sl], st["v"][sl], w.hparams,
                                  t, step_seed(t), scale=res)
        return host_copy(st)

    one = run(1)
    for world in (2, 4, 8):
        other = run(world)
        for k in ("P", "M", "m", "v"):
            assert np.array_equal(one[k].view(np.uint8), other[k].view(np.uint8)), (world, k)


def test_master_to_bf16_sr_special_values(bfo):
    rs = np.random.default_rng(8)
    n = 4096 * 2 + 6
    bits = rs.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    bits[:12] = [0x7F800000, 0xFF800000, 0x7FC00001, 0xFFFFFFFF, 0x7F7FFFFF, 0x00000001,
                 0x80000001, 0x007FFFFF, 0x00000000, 0x80000000, 0x3F808000, 0xBF80FFFF]
    M = bits.view(np.float32)
    T = bfo.Table([(0, n, 0)])
    P = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    for seed in (0, step_seed(3), 2 ** 64 - 1):
        bfo.master_to_bf16_sr(T, dev_f32(M, DEV), P, seed)
        got = u16(P)
        ref = o.master_to_bf16_sr(M, 0, seed)
        nan = (ref & 0x7FFF) > 0x7F80
        assert np.array_equal((got & 0x7FFF) > 0x7F80, nan)
        assert np.array_equal(got[~nan], ref[~nan])


def test_update_non_finite_grads(bfo):
    w = ragged_workload(2, 3)
    T = bfo.Table(w.entries())
    st = device_state(w, 0, w.n, DEV)
    W.fill_grads(torch, w, st["G"], 0, 1)
    st["G"][10] = float("nan")
    st["G"][4000] = float("inf")
    st["G"][4001] = float("-inf")
    h = host_copy(st)
    bfo.adamw_sr_step(T, st["P"], st["G"], st["M"], st["m"], st["v"], w.hparams, 1, step_seed(1), scale=None)
    oracle_step(o.table(w.entries()), 0, h, w.hparams, 1.0, 1, step_seed(1))
    assert_state_parity(host_copy(st), h, "non-finite")


def _special_state(n, master, seed=11):
    """Finite state built from edge values: fp32 subnormals of both signs,
    signed zeros, the smallest normal, values near the fp32 maximum, bf16
    subnormal and near-boundary grads; no NaN (its payload is not pinned)."""
    rs = np.random.default_rng(seed)
    f = np.float32
    m_vals = np.array([0.0, -0.0, 1e-40, -1e-40, 1.4e-45, -1.4e-45, 1.17549435e-38, -3.5e-39, 2.5e-3, -7.0e-4],
                      f)
    v_vals = np.array([0.0, 1e-40, 1.4e-45, 1.17549435e-38, 3.0e-39, 6.25e-6, 1e-12, 0.5], f)
    w_vals = np.array([0.0, -0.0, 1e-40, -1e-40, 1.17549435e-38, 1.0, -1.0, 3.3e38, -3.3e38, 65504.0, 1e-3,
                       -2.0 ** -126, 1.0 + 2.0 ** -9], f)
    g_bits = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x5F0B, 0xDF0B,
                       0x3A83, 0x2F80], np.uint16)     # 0x5F0B ~ 1e19: its square stays finite in fp32
    pick = lambda vals: vals[rs.integers(0, vals.size, n)]
    st = {"m": pick(m_vals), "v": pick(v_vals), "G": pick(g_bits)}
    M = pick(w_vals)
    st["M"] = M if master else None
    st["P"] = (M.view(np.uint32) >> 16).astype(np.uint16) if master else pick(g_bits ^ np.uint16(0x0100))
    return st


@pytest.mark.parametrize("master", [True, False])
@pytest.mark.parametrize("rounding", [o.ROUND_SR, o.ROUND_RNE])
@pytest.mark.parametrize("bias_correction,t", [(True, 1), (True, 1000), (False, 7)])
def test_update_edge_values_bit_exact(bfo, master, rounding, bias_correction, t):
    # Subnormal moments and weights, signed zeros, near-overflow weights and
    # bf16-subnormal grads go through the fp32 sequence with denormals kept:
    # every output bit must equal the oracle's.
    w = ragged_workload(3, 13, seed=9)
    ents = w.entries()
    T = bfo.Table(ents)
    h = _special_state(w.n, master)
    hp = W.HParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, bias_correction=bias_correction)
    st = {"P": dev_bf16(h["P"], DEV), "G": dev_bf16(h["G"], DEV), "m": dev_f32(h["m"], DEV),
          "v": dev_f32(h["v"], DEV), "M": dev_f32(h["M"], DEV) if master else None}
    bfo.adamw_sr_step(T, st["P"], st["G"], st["M"], st["m"], st["v"], hp, t, step_seed(t), scale=None,
                      rounding=rounding)
    ref = {k: (None if a is None else a.copy()) for k, a in h.items()}
    o.adamw_step(o.table(ents), 0, ref["P"], ref["G"], ref["M"], ref["m"], ref["v"], oracle_hparams(hp), 1.0, t,
                 step_seed(t), rounding)
    got = host_copy(st)
    assert np.array_equal(got["P"], ref["P"]), "bf16 params differ"
    for k in ("m", "v") + (("M",) if master else ()):
        assert np.array_equal(got[k].view(np.uint32), ref[k].view(np.uint32)), f"{k} differs"
    sub = (np.abs(ref["m"]) < 1.17549435e-38) & (ref["m"] != 0)
    assert sub.any(), "the case should leave subnormal moments"


def test_empty_shard(bfo):
    T = bfo.Table([])
    res = bfo.new_norm_result(DEV)
    e16 = torch.empty(0, dtype=torch.bfloat16, device=DEV)
    e32 = torch.empty(0, dtype=torch.float32, device=DEV)
    bfo.grad_global_norm(T, e16, res)
    assert bfo.read_norm_result(res) == (0.0, 0.0, 1.0)
    bfo.adamw_sr_step(T, e16, e16, e32, e32, e32, W.HParams(), 1, 1, scale=res)
    bfo.master_to_bf16_sr(T, e32, e16, 1)
    torch.cuda.synchronize()


def test_misaligned_and_wrong_size_rejected(bfo):
    w = W.tiny()
    T = bfo.Table(w.entries())
    st = device_state(w, 0, w.n + 8, DEV)
    sl = slice(1, w.n + 1)                               # 2-byte / 4-byte offset views
    with pytest.raises(bfo.BfoError) as e:
        bfo.adamw_sr_step(T, st["P"][sl], st["G"][sl], st["M"][sl], st["m"][sl], st["v"][sl], w.hparams, 1, 1)
    assert e.value.status == bfo.EMISALIGNED
    with pytest.raises(ValueError):
        bfo.adamw_sr_step(T, st["P"], st["G"], st["M"], st["m"], st["v"], w.hparams, 1, 1)
    with pytest.raises(bfo.BfoError) as e:
        bfo.adamw_sr_step(T, st["P"][:w.n], st["G"][:w.n], st["M"][:w.n], st["m"][:w.n], st["v"][:w.n],
                          w.hparams, 0, 1)
    assert e.value.status == bfo.EINVAL


def test_overlapping_arrays_rejected(bfo):
    # Arrays of one call that share bytes are refused before any work is
    # queued; arrays that only touch (one ends where the next begins) are
    # fine.
    import ctypes
    w = W.tiny()
    n = w.n
    T = bfo.Table(w.entries())
    st = device_state(w, 0, n, DEV)
    W.fill_grads(torch, w, st["G"], 0, 1)
    both = torch.zeros(2 * n + 8, dtype=torch.float32, device=DEV)
    before = {k: t.clone() for k, t in st.items()}
    cases = [
        (st["P"], st["P"], st["M"], st["m"], st["v"], None),          # params are the grads
        (st["P"], st["G"], st["M"], both[:n], both[8:n + 8], None),   # m and v overlap
        (st["P"], st["G"], st["m"], st["m"], st["v"], None),          # master is m
        (st["P"], st["G"], st["M"], st["m"], st["v"], st["v"].data_ptr() + 64),  # scale inside v
    ]
    for P, G, M, m, v, scale in cases:
        with pytest.raises(bfo.BfoError) as e:
            bfo.adamw_sr_step(T, P, G, M, m, v, w.hparams, 1, 1, scale=scale)
        assert e.value.status == bfo.EINVAL
    lib, stream = bfo.library(), ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    g = ctypes.c_void_p(st["G"].data_ptr())
    assert lib.grad_global_norm(T.handle, g, ctypes.c_float(1.0), None, g, stream) == bfo.EINVAL
    mp = ctypes.c_void_p(st["M"].data_ptr())
    assert lib.master_to_bf16_sr(T.handle, mp, mp, ctypes.c_uint64(1), stream) == bfo.EINVAL
    torch.cuda.synchronize()
    for k, t in st.items():
        assert torch.equal(t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32),
                           before[k].view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)), k
    # touching, not overlapping: m and v as the two halves of one buffer
    bfo.adamw_sr_step(T, st["P"], st["G"], st["M"], both[:n], both[n:2 * n], w.hparams, 1, 1)
    torch.cuda.synchronize()


# --------------------------------------------------------------------- stall


def test_stall16m_sr_tracks_master_rne_freezes(bfo):
    w = W.stall16m()
    n = w.n
    T = bfo.Table(w.entries())
    P0, M0, _, _ = W.init_state(torch, w, 0, n, DEV)
    G = torch.full((n,), w.grad_const, dtype=torch.bfloat16, device=DEV)
    runs = {}
    for name, master, rnd in (("A", True, o.ROUND_SR), ("B", False, o.ROUND_SR), ("C", False, o.ROUND_RNE)):
        st = {"P": P0.clone(), "M": M0.clone() if master else None,
              "m": torch.zeros(n, device=DEV), "v": torch.zeros(n, device=DEV), "G": G}
        h = host_copy(st)
        for t in range(1, w.steps + 1):
            bfo.adamw_sr_step(T, st["P"], G, st["M"], st["m"], st["v"], w.hparams, t, step_seed(t),
                              scale=None, rounding=rnd)
            if t == 1:   # first step bit-compared in full against the oracle
                oracle_step(o.table(w.entries()), 0, h, w.hparams, 1.0, 1, step_seed(1), rnd)
                assert_state_parity(host_copy(st), h, f"stall {name} t=1")
        runs[name] = st
    p0 = P0.double()
    drift_master = runs["A"]["M"].double() - p0
    drift_sr = runs["B"]["P"].double() - p0
    diff = runs["B"]["P"].double() - runs["A"]["M"].double()
    bound = 3 * diff.std().item() / math.sqrt(n)
    print(f"stall: master drift {drift_master.mean().item():.6f}, SR drift {drift_sr.mean().item():.6f}, "
          f"3-sigma {bound:.2e}", flush=True)
    assert abs(drift_master.mean().item() - 0.78) < 0.01
    assert abs(drift_sr.mean().item() - drift_master.mean().item()) <= bound
    assert torch.equal(runs["C"]["P"].view(torch.int16), P0.view(torch.int16))


# --------------------------------------------------------------------- full sizes


def report(what, rep):
    """Print a full-state parity report and, when BFO_PARITY_REPORT names a
    file, append it there as one JSON line."""
    import json
    import os
    line = json.dumps({"case": what, **rep})
    print(line, flush=True)
    path = os.environ.get("BFO_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


def full_size_step(bfo, w, rank, steps=1, master=True, rounding=o.ROUND_SR, check=None, what=None):
    """One rank of a full-size workload in the layout the benchmark times:
    full-length P and G buffers (ZeRO-1), shard-local M, m, v.  Steps `check`
    (default: all) are compared with the oracle over every element of the
    shard: the state before the step is kept in device memory, and the
    oracle steps it chunk by chunk on the host threads (full_state)."""
    check = set(range(1, steps + 1)) if check is None else set(check)
    ents = w.entries()
    T = bfo.Table(ents, w.world, rank)
    b, e = T.begin, T.end
    S = e - b
    P_full = torch.empty(w.n if w.world > 1 else 0, dtype=torch.bfloat16, device=DEV)
    P, M, m, v = W.init_state(torch, w, b, e, DEV, master=master)
    if w.world > 1:
        P_full.view(torch.int16).fill_(0x7FA5)                             # sentinel NaN pattern
        P_full[b:e] = P
        del P
        P = P_full[b:e]
    G = torch.empty(S, dtype=torch.bfloat16, device=DEV)
    st = {"P": P, "M": M, "m": m, "v": v}
    res = bfo.new_norm_result(DEV)
    chk = FullStateChecker(o.table(ents), oracle_hparams(w.hparams), w.hparams.max_norm, master, DEV)
    label = what or f"{w.name} rank {rank}/{w.world} master={master} rounding={rounding}"
    for t in range(1, steps + 1):
        W.fill_grads(torch, w, G, b, t)
        pre = snapshot(st) if t in check else None
        bfo.grad_global_norm(T, G, res, w.hparams.max_norm)
        bfo.adamw_sr_step(T, P, G, M, m, v, w.hparams, t, step_seed(t), scale=res, rounding=rounding)
        got_norm = bfo.read_norm_result(res)
        if t not in check:
            continue
        counts, sumsq = chk.check_step(pre, st, G, b, got_norm[2], t, step_seed(t), rounding)
        del pre
        torch.cuda.empty_cache()
        assert_norm_parity(got_norm, (sumsq, *o.norm_from_sumsq(sumsq, w.hparams.max_norm)))
        report(f"{label} t={t}", assert_counts(counts, S, f"{label} t={t}"))
    chk.close()
    if w.world > 1:
        outside = torch.cat([P_full[:b], P_full[e:]]).view(torch.int16)
        assert bool((outside == 0x7FA5).all()), "a write escaped the shard"
    return got_norm


def test_full_size_gpt2_1p5b_shard(bfo):
    w = W.gpt2_1p5b_shard()
    # Every rank of the 1/8 shards, two steps each, every element of P, M, m
    # and v against the oracle.
    for rank in (1, 0, 2, 3, 4, 5, 6, 7):
        got = full_size_step(bfo, w, rank, steps=2)
        print(f"gpt2_1p5b rank {rank}: norm {got[1]:.6f} scale {got[2]:.6f}", flush=True)


@pytest.mark.parametrize("master,rounding", [(False, o.ROUND_SR), (False, o.ROUND_RNE), (True, o.ROUND_RNE)])
def test_full_size_gpt2_1p5b_shard_variants(bfo, master, rounding):
    # The other update variants at the benchmark's size and shard: no master
    # (old weights read from the bf16 params), round to nearest even.
    w = W.gpt2_1p5b_shard()
    got = full_size_step(bfo, w, w.rank, steps=2, master=master, rounding=rounding)
    print(f"gpt2_1p5b rank {w.rank} master={master} rounding={rounding}: scale {got[2]:.6f}", flush=True)


def test_full_size_gpt2_1p5b_shard_in_the_benchmark_placement(bfo):
    # The benchmark's own arrays: params, a two-buffer grads pool, master, m
    # and v carved from one arena of most of device memory, each on its own
    # 16 GiB region (bench.state_arrays, spread placement), the launches
    # bench.py times; two steps, sampled windows against the oracle.
    import bench
    w = W.gpt2_1p5b_shard()
    ents = w.entries()
    T = bfo.Table(ents, w.world, w.rank)
    b, e = T.begin, T.end
    S = e - b
    g_stride = (S + 127) // 128 * 128
    arrays = bench.state_arrays(torch, bfo, torch.device(DEV), "spread", w.n, g_stride, 2, S, True,
                                (16 << 30) + S * 6)
    P_full, pool_mem, M, m, v = (arrays[k] for k in ("P", "G", "M", "m", "v"))
    assert arrays["arena_bytes"] > 0
    P_full.view(torch.int16).fill_(0x7FA5)                                 # sentinel NaN pattern
    P = P_full[b:e]
    W.init_params_into(torch, w, b, P, M)
    m.zero_()
    v.zero_()
    pool = [pool_mem[k * g_stride:k * g_stride + S] for k in range(2)]
    st = {"P": P, "M": M, "m": m, "v": v}
    res = bfo.new_norm_result(DEV)
    chk = FullStateChecker(o.table(ents), oracle_hparams(w.hparams), w.hparams.max_norm, True, DEV)
    for t in (1, 2):
        G = pool[t - 1]
        W.fill_grads(torch, w, G, b, t)
        pre = snapshot(st)
        bfo.grad_global_norm(T, G, res, w.hparams.max_norm)
        bfo.adamw_sr_step(T, P, G, M, m, v, w.hparams, t, step_seed(t), scale=res)
        got_norm = bfo.read_norm_result(res)
        counts, sumsq = chk.check_step(pre, st, G, b, got_norm[2], t, step_seed(t), o.ROUND_SR)
        del pre
        assert_norm_parity(got_norm, (sumsq, *o.norm_from_sumsq(sumsq, w.hparams.max_norm)))
        report(f"gpt2_1p5b_shard rank {w.rank} spread placement t={t}", assert_counts(counts, S, f"spread t={t}"))
    chk.close()
    outside = torch.cat([P_full[:b], P_full[e:]]).view(torch.int16)
    assert bool((outside == 0x7FA5).all()), "a write escaped the shard"
    del arrays, P_full, pool_mem, M, m, v, P, pool, st


def test_full_size_rebuild_gpt2_1p5b_shard(bfo):
    # The resume rebuild at the benchmark's size and shard: after a step, the
    # master and that step's seed give back the step's bf16 params bit for
    # bit, and sampled windows equal the oracle's rebuild of the same master.
    w = W.gpt2_1p5b_shard()
    ents = w.entries()
    T = bfo.Table(ents, w.world, w.rank)
    b, e = T.begin, T.end
    P, M, m, v = W.init_state(torch, w, b, e, DEV)
    G = torch.empty(e - b, dtype=torch.bfloat16, device=DEV)
    W.fill_grads(torch, w, G, b, 1)
    res = bfo.new_norm_result(DEV)
    bfo.grad_global_norm(T, G, res, w.hparams.max_norm)
    bfo.adamw_sr_step(T, P, G, M, m, v, w.hparams, 1, step_seed(1), scale=res)
    P2 = torch.zeros_like(P)
    bfo.master_to_bf16_sr(T, M, P2, step_seed(1))
    assert torch.equal(P2.view(torch.int16), P.view(torch.int16))
    chk = FullStateChecker(o.table(ents), oracle_hparams(w.hparams), w.hparams.max_norm, True, DEV)
    assert chk.check_rebuild(M, P2, b, step_seed(1)) == e - b           # every element, bit for bit
    chk.close()


@pytest.mark.timeout(900)
def test_full_size_llama7b(bfo):
    # 20 steps of the 6.74e9-element state (all in one shard, past 2^32
    # elements); steps 1, 2, 10 and 20 compared with the oracle over every
    # element (the pre-step state is kept beside the live one: 94 GB more).
    w = W.llama7b()
    got = full_size_step(bfo, w, 0, steps=20, check=(1, 2, 10, 20))
    print(f"llama7b: norm {got[1]:.6f} scale {got[2]:.6f}", flush=True)
    assert got[2] < 1.0


@pytest.mark.timeout(600)
def test_full_size_llama7b_no_master(bfo):
    # The no-master update (old weights read from the bf16 params; lanes pair
    # up to share Philox blocks) over the whole 6.74e9-element state, global
    # indices past 2^32: steps 1 and 2 against the oracle on every element.
    w = W.llama7b()
    got = full_size_step(bfo, w, 0, steps=2, master=False)
    print(f"llama7b no master: norm {got[1]:.6f} scale {got[2]:.6f}", flush=True)


def test_full_size_gpt2_1p5b_eight_shards_equal_the_unsharded_step(bfo):
    # The ZeRO-1 invariant at full size: the 8 ranks' flat shards, stepped
    # with the global clip scale into one shared param buffer, reproduce the
    # unsharded two-step run bit for bit (P, M, m, v), and the 8 per-rank
    # sums of squares add up to the global one.
    w = W.gpt2_1p5b_shard()
    ents = w.entries()
    n = w.n
    P0, M0, _, _ = W.init_state(torch, w, 0, n, DEV)
    G = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    Tfull = bfo.Table(ents)
    res = bfo.new_norm_result(DEV)
    ref = {"P": P0.clone(), "M": M0.clone(), "m": torch.zeros(n, device=DEV), "v": torch.zeros(n, device=DEV)}
    sh = {"P": P0, "M": M0, "m": torch.zeros(n, device=DEV), "v": torch.zeros(n, device=DEV)}
    tables = [bfo.Table(ents, w.world, r) for r in range(w.world)]
    rres = bfo.new_norm_result(DEV)
    for t in (1, 2):
        W.fill_grads(torch, w, G, 0, t)
        bfo.grad_global_norm(Tfull, G, res, w.hparams.max_norm)
        bfo.adamw_sr_step(Tfull, ref["P"], G, ref["M"], ref["m"], ref["v"], w.hparams, t, step_seed(t), scale=res)
        total = 0.0
        for T in tables:
            b, e = T.begin, T.end
            bfo.grad_global_norm(T, G[b:e], rres, w.hparams.max_norm)
            total += bfo.read_norm_result(rres)[0]
            bfo.adamw_sr_step(T, sh["P"][b:e], G[b:e], sh["M"][b:e], sh["m"][b:e], sh["v"][b:e], w.hparams, t,
                              step_seed(t), scale=res)
        glob = bfo.read_norm_result(res)[0]
        assert abs(total - glob) <= 1e-12 * glob, (total, glob)
        for k in ("P", "M", "m", "v"):
            a = sh[k].view(torch.int16 if k == "P" else torch.int32)
            r = ref[k].view(torch.int16 if k == "P" else torch.int32)
            assert torch.equal(a, r), f"{k} differs from the unsharded run at t={t}"
        print(f"t={t}: 8 shards == unsharded (n={n}), sumsq {glob:.6f}", flush=True)


def per_tensor_full_size(bfo, w, world, rank, steps=2):
    """llm.c's ZeRO-1 layout at full size: rank `rank` of `world` owns 1/world
    of every tensor; P and G are the full n-element buffers.  Every shard
    element of P, M, m and v is compared with the oracle after each step
    (gathered to shard order on the device, the oracle stepping each run of
    consecutive global indices), the norm over the whole shard, and every
    params position outside the shard must keep its bits."""
    ents = w.entries()
    tbl = o.table(ents)
    T = bfo.Table(ents, world, rank, layout=bfo.LAYOUT_PER_TENSOR)
    S = T.size
    gidx = _oracle_gidx(bfo, tbl, w, world, rank, bfo.LAYOUT_PER_TENSOR)
    assert S == w.n // world and np.array_equal(T.global_index(), gidx)
    P, M_full, m0, v0 = W.init_state(torch, w, 0, w.n, DEV)
    del m0, v0
    gi = torch.from_numpy(gidx.astype(np.int64)).to(DEV)
    del gidx
    st = {"M": M_full[gi].clone(), "m": torch.zeros(S, device=DEV), "v": torch.zeros(S, device=DEV)}
    del M_full
    torch.cuda.empty_cache()
    G = torch.empty(w.n, dtype=torch.bfloat16, device=DEV)
    res = bfo.new_norm_result(DEV)
    segs = [(local, local + length, glob) for local, _addr, glob, length, _flags in T.runs()]
    chk = FullStateChecker(tbl, oracle_hparams(w.hparams), w.hparams.max_norm, True, DEV)
    for t in range(1, steps + 1):
        W.fill_grads(torch, w, G, 0, t)
        P_before = P.clone()
        pre = {"P": P[gi], "M": st["M"].clone(), "m": st["m"].clone(), "v": st["v"].clone()}
        G_loc = G[gi]
        bfo.grad_global_norm(T, G, res, w.hparams.max_norm)
        bfo.adamw_sr_step(T, P, G, st["M"], st["m"], st["v"], w.hparams, t, step_seed(t), scale=res)
        got = bfo.read_norm_result(res)
        post = {"P": P[gi], "M": st["M"], "m": st["m"], "v": st["v"]}
        counts, sumsq = chk.check_step(pre, post, G_loc, 0, got[2], t, step_seed(t), o.ROUND_SR, segments=segs)
        assert_norm_parity(got, (sumsq, *o.norm_from_sumsq(sumsq, w.hparams.max_norm)))
        report(f"{w.name} per-tensor rank {rank}/{world} t={t}", assert_counts(counts, S, f"per-tensor t={t}"))
        P_before[gi] = post["P"]
        assert torch.equal(P_before.view(torch.int16), P.view(torch.int16)), "a write escaped the shard"
        del pre, post, G_loc, P_before
        torch.cuda.empty_cache()
    chk.close()


def test_full_size_gpt2_1p5b_per_tensor(bfo):
    w = W.gpt2_1p5b_shard()
    per_tensor_full_size(bfo, w, w.world, w.rank)


def test_full_size_llama7b_per_tensor_last_rank(bfo):
    # Rank 7 of 8 holds the last eighth of every tensor: its positions in the
    # 6.74e9-element params and grads run past 2^32 and 2^32 - 1 bytes.
    per_tensor_full_size(bfo, W.llama7b(), 8, 7)


# --------------------------------------------------------------------- layouts


def padded_tiny(pad):
    """The d=32 model plus a trailing 1-D tensor of `pad` elements, so that
    n / world stops being a multiple of 8 (misaligned flat shard starts)."""
    w = W.tiny()
    w.tensors = list(w.tensors) + [("pad", (pad,))]
    return w


LAYOUT_CASES = [("flat", W.tiny, 8), ("flat_misaligned", lambda: padded_tiny(4), 4),
                ("per_tensor", W.tiny, 8), ("per_tensor", W.tiny, 2)]


def _oracle_gidx(bfo, tbl, w, world, rank, layout):
    if layout == bfo.LAYOUT_PER_TENSOR:
        rc, g = o.shard_map_per_tensor(tbl, world, rank)
        assert rc == o.OK
        return g
    rc, b, e = o.shard_range(w.n, world, rank)
    assert rc == o.OK
    return np.arange(b, e, dtype=np.uint64)


@pytest.mark.parametrize("name,make,world", LAYOUT_CASES)
def test_shard_plan_matches_oracle(bfo, name, make, world):
    w = make()
    ents = w.entries()
    tbl = o.table(ents)
    layout = bfo.LAYOUT_PER_TENSOR if name == "per_tensor" else bfo.LAYOUT_FLAT
    decay_all = o.decay_mask(tbl, 0, w.n)
    for r in range(world):
        T = bfo.Table(ents, world, r, layout=layout)
        gidx = _oracle_gidx(bfo, tbl, w, world, r, layout)
        assert np.array_equal(T.global_index(), gidx), (name, r)
        dm = bfo.decay_mask_dump(T).cpu().numpy()
        assert np.array_equal(dm, decay_all[gidx]), (name, r)


@pytest.mark.parametrize("name,make,world", LAYOUT_CASES)
@pytest.mark.parametrize("master", [True, False])
def test_update_layouts_all_ranks(bfo, name, make, world, master):
    # Every rank's shard is stepped on the GPU and by the oracle from the same
    # full initial state; the shards together must also rebuild the unsharded
    # GPU run bit for bit.  The clip scale is the global one (world=1 norm).
    w = make()
    w.grad_std = 0.05                                    # clip active
    ents = w.entries()
    tbl = o.table(ents)
    layout = bfo.LAYOUT_PER_TENSOR if name == "per_tensor" else bfo.LAYOUT_FLAT
    P0, M0, _, _ = W.init_state(torch, w, 0, w.n, DEV)
    Gs = []
    for t in range(1, 4):
        G = torch.empty(w.n, dtype=torch.bfloat16, device=DEV)
        W.fill_grads(torch, w, G, 0, t)
        Gs.append(G)
    Tfull = bfo.Table(ents)
    res = bfo.new_norm_result(DEV)

    # unsharded reference run on the GPU
    ref = {"P": P0.clone(), "M": M0.clone(), "m": torch.zeros(w.n, device=DEV), "v": torch.zeros(w.n, device=DEV)}
    for t, G in enumerate(Gs, 1):
        bfo.grad_global_norm(Tfull, G, res)
        bfo.adamw_sr_step(Tfull, ref["P"], G, ref["M"] if master else None, ref["m"], ref["v"], w.hparams, t,
                          step_seed(t), scale=res)

    P = P0.clone()
    Ph = u16(P0)
    Gh = [u16(G) for G in Gs]
    ranks = []
    for r in range(world):
        T = bfo.Table(ents, world, r, layout=layout)
        gidx = _oracle_gidx(bfo, tbl, w, world, r, layout)
        gi = torch.from_numpy(gidx.astype(np.int64)).to(DEV)
        st = {"M": M0[gi].clone() if master else None, "m": torch.zeros(T.size, device=DEV),
              "v": torch.zeros(T.size, device=DEV)}
        h = {"M": f32(st["M"]) if master else None, "m": np.zeros(T.size, np.float32),
             "v": np.zeros(T.size, np.float32)}
        ranks.append((T, gidx, st, h))
    for t, G in enumerate(Gs, 1):
        bfo.grad_global_norm(Tfull, G, res)
        scale = bfo.read_norm_result(res)[2]
        for T, gidx, st, h in ranks:
            if layout == bfo.LAYOUT_PER_TENSOR:
                Pa, Ga = P, G
            else:
                Pa, Ga = P[T.begin:T.end], G[T.begin:T.end]
            rres = bfo.new_norm_result(DEV)
            bfo.grad_global_norm(T, Ga, rres)
            assert_norm_parity(bfo.read_norm_result(rres), o.grad_norm(np.ascontiguousarray(Gh[t - 1][gidx])))
            bfo.adamw_sr_step(T, Pa, Ga, st["M"], st["m"], st["v"], w.hparams, t, step_seed(t), scale=res)
            o.adamw_step_mapped(tbl, gidx, Ph, Gh[t - 1], h["M"], h["m"], h["v"], oracle_hparams(w.hparams), scale,
                                t, step_seed(t))
    assert_bf16_parity(u16(P), Ph, f"{name} params")
    assert np.array_equal(u16(P), u16(ref["P"])), "sharded run differs from the unsharded one"
    for T, gidx, st, h in ranks:
        gi = torch.from_numpy(gidx.astype(np.int64)).to(DEV)
        for k in ("m", "v") + (("M",) if master else ()):
            assert_f32_parity(f32(st[k]), h[k], f"{name} {k}")
            assert np.array_equal(f32(st[k]).view(np.uint32), f32(ref[k][gi]).view(np.uint32)), (name, k)
    if master:
        # replay: every rank rebuilds its own bf16 params from its master
        Pr = torch.zeros_like(P)
        for T, gidx, st, h in ranks:
            Pa = Pr if layout == bfo.LAYOUT_PER_TENSOR else Pr[T.begin:T.end]
            bfo.master_to_bf16_sr(T, st["M"], Pa, step_seed(3))
        assert np.array_equal(u16(Pr), u16(P))


def test_update_per_tensor_gpt2_124m(bfo):
    w = W.gpt2_124m()
    ents = w.entries()
    tbl = o.table(ents)
    world, r = 4, 1
    T = bfo.Table(ents, world, r, layout=bfo.LAYOUT_PER_TENSOR)
    gidx = _oracle_gidx(bfo, tbl, w, world, r, bfo.LAYOUT_PER_TENSOR)
    assert np.array_equal(T.global_index(), gidx)
    P, M0, _, _ = W.init_state(torch, w, 0, w.n, DEV)
    gi = torch.from_numpy(gidx.astype(np.int64)).to(DEV)
    st = {"M": M0[gi].clone(), "m": torch.zeros(T.size, device=DEV), "v": torch.zeros(T.size, device=DEV)}
    del M0
    h = {"M": f32(st["M"]), "m": np.zeros(T.size, np.float32), "v": np.zeros(T.size, np.float32)}
    Ph = u16(P)
    G = torch.empty(w.n, dtype=torch.bfloat16, device=DEV)
    res = bfo.new_norm_result(DEV)
    for t in (1, 2):
        W.fill_grads(torch, w, G, 0, t)
        Gh = u16(G)
        bfo.grad_global_norm(T, G, res)
        got = bfo.read_norm_result(res)
        assert_norm_parity(got, o.grad_norm(np.ascontiguousarray(Gh[gidx])))
        bfo.adamw_sr_step(T, P, G, st["M"], st["m"], st["v"], w.hparams, t, step_seed(t), scale=res)
        o.adamw_step_mapped(tbl, gidx, Ph, Gh, h["M"], h["m"], h["v"], oracle_hparams(w.hparams), got[2], t,
                            step_seed(t))
        assert_bf16_parity(u16(P), Ph, "per-tensor 124M params")
        for k in ("M", "m", "v"):
            assert_f32_parity(f32(st[k]), h[k], f"per-tensor 124M {k}")


# --------------------------------------------------------------------- step control


def test_outlier_detector_matches_oracle(bfo):
    rs = np.random.default_rng(21)
    window, thr = 32, 3.0
    xs = list(rs.normal(8.0, 0.5, 160).astype(np.float32))
    xs[70] = np.float32(80.0)
    xs[90] = np.float32(np.inf)
    xs[91] = np.float32(np.nan)
    xs[120] = np.float32(8.0 + 2.9 * 0.5)
    dev = bfo.Outlier(window, thr, device=DEV)
    ref = o.Outlier(window, thr)
    val = torch.zeros(1, dtype=torch.float32, device=DEV)
    for k, x in enumerate(xs):
        val.fill_(float(x))
        dev.update(val)
        z, skip = float(dev.z.item()), int(dev.skip.item())
        rz, rskip = ref.update(float(x))
        assert skip == rskip, (k, z, rz)
        assert (math.isnan(z) and math.isnan(rz)) or np.float32(z).view(np.uint32) == np.float32(rz).view(np.uint32), \
            (k, z, rz)
    dev.reset()
    val.fill_(100.0)
    dev.update(val)
    assert math.isnan(dev.z.item()) and dev.skip.item() == 0


@pytest.mark.parametrize("master", [True, False])
def test_skip_flag_freezes_the_step(bfo, master):
    w = ragged_workload(3, 5)
    T = bfo.Table(w.entries())
    st = device_state(w, 0, w.n, DEV, master=master)
    W.fill_grads(torch, w, st["G"], 0, 1)
    before = host_copy(st)
    skip = torch.ones(1, dtype=torch.int32, device=DEV)
    bfo.adamw_sr_step(T, st["P"], st["G"], st["M"], st["m"], st["v"], w.hparams, 1, step_seed(1), skip=skip)
    after = host_copy(st)
    for k in ("P", "M", "m", "v"):
        if before[k] is not None:
            assert np.array_equal(before[k].view(np.uint8), after[k].view(np.uint8)), k
    skip.zero_()
    bfo.adamw_sr_step(T, st["P"], st["G"], st["M"], st["m"], st["v"], w.hparams, 1, step_seed(1), skip=skip)
    oracle_step(o.table(w.entries()), 0, before, w.hparams, 1.0, 1, step_seed(1))
    assert_state_parity(host_copy(st), before, "skip=0")


def test_step_control_pipeline_skips_the_spike(bfo):
    # norm -> detector(norm) -> update(skip) with no host round trip; a
    # gradient spike at one step must be skipped, the others applied, and the
    # trajectory must match the oracle driven by the same decisions.
    w = ragged_workload(6, 3)
    w.grad_std = 1e-3
    ents = w.entries()
    T = bfo.Table(ents)
    tbl = o.table(ents)
    st = device_state(w, 0, w.n, DEV)
    h = host_copy(st)
    res = bfo.new_norm_result(DEV)
    det = bfo.Outlier(16, 5.0, device=DEV)
    ref = o.Outlier(16, 5.0)
    skipped = []
    for t in range(1, 41):
        lr = bfo.lr_at(bfo.LR_COSINE, t - 1, 5, 40, 1e-3, 0.1)
        hp = W.HParams(lr=lr)
        W.fill_grads(torch, w, st["G"], 0, t)
        if t == 30:
            st["G"].mul_(1000.0)
        bfo.grad_global_norm(T, st["G"], res)
        det.update(bfo.norm_ptr(res))
        bfo.adamw_sr_step(T, st["P"], st["G"], st["M"], st["m"], st["v"], hp, t, step_seed(t), scale=res,
                          skip=det.skip)
        _, norm, scale = bfo.read_norm_result(res)
        _, rskip = ref.update(norm)
        assert int(det.skip.item()) == rskip, t
        if rskip:
            skipped.append(t)
            continue
        h["G"] = u16(st["G"])
        oracle_step(tbl, 0, h, hp, scale, t, step_seed(t))
    assert skipped == [30]
    assert_state_parity(host_copy(st), h, "step control")


# --------------------------------------------------------------------- checkpoint / resume


def _same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


class _Run:
    """A GPU run of the ragged workload beside the oracle's own run of it:
    both start from the same state and take the same grads; the oracle is
    fed the GPU's clip scale (norms compared separately)."""

    def __init__(self, bfo, master=True, rounding=o.ROUND_SR):
        self.bfo = bfo
        self.w = ragged_workload(6, 3)
        self.w.grad_std = 0.05
        self.T = bfo.Table(self.w.entries())
        self.tbl = o.table(self.w.entries())
        self.st = device_state(self.w, 0, self.w.n, DEV, master=master)
        self.h = host_copy(self.st)
        self.res = bfo.new_norm_result(DEV)
        self.rounding = rounding

    def gpu_step(self, state, t, skip=None, rounding=None):
        rounding = self.rounding if rounding is None else rounding
        W.fill_grads(torch, self.w, state["G"], 0, t)
        self.bfo.grad_global_norm(self.T, state["G"], self.res)
        self.bfo.adamw_sr_step(self.T, state["P"], state["G"], state.get("M"), state["m"], state["v"],
                               self.w.hparams, t, step_seed(t), scale=self.res, rounding=rounding, skip=skip)
        got = self.bfo.read_norm_result(self.res)
        return got[2]

    def both_step(self, t):
        scale = self.gpu_step(self.st, t)
        self.h["G"] = u16(self.st["G"])
        assert_norm_parity(self.bfo.read_norm_result(self.res), o.grad_norm(self.h["G"], 1.0))
        oracle_step(self.tbl, 0, self.h, self.w.hparams, scale, t, step_seed(t), self.rounding)
        return scale

    def fresh(self, master=True):
        return {"P": torch.empty_like(self.st["P"]),
                "M": torch.empty(self.w.n, dtype=torch.float32, device=DEV) if master else None,
                "m": torch.empty_like(self.st["m"]), "v": torch.empty_like(self.st["v"]),
                "G": torch.empty_like(self.st["G"])}


def test_checkpoint_resume_matches_the_oracle(bfo, tmp_path):
    # "04 · 多 GPU 与混合精度" §5.1-5.2: save (master, m, v, last seed) at
    # step 4 -- not the bf16 weights --, resume in fresh buffers (the load
    # rebuilds the params from the master with the saved draws), run to step
    # 8.  The oracle runs steps 1-8 from the same start: the rebuilt params
    # equal its step-4 params and the resumed run its step-8 state, bit for
    # bit, as does the run that never stopped.
    run = _Run(bfo)
    d = str(tmp_path)
    scales = {}
    for t in range(1, 9):
        scales[t] = run.both_step(t)
        if t == 4:
            bfo.checkpoint_save(d, run.T, run.st["m"], run.st["v"], 4, step_seed(4), master=run.st["M"])
            assert bfo.checkpoint_latest(d) is None            # not done until marked
            bfo.checkpoint_done(d, 4)
            at4 = {k: (None if a is None else a.copy()) for k, a in run.h.items()}
    uninterrupted = host_copy(run.st)
    for k in ("P", "M", "m", "v"):
        assert _same_bits(uninterrupted[k], run.h[k]), f"uninterrupted run vs oracle: {k}"

    fresh = run.fresh()
    last = bfo.checkpoint_latest(d)
    assert last == 4
    assert bfo.checkpoint_load(d, last, run.T, fresh["m"], fresh["v"], master=fresh["M"],
                               params=fresh["P"]) == step_seed(4)
    got = host_copy(fresh)
    for k in ("P", "M", "m", "v"):
        assert _same_bits(got[k], at4[k]), f"loaded step-4 {k} vs oracle"
    for t in range(5, 9):
        assert run.gpu_step(fresh, t) == scales[t]
    got = host_copy(fresh)
    for k in ("P", "M", "m", "v"):
        assert _same_bits(got[k], run.h[k]), f"resumed step-8 {k} vs oracle"


@pytest.mark.parametrize("stored_params", [False, True])
def test_checkpoint_resumes_a_run_without_master(bfo, tmp_path, stored_params):
    # "04 · 多 GPU 与混合精度" §5.2: only the fp32 master is needed, so the
    # same state can resume under another precision setup.  A master run
    # saves at step 4; a run without a master loads it (params rebuilt by SR
    # with the saved seed, the master staged in v's buffer -- or the stored
    # params taken as they are) and goes on with the no-master update.  The
    # oracle does the same from its own step-4 state.
    run = _Run(bfo)
    d = str(tmp_path)
    for t in range(1, 5):
        run.both_step(t)
    bfo.checkpoint_save(d, run.T, run.st["m"], run.st["v"], 4, step_seed(4), master=run.st["M"],
                        params=run.st["P"] if stored_params else None)
    bfo.checkpoint_done(d, 4)
    fresh = run.fresh(master=False)
    fresh["P"].view(torch.int16).fill_(0x7FA5)
    fresh["v"].fill_(float("nan"))
    assert bfo.checkpoint_load(d, 4, run.T, fresh["m"], fresh["v"], params=fresh["P"]) == step_seed(4)
    got = host_copy(fresh)
    for k in ("P", "m", "v"):
        assert _same_bits(got[k], run.h[k]), f"step-4 {k} vs oracle"
    oracle_h = {k: (None if k == "M" else a) for k, a in run.h.items()}
    for t in range(5, 9):
        scale = run.gpu_step(fresh, t)
        oracle_h["G"] = u16(fresh["G"])
        oracle_step(run.tbl, 0, oracle_h, run.w.hparams, scale, t, step_seed(t), o.ROUND_SR)
    got = host_copy(fresh)
    for k in ("P", "m", "v"):
        assert _same_bits(got[k], oracle_h[k]), f"no-master step-8 {k} vs oracle"


def test_checkpoint_round_to_nearest_master_run(bfo, tmp_path):
    # A master run that writes its bf16 weights by round-to-nearest: the
    # header keeps the mode, and the load rebuilds the params as RNE(master),
    # the oracle's step-3 params; master_to_bf16 with RNE does the same, and
    # an SR rebuild of the same master would not.
    run = _Run(bfo, rounding=o.ROUND_RNE)
    d = str(tmp_path)
    for t in range(1, 4):
        run.both_step(t)
    bfo.checkpoint_save(d, run.T, run.st["m"], run.st["v"], 3, step_seed(3), master=run.st["M"],
                        rounding=bfo.ROUND_RNE)
    fresh = run.fresh()
    bfo.checkpoint_load(d, 3, run.T, fresh["m"], fresh["v"], master=fresh["M"], params=fresh["P"])
    assert _same_bits(u16(fresh["P"]), run.h["P"])
    assert _same_bits(o.round_nearest_even(run.h["M"]), run.h["P"])
    P2 = torch.empty_like(fresh["P"])
    bfo.master_to_bf16(run.T, fresh["M"], P2, 0, bfo.ROUND_RNE)
    assert _same_bits(u16(P2), run.h["P"])
    bfo.master_to_bf16(run.T, fresh["M"], P2, step_seed(3), bfo.ROUND_SR)
    assert not _same_bits(u16(P2), run.h["P"])
    with pytest.raises(bfo.BfoError) as e:
        bfo.master_to_bf16(run.T, fresh["M"], P2, 0, 7)
    assert e.value.status == bfo.EINVAL


def test_checkpoint_after_a_skipped_update_keeps_the_stored_params(bfo, tmp_path):
    # A step whose update a device flag skipped leaves the step-3 state, but
    # the caller, which does not wait for the flag, saves "step 4, seed 4".
    # With the params stored, the load restores them as they are (the
    # oracle's step-3 params); a rebuild with seed 4 would not give them.
    run = _Run(bfo)
    d = str(tmp_path)
    for t in range(1, 4):
        run.both_step(t)
    skip = torch.ones(1, dtype=torch.int32, device=DEV)
    run.gpu_step(run.st, 4, skip=skip)
    assert _same_bits(u16(run.st["P"]), run.h["P"]) and _same_bits(f32(run.st["M"]), run.h["M"])
    bfo.checkpoint_save(d, run.T, run.st["m"], run.st["v"], 4, step_seed(4), master=run.st["M"],
                        params=run.st["P"])
    fresh = run.fresh()
    bfo.checkpoint_load(d, 4, run.T, fresh["m"], fresh["v"], master=fresh["M"], params=fresh["P"])
    got = host_copy(fresh)
    for k in ("P", "M", "m", "v"):
        assert _same_bits(got[k], run.h[k]), k
    rebuilt = o.master_to_bf16_sr(run.h["M"], 0, step_seed(4))
    assert not _same_bits(rebuilt, run.h["P"])


def test_checkpoint_refuses_a_corrupted_file(bfo, tmp_path):
    # One flipped byte anywhere in the payload, or in the header, is refused
    # (BFO_EFORMAT) by the per-array and header checksums; the intact file
    # loads.
    run = _Run(bfo)
    for t in (1, 2):
        run.both_step(t)
    d = str(tmp_path)
    bfo.checkpoint_save(d, run.T, run.st["m"], run.st["v"], 2, step_seed(2), master=run.st["M"],
                        params=run.st["P"])
    path = tmp_path / "state_00000002_00000.bin"
    data = bytearray(path.read_bytes())
    n = run.w.n
    header = 128
    assert len(data) == header + (4 + 2 + 4 + 4) * n
    offsets = {"header (seed)": 24, "master": header + 4 * 17 + 1, "params": header + 4 * n + 2 * 5,
               "m": header + 6 * n + 4 * (n - 1) + 3, "v": header + 10 * n + 4 * (n // 2)}
    fresh = run.fresh()
    for what, pos in offsets.items():
        data[pos] ^= 0x10
        path.write_bytes(bytes(data))
        with pytest.raises(bfo.BfoError) as e:
            bfo.checkpoint_load(d, 2, run.T, fresh["m"], fresh["v"], master=fresh["M"], params=fresh["P"])
        assert e.value.status == bfo.EFORMAT, what
        data[pos] ^= 0x10
    path.write_bytes(bytes(data))
    bfo.checkpoint_load(d, 2, run.T, fresh["m"], fresh["v"], master=fresh["M"], params=fresh["P"])
    got = host_copy(fresh)
    for k in ("P", "M", "m", "v"):
        assert _same_bits(got[k], run.h[k]), k


def test_checkpoint_no_master_per_tensor_round_trip_and_errors(bfo, tmp_path):
    w = W.tiny()
    ents = w.entries()
    world, r = 4, 2
    T = bfo.Table(ents, world, r, layout=bfo.LAYOUT_PER_TENSOR)
    P, _, _, _ = W.init_state(torch, w, 0, w.n, DEV, master=False)
    m = torch.randn(T.size, device=DEV)
    v = torch.rand(T.size, device=DEV)
    d = str(tmp_path)
    bfo.checkpoint_save(d, T, m, v, 7, 99, params=P)
    P2 = torch.zeros_like(P)
    m2, v2 = torch.empty_like(m), torch.empty_like(v)
    assert bfo.checkpoint_load(d, 7, T, m2, v2, params=P2) == 99
    gi = torch.from_numpy(T.global_index().astype(np.int64)).to(DEV)
    assert torch.equal(P2[gi].view(torch.int16), P[gi].view(torch.int16))
    mask = torch.ones(w.n, dtype=torch.bool, device=DEV)
    mask[gi] = False
    assert not bool(P2.view(torch.int16)[mask].any())    # only this rank's elements were written
    assert torch.equal(m2, m) and torch.equal(v2, v)
    # refusals: another rank's table, a master where none was saved, a missing step, a truncated file
    with pytest.raises(bfo.BfoError) as e:
        bfo.checkpoint_load(d, 7, bfo.Table(ents, world, r, layout=bfo.LAYOUT_FLAT), m2, v2, params=P2[:T.size])
    assert e.value.status == bfo.EFORMAT
    with pytest.raises(bfo.BfoError) as e:
        bfo.checkpoint_load(d, 7, T, m2, v2, master=torch.empty_like(m))
    assert e.value.status == bfo.EFORMAT
    with pytest.raises(bfo.BfoError) as e:
        bfo.checkpoint_load(d, 8, T, m2, v2, params=P2)
    assert e.value.status == bfo.ENOTFOUND
    path = tmp_path / "state_00000007_00002.bin"
    data = path.read_bytes()
    path.write_bytes(data[:-4])
    with pytest.raises(bfo.BfoError) as e:
        bfo.checkpoint_load(d, 7, T, m2, v2, params=P2)
    assert e.value.status == bfo.EFORMAT
