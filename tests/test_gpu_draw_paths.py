"""GPU parity of the update's two ways of drawing the rounding noise.

A lane of the update owns four 4-element quads.  Without a master, when a
whole wave's quads sit in runs at global indices 0 / 4 mod 8 (even / odd
lane), lanes 2i and 2i+1 each compute two of their four shared Philox blocks
and swap halves; any other wave computes every quad's block itself.  These
shards put both kinds of wave, and the seams between them, into one launch:

  - a flat shard starting at global index 0 mod 8 whose last wave is cut by
    the shard end (paired waves, then a fallback wave);
  - flat shards starting 4 mod 8 and 2 mod 8 (no wave can pair; quads that
    straddle two Philox blocks);
  - a per-tensor shard whose runs change mid-wave (tiles that cross runs).

Each runs two steps (norm, then SR update) with and without a master,
against the oracle on every element (draws are exact, so params must be
equal)."""
import numpy as np
import pytest
import torch

import oracle as o
from gpu_harness import (assert_bf16_parity, assert_f32_parity, assert_norm_parity, f32, oracle_hparams,
                         step_seed, u16)
from bf16_numerics_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (name, tensor sizes, world, rank, layout, shard begin mod 8 for flat
# shards); flags alternate decay / no decay
CASES = [
    ("flat, begins 0 mod 8, ragged end", [12288, 3000, 9001, 5], 1, 0, 0, 0),
    ("flat, begins 4 mod 8", [20000, 20008], 2, 1, 0, 4),
    ("flat, begins 2 mod 8", [20002, 20002], 2, 1, 0, 2),
    ("per-tensor, runs change mid-wave", [4100, 1030, 8192, 60, 2050, 6006], 2, 1, 1, None),
]


@pytest.fixture(scope="module")
def bfo():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from bf16_numerics_amd import binding
    torch.cuda.set_device(0)
    return binding


@pytest.mark.parametrize("master", [False, True])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_draw_paths_match_the_oracle(bfo, case, master):
    name, sizes, world, rank, layout, begin_mod8 = case
    print(f"draw paths: {name}, master={master}", flush=True)
    entries, off = [], 0
    for i, s in enumerate(sizes):
        entries.append((off, s, i % 2))
        off += s
    n = off
    tbl = o.table(entries)
    hp = W.tiny().hparams
    T = bfo.Table(entries, world, rank, layout=layout)
    S = T.size
    if layout == bfo.LAYOUT_PER_TENSOR:
        rc, gidx = o.shard_map_per_tensor(tbl, world, rank)
    else:
        rc, b, e = o.shard_range(n, world, rank)
        gidx = np.arange(b, e, dtype=np.uint64)
    assert rc == o.OK and S == gidx.size
    gi = gidx.astype(np.int64)
    if begin_mod8 is not None:
        assert int(gidx[0]) % 8 == begin_mod8

    rs = np.random.default_rng(4242 + len(name))
    P_all = (rs.normal(0, 0.02, n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    M = (P_all[gi].astype(np.uint32) << 16).view(np.float32).copy() if master else None
    m = rs.normal(0, 1e-4, S).astype(np.float32)
    v = (rs.random(S) * 1e-7).astype(np.float32)
    pg_src = P_all if layout == bfo.LAYOUT_PER_TENSOR else P_all[gi]
    dP = W.from_bf16_bits(torch, pg_src, DEV)
    dG = torch.empty_like(dP)
    dM = torch.from_numpy(M).to(DEV) if master else None
    dm, dv = torch.from_numpy(m).to(DEV), torch.from_numpy(v).to(DEV)
    res = bfo.new_norm_result(DEV)
    h = {"P": P_all.copy(), "M": None if M is None else M.copy(), "m": m.copy(), "v": v.copy()}
    for t in (1, 2):
        G_all = (rs.normal(0, 1e-2, n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        dG.copy_(W.from_bf16_bits(torch, G_all if layout == bfo.LAYOUT_PER_TENSOR else G_all[gi], DEV))
        bfo.grad_global_norm(T, dG, res, hp.max_norm)
        bfo.adamw_sr_step(T, dP, dG, dM, dm, dv, hp, t, step_seed(t), scale=res)
        got = bfo.read_norm_result(res)
        assert_norm_parity(got, o.grad_norm(np.ascontiguousarray(G_all[gi]), hp.max_norm))
        o.adamw_step_mapped(tbl, gidx, h["P"], G_all, h["M"], h["m"], h["v"], oracle_hparams(hp), got[2], t,
                            step_seed(t))
    ref = h["P"] if layout == bfo.LAYOUT_PER_TENSOR else h["P"][gi]
    assert_bf16_parity(u16(dP), ref, f"{name} params")
    if master:
        assert_f32_parity(f32(dM), h["M"], f"{name} master")
    assert_f32_parity(f32(dm), h["m"], f"{name} m")
    assert_f32_parity(f32(dv), h["v"], f"{name} v")
