"""Randomised GPU parity: many small seeded cases against the oracle.

Each case draws a tensor table (tensors of 0-5,000 elements, random decay
flags), a shard count and rank, a layout, master or no master, a rounding
mode, and an element offset of 0-7 for the params and grads arrays (so their
start is 2-byte aligned only, or any 16-byte phase), then runs the grad norm
and two update steps on the GPU (odd cases through the one-call step) and the
oracle on the same inputs; with a master, the rebuild must give the last
step's params back.  Bars as
in the other parity tests: draws, maps and masks exact; bf16 params equal or
one step apart in at most 1e-6 of the elements (none at these sizes); fp32
state within relative 1e-6; norm within relative 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle as o
from gpu_harness import (assert_bf16_parity, assert_f32_parity, assert_norm_parity, f32, oracle_hparams,
                         step_seed, u16)
from bf16_numerics_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CASES = 256


@pytest.fixture(scope="module")
def bfo():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from bf16_numerics_amd import binding
    torch.cuda.set_device(0)
    return binding


def draw_case(k):
    rs = np.random.default_rng(9000 + k)
    world = int(rs.integers(1, 9))
    layout = int(rs.integers(0, 2))
    sizes = [int(x) for x in rs.integers(0, 5000, int(rs.integers(1, 16)))]
    if layout == 1:
        sizes = [s - s % world for s in sizes]
    entries, off = [], 0
    for s in sizes:
        entries.append((off, s, int(rs.integers(0, 2))))
        off += s
    pad = (-off) % world
    if pad:
        entries.append((off, pad, 0))
        off += pad
    return {"entries": entries, "n": off, "world": world, "rank": int(rs.integers(0, world)),
            "layout": layout, "master": bool(rs.integers(0, 2)), "rounding": int(rs.integers(0, 2)),
            "shift": int(rs.integers(0, 8)), "grad_std": float(10 ** rs.uniform(-4, -1)), "seed": 9000 + k}


@pytest.mark.parametrize("k", range(CASES))
def test_random_case_matches_the_oracle(bfo, k):
    c = draw_case(k)
    print(f"case {k}: n={c['n']} world={c['world']} rank={c['rank']} layout={c['layout']} "
          f"master={c['master']} rounding={c['rounding']} shift={c['shift']}", flush=True)
    entries, n, world, rank = c["entries"], c["n"], c["world"], c["rank"]
    tbl = o.table(entries)
    hp = W.tiny().hparams
    rs = np.random.default_rng(c["seed"])
    T = bfo.Table(entries, world, rank, layout=c["layout"])
    S = T.size
    if c["layout"] == bfo.LAYOUT_PER_TENSOR:
        rc, gidx = o.shard_map_per_tensor(tbl, world, rank)
        pg_len = n
    else:
        rc, b, e = o.shard_range(n, world, rank)
        gidx = np.arange(b, e, dtype=np.uint64)
        pg_len = S
    assert rc == o.OK and S == gidx.size
    assert np.array_equal(T.global_index(), gidx)

    # host inputs: params of the whole buffer, the shard's fp32 state
    P_all = (rs.normal(0, 0.02, n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    M = P_all[gidx.astype(np.int64)].astype(np.uint32) << 16
    M = M.view(np.float32).copy() if c["master"] else None
    m = rs.normal(0, 1e-4, S).astype(np.float32)
    v = (rs.random(S) * 1e-7).astype(np.float32)
    sh = c["shift"]
    # device buffers with the params/grads arrays starting `shift` elements in
    buf_P = torch.zeros(pg_len + 8, dtype=torch.bfloat16, device=DEV)
    buf_G = torch.zeros(pg_len + 8, dtype=torch.bfloat16, device=DEV)
    dP, dG = buf_P[sh:sh + pg_len], buf_G[sh:sh + pg_len]
    pg_src = P_all if c["layout"] == bfo.LAYOUT_PER_TENSOR else P_all[gidx.astype(np.int64)]
    dP.copy_(W.from_bf16_bits(torch, pg_src, DEV))
    dM = torch.from_numpy(M).to(DEV) if M is not None else None
    dm, dv = torch.from_numpy(m).to(DEV), torch.from_numpy(v).to(DEV)
    res = bfo.new_norm_result(DEV)
    h = {"P": P_all.copy(), "M": None if M is None else M.copy(), "m": m.copy(), "v": v.copy()}
    for t in (1, 2):
        G_all = (rs.normal(0, c["grad_std"], n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        g_src = G_all if c["layout"] == bfo.LAYOUT_PER_TENSOR else G_all[gidx.astype(np.int64)]
        dG.copy_(W.from_bf16_bits(torch, g_src, DEV))
        if k % 2:       # odd cases take the one-call step (one launch when S <= 65,536)
            bfo.adamw_sr_step_with_norm(T, dP, dG, dM, dm, dv, hp, t, step_seed(t), res, hp.max_norm,
                                        rounding=c["rounding"], workspace=bfo.new_norm_workspace(T))
        else:
            bfo.grad_global_norm(T, dG, res, hp.max_norm)
            bfo.adamw_sr_step(T, dP, dG, dM, dm, dv, hp, t, step_seed(t), scale=res, rounding=c["rounding"])
        got = bfo.read_norm_result(res)
        assert_norm_parity(got, o.grad_norm(np.ascontiguousarray(G_all[gidx.astype(np.int64)]), hp.max_norm))
        o.adamw_step_mapped(tbl, gidx, h["P"], G_all, h["M"], h["m"], h["v"], oracle_hparams(hp), got[2], t,
                            step_seed(t), c["rounding"])
    gp = u16(dP)
    ref = h["P"] if c["layout"] == bfo.LAYOUT_PER_TENSOR else h["P"][gidx.astype(np.int64)]
    assert_bf16_parity(gp, ref, f"case {k} params")
    assert np.array_equal(u16(buf_P[:sh]), np.zeros(sh, np.uint16)), "write before the params array"
    assert np.array_equal(u16(buf_P[sh + pg_len:]), np.zeros(8 - sh, np.uint16)), "write past the params array"
    if M is not None:
        assert_f32_parity(f32(dM), h["M"], f"case {k} master")
        # the rebuild from the master, in the step's rounding mode, gives the step's params back
        P2 = dP.clone()
        if c["layout"] == bfo.LAYOUT_PER_TENSOR:
            P2.view(torch.int16)[torch.from_numpy(gidx.astype(np.int64)).to(DEV)] = 0x7FA5
        else:
            P2.view(torch.int16).fill_(0x7FA5)
        bfo.master_to_bf16(T, dM, P2, step_seed(2), c["rounding"])
        assert np.array_equal(u16(P2), gp), f"case {k} rebuild"
    assert_f32_parity(f32(dm), h["m"], f"case {k} m")
    assert_f32_parity(f32(dv), h["v"], f"case {k} v")
