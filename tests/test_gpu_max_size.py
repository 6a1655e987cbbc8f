"""GPU parity at sizes past one launch.

The library splits a grid longer than 2^22 workgroups into several launches
(a launch's lane count has to stay below 2^32), each starting at its own
tile offset.  Every shard of the models up to Llama-7B fits in one launch, so
these cases size the input just past that split, with tensor boundaries and
a ragged end around it, at the largest sizes one GPU's memory takes:

  - grad norm over 3.4e10 elements (69 GB of grads; both stage-1 kernels):
    a pattern whose sum of squares is an exact binary64 value, so the result
    must equal the closed form bit for bit;
  - the no-master update over 1.7e10 elements (206 GB of state) and the
    master-to-bf16 rebuild over the same length: sampled windows against the
    oracle, around the split, the tensor boundaries, the ends;
  - the draw dump (2^30 + 777 draws) and the decay-mask dump (8.6e9
    elements) against the oracle around their own splits.
"""
import math

import numpy as np
import pytest
import torch

import oracle as o
from bf16_numerics_amd import workloads as W
from gpu_harness import assert_norm_parity, assert_state_parity, f32, host_copy, oracle_step, step_seed, u16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SPLIT = 1 << 22              # workgroups per launch before the library splits a grid
UPDATE_TILE = 4096           # elements per update / rebuild workgroup
NORM_TILE = 8192             # elements per grad-norm stage-1 workgroup
CHUNK = 1 << 28              # elements per fill step (bounds the fill's temporaries)


@pytest.fixture(scope="module")
def bfo():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from bf16_numerics_amd import binding
    torch.cuda.set_device(0)
    return binding


@pytest.fixture(autouse=True)
def _free_memory():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def need_bytes(nbytes):
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < nbytes + (8 << 30):
        pytest.skip(f"needs {nbytes / 1e9:.0f} GB of free device memory, {free / 1e9:.0f} GB free")


def fill(dst, make, seed):
    """dst[c0:c1] = make(generator, c0, c1) chunk by chunk, one seeded
    generator per chunk."""
    for k, c0 in enumerate(range(0, dst.numel(), CHUNK)):
        c1 = min(dst.numel(), c0 + CHUNK)
        gen = torch.Generator(device=DEV).manual_seed(seed * 1_000_003 + k)
        dst[c0:c1] = make(gen, c0, c1)


def sample_windows(points, S, half=64, n_random=16, seed=0):
    rs = np.random.default_rng(seed)
    rng = [(max(0, p - half), min(S, p + half)) for p in points]
    rng += [(int(x), int(x) + 64) for x in rs.integers(0, S - 64, n_random)]
    rng.sort()
    merged = []
    for lo, hi in rng:
        if merged and lo <= merged[-1][1]:
            merged[-1] = (merged[-1][0], max(merged[-1][1], hi))
        elif hi > lo:
            merged.append((lo, hi))
    return merged


# --------------------------------------------------------------------- norm


def norm_pattern_sumsq(S):
    """Sum of squares of g[j] = (1 + (j >> 13) mod 7) * 2^-10 over [0, S),
    as an exact binary64 value (an integer count of 2^-20 below 2^53)."""
    full, rem = S // NORM_TILE, S % NORM_TILE
    total = 0
    for r in range(7):
        tiles = full // 7 + (1 if r < full % 7 else 0)
        total += tiles * NORM_TILE * (r + 1) ** 2
    total += rem * (full % 7 + 1) ** 2
    assert total < 2 ** 53
    return float(total) * 2.0 ** -20


def test_norm_past_one_launch_is_exact(bfo):
    S = SPLIT * NORM_TILE + 3 * NORM_TILE + 5          # one full launch, then four tiles, the last ragged
    need_bytes(2 * S)
    G = torch.empty(S, dtype=torch.bfloat16, device=DEV)
    fill(G, lambda gen, c0, c1: (((torch.arange(c0, c1, device=DEV) >> 13) % 7 + 1).float() * 2.0 ** -10)
         .to(torch.bfloat16), 0)
    sumsq = norm_pattern_sumsq(S)
    norm = np.float32(math.sqrt(sumsq))
    ref = (sumsq, float(norm), float(np.float32(1.0) / norm))
    res = bfo.new_norm_result(DEV)
    for layout in (bfo.LAYOUT_FLAT, bfo.LAYOUT_PER_TENSOR):
        T = bfo.Table([(0, S, 1)], layout=layout)
        res.zero_()
        bfo.grad_global_norm(T, G, res, 1.0)
        got = bfo.read_norm_result(res)
        print(f"norm S={S} layout={layout}: sumsq {got[0]!r} (closed form {sumsq!r})", flush=True)
        assert got[0] == sumsq, (layout, got[0], sumsq)
        assert_norm_parity(got, ref)
        T.close()


# --------------------------------------------------------------------- update and rebuild


def split_table():
    """Three tensors (decay, no decay, decay) whose boundaries sit 5 elements
    either side of the first element of the second launch, and a ragged
    end one tile and 24 elements later."""
    first = SPLIT * UPDATE_TILE
    S = first + UPDATE_TILE + 24
    entries = [(0, first - 5, 1), (first - 5, 10, 0), (first + 5, S - first - 5, 1)]
    return S, first, entries


def test_update_no_master_past_one_launch(bfo):
    S, first, entries = split_table()
    need_bytes(12 * S)
    hp = W.tiny().hparams
    T = bfo.Table(entries)
    P = torch.empty(S, dtype=torch.bfloat16, device=DEV)
    G = torch.empty(S, dtype=torch.bfloat16, device=DEV)
    m = torch.empty(S, dtype=torch.float32, device=DEV)
    v = torch.empty(S, dtype=torch.float32, device=DEV)
    fill(P, lambda gen, c0, c1: (torch.randn(c1 - c0, generator=gen, device=DEV) * 0.02).to(torch.bfloat16), 1)
    fill(G, lambda gen, c0, c1: (torch.randn(c1 - c0, generator=gen, device=DEV) * 1e-3).to(torch.bfloat16), 2)
    fill(m, lambda gen, c0, c1: torch.randn(c1 - c0, generator=gen, device=DEV) * 1e-4, 3)
    fill(v, lambda gen, c0, c1: torch.rand(c1 - c0, generator=gen, device=DEV) * 1e-8, 4)
    st = {"P": P, "M": None, "m": m, "v": v, "G": G}
    wins = sample_windows([0, first - 5, first, first + 5, S - 24, S], S)
    pre = [host_copy(st, lo, hi) for lo, hi in wins]
    res = bfo.new_norm_result(DEV)
    t = 3
    bfo.grad_global_norm(T, G, res, hp.max_norm)
    bfo.adamw_sr_step(T, P, G, None, m, v, hp, t, step_seed(t), scale=res)
    scale = bfo.read_norm_result(res)[2]
    tbl = o.table(entries)
    for (lo, hi), h in zip(wins, pre):
        oracle_step(tbl, lo, h, hp, scale, t, step_seed(t))
        assert_state_parity(host_copy(st, lo, hi), h, f"S={S} [{lo},{hi})")
    print(f"no-master update S={S}: {len(wins)} windows equal the oracle (scale {scale:.6f})", flush=True)
    T.close()


def test_rebuild_past_one_launch(bfo):
    S, first, entries = split_table()
    need_bytes(6 * S)
    T = bfo.Table(entries)
    M = torch.empty(S, dtype=torch.float32, device=DEV)
    fill(M, lambda gen, c0, c1: torch.randn(c1 - c0, generator=gen, device=DEV) * 0.02, 5)
    P = torch.zeros(S, dtype=torch.bfloat16, device=DEV)
    seed = step_seed(7)
    bfo.master_to_bf16_sr(T, M, P, seed)
    wins = sample_windows([0, first - 5, first, first + 5, S - 24, S], S, seed=1)
    for lo, hi in wins:
        ref = o.master_to_bf16_sr(f32(M[lo:hi]), lo, seed)
        assert np.array_equal(u16(P[lo:hi]), ref), (lo, hi)
    T.close()


# --------------------------------------------------------------------- test exports


def test_rng_dump_past_one_launch(bfo):
    count = SPLIT * 256 + 777                     # 256 draws per workgroup
    first, seed = (1 << 36) + 5, 0x0123456789ABCDEF
    out = bfo.rng_dump(first, count, seed, DEV)
    for lo, hi in ((0, 512), (SPLIT * 256 - 512, SPLIT * 256 + 512), (count - 512, count)):
        got = out[lo:hi].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, o.rng16(first + lo, hi - lo, seed)), (lo, hi)


def test_decay_mask_dump_past_one_launch(bfo):
    first = SPLIT * 256 * 8                       # 256 vectors of 8 elements per workgroup
    S = first + 4096 + 3
    entries = [(0, first - 1, 1), (first - 1, 2, 0), (first + 1, S - first - 1, 1)]
    need_bytes(S)
    T = bfo.Table(entries)
    dm = bfo.decay_mask_dump(T)
    tbl = o.table(entries)
    for lo, hi in sample_windows([0, first - 1, first, first + 1, S], S, seed=2):
        assert np.array_equal(dm[lo:hi].cpu().numpy(), o.decay_mask(tbl, lo, hi - lo)), (lo, hi)
    T.close()
