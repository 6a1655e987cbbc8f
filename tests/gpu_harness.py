"""Shared helpers of the GPU parity tests: seeded state on the device, host
copies for the oracle, and the comparison bars.

Bars (floating point decides only the fp32 values; the draws, shard offsets
and decay masks are integers and must be bit-exact):
  - bf16 params equal the oracle's, or differ by one bf16 step in at most
    1e-6 of the elements (floor of 1e-6 * n, so none for small shards);
  - fp32 master, m and v within relative 1e-6 of the oracle's;
  - grad norm within relative 1e-5.
"""
import numpy as np
import torch

import oracle as o
from bf16_numerics_amd import workloads as W

SEED = W.SEED


def step_seed(t):
    """Per-step rounding seed: base seed in the high word, step in the low."""
    return (SEED << 32) | (t & 0xFFFFFFFF)


def u16(t):
    return W.bf16_bits_numpy(torch, t).copy()


def f32(t):
    return t.detach().cpu().numpy().copy()


def dev_bf16(bits, device):
    return W.from_bf16_bits(torch, bits, device)


def dev_f32(a, device):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def oracle_hparams(hp):
    return o.hparams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.bias_correction)


def assert_bf16_parity(got, ref, what="params"):
    got = np.asarray(got, np.uint16)
    ref = np.asarray(ref, np.uint16)
    assert got.shape == ref.shape
    diff = got != ref
    nan_g = (got & 0x7FFF) > 0x7F80
    nan_r = (ref & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN positions differ"
    diff &= ~(nan_g & nan_r)
    ndiff = int(diff.sum())
    if ndiff:
        steps = np.abs(got[diff].astype(np.int32) - ref[diff].astype(np.int32))
        same_sign = (got[diff] >> 15) == (ref[diff] >> 15)
        assert np.all((steps <= 1) & same_sign), f"{what}: a difference above one bf16 step"
    allowed = int(1e-6 * got.size)
    assert ndiff <= allowed, f"{what}: {ndiff} of {got.size} differ by one step (allowed {allowed})"
    return ndiff


def assert_f32_parity(got, ref, what, rtol=1e-6):
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    assert got.shape == ref.shape
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN positions differ"
    ok = ~nan_r
    g64, r64 = got[ok].astype(np.float64), ref[ok].astype(np.float64)
    same = g64 == r64
    err = np.abs(g64 - r64)
    bad = ~same & ~(err <= rtol * np.abs(r64))
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond relative {rtol}; worst " \
                          f"{float((err / np.maximum(np.abs(r64), 1e-300))[bad].max())}"
    return int((~same).sum())


def assert_norm_parity(got, ref, rtol=1e-5):
    gs, gn, gsc = got
    rs, rn, rsc = ref
    for a, b, name in ((gs, rs, "sumsq"), (gn, rn, "norm"), (gsc, rsc, "scale")):
        if np.isnan(b):
            assert np.isnan(a), name
        elif np.isinf(b):
            assert a == b, name
        else:
            assert abs(a - b) <= rtol * abs(b), f"{name}: {a} vs {b}"


def device_state(w, begin, end, device, master=True, seed=SEED):
    P, M, m, v = W.init_state(torch, w, begin, end, device, seed=seed, master=master)
    G = torch.empty(end - begin, dtype=torch.bfloat16, device=device)
    return {"P": P, "M": M, "m": m, "v": v, "G": G}


def host_copy(st, lo=0, hi=None):
    out = {}
    for k, t in st.items():
        if t is None:
            out[k] = None
            continue
        piece = t[lo:hi]
        out[k] = u16(piece) if t.dtype == torch.bfloat16 else f32(piece)
    return out


def oracle_step(tbl, begin, h, hp, scale, t, seed, rounding=o.ROUND_SR):
    """Apply the oracle update in place to host copy h (from host_copy)."""
    o.adamw_step(tbl, begin, h["P"], h["G"], h["M"], h["m"], h["v"], oracle_hparams(hp),
                 scale, t, seed, rounding)


def assert_state_parity(gpu, ref, what=""):
    nb = assert_bf16_parity(gpu["P"], ref["P"], f"{what} params")
    nm = 0
    if ref.get("M") is not None:
        nm = assert_f32_parity(gpu["M"], ref["M"], f"{what} master")
    n1 = assert_f32_parity(gpu["m"], ref["m"], f"{what} m")
    n2 = assert_f32_parity(gpu["v"], ref["v"], f"{what} v")
    return {"P": nb, "M": nm, "m": n1, "v": n2}
