"""Python access to the CPU oracle (oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It marshals numpy arrays into the plain C reference and
adds no arithmetic of its own.  bf16 values travel as their uint16 bit
patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

ROUND_SR = 0
ROUND_RNE = 1

OK = 0
EINVAL = -1
ENOTDIVISIBLE = -2
ERANGE = -3
ETABLE = -5

TENSOR_DTYPE = np.dtype([("offset", "<u8"), ("numel", "<u8"), ("flags", "<u4"), ("pad", "<u4")])


class _HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("bias_correction", ctypes.c_int32)]


_u8 = ctypes.c_uint8
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_vp = ctypes.c_void_p

_LIB = None


def _load():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    sig = {
        "oracle_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "oracle_bf16_to_f32_array": (None, [_vp, ctypes.c_uint64, _vp]),
        "oracle_round_nearest_even": (ctypes.c_uint16, [ctypes.c_float]),
        "oracle_round_stochastic": (ctypes.c_uint16, [ctypes.c_float, ctypes.c_uint16]),
        "oracle_round_stochastic_array": (None, [_vp, _vp, ctypes.c_uint64, _vp]),
        "oracle_round_nearest_even_array": (None, [_vp, ctypes.c_uint64, _vp]),
        "oracle_philox4x32_10": (None, [_u32p, _u32p, _u32p]),
        "oracle_rng16": (ctypes.c_uint16, [ctypes.c_uint64, ctypes.c_uint64]),
        "oracle_rng16_fill": (None, [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, _vp]),
        "oracle_shard_range": (ctypes.c_int, [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, _u64p, _u64p]),
        "oracle_table_check": (ctypes.c_int, [_vp, ctypes.c_uint32, _u64p]),
        "oracle_decay_mask": (ctypes.c_int, [_vp, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64, _vp]),
        "oracle_grad_norm": (None, [_vp, ctypes.c_uint64, ctypes.c_float, _f64p, _f32p, _f32p]),
        "oracle_norm_from_sumsq": (None, [ctypes.c_double, ctypes.c_float, _f32p, _f32p]),
        "oracle_bias_corrections": (None, [ctypes.c_float, ctypes.c_float, ctypes.c_uint64, ctypes.c_int, _f32p, _f32p]),
        "oracle_adamw_step": (ctypes.c_int, [_vp, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint64,
                                             _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_HParams),
                                             ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int]),
        "oracle_master_to_bf16_sr": (None, [_vp, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, _vp]),
        "oracle_adamw_step_mapped": (ctypes.c_int, [_vp, ctypes.c_uint32, _vp, ctypes.c_uint64,
                                                    _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_HParams),
                                                    ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int]),
        "oracle_shard_map_per_tensor": (ctypes.c_int, [_vp, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                                       _vp, ctypes.c_uint64, _u64p]),
        "oracle_master_to_bf16_sr_mapped": (None, [_vp, _vp, ctypes.c_uint64, ctypes.c_uint64, _vp]),
        "oracle_lr_at": (ctypes.c_float, [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_float, ctypes.c_float, ctypes.c_float]),
        "oracle_outlier_init": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint32]),
        "oracle_outlier_update": (None, [ctypes.c_void_p, ctypes.c_float, ctypes.c_float,
                                         ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _need(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != np.dtype(dtype) or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"{name} must be a C-contiguous numpy array of {np.dtype(dtype)}")
    return a


def table(entries):
    """Build a tensor table from (offset, numel, flags) triples."""
    t = np.zeros(len(entries), dtype=TENSOR_DTYPE)
    for k, (off, numel, flags) in enumerate(entries):
        t[k] = (off, numel, flags, 0)
    return t


def hparams(lr, beta1, beta2, eps, weight_decay, bias_correction=True):
    return _HParams(lr, beta1, beta2, eps, weight_decay, 1 if bias_correction else 0)


def bf16_to_f32(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().oracle_bf16_to_f32_array(_ptr(h), h.size, _ptr(out))
    return out


def round_nearest_even(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_round_nearest_even_array(_ptr(x), x.size, _ptr(out))
    return out


def round_stochastic(x, r):
    x = np.ascontiguousarray(x, dtype=np.float32)
    r = np.ascontiguousarray(np.broadcast_to(r, x.shape), dtype=np.uint16)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_round_stochastic_array(_ptr(x), _ptr(r), x.size, _ptr(out))
    return out


def philox4x32_10(counter, key):
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in counter])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    out = (ctypes.c_uint32 * 4)()
    _load().oracle_philox4x32_10(c, k, out)
    return [int(v) for v in out]


def rng16(first, count, seed):
    out = np.empty(count, np.uint16)
    _load().oracle_rng16_fill(first, count, seed, _ptr(out))
    return out


def shard_range(n, world, rank):
    """Returns (status, begin, end)."""
    b = ctypes.c_uint64(0)
    e = ctypes.c_uint64(0)
    rc = _load().oracle_shard_range(n, world, rank, ctypes.byref(b), ctypes.byref(e))
    return rc, b.value, e.value


def table_check(tbl):
    n = ctypes.c_uint64(0)
    rc = _load().oracle_table_check(_ptr(tbl), len(tbl), ctypes.byref(n))
    return rc, n.value


def decay_mask(tbl, begin, count):
    out = np.empty(count, np.uint8)
    rc = _load().oracle_decay_mask(_ptr(tbl), len(tbl), begin, count, _ptr(out))
    if rc != OK:
        raise ValueError(f"oracle_decay_mask failed: {rc}")
    return out


def grad_norm(g, max_norm=1.0):
    """Returns (sumsq, norm, scale)."""
    g = _need(g, np.uint16, "g")
    s = ctypes.c_double(0.0)
    nrm = ctypes.c_float(0.0)
    sc = ctypes.c_float(0.0)
    _load().oracle_grad_norm(_ptr(g), g.size, max_norm, ctypes.byref(s), ctypes.byref(nrm), ctypes.byref(sc))
    return s.value, nrm.value, sc.value


def norm_from_sumsq(sumsq, max_norm=1.0):
    """(norm, scale) for a sum of squares formed elsewhere."""
    nrm = ctypes.c_float(0.0)
    sc = ctypes.c_float(0.0)
    _load().oracle_norm_from_sumsq(sumsq, max_norm, ctypes.byref(nrm), ctypes.byref(sc))
    return nrm.value, sc.value


def bias_corrections(beta1, beta2, t, bias_correction=True):
    b1 = ctypes.c_float(0.0)
    b2 = ctypes.c_float(0.0)
    _load().oracle_bias_corrections(beta1, beta2, t, 1 if bias_correction else 0,
                                    ctypes.byref(b1), ctypes.byref(b2))
    return b1.value, b2.value


def adamw_step(tbl, begin, P, G, M, m, v, hp, grad_scale, t, seed, rounding=ROUND_SR):
    """One step in place over global elements [begin, begin + len(P))."""
    n = P.size
    _need(P, np.uint16, "P")
    _need(G, np.uint16, "G")
    _need(m, np.float32, "m")
    _need(v, np.float32, "v")
    if M is not None:
        _need(M, np.float32, "M")
        if M.size != n:
            raise ValueError("size mismatch")
    if G.size != n or m.size != n or v.size != n:
        raise ValueError("size mismatch")
    rc = _load().oracle_adamw_step(_ptr(tbl), len(tbl), begin, n, _ptr(P), _ptr(G), _ptr(M),
                                   _ptr(m), _ptr(v), ctypes.byref(hp), grad_scale, t, seed, rounding)
    if rc != OK:
        raise ValueError(f"oracle_adamw_step failed: {rc}")


def master_to_bf16_sr(M, begin, seed):
    _need(M, np.float32, "M")
    out = np.empty(M.size, np.uint16)
    _load().oracle_master_to_bf16_sr(_ptr(M), begin, M.size, seed, _ptr(out))
    return out


def shard_map_per_tensor(tbl, world, rank):
    """(status, global index of every shard position) for the per-tensor layout."""
    total = int(tbl["numel"].sum()) if len(tbl) else 0
    cap = total // world if world else 0
    out = np.empty(max(cap, 1), np.uint64)
    cnt = ctypes.c_uint64(0)
    rc = _load().oracle_shard_map_per_tensor(_ptr(tbl), len(tbl), world, rank, _ptr(out), cap, ctypes.byref(cnt))
    return rc, out[:cnt.value]


def adamw_step_mapped(tbl, gidx, P_full, G_full, M, m, v, hp, grad_scale, t, seed, rounding=ROUND_SR):
    """One step in place for shard positions j -> global gidx[j]; P_full, G_full
    are full buffers, M/m/v shard-local."""
    gidx = _need(np.ascontiguousarray(gidx, np.uint64), np.uint64, "gidx")
    _need(P_full, np.uint16, "P_full")
    _need(G_full, np.uint16, "G_full")
    _need(m, np.float32, "m")
    _need(v, np.float32, "v")
    if M is not None:
        _need(M, np.float32, "M")
    n = gidx.size
    if m.size != n or v.size != n or (M is not None and M.size != n):
        raise ValueError("size mismatch")
    rc = _load().oracle_adamw_step_mapped(_ptr(tbl), len(tbl), _ptr(gidx), n, _ptr(P_full), _ptr(G_full), _ptr(M),
                                          _ptr(m), _ptr(v), ctypes.byref(hp), grad_scale, t, seed, rounding)
    if rc != OK:
        raise ValueError(f"oracle_adamw_step_mapped failed: {rc}")


def master_to_bf16_sr_mapped(M, gidx, seed, P_full):
    gidx = np.ascontiguousarray(gidx, np.uint64)
    _need(M, np.float32, "M")
    _need(P_full, np.uint16, "P_full")
    _load().oracle_master_to_bf16_sr_mapped(_ptr(M), _ptr(gidx), gidx.size, seed, _ptr(P_full))


LR_CONSTANT, LR_LINEAR, LR_COSINE, LR_WSD = 0, 1, 2, 3


def lr_at(kind, step, warmup, total, lr_max, final_frac=0.0, decay_frac=0.0):
    return _load().oracle_lr_at(kind, step, warmup, total, lr_max, final_frac, decay_frac)


class _OutlierState(ctypes.Structure):
    _fields_ = [("window", ctypes.c_uint32), ("count", ctypes.c_uint32), ("head", ctypes.c_uint32),
                ("pad", ctypes.c_uint32), ("values", ctypes.c_float * 4096)]


class Outlier:
    """The oracle's z-score detector (window of previous finite values)."""

    def __init__(self, window=128, threshold=0.0):
        self._st = _OutlierState()
        rc = _load().oracle_outlier_init(ctypes.byref(self._st), window)
        if rc != OK:
            raise ValueError(f"oracle_outlier_init failed: {rc}")
        self.threshold = threshold

    def update(self, x):
        """Returns (z, skip) for value x, then appends x if finite."""
        z = ctypes.c_float(0.0)
        sk = ctypes.c_int32(0)
        _load().oracle_outlier_update(ctypes.byref(self._st), x, self.threshold, ctypes.byref(z), ctypes.byref(sk))
        return z.value, sk.value
