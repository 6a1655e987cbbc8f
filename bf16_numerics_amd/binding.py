"""Thin Python binding of libbf16opt.so (include/bf16opt.h).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the optimizer runs in the library's
kernels.  Importing this module fails loudly when the library has not been
built -- there is no fallback path.
"""
import ctypes
import os

import torch

from .build import LIB as _LIB_PATH

OK = 0
EINVAL = -1
ENOTDIVISIBLE = -2
ERANGE = -3
EMISALIGNED = -4
ETABLE = -5
EHIP = -6
EDEVICE = -7
EIO = -8
EFORMAT = -9
ENOTFOUND = -10

ROUND_SR = 0
ROUND_RNE = 1
FLAG_DECAY = 1
LAYOUT_FLAT = 0
LAYOUT_PER_TENSOR = 1

# Symbols declared in include/bf16opt.h.
EXPORTS = ("shard_range", "bfo_table_create", "bfo_table_create_layout", "bfo_table_destroy",
           "bfo_table_info", "bfo_table_runs",
           "grad_global_norm", "adamw_sr_step", "master_to_bf16_sr", "bfo_rng_dump",
           "bfo_decay_mask_dump", "bfo_status_string", "bfo_last_hip_error", "bfo_lr_at",
           "bfo_outlier_create", "bfo_outlier_destroy", "bfo_outlier_reset", "bfo_outlier_update",
           "bfo_checkpoint_save", "bfo_checkpoint_done", "bfo_checkpoint_latest", "bfo_checkpoint_load",
           "bfo_stream_mix", "bfo_plan_runs", "bfo_step_scalars_fill", "adamw_sr_step_scheduled",
           "bfo_cursor_advance", "bfo_spread_layout", "bfo_norm_workspace_bytes", "grad_global_norm_noalloc", "master_to_bf16",
           "bfo_checksum64", "adamw_sr_step_with_norm")

LR_CONSTANT, LR_LINEAR, LR_COSINE, LR_WSD = 0, 1, 2, 3


class BfoTensor(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("numel", ctypes.c_uint64),
                ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class BfoRun(ctypes.Structure):
    _fields_ = [("local", ctypes.c_uint64), ("addr", ctypes.c_uint64), ("global_", ctypes.c_uint64),
                ("length", ctypes.c_uint64), ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class AdamwHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("bias_correction", ctypes.c_int32)]


class LrSchedule(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("reserved", ctypes.c_uint32), ("warmup_steps", ctypes.c_uint64),
                ("total_steps", ctypes.c_uint64), ("lr_max", ctypes.c_float), ("final_frac", ctypes.c_float),
                ("decay_frac", ctypes.c_float), ("reserved2", ctypes.c_uint32)]


class StepScalars(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("bc1", ctypes.c_float), ("bc2", ctypes.c_float),
                ("reserved", ctypes.c_uint32), ("t", ctypes.c_uint64), ("seed", ctypes.c_uint64)]


NORM_RESULT_BYTES = 16  # bfo_norm_result: double sumsq; float norm; float scale
STEP_SCALARS_BYTES = 32


class BfoError(RuntimeError):
    def __init__(self, fn, status):
        msg = _lib().bfo_status_string(status).decode()
        if status == EHIP:
            msg += f" (hipError {_lib().bfo_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [{status}]")
        self.status = status


_L = None


def _lib():
    global _L
    if _L is not None:
        return _L
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it first (python -m bf16_numerics_amd.build "
                          "or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    u64, u32, vp, i32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
    pu64 = ctypes.POINTER(ctypes.c_uint64)
    sig = {
        "shard_range": (i32, [u64, u32, u32, pu64, pu64]),
        "bfo_table_create": (i32, [ctypes.POINTER(BfoTensor), u32, u32, u32, ctypes.POINTER(vp)]),
        "bfo_table_create_layout": (i32, [ctypes.POINTER(BfoTensor), u32, u32, u32, i32, ctypes.POINTER(vp)]),
        "bfo_table_runs": (i32, [vp, ctypes.POINTER(BfoRun), u32, ctypes.POINTER(u32)]),
        "bfo_table_destroy": (i32, [vp]),
        "bfo_table_info": (i32, [vp, pu64, pu64, pu64]),
        "grad_global_norm": (i32, [vp, vp, ctypes.c_float, vp, vp, vp]),
        "bfo_norm_workspace_bytes": (i32, [vp, pu64]),
        "grad_global_norm_noalloc": (i32, [vp, vp, ctypes.c_float, vp, vp]),
        "adamw_sr_step": (i32, [vp, vp, vp, vp, vp, vp, ctypes.POINTER(AdamwHParams), vp, vp, u64, u64, i32, vp]),
        "adamw_sr_step_with_norm": (i32, [vp, vp, vp, vp, vp, vp, ctypes.POINTER(AdamwHParams), ctypes.c_float, vp,
                                          vp, vp, u64, u64, i32, vp]),
        "bfo_lr_at": (i32, [ctypes.POINTER(LrSchedule), u64, ctypes.POINTER(ctypes.c_float)]),
        "bfo_outlier_create": (i32, [u32, ctypes.c_float, ctypes.POINTER(vp)]),
        "bfo_outlier_destroy": (i32, [vp]),
        "bfo_outlier_reset": (i32, [vp, vp]),
        "bfo_outlier_update": (i32, [vp, vp, vp, vp, vp]),
        "bfo_checkpoint_save": (i32, [ctypes.c_char_p, vp, vp, vp, vp, vp, u64, u64, i32, vp]),
        "bfo_checksum64": (u64, [vp, u64]),
        "master_to_bf16": (i32, [vp, vp, vp, u64, i32, vp]),
        "bfo_checkpoint_done": (i32, [ctypes.c_char_p, u64]),
        "bfo_checkpoint_latest": (i32, [ctypes.c_char_p, pu64]),
        "bfo_checkpoint_load": (i32, [ctypes.c_char_p, u64, vp, vp, vp, vp, vp, pu64, vp]),
        "master_to_bf16_sr": (i32, [vp, vp, vp, u64, vp]),
        "bfo_rng_dump": (i32, [u64, u64, u64, vp, vp]),
        "bfo_decay_mask_dump": (i32, [vp, vp, vp]),
        "bfo_stream_mix": (i32, [vp, vp, vp, vp, vp, u64, u32, i32, vp]),
        "bfo_plan_runs": (i32, [ctypes.POINTER(BfoTensor), u32, u32, u32, i32, ctypes.POINTER(BfoRun), u32,
                                ctypes.POINTER(u32), pu64]),
        "bfo_step_scalars_fill": (i32, [ctypes.POINTER(AdamwHParams), u64, ctypes.c_float, u64,
                                        ctypes.POINTER(StepScalars)]),
        "adamw_sr_step_scheduled": (i32, [vp, vp, vp, vp, vp, vp, ctypes.POINTER(AdamwHParams), vp, u64, vp, vp,
                                          vp, i32, vp]),
        "bfo_cursor_advance": (i32, [vp, vp]),
        "bfo_spread_layout": (i32, [pu64, u32, pu64, pu64]),
        "bfo_status_string": (ctypes.c_char_p, [i32]),
        "bfo_last_hip_error": (i32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _L = lib
    return lib


def library():
    """The loaded ctypes library (raises ImportError if it was not built)."""
    return _lib()


_lib()  # fail at import time when the library is missing


def _check(fn, status):
    if status != OK:
        raise BfoError(fn, status)


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _arg(t, dtype, count, name, dev):
    """Device pointer of a contiguous tensor holding exactly `count` elements."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != count:
        raise ValueError(f"{name} has {t.numel()} elements, the shard has {count}")
    return ctypes.c_void_p(t.data_ptr())


def shard_range(n, world, rank):
    b, e = ctypes.c_uint64(0), ctypes.c_uint64(0)
    _check("shard_range", _lib().shard_range(n, world, rank, ctypes.byref(b), ctypes.byref(e)))
    return b.value, e.value


def _tensor_array(entries):
    arr = (BfoTensor * max(1, len(entries)))()
    for k, (off, numel, flags) in enumerate(entries):
        arr[k].offset, arr[k].numel, arr[k].flags, arr[k].reserved = off, numel, flags, 0
    return arr


def plan_runs(entries, world=1, rank=0, layout=LAYOUT_FLAT):
    """The shard plan on the host (no GPU): (status, S, [(local, addr, global, length, flags)])."""
    arr = _tensor_array(entries)
    cnt, S = ctypes.c_uint32(0), ctypes.c_uint64(0)
    rc = _lib().bfo_plan_runs(arr, len(entries), world, rank, layout, None, 0, ctypes.byref(cnt), ctypes.byref(S))
    if rc != OK:
        return rc, 0, []
    out = (BfoRun * max(1, cnt.value))()
    rc = _lib().bfo_plan_runs(arr, len(entries), world, rank, layout, out, cnt.value, ctypes.byref(cnt),
                              ctypes.byref(S))
    return rc, S.value, [(r.local, r.addr, r.global_, r.length, r.flags) for r in out[:cnt.value]]


def shard_range_status(n, world, rank):
    b, e = ctypes.c_uint64(0), ctypes.c_uint64(0)
    rc = _lib().shard_range(n, world, rank, ctypes.byref(b), ctypes.byref(e))
    return rc, b.value, e.value


class Table:
    """A validated tensor table intersected with one ZeRO-1 shard (device-resident plan).

    entries: (offset, numel, flags) triples in buffer order; flags bit 0 = decay.
    layout: LAYOUT_FLAT (contiguous range [begin, end); params/grads passed as
    shard-local arrays) or LAYOUT_PER_TENSOR (1/world of every tensor;
    params/grads passed as the full n-element buffers).
    Created on the current device; every call must use that device.
    """

    def __init__(self, entries, world=1, rank=0, device=None, layout=LAYOUT_FLAT):
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None else
                                   torch.device(device).index or 0)
        arr = _tensor_array(entries)
        h = ctypes.c_void_p(None)
        with torch.cuda.device(self.device):
            _check("bfo_table_create_layout",
                   _lib().bfo_table_create_layout(arr, len(entries), world, rank, layout, ctypes.byref(h)))
        self._h = h
        n, b, e = ctypes.c_uint64(0), ctypes.c_uint64(0), ctypes.c_uint64(0)
        _check("bfo_table_info", _lib().bfo_table_info(h, ctypes.byref(n), ctypes.byref(b), ctypes.byref(e)))
        self.n, self.begin, self.end = n.value, b.value, e.value
        self.world, self.rank, self.layout = world, rank, layout

    @property
    def size(self):
        """Shard length S (elements of master / m / v)."""
        return self.end - self.begin

    @property
    def pg_size(self):
        """Elements the params / grads arrays must hold for this layout."""
        return self.n if self.layout == LAYOUT_PER_TENSOR else self.size

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("table destroyed")
        return self._h

    def runs(self):
        """The shard plan: list of (local, addr, global, length, flags)."""
        cnt = ctypes.c_uint32(0)
        _check("bfo_table_runs", _lib().bfo_table_runs(self.handle, None, 0, ctypes.byref(cnt)))
        arr = (BfoRun * max(1, cnt.value))()
        _check("bfo_table_runs", _lib().bfo_table_runs(self.handle, arr, cnt.value, ctypes.byref(cnt)))
        return [(r.local, r.addr, r.global_, r.length, r.flags) for r in arr[:cnt.value]]

    def global_index(self):
        """Global index of every shard position, expanded from the plan (numpy uint64)."""
        import numpy as np
        out = np.empty(self.size, np.uint64)
        for local, _addr, glob, length, _flags in self.runs():
            out[local:local + length] = np.arange(glob, glob + length, dtype=np.uint64)
        return out

    def close(self):
        if getattr(self, "_h", None) is not None:
            torch.cuda.synchronize(self.device)
            _check("bfo_table_destroy", _lib().bfo_table_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def new_norm_result(device):
    """A zeroed device buffer for bfo_norm_result (16 bytes, 16-byte aligned)."""
    return torch.zeros(2, dtype=torch.float64, device=device)


def read_norm_result(res):
    """(sumsq, norm, scale) from a bfo_norm_result buffer (synchronises)."""
    raw = res.detach().cpu()
    sumsq = float(raw[0])
    tail = raw[1:2].view(torch.float32)
    return sumsq, float(tail[0]), float(tail[1])


def scale_ptr(res):
    """Address of bfo_norm_result.scale inside a norm-result buffer."""
    return res.data_ptr() + 12


def norm_workspace_bytes(table):
    """Device bytes grad_global_norm needs as workspace for this table."""
    out = ctypes.c_uint64(0)
    _check("bfo_norm_workspace_bytes", _lib().bfo_norm_workspace_bytes(table.handle, ctypes.byref(out)))
    return out.value


def new_norm_workspace(table):
    """A device buffer of norm_workspace_bytes(table) bytes (at least 8)."""
    return torch.empty(max(8, norm_workspace_bytes(table)), dtype=torch.uint8, device=table.device)


def grad_global_norm(table, grads, out, max_norm=1.0, workspace=None):
    """workspace: new_norm_workspace(table), or None for the table's own buffer."""
    dev = table.device
    g = _arg(grads, torch.bfloat16, table.pg_size, "grads", dev)
    if out.dtype != torch.float64 or out.numel() != 2 or out.device != dev:
        raise ValueError("out must be new_norm_result(device)")
    ws = None
    if workspace is not None:
        if workspace.device != dev or not workspace.is_contiguous() or \
                workspace.numel() * workspace.element_size() < norm_workspace_bytes(table):
            raise ValueError("workspace must be new_norm_workspace(table)")
        ws = ctypes.c_void_p(workspace.data_ptr())
    with torch.cuda.device(dev):
        _check("grad_global_norm", _lib().grad_global_norm(table.handle, g, max_norm, ws,
                                                           ctypes.c_void_p(out.data_ptr()), _stream(dev)))
    return out


def grad_global_norm_noalloc(table, grads, out, max_norm=1.0):
    """grad_global_norm with the library's fixed device array as workspace
    (allocates nothing; calls on one GPU must not overlap in time)."""
    dev = table.device
    g = _arg(grads, torch.bfloat16, table.pg_size, "grads", dev)
    if out.dtype != torch.float64 or out.numel() != 2 or out.device != dev:
        raise ValueError("out must be new_norm_result(device)")
    with torch.cuda.device(dev):
        _check("grad_global_norm_noalloc", _lib().grad_global_norm_noalloc(table.handle, g, max_norm,
                                                                           ctypes.c_void_p(out.data_ptr()),
                                                                           _stream(dev)))
    return out


def _scale_arg(scale, dev):
    """A norm-result buffer (its .scale is used), an int device address, or None for 1.0."""
    if isinstance(scale, torch.Tensor):
        if scale.dtype != torch.float64 or scale.numel() != 2 or scale.device != dev:
            raise ValueError("scale must be a norm-result buffer on the table's device")
        return ctypes.c_void_p(scale_ptr(scale))
    if scale is None:
        return None
    return ctypes.c_void_p(int(scale))


def adamw_sr_step(table, params, grads, master, m, v, hp, t, seed, scale=None,
                  rounding=ROUND_SR, skip=None):
    """One fused AdamW step over the shard.  scale: a norm-result buffer
    (its .scale is used), an int device address, or None for 1.0.  skip: an
    int32 device tensor of one element (nonzero -> the step changes nothing)
    or None."""
    dev = table.device
    S = table.size
    p = _arg(params, torch.bfloat16, table.pg_size, "params", dev)
    g = _arg(grads, torch.bfloat16, table.pg_size, "grads", dev)
    M = _arg(master, torch.float32, S, "master", dev)
    mm = _arg(m, torch.float32, S, "m", dev)
    vv = _arg(v, torch.float32, S, "v", dev)
    sp = _scale_arg(scale, dev)
    sk = _arg(skip, torch.int32, 1, "skip", dev) if skip is not None else None
    h = _hparams(hp)
    with torch.cuda.device(dev):
        _check("adamw_sr_step", _lib().adamw_sr_step(table.handle, p, g, M, mm, vv, ctypes.byref(h), sp, sk,
                                                     t, seed, rounding, _stream(dev)))


def adamw_sr_step_with_norm(table, params, grads, master, m, v, hp, t, seed, out, max_norm=1.0,
                            rounding=ROUND_SR, skip=None, workspace=None):
    """grad_global_norm into `out` (a norm-result buffer) and the update with
    its scale, in one call (one launch for shards of at most 65,536 elements)."""
    dev = table.device
    S = table.size
    p = _arg(params, torch.bfloat16, table.pg_size, "params", dev)
    g = _arg(grads, torch.bfloat16, table.pg_size, "grads", dev)
    M = _arg(master, torch.float32, S, "master", dev)
    mm = _arg(m, torch.float32, S, "m", dev)
    vv = _arg(v, torch.float32, S, "v", dev)
    if out.dtype != torch.float64 or out.numel() != 2 or out.device != dev:
        raise ValueError("out must be new_norm_result(device)")
    sk = _arg(skip, torch.int32, 1, "skip", dev) if skip is not None else None
    ws = None
    if workspace is not None:
        if workspace.device != dev or not workspace.is_contiguous() or \
                workspace.numel() * workspace.element_size() < norm_workspace_bytes(table):
            raise ValueError("workspace must be new_norm_workspace(table)")
        ws = ctypes.c_void_p(workspace.data_ptr())
    with torch.cuda.device(dev):
        _check("adamw_sr_step_with_norm", _lib().adamw_sr_step_with_norm(
            table.handle, p, g, M, mm, vv, ctypes.byref(_hparams(hp)), max_norm, ws,
            ctypes.c_void_p(out.data_ptr()), sk, t, seed, rounding, _stream(dev)))


def _hparams(hp):
    if isinstance(hp, AdamwHParams):
        return hp
    return AdamwHParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, 1 if hp.bias_correction else 0)


def step_scalars(hp, t, lr, seed):
    """The per-step scalars of step t (bfo_step_scalars_fill), as a StepScalars."""
    out = StepScalars()
    _check("bfo_step_scalars_fill", _lib().bfo_step_scalars_fill(ctypes.byref(_hparams(hp)), t, lr, seed,
                                                                 ctypes.byref(out)))
    return out


def step_schedule(hp, steps, device):
    """A device array of bfo_step_scalars for [(t, lr, seed), ...] (uint8 tensor, 32 bytes per step)."""
    arr = (StepScalars * max(1, len(steps)))()
    for k, (t, lr, seed) in enumerate(steps):
        arr[k] = step_scalars(hp, t, lr, seed)
    host = torch.frombuffer(bytearray(bytes(arr)[:STEP_SCALARS_BYTES * len(steps)]), dtype=torch.uint8)
    return host.to(device)


def adamw_sr_step_scheduled(table, params, grads, master, m, v, hp, steps, cursor, scale=None,
                            rounding=ROUND_SR, skip=None):
    """adamw_sr_step with lr, bias corrections and seed read on the device from
    steps[cursor] (steps: step_schedule(...); cursor: an int64 device tensor of
    one element).  Nothing passed here changes from step to step."""
    dev = table.device
    S = table.size
    p = _arg(params, torch.bfloat16, table.pg_size, "params", dev)
    g = _arg(grads, torch.bfloat16, table.pg_size, "grads", dev)
    M = _arg(master, torch.float32, S, "master", dev)
    mm = _arg(m, torch.float32, S, "m", dev)
    vv = _arg(v, torch.float32, S, "v", dev)
    if steps.dtype != torch.uint8 or steps.numel() % STEP_SCALARS_BYTES or steps.device != dev \
            or not steps.is_contiguous():
        raise ValueError("steps must be step_schedule(...) on the table's device")
    cur = _arg(cursor, torch.int64, 1, "cursor", dev)
    sp = _scale_arg(scale, dev)
    sk = _arg(skip, torch.int32, 1, "skip", dev) if skip is not None else None
    with torch.cuda.device(dev):
        _check("adamw_sr_step_scheduled", _lib().adamw_sr_step_scheduled(
            table.handle, p, g, M, mm, vv, ctypes.byref(_hparams(hp)), ctypes.c_void_p(steps.data_ptr()),
            steps.numel() // STEP_SCALARS_BYTES, cur, sp, sk, rounding, _stream(dev)))


def cursor_advance(cursor):
    """cursor += 1 on the device (an int64 tensor of one element)."""
    c = _arg(cursor, torch.int64, 1, "cursor", cursor.device)
    with torch.cuda.device(cursor.device):
        _check("bfo_cursor_advance", _lib().bfo_cursor_advance(c, _stream(cursor.device)))


REGION_BYTES = 1 << 34


def spread_layout(sizes):
    """(offsets, total) placing arrays of `sizes` bytes each on its own 16 GiB
    boundary after the previous (bfo_spread_layout)."""
    n = len(sizes)
    b = (ctypes.c_uint64 * max(1, n))(*sizes)
    off = (ctypes.c_uint64 * max(1, n))()
    tot = ctypes.c_uint64(0)
    _check("bfo_spread_layout", _lib().bfo_spread_layout(b, n, off, ctypes.byref(tot)))
    return list(off[:n]), tot.value


def lr_at(kind, step, warmup_steps, total_steps, lr_max, final_frac=0.0, decay_frac=0.0):
    """The library's learning-rate schedule at 0-based `step` (host only)."""
    sch = LrSchedule(kind, 0, warmup_steps, total_steps, lr_max, final_frac, decay_frac, 0)
    out = ctypes.c_float(0.0)
    _check("bfo_lr_at", _lib().bfo_lr_at(ctypes.byref(sch), step, ctypes.byref(out)))
    return out.value


class Outlier:
    """Device-side z-score detector over the last `window` values."""

    def __init__(self, window=128, threshold=0.0, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None else
                                   torch.device(device).index or 0)
        h = ctypes.c_void_p(None)
        with torch.cuda.device(self.device):
            _check("bfo_outlier_create", _lib().bfo_outlier_create(window, threshold, ctypes.byref(h)))
        self._h = h
        self.z = torch.zeros(1, dtype=torch.float32, device=self.device)
        self.skip = torch.zeros(1, dtype=torch.int32, device=self.device)

    def update(self, value_ptr):
        """Queue an update reading the device float at `value_ptr` (an int
        address or a one-element float32 tensor); fills self.z, self.skip."""
        vp = value_ptr.data_ptr() if isinstance(value_ptr, torch.Tensor) else int(value_ptr)
        with torch.cuda.device(self.device):
            _check("bfo_outlier_update", _lib().bfo_outlier_update(
                self._h, ctypes.c_void_p(vp), ctypes.c_void_p(self.z.data_ptr()),
                ctypes.c_void_p(self.skip.data_ptr()), _stream(self.device)))
        return self

    def reset(self):
        with torch.cuda.device(self.device):
            _check("bfo_outlier_reset", _lib().bfo_outlier_reset(self._h, _stream(self.device)))

    def close(self):
        if getattr(self, "_h", None) is not None:
            torch.cuda.synchronize(self.device)
            _check("bfo_outlier_destroy", _lib().bfo_outlier_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def norm_ptr(res):
    """Address of bfo_norm_result.norm inside a norm-result buffer."""
    return res.data_ptr() + 8


def master_to_bf16_sr(table, master, params, seed):
    dev = table.device
    M = _arg(master, torch.float32, table.size, "master", dev)
    p = _arg(params, torch.bfloat16, table.pg_size, "params", dev)
    with torch.cuda.device(dev):
        _check("master_to_bf16_sr", _lib().master_to_bf16_sr(table.handle, M, p, seed, _stream(dev)))


def master_to_bf16(table, master, params, seed, rounding=ROUND_SR):
    dev = table.device
    M = _arg(master, torch.float32, table.size, "master", dev)
    p = _arg(params, torch.bfloat16, table.pg_size, "params", dev)
    with torch.cuda.device(dev):
        _check("master_to_bf16", _lib().master_to_bf16(table.handle, M, p, seed, rounding, _stream(dev)))


def checksum64(data):
    """bfo_checksum64 of a bytes-like object (host only)."""
    buf = (ctypes.c_char * len(data)).from_buffer_copy(bytes(data))
    return _lib().bfo_checksum64(buf, len(data))


def rng_dump(first, count, seed, device=None):
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else torch.device(device).index or 0)
    out = torch.empty(count, dtype=torch.int16, device=dev)
    with torch.cuda.device(dev):
        _check("bfo_rng_dump", _lib().bfo_rng_dump(first, count, seed, ctypes.c_void_p(out.data_ptr()),
                                                   _stream(dev)))
    return out


def decay_mask_dump(table):
    dev = table.device
    out = torch.empty(table.size, dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check("bfo_decay_mask_dump", _lib().bfo_decay_mask_dump(table.handle, ctypes.c_void_p(out.data_ptr()),
                                                                 _stream(dev)))
    return out


MIX_BOTH, MIX_READS, MIX_WRITES = 0, 1, 2


def stream_mix(params, grads, master, m, v, key=0, mode=MIX_BOTH):
    """The update's memory traffic without its arithmetic (bandwidth ceiling).

    MIX_BOTH with a master: m, v, master ^= key as bit patterns and params =
    grads ^ (key & 0xFFFF); master None: m, v ^= key and params ^= grads ^
    (key & 0xFFFF).  MIX_READS: the same reads, nothing written.  MIX_WRITES:
    the same writes (key- and index-made words), nothing read."""
    count = m.numel()
    dev = m.device
    args = [_arg(params, torch.bfloat16, count, "params", dev), _arg(grads, torch.bfloat16, count, "grads", dev),
            _arg(master, torch.float32, count, "master", dev), _arg(m, torch.float32, count, "m", dev),
            _arg(v, torch.float32, count, "v", dev)]
    with torch.cuda.device(dev):
        _check("bfo_stream_mix", _lib().bfo_stream_mix(*args, count, key & 0xFFFFFFFF, mode, _stream(dev)))


def checkpoint_save(directory, table, m, v, step, seed, master=None, params=None, rounding=ROUND_SR):
    """Write this rank's state of `step`: master and/or params (at least one),
    m, v, and the seed and rounding mode of the last update."""
    dev = table.device
    M = _arg(master, torch.float32, table.size, "master", dev)
    p = _arg(params, torch.bfloat16, table.pg_size, "params", dev)
    mm = _arg(m, torch.float32, table.size, "m", dev)
    vv = _arg(v, torch.float32, table.size, "v", dev)
    with torch.cuda.device(dev):
        _check("bfo_checkpoint_save", _lib().bfo_checkpoint_save(os.fsencode(directory), table.handle, p, M, mm, vv,
                                                               step, seed, rounding, _stream(dev)))


def checkpoint_done(directory, step):
    _check("bfo_checkpoint_done", _lib().bfo_checkpoint_done(os.fsencode(directory), step))


def checkpoint_latest(directory):
    """Largest step with a DONE marker, or None."""
    out = ctypes.c_uint64(0)
    rc = _lib().bfo_checkpoint_latest(os.fsencode(directory), ctypes.byref(out))
    if rc == ENOTFOUND:
        return None
    _check("bfo_checkpoint_latest", rc)
    return out.value


def checkpoint_load(directory, step, table, m, v, master=None, params=None):
    """Read this rank's state of `step` (params stored or rebuilt from the
    stored master when given); returns the saved seed."""
    dev = table.device
    M = _arg(master, torch.float32, table.size, "master", dev)
    p = _arg(params, torch.bfloat16, table.pg_size, "params", dev)
    mm = _arg(m, torch.float32, table.size, "m", dev)
    vv = _arg(v, torch.float32, table.size, "v", dev)
    seed = ctypes.c_uint64(0)
    with torch.cuda.device(dev):
        _check("bfo_checkpoint_load", _lib().bfo_checkpoint_load(os.fsencode(directory), step, table.handle, p, M,
                                                               mm, vv, ctypes.byref(seed), _stream(dev)))
    return seed.value
