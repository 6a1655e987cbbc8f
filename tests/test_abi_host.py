"""Host-side checks of the C-ABI library (no GPU): it loads, exports every
symbol include/bf16opt.h declares, and rejects bad arguments before any HIP
call.  No compute entry point is called with valid device arguments here."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "bf16opt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def bfo():
    from bf16_numerics_amd import binding
    return binding


def test_header_declares_the_four_entry_points():
    fns = header_functions()
    for name in ("shard_range", "grad_global_norm", "adamw_sr_step", "master_to_bf16_sr"):
        assert name in fns


def test_library_exports_every_declared_symbol(bfo):
    lib = bfo.library()
    fns = header_functions()
    assert fns, "no declarations parsed"
    for name in fns:
        assert hasattr(lib, name), name
    assert sorted(bfo.EXPORTS) == fns


def test_status_strings(bfo):
    lib = bfo.library()
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10):
        s = lib.bfo_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.bfo_status_string(-99).decode() == "unknown status"


def test_shard_range_host(bfo):
    assert bfo.shard_range_status(10, 0, 0)[0] == bfo.EINVAL
    assert bfo.shard_range_status(12, 4, 4)[0] == bfo.ERANGE
    assert bfo.shard_range_status(10, 4, 0)[0] == bfo.ENOTDIVISIBLE
    assert bfo.shard_range(1_557_686_400, 8, 1) == (194_710_800, 389_421_600)
    assert bfo.shard_range(0, 3, 2) == (0, 0)
    n = 7 << 37
    spans = [bfo.shard_range(n, 7, r) for r in range(7)]
    assert spans[0][0] == 0 and spans[-1][1] == n
    assert all(spans[k][1] == spans[k + 1][0] for k in range(6))


def _create(bfo, entries, world=1, rank=0):
    arr = (bfo.BfoTensor * max(1, len(entries)))()
    for k, e in enumerate(entries):
        arr[k].offset, arr[k].numel, arr[k].flags = e[0], e[1], e[2]
        arr[k].reserved = e[3] if len(e) > 3 else 0
    h = ctypes.c_void_p(None)
    return bfo.library().bfo_table_create(arr, len(entries), world, rank, ctypes.byref(h)), h


def test_table_create_rejects_bad_tables_before_touching_the_gpu(bfo):
    assert _create(bfo, [(0, 10, 1), (11, 5, 0)])[0] == bfo.ETABLE      # gap
    assert _create(bfo, [(0, 10, 1), (8, 5, 0)])[0] == bfo.ETABLE       # overlap
    assert _create(bfo, [(1, 10, 1)])[0] == bfo.ETABLE                  # not from 0
    assert _create(bfo, [(0, 10, 2)])[0] == bfo.ETABLE                  # undefined flag bit
    assert _create(bfo, [(0, 10, 1, 7)])[0] == bfo.ETABLE               # reserved field set
    assert _create(bfo, [(0, 2**64 - 1, 0), (2**64 - 1, 5, 0)])[0] == bfo.ETABLE  # overflow
    assert _create(bfo, [(0, 30, 1)], world=4)[0] == bfo.ENOTDIVISIBLE
    assert _create(bfo, [(0, 32, 1)], world=4, rank=4)[0] == bfo.ERANGE
    assert _create(bfo, [(0, 32, 1)], world=0)[0] == bfo.EINVAL
    lib = bfo.library()
    arr = (bfo.BfoTensor * 2)()
    arr[0].offset, arr[0].numel, arr[1].offset, arr[1].numel = 0, 8, 8, 6   # 6 % 4 != 0
    h = ctypes.c_void_p(None)
    assert lib.bfo_table_create_layout(arr, 2, 4, 0, bfo.LAYOUT_PER_TENSOR, ctypes.byref(h)) == bfo.ENOTDIVISIBLE
    assert lib.bfo_table_create_layout(arr, 2, 2, 0, 7, ctypes.byref(h)) == bfo.EINVAL   # unknown layout
    lib = bfo.library()
    assert lib.bfo_table_create(None, 3, 1, 0, ctypes.byref(ctypes.c_void_p())) == bfo.EINVAL
    arr = (bfo.BfoTensor * 1)()
    assert lib.bfo_table_create(arr, 1, 1, 0, None) == bfo.EINVAL


def test_entry_points_reject_null_table_and_bad_scalars(bfo):
    lib = bfo.library()
    hp = bfo.AdamwHParams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)
    assert lib.grad_global_norm(None, None, 1.0, None, None, None) == bfo.EINVAL
    assert lib.adamw_sr_step(None, None, None, None, None, None, ctypes.byref(hp), None, None, 1, 0, 0,
                             None) == bfo.EINVAL
    assert lib.master_to_bf16_sr(None, None, None, 0, None) == bfo.EINVAL
    assert lib.bfo_decay_mask_dump(None, None, None) == bfo.EINVAL
    assert lib.bfo_table_info(None, None, None, None) == bfo.EINVAL
    assert lib.bfo_table_runs(None, None, 0, ctypes.byref(ctypes.c_uint32())) == bfo.EINVAL
    assert lib.bfo_table_destroy(None) == bfo.OK
    assert lib.bfo_rng_dump(0, 10, 0, None, None) == bfo.EINVAL
    assert lib.bfo_rng_dump(0, 10, 0, ctypes.c_void_p(1), None) == bfo.EMISALIGNED
    assert lib.bfo_rng_dump(2**64 - 5, 10, 0, ctypes.c_void_p(16), None) == bfo.ERANGE
    assert lib.bfo_stream_mix(None, None, None, None, None, 0, 0, 0, None) == bfo.OK
    assert lib.bfo_stream_mix(None, None, None, None, None, 8, 0, 0, None) == bfo.EINVAL
    assert lib.bfo_stream_mix(None, None, None, None, None, 0, 0, 3, None) == bfo.EINVAL
    p16, p8 = ctypes.c_void_p(16), ctypes.c_void_p(24)
    assert lib.bfo_stream_mix(p16, p16, p16, p16, p8, 8, 0, 0, None) == bfo.EMISALIGNED
    st = bfo.StepScalars()
    assert lib.bfo_step_scalars_fill(ctypes.byref(hp), 0, 1e-3, 1, ctypes.byref(st)) == bfo.EINVAL
    assert lib.bfo_step_scalars_fill(None, 1, 1e-3, 1, ctypes.byref(st)) == bfo.EINVAL
    assert lib.bfo_step_scalars_fill(ctypes.byref(hp), 1, 1e-3, 1, None) == bfo.EINVAL
    assert lib.adamw_sr_step_scheduled(None, None, None, None, None, None, ctypes.byref(hp), p16, 1, p16, None,
                                       None, 0, None) == bfo.EINVAL
    assert lib.adamw_sr_step_scheduled(None, None, None, None, None, None, ctypes.byref(hp), p8, 1, p16, None,
                                       None, 0, None) == bfo.EMISALIGNED
    assert lib.adamw_sr_step_scheduled(None, None, None, None, None, None, ctypes.byref(hp), p16, 1, None, None,
                                       None, 0, None) == bfo.EINVAL
    assert lib.bfo_cursor_advance(None, None) == bfo.EINVAL
    assert lib.bfo_cursor_advance(ctypes.c_void_p(20), None) == bfo.EMISALIGNED


def test_step_scalars_match_the_oracles_bias_corrections(bfo):
    # The device-resident step scalars carry the same 1 - beta^t the
    # by-value step forms; the oracle's bias corrections are pinned to the
    # printed multipliers.
    import oracle as o
    for beta1, beta2 in ((0.9, 0.95), (0.9, 0.999), (0.8, 0.99)):
        for t in (1, 2, 3, 10, 100, 1000, 123_457, 10 ** 9):
            for on in (True, False):
                hp = bfo.AdamwHParams(5e-4, beta1, beta2, 1e-8, 0.1, 1 if on else 0)
                st = bfo.step_scalars(hp, t, 2.5e-4, (1337 << 32) | t)
                assert (st.bc1, st.bc2) == o.bias_corrections(beta1, beta2, t, on), (beta1, beta2, t, on)
                assert st.t == t and st.seed == (1337 << 32) | t and st.reserved == 0
                assert st.lr == float(ctypes.c_float(2.5e-4).value)


def test_binding_refuses_a_missing_library(tmp_path, monkeypatch):
    import importlib
    import sys
    from bf16_numerics_amd import build
    monkeypatch.setattr(build, "LIB", str(tmp_path / "missing.so"))
    sys.modules.pop("bf16_numerics_amd.binding", None)
    try:
        with pytest.raises(ImportError):
            importlib.import_module("bf16_numerics_amd.binding")
    finally:
        monkeypatch.undo()
        sys.modules.pop("bf16_numerics_amd.binding", None)
        importlib.import_module("bf16_numerics_amd.binding")


def test_lr_schedule_library_matches_oracle(bfo):
    import oracle as o
    for kind in (bfo.LR_CONSTANT, bfo.LR_LINEAR, bfo.LR_COSINE, bfo.LR_WSD):
        for (W_, T_, peak, frac, dfrac) in ((0, 100, 6e-4, 0.0, 0.25), (700, 18_865, 6e-4, 0.1, 0.2),
                                           (5, 5, 1e-3, 0.5, 0.0)):
            for s in list(range(0, 40)) + list(range(T_ - 40, T_ + 5)) + [T_ // 2, 10 ** 9]:
                assert bfo.lr_at(kind, s, W_, T_, peak, frac, dfrac) == o.lr_at(kind, s, W_, T_, peak, frac, dfrac)
    lib = bfo.library()
    bad = bfo.LrSchedule(9, 0, 0, 10, 1e-3, 0.0, 0.0, 0)
    assert lib.bfo_lr_at(ctypes.byref(bad), 0, ctypes.byref(ctypes.c_float())) == bfo.EINVAL
    bad = bfo.LrSchedule(0, 0, 20, 10, 1e-3, 0.0, 0.0, 0)
    assert lib.bfo_lr_at(ctypes.byref(bad), 0, ctypes.byref(ctypes.c_float())) == bfo.EINVAL


def test_checkpoint_latest_reads_done_markers(bfo, tmp_path):
    d = str(tmp_path)
    assert bfo.checkpoint_latest(d) is None
    for name in ("state_00000012_00000.bin", "DONE_x", "DONE_", "DONEX_00000099", "DONE_00000003"):
        (tmp_path / name).write_bytes(b"")
    assert bfo.checkpoint_latest(d) == 3
    bfo.checkpoint_done(d, 12)
    assert (tmp_path / "DONE_00000012").exists()
    assert bfo.checkpoint_latest(d) == 12
    lib = bfo.library()
    assert lib.bfo_checkpoint_latest(os.fsencode(str(tmp_path / "missing")), ctypes.byref(ctypes.c_uint64())) == bfo.EIO
    assert lib.bfo_checkpoint_latest(None, None) == bfo.EINVAL
    assert lib.bfo_checkpoint_done(None, 1) == bfo.EINVAL
    assert lib.bfo_checkpoint_save(b"/tmp", None, None, None, None, None, 1, 1, 0, None) == bfo.EINVAL
    assert lib.bfo_checkpoint_load(b"/tmp", 1, None, None, None, None, None, None, None) == bfo.EINVAL


def _checksum_by_definition(data):
    """The checksum as bf16opt.h defines it, step by step in Python integers."""
    mask = (1 << 64) - 1
    prime, basis = 1099511628211, 14695981039346656037
    lanes = [basis + l for l in range(4)]
    padded = bytes(data) + b"\0" * (-len(data) % 32)
    for blk in range(0, len(padded), 32):
        for l in range(4):
            w = int.from_bytes(padded[blk + 8 * l:blk + 8 * l + 8], "little")
            lanes[l] = ((lanes[l] ^ w) * prime) & mask
    x = basis ^ len(data)
    for h in lanes:
        x = ((x ^ h) * prime) & mask
        x ^= x >> 29
    return x


def test_checksum64_follows_its_definition_and_sees_every_flipped_byte(bfo):
    rs = np.random.default_rng(9)
    for n in (0, 1, 7, 8, 31, 32, 33, 100, 1000):
        data = rs.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert bfo.checksum64(data) == _checksum_by_definition(data), n
    data = bytearray(rs.integers(0, 256, 4096 + 5, dtype=np.uint8).tobytes())
    base = bfo.checksum64(data)
    for pos in range(len(data)):                      # every single-byte change is seen
        for flip in (0x01, 0x80):
            data[pos] ^= flip
            assert bfo.checksum64(data) != base, pos
            data[pos] ^= flip
    # appending zero bytes changes the length, hence the sum
    assert bfo.checksum64(bytes(data) + b"\0") != base


def test_spread_layout_puts_each_array_on_its_own_16_gib_boundary(bfo):
    R = 1 << 34
    sizes = [3_115_372_800, 4 * 389_421_600, 778_843_200, 778_843_200, 778_843_200]
    offsets, total = bfo.spread_layout(sizes)
    assert offsets == [0, R, 2 * R, 4 * R, 5 * R] and total == 5 * R + sizes[-1]   # region 3 is skipped
    # arrays larger than a region take as many whole regions as they need
    offsets, total = bfo.spread_layout([R + 1, 5, R])
    assert offsets == [0, 2 * R, 4 * R] and total == 5 * R
    offsets, _ = bfo.spread_layout([1] * 8)
    assert offsets == [r * R for r in (0, 1, 2, 4, 5, 6, 8, 9)]
    # at every element index, arrays of non-decreasing element size stay a region or more apart
    for a, b in zip(offsets, offsets[1:]):
        assert b - a >= R
    assert bfo.spread_layout([]) == ([], 0)
    assert bfo.spread_layout([0, 0]) == ([0, 0], 0)
    lib = bfo.library()
    tot = ctypes.c_uint64()
    big = (ctypes.c_uint64 * 2)(2 ** 64 - R + 5, 8)       # the second start would pass 2^64
    off = (ctypes.c_uint64 * 2)()
    assert lib.bfo_spread_layout(big, 2, off, ctypes.byref(tot)) == bfo.ERANGE
    assert lib.bfo_spread_layout(None, 1, off, ctypes.byref(tot)) == bfo.EINVAL
    assert lib.bfo_spread_layout(big, 1, off, None) == bfo.EINVAL
