"""The host shard plan (bfo_plan_runs: the runs a table is built from)
against the oracle's shard range, per-tensor map and decay mask, on the CPU.
Small tables are expanded element by element; the full-size models are
checked at every run boundary."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as o
from bf16_numerics_amd import binding as bfo
from bf16_numerics_amd import workloads as W


def random_table(seed, n_tensors=40, world=8):
    """Tensor sizes 0..3000 (multiples of `world` when asked), random flags."""
    rs = np.random.default_rng(seed)
    entries, off = [], 0
    for _ in range(n_tensors):
        numel = int(rs.integers(0, 3000)) * (world if seed % 2 else 1)
        entries.append((off, numel, int(rs.integers(0, 2))))
        off += numel
    # pad so that flat shards over `world` ranks divide
    pad = (-off) % world
    if pad:
        entries.append((off, pad, 0))
    return entries


def expand(runs):
    """(local, addr, global, flag) of every shard position, from the runs."""
    if not runs:
        z = np.zeros(0, np.uint64)
        return z, z, z, np.zeros(0, np.uint8)
    local = np.concatenate([np.arange(lo, lo + n, dtype=np.uint64) for lo, _, _, n, _ in runs])
    addr = np.concatenate([np.arange(a, a + n, dtype=np.uint64) for _, a, _, n, _ in runs])
    glob = np.concatenate([np.arange(g, g + n, dtype=np.uint64) for _, _, g, n, _ in runs])
    flag = np.concatenate([np.full(n, f, np.uint8) for _, _, _, n, f in runs])
    return local, addr, glob, flag


def assert_maximal(runs):
    for p, q in zip(runs, runs[1:]):
        continues = p[1] + p[3] == q[1] and p[2] + p[3] == q[2]
        assert not (continues and p[4] == q[4]), f"runs {p} and {q} should have merged"


SMALL = [("tiny", W.tiny().entries())] + [(f"random{s}", random_table(s)) for s in range(6)]


@pytest.mark.parametrize("name,entries", SMALL)
@pytest.mark.parametrize("world", [1, 2, 8])
def test_flat_plan_matches_oracle_elementwise(name, entries, world):
    tbl = o.table(entries)
    n = sum(e[1] for e in entries)
    mask = o.decay_mask(tbl, 0, n)
    for rank in range(world):
        rc, S, runs = bfo.plan_runs(entries, world, rank, bfo.LAYOUT_FLAT)
        rc_o, b, e = o.shard_range(n, world, rank)
        assert rc == rc_o
        if rc != o.OK:
            continue
        assert S == e - b
        local, addr, glob, flag = expand(runs)
        assert np.array_equal(local, np.arange(S, dtype=np.uint64))
        assert np.array_equal(addr, local)
        assert np.array_equal(glob, np.arange(b, e, dtype=np.uint64))
        assert np.array_equal(flag, mask[b:e])
        assert_maximal(runs)


@pytest.mark.parametrize("name,entries", SMALL)
@pytest.mark.parametrize("world", [1, 2, 8])
def test_per_tensor_plan_matches_oracle_elementwise(name, entries, world):
    tbl = o.table(entries)
    n = sum(e[1] for e in entries)
    mask = o.decay_mask(tbl, 0, n)
    for rank in range(world):
        rc, S, runs = bfo.plan_runs(entries, world, rank, bfo.LAYOUT_PER_TENSOR)
        rc_o, gidx = o.shard_map_per_tensor(tbl, world, rank)
        assert rc == rc_o, (name, world, rank)
        if rc != o.OK:
            continue
        assert S == gidx.size
        local, addr, glob, flag = expand(runs)
        assert np.array_equal(local, np.arange(S, dtype=np.uint64))
        assert np.array_equal(glob, gidx)
        assert np.array_equal(addr, glob)
        assert np.array_equal(flag, mask[gidx.astype(np.int64)])
        assert_maximal(runs)


@pytest.mark.parametrize("make,world,layout", [
    (W.gpt2_1p5b_shard, 8, bfo.LAYOUT_FLAT), (W.gpt2_1p5b_shard, 8, bfo.LAYOUT_PER_TENSOR),
    (W.llama7b, 1, bfo.LAYOUT_FLAT), (W.llama7b, 8, bfo.LAYOUT_FLAT), (W.llama7b, 8, bfo.LAYOUT_PER_TENSOR)])
def test_full_size_plans_at_every_run_boundary(make, world, layout):
    w = make()
    entries = w.entries()
    tbl = o.table(entries)
    n = w.n
    offsets = np.array([e[0] for e in entries], np.uint64)
    for rank in range(world):
        rc, S, runs = bfo.plan_runs(entries, world, rank, layout)
        assert rc == o.OK
        assert S == n // world
        assert sum(r[3] for r in runs) == S
        expect_local = 0
        for local, addr, glob, length, flag in runs:
            assert local == expect_local
            expect_local += length
            if layout == bfo.LAYOUT_FLAT:
                assert addr == local and glob == rank * S + local
            else:
                assert addr == glob
                # the run is rank `rank`'s slice of one tensor (or of several adjacent equal-flag ones)
                k = int(np.searchsorted(offsets, np.uint64(glob), side="right")) - 1
                slice_len = entries[k][1] // world
                assert glob == entries[k][0] + rank * slice_len
            for g in (glob, glob + length - 1):
                assert o.decay_mask(tbl, int(g), 1)[0] == flag
        assert_maximal(runs)
    if layout == bfo.LAYOUT_PER_TENSOR and n < 2_000_000_000:
        # rank 1 in full: every shard position's global index equals the oracle's map
        rc_o, gidx = o.shard_map_per_tensor(tbl, world, 1)
        assert rc_o == o.OK
        pos = 0
        for _, _, glob, length, _ in bfo.plan_runs(entries, world, 1, layout)[2]:
            seg = gidx[pos:pos + length]
            assert seg[0] == glob and seg[-1] == glob + length - 1
            assert np.all(np.diff(seg.astype(np.int64)) == 1)
            pos += length
        assert pos == gidx.size


def test_plan_errors_match_oracle():
    good = [(0, 8, 1), (8, 8, 0)]
    cases = [
        ([(0, 8, 1), (9, 8, 0)], 2, 0, bfo.LAYOUT_FLAT),        # gap
        ([(0, 8, 2)], 1, 0, bfo.LAYOUT_FLAT),                   # undefined flag bit
        (good, 0, 0, bfo.LAYOUT_FLAT),                          # no ranks
        (good, 2, 2, bfo.LAYOUT_FLAT),                          # rank out of range
        (good, 3, 0, bfo.LAYOUT_FLAT),                          # 16 over 3 does not divide
        ([(0, 6, 1), (6, 10, 0)], 4, 0, bfo.LAYOUT_PER_TENSOR),  # n divides, tensor sizes do not
        (good, 2, 0, 7),                                        # unknown layout
    ]
    expect = [o.ETABLE, o.ETABLE, o.EINVAL, o.ERANGE, o.ENOTDIVISIBLE, o.ENOTDIVISIBLE, o.EINVAL]
    for (entries, world, rank, layout), want in zip(cases, expect):
        rc, _, _ = bfo.plan_runs(entries, world, rank, layout)
        assert rc == want, (entries, world, rank, layout, rc)
        if layout == bfo.LAYOUT_PER_TENSOR:
            assert o.shard_map_per_tensor(o.table(entries), world, rank)[0] == want
        elif layout == bfo.LAYOUT_FLAT:
            rc_t, n = o.table_check(o.table(entries))
            rc_o = rc_t if rc_t != o.OK else o.shard_range(n, world, rank)[0]
            assert rc_o == want


def test_plan_capacity_and_null_arguments():
    lib = bfo.library()
    import ctypes
    arr = (bfo.BfoTensor * 2)()
    arr[0].offset, arr[0].numel, arr[0].flags = 0, 8, 1
    arr[1].offset, arr[1].numel, arr[1].flags = 8, 8, 0
    cnt, S = ctypes.c_uint32(0), ctypes.c_uint64(0)
    out = (bfo.BfoRun * 1)()
    assert lib.bfo_plan_runs(arr, 2, 1, 0, bfo.LAYOUT_FLAT, None, 0, None, None) == bfo.EINVAL
    assert lib.bfo_plan_runs(arr, 2, 1, 0, bfo.LAYOUT_FLAT, None, 0, ctypes.byref(cnt), ctypes.byref(S)) == bfo.OK
    assert (cnt.value, S.value) == (2, 16)
    assert lib.bfo_plan_runs(arr, 2, 1, 0, bfo.LAYOUT_FLAT, out, 1, ctypes.byref(cnt), None) == bfo.ERANGE
    assert lib.bfo_plan_runs(None, 2, 1, 0, bfo.LAYOUT_FLAT, None, 0, ctypes.byref(cnt), None) == bfo.EINVAL
    assert lib.bfo_plan_runs(None, 0, 1, 0, bfo.LAYOUT_FLAT, None, 0, ctypes.byref(cnt), ctypes.byref(S)) == bfo.OK
    assert (cnt.value, S.value) == (0, 0)


@st.composite
def tables_and_shards(draw):
    """A random table (0-12 tensors of 0-70 elements, random flags, some
    sizes multiples of the shard count), a shard count, a rank and a layout."""
    world = draw(st.integers(1, 9))
    sizes = draw(st.lists(st.integers(0, 70), max_size=12))
    if draw(st.booleans()):
        sizes = [s * world for s in sizes]
    flags = draw(st.lists(st.integers(0, 1), min_size=len(sizes), max_size=len(sizes)))
    entries, off = [], 0
    for numel, f in zip(sizes, flags):
        entries.append((off, numel, f))
        off += numel
    rank = draw(st.integers(0, world - 1))
    layout = draw(st.sampled_from([bfo.LAYOUT_FLAT, bfo.LAYOUT_PER_TENSOR]))
    return entries, world, rank, layout


@settings(max_examples=400, deadline=None)
@given(tables_and_shards())
def test_random_plans_match_the_oracle(case):
    # Any table, shard count, rank and layout: the host plan either fails with
    # the oracle's status or expands, element by element, to the oracle's
    # global index map and decay mask, in maximal runs.
    entries, world, rank, layout = case
    tbl = o.table(entries)
    n = sum(e[1] for e in entries)
    rc, S, runs = bfo.plan_runs(entries, world, rank, layout)
    if layout == bfo.LAYOUT_PER_TENSOR:
        rc_o, gidx = o.shard_map_per_tensor(tbl, world, rank)
    else:
        rc_o, b, e = o.shard_range(n, world, rank)
        gidx = np.arange(b, e, dtype=np.uint64) if rc_o == o.OK else None
    assert rc == rc_o, (entries, world, rank, layout)
    if rc != o.OK:
        return
    local, addr, glob, flag = expand(runs)
    assert S == gidx.size
    assert np.array_equal(local, np.arange(S, dtype=np.uint64))
    assert np.array_equal(glob, gidx)
    assert np.array_equal(addr, glob if layout == bfo.LAYOUT_PER_TENSOR else local)
    assert np.array_equal(flag, o.decay_mask(tbl, 0, n)[gidx.astype(np.int64)] if n else flag)
    assert_maximal(runs)
