"""Full-state parity of one optimizer step against the CPU oracle.

For the large shards, comparing a few windows leaves almost every element
unchecked, and the host cannot hold the oracle's copy of a 6.7e9-element
state next to the GPU's.  This helper checks every element, chunk by chunk:

  - `pre` holds device copies of the state before the step (P, M or None,
    m, v; shard-local, S elements each), `post` the live state after the
    GPU step, `G` the step's grads (S elements, shard-local);
  - each chunk of pre-state and grads is copied to pinned host memory, the
    oracle steps it in place on K host threads (static contiguous parts,
    each one call of the oracle on its own elements: the oracle's result
    for an element does not depend on the others);
  - the oracle's result is copied back to the device and compared there,
    element by element, with the GPU's post-state.

The bars are the ones the parity tests use everywhere: bf16 params equal,
or one bf16 step apart with the same sign in at most 1e-6 of the elements;
fp32 master, m and v within relative 1e-6 (NaN where the oracle has NaN).
The comparison is plain torch on whatever device the tensors live on, so the
same code is exercised on the CPU by the host test suite.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle as o

CHUNK = 1 << 26
F32_RTOL = 1e-6
BF16_FRACTION = 1e-6


def host_threads():
    """Host threads this process may use (its CPU share)."""
    k = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(k, int(cap))) if cap and cap.isdigit() else k


def parts(count, k):
    """k contiguous parts of [0, count) cut at multiples of 8 (empty ones dropped)."""
    cuts = [count * i // k // 8 * 8 for i in range(k)] + [count]
    return [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]


def compare_bf16(got, ref, what):
    """Number of bf16 patterns (int16 tensors) that differ; raises unless every
    difference is one step with the same sign and NaNs sit at the same places."""
    nan_g = (got & 0x7FFF) > 0x7F80
    nan_r = (ref & 0x7FFF) > 0x7F80
    if not torch.equal(nan_g, nan_r):
        raise AssertionError(f"{what}: NaN positions differ")
    diff = (got != ref) & ~nan_r
    nd = int(diff.sum())
    if nd:
        g, r = got[diff].to(torch.int32), ref[diff].to(torch.int32)
        far = ((g - r).abs() > 1) | ((g < 0) != (r < 0))
        if bool(far.any()):
            raise AssertionError(f"{what}: {int(far.sum())} elements more than one bf16 step apart")
    return nd


def compare_f32(got, ref, what, rtol=F32_RTOL):
    """Number of fp32 values whose bits differ; raises if any is beyond rtol
    relative to the oracle's value or NaN positions differ."""
    nan_g, nan_r = torch.isnan(got), torch.isnan(ref)
    if not torch.equal(nan_g, nan_r):
        raise AssertionError(f"{what}: NaN positions differ")
    diff = (got.view(torch.int32) != ref.view(torch.int32)) & ~nan_r
    nd = int(diff.sum())
    if nd:
        g, r = got[diff].to(torch.float64), ref[diff].to(torch.float64)
        bad = (g - r).abs() > rtol * r.abs()
        if bool(bad.any()):
            worst = float(((g - r).abs() / r.abs().clamp_min(1e-300)).max())
            raise AssertionError(f"{what}: {int(bad.sum())} elements beyond relative {rtol} (worst {worst:.3e})")
    return nd


class FullStateChecker:
    """Oracle steps and element-by-element comparisons for one shard layout
    (flat: shard element j is global index begin + j)."""

    def __init__(self, tbl, hp, max_norm, master, device, chunk=CHUNK, threads=None):
        self.tbl, self.hp, self.max_norm, self.master = tbl, hp, max_norm, master
        self.device = torch.device(device)
        self.chunk = chunk
        self.k = threads or host_threads()
        self.pool = ThreadPoolExecutor(self.k)
        pin = self.device.type == "cuda"
        self.h = {"P": torch.empty(chunk, dtype=torch.int16, pin_memory=pin),
                  "G": torch.empty(chunk, dtype=torch.int16, pin_memory=pin),
                  "m": torch.empty(chunk, dtype=torch.float32, pin_memory=pin),
                  "v": torch.empty(chunk, dtype=torch.float32, pin_memory=pin)}
        if master:
            self.h["M"] = torch.empty(chunk, dtype=torch.float32, pin_memory=pin)
        self.d = {k: torch.empty(chunk, dtype=t.dtype, device=self.device) for k, t in self.h.items() if k != "G"}

    def close(self):
        self.pool.shutdown()
        self.h = self.d = None

    def _np(self, name, n):
        a = self.h[name][:n].numpy()
        return a.view(np.uint16) if a.dtype == np.int16 else a

    def oracle_norm_parts(self, G_host_u16):
        """Sum of squares of a host chunk, as the oracle's per-part sums in part order."""
        return sum(self.pool.map(lambda r: o.grad_norm(G_host_u16[r[0]:r[1]], self.max_norm)[0],
                                 parts(G_host_u16.size, self.k)))

    def oracle_step_host(self, h, begin, scale, t, seed, rounding, segments=None, offset=0):
        """The oracle step in place over host arrays h (numpy; P, G uint16; M, m,
        v float32).  Element j holds global index begin + j; or, with
        `segments` [(local_lo, local_hi, global_lo), ...] covering the shard,
        shard element offset + j lies in the segment that holds it, at global
        index global_lo + (offset + j - local_lo)."""
        n = h["P"].size
        jobs = []
        for a, b in parts(n, self.k):
            if segments is None:
                jobs.append((a, b, begin + a))
                continue
            for lo, hi, g in segments:
                x, y = max(a, lo - offset), min(b, hi - offset)
                if x < y:
                    jobs.append((x, y, g + (offset + x - lo)))
        sl = (lambda arr, j: None if arr is None else arr[j[0]:j[1]])
        list(self.pool.map(lambda j: o.adamw_step(self.tbl, j[2], sl(h["P"], j), sl(h["G"], j), sl(h.get("M"), j),
                                                  sl(h["m"], j), sl(h["v"], j), self.hp, scale, t, seed, rounding),
                           jobs))

    def compare_host_to_device(self, got, ref, what):
        """Compare device state `got` (P int16/bf16, M, m, v) with host numpy
        `ref`, uploading the reference chunk by chunk.  Returns diff counts."""
        S = got["m"].numel()
        counts = {k: 0 for k in self.d}
        for lo in range(0, S, self.chunk):
            hi = min(S, lo + self.chunk)
            n = hi - lo
            for k in self.d:
                src = ref[k][lo:hi]
                self.h[k][:n].copy_(torch.from_numpy(src.view(np.int16) if src.dtype == np.uint16 else src))
                self.d[k][:n].copy_(self.h[k][:n])
            counts = self._add(counts, self._compare_chunk(got, lo, hi, f"{what} [{lo},{hi})"))
        return counts

    def _compare_chunk(self, got, lo, hi, what):
        n = hi - lo
        out = {"P": compare_bf16(got["P"][lo:hi].view(torch.int16), self.d["P"][:n], f"{what} params")}
        for k in ("M", "m", "v"):
            if k in self.d:
                out[k] = compare_f32(got[k][lo:hi], self.d[k][:n], f"{what} {k}")
        return out

    @staticmethod
    def _add(a, b):
        return {k: a.get(k, 0) + b.get(k, 0) for k in set(a) | set(b)}

    def check_step(self, pre, post, G, begin, scale, t, seed, rounding, segments=None):
        """Oracle(pre, G, scale) against the GPU's post-state over every element.
        All arrays shard-local; element j is global index begin + j, or as
        `segments` map it (see oracle_step_host).  Returns (diff counts per
        array, oracle sum of squares of G)."""
        S = post["m"].numel()
        counts = {k: 0 for k in self.d}
        sumsq = 0.0
        for lo in range(0, S, self.chunk):
            hi = min(S, lo + self.chunk)
            n = hi - lo
            self.h["G"][:n].copy_(G[lo:hi].view(torch.int16))
            for k in self.d:
                src = pre[k][lo:hi]
                self.h[k][:n].copy_(src.view(torch.int16) if k == "P" else src)
            h = {k: self._np(k, n) for k in self.h}
            sumsq += self.oracle_norm_parts(h["G"])
            self.oracle_step_host(h, begin + lo, scale, t, seed, rounding, segments, lo)
            for k in self.d:
                self.d[k][:n].copy_(self.h[k][:n])
            counts = self._add(counts, self._compare_chunk(post, lo, hi, f"t={t} [{lo},{hi})"))
        return counts, sumsq


    def check_rebuild(self, M, P, begin, seed):
        """The oracle's rebuild of device master M (S fp32) against device
        params P (S bf16) over every element; rounding decisions are exact, so
        every pattern must be equal.  Returns the number of elements checked."""
        S = M.numel()
        for lo in range(0, S, self.chunk):
            hi = min(S, lo + self.chunk)
            n = hi - lo
            self.h["M" if self.master else "m"][:n].copy_(M[lo:hi])
            Mh = self._np("M" if self.master else "m", n)
            Ph = self._np("P", n)

            def one(r):
                Ph[r[0]:r[1]] = o.master_to_bf16_sr(Mh[r[0]:r[1]], begin + lo + r[0], seed)
            list(self.pool.map(one, parts(n, self.k)))
            self.d["P"][:n].copy_(self.h["P"][:n])
            got = P[lo:hi].view(torch.int16)
            nd = int((got != self.d["P"][:n]).sum())
            if nd:
                raise AssertionError(f"rebuild [{lo},{hi}): {nd} params differ from the oracle")
        return S


def assert_counts(counts, S, what):
    """The bf16 allowance: at most floor(1e-6 * S) elements one step apart."""
    allowed = int(BF16_FRACTION * S)
    assert counts["P"] <= allowed, f"{what}: {counts['P']} of {S} params one step apart (allowed {allowed})"
    frac = {k: v / S if S else 0.0 for k, v in counts.items()}
    return {"counts": counts, "fraction": frac, "allowed_bf16": allowed, "elements": S}


def snapshot(st):
    """Device copies of the state arrays a step overwrites."""
    return {k: (None if st.get(k) is None else st[k].clone()) for k in ("P", "M", "m", "v")}
