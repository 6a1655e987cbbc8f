"""Benchmark of the mixed-precision AdamW step on one MI355X.

A step is one pass of the whole hot path over one shard: the grad norm
(stage 1 + stage 2 with clip scale) and the fused AdamW/SR update, both
through the C ABI on torch's current stream.  Inputs (state and a small pool
of pre-generated gradient buffers) are resident in HBM before timing starts.

Prints one JSON line: Gparams/s of the whole step, the HBM roofline of the
dominant kernel (the update, 28 algorithmic bytes per parameter), the CPU
oracle timed on a bounded sample of the same workload, and an achievable
ceiling: a kernel that moves the update's bytes with none of its arithmetic.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
UPDATE_BYTES = 28              # G 2 + m 4+4 + v 4+4 + M 4+4 + P 2 per parameter
UPDATE_BYTES_NO_MASTER = 22    # G 2 + P 2+2 + m 4+4 + v 4+4
NORM_BYTES = 2                 # G read once
REBUILD_BYTES = 6              # master_to_bf16_sr: M 4 read + P 2 written
TARGET_FRAC = 0.80             # the bar set for the step's kernels: 80% of HBM peak
METRIC = "optimizer Gparams/s per step + achieved HBM GB/s (% of peak), 1 MI355X"
WORKLOAD_NAMES = ("tiny_gpt_d32", "gpt2_124m", "gpt2_1p5b_shard", "stall16m", "llama7b")


def kernel_source_digest():
    path = os.path.join(ROOT, "bf16_numerics_amd", "csrc", "bfo_kernels.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_record(workload):
    """The committed counter summary of a workload, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"adamw_update_{workload}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("kernel_source_sha256_16") == kernel_source_digest() else None


def measured_traffic(workload):
    """HBM bytes per update launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    rec = traffic_record(workload)
    return rec.get("bytes_per_launch") if rec else None


def measured_rebuild_traffic(workload):
    """HBM bytes per rebuild launch from the same summary, or None."""
    rec = traffic_record(workload)
    return (rec.get("rebuild") or {}).get("bytes_per_launch") if rec else None


def cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_threads():
    """Host threads this process may use (the CPU share, not the machine)."""
    k = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(k, int(cap))) if cap and cap.isdigit() else k


def cpu_baseline(torch, w, st, begin, target_s, rounding_sr=True):
    """The oracle, as it stands, on a contiguous slice of the same shard: grad
    norm + the timed AdamW variant per step, first on one thread, then on K threads
    (a static contiguous partition of the slice; each thread calls the oracle
    on its part, and the per-part sums of squares are added in part order
    before the clip scale).  The oracle's C functions run without the GIL."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle as o
    from bf16_numerics_amd import workloads as W

    count = min(1 << 23, st["P"].numel())
    h = {k: (None if t is None else W.bf16_bits_numpy(torch, t[:count]).copy() if t.dtype == torch.bfloat16
             else t[:count].cpu().numpy().copy()) for k, t in st.items()}
    rounding = o.ROUND_SR if rounding_sr else o.ROUND_RNE
    sl = (lambda a, r: None if a is None else a[r[0]:r[1]])
    tbl = o.table(w.entries())
    hp = o.hparams(w.hparams.lr, w.hparams.beta1, w.hparams.beta2, w.hparams.eps,
                   w.hparams.weight_decay, w.hparams.bias_correction)
    max_norm = w.hparams.max_norm

    def run(parts, pool, budget, first_step):
        steps, t0 = 0, time.perf_counter()
        while True:
            steps += 1
            t = first_step + steps
            sums = list(pool.map(lambda r: o.grad_norm(h["G"][r[0]:r[1]], max_norm)[0], parts))
            _, scale = o.norm_from_sumsq(sum(sums), max_norm)
            list(pool.map(lambda r: o.adamw_step(tbl, begin + r[0], h["P"][r[0]:r[1]], h["G"][r[0]:r[1]],
                                                 sl(h["M"], r), h["m"][r[0]:r[1]], h["v"][r[0]:r[1]], hp,
                                                 scale, t, (1337 << 32) | t, rounding), parts))
            el = time.perf_counter() - t0
            if el >= budget or steps >= 4096:
                return steps, el

    with ThreadPoolExecutor(1) as pool:
        s1, el1 = run([(0, count)], pool, target_s / 2, 0)
    k = cpu_threads()
    cuts = [count * i // k // 8 * 8 for i in range(k)] + [count]
    with ThreadPoolExecutor(k) as pool:
        sk, elk = run(list(zip(cuts[:-1], cuts[1:])), pool, target_s / 2, s1)
    one = count * s1 / el1 / 1e9
    return {"value": count * sk / elk / 1e9, "unit": "Gparams/s", "cores": k, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"contiguous {count}-element slice of the {w.name} shard, grad norm + AdamW update "
                      f"({'master' if h['M'] is not None else 'no master'}, {'SR' if rounding_sr else 'RNE'}) "
                      f"per step: {sk} steps in {elk:.1f} s on {k} threads (static contiguous partition); "
                      f"before that {s1} steps in {el1:.1f} s on 1 thread",
            "single_thread_value": one}


def checkpoint_rate(torch, bfo, T, P, M, m, v, seed, rounding, directory):
    """Save this rank's optimizer state, mark it done, find it as the latest,
    load it into fresh buffers (with a master, the params are rebuilt from it
    during the load) and check every byte; time save and load."""
    import shutil

    step_no = 1
    os.makedirs(directory, exist_ok=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bfo.checkpoint_save(directory, T, m, v, step_no, seed, master=M, params=None if M is not None else P,
                        rounding=rounding)
    bfo.checkpoint_done(directory, step_no)
    t_save = time.perf_counter() - t0
    assert bfo.checkpoint_latest(directory) == step_no
    m2, v2 = torch.empty_like(m), torch.empty_like(v)
    M2 = torch.empty_like(M) if M is not None else None
    # the shard's positions of P2 start as a NaN pattern; the load must fill them
    P2 = P.clone()
    if T.layout == bfo.LAYOUT_PER_TENSOR:
        P2.view(torch.int16)[torch.from_numpy(T.global_index().astype("int64")).to(P.device)] = 0x7FA5
    else:
        P2.view(torch.int16).fill_(0x7FA5)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    got_seed = bfo.checkpoint_load(directory, step_no, T, m2, v2, master=M2, params=P2)
    torch.cuda.synchronize()
    t_load = time.perf_counter() - t0
    same = got_seed == seed and all(torch.equal(a.view(torch.int32), b.view(torch.int32))
                                   for a, b in ((m, m2), (v, v2)) + (((M, M2),) if M is not None else ()))
    same = same and torch.equal(P.view(torch.int16), P2.view(torch.int16))
    nbytes = sum(os.path.getsize(os.path.join(directory, f)) for f in os.listdir(directory))
    shutil.rmtree(directory, ignore_errors=True)
    del m2, v2, M2, P2
    return {"bytes": nbytes, "save_s": round(t_save, 3), "load_s": round(t_load, 3),
            "save_GBps": round(nbytes / t_save / 1e9, 2), "load_GBps": round(nbytes / t_load / 1e9, 2),
            "round_trip_bit_exact": bool(same), "dir": directory}


def rebuild_rate(torch, bfo, stream, T, M, P, seed, launches):
    """master_to_bf16_sr (the resume-time rebuild, 6 B per parameter) timed per
    launch with HIP events on the launch stream.  It rewrites P from the
    master with the last update's seed (after an SR update, the same bits)."""
    for _ in range(2):
        bfo.master_to_bf16_sr(T, M, P, seed)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for a, z in evs:
        a.record(stream)
        bfo.master_to_bf16_sr(T, M, P, seed)
        z.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(z) for a, z in evs) / launches
    gbs = REBUILD_BYTES * M.numel() / (ms * 1e-3) / 1e9
    return {"kernel": "masterToBf16Kernel", "achieved": round(gbs, 1), "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "ms_avg": round(ms, 5),
            "algorithmic_bytes_per_launch": REBUILD_BYTES * M.numel()}


def settle(torch, bfo, P, G, M, m, v, count, seconds):
    """Sustained read-only passes over the step's arrays for `seconds` before
    any step runs.  Measured on MI355X: from a standing start the 7B step runs
    32.2 ms for its first 20 steps, 31.9 for the next 20 and 31.56-31.62 from
    then on (the 1.5B shard: 0.962 ms over its first 200 steps, 0.932 after);
    two seconds of these reads first (or of the update's own loads and stores)
    take the ramp away, an unrelated fill only part of it.  Reads only
    (bfo_stream_mix READS): no array changes.  P and G views start on 16-byte
    boundaries (the kernel's requirement), the state arrays at their start.
    Returns (passes, seconds spent)."""
    if seconds <= 0 or count < 16:
        return 0, 0.0
    def aligned(t):
        k = (-t.data_ptr() % 16) // t.element_size()
        return t[k:]
    Pa, Ga = aligned(P), aligned(G)
    n = min(count, Pa.numel(), Ga.numel()) // 8 * 8
    passes, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            bfo.stream_mix(Pa[:n], Ga[:n], None if M is None else M[:n], m[:n], v[:n], 0, bfo.MIX_READS)
            passes += 1
        torch.cuda.synchronize()
    return passes, round(time.perf_counter() - t0, 3)


def stream_ceiling(torch, bfo, stream, P, G, M, m, v, launches, update_gbs, norm=None, grads=None,
                   ms_step=None):
    """Achievable bandwidth for the update's own traffic on this device: the
    library's stream-mix kernel (the update's bytes per element -- 14 read and
    14 written with a master, 12 and 10 without -- in its vector and
    workgroup plan, no arithmetic; key 0 leaves m, v and the master
    unchanged), timed per launch with HIP events on the launch stream, as the
    update is.  Then the same reads alone and the same writes alone (which
    overwrite the state, so they run last): `serial_bound` is the rate the
    mix would reach if HBM served its reads and its writes one after the
    other at those rates.  With `norm` (enqueues the real grad norm of
    grads[k]) it also times K steps of norm + stream mix over the same grads,
    back to back like the timed region: the step's own ceiling."""
    def per_launch(mode):
        # events recorded once beforehand and two untimed launches ahead, so
        # that the host is ahead of the GPU when the timed intervals start
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(launches)]
        for a, z in evs:
            a.record(stream)
            z.record(stream)
        for _ in range(2):
            bfo.stream_mix(P, G, M, m, v, 0, mode)
        for a, z in evs:
            a.record(stream)
            bfo.stream_mix(P, G, M, m, v, 0, mode)
            z.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(z) for a, z in evs) / launches

    ms = per_launch(bfo.MIX_BOTH)
    rd_b, wr_b = (14, 14) if M is not None else (12, 10)
    per = rd_b + wr_b
    gbs = per * m.numel() / (ms * 1e-3) / 1e9
    out = {"kernel": "streamMixKernel (update traffic, no arithmetic)", "achieved": round(gbs, 1),
           "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "ms_avg": round(ms, 5),
           "update_over_ceiling": round(update_gbs / gbs, 4)}
    if norm is not None:
        n = m.numel()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for k in range(launches):
            norm(k)
            bfo.stream_mix(P, grads[k % len(grads)][:n], M, m, v, 0)
        z.record(stream)
        torch.cuda.synchronize()
        step_ms = a.elapsed_time(z) / launches
        out["step_ms"] = round(step_ms, 5)
        out["step_over_ceiling"] = round(step_ms / ms_step, 4)
    ms_r = per_launch(bfo.MIX_READS)
    ms_w = per_launch(bfo.MIX_WRITES)          # overwrites m, v, the master and the params
    r_gbs = rd_b * m.numel() / (ms_r * 1e-3) / 1e9
    w_gbs = wr_b * m.numel() / (ms_w * 1e-3) / 1e9
    bound = per / (rd_b / r_gbs + wr_b / w_gbs)
    out["reads_only"] = {"GBps": round(r_gbs, 1), "frac": round(r_gbs / HBM_PEAK_GBS, 4), "ms_avg": round(ms_r, 5)}
    out["writes_only"] = {"GBps": round(w_gbs, 1), "frac": round(w_gbs / HBM_PEAK_GBS, 4), "ms_avg": round(ms_w, 5)}
    out["serial_bound"] = {"GBps": round(bound, 1), "frac": round(bound / HBM_PEAK_GBS, 4),
                           "mix_over_bound": round(gbs / bound, 4), "update_over_bound": round(update_gbs / bound, 4)}
    return out


ARENA_FRAC = 0.8               # spread placement: the arena covers this share of device memory


def state_arrays(torch, bfo, dev, placement, n, g_len, n_grads, S, master, reserve):
    """The step's device arrays: P (n bf16), G (n_grads * g_len bf16), M (S
    fp32, or None), m and v (S fp32).

    "packed": one allocation per array.  "spread": one arena covering most of
    device memory, as a framework that preallocates its memory pool holds it,
    with the five groups starting on successive 16 GiB boundaries
    (bfo_spread_layout) so that at any element index the arrays lie in
    different 16 GiB regions; the rest of the arena is what such a framework
    would give its other buffers.  `reserve` bytes stay outside the arena for
    input generation."""
    specs = [("P", n, torch.bfloat16, 2), ("G", n_grads * g_len, torch.bfloat16, 2)]
    specs += [("M", S, torch.float32, 4)] if master else []
    specs += [("m", S, torch.float32, 4), ("v", S, torch.float32, 4)]
    out = {"M": None, "arena_bytes": 0}
    if placement == "packed":
        for name, count, dt, _ in specs:
            out[name] = torch.empty(count, dtype=dt, device=dev)
        return out
    offsets, needed = bfo.spread_layout([count * es for _, count, _, es in specs])
    free, total_mem = torch.cuda.mem_get_info(dev)
    size = max(needed, min(int(ARENA_FRAC * total_mem), free - reserve)) // 4096 * 4096
    arena = torch.empty(size, dtype=torch.uint8, device=dev)
    for (name, count, dt, es), off in zip(specs, offsets):
        out[name] = arena[off:off + count * es].view(dt)
    out["arena_bytes"] = size
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-seconds", type=float, default=2.0,
                    help="read-only passes over the step's arrays before the warm-up steps, so that the "
                         "timed steps see the GPU's steady state (0: none)")
    ap.add_argument("--workload", default="llama7b", choices=WORKLOAD_NAMES,
                    help="llama7b (default: the largest configuration that fits one GPU, 6.74e9 parameters "
                         "in one shard), gpt2_1p5b_shard (rank 1 of 8 of the 1.5B model), gpt2_124m, "
                         "stall16m, tiny_gpt_d32")
    ap.add_argument("--grad-pool", type=int, default=4)
    ap.add_argument("--layout", choices=("flat", "per_tensor"), default="flat",
                    help="ZeRO-1 shard layout: contiguous range, or 1/N of every tensor")
    ap.add_argument("--rank", type=int, default=None,
                    help="ZeRO-1 rank whose shard is timed (default: the workload's own, rank 1 of 8 for the "
                         "1.5B shard)")
    ap.add_argument("--pad", type=int, default=0,
                    help="append a 1-D tensor of this many elements (e.g. 8 makes n/8 odd: misaligned shards)")
    ap.add_argument("--no-master", action="store_true",
                    help="time the no-master update (old weights read from the bf16 params, 22 B/param)")
    ap.add_argument("--rounding", choices=("sr", "rne"), default="sr",
                    help="bf16 write-back: stochastic (default) or round to nearest even")
    ap.add_argument("--step-control", action="store_true",
                    help="per-step learning rate from a cosine schedule (host) and the device outlier "
                         "detector (window 128, z > 6 skips) between the norm and the update")
    ap.add_argument("--checkpoint-dir", default=None,
                    help="after timing, save this rank's state there, load it back, check it bit for bit, "
                         "time both and delete the files")
    ap.add_argument("--graph", action="store_true",
                    help="record the step once per grads buffer as a HIP graph (norm, outlier update, scheduled "
                         "update, cursor advance) and time graph replays")
    ap.add_argument("--one-call", action="store_true",
                    help="each step is one adamw_sr_step_with_norm call (norm, clip and update; a single kernel "
                         "launch for shards of at most 65,536 elements) instead of grad_global_norm + adamw_sr_step")
    ap.add_argument("--placement", choices=("spread", "packed"), default="spread",
                    help="spread: params, grads, master, m and v carved from one arena covering most of device "
                         "memory, each starting on its own 16 GiB boundary (bfo_spread_layout); packed: one "
                         "allocation per array")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the same-traffic streaming kernel timed after the step (achievable ceiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, copy 2 GiB -> 2 GiB three times (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the step is measured on one "
              "GPU's ZeRO-1 shard; no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)

    if args.one_call and (args.graph or args.step_control):
        ap.error("--one-call takes the clip scale from its own norm: no --graph or --step-control")

    import torch
    from bf16_numerics_amd import binding as bfo
    from bf16_numerics_amd import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[args.workload]()
    if args.pad:
        w.tensors = list(w.tensors) + [("pad", (args.pad,))]
    if args.rank is not None:
        if not 0 <= args.rank < w.world:
            ap.error(f"--rank must be in [0, {w.world}) for {w.name}")
        w.rank = args.rank
    layout = bfo.LAYOUT_PER_TENSOR if args.layout == "per_tensor" else bfo.LAYOUT_FLAT
    bfo.Table(w.entries(), w.world, w.rank, layout=layout).close()     # first call pays library start-up
    t0 = time.perf_counter()
    T = bfo.Table(w.entries(), w.world, w.rank, layout=layout)      # host plan + one upload, once per table
    table_ms = (time.perf_counter() - t0) * 1e3
    S = T.size

    # Device arrays: the full-length bf16 params (ZeRO-1: every rank holds
    # them), the gradient buffers, and the shard's fp32 master, m and v.
    per_tensor = layout == bfo.LAYOUT_PER_TENSOR
    g_len, g_begin = (w.n, 0) if per_tensor else (S, T.begin)
    n_grads = max(1, args.grad_pool)
    g_stride = (g_len + 127) // 128 * 128          # each gradient buffer starts on a 256-byte line
    reserve = (16 << 30) + g_len * 6 + (S * 8 if per_tensor else 0)   # grads generation, index map
    arrays = state_arrays(torch, bfo, dev, args.placement, w.n, g_stride, n_grads, S, not args.no_master,
                          reserve)
    P_full, grads_all, M, m, v = (arrays[k] for k in ("P", "G", "M", "m", "v"))
    if per_tensor:
        # llm.c-style ZeRO-1: this rank's 1/N of every tensor.
        P = P_full
        W.init_params_into(torch, w, 0, P)
        if M is not None:
            M.copy_(P[torch.from_numpy(T.global_index().astype("int64")).to(dev)].to(torch.float32))
        b, e = 0, S
    else:
        # Contiguous ZeRO-1 layout: the shard [b, e) of the params, the rest shard-local.
        b, e = T.begin, T.end
        P = P_full[b:e]
        W.init_params_into(torch, w, b, P, M)
    m.zero_()
    v.zero_()
    pool = [grads_all[k * g_stride:k * g_stride + g_len] for k in range(n_grads)]
    for k, G in enumerate(pool):
        W.fill_grads(torch, w, G, g_begin, k + 1)
    torch.cuda.empty_cache()
    res = bfo.new_norm_result(dev)
    norm_ws = bfo.new_norm_workspace(T)
    hp = bfo.AdamwHParams(w.hparams.lr, w.hparams.beta1, w.hparams.beta2, w.hparams.eps,
                          w.hparams.weight_decay, 1)
    stream = torch.cuda.current_stream(dev)
    rounding = bfo.ROUND_RNE if args.rounding == "rne" else bfo.ROUND_SR
    upd_bytes = UPDATE_BYTES_NO_MASTER if args.no_master else UPDATE_BYTES
    step_bytes = upd_bytes + NORM_BYTES
    if args.one_call:
        upd_bytes = step_bytes           # the timed call reads the grads for the norm too
    variant = ("no-master" if args.no_master else "master") + "," + args.rounding.upper()
    last_t = args.warmup + 2 * args.steps + 1   # warm-up, timed, lead, event-bracketed steps
    outlier, hps = None, None
    if args.step_control:
        # Cosine schedule over every step this run makes; the detector's window
        # is filled beforehand with the norms of the gradient pool in the order
        # the steps use them, so that the timed steps pay for the full z-score
        # pass (an identical value throughout would give a zero variance).
        hps = [None] + [bfo.AdamwHParams(bfo.lr_at(bfo.LR_COSINE, t - 1, 10, last_t, w.hparams.lr, 0.1),
                                         w.hparams.beta1, w.hparams.beta2, w.hparams.eps,
                                         w.hparams.weight_decay, 1) for t in range(1, last_t + 1)]
        outlier = bfo.Outlier(window=128, threshold=6.0, device=dev)
        for k in range(128):
            bfo.grad_global_norm(T, pool[k % len(pool)], res, w.hparams.max_norm)
            outlier.update(bfo.norm_ptr(res))
    skips = torch.zeros(1, dtype=torch.int64, device=dev)
    sched = cursor = None
    if args.graph:
        # Per-step scalars for every step this run makes (the check pass
        # included), read on the device through a cursor each update advances.
        n_sched = last_t + args.steps
        sched = bfo.step_schedule(hp, [(t, hps[min(t, last_t)].lr if hps else hp.lr, (1337 << 32) | t)
                                       for t in range(1, n_sched + 1)], dev)
        cursor = torch.zeros(1, dtype=torch.int64, device=dev)

    def update(t, G, skip):
        if args.graph:
            bfo.adamw_sr_step_scheduled(T, P, G, M, m, v, hp, sched, cursor, scale=res, rounding=rounding,
                                        skip=skip)
        else:
            bfo.adamw_sr_step(T, P, G, M, m, v, hps[t] if hps else hp, t, (1337 << 32) | t, scale=res,
                              rounding=rounding, skip=skip)

    def record_step(G):
        bfo.grad_global_norm(T, G, res, w.hparams.max_norm, workspace=norm_ws)
        return outlier.update(bfo.norm_ptr(res)).skip if outlier is not None else None

    graphs = []
    if args.graph:
        torch.cuda.synchronize()
        for G in pool:                       # one graph per grads buffer; nothing else differs
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                update(None, G, record_step(G))
                bfo.cursor_advance(cursor)
            graphs.append(g)
        torch.cuda.synchronize()

    def step(t, ev=None):
        G = pool[(t - 1) % len(pool)]
        if graphs and ev is None:
            graphs[(t - 1) % len(pool)].replay()
            return
        if ev is not None:
            ev[2].record(stream)
        if args.one_call:
            if ev is not None:
                ev[0].record(stream)
            bfo.adamw_sr_step_with_norm(T, P, G, M, m, v, hp, t, (1337 << 32) | t, res, w.hparams.max_norm,
                                        rounding=rounding, workspace=norm_ws)
            if ev is not None:
                ev[1].record(stream)
            return
        skip = record_step(G)
        if ev is not None:
            ev[0].record(stream)
        update(t, G, skip)
        if ev is not None:
            ev[1].record(stream)
        if args.graph:
            bfo.cursor_advance(cursor)

    settle_passes, settle_s = settle(torch, bfo, P, pool[0], M, m, v, S, args.settle_seconds)
    for t in range(1, args.warmup + 1):
        step(t)
    torch.cuda.synchronize()

    # Timed region: exactly K steps, nothing but the optimizer's own launches.
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_begin.record(stream)
    for k in range(args.steps):
        step(args.warmup + 1 + k)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step_ev = t_begin.elapsed_time(t_end) / args.steps
    ms_step = max(wall * 1e3 / args.steps, ms_step_ev)

    # Per-launch duration of the dominant kernel (the update): K more steps with
    # HIP events recorded on the launch stream around each update call.  Kept
    # out of the region above because each event adds a few microseconds of gap.
    # The events are created (first record) beforehand and an untimed step
    # leads the pass, so the host is ahead of the GPU from the first interval
    # on and no host delay can fall inside one.
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    for tpl in evs:
        for ev_k in tpl:
            ev_k.record(stream)
    t_lead = args.warmup + args.steps + 1
    step(t_lead)
    for k in range(args.steps):
        step(t_lead + 1 + k, evs[k])
    torch.cuda.synchronize()
    if outlier is not None:
        # Evidence that no timed step was skipped: the event-bracketed pass
        # uses the same grads in the same order, so count its skips.
        for k in range(args.steps):
            step(t_lead + 1 + k)
            skips.add_(outlier.skip)
        torch.cuda.synchronize()
    upd_ms = [a.elapsed_time(z) for a, z, _ in evs]
    upd_avg = sum(upd_ms) / len(upd_ms)
    upd_median = statistics.median(upd_ms)
    norm_ms = [s0.elapsed_time(a) for a, _, s0 in evs]
    step_ev_ms = sorted(s0.elapsed_time(z) for _, z, s0 in evs)
    gparams = S / (ms_step * 1e-3) / 1e9
    step_gbs = step_bytes * S / (ms_step * 1e-3) / 1e9
    achieved = upd_bytes * S / (upd_avg * 1e-3) / 1e9
    default_variant = (args.layout == "flat" and not args.pad and not args.no_master and args.rounding == "sr"
                       and args.rank is None and not args.graph and args.placement == "spread"
                       and not args.one_call)
    traffic = measured_traffic(w.name) if default_variant else None
    last_seed = (1337 << 32) | last_t      # seed of the last update (the check pass repeats the same t)
    sumsq, norm, scale = bfo.read_norm_result(res)

    out = {
        "metric": METRIC,
        "value": round(gparams, 3),
        "unit": "Gparams/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name + (f"+pad{args.pad}" if args.pad else ""), "n_total": w.n,
                   "layout": args.layout, "shard": [b, e], "shard_elems": S,
                   "world": w.world, "rank": w.rank, "tensors": len(w.tensors),
                   "grad_pool": len(pool), "bytes_per_param_step": step_bytes,
                   "update": variant,
                   "launch": "graph" if args.graph else ("one-call" if args.one_call else "stream"),
                   "placement": args.placement, "arena_bytes": arrays["arena_bytes"]},
        "hbm_gbs_step": round(step_gbs, 1),
        "hbm_frac_step": round(step_gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm",
                     "kernel": (f"adamw_sr_step_with_norm<{variant}> (norm + update"
                                f"{', one launch' if S <= 65536 else ''})") if args.one_call else
                               f"adamwTileKernel<{variant}{',scheduled' if args.graph else ''}>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "target_frac": TARGET_FRAC,
                     "shortfall_vs_target": round(TARGET_FRAC - achieved / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": upd_bytes * S,
                     "update_ms_avg": round(upd_avg, 5), "update_ms_median": round(upd_median, 5)},
        "settle": {"seconds": settle_s, "passes": settle_passes, "kernel": "streamMixKernel (reads only)"},
        "timed_region_ms_per_step": {"events": round(ms_step_ev, 5), "wall": round(wall * 1e3 / args.steps, 5)},
        "step_ms_events": {"mean": round(sum(step_ev_ms) / len(step_ev_ms), 5),
                           "median": round(statistics.median(step_ev_ms), 5),
                           "min": round(step_ev_ms[0], 5), "max": round(step_ev_ms[-1], 5),
                           "norm_mean": round(sum(norm_ms) / len(norm_ms), 5)},
        "last_norm": {"norm": norm, "scale": scale},
        "table_ms": round(table_ms, 3),
    }
    if outlier is not None:
        out["step_control"] = {"lr": "cosine, 10 warm-up steps, floor 0.1", "outlier_window": 128,
                               "z_threshold": 6.0, "last_z": float(outlier.z.item()),
                               "skipped_in_check_pass": int(skips.item())}
    if args.checkpoint_dir:
        out["checkpoint"] = checkpoint_rate(torch, bfo, T, P, M, m, v, last_seed, rounding, args.checkpoint_dir)
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
        del src, dst
    if M is not None:
        out["rebuild"] = rebuild_rate(torch, bfo, stream, T, M, P, last_seed, args.steps)
        out["rebuild"]["traffic"] = measured_rebuild_traffic(w.name) if default_variant else None
    if not args.no_cpu_baseline and args.layout == "flat":
        st = {"P": P, "G": pool[0], "M": M, "m": m, "v": v}
        out["cpu_baseline"] = cpu_baseline(torch, w, st, b, args.cpu_seconds, args.rounding == "sr")
    if not args.no_ceiling and (P.data_ptr() % 16 or pool[0].data_ptr() % 16):
        # the streaming kernel moves 16-byte vectors only
        out["ceiling"] = {"skipped": "params or grads not 16-byte aligned (the update takes its per-element "
                                     "path for them)"}
    elif not args.no_ceiling:
        out["ceiling"] = stream_ceiling(
            torch, bfo, stream, P[:S], pool[0][:S], M, m, v, args.steps, achieved,
            norm=lambda k: bfo.grad_global_norm(T, pool[k % len(pool)], res, w.hparams.max_norm),
            grads=pool, ms_step=ms_step)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
