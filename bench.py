"""Benchmark of the mixed-precision AdamW step on one MI355X.

A step is one pass of the whole hot path over one shard: the grad norm
(stage 1 + stage 2 with clip scale) and the fused AdamW/SR update, both
through the C ABI on torch's current stream.  Inputs (state and a small pool
of pre-generated gradient buffers) are resident in HBM before timing starts.

Prints one JSON line: Gparams/s of the whole step, the HBM roofline of the
dominant kernel (the update, 28 algorithmic bytes per parameter), and the CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
UPDATE_BYTES = 28              # G 2 + m 4+4 + v 4+4 + M 4+4 + P 2 per parameter
NORM_BYTES = 2                 # G read once
METRIC = "optimizer Gparams/s per step + achieved HBM GB/s (% of peak), 1 MI355X"


def kernel_source_digest():
    path = os.path.join(ROOT, "bf16_numerics_amd", "csrc", "bfo_kernels.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per update launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"adamw_update_{workload}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_digest():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(torch, w, st, begin, target_s):
    """The oracle, as it stands, on a contiguous slice of the same shard:
    grad norm + AdamW/SR update per step, one thread."""
    import numpy as np
    import oracle as o
    from bf16_numerics_amd import workloads as W

    count = min(1 << 23, st["P"].numel())
    h = {k: (W.bf16_bits_numpy(torch, t[:count]).copy() if t.dtype == torch.bfloat16
             else t[:count].cpu().numpy().copy()) for k, t in st.items()}
    tbl = o.table(w.entries())
    hp = o.hparams(w.hparams.lr, w.hparams.beta1, w.hparams.beta2, w.hparams.eps,
                   w.hparams.weight_decay, w.hparams.bias_correction)
    steps = 0
    t0 = time.perf_counter()
    while True:
        steps += 1
        _, _, scale = o.grad_norm(h["G"], w.hparams.max_norm)
        o.adamw_step(tbl, begin, h["P"], h["G"], h["M"], h["m"], h["v"], hp, scale, steps,
                     (1337 << 32) | steps, o.ROUND_SR)
        el = time.perf_counter() - t0
        if el >= target_s or steps >= 64:
            break
    return {"value": count * steps / el / 1e9, "unit": "Gparams/s", "cores": 1, "kind": "oracle",
            "sample": f"contiguous {count}-element slice of the {w.name} shard, {steps} steps of "
                      f"grad norm + AdamW/SR update, {el:.1f} s single-threaded"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2_1p5b_shard")
    ap.add_argument("--grad-pool", type=int, default=4)
    ap.add_argument("--layout", choices=("flat", "per_tensor"), default="flat",
                    help="ZeRO-1 shard layout: contiguous range, or 1/N of every tensor")
    ap.add_argument("--pad", type=int, default=0,
                    help="append a 1-D tensor of this many elements (e.g. 8 makes n/8 odd: misaligned shards)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, copy 2 GiB -> 2 GiB three times (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the step is measured on one "
              "GPU's ZeRO-1 shard; no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)

    import torch
    from bf16_numerics_amd import binding as bfo
    from bf16_numerics_amd import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[args.workload]()
    if args.pad:
        w.tensors = list(w.tensors) + [("pad", (args.pad,))]
    layout = bfo.LAYOUT_PER_TENSOR if args.layout == "per_tensor" else bfo.LAYOUT_FLAT
    T = bfo.Table(w.entries(), w.world, w.rank, layout=layout)
    S = T.size

    if layout == bfo.LAYOUT_PER_TENSOR:
        # llm.c-style ZeRO-1: full-length bf16 params and grads, shard-local
        # fp32 master/m/v for this rank's 1/N of every tensor.
        P, M_full, _, _ = W.init_state(torch, w, 0, w.n, dev)
        gi = torch.from_numpy(T.global_index().astype("int64")).to(dev)
        M = M_full[gi].clone()
        del M_full, gi
        m = torch.zeros(S, dtype=torch.float32, device=dev)
        v = torch.zeros(S, dtype=torch.float32, device=dev)
        b, e = 0, S
        g_len, g_begin = w.n, 0
    else:
        # Contiguous ZeRO-1 layout: full-length bf16 params, shard-local rest.
        b, e = T.begin, T.end
        P_full = torch.empty(w.n if w.world > 1 else 0, dtype=torch.bfloat16, device=dev)
        P, M, m, v = W.init_state(torch, w, b, e, dev)
        if w.world > 1:
            P_full[b:e] = P
            del P
            P = P_full[b:e]
        g_len, g_begin = S, b
    pool = []
    for k in range(max(1, args.grad_pool)):
        G = torch.empty(g_len, dtype=torch.bfloat16, device=dev)
        W.fill_grads(torch, w, G, g_begin, k + 1)
        pool.append(G)
    res = bfo.new_norm_result(dev)
    hp = bfo.AdamwHParams(w.hparams.lr, w.hparams.beta1, w.hparams.beta2, w.hparams.eps,
                          w.hparams.weight_decay, 1)
    stream = torch.cuda.current_stream(dev)

    def step(t, ev=None):
        G = pool[(t - 1) % len(pool)]
        bfo.grad_global_norm(T, G, res, w.hparams.max_norm)
        if ev is not None:
            ev[0].record(stream)
        bfo.adamw_sr_step(T, P, G, M, m, v, hp, t, (1337 << 32) | t, scale=res)
        if ev is not None:
            ev[1].record(stream)

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
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for k in range(args.steps):
        step(args.warmup + args.steps + 1 + k, evs[k])
    torch.cuda.synchronize()
    upd_ms = [a.elapsed_time(z) for a, z in evs]
    upd_avg = sum(upd_ms) / len(upd_ms)
    gparams = S / (ms_step * 1e-3) / 1e9
    step_gbs = (UPDATE_BYTES + NORM_BYTES) * S / (ms_step * 1e-3) / 1e9
    achieved = UPDATE_BYTES * S / (upd_avg * 1e-3) / 1e9
    traffic = measured_traffic(w.name) if (args.layout == "flat" and not args.pad) else None
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
                   "grad_pool": len(pool), "bytes_per_param_step": UPDATE_BYTES + NORM_BYTES},
        "hbm_gbs_step": round(step_gbs, 1),
        "hbm_frac_step": round(step_gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "adamwTileKernel<master,SR>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": UPDATE_BYTES * S,
                     "update_ms_avg": round(upd_avg, 5)},
        "last_norm": {"norm": norm, "scale": scale},
    }
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
        del src, dst
    if not args.no_cpu_baseline and args.layout == "flat":
        st = {"P": P, "G": pool[0], "M": M, "m": m, "v": v}
        out["cpu_baseline"] = cpu_baseline(torch, w, st, b, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
