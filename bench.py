"""Benchmark of the PASA forward hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  * PASA prefill on the Qwen2-7B-shaped causal workload (batch 1, 28 query
    heads, 4 key/value heads, head_dim 128, seq 4096, bias 30 on q and k), and
  * PASA split-KV decode + combine on the decode workload (batch 64, one query
    token, 28/4 heads, head_dim 128, KV length 8192).
`value` is the prefill's TFLOP/s over algorithmic flops (4 * head_dim per
visible query/key pair), from HIP events recorded on the launch stream around
each prefill call inside the timed steps; the decode's achieved HBM GB/s is
reported beside it.  Inputs are resident in HBM before timing starts.

Also reported: relative RMSE of sampled output rows against the binary64
oracle, the naive fp16 kernel's inf/NaN count on the same input (the overflow
PASA avoids), and the oracle itself timed on this host's cores over a bounded
row sample (`cpu_baseline`).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0      # MI355X dense fp16 matrix peak
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E peak

# HBM traffic of the prefill kernel per launch, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs scaled by a copy-kernel calibration; None until measured for
# the current kernel.
PREFILL_TRAFFIC_BYTES = None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing and the sampled parity check")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times "
                         "(reference for the HBM byte counters), then exit")
    return ap.parse_args()


def calibrate_copy(mib):
    """A plain copy kernel of known size: reads and writes exactly mib MiB."""
    import torch
    src = torch.ones(mib * (1 << 20) // 2, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": mib * (1 << 20)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every workload here fits one MI355X); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import numpy as np
    import torch

    import precision_flashattention_numerics_amd as pasa
    import workloads as W
    from workloads.metrics import nonfinite, rel_rmse

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    wp = W.CONFIGS["c2"]
    wd = W.CONFIGS["c5"]
    log("generating inputs ...")
    qp, kp, vp = W.generate(wp)
    qd, kd, vd = W.generate(wd)
    tqp, tkp, tvp = (torch.from_numpy(x).cuda() for x in (qp, kp, vp))
    tqd, tkd, tvd = (torch.from_numpy(x).cuda() for x in (qd, kd, vd))
    op = torch.empty_like(tqp)
    lp = torch.empty((wp.batch, wp.heads_q, wp.seqlen_q), dtype=torch.float32, device="cuda")
    od = torch.empty_like(tqd)
    ld = torch.empty((wd.batch, wd.heads_q), dtype=torch.float32, device="cuda")
    ws, nsplit = pasa.decode_workspace(tqd, tkd)
    stream = torch.cuda.current_stream()

    def prefill():
        pasa.attn_fwd(tqp, tkp, tvp, causal=wp.causal, scale=wp.scale, out=op, lse=lp)

    def decode():
        pasa.attn_decode(tqd, tkd, tvd, scale=wd.scale, out=od, lse=ld, workspace=ws,
                         num_splits=nsplit)

    log(f"warmup {args.warmup} steps ...")
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        prefill()
        ev[i][1].record(stream)
        decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    dec_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]
    pre_avg = sum(pre_ms) / K
    dec_avg = sum(dec_ms) / K
    log(f"timed {K} steps: prefill {pre_avg:.4f} ms, decode {dec_avg:.4f} ms, wall {wall:.3f} s")

    flops = wp.flops()
    tflops = flops / (pre_avg * 1e-3) / 1e12
    dec_bytes = wd.io_bytes()
    dec_gbps = dec_bytes / (dec_avg * 1e-3) / 1e9

    # parity of the benchmarked outputs on sampled rows, and the naive kernel
    out = {}
    o_np = op.cpu().numpy()
    l_np = lp.cpu().numpy()
    od_np = od.cpu().numpy()
    out["pasa_nonfinite"] = nonfinite(o_np) + nonfinite(od_np)
    on, _ = pasa.naive_attn_fwd(tqp, tkp, tvp, causal=wp.causal, scale=wp.scale)
    torch.cuda.synchronize()
    out["naive_nonfinite"] = nonfinite(on.cpu().numpy())

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import attn_fp64, num_threads
        rng = np.random.default_rng(2024)
        total_rows = wp.batch * wp.heads_q * wp.seqlen_q

        def run_rows(rows):
            t = time.perf_counter()
            ro, rl = attn_fp64(qp, kp, vp, wp.scale, wp.causal, rows=rows)
            return ro, rl, time.perf_counter() - t

        def pairs(rows):
            i = rows % wp.seqlen_q
            return int(np.sum(np.minimum(i + 1 + wp.seqlen_kv - wp.seqlen_q, wp.seqlen_kv)))

        probe = rng.choice(total_rows, 256, replace=False)
        _, _, tp = run_rows(probe)
        rate = pairs(probe) / max(tp, 1e-6)          # visible pairs per second
        n_rows = int(min(total_rows, max(256, args.cpu_seconds * rate / (pairs(probe) / 256))))
        rows = np.sort(rng.choice(total_rows, n_rows, replace=False))
        ro, rl, tc = run_rows(rows)
        cpu_flops = 4 * wp.head_dim * pairs(rows)
        b, rem = np.divmod(rows, wp.heads_q * wp.seqlen_q)
        h, i = np.divmod(rem, wp.seqlen_q)
        out["rel_rmse_sampled"] = rel_rmse(o_np[b, i, h], ro)
        out["lse_max_abs_err_sampled"] = float(np.max(np.abs(l_np[b, h, i] - rl)))
        cpu = {"value": cpu_flops / tc / 1e12, "unit": "TFLOP/s", "cores": num_threads(),
               "kind": "oracle",
               "sample": f"{n_rows} random query rows of the prefill workload "
                         f"({cpu_flops:.3e} algorithmic flops, {tc:.1f} s, binary64, OpenMP)"}
        log(f"oracle: {n_rows} rows in {tc:.1f} s")

    line = {
        "metric": "PASA fwd TFLOP/s (fraction of fp16 MFMA peak); decode HBM GB/s; RMSE vs fp64",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "qwen2-7b-shaped causal prefill + split-KV decode",
                   "prefill": {"batch": wp.batch, "seq": wp.seqlen_q, "heads_q": wp.heads_q,
                               "heads_kv": wp.heads_kv, "head_dim": wp.head_dim,
                               "causal": wp.causal, "bias": 30},
                   "decode": {"batch": wd.batch, "kv_len": wd.seqlen_kv, "heads_q": wd.heads_q,
                              "heads_kv": wd.heads_kv, "head_dim": wd.head_dim,
                              "splits": nsplit, "bias": 30}},
        "prefill_ms": round(pre_avg, 5),
        "prefill_frac_of_peak": round(tflops / PEAK_FP16_TFLOPS, 4),
        "decode_ms": round(dec_avg, 5),
        "decode_GBps": round(dec_gbps, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP16_TFLOPS, 4),
                     "traffic": PREFILL_TRAFFIC_BYTES},
        "roofline_decode": {"bound": "hbm", "achieved": round(dec_gbps, 1),
                            "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                            "frac": round(dec_gbps / PEAK_HBM_GBPS, 4), "traffic": None},
        "cpu_baseline": cpu,
        **out,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
