"""Benchmark of the PASA forward hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  * PASA prefill on the Qwen2-7B-shaped causal workload (batch 1, 28 query
    heads, 4 key/value heads, head_dim 128, seq 4096, bias 30 on q and k), and
  * PASA split-KV decode + combine on the decode workload (batch 64, one query
    token, 28/4 heads, head_dim 128, KV length 8192).
`value` is the prefill's TFLOP/s over algorithmic flops (4 * head_dim per
visible query/key pair), from HIP events recorded on the launch stream around
the prefill launches inside the timed steps; the decode's achieved HBM GB/s is
reported beside it.  Inputs are resident in HBM before timing starts, and the
timed steps follow back-to-back warmup steps -- at least --warmup of them and
at least --warm-seconds of wall time, both counted in the line: the GPU raises
its clock only after tens of milliseconds of sustained load, so a burst timed
right after an idle spell measures the clock ramp instead of the kernel (that
cold figure is reported beside it as prefill_ms_cold).

Also reported: the roofline fractions against the published peaks and against
peaks measured on this GPU by two microbenchmarks (back-to-back fp16 matrix
products; a streaming HBM read); the other prefill workloads (single head,
Stable-Video-Diffusion-shaped resonance, 32K long context) with the naive fp16
kernel's overflow on each; relative RMSE of sampled output rows against the
binary64 oracle; and the oracle itself timed on this host's cores over a
bounded row sample (`cpu_baseline`).

`--profile-config c3|c4` runs only that prefill workload, `--profile-config
c5paged` only the decode over the shuffled 64-key-page cache (both for
rocprofv3), and `--summarize-profile DIR SET` writes the text summaries under
profiles/.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2500.0      # MI355X dense fp16 matrix peak (published)
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E peak (published)

PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "precision_flashattention_numerics_amd", "csrc")
PEAK_LIB = os.path.join(ROOT, "precision_flashattention_numerics_amd", "peak", "libpasa_peak.so")

# Kernel symbols (substrings) of the profiled launches:
# fwd_kernel<head_dim, causal, variant (0 PASA, 1 strict, 2 naive, 3 e4m3), key split>
K_PREFILL = "fwd_kernelILi128ELb1ELi0ELb0E"  # PASA prefill, head_dim 128, causal
K_STRICT = "fwd_kernelILi128ELb1ELi1ELb0E"   # strict PASA prefill, same shape
K_NAIVE = "fwd_kernelILi128ELb1ELi2ELb0E"    # naive fp16 prefill, same shape
K_C3 = "fwd_kernelILi64ELb0ELi0ELb1E"        # PASA prefill, head_dim 64, non-causal, key split
K_SPLIT = "decode_split_kernelILi128ELb0E"   # decode split, head_dim 128, contiguous cache
K_SPLIT_PAGED = "decode_split_kernelILi128ELb1E"   # decode split, head_dim 128, paged cache
K_COMBINE = "decode_combine_kernel"

# Profile sets: which bench invocation each rocprofv3 run wraps, and the file
# name stem of its summaries under profiles/.
PROFILE_SETS = {
    "qwen2": dict(
        stem="pasa_prefill_qwen2shape_s4096_decode_b64_kv8192", config="c2",
        trace_args="--steps 20 --warmup 5 --no-cpu-baseline --no-other-configs",
        pmc_args="--steps 3 --warmup 1 --warm-seconds 0 --no-cpu-baseline --no-other-configs",
        prefill=K_PREFILL, decode=K_SPLIT),
    "svd": dict(
        stem="pasa_prefill_svdshape_b2_s9216_d64", config="c3",
        trace_args="--profile-config c3 --steps 100",
        pmc_args="--profile-config c3 --steps 3 --warm-seconds 0",
        prefill=K_C3, decode=None),
    "longctx": dict(
        stem="pasa_prefill_longctx_s32768_h32_8_d128", config="c4",
        trace_args="--profile-config c4 --steps 20",
        pmc_args="--profile-config c4 --steps 2 --warm-seconds 0",
        prefill=K_PREFILL, decode=None),
    "paged": dict(
        stem="pasa_decode_paged64_shuffled_b64_kv8192", config="c5",
        trace_args="--profile-config c5paged --steps 100",
        pmc_args="--profile-config c5paged --steps 3 --warm-seconds 0",
        prefill=None, decode=K_SPLIT_PAGED),
}
PMC_SETS = {
    "pmc1": "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_VMEM "
            "SQ_BUSY_CYCLES SQ_WAVE_CYCLES",
    "pmc2": "SQ_LDS_BANK_CONFLICT SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
            "SQ_WAIT_INST_LDS SQ_ACTIVE_INST_ANY SQ_WAIT_ANY GRBM_GUI_ACTIVE",
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
}


def profile_cmd(set_name, kind):
    """The rocprofv3 command of one profile run (kind: trace, a PMC_SETS key,
    or cfetch / cwrite for the copy calibration)."""
    ps = PROFILE_SETS[set_name]
    d = f"rocprof_out/{set_name}/{kind}"
    if kind == "trace":
        return (f"rocprofv3 --kernel-trace --stats -d {d} -o run --output-format csv "
                f"-- python bench.py {ps['trace_args']}")
    if kind in ("cfetch", "cwrite"):
        c = "FETCH_SIZE" if kind == "cfetch" else "WRITE_SIZE"
        return (f"rocprofv3 --pmc {c} -d {d} -o run --output-format csv "
                f"-- python bench.py --calibrate-copy 1024")
    return (f"rocprofv3 --pmc {PMC_SETS[kind]} -d {d} -o run --output-format csv "
            f"-- python bench.py {ps['pmc_args']}")


def source_hash():
    """sha256 over the kernel sources and the ABI header (what the counters
    describe), with comments and whitespace removed so that a comment edit
    does not invalidate recorded counters, and over the compiler options the
    library is built with."""
    import glob
    import hashlib
    import re
    from precision_flashattention_numerics_amd import build as hip_build
    h = hashlib.sha256()
    h.update(repr((hip_build.FLAGS, sorted(hip_build.SOURCE_FLAGS.items()))).encode())
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp")))
    files.append(os.path.join(ROOT, "include", "pasa_attn.h"))
    for f in files:
        text = open(f).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(os.path.basename(f).encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def traffic_file(set_name):
    return os.path.join(PROFILES, PROFILE_SETS[set_name]["stem"] + "_hbm_traffic.txt")


def recorded_traffic(set_name="qwen2"):
    """(prefill_bytes, decode_bytes) per launch from the committed profile summary,
    or (None, None) if it is missing or was taken on other kernel sources."""
    try:
        kv = {}
        for line in open(traffic_file(set_name)):
            if "=" in line and not line.startswith("#"):
                a, b = line.split("=", 1)
                kv[a.strip()] = b.strip()
        if kv.get("source_sha256") != source_hash():
            return None, None
        dec = kv.get("decode_split_traffic_bytes")
        return int(kv["prefill_traffic_bytes"]), (int(dec) if dec else None)
    except (OSError, KeyError, ValueError):
        return None, None


def _counters(path):
    """{kernel name: {counter: mean value per dispatch}} from a rocprofv3 csv."""
    import csv
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = {}
    for kname, cs in acc.items():
        out[kname] = {c: sum(v) / len(v) for c, v in cs.items()}
    return out


def _pick(table, sub):
    for k, v in table.items():
        if sub in k:
            return v
    raise KeyError(sub)


def summarize_profile(d, set_name):
    """Write the text summaries under profiles/ from a rocprofv3 output directory
    laid out as profile_cmd() produces it (d/<kind>/run_*.csv)."""
    import csv
    import workloads as W
    ps = PROFILE_SETS[set_name]
    os.makedirs(PROFILES, exist_ok=True)
    wp, wd = W.CONFIGS[ps["config"]], W.CONFIGS["c5"]
    stats = {r["Name"]: r for r in csv.DictReader(open(os.path.join(d, "trace", "run_kernel_stats.csv")))}

    def st(sub):
        for k, v in stats.items():
            if sub in k:
                return v
        raise KeyError(sub)
    title = {"c2": "the Qwen2-7B-shaped causal prefill (batch 1, seq 4096, 28 query / 4 kv heads, "
                   "head_dim 128) and split-KV decode (batch 64, kv length 8192, 28/4 heads, head_dim 128)",
             "c5": "the split-KV decode (batch 64, kv length 8192, 28/4 heads, head_dim 128) over a paged "
                   "cache of 64-key pages in a seeded shuffled order",
             "c3": "the Stable-Video-Diffusion-shaped resonance prefill (batch 2, seq 9216, 5 heads, "
                   "head_dim 64, non-causal)",
             "c4": "the long-context causal prefill (batch 1, seq 32768, 32 query / 8 kv heads, "
                   "head_dim 128)"}[ps["config"]]
    lines = [f"# rocprofv3 kernel trace of bench.py on {title}, one MI355X.",
             "# command: " + profile_cmd(set_name, "trace"),
             f"# kernel sources sha256: {source_hash()}",
             "kernel                         calls  avg_us    min_us    max_us   algorithmic    rate"]
    if ps["prefill"]:
        pre = st(ps["prefill"])
        avg_p = float(pre["AverageNs"]) * 1e-3
        lines.append(f"pasa prefill                 {int(pre['Calls']):6d} {avg_p:8.2f} "
                     f"{float(pre['MinNs'])*1e-3:8.2f} {float(pre['MaxNs'])*1e-3:8.2f}  "
                     f"{wp.flops():.4e} flop  {wp.flops()/avg_p/1e6:8.1f} TFLOP/s "
                     f"({wp.flops()/avg_p/1e6/PEAK_FP16_TFLOPS:.3f} of 2500)")
    if ps["decode"]:
        sp = st(ps["decode"])
        avg_s = float(sp["AverageNs"]) * 1e-3
        cb = st(K_COMBINE)
        avg_c = float(cb["AverageNs"]) * 1e-3
        lines.append(f"pasa decode split            {int(sp['Calls']):6d} {avg_s:8.2f} "
                     f"{float(sp['MinNs'])*1e-3:8.2f} {float(sp['MaxNs'])*1e-3:8.2f}  "
                     f"{wd.io_bytes():.4e} B     {wd.io_bytes()/avg_s/1e3:8.1f} GB/s "
                     f"({wd.io_bytes()/avg_s/1e3/PEAK_HBM_GBPS:.3f} of 8000)")
        lines.append(f"pasa decode combine          {int(cb['Calls']):6d} {avg_c:8.2f} "
                     f"{float(cb['MinNs'])*1e-3:8.2f} {float(cb['MaxNs'])*1e-3:8.2f}")
        for label, key in (("naive fp16 prefill", K_NAIVE), ("strict PASA prefill", K_STRICT)):
            try:
                kv = st(key)
            except KeyError:
                continue
            lines.append(f"{label:<28} {int(kv['Calls']):6d} {float(kv['AverageNs'])*1e-3:8.2f} "
                         f"{float(kv['MinNs'])*1e-3:8.2f} {float(kv['MaxNs'])*1e-3:8.2f}")
    open(os.path.join(PROFILES, ps["stem"] + "_kernel_trace.txt"), "w").write("\n".join(lines) + "\n")

    t = []
    fp = os.path.join(d, "fetch", "run_counter_collection.csv")
    if os.path.exists(fp):
        fetch = _counters(fp)
        write = _counters(os.path.join(d, "write", "run_counter_collection.csv"))
        # the copy calibration is taken once (under the qwen2 set) and reused
        cal = d if os.path.exists(os.path.join(d, "cfetch")) else os.path.join(os.path.dirname(d), "qwen2")
        cfetch = _counters(os.path.join(cal, "cfetch", "run_counter_collection.csv"))
        cwrite = _counters(os.path.join(cal, "cwrite", "run_counter_collection.csv"))
        copy_bytes = 1024 * (1 << 20)
        cf = _pick(cfetch, "copyBuffer")["FETCH_SIZE"] * 1024
        cw = _pick(cwrite, "copyBuffer")["WRITE_SIZE"] * 1024
        ff, wf = copy_bytes / cf, copy_bytes / cw
        t = ["# HBM traffic per dispatch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch),",
             "# each scaled by what the same counter reads for a plain 1 GiB device-to-device copy.",
             "# commands:",
             "#   " + profile_cmd(set_name, "fetch"), "#   " + profile_cmd(set_name, "write"),
             "#   " + profile_cmd("qwen2", "cfetch"), "#   " + profile_cmd("qwen2", "cwrite"),
             f"source_sha256={source_hash()}",
             f"copy_bytes={copy_bytes}",
             f"copy_fetch_kib={cf/1024:.1f}", f"copy_write_kib={cw/1024:.1f}",
             f"fetch_factor={ff:.4f}", f"write_factor={wf:.4f}"]
        if ps["prefill"]:
            pf = _pick(fetch, ps["prefill"])["FETCH_SIZE"]
            pw = _pick(write, ps["prefill"])["WRITE_SIZE"]
            p_bytes = int(pf * 1024 * ff + pw * 1024 * wf)
            t += [f"prefill_fetch_kib={pf:.1f}", f"prefill_write_kib={pw:.1f}",
                  f"prefill_traffic_bytes={p_bytes}",
                  f"prefill_algorithmic_bytes={wp.io_bytes()}"]
        if ps["decode"]:
            sf = _pick(fetch, ps["decode"])["FETCH_SIZE"]
            sw = _pick(write, ps["decode"])["WRITE_SIZE"]
            s_bytes = int(sf * 1024 * ff + sw * 1024 * wf)
            t += [f"decode_split_fetch_kib={sf:.1f}", f"decode_split_write_kib={sw:.1f}",
                  f"decode_split_traffic_bytes={s_bytes}",
                  f"decode_algorithmic_bytes={wd.io_bytes()}"]
        open(traffic_file(set_name), "w").write("\n".join(t) + "\n")

    rows = []
    for key, title2 in (("pmc1", "instruction counts"), ("pmc2", "busy / wait cycles")):
        path = os.path.join(d, key, "run_counter_collection.csv")
        if not os.path.exists(path):
            continue
        c = _counters(path)
        rows.append(f"# {title2}: " + profile_cmd(set_name, key))
        kernels = ([("pasa prefill", ps["prefill"])] if ps["prefill"] else []) + \
            ([("pasa decode split", ps["decode"])] if ps["decode"] else [])
        for name, sub in kernels:
            vals = _pick(c, sub)
            rows.append(f"{name}: " + ", ".join(f"{k}={v:.0f}" for k, v in sorted(vals.items())))
    if rows:
        rows.append(f"# kernel sources sha256: {source_hash()}")
        open(os.path.join(PROFILES, ps["stem"] + "_counters.txt"), "w").write("\n".join(rows) + "\n")
    print("\n".join(lines + t + rows))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5,
                    help="at least this many untimed warmup steps (more run until --warm-seconds)")
    ap.add_argument("--warm-seconds", type=float, default=0.3,
                    help="keep running warmup steps until this much wall time has passed "
                         "(the GPU clock ramps up over the first ~40 ms of sustained load)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing and the sampled parity checks")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the other prefill workloads (c1, c3, c4), the paged and e4m3 "
                         "variants and the peak microbenchmarks; profiling runs use this so "
                         "that the c2 kernel's averages are its own")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--profile-config", choices=("c3", "c4", "c5paged"), default=None,
                    help="run only this prefill workload: --steps launches after the warmup")
    ap.add_argument("--summarize-profile", nargs=2, metavar=("DIR", "SET"), default=None,
                    help="write the text summaries under profiles/ from a rocprofv3 output "
                         "directory (subdirectories trace, fetch, write, pmc1, pmc2, and for the "
                         "qwen2 set cfetch, cwrite, made by profile_cmd()), then exit")
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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def warm(fn, seconds, min_iters=1):
    """Run fn back to back until min_iters calls and `seconds` of wall time:
    the GPU raises its clock only after tens of milliseconds of sustained
    load, so timings taken right after an idle spell measure the ramp.
    Returns (calls, seconds)."""
    import torch
    t = time.perf_counter()
    i = 0
    while i < min_iters or time.perf_counter() - t < seconds:
        for _ in range(min(8, max(1, min_iters - i)) if seconds <= 0 else 8):
            fn()
            i += 1
        torch.cuda.synchronize()
    return i, time.perf_counter() - t


def timed_batches(fn, reps, batches, stream):
    """Median and min over `batches` runs of `reps` back-to-back calls, each run
    bracketed by events on the launch stream (ms per call)."""
    import torch
    ts = []
    for _ in range(batches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / reps)
    ts.sort()
    return ts[len(ts) // 2], ts[0]


def measure_peaks(stream):
    """Achievable peaks on this GPU: fp16 matrix-core TFLOP/s (back-to-back
    v_mfma_f32_32x32x16_f16, four chains per wave, four waves per SIMD) and HBM
    read GB/s (a non-temporal 16-byte streaming read of 4 GiB)."""
    import ctypes
    import torch
    if not os.path.exists(PEAK_LIB):
        return None
    lib = ctypes.CDLL(PEAK_LIB)
    lib.peak_mfma_f16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p]
    s = ctypes.c_void_p(stream.cuda_stream)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 4 * n_cu, 2048          # 4 workgroups of 4 waves per CU
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")

    def mfma():
        assert lib.peak_mfma_f16(out.data_ptr(), blocks, iters, s) == 0
    warm(mfma, 0.1)
    med, _ = timed_batches(mfma, 3, 5, stream)
    flops = blocks * 4 * 4 * iters * 32768.0
    # the HBM read: the best of a few launch shapes (workgroups per CU, loads
    # in flight per lane), each over a 2 GiB buffer (8x the last-level cache)
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    hout = torch.empty(32 * n_cu * 256, dtype=torch.int32, device="cuda")
    best, shape = 0.0, None
    for per_cu in (4, 8, 16, 32):
        for unroll in (4, 8, 16):
            def hbm():
                assert lib.peak_hbm_read(src.data_ptr(), nbytes // 16, hout.data_ptr(),
                                         per_cu * n_cu, unroll, s) == 0
            warm(hbm, 0.03)
            hmed, _ = timed_batches(hbm, 3, 3, stream)
            gbps = nbytes / (hmed * 1e-3) / 1e9
            if gbps > best:
                best, shape = gbps, (per_cu, unroll)
    del src, hout, out
    torch.cuda.empty_cache()
    return {"mfma_f16_tflops": round(flops / (med * 1e-3) / 1e12, 1),
            "hbm_read_gbps": round(best, 1),
            "how": "fp16 32x32x16 matrix products back to back (4 chains per wave, 16 waves per CU); "
                   f"non-temporal 16-byte streaming read of 2 GiB, best of 12 launch shapes "
                   f"({shape[0]} workgroups of 256 per CU, {shape[1]} loads in flight per lane)"}


def paged_pool(wd, tk, tv):
    """The decode workload's cache (tk, tv [B, Skv, Hkv, D]) as a pool of 64-key
    pages scattered in a seeded random order: (k pool, v pool, block table,
    sequence lengths)."""
    import numpy as np
    import torch
    ps = 64
    n_pages = wd.batch * wd.seqlen_kv // ps
    perm = torch.from_numpy(np.random.default_rng(5).permutation(n_pages).astype(np.int32)).cuda()
    kpool = torch.empty((n_pages, ps, wd.heads_kv, wd.head_dim), dtype=torch.float16, device="cuda")
    vpool = torch.empty_like(kpool)
    kpool[perm.long()] = tk.reshape(n_pages, ps, wd.heads_kv, wd.head_dim)
    vpool[perm.long()] = tv.reshape(n_pages, ps, wd.heads_kv, wd.head_dim)
    table = perm.reshape(wd.batch, wd.seqlen_kv // ps).contiguous()
    lens = torch.full((wd.batch,), wd.seqlen_kv, dtype=torch.int32, device="cuda")
    return kpool, vpool, table, lens


def profile_only(args):
    """--profile-config: one prefill workload (or the paged decode) alone,
    --steps launches after the warmup, for rocprofv3 runs of that workload."""
    import torch
    import precision_flashattention_numerics_amd as pasa
    import workloads as W
    if args.profile_config == "c5paged":
        wd = W.CONFIGS["c5"]
        tq, tk, tv = (torch.from_numpy(x).cuda() for x in W.generate(wd))
        kpool, vpool, table, lens = paged_pool(wd, tk, tv)
        del tk, tv
        od, ld = pasa.attn_decode_paged(tq, kpool, vpool, table, lens, scale=wd.scale)

        def paged():
            pasa.attn_decode_paged(tq, kpool, vpool, table, lens, scale=wd.scale, out=od, lse=ld)
        n_warm, s_warm = warm(paged, args.warm_seconds, args.warmup)
        med, _ = timed_batches(paged, args.steps, 1, torch.cuda.current_stream())
        gbps = wd.io_bytes() / (med * 1e-3) / 1e9
        print(json.dumps({"config": "c5 paged (64-key pages, shuffled)", "launches": args.steps,
                          "ms": round(med, 5), "GBps": round(gbps, 1),
                          "frac": round(gbps / PEAK_HBM_GBPS, 4), "warmup_launches": n_warm,
                          "warmup_seconds": round(s_warm, 3)}), flush=True)
        return
    w = W.CONFIGS[args.profile_config]
    tq, tk, tv = (torch.from_numpy(x).cuda() for x in W.generate(w))
    o = torch.empty_like(tq)
    lse = torch.empty((w.batch, w.heads_q, w.seqlen_q), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def fwd():
        pasa.attn_fwd(tq, tk, tv, causal=w.causal, scale=w.scale, out=o, lse=lse)
    n_warm, s_warm = warm(fwd, args.warm_seconds, args.warmup)
    med, mn = timed_batches(fwd, args.steps, 1, stream)
    tf = w.flops() / (med * 1e-3) / 1e12
    print(json.dumps({"config": w.name, "launches": args.steps, "ms": round(med, 5),
                      "tflops": round(tf, 2), "frac": round(tf / PEAK_FP16_TFLOPS, 4),
                      "warmup_launches": n_warm, "warmup_seconds": round(s_warm, 3)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every workload here fits one MI355X); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.summarize_profile:
        summarize_profile(*args.summarize_profile)
        return
    if args.profile_config:
        profile_only(args)
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

    def step():
        prefill()
        decode()

    # the first prefill launches after the idle spell (clock not yet raised),
    # reported beside the steady-state figure
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        prefill()
    e1.record(stream)
    torch.cuda.synchronize()
    cold_ms = e0.elapsed_time(e1) / 5
    n_warm, s_warm = warm(step, args.warm_seconds, args.warmup)
    log(f"warmup {n_warm} steps ({s_warm:.2f} s) ...")

    # K steps: the K prefill launches back to back, then the K decode launches,
    # each run bracketed by events on the launch stream, so that a kernel's
    # average is its launch-to-launch time (as rocprofv3 reports it) rather
    # than including an event round trip per launch
    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(K):
        prefill()
    ev[1].record(stream)
    for i in range(K):
        decode()
    ev[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_avg = ev[0].elapsed_time(ev[1]) / K
    dec_avg = ev[1].elapsed_time(ev[2]) / K
    log(f"timed {K} steps: prefill {pre_avg:.4f} ms, decode {dec_avg:.4f} ms, wall {wall:.3f} s")

    traffic_p, traffic_d = recorded_traffic("qwen2")
    flops = wp.flops()
    tflops = flops / (pre_avg * 1e-3) / 1e12
    dec_bytes = wd.io_bytes()
    dec_gbps = dec_bytes / (dec_avg * 1e-3) / 1e9

    out = {}
    o_np = op.cpu().numpy()
    l_np = lp.cpu().numpy()
    od_np = od.cpu().numpy()
    out["pasa_nonfinite"] = nonfinite(o_np) + nonfinite(od_np)

    def naive_report(tq, tk, tv, w):
        """The naive fp16 kernel on the same input: inf/NaN outputs, and which
        heads have any (the overflow PASA avoids)."""
        on, _ = pasa.naive_attn_fwd(tq, tk, tv, causal=w.causal, scale=w.scale)
        torch.cuda.synchronize()
        on = on.cpu().numpy()
        per_head = [nonfinite(on[:, :, h]) for h in range(w.heads_q)]
        rep = {"nonfinite": int(sum(per_head)), "of": int(on.size),
               "heads_nonfinite": int(sum(1 for x in per_head if x)), "heads": w.heads_q}
        return rep, on, [h for h in range(w.heads_q) if per_head[h] == 0]

    naive = {}
    naive["c2"], _, _ = naive_report(tqp, tkp, tvp, wp)
    out["naive_nonfinite"] = naive["c2"]["nonfinite"]
    # the variant with fp16 running maximum and offset: its error is reported
    # beside the default's (and its speed, outside the timed steps)
    os_, ls_ = pasa.attn_fwd_strict(tqp, tkp, tvp, causal=wp.causal, scale=wp.scale)

    def strict():
        pasa.attn_fwd_strict(tqp, tkp, tvp, causal=wp.causal, scale=wp.scale, out=os_, lse=ls_)
    warm(strict, 0.1)
    med, _ = timed_batches(strict, K, 1, stream)
    out["strict_tflops"] = round(flops / (med * 1e-3) / 1e12, 3)
    os_np, ls_np = os_.cpu().numpy(), ls_.cpu().numpy()
    out["strict_nonfinite"] = nonfinite(os_np)

    # the other prefill configs, outside the timed steps: c1 is launch-bound
    # (its latency is reported), c3 and c4 against the same MFMA peak
    kept = {}      # inputs and sampled outputs for the oracle leg
    peaks = None
    if not args.no_other_configs:
        other = {}
        for name, reps in (("c1", 20), ("c3", 10), ("c4", 2)):
            w = W.CONFIGS[name]
            log(f"config {name} ...")
            q_, k_, v_ = W.generate(w)
            tq, tk, tv = (torch.from_numpy(x).cuda() for x in (q_, k_, v_))
            o2 = torch.empty_like(tq)
            l2 = torch.empty((w.batch, w.heads_q, w.seqlen_q), dtype=torch.float32, device="cuda")

            def fwd2():
                pasa.attn_fwd(tq, tk, tv, causal=w.causal, scale=w.scale, out=o2, lse=l2)
            if name == "c1":
                # launch-bound: the latency of single launches
                warm(fwd2, 0.0, 2)
                ts = sorted(timed_batches(fwd2, 1, 1, stream)[0] for _ in range(reps))
                med, mn = ts[len(ts) // 2], ts[0]
            else:
                # throughput: warm, then batches of back-to-back launches
                warm(fwd2, 0.15)
                med, mn = timed_batches(fwd2, reps, 5, stream)
            tf = w.flops() / (med * 1e-3) / 1e12
            o2_np = o2.cpu().numpy()
            other[name] = {"median_ms": round(med, 5), "min_ms": round(mn, 5),
                           "tflops": round(tf, 2), "frac": round(tf / PEAK_FP16_TFLOPS, 4),
                           "nonfinite": nonfinite(o2_np)}
            if name != "c1":
                naive[name], on, fin_heads = naive_report(tq, tk, tv, w)
                rng = np.random.default_rng(7)
                rows = np.sort(rng.choice(w.batch * w.heads_q * w.seqlen_q, 256, replace=False))
                b, rem = np.divmod(rows, w.heads_q * w.seqlen_q)
                h, i = np.divmod(rem, w.seqlen_q)
                keep = dict(w=w, q=q_, k=k_, v=v_, rows=rows, o=o2_np[b, i, h])
                if fin_heads:
                    nrows = np.concatenate([
                        np.sort(rng.choice(w.seqlen_q, 64, replace=False)) + (bb * w.heads_q + hh) * w.seqlen_q
                        for bb in range(w.batch) for hh in fin_heads]).astype(np.int64)
                    b, rem = np.divmod(nrows, w.heads_q * w.seqlen_q)
                    h, i = np.divmod(rem, w.seqlen_q)
                    keep.update(naive_rows=nrows, naive_o=on[b, i, h])
                kept[name] = keep
                del on
            del tq, tk, tv, o2, l2, o2_np
            torch.cuda.empty_cache()
        # the decode workload over a paged cache: 64-key pages scattered over
        # the pool in a seeded random order (HBM-bound like the contiguous one)
        kpool, vpool, table, lens = paged_pool(wd, tkd, tvd)
        opg, lpg = pasa.attn_decode_paged(tqd, kpool, vpool, table, lens, scale=wd.scale)

        def paged():
            pasa.attn_decode_paged(tqd, kpool, vpool, table, lens, scale=wd.scale, out=opg, lse=lpg)
        warm(paged, 0.1)
        pg_ms, _ = timed_batches(paged, 10, 1, stream)
        other["c5_paged64"] = {"ms": round(pg_ms, 5),
                               "GBps": round(wd.io_bytes() / (pg_ms * 1e-3) / 1e9, 1),
                               "frac": round(wd.io_bytes() / (pg_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                               "equal_to_contiguous": bool(torch.equal(opg, od))}
        del kpool, vpool
        torch.cuda.empty_cache()
        # c2 with e4m3 queries and keys (per-tensor scales; values fp16)
        q8s = float(tqp.abs().max()) / 448.0
        k8s = float(tkp.abs().max()) / 448.0
        q8 = torch.clamp(tqp.float() / q8s, -448.0, 448.0).to(torch.float8_e4m3fn)
        k8 = torch.clamp(tkp.float() / k8s, -448.0, 448.0).to(torch.float8_e4m3fn)
        o8, l8 = pasa.attn_fwd_fp8(q8, k8, tvp, q8s, k8s, causal=wp.causal, scale=wp.scale)

        def fp8():
            pasa.attn_fwd_fp8(q8, k8, tvp, q8s, k8s, causal=wp.causal, scale=wp.scale, out=o8, lse=l8)
        warm(fp8, 0.1)
        f8_ms, _ = timed_batches(fp8, 10, 1, stream)
        other["c2_fp8_qk"] = {"ms": round(f8_ms, 5),
                              "tflops": round(flops / (f8_ms * 1e-3) / 1e12, 2),
                              "nonfinite": nonfinite(o8.cpu().numpy())}
        del q8, k8, o8, l8
        torch.cuda.empty_cache()
        # a short causal prefill of few work items (Qwen2-shaped heads, 2048
        # tokens), where the longest causal items set the time: the library
        # runs it as key-split items
        ws_ = W.custom(1, 2048, 2048, 32, 8, 128, True, kind="bias", seed=12, bias=30.0)
        tq, tk, tv = (torch.from_numpy(x).cuda() for x in W.generate(ws_))
        os2, ls2 = pasa.attn_fwd(tq, tk, tv, causal=True, scale=ws_.scale)

        def short():
            pasa.attn_fwd(tq, tk, tv, causal=True, scale=ws_.scale, out=os2, lse=ls2)
        warm(short, 0.1)
        sh_ms, _ = timed_batches(short, 10, 5, stream)
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        other["causal_s2048_h32"] = {"ms": round(sh_ms, 5),
                                     "tflops": round(ws_.flops() / (sh_ms * 1e-3) / 1e12, 2),
                                     "key_split": pasa.fwd_key_split(1, 2048, 2048, 32, 128, True, n_cu),
                                     "nonfinite": nonfinite(os2.cpu().numpy())}
        del tq, tk, tv, os2, ls2
        torch.cuda.empty_cache()
        out["other_configs"] = other
        log("peak microbenchmarks ...")
        peaks = measure_peaks(stream)
    out["naive"] = naive

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
        # when the sample is the whole workload and takes less than the budget,
        # repeat it until the budget is spent and take the median run
        times = [tc]
        while sum(times) < args.cpu_seconds and len(times) < 64:
            times.append(run_rows(rows)[2])
        tc = float(np.median(times))
        cpu_flops = 4 * wp.head_dim * pairs(rows)
        b, rem = np.divmod(rows, wp.heads_q * wp.seqlen_q)
        h, i = np.divmod(rem, wp.seqlen_q)
        out["rel_rmse_sampled"] = rel_rmse(o_np[b, i, h], ro)
        out["lse_max_abs_err_sampled"] = float(np.max(np.abs(l_np[b, h, i] - rl)))
        out["strict_rel_rmse_sampled"] = rel_rmse(os_np[b, i, h], ro)
        out["strict_lse_max_abs_err_sampled"] = float(np.max(np.abs(ls_np[b, h, i] - rl)))
        # the other workloads' sampled rows, and the naive kernel's error on
        # the heads where it stayed finite
        for name, kp_ in kept.items():
            w = kp_["w"]
            r_o, _ = attn_fp64(kp_["q"], kp_["k"], kp_["v"], w.scale, w.causal, rows=kp_["rows"])
            out["other_configs"][name]["rel_rmse_sampled"] = rel_rmse(kp_["o"], r_o)
            if "naive_rows" in kp_:
                r_n, _ = attn_fp64(kp_["q"], kp_["k"], kp_["v"], w.scale, w.causal,
                                   rows=kp_["naive_rows"])
                naive[name]["finite_heads_rel_rmse_sampled"] = rel_rmse(kp_["naive_o"], r_n)
        cpu = {"value": cpu_flops / tc / 1e12, "unit": "TFLOP/s", "cores": num_threads(),
               "cpu_model": cpu_model(), "kind": "oracle",
               "sample": (f"{'all ' if n_rows == total_rows else ''}{n_rows} "
                          f"{'' if n_rows == total_rows else 'random '}query rows of the prefill "
                          f"workload ({cpu_flops:.3e} algorithmic flops, binary64, OpenMP), "
                          f"median of {len(times)} runs over {sum(times):.1f} s: {tc:.2f} s per run")}
        log(f"oracle: {n_rows} rows, {len(times)} runs, median {tc:.2f} s")

    roof = {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_FP16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP16_TFLOPS, 4), "traffic": traffic_p}
    roof_d = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
              "frac": round(dec_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic_d}
    if peaks:
        roof["measured_peak"] = peaks["mfma_f16_tflops"]
        roof["frac_of_measured_peak"] = round(tflops / peaks["mfma_f16_tflops"], 4)
        roof_d["measured_peak"] = peaks["hbm_read_gbps"]
        roof_d["frac_of_measured_peak"] = round(dec_gbps / peaks["hbm_read_gbps"], 4)
    line = {
        "metric": "PASA fwd TFLOP/s (fraction of fp16 MFMA peak); decode HBM GB/s; RMSE vs fp64",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": n_warm,
        "warmup_seconds": round(s_warm, 3),
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
        "prefill_ms_cold": round(cold_ms, 5),
        "prefill_frac_of_peak": round(tflops / PEAK_FP16_TFLOPS, 4),
        "decode_ms": round(dec_avg, 5),
        "decode_GBps": round(dec_gbps, 1),
        "roofline": roof,
        "roofline_decode": roof_d,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        **out,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
