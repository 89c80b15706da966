#!/usr/bin/env python3
"""Throughput of the gated delta rule hot path on one MI355X (gfx950).

    python bench.py [--steps K] [--warmup W] [--workload prefill_1k]

Headline: chunked-prefill tokens/s of one Qwen3.5-9B Gated DeltaNet layer
(16 query/key heads, 32 value heads, head dim 128, chunk 64; B=1, T=1024,
bf16 q/k/v, fp32 g/beta/state).  One step = one gdn_prefill_chunked call
(chunk table, prep, chunk scan) over one batch already resident in HBM.
Several copies of the batch are rotated so that repeated steps do not run
out of the 256 MB last-level cache.  The same run also measures the decode
step (64 sequences, state updated in place, state sets rotated), the long
32k prefill and the 16-sequence varlen prefill, each with its per-kernel
durations from HIP events recorded on the library's launch stream; the conv1d
ahead of the scan and the gated RMSNorm after it, on the 1k and 32k shapes; and
the fp64 CPU oracle on a bounded sample of the headline workload.

Prints ONE JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0       # dense bf16 matrix cores
PEAK_FP32_MFMA_TFLOPS = 157.3   # dense fp32 matrix cores
CACHE_DEFEAT_BYTES = 600e6      # rotate copies until the working set exceeds the 256 MB MALL twice over

METRIC = "prefill tokens/s + decode tokens/s (Qwen3.5-9B GDN layer), % MFMA/HBM peak"

# HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, each
# scaled by what the counter reads for a plain copy of known size).  A figure is used only
# while the kernel's sources still hash to the digest stored beside it.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
KERNEL_SOURCES = {
    "gdn_chunk_scan_rows_kernel": ("gated_deltanet_scan_amd/csrc/gdn_prefill.hip", "gated_deltanet_scan_amd/csrc/gdn_device.hpp"),
    "gdn_chunk_scan_bf16_kernel": ("gated_deltanet_scan_amd/csrc/gdn_prefill.hip", "gated_deltanet_scan_amd/csrc/gdn_device.hpp"),
    "gdn_chunk_scan_kernel": ("gated_deltanet_scan_amd/csrc/gdn_prefill.hip", "gated_deltanet_scan_amd/csrc/gdn_device.hpp"),
    "gdn_prep_kernel": ("gated_deltanet_scan_amd/csrc/gdn_prefill.hip", "gated_deltanet_scan_amd/csrc/gdn_device.hpp"),
    "gdn_decode_kernel": ("gated_deltanet_scan_amd/csrc/gdn_decode.hip", "gated_deltanet_scan_amd/csrc/gdn_device.hpp"),
    "gdn_gated_rmsnorm_kernel": ("gated_deltanet_scan_amd/csrc/gdn_norm.hip", "gated_deltanet_scan_amd/csrc/gdn_device.hpp"),
    "gdn_conv_kernel": ("gated_deltanet_scan_amd/csrc/gdn_conv.hip", "gated_deltanet_scan_amd/csrc/gdn_device.hpp"),
}


def sources_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter summary, or
    None when there is none or the kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    want = sources_digest(kernel)
    for line in lines:
        if not line.startswith("traffic:"):
            continue
        kv = dict(tok.split("=", 1) for tok in line[len("traffic:"):].split())
        if kv.get("kernel") == kernel and kv.get("workload") == workload and kv.get("sources") == want:
            return float(kv["bytes_per_launch"])
    return None


def esize(dtype):
    import torch
    return 2 if dtype == torch.bfloat16 else 4


def prefill_costs(w, lengths):
    """Algorithmic bytes and flops per launch of each prefill kernel.

    Bytes are what the kernel must move between HBM and the chip at least: its inputs
    read once and its outputs written once.  Flops count the dense contractions only
    (a multiply-add is two flops): per real token for the scan, per chunk for the prep."""
    es = esize(w.io_dtype)
    T = sum(lengths)
    N = len(lengths)
    C, dk, dv, hqk, hv = w.chunk, w.dk, w.dv, w.hqk, w.hv
    E = sum((L + C - 1) // C for L in lengths)
    qk_bytes = 2 * T * hqk * dk * es
    gb_bytes = 2 * T * hv * 4
    ta_bytes = 2 * E * hv * C * C * es + E * hv * 4 * C * 4     # T, A and the decay record
    s_in = N * hv * dk * dv * 4 if w.s0_std is not None else 0
    s_out = N * hv * dk * dv * 4
    prep = {
        "bytes": qk_bytes + gb_bytes + ta_bytes,
        # two lower-triangular Gram products per chunk and query/key head, plus the
        # forward substitution (C^3/3 flops per chunk and value head)
        "flops": E * hqk * 2 * (C * (C + 1) // 2) * dk * 2 + E * hv * (C ** 3) // 3,
    }
    scan = {
        "bytes": qk_bytes + T * hv * dv * es + gb_bytes + ta_bytes + T * hv * dv * es + s_in + s_out,
        # [Q;K] S, S update: 6 dk dv; T X and A D: 4 C dv  (per token and value head)
        "flops": T * hv * (6 * dk * dv + 4 * C * dv),
    }
    io_bytes = qk_bytes + 2 * T * hv * dv * es + gb_bytes + s_in + s_out   # what a step must move at least
    return {"prep": prep, "scan": scan, "io_bytes": io_bytes, "chunks": E}


def decode_costs(w):
    es = esize(w.io_dtype)
    N = len(w.lengths)
    state = 2 * N * w.hv * w.dk * w.dv * 4
    other = 2 * N * w.hqk * w.dk * es + 2 * N * w.hv * w.dv * es + 2 * N * w.hv * 4
    return {"bytes": state + other, "state_bytes": state, "flops": N * w.hv * 7 * w.dk * w.dv}


def _sync():
    import torch
    torch.cuda.synchronize()


def _clone_inputs(d):
    return {k: (v.clone() if hasattr(v, "clone") else v) for k, v in d.items()}


def measure_prefill(name, steps, warmup, lengths=None):
    import torch

    import gated_deltanet_scan_amd as gdn
    from gated_deltanet_scan_amd import synthetic
    w = synthetic.workload(name)
    lengths = lengths or w.lengths
    x = synthetic.make_workload_inputs(w, lengths=lengths)
    dev = torch.device("cuda:0")
    base = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    costs = prefill_costs(w, lengths)
    shape = gdn.make_shape(w.hqk, w.hv, w.dk, w.dv, w.chunk, 1 if w.io_dtype == torch.bfloat16 else 0, 1.0)
    ws_bytes = gdn.workspace_bytes(shape, sum(lengths), len(lengths))
    per_set = costs["io_bytes"] + ws_bytes
    n_sets = int(min(16, max(1, math.ceil(CACHE_DEFEAT_BYTES / per_set))))
    calls = []
    for i in range(n_sets):
        d = base if i == 0 else _clone_inputs(base)
        # host copy of the offsets: the library validates them and plans its segments
        calls.append(gdn.prepare_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], x["cu_seqlens"],
                                         d["initial_state"], chunk=w.chunk))
    for i in range(warmup):
        calls[i % n_sets]()
    _sync()
    t0 = time.perf_counter()
    for i in range(steps):
        calls[i % n_sets]()
    _sync()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / steps

    # per-kernel durations: HIP events on the launch stream over a second timed pass
    gdn.profile_enable(True)
    for i in range(steps):
        calls[i % n_sets]()
    _sync()
    kern = {}
    for kid, kname in ((0, "chunk_table"), (1, "prep"), (2, "scan")):
        n, tot = gdn.profile_collect(kid)
        kern[kname] = {"launches_per_step": n / steps, "avg_us": (tot / n * 1e3) if n else None,
                       "per_step_us": tot * 1e3 / steps}
    gdn.profile_enable(False)
    T = sum(lengths)
    flops = costs["prep"]["flops"] + costs["scan"]["flops"]
    peak = PEAK_BF16_TFLOPS if w.io_dtype == torch.bfloat16 else PEAK_FP32_MFMA_TFLOPS
    out = {
        "workload": name, "tokens": T, "sequences": len(lengths), "ms_per_step": ms,
        "tokens_per_s": T / (ms * 1e-3), "rotated_copies": n_sets,
        "mfma_frac": flops / (ms * 1e-3) / (peak * 1e12),
        "hbm_frac": costs["io_bytes"] / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "kernels": kern,
        "scan_kernel": scan_kernel_name(w, lengths),
    }
    # whole-step costs over the kernel's summed launch time (a long or batched prefill is
    # cut into several launches of each kernel)
    for kname in ("prep", "scan"):
        us = kern[kname]["per_step_us"]
        c = costs[kname]
        if us:
            out[kname + "_gbs"] = c["bytes"] / (us * 1e-6) / 1e9
            out[kname + "_tflops"] = c["flops"] / (us * 1e-6) / 1e12
    out["_costs"] = costs
    out["_peak_tflops"] = peak
    return out


def scan_kernel_name(w, lengths):
    """Which scan kernel the library runs for this batch (bf16 io, chunk 64: whole-head
    workgroups for wide batches of 128-dim heads, the row-split kernel otherwise)."""
    import torch
    if w.io_dtype == torch.bfloat16 and w.chunk == 64:
        if w.dv == 128 and len(lengths) * w.hv >= 256:
            return "gdn_chunk_scan_bf16_kernel"
        return "gdn_chunk_scan_rows_kernel"
    return "gdn_chunk_scan_kernel"


def roofline_for(pre):
    """Roofline object of the dominant prefill kernel (the one with the longest average launch)."""
    kern = pre["kernels"]
    name = max(("prep", "scan"), key=lambda k: kern[k]["per_step_us"] or 0.0)
    launches = kern[name]["launches_per_step"]
    us = kern[name]["avg_us"]
    # algorithmic cost of one launch: the step's cost over its launches of this kernel
    c = {k: v / launches for k, v in pre["_costs"][name].items()}
    intensity = c["flops"] / c["bytes"]
    ridge = pre["_peak_tflops"] * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity < ridge:
        achieved = c["bytes"] / (us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = c["flops"] / (us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": pre["_peak_tflops"], "unit": "TFLOP/s",
                "frac": achieved / pre["_peak_tflops"]}
    kernel = "gdn_prep_kernel" if name == "prep" else pre["scan_kernel"]
    roof.update({"traffic": measured_traffic(kernel, pre["workload"]), "kernel": kernel,
                 "avg_us": us, "algorithmic_bytes": c["bytes"], "algorithmic_flops": c["flops"],
                 "intensity_flop_per_byte": intensity})
    return roof


def measure_decode(name, steps, warmup):
    import torch

    import gated_deltanet_scan_amd as gdn
    from gated_deltanet_scan_amd import synthetic
    w = synthetic.workload(name)
    x = synthetic.make_workload_inputs(w)
    dev = torch.device("cuda:0")
    base = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    costs = decode_costs(w)
    n_sets = int(min(16, max(3, math.ceil(CACHE_DEFEAT_BYTES / costs["bytes"]))))
    calls = []
    for i in range(n_sets):
        d = base if i == 0 else _clone_inputs(base)
        calls.append(gdn.prepare_decode(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"]))
    for i in range(warmup):
        calls[i % n_sets]()
    _sync()
    t0 = time.perf_counter()
    for i in range(steps):
        calls[i % n_sets]()
    _sync()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    gdn.profile_enable(True)
    for i in range(steps):
        calls[i % n_sets]()
    _sync()
    n, tot = gdn.profile_collect(3)
    gdn.profile_enable(False)
    us = tot / n * 1e3
    achieved = costs["bytes"] / (us * 1e-6) / 1e9
    N = len(w.lengths)
    return {
        "workload": name, "sequences": N, "ms_per_step": ms, "tokens_per_s": N / (ms * 1e-3),
        "kernel_avg_us": us, "kernel_tokens_per_s": N / (us * 1e-6),
        "state_gbs": costs["state_bytes"] / (us * 1e-6) / 1e9, "rotated_state_sets": n_sets,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic("gdn_decode_kernel", name),
                     "kernel": "gdn_decode_kernel",
                     "avg_us": us, "algorithmic_bytes": costs["bytes"]},
    }


def measure_norm(tokens, steps, warmup, hv=32, dv=128):
    """The gated RMSNorm after the scan (gdn_gated_rmsnorm) on a [tokens, HV, dv] bf16 output:
    algorithmic bytes = o and z read once, y written once (3 * tokens * HV * dv * 2) plus the
    weight.  Input sets are rotated so that the working set exceeds the last-level cache."""
    import torch

    import gated_deltanet_scan_amd as gdn
    from gated_deltanet_scan_amd import synthetic
    x = synthetic.make_norm_inputs(tokens, hv, dv, torch.bfloat16, seed=2000)
    dev = torch.device("cuda:0")
    base = {k: v.to(dev) for k, v in x.items()}
    nbytes = 3 * tokens * hv * dv * 2 + dv * 4
    n_sets = int(min(16, max(1, math.ceil(CACHE_DEFEAT_BYTES / nbytes))))
    calls = []
    for i in range(n_sets):
        d = base if i == 0 else {k: v.clone() for k, v in base.items()}
        calls.append(gdn.prepare_gated_rmsnorm(d["o"], d["z"], d["weight"], eps=1e-6))
    for i in range(warmup):
        calls[i % n_sets]()
    _sync()
    gdn.profile_enable(True)
    for i in range(steps):
        calls[i % n_sets]()
    _sync()
    n, tot = gdn.profile_collect(5)
    gdn.profile_enable(False)
    us = tot / n * 1e3
    achieved = nbytes / (us * 1e-6) / 1e9
    return {"shape": [tokens, hv, dv], "dtype": "bf16", "eps": 1e-6, "kernel_avg_us": us,
            "tokens_per_s": tokens / (us * 1e-6), "rotated_sets": n_sets,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": achieved / PEAK_HBM_GBS, "kernel": "gdn_gated_rmsnorm_kernel",
                         "traffic": measured_traffic("gdn_gated_rmsnorm_kernel", "norm_%d" % tokens),
                         "avg_us": us, "algorithmic_bytes": nbytes}}


def measure_conv(tokens, steps, warmup, hqk=16, hv=32, d=128, width=4):
    """The conv1d ahead of the scan (gdn_conv1d_qkv, q/k head L2 norms, conv state read and
    updated in place) on one sequence of `tokens` bf16 tokens with the Qwen3.5-9B heads.
    Algorithmic bytes of the conv kernel: x read once and q, k, v written once (2 * T * C * 2),
    the taps (C * K * 4) and the state entries it reads (C * (K-1) * 4).  The state update is
    its own small kernel (timed apart; the step is both).  Input sets are rotated past the
    last-level cache."""
    import torch

    import gated_deltanet_scan_amd as gdn
    from gated_deltanet_scan_amd import synthetic
    x = synthetic.make_conv_inputs([tokens], hqk, hv, d, d, width, torch.bfloat16, seed=3000)
    dev = torch.device("cuda:0")
    C = 2 * hqk * d + hv * d
    nbytes = 2 * tokens * C * 2 + C * width * 4 + C * (width - 1) * 4
    n_sets = int(min(16, max(1, math.ceil(CACHE_DEFEAT_BYTES / nbytes))))
    calls = []
    for i in range(n_sets):
        xx, w, cu, st = (x["x"].to(dev).clone(), x["weight"].to(dev), x["cu_seqlens"].to(dev),
                         x["state"].to(dev).clone())
        calls.append(gdn.prepare_conv1d_qkv(xx, w, hqk, hv, d, d, cu, st, st, l2norm=True, eps=1e-6))
    for i in range(warmup):
        calls[i % n_sets]()
    _sync()
    gdn.profile_enable(True)
    for i in range(steps):
        calls[i % n_sets]()
    _sync()
    n, tot = gdn.profile_collect(6)      # the conv
    n_st, tot_st = gdn.profile_collect(7)   # its state update
    gdn.profile_enable(False)
    us = tot / steps * 1e3
    us_state = tot_st / steps * 1e3
    achieved = nbytes / (us * 1e-6) / 1e9
    return {"shape": {"tokens": tokens, "channels": C, "width": width}, "dtype": "bf16", "kernel_avg_us": us,
            "state_update_avg_us": us_state, "step_us": us + us_state,
            "launches_per_step": (n + n_st) / steps, "tokens_per_s": tokens / ((us + us_state) * 1e-6),
            "rotated_sets": n_sets,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": achieved / PEAK_HBM_GBS, "kernel": "gdn_conv_kernel",
                         "traffic": measured_traffic("gdn_conv_kernel", "conv_%d" % tokens),
                         "avg_us": us, "algorithmic_bytes": nbytes}}


def cpu_baseline(name, seconds):
    import oracle
    from gated_deltanet_scan_amd import synthetic
    w = synthetic.workload(name)
    x = synthetic.make_workload_inputs(w)
    threads = oracle.default_threads()
    T = w.total_tokens
    runs = 0
    t0 = time.perf_counter()
    while True:
        oracle.gdn_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"], x["initial_state"],
                           threads=threads)
        runs += 1
        wall = time.perf_counter() - t0
        if wall >= seconds or runs >= 1000:
            break
    return {"value": runs * T / wall, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d full passes of %s (%d tokens x %d value heads, fp64 sequential recurrence, "
                      "%d threads over (sequence, head) items), %.1f s wall" % (runs, name, T, w.hv, threads,
                                                                                 wall)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_1k")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the long and varlen prefill lines")
    ap.add_argument("--profile-prefill", action="store_true",
                    help="run only the headline prefill loop (for rocprofv3 kernel traces and counters)")
    ap.add_argument("--profile-decode", action="store_true",
                    help="run only the decode loop (for rocprofv3 kernel traces and counters)")
    ap.add_argument("--profile-norm", action="store_true",
                    help="run only the gated RMSNorm loop at 32768 tokens (for rocprofv3)")
    ap.add_argument("--profile-conv", action="store_true",
                    help="run only the conv1d loop at 32768 tokens (for rocprofv3)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run only a plain device copy of MIB MiB, 10 times (scale for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the gated delta rule shards over heads and sequences with no "
              "exchange; more than one GPU is not measured here (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            torch.neg(src, out=dst)     # one elementwise kernel: reads n bytes, writes n bytes
        _sync()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 10}))
        return
    import gated_deltanet_scan_amd as gdn
    gdn.load_library()

    if args.profile_decode:
        dec = measure_decode("decode_64", args.steps, args.warmup)
        print(json.dumps(dec))
        return
    if args.profile_norm or args.profile_conv:
        fn = measure_norm if args.profile_norm else measure_conv
        print(json.dumps(fn(32768, args.steps, args.warmup)))
        return
    print("[bench] prefill %s" % args.workload, file=sys.stderr, flush=True)
    pre = measure_prefill(args.workload, args.steps, args.warmup)
    if args.profile_prefill:
        print(json.dumps({k: v for k, v in pre.items() if not k.startswith("_")}))
        return
    print("[bench] decode_64", file=sys.stderr, flush=True)
    dec = measure_decode("decode_64", max(args.steps, 20), args.warmup)
    extra = {}
    if not args.no_extra:
        for name in ("prefill_32k", "varlen_16"):
            if name == args.workload:
                continue
            print("[bench] prefill %s" % name, file=sys.stderr, flush=True)
            r = measure_prefill(name, max(5, min(args.steps, 20)), 2)
            extra[name] = {k: v for k, v in r.items() if not k.startswith("_")}
        for tokens in (1024, 32768):
            print("[bench] gated RMSNorm %d tokens" % tokens, file=sys.stderr, flush=True)
            extra["gated_rmsnorm_%d" % tokens] = measure_norm(tokens, max(10, min(args.steps, 50)), 3)
        for tokens in (1024, 32768):
            print("[bench] conv1d %d tokens" % tokens, file=sys.stderr, flush=True)
            extra["conv1d_qkv_%d" % tokens] = measure_conv(tokens, max(10, min(args.steps, 50)), 3)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.workload, args.cpu_seconds)

    from gated_deltanet_scan_amd import synthetic
    w = synthetic.workload(args.workload)
    line = {
        "metric": METRIC,
        "value": pre["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.io_dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": "%s: Qwen3.5-9B GDN layer prefill, %d sequence(s), %d tokens, %d QK / %d V heads, "
                               "dk=dv=%d, chunk %d, bf16 q/k/v, fp32 g/beta/state"
                               % (args.workload, len(w.lengths), w.total_tokens, w.hqk, w.hv, w.dk, w.chunk),
                   "global_batch": len(w.lengths), "seq_len": w.total_tokens},
        "roofline": roofline_for(pre),
        "cpu_baseline": cpu,
        "prefill": {k: v for k, v in pre.items() if not k.startswith("_")},
        "decode": dec,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
