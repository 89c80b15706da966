#!/usr/bin/env python3
"""Throughput of the gated delta rule hot path on one MI355X (gfx950).

    python bench.py [--steps K] [--warmup W] [--workload varlen_16]

Headline: the packed variable-length prefill of one Qwen3.5-9B Gated DeltaNet
layer (16 query/key heads, 32 value heads, head dim 128, chunk 64; 16
sequences of U{256..8192} tokens, each from its own fp32 initial state; bf16
q/k/v, fp32 g/beta/state) with the verify protocol of that workload: after the
prompts, the states are snapshotted, a 16-token draft of every sequence is run
through the chunked prefill, the states are restored, and the accepted prefix of
every draft (m ~ U{1..15} tokens) is fed again.  One step = that whole sequence
of library calls (prefill, snapshot, verify prefill, restore, re-feed prefill)
over one batch already resident in HBM; `value` counts every token the
recurrence processes in it (prompts + drafts + re-fed tokens).

The same run measures the 1k and 32k single-sequence prefills, a skewed batch
(one 32k sequence among 63 short ones), the decode step (64 sequences, state
updated in place, state sets rotated past the last-level cache), the conv1d
ahead of the scan and the gated RMSNorm after it, each with per-kernel durations
from HIP events that the library records on its launch stream, and the fp64 CPU
oracle on a bounded sample of the headline workload.

Algorithmic work per token and value head (chunk C, head dims dk, dv):
  flops = 4 C dk HQK/HV (K K^T and Q K^T, shared by a query/key head's value heads)
        + 2 C (dk + dv) (the two products with the chunk's triangular inverse)
        + 6 dk dv (the three products with the state) + 2 C dv (the intra-chunk output)
        = 163,840 at the Qwen3.5-9B shapes;
  bytes per token = q, k, v read and o written in the io dtype, g and beta in fp32
        = 24,832 at the Qwen3.5-9B shapes; plus every state read and written once per call.
Workspace round trips (the chunk matrices written by the prep and read by the scan)
are not algorithmic: they show up in `traffic`, the HBM bytes that the rocprofv3
counters measured per launch.

Warm-up: the first few dozen steps of a run are slower while the GPU's clocks
ramp up (varlen_16, 30 timed steps: 1.166 ms per step after 3 untimed steps,
1.108 after 20, 1.082 after 60, 1.088 after 120), so the default is 60 untimed
steps before the timed ones.

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
    "gdn_chunk_scan_tform_kernel": ("gated_deltanet_scan_amd/csrc/gdn_prefill.hip", "gated_deltanet_scan_amd/csrc/gdn_device.hpp"),
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


def flops_per_token_head(w):
    """Dense-contraction flops per token and value head of the chunked form (a multiply-add is
    two flops); 163,840 at C = 64, dk = dv = 128, HQK / HV = 1/2."""
    C, dk, dv = w.chunk, w.dk, w.dv
    return (4 * C * dk * w.hqk) // w.hv + 2 * C * (dk + dv) + 6 * dk * dv + 2 * C * dv


def bytes_per_token(w):
    """Algorithmic HBM bytes per token: q, k, v read and o written once, g and beta in fp32."""
    es = esize(w.io_dtype)
    return es * (2 * w.hqk * w.dk + 2 * w.hv * w.dv) + 2 * 4 * w.hv


def prefill_costs(w, tokens, calls, seqs):
    """Algorithmic bytes and flops of `calls` prefill calls that process `tokens` tokens in all,
    each reading and writing the states of `seqs` sequences once."""
    state = seqs * w.hv * w.dk * w.dv * 4
    return {"bytes": bytes_per_token(w) * tokens + 2 * state * calls,
            "flops": flops_per_token_head(w) * w.hv * tokens}


def decode_costs(w):
    es = esize(w.io_dtype)
    N = len(w.lengths)
    state = 2 * N * w.hv * w.dk * w.dv * 4
    other = 2 * N * w.hqk * w.dk * es + 2 * N * w.hv * w.dv * es + 2 * N * w.hv * 4
    return {"bytes": state + other, "state_bytes": state, "flops": N * w.hv * 7 * w.dk * w.dv}


def _sync():
    import torch
    torch.cuda.synchronize()


SCAN_VARIANTS = ((8, "gdn_chunk_scan_rows_kernel"), (9, "gdn_chunk_scan_bf16_kernel"), (10, "gdn_chunk_scan_kernel"),
                 (11, "gdn_chunk_scan_tform_kernel"))


def _kernel_times(steps):
    """Per-step launches and time of each library kernel recorded since profile_enable."""
    import gated_deltanet_scan_amd as gdn
    kern = {}
    for kid, kname in ((0, "chunk_table"), (1, "prep"), (2, "scan"), (12, "short"), (4, "snapshot")):
        n, tot = gdn.profile_collect(kid)
        kern[kname] = {"launches_per_step": n / steps, "avg_us": (tot / n * 1e3) if n else None,
                       "per_step_us": tot * 1e3 / steps}
    # the scan kernel the library chose (it reports each launch under its kernel's identifier)
    ran = [(name, gdn.profile_collect(kid)[0]) for kid, name in SCAN_VARIANTS]
    kern["scan"]["kernel"] = "+".join(name for name, n in ran if n) or None
    return kern


def _timed(fn, steps, warmup):
    """Wall-clock ms per step of `steps` calls after `warmup` calls (synchronised on both sides),
    then the per-kernel HIP-event times of a second pass of `steps` calls."""
    import gated_deltanet_scan_amd as gdn
    for i in range(warmup):
        fn(i)
    _sync()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    _sync()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    gdn.profile_enable(True)
    for i in range(steps):
        fn(i)
    _sync()
    kern = _kernel_times(steps)
    gdn.profile_enable(False)
    return ms, kern


def _to_dev(x):
    import torch
    dev = torch.device("cuda:0")
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def _pack_drafts(w, accepted):
    """The verify drafts (16 fresh tokens per sequence, drawn from the workload's laws) and the
    accepted prefixes to re-feed (the first m_n draft tokens of sequence n), packed."""
    import torch
    from gated_deltanet_scan_amd import synthetic
    n = len(w.lengths)
    V = w.verify_tokens
    draft = synthetic.make_inputs([V] * n, w.hqk, w.hv, w.dk, w.dv, w.io_dtype, seed=w.seed + 100,
                                  g_law=w.g_law, s0_std=None)
    idx = torch.cat([torch.arange(i * V, i * V + m) for i, m in enumerate(accepted)])
    refeed = {key: draft[key][idx].contiguous() for key in ("q", "k", "v", "g", "beta")}
    cu = torch.zeros(n + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(accepted, dtype=torch.int64), 0).to(torch.int32)
    refeed["cu_seqlens"] = cu
    refeed["initial_state"] = None
    return draft, refeed


def measure_prefill(name, steps, warmup, lengths=None, verify=None):
    """One prefill workload.  With `verify` (the headline varlen workload), a step is the whole
    verify protocol: prompt prefill, snapshot, draft prefill, restore, re-feed prefill."""
    import torch

    import gated_deltanet_scan_amd as gdn
    from gated_deltanet_scan_amd import synthetic
    w = synthetic.workload(name)
    lengths = lengths or w.lengths
    x = synthetic.make_workload_inputs(w, lengths=lengths)
    base = _to_dev(x)
    N, T = len(lengths), sum(lengths)
    verify = bool(verify and w.verify_tokens)
    es = esize(w.io_dtype)
    ws_bytes = gdn.workspace_bytes(gdn.make_shape(w.hqk, w.hv, w.dk, w.dv, w.chunk,
                                                  1 if w.io_dtype == torch.bfloat16 else 0, 1.0), T, N)
    per_set = bytes_per_token(w) * T + ws_bytes
    n_sets = 1 if verify else int(min(16, max(1, math.ceil(CACHE_DEFEAT_BYTES / per_set))))
    calls = []
    for i in range(n_sets):
        d = base if i == 0 else {k: (v.clone() if hasattr(v, "clone") else v) for k, v in base.items()}
        # host copy of the offsets: the library validates them and plans its launches
        calls.append(gdn.prepare_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], x["cu_seqlens"],
                                         d["initial_state"], chunk=w.chunk))
    tokens, n_calls = T, 1
    if verify:
        accepted = synthetic.accept_counts(w.seed + 1, N, w.verify_tokens)
        draft, refeed = _pack_drafts(w, accepted)
        state = calls[0].result[1]                  # the prompts' final states, updated in place
        snap = torch.empty_like(state)
        dd, dr = _to_dev(draft), _to_dev(refeed)
        ver = gdn.prepare_prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], draft["cu_seqlens"], state,
                                  chunk=w.chunk, final_state=state)
        ref = gdn.prepare_prefill(dr["q"], dr["k"], dr["v"], dr["g"], dr["beta"], refeed["cu_seqlens"], state,
                                  chunk=w.chunk, final_state=state)

        def step(i):
            calls[0]()
            gdn.state_snapshot(state, snap)
            ver()
            gdn.state_snapshot(snap, state)
            ref()
        tokens = T + N * w.verify_tokens + sum(accepted)
        n_calls = 3
    else:
        def step(i):
            calls[i % n_sets]()
    ms, kern = _timed(step, steps, warmup)
    costs = prefill_costs(w, tokens, n_calls, N)
    peak = PEAK_BF16_TFLOPS if w.io_dtype == torch.bfloat16 else PEAK_FP32_MFMA_TFLOPS
    out = {
        "workload": name, "tokens": tokens, "prompt_tokens": T, "sequences": N, "ms_per_step": ms,
        "tokens_per_s": tokens / (ms * 1e-3), "rotated_copies": n_sets,
        "algorithmic_flops": costs["flops"], "algorithmic_bytes": costs["bytes"],
        "mfma_frac": costs["flops"] / (ms * 1e-3) / (peak * 1e12),
        "hbm_frac": costs["bytes"] / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "kernels": kern,
        "scan_kernel": kern["scan"]["kernel"],
    }
    if verify:
        out["verify"] = {"draft_tokens": N * w.verify_tokens, "refed_tokens": sum(accepted),
                         "accepted": accepted,
                         "step": "prefill, snapshot, %d-token draft prefill, restore, re-feed prefill"
                                 % w.verify_tokens}
    scan_costs = costs
    if verify and kern["short"]["launches_per_step"]:
        # the draft and re-feed calls ran the token-recurrent kernel (every sequence of each at
        # most 8 tokens), so the scan launches did the prompts' work alone
        scan_costs = prefill_costs(w, T, 1, N)
    out["roofline"] = roofline_for(out, scan_costs, peak)
    return out


def roofline_for(pre, costs, peak_tflops):
    """Roofline object of the scan kernel, the step's dominant kernel: the algorithmic bytes (or
    flops) of the calls its launches served, spread over those launches, divided by their
    average duration."""
    k = pre["kernels"]["scan"]
    launches, us = k["launches_per_step"], k["avg_us"]
    c = {key: v / launches for key, v in costs.items()}
    intensity = c["flops"] / c["bytes"]
    ridge = peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9)
    if intensity < ridge:
        achieved = c["bytes"] / (us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = c["flops"] / (us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak_tflops, "unit": "TFLOP/s",
                "frac": achieved / peak_tflops}
    kernel = pre["scan_kernel"]
    roof.update({"traffic": measured_traffic(kernel, pre["workload"]) if kernel and "+" not in kernel else None,
                 "kernel": kernel, "avg_us": us, "launches_per_step": launches,
                 "algorithmic_bytes": c["bytes"], "algorithmic_flops": c["flops"],
                 "intensity_flop_per_byte": intensity,
                 "mfma_frac_of_kernel": c["flops"] / (us * 1e-6) / (peak_tflops * 1e12)})
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
        d = base if i == 0 else {k: (v.clone() if hasattr(v, "clone") else v) for k, v in base.items()}
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


def cpu_baseline(name, seconds, verify=False):
    """The fp64 oracle as it stands, timed on this host's cores over full passes of the
    workload (with `verify`, each pass also runs the drafts and the re-fed prefixes from the
    prompts' final states, as the GPU step does)."""
    import oracle
    from gated_deltanet_scan_amd import synthetic
    w = synthetic.workload(name)
    x = synthetic.make_workload_inputs(w)
    threads = oracle.default_threads()
    passes = []
    tokens = w.total_tokens
    if verify and w.verify_tokens:
        accepted = synthetic.accept_counts(w.seed + 1, len(w.lengths), w.verify_tokens)
        draft, refeed = _pack_drafts(w, accepted)
        tokens += len(w.lengths) * w.verify_tokens + sum(accepted)

    def one_pass():
        _, st = oracle.gdn_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"], x["initial_state"],
                                   threads=threads)
        if verify and w.verify_tokens:
            oracle.gdn_forward(draft["q"], draft["k"], draft["v"], draft["g"], draft["beta"], draft["cu_seqlens"],
                               st, threads=threads)
            oracle.gdn_forward(refeed["q"], refeed["k"], refeed["v"], refeed["g"], refeed["beta"],
                               refeed["cu_seqlens"], st, threads=threads)
    runs = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        runs += 1
        wall = time.perf_counter() - t0
        if wall >= seconds or runs >= 1000:
            break
    what = "prompts, drafts and re-fed prefixes" if verify and w.verify_tokens else "the batch"
    return {"value": runs * tokens / wall, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d full passes of %s over %s (%d tokens x %d value heads per pass, fp64 sequential "
                      "recurrence, %d threads over (sequence, head) items), %.1f s wall"
                      % (runs, name, what, tokens, w.hv, threads, wall)}


def skewed_lengths():
    """One 32768-token sequence among 63 sequences of 64 tokens."""
    return [32768] + [64] * 63


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="varlen_16")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other prefill, decode, conv and norm lines")
    ap.add_argument("--profile-prefill", action="store_true",
                    help="run only the headline loop (for rocprofv3 kernel traces and counters)")
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
    if args.workload == "skewed_64":
        # the skewed batch alone (prefill_32k's shapes, one 32k sequence among 63 of 64 tokens)
        if not args.profile_prefill:
            print("--workload skewed_64 goes with --profile-prefill", file=sys.stderr)
            sys.exit(2)
        print("[bench] prefill skewed batch (one 32k sequence among 63 of 64 tokens)", file=sys.stderr, flush=True)
        pre = measure_prefill("prefill_32k", args.steps, args.warmup, lengths=skewed_lengths())
        pre["workload"] = "skewed_64"
        print(json.dumps(pre))
        return
    from gated_deltanet_scan_amd import synthetic
    w = synthetic.workload(args.workload)
    verify = w.verify_tokens > 0
    print("[bench] prefill %s%s" % (args.workload, " with the verify protocol" if verify else ""),
          file=sys.stderr, flush=True)
    pre = measure_prefill(args.workload, args.steps, args.warmup, verify=verify)
    if args.profile_prefill:
        print(json.dumps(pre))
        return
    extra = {}
    dec = None
    if not args.no_extra:
        print("[bench] decode_64", file=sys.stderr, flush=True)
        dec = measure_decode("decode_64", max(args.steps, 20), args.warmup)
        for name in ("prefill_1k", "prefill_32k", "varlen_16"):
            if name == args.workload:
                continue
            print("[bench] prefill %s" % name, file=sys.stderr, flush=True)
            extra[name] = measure_prefill(name, max(5, min(args.steps, 20)), 10)
        print("[bench] prefill skewed batch (one 32k sequence among 63 of 64 tokens)", file=sys.stderr, flush=True)
        extra["skewed_64"] = measure_prefill("prefill_32k", max(5, min(args.steps, 20)), 10, lengths=skewed_lengths())
        extra["skewed_64"]["workload"] = "skewed_64"
        for tokens in (1024, 32768):
            print("[bench] gated RMSNorm %d tokens" % tokens, file=sys.stderr, flush=True)
            extra["gated_rmsnorm_%d" % tokens] = measure_norm(tokens, max(10, min(args.steps, 50)), 10)
        for tokens in (1024, 32768):
            print("[bench] conv1d %d tokens" % tokens, file=sys.stderr, flush=True)
            extra["conv1d_qkv_%d" % tokens] = measure_conv(tokens, max(10, min(args.steps, 50)), 10)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.workload, args.cpu_seconds, verify=verify)

    what = ("%d sequences of U{256..8192} tokens (%d in all) from their own fp32 states, then per sequence a "
            "%d-token draft from a state snapshot, restore, and re-feed of the accepted prefix"
            % (len(w.lengths), w.total_tokens, w.verify_tokens)) if verify else \
        "%d sequence(s), %d tokens" % (len(w.lengths), w.total_tokens)
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
        "config": {"workload": "%s: Qwen3.5-9B GDN layer prefill, %s; %d QK / %d V heads, dk=dv=%d, chunk %d, "
                               "bf16 q/k/v, fp32 g/beta/state" % (args.workload, what, w.hqk, w.hv, w.dk, w.chunk),
                   "global_batch": len(w.lengths), "seq_len": w.total_tokens},
        "roofline": pre["roofline"],
        "cpu_baseline": cpu,
        "prefill": {k: v for k, v in pre.items() if k != "roofline"},
        "decode": dec,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
