"""Shared helpers of the GPU parity tests: run the HIP path and the fp64 oracle on
the same seeded inputs and compare them.

Error metric: per tensor, max |x - x_ref| / max |x_ref| (max-norm relative
error), taken separately for the outputs and the final states, per sequence for
packed batches, and also per (sequence, value head): a head whose outputs are
much smaller than the others' must meet the same relative bar on its own scale.
Bars: 1e-4 for fp32 io; 2e-2 on outputs and 1e-2 on final states for bf16 io
(fp32 state).
"""
import sys

import numpy as np
import torch

import oracle

TOL = {torch.float32: (1e-4, 1e-4), torch.bfloat16: (2e-2, 1e-2)}


def say(*args):
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref))
    if den == 0.0:
        return float(num)
    return float(num / den)


def to_dev(inp, device="cuda"):
    out = {}
    for key, val in inp.items():
        out[key] = val.to(device) if isinstance(val, torch.Tensor) else val
    return out


def gpu_prefill(inp, chunk, scale=None, initial_state="from_inputs", inplace=False, host_offsets=True):
    """Run gdn_prefill_chunked.  host_offsets=True hands the library a host copy of cu_seqlens
    (segmented launch); False passes device offsets only (single launch over a chunk table)."""
    import gated_deltanet_scan_amd as gdn
    d = to_dev(inp)
    s0 = d["initial_state"] if initial_state == "from_inputs" else initial_state
    fs = None
    if inplace:
        fs = s0
    cu = inp["cu_seqlens"].cpu() if host_offsets else d["cu_seqlens"]
    o, S = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, s0,
                               scale=scale, chunk=chunk, final_state=fs)
    torch.cuda.synchronize()
    return o, S


def oracle_prefill(inp, scale=None, initial_state="from_inputs"):
    s0 = inp["initial_state"] if initial_state == "from_inputs" else initial_state
    return oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"], s0,
                              scale=scale)


def check_prefill(o, S, o_ref, S_ref, cu, io_dtype, label=""):
    """Assert the bars per sequence and per (sequence, value head); returns the worst
    per-sequence errors (o, S).  The worst per-head errors are printed."""
    tol_o, tol_s = TOL[io_dtype]
    o = o.double().cpu().numpy()
    S = S.double().cpu().numpy()
    assert np.all(np.isfinite(o)), label + ": non-finite output"
    assert np.all(np.isfinite(S)), label + ": non-finite state"
    cu = [int(x) for x in cu]
    worst_o = worst_s = 0.0
    head_o = head_s = 0.0
    hv = S.shape[1] if S.ndim == 4 else 1
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        eo = rel_err(o[a:b], o_ref[a:b]) if b > a else 0.0
        es = rel_err(S[n], S_ref[n])
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
        assert eo <= tol_o, "%s seq %d: output rel err %.3e > %.1e" % (label, n, eo, tol_o)
        assert es <= tol_s, "%s seq %d: state rel err %.3e > %.1e" % (label, n, es, tol_s)
        for h in range(hv):
            eho = rel_err(o[a:b, h], o_ref[a:b, h]) if b > a else 0.0
            ehs = rel_err(S[n, h], S_ref[n, h])
            head_o, head_s = max(head_o, eho), max(head_s, ehs)
            assert eho <= tol_o, "%s seq %d head %d: output rel err %.3e > %.1e" % (label, n, h, eho, tol_o)
            assert ehs <= tol_s, "%s seq %d head %d: state rel err %.3e > %.1e" % (label, n, h, ehs, tol_s)
    say(label, "worst per-head rel err: o %.3e  S %.3e" % (head_o, head_s))
    return worst_o, worst_s
