"""GPU parity of the chunked prefill with the gated RMSNorm on its output rows
(gdn_prefill_chunked_gated_rmsnorm) against the fp64 oracles: the recurrence
(oracle.gdn_forward), then the norm (oracle/output_norm.py) on its fp64 output.

Cases: a batch on the whole-head scan (more than 64 (sequence, head) pairs, dk =
dv = 128, bf16), a batch on the row-split scan, an fp32 batch, and the 16-sequence
varlen workload (two segments, sampled rows).  The norm runs once, in place, after
the scans (its launch count is checked).  Bars: 2e-2 (bf16 io) and 1e-4 (fp32 io)
on y, and the prefill's own bars on the final states.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_scan_amd as gdn
import oracle
from gated_deltanet_scan_amd import synthetic as S
from gpu_helpers import TOL, rel_err, say, to_dev
from oracle.output_norm import gated_rmsnorm as ref_norm

pytestmark = pytest.mark.gpu


def _gate_and_weight(T, hv, dv, io, seed):
    gen = torch.Generator().manual_seed(seed)
    z = (2.0 * torch.randn(T, hv, dv, generator=gen)).to(io)
    w = torch.empty(dv).uniform_(0.5, 1.5, generator=gen).float()
    return z, w


def _run(inp, io, chunk, label, rows=None):
    T = int(inp["cu_seqlens"][-1])
    hv, dv = inp["v"].shape[1], inp["v"].shape[2]
    z, w = _gate_and_weight(T, hv, dv, io, seed=T + hv)
    d = to_dev(inp)
    say(label, "T=%d" % T, "N=%d" % (len(inp["cu_seqlens"]) - 1), "q", tuple(inp["q"].shape), io)
    gdn.profile_enable(True)
    y, S_gpu = gdn.prefill_chunked_gated_rmsnorm(d["q"], d["k"], d["v"], d["g"], d["beta"], z.cuda(), w.cuda(),
                                                 inp["cu_seqlens"].cpu(), d["initial_state"], eps=1e-6, chunk=chunk)
    torch.cuda.synchronize()
    norm_launches, _ = gdn.profile_collect(5)
    gdn.profile_enable(False)
    o_ref, S_ref = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                                      inp["initial_state"])
    sel = np.arange(T) if rows is None else rows
    y_ref = ref_norm(o_ref[sel], z[sel], w, 1e-6)
    ey = rel_err(y[torch.as_tensor(sel).cuda()].double().cpu().numpy(), y_ref)
    es = rel_err(S_gpu.double().cpu().numpy(), S_ref)
    say(label, "norm kernel launches %d; max rel err y %.3e  S %.3e" % (norm_launches, ey, es))
    tol_o, tol_s = TOL[io]
    assert ey <= tol_o and es <= tol_s, (label, ey, es)
    return norm_launches


def test_norm_after_the_whole_head_scan():
    inp = S.make_inputs([300, 64, 1, 190], 16, 32, 128, 128, torch.bfloat16, seed=71, s0_std=0.05)
    assert _run(inp, torch.bfloat16, 64, "norm_after_wide") == 1


def test_norm_after_the_row_split_scan():
    inp = S.make_inputs([500, 37], 2, 4, 128, 128, torch.bfloat16, seed=72, s0_std=0.05)
    assert _run(inp, torch.bfloat16, 64, "norm_after_rows") == 1


def test_norm_after_the_fp32_scan():
    inp = S.make_inputs([129, 16, 3], 2, 4, 64, 64, torch.float32, seed=73, s0_std=0.05)
    assert _run(inp, torch.float32, 64, "norm_after_fp32") == 1


def test_norm_varlen_16_workload_sampled():
    w = S.workload("varlen_16")
    inp = S.make_workload_inputs(w)
    T = w.total_tokens
    rows = np.unique(np.concatenate([np.arange(0, T, 37), np.asarray(inp["cu_seqlens"][1:]) - 1]))
    assert _run(inp, torch.bfloat16, 64, "norm_varlen16", rows=rows) == 1
