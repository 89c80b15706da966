"""GPU parity of the token-recurrent prefill (gdn_prefill_chunked on a batch whose sequences
are all at most 8 tokens long, with host offsets) against the fp64 oracle.

The library takes this path when cu_seqlens_host shows every sequence at most 8 tokens
long: one launch (profile identifier 12) and no prep or chunk scan.  Cases: every head size
in both io dtypes, lengths 0 .. 8 with a
zero-length sequence, the limit itself (8 tokens: recurrent; 9: chunked), no initial state,
in-place prefix reuse, a short verify block at the Qwen3.5-9B shape (16 sequences of 8
tokens, 16 QK / 32 V heads, dk = dv = 128, bf16) and the gated RMSNorm after it.  Bars as
for the chunked prefill: 1e-4 for fp32 io, 2e-2 (outputs) and 1e-2 (states) for bf16 io.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_scan_amd as gdn
import oracle
from gated_deltanet_scan_amd import synthetic as S
from gpu_helpers import TOL, check_prefill, oracle_prefill, rel_err, say, to_dev
from oracle.output_norm import gated_rmsnorm as ref_norm

pytestmark = pytest.mark.gpu

PROF_PREP, PROF_SCAN, PROF_SHORT = 1, 2, 12


def _launches(fn):
    """Run fn with kernel timing on; returns (result, {kernel id: launches})."""
    gdn.profile_enable(True)
    out = fn()
    torch.cuda.synchronize()
    counts = {kid: gdn.profile_collect(kid)[0] for kid in (PROF_PREP, PROF_SCAN, PROF_SHORT)}
    gdn.profile_enable(False)
    return out, counts


def _run(inp, io, label, chunk=64, initial_state="from_inputs", inplace=False):
    d = to_dev(inp)
    s0 = d["initial_state"] if initial_state == "from_inputs" else initial_state
    say(label, "T=%d" % int(inp["cu_seqlens"][-1]), "N=%d" % (len(inp["cu_seqlens"]) - 1),
        "q", tuple(inp["q"].shape), "v", tuple(inp["v"].shape), io, "in place" if inplace else "")
    fs = s0 if inplace else None
    (o, St), counts = _launches(lambda: gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                            inp["cu_seqlens"].cpu(), s0, chunk=chunk,
                                                            final_state=fs))
    s0_ref = inp["initial_state"] if initial_state == "from_inputs" else (
        None if initial_state is None else initial_state.cpu())
    o_ref, S_ref = oracle_prefill(inp, initial_state=s0_ref)
    eo, es = check_prefill(o, St, o_ref, S_ref, inp["cu_seqlens"], io, label)
    say(label, "launches", counts, "max rel err: o %.3e  S %.3e" % (eo, es))
    return counts


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_short_batch_every_head_size(io, d):
    inp = S.make_inputs([5, 0, 8, 1, 7, 3], 2, 4, d, d, io, seed=900 + d, s0_std=0.05)
    counts = _run(inp, io, "short_d%d" % d)
    assert counts[PROF_SHORT] == 1 and counts[PROF_PREP] == 0 and counts[PROF_SCAN] == 0, counts


@pytest.mark.parametrize("hqk,hv", [(4, 16), (1, 8), (8, 8)])
def test_short_batch_query_key_groups(hqk, hv):
    """4, 8 and 1 value heads per query/key head on the token-recurrent path."""
    inp = S.make_inputs([8, 3, 0, 6], hqk, hv, 128, 128, torch.bfloat16, seed=910 + hv + hqk, s0_std=0.05)
    counts = _run(inp, torch.bfloat16, "short_groups_%d_%d" % (hqk, hv))
    assert counts[PROF_SHORT] == 1 and counts[PROF_PREP] == 0, counts


@pytest.mark.parametrize("longest,recurrent", [(8, True), (9, False)])
def test_limit_of_the_recurrent_path(longest, recurrent):
    inp = S.make_inputs([longest, 7, 2], 2, 4, 128, 128, torch.bfloat16, seed=930 + longest, s0_std=0.05)
    counts = _run(inp, torch.bfloat16, "limit_%d" % longest)
    if recurrent:
        assert counts[PROF_SHORT] == 1 and counts[PROF_PREP] == 0, counts
    else:
        assert counts[PROF_SHORT] == 0 and counts[PROF_PREP] >= 1 and counts[PROF_SCAN] >= 1, counts


def test_short_batch_without_initial_state():
    inp = S.make_inputs([6, 3, 8], 2, 4, 64, 64, torch.float32, seed=941, s0_std=None)
    counts = _run(inp, torch.float32, "short_zero_state", initial_state=None)
    assert counts[PROF_SHORT] == 1, counts


def test_short_batch_in_place_prefix_reuse():
    inp = S.make_inputs([8, 4, 0, 7], 2, 4, 128, 128, torch.bfloat16, seed=947, s0_std=0.05)
    counts = _run(inp, torch.bfloat16, "short_in_place", inplace=True)
    assert counts[PROF_SHORT] == 1, counts


def test_short_verify_block_at_the_model_shape():
    """A verify block of 8 tokens per sequence for 16 sequences, correlated keys with weak
    decay from nonzero states (the hardest case for accumulated rounding)."""
    inp = S.make_inputs([8] * 16, 16, 32, 128, 128, torch.bfloat16, seed=953, s0_std=0.05,
                        key_law="correlated", g_law="weak")
    counts = _run(inp, torch.bfloat16, "verify_16x8")
    assert counts[PROF_SHORT] == 1 and counts[PROF_PREP] == 0, counts


def test_gated_rmsnorm_after_the_recurrent_path():
    inp = S.make_inputs([8, 5, 2, 1], 16, 32, 128, 128, torch.bfloat16, seed=959, s0_std=0.05)
    T, hv, dv = int(inp["cu_seqlens"][-1]), 32, 128
    gen = torch.Generator().manual_seed(961)
    z = (2.0 * torch.randn(T, hv, dv, generator=gen)).to(torch.bfloat16)
    w = torch.empty(dv).uniform_(0.5, 1.5, generator=gen).float()
    d = to_dev(inp)
    say("short_norm", "T=%d" % T)
    gdn.profile_enable(True)
    y, S_gpu = gdn.prefill_chunked_gated_rmsnorm(d["q"], d["k"], d["v"], d["g"], d["beta"], z.cuda(), w.cuda(),
                                                 inp["cu_seqlens"].cpu(), d["initial_state"], eps=1e-6, chunk=64)
    torch.cuda.synchronize()
    short_launches, _ = gdn.profile_collect(PROF_SHORT)
    norm_launches, _ = gdn.profile_collect(5)
    gdn.profile_enable(False)
    o_ref, S_ref = oracle.gdn_forward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                                      inp["initial_state"])
    y_ref = ref_norm(o_ref, z, w, 1e-6)
    ey = rel_err(y.double().cpu().numpy(), y_ref)
    es = rel_err(S_gpu.double().cpu().numpy(), S_ref)
    say("short_norm", "launches short %d norm %d; max rel err y %.3e  S %.3e" % (short_launches, norm_launches,
                                                                               ey, es))
    tol_o, tol_s = TOL[torch.bfloat16]
    assert short_launches == 1 and norm_launches == 1
    assert ey <= tol_o and es <= tol_s, (ey, es)


@pytest.mark.parametrize("chunk", [16, 64])
def test_fp32_at_dk_128_any_length(chunk):
    """fp32 io at dk = dv = 128 has no chunked kernel: every call runs the token-recurrent
    kernel, block of 8 tokens after block, whatever the lengths (here up to 300 tokens, with
    and without host offsets)."""
    inp = S.make_inputs([300, 1, 0, 17, 64], 2, 4, 128, 128, torch.float32, seed=971 + chunk, s0_std=0.05)
    counts = _run(inp, torch.float32, "fp32_d128_c%d" % chunk, chunk=chunk)
    assert counts[PROF_SHORT] == 1 and counts[PROF_PREP] == 0 and counts[PROF_SCAN] == 0, counts
    d = to_dev(inp)
    say("fp32_d128 device offsets")
    o, St = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["initial_state"],
                                chunk=chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(o, St, o_ref, S_ref, inp["cu_seqlens"], torch.float32, "fp32_d128_device_offsets")
