"""GPU parity of the gated RMSNorm (gdn_gated_rmsnorm) against the fp64 oracle
(oracle/output_norm.py).

Cases: both io dtypes, every supported dv, token counts that leave a ragged last
wave, the 1k prefill output shape (1024 tokens x 32 value heads x 128), per-head
output RMS across the pages' 1e-3..2e-2 range with eps = 1e-6 (eps matters there)
and eps = 1, the 32768-token shape the benchmark times (sampled rows), in place on
o and on z, all-zero rows, a large dynamic range, zero tokens, and run-to-run
determinism.  Bars as for the prefill outputs: 1e-4 for fp32 io, 2e-2 for bf16 io
(max-norm relative error per tensor).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_scan_amd as gdn
from gated_deltanet_scan_amd import synthetic as S
from gpu_helpers import rel_err, say
from oracle.output_norm import gated_rmsnorm as ref_norm

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def _run(inp, io, eps, label, inplace=None):
    o, z, w = (inp[k].cuda() for k in ("o", "z", "weight"))
    say(label, "o", tuple(o.shape), io, "eps", eps, "in place on %s" % inplace if inplace else "")
    want = ref_norm(inp["o"], inp["z"], inp["weight"], eps)
    out = {"o": o, "z": z}.get(inplace)
    y = gdn.gated_rmsnorm(o, z, w, eps=eps, out=out)
    torch.cuda.synchronize()
    err = rel_err(y.double().cpu().numpy(), want)
    say(label, "max rel err %.3e" % err)
    assert err <= TOL[io], (label, err)
    return y


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("dv", [32, 64, 128])
@pytest.mark.parametrize("tokens,hv", [(1, 1), (37, 3), (300, 8)])
def test_shapes(io, dv, tokens, hv):
    inp = S.make_norm_inputs(tokens, hv, dv, io, seed=dv * 1000 + tokens + hv)
    _run(inp, io, 1e-6, "shape_t%d_h%d_d%d" % (tokens, hv, dv))


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("eps", [1e-6, 1.0])
def test_prefill_1k_output_shape(io, eps):
    inp = S.make_norm_inputs(1024, 32, 128, io, seed=1001)
    _run(inp, io, eps, "prefill_1k_out")


def test_full_32k_shape_sampled():
    """The size the benchmark times (32768 tokens x 32 value heads x 128, bf16), checked on
    every 61st token row (rows are independent) and the last one."""
    inp = S.make_norm_inputs(32768, 32, 128, torch.bfloat16, seed=3001)
    say("norm_32k", "o", tuple(inp["o"].shape), "bf16, eps 1e-6")
    y = gdn.gated_rmsnorm(inp["o"].cuda(), inp["z"].cuda(), inp["weight"].cuda(), eps=1e-6)
    torch.cuda.synchronize()
    rows = torch.cat([torch.arange(0, 32768, 61), torch.tensor([32767])])
    want = ref_norm(inp["o"][rows], inp["z"][rows], inp["weight"], 1e-6)
    err = rel_err(y[rows.cuda()].double().cpu().numpy(), want)
    say("norm_32k", "%d sampled tokens, max rel err %.3e" % (len(rows), err))
    assert err <= TOL[torch.bfloat16], err


@pytest.mark.parametrize("where", ["o", "z"])
def test_in_place(where):
    inp = S.make_norm_inputs(100, 4, 128, torch.bfloat16, seed=7)
    _run(inp, torch.bfloat16, 1e-6, "in_place", inplace=where)


def test_zero_rows_and_dynamic_range():
    inp = S.make_norm_inputs(64, 4, 128, torch.float32, seed=11)
    inp["o"][3] = 0.0                       # zero rows: y = 0 exactly
    inp["o"][5, 1] *= 1e6                   # large and small rows side by side
    inp["o"][6, 2] *= 1e-3
    y = _run(inp, torch.float32, 1e-6, "zero_rows")
    assert torch.all(y[3] == 0)


def test_zero_tokens_is_a_no_op():
    o = torch.zeros(0, 4, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, device="cuda")
    y = gdn.gated_rmsnorm(o, o, w)
    assert y.shape == (0, 4, 64)


def test_run_to_run_bitwise_determinism():
    inp = S.make_norm_inputs(256, 16, 128, torch.bfloat16, seed=3)
    o, z, w = (inp[k].cuda() for k in ("o", "z", "weight"))
    a = gdn.gated_rmsnorm(o, z, w)
    b = gdn.gated_rmsnorm(o, z, w)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
