"""GPU parity of gdn_prefill_chunked_noalloc, the prefill that allocates nothing (its chunk
workspace is the library's own device scratch), against gdn_prefill_chunked with a workspace,
through the C ABI: two calls in a row, the first on a batch larger than the scratch (cut
into segments sized to it), the second on a smaller one; and the batches it must refuse.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_scan_amd as gdn
from gated_deltanet_scan_amd import synthetic as S
from gpu_helpers import TOL, check_prefill, oracle_prefill, rel_err, say, to_dev

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def _inputs(lengths, seed):
    return S.make_inputs(lengths, 16, 32, 128, 128, torch.bfloat16, seed=seed, g_law="uniform", s0_std=0.05)


def _both(inp, label, host_offsets=True):
    """Run both entry points on the same inputs; compare them to the parity bar (and report
    whether they agree bit for bit), and the no-allocation one to the fp64 oracle."""
    d = to_dev(inp)
    cu = inp["cu_seqlens"] if host_offsets else d["cu_seqlens"]
    T, N = int(inp["cu_seqlens"][-1]), len(inp["cu_seqlens"]) - 1
    need = gdn.workspace_bytes(gdn.make_shape(16, 32, 128, 128, 64, 1, 128 ** -0.5), T, N)
    say(label, "T=%d N=%d workspace %d bytes (scratch %d)" % (T, N, need, SCRATCH_BYTES))
    o_ws, s_ws = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["initial_state"])
    o_na, s_na = gdn.prefill_chunked_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["initial_state"])
    torch.cuda.synchronize()
    tol_o, tol_s = TOL[torch.bfloat16]
    eo = rel_err(o_na.double().cpu().numpy(), o_ws.double().cpu().numpy())
    es = rel_err(s_na.double().cpu().numpy(), s_ws.double().cpu().numpy())
    say(label, "no-alloc vs workspace entry: o %.3e S %.3e, bitwise %s" %
        (eo, es, bool(torch.equal(o_na, o_ws) and torch.equal(s_na, s_ws))))
    assert eo <= tol_o and es <= tol_s
    o_ref, s_ref = oracle_prefill(inp)
    check_prefill(o_na, s_na, o_ref, s_ref, inp["cu_seqlens"], torch.bfloat16, label)
    return need


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    need1 = _both(_inputs([4000, 3000, 4100], seed=41), "noalloc_call1")
    assert need1 > SCRATCH_BYTES, "the first batch must exceed the scratch (segmented)"
    need2 = _both(_inputs([700, 90], seed=42), "noalloc_call2")
    assert need2 < need1


def test_noalloc_batch_within_the_scratch_without_host_offsets():
    _both(_inputs([900, 33, 0, 250], seed=43), "noalloc_device_offsets", host_offsets=False)


def test_noalloc_rejects_batches_beyond_its_scratch():
    """Without host offsets a batch whose workspace exceeds the scratch, and with them a batch
    of more sequences than the scratch holds chunk slots, fail with GDN_ERR_WORKSPACE before
    anything is enqueued: the outputs keep their contents."""
    for lengths, host in (([6000, 6000], False), ([70] * 120, True)):
        inp = _inputs(lengths, seed=44)
        d = to_dev(inp)
        cu = inp["cu_seqlens"] if host else d["cu_seqlens"]
        o = torch.full((sum(lengths), 32, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        fs = torch.full_like(d["initial_state"], float("nan"))
        say("noalloc_reject", "N=%d host offsets %s" % (len(lengths), host))
        with pytest.raises(gdn.GdnError) as ei:
            gdn.prefill_chunked_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["initial_state"],
                                        final_state=fs, out=o)
        assert ei.value.status == 3, ei.value
        torch.cuda.synchronize()
        assert bool(torch.isnan(o).all()) and bool(torch.isnan(fs).all())
