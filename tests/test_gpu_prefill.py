"""GPU parity of the chunked prefill (gdn_prefill_chunked) against the fp64 oracle.

Cases: the five workloads at their full sizes (the tiny fp32 one, 1k prefill,
32k prefill, the 16-sequence varlen batch), lengths below, at and above the
chunk, multi-chunk ragged tails, zero-length sequences, batches without tokens
(and without sequences), batches at and past
the 4096-sequence ordering limit, every supported head size and chunk length
in both io dtypes, the strong-decay (-6.72) segment,
a weak-decay long-memory stress (also at the full 32k shape), highly
correlated keys, scale 0, in-place prefix reuse and run-to-run determinism.
With host offsets, a batch whose sequences are all at most 8 tokens long takes the
token-recurrent path instead (tests/test_gpu_short_prefill.py); the device-offset runs
keep the chunked kernels covered at those lengths.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_scan_amd as gdn
from gated_deltanet_scan_amd import synthetic as S
from gpu_helpers import check_prefill, gpu_prefill, oracle_prefill, rel_err, say

pytestmark = pytest.mark.gpu


def _case(lengths, hqk, hv, d, io, seed, g_law="uniform", s0_std=0.05, strong=False, key_law="gaussian"):
    return S.make_inputs(lengths, hqk, hv, d, d, io, seed=seed, g_law=g_law, s0_std=s0_std,
                         strong_segment=strong, key_law=key_law)


def _run(inp, chunk, io, label, scale=None, host_offsets=True):
    say(label, "T=%d" % int(inp["cu_seqlens"][-1]), "N=%d" % (len(inp["cu_seqlens"]) - 1),
        "q", tuple(inp["q"].shape), "v", tuple(inp["v"].shape), "chunk", chunk, io,
        "host offsets" if host_offsets else "device offsets")
    o, St = gpu_prefill(inp, chunk, scale=scale, host_offsets=host_offsets)
    o_ref, S_ref = oracle_prefill(inp, scale=scale)
    eo, es = check_prefill(o, St, o_ref, S_ref, inp["cu_seqlens"], io, label)
    say(label, "max rel err: o %.3e  S %.3e" % (eo, es))
    return eo, es


def test_tiny_fp32_workload():
    w = S.workload("tiny_fp32")
    _run(S.make_workload_inputs(w), w.chunk, w.io_dtype, "tiny_fp32")


def test_prefill_1k_workload():
    w = S.workload("prefill_1k")
    _run(S.make_workload_inputs(w), w.chunk, w.io_dtype, "prefill_1k")


@pytest.mark.parametrize("host_offsets", [True, False])
def test_prefill_32k_workload(host_offsets):
    w = S.workload("prefill_32k")
    _run(S.make_workload_inputs(w), w.chunk, w.io_dtype, "prefill_32k", host_offsets=host_offsets)


@pytest.mark.parametrize("host_offsets", [True, False])
def test_varlen_16_workload(host_offsets):
    w = S.workload("varlen_16")
    _run(S.make_workload_inputs(w), w.chunk, w.io_dtype, "varlen_16", host_offsets=host_offsets)


@pytest.mark.parametrize("host_offsets", [True, False])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 127, 128, 129])
@pytest.mark.parametrize("io,d,chunk", [(torch.float32, 32, 16), (torch.bfloat16, 128, 64)])
def test_lengths_around_the_chunk(T, io, d, chunk, host_offsets):
    """With host offsets the length 1 takes the token-recurrent path; with device offsets every
    length runs the chunked kernels."""
    _run(_case([T], 1, 2, d, io, seed=100 + T), chunk, io, "len%d_d%d_c%d" % (T, d, chunk),
         host_offsets=host_offsets)


@pytest.mark.parametrize("host_offsets", [True, False])
@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,chunk", [(32, 16), (64, 16), (32, 64), (64, 64), (128, 64)])
def test_every_kernel_instance(io, d, chunk, host_offsets):
    """Every (io dtype, head size, chunk) instance; fp32 io at dk = 128 runs the token-recurrent
    kernel at any length."""
    lengths = [3 * chunk + 5, chunk, 1, 2 * chunk - 1]
    _run(_case(lengths, 2, 4, d, io, seed=7 * d + chunk), chunk, io, "inst_d%d_c%d" % (d, chunk),
         host_offsets=host_offsets)


@pytest.mark.parametrize("nseq", [40, 160])
def test_wide_slices_many_sequences(nseq):
    """Enough (sequence, head) pairs that the scan takes whole 128-column heads per workgroup
    (the wide-batch kernel) instead of the row-split one."""
    gen = torch.Generator().manual_seed(nseq)
    lengths = [int(x) for x in torch.randint(0, 200, (nseq,), generator=gen)]
    for host_offsets in (True, False):
        _run(_case(lengths, 2, 4, 128, torch.bfloat16, seed=500 + nseq), 64, torch.bfloat16,
             "wide_n%d" % nseq, host_offsets=host_offsets)


@pytest.mark.parametrize("hqk,hv,nseq", [(8, 8, 10), (4, 16, 6), (2, 16, 5), (1, 4, 2)])
def test_query_key_groups(hqk, hv, nseq):
    """1, 4 and 8 value heads per query/key head (the other cases use 2): the prep deals a
    group's value heads to one XCD and forms the group's Gram products per value head, and the
    scans read the group's q and k rows.  Whole-head scan (80-96 pairs) and row-split scan (8
    pairs), sequences of several chunks with ragged ends, both launch modes."""
    gen = torch.Generator().manual_seed(hqk * 100 + hv)
    lengths = [int(x) for x in torch.randint(1, 300, (nseq,), generator=gen)]
    inp = _case(lengths, hqk, hv, 128, torch.bfloat16, seed=40 + hv + hqk)
    for host_offsets in (True, False):
        _run(inp, 64, torch.bfloat16, "groups_%d_%d" % (hqk, hv), host_offsets=host_offsets)


@pytest.mark.parametrize("nseq", [4096, 4100])
def test_batches_at_and_past_the_ordering_limit(nseq):
    """Up to 4096 sequences a ranking kernel orders the batch so that the scans start the
    longest sequences first; past that the scans take the sequences in batch order.  Both
    sides of the limit, with host and device offsets: mostly sequences of 0..4 tokens, with a
    130-token one every 997, one value head per query/key head (4096+ pairs: the whole-head
    scan)."""
    gen = torch.Generator().manual_seed(nseq)
    lengths = [int(x) for x in torch.randint(0, 5, (nseq,), generator=gen)]
    for i in range(0, nseq, 997):
        lengths[i] = 130
    inp = _case(lengths, 1, 1, 128, torch.bfloat16, seed=700 + nseq)
    for host_offsets in (True, False):
        _run(inp, 64, torch.bfloat16, "ordering_n%d" % nseq, host_offsets=host_offsets)


def test_long_sequence_spans_several_segments():
    """With host offsets the launch is cut into segments of local chunks; 20000 tokens of one
    sequence with 32 value heads span several of them (state carried in final_state)."""
    _run(_case([20000, 300], 16, 32, 128, torch.bfloat16, seed=29), 64, torch.bfloat16, "segments")


def test_zero_length_sequences_pass_state_through():
    lengths = [0, 70, 0, 0, 5, 0]
    inp = _case(lengths, 2, 4, 128, torch.bfloat16, seed=21)
    _run(inp, 64, torch.bfloat16, "zero_lengths")
    o, St = gpu_prefill(inp, 64)
    s0 = inp["initial_state"]
    for n in (0, 2, 3, 5):
        assert torch.equal(St[n].cpu(), s0[n]), "empty sequence %d changed its state" % n


@pytest.mark.parametrize("host_offsets", [True, False])
def test_batches_without_tokens(host_offsets):
    """No tokens at all: every final state is its initial state bit for bit (also in place),
    or zeros without initial states (written over a NaN-filled buffer); a batch of no
    sequences is a no-op."""
    import gated_deltanet_scan_amd as gdn
    inp = _case([0, 0, 0], 1, 2, 128, torch.bfloat16, seed=31)
    say("no_tokens", "host offsets" if host_offsets else "device offsets")
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    cu = inp["cu_seqlens"] if host_offsets else d["cu_seqlens"]
    o, St = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["initial_state"])
    torch.cuda.synchronize()
    assert o.shape[0] == 0
    assert torch.equal(St.cpu(), inp["initial_state"])
    state = d["initial_state"].clone()
    gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, state, final_state=state)
    torch.cuda.synchronize()
    assert torch.equal(state.cpu(), inp["initial_state"])
    fs = torch.full_like(d["initial_state"], float("nan"))
    o, St = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, None, final_state=fs)
    torch.cuda.synchronize()
    assert St.data_ptr() == fs.data_ptr()
    assert not bool(torch.isnan(St).any()) and int(torch.count_nonzero(St)) == 0
    cu0 = torch.zeros(1, dtype=torch.int32)
    e = {k: d[k][:0] for k in ("q", "k", "v", "g", "beta")}
    o, St = gdn.prefill_chunked(e["q"], e["k"], e["v"], e["g"], e["beta"], cu0 if host_offsets else cu0.cuda(), None)
    torch.cuda.synchronize()
    assert o.shape[0] == 0 and St.shape[0] == 0


def test_zero_initial_state_and_gqa_groups_of_four():
    inp = _case([150, 90], 2, 8, 64, torch.bfloat16, seed=22, s0_std=None)
    _run(inp, 64, torch.bfloat16, "gqa4_zero_s0")


def test_strong_decay_segment_stays_finite():
    """Tokens 64..127 of head 0 decay by exactly -6.72 per step: the upper-triangle exponent
    would overflow fp32 without log-space masking."""
    inp = _case([256], 1, 2, 128, torch.bfloat16, seed=23, strong=True)
    assert float(inp["g"][100, 0]) == np.float32(-6.72)
    _run(inp, 64, torch.bfloat16, "strong_decay")


def test_weak_decay_long_memory():
    """g ~ -U(0, 0.02): the state remembers thousands of tokens, so rounding can accumulate
    across many chunks."""
    inp = _case([4096], 1, 2, 128, torch.bfloat16, seed=24, g_law="weak")
    _run(inp, 64, torch.bfloat16, "weak_decay")


def test_weak_decay_at_the_32k_shape():
    """The 32k prefill shape (one 32768-token sequence, 16 query/key -> 32 value heads, d = 128,
    initial state N(0, 0.05^2)) with weak decay g ~ -U(0, 0.02): the state remembers thousands
    of tokens, so rounding on the 512-chunk chain accumulates instead of being forgotten within
    a chunk as under the workload's strong decay.  Both launch modes."""
    inp = _case([32768], 16, 32, 128, torch.bfloat16, seed=1013, g_law="weak")
    for host_offsets in (True, False):
        _run(inp, 64, torch.bfloat16, "weak_decay_32k", host_offsets=host_offsets)


@pytest.mark.parametrize("g_law", ["uniform", "weak"])
def test_correlated_keys_through_the_solve(g_law):
    """Highly correlated keys (one shared direction per head plus 10% noise, normalised; the
    NPU page, section "How it works", warns that real keys are highly correlated and break
    naive triangular inverses) at the 1k prefill shape: the off-diagonal entries of the
    chunk's triangular system are near beta, so the fp32 solve and the bf16 inverse carry
    large, alternating entries.  With the workload's decay law and with weak decay."""
    inp = _case([1024], 16, 32, 128, torch.bfloat16, seed=1011, g_law=g_law, s0_std=None, strong=True,
                key_law="correlated")
    k = inp["k"].double()
    cos = (k[1:] * k[:-1]).sum(-1)
    assert float(cos.mean()) > 0.95, "keys are not correlated"
    _run(inp, 64, torch.bfloat16, "correlated_keys_" + g_law)


def test_scale_argument():
    inp = _case([100], 1, 2, 64, torch.float32, seed=25)
    _run(inp, 64, torch.float32, "scale_0.3", scale=0.3)


@pytest.mark.parametrize("io,d", [(torch.float32, 64), (torch.bfloat16, 128)])
def test_scale_zero(io, d):
    """scale = 0: every output is exactly zero and the state is that of any other scale (the
    scale multiplies the queries only).  Sequences of several chunks, both launch modes, and
    for bf16 both scan kernels (8 and 80 (sequence, head) pairs)."""
    for lengths, hv in (([200, 70], 4), ([130] * 20, 4)):
        if io == torch.float32 and len(lengths) > 2:
            continue
        inp = _case(lengths, 2, hv, d, io, seed=33 + len(lengths))
        for host_offsets in (True, False):
            o, St = gpu_prefill(inp, 64, scale=0.0, host_offsets=host_offsets)
            assert int(torch.count_nonzero(o)) == 0, "scale 0 gave nonzero outputs"
            o_ref, S_ref = oracle_prefill(inp, scale=0.0)
            check_prefill(o, St, o_ref, S_ref, inp["cu_seqlens"], io, "scale_0_n%d" % len(lengths))


def test_in_place_prefix_reuse_matches_two_calls():
    """Prefill [0, a) then [a, T) from the carried state (final_state aliasing initial_state)
    matches the oracle on [0, T)."""
    inp = _case([300], 2, 4, 128, torch.bfloat16, seed=26)
    a = 130
    part1 = {k: (v[:a].contiguous() if k in ("q", "k", "v", "g", "beta") else v) for k, v in inp.items()}
    part1["cu_seqlens"] = torch.tensor([0, a], dtype=torch.int32)
    part2 = {k: (v[a:].contiguous() if k in ("q", "k", "v", "g", "beta") else v) for k, v in inp.items()}
    part2["cu_seqlens"] = torch.tensor([0, 300 - a], dtype=torch.int32)
    import gated_deltanet_scan_amd as gdn
    state = inp["initial_state"].cuda().clone()
    outs = []
    for part in (part1, part2):
        say("prefix_reuse part", tuple(part["q"].shape))
        d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in part.items()}
        o, st = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], state,
                                    final_state=state)
        assert st.data_ptr() == state.data_ptr()
        outs.append(o)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp)
    check_prefill(torch.cat(outs), state, o_ref, S_ref, inp["cu_seqlens"], torch.bfloat16, "prefix_reuse")


@pytest.mark.parametrize("lengths,hqk,hv", [([700, 33], 2, 4), ([300, 5, 0, 129] * 5, 2, 4)])
def test_run_to_run_bitwise_determinism(lengths, hqk, hv):
    """Two runs give the same bits, for the row-split scan (8 pairs) and the whole-head scan
    (80 pairs), with host offsets (segmented launches) and device offsets (one launch over the
    chunk table); the two launch modes also agree bit for bit (same per-chunk arithmetic, the
    state carried in fp32 between segments)."""
    inp = _case(lengths, hqk, hv, 128, torch.bfloat16, seed=27)
    say("determinism", "N=%d" % len(lengths), "pairs=%d" % (len(lengths) * hv))
    runs = {}
    for host_offsets in (True, False):
        o1, s1 = gpu_prefill(inp, 64, host_offsets=host_offsets)
        o2, s2 = gpu_prefill(inp, 64, host_offsets=host_offsets)
        assert torch.equal(o1, o2) and torch.equal(s1, s2)
        runs[host_offsets] = (o1, s1)
    assert torch.equal(runs[True][0], runs[False][0]) and torch.equal(runs[True][1], runs[False][1])


def test_chunk_length_does_not_change_the_answer():
    """The chunked form is exact, so chunk 16 and chunk 64 agree with each other to rounding."""
    inp = _case([257], 1, 2, 32, torch.float32, seed=28)
    o16, s16 = gpu_prefill(inp, 16)
    o64, s64 = gpu_prefill(inp, 64)
    assert rel_err(o16.double().cpu(), o64.double().cpu()) < 1e-4
    assert rel_err(s16.double().cpu(), s64.double().cpu()) < 1e-4


def test_workspace_smaller_than_the_batch():
    """With host offsets a workspace smaller than gdn_prefill_workspace_bytes() is accepted: the
    batch runs in segments sized to it.  The whole-batch workspace, the size of the plan
    (gdn_prefill_workspace_bytes_for) and a workspace of 5 chunk slots per sequence give the
    same bits (per-chunk arithmetic does not depend on the plan; the state is carried in fp32
    between segments), and agree with the oracle."""
    import gated_deltanet_scan_amd as gdn
    from gated_deltanet_scan_amd import binding
    lengths = [3000, 700, 1500, 64]
    inp = _case(lengths, 2, 4, 128, torch.bfloat16, seed=31)
    d = {key: (val.cuda() if isinstance(val, torch.Tensor) else val) for key, val in inp.items()}
    cu = inp["cu_seqlens"].cpu()
    sh = binding.make_shape(2, 4, 128, 128, 64, binding.GDN_DTYPE_BF16, 128 ** -0.5)
    full = gdn.workspace_bytes(sh, int(cu[-1]), len(lengths))
    plan = gdn.workspace_bytes_for(sh, cu)
    slot = 4 * ((128 + 64) * 64 * 2 + 4 * 64 * 4)
    tight = 256 + len(lengths) * 5 * slot
    assert tight < plan <= full, (tight, plan, full)
    runs = []
    for nbytes in (full, plan, tight):
        say("workspace", nbytes, "bytes of", full)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        o, st = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["initial_state"], chunk=64,
                                    workspace=ws)
        torch.cuda.synchronize()
        runs.append((o, st))
    for o, st in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(st, runs[0][1])
    o_ref, s_ref = oracle_prefill(inp)
    check_prefill(runs[2][0], runs[2][1], o_ref, s_ref, inp["cu_seqlens"], torch.bfloat16, "tight_workspace")
    # one slot short of a chunk per sequence: refused, outputs untouched
    ws = torch.empty(256 + len(lengths) * slot - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(gdn.GdnError):
        gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["initial_state"], chunk=64,
                            workspace=ws)


def test_planned_workspace_at_the_32k_shape():
    """prefill_32k with the workspace of its plan (128-chunk segments, about a quarter of the
    whole-batch size) gives the bits of the whole-batch workspace."""
    import gated_deltanet_scan_amd as gdn
    from gated_deltanet_scan_amd import binding
    w = S.workload("prefill_32k")
    inp = S.make_workload_inputs(w)
    d = {key: (val.cuda() if isinstance(val, torch.Tensor) else val) for key, val in inp.items()}
    cu = inp["cu_seqlens"].cpu()
    sh = binding.make_shape(w.hqk, w.hv, w.dk, w.dv, w.chunk, binding.GDN_DTYPE_BF16, w.dk ** -0.5)
    full = gdn.workspace_bytes(sh, int(cu[-1]), 1)
    plan = gdn.workspace_bytes_for(sh, cu)
    say("prefill_32k workspace", plan, "of", full)
    assert plan < full // 3
    runs = []
    for nbytes in (full, plan):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        runs.append(gdn.prefill_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["initial_state"],
                                        chunk=w.chunk, workspace=ws))
        torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])


@pytest.mark.parametrize("hv", [4, 32])
def test_batch_already_longest_first(hv):
    """Host offsets whose chunk counts never increase along the batch: the scans take the batch
    order as it stands (no ordering launch).  Same bits as with device offsets (ordered on the
    device), and parity with the oracle; with 32 value heads the whole-head scan runs."""
    lengths = [700, 300, 300, 65, 64, 1, 0]
    inp = _case(lengths, hv // 2, hv, 128, torch.bfloat16, seed=33)
    o_h, s_h = gpu_prefill(inp, 64, host_offsets=True)
    o_d, s_d = gpu_prefill(inp, 64, host_offsets=False)
    assert torch.equal(o_h, o_d) and torch.equal(s_h, s_d)
    _run(inp, 64, torch.bfloat16, "longest_first_hv%d" % hv)


@pytest.mark.parametrize("host_offsets", [True, False])
def test_skewed_batch(host_offsets):
    """One long sequence among short ones.  With host offsets its chains run in the row-split
    scan and the short sequences in the whole-head scan (two launches over disjoint ranks);
    with device offsets everything runs in the whole-head scan.  Both against the oracle."""
    lengths = [8192] + [64] * 20 + [37, 0]
    _run(_case(lengths, 16, 32, 128, torch.bfloat16, seed=35), 64, torch.bfloat16, "skewed",
         host_offsets=host_offsets)


def test_skewed_batch_windows():
    """A long sequence whose row-split chain spans several windows of local chunks, each with a
    chunk table of its own; a second sequence reaches past the first window, the rest (one
    chunk or none) end in it.  At this shape (16 QK / 32 V heads, dk = dv = 128, bf16) the
    375-chunk sequence takes windows of 125 chunks: three table launches and three row-split
    scans, and the whole-head scan of the other sequences in the two windows that hold their
    chunks (the third holds none).  Against the oracle, states and outputs."""
    import gated_deltanet_scan_amd as gdn
    lengths = [24000, 9000] + [64] * 20 + [37, 0, 1]
    inp = _case(lengths, 16, 32, 128, torch.bfloat16, seed=36)
    gdn.profile_enable(True)
    try:
        eo, es = _run(inp, 64, torch.bfloat16, "skewed_windows")
        torch.cuda.synchronize()
        counts = {kid: gdn.profile_collect(kid)[0] for kid in (0, 8, 9)}
    finally:
        gdn.profile_enable(False)
    say("skewed_windows", "launches: chunk table %d, row-split scan %d, whole-head scan %d"
        % (counts[0], counts[8], counts[9]))
    assert counts == {0: 3, 8: 3, 9: 2}, counts
