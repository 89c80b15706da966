"""GPU parity of the decode step, the state snapshot and the verify / rollback /
re-feed protocol against the fp64 oracle.

The protocol (NPU page, "New in v2"): the recurrent state cannot be rewound,
so it is snapshotted before a 16-token draft is checked in one pass; after
m tokens are accepted the state is restored from the snapshot and the m
accepted tokens are fed again.  Expected: the final state equals the oracle
run over the L + m tokens.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_scan_amd as gdn
import oracle
from gated_deltanet_scan_amd import synthetic as S
from gpu_helpers import TOL, check_prefill, gpu_prefill, oracle_prefill, rel_err, say, to_dev

pytestmark = pytest.mark.gpu


def _decode_inputs(n, hqk, hv, d, io, seed, s0_std=0.05, g_law="uniform"):
    return S.make_inputs([1] * n, hqk, hv, d, d, io, seed=seed, g_law=g_law, s0_std=s0_std)


def _check_decode(inp, io, label, scale=None):
    n = len(inp["cu_seqlens"]) - 1
    say(label, "decode N=%d" % n, tuple(inp["q"].shape), tuple(inp["v"].shape), io)
    d = to_dev(inp)
    state = d["initial_state"].clone()
    o = gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, scale=scale)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp, scale=scale)
    tol_o, tol_s = TOL[io]
    o = o.double().cpu().numpy()
    st = state.double().cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(st))
    eo, es = rel_err(o, o_ref), rel_err(st, S_ref)
    say(label, "max rel err: o %.3e  S %.3e" % (eo, es))
    assert eo <= tol_o and es <= tol_s, (eo, es)
    # per sequence, and per (sequence, value head) on the head's own scale
    for i in range(n):
        assert rel_err(o[i], o_ref[i]) <= tol_o
        assert rel_err(st[i], S_ref[i]) <= tol_s
        for h in range(o.shape[1]):
            assert rel_err(o[i, h], o_ref[i, h]) <= tol_o, (label, i, h)
            assert rel_err(st[i, h], S_ref[i, h]) <= tol_s, (label, i, h)


def test_decode_64_workload():
    w = S.workload("decode_64")
    _check_decode(S.make_workload_inputs(w), w.io_dtype, "decode_64")


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_decode_every_head_size(io, d):
    _check_decode(_decode_inputs(5, 2, 4, d, io, seed=300 + d), io, "decode_d%d" % d)


def test_decode_large_batch_and_empty_batch():
    """A batch of 3000 sequences (one query/key head, one value head each: 12000 waves) at
    parity, then a batch of no sequences, which must leave the state untouched."""
    _check_decode(_decode_inputs(3000, 1, 1, 128, torch.bfloat16, seed=305), torch.bfloat16, "decode_n3000")
    inp = _decode_inputs(2, 1, 2, 128, torch.bfloat16, seed=306)
    d = to_dev(inp)
    state = d["initial_state"].clone()
    o = gdn.decode_step(d["q"][:0], d["k"][:0], d["v"][:0], d["g"][:0], d["beta"][:0], state[:0])
    torch.cuda.synchronize()
    assert o.shape[0] == 0 and torch.equal(state.cpu(), inp["initial_state"])


@pytest.mark.parametrize("hqk,hv", [(4, 16), (1, 8), (8, 8)])
def test_decode_query_key_groups(hqk, hv):
    """4, 8 and 1 value heads per query/key head (the cases above use 1 and 2): each value
    head's wave reads its group's query and key rows."""
    _check_decode(_decode_inputs(6, hqk, hv, 128, torch.bfloat16, seed=320 + hv + hqk), torch.bfloat16,
                  "decode_groups_%d_%d" % (hqk, hv))


def test_decode_strong_decay_and_scale():
    inp = _decode_inputs(3, 1, 2, 128, torch.bfloat16, seed=310)
    inp["g"][:] = S.STRONG_DECAY
    _check_decode(inp, torch.bfloat16, "decode_strong", scale=0.5)


def test_prefill_then_decode_handoff():
    """Chunked prefill of L tokens, then m one-token decode steps from its final state, equals the
    oracle over L + m tokens (the chunked-prefill -> sequential-decode handoff)."""
    L, m = 200, 5
    full = S.make_inputs([L + m], 2, 4, 128, 128, torch.bfloat16, seed=320, s0_std=0.05)
    pre = {k: (v[:L].contiguous() if k in ("q", "k", "v", "g", "beta") else v) for k, v in full.items()}
    pre["cu_seqlens"] = torch.tensor([0, L], dtype=torch.int32)
    say("handoff prefill L=%d" % L)
    o_pre, state = gpu_prefill(pre, 64)
    dev = to_dev(full)
    outs = [o_pre]
    for t in range(L, L + m):
        say("handoff decode t=%d" % t)
        outs.append(gdn.decode_step(dev["q"][t:t + 1].contiguous(), dev["k"][t:t + 1].contiguous(),
                                    dev["v"][t:t + 1].contiguous(), dev["g"][t:t + 1].contiguous(),
                                    dev["beta"][t:t + 1].contiguous(), state))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(full)
    check_prefill(torch.cat(outs), state, o_ref, S_ref, full["cu_seqlens"], torch.bfloat16, "handoff")


def test_snapshot_gather_scatter_and_bounds():
    n, hv, d = 6, 4, 32
    src = torch.randn(n, hv, d, d, device="cuda")
    dst = torch.zeros(4, hv, d, d, device="cuda")
    rows = torch.tensor([5, 0, 3, 99], dtype=torch.int32, device="cuda")   # 99: out of range, skipped
    say("snapshot gather")
    gdn.state_snapshot(src, dst, src_rows=rows)
    torch.cuda.synchronize()
    assert torch.equal(dst[0], src[5]) and torch.equal(dst[1], src[0]) and torch.equal(dst[2], src[3])
    assert torch.equal(dst[3], torch.zeros_like(dst[3]))
    back = torch.zeros_like(src)
    say("snapshot scatter")
    gdn.state_snapshot(dst, back, dst_rows=rows[:3].contiguous(), num_rows=3)
    torch.cuda.synchronize()
    assert torch.equal(back[5], src[5]) and torch.equal(back[0], src[0]) and torch.equal(back[3], src[3])
    assert torch.equal(back[1], torch.zeros_like(back[1]))


def _slice_tokens(inp, lengths_take, offsets):
    """Per sequence n take tokens [offsets[n], offsets[n] + lengths_take[n]) of a packed batch."""
    idx = torch.cat([torch.arange(int(o), int(o) + int(t)) for o, t in zip(offsets, lengths_take)]) \
        if sum(lengths_take) else torch.zeros(0, dtype=torch.long)
    out = {k: (v[idx].contiguous() if k in ("q", "k", "v", "g", "beta") else v) for k, v in inp.items()}
    cu = torch.zeros(len(lengths_take) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths_take, dtype=torch.int64), 0).to(torch.int32)
    out["cu_seqlens"] = cu
    return out


def _verify_protocol(w, accepted, label, host_offsets=False):
    """Packed prefill -> snapshot -> one 16-token verify block per sequence -> restore -> re-feed
    the accepted prefix.  Checks the prompt outputs, the verify outputs, the re-fed outputs and the
    final states (per sequence and per value head).  With host offsets, a re-feed of at most 8
    tokens per sequence takes the token-recurrent prefill; the other calls, and every call with
    device offsets, the chunked kernels."""
    V = w.verify_tokens
    n = len(w.lengths)
    # one draw holds prompt + verify tokens of every sequence; sequences are split below
    total = [L + V for L in w.lengths]
    allx = S.make_inputs(total, w.hqk, w.hv, w.dk, w.dv, w.io_dtype, seed=w.seed, g_law=w.g_law,
                         s0_std=w.s0_std, strong_segment=w.strong_segment)
    starts = [int(x) for x in allx["cu_seqlens"][:-1]]
    prompt = _slice_tokens(allx, w.lengths, starts)
    verify = _slice_tokens(allx, [V] * n, [s + L for s, L in zip(starts, w.lengths)])
    refeed = _slice_tokens(allx, accepted, [s + L for s, L in zip(starts, w.lengths)])

    say(label, "prompt prefill", sum(w.lengths), "tokens")
    dev_p = to_dev(prompt)
    state = dev_p["initial_state"].clone()
    cu_of = lambda part, dev: part["cu_seqlens"] if host_offsets else dev["cu_seqlens"]
    o_prompt, _ = gdn.prefill_chunked(dev_p["q"], dev_p["k"], dev_p["v"], dev_p["g"], dev_p["beta"],
                                      cu_of(prompt, dev_p), state, final_state=state)
    snap = torch.empty_like(state)
    say(label, "snapshot")
    gdn.state_snapshot(state, snap)
    say(label, "verify block")
    dev_v = to_dev(verify)
    o_verify, _ = gdn.prefill_chunked(dev_v["q"], dev_v["k"], dev_v["v"], dev_v["g"], dev_v["beta"],
                                      cu_of(verify, dev_v), state, final_state=state)
    say(label, "restore")
    gdn.state_snapshot(snap, state)
    say(label, "re-feed", accepted)
    dev_r = to_dev(refeed)
    o_refeed, _ = gdn.prefill_chunked(dev_r["q"], dev_r["k"], dev_r["v"], dev_r["g"], dev_r["beta"],
                                      cu_of(refeed, dev_r), state, final_state=state)
    torch.cuda.synchronize()

    # oracle: prompt + accepted tokens in one pass per sequence
    kept = _slice_tokens(allx, [L + m for L, m in zip(w.lengths, accepted)], starts)
    o_kept, S_kept = oracle_prefill(kept)
    tol_o, tol_s = TOL[w.io_dtype]
    st = state.double().cpu().numpy()
    for i in range(n):
        assert rel_err(st[i], S_kept[i]) <= tol_s, "%s seq %d final state" % (label, i)
    # verify outputs over the draft equal the oracle over prompt + draft
    o_draft_ref, _ = oracle_prefill(allx)
    ov = o_verify.double().cpu().numpy()
    orf = o_refeed.double().cpu().numpy()
    cu_v = [int(x) for x in verify["cu_seqlens"]]
    cu_r = [int(x) for x in refeed["cu_seqlens"]]
    cu_k = [int(x) for x in kept["cu_seqlens"]]
    op = o_prompt.double().cpu().numpy()
    cu_p = [int(x) for x in prompt["cu_seqlens"]]
    for i in range(n):
        # the prompt outputs: the first L tokens of the oracle over prompt + draft
        ref_prompt = o_draft_ref[starts[i]: starts[i] + w.lengths[i]]
        assert rel_err(op[cu_p[i]:cu_p[i + 1]], ref_prompt) <= tol_o, "%s seq %d prompt outputs" % (label, i)
        for h in range(st.shape[1]):
            assert rel_err(st[i, h], S_kept[i, h]) <= tol_s, "%s seq %d head %d final state" % (label, i, h)
        ref_draft = o_draft_ref[starts[i] + w.lengths[i]: starts[i] + w.lengths[i] + V]
        assert rel_err(ov[cu_v[i]:cu_v[i + 1]], ref_draft) <= tol_o, "%s seq %d verify outputs" % (label, i)
        ref_acc = o_kept[cu_k[i] + w.lengths[i]: cu_k[i + 1]]
        if accepted[i]:
            assert rel_err(orf[cu_r[i]:cu_r[i + 1]], ref_acc) <= tol_o, "%s seq %d re-fed outputs" % (label, i)


@pytest.mark.parametrize("host_offsets", [False, True])
def test_varlen_verify_rollback_refeed_workload(host_offsets):
    w = S.workload("varlen_16")
    accepted = S.accept_counts(w.seed + 1, len(w.lengths), w.verify_tokens)
    _verify_protocol(w, accepted, "varlen_16_protocol", host_offsets=host_offsets)


@pytest.mark.parametrize("host_offsets", [False, True])
def test_verify_protocol_accept_none_and_all(host_offsets):
    w = S.Workload("small_protocol", [300, 64, 17], 2, 4, 128, 128, 64, torch.bfloat16, "uniform", 0.05, 330,
                   verify_tokens=16)
    _verify_protocol(w, [0, 16, 7], "protocol_edges", host_offsets=host_offsets)
