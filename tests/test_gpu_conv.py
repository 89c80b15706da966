"""GPU parity of the depthwise causal conv1d with q/k head L2 norms (gdn_conv1d_qkv)
against the fp64 oracle (oracle/conv1d.py).

Cases: both io dtypes, dk = dv in {32, 64, 128}, conv widths 1, 2, 4 and 8, packed
batches with empty sequences and sequences shorter than the window, with and without
a conv state, silu on and off, the L2 norm on and off, the state updated in place, a
sequence split in two calls with the state carried (bitwise equal to one call), the
Qwen3.5-9B 1k prefill shape, packed batches large enough that each wave walks several
token blocks, runs of empty sequences longer than a wave's offset window, the
32768-token shape the benchmark times (sampled slices), a verify-and-rollback of the
conv states through gdn_conv_state_snapshot, and the conv feeding the chunked
prefill end to end.
Bars: 1e-4 (fp32 io) and 2e-2 (bf16 io) on q, k and v (max-norm relative per tensor);
the new conv state is a copy of inputs and must match bit for bit.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_scan_amd as gdn
import oracle
from gated_deltanet_scan_amd import synthetic as S
from gpu_helpers import rel_err, say
from oracle.conv1d import conv_qkv

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def _gpu(inp, hqk, hv, dk, dv, silu, l2norm, inplace=False):
    x, w, cu = inp["x"].cuda(), inp["weight"].cuda(), inp["cu_seqlens"].cuda()
    s_in = inp["state"].cuda() if inp["state"] is not None else None
    K = w.shape[1]
    n = cu.numel() - 1
    if inplace and s_in is not None:
        s_out = s_in
    else:
        s_out = torch.full((n, x.shape[1], K - 1), float("nan"), device="cuda") if K > 1 else None
    q, k, v = gdn.conv1d_qkv(x, w, hqk, hv, dk, dv, cu, s_in, s_out, silu=silu, l2norm=l2norm, eps=1e-6)
    torch.cuda.synchronize()
    return q, k, v, s_out


def _check(inp, hqk, hv, dk, dv, io, silu, l2norm, label, inplace=False):
    K = inp["weight"].shape[1]
    say(label, "T=%d" % inp["x"].shape[0], "N=%d" % (inp["cu_seqlens"].numel() - 1), "heads", hqk, hv, "d", dk, dv,
        "K", K, io, "silu" if silu else "", "l2norm" if l2norm else "", "in place" if inplace else "")
    q_ref, k_ref, v_ref, s_ref = conv_qkv(inp["x"], inp["weight"], hqk, hv, dk, dv, inp["cu_seqlens"],
                                          inp["state"], silu=silu, l2norm=l2norm, eps=1e-6)
    q, k, v, s_out = _gpu(inp, hqk, hv, dk, dv, silu, l2norm, inplace)
    errs = [rel_err(t.double().cpu().numpy(), r) for t, r in ((q, q_ref), (k, k_ref), (v, v_ref))]
    say(label, "max rel err q %.3e k %.3e v %.3e" % tuple(errs))
    assert max(errs) <= TOL[io], (label, errs)
    if s_out is not None:
        np.testing.assert_array_equal(s_out.cpu().numpy(), s_ref.astype(np.float32))
    return q, k, v, s_out


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("K", [1, 2, 4, 8])
def test_shapes_and_widths(io, d, K):
    lengths = [5, 1, 0, 37, 3]
    inp = S.make_conv_inputs(lengths, 2, 4, d, d, K, io, seed=100 * d + K)
    _check(inp, 2, 4, d, d, io, silu=False, l2norm=True, label="shape_d%d_K%d" % (d, K))


@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("l2norm", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
def test_options(silu, l2norm, with_state):
    inp = S.make_conv_inputs([9, 2, 20], 2, 4, 64, 64, 4, torch.float32, seed=7, with_state=with_state)
    _check(inp, 2, 4, 64, 64, torch.float32, silu, l2norm, "options")


def test_state_in_place():
    inp = S.make_conv_inputs([6, 1, 0, 2, 40], 2, 4, 128, 128, 4, torch.bfloat16, seed=9)
    _check(inp, 2, 4, 128, 128, torch.bfloat16, False, True, "in_place", inplace=True)


def test_split_with_carried_state_is_bitwise_one_call():
    inp = S.make_conv_inputs([50], 2, 4, 128, 128, 4, torch.bfloat16, seed=11)
    x, w = inp["x"].cuda(), inp["weight"].cuda()
    s0 = inp["state"].cuda()
    whole = gdn.conv1d_qkv(x, w, 2, 4, 128, 128, None, s0, None)
    s1 = torch.empty_like(s0)
    a = gdn.conv1d_qkv(x[:17].contiguous(), w, 2, 4, 128, 128, None, s0, s1)
    b = gdn.conv1d_qkv(x[17:].contiguous(), w, 2, 4, 128, 128, None, s1, None)
    torch.cuda.synchronize()
    for part in range(3):
        assert torch.equal(torch.cat([a[part], b[part]]), whole[part])


def test_prefill_1k_shape():
    inp = S.make_conv_inputs([1024], 16, 32, 128, 128, 4, torch.bfloat16, seed=1001)
    _check(inp, 16, 32, 128, 128, torch.bfloat16, False, True, "prefill_1k_shape")


# Large enough that each wave walks several 16-token blocks (the launcher spreads the token
# blocks over about one round of resident waves): sequence starts then fall inside later
# blocks of a wave and at wave boundaries, and the window is carried from block to block.
@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
@pytest.mark.parametrize("inplace", [False, True], ids=["state_out", "in_place"])
def test_waves_over_several_blocks(io, inplace):
    lengths = [6000, 3, 700, 1, 1, 0, 9500, 40, 17, 2, 255, 257, 3000]   # 3 (bf16) or 5 (fp32) blocks a wave
    inp = S.make_conv_inputs(lengths, 16, 32, 128, 128, 4, io, seed=21 + int(inplace))
    _check(inp, 16, 32, 128, 128, io, False, True, "multi_block_waves", inplace=inplace)


def test_runs_of_empty_sequences():
    """More sequence ends at one token than a wave fetches offsets for (63): the sequence of
    a token is then searched for again."""
    lengths = [1000] + [0] * 70 + [17] + [0] * 5 + [1] * 30 + [12000]   # 2 blocks a wave
    inp = S.make_conv_inputs(lengths, 16, 32, 128, 128, 4, torch.bfloat16, seed=23)
    _check(inp, 16, 32, 128, 128, torch.bfloat16, True, True, "empty_runs")


def test_full_32k_shape_sampled():
    """The conv at the size the benchmark times (32768 tokens of the Qwen3.5-9B heads, 4
    blocks per wave), checked on sampled slices: each slice's outputs come from the oracle run
    on the slice with the K-1 inputs before it as its state (a sequence split with the state
    carried equals the whole), the first slice with the real state."""
    hqk, hv, d, K, T = 16, 32, 128, 4, 32768
    inp = S.make_conv_inputs([T], hqk, hv, d, d, K, torch.bfloat16, seed=25)
    say("full_32k", "T=%d" % T)
    q, k, v, s_out = _gpu(inp, hqk, hv, d, d, silu=False, l2norm=True)
    x = inp["x"]
    slices = [(0, 40), (250, 262), (4090, 4100), (16370, 16400), (20000, 20017), (32700, 32768)]
    for a, b in slices:
        if a == 0:
            st = inp["state"]
        else:
            st = x[a - (K - 1):a].float().t().unsqueeze(0).contiguous()
        q_ref, k_ref, v_ref, _ = conv_qkv(x[a:b], inp["weight"], hqk, hv, d, d, None, st, l2norm=True, eps=1e-6)
        errs = [rel_err(t[a:b].double().cpu().numpy(), r) for t, r in ((q, q_ref), (k, k_ref), (v, v_ref))]
        say("full_32k", "tokens %d..%d max rel err q %.3e k %.3e v %.3e" % ((a, b) + tuple(errs)))
        assert max(errs) <= TOL[torch.bfloat16], (a, b, errs)
    np.testing.assert_array_equal(s_out[0].cpu().numpy(), x[T - (K - 1):].float().t().numpy())


def test_conv_state_snapshot_verify_and_rollback():
    """Verify and roll back through the conv (NPU page, "New in v2"): after a prefix, the conv
    states are saved (scattered into a pool), a 16-token draft per sequence moves them on,
    they are restored, and the m_n accepted draft tokens are fed again.  The states then equal
    the oracle's over the prefix plus the accepted tokens (bit for bit), and so do the outputs
    of the accepted tokens."""
    hqk, hv, d, K = 2, 4, 128, 4
    prefix = [40, 3, 0, 70, 17]
    m = [0, 1, 7, 15, 16]
    N = len(prefix)
    inp = S.make_conv_inputs(prefix, hqk, hv, d, d, K, torch.bfloat16, seed=61)
    x, w = inp["x"].cuda(), inp["weight"].cuda()
    C = x.shape[1]
    state = inp["state"].cuda().clone()
    say("conv_rollback", "prefix", prefix, "accepted", m)
    gdn.conv1d_qkv(x, w, hqk, hv, d, d, inp["cu_seqlens"].cuda(), state, state)
    pool = torch.full((8, C, K - 1), float("nan"), device="cuda")
    rows = torch.tensor([6, 0, 3, 1, 5], dtype=torch.int32, device="cuda")
    gdn.conv_state_snapshot(state, pool, dst_rows=rows)
    draft = S.make_conv_inputs([16] * N, hqk, hv, d, d, K, torch.bfloat16, seed=62)["x"]
    cu16 = torch.arange(0, 16 * N + 1, 16, dtype=torch.int32)
    gdn.conv1d_qkv(draft.cuda(), w, hqk, hv, d, d, cu16.cuda(), state, state)
    gdn.conv_state_snapshot(pool, state, src_rows=rows)
    acc = torch.cat([draft[16 * n:16 * n + m[n]] for n in range(N)])
    cu_m = torch.tensor([0] + list(np.cumsum(m)), dtype=torch.int32)
    q, k, v = gdn.conv1d_qkv(acc.cuda(), w, hqk, hv, d, d, cu_m.cuda(), state, state)
    torch.cuda.synchronize()

    cu = [int(t) for t in inp["cu_seqlens"]]
    full = torch.cat([torch.cat([inp["x"][cu[n]:cu[n + 1]], draft[16 * n:16 * n + m[n]]]) for n in range(N)])
    cu_full = torch.tensor([0] + list(np.cumsum([prefix[n] + m[n] for n in range(N)])), dtype=torch.int32)
    q_ref, k_ref, v_ref, s_ref = conv_qkv(full, inp["weight"], hqk, hv, d, d, cu_full, inp["state"], l2norm=True,
                                          eps=1e-6)
    np.testing.assert_array_equal(state.cpu().numpy(), s_ref.astype(np.float32))
    tail = torch.cat([torch.arange(int(cu_full[n]) + prefix[n], int(cu_full[n + 1])) for n in range(N)])
    for got, ref, name in ((q, q_ref, "q"), (k, k_ref, "k"), (v, v_ref, "v")):
        err = rel_err(got.double().cpu().numpy(), ref[tail.numpy()])
        say("conv_rollback", "%s max rel err %.3e" % (name, err))
        assert err <= TOL[torch.bfloat16], (name, err)


def test_conv_feeds_the_chunked_prefill():
    """Upstream step end to end: conv (with state) -> chunked prefill, against the oracle's
    conv followed by the oracle's recurrence."""
    hqk, hv, d = 2, 4, 128
    lengths = [70, 5, 130]
    inp = S.make_conv_inputs(lengths, hqk, hv, d, d, 4, torch.bfloat16, seed=13)
    gen = torch.Generator().manual_seed(14)
    T = sum(lengths)
    g = -(0.5 + 6.5 * torch.rand(T, hv, generator=gen))
    beta = torch.sigmoid(torch.randn(T, hv, generator=gen))
    say("conv_then_prefill", "lengths", lengths)
    q, k, v, _ = _gpu(inp, hqk, hv, d, d, silu=False, l2norm=True)
    cu = inp["cu_seqlens"]
    o, _ = gdn.prefill_chunked(q, k, v, g.cuda(), beta.cuda(), cu, None, chunk=64)
    torch.cuda.synchronize()
    q_ref, k_ref, v_ref, _ = conv_qkv(inp["x"], inp["weight"], hqk, hv, d, d, cu, inp["state"], l2norm=True)
    # the recurrence of the oracle on the GPU's rounded conv outputs (the scan's own inputs)
    o_ref, _ = oracle.gdn_forward(q.cpu(), k.cpu(), v.cpu(), g, beta, cu)
    err = rel_err(o.double().cpu().numpy(), o_ref)
    say("conv_then_prefill", "max rel err o %.3e" % err)
    assert err <= 2e-2
    # and the conv outputs themselves against the oracle's
    assert rel_err(q.double().cpu().numpy(), q_ref) <= 2e-2
