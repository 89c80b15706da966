"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None of them compares the oracle with
itself or with a retyped copy of its loop: each uses a different statement
of the rule (closed-form factor products, chunkwise-parallel form), a closed
form for a special case, or an invariant that a dropped term, a wrong sign,
a wrong index or a transposed operand would break.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_forms import chunkwise, closed_form_products
from gated_deltanet_scan_amd import synthetic


def _rand_case(rng, T, hqk, hv, dk, dv, unit_keys=True, s0=True):
    q = rng.standard_normal((T, hqk, dk))
    k = rng.standard_normal((T, hqk, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, hv, dv))
    g = -np.log1p(np.exp(rng.standard_normal((T, hv)) + 1.0))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, hv))))
    S0 = 0.3 * rng.standard_normal((1, hv, dk, dv)) if s0 else None
    return q, k, v, g, beta, S0


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("unit_keys", [True, False])
def test_against_closed_form_factor_products(unit_keys):
    """Qwen3.5-9B architecture page, Gated DeltaNet: S_t = a_t(I - b_t k k^T)S_{t-1} + b_t k v^T,
    summed out as explicit products of materialised dk x dk factors (dk != dv so a
    transposed state would fail)."""
    rng = np.random.default_rng(1)
    T, hqk, hv, dk, dv = 11, 1, 2, 5, 3
    q, k, v, g, beta, S0 = _rand_case(rng, T, hqk, hv, dk, dv, unit_keys)
    scale = 0.7
    o, S = oracle.gdn_forward(q, k, v, g, beta, None, S0, scale=scale)
    for h in range(hv):
        o_ref, S_ref = closed_form_products(q[:, 0], k[:, 0], v[:, h], g[:, h], beta[:, h], S0[0, h], scale)
        assert _rel(o[:, h], o_ref) < 1e-12
        assert _rel(S[0, h], S_ref) < 1e-12


def test_pure_decay_when_beta_is_zero():
    """beta = 0: nothing is written, S_t = exp(G_t) S_0 and o_t = scale exp(G_t) S_0^T q_t."""
    rng = np.random.default_rng(2)
    T, hqk, hv, dk, dv = 20, 2, 4, 6, 5
    q, k, v, g, beta, S0 = _rand_case(rng, T, hqk, hv, dk, dv)
    beta[:] = 0.0
    o, S = oracle.gdn_forward(q, k, v, g, beta, None, S0, scale=1.0)
    G = np.cumsum(g, axis=0)
    for h in range(hv):
        hq = h * hqk // hv
        assert _rel(S[0, h], np.exp(G[-1, h]) * S0[0, h]) < 1e-13
        o_ref = np.exp(G[:, h])[:, None] * (q[:, hq] @ S0[0, h])
        assert _rel(o[:, h], o_ref) < 1e-13


def test_exact_recall_alpha_one_beta_one_unit_keys():
    """alpha = 1, beta = 1, |k| = 1: the update stores v_t under k_t exactly, so
    S_t^T k_t = v_t after every step; with q_t = k_t the output is scale * v_t."""
    rng = np.random.default_rng(3)
    T, hqk, hv, dk, dv = 30, 2, 2, 8, 7
    q, k, v, g, beta, S0 = _rand_case(rng, T, hqk, hv, dk, dv)
    g[:] = 0.0
    beta[:] = 1.0
    o, S = oracle.gdn_forward(k, k, v, g, beta, None, S0, scale=0.5)
    for h in range(hv):
        assert np.max(np.abs(o[:, h] - 0.5 * v[:, h])) < 1e-12
        assert np.max(np.abs(S[0, h].T @ k[-1, h] - v[-1, h])) < 1e-12


def test_one_hot_keys_overwrite_rows():
    """alpha = 1, beta = 1, k_t = e_{i_t}: row i_t of S becomes v_t, other rows stay (a plain
    key-value memory overwrite)."""
    rng = np.random.default_rng(4)
    T, dk, dv = 12, 6, 4
    idx = rng.integers(0, dk, size=T)
    k = np.zeros((T, 1, dk))
    k[np.arange(T), 0, idx] = 1.0
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    g = np.zeros((T, 1))
    beta = np.ones((T, 1))
    S0 = rng.standard_normal((1, 1, dk, dv))
    _, S = oracle.gdn_forward(q, k, v, g, beta, None, S0, scale=1.0)
    expect = S0[0, 0].copy()
    for t in range(T):
        expect[idx[t]] = v[t, 0]
    assert np.max(np.abs(S[0, 0] - expect)) <= 4 * np.finfo(np.float64).eps * np.max(np.abs(expect))


def test_padding_tokens_leave_state_bitwise():
    """NPU page, How it works: g = 0, beta = 0 tokens leave the state exactly as after the last
    real token."""
    rng = np.random.default_rng(5)
    T, hqk, hv, dk, dv = 9, 1, 2, 5, 5
    q, k, v, g, beta, S0 = _rand_case(rng, T, hqk, hv, dk, dv)
    pad = 6
    qp = np.concatenate([q, rng.standard_normal((pad, hqk, dk))])
    kp = np.concatenate([k, rng.standard_normal((pad, hqk, dk))])
    vp = np.concatenate([v, rng.standard_normal((pad, hv, dv))])
    gp = np.concatenate([g, np.zeros((pad, hv))])
    bp = np.concatenate([beta, np.zeros((pad, hv))])
    _, S_a = oracle.gdn_forward(q, k, v, g, beta, None, S0)
    _, S_b = oracle.gdn_forward(qp, kp, vp, gp, bp, None, S0)
    assert np.array_equal(S_a, S_b)


def test_composition_prefix_reuse_bitwise():
    """Running [0, a) then [a, T) from the carried state equals running [0, T) (prefix reuse)."""
    rng = np.random.default_rng(6)
    T, hqk, hv, dk, dv = 25, 2, 4, 4, 6
    q, k, v, g, beta, S0 = _rand_case(rng, T, hqk, hv, dk, dv)
    o_full, S_full = oracle.gdn_forward(q, k, v, g, beta, None, S0)
    a = 11
    o1, S1 = oracle.gdn_forward(q[:a], k[:a], v[:a], g[:a], beta[:a], None, S0)
    o2, S2 = oracle.gdn_forward(q[a:], k[a:], v[a:], g[a:], beta[a:], None, S1)
    assert np.array_equal(np.concatenate([o1, o2]), o_full)
    assert np.array_equal(S2, S_full)


@pytest.mark.parametrize("inverse", ["forward", "doubling", "series"])
@pytest.mark.parametrize("chunk", [1, 2, 16, 64])
def test_chunkwise_parallel_form(chunk, inverse):
    """NPU page, How it works: the chunkwise-parallel N, D, O, S_T is exact, so in fp64 it must
    agree with the sequential oracle for any chunk length, including a ragged last chunk."""
    rng = np.random.default_rng(7)
    T, hqk, hv, dk, dv = 77, 1, 2, 8, 6
    q, k, v, g, beta, S0 = _rand_case(rng, T, hqk, hv, dk, dv)
    o, S = oracle.gdn_forward(q, k, v, g, beta, None, S0, scale=0.25)
    for h in range(hv):
        oc, Sc = chunkwise(q[:, 0], k[:, 0], v[:, h], g[:, h], beta[:, h], S0[0, h], 0.25, chunk,
                           inverse=inverse)
        assert _rel(oc, o[:, h]) < 1e-10
        assert _rel(Sc, S[0, h]) < 1e-10


def test_strong_decay_overflow_needs_log_space_masking():
    """Candle pull-request page, Chunked GatedDeltaNet Scan: at about -6.72 per step the naive
    fp32 exp(G_i - G_j) overflows in the upper triangle and inf * 0 gives NaN; masking the
    exponent before exp keeps fp32 finite and within 1e-4 of the sequential result."""
    rng = np.random.default_rng(8)
    T, dk, dv = 64, 16, 16
    q, k, v, g, beta, _ = _rand_case(rng, T, 1, 1, dk, dv, s0=False)
    g[:] = synthetic.STRONG_DECAY
    S0 = np.zeros((1, 1, dk, dv))
    o_ref, S_ref = oracle.gdn_forward(q, k, v, g, beta, None, S0, scale=1.0)
    args = (q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0[0, 0], 1.0, 64)
    o_naive, _ = chunkwise(*args, masked=False, dtype=np.float32)
    assert not np.all(np.isfinite(o_naive))
    o_fix, S_fix = chunkwise(*args, masked=True, dtype=np.float32)
    assert np.all(np.isfinite(o_fix)) and np.all(np.isfinite(S_fix))
    assert np.max(np.abs(o_fix - o_ref[:, 0])) < 1e-4
    assert np.max(np.abs(S_fix - S_ref[0, 0])) < 1e-4


def test_first_overflowing_distance():
    """The overflow claim made concrete: at -6.72 per step, exp of the upper-triangle difference
    (6.72 * distance) leaves fp32 once the distance reaches 14 (the first t >= 15)."""
    d = np.arange(1, 64)
    over = ~np.isfinite(np.exp(np.float32(6.72) * d.astype(np.float32)))
    assert d[over][0] == 14


def test_output_is_linear_in_scale():
    rng = np.random.default_rng(9)
    q, k, v, g, beta, S0 = _rand_case(rng, 15, 1, 1, 4, 4)
    o1, S1 = oracle.gdn_forward(q, k, v, g, beta, None, S0, scale=1.0)
    o2, S2 = oracle.gdn_forward(q, k, v, g, beta, None, S0, scale=0.125)
    assert np.array_equal(S1, S2)
    assert np.max(np.abs(o2 - 0.125 * o1)) <= 1e-15 * np.max(np.abs(o1))


def test_packed_batch_equals_separate_runs():
    rng = np.random.default_rng(10)
    lengths = [5, 0, 13, 1, 7]
    T = sum(lengths)
    q, k, v, g, beta, _ = _rand_case(rng, T, 2, 4, 4, 3)
    S0 = rng.standard_normal((len(lengths), 4, 4, 3))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, S = oracle.gdn_forward(q, k, v, g, beta, cu, S0)
    for n in range(len(lengths)):
        a, b = cu[n], cu[n + 1]
        on, Sn = oracle.gdn_forward(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], None, S0[n:n + 1])
        assert np.array_equal(o[a:b], on)
        assert np.array_equal(S[n], Sn[0])
    assert np.array_equal(S[1], S0[1])   # an empty sequence passes its state through


def test_grouped_heads_read_their_block_of_query_key_heads():
    """Value head h reads query/key head floor(h * HQK / HV): the grouped run equals a run with
    the query/key heads replicated to one per value head."""
    rng = np.random.default_rng(11)
    T, hqk, hv, dk, dv = 10, 2, 6, 4, 4
    q, k, v, g, beta, S0 = _rand_case(rng, T, hqk, hv, dk, dv)
    o, S = oracle.gdn_forward(q, k, v, g, beta, None, S0)
    rep = [h * hqk // hv for h in range(hv)]
    assert rep == [0, 0, 0, 1, 1, 1]
    o2, S2 = oracle.gdn_forward(q[:, rep], k[:, rep], v, g, beta, None, S0)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(12)
    q, k, v, g, beta, S0 = _rand_case(rng, 40, 2, 8, 8, 8)
    a = oracle.gdn_forward(q, k, v, g, beta, None, S0, threads=1)
    b = oracle.gdn_forward(q, k, v, g, beta, None, S0, threads=5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_accepts_bf16_torch_tensors_exactly():
    x = synthetic.make_inputs([9], 1, 2, 8, 8, torch.bfloat16, seed=3, g_law="uniform")
    o, S = oracle.gdn_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"])
    o2, S2 = oracle.gdn_forward(x["q"].double().numpy(), x["k"].double().numpy(),
                                x["v"].double().numpy(), x["g"].double().numpy(),
                                x["beta"].double().numpy(), [0, 9])
    assert np.array_equal(o, o2) and np.array_equal(S, S2)


def test_rejects_bad_arguments():
    q = np.zeros((4, 1, 2))
    v = np.zeros((4, 2, 2))
    g = np.zeros((4, 2))
    with pytest.raises(ValueError):
        oracle.gdn_forward(q, q, v, g, g, [0, 3])         # cu_seqlens does not end at T
    with pytest.raises(ValueError):
        oracle.gdn_forward(q, q, v, g, g, [0, 3, 2, 4])   # decreasing offsets
