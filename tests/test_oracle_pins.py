"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names the passage or the mathematics that fixes the expected value.
Shapes use K != V wherever the state's orientation could be confused.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
from tests.reference_forms import LOG2E, brute_force, chunk_form, chunk_intra

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, B, T, H, K, V, state=True, N=None, g_scale=1.0):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    g = g_scale * rng.standard_normal((B, T, H, K))
    beta = rng.standard_normal((B, T, H))
    A_log = rng.uniform(0, 1, H)
    dt_bias = rng.uniform(0, 1, (H, K))
    N = B if N is None else N
    s0 = 0.1 * rng.standard_normal((N, H, V, K)) if state else None
    return q, k, v, g, beta, A_log, dt_bias, s0


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------------------
# gate: closed forms and range (the formula is a reading; these pin its shape)
# ---------------------------------------------------------------------------

def test_gate_closed_forms():
    lb = -5.0
    H, K = 3, 4
    dt_bias = np.array([[0.1, 0.2, 0.3, 0.4]] * H)
    A_log = np.array([0.0, math.log(2.0), 0.7])
    # g + dt_bias = 0: sigmoid(0) = 1/2 whatever A_log, so lam = lb / 2.
    lam = oracle.gate(-dt_bias[None], A_log, dt_bias, lb)
    np.testing.assert_allclose(lam, np.full((1, H, K), lb / 2), rtol=0, atol=1e-15)
    # exp(A_log) (g + dt_bias) = ln 3: sigmoid(ln 3) = 3/4, so lam = 0.75 lb.
    x = math.log(3.0) / np.exp(A_log)[:, None] - dt_bias
    lam = oracle.gate(x[None], A_log, dt_bias, lb)
    np.testing.assert_allclose(lam, np.full((1, H, K), 0.75 * lb), rtol=1e-14)
    # saturation: a large positive argument reaches lb, a large negative one 0.
    lam_hi = oracle.gate(np.full((1, H, K), 100.0), A_log, dt_bias, lb)
    lam_lo = oracle.gate(np.full((1, H, K), -100.0), A_log, dt_bias, lb)
    np.testing.assert_allclose(lam_hi, lb, rtol=1e-14)
    assert np.all(np.abs(lam_lo) < 1e-40)


def test_gate_range_and_prefix_bound():
    # Per-token decay in (lb, 0), so the inclusive base-2 prefix over i+1 tokens
    # lies in ((i+1) lb log2(e), 0): the range stated in section 2 of the
    # FlashInfer PR #4262 summary (G_i in [32 b, 0] for a 32-token chunk).
    rng = np.random.default_rng(11)
    lb = -5.0
    H, K = 4, 32
    g = 3.0 * rng.standard_normal((64, H, K))
    lam = oracle.gate(g, rng.uniform(0, 1, H), rng.uniform(0, 1, (H, K)), lb)
    assert np.all(lam < 0) and np.all(lam > lb)
    G = np.cumsum(lam[:32] * LOG2E, axis=0)
    b = lb * LOG2E
    assert np.all(G <= 0) and np.all(G >= 32 * b)
    assert np.all(G[-1] > 32 * b)


def test_anchor_constants_match_printed_values():
    with open(os.path.join(GOLDEN, "anchor_constants.json")) as f:
        gold = json.load(f)
    lb = gold["lower_bound"]
    b = lb * math.log2(math.e)
    anchor = gold["anchor_multiplier"] * b
    assert round(b, gold["b_decimals"]) == gold["b_printed"]
    assert round(anchor, gold["anchor_decimals"]) == gold["anchor_printed"]
    # the centred radius equals half the chunk's prefix range: (32/2)|b| = 16|b|
    radius = gold["prefix_range_factor"] / 2 * abs(b)
    assert round(radius, 2) == gold["centred_radius_printed"]
    assert abs(radius - abs(anchor)) < 1e-12


# ---------------------------------------------------------------------------
# closed forms of the recurrence
# ---------------------------------------------------------------------------

def test_t1_closed_form_with_state():
    # One token, q = k = 3 e_0, g = -dt_bias (alpha = exp(lb/2) on every key
    # column), beta logit 0 (beta = 1/2).  By hand:
    #   S_1 = S_0 alpha + beta (v - r alpha S_0[:,0]) r e_0^T,  r = 3 / sqrt(9 + eps)
    #   o   = scale r S_1[:, 0]
    K, V, H = 4, 3, 1
    lb, scale = -0.8, 0.37
    rng = np.random.default_rng(1)
    S0 = rng.standard_normal((1, H, V, K))
    dt_bias = rng.uniform(0, 1, (H, K))
    q = np.zeros((1, 1, H, K)); q[..., 0] = 3.0
    k = q.copy()
    v = rng.standard_normal((1, 1, H, V))
    g = -dt_bias[None, None]
    beta = np.zeros((1, 1, H))
    out, fin = oracle.kda_fwd(q, k, v, g, beta, scale, np.array([0.3]), dt_bias, lb, S0)
    r = 3.0 / math.sqrt(9.0 + 1e-6)
    alpha = math.exp(lb / 2)
    S1 = S0[0, 0] * alpha
    S1[:, 0] += 0.5 * (v[0, 0, 0] - r * alpha * S0[0, 0][:, 0]) * r
    np.testing.assert_allclose(fin[0, 0], S1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(out[0, 0, 0], scale * r * S1[:, 0], rtol=1e-13, atol=1e-15)


def test_t1_closed_form_zero_state():
    # S_0 = 0: o = scale beta (qh . kh) v and S_1 = beta v kh^T.
    rng = np.random.default_rng(2)
    K, V, H = 8, 5, 2
    q, k, v, g, beta, A_log, dt_bias, _ = _rand_inputs(rng, 1, 1, H, K, V, state=False)
    out, fin = oracle.kda_fwd(q, k, v, g, beta, 0.5, A_log, dt_bias, -5.0)
    for h in range(H):
        qh = q[0, 0, h] / math.sqrt(np.sum(q[0, 0, h] ** 2) + 1e-6)
        kh = k[0, 0, h] / math.sqrt(np.sum(k[0, 0, h] ** 2) + 1e-6)
        b = 1.0 / (1.0 + math.exp(-beta[0, 0, h]))
        np.testing.assert_allclose(out[0, 0, h], 0.5 * b * (qh @ kh) * v[0, 0, h], rtol=1e-13)
        np.testing.assert_allclose(fin[0, h], b * np.outer(v[0, 0, h], kh), rtol=1e-13)


def test_projection_property():
    # beta logit +30 (beta = 1 to 1e-13) and q = k: the delta rule makes S_t kh_t = v_t
    # (up to eps / |k|^2, made negligible by |k| ~ 1e3), so out_t = scale v_t whatever
    # the gates and the initial state.
    rng = np.random.default_rng(3)
    B, T, H, K, V = 1, 40, 2, 16, 12
    q, k, v, g, beta, A_log, dt_bias, s0 = _rand_inputs(rng, B, T, H, K, V)
    beta[:] = 30.0
    scale = 0.25
    k = 1e3 * k
    out, _ = oracle.kda_fwd(k, k, v, g, beta, scale, A_log, dt_bias, -5.0, s0)
    np.testing.assert_allclose(out, scale * v, rtol=0, atol=1e-11 * scale)


def test_pure_decay():
    # beta logit -30 (beta ~ 1e-13) and g = -dt_bias (lam = lb/2 every token):
    # S_T = S_0 exp(T lb/2) and o_t = scale exp((t+1) lb/2) S_0 qh_t.
    rng = np.random.default_rng(4)
    B, T, H, K, V = 1, 20, 2, 6, 5
    q, k, v, g, beta, A_log, dt_bias, s0 = _rand_inputs(rng, B, T, H, K, V)
    beta[:] = -30.0
    g = np.broadcast_to(-dt_bias, (B, T, H, K)).copy()
    lb, scale = -0.1, 0.7
    out, fin = oracle.kda_fwd(q, k, v, g, beta, scale, A_log, dt_bias, lb, s0)
    np.testing.assert_allclose(fin, s0 * math.exp(T * lb / 2), rtol=1e-11, atol=1e-12)
    qh = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + 1e-6)
    for t in range(T):
        for h in range(H):
            want = scale * math.exp((t + 1) * lb / 2) * s0[0, h] @ qh[0, t, h]
            np.testing.assert_allclose(out[0, t, h], want, rtol=1e-10, atol=1e-12)


def test_basis_keys_ungated_delta_rule():
    # S_0 = 0, k_t = 2 e_t (t < T <= K), beta logit 30, g = -dt_bias so that
    # alpha = exp(lb/2) with lb = -1e-4 (nearly ungated).  Column t of S_{t-1} is
    # zero, so the prediction S kh_t vanishes and token t adds beta r v_t e_t^T
    # (kh_t = r e_t, r = 2/sqrt(4+eps)); column t of S_T is beta r v_t alpha^(T-1-t),
    # and with q_t = e_0, o_t = scale r_q beta r v_0 alpha^t, r_q = 1/sqrt(1+eps).
    T, H, K, V = 6, 1, 8, 3
    lb, scale = -1e-4, 0.9
    rng = np.random.default_rng(5)
    v = rng.standard_normal((1, T, H, V))
    k = np.zeros((1, T, H, K))
    for t in range(T):
        k[0, t, 0, t] = 2.0
    q = np.zeros((1, T, H, K)); q[..., 0] = 1.0
    dt_bias = rng.uniform(0, 1, (H, K))
    g = np.broadcast_to(-dt_bias, (1, T, H, K)).copy()
    beta = np.full((1, T, H), 30.0)
    out, fin = oracle.kda_fwd(q, k, v, g, beta, scale, np.zeros(H), dt_bias, lb)
    b = 1.0 / (1.0 + math.exp(-30.0))
    r = 2.0 / math.sqrt(4.0 + 1e-6)
    alpha = math.exp(lb / 2)
    want = np.zeros((V, K))
    for t in range(T):
        want[:, t] = b * r * v[0, t, 0] * alpha ** (T - 1 - t)
    np.testing.assert_allclose(fin[0, 0], want, rtol=1e-13, atol=1e-15)
    rq = 1.0 / math.sqrt(1.0 + 1e-6)
    for t in range(T):
        np.testing.assert_allclose(out[0, t, 0], scale * rq * b * r * v[0, 0, 0] * alpha ** t,
                                   rtol=1e-13)


# ---------------------------------------------------------------------------
# independent forms: brute force and the pages' chunk decomposition
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("K,V", [(5, 3), (4, 6)])
def test_brute_force(K, V):
    rng = np.random.default_rng(6 + K)
    B, T, H = 2, 7, 2
    q, k, v, g, beta, A_log, dt_bias, s0 = _rand_inputs(rng, B, T, H, K, V, g_scale=0.5)
    lb, scale = -0.7, 0.6
    out, fin = oracle.kda_fwd(q, k, v, g, beta, scale, A_log, dt_bias, lb, s0)
    lam = oracle.gate(g, A_log, dt_bias, lb)
    out_bf, fin_bf = brute_force(q, k, v, lam, beta, scale, s0)
    assert _rel(out, out_bf) < 1e-12
    assert _rel(fin, fin_bf) < 1e-12


def test_brute_force_varlen():
    rng = np.random.default_rng(7)
    K, V, H = 4, 3, 2
    cu = np.array([0, 3, 3, 9, 12])
    q, k, v, g, beta, A_log, dt_bias, s0 = _rand_inputs(rng, 1, 12, H, K, V, N=4)
    out, fin = oracle.kda_fwd(q, k, v, g, beta, 0.5, A_log, dt_bias, -2.0, s0, cu_seqlens=cu)
    lam = oracle.gate(g, A_log, dt_bias, -2.0)
    out_bf, fin_bf = brute_force(q, k, v, lam, beta, 0.5, s0, cu=cu)
    assert _rel(out, out_bf) < 1e-12
    assert _rel(fin, fin_bf) < 1e-12


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 32])
@pytest.mark.parametrize("centred", [False, True])
def test_chunk_form_equals_recurrence(chunk, centred):
    # The page's chunk equations (partial last chunks included: T = 100) give the
    # oracle's per-token result, with or without the fixed anchor 16 lb log2(e).
    rng = np.random.default_rng(100 + chunk)
    B, T, H, K, V = 2, 100, 2, 16, 12
    lb, scale = -5.0, 1.0 / math.sqrt(K)
    q, k, v, g, beta, A_log, dt_bias, s0 = _rand_inputs(rng, B, T, H, K, V)
    out, fin = oracle.kda_fwd(q, k, v, g, beta, scale, A_log, dt_bias, lb, s0)
    lam = oracle.gate(g, A_log, dt_bias, lb)
    anchor = 16 * lb * LOG2E if centred else 0.0
    out_c, fin_c = chunk_form(q, k, v, lam, beta, scale, chunk, anchor, s0)
    assert _rel(out, out_c) < 1e-12
    assert _rel(fin, fin_c) < 1e-12


def test_chunk_form_varlen():
    rng = np.random.default_rng(8)
    H, K, V = 2, 16, 16
    cu = np.array([0, 30, 31, 31, 95])
    q, k, v, g, beta, A_log, dt_bias, s0 = _rand_inputs(rng, 1, 95, H, K, V, N=4)
    out, fin = oracle.kda_fwd(q, k, v, g, beta, 0.25, A_log, dt_bias, -5.0, s0, cu_seqlens=cu)
    lam = oracle.gate(g, A_log, dt_bias, -5.0)
    out_c, fin_c = chunk_form(q, k, v, lam, beta, 0.25, 32, 16 * -5.0 * LOG2E, s0, cu=cu)
    assert _rel(out, out_c) < 1e-12
    assert _rel(fin, fin_c) < 1e-12


def test_centring_invariance():
    # The anchor cancels inside the product (2^(G_i - C) 2^(C - G_j) = 2^(G_i - G_j)),
    # so L and Mqk do not depend on it (section 2 of the PR #4262 summary).
    rng = np.random.default_rng(9)
    m, K = 32, 16
    lb = -5.0
    q, k = rng.standard_normal((m, K)), rng.standard_normal((m, K))
    lam = oracle.gate(rng.standard_normal((m, 1, K)), rng.uniform(0, 1, 1),
                      rng.uniform(0, 1, (1, K)), lb)[:, 0]
    beta = rng.standard_normal(m)
    ref = chunk_intra(q, k, lam, beta, 0.3, 0.0)
    for anchor in (16 * lb * LOG2E, -115.0, 37.25):
        L, M = chunk_intra(q, k, lam, beta, 0.3, anchor)
        np.testing.assert_allclose(L, ref[0], rtol=1e-12, atol=1e-14 * np.abs(ref[0]).max())
        np.testing.assert_allclose(M, ref[1], rtol=1e-12, atol=1e-14 * np.abs(ref[1]).max())


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_varlen_equals_separate_runs_and_batched():
    rng = np.random.default_rng(10)
    H, K, V = 3, 8, 6
    lens = [5, 0, 17, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    Tt = int(cu[-1])
    q, k, v, g, beta, A_log, dt_bias, s0 = _rand_inputs(rng, 1, Tt, H, K, V, N=len(lens))
    out, fin = oracle.kda_fwd(q, k, v, g, beta, 0.3, A_log, dt_bias, -5.0, s0, cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        sl = (slice(None), slice(a, b))
        o1, f1 = oracle.kda_fwd(q[sl], k[sl], v[sl], g[sl], beta[sl], 0.3, A_log, dt_bias, -5.0,
                                s0[n:n + 1])
        assert np.array_equal(out[:, a:b], o1)
        assert np.array_equal(fin[n], f1[0])
    assert np.array_equal(fin[1], s0[1])  # empty sequence: state passes through
    # batched [B,T] equals varlen over the flattened tokens with cu = [0, T, 2T, ...]
    B, T = 3, 11
    q, k, v, g, beta, A_log, dt_bias, s0 = _rand_inputs(rng, B, T, H, K, V)
    ob, fb = oracle.kda_fwd(q, k, v, g, beta, 0.3, A_log, dt_bias, -5.0, s0)
    flat = lambda x: x.reshape((1, B * T) + x.shape[2:])
    ov, fv = oracle.kda_fwd(flat(q), flat(k), flat(v), flat(g), flat(beta), 0.3, A_log, dt_bias,
                            -5.0, s0, cu_seqlens=np.arange(B + 1) * T)
    assert np.array_equal(ob.reshape(ov.shape), ov) and np.array_equal(fb, fv)


def test_linearity_in_v_and_state_and_scale():
    rng = np.random.default_rng(12)
    B, T, H, K, V = 1, 25, 2, 8, 5
    q, k, v1, g, beta, A_log, dt_bias, s1 = _rand_inputs(rng, B, T, H, K, V)
    v2 = rng.standard_normal(v1.shape)
    s2 = rng.standard_normal(s1.shape)
    run = lambda v, s, sc=0.4: oracle.kda_fwd(q, k, v, g, beta, sc, A_log, dt_bias, -3.0, s)
    o1, f1 = run(v1, s1)
    o2, f2 = run(v2, s2)
    o3, f3 = run(2.0 * v1 - 3.0 * v2, 2.0 * s1 - 3.0 * s2)
    assert _rel(o3, 2.0 * o1 - 3.0 * o2) < 1e-12
    assert _rel(f3, 2.0 * f1 - 3.0 * f2) < 1e-12
    o4, f4 = run(v1, s1, sc=1.2)
    assert _rel(o4, 3.0 * o1) < 1e-14 and np.array_equal(f4, f1)


def test_split_invariance():
    # Running [0, t1) then [t1, T) from the returned state equals one run
    # (the continued-generation use of final_state).
    rng = np.random.default_rng(13)
    B, T, H, K, V = 1, 90, 2, 8, 8
    q, k, v, g, beta, A_log, dt_bias, s0 = _rand_inputs(rng, B, T, H, K, V)
    o, f = oracle.kda_fwd(q, k, v, g, beta, 0.3, A_log, dt_bias, -5.0, s0)
    t1 = 37
    a = (slice(None), slice(0, t1))
    b = (slice(None), slice(t1, T))
    oa, fa = oracle.kda_fwd(q[a], k[a], v[a], g[a], beta[a], 0.3, A_log, dt_bias, -5.0, s0)
    ob, fb = oracle.kda_fwd(q[b], k[b], v[b], g[b], beta[b], 0.3, A_log, dt_bias, -5.0, fa)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o) and np.array_equal(fb, f)


def test_value_row_permutation():
    # Each value row of the state evolves independently: permuting the V index
    # of v and of S_0's rows permutes out and S_T the same way.
    rng = np.random.default_rng(14)
    B, T, H, K, V = 1, 30, 2, 8, 7
    q, k, v, g, beta, A_log, dt_bias, s0 = _rand_inputs(rng, B, T, H, K, V)
    perm = rng.permutation(V)
    o, f = oracle.kda_fwd(q, k, v, g, beta, 0.3, A_log, dt_bias, -5.0, s0)
    op, fp = oracle.kda_fwd(q, k, v[..., perm], g, beta, 0.3, A_log, dt_bias, -5.0,
                            s0[:, :, perm, :])
    assert np.array_equal(op, o[..., perm]) and np.array_equal(fp, f[:, :, perm, :])


def test_norm_scale_invariance():
    rng = np.random.default_rng(15)
    B, T, H, K, V = 1, 20, 1, 16, 4
    q, k, v, g, beta, A_log, dt_bias, s0 = _rand_inputs(rng, B, T, H, K, V)
    o, f = oracle.kda_fwd(q, k, v, g, beta, 0.3, A_log, dt_bias, -5.0, s0)
    o2, f2 = oracle.kda_fwd(7.0 * q, 0.5 * k, v, g, beta, 0.3, A_log, dt_bias, -5.0, s0)
    assert _rel(o2, o) < 1e-6 and _rel(f2, f) < 1e-6


def test_bad_cu_seqlens_rejected():
    rng = np.random.default_rng(16)
    q, k, v, g, beta, A_log, dt_bias, _ = _rand_inputs(rng, 1, 10, 1, 4, 4, state=False)
    with pytest.raises(ValueError):
        oracle.kda_fwd(q, k, v, g, beta, 0.3, A_log, dt_bias, -5.0, cu_seqlens=[0, 6, 4, 10])
    with pytest.raises(ValueError):
        oracle.kda_fwd(q, k, v, g, beta, 0.3, A_log, dt_bias, -5.0, cu_seqlens=[0, 6, 9])
