"""Pins for the fp64 oracle: each test checks the oracle against something other
than itself -- the KDA equation written as explicit matrix products (a second
published form of the recurrence), exact rational arithmetic, closed forms,
invariants, and numbers printed on the pages.

Pages (cited by title and section):
  [P1] "How Kimi K3 Engineered Its Way to the Frontier" -- "How KDA updates its
       state" (token loop, decay on the key axis, erase reads the decayed state,
       beta near 1 clears the old value); "FlashKDA steps the state once per 16
       tokens" (chunked result matches the token loop); "What the hybrid saves".
  [P2] "Kimi K3: Open Frontier Intelligence", section 6 (the KDA equation).
  [P3] "Kimi K3 -- Training and Infrastructure Notes", section 4.1 (segment
       transition M and zero-start state S~ compose exactly).
  [P4] "Kimi K3: a 2.8T open model ...", "Kimi Delta Attention" (same equation);
       "FlashKDA: the equation, shipped as a kernel" (beta logits pass through a
       sigmoid).
  The lower-bounded gate: [P1] "How KDA updates its state" (K3's gate from
  flash-linear-attention's gate.py: g = lower_bound * sigmoid(exp(A_log) *
  (x + dt_bias)), so g stays in (lower_bound, 0) and exp(g) above exp(-5)).
  The decode front end: [P1] "How KDA updates its state" and "What the hybrid
  saves" (three ShortConv caches of kernel size 4, 216 KiB per layer in bf16);
  [P4] "Kimi Delta Attention" (short convolution, Swish, L2 normalisation).
"""
import json
import math
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.build import SOURCE, build_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def rand_inputs(rng, T, H, K, V, unit=True, g_scale=1.0):
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    g = -np.logaddexp(0.0, rng.standard_normal((T, H, K))) * g_scale  # -softplus
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def equation_form(q, k, v, g, beta, S0, scale=1.0):
    """The KDA equation of [P2] section 6 / [P4] "Kimi Delta Attention", written
    as explicit matrix products for one head:
        S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t
    q, k, g: [T, K]; v: [T, V]; beta: [T]; S0: [K, V]."""
    T, K = k.shape
    S = S0.copy()
    outs = []
    for t in range(T):
        kt = k[t][:, None]
        Mt = (np.eye(K) - beta[t] * kt @ kt.T) @ np.diag(np.exp(g[t]))
        S = Mt @ S + beta[t] * kt @ v[t][None, :]
        outs.append(scale * S.T @ q[t])
    return np.array(outs), S


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("K,V,T", [(1, 1, 3), (2, 3, 2), (3, 2, 3), (4, 4, 3), (5, 2, 1)])
def test_tiny_matches_equation_form(K, V, T):
    """Tiny inputs (K != V catches a transposed operand): the token loop equals
    the matrix-product form of the KDA equation."""
    rng = np.random.default_rng(100 + 10 * K + V)
    H = 2
    q, k, v, g, beta = rand_inputs(rng, T, H, K, V, unit=False)
    S0 = rng.standard_normal((1, H, K, V))
    o, sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0, scale=0.75)
    for h in range(H):
        o_ref, s_ref = equation_form(q[:, h], k[:, h], v[:, h], g[:, h], beta[:, h],
                                     S0[0, h], scale=0.75)
        np.testing.assert_allclose(o[:, h], o_ref, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(sf[0, h], s_ref, rtol=1e-13, atol=1e-13)


def test_exact_rational_two_tokens():
    """d_k = d_v = 2, two tokens, hand-chosen rational values, expanded in exact
    rational arithmetic from the KDA equation.  Decays are chosen as exp(g) with
    g = ln(1/2), ln(1/4), so alpha is 1/2, 1/4 up to one rounding of exp/log."""
    F = Fraction
    alphas = [[F(1, 2), F(1, 4)], [F(1, 4), F(1, 2)]]
    ks = [[F(3, 5), F(4, 5)], [F(1), F(0)]]
    vs = [[F(2), F(-1)], [F(1, 2), F(3)]]
    qs = [[F(1), F(2)], [F(-1), F(1)]]
    betas = [F(1, 2), F(1, 3)]
    S = [[F(1), F(0)], [F(2), F(-1)]]  # initial state, rows = key channels
    outs = []
    for t in range(2):
        a, kk, vv, qq, b = alphas[t], ks[t], vs[t], qs[t], betas[t]
        D = [[a[i] * S[i][j] for j in range(2)] for i in range(2)]       # Diag(a) S
        kTD = [sum(kk[i] * D[i][j] for i in range(2)) for j in range(2)]  # k^T D S
        S = [[D[i][j] - b * kk[i] * kTD[j] + b * kk[i] * vv[j] for j in range(2)]
             for i in range(2)]
        outs.append([sum(qq[i] * S[i][j] for i in range(2)) for j in range(2)])
    fl = lambda m: np.array(m, dtype=np.float64)
    q = fl(qs)[:, None, :]
    k = fl(ks)[:, None, :]
    v = fl(vs)[:, None, :]
    g = np.log(fl(alphas))[:, None, :]
    beta = fl(betas)[:, None]
    S0 = fl([[1, 0], [2, -1]])[None, None]
    o, sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
    np.testing.assert_allclose(o[:, 0], fl(outs), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(sf[0, 0], fl(S), rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------- closed forms
def test_beta0_alpha1_leaves_state_unchanged():
    rng = np.random.default_rng(1)
    T, H, K, V = 37, 3, 8, 6
    q, k, v, g, beta = rand_inputs(rng, T, H, K, V)
    g[:] = 0.0
    beta[:] = 0.0
    S0 = rng.standard_normal((1, H, K, V))
    o, sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
    assert np.array_equal(sf, S0)
    np.testing.assert_allclose(o, np.einsum("thk,hkv->thv", q, S0[0]), rtol=1e-13)


def test_beta0_pure_decay_closed_form():
    """beta = 0: S_T = Diag(exp(sum_t g_t)) S0, o_t = (Diag(exp(G_t)) S0)^T q_t."""
    rng = np.random.default_rng(2)
    T, H, K, V = 29, 2, 8, 5
    q, k, v, g, beta = rand_inputs(rng, T, H, K, V, g_scale=0.1)
    beta[:] = 0.0
    S0 = rng.standard_normal((1, H, K, V))
    o, sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
    G = np.cumsum(g, axis=0)
    np.testing.assert_allclose(sf[0], np.exp(G[-1])[:, :, None] * S0[0], rtol=1e-12)
    o_ref = np.einsum("thk,thk,hkv->thv", q, np.exp(G), S0[0])
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)


def test_beta1_unit_key_reads_back_its_value():
    """[P1] "How KDA updates its state": beta near 1 clears the old value and the
    next read for k_t returns what this token wrote.  With beta = 1, |k| = 1 and
    q = k the read returns v_t exactly, for any prior state and decay."""
    rng = np.random.default_rng(3)
    T, H, K, V = 41, 2, 16, 12
    q, k, v, g, beta = rand_inputs(rng, T, H, K, V)
    beta[:] = 1.0
    q = k.copy()
    S0 = rng.standard_normal((1, H, K, V))
    o, _ = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_exact_retrieval():
    """alpha = 1, beta = 1, S0 = 0 and orthonormal keys: every written value is
    retrieved exactly, k_j^T S_T = v_j^T for all j."""
    rng = np.random.default_rng(4)
    K = V = 16
    T = 16
    Q, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = Q.T[:T][:, None, :]  # rows are orthonormal keys
    v = rng.standard_normal((T, 1, V))
    q = rng.standard_normal((T, 1, K))
    g = np.zeros((T, 1, K))
    beta = np.ones((T, 1))
    _, sf = oracle.recurrent(q, k, v, g, beta)
    np.testing.assert_allclose(k[:, 0] @ sf[0, 0], v[:, 0], rtol=1e-12, atol=1e-12)


def test_decay_is_natural_exponential_of_gate():
    """The page's decay floor: with g = -5 the state survives as exp(-5) ~ 0.0067
    (a base-2 reading would give 2^-5 = 0.031)."""
    c = json.load(open(GOLDEN))["decay_floor"]
    H, K, V = 1, 4, 3
    S0 = np.ones((1, H, K, V))
    q = np.zeros((1, H, K))
    k = np.zeros((1, H, K))
    v = np.zeros((1, H, V))
    g = np.full((1, H, K), c["gate_lower_bound"])
    beta = np.zeros((1, H))
    _, sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
    assert abs(sf[0, 0, 0, 0] - c["alpha_floor_printed"]) <= c["printed_digits_tol"]


def test_cumulative_16_token_bound_of_lower_bounded_gate():
    """[P2] section 6: with every g >= -5 a 16-token cumulative log-decay lies in
    [-80, 0]; checked on the clamped synthetic gate the prefill workload uses."""
    import torch
    import kda_inputs as ki
    c = json.load(open(GOLDEN))["cumulative_bound_16"]
    cfg = ki.PrefillConfig("t", (4096,), 2, "bf16", g_lower_bound=c["gate_lower_bound"])
    x = ki.make_prefill(cfg, heads=2)
    G16 = x["g"].double().view(-1, c["tokens"], 2, 128).sum(dim=1)
    assert float(G16.min()) >= c["lower"] and float(G16.max()) <= c["upper"]
    assert float(x["g"].min()) >= c["gate_lower_bound"]
    assert math.isclose(c["lower"], c["tokens"] * c["gate_lower_bound"])


# ----------------------------------------------------------------- invariants
@pytest.mark.parametrize("C", [1, 7, 16, 64])
def test_chunked_equals_sequential(C):
    """[P1] "FlashKDA steps the state once per 16 tokens": the chunked result
    matches the token loop.  Packed batch, partial last chunks, initial state."""
    rng = np.random.default_rng(10 + C)
    lens = [1, 63, 64, 65, 150, 0, 29]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, K, V = int(cu[-1]), 2, 16, 12
    q, k, v, g, beta = rand_inputs(rng, T, H, K, V)
    S0 = 0.3 * rng.standard_normal((len(lens), H, K, V))
    o1, s1 = oracle.recurrent(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0, scale=0.5)
    o2, s2 = oracle.chunked(q, k, v, g, beta, C, cu_seqlens=cu, initial_state=S0, scale=0.5)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 * np.max(np.abs(o1))
    assert np.max(np.abs(s1 - s2)) <= 1e-12 * np.max(np.abs(s1))


def test_chunked_equals_sequential_at_head_dim_128():
    rng = np.random.default_rng(11)
    T, H, K, V = 200, 1, 128, 128
    q, k, v, g, beta = rand_inputs(rng, T, H, K, V)
    o1, s1 = oracle.recurrent(q, k, v, g, beta)
    o2, s2 = oracle.chunked(q, k, v, g, beta, 64)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 * np.max(np.abs(o1))
    assert np.max(np.abs(s1 - s2)) <= 1e-12 * np.max(np.abs(s1))


def test_segment_transition_composes_exactly():
    """[P3] section 4.1: a segment maps S_in to M S_in + S~; M is the ordered
    product of (I - b k k^T) Diag(a) (built here with numpy), S~ the state from
    zero; composing two segments equals running both."""
    rng = np.random.default_rng(12)
    T1, T2, K, V = 23, 31, 8, 6
    q, k, v, g, beta = rand_inputs(rng, T1 + T2, 1, K, V)
    k1, v1, g1, b1 = k[:, 0], v[:, 0], g[:, 0], beta[:, 0]
    M, St = oracle.transition(k1, v1, g1, b1)
    Mref = np.eye(K)
    for t in range(T1 + T2):
        kt = k1[t][:, None]
        Mref = (np.eye(K) - b1[t] * kt @ kt.T) @ np.diag(np.exp(g1[t])) @ Mref
    np.testing.assert_allclose(M, Mref, rtol=1e-12, atol=1e-14)
    S0 = rng.standard_normal((1, 1, K, V))
    _, sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
    np.testing.assert_allclose(sf[0, 0], M @ S0[0, 0] + St, rtol=1e-12, atol=1e-13)
    # two segments composed
    Ma, Sa = oracle.transition(k1[:T1], v1[:T1], g1[:T1], b1[:T1])
    Mb, Sb = oracle.transition(k1[T1:], v1[T1:], g1[T1:], b1[T1:])
    np.testing.assert_allclose(Mb @ (Ma @ S0[0, 0] + Sa) + Sb, sf[0, 0], rtol=1e-12,
                               atol=1e-13)


def test_outputs_affine_in_initial_state():
    rng = np.random.default_rng(13)
    T, H, K, V = 40, 2, 8, 8
    q, k, v, g, beta = rand_inputs(rng, T, H, K, V)
    Sa = rng.standard_normal((1, H, K, V))
    Sb = rng.standard_normal((1, H, K, V))
    oa, sa = oracle.recurrent(q, k, v, g, beta, initial_state=Sa)
    ob, sb = oracle.recurrent(q, k, v, g, beta, initial_state=Sb)
    oab, sab = oracle.recurrent(q, k, v, g, beta, initial_state=Sa + Sb)
    o0, s0 = oracle.recurrent(q, k, v, g, beta)
    np.testing.assert_allclose(oab, oa + ob - o0, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sab, sa + sb - s0, rtol=1e-11, atol=1e-12)


def test_split_and_resume_is_bitwise():
    rng = np.random.default_rng(14)
    T, H, K, V = 90, 2, 8, 4
    q, k, v, g, beta = rand_inputs(rng, T, H, K, V)
    S0 = rng.standard_normal((1, H, K, V))
    o, sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
    t = 37
    o1, s1 = oracle.recurrent(q[:t], k[:t], v[:t], g[:t], beta[:t], initial_state=S0)
    o2, s2 = oracle.recurrent(q[t:], k[t:], v[t:], g[t:], beta[t:], initial_state=s1)
    assert np.array_equal(np.concatenate([o1, o2]), o)
    assert np.array_equal(s2, sf)


def test_varlen_equals_separate_runs():
    rng = np.random.default_rng(15)
    lens = [5, 0, 17, 1, 33]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, K, V = int(cu[-1]), 2, 8, 4
    q, k, v, g, beta = rand_inputs(rng, T, H, K, V)
    S0 = rng.standard_normal((len(lens), H, K, V))
    o, sf = oracle.recurrent(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, sn = oracle.recurrent(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b],
                                  initial_state=S0[n:n + 1])
        assert np.array_equal(o[a:b], on)
        assert np.array_equal(sf[n], sn[0])


def test_decode_steps_equal_token_loop():
    """T decode steps through a slot pool equal the token loop per sequence; a
    negative slot leaves its state untouched."""
    rng = np.random.default_rng(16)
    B, H, K, V, T = 5, 2, 8, 6, 7
    q, k, v, g, beta = rand_inputs(rng, T * B, H, K, V)
    shp = lambda x: x.reshape((T, B) + x.shape[1:])
    q, k, v, g, beta = map(shp, (q, k, v, g, beta))
    pool = rng.standard_normal((8, H, K, V))
    slots = np.array([6, 0, -1, 3, 1])
    cur = pool.copy()
    outs = []
    for t in range(T):
        o_t, cur = oracle.decode_step(q[t], k[t], v[t], g[t], beta[t], cur, slots)
        outs.append(o_t)
    for b, s in enumerate(slots):
        if s < 0:
            continue
        o_ref, s_ref = oracle.recurrent(q[:, b], k[:, b], v[:, b], g[:, b], beta[:, b],
                                        initial_state=pool[s:s + 1])
        np.testing.assert_allclose(np.array(outs)[:, b], o_ref, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(cur[s], s_ref[0], rtol=1e-13, atol=1e-14)
    untouched = [s for s in range(8) if s not in set(slots.tolist())]
    assert np.array_equal(cur[untouched], pool[untouched])
    assert np.all(np.isnan(np.array(outs)[:, 2]))


# ------------------------------------------------ gate and beta front end
def _gate_case(rng, T=5, H=3, K=4):
    return (rng.standard_normal((T, H, K)), rng.standard_normal(H) * 0.7,
            rng.standard_normal((H, K)))


def test_gate_zero_argument_gives_half_the_bound():
    """sigmoid(0) = 1/2 exactly: with x = -dt_bias[h, c] every g is lower_bound / 2
    whatever A_log is (pins the bias indexing [h, c] against a transposed read)."""
    rng = np.random.default_rng(11)
    T, H, K = 4, 3, 5
    dt = rng.standard_normal((H, K))
    x = np.broadcast_to(-dt, (T, H, K)).copy()
    A = rng.standard_normal(H) * 2.0
    for lb in (-5.0, -1.25):
        g = oracle.lowerbound_gate(x, A, dt, lb)
        assert np.array_equal(g, np.full((T, H, K), lb / 2))


def test_gate_closed_form_per_head():
    """With x + dt_bias = 1 and A_log[h] = ln(ln m_h), the gate's argument is ln m_h and
    sigmoid(ln m) = m / (1 + m): g = lower_bound m_h / (1 + m_h), a different exact
    value per head (pins exp(A_log) rather than A_log, the head index and the sign
    inside the sigmoid)."""
    rng = np.random.default_rng(12)
    T, H, K = 3, 4, 6
    m = np.array([2.0, 3.0, 5.0, 9.0])
    A = np.log(np.log(m))
    dt = rng.standard_normal((H, K))
    x = 1.0 - dt[None]
    x = np.broadcast_to(x, (T, H, K)).copy()
    lb = -5.0
    g = oracle.lowerbound_gate(x, A, dt, lb)
    want = lb * m / (1.0 + m)
    np.testing.assert_allclose(g, np.broadcast_to(want[None, :, None], g.shape),
                               rtol=1e-14, atol=0)


def test_gate_reflection_sums_to_the_bound():
    """sigmoid(z) + sigmoid(-z) = 1, so reflecting x + dt_bias about zero maps g to
    lower_bound - g."""
    rng = np.random.default_rng(13)
    x, A, dt = _gate_case(rng)
    xr = -x - 2.0 * dt[None]  # (xr + dt) = -(x + dt)
    g1 = oracle.lowerbound_gate(x, A, dt, -5.0)
    g2 = oracle.lowerbound_gate(xr, A, dt, -5.0)
    np.testing.assert_allclose(g1 + g2, -5.0, rtol=0, atol=1e-14)


def test_gate_range_limits_and_page_floor():
    """[P1]: g lies between the bound and 0, so exp(g) stays above exp(-5) ~ 0.0067
    (printed); large positive logits reach the bound, large negative ones 0, and
    g falls as the logit rises."""
    c = json.load(open(GOLDEN))["decay_floor"]
    lb = c["gate_lower_bound"]
    x = np.linspace(-8.0, 8.0, 161).reshape(161, 1, 1) * np.ones((1, 2, 3))
    A = np.array([0.0, 0.5])
    g = oracle.lowerbound_gate(x, A, None, lb)
    assert np.all(g > lb) and np.all(g < 0.0)
    assert np.all(np.diff(g, axis=0) < 0.0)
    assert float(np.exp(g).min()) >= c["alpha_floor_printed"] - c["printed_digits_tol"]
    far = oracle.lowerbound_gate(np.array([[[60.0, -60.0]]]), np.array([0.0]), None, lb)
    assert far[0, 0, 0] == lb and -1e-25 < far[0, 0, 1] < 0.0
    # A_log -> -inf: exp(A_log) = 0 and every g is the bound's half
    flat = oracle.lowerbound_gate(x, np.array([-np.inf, -np.inf]), None, lb)
    assert np.array_equal(flat, np.full_like(flat, lb / 2))


def test_gate_without_bias_equals_zero_bias():
    rng = np.random.default_rng(14)
    x, A, dt = _gate_case(rng)
    np.testing.assert_array_equal(oracle.lowerbound_gate(x, A, None, -5.0),
                                  oracle.lowerbound_gate(x, A, np.zeros_like(dt), -5.0))


def test_beta_sigmoid_values():
    """sigmoid(0) = 1/2, sigmoid(+-ln 3) = 3/4 and 1/4; the library's logistic
    function agrees to rounding."""
    from scipy.special import expit
    y = oracle.sigmoid(np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -40.0]))
    np.testing.assert_allclose(y[:3], [0.5, 0.75, 0.25], rtol=1e-15, atol=0)
    assert y[3] == 1.0 or abs(y[3] - 1.0) < 1e-17
    assert 0.0 < y[4] < 1e-17
    z = np.random.default_rng(15).standard_normal((7, 3)) * 4.0
    np.testing.assert_allclose(oracle.sigmoid(z), expit(z), rtol=1e-15, atol=0)


# ------------------------------------------------------- decode front end
def test_short_conv_matches_library_correlation():
    """The causal depthwise convolution equals numpy's 'valid' correlation of the
    cache followed by the inputs with each channel's taps (oldest tap first)."""
    rng = np.random.default_rng(21)
    T, C, W = 7, 5, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    cache = rng.standard_normal((W - 1, C))
    y, new_cache = oracle.short_conv(x, w, cache)
    ext = np.concatenate([cache, x])
    for c in range(C):
        np.testing.assert_allclose(y[:, c], np.correlate(ext[:, c], w[c], mode="valid"),
                                   rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(new_cache, x[-(W - 1):])


def test_short_conv_identity_and_delay_taps():
    """Tap on the newest input reproduces x; tap on the oldest delays it by
    W - 1 tokens, reading the cache first."""
    rng = np.random.default_rng(22)
    T, C, W = 6, 3, 4
    x = rng.standard_normal((T, C))
    cache = rng.standard_normal((W - 1, C))
    ident = np.zeros((C, W)); ident[:, -1] = 1.0
    delay = np.zeros((C, W)); delay[:, 0] = 1.0
    np.testing.assert_array_equal(oracle.short_conv(x, ident, cache)[0], x)
    np.testing.assert_array_equal(oracle.short_conv(x, delay, cache)[0],
                                  np.concatenate([cache, x])[:T])


def test_short_conv_streams_token_by_token():
    """One call over T tokens equals T one-token calls chained through the cache
    (the decode step's use)."""
    rng = np.random.default_rng(23)
    T, C, W = 9, 4, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    cache0 = rng.standard_normal((W - 1, C))
    y_all, c_all = oracle.short_conv(x, w, cache0)
    cache = cache0
    for t in range(T):
        y_t, cache = oracle.short_conv(x[t:t + 1], w, cache)
        np.testing.assert_allclose(y_t[0], y_all[t], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(cache, c_all)


def test_conv_cache_bytes_match_page_accounting():
    """[P1] "What the hybrid saves": three caches of kernel size 4 (W - 1 = 3
    previous inputs) over 96 heads x 128 channels in bf16 are 216 KiB."""
    c = json.load(open(GOLDEN))["state_memory"]
    W = c["conv_kernel_size"]
    assert 3 * (W - 1) * c["heads"] * c["head_dim"] * 2 == c["conv_cache_bytes_per_layer"]


def test_swish_identities():
    """swish(0) = 0, swish(x) - swish(-x) = x, swish(ln 3) = 0.75 ln 3, and the
    library logistic function times x."""
    from scipy.special import expit
    assert oracle.swish(np.array([0.0]))[0] == 0.0
    x = np.random.default_rng(24).standard_normal(50) * 5
    np.testing.assert_allclose(oracle.swish(x) - oracle.swish(-x), x, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.swish(np.array([math.log(3.0)])), [0.75 * math.log(3.0)],
                               rtol=1e-15)
    np.testing.assert_allclose(oracle.swish(x), x * expit(x), rtol=1e-14, atol=1e-15)


def test_l2norm_closed_forms():
    """(3, 4) -> (0.6, 0.8) with eps = 0; with eps the norm is |x| / sqrt(|x|^2 + eps);
    zero stays zero."""
    np.testing.assert_allclose(oracle.l2norm(np.array([[3.0, 4.0]]), eps=0.0), [[0.6, 0.8]],
                               rtol=1e-15)
    x = np.random.default_rng(25).standard_normal((4, 128))
    y = oracle.l2norm(x, eps=1e-6)
    nx = np.linalg.norm(x, axis=-1)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), nx / np.sqrt(nx ** 2 + 1e-6),
                               rtol=1e-13)
    np.testing.assert_allclose(y / np.linalg.norm(y, axis=-1, keepdims=True),
                               x / nx[:, None], rtol=1e-12)
    assert np.array_equal(oracle.l2norm(np.zeros((1, 8))), np.zeros((1, 8)))


def test_rmsnorm_closed_forms():
    """An alternating +-c vector has mean square c^2: it maps to +-w / sqrt(1 + eps/c^2);
    the weight multiplies per element; scaling x by 7 leaves the eps = 0 result."""
    c, eps = 3.0, 1e-6
    x = np.array([[c, -c, c, -c]])
    w = np.array([1.0, 2.0, 0.5, -1.0])
    np.testing.assert_allclose(oracle.rmsnorm(x, w, eps),
                               np.array([[1, -2, 0.5, 1.0]]) / math.sqrt(1 + eps / c ** 2),
                               rtol=1e-15)
    z = np.random.default_rng(26).standard_normal((3, 128))
    np.testing.assert_allclose(oracle.rmsnorm(7 * z, None, 0.0), oracle.rmsnorm(z, None, 0.0),
                               rtol=1e-13)
    np.testing.assert_allclose(np.mean(oracle.rmsnorm(z, None, 0.0) ** 2, axis=-1), 1.0,
                               rtol=1e-13)


def test_fused_decode_steps_equal_whole_sequence_front_end():
    """T fused decode steps from an empty (zero) cache equal the whole sequence
    pushed through the short convolution at once, Swish, L2 normalisation, the
    token loop and the output RMSNorm (streaming = batch)."""
    rng = np.random.default_rng(27)
    T, H, K, W = 6, 2, 4, 4
    raw = [rng.standard_normal((T, H, K)) for _ in range(3)]
    w = rng.standard_normal((3, H, K, W))
    g = -np.logaddexp(0.0, rng.standard_normal((T, H, K)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, H))))
    nw = rng.standard_normal(K)
    pool = rng.standard_normal((1, H, K, K)) * 0.1
    cache = np.zeros((1, 3, W - 1, H, K))
    outs = []
    st = pool
    for t in range(T):
        o, st, cache = oracle.fused_decode_step(raw[0][t:t + 1], raw[1][t:t + 1],
                                                raw[2][t:t + 1], g[t:t + 1], beta[t:t + 1],
                                                w, cache, st, norm_weight=nw, scale=0.5)
        outs.append(o[0])
    conv = []
    for i in range(3):
        y, _ = oracle.short_conv(raw[i].reshape(T, H * K), w[i].reshape(H * K, W),
                                 np.zeros((W - 1, H * K)))
        conv.append(oracle.swish(y).reshape(T, H, K))
    q, k = oracle.l2norm(conv[0]), oracle.l2norm(conv[1])
    o_ref, s_ref = oracle.recurrent(q, k, conv[2], g, beta, initial_state=pool, scale=0.5)
    np.testing.assert_allclose(np.array(outs), oracle.rmsnorm(o_ref, nw), rtol=1e-11,
                               atol=1e-12)
    np.testing.assert_allclose(st, s_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(cache[0, 0], raw[0][-(W - 1):])


def _spec_inputs(rng, B, T, H, K):
    return {"q": rng.standard_normal((B, T, H, K)), "k": rng.standard_normal((B, T, H, K)),
            "v": rng.standard_normal((B, T, H, K)),
            "g": -np.logaddexp(0.0, rng.standard_normal((B, T, H, K))),
            "beta": 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))}


def test_spec_verify_replay_equals_accepted_token_stream():
    """Two verification rounds with replay: the committed state and cache equal
    plain fused steps over exactly the accepted tokens, and each window's outputs
    equal plain fused steps from the committed point (the draft tokens that are
    rejected leave no trace)."""
    rng = np.random.default_rng(31)
    B, T, H, K = 3, 3, 2, 4
    w = rng.standard_normal((3, H, K, 4))
    pool0 = rng.standard_normal((B, H, K, K)) * 0.1
    cache0 = rng.standard_normal((B, 3, 3, H, K))
    win1, win2 = _spec_inputs(rng, B, T, H, K), _spec_inputs(rng, B, T, H, K)
    acc = np.array([0, 2, 3])  # tokens of window 1 accepted per row
    o1, pool1, cache1 = oracle.spec_verify_step(win1, None, np.zeros(B), w, cache0, pool0)
    assert np.array_equal(pool1, pool0) and np.array_equal(cache1, cache0)
    o2, pool2, cache2 = oracle.spec_verify_step(win2, win1, acc, w, cache1, pool1)
    for b in range(B):
        st, cc = pool0[b:b + 1], cache0[b:b + 1]
        for t in range(T):  # window 1's outputs: plain steps from the committed point
            args = [win1[n][b, t][None] for n in ("q", "k", "v", "g", "beta")]
            o_t, st, cc = oracle.fused_decode_step(*args, w, cc, st)
            np.testing.assert_allclose(o1[b, t], o_t[0], rtol=1e-13, atol=1e-14)
        st, cc = pool0[b:b + 1], cache0[b:b + 1]
        for t in range(int(acc[b])):
            args = [win1[n][b, t][None] for n in ("q", "k", "v", "g", "beta")]
            _, st, cc = oracle.fused_decode_step(*args, w, cc, st)
        np.testing.assert_allclose(pool2[b], st[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_array_equal(cache2[b], cc[0])
        for t in range(T):
            args = [win2[n][b, t][None] for n in ("q", "k", "v", "g", "beta")]
            o_t, st, cc = oracle.fused_decode_step(*args, w, cc, st)
            np.testing.assert_allclose(o2[b, t], o_t[0], rtol=1e-13, atol=1e-14)


def test_spec_verify_one_token_window_is_the_decode_step():
    """A window of one new token with nothing to replay is one fused step, except
    that the state and cache are not advanced; replaying that token next time
    advances them exactly as the step does."""
    rng = np.random.default_rng(32)
    B, H, K = 2, 2, 4
    w = rng.standard_normal((3, H, K, 4))
    pool0 = rng.standard_normal((B, H, K, K)) * 0.1
    cache0 = rng.standard_normal((B, 3, 3, H, K))
    win = _spec_inputs(rng, B, 1, H, K)
    o, pool1, cache1 = oracle.spec_verify_step(win, None, np.zeros(B), w, cache0, pool0,
                                               norm_weight=np.ones(K) * 2)
    args = [win[n][:, 0] for n in ("q", "k", "v", "g", "beta")]
    o_ref, pool_ref, cache_ref = oracle.fused_decode_step(*args, w, cache0, pool0,
                                                          norm_weight=np.ones(K) * 2)
    np.testing.assert_array_equal(o[:, 0], o_ref)
    assert np.array_equal(pool1, pool0)
    _, pool2, cache2 = oracle.spec_verify_step(_spec_inputs(rng, B, 1, H, K), win,
                                               np.ones(B), w, cache1, pool1,
                                               norm_weight=np.ones(K) * 2)
    np.testing.assert_array_equal(pool2, pool_ref)
    np.testing.assert_array_equal(cache2, cache_ref)


# ------------------------------------------------------------ backward pass
def _bwd_case(seed=41):
    rng = np.random.default_rng(seed)
    H, K, V = 2, 3, 2
    lens = [3, 2]
    T = sum(lens)
    x = {"q": rng.standard_normal((T, H, K)), "k": rng.standard_normal((T, H, K)) * 0.7,
         "v": rng.standard_normal((T, H, V)),
         "g": -np.logaddexp(0.0, rng.standard_normal((T, H, K))),
         "beta": 1 / (1 + np.exp(-rng.standard_normal((T, H)))),
         "S0": rng.standard_normal((2, H, K, V)) * 0.5}
    dO = rng.standard_normal((T, H, V))
    dSf = rng.standard_normal((2, H, K, V))
    return x, dO, dSf, [0, 3, 5]


def _loss(x, dO, dSf, cu, scale):
    o, sf = oracle.recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], cu_seqlens=cu,
                             initial_state=x["S0"], scale=scale)
    return float(np.sum(o * dO) + np.sum(sf * dSf))


def test_backward_matches_central_differences():
    """Every gradient of L = <dO, o> + <dS_final, S_T>, entry by entry, against the
    central difference (L(x + h) - L(x - h)) / 2h of the forward token loop, over
    a two-sequence pack with nonzero initial states and a non-unit scale."""
    x, dO, dSf, cu = _bwd_case()
    scale = 0.8
    got = oracle.recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, cu_seqlens=cu,
                               initial_state=x["S0"], dS_final=dSf, scale=scale)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "dS0"}
    h = 1e-6
    for name, gname in names.items():
        num = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xm = {kk: vv.copy() for kk, vv in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            num[idx] = (_loss(xp, dO, dSf, cu, scale) - _loss(xm, dO, dSf, cu, scale)) / (2 * h)
        np.testing.assert_allclose(got[gname], num, rtol=1e-6, atol=1e-8, err_msg=gname)


def test_backward_special_cases():
    """With beta = 0 and g = 0 the state never changes: dv = 0, dq = scale S0 dO,
    dS0 = scale sum_t q_t dO_t^T + dS_final, dk = 0 (k only enters through the
    erase and the write, both scaled by beta) and dg_t = <dS'_t, S0>."""
    x, dO, dSf, cu = _bwd_case(42)
    x["beta"][:] = 0.0
    x["g"][:] = 0.0
    got = oracle.recurrent_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, cu_seqlens=cu,
                               initial_state=x["S0"], dS_final=dSf, scale=0.5)
    assert np.array_equal(got["dv"], np.zeros_like(got["dv"]))
    assert np.allclose(got["dk"], 0.0, atol=1e-15)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        for h in range(x["q"].shape[1]):
            S0 = x["S0"][n, h]
            np.testing.assert_allclose(got["dq"][a:b, h], 0.5 * dO[a:b, h] @ S0.T, rtol=1e-13)
            ds0 = dSf[n, h] + 0.5 * x["q"][a:b, h].T @ dO[a:b, h]
            np.testing.assert_allclose(got["dS0"][n, h], ds0, rtol=1e-13, atol=1e-14)
            # dL/dS' at token t: dS_final plus the reads of tokens t .. end
            for t in range(a, b):
                dsp = dSf[n, h] + 0.5 * x["q"][t:b, h].T @ dO[t:b, h]
                np.testing.assert_allclose(got["dg"][t, h], np.sum(dsp * S0, axis=1),
                                           rtol=1e-12, atol=1e-13)


# ------------------------------------------- planted mistakes must be caught
def _pins_pass():
    """Run a compact set of the pins above; True if all hold."""
    checks = [
        lambda: test_tiny_matches_equation_form(3, 2, 3),
        test_exact_rational_two_tokens,
        test_beta1_unit_key_reads_back_its_value,
        test_beta0_pure_decay_closed_form,
        test_decay_is_natural_exponential_of_gate,
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def _swap_blocks(src, a, b):
    """Move the text between markers ``b`` before the text between markers ``a``."""
    ia0, ia1 = src.index(f"/*{a}_BEGIN*/"), src.index(f"/*{a}_END*/") + len(f"/*{a}_END*/")
    ib0, ib1 = src.index(f"/*{b}_BEGIN*/"), src.index(f"/*{b}_END*/") + len(f"/*{b}_END*/")
    assert ia1 <= ib0
    return src[:ia0] + src[ib0:ib1] + src[ia1:ib0] + src[ia0:ia1] + src[ib1:]


MUTANTS = {
    # erase term dropped (plain linear attention with decay)
    "no_erase": lambda s: s.replace("bk * (v[j] - r[j]); /*MUT_ERASE*/", "bk * v[j];"),
    # sign of the erase flipped
    "erase_sign": lambda s: s.replace("bk * (v[j] - r[j]); /*MUT_ERASE*/",
                                      "bk * (v[j] + r[j]);"),
    # decay applied to the value axis (columns) instead of the key axis (rows)
    "decay_on_value_axis": lambda s: s.replace(
        "S[(size_t)i * V + j] *= a; /*MUT_DECAY*/",
        "S[(size_t)i * V + j] *= exp(g[j % K]); (void)a;"),
    # base-2 gate instead of natural log
    "base2_gate": lambda s: s.replace("const double a = exp(g[i]);",
                                      "const double a = exp2(g[i]);"),
    # read before the write
    "read_before_write": lambda s: _swap_blocks(s, "MUT_WRITE", "MUT_READ"),
    # erase measured with the query instead of the key
    "erase_with_query": lambda s: s.replace(
        "const double bk = beta * k[i];", "const double bk = beta * q[i];"),
}


def _gate_pins_pass():
    checks = [test_gate_zero_argument_gives_half_the_bound, test_gate_closed_form_per_head,
              test_gate_range_limits_and_page_floor, test_beta_sigmoid_values]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


GATE_MUTANTS = {
    # A_log used without its exponential
    "gate_no_exp": lambda s: s.replace("const double a = exp(A_log[h]);",
                                       "const double a = A_log[h];"),
    # sign inside the sigmoid flipped
    "sigmoid_sign": lambda s: s.replace("return 1.0 / (1.0 + exp(-z));",
                                        "return 1.0 / (1.0 + exp(z));"),
    # bias read as [c, h] instead of [h, c]
    "gate_bias_transposed": lambda s: s.replace("dt_bias[(size_t)h * K + c]",
                                                "dt_bias[(size_t)c * H + h]"),
    # bias added outside the scale
    "gate_bias_unscaled": lambda s: s.replace("lower_bound * sigmoid(a * z);",
                                              "lower_bound * sigmoid(a * x[i] + (z - x[i]));"),
    # every head given head 0's A_log
    "gate_head0": lambda s: s.replace("const double a = exp(A_log[h]);",
                                      "const double a = exp(A_log[0]);"),
}


def _front_pins_pass():
    checks = [test_short_conv_matches_library_correlation, test_short_conv_streams_token_by_token,
              test_swish_identities, test_l2norm_closed_forms, test_rmsnorm_closed_forms]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


FRONT_MUTANTS = {
    # taps applied newest first
    "conv_taps_reversed": lambda s: s.replace("acc += w[(size_t)c * W + i] * ext",
                                              "acc += w[(size_t)c * W + (W - 1 - i)] * ext"),
    # cache left as it was
    "conv_cache_not_updated": lambda s: s.replace(
        "memcpy(cache, ext + (size_t)T * C, sizeof(double) * (size_t)(W - 1) * C);", ""),
    # Swish with the reflected sigmoid
    "swish_sign": lambda s: s.replace("y[i] = x[i] * sigmoid(x[i]);",
                                      "y[i] = x[i] * sigmoid(-x[i]);"),
    # L2 normalisation without the square root
    "l2_no_sqrt": lambda s: s.replace("const double inv = 1.0 / sqrt(ss + eps);",
                                      "const double inv = 1.0 / (ss + eps);"),
    # RMSNorm over the sum instead of the mean
    "rms_sum": lambda s: s.replace("const double inv = 1.0 / sqrt(ss / n + eps);",
                                   "const double inv = 1.0 / sqrt(ss + eps);"),
}


@pytest.mark.parametrize("name", sorted(FRONT_MUTANTS))
def test_front_pins_catch_planted_mistake(name, tmp_path):
    """Plausible mistakes in the decode front end's pieces, planted in a copy of
    the oracle on the CPU, each fail one of their pins."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(SOURCE).read()
    mutated = FRONT_MUTANTS[name](src)
    assert mutated != src, "mutation did not apply"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(mutated)
    lib_path = build_oracle(str(path), str(tmp_path / f"libmut_{name}.so"))
    assert _front_pins_pass(), "unmodified oracle must pass the front-end pins"
    with oracle.using(oracle.open_library(lib_path)):
        assert not _front_pins_pass(), f"planted mistake '{name}' was not caught"


def _bwd_pins_pass():
    for c in (test_backward_matches_central_differences, test_backward_special_cases):
        try:
            c()
        except AssertionError:
            return False
    return True


BWD_MUTANTS = {
    # decay gradient taken against the undecayed state
    "dg_undecayed": lambda s: s.replace("dgi += dSp * Sp[i * V + j];",
                                        "dgi += dSp * Sprev[i * V + j];"),
    # state gradient carried back without the decay
    "dS_no_decay": lambda s: s.replace("dS[i * V + j] = exp(gt[i]) * dSp;",
                                       "dS[i * V + j] = dSp;"),
    # beta gradient with the wrong sign of r
    "dbeta_sign": lambda s: s.replace("db += (vt[j] - r[j]) * du[j];",
                                      "db += (vt[j] + r[j]) * du[j];"),
    # erase path of dk dropped
    "dk_no_erase": lambda s: s.replace("dki += dS[i * V + j] * u[j] + Sp[i * V + j] * dr[j];",
                                       "dki += dS[i * V + j] * u[j];"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_pins_catch_planted_mistake(name, tmp_path):
    """Plausible mistakes in the backward pass, planted in a copy of the oracle on
    the CPU, each fail the finite-difference or special-case pin."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(SOURCE).read()
    mutated = BWD_MUTANTS[name](src)
    assert mutated != src, "mutation did not apply"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(mutated)
    lib_path = build_oracle(str(path), str(tmp_path / f"libmut_{name}.so"))
    assert _bwd_pins_pass(), "unmodified oracle must pass the backward pins"
    with oracle.using(oracle.open_library(lib_path)):
        assert not _bwd_pins_pass(), f"planted mistake '{name}' was not caught"


@pytest.mark.parametrize("name", sorted(GATE_MUTANTS))
def test_gate_pins_catch_planted_mistake(name, tmp_path):
    """Plausible mistakes in the gate and beta front end, planted in a copy of the
    oracle on the CPU, each fail one of the gate pins."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(SOURCE).read()
    mutated = GATE_MUTANTS[name](src)
    assert mutated != src, "mutation did not apply"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(mutated)
    lib_path = build_oracle(str(path), str(tmp_path / f"libmut_{name}.so"))
    assert _gate_pins_pass(), "unmodified oracle must pass the gate pins"
    with oracle.using(oracle.open_library(lib_path)):
        assert not _gate_pins_pass(), f"planted mistake '{name}' was not caught"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    """Each plausible mistake, planted in a copy of the oracle on the CPU, fails
    at least one pin; the unmodified oracle passes them all."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(SOURCE).read()
    mutated = MUTANTS[name](src)
    assert mutated != src, "mutation did not apply"
    path = tmp_path / f"mut_{name}.c"
    path.write_text(mutated)
    lib_path = build_oracle(str(path), str(tmp_path / f"libmut_{name}.so"))
    assert _pins_pass(), "unmodified oracle must pass the pins"
    with oracle.using(oracle.open_library(lib_path)):
        assert not _pins_pass(), f"planted mistake '{name}' was not caught"
