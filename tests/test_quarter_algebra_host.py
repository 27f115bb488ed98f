"""The algebra of the gate prefill's quarter-mode window, checked on the host.

A 64-token window whose decay range is too wide for one reference keeps one
reference per 16-token quarter (its token 8).  The kernel then runs the window
as one pipeline step ("How Kimi K3 Engineered Its Way to the Frontier",
section "FlashKDA steps the state once per 16 tokens": the chunk's work as
dense products, exponentials of cumulative decays kept in range):

- operands per quarter q against its reference Gm_q:
  nKr = -beta k e^{G - Gm_q}, Qr = q e^{G - Gm_q}, Kc = k e^{Gm_q - G};
- Gram tile (i, j), i > j: quarter j's Kc scaled per channel by
  e_ij = e^{Gm_i - Gm_j} <= 1 before the product, diagonal tiles as they are;
- Y and O rows of quarter q against d_q S' (S' = e^{Gm_0} S, d_q = e^{Gm_q - Gm_0});
- U from the whole lower-triangular system, O += P U over all tiles;
- the state quarter by quarter: S' <- r_{q-1} S' + Kc_q^T U_q with
  r_q = e^{Gm_{q+1} - Gm_q}, and S_next = e^{G_end - Gm_3} S'.

This test evaluates exactly that sequence of steps in fp64, with the
per-channel factors (e, d, r and the window multipliers) rounded to fp32 as the
kernel stores them, and compares it with the oracle's token loop (the
definition).  Decays at the page's -5 floor make the far cross-quarter factors
underflow to zero in fp32; the test checks that they do and that the result
still matches, i.e. that what underflows is negligible where it is added.
"""
import numpy as np
import pytest

import oracle

C = 64   # tokens per window
Q = 16   # tokens per quarter
D = 128  # head dimension


def f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def quarter_window(q, k, v, beta, g, S, scale):
    """One window (tokens 0..63) from incoming state S [D, D], the quarter-mode
    steps in order.  Returns (o [64, D], S_next [D, D])."""
    G = np.cumsum(g, axis=0)                    # [64, D] cumulative log-decay (natural)
    Gm = G[np.arange(4) * Q + 8]                # [4, D] quarter references
    quarter = np.arange(C) // Q
    # operands against each row's quarter reference
    nkr = -beta[:, None] * k * np.exp(G - Gm[quarter])
    qr = q * np.exp(G - Gm[quarter])
    kc = k * np.exp(Gm[quarter] - G)
    # factors as the kernel stores them (fp32, all <= 1)
    r = f32(np.exp(Gm[1:] - Gm[:-1]))           # r_q, q = 0..2
    d = f32(np.exp(Gm - Gm[0]))                 # d_q (d_0 = 1)
    mfac = f32(np.exp(Gm[0]))                   # window multiplier (start reference)
    post = f32(np.exp(G[-1] - Gm[3]))           # end factor
    e = np.ones((4, 4, D))
    for i in range(4):
        for j in range(i):
            e[i, j] = np.prod(r[j:i], axis=0)   # the Gram's product of slot factors
    # Gram tiles into Lm (-beta A, strictly lower) and P (lower incl. diagonal)
    Lm = np.zeros((C, C))
    P = np.zeros((C, C))
    for i in range(4):
        for j in range(i + 1):
            ri, rj = slice(Q * i, Q * i + Q), slice(Q * j, Q * j + Q)
            kcj = kc[rj] * (e[i, j] if i > j else 1.0)
            Lm[ri, rj] = nkr[ri] @ kcj.T
            P[ri, rj] = qr[ri] @ kcj.T
    Lm = np.tril(Lm, -1)
    P = np.tril(P)
    # Y and O^T rows per quarter against the state at that quarter's reference
    Sp = mfac[:, None] * S                      # S' at reference 0 (rows = channels)
    Y = np.zeros((C, D))
    O = np.zeros((C, D))
    for i in range(4):
        ri = slice(Q * i, Q * i + Q)
        Sq = d[i][:, None] * Sp
        Y[ri] = beta[ri, None] * v[ri] + nkr[ri] @ Sq
        O[ri] = qr[ri] @ Sq
    U = np.linalg.solve(np.eye(C) - Lm, Y)     # (I + beta A) U = Y
    O = O + P @ U
    # state update quarter by quarter
    acc = Sp.copy()
    for i in range(4):
        ri = slice(Q * i, Q * i + Q)
        if i > 0:
            acc = r[i - 1][:, None] * acc
        acc = acc + kc[ri].T @ U[ri]
    return scale * O, post[:, None] * acc


def run_windows(q, k, v, beta, g, S0, scale):
    S = S0
    outs = []
    for w in range(q.shape[0] // C):
        t = slice(C * w, C * w + C)
        o, S = quarter_window(q[t], k[t], v[t], beta[t], g[t], S, scale)
        outs.append(o)
    return np.concatenate(outs), S


@pytest.mark.parametrize("case", ["floor", "mixed"])
def test_quarter_mode_window_matches_token_loop(case):
    rng = np.random.default_rng(17 if case == "floor" else 29)
    T = 3 * C
    q = rng.standard_normal((T, D)) / np.sqrt(D)
    k = rng.standard_normal((T, D))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, D))
    beta = rng.uniform(0.1, 0.9, T)
    if case == "floor":  # every channel at or near the page's -5 floor
        g = -5.0 + rng.uniform(0.0, 0.5, (T, D))
    else:  # half the channels at the floor, half slow
        g = np.where(rng.uniform(size=(1, D)) < 0.5, -5.0 + rng.uniform(0, 0.3, (T, D)),
                     -rng.uniform(0.0, 0.1, (T, D)))
    S0 = 0.3 * rng.standard_normal((D, D))
    scale = D ** -0.5
    o, S = run_windows(q, k, v, beta, g, S0, scale)
    o_ref, s_ref = oracle.recurrent(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None],
                                    initial_state=S0[None, None], scale=scale)
    o_ref, s_ref = o_ref[:, 0], s_ref[0, 0]
    err_o = np.abs(o - o_ref).max() / np.abs(o_ref).max()
    err_s = np.abs(S - s_ref).max() / max(np.abs(s_ref).max(), 1e-300)
    assert err_o < 1e-6 and err_s < 1e-6, (err_o, err_s)
    # per 16-token quarter too, so small rows after strong decay are checked on their own scale
    for t0 in range(0, T, Q):
        blk = slice(t0, t0 + Q)
        assert np.abs(o[blk] - o_ref[blk]).max() <= 1e-6 * np.abs(o_ref[blk]).max() + 1e-300
    # the far cross-quarter factors do underflow in fp32 at the floor
    G = np.cumsum(g[:C], axis=0)
    far = np.exp(G[3 * Q + 8] - G[8]).astype(np.float32)
    assert (far == 0).any() if case == "floor" else True


def test_single_reference_would_overflow():
    """The reason for quarter mode: at the floor, one reference per 64-token
    window puts factors far outside fp32 (and bf16, the operands' type)."""
    g = np.full(C, -5.0)
    G = np.cumsum(g)
    assert np.exp(G[31] - G[63]) > np.finfo(np.float32).max
    quarter = np.arange(C) // Q
    Gm = G[np.arange(4) * Q + 8]
    assert np.abs(G - Gm[quarter]).max() * np.log2(np.e) < 64  # per-quarter: within 2^64
