"""fp64 CPU oracle for Kimi Delta Attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  The HIP product library never calls it, and this
package imports nothing from the product package.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, OpenMP over
(sequence, head)); this module only marshals numpy arrays through ctypes.
Sources are cited in the C file: the token loop of "How Kimi K3 Engineered Its
Way to the Frontier" (section "How KDA updates its state"), the KDA equation of
"Kimi K3: Open Frontier Intelligence" (section 6) and of "Kimi K3: a 2.8T open
model ..." (section "Kimi Delta Attention"), and the segment transition of
"Kimi K3 -- Training and Infrastructure Notes" (section 4.1).
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np

from .build import build_oracle, library_path

__all__ = [
    "recurrent",
    "recurrent_bwd",
    "chunked",
    "decode_step",
    "transition",
    "lowerbound_gate",
    "sigmoid",
    "short_conv",
    "swish",
    "l2norm",
    "rmsnorm",
    "fused_decode_step",
    "spec_verify_step",
    "max_threads",
    "load",
    "open_library",
    "using",
]

_LIB = None
_DP = ctypes.POINTER(ctypes.c_double)
_I64P = ctypes.POINTER(ctypes.c_int64)


def load(rebuild: bool = False):
    """Load (building with gcc first if needed) the oracle shared library."""
    global _LIB
    if _LIB is not None and not rebuild:
        return _LIB
    path = library_path()
    if rebuild or not os.path.exists(path):
        build_oracle()
    _LIB = open_library(path)
    return _LIB


@contextlib.contextmanager
def using(lib):
    """Temporarily route this module's functions through another build of the
    oracle (the tests use it to run the pins against planted mistakes)."""
    global _LIB
    saved = _LIB
    _LIB = lib
    try:
        yield lib
    finally:
        _LIB = saved


def open_library(path):
    """Open an oracle shared library at ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    lib.kda_oracle_recurrent.argtypes = [
        ctypes.c_int, _I64P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _DP, _DP, _DP, _DP, _DP, ctypes.c_double, _DP, _DP, _DP, ctypes.c_int,
    ]
    lib.kda_oracle_chunked.argtypes = [
        ctypes.c_int, _I64P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _DP, _DP, _DP, _DP, _DP, ctypes.c_double, _DP, _DP, _DP, ctypes.c_int,
    ]
    lib.kda_oracle_decode_step.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _DP, _DP, _DP, _DP, _DP, ctypes.c_double, _DP, _I64P, ctypes.c_int64, _DP,
        ctypes.c_int,
    ]
    lib.kda_oracle_transition.argtypes = [
        ctypes.c_int64, ctypes.c_int, ctypes.c_int, _DP, _DP, _DP, _DP, _DP, _DP,
    ]
    lib.kda_oracle_recurrent_bwd.argtypes = [
        ctypes.c_int, _I64P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _DP, _DP, _DP, _DP, _DP, ctypes.c_double, _DP, _DP, _DP, _DP, _DP, _DP, _DP, _DP, _DP,
    ]
    lib.kda_oracle_recurrent_bwd.restype = ctypes.c_int
    lib.kda_oracle_lowerbound_gate.argtypes = [
        ctypes.c_int64, ctypes.c_int, ctypes.c_int, _DP, _DP, _DP, ctypes.c_double, _DP,
    ]
    lib.kda_oracle_sigmoid.argtypes = [ctypes.c_int64, _DP, _DP]
    lib.kda_oracle_short_conv.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, _DP, _DP,
                                          _DP, _DP]
    lib.kda_oracle_swish.argtypes = [ctypes.c_int64, _DP, _DP]
    lib.kda_oracle_l2norm.argtypes = [ctypes.c_int64, ctypes.c_int, _DP, ctypes.c_double, _DP]
    lib.kda_oracle_rmsnorm.argtypes = [ctypes.c_int64, ctypes.c_int, _DP, _DP, ctypes.c_double,
                                       _DP]
    lib.kda_oracle_max_threads.argtypes = []
    for fn in ("kda_oracle_recurrent", "kda_oracle_chunked", "kda_oracle_decode_step",
               "kda_oracle_transition", "kda_oracle_lowerbound_gate", "kda_oracle_sigmoid",
               "kda_oracle_short_conv", "kda_oracle_swish", "kda_oracle_l2norm",
               "kda_oracle_rmsnorm", "kda_oracle_max_threads"):
        getattr(lib, fn).restype = ctypes.c_int
    return lib


def _f64(a, name):
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor: upcast exactly what it holds
        a = a.detach().to("cpu").double().numpy()
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_DP)


def _cu(cu_seqlens, T):
    if cu_seqlens is None:
        raise ValueError("cu_seqlens is required")
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if cu.ndim != 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be non-decreasing, start at 0 and end at T_total")
    return cu


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def _common(q, k, v, g, beta, cu_seqlens, initial_state):
    q, k, v, g, beta = (_f64(x, n) for x, n in
                        ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta")))
    if q.ndim != 3 or k.shape != q.shape or g.shape != q.shape:
        raise ValueError("q, k, g must be [T, H, K] with equal shapes")
    T, H, K = q.shape
    if v.ndim != 3 or v.shape[:2] != (T, H):
        raise ValueError("v must be [T, H, V]")
    V = v.shape[2]
    if beta.shape != (T, H):
        raise ValueError("beta must be [T, H]")
    if cu_seqlens is None:
        cu_seqlens = [0, T]
    cu = _cu(cu_seqlens, T)
    N = cu.shape[0] - 1
    s0 = _f64(initial_state, "initial_state")
    if s0 is not None and s0.shape != (N, H, K, V):
        raise ValueError(f"initial_state must be [{N}, {H}, {K}, {V}]")
    return q, k, v, g, beta, cu, s0, T, H, K, V, N


def recurrent(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=1.0,
              nthreads=0):
    """Token-by-token KDA (the definition). Returns (o [T,H,V], S_final [N,H,K,V])."""
    lib = load()
    q, k, v, g, beta, cu, s0, T, H, K, V, N = _common(q, k, v, g, beta, cu_seqlens,
                                                      initial_state)
    o = np.zeros((T, H, V))
    sf = np.zeros((N, H, K, V))
    rc = lib.kda_oracle_recurrent(N, cu.ctypes.data_as(_I64P), H, K, V, _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(s0),
                                  _ptr(o), _ptr(sf), int(nthreads))
    _check(rc, "kda_oracle_recurrent")
    return o, sf


def recurrent_bwd(q, k, v, g, beta, dO, cu_seqlens=None, initial_state=None, dS_final=None,
                  scale=1.0):
    """Gradients of L = sum <dO, o> + <dS_final, S_T> through the token loop.

    Shapes as in ``recurrent``; dO: [T, H, V]; dS_final: [N, H, K, V] or None.
    Returns a dict of dq, dk, dg [T, H, K], dv [T, H, V], dbeta [T, H] and
    dS0 [N, H, K, V] (fp64).
    """
    lib = load()
    q, k, v, g, beta, cu, s0, T, H, K, V, N = _common(q, k, v, g, beta, cu_seqlens,
                                                        initial_state)
    dO = _f64(dO, "dO")
    if dO.shape != (T, H, V):
        raise ValueError("dO must be [T, H, V]")
    dsf = _f64(dS_final, "dS_final")
    if dsf is not None and dsf.shape != (N, H, K, V):
        raise ValueError(f"dS_final must be [{N}, {H}, {K}, {V}]")
    out = {"dq": np.zeros((T, H, K)), "dk": np.zeros((T, H, K)), "dv": np.zeros((T, H, V)),
           "dg": np.zeros((T, H, K)), "dbeta": np.zeros((T, H)), "dS0": np.zeros((N, H, K, V))}
    rc = lib.kda_oracle_recurrent_bwd(N, cu.ctypes.data_as(_I64P), H, K, V, _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(s0),
                                      _ptr(dO), _ptr(dsf), *(_ptr(out[n]) for n in
                                      ("dq", "dk", "dv", "dg", "dbeta", "dS0")))
    _check(rc, "kda_oracle_recurrent_bwd")
    return out


def chunked(q, k, v, g, beta, chunk_size, cu_seqlens=None, initial_state=None, scale=1.0,
            nthreads=0):
    """Chunkwise KDA in fp64 (block form of the same recurrence). Same returns."""
    lib = load()
    q, k, v, g, beta, cu, s0, T, H, K, V, N = _common(q, k, v, g, beta, cu_seqlens,
                                                      initial_state)
    o = np.zeros((T, H, V))
    sf = np.zeros((N, H, K, V))
    rc = lib.kda_oracle_chunked(N, cu.ctypes.data_as(_I64P), H, K, V, int(chunk_size),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                float(scale), _ptr(s0), _ptr(o), _ptr(sf), int(nthreads))
    _check(rc, "kda_oracle_chunked")
    return o, sf


def decode_step(q, k, v, g, beta, state_pool, slot_idx=None, scale=1.0, nthreads=0):
    """One decode token per row, in place on a copy of ``state_pool``.

    q, k, g: [B, H, K]; v: [B, H, V]; beta: [B, H]; state_pool: [S, H, K, V].
    Returns (o [B, H, V] -- NaN rows for skipped slots, new_state_pool).
    """
    lib = load()
    q, k, v, g, beta = (_f64(x, "x") for x in (q, k, v, g, beta))
    B, H, K = q.shape
    V = v.shape[2]
    pool = np.array(_f64(state_pool, "state_pool"), copy=True)
    if pool.shape[1:] != (H, K, V):
        raise ValueError("state_pool must be [slots, H, K, V]")
    idx = None
    if slot_idx is not None:
        idx = np.ascontiguousarray(np.asarray(slot_idx, dtype=np.int64))
        if idx.shape != (B,):
            raise ValueError("slot_idx must be [B]")
    o = np.full((B, H, V), np.nan)
    rc = lib.kda_oracle_decode_step(B, H, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), float(scale), _ptr(pool),
                                    None if idx is None else idx.ctypes.data_as(_I64P),
                                    pool.shape[0], _ptr(o), int(nthreads))
    _check(rc, "kda_oracle_decode_step")
    return o, pool


def transition(k, v, g, beta):
    """Segment transition of one head: returns (M [K,K], S_tilde [K,V]).

    k, g: [T, K]; v: [T, V]; beta: [T].  S_out = M @ S_in + S_tilde.
    """
    lib = load()
    k, v, g, beta = (_f64(x, "x") for x in (k, v, g, beta))
    T, K = k.shape
    V = v.shape[1]
    M = np.zeros((K, K))
    St = np.zeros((K, V))
    rc = lib.kda_oracle_transition(T, K, V, _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(M), _ptr(St))
    _check(rc, "kda_oracle_transition")
    return M, St


def lowerbound_gate(x, A_log, dt_bias=None, lower_bound=-5.0):
    """K3's lower-bounded gate: g = lower_bound * sigmoid(exp(A_log[h]) * (x + dt_bias[h])).

    x: [..., H, K] raw gate logits; A_log: [H]; dt_bias: [H, K] (or anything of
    H*K values) or None.  Returns fp64 g of x's shape.
    """
    lib = load()
    x = _f64(x, "x")
    if x.ndim < 2:
        raise ValueError("x must be [..., H, K]")
    H, K = x.shape[-2:]
    A = _f64(A_log, "A_log").reshape(-1)
    if A.shape != (H,):
        raise ValueError(f"A_log must hold {H} values")
    dt = _f64(dt_bias, "dt_bias")
    if dt is not None:
        dt = np.ascontiguousarray(dt.reshape(-1))
        if dt.shape != (H * K,):
            raise ValueError(f"dt_bias must hold {H * K} values")
    T = x.size // (H * K)
    g = np.empty_like(x)
    rc = lib.kda_oracle_lowerbound_gate(T, H, K, _ptr(x), _ptr(A), _ptr(dt),
                                        float(lower_bound), _ptr(g))
    _check(rc, "kda_oracle_lowerbound_gate")
    return g


def sigmoid(x):
    """beta from beta logits: 1 / (1 + exp(-x)), elementwise, fp64."""
    lib = load()
    x = _f64(x, "x")
    y = np.empty_like(x)
    rc = lib.kda_oracle_sigmoid(x.size, _ptr(x), _ptr(y))
    _check(rc, "kda_oracle_sigmoid")
    return y


def short_conv(x, w, cache):
    """Causal depthwise convolution continuing from ``cache``.

    x: [T, C] inputs; w: [C, W] taps (oldest first); cache: [W - 1, C] previous
    inputs (oldest first).  Returns (y [T, C], new cache [W - 1, C]).
    """
    lib = load()
    x = _f64(x, "x")
    w = _f64(w, "w")
    T, C = x.shape
    if w.ndim != 2 or w.shape[0] != C:
        raise ValueError("w must be [C, W]")
    W = w.shape[1]
    cache = np.array(_f64(cache, "cache"), copy=True)
    if cache.shape != (W - 1, C):
        raise ValueError(f"cache must be [{W - 1}, {C}]")
    y = np.empty_like(x)
    rc = lib.kda_oracle_short_conv(T, C, W, _ptr(x), _ptr(w), _ptr(cache), _ptr(y))
    _check(rc, "kda_oracle_short_conv")
    return y, cache


def swish(x):
    """x * sigmoid(x), elementwise."""
    lib = load()
    x = _f64(x, "x")
    y = np.empty_like(x)
    _check(lib.kda_oracle_swish(x.size, _ptr(x), _ptr(y)), "kda_oracle_swish")
    return y


def l2norm(x, eps=1e-6):
    """x / sqrt(sum x^2 + eps) over the last axis."""
    lib = load()
    x = _f64(x, "x")
    y = np.empty_like(x)
    n = x.shape[-1]
    _check(lib.kda_oracle_l2norm(x.size // n, n, _ptr(x), float(eps), _ptr(y)),
           "kda_oracle_l2norm")
    return y


def rmsnorm(x, weight=None, eps=1e-6):
    """x / sqrt(mean x^2 + eps) * weight over the last axis (weight [n] or None)."""
    lib = load()
    x = _f64(x, "x")
    y = np.empty_like(x)
    n = x.shape[-1]
    w = _f64(weight, "weight")
    if w is not None:
        w = np.ascontiguousarray(w.reshape(-1))
        if w.shape != (n,):
            raise ValueError(f"weight must hold {n} values")
    _check(lib.kda_oracle_rmsnorm(x.size // n, n, _ptr(x), _ptr(w), float(eps), _ptr(y)),
           "kda_oracle_rmsnorm")
    return y


def fused_decode_step(q_in, k_in, v_in, g, beta, conv_w, conv_cache, state_pool,
                      slot_idx=None, scale=1.0, l2_eps=1e-6, norm_weight=None,
                      norm_eps=1e-6, out_norm=True, gate=None):
    """One decode token per row with the layer's front and back end, composed from
    the functions above ("Kimi K3 -- Training and Infrastructure Notes", section 4.5:
    one kernel covers short convolution, input normalisation, gating, the
    recurrence and output normalisation; "Kimi K3: a 2.8T open model ...",
    "Kimi Delta Attention": q, k from a short convolution, Swish and L2
    normalisation, v from a short convolution and Swish).

    Per row b with slot s = slot_idx[b] (b when None; negative = skipped):
      for each of q, k, v (index i = 0, 1, 2): the short convolution of the row's
      raw input continuing from conv_cache[s, i] with taps conv_w[i] (width 4),
      then Swish; q and k L2-normalised per head; with ``gate`` (dict A_log,
      dt_bias, lower_bound, beta_logits) g and beta are logits turned by the
      lower-bounded gate and the sigmoid; the KDA step on state_pool[s]; o
      RMSNorm-ed per head with ``norm_weight`` [V] (or weight 1) if out_norm.

    q_in, k_in, v_in, g: [B, H, K]; beta: [B, H]; conv_w: [3, H, K, W];
    conv_cache: [slots, 3, W - 1, H, K]; state_pool: [slots, H, K, V].
    Returns (o [B, H, V] (NaN for skipped rows), new state_pool, new conv_cache).
    """
    ins = [_f64(t, "x") for t in (q_in, k_in, v_in)]
    B, H, K = ins[0].shape
    w = _f64(conv_w, "conv_w")
    W = w.shape[-1]
    cache = np.array(_f64(conv_cache, "conv_cache"), copy=True)
    if w.shape != (3, H, K, W) or cache.shape[1:] != (3, W - 1, H, K):
        raise ValueError("conv_w must be [3, H, K, W] and conv_cache [slots, 3, W-1, H, K]")
    slots = (np.arange(B) if slot_idx is None
             else np.asarray(_f64(slot_idx, "slot_idx")).astype(np.int64))
    conv = [np.zeros((B, H, K)) for _ in range(3)]
    for b in range(B):
        s = int(slots[b])
        if s < 0:
            continue
        for i in range(3):
            y, c_new = short_conv(ins[i][b].reshape(1, H * K), w[i].reshape(H * K, W),
                                  cache[s, i].reshape(W - 1, H * K))
            conv[i][b] = swish(y).reshape(H, K)
            cache[s, i] = c_new.reshape(W - 1, H, K)
    q = l2norm(conv[0], l2_eps)
    k = l2norm(conv[1], l2_eps)
    v = conv[2]
    g = _f64(g, "g")
    beta = _f64(beta, "beta")
    if gate is not None:
        if gate.get("A_log") is not None:
            g = lowerbound_gate(g, gate["A_log"], gate.get("dt_bias"), gate["lower_bound"])
        if gate.get("beta_logits"):
            beta = sigmoid(beta)
    o, pool = decode_step(q, k, v, g, beta, state_pool,
                          None if slot_idx is None else slots, scale=scale)
    if out_norm:
        live = slots >= 0
        o[live] = rmsnorm(o[live], norm_weight, norm_eps)
    return o, pool, cache


def spec_verify_step(new, replay, num_replay, conv_w, conv_cache, state_pool, slot_idx=None,
                     **kw):
    """Speculative-decode verification with replay ("Kimi K3 -- Training and
    Infrastructure Notes", section 4.5, KDA decoding: the state after an accepted
    draft prefix is determined by the drafts' projected inputs, so only those are
    kept; the accepted tokens are replayed to rebuild the state, the state of the
    verified tokens is written back, and the replayed tokens and the next window
    run in one recurrent loop).

    Per row b with slot s (skipped when negative): first the first num_replay[b]
    (clamped to [0, Tr]) tokens of ``replay`` (the previous window's projected inputs) go through
    ``fused_decode_step`` in order; the state and conv cache reached are the ones
    written back.  Then the T tokens of ``new`` go through the same steps from
    there, and their outputs are returned; the state they reach is dropped.

    new, replay: dicts of q, k, v, g [B, T, H, K] and beta [B, T, H] (replay may
    have a different T, or be None with num_replay all zero); num_replay: [B];
    the other arguments as in ``fused_decode_step``.
    Returns (o [B, T, H, V], new state_pool, new conv_cache).
    """
    nq = _f64(new["q"], "q")
    B, T, H, K = nq.shape
    slots = np.arange(B) if slot_idx is None else np.asarray(slot_idx).astype(np.int64)
    num_replay = np.asarray(num_replay).astype(np.int64)
    pool = np.array(_f64(state_pool, "state_pool"), copy=True)
    cache = np.array(_f64(conv_cache, "conv_cache"), copy=True)
    V = pool.shape[-1]
    o = np.full((B, T, H, V), np.nan)
    names = ("q", "k", "v", "g", "beta")
    for b in range(B):
        s = int(slots[b])
        if s < 0:
            continue
        st, cc = pool[s:s + 1], cache[s:s + 1]
        n_rep = 0 if replay is None else min(max(int(num_replay[b]), 0), replay["q"].shape[1])
        for t in range(n_rep):
            args = [_f64(replay[n], n)[b, t][None] for n in names]
            _, st, cc = fused_decode_step(*args, conv_w, cc, st, **kw)
        pool[s:s + 1], cache[s:s + 1] = st, cc  # written back
        for t in range(T):
            args = [_f64(new[n], n)[b, t][None] for n in names]
            o_t, st, cc = fused_decode_step(*args, conv_w, cc, st, **kw)
            o[b, t] = o_t[0]
    return o, pool, cache


def max_threads() -> int:
    return int(load().kda_oracle_max_threads())
