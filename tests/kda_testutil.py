"""Helpers shared by the GPU parity tests (not a test module)."""
import sys

import numpy as np
import torch

import oracle

# Tolerances of max|x_gpu - x_ref| / max|x_ref| per output tensor: 2e-2 for bf16
# inputs with an fp32 state, 1e-4 for fp32 inputs.
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
# The same ratio taken per 64-token chunk of a chain's outputs, each chunk's
# error over that chunk's own max|ref|: an error confined to small-magnitude
# rows (after strong decay, in the 16-token fallback windows, right after a
# hand-over cut) shows here while the chain-wide ratio hides it.
TOL_CHUNK = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    assert np.all(np.isfinite(x)), "non-finite values in GPU output"
    denom = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / denom) if denom > 0 else float(np.max(np.abs(x)))


def chunk_rel_err(x, ref, chunk: int = 64):
    """Largest per-chunk ratio max|x - ref| / max|ref| over the chunks of rows
    [c chunk, (c + 1) chunk) of a chain's outputs, and the chunk it occurs in.
    A chunk whose reference is all zero must come out all zero."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    assert np.all(np.isfinite(x)), "non-finite values in GPU output"
    worst, at = 0.0, -1
    for c in range(0, x.shape[0], chunk):
        d = np.max(np.abs(x[c:c + chunk] - ref[c:c + chunk]))
        m = np.max(np.abs(ref[c:c + chunk]))
        e = d / m if m > 0 else (0.0 if d == 0 else np.inf)
        if e > worst:
            worst, at = float(e), c // chunk
    return worst, at


def to64(t) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def oracle_chains(inp: dict, chains, scale=1.0, nthreads=0, front=None):
    """Run the oracle on selected (sequence n, head h) chains of a prefill batch.

    Returns {(n, h): (o [L, 128], S_final [128, 128])} computed from exactly the
    tensors in ``inp`` (the values the GPU received).  ``front`` (optional dict:
    A_log, dt_bias, lower_bound for the lower-bounded gate when A_log is not None;
    beta_logits) says that g and beta hold logits: the oracle's gate and sigmoid
    turn each chain's logits into g and beta first."""
    cu = inp["cu_seqlens_host"]
    # gather every chain into one packed single-head batch for one oracle call
    qs, ks, vs, gs, bs, s0s, lens = [], [], [], [], [], [], []
    for n, h in chains:
        a, b = cu[n], cu[n + 1]
        qs.append(to64(inp["q"][a:b, h]))
        ks.append(to64(inp["k"][a:b, h]))
        vs.append(to64(inp["v"][a:b, h]))
        g = to64(inp["g"][a:b, h])
        beta = to64(inp["beta"][a:b, h])
        if front is not None and front.get("A_log") is not None:
            dt = front.get("dt_bias")
            g = oracle.lowerbound_gate(g[:, None], to64(front["A_log"][h:h + 1]),
                                       None if dt is None else to64(dt[h:h + 1]),
                                       front["lower_bound"])[:, 0]
        if front is not None and front.get("beta_logits"):
            beta = oracle.sigmoid(beta)
        gs.append(g)
        bs.append(beta)
        s0 = inp.get("initial_state")
        s0s.append(to64(s0[n, h]) if s0 is not None else np.zeros((128, 128)))
        lens.append(b - a)
    cu2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    cat = lambda xs: np.concatenate(xs, axis=0)[:, None]
    o, sf = oracle.recurrent(cat(qs), cat(ks), cat(vs), cat(gs),
                             np.concatenate(bs)[:, None], cu_seqlens=cu2,
                             initial_state=np.stack(s0s)[:, None], scale=scale,
                             nthreads=nthreads)
    out = {}
    for i, (n, h) in enumerate(chains):
        out[(n, h)] = (o[cu2[i]:cu2[i + 1], 0], sf[i, 0])
    return out


def check_prefill_chains(inp: dict, o, sf, chains, dtype, scale=1.0, front=None):
    """Compare a prefill's o and final states on (sequence, head) chains with the
    oracle: chain-wide ratios within TOL and every 64-token chunk of o within
    TOL_CHUNK of its own magnitude; prints the worst of each."""
    ref = oracle_chains(inp, chains, scale=scale, front=front)
    cu = inp["cu_seqlens_host"]
    worst_o = worst_s = 0.0
    worst_c, where_c = 0.0, None
    for (n, h), (o_ref, s_ref) in ref.items():
        a, b = cu[n], cu[n + 1]
        if b > a:
            x = to64(o[a:b, h])
            worst_o = max(worst_o, rel_err(x, o_ref))
            ec, c = chunk_rel_err(x, o_ref)
            if ec > worst_c:
                worst_c, where_c = ec, (n, h, c)
        worst_s = max(worst_s, rel_err(to64(sf[n, h]), s_ref))
    print(f"  max rel err: o {worst_o:.3e}  S_final {worst_s:.3e}  "
          f"o per chunk {worst_c:.3e} at (seq, head, chunk) {where_c}", flush=True)
    assert worst_o <= TOL[dtype], worst_o
    assert worst_s <= TOL[dtype], worst_s
    assert worst_c <= TOL_CHUNK[dtype], (worst_c, where_c)
