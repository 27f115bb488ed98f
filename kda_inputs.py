"""Seeded synthetic inputs for KDA prefill and decode.

This module is shared by the tests, the benchmark and the smoke check.  It holds
only the input recipe (distributions, shapes, sequence-length mixes); none of
the KDA arithmetic.  Both the HIP path and the fp64 oracle consume the tensors
it returns -- the oracle always receives exactly the values the GPU received.

Recipe (the workload statements of the prefill/decode configurations):
  q, k  ~ N(0, 1) per entry, then L2-normalised over the 128 channels of each
          (token, head) in fp32, then cast to the I/O dtype;
  v     ~ N(0, 1), cast to the I/O dtype;
  beta  = sigmoid(N(0, 1)), fp32, one per (token, head);
  g     = -softplus(N(0, 1)), fp32, one per (token, head, key channel)
          (natural-log decay, alpha = exp(g)); with ``g_lower_bound`` the values
          are clamped below at that bound (alpha >= exp(-5) for bound -5);
  S0    = zeros, or N(0, 0.02^2) fp32 when ``init_std`` is given.
Variable-length packs draw lengths log-uniformly (see ``varlen_lengths``).

Gate front end (``gate_logits`` / ``beta_logits``): the same generators give the
raw N(0, 1) draws instead -- gate logits in place of g and beta logits in place
of beta (whose sigmoid is the recipe's beta) -- and ``make_gate_params`` draws
per-head A_log ~ N(a_log_mean, a_log_std^2) and per-channel
dt_bias ~ N(dt_mean, dt_std^2) (the pages give no initialisation; these are
synthetic parameters of the right shapes).

Decode front end (``raw_qk`` and ``make_conv_front``): q and k are the raw
N(0, 1) projections (the kernel's short convolution, Swish and L2 norm make
the unit vectors); conv taps ~ N(0, 0.5^2) per (input, head, channel, tap),
caches ~ N(0, 1) (as if earlier tokens had been seen), cast to the I/O dtype;
output-norm weight 1 + N(0, 0.1^2).  The pages give none of these
distributions.

Every tensor has its own generator seeded from (seed, tensor id), and large
tensors are filled slice by slice (fixed slice size) so that no fp32 staging
copy of a whole bf16 tensor is ever made.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

D = 128
_SLICE_ROWS = 1 << 15  # rows of [rows, H, D] generated per step

_TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "g": 4, "beta": 5, "s0": 6, "A_log": 7, "dt_bias": 8,
               "conv_w": 9, "conv_cache": 10, "norm_w": 11}


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    lengths: tuple            # sequence lengths (one entry per packed sequence)
    heads: int
    dtype: str                # "bf16" or "f32" for q, k, v, o
    init_std: Optional[float] = None   # None -> zero initial state
    g_lower_bound: Optional[float] = None
    chunk: int = 64
    varlen: bool = False      # pass cu_seqlens (True) or a fixed [B, T] batch

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def num_seqs(self) -> int:
        return len(self.lengths)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    heads: int
    steps: int
    init_std: float = 0.02
    ring: int = 16            # distinct per-step inputs, reused cyclically
    dtype: str = "bf16"


def varlen_lengths(n: int = 32, total: int = 1 << 20, lo: int = 1024, hi: int = 1 << 18,
                   seed: int = 1003) -> list:
    """Lengths drawn log-uniformly in [lo, hi], rescaled to sum exactly to ``total``.

    u_i ~ U(ln lo, ln hi); l_i = round(e^{u_i} * total / sum e^u), clipped to
    [lo, hi]; the residual is spread one token at a time, round robin, over the
    entries that are not at a clip bound.  Lengths are not rounded to the chunk
    size, so packed sequences end inside chunks.
    """
    rng = np.random.default_rng(seed)
    e = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
    lengths = np.clip(np.rint(e * total / e.sum()).astype(np.int64), lo, hi)
    resid = int(total - lengths.sum())
    i = 0
    guard = 0
    while resid != 0:
        step = 1 if resid > 0 else -1
        j = i % n
        if lo <= lengths[j] + step <= hi:
            lengths[j] += step
            resid -= step
        i += 1
        guard += 1
        if guard > 100 * n * (abs(resid) + 1):
            raise ValueError("cannot distribute residual within bounds")
    return [int(x) for x in lengths]


# Workloads of the five configurations (names describe the workload itself).
CONFIGS = {
    "kda_fwd_b1_t256_h2_f32": PrefillConfig("kda_fwd_b1_t256_h2_f32", (256,), 2, "f32"),
    "kda_prefill_b4_t8192_h96_bf16": PrefillConfig(
        "kda_prefill_b4_t8192_h96_bf16", (8192,) * 4, 96, "bf16"),
    "kda_prefill_t65536_h96_bf16_s0_gclamp5": PrefillConfig(
        "kda_prefill_t65536_h96_bf16_s0_gclamp5", (65536,), 96, "bf16", init_std=0.02,
        g_lower_bound=-5.0),
    "kda_prefill_varlen32_t1m_h96_bf16": PrefillConfig(
        "kda_prefill_varlen32_t1m_h96_bf16", tuple(varlen_lengths()), 96, "bf16",
        varlen=True),
}
DECODE_CONFIGS = {
    "kda_decode_b512_h96_bf16_f32state": DecodeConfig(
        "kda_decode_b512_h96_bf16_f32state", 512, 96, 1000),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _gen(device, seed: int, tid: int) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + tid)
    return gen


def _fill(out: torch.Tensor, gen: torch.Generator, kind: str, bound=None) -> None:
    """Fill ``out`` ([rows, ...]) slice by slice from ``gen``."""
    rows = out.shape[0]
    for r0 in range(0, rows, _SLICE_ROWS):
        r1 = min(rows, r0 + _SLICE_ROWS)
        shape = (r1 - r0,) + tuple(out.shape[1:])
        x = torch.randn(shape, generator=gen, device=out.device, dtype=torch.float32)
        if kind == "unit":      # L2-normalised over the last dim
            x = x / x.norm(dim=-1, keepdim=True)
        elif kind == "logdecay":  # -softplus(N(0,1)), optionally clamped below
            x = -torch.nn.functional.softplus(x)
            if bound is not None:
                x = torch.clamp(x, min=float(bound))
        elif kind == "sigmoid":
            x = torch.sigmoid(x)
        elif kind == "normal":
            pass
        else:
            raise ValueError(kind)
        out[r0:r1].copy_(x)
        del x


# Gate parameter sets.  "matched": with N(0, 1) gate logits the log-decay has
# about the statistics of the recipe's -softplus(N(0, 1)) (mean ~ -0.8, the same on
# every channel); "heavy": a spread of per-channel biases and per-head scales,
# so that some channels of every head decay fast (near the bound) on many tokens.
GATE_PARAM_SETS = {
    "matched": dict(a_log_mean=0.0, a_log_std=0.1, dt_mean=-2.0, dt_std=0.1),
    "heavy": dict(a_log_mean=0.0, a_log_std=0.5, dt_mean=-2.0, dt_std=0.5),
}


def make_gate_params(heads: int, device="cpu", seed: int = 1009, a_log_mean: float = 0.0,
                     a_log_std: float = 0.1, dt_mean: float = -2.0, dt_std: float = 0.1) -> dict:
    """Per-head A_log [H] and per-channel dt_bias [H, 128], fp32 (defaults: "matched")."""
    A = torch.empty((heads,), dtype=torch.float32, device=device)
    _fill(A.view(heads, 1), _gen(device, seed, _TENSOR_IDS["A_log"]), "normal")
    A.mul_(float(a_log_std)).add_(float(a_log_mean))
    dt = torch.empty((heads, D), dtype=torch.float32, device=device)
    _fill(dt, _gen(device, seed, _TENSOR_IDS["dt_bias"]), "normal")
    dt.mul_(float(dt_std)).add_(float(dt_mean))
    return {"A_log": A, "dt_bias": dt}


def make_prefill(cfg: PrefillConfig, device="cpu", seed: int = 1001, dtype=None,
                 heads: Optional[int] = None, lengths: Optional[Sequence[int]] = None,
                 init_std="cfg", g_lower_bound="cfg", gate_logits: bool = False,
                 beta_logits: bool = False) -> dict:
    """Generate one batch of prefill inputs for ``cfg`` (overrides allowed).

    Returns a dict with q, k, v ([T, H, 128], I/O dtype), g ([T, H, 128] fp32),
    beta ([T, H] fp32), initial_state ([N, H, 128, 128] fp32 or None),
    cu_seqlens (int32 tensor on ``device``), cu_seqlens_host (list) and the
    resolved scalars.
    """
    H = cfg.heads if heads is None else heads
    lens = list(cfg.lengths if lengths is None else lengths)
    dt = torch_dtype(cfg.dtype if dtype is None else dtype)
    std = cfg.init_std if init_std == "cfg" else init_std
    lb = cfg.g_lower_bound if g_lower_bound == "cfg" else g_lower_bound
    T = int(sum(lens))
    out = {}
    for name, kind, tdt in (("q", "unit", dt), ("k", "unit", dt), ("v", "normal", dt)):
        t = torch.empty((T, H, D), dtype=tdt, device=device)
        _fill(t, _gen(device, seed, _TENSOR_IDS[name]), kind)
        out[name] = t
    g = torch.empty((T, H, D), dtype=torch.float32, device=device)
    _fill(g, _gen(device, seed, _TENSOR_IDS["g"]), "normal" if gate_logits else "logdecay", lb)
    beta = torch.empty((T, H), dtype=torch.float32, device=device)
    _fill(beta, _gen(device, seed, _TENSOR_IDS["beta"]), "normal" if beta_logits else "sigmoid")
    out["g"], out["beta"] = g, beta
    if std is None:
        out["initial_state"] = None
    else:
        s0 = torch.empty((len(lens), H, D, D), dtype=torch.float32, device=device)
        _fill(s0, _gen(device, seed, _TENSOR_IDS["s0"]), "normal")
        s0.mul_(float(std))
        out["initial_state"] = s0
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    out["cu_seqlens_host"] = cu
    out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=device)
    out["lengths"] = lens
    out["heads"] = H
    out["dtype"] = dt
    return out


def make_conv_front(slots: int, heads: int, dtype: str = "bf16", device="cpu",
                    seed: int = 1011) -> dict:
    """conv_cache [slots, 3, 3, H, 128] (I/O dtype), conv_weight [3, H, 128, 4] and
    norm_weight [128] (fp32) for the fused decode step."""
    w = torch.empty((3 * heads * D, 4), dtype=torch.float32, device=device)
    _fill(w, _gen(device, seed, _TENSOR_IDS["conv_w"]), "normal")
    w.mul_(0.5)
    cache = torch.empty((slots * 3 * 3 * heads, D), dtype=torch_dtype(dtype), device=device)
    _fill(cache, _gen(device, seed, _TENSOR_IDS["conv_cache"]), "normal")
    nw = torch.empty((D, 1), dtype=torch.float32, device=device)
    _fill(nw, _gen(device, seed, _TENSOR_IDS["norm_w"]), "normal")
    nw.mul_(0.1).add_(1.0)
    return {"conv_weight": w.view(3, heads, D, 4), "conv_cache": cache.view(slots, 3, 3, heads, D),
            "norm_weight": nw.view(D)}


def make_decode_ring(cfg: DecodeConfig, device="cpu", seed: int = 1005,
                     batch: Optional[int] = None, heads: Optional[int] = None,
                     ring: Optional[int] = None, gate_logits: bool = False,
                     beta_logits: bool = False, raw_qk: bool = False) -> dict:
    """Per-step decode inputs for ``ring`` distinct steps plus the initial state pool.

    q, k, g: [ring, B, H, 128]; v: [ring, B, H, 128]; beta: [ring, B, H];
    state: [B, H, 128, 128] fp32 ~ N(0, init_std^2).
    """
    B = cfg.batch if batch is None else batch
    H = cfg.heads if heads is None else heads
    R = cfg.ring if ring is None else ring
    dt = torch_dtype(cfg.dtype)
    out = {}
    for name, kind in (("q", "normal" if raw_qk else "unit"), ("k", "normal" if raw_qk else "unit"),
                       ("v", "normal")):
        t = torch.empty((R * B, H, D), dtype=dt, device=device)
        _fill(t, _gen(device, seed, _TENSOR_IDS[name]), kind)
        out[name] = t.view(R, B, H, D)
    g = torch.empty((R * B, H, D), dtype=torch.float32, device=device)
    _fill(g, _gen(device, seed, _TENSOR_IDS["g"]), "normal" if gate_logits else "logdecay")
    beta = torch.empty((R * B, H), dtype=torch.float32, device=device)
    _fill(beta, _gen(device, seed, _TENSOR_IDS["beta"]), "normal" if beta_logits else "sigmoid")
    out["g"], out["beta"] = g.view(R, B, H, D), beta.view(R, B, H)
    s = torch.empty((B, H, D, D), dtype=torch.float32, device=device)
    _fill(s, _gen(device, seed, _TENSOR_IDS["s0"]), "normal")
    s.mul_(float(cfg.init_std))
    out["state"] = s
    return out
