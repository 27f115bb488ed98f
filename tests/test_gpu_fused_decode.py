"""GPU parity of the fused decode step (kda_fused_decode_step) against the oracle.

The kernel runs the layer's front end (short convolution of q, k, v continuing
from per-slot caches, Swish, L2 norm of q and k), the recurrent step and the
output RMSNorm in one launch ("Kimi K3 -- Training and Infrastructure Notes",
section 4.5; "Kimi K3: a 2.8T open model ...", "Kimi Delta Attention"); the
oracle composes its pinned pieces in fp64 on exactly the values the GPU read.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testutil import TOL, announce, rel_err, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_10_amd as m
    m.library()
    return m


def step_both(kda, x, t, front, pool_gpu, pool_ref, cache_ref, idx, **kw):
    """One fused step on the GPU (in place) and in the oracle; returns both outputs
    and the oracle's new pool and cache."""
    gate = kw.pop("gate", None)
    gkw = {}
    if gate is not None:
        gkw = dict(A_log=gate.get("A_log"), dt_bias=gate.get("dt_bias"),
                   lower_bound=gate["lower_bound"], beta_logits=gate.get("beta_logits", False))
    o = kda.fused_decode_step(x["q"][t], x["k"][t], x["v"][t], x["g"][t], x["beta"][t],
                              pool_gpu, front["conv_cache"], front["conv_weight"],
                              state_indices=idx, **kw, **gkw)
    o_ref, pool_ref, cache_ref = oracle.fused_decode_step(
        x["q"][t], x["k"][t], x["v"][t], x["g"][t], x["beta"][t], front["conv_weight"],
        cache_ref, pool_ref, None if idx is None else idx.cpu().numpy(),
        scale=kw.get("scale", 1.0), l2_eps=kw.get("l2_eps", 1e-6),
        norm_weight=kw.get("norm_weight"), norm_eps=kw.get("norm_eps", 1e-6),
        out_norm=kw.get("out_norm", True), gate=gate)
    return o, o_ref, pool_ref, cache_ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fused_steps_with_slots_vs_oracle(kda, dtype):
    """Five chained steps, a skipped row, scattered slots, the output RMSNorm with
    a weight; the conv caches match the oracle's exactly (raw inputs shifted)."""
    announce(f"fused decode slots dtype={dtype}")
    dev = "cuda"
    B, H, slots, steps = 6, 3, 9, 5
    name = "bf16" if dtype == torch.bfloat16 else "f32"
    cfg = ki.DecodeConfig("t", B, H, steps, dtype=name)
    x = ki.make_decode_ring(cfg, device=dev, ring=steps, raw_qk=True)
    front = ki.make_conv_front(slots, H, name, device=dev)
    pool = torch.randn((slots, H, 128, 128), device=dev, dtype=torch.float32) * 0.05
    idx = torch.tensor([4, 0, -1, 8, 2, 7], dtype=torch.int32, device=dev)
    cache0 = front["conv_cache"].clone()
    pool_ref, cache_ref = to64(pool), to64(cache0)
    gpu_pool = pool.clone()
    live = [b for b in range(B) if idx[b] >= 0]
    for t in range(steps):
        o, o_ref, pool_ref, cache_ref = step_both(kda, x, t, front, gpu_pool, pool_ref, cache_ref,
                                                  idx, scale=0.7,
                                                  norm_weight=front["norm_weight"])
        torch.cuda.synchronize()
        err = rel_err(to64(o)[live], o_ref[live])
        print(f"  step {t}: o rel err {err:.3e}", flush=True)
        assert err <= TOL[dtype]
    assert rel_err(to64(gpu_pool), pool_ref) <= 1e-4
    assert np.array_equal(to64(front["conv_cache"]), cache_ref)
    for s in (1, 3, 5, 6):  # the skipped row's slot and the unused slots are untouched
        assert torch.equal(gpu_pool[s], pool[s])
        assert torch.equal(front["conv_cache"][s], cache0[s])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fused_gate_beta_logits_without_norm_weight(kda, dtype):
    """Gate logits and beta logits, output norm without a weight, then with the
    norm switched off; identity slots."""
    announce(f"fused decode gate dtype={dtype}")
    dev = "cuda"
    B, H, steps = 4, 2, 3
    name = "bf16" if dtype == torch.bfloat16 else "f32"
    cfg = ki.DecodeConfig("t", B, H, steps, dtype=name)
    x = ki.make_decode_ring(cfg, device=dev, ring=steps, raw_qk=True, gate_logits=True,
                            beta_logits=True)
    front = ki.make_conv_front(B, H, name, device=dev, seed=1013)
    gp = ki.make_gate_params(H, device=dev, seed=1015, **ki.GATE_PARAM_SETS["heavy"])
    gate = {"A_log": gp["A_log"], "dt_bias": gp["dt_bias"], "lower_bound": -5.0,
            "beta_logits": True}
    pool = torch.randn((B, H, 128, 128), device=dev, dtype=torch.float32) * 0.05
    pool_ref, cache_ref = to64(pool), to64(front["conv_cache"])
    for t in range(steps):
        out_norm = t < 2
        o, o_ref, pool_ref, cache_ref = step_both(kda, x, t, front, pool, pool_ref, cache_ref,
                                                  None, gate=gate, out_norm=out_norm)
        torch.cuda.synchronize()
        assert rel_err(to64(o), o_ref) <= TOL[dtype]
    assert rel_err(to64(pool), pool_ref) <= 1e-4
    assert np.array_equal(to64(front["conv_cache"]), cache_ref)


def test_fused_full_b512_h96_sampled(kda):
    """512 rows x 96 heads, bf16, fp32 states in place, the decode workload's
    launch; three rows (all heads) replayed by the oracle."""
    announce("fused decode full b512 h96")
    dev = "cuda"
    cfg = ki.DECODE_CONFIGS["kda_decode_b512_h96_bf16_f32state"]
    x = ki.make_decode_ring(cfg, device=dev, ring=1, raw_qk=True)
    front = ki.make_conv_front(cfg.batch, cfg.heads, "bf16", device=dev)
    state = x["state"]
    rows = [0, 257, 511]
    pool_ref = to64(state[rows])
    cache_ref = to64(front["conv_cache"][rows])
    o = kda.fused_decode_step(x["q"][0], x["k"][0], x["v"][0], x["g"][0], x["beta"][0], state,
                              front["conv_cache"], front["conv_weight"],
                              norm_weight=front["norm_weight"])
    torch.cuda.synchronize()
    sel = lambda t: t[0][rows]
    o_ref, pool_ref, cache_ref = oracle.fused_decode_step(
        sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["g"]), sel(x["beta"]),
        front["conv_weight"], cache_ref, pool_ref, norm_weight=front["norm_weight"])
    assert rel_err(to64(o[rows]), o_ref) <= TOL[torch.bfloat16]
    assert rel_err(to64(state[rows]), pool_ref) <= 1e-4
    assert np.array_equal(to64(front["conv_cache"][rows]), cache_ref)
    del x, state, front
    torch.cuda.empty_cache()
