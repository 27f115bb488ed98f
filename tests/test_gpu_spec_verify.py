"""GPU parity of the speculative-decode verification with replay
(kda_spec_verify_step) against the oracle.

"Kimi K3 -- Training and Infrastructure Notes", section 4.5 (KDA decoding): the
accepted draft tokens are replayed from their cached projected inputs, the state
of the verified tokens is written back, and the new draft window runs in the same
loop for its outputs.  The oracle composes its fused decode step in fp64.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testutil import TOL, announce, rel_err, to64

pytestmark = pytest.mark.gpu
NAMES = ("q", "k", "v", "g", "beta")


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_10_amd as m
    m.library()
    return m


def window(B, T, H, dtype, seed, dev="cuda", gate=False):
    """One draft window of raw projections, [B, T, H, ...]."""
    cfg = ki.DecodeConfig("t", B, H, T, dtype=dtype)
    x = ki.make_decode_ring(cfg, device=dev, ring=T, seed=seed, raw_qk=True,
                            gate_logits=gate, beta_logits=gate)
    return {n: x[n].transpose(0, 1).contiguous() for n in NAMES}


def verify_both(kda, new, replay, nrep, front, pool, pool_ref, cache_ref, idx=None, gate=None,
                **kw):
    gkw = {}
    if gate is not None:
        gkw = dict(A_log=gate["A_log"], dt_bias=gate["dt_bias"], lower_bound=gate["lower_bound"],
                   beta_logits=gate["beta_logits"])
    o = kda.spec_verify_step(*(new[n] for n in NAMES), pool, front["conv_cache"],
                             front["conv_weight"], replay=replay, num_replay=nrep,
                             state_indices=idx, **kw, **gkw)
    nr = np.zeros(new["q"].shape[0]) if replay is None else (
        nrep.cpu().numpy() if nrep is not None else np.full(new["q"].shape[0], replay["q"].shape[1]))
    o_ref, pool_ref, cache_ref = oracle.spec_verify_step(
        new, replay, nr, front["conv_weight"], cache_ref, pool_ref,
        None if idx is None else idx.cpu().numpy(), gate=gate, **kw)
    return o, o_ref, pool_ref, cache_ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_three_rounds_with_accepted_counts(kda, dtype):
    """Three verification rounds of a 4-token window; per-row accepted counts 0
    to 4 (a row whose count is above the window is clamped); a skipped row and
    scattered slots; outputs, states and caches against the oracle each round."""
    announce(f"spec verify rounds dtype={dtype}")
    dev = "cuda"
    B, T, H, slots = 5, 4, 2, 8
    tol = TOL[torch.bfloat16 if dtype == "bf16" else torch.float32]
    front = ki.make_conv_front(slots, H, dtype, device=dev)
    pool = torch.randn((slots, H, 128, 128), device=dev, dtype=torch.float32) * 0.05
    idx = torch.tensor([6, 1, -1, 3, 0], dtype=torch.int32, device=dev)
    pool0, cache0 = pool.clone(), front["conv_cache"].clone()
    pool_ref, cache_ref = to64(pool), to64(front["conv_cache"])
    live = [b for b in range(B) if idx[b] >= 0]
    replay, nrep = None, None
    counts = [[0, 4, 9, 2, 1], [3, 0, 1, 4, 2], [1, 1, 1, 1, 1]]
    for rnd in range(3):
        new = window(B, T, H, dtype, seed=200 + rnd)
        o, o_ref, pool_ref, cache_ref = verify_both(kda, new, replay, nrep, front, pool,
                                                    pool_ref, cache_ref, idx=idx,
                                                    norm_weight=front["norm_weight"], scale=0.8)
        torch.cuda.synchronize()
        err = rel_err(to64(o)[live], o_ref[live])
        print(f"  round {rnd}: o rel err {err:.3e}", flush=True)
        assert err <= tol
        assert rel_err(to64(pool), pool_ref) <= 1e-4
        assert np.array_equal(to64(front["conv_cache"]), cache_ref)
        replay = new
        nrep = torch.tensor(counts[rnd], dtype=torch.int32, device=dev)
    for s in (2, 4, 5, 7):  # slots no row names stay untouched
        assert torch.equal(pool[s], pool0[s])
        assert torch.equal(front["conv_cache"][s], cache0[s])


def test_gate_logits_and_replay_only(kda):
    """Gate and beta logits; then a call with an empty new window that only
    commits the accepted tokens."""
    announce("spec verify gate, replay only")
    dev = "cuda"
    B, T, H = 3, 3, 2
    front = ki.make_conv_front(B, H, "bf16", device=dev, seed=1017)
    gp = ki.make_gate_params(H, device=dev, seed=1019, **ki.GATE_PARAM_SETS["heavy"])
    gate = {"A_log": gp["A_log"], "dt_bias": gp["dt_bias"], "lower_bound": -5.0,
            "beta_logits": True}
    pool = torch.randn((B, H, 128, 128), device=dev, dtype=torch.float32) * 0.05
    pool_ref, cache_ref = to64(pool), to64(front["conv_cache"])
    w1 = window(B, T, H, "bf16", seed=300, gate=True)
    o, o_ref, pool_ref, cache_ref = verify_both(kda, w1, None, None, front, pool, pool_ref,
                                                cache_ref, gate=gate)
    torch.cuda.synchronize()
    assert rel_err(to64(o), o_ref) <= TOL[torch.bfloat16]
    empty = {n: w1[n][:, :0].contiguous() for n in NAMES}
    nrep = torch.tensor([3, 0, 2], dtype=torch.int32, device=dev)
    o2, o2_ref, pool_ref, cache_ref = verify_both(kda, empty, w1, nrep, front, pool, pool_ref,
                                                  cache_ref, gate=gate)
    torch.cuda.synchronize()
    assert o2.numel() == 0
    assert rel_err(to64(pool), pool_ref) <= 1e-4
    assert np.array_equal(to64(front["conv_cache"]), cache_ref)


def test_full_b512_h96_window4_sampled(kda):
    """512 rows x 96 heads, bf16, a 4-token window and per-row accepted counts of
    the previous window 0..4; three rows (all heads) replayed by the oracle."""
    announce("spec verify full b512 h96 window 4")
    dev = "cuda"
    cfg = ki.DECODE_CONFIGS["kda_decode_b512_h96_bf16_f32state"]
    B, H, T = cfg.batch, cfg.heads, 4
    state = ki.make_decode_ring(cfg, device=dev, ring=1)["state"]
    front = ki.make_conv_front(B, H, "bf16", device=dev)
    prev, new = window(B, T, H, "bf16", seed=400), window(B, T, H, "bf16", seed=401)
    nrep = torch.randint(0, T + 1, (B,), generator=torch.Generator().manual_seed(5),
                         dtype=torch.int32).to(dev)
    rows = [0, 300, 511]
    pool_ref, cache_ref = to64(state[rows]), to64(front["conv_cache"][rows])
    o = kda.spec_verify_step(*(new[n] for n in NAMES), state, front["conv_cache"],
                             front["conv_weight"], replay=prev, num_replay=nrep,
                             norm_weight=front["norm_weight"])
    torch.cuda.synchronize()
    sel = lambda d: {n: d[n][rows] for n in NAMES}
    o_ref, pool_ref, cache_ref = oracle.spec_verify_step(
        sel(new), sel(prev), nrep.cpu().numpy()[rows], front["conv_weight"], cache_ref, pool_ref,
        norm_weight=front["norm_weight"])
    assert rel_err(to64(o[rows]), o_ref) <= TOL[torch.bfloat16]
    assert rel_err(to64(state[rows]), pool_ref) <= 1e-4
    assert np.array_equal(to64(front["conv_cache"][rows]), cache_ref)
    del state, front, prev, new
    torch.cuda.empty_cache()
