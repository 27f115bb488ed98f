"""GPU parity of the gate and beta front end against the fp64 oracle.

With the lower-bounded gate selected, g holds raw gate logits and the kernels
apply K3's gate ("How Kimi K3 Engineered Its Way to the Frontier", section "How
KDA updates its state": g = lower_bound * sigmoid(exp(A_log) (x + dt_bias)));
with beta logits, beta passes through a sigmoid ("Kimi K3: a 2.8T open model
...", subsection "FlashKDA: the equation, shipped as a kernel").  The oracle
computes the gate and the sigmoid in fp64 from the same logits and then runs the
token loop.
"""
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testutil import TOL, announce, check_prefill_chains, rel_err, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_10_amd as m
    m.library()
    return m


def front(gp, lower_bound, gate=True, beta_logits=True):
    """How the oracle reads g and beta: logits through its gate and sigmoid."""
    return {"A_log": gp["A_log"] if gate else None, "dt_bias": gp.get("dt_bias"),
            "lower_bound": lower_bound, "beta_logits": beta_logits}


def run(kda, inp, gp, lower_bound=-5.0, gate=True, beta_logits=True, varlen=True, **kw):
    return kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                         cu_seqlens=inp["cu_seqlens"] if varlen else None,
                         cu_seqlens_host=inp["cu_seqlens_host"] if varlen else None,
                         initial_state=inp["initial_state"], num_seqs=len(inp["lengths"]),
                         A_log=gp["A_log"] if gate else None,
                         dt_bias=gp.get("dt_bias") if gate else None,
                         lower_bound=lower_bound, beta_logits=beta_logits, **kw)


def check(inp, fr, o, sf, chains, dtype, scale=1.0):
    check_prefill_chains(inp, o, sf, chains, dtype, scale=scale, front=fr)


# Gate parameter sets: "floor" puts many tokens near the bound (16-token windows),
# "gentle" keeps decays small (one reference per 64-token window).
GATE_PARAMS = {
    "floor": dict(a_log_mean=1.0, a_log_std=0.5, dt_mean=0.0, dt_std=1.0),
    "gentle": dict(a_log_mean=0.0, a_log_std=0.3, dt_mean=-4.0, dt_std=0.5),
    **ki.GATE_PARAM_SETS,
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("params", sorted(GATE_PARAMS))
def test_prefill_gate_and_beta_logits_vs_oracle(kda, dtype, params):
    """Ragged packed sequences (an empty one, one token, ends inside chunks),
    nonzero initial states, gate logits and beta logits."""
    announce(f"gate prefill params={params} dtype={dtype}")
    lens = (1, 63, 64, 65, 130, 0, 300, 17, 700)
    H = 3
    cfg = ki.PrefillConfig("t", lens, H, dtype, init_std=0.3, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=41, gate_logits=True, beta_logits=True)
    gp = ki.make_gate_params(H, device="cuda", seed=43, **GATE_PARAMS[params])
    o, sf = run(kda, inp, gp, scale=0.8)
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(len(lens)) for h in range(H)]
    check(inp, front(gp, -5.0), o, sf, chains, inp["dtype"], scale=0.8)


def test_prefill_gate_quarter_mode_boundaries(kda):
    """The "floor" parameters put most decays near the bound, so chunks take one
    reference per 16-token quarter (quarter mode: one window whose quarters the
    consumer waves take in four steps).  Sequences end at, just before and just
    after every quarter boundary, leaving quarters partly or wholly past the end."""
    announce("gate prefill quarter mode boundaries")
    lens = (1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 127, 128, 129, 200)
    H = 2
    cfg = ki.PrefillConfig("t", lens, H, "bf16", init_std=0.3, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=61, gate_logits=True, beta_logits=True)
    gp = ki.make_gate_params(H, device="cuda", seed=63, **GATE_PARAMS["floor"])
    o, sf = run(kda, inp, gp)
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(len(lens)) for h in range(H)]
    check(inp, front(gp, -5.0), o, sf, chains, inp["dtype"])


@pytest.mark.parametrize("lower_bound", [-2.5, 0.0])
def test_prefill_gate_other_bounds_without_bias(kda, lower_bound):
    """Other bounds in the accepted range, no dt_bias, beta given directly."""
    announce(f"gate prefill lower_bound={lower_bound}")
    lens = (200, 77)
    H = 2
    cfg = ki.PrefillConfig("t", lens, H, "bf16", init_std=0.2, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=47, gate_logits=True)
    gp = {"A_log": ki.make_gate_params(H, device="cuda", seed=49)["A_log"], "dt_bias": None}
    o, sf = run(kda, inp, gp, lower_bound=lower_bound, beta_logits=False)
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(len(lens)) for h in range(H)]
    check(inp, front(gp, lower_bound, beta_logits=False), o, sf, chains, torch.bfloat16)


def test_prefill_beta_logits_with_log_decay(kda):
    """Beta logits alone, with g given as the log-decay."""
    announce("gate prefill beta logits only")
    lens = (129, 64)
    cfg = ki.PrefillConfig("t", lens, 2, "bf16", init_std=0.1, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=51, beta_logits=True)
    o, sf = run(kda, inp, {}, gate=False)
    torch.cuda.synchronize()
    check(inp, front({}, -5.0, gate=False), o, sf, [(0, 0), (0, 1), (1, 0), (1, 1)],
          torch.bfloat16)


@pytest.mark.parametrize("dtype,segments", [("bf16", 3), ("f32", 2)])
def test_prefill_gate_with_segments(kda, dtype, segments):
    """The segment passes (transition trackers, composition, re-runs) read the
    gate logits the same way."""
    announce(f"gate prefill segments={segments} dtype={dtype}")
    lens = (1000, 65, 0, 333)
    H = 2
    cfg = ki.PrefillConfig("t", lens, H, dtype, init_std=0.3, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=53, gate_logits=True, beta_logits=True)
    gp = ki.make_gate_params(H, device="cuda", seed=55, **GATE_PARAMS["floor"])
    o, sf = run(kda, inp, gp, segments=segments)
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(len(lens)) for h in range(H)]
    check(inp, front(gp, -5.0), o, sf, chains, inp["dtype"])


def test_prefill_gate_matches_precomputed_log_decay(kda):
    """fp32 I/O: the fused gate and the plain kernel fed the oracle's gate and
    sigmoid (rounded to fp32) agree to 2e-5 -- the in-kernel gate is the
    oracle's up to fp32 rounding.  (With bf16 operands the two can differ by
    flipped bf16 roundings inside the chunk products, which the oracle parity
    tests bound instead.)"""
    announce("gate prefill fused vs precomputed")
    lens = (513, 64, 7)
    H = 2
    cfg = ki.PrefillConfig("t", lens, H, "f32", init_std=0.1, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=57, gate_logits=True, beta_logits=True)
    gp = ki.make_gate_params(H, device="cuda", seed=59)
    o1, s1 = run(kda, inp, gp)
    g64 = oracle.lowerbound_gate(inp["g"], gp["A_log"], gp["dt_bias"], -5.0)
    b64 = oracle.sigmoid(inp["beta"])
    plain = {**inp, "g": torch.from_numpy(g64).float().cuda(),
             "beta": torch.from_numpy(b64).float().cuda()}
    o2, s2 = run(kda, plain, gp, gate=False, beta_logits=False)
    torch.cuda.synchronize()
    assert rel_err(to64(o1), to64(o2)) <= 2e-5
    assert rel_err(to64(s1), to64(s2)) <= 2e-5


@pytest.mark.parametrize("params", sorted(ki.GATE_PARAM_SETS))
def test_full_b4_t8192_h96_gate_sampled(kda, params):
    """The B=4, T=8192, H=96 bf16 workload with gate and beta logits, in the
    launch configuration the benchmark's gate leg times; sampled chains."""
    announce(f"gate prefill full b4 t8192 h96 params={params}")
    cfg = ki.CONFIGS["kda_prefill_b4_t8192_h96_bf16"]
    inp = ki.make_prefill(cfg, device="cuda", seed=1002, gate_logits=True, beta_logits=True)
    gp = ki.make_gate_params(cfg.heads, device="cuda", seed=1009, **ki.GATE_PARAM_SETS[params])
    o, sf = run(kda, inp, gp, varlen=False)
    torch.cuda.synchronize()
    chains = [(0, 0), (1, 17), (2, 50), (3, 95)]
    check(inp, front(gp, -5.0), o, sf, chains, torch.bfloat16)


# ---------------------------------------------------------------- decode step
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_gate_and_beta_logits_vs_oracle(kda, dtype):
    announce(f"gate decode dtype={dtype}")
    dev = "cuda"
    B, H, slots, steps = 6, 3, 9, 4
    cfg = ki.DecodeConfig("t", B, H, steps, dtype="bf16" if dtype == torch.bfloat16 else "f32")
    x = ki.make_decode_ring(cfg, device=dev, ring=steps, gate_logits=True, beta_logits=True)
    gp = ki.make_gate_params(H, device=dev, seed=61, **GATE_PARAMS["floor"])
    pool = torch.randn((slots, H, 128, 128), device=dev, dtype=torch.float32) * 0.05
    idx = torch.tensor([4, 0, -1, 8, 2, 7], dtype=torch.int32, device=dev)
    ref_pool = to64(pool)
    gpu_pool = pool.clone()
    for t in range(steps):
        o = kda.recurrent_step(x["q"][t], x["k"][t], x["v"][t], x["g"][t], x["beta"][t],
                               gpu_pool, idx, scale=0.5, A_log=gp["A_log"],
                               dt_bias=gp["dt_bias"], lower_bound=-5.0, beta_logits=True)
        g_ref = oracle.lowerbound_gate(x["g"][t], gp["A_log"], gp["dt_bias"], -5.0)
        b_ref = oracle.sigmoid(x["beta"][t])
        o_ref, ref_pool = oracle.decode_step(x["q"][t], x["k"][t], x["v"][t], g_ref, b_ref,
                                             ref_pool, idx.cpu().numpy(), scale=0.5)
        torch.cuda.synchronize()
        live = [b for b in range(B) if idx[b] >= 0]
        assert rel_err(to64(o)[live], o_ref[live]) <= TOL[dtype]
    assert rel_err(to64(gpu_pool), ref_pool) <= 1e-4
    for s in (1, 3, 5, 6):
        assert torch.equal(gpu_pool[s], pool[s])


def test_decode_gate_without_bias_equals_prefill(kda):
    """T decode steps with gate logits reproduce the gated prefill of the same tokens."""
    announce("gate decode == gate prefill")
    H, T = 2, 70
    cfg = ki.PrefillConfig("t", (T,), H, "bf16", init_std=0.1)
    inp = ki.make_prefill(cfg, device="cuda", seed=63, gate_logits=True, beta_logits=True)
    gp = {"A_log": ki.make_gate_params(H, device="cuda", seed=65)["A_log"], "dt_bias": None}
    o, sf = run(kda, inp, gp, lower_bound=-4.0, varlen=False)
    state = inp["initial_state"].clone()
    outs = []
    for t in range(T):
        sl = lambda z: z[t:t + 1].contiguous()
        outs.append(kda.recurrent_step(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]),
                                       sl(inp["beta"]), state, A_log=gp["A_log"],
                                       lower_bound=-4.0, beta_logits=True))
    torch.cuda.synchronize()
    assert rel_err(to64(torch.cat(outs)), to64(o)) <= TOL[torch.bfloat16]
    assert rel_err(to64(state), to64(sf)) <= TOL[torch.bfloat16]
