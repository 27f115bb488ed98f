"""GPU parity of the chunked prefill (kda_chunk_fwd) against the fp64 oracle.

The kernel evaluates the chunkwise form of the recurrence ("How Kimi K3
Engineered Its Way to the Frontier", section "FlashKDA steps the state once per
16 tokens"); the oracle is the token loop, so these tests also check that the
chunked schedule reproduces the loop.  Small cases are checked element by
element in full; full-size workloads on sampled (sequence, head) chains.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
from kda_testutil import TOL, announce, check_prefill_chains, rel_err, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_10_amd as m
    m.library()
    return m


def run(kda, inp, scale=1.0, varlen=True, **kw):
    return kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                         cu_seqlens=inp["cu_seqlens"] if varlen else None,
                         cu_seqlens_host=inp["cu_seqlens_host"] if varlen else None,
                         initial_state=inp["initial_state"],
                         num_seqs=len(inp["lengths"]), scale=scale, **kw)


def check_chains(inp, o, sf, chains, dtype, scale=1.0):
    check_prefill_chains(inp, o, sf, chains, dtype, scale=scale)


def test_fp32_forward_b1_t256_h2(kda):
    """The fp32 workload in full: B=1, T=256, H=2, chunk 64, zero initial state."""
    announce("chunk fp32 b1 t256 h2")
    cfg = ki.CONFIGS["kda_fwd_b1_t256_h2_f32"]
    inp = ki.make_prefill(cfg, device="cuda")
    o, sf = run(kda, inp, varlen=False)
    torch.cuda.synchronize()
    check_chains(inp, o, sf, [(0, 0), (0, 1)], torch.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_ragged_with_initial_state(kda, dtype):
    """Packed sequences ending inside chunks, an empty sequence, a one-token
    sequence, nonzero initial states, a non-unit output scale."""
    announce(f"chunk varlen ragged dtype={dtype}")
    lens = (1, 63, 64, 65, 130, 0, 300, 17)
    cfg = ki.PrefillConfig("t", lens, 3, dtype, init_std=0.3, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=7)
    o, sf = run(kda, inp, scale=0.7)
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(len(lens)) for h in range(3)]
    check_chains(inp, o, sf, chains, inp["dtype"], scale=0.7)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", ["beta0_g0", "scale0", "no_write"])
def test_prefill_degenerate_parameters(kda, dtype, case):
    """Degenerate values the recurrence allows ("How Kimi K3 Engineered Its Way
    to the Frontier", "How KDA updates its state"): beta = 0 on every third token
    (no write there) with g = 0 on 40 channels (no decay); scale = 0 (o is
    exactly 0, the state evolves as usual); beta = 0 and g = 0 everywhere (the
    state passes through unchanged and o_t = scale S0^T q_t)."""
    announce(f"chunk degenerate {case} dtype={dtype}")
    lens = (150, 77, 64)
    cfg = ki.PrefillConfig("t", lens, 2, dtype, init_std=0.3, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=91)
    scale = 0.8
    if case == "beta0_g0":
        inp["beta"][::3] = 0.0
        inp["g"][:, :, :40] = 0.0
    elif case == "scale0":
        scale = 0.0
    else:
        inp["beta"].zero_()
        inp["g"].zero_()
    o, sf = run(kda, inp, scale=scale)
    torch.cuda.synchronize()
    if case == "scale0":
        assert float(o.abs().max()) == 0.0
    if case == "no_write":
        assert rel_err(to64(sf), to64(inp["initial_state"])) <= 1e-6
    chains = [(n, h) for n in range(len(lens)) for h in range(2)]
    check_chains(inp, o, sf, chains, inp["dtype"], scale=scale)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_all_sequences_empty(kda, dtype):
    """A pack whose sequences are all empty: no output rows, and every final
    state is its initial state bit for bit (zero without one)."""
    announce(f"chunk all sequences empty dtype={dtype}")
    cfg = ki.PrefillConfig("t", (0, 0, 0), 2, dtype, init_std=0.3, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=5)
    o, sf = run(kda, inp)
    torch.cuda.synchronize()
    assert o.shape[0] == 0
    assert torch.equal(sf, inp["initial_state"])
    inp["initial_state"] = None
    o, sf = run(kda, inp)
    torch.cuda.synchronize()
    assert torch.equal(sf, torch.zeros_like(sf))


def test_fixed_batch_matches_varlen(kda):
    announce("chunk fixed batch vs varlen")
    cfg = ki.PrefillConfig("t", (200, 200, 200), 4, "bf16", init_std=0.1)
    inp = ki.make_prefill(cfg, device="cuda", seed=11)
    o1, s1 = run(kda, inp, varlen=False)
    o2, s2 = run(kda, inp, varlen=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    check_chains(inp, o1, s1, [(0, 0), (1, 3), (2, 1)], torch.bfloat16)


def test_bounded_gate_slow_decay_and_long_memory(kda):
    """Gates near zero (slow forgetting) keep the state alive across many chunks
    and exercise the recurrence rather than the decay; gates at the -5 floor
    exercise the reference-point scaling inside 16-token sub-tiles."""
    announce("chunk slow and floor decay")
    cfg = ki.PrefillConfig("t", (700, 333), 2, "bf16", init_std=0.2)
    inp = ki.make_prefill(cfg, device="cuda", seed=13)
    T = inp["g"].shape[0]
    g = inp["g"]
    g[: T // 2] *= 0.01                    # alpha ~ 0.99
    g[T // 2:] = -5.0                      # alpha = exp(-5), the page's floor
    o, sf = run(kda, inp)
    torch.cuda.synchronize()
    check_chains(inp, o, sf, [(0, 0), (0, 1), (1, 0), (1, 1)], torch.bfloat16)


def poisoned_run(kda, inp, poison, segments=0):
    """One prefill whose o, final state and workspace start filled with `poison`,
    so that any element no launch writes (or any read of unwritten workspace)
    shows up in the result."""
    N = len(inp["lengths"])
    T, H, D = inp["q"].shape
    o = torch.full_like(inp["q"], poison)
    sf = torch.full((N, H, D, D), poison, dtype=torch.float32, device=inp["q"].device)
    wsb = kda.chunk_fwd_workspace_size(inp["q"], num_seqs=N,
                                       cu_seqlens_host=inp["cu_seqlens_host"], segments=segments)
    ws = torch.full(((wsb + 3) // 4 + 1,), poison, dtype=torch.float32, device=inp["q"].device)
    kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                  cu_seqlens=inp["cu_seqlens"], cu_seqlens_host=inp["cu_seqlens_host"],
                  initial_state=inp["initial_state"], num_seqs=N, out=o, final_state=sf,
                  workspace=ws.view(torch.uint8), segments=segments)
    torch.cuda.synchronize()
    return o, sf


def where_different(name, a, b, cu=None):
    """'' when a and b are the same bits, else which (token, head) rows or
    (sequence, head) states differ and by how much."""
    a = a.float().cpu().numpy()
    b = b.float().cpu().numpy()
    d = a.view(np.uint32) != b.view(np.uint32)
    if not d.any():
        return ""
    idx = np.argwhere(d)
    if cu is not None:  # o: map tokens to (sequence, row in sequence)
        seq = np.searchsorted(np.asarray(cu), idx[:, 0], side="right") - 1
        where = sorted({(int(s), int(h)) for s, h in zip(seq, idx[:, 1])})
        rows = f"tokens {int(idx[:, 0].min())}..{int(idx[:, 0].max())}"
    else:
        where = sorted({(int(n), int(h)) for n, h in idx[:, :2]})
        rows = f"key rows {int(idx[:, 2].min())}..{int(idx[:, 2].max())}"
    return (f"{name}: {int(d.sum())} elements differ in (sequence, head) {where[:12]}, {rows}, "
            f"max |diff| {float(np.nanmax(np.abs(a[d] - b[d]))):.3e}")


@pytest.mark.parametrize("segments", [0, 1])
def test_deterministic(kda, segments):
    """The same inputs give the same bits, with the outputs and the workspace
    poisoned before each call (NaN, then a finite value): every output element
    is written and nothing unwritten is read.  segments = 0 takes the automatic
    three-segment split here (16 chains of up to 16 chunks); 1 runs whole chains."""
    announce(f"chunk determinism segments={segments}")
    cfg = ki.PrefillConfig("t", (1000, 37), 8, "bf16", init_std=0.1, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=3)
    cu = inp["cu_seqlens_host"]
    o1, s1 = poisoned_run(kda, inp, float("nan"), segments)
    assert torch.isfinite(o1).all(), "o has elements no launch wrote (or non-finite values)"
    assert torch.isfinite(s1).all(), "final state not fully written (or non-finite)"
    for poison in (float("nan"), 7.0, 0.0):
        o2, s2 = poisoned_run(kda, inp, poison, segments)
        msg = "; ".join(m for m in (where_different("o", o1, o2, cu),
                                     where_different("S_final", s1, s2)) if m)
        assert not msg, f"poison {poison}: {msg}"


def test_split_and_resume(kda):
    """Prefill [0, t) then [t, T) from the carried state equals one pass."""
    announce("chunk split/resume")
    cfg = ki.PrefillConfig("t", (500,), 2, "bf16", init_std=0.1)
    inp = ki.make_prefill(cfg, device="cuda", seed=5)
    o, sf = run(kda, inp, varlen=False)
    t = 200
    part = lambda d, a, b: {**d, "q": d["q"][a:b].contiguous(), "k": d["k"][a:b].contiguous(),
                            "v": d["v"][a:b].contiguous(), "g": d["g"][a:b].contiguous(),
                            "beta": d["beta"][a:b].contiguous(), "lengths": [b - a]}
    o1, s1 = run(kda, part(inp, 0, t), varlen=False)
    p2 = part(inp, t, 500)
    p2["initial_state"] = s1
    o2, s2 = run(kda, p2, varlen=False)
    torch.cuda.synchronize()
    assert rel_err(to64(torch.cat([o1, o2])), to64(o)) <= TOL[torch.bfloat16]
    assert rel_err(to64(s2), to64(sf)) <= TOL[torch.bfloat16]


def test_decode_steps_equal_prefill(kda):
    """T recurrent decode steps reproduce the prefill of the same T tokens."""
    announce("decode == prefill")
    H, T = 4, 90
    cfg = ki.PrefillConfig("t", (T,), H, "bf16", init_std=0.1)
    inp = ki.make_prefill(cfg, device="cuda", seed=21)
    o, sf = run(kda, inp, varlen=False)
    state = inp["initial_state"].clone()
    outs = []
    for t in range(T):
        sl = lambda x: x[t:t + 1].contiguous()
        outs.append(kda.recurrent_step(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]),
                                       sl(inp["beta"]), state))
    torch.cuda.synchronize()
    assert rel_err(to64(torch.cat(outs)), to64(o)) <= TOL[torch.bfloat16]
    assert rel_err(to64(state), to64(sf)) <= TOL[torch.bfloat16]


# ------------------------------------------------- intra-device segment parallelism
@pytest.mark.parametrize("dtype,segments", [("bf16", 2), ("bf16", 3), ("bf16", 5), ("f32", 3)])
def test_segments_match_oracle(kda, dtype, segments):
    """Sequences split into segments whose transitions are evaluated from a zero
    state, composed in order and re-run ("Kimi K3 -- Training and Infrastructure
    Notes", section 4.1) give the token loop's result.  The lengths include
    sequences shorter than the segment count (fewer, or a single segment), an
    empty one, and ragged ends."""
    announce(f"chunk segments={segments} dtype={dtype}")
    lens = (1, 63, 64, 65, 130, 0, 300, 17, 1000, 333)
    cfg = ki.PrefillConfig("t", lens, 3, dtype, init_std=0.3, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=31)
    o, sf = run(kda, inp, scale=0.9, segments=segments)
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(len(lens)) for h in range(3)]
    check_chains(inp, o, sf, chains, inp["dtype"], scale=0.9)


def test_automatic_split_matches_oracle(kda):
    """Automatic mode on a batch that leaves compute units idle splits every
    sequence of at least 8 chunks into three segments with shares 2:1:1; the
    outputs match the token loop and the unsplit run (short sequences, an empty
    one and ragged ends are mixed in)."""
    announce("chunk automatic split")
    lens = (1000, 17, 0, 513, 4100, 64)
    cfg = ki.PrefillConfig("t", lens, 2, "bf16", init_std=0.3, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=37)
    ws_auto = kda.chunk_fwd_workspace_size(inp["q"], num_seqs=len(lens),
                                           cu_seqlens_host=inp["cu_seqlens_host"], segments=0)
    ws_one = kda.chunk_fwd_workspace_size(inp["q"], num_seqs=len(lens),
                                          cu_seqlens_host=inp["cu_seqlens_host"], segments=1)
    assert ws_auto > ws_one  # the split's segment states are in the workspace
    o0, s0 = run(kda, inp, segments=0)
    o1, s1 = run(kda, inp, segments=1)
    torch.cuda.synchronize()
    chains = [(n, h) for n in range(len(lens)) for h in range(2)]
    check_chains(inp, o0, s0, chains, torch.bfloat16)
    assert rel_err(to64(o0), to64(o1)) <= TOL[torch.bfloat16]
    assert rel_err(to64(s0), to64(s1)) <= TOL[torch.bfloat16]


def test_segments_fixed_batch_without_initial_state(kda):
    announce("chunk segments fixed batch")
    cfg = ki.PrefillConfig("t", (777, 777), 4, "bf16")
    inp = ki.make_prefill(cfg, device="cuda", seed=33)
    o1, s1 = run(kda, inp, varlen=False, segments=4)
    o0, s0 = run(kda, inp, varlen=False, segments=1)
    torch.cuda.synchronize()
    check_chains(inp, o1, s1, [(0, 0), (1, 3)], torch.bfloat16)
    assert rel_err(to64(o1), to64(o0)) <= TOL[torch.bfloat16]
    assert rel_err(to64(s1), to64(s0)) <= TOL[torch.bfloat16]


def test_balanced_schedule_hands_states_over(kda):
    """A fixed-length batch with more chains than compute units (3 x 96 = 288
    chains of 16 chunks, the last one ragged) and a nonzero initial state: the
    automatic schedule cuts chains between workgroups, which hand the state over;
    against the oracle on cut chains and against whole chains (segments=1)."""
    announce("chunk balanced schedule b3 t1000 h96")
    cfg = ki.PrefillConfig("t", (1000, 1000, 1000), 96, "bf16", init_std=0.02)
    inp = ki.make_prefill(cfg, device="cuda", seed=71)
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the cut points below assume 256 compute units")
    assert kda.chunk_fwd_workspace_size(inp["q"], num_seqs=3, segments=0) > 0
    o0, s0 = run(kda, inp, varlen=False)
    o1, s1 = run(kda, inp, varlen=False, segments=1)
    torch.cuda.synchronize()
    # runs of 18 chunks: chain 1 cut at chunk 2, chain 112 = (1, 16) at chunk 8,
    # chain 286 = (2, 94) at chunk 14; chain 0 whole
    check_chains(inp, o0, s0, [(0, 0), (0, 1), (1, 16), (2, 94)], torch.bfloat16)
    assert rel_err(to64(o0), to64(o1)) <= TOL[torch.bfloat16]
    assert rel_err(to64(s0), to64(s1)) <= 1e-4


# ----------------------------------------------------------- full-size workloads
def test_full_b4_t8192_h96_sampled(kda):
    """B=4, T=8192, H=96, bf16, zero initial state -- the benchmark workload, in the
    launch configuration the benchmark times; six chains replayed by the oracle."""
    announce("chunk full b4 t8192 h96")
    cfg = ki.CONFIGS["kda_prefill_b4_t8192_h96_bf16"]
    inp = ki.make_prefill(cfg, device="cuda", seed=1002)
    o, sf = run(kda, inp, varlen=False)
    torch.cuda.synchronize()
    # 384 chains on 256 units run as 256 runs of 192 chunks; (0, 1) and (3, 1)
    # are cut at chunk 64 and handed over between two workgroups
    check_chains(inp, o, sf, [(0, 0), (0, 1), (1, 17), (2, 50), (3, 95), (0, 63), (3, 1)],
                 torch.bfloat16)


def test_full_t65536_h96_initial_state_sampled(kda):
    """One 65,536-token sequence, H=96, N(0, 0.02) initial state, gate clamped at -5."""
    announce("chunk full t65536 h96 s0")
    cfg = ki.CONFIGS["kda_prefill_t65536_h96_bf16_s0_gclamp5"]
    inp = ki.make_prefill(cfg, device="cuda", seed=1003)
    o, sf = run(kda, inp, varlen=False)
    torch.cuda.synchronize()
    check_chains(inp, o, sf, [(0, 0), (0, 47), (0, 95)], torch.bfloat16)


@pytest.mark.parametrize("segments", [0, 8])
def test_full_t65536_h96_segmented_sampled(kda, segments):
    """The 65,536-token workload with its chains split into segments (0 = the
    library's automatic choice), against the oracle on sampled heads."""
    announce(f"chunk full t65536 h96 s0 segments={segments}")
    cfg = ki.CONFIGS["kda_prefill_t65536_h96_bf16_s0_gclamp5"]
    inp = ki.make_prefill(cfg, device="cuda", seed=1003)
    o, sf = run(kda, inp, varlen=False, segments=segments)
    torch.cuda.synchronize()
    check_chains(inp, o, sf, [(0, 5), (0, 64)], torch.bfloat16)


def test_full_varlen32_t1m_h96_sampled(kda):
    """32 packed sequences (log-uniform 1K..256K tokens, 1,048,576 total), H=96."""
    announce("chunk full varlen32 t1m h96")
    cfg = ki.CONFIGS["kda_prefill_varlen32_t1m_h96_bf16"]
    inp = ki.make_prefill(cfg, device="cuda", seed=1004)
    o, sf = run(kda, inp)
    torch.cuda.synchronize()
    lens = inp["lengths"]
    longest = int(np.argmax(lens))
    shortest = int(np.argmin(lens))
    chains = [(longest, 3), (shortest, 95), (5, 40), (31, 0)]
    check_chains(inp, o, sf, chains, torch.bfloat16)
    del inp, o, sf
    torch.cuda.empty_cache()
