"""GPU parity of the chunked backward (kda_chunk_bwd) against the fp64 oracle.

The oracle is the reverse-mode token loop (pinned by central differences on the
CPU); the kernel works on 16-token sub-chunks ("How Kimi K3 Engineered Its Way to
the Frontier", sections "How KDA updates its state" and "FlashKDA steps the state
once per 16 tokens").  All gradients are fp32; the inputs are the bf16 or fp32
values the forward takes.
"""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testutil import announce, rel_err, to64

pytestmark = pytest.mark.gpu
NAMES = ("dq", "dk", "dv", "dg", "dbeta")
# Gradients are computed in fp32 from the exact input values (bf16 inputs are
# exact in fp32), so the fp32 bound applies to both input dtypes.
TOL_BWD = 1e-4


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_10_amd as m
    m.library()
    return m


def grads_gpu(kda, inp, dO, dSf, scale=1.0, varlen=True):
    return kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dO,
                         cu_seqlens=inp["cu_seqlens"] if varlen else None,
                         cu_seqlens_host=inp["cu_seqlens_host"] if varlen else None,
                         initial_state=inp["initial_state"], dfinal_state=dSf, scale=scale,
                         num_seqs=len(inp["lengths"]))


def compare(got, ref, tol=TOL_BWD, rows=None):
    worst = {}
    for n in NAMES + ("dinitial_state",):
        r = ref["dS0" if n == "dinitial_state" else n]
        gt = got[n]
        if gt is None:
            continue
        gt = to64(gt)
        if rows is not None and n != "dinitial_state":
            gt, r = gt[rows], r[rows]
        worst[n] = rel_err(gt, r)
    print("  max rel err: " + "  ".join(f"{k} {v:.2e}" for k, v in worst.items()), flush=True)
    for k, v in worst.items():
        assert v <= tol, (k, v)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_varlen_ragged_vs_oracle(kda, dtype):
    """Sequences ending inside sub-chunks, one of exactly 16 tokens, an empty one,
    nonzero initial states and final-state gradients, a non-unit scale."""
    announce(f"chunk bwd varlen dtype={dtype}")
    lens = (1, 15, 16, 17, 40, 0, 100, 77)
    H = 2
    cfg = ki.PrefillConfig("t", lens, H, dtype, init_std=0.3, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=71)
    gen = torch.Generator(device="cuda").manual_seed(72)
    T = inp["q"].shape[0]
    dO = torch.randn((T, H, 128), generator=gen, device="cuda").to(inp["q"].dtype)
    dSf = torch.randn((len(lens), H, 128, 128), generator=gen, device="cuda") * 0.1
    got = grads_gpu(kda, inp, dO, dSf, scale=0.8)
    torch.cuda.synchronize()
    ref = oracle.recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dO,
                               cu_seqlens=inp["cu_seqlens_host"],
                               initial_state=inp["initial_state"], dS_final=dSf, scale=0.8)
    compare(got, ref)


def test_backward_strong_decay_and_no_state(kda):
    """Half the tokens at the gate's floor g = -5 (every e^{G} factor far below
    1), no initial state and no final-state gradient (dS_final = 0)."""
    announce("chunk bwd strong decay")
    cfg = ki.PrefillConfig("t", (150, 64), 2, "bf16", varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=73)
    T = inp["g"].shape[0]
    inp["g"][: T // 2] = -5.0
    gen = torch.Generator(device="cuda").manual_seed(74)
    dO = torch.randn((T, 2, 128), generator=gen, device="cuda").to(torch.bfloat16)
    got = grads_gpu(kda, inp, dO, None)
    torch.cuda.synchronize()
    ref = oracle.recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dO,
                               cu_seqlens=inp["cu_seqlens_host"])
    compare(got, ref)


def test_backward_extreme_decay_exact_pairs(kda):
    """Stretches of g = -20 per token: inside such a sub-chunk the reference
    factors e^{+-(G - G_7)} would exceed e^60, so the prep and finalize passes
    take every token pair with its own exponential there (the matrix-core path
    elsewhere, in the same launch)."""
    announce("chunk bwd extreme decay")
    cfg = ki.PrefillConfig("t", (70, 41), 2, "f32", init_std=0.3, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=79)
    g = inp["g"]
    g[3:19] = -20.0          # the first sequence's first sub-chunk and into the second
    g[75:90, 1] = -20.0      # one head of the second sequence
    gen = torch.Generator(device="cuda").manual_seed(80)
    T = g.shape[0]
    dO = torch.randn((T, 2, 128), generator=gen, device="cuda")
    dSf = torch.randn((2, 2, 128, 128), generator=gen, device="cuda") * 0.1
    got = grads_gpu(kda, inp, dO, dSf, scale=0.9)
    torch.cuda.synchronize()
    ref = oracle.recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dO,
                               cu_seqlens=inp["cu_seqlens_host"],
                               initial_state=inp["initial_state"], dS_final=dSf, scale=0.9)
    compare(got, ref)


@pytest.mark.parametrize("case", ["beta0_g0", "scale0"])
def test_backward_degenerate_parameters(kda, case):
    """Degenerate values the method allows: beta = 0 on some tokens (no write,
    A = 0 there) with g = 0 on some channels (no decay), and scale = 0 (o = 0,
    so only the final-state gradient drives dq..dbeta)."""
    announce(f"chunk bwd degenerate {case}")
    cfg = ki.PrefillConfig("t", (45, 38), 2, "f32", init_std=0.3, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=84)
    gen = torch.Generator(device="cuda").manual_seed(85)
    T = inp["q"].shape[0]
    scale = 1.0
    if case == "beta0_g0":
        inp["beta"][::3] = 0.0
        inp["g"][:, :, :40] = 0.0
    else:
        scale = 0.0
    dO = torch.randn((T, 2, 128), generator=gen, device="cuda")
    dSf = torch.randn((2, 2, 128, 128), generator=gen, device="cuda") * 0.1
    got = grads_gpu(kda, inp, dO, dSf, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dO,
                               cu_seqlens=inp["cu_seqlens_host"],
                               initial_state=inp["initial_state"], dS_final=dSf, scale=scale)
    if case == "scale0":
        assert float(got["dq"].abs().max()) == 0.0  # q only reaches the loss through o
    compare(got, ref)


def test_backward_rejects_missized_outputs(kda):
    """Caller-supplied gradient buffers and workspace are checked on the host
    (the kernels only see pointers); nothing is launched."""
    cfg = ki.PrefillConfig("t", (32, 32), 2, "bf16")
    inp = ki.make_prefill(cfg, device="cuda", seed=83)
    dO = torch.zeros_like(inp["q"])
    T, H = inp["q"].shape[:2]
    bad = {"dq": torch.empty((T - 1, H, 128), device="cuda")}
    with pytest.raises(ValueError):
        kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dO, num_seqs=2,
                      grads=bad)
    with pytest.raises(TypeError):
        kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dO, num_seqs=2,
                      grads={"dbeta": torch.empty((T, H), device="cuda", dtype=torch.float64)})
    with pytest.raises(TypeError):
        kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dO, num_seqs=2,
                      workspace=torch.empty(16, device="cuda"))


def test_backward_small_workspace_runs_sequence_groups_bitwise(kda):
    """A workspace below the whole pack's is used for groups of sequences in
    turn: the same bits as one pass, down to the minimum (the largest single
    sequence's requirement); fixed batches group the same way."""
    announce("chunk bwd sequence groups")
    lens = (40, 200, 17, 0, 96, 150, 33)
    cfg = ki.PrefillConfig("t", lens, 2, "bf16", init_std=0.2, varlen=True)
    inp = ki.make_prefill(cfg, device="cuda", seed=86)
    gen = torch.Generator(device="cuda").manual_seed(87)
    T = inp["q"].shape[0]
    dO = torch.randn((T, 2, 128), generator=gen, device="cuda").to(torch.bfloat16)
    dSf = torch.randn((len(lens), 2, 128, 128), generator=gen, device="cuda") * 0.1
    kw = dict(cu_seqlens=inp["cu_seqlens"], cu_seqlens_host=inp["cu_seqlens_host"],
              initial_state=inp["initial_state"], dfinal_state=dSf, scale=0.9,
              num_seqs=len(lens))
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dO)
    whole = kda.chunk_bwd(*args, **kw)
    full = kda.chunk_bwd_workspace_size(inp["q"], cu_seqlens_host=inp["cu_seqlens_host"])
    least = kda.chunk_bwd_workspace_size(inp["q"], cu_seqlens_host=inp["cu_seqlens_host"],
                                         minimum=True)
    assert least < full
    for size in (least, (least + full) // 2):
        ws = torch.empty(size, dtype=torch.uint8, device="cuda")
        got = kda.chunk_bwd(*args, workspace=ws, **kw)
        torch.cuda.synchronize()
        for n in NAMES + ("dinitial_state",):
            assert torch.equal(got[n], whole[n]), (size, n)
    fb = ki.PrefillConfig("t", (80,) * 5, 2, "bf16")
    x = ki.make_prefill(fb, device="cuda", seed=88)
    dO2 = torch.randn(x["q"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    a2 = (x["q"], x["k"], x["v"], x["g"], x["beta"], dO2)
    one = kda.chunk_bwd(*a2, num_seqs=5)
    small = kda.chunk_bwd(*a2, num_seqs=5, max_workspace_bytes=1)  # one sequence per group
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(small[n], one[n]), n


def test_backward_fixed_batch_equals_varlen(kda):
    announce("chunk bwd fixed batch vs varlen")
    cfg = ki.PrefillConfig("t", (96, 96), 3, "bf16", init_std=0.1)
    inp = ki.make_prefill(cfg, device="cuda", seed=75)
    gen = torch.Generator(device="cuda").manual_seed(76)
    dO = torch.randn((192, 3, 128), generator=gen, device="cuda").to(torch.bfloat16)
    a = grads_gpu(kda, inp, dO, None, varlen=False)
    b = grads_gpu(kda, inp, dO, None, varlen=True)
    torch.cuda.synchronize()
    for n in NAMES + ("dinitial_state",):
        assert torch.equal(a[n], b[n]), n


def test_backward_full_b4_t8192_h96_whole_chains(kda):
    """The 4 x 8,192 x 96 bf16 workload's backward, in the launch the benchmark
    times; three whole chains (every token's gradients) against the oracle's
    reverse pass over the same 8,192 tokens."""
    announce("chunk bwd full b4 t8192 h96 whole chains")
    cfg = ki.CONFIGS["kda_prefill_b4_t8192_h96_bf16"]
    inp = ki.make_prefill(cfg, device="cuda", seed=1002)
    T, H = inp["q"].shape[0], inp["heads"]
    gen = torch.Generator(device="cuda").manual_seed(77)
    dO = torch.randn((T, H, 128), generator=gen, device="cuda").to(torch.bfloat16)
    got = grads_gpu(kda, inp, dO, None, varlen=False)
    torch.cuda.synchronize()
    chains = ((0, 0), (2, 41), (3, 95))
    # one oracle call over the three chains packed one after another
    pack = lambda t: torch.cat([t[n * 8192:(n + 1) * 8192, h:h + 1] for n, h in chains])
    cu = [0, 8192, 16384, 24576]
    ref = oracle.recurrent_bwd(pack(inp["q"]), pack(inp["k"]), pack(inp["v"]), pack(inp["g"]),
                               pack(inp["beta"]), pack(dO), cu_seqlens=cu)
    sub = {k: (pack(v) if v is not None and k != "dinitial_state" else None) for k, v in got.items()}
    compare(sub, ref)
    del inp, got, ref
    torch.cuda.empty_cache()


def test_backward_b1_t256_h2_f32_whole(kda):
    """The 256-token, 2-head fp32 workload, every gradient against the oracle."""
    announce("chunk bwd b1 t256 h2 f32")
    cfg = ki.CONFIGS["kda_fwd_b1_t256_h2_f32"]
    inp = ki.make_prefill(cfg, device="cuda", seed=1001)
    gen = torch.Generator(device="cuda").manual_seed(81)
    dO = torch.randn(inp["q"].shape, generator=gen, device="cuda")
    got = grads_gpu(kda, inp, dO, None, varlen=False)
    torch.cuda.synchronize()
    ref = oracle.recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dO,
                               initial_state=inp["initial_state"])
    compare(got, ref)


def test_backward_t65536_h96_last_and_middle_tokens(kda):
    """One 65,536-token sequence, 96 heads, bf16, nonzero initial state, decay
    floored at -5 (4,096 sub-chunks per chain in the serial passes).  The last 64
    tokens of two chains against the oracle run from the state the forward
    reaches at token 65,472; and a middle window, tokens 32,768 .. 32,831 of one
    chain, against the oracle run from the forward state at token 32,768 with
    the state gradient the oracle's reverse pass over tokens 32,832 .. 65,535
    brings back to token 32,832."""
    announce("chunk bwd t65536 h96 last and middle tokens")
    cfg = ki.CONFIGS["kda_prefill_t65536_h96_bf16_s0_gclamp5"]
    inp = ki.make_prefill(cfg, device="cuda", seed=1003)
    T, H = inp["q"].shape[0], inp["heads"]
    gen = torch.Generator(device="cuda").manual_seed(82)
    dO = torch.randn((T, H, 128), generator=gen, device="cuda").to(torch.bfloat16)
    got = grads_gpu(kda, inp, dO, None, varlen=False)
    torch.cuda.synchronize()
    tail = 64
    for h in (5, 90):
        sl = lambda t: t[: T - tail, h:h + 1]
        s0 = inp["initial_state"][:, h:h + 1]
        _, s_mid = oracle.recurrent(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]),
                                    sl(inp["beta"]), initial_state=s0)
        tl = lambda t: t[T - tail:, h:h + 1]
        ref = oracle.recurrent_bwd(tl(inp["q"]), tl(inp["k"]), tl(inp["v"]), tl(inp["g"]),
                                   tl(inp["beta"]), tl(dO), initial_state=s_mid)
        sub = {k: (v[T - tail:, h:h + 1] if v is not None and k != "dinitial_state" else None)
               for k, v in got.items()}
        compare(sub, ref)
    # middle window
    h, a, b = 5, 32768, 32832
    rng = lambda t, lo, hi: t[lo:hi, h:h + 1]
    args = lambda lo, hi: [rng(inp[n], lo, hi) for n in ("q", "k", "v", "g", "beta")]
    s0 = inp["initial_state"][:, h:h + 1]
    _, s_a = oracle.recurrent(*args(0, a), initial_state=s0)
    _, s_b = oracle.recurrent(*args(a, b), initial_state=s_a)
    back = oracle.recurrent_bwd(*args(b, T), rng(dO, b, T), initial_state=s_b)
    ref = oracle.recurrent_bwd(*args(a, b), rng(dO, a, b), initial_state=s_a,
                               dS_final=back["dS0"])
    sub = {k: (v[a:b, h:h + 1] if v is not None and k != "dinitial_state" else None)
           for k, v in got.items()}
    compare(sub, ref)
    del inp, got
    torch.cuda.empty_cache()
