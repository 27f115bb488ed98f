"""Benchmark of the KDA hot path on one MI355X.

A step is one chunked prefill forward (chunk 64, fp32 state, outputs + final
states) of the largest workload that fits one GPU: the varlen pack of 32
sequences, lengths log-uniform in [1K, 256K] summing to 1,048,576 tokens, 96
heads, bf16 -- inputs resident in HBM before the timed region.  The 4 x 8,192 x
96 batch and the single 65,536-token sequence (nonzero initial state, decay
floor -5) are timed after it and reported as extra prefill lines; the recurrent
decode workload (512 sequences x 96 heads, fp32 states in HBM, 1000 in-place
steps) last, in the same JSON line, after a kda_state_io line (a gather of
512 fp32 states of 96 heads from a 1,024-slot pool in random order).

With --front gate the prefill reads raw gate logits (fp32, in place of g), per-head
A_log and per-channel dt_bias, and beta logits, and applies K3's lower-bounded gate
and the beta sigmoid in the kernel ("How Kimi K3 Engineered Its Way to the
Frontier", section "How KDA updates its state"); the byte count is the same.

Algorithmic accounting (fixed; it does not depend on the implementation):
  prefill FLOP per token-head = 6 d^2 + C (3 d + 2 d) = 139,264   (d = 128, C = 64)
  prefill bytes per token-head = q, k, v, o in bf16 (4 x 256) + g fp32 (512) + beta (4)
                                 = 1,540, plus 64 KiB per (sequence, head) final state
  decode bytes per (row, head) per step = 2 x 65,536 (state read + write)
                                 + 3 x 256 (q, k, v) + 512 (g) + 4 (beta) + 256 (o) = 132,612
                                 (+ 4,608 for the fused step's three bf16 conv caches,
                                 read and rewritten; per-head weights are not counted)
  state_io bytes per gathered (state, head) = 2 x 65,536 (read + write)
Roofline peaks: HBM 8.0 TB/s; bf16 dense matrix 2.5 PFLOP/s (2,516.6 TFLOP/s).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s + % MFMA peak; decode step GB/s + % HBM peak"
PREFILL_WORKLOAD = "kda_prefill_varlen32_t1m_h96_bf16"
EXTRA_WORKLOADS = "kda_prefill_b4_t8192_h96_bf16,kda_prefill_t65536_h96_bf16_s0_gclamp5"
DECODE_WORKLOAD = "kda_decode_b512_h96_bf16_f32state"
D, C = 128, 64
FLOP_PER_TOKEN_HEAD = 6 * D * D + C * (3 * D + 2 * D)          # 139,264
BYTES_PER_TOKEN_HEAD = 4 * 2 * D + 4 * D + 4                   # 1,540
STATE_BYTES = D * D * 4                                        # 65,536
DECODE_BYTES_PER_HEAD = 2 * STATE_BYTES + 3 * 2 * D + 4 * D + 4 + 2 * D   # 132,612
CONV_CACHE_BYTES_PER_HEAD = 2 * 3 * 3 * D * 2                              # 4,608 (read + write)
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-state-io", action="store_true",
                    help="skip the kda_state_io gather line (512 x 96 fp32 states)")
    ap.add_argument("--decode-kernel", choices=("step", "fused", "spec"), default="step",
                    help="decode leg: the plain step (default), the fused step with the "
                         "short-convolution front end and the output RMSNorm, or the "
                         "speculative-decode verification (replay of a --spec-window-token "
                         "window, all accepted, plus a new window of as many tokens)")
    ap.add_argument("--spec-window", type=int, default=4)
    ap.add_argument("--bwd", action="store_true",
                    help="also time the chunked backward on the prefill workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle sample until this much wall time has passed")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, copy a state pool of this many MiB once (the plain "
                         "copy kernel whose hardware byte counters scale the prefill's)")
    ap.add_argument("--workload", default=PREFILL_WORKLOAD)
    ap.add_argument("--extra", default=EXTRA_WORKLOADS,
                    help="comma-separated further prefill workloads, timed after the headline "
                         "one and reported under prefill_workloads ('' for none)")
    ap.add_argument("--segments", type=int, default=0,
                    help="segments per sequence (0 = the library's automatic choice)")
    ap.add_argument("--gate-params", choices=("matched", "heavy"), default="matched",
                    help="gate parameter set for --front gate (see kda_inputs.GATE_PARAM_SETS)")
    ap.add_argument("--front", choices=("logdecay", "gate"), default="logdecay",
                    help="prefill inputs: log-decay g and beta (default), or gate logits "
                         "with A_log, dt_bias and beta logits (the lower-bounded gate and "
                         "the beta sigmoid computed in the kernel)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic record from rocprofv3 --pmc FETCH_SIZE and "
                         "WRITE_SIZE counter_collection.csv files (taken with "
                         "--copy-calibration-mib) and exit; needs no GPU")
    return ap.parse_args()


def prefill_summary(pre, steps):
    """Throughput of a timed prefill against the fixed accounting (per token-head
    139,264 FLOP and 1,540 B, plus 64 KiB per chain for the final state and,
    when given, the initial state)."""
    H, tokens, N, ms = pre["heads"], pre["tokens"], pre["seqs"], pre["ms"]
    tok_s = tokens / (ms * 1e-3)
    tflops = tok_s * H * FLOP_PER_TOKEN_HEAD / 1e12
    alg = tokens * H * BYTES_PER_TOKEN_HEAD + N * H * STATE_BYTES * (
        2 if pre["x"]["initial_state"] is not None else 1)
    gbs = alg / (ms * 1e-3) / 1e9
    return {"ms_per_step": ms, "steps": steps, "sequences": N, "tokens": tokens, "heads": H,
            "tokens_per_s": tok_s, "tflops": tflops, "mfma_peak_frac": tflops / BF16_PEAK_TFLOPS,
            "gb_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": alg}


def time_prefill(kda, ki, workload, steps, warmup, segments=0, front="logdecay",
                 gate_params="matched"):
    import torch
    cfg = ki.CONFIGS[workload]
    gate = front == "gate"
    x = ki.make_prefill(cfg, device="cuda", seed=1002, gate_logits=gate, beta_logits=gate)
    gp = (ki.make_gate_params(x["heads"], device="cuda", seed=1009,
                              **ki.GATE_PARAM_SETS[gate_params]) if gate else {})
    fkw = dict(A_log=gp.get("A_log"), dt_bias=gp.get("dt_bias"), lower_bound=-5.0,
               beta_logits=gate)
    N, H = len(x["lengths"]), x["heads"]
    varlen = cfg.varlen
    o = torch.empty_like(x["q"])
    sf = torch.empty((N, H, D, D), dtype=torch.float32, device="cuda")
    ws_bytes = kda.chunk_fwd_workspace_size(
        x["q"], num_seqs=N, cu_seqlens_host=x["cu_seqlens_host"] if varlen else None,
        segments=segments)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"],
                      cu_seqlens=x["cu_seqlens"] if varlen else None,
                      cu_seqlens_host=x["cu_seqlens_host"] if varlen else None,
                      initial_state=x["initial_state"], num_seqs=N, out=o, final_state=sf,
                      workspace=ws, segments=segments, **fkw)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    tokens = x["q"].shape[0]
    res = dict(ms=ms, wall_s=wall, tokens=tokens, heads=H, seqs=N, x=x, cfg=cfg,
               gate_params=gp if gate else None)
    return res


PREFILL_BWD_WORKLOAD = "kda_prefill_b4_t8192_h96_bf16"  # the backward's timed workload
BWD_BYTES_PER_TOKEN_HEAD = 4 * 2 * D + 4 * D + 4 + 4 * 4 * D + 4     # 3,592
# Matrix-core work of the backward per 16-token sub-chunk of one head (all 128
# value columns, d = 128), product by product as the passes compute them; the
# products run on fp32 matrix cores for both I/O dtypes.
BWD_FLOPS_PER_SUBCHUNK_HEAD = (
    (2 * 16 * D * D + 2 * 16 * 16 * D + 2 * D * 16 * D)            # states: KS, U, S update
    + (2 * 16 * D * D * 2 + 2 * 16 * 16 * D * 5                    # serial: KS, Kb dS; U, P^T dO, dW, dA, dP
       + 2 * 16 * D * D * 3 + 2 * 2 * D * 16 * D)                  #   dKt, dQt, dKb; dS update
    + 2 * 2 * 16 * 16 * D                                          # prep: Ab, P
    + 4 * 2 * 16 * 16 * D)                                         # finalize: pair terms
BWD_FLOPS_PER_TOKEN_HEAD = BWD_FLOPS_PER_SUBCHUNK_HEAD // 16       # 344,064
FP32_MFMA_PEAK_TFLOPS = 157.3


def time_backward(kda, ki, workload, steps, warmup, cpu_seconds=0.0):
    """The chunked backward on the prefill workload: gradients of <dO, o> with
    dO ~ N(0, 1) in the I/O dtype; grads and workspace allocated once.  With
    cpu_seconds > 0 the oracle's backward is timed beside it (cpu_baseline_bwd)."""
    import torch
    cfg = ki.CONFIGS[workload]
    x = ki.make_prefill(cfg, device="cuda", seed=1002)
    T, H = x["q"].shape[0], x["heads"]
    N = len(x["lengths"])
    gen = torch.Generator(device="cuda").manual_seed(1007)
    dO = torch.randn((T, H, D), generator=gen, device="cuda").to(x["q"].dtype)
    varlen = cfg.varlen
    grads = kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO,
                          cu_seqlens=x["cu_seqlens"] if varlen else None,
                          cu_seqlens_host=x["cu_seqlens_host"] if varlen else None,
                          initial_state=x["initial_state"], num_seqs=N)
    ws = [None]

    def step():
        kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO,
                      cu_seqlens=x["cu_seqlens"] if varlen else None,
                      cu_seqlens_host=x["cu_seqlens_host"] if varlen else None,
                      initial_state=x["initial_state"], num_seqs=N, grads=grads,
                      workspace=ws[0])

    # one workspace for every step
    ws_bytes = kda.chunk_bwd_workspace_size(
        x["q"], num_seqs=N, cu_seqlens_host=x["cu_seqlens_host"] if varlen else None)
    ws[0] = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    alg = T * H * BWD_BYTES_PER_TOKEN_HEAD
    flops = T * H * BWD_FLOPS_PER_TOKEN_HEAD
    cpu = cpu_baseline_bwd(x, dO, cpu_seconds) if cpu_seconds > 0 else None
    del x, grads, ws, dO
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "steps": steps, "tokens_per_s": T / (ms * 1e-3),
            "algorithmic_bytes": alg, "gb_per_s": alg / (ms * 1e-3) / 1e9,
            "hbm_frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "flops": flops, "tflops": flops / (ms * 1e-3) / 1e12,
            "mfma_fp32_frac": flops / (ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS,
            "workload": workload,
            "kernels": ["bwd_prep_kernel", "bwd_states_kernel", "bwd_serial_kernel",
                        "bwd_finalize_kernel"],
            "cpu_baseline": cpu}


BWD_CPU_TOKENS = 1024  # tokens per chain in the oracle's backward sample


def cpu_baseline_bwd(x, dO, seconds):
    """Time the oracle's backward (the fp64 token loop in reverse mode, as it
    stands: single-threaded, every state kept) on a bounded sample: one
    (sequence, head) chain per host thread, its first BWD_CPU_TOKENS tokens,
    the chains run concurrently from Python threads (the C call releases the
    interpreter lock), repeated until `seconds` of wall time have passed."""
    import concurrent.futures as cf
    import numpy as np
    import oracle
    oracle.load()
    cores = min(len(os.sched_getaffinity(0)), oracle.max_threads())
    cu = x["cu_seqlens_host"]
    N, H = len(cu) - 1, x["heads"]
    to = lambda t: t.detach().cpu().double().numpy()
    samples = []
    for i in range(cores):
        n, h = i % N, (i * 7) % H
        a = cu[n]
        b = min(cu[n + 1], a + BWD_CPU_TOKENS)
        sl = lambda t: to(t[a:b, h:h + 1])
        samples.append((sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]),
                        sl(dO)))
    run = lambda smp: oracle.recurrent_bwd(*smp)
    passes, t0 = 0, time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        while True:
            list(ex.map(run, samples))
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= seconds:
                break
    token_heads = sum(smp[0].shape[0] for smp in samples) * passes
    return {"value": token_heads / H / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{cores} (sequence, head) chains, the first {BWD_CPU_TOKENS} tokens of "
                      f"each, oracle backward (fp64 reverse-mode token loop), one chain per "
                      f"thread, run {passes} times; value = token-heads/s divided by {H} heads",
            "token_heads_per_s": token_heads / dt, "seconds": dt}


def time_decode(kda, ki, steps, warmup=10, kernel="step", window=4):
    import torch
    cfg = ki.DECODE_CONFIGS[DECODE_WORKLOAD]
    fused = kernel != "step"
    x = ki.make_decode_ring(cfg, device="cuda", raw_qk=fused)
    state = x["state"]
    o = torch.empty_like(x["q"][0])
    front = ki.make_conv_front(cfg.batch, cfg.heads, cfg.dtype, device="cuda") if fused else None
    if kernel == "spec":  # windows of `window` tokens: [B, T, H, ...], two alternating
        wins = []
        for w in range(2):
            xw = ki.make_decode_ring(cfg, device="cuda", ring=window, seed=2000 + w, raw_qk=True)
            wins.append({n: xw[n].transpose(0, 1).contiguous()
                         for n in ("q", "k", "v", "g", "beta")})
            del xw
        o = torch.empty_like(wins[0]["q"])

    def step(t):
        r = t % cfg.ring
        if kernel == "spec":
            new, prev = wins[t % 2], wins[(t + 1) % 2]
            kda.spec_verify_step(new["q"], new["k"], new["v"], new["g"], new["beta"], state,
                                 front["conv_cache"], front["conv_weight"], replay=prev,
                                 norm_weight=front["norm_weight"], out=o)
        elif fused:
            kda.fused_decode_step(x["q"][r], x["k"][r], x["v"][r], x["g"][r], x["beta"][r], state,
                                  front["conv_cache"], front["conv_weight"],
                                  norm_weight=front["norm_weight"], out=o)
        else:
            kda.recurrent_step(x["q"][r], x["k"][r], x["v"][r], x["g"][r], x["beta"][r], state,
                               out=o)

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for t in range(steps):
        step(warmup + t)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    heads = cfg.batch * cfg.heads
    per_head = DECODE_BYTES_PER_HEAD + (CONV_CACHE_BYTES_PER_HEAD if fused else 0)
    extra = {}
    if kernel == "spec":  # replayed and new tokens' inputs, new tokens' outputs
        tok_in = 3 * 2 * D + 4 * D + 4
        per_head = 2 * STATE_BYTES + CONV_CACHE_BYTES_PER_HEAD + 2 * window * tok_in + \
            window * 2 * D
        extra = {"window": window, "replayed": window,
                 "tokens_verified_per_s": cfg.batch * window / (ms * 1e-3)}
    gbs = heads * per_head / (ms * 1e-3) / 1e9
    del x, state, front
    torch.cuda.empty_cache()
    return dict(ms_per_step=ms, steps=steps, gb_per_s=gbs, hbm_frac=gbs / HBM_PEAK_GBS,
                bytes_per_step=heads * per_head, batch=cfg.batch, heads=cfg.heads,
                kernel="decode_loop_kernel", entry={"step": "kda_recurrent_step",
                "fused": "kda_fused_decode_step", "spec": "kda_spec_verify_step"}[kernel],
                **extra)


def time_state_io(kda, steps=20, warmup=3, states=512, heads=96):
    """kda_state_io gathering `states` fp32 states of `heads` heads (a prefix-cache
    restore: snapshots copied into request slots) from a pool of twice as many
    slots, in a seeded random order; algorithmic bytes = the states read + written."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(3001)
    pool = torch.randn((2 * states, heads, D, D), generator=gen, device="cuda")
    dst = torch.empty((states, heads, D, D), device="cuda")
    idx = torch.randperm(2 * states, generator=gen, device="cuda")[:states].to(torch.int32)
    for _ in range(warmup):
        kda.state_io(kda.STATE_GATHER, dst, pool, idx)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        kda.state_io(kda.STATE_GATHER, dst, pool, idx)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    nbytes = 2 * states * heads * STATE_BYTES
    del pool, dst, idx
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return dict(op="gather", states=states, heads=heads, dtype="f32", ms_per_call=ms, calls=steps,
                bytes_per_call=nbytes, gb_per_s=gbs, hbm_frac=gbs / HBM_PEAK_GBS,
                kernel="state_io_kernel", entry="kda_state_io")


def baseline_chains(x):
    """The (sequence, head) chains the oracle baseline times: heads 0, 31, 63 and
    95 (spread over the 96) of every sequence, up to 32 sequences."""
    N, H = len(x["lengths"]), x["heads"]
    heads = sorted({i * (H - 1) // 3 for i in range(4)}) if H >= 4 else list(range(H))
    return [(n, h) for h in heads for n in range(min(N, 32))]


def cpu_baseline(x, seconds, gp=None):
    """Time the fp64 oracle (as it stands: OpenMP over chains) on a bounded
    sample of the same workload: the chains of baseline_chains, whole, run
    repeatedly until `seconds` of wall time have passed (at least once); the rate
    is the mean.  With gate parameters `gp` the oracle's gate and beta sigmoid run
    inside the timed loop too."""
    import numpy as np
    import oracle
    chains = baseline_chains(x)
    cu = x["cu_seqlens_host"]
    H = x["heads"]
    to = lambda t: t.detach().cpu().double().numpy()
    qs, ks, vs, gs, bs, lens = [], [], [], [], [], []
    for n, h in chains:
        a, b = cu[n], cu[n + 1]
        qs.append(to(x["q"][a:b, h])); ks.append(to(x["k"][a:b, h])); vs.append(to(x["v"][a:b, h]))
        gs.append(to(x["g"][a:b, h])); bs.append(to(x["beta"][a:b, h])); lens.append(b - a)
    cu2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    cat = lambda xs: np.concatenate(xs, axis=0)[:, None]
    args = (cat(qs), cat(ks), cat(vs), cat(gs), np.concatenate(bs)[:, None])
    del qs, ks, vs, gs, bs
    if gp is not None:
        A_np, dt_np = to(gp["A_log"]), to(gp["dt_bias"])
    oracle.load()
    cores = len(os.sched_getaffinity(0))
    threads = min(cores, oracle.max_threads(), len(chains))
    passes, t0 = 0, time.perf_counter()
    while True:
        if gp is not None:  # per token: the gate of its chain's head, then the loop
            g = np.empty_like(args[3])
            for i, (n, h) in enumerate(chains):
                g[cu2[i]:cu2[i + 1]] = oracle.lowerbound_gate(
                    args[3][cu2[i]:cu2[i + 1]], A_np[h:h + 1], dt_np[h:h + 1], -5.0)
            run = (*args[:3], g, oracle.sigmoid(args[4]))
        else:
            run = args
        oracle.recurrent(*run, cu_seqlens=cu2, nthreads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    token_heads = int(cu2[-1]) * passes
    heads = sorted({h for _, h in chains})
    nseq = len({n for n, _ in chains})
    return {"value": token_heads / H / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"heads {heads} of {nseq} sequences of the same workload: {len(chains)} "
                      f"(sequence, head) chains, {int(cu2[-1])} token-heads (fp64 token loop, "
                      f"OpenMP over chains on {threads} threads), run {passes} times; value = "
                      f"token-heads/s divided by {H} heads",
            "token_heads_per_s": token_heads / dt, "seconds": dt}


PREFILL_KERNEL = "chunk_fwd_pipe_kernel"
PREFILL_SOURCES = ["gated_delta_rule_10_amd/csrc/kda_chunk_pipe.hip",
                   "gated_delta_rule_10_amd/csrc/kda_chunk_common.h",
                   "gated_delta_rule_10_amd/csrc/kda_device.h",
                   "gated_delta_rule_10_amd/csrc/kda_pipe_layout.h"]
TRAFFIC_NAMES = {
    "kda_prefill_varlen32_t1m_h96_bf16": "chunk_fwd_bf16_varlen32_t1m_h96",
    "kda_prefill_b4_t8192_h96_bf16": "chunk_fwd_bf16_b4_t8192_h96",
    "kda_prefill_t65536_h96_bf16_s0_gclamp5": "chunk_fwd_bf16_t65536_h96",
}


def traffic_record_path(workload, front="logdecay"):
    name = TRAFFIC_NAMES.get(workload, workload)
    if front == "gate":
        name = name.replace("chunk_fwd_", "chunk_fwd_gate_")
    return os.path.join(ROOT, "profiles", name + "_traffic.json")


def sources_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def measured_traffic(workload, front="logdecay"):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE readings,
    or None when they were taken on other kernel sources or another workload."""
    path = traffic_record_path(workload, front)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if sources_digest(rec["sources"]) != rec["source_sha256"] or rec["workload"] != workload:
        return None
    return rec["traffic_bytes"]


def copy_bytes_for(mib, heads=96):
    """Bytes the calibration copy moves each way for a pool of `mib` MiB."""
    return max(1, (mib << 20) // (heads * D * D * 4)) * heads * D * D * 4


def record_traffic(fetch_csv, write_csv, workload, mib, front="logdecay"):
    """Scale the prefill kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by
    what the same counters read for the state-pool copy of known size, and store
    the result with a digest of the kernel's sources."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("prefill" if PREFILL_KERNEL in name else
                   "copy" if "state_io_kernel" in name else None)
            if key:
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
        return vals

    f, w = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = copy_bytes_for(mib)
    fscale = copy_bytes / 1024 / (sum(f["copy"]) / len(f["copy"]))
    wscale = copy_bytes / 1024 / (sum(w["copy"]) / len(w["copy"]))
    fk = sum(f["prefill"]) / len(f["prefill"])
    wk = sum(w["prefill"]) / len(w["prefill"])
    rec = {"kernel": PREFILL_KERNEL, "workload": workload, "front": front,
           "sources": PREFILL_SOURCES,
           "source_sha256": sources_digest(PREFILL_SOURCES),
           "fetch_size_kib": fk, "write_size_kib": wk, "dispatches": len(f["prefill"]),
           "copy_calibration": {"bytes_each_way": copy_bytes,
                                "fetch_size_kib": sum(f["copy"]) / len(f["copy"]),
                                "write_size_kib": sum(w["copy"]) / len(w["copy"]),
                                "fetch_scale": fscale, "write_scale": wscale},
           "read_bytes": round(fk * 1024 * fscale), "write_bytes": round(wk * 1024 * wscale)}
    rec["traffic_bytes"] = rec["read_bytes"] + rec["write_bytes"]
    with open(traffic_record_path(workload, front), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def copy_calibration(kda, mib):
    """One fp32 state-pool copy of `mib` MiB read + `mib` MiB written: the plain
    copy kernel whose FETCH_SIZE / WRITE_SIZE readings scale the prefill's."""
    import torch
    H = 96
    slots = max(1, (mib << 20) // (H * D * D * 4))
    src = torch.ones((slots, H, D, D), dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    kda.state_io(kda.STATE_COPY, dst, src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    start.record(stream)
    for _ in range(reps):
        kda.state_io(kda.STATE_COPY, dst, src)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    nbytes = src.numel() * 4
    return {"bytes_read": nbytes, "bytes_written": nbytes, "kernel": "state_io_kernel",
            "ms": ms, "gb_per_s": 2 * nbytes / (ms * 1e-3) / 1e9}


def note(msg):
    """A progress line on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(*args.record_traffic, args.workload, args.copy_calibration_mib or 1536,
                       args.front)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    import gated_delta_rule_10_amd as kda
    import kda_inputs as ki
    kda.library()
    torch.cuda.set_device(0)

    pre = time_prefill(kda, ki, args.workload, args.steps, args.warmup, args.segments,
                       args.front, args.gate_params)
    head = prefill_summary(pre, args.steps)
    note(f"{args.workload}: {head['ms_per_step']:.3f} ms per prefill")
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "sequences": pre["seqs"],
                   "tokens": pre["tokens"], "heads": pre["heads"], "head_dim": D, "chunk": C,
                   "state": "fp32", "segments": args.segments, "front": args.front,
                   **({"gate_params": args.gate_params} if args.front == "gate" else {})},
        "tflops": head["tflops"],
        "mfma_peak_frac": head["mfma_peak_frac"],
        "roofline": {"bound": "hbm", "achieved": head["gb_per_s"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": head["hbm_frac"],
                     "traffic": measured_traffic(args.workload, args.front),
                     "kernel": PREFILL_KERNEL,
                     "bytes_per_launch": head["bytes_per_launch"]},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pre["x"], args.cpu_seconds, pre["gate_params"])
        note(f"oracle baseline: {line['cpu_baseline']['value']:.0f} tokens/s")
    del pre
    torch.cuda.empty_cache()
    extras = [w for w in args.extra.split(",") if w and w != args.workload]
    if extras:
        line["prefill_workloads"] = {}
    for wl in extras:
        steps = max(args.steps, 20)
        p = time_prefill(kda, ki, wl, steps, max(args.warmup, 5), args.segments, args.front,
                         args.gate_params)
        line["prefill_workloads"][wl] = {**prefill_summary(p, steps),
                                         "traffic": measured_traffic(wl, args.front)}
        note(f"{wl}: {line['prefill_workloads'][wl]['ms_per_step']:.3f} ms per prefill")
        del p
        torch.cuda.empty_cache()
    # (not in a counter-calibration run: the traffic record takes every state_io
    # dispatch of that run as the calibration copy)
    if not args.no_state_io and not args.copy_calibration_mib:
        line["state_io"] = time_state_io(kda)
        note("state_io timed")
    if not args.no_decode:
        line["decode"] = time_decode(kda, ki, args.decode_steps, kernel=args.decode_kernel,
                                     window=args.spec_window)
        line["decode"]["workload"] = DECODE_WORKLOAD
        note("decode timed")
    if args.bwd:
        line["backward"] = time_backward(kda, ki, PREFILL_BWD_WORKLOAD, max(2, args.steps // 2),
                                         max(1, args.warmup // 2),
                                         0.0 if args.no_cpu_baseline else args.cpu_seconds)
    if args.copy_calibration_mib > 0:
        line["copy_calibration"] = copy_calibration(kda, args.copy_calibration_mib)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
