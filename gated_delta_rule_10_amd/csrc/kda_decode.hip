// kda_decode.hip -- decode tokens per (row, head), in place on an fp32 state pool:
// the plain recurrent step, the fused step with the layer's front end and output
// normalisation, and the speculative-decode verification that replays accepted
// draft tokens -- one loop kernel for all three.
//
// Pages (cited by title and section):
//  "Kimi K3 -- Training and Infrastructure Notes", section 4.5 (KDA decoding):
//    the decode kernel fuses short convolution, input normalisation, gating, the
//    KDA recurrence and output normalisation and updates the state in place;
//    under speculative decoding only the drafts' projected inputs are kept, the
//    accepted tokens are replayed to rebuild the state on chip, the state of the
//    verified tokens is written back, and the replayed tokens and the next draft
//    window share one recurrent loop in one kernel.
//  "Kimi K3: a 2.8T open model ...", "Kimi Delta Attention": queries and keys come
//    from a short convolution followed by Swish and L2 normalisation, values
//    from a short convolution and Swish.
//  "How Kimi K3 Engineered Its Way to the Frontier", "How KDA updates its state"
//    and "What the hybrid saves": one ShortConv cache each for the query, key and
//    value projections, kernel size 4; the recurrence (decay, erase + write,
//    read) and K3's lower-bounded gate.
//
// The step is bound by HBM: it reads and writes the 64 KiB fp32 state of every
// (row, head) once, against ~7 * 128^2 flops per token.  One 512-thread
// workgroup per (row, head) owns that head's state and its three conv caches for
// the whole call: the state stays in registers and the conv window in the
// registers of the threads that convolve, across all tokens of the call, so the
// state costs one read and at most one write however many tokens run (a split of
// a state's value columns over two workgroups would have both read the q and k
// caches while one rewrites them).  The first token's q, k, v and g are loaded
// before the state: the load counter is in order, so the front end waits only
// for those bytes while the state streams in (measured 1.07 ms against 1.17 ms
// per 512 x 96 step with the order reversed).  A call has two phases of tokens:
//   A: tokens whose state is committed -- the fused step's one token, or the
//      verification's replayed accepted tokens; after them the state and the
//      conv window are written back (when at least one ran);
//   B: tokens whose outputs are wanted but whose state is not kept -- the new
//      verification window.
// The plain step is phase A with one token and the front end compiled out
// (FRONT = false).  Per token:
//   1. threads 0..383 run the convolution of one (input, channel) -- q, k, v
//      for t / 128 = 0, 1, 2 -- shift their window and apply Swish (or stage
//      the input as given); threads 384..511 stage the per-channel decay;
//   2. one wave reduces |q|^2, |k|^2 and q.k for the L2 norms;
//   3. decay, r = S^T k and y = S^T q (thread t: value columns 4 (t % 32) .. +3
//      of key rows t / 32 + 16 i), reduced over key rows in registers and then
//      through LDS;
//   4. u = beta (v - r), o = scale (y + (q.k) u) and the output norm's sum of
//      squares; S += k u^T; o stored.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kD = KDA_HEAD_DIM;  // 128
constexpr int kW = KDA_CONV_WIDTH;  // 4
constexpr int kNT = 512;
constexpr int kCG = kD / 4;       // 32 column groups of 4 value columns
constexpr int kRG = kNT / kCG;    // 16 row groups
constexpr int kRPT = kD / kRG;    // 8 key rows per thread

// Token inputs of one phase: [B, T, H, 128] (q, k, v, g, o) and [B, T, H] (beta).
struct Tokens {
  const void *q, *k, *v;
  const float *g, *beta;
  void *o;               // null: outputs not written
  int32_t T;             // tokens per row in the arrays
  const int32_t *count;  // device [B]: tokens to run, clamped to [0, T]; null = T
};

struct LoopParams {
  Tokens a, b;             // committed phase, then the phase whose state is dropped
  const float *conv_w;     // [3][H][128][4]
  void *conv_cache;        // [slots][3][3][H][128]
  float *state;            // [slots][H][128][128]
  const int32_t *slot_of_row;
  int32_t num_slots, H;
  float scale, l2_eps, norm_eps;
  int32_t out_norm;
  const float *norm_w;     // [128] or null
  const float *A_log, *dt_bias;
  float gate_scale;        // lower_bound log2(e)
  int32_t beta_logits;
  int32_t stagger;         // sleep before the state loads: 0 none, 1 long, 2 short (launch)
};

// FRONT: the short-convolution front end, the L2 norms and the output norm; without
// it q, k, v are used as given (the plain step).
template <class IO, bool GATE, bool FRONT>
__global__ __launch_bounds__(kNT) void decode_loop_kernel(LoopParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int slot = p.slot_of_row ? p.slot_of_row[b] : b;
  if (slot < 0 || slot >= p.num_slots) return;  // uniform over the workgroup
  auto count_of = [&](const Tokens &tk) {
    int n = tk.T;
    if (tk.count) {
      const int c = tk.count[b];
      n = c < 0 ? 0 : (c > tk.T ? tk.T : c);
    }
    return n;
  };
  const int na = count_of(p.a), nb = count_of(p.b);

  const int t = threadIdx.x;
  const int cg = t % kCG;  // value columns 4 cg .. 4 cg + 3
  const int rg = t / kCG;  // key rows rg + kRG i
  float *__restrict__ S = p.state + ((int64_t)slot * p.H + h) * (kD * kD);
  const bool conv_thread = t < 3 * kD;
  const int ci = t / kD, cc = t % kD;  // input (q, k, v) and channel; decay channel t - 384

  // This thread's input of the first token, loaded before the state: the load
  // counter is in order, so the first token's front end then waits only for
  // these few bytes while the state streams in.
  // (a copy, not a reference: a reference into the arguments chosen at run time
  // would make the compiler keep the arguments in per-lane scratch memory)
  const Tokens first = na > 0 ? p.a : p.b;
  const bool any = na > 0 || nb > 0;
  auto input_ptr = [&](const Tokens &tk) -> const IO * {
    return reinterpret_cast<const IO *>(ci == 0 ? tk.q : ci == 1 ? tk.k : tk.v);
  };
  // (every thread loads both values, so no branch -- and no wait at its join --
  // comes before the state loads; t / 128 = 3 reads v, unused)
  IO x_cur = IO(0.f);
  float g_cur = 0.f, b_cur = 0.f;
  if (any) {
    const int64_t row0 = (int64_t)b * first.T * p.H + h;  // (b, 0, h)
    x_cur = input_ptr(first)[row0 * kD + cc];
    g_cur = first.g[row0 * kD + cc];
    b_cur = first.beta[row0];
  }

  // conv window of this thread's (input, channel): the three previous raw inputs,
  // also loaded before the state (the first token's front end waits only for them)
  IO *cache = nullptr;
  const int64_t tap = (int64_t)p.H * kD;  // elements between a cache's taps
  IO w0 = IO(0.f), w1 = IO(0.f), w2 = IO(0.f);
  f32x4 wt = {0.f, 0.f, 0.f, 0.f};
  if (FRONT && conv_thread) {
    cache = reinterpret_cast<IO *>(p.conv_cache) + ((int64_t)slot * 3 + ci) * (kW - 1) * tap +
            (int64_t)h * kD + cc;
    wt = *reinterpret_cast<const f32x4 *>(p.conv_w + (((int64_t)ci * p.H + h) * kD + cc) * kW);
    w0 = cache[0];
    w1 = cache[tap];
    w2 = cache[2 * tap];
  }
  // the output norm's weight of channel t (the two waves that write o)
  float nw = 1.f;
  if (FRONT && t < kD && p.norm_w) nw = p.norm_w[t];
  // On large grids each workgroup idles before its state loads (the small loads
  // above are issued first): ~3.4 us (127 x 64 clocks) when the call runs one
  // token per row, half that for longer windows.  Sweep on the 512 x 96 step in
  // steps of 512 clocks, 4,096 .. 12,288: plain step 1.177 / 1.110 / 0.995 /
  // 1.010 / 1.052 ms, with the front end 1.086 / 1.032 / 1.016 / 1.054 / 1.112
  // ms; verification of 4 + 4 tokens 2.17 ms at 4,096 clocks, 2.31 at 8,128.
  if (p.stagger == 1) __builtin_amdgcn_s_sleep(127);
  if (p.stagger == 2) __builtin_amdgcn_s_sleep(64);

  // the state, before anything waits on it
  f32x4 s[kRPT];
#pragma unroll
  for (int i = 0; i < kRPT; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (rg + kRG * i) * kD + 4 * cg));

  __shared__ float sx[3][kD];          // Swish(conv) of q, k, v (q, k not yet normalised)
  __shared__ float sa[kD];             // per-channel decay exp(g)
  __shared__ f32x4 red[2][kRG][kCG];   // partial column sums of r and y
  __shared__ float sc[4];              // 1/|q|, 1/|k|, q.k of the unit vectors
  __shared__ float sss[2];             // output norm: sums of squares of two waves
  __shared__ float su[kD];

  float gate_a = 0.f, gate_dt = 0.f;
  if constexpr (GATE) {
    if (!conv_thread) {
      gate_a = gate_head_factor(p.A_log[h]);
      gate_dt = p.dt_bias ? p.dt_bias[h * kD + (t - 3 * kD)] : 0.f;
    }
  }

  // Inputs of the call's token k (phase a's tokens, then phase b's), clamped to
  // the last one: issued one token ahead, so no token waits on its own loads.
  // (the phase's pointers are picked with the token-uniform condition first and
  // only then per lane: a per-lane pick through a reference into the arguments
  // would load the pointer itself from memory before every prefetch)
  auto load_inputs = [&](int k, IO &x, float &g, float &bt) {
    const int kk = k < na + nb ? k : na + nb - 1;
    const bool in_a = kk < na;
    const int j = in_a ? kk : kk - na;
    const int64_t row = ((int64_t)b * (in_a ? p.a.T : p.b.T) + j) * p.H + h;
    const IO *qp = reinterpret_cast<const IO *>(in_a ? p.a.q : p.b.q);
    const IO *kp = reinterpret_cast<const IO *>(in_a ? p.a.k : p.b.k);
    const IO *vp = reinterpret_cast<const IO *>(in_a ? p.a.v : p.b.v);
    const float *gp = in_a ? p.a.g : p.b.g;
    const float *bp = in_a ? p.a.beta : p.b.beta;
    const IO *src = ci == 0 ? qp : ci == 1 ? kp : vp;
    x = src[row * kD + cc];
    g = gp[row * kD + cc];
    bt = bp[row];
  };
  // token j of phase tk, the call's token k; its inputs are in x_cur, g_cur, b_cur
  auto token = [&](const Tokens &tk, int j, int k) {
    const int64_t row = ((int64_t)b * tk.T + j) * p.H + h;  // (b, j, h)
    const int64_t tok = row * kD;
    IO x_nxt;
    float g_nxt, b_nxt;
    // 1. front end
    if (conv_thread && !FRONT) {
      sx[ci][cc] = to_f32(x_cur);
    } else if (conv_thread) {
      const IO xn = x_cur;
      float y = wt[0] * to_f32(w0);
      y = fmaf(wt[1], to_f32(w1), y);
      y = fmaf(wt[2], to_f32(w2), y);
      y = fmaf(wt[3], to_f32(xn), y);
      w0 = w1;  // the window keeps raw inputs: an exact shift
      w1 = w2;
      w2 = xn;
      sx[ci][cc] = y * sigmoid_fast(y);
    } else {
      const int c = t - 3 * kD;
      const float x = g_cur;
      if constexpr (GATE)
        sa[c] = fast_exp2(gate_log2(x, gate_a, gate_dt, p.gate_scale));
      else
        sa[c] = fast_exp2(x * kLog2e);
    }
    load_inputs(k + 1, x_nxt, g_nxt, b_nxt);
    block_sync();
    // 2. L2 norms of q and k, and q.k of the normalised vectors
    if (t < 64) {
      const float q0 = sx[0][2 * t], q1 = sx[0][2 * t + 1];
      const float k0 = sx[1][2 * t], k1 = sx[1][2 * t + 1];
      float qq = q0 * q0 + q1 * q1, kk = k0 * k0 + k1 * k1, qk = q0 * k0 + q1 * k1;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        qq += __shfl_xor(qq, off, 64);
        kk += __shfl_xor(kk, off, 64);
        qk += __shfl_xor(qk, off, 64);
      }
      if (t == 0) {
        const float iq = FRONT ? 1.f / sqrtf(qq + p.l2_eps) : 1.f;
        const float ik = FRONT ? 1.f / sqrtf(kk + p.l2_eps) : 1.f;
        sc[0] = iq;
        sc[1] = ik;
        sc[2] = qk * iq * ik;
      }
    }
    block_sync();
    // 3. decay, then r = S'^T k and y = S'^T q with the unnormalised q, k
    f32x4 r4 = {0.f, 0.f, 0.f, 0.f}, y4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kRPT; ++i) {
      const int kr = rg + kRG * i;
      s[i] *= sa[kr];
      r4 += s[i] * sx[1][kr];
      y4 += s[i] * sx[0][kr];
    }
    red[0][rg][cg] = r4;
    red[1][rg][cg] = y4;
    block_sync();
    // 4. outputs, the write vector u and the output norm's sum of squares
    const float iq = sc[0], ik = sc[1];
    float o = 0.f;
    if (t < kD) {
      const float *rr = reinterpret_cast<const float *>(&red[0][0][0]);
      const float *yy = reinterpret_cast<const float *>(&red[1][0][0]);
      float r = 0.f, y = 0.f;
#pragma unroll
      for (int j2 = 0; j2 < kRG; ++j2) {
        r += rr[j2 * kD + t];
        y += yy[j2 * kD + t];
      }
      const float bt = p.beta_logits ? sigmoid_fast(b_cur) : b_cur;
      const float u = bt * (sx[2][t] - ik * r);
      su[t] = u;
      o = p.scale * (iq * y + sc[2] * u);
      float sq = o * o;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 64);
      if ((t & 63) == 0) sss[t >> 6] = sq;
    }
    block_sync();
    const f32x4 u4 = *reinterpret_cast<const f32x4 *>(&su[4 * cg]);
#pragma unroll
    for (int i = 0; i < kRPT; ++i) s[i] += (ik * sx[1][rg + kRG * i]) * u4;
    if (t < kD && tk.o) {
      if (FRONT && p.out_norm) {
        const float inv = 1.f / sqrtf((sss[0] + sss[1]) * (1.f / kD) + p.norm_eps);
        o *= inv * nw;
      }
      reinterpret_cast<IO *>(tk.o)[tok + t] = from_f32<IO>(o);
    }
    x_cur = x_nxt;  // many barriers after the loads were issued
    g_cur = g_nxt;
    b_cur = b_nxt;
  };

  for (int j = 0; j < na; ++j) {
    if (j > 0) block_sync();  // the previous token's reads of sx, su, sc are done
    token(p.a, j, j);
  }
  if (na > 0) {  // write back the committed state and conv window
#pragma unroll
    for (int i = 0; i < kRPT; ++i)
      __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4 *>(S + (rg + kRG * i) * kD + 4 * cg));
    if (FRONT && conv_thread) {
      cache[0] = w0;
      cache[tap] = w1;
      cache[2 * tap] = w2;
    }
  }
  for (int j = 0; j < nb; ++j) {
    if (na > 0 || j > 0) block_sync();
    token(p.b, j, na + j);
  }
}

template <class IO, bool GATE, bool FRONT>
hipError_t launch_typed(const LoopParams &lp, unsigned blocks, hipStream_t stream) {
  hipLaunchKernelGGL((decode_loop_kernel<IO, GATE, FRONT>), dim3(blocks), dim3(kNT), 0, stream,
                     lp);
  return hipGetLastError();
}

// The fields shared by the fused step and the verification.
LoopParams common(const kda_fused_step_args &a) {
  LoopParams lp;
  lp.conv_w = a.conv_weight;
  lp.conv_cache = a.conv_cache;
  lp.state = a.state;
  lp.slot_of_row = a.state_indices;
  lp.num_slots = a.num_slots;
  lp.H = a.num_heads;
  lp.scale = a.scale;
  lp.l2_eps = a.l2_eps;
  lp.norm_eps = a.norm_eps;
  lp.out_norm = a.out_norm;
  lp.norm_w = a.norm_weight;
  lp.A_log = a.gate.A_log;
  lp.dt_bias = a.gate.dt_bias;
  lp.gate_scale = (float)((double)a.gate.lower_bound * 1.4426950408889634);  // lower_bound log2(e)
  lp.beta_logits = a.gate.beta_logits;
  lp.stagger = 0;
  return lp;
}

template <bool FRONT>
hipError_t launch(const kda_fused_step_args &a, LoopParams lp, hipStream_t stream) {
  const unsigned blocks = (unsigned)a.batch * (unsigned)a.num_heads;
  // The start delay pays off when the grid is many times what the device holds at
  // once (measured: 12,288 and 49,152 workgroups 10-11% faster, 3,072 2.5% slower).
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  const bool one_token = (int64_t)lp.a.T + lp.b.T <= 1;
  lp.stagger = cus > 0 && blocks >= 32u * (unsigned)cus ? (one_token ? 1 : 2) : 0;
  const bool gate = a.gate.mode == KDA_GATE_LOWER_BOUND;
  if (a.io_dtype == KDA_BF16)
    return gate ? launch_typed<bf16, true, FRONT>(lp, blocks, stream)
                : launch_typed<bf16, false, FRONT>(lp, blocks, stream);
  return gate ? launch_typed<float, true, FRONT>(lp, blocks, stream)
              : launch_typed<float, false, FRONT>(lp, blocks, stream);
}

}  // namespace

hipError_t launch_fused_decode_step(const kda_fused_step_args &a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  LoopParams lp = common(a);
  lp.a = Tokens{a.q, a.k, a.v, a.g, a.beta, a.o, 1, nullptr};
  lp.b = Tokens{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr};
  return launch<true>(a, lp, stream);
}

hipError_t launch_recurrent_step(const kda_recurrent_step_args &r, hipStream_t stream) {
  if (r.batch == 0) return hipSuccess;
  kda_fused_step_args a = {};
  a.batch = r.batch;
  a.num_heads = r.num_heads;
  a.io_dtype = r.io_dtype;
  a.scale = r.scale;
  a.state = r.state;
  a.state_indices = r.state_indices;
  a.num_slots = r.num_slots;
  a.gate = r.gate;
  LoopParams lp = common(a);
  lp.a = Tokens{r.q, r.k, r.v, r.g, r.beta, r.o, 1, nullptr};
  lp.b = Tokens{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr};
  return launch<false>(a, lp, stream);
}

hipError_t launch_spec_verify(const kda_spec_verify_args &v, hipStream_t stream) {
  const kda_fused_step_args &a = v.step;
  if (a.batch == 0) return hipSuccess;
  LoopParams lp = common(a);
  lp.a = Tokens{v.replay_q, v.replay_k, v.replay_v, v.replay_g, v.replay_beta, nullptr,
                v.replay_window, v.num_replay};
  lp.b = Tokens{a.q, a.k, a.v, a.g, a.beta, a.o, v.window, nullptr};
  return launch<true>(a, lp, stream);
}

}  // namespace kda
