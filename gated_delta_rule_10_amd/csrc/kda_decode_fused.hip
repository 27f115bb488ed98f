// kda_decode_fused.hip -- one decode token per (row, head) with the layer's front
// end and output normalisation in the same kernel.
//
// Pages (cited by title and section):
//  "Kimi K3 -- Training and Infrastructure Notes", section 4.5: the decode kernel
//    fuses short convolution, input normalisation, gating, the KDA recurrence and
//    output normalisation; the state is updated in place.
//  "Kimi K3: a 2.8T open model ...", "Kimi Delta Attention": queries and keys come
//    from a short convolution followed by Swish and L2 normalisation, values
//    from a short convolution and Swish.
//  "How Kimi K3 Engineered Its Way to the Frontier", "How KDA updates its state"
//    and "What the hybrid saves": one ShortConv cache each for the query, key and
//    value projections, kernel size 4; the recurrence (decay, erase + write,
//    read) and K3's lower-bounded gate.
//
// One 512-thread workgroup per (row, head) owns that head's state and its three
// conv caches, so the caches are read and rewritten without any other workgroup
// touching them (splitting a state's value columns over two workgroups, as the
// plain step does, would have both read the q and k caches while one rewrites
// them).  The fp32 state is the traffic (64 KiB in and out); everything else is
// a few KiB:
//   1. the state loads are issued first (thread t: value columns 4 (t % 32) ..
//      +3 of key rows t / 32 + 16 i, i < 8, nontemporal 16-byte accesses);
//   2. threads 0..383 run the convolution of one (input, channel) -- q, k, v
//      for t / 128 = 0, 1, 2 -- shift its cache and apply Swish; threads
//      384..511 stage the per-channel decay;
//   3. one wave reduces |q|^2, |k|^2 and q.k for the L2 norms;
//   4. decay, r = S^T k and y = S^T q from the loaded state, reduced over key
//      rows in registers and then through LDS;
//   5. u = beta (v - r), o = scale (y + (q.k) u), the output norm's sum of
//      squares; S += k u^T written back.
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

struct FusedParams {
  const void *q, *k, *v;
  const float *g, *beta;
  const float *conv_w;     // [3][H][128][4]
  void *conv_cache;        // [slots][3][3][H][128]
  float *state;            // [slots][H][128][128]
  const int32_t *slot_of_row;
  int32_t num_slots, H;
  float scale, l2_eps, norm_eps;
  int32_t out_norm;
  const float *norm_w;     // [128] or null
  void *o;
  const float *A_log, *dt_bias;
  float gate_scale;        // lower_bound log2(e)
  int32_t beta_logits;
};

template <class IO, bool GATE>
__global__ __launch_bounds__(kNT) void fused_step_kernel(FusedParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int slot = p.slot_of_row ? p.slot_of_row[b] : b;
  if (slot < 0 || slot >= p.num_slots) return;  // uniform over the workgroup

  const int t = threadIdx.x;
  const int cg = t % kCG;  // value columns 4 cg .. 4 cg + 3
  const int rg = t / kCG;  // key rows rg + kRG i
  float *__restrict__ S = p.state + ((int64_t)slot * p.H + h) * (kD * kD);

  // 1. the state, before anything waits
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

  const int64_t tok = (int64_t)bh * kD;
  // 2. front end
  if (t < 3 * kD) {
    const int i = t / kD, c = t % kD;
    const IO *X = reinterpret_cast<const IO *>(i == 0 ? p.q : i == 1 ? p.k : p.v);
    IO *cache = reinterpret_cast<IO *>(p.conv_cache) +
                ((int64_t)slot * 3 + i) * (kW - 1) * ((int64_t)p.H * kD) + (int64_t)h * kD + c;
    const int64_t tap = (int64_t)p.H * kD;  // elements between a cache's taps
    const f32x4 w = *reinterpret_cast<const f32x4 *>(p.conv_w + (((int64_t)i * p.H + h) * kD + c) * kW);
    const IO x0 = cache[0], x1 = cache[tap], x2 = cache[2 * tap], xn = X[tok + c];
    float y = w[0] * to_f32(x0);
    y = fmaf(w[1], to_f32(x1), y);
    y = fmaf(w[2], to_f32(x2), y);
    y = fmaf(w[3], to_f32(xn), y);
    cache[0] = x1;  // the cache keeps raw inputs: an exact shift
    cache[tap] = x2;
    cache[2 * tap] = xn;
    sx[i][c] = y * sigmoid_fast(y);
  } else {
    const int c = t - 3 * kD;
    const float x = p.g[tok + c];
    if constexpr (GATE)
      sa[c] = fast_exp2(gate_log2(x, gate_head_factor(p.A_log[h]),
                                  p.dt_bias ? p.dt_bias[h * kD + c] : 0.f, p.gate_scale));
    else
      sa[c] = fast_exp2(x * kLog2e);
  }
  block_sync();

  // 3. L2 norms of q and k, and q.k of the normalised vectors
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
      const float iq = 1.f / sqrtf(qq + p.l2_eps), ik = 1.f / sqrtf(kk + p.l2_eps);
      sc[0] = iq;
      sc[1] = ik;
      sc[2] = qk * iq * ik;
    }
  }
  block_sync();

  // 4. decay, then r = S'^T k and y = S'^T q with the unnormalised q, k (scaled below)
  f32x4 r4 = {0.f, 0.f, 0.f, 0.f}, y4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kRPT; ++i) {
    const int row = rg + kRG * i;
    s[i] *= sa[row];
    r4 += s[i] * sx[1][row];
    y4 += s[i] * sx[0][row];
  }
  red[0][rg][cg] = r4;
  red[1][rg][cg] = y4;
  block_sync();

  // 5. outputs, the write vector u and the output norm's sum of squares
  const float iq = sc[0], ik = sc[1];
  float o = 0.f;
  if (t < kD) {
    const float *rr = reinterpret_cast<const float *>(&red[0][0][0]);
    const float *yy = reinterpret_cast<const float *>(&red[1][0][0]);
    float r = 0.f, y = 0.f;
#pragma unroll
    for (int j = 0; j < kRG; ++j) {
      r += rr[j * kD + t];
      y += yy[j * kD + t];
    }
    const float bt = p.beta_logits ? sigmoid_fast(p.beta[bh]) : p.beta[bh];
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
  for (int i = 0; i < kRPT; ++i) {
    const int row = rg + kRG * i;
    const f32x4 nv = s[i] + (ik * sx[1][row]) * u4;
    __builtin_nontemporal_store(nv, reinterpret_cast<f32x4 *>(S + row * kD + 4 * cg));
  }
  if (t < kD) {
    if (p.out_norm) {
      const float inv = 1.f / sqrtf((sss[0] + sss[1]) * (1.f / kD) + p.norm_eps);
      o *= inv * (p.norm_w ? p.norm_w[t] : 1.f);
    }
    reinterpret_cast<IO *>(p.o)[tok + t] = from_f32<IO>(o);
  }
}

template <class IO, bool GATE>
hipError_t launch_typed(const FusedParams &fp, unsigned blocks, hipStream_t stream) {
  hipLaunchKernelGGL((fused_step_kernel<IO, GATE>), dim3(blocks), dim3(kNT), 0, stream, fp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fused_decode_step(const kda_fused_step_args &a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  FusedParams fp;
  fp.q = a.q;
  fp.k = a.k;
  fp.v = a.v;
  fp.g = a.g;
  fp.beta = a.beta;
  fp.conv_w = a.conv_weight;
  fp.conv_cache = a.conv_cache;
  fp.state = a.state;
  fp.slot_of_row = a.state_indices;
  fp.num_slots = a.num_slots;
  fp.H = a.num_heads;
  fp.scale = a.scale;
  fp.l2_eps = a.l2_eps;
  fp.norm_eps = a.norm_eps;
  fp.out_norm = a.out_norm;
  fp.norm_w = a.norm_weight;
  fp.o = a.o;
  fp.A_log = a.gate.A_log;
  fp.dt_bias = a.gate.dt_bias;
  fp.gate_scale = (float)((double)a.gate.lower_bound * 1.4426950408889634);  // lower_bound log2(e)
  fp.beta_logits = a.gate.beta_logits;
  const unsigned blocks = (unsigned)a.batch * (unsigned)a.num_heads;
  const bool gate = a.gate.mode == KDA_GATE_LOWER_BOUND;
  if (a.io_dtype == KDA_BF16)
    return gate ? launch_typed<bf16, true>(fp, blocks, stream)
                : launch_typed<bf16, false>(fp, blocks, stream);
  return gate ? launch_typed<float, true>(fp, blocks, stream)
              : launch_typed<float, false>(fp, blocks, stream);
}

}  // namespace kda
