// kda_decode.hip -- recurrent KDA decode step, in place on an fp32 state pool.
//
// Computes, per (row b, head h), one token of the recurrence of "How Kimi K3
// Engineered Its Way to the Frontier" (section "How KDA updates its state"):
// forget (rows of S scaled by exp(g)), erase+write against the decayed state,
// read from the updated state; the state stays in HBM and is rewritten in place
// ("Kimi K3 -- Training and Infrastructure Notes", section 4.5).
//
//   S' = Diag(exp g) S,  r = S'^T k,  y = S'^T q,  u = beta (v - r)
//   S  = S' + k u^T,     o = scale (y + (q . k) u)
//
// The step is bound by HBM: it reads and writes the 64 KiB fp32 state of every
// (row, head) once, against ~7 * 128^2 flops.  Value columns are independent
// (every sum runs over key rows), so a state is split by columns: NC columns
// per NT-thread workgroup, thread t holding four columns (4 (t % (NC/4)) .. +3)
// of key rows t / (NC/4) + RG i.  With NC = 64 each wave load/store covers four
// 256-byte half rows, and the two workgroups of a state run side by side; this
// measured faster than one 128-column workgroup per state (5.46 vs 5.16 TB/s),
// than 32-column quarters (128-byte segments) and than caching the state
// accesses.  Column sums over the key rows are reduced first in registers, then
// across the row groups through LDS.  All state loads are issued before anything
// waits on them.
//
// GATE: g holds gate logits of K3's lower-bounded gate ("How Kimi K3 Engineered
// Its Way to the Frontier", "How KDA updates its state"), turned into the decay
// as it is staged; beta logits (beta_logits) pass through a sigmoid.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kD = KDA_HEAD_DIM;  // 128
constexpr int kCols = 64;     // value columns per workgroup: two workgroups per state
constexpr int kThreads = 256;

struct GateArgs {
  const float *A_log, *dt_bias;  // [H], [H][128] or null
  float scale;                   // lower_bound log2(e)
  int32_t beta_logits;
};

template <class IO, int NC, int NT, bool GATE>
__global__ __launch_bounds__(NT) void recurrent_step_kernel(
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ state,
    const int32_t *__restrict__ slot_of_row, int32_t num_slots, int32_t H, float scale,
    IO *__restrict__ o, GateArgs ga) {
  constexpr int NP = kD / NC;        // workgroups per state
  constexpr int CG = NC / 4;         // column groups (4 columns each)
  constexpr int RG = NT / CG;        // row groups
  constexpr int RPT = kD / RG;       // rows per thread
  const int bh = blockIdx.x / NP;    // (row, head)
  const int part = blockIdx.x - bh * NP;
  const int b = bh / H;
  const int h = bh - b * H;
  const int slot = slot_of_row ? slot_of_row[b] : b;
  if (slot < 0 || slot >= num_slots) return;  // uniform over the workgroup

  float *__restrict__ S = state + ((int64_t)slot * H + h) * (kD * kD) + NC * part;
  const int t = threadIdx.x;
  const int cg = t % CG;  // value columns 4*cg .. 4*cg+3 of the part
  const int rg = t / CG;  // key rows rg + RG*i

  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (rg + RG * i) * kD + 4 * cg));

  __shared__ float sq[kD], sk[kD], sa[kD], su[NC];
  __shared__ f32x4 red[2][RG][CG];
  __shared__ float sqk;
  const int64_t tok = (int64_t)bh * kD;
  auto decay = [&](int c) -> float {  // alpha of key channel c
    const float x = g[tok + c];
    if constexpr (GATE)
      return fast_exp2(gate_log2(x, gate_head_factor(ga.A_log[h]),
                                 ga.dt_bias ? ga.dt_bias[h * kD + c] : 0.f, ga.scale));
    else
      return fast_exp2(x * kLog2e);
  };
  if (t < kD) {
    sq[t] = to_f32(q[tok + t]);
    sk[t] = to_f32(k[tok + t]);
  } else if (t < 2 * kD) {
    sa[t - kD] = decay(t - kD);
  }
  if (NT < 2 * kD && t < kD) sa[t] = decay(t);
  block_sync();

  if (t < 64) {  // q . k, one wave
    float p = sq[2 * t] * sk[2 * t] + sq[2 * t + 1] * sk[2 * t + 1];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off, 64);
    if (t == 0) sqk = p;
  }
  f32x4 r4 = {0.f, 0.f, 0.f, 0.f}, y4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    s[i] *= sa[row];
    r4 += s[i] * sk[row];
    y4 += s[i] * sq[row];
  }
  red[0][rg][cg] = r4;
  red[1][rg][cg] = y4;
  block_sync();

  if (t < NC) {
    const float *rr = reinterpret_cast<const float *>(&red[0][0][0]);
    const float *yy = reinterpret_cast<const float *>(&red[1][0][0]);
    float r = 0.f, y = 0.f;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      r += rr[j * NC + t];
      y += yy[j * NC + t];
    }
    const int col = NC * part + t;
    const float bt = ga.beta_logits ? sigmoid_fast(beta[bh]) : beta[bh];
    const float u = bt * (to_f32(v[tok + col]) - r);
    su[t] = u;
    o[tok + col] = from_f32<IO>(scale * (y + sqk * u));
  }
  block_sync();

  const f32x4 u4 = *reinterpret_cast<const f32x4 *>(&su[4 * cg]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg + RG * i;
    const f32x4 nv = s[i] + sk[row] * u4;
    __builtin_nontemporal_store(nv, reinterpret_cast<f32x4 *>(S + row * kD + 4 * cg));
  }
}

template <class IO, bool GATE>
hipError_t launch_typed(const kda_recurrent_step_args &a, const GateArgs &ga, hipStream_t stream) {
  constexpr int NC = kCols, NT = kThreads;
  const dim3 grid((unsigned)a.batch * (unsigned)a.num_heads * (unsigned)(kD / NC));
  hipLaunchKernelGGL((recurrent_step_kernel<IO, NC, NT, GATE>), grid, dim3(NT), 0, stream,
                     (const IO *)a.q, (const IO *)a.k, (const IO *)a.v, a.g, a.beta, a.state,
                     a.state_indices, a.num_slots, a.num_heads, a.scale, (IO *)a.o, ga);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_recurrent_step(const kda_recurrent_step_args &a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  GateArgs ga;
  ga.A_log = a.gate.A_log;
  ga.dt_bias = a.gate.dt_bias;
  ga.scale = (float)((double)a.gate.lower_bound * 1.4426950408889634);  // lower_bound log2(e)
  ga.beta_logits = a.gate.beta_logits;
  const bool gate = a.gate.mode == KDA_GATE_LOWER_BOUND;
  if (a.io_dtype == KDA_BF16)
    return gate ? launch_typed<bf16, true>(a, ga, stream) : launch_typed<bf16, false>(a, ga, stream);
  return gate ? launch_typed<float, true>(a, ga, stream) : launch_typed<float, false>(a, ga, stream);
}

}  // namespace kda
