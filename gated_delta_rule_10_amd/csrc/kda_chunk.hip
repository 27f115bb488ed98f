// kda_chunk.hip -- chunkwise KDA prefill forward on gfx950 matrix cores.
//
// Pages (cited by title and section):
//  [P1] "How Kimi K3 Engineered Its Way to the Frontier": "How KDA updates its
//       state" (the recurrence; decay per key channel = per row of S) and
//       "FlashKDA steps the state once per 16 tokens" (split into chunks, compute
//       inside a chunk with dense products, step the state once per chunk; the
//       lower-bounded gate keeps reciprocal cumulative decays of a 16-token tile
//       in range so every tile is a dense matrix product; 16x16 unit-triangular
//       inverse by a Neumann series, exact after three doubling rounds).
//  [P2] "Kimi K3: Open Frontier Intelligence", section 6 (the equation; with
//       log-decay >= -5 a 16-token tile's cumulative log-decay lies in (-80, 0)).
//  [P3] "Kimi K3 -- Training and Infrastructure Notes", section 4.1 (overlap
//       chunk-local work with the cross-chunk state recurrence; segment
//       transitions composed exactly).
//
// Chunk algebra (chunk of C = 64 tokens, incoming state S, 128 x 128):
//   G_r = sum_{s<=r} g_s (per key channel);   Q~ = q e^{G}, K~ = k e^{G},
//   Kbar = k e^{G_C - G}, Gamma = e^{G_C};
//   A[r,s] = beta_r k_r.(e^{G_r-G_s} k_s)  (s < r),  P[r,s] = q_r.(e^{G_r-G_s} k_s) (s <= r)
//   X = (I + A)^{-1}                          (unit lower triangular)
//   U = X (beta V - beta K~ S)                (the chunk's delta-rule updates)
//   O = scale (Q~ S + P U),  S <- Gamma S + Kbar^T U.
// This equals the token loop exactly; only rounding differs.
//
// MI355X design (one workgroup of 4 waves per (sequence, head[, value block])):
//  * The whole chain of chunks of one (sequence, head) runs in one workgroup, so
//    the fp32 state never leaves registers and no chunk-local matrix makes a
//    round trip through HBM: every input byte is read once and o written once.
//  * Wave w owns the 16 tokens of sub-tile w for the elementwise work (lane =
//    channel pair), and a quarter of the value columns for the recurrence
//    (columns of S evolve independently).  S (fp32) is the MFMA accumulator of
//    the state update and is repacked to bf16 in registers as the operand of the
//    next chunk's products -- it is never staged in LDS.
//  * Decay factors use a reference inside every 16-token sub-tile (its token 8),
//    so every factor fed to the matrix cores is a product of exponentials of at
//    most 8-token cumulative decays: below 2^58 under the page's -5 bound.
//    Off-diagonal sub-tile pairs (i > j) get their column operand pre-multiplied
//    by e^{G_ref(i) - G_ref(j)} <= 1.  (Valid whenever every 8-token cumulative
//    log-decay is above about -87; beyond that, exponents saturate.)
//  * The next chunk's q/k/v/g/beta are loaded into registers while the current
//    chunk runs its recurrence products.
//  * fp32 I/O uses the same kernel with fp32 operands (V_MFMA_F32_16X16X4_F32),
//    the intra-chunk products in two channel halves, and 64 value columns per
//    workgroup so the operand buffers fit in the 160 KiB of LDS.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = KDA_CHUNK;     // 64 tokens per chunk
constexpr int kD = KDA_HEAD_DIM;  // 128 channels
constexpr int kThreads = 256;
constexpr int kRef = 8;           // reference token inside each 16-token sub-tile

struct ChunkParams {
  const void *q, *k, *v;
  const float *g, *beta;
  const float *s0;
  float *sfinal;
  void *o;
  const int32_t *cu;     // device cu_seqlens or null
  const int32_t *order;  // device sequence order (longest first) or null
  int64_t total_tokens;  // T_total from the host-validated sizes
  int32_t H;
  int32_t seq_len;
  float scale;
};

// Tile list of the 10 lower (row-tile i, column-tile j) pairs and their owner wave.
__device__ __forceinline__ int tri_index(int i, int j) { return i * (i + 1) / 2 + j; }

template <class OpT, int DV>
struct Layout {
  static constexpr int NH = sizeof(OpT) == 4 ? 2 : 1;   // channel passes of the Gram products
  static constexpr int KH = kD / NH;                     // channels per pass
  static constexpr int PADE = 16 / (int)sizeof(OpT);     // 16-byte row padding
  static constexpr int LD_KH = KH + PADE;
  static constexpr int LD_D = kD + PADE;
  static constexpr int LD_C = kC + PADE;
  static constexpr int LD_O = DV + PADE;
  static constexpr int LD_F = kC + 4;                    // fp32 solve buffers
  static constexpr int LD_W = 17;                        // per-wave 16x16 fp32 scratch
  static constexpr int NVT = DV / 64;                    // 16-column value tiles per wave
  // Region R: three phases reuse the same bytes.
  //  Gram:       Kr[64][LD_KH], Qr[64][LD_KH], Kc[160][LD_KH]                 (OpT)
  //  solve:      A[64][LD_F], X[64][LD_F], 4 waves x 4 x [16][LD_W]          (fp32)
  //  recurrence: Qt[64][LD_D], nBKt[64][LD_D], KbT[128][LD_C], BVT[DV][LD_C]  (OpT)
  //  output:     Ost[64][LD_O]                                               (OpT)
  static constexpr size_t kGram = (size_t)(64 + 64 + 160) * LD_KH * sizeof(OpT);
  static constexpr size_t kSolve = (size_t)2 * 64 * LD_F * 4 + (size_t)4 * 4 * 16 * LD_W * 4;
  static constexpr size_t kRec =
      ((size_t)2 * 64 * LD_D + (size_t)128 * LD_C + (size_t)DV * LD_C) * sizeof(OpT);
  static constexpr size_t kOut = (size_t)64 * LD_O * sizeof(OpT);
  static constexpr size_t kRegion =
      kGram > kSolve ? (kGram > kRec ? (kGram > kOut ? kGram : kOut) : (kRec > kOut ? kRec : kOut))
                     : (kSolve > kRec ? (kSolve > kOut ? kSolve : kOut) : (kRec > kOut ? kRec : kOut));
  static constexpr size_t kXinv = (size_t)64 * LD_C * sizeof(OpT);
  static constexpr size_t kP = kXinv;
  static constexpr size_t kSmall = (size_t)(4 * 128 + 4 * 128 + 64 + 128) * 4;
  static constexpr size_t kTotal = kRegion + kXinv + kP + kSmall;
  static_assert(kTotal <= 160 * 1024, "LDS budget exceeded");
};

template <class OpT> struct Raw;  // two consecutive channels of one token
template <> struct Raw<bf16> {
  uint32_t u;
  __device__ __forceinline__ float lo() const { return __uint_as_float(u << 16); }
  __device__ __forceinline__ float hi() const { return __uint_as_float(u & 0xffff0000u); }
};
template <> struct Raw<float> {
  f32x2 f;
  __device__ __forceinline__ float lo() const { return f[0]; }
  __device__ __forceinline__ float hi() const { return f[1]; }
};
__device__ __forceinline__ void raw_load(Raw<bf16> &r, const bf16 *p) {
  r.u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}
__device__ __forceinline__ void raw_load(Raw<float> &r, const float *p) {
  r.f = __builtin_nontemporal_load(reinterpret_cast<const f32x2 *>(p));
}
template <class OpT> __device__ __forceinline__ void raw_zero(Raw<OpT> &r);
template <> __device__ __forceinline__ void raw_zero(Raw<bf16> &r) { r.u = 0u; }
template <> __device__ __forceinline__ void raw_zero(Raw<float> &r) { r.f = f32x2{0.f, 0.f}; }

// acc += X * Y for 16x16 fp32 blocks held in LDS (row-major), fp32 matrix cores.
// X rows/cols at x[r * ldx + c], Y at y[r * ldy + c]; result layout as mma().
__device__ __forceinline__ void mm16_f32(f32x4 &acc, const float *x, int ldx, const float *y,
                                         int ldy, int lane) {
  const int col = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = x[col * ldx + 4 * j + g];
    const float b = y[(4 * j + g) * ldy + col];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
  }
}
__device__ __forceinline__ void st16(float *c, int ldc, const f32x4 &acc, int lane) {
  const int col = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[(4 * g + i) * ldc + col] = acc[i];
}
__device__ __forceinline__ f32x4 ld16(const float *c, int ldc, int lane) {
  const int col = lane & 15, g = lane >> 4;
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = c[(4 * g + i) * ldc + col];
  return r;
}
__device__ __forceinline__ void wave_lds_fence() { __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <class OpT, int DV>
__global__ __launch_bounds__(kThreads, 1) void chunk_fwd_kernel(ChunkParams p) {
  typedef Layout<OpT, DV> L;
  constexpr int VS = kD / DV;  // value blocks per head
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::kTotal];

  unsigned char *region = smem;
  OpT *Xinv = reinterpret_cast<OpT *>(smem + L::kRegion);
  OpT *Pm = reinterpret_cast<OpT *>(smem + L::kRegion + L::kXinv);
  float *gtot = reinterpret_cast<float *>(smem + L::kRegion + L::kXinv + L::kP);
  float *gmid = gtot + 4 * 128;
  float *sbeta = gmid + 4 * 128;
  float *sgam = sbeta + 64;

  // Gram phase views
  OpT *Kr = reinterpret_cast<OpT *>(region);
  OpT *Qr = Kr + 64 * L::LD_KH;
  OpT *Kc = Qr + 64 * L::LD_KH;
  // solve phase views
  float *A32 = reinterpret_cast<float *>(region);
  float *X32 = A32 + 64 * L::LD_F;
  float *Wscr = X32 + 64 * L::LD_F;
  // recurrence phase views
  OpT *Qt = reinterpret_cast<OpT *>(region);
  OpT *nBKt = Qt + 64 * L::LD_D;
  OpT *KbT = nBKt + 64 * L::LD_D;
  OpT *BVT = KbT + 128 * L::LD_C;
  // output staging
  OpT *Ost = reinterpret_cast<OpT *>(region);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // ---- work item: (sequence rank, head, value block)
  const int item = blockIdx.x;
  const int vs = item % VS;
  const int chain = item / VS;
  const int srank = chain / p.H;
  const int h = chain - srank * p.H;
  const int n = p.order ? p.order[srank] : srank;
  int64_t bos = (int64_t)n * p.seq_len, len = p.seq_len;
  if (p.cu) {  // device offsets, clamped to the validated token range
    const int64_t a = p.cu[n], b = p.cu[n + 1];
    bos = a < 0 ? 0 : (a > p.total_tokens ? p.total_tokens : a);
    const int64_t e = b < bos ? bos : (b > p.total_tokens ? p.total_tokens : b);
    len = e - bos;
  }
  const int nchunks = (int)((len + kC - 1) / kC);
  const int H = p.H;
  const int vblk = vs * DV;               // first value column of this workgroup
  const int vw = vblk + w * (DV / 4);     // first value column of this wave

  const OpT *__restrict__ qg = reinterpret_cast<const OpT *>(p.q);
  const OpT *__restrict__ kg = reinterpret_cast<const OpT *>(p.k);
  const OpT *__restrict__ vg = reinterpret_cast<const OpT *>(p.v);
  OpT *__restrict__ og = reinterpret_cast<OpT *>(p.o);

  // One-time zero of the strictly-upper blocks of X and P that the 32-wide
  // k-steps read: blocks (0,1) and (2,3).
  for (int e = tid; e < 2 * 256; e += kThreads) {
    const int b = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
    const int r = 16 * (2 * b) + rr, c = 16 * (2 * b + 1) + cc;
    Xinv[r * L::LD_C + c] = from_f32<OpT>(0.f);
    Pm[r * L::LD_C + c] = from_f32<OpT>(0.f);
  }

  // ---- state (fp32 accumulators): S[ct][vt] holds S[16ct+4g4+i][vw+16vt+l16]
  f32x4 S[8][L::NVT];
  {
    const float *s0 = p.s0 ? p.s0 + ((int64_t)n * H + h) * (kD * kD) : nullptr;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int vt = 0; vt < L::NVT; ++vt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[ct][vt][i] = s0 ? s0[(16 * ct + 4 * g4 + i) * kD + vw + 16 * vt + l16] : 0.f;
  }

  // ---- register prefetch of a chunk's raw inputs: wave w = tokens 16w..16w+15,
  //      lane = channels 2*lane, 2*lane+1 (value channels vblk + 2*lane for DV=128;
  //      lanes < 32 cover the 64 columns when DV=64).
  Raw<OpT> rq[16], rk[16], rv[16];
  f32x2 rg[16];
  float rb = 0.f;
  const int c0 = 2 * lane;
  const bool has_v = (DV == 128) || (lane < 32);
  auto prefetch = [&](int j) {
    const int64_t t0 = bos + (int64_t)j * kC + 16 * w;
    const int64_t lim = bos + len;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int64_t tok = t0 + t;
      if (tok < lim) {
        const int64_t base = (tok * H + h) * kD;
        raw_load(rq[t], qg + base + c0);
        raw_load(rk[t], kg + base + c0);
        if (has_v) raw_load(rv[t], vg + base + vblk + c0); else raw_zero(rv[t]);
        rg[t] = __builtin_nontemporal_load(reinterpret_cast<const f32x2 *>(p.g + base + c0));
      } else {
        raw_zero(rq[t]); raw_zero(rk[t]); raw_zero(rv[t]);
        rg[t] = f32x2{0.f, 0.f};
      }
    }
    const int64_t tb = t0 + (lane & 15);
    rb = (lane < 16 && tb < lim) ? p.beta[tb * H + h] : 0.f;
  };
  if (nchunks > 0) prefetch(0);

  for (int j = 0; j < nchunks; ++j) {
    const int Lc = (int)((len - (int64_t)j * kC) < kC ? (len - (int64_t)j * kC) : kC);

    // ===== P0: per-channel cumulative log2-decay inside the sub-tile
    float G0[16], G1[16];
    {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        a0 += rg[t][0] * kLog2e;
        a1 += rg[t][1] * kLog2e;
        G0[t] = a0;
        G1[t] = a1;
      }
      gtot[w * 128 + c0] = a0;
      gtot[w * 128 + c0 + 1] = a1;
      gmid[w * 128 + c0] = G0[kRef];
      gmid[w * 128 + c0 + 1] = G1[kRef];
      if (lane < 16) sbeta[16 * w + lane] = rb;
    }
    block_sync();

    // chunk-relative reference values G(16i + kRef) for all sub-tiles, and G(last)
    float gref0[4], gref1[4], glast0 = 0.f, glast1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gref0[i] = glast0 + gmid[i * 128 + c0];
      gref1[i] = glast1 + gmid[i * 128 + c0 + 1];
      glast0 += gtot[i * 128 + c0];
      glast1 += gtot[i * 128 + c0 + 1];
    }
    // E1 = e^{G_t - G_ref} (row factor), E2 = e^{G_ref - G_t} (column factor)
    float E1a[16], E1b[16], E2a[16], E2b[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float d0 = G0[t] - G0[kRef], d1 = G1[t] - G1[kRef];
      E1a[t] = fast_exp2(d0);
      E1b[t] = fast_exp2(d1);
      E2a[t] = fast_exp2(-d0);
      E2b[t] = fast_exp2(-d1);
    }

    // ===== P1 + Gram: A = beta (Kr Kc^T), P = Qr Kc^T over the 10 lower tile pairs.
    // Tile t of the list (0,0),(1,0),(1,1),(2,0),(2,1),(2,2),(3,0),(3,1),(3,2),(3,3)
    // belongs to wave t % 4.
    f32x4 accA[3], accP[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      accA[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      accP[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int hc = 0; hc < L::NH; ++hc) {
      if (c0 / L::KH == hc) {
        const int cc = c0 - hc * L::KH;
        float F0[4], F1[4];  // e^{G_ref(i) - G_ref(w)} for i > w
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          F0[i] = i > w ? fast_exp2(gref0[i] - gref0[w]) : 1.f;
          F1[i] = i > w ? fast_exp2(gref1[i] - gref1[w]) : 1.f;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int r = 16 * w + t;
          const float k0 = rk[t].lo(), k1 = rk[t].hi();
          const float q0 = rq[t].lo(), q1 = rq[t].hi();
          store2<OpT>(Kr + r * L::LD_KH + cc, k0 * E1a[t], k1 * E1b[t]);
          store2<OpT>(Qr + r * L::LD_KH + cc, q0 * E1a[t], q1 * E1b[t]);
          const float b0 = k0 * E2a[t], b1 = k1 * E2b[t];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (i >= w) {
              OpT *dst = Kc + (tri_index(i, w) * 16 + t) * L::LD_KH + cc;
              store2<OpT>(dst, b0 * F0[i], b1 * F1[i]);
            }
          }
        }
      }
      block_sync();
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int tile = w + 4 * u;
        if (tile < 10) {
          const int ti = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
#pragma unroll
          for (int kk = 0; kk < L::KH / 32; ++kk) {
            Frag<OpT> xs, yk, yq;
            lds_frag_ck(xs, Kc + tile * 16 * L::LD_KH, L::LD_KH, l16, 32 * kk, g4);
            lds_frag_ck(yk, Kr + 16 * ti * L::LD_KH, L::LD_KH, l16, 32 * kk, g4);
            lds_frag_ck(yq, Qr + 16 * ti * L::LD_KH, L::LD_KH, l16, 32 * kk, g4);
            mma(accA[u], xs, yk);
            mma(accP[u], xs, yq);
          }
        }
      }
      block_sync();
    }
    // results: lane holds A[r = 16 ti + l16][s = 16 tj + 4 g4 + i]
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int tile = w + 4 * u;
      if (tile < 10) {
        const int ti = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
        const int tj = tile - tri_index(ti, 0);
        const int r = 16 * ti + l16;
        const float br = sbeta[r];
        f32x4 av, pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * tj + 4 * g4 + i;
          av[i] = s < r ? br * accA[u][i] : 0.f;
          pv[i] = s <= r ? accP[u][i] : 0.f;
        }
        *reinterpret_cast<f32x4 *>(A32 + r * L::LD_F + 16 * tj + 4 * g4) = av;
        OpT *pp = Pm + r * L::LD_C + 16 * tj + 4 * g4;
        store2<OpT>(pp, pv[0], pv[1]);
        store2<OpT>(pp + 2, pv[2], pv[3]);
      }
    }
    block_sync();

    // ===== solve: X = (I + A)^{-1}, fp32 matrix cores.
    {
      float *scr = Wscr + w * 4 * 16 * L::LD_W;  // four 16x16 scratch blocks of this wave
      float *s0b = scr, *s1b = scr + 16 * L::LD_W, *s2b = scr + 32 * L::LD_W,
            *s3b = scr + 48 * L::LD_W;
      // diagonal block w: Neumann series (I+N)^{-1} = (I-N)(I+N^2)(I+N^4)(I+N^8)
      const float *Nb = A32 + 16 * w * L::LD_F + 16 * w;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mm16_f32(acc, Nb, L::LD_F, Nb, L::LD_F, lane);  // N^2
      st16(s0b, L::LD_W, acc, lane);
      wave_lds_fence();
      f32x4 n3 = {0.f, 0.f, 0.f, 0.f};
      mm16_f32(n3, Nb, L::LD_F, s0b, L::LD_W, lane);  // N^3
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mm16_f32(acc, s0b, L::LD_W, s0b, L::LD_W, lane);  // N^4
      st16(s1b, L::LD_W, acc, lane);
      {
        const f32x4 nn = ld16(Nb, L::LD_F, lane), n2 = ld16(s0b, L::LD_W, lane);
        f32x4 p1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p1[i] = ((4 * g4 + i) == l16 ? 1.f : 0.f) - nn[i] + n2[i] - n3[i];
        st16(s2b, L::LD_W, p1, lane);  // P1 = (I - N)(I + N^2)
      }
      wave_lds_fence();
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mm16_f32(acc, s1b, L::LD_W, s1b, L::LD_W, lane);  // N^8
      st16(s3b, L::LD_W, acc, lane);
      f32x4 p2 = ld16(s2b, L::LD_W, lane);
      mm16_f32(p2, s2b, L::LD_W, s1b, L::LD_W, lane);  // P2 = P1 + P1 N^4
      st16(s0b, L::LD_W, p2, lane);
      wave_lds_fence();
      f32x4 xd = p2;
      mm16_f32(xd, s0b, L::LD_W, s3b, L::LD_W, lane);  // X = P2 + P2 N^8
      st16(X32 + 16 * w * L::LD_F + 16 * w, L::LD_F, xd, lane);
      block_sync();
      // off-diagonal blocks, X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj, by distance
#pragma unroll
      for (int dist = 1; dist <= 3; ++dist) {
        if (w < 4 - dist) {
          const int jj = w, ii = w + dist;
          f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
          for (int kk = jj; kk < ii; ++kk)
            mm16_f32(tacc, A32 + 16 * ii * L::LD_F + 16 * kk, L::LD_F,
                     X32 + 16 * kk * L::LD_F + 16 * jj, L::LD_F, lane);
          st16(s0b, L::LD_W, tacc, lane);
          wave_lds_fence();
          f32x4 xo = {0.f, 0.f, 0.f, 0.f};
          mm16_f32(xo, X32 + 16 * ii * L::LD_F + 16 * ii, L::LD_F, s0b, L::LD_W, lane);
          st16(X32 + 16 * ii * L::LD_F + 16 * jj, L::LD_F, -xo, lane);
        }
        block_sync();
      }
      // X (lower blocks) -> Xinv in the operand type
      for (int e = tid; e < 10 * 256; e += kThreads) {
        const int tile = e >> 8;
        const int ti = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
        const int tj = tile - tri_index(ti, 0);
        const int r = 16 * ti + ((e >> 4) & 15), c = 16 * tj + (e & 15);
        Xinv[r * L::LD_C + c] = from_f32<OpT>(X32[r * L::LD_F + c]);
      }
      block_sync();
    }

    // ===== P2: operands of the state products (region now holds the recurrence views)
    {
      const float eB0 = fast_exp2(gref0[w]), eB1 = fast_exp2(gref1[w]);               // e^{G_ref}
      const float eK0 = fast_exp2(glast0 - gref0[w]), eK1 = fast_exp2(glast1 - gref1[w]);  // e^{G_C-G_ref}
      OpT kb0[16], kb1[16], bv0[16], bv1[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int r = 16 * w + t;
        const float br = sbeta[r];
        const float e0 = E1a[t] * eB0, e1 = E1b[t] * eB1;
        store2<OpT>(Qt + r * L::LD_D + c0, rq[t].lo() * e0, rq[t].hi() * e1);
        store2<OpT>(nBKt + r * L::LD_D + c0, -br * rk[t].lo() * e0, -br * rk[t].hi() * e1);
        kb0[t] = from_f32<OpT>(rk[t].lo() * E2a[t] * eK0);
        kb1[t] = from_f32<OpT>(rk[t].hi() * E2b[t] * eK1);
        bv0[t] = from_f32<OpT>(br * rv[t].lo());
        bv1[t] = from_f32<OpT>(br * rv[t].hi());
      }
      // transposed rows: 16 consecutive tokens of one channel
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        KbT[c0 * L::LD_C + 16 * w + t] = kb0[t];
        KbT[(c0 + 1) * L::LD_C + 16 * w + t] = kb1[t];
      }
      if (has_v) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          BVT[c0 * L::LD_C + 16 * w + t] = bv0[t];
          BVT[(c0 + 1) * L::LD_C + 16 * w + t] = bv1[t];
        }
      }
      if (w == 0) {
        sgam[c0] = fast_exp2(glast0);
        sgam[c0 + 1] = fast_exp2(glast1);
      }
    }
    // raw registers are free: start loading the next chunk
    if (j + 1 < nchunks) prefetch(j + 1);
    block_sync();

    // ===== recurrence on this wave's value columns
    f32x4 accY[4][L::NVT], accO[4][L::NVT];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int vt = 0; vt < L::NVT; ++vt) {
        // Y starts at beta V: lane holds (s = 16 st + 4 g4 + i, v = local col)
        const int vc = vw - vblk + 16 * vt + l16;
        const OpT *src = BVT + vc * L::LD_C + 16 * st + 4 * g4;
#pragma unroll
        for (int i = 0; i < 4; ++i) accY[st][vt][i] = to_f32(src[i]);
        accO[st][vt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    // Y -= beta K~ S ; O = Q~ S   (S from registers as the Y operand)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      Frag<OpT> sf[L::NVT];
#pragma unroll
      for (int vt = 0; vt < L::NVT; ++vt) acc_frag_sk(sf[vt], S[2 * kk][vt], S[2 * kk + 1][vt]);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        Frag<OpT> xb, xq;
        lds_frag_sk(xb, nBKt, L::LD_D, 16 * st + l16, 32 * kk, g4);
        lds_frag_sk(xq, Qt, L::LD_D, 16 * st + l16, 32 * kk, g4);
#pragma unroll
        for (int vt = 0; vt < L::NVT; ++vt) {
          mma(accY[st][vt], xb, sf[vt]);
          mma(accO[st][vt], xq, sf[vt]);
        }
      }
    }
    // U = X Y
    Frag<OpT> yf[2][L::NVT];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int vt = 0; vt < L::NVT; ++vt)
        acc_frag_sk(yf[kk][vt], accY[2 * kk][vt], accY[2 * kk + 1][vt]);
    f32x4 accU[4][L::NVT];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int vt = 0; vt < L::NVT; ++vt) {
        accU[st][vt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk <= st / 2) {
            Frag<OpT> xi;
            lds_frag_sk(xi, Xinv, L::LD_C, 16 * st + l16, 32 * kk, g4);
            mma(accU[st][vt], xi, yf[kk][vt]);
          }
        }
      }
    Frag<OpT> uf[2][L::NVT];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int vt = 0; vt < L::NVT; ++vt)
        acc_frag_sk(uf[kk][vt], accU[2 * kk][vt], accU[2 * kk + 1][vt]);
    // O += P U
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk <= rt / 2) {
          Frag<OpT> xp;
          lds_frag_sk(xp, Pm, L::LD_C, 16 * rt + l16, 32 * kk, g4);
#pragma unroll
          for (int vt = 0; vt < L::NVT; ++vt) mma(accO[rt][vt], xp, uf[kk][vt]);
        }
      }
    // S <- Gamma S + Kbar^T U
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(sgam + 16 * ct + 4 * g4);
#pragma unroll
      for (int vt = 0; vt < L::NVT; ++vt) S[ct][vt] *= gm;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        Frag<OpT> xk;
        lds_frag_sk(xk, KbT, L::LD_C, 16 * ct + l16, 32 * kk, g4);
#pragma unroll
        for (int vt = 0; vt < L::NVT; ++vt) mma(S[ct][vt], xk, uf[kk][vt]);
      }
    }
    block_sync();

    // ===== output: stage O (scaled, io dtype) in LDS, then row-contiguous stores
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int vt = 0; vt < L::NVT; ++vt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Ost[(16 * rt + 4 * g4 + i) * L::LD_O + (vw - vblk) + 16 * vt + l16] =
              from_f32<OpT>(p.scale * accO[rt][vt][i]);
    block_sync();
    {
      constexpr int kVec = 16 / (int)sizeof(OpT);       // elements per 16-byte store
      constexpr int kPerRow = DV / kVec;                // stores per output row
      constexpr int kRowsPerPass = kThreads / kPerRow;
      const int col = (tid % kPerRow) * kVec;
      for (int r = tid / kPerRow; r < Lc; r += kRowsPerPass) {
        const int64_t tok = bos + (int64_t)j * kC + r;
        const f32x4 val = *reinterpret_cast<const f32x4 *>(Ost + r * L::LD_O + col);
        __builtin_nontemporal_store(
            val, reinterpret_cast<f32x4 *>(og + (tok * H + h) * kD + vblk + col));
      }
    }
    // (the next chunk's first barrier orders these LDS reads before its writes)
  }

  if (p.sfinal) {
    float *sf = p.sfinal + ((int64_t)n * H + h) * (kD * kD);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int vt = 0; vt < L::NVT; ++vt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sf[(16 * ct + 4 * g4 + i) * kD + vw + 16 * vt + l16] = S[ct][vt][i];
  }
}

// Longest-first order of the sequences of a packed batch (N <= 4096): one
// workgroup, bitonic sort of (chunks, index) keys in LDS.
__global__ __launch_bounds__(1024) void order_longest_first_kernel(const int32_t *__restrict__ cu,
                                                                   int32_t N,
                                                                   int32_t *__restrict__ order) {
  __shared__ uint64_t key[4096];
  int M = 1;
  while (M < N) M <<= 1;
  for (int i = threadIdx.x; i < M; i += blockDim.x) {
    // larger length first; ties keep the lower index first; padding sorts last
    uint64_t kv = ~0ull;
    if (i < N) {
      const uint32_t lenv = (uint32_t)(cu[i + 1] - cu[i]);
      kv = ((uint64_t)(0xffffffffu - lenv) << 32) | (uint32_t)i;
    }
    key[i] = kv;
  }
  __syncthreads();
  for (int size = 2; size <= M; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < M; i += blockDim.x) {
        const int jx = i ^ stride;
        if (jx > i) {
          const bool up = (i & size) == 0;
          const uint64_t a = key[i], b = key[jx];
          if ((a > b) == up) {
            key[i] = b;
            key[jx] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < N; i += blockDim.x) order[i] = (int32_t)(key[i] & 0xffffffffu);
}

template <class OpT, int DV>
hipError_t launch_typed(const ChunkParams &p, int64_t items, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_fwd_kernel<OpT, DV>), dim3((unsigned)items), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

kda_status plan_chunk_fwd(const kda_chunk_fwd_args &a, ChunkPlan *plan) {
  ChunkPlan pl;
  pl.num_seqs = a.num_seqs;
  pl.heads = a.num_heads;
  pl.varlen = a.cu_seqlens != nullptr;
  int64_t maxlen = 0;
  if (pl.varlen) {
    pl.total_tokens = a.cu_seqlens_host[a.num_seqs];
    for (int i = 0; i < a.num_seqs; ++i) {
      const int64_t l = (int64_t)a.cu_seqlens_host[i + 1] - a.cu_seqlens_host[i];
      if (l > maxlen) maxlen = l;
    }
  } else {
    pl.total_tokens = (int64_t)a.num_seqs * a.seq_len;
    maxlen = a.seq_len;
  }
  pl.max_chunks = (maxlen + KDA_CHUNK - 1) / KDA_CHUNK;
  pl.segments = 1;
  size_t off = 0;
  if (pl.varlen && a.num_seqs > 1 && a.num_seqs <= 4096) {
    pl.order_off = off;
    pl.order_bytes = (size_t)a.num_seqs * sizeof(int32_t);
    off += (pl.order_bytes + 255) & ~(size_t)255;
  }
  pl.total_bytes = off;
  *plan = pl;
  return KDA_SUCCESS;
}

hipError_t launch_chunk_fwd(const kda_chunk_fwd_args &a, const ChunkPlan &plan,
                            hipStream_t stream) {
  ChunkParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.g = a.g;
  p.beta = a.beta;
  p.s0 = a.initial_state;
  p.sfinal = a.final_state;
  p.o = a.o;
  p.cu = a.cu_seqlens;
  p.order = nullptr;
  p.total_tokens = plan.total_tokens;
  p.H = a.num_heads;
  p.seq_len = a.seq_len;
  p.scale = a.scale;
  if (plan.order_bytes) {
    int32_t *order = reinterpret_cast<int32_t *>((char *)a.workspace + plan.order_off);
    hipLaunchKernelGGL(order_longest_first_kernel, dim3(1), dim3(1024), 0, stream,
                       a.cu_seqlens, a.num_seqs, order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.order = order;
  }
  const int64_t chains = (int64_t)a.num_seqs * a.num_heads;
  if (a.io_dtype == KDA_BF16) return launch_typed<bf16, 128>(p, chains, stream);
  return launch_typed<float, 64>(p, chains * 2, stream);
}

}  // namespace kda
