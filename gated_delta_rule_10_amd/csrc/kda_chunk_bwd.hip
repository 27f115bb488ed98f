// kda_chunk_bwd.hip -- backward pass of the chunked KDA forward: dq, dk, dv, dg,
// dbeta and the initial-state gradient, for training.
//
// Pages (cited by title and section):
//  "How Kimi K3 Engineered Its Way to the Frontier", "How KDA updates its state"
//    (the recurrence: decay per key channel, erase + write, read) and "FlashKDA
//    steps the state once per 16 tokens" (the chunkwise form; FlashKDA itself is
//    forward-only).
//  "Kimi K3 -- Training and Infrastructure Notes", section 4.1 (the KDA kernels
//    serve training as well as inference prefill).
//
// The sequence is cut into 16-token sub-chunks.  For a sub-chunk with incoming
// state S (128 x 128), cumulative log-decays G_r = sum_{s<=r} g_s (natural log),
// and L <= 16 tokens:
//   Kt = k e^{G},  Qt = q e^{G},  Kb = k e^{G_last - G},  Gam = e^{G_last}
//   Ab_rs = sum_c k_rc k_sc e^{G_rc - G_sc} (s < r),  A = diag(beta) Ab
//   P_rs  = sum_c q_rc k_sc e^{G_rc - G_sc} (s <= r)
//   W = beta (V - Kt S),  U = (I + A)^{-1} W,  O = scale (Qt S + P U),
//   S_next = Gam S + Kb^T U.
// Every exponent is <= 0 (a cumulative decay, or a difference G_r - G_s with
// s <= r), so nothing overflows in fp32 for any decay; the matrix-core form of
// the e^{G_r - G_s} terms splits them at the sub-chunk's token 7 into two
// factors and is used only while those stay within e^60.  The backward of one
// sub-chunk, with dS the gradient of its outgoing state:
//   dU = scale P^T dO + Kb dS,   dW = (I + A)^{-T} dU,
//   dA = -tril(dW U^T, -1),      dP = scale tril(dO U^T),
//   dbeta_r = sum_v dW_rv (V - Kt S)_rv + sum_s dA_rs Ab_rs,   dV = beta dW,
//   dKt = -(beta dW) S^T,  dQt = scale dO S^T,  dKb = U dS^T,  dGam = rowsum(dS S),
//   dS_in = Gam dS + Kt^T (-beta dW) + Qt^T (scale dO),
// and dk, dq, dG follow from Kt, Qt, Kb, Gam and the e^{G_r - G_s} inside Ab and P;
// dg is the reverse cumulative sum of dG within the sub-chunk.
//
// Four launches:
//  0. prep: per (sub-chunk, head), fully parallel, the matrices that do not
//     depend on the state: Ab, P (matrix-core products of reference-scaled
//     operands, or one exponential per channel and pair where the decay range
//     is too wide) and X = (I + A)^{-1} (forward substitution), kept in the
//     workspace;
//  1. states: per (sequence, head, half of the value columns) the sub-chunk
//     forward from the initial state, writing the state at every sub-chunk
//     start to the workspace;
//  2. serial: per (sequence, head, half) the sub-chunks in reverse, the state
//     gradient carried in LDS; it writes dv and, for the terms that sum over
//     value columns, this half's partial sums to the workspace;
//  3. finalize: per (sub-chunk, head, half of the key channels) the two
//     value halves' partials summed and dq, dk, dg, dbeta formed (the
//     e^{G_r - G_s} terms again as reference-scaled matrix-core products, with
//     the same per-pair fallback).
// The 16 x 16 x K products run on fp32 matrix cores (V_MFMA_F32_16X16X4_F32).
// In the two serial passes eight waves share a sub-chunk: chains of products
// whose operands a wave produced itself (KS -> W -> U, dU -> dW) stay in
// registers in the matrix-core result layout, the rest go through LDS, and the
// next sub-chunk's inputs are loaded into registers while the current one is
// processed.
#include "kda_chunk_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kSC = 16;          // tokens per sub-chunk
constexpr int kNB = 2;           // value-column halves per chain
constexpr int kNC = kD / kNB;    // 64 value columns per workgroup
constexpr int kBT = 512;         // threads of the serial passes (8 waves)
constexpr int kPT = 256;         // threads of the prep pass
// LDS row strides of the serial passes: multiples of 4 floats, so a lane reads
// four consecutive k-values of a k-contiguous operand with one 16-byte load; 4
// mod 64 banks, so the 16 rows x 4 lane groups of a fragment read hit distinct
// banks in each 8-lane phase, and column reads (16 g4 + l16) do too.
constexpr int kLS = kNC + 4;     // row stride of the state halves
constexpr int kLT = kD + 4;      // row stride of 16 x 128 token matrices
constexpr int kLB = kNC + 4;     // row stride of 16 x 64 token blocks
constexpr int kLM = kSC + 1;     // row stride of 16 x 16 matrices (odd: column reads)

struct BwdParams {
  const void *q, *k, *v, *dO;
  const float *g, *beta, *s0, *dsf;
  float *dq, *dk, *dv, *dg, *dbeta, *ds0;
  const int32_t *cu;
  int64_t total_tokens;
  int64_t chains;   // (sequence, head) chains of this launch: sequences seq0 .. seq0 + chains / H
  int64_t slot0;    // sub-chunk slot of the launch's first sub-chunk (workspace origin)
  int32_t H, seq_len, seq0;
  float scale;
  float *ckpt;     // [slots][H][128][128] states at sub-chunk starts
  float *part;     // [slots][H][kNB][kPart] partial sums of the serial pass
  float *rec;      // [slots][H][kRec] Ab, P, X of the prep pass
};

// Per (sub-chunk, head) record of the prep pass (row-major 16 x 16 each).
constexpr int kRecAb = 0, kRecP = 256, kRecX = 512, kRec = 768;
// Partial sums one workgroup leaves for the finalize pass, per (sub-chunk, head, half).
constexpr int kPdA = 0, kPdP = 256, kPdB = 512, kPdKt = 528, kPdQt = kPdKt + 2048,
              kPdKb = kPdQt + 2048, kPdGam = kPdKb + 2048, kPart = kPdGam + 128;

// Sub-chunk slot of sub-chunk j of sequence n starting at token bos, relative
// to the launch's first: distinct for all (n, j) of the launch, below the slot
// count its workspace was laid out for (slot_count on the host).
__device__ __forceinline__ int64_t slot_of(const BwdParams &p, int64_t bos, int n, int j) {
  return bos / kSC + n + j - p.slot0;
}

__device__ __forceinline__ void seq_range(const BwdParams &p, int n, int64_t &bos, int64_t &len) {
  bos = (int64_t)n * p.seq_len;
  len = p.seq_len;
  if (p.cu) {  // device offsets, clamped to the validated token range
    const int64_t a = p.cu[n], b = p.cu[n + 1];
    bos = a < 0 ? 0 : (a > p.total_tokens ? p.total_tokens : a);
    const int64_t e = b < bos ? bos : (b > p.total_tokens ? p.total_tokens : b);
    len = e - bos;
  }
}

// Workgroups are dealt to the eight XCDs (each with its own L2) by block index
// mod 8.  A unit of work split into nb parts that read the same inputs gets
// blocks that share the index mod 8, so its parts meet in one L2: unit =
// (b / (8 nb)) 8 + b % 8, part = (b % (8 nb)) / 8.  The grid is rounded up
// to whole groups of 8 units; the surplus blocks return at once.
__device__ __forceinline__ void xcd_unit(int64_t b, int nb, int64_t &unit, int &part) {
  unit = (b / (8 * nb)) * 8 + b % 8;
  part = (int)((b % (8 * nb)) / 8);
}
inline int64_t xcd_grid(int64_t units, int nb) { return (units + 7) / 8 * 8 * nb; }

__device__ __forceinline__ int sub_len(int64_t len, int j) {
  const int64_t rest = len - (int64_t)j * kSC;
  return (int)(rest < kSC ? rest : kSC);
}

// acc += a b on fp32 matrix cores (V_MFMA_F32_16X16X4_F32): acc is a 16 x 16
// tile, lane (l16, g4) holding rows 4 g4 + i of column l16; per instruction
// lane (l16, g4) supplies A[l16][k] and B[k][l16] for its own k, so a 16-deep
// contraction is four instructions with k = 4 g4 + t (t = 0..3).
__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Element at a wave-uniform base plus a 32-bit per-lane byte offset: the
// address needs no 64-bit per-lane arithmetic (scalar base + vector offset).
template <class T>
__device__ __forceinline__ T at(const void *base, uint32_t byte_off) {
  return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}
template <class T>
__device__ __forceinline__ void put(void *base, uint32_t byte_off, T v) {
  *reinterpret_cast<T *>(reinterpret_cast<char *>(base) + byte_off) = v;
}
// Base of token t0, head h in a [T, H, 128] tensor of T_ elements.
template <class T_>
__device__ __forceinline__ const T_ *row_base(const void *x, int64_t t0, int64_t rowstride, int h) {
  return reinterpret_cast<const T_ *>(x) + t0 * rowstride + (int64_t)h * kD;
}

__device__ __forceinline__ f32x4 ld4(const float *p) {
  return *reinterpret_cast<const f32x4 *>(p);
}

// acc += A B over K (a multiple of 16), with A row m at a + m lda and B column
// n at b + n ldb both stored k-contiguous (16-byte aligned): four k-values per
// 16-byte LDS read.
__device__ __forceinline__ void mm4(f32x4 &acc, int K, int l16, int g4, const float *a, int lda,
                                    const float *b, int ldb) {
  const float *ar = a + l16 * lda + 4 * g4, *bc = b + l16 * ldb + 4 * g4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 16) {
    const f32x4 x = ld4(ar + k0), y = ld4(bc + k0);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = mfma(x[t], y[t], acc);
  }
}
// A k-contiguous as in mm4, B read by b(k, n); two accumulator chains.
template <class FB>
__device__ __forceinline__ void mmA4(f32x4 &acc, int K, int l16, int g4, const float *a, int lda,
                                     FB b) {
  const float *ar = a + l16 * lda + 4 * g4;
  f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    const f32x4 x = ld4(ar + k0), y = ld4(ar + k0 + 16);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc = mfma(x[t], b(k0 + 4 * g4 + t, l16), acc);
      acc2 = mfma(y[t], b(k0 + 16 + 4 * g4 + t, l16), acc2);
    }
  }
  acc += acc2;
}

// ---------------------------------------------------------------- 0. prep
// Workgroup per (sequence, head, j0): sub-chunks j0, j0 + stride, ...
// Ab and P on the matrix cores with the reference M = G at the sub-chunk's
// token 7: Ab_rs = sum_c (k_rc e^{G_rc - M_c}) (k_sc e^{M_c - G_sc}) and the same
// with q_r for P, exact up to rounding while every |G - M| stays within
// kRefSpan (each factor below e^60; masked entries may overflow and are
// discarded).  Otherwise every pair takes its own exponential per channel.
constexpr float kRefSpan = 60.f;
template <class IO>
__global__ __launch_bounds__(kPT) void bwd_prep_kernel(BwdParams p, int stride) {
  __shared__ __attribute__((aligned(16))) float kx[kSC * kLT], qx[kSC * kLT], G[kSC * kLT];
  __shared__ __attribute__((aligned(16))) float Ke[kSC * kLT], Kd[kSC * kLT], Qe[kSC * kLT];
  __shared__ float A[kSC * kLM], bt[kSC], tot[kD], wspan[kPT / 64];
  const int chain = p.seq0 * p.H + blockIdx.x / stride, j0 = blockIdx.x % stride;
  const int n = chain / p.H, h = chain % p.H;
  int64_t bos, len;
  seq_range(p, n, bos, len);
  const int t = threadIdx.x;
  const int c = t & (kD - 1), hh = t >> 7;  // channel; rows 8 hh .. 8 hh + 7
  const IO *q = reinterpret_cast<const IO *>(p.q), *k = reinterpret_cast<const IO *>(p.k);
  const int64_t rowstride = (int64_t)p.H * kD;
  const int nsub = (int)((len + kSC - 1) / kSC);
  for (int j = j0; j < nsub; j += stride) {
    const int64_t t0 = bos + (int64_t)j * kSC;
    const int L = sub_len(len, j);
    IO kv[8], qv[8];
    float gv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // unconditional loads (rows past L read row L - 1)
      const int64_t off = (t0 + min(8 * hh + i, L - 1)) * rowstride + (int64_t)h * kD + c;
      kv[i] = k[off];
      qv[i] = q[off];
      gv[i] = p.g[off];
    }
    const float bv = p.beta[(t0 + min(t & 15, L - 1)) * p.H + h];
    float gr[8];
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * hh + i;
      const bool live = r < L;
      kx[r * kLT + c] = live ? to_f32(kv[i]) : 0.f;
      qx[r * kLT + c] = live ? to_f32(qv[i]) : 0.f;
      a += live ? gv[i] : 0.f;
      gr[i] = a;
    }
    if (hh == 0) tot[c] = a;
    if (t < kSC) bt[t] = t < L ? bv : 0.f;
    block_sync();
    const float base = hh ? tot[c] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) G[(8 * hh + i) * kLT + c] = base + gr[i];
    {  // reference-scaled operands; the half-to-token-7 prefix of channel c is known here
      const float M = hh ? tot[c] : gr[7];  // G_7: the first half's total
      float span = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * hh + i;
        const float Gv = base + gr[i], d = Gv - M;
        const float up = __expf(d), dn = __expf(-d);
        const float kv_ = kx[r * kLT + c], qv_ = qx[r * kLT + c];
        Ke[r * kLT + c] = kv_ * up;
        Qe[r * kLT + c] = qv_ * up;
        Kd[r * kLT + c] = kv_ * dn;
        span = fmaxf(span, fabsf(d));
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) span = fmaxf(span, __shfl_xor(span, m));
      if ((t & 63) == 0) wspan[t >> 6] = span;
    }
    block_sync();
    float *rec = p.rec + (slot_of(p, bos, n, j) * p.H + h) * (int64_t)kRec;
    float maxspan = 0.f;
#pragma unroll
    for (int u = 0; u < kPT / 64; ++u) maxspan = fmaxf(maxspan, wspan[u]);
    if (maxspan <= kRefSpan) {  // waves 0 and 1: Ab and P tiles
      const int lane = t & 63, w = t >> 6, l16 = lane & 15, g4 = lane >> 4;
      if (w < 2) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        mm4(acc, kD, l16, g4, w == 0 ? Ke : Qe, kLT, Kd, kLT);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g4 + i, s = l16;
          if (w == 0) {
            const float ab = s < r ? acc[i] : 0.f;
            A[r * kLM + s] = bt[r] * ab;
            rec[kRecAb + r * kSC + s] = ab;
          } else {
            rec[kRecP + r * kSC + s] = s <= r ? acc[i] : 0.f;
          }
        }
      }
    } else {  // Ab and P: thread (r, s), every channel, with e^{G_rc - G_sc} (s <= r)
      const int r = t / kSC, s = t % kSC;
      float ab = 0.f, pp = 0.f;
      if (s <= r) {
        for (int cc = 0; cc < kD; ++cc) {
          const float e = __expf(G[r * kLT + cc] - G[s * kLT + cc]);
          const float ks = kx[s * kLT + cc] * e;
          ab = fmaf(kx[r * kLT + cc], ks, ab);
          pp = fmaf(qx[r * kLT + cc], ks, pp);
        }
      }
      ab = s < r ? ab : 0.f;
      A[r * kLM + s] = bt[r] * ab;
      rec[kRecAb + t] = ab;
      rec[kRecP + t] = pp;
    }
    block_sync();
    if (t < kSC) {  // X = (I + A)^{-1}, column t, by forward substitution
      float xc[kSC];
#pragma unroll
      for (int i = 0; i < kSC; ++i) {
        float x = i == t ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) x = fmaf(-A[i * kLM + m], xc[m], x);
        xc[i] = x;
        rec[kRecX + i * kSC + t] = x;
      }
    }
    block_sync();
  }
}

// Decay-weighted operands of one sub-chunk from the token inputs held in
// registers: thread (channel c, rows 4 qr .. 4 qr + 3) holds k, q and the
// inclusive prefix of g over its four rows; tot[qr][c] holds the row-quarter
// totals.  Writes Kt, Qt (if QT) and Kb rows and, for qr == 0, gam.
template <bool QT>
__device__ __forceinline__ void decay_operands(const float *kr, const float *qr_, const float *gp,
                                               const float *tot, int c, int qr, float *Kt,
                                               float *Qt, float *Kb, float *gam) {
  float base = 0.f, Gl = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float x = tot[u * kD + c];
    base += u < qr ? x : 0.f;
    Gl += x;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * qr + i;
    const float G = base + gp[i];
    const float eg = __expf(G), eb = __expf(Gl - G);
    Kt[r * kLT + c] = kr[i] * eg;
    if (QT) Qt[r * kLT + c] = qr_[i] * eg;
    Kb[r * kLT + c] = kr[i] * eb;
  }
  if (qr == 0) gam[c] = __expf(Gl);
}

// Prefetched loads are unconditional (rows past the sub-chunk's L valid tokens
// read its last token instead) and are masked where they are consumed, so no
// load sits in a branch that waits for it on the spot.

// Token inputs of one sub-chunk for thread (channel c, rows 4 qr + i), raw.
template <class IO, bool QT> struct TokRegs {
  IO k[4], q[QT ? 4 : 1];
  float g[4];
};
template <class IO, bool QT>
__device__ __forceinline__ void load_tokens(const BwdParams &p, int64_t t0, int L, int h, int c,
                                            int qr, TokRegs<IO, QT> &x) {
  const int64_t rowstride = (int64_t)p.H * kD;
  const IO *kb = row_base<IO>(p.k, t0, rowstride, h), *qb = row_base<IO>(p.q, t0, rowstride, h);
  const float *gb = row_base<float>(p.g, t0, rowstride, h);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t e = (uint32_t)(min(4 * qr + i, L - 1) * (int)rowstride + c);
    x.k[i] = at<IO>(kb, e * sizeof(IO));
    if (QT) x.q[i] = at<IO>(qb, e * sizeof(IO));
    x.g[i] = at<float>(gb, e * 4u);
  }
}
// Masked values: rows past L are zero.
template <class IO, bool QT>
__device__ __forceinline__ void take_tokens(const TokRegs<IO, QT> &x, int L, int qr, float *kr,
                                            float *qv, float *gr) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool live = 4 * qr + i < L;
    kr[i] = live ? to_f32(x.k[i]) : 0.f;
    if (QT) qv[i] = live ? to_f32(x.q[i]) : 0.f;
    gr[i] = live ? x.g[i] : 0.f;
  }
}

// A 16 x 16 tile of a [T, H, 128] tensor (columns col0 .. col0 + 15) in the
// matrix-core result layout: rows 4 g4 + i, column l16, raw.
template <class IO>
__device__ __forceinline__ void load_tile(const void *base, const BwdParams &p, int64_t t0, int L,
                                          int h, int col0, int l16, int g4, IO *x) {
  const int64_t rowstride = (int64_t)p.H * kD;
  const IO *b = row_base<IO>(base, t0, rowstride, h);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t e = (uint32_t)(min(4 * g4 + i, L - 1) * (int)rowstride + col0 + l16);
    x[i] = at<IO>(b, e * sizeof(IO));
  }
}
template <class IO>
__device__ __forceinline__ void take_tile(const IO *x, int L, int g4, float *y) {
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = 4 * g4 + i < L ? to_f32(x[i]) : 0.f;
}

struct StatesSmem {
  float S[kD * kLS];
  float Kt[2][kSC * kLT], Kb[2][kSC * kLT];  // by sub-chunk parity
  float U[kSC * kLB];
  float X[kSC * kLM];
  float beta[kSC];
  float gam[2][kD];
  float tot[4 * kD];
};

// ---------------------------------------------------------------- 1. states
// Per sub-chunk j, three barriers: A stage beta, X; C waves 0-3: KS = Kt S,
// W = beta (V - KS), U = X W for value tile w (registers), waves 4-7: the state
// checkpoint, every thread the decay totals of sub-chunk j + 1; D all eight:
// S <- Gam S + Kb^T U (wave w owns channel tile w) and the decay-weighted
// operands of sub-chunk j + 1 into the other LDS buffer.
template <class IO>
__global__ __launch_bounds__(kBT) void bwd_states_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) StatesSmem sm;
  int64_t unit;
  int blk;
  xcd_unit(blockIdx.x, kNB, unit, blk);
  if (unit >= p.chains) return;
  const int chain = p.seq0 * p.H + (int)unit;
  const int n = chain / p.H, h = chain % p.H;
  int64_t bos, len;
  seq_range(p, n, bos, len);
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, l16 = lane & 15, g4 = lane >> 4;
  const int c = t & (kD - 1), qr = t >> 7;
  for (int e = t; e < kD * kNC; e += kBT) {
    const int cc = e / kNC, vv = e % kNC;
    sm.S[cc * kLS + vv] = p.s0 ? p.s0[((int64_t)chain * kD + cc) * kD + blk * kNC + vv] : 0.f;
  }
  const int nsub = (int)((len + kSC - 1) / kSC);
  if (nsub == 0) return;
  // Registers in flight (unconditional loads; X and beta are written to LDS by
  // every thread, copies of equal values, so every thread consumes its loads):
  // tokens two sub-chunks ahead, beta and X one ahead, the v tile one ahead.
  TokRegs<IO, false> tok;
  IO vraw[4];
  float braw = 0.f, xr = 0.f;
  auto fetch_tokens = [&](int j) {
    load_tokens<IO, false>(p, bos + (int64_t)j * kSC, sub_len(len, j), h, c, qr, tok);
  };
  auto fetch_small = [&](int j) {
    const int64_t t0 = bos + (int64_t)j * kSC;
    braw = at<float>(p.beta + t0 * p.H + h, (uint32_t)(min(t & 15, sub_len(len, j) - 1) * p.H) * 4u);
    xr = at<float>(p.rec + (slot_of(p, bos, n, j) * p.H + h) * (int64_t)kRec + kRecX,
                   (uint32_t)(t & 255) * 4u);
  };
  auto fetch_v = [&](int j) {
    load_tile<IO>(p.v, p, bos + (int64_t)j * kSC, sub_len(len, j), h, blk * kNC + 16 * (w & 3),
                  l16, g4, vraw);
  };
  auto totals = [&](int L) {
    float kr[4], gr[4];
    take_tokens<IO, false>(tok, L, qr, kr, nullptr, gr);
    sm.tot[qr * kD + c] = (gr[0] + gr[1]) + (gr[2] + gr[3]);
  };
  auto operands = [&](int L, int b) {
    float kr[4], gr[4];
    take_tokens<IO, false>(tok, L, qr, kr, nullptr, gr);
#pragma unroll
    for (int i = 1; i < 4; ++i) gr[i] += gr[i - 1];
    decay_operands<false>(kr, nullptr, gr, sm.tot, c, qr, sm.Kt[b], nullptr, sm.Kb[b], sm.gam[b]);
  };
  // prologue: operands of sub-chunk 0 into buffer 0
  fetch_tokens(0);
  fetch_small(0);
  fetch_v(0);
  totals(sub_len(len, 0));
  block_sync();
  operands(sub_len(len, 0), 0);
  fetch_tokens(min(1, nsub - 1));
  for (int j = 0; j < nsub; ++j) {
    const int L = sub_len(len, j);
    const int b = j & 1;
    const int jn = min(j + 1, nsub - 1);  // next sub-chunk (the last one: itself, unused)
    const int Ln = sub_len(len, jn);
    // A: beta and X of this sub-chunk
    sm.beta[t & 15] = (t & 15) < L ? braw : 0.f;
    sm.X[((t & 255) >> 4) * kLM + (t & 15)] = xr;
    fetch_small(jn);  // unconditional: static wait counts
    block_sync();
    // C
    if (w < 4) {
      float vt[4];
      take_tile<IO>(vraw, L, g4, vt);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mmA4(acc, kD, l16, g4, sm.Kt[b], kLT,
           [&](int kk, int nn) { return sm.S[kk * kLS + 16 * w + nn]; });
      f32x4 wr;
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[i] = sm.beta[4 * g4 + i] * (vt[i] - acc[i]);
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) u = mfma(sm.X[l16 * kLM + 4 * g4 + tt], wr[tt], u);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.U[(4 * g4 + i) * kLB + 16 * w + l16] = u[i];
    } else {  // checkpoint of the state at this sub-chunk's start (16 lanes per row)
      float *ck = p.ckpt + (slot_of(p, bos, n, j) * p.H + h) * (int64_t)(kD * kD) + blk * kNC;
      const int tw = t - 256, col = 4 * (tw & 15);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int row = (tw >> 4) + 16 * m;
        *reinterpret_cast<f32x4 *>(ck + row * kD + col) = ld4(sm.S + row * kLS + col);
      }
    }
    fetch_v(jn);
    totals(Ln);  // of the next sub-chunk, for its operands in D
    block_sync();
    // D: S <- Gam S + Kb^T U, channel tile w, value tiles 0..3 (independent chains);
    // the next sub-chunk's operands into the other buffer
    operands(Ln, b ^ 1);
    fetch_tokens(min(j + 2, nsub - 1));  // unconditional: static wait counts
    {
      f32x4 acc[4];
      float kbv[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) kbv[tt] = sm.Kb[b][(4 * g4 + tt) * kLT + 16 * w + l16];
#pragma unroll
      for (int vtile = 0; vtile < 4; ++vtile)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cc = 16 * w + 4 * g4 + i;
          acc[vtile][i] = sm.gam[b][cc] * sm.S[cc * kLS + 16 * vtile + l16];
        }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int kk = 4 * g4 + tt;
#pragma unroll
        for (int vtile = 0; vtile < 4; ++vtile)
          acc[vtile] = mfma(kbv[tt], sm.U[kk * kLB + 16 * vtile + l16], acc[vtile]);
      }
#pragma unroll
      for (int vtile = 0; vtile < 4; ++vtile)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.S[(16 * w + 4 * g4 + i) * kLS + 16 * vtile + l16] = acc[vtile][i];
    }
    block_sync();
  }
}

struct SerialSmem {
  float S[kD * kLS];         // incoming state of the sub-chunk, this half's columns
  float dS[kD * kLS];        // state gradient
  float Kt[2][kSC * kLT], Qt[2][kSC * kLT], Kb[2][kSC * kLT];  // by sub-chunk parity
  float VmKS[kSC * kLB], U[kSC * kLB], dW[kSC * kLB], dOb[kSC * kLB];
  float P[kSC * kLM], X[kSC * kLM];
  float beta[kSC];
  float gam[2][kD];
  float tot[4 * kD];
};

// ---------------------------------------------------------------- 2. serial
// Per sub-chunk j, in reverse, three barriers: A stage S, beta, P, X; C waves
// 0-3: KS, W, U (value tile w), waves 4-7: dU = scale P^T dO + Kb dS,
// dW = X^T dU, dv (value tile w - 4), and every thread the decay totals of
// sub-chunk j - 1; D wave w, channel tile w: dKt, dQt, dKb, dGam partials and
// dS <- Gam dS + Kt^T (-beta dW) + Qt^T (scale dO), waves 0-2 also dA, dP and
// the W part of dbeta, and every thread the decay-weighted operands of
// sub-chunk j - 1 into the other LDS buffer (vector work in the shadow of the
// matrix-core chains).
template <class IO>
__global__ __launch_bounds__(kBT) void bwd_serial_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) SerialSmem sm;
  int64_t unit;
  int blk;
  xcd_unit(blockIdx.x, kNB, unit, blk);
  if (unit >= p.chains) return;
  const int chain = p.seq0 * p.H + (int)unit;
  const int n = chain / p.H, h = chain % p.H;
  int64_t bos, len;
  seq_range(p, n, bos, len);
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, l16 = lane & 15, g4 = lane >> 4;
  const int c = t & (kD - 1), qr = t >> 7;
  const float scale = p.scale;
  for (int e = t; e < kD * kNC; e += kBT) {
    const int cc = e / kNC, vv = e % kNC;
    sm.dS[cc * kLS + vv] = p.dsf ? p.dsf[((int64_t)chain * kD + cc) * kD + blk * kNC + vv] : 0.f;
  }
  const int nsub = (int)((len + kSC - 1) / kSC);
  if (nsub == 0) {  // empty sequence: dS0 = dS_final
    block_sync();
    if (p.ds0)
      for (int e = t; e < kD * kNC; e += kBT) {
        const int cc = e / kNC, vv = e % kNC;
        p.ds0[((int64_t)chain * kD + cc) * kD + blk * kNC + vv] = sm.dS[cc * kLS + vv];
      }
    return;
  }
  const int64_t rowstride = (int64_t)p.H * kD;
  // Registers in flight (unconditional loads, every thread consumes what it loads):
  // tokens of the next sub-chunk, its state / beta / P / X, the v or dO tile.
  TokRegs<IO, true> tok;
  IO vraw[4];
  float braw = 0.f, pr = 0.f;
  f32x4 sr[4];
  const int scol = 4 * (t & 15);  // state load: rows (t >> 4) + 32 m, columns scol..scol+3
  auto fetch_tokens = [&](int j) {
    load_tokens<IO, true>(p, bos + (int64_t)j * kSC, sub_len(len, j), h, c, qr, tok);
  };
  auto fetch_state = [&](int j) {
    const int64_t t0 = bos + (int64_t)j * kSC;
    const int L = sub_len(len, j);
    const int64_t slot = slot_of(p, bos, n, j);
    braw = at<float>(p.beta + t0 * p.H + h, (uint32_t)(min(t & 15, L - 1) * p.H) * 4u);
    const float *ck = p.ckpt + (slot * p.H + h) * (int64_t)(kD * kD) + blk * kNC;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      sr[m] = at<f32x4>(ck, (uint32_t)((((t >> 4) + 32 * m) * kD + scol) * 4));
    pr = at<float>(p.rec + (slot * p.H + h) * (int64_t)kRec + kRecP, (uint32_t)t * 4u);  // P, X
  };
  auto fetch_vd = [&](int j) {  // v tile (waves 0-3) or dO tile (waves 4-7)
    load_tile<IO>(w < 4 ? p.v : p.dO, p, bos + (int64_t)j * kSC, sub_len(len, j), h,
                  blk * kNC + 16 * (w & 3), l16, g4, vraw);
  };
  // decay totals of the tokens in `tok` (sub-chunk of length L) to sm.tot
  auto totals = [&](int L) {
    float kr[4], qv[4], gr[4];
    take_tokens<IO, true>(tok, L, qr, kr, qv, gr);
    sm.tot[qr * kD + c] = (gr[0] + gr[1]) + (gr[2] + gr[3]);
  };
  // decay-weighted operands of the tokens in `tok` into buffer b (after totals)
  auto operands = [&](int L, int b) {
    float kr[4], qv[4], gr[4];
    take_tokens<IO, true>(tok, L, qr, kr, qv, gr);
#pragma unroll
    for (int i = 1; i < 4; ++i) gr[i] += gr[i - 1];
    decay_operands<true>(kr, qv, gr, sm.tot, c, qr, sm.Kt[b], sm.Qt[b], sm.Kb[b], sm.gam[b]);
  };
  // prologue: operands of the last sub-chunk into buffer 0
  fetch_tokens(nsub - 1);
  fetch_state(nsub - 1);
  fetch_vd(nsub - 1);
  totals(sub_len(len, nsub - 1));
  block_sync();
  operands(sub_len(len, nsub - 1), 0);
  fetch_tokens(max(nsub - 2, 0));
  for (int j = nsub - 1; j >= 0; --j) {
    const int64_t t0 = bos + (int64_t)j * kSC;
    const int L = sub_len(len, j);
    const int64_t slot = slot_of(p, bos, n, j);
    const int b = (nsub - 1 - j) & 1;  // LDS buffer of this sub-chunk's operands
    const int jn = max(j - 1, 0);      // next sub-chunk (j = 0: sub-chunk 0 again, unused)
    const int Ln = sub_len(len, jn);
    // A: stage the state, beta, P, X
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<f32x4 *>(sm.S + ((t >> 4) + 32 * m) * kLS + scol) = sr[m];
    sm.beta[t & 15] = (t & 15) < L ? braw : 0.f;
    (t < 256 ? sm.P : sm.X)[((t >> 4) & 15) * kLM + (t & 15)] = pr;
    fetch_state(jn);  // unconditional: static wait counts
    block_sync();
    // C
    float vd[4];  // v tile (waves 0-3) or dO tile (waves 4-7)
    take_tile<IO>(vraw, L, g4, vd);
    if (w < 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mmA4(acc, kD, l16, g4, sm.Kt[b], kLT, [&](int kk, int nn) { return sm.S[kk * kLS + 16 * w + nn]; });
      f32x4 wr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = vd[i] - acc[i];
        sm.VmKS[(4 * g4 + i) * kLB + 16 * w + l16] = d;
        wr[i] = sm.beta[4 * g4 + i] * d;
      }
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) u = mfma(sm.X[l16 * kLM + 4 * g4 + tt], wr[tt], u);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.U[(4 * g4 + i) * kLB + 16 * w + l16] = u[i];
    } else {
      const int vt = w - 4;
      float *dvb = p.dv + t0 * rowstride + (int64_t)h * kD + blk * kNC;
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.dOb[(4 * g4 + i) * kLB + 16 * vt + l16] = vd[i];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc = mfma(scale * sm.P[(4 * g4 + tt) * kLM + l16], vd[tt], acc);
      mmA4(acc, kD, l16, g4, sm.Kb[b], kLT, [&](int kk, int nn) { return sm.dS[kk * kLS + 16 * vt + nn]; });
      f32x4 dw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) dw = mfma(sm.X[(4 * g4 + tt) * kLM + l16], acc[tt], dw);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i, col = 16 * vt + l16;
        sm.dW[r * kLB + col] = dw[i];
        if (r < L)  // dV = beta dW
          put<float>(dvb, (uint32_t)(r * (int)rowstride + col) * 4u, sm.beta[r] * dw[i]);
      }
    }
    fetch_vd(jn);
    totals(Ln);  // of sub-chunk jn, for its operands in D
    block_sync();
    // D
    float *part = p.part + ((slot * p.H + h) * kNB + blk) * (int64_t)kPart;
    const int ct = w;
    if (w == 0) {  // dA = -tril(dW U^T)
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mm4(acc, kNC, l16, g4, sm.dW, kLB, sm.U, kLB);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        put<float>(part, (uint32_t)(kPdA + r * kSC + l16) * 4u, l16 < r ? -acc[i] : 0.f);
      }
    } else if (w == 1) {  // dP = scale tril(dO U^T)
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mm4(acc, kNC, l16, g4, sm.dOb, kLB, sm.U, kLB);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        put<float>(part, (uint32_t)(kPdP + r * kSC + l16) * 4u, l16 <= r ? scale * acc[i] : 0.f);
      }
    } else if (w == 2) {  // dbeta, W part: sum_v dW (V - KS)
      float a = 0.f;
#pragma unroll
      for (int v4 = 0; v4 < 16; v4 += 4) {
        const f32x4 x = ld4(sm.dW + l16 * kLB + 16 * g4 + v4);
        const f32x4 y = ld4(sm.VmKS + l16 * kLB + 16 * g4 + v4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a = fmaf(x[e], y[e], a);
      }
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      if (g4 == 0) put<float>(part, (uint32_t)(kPdB + l16) * 4u, a);
    }
    // operands of the next sub-chunk into the other buffer, then its tokens' loads
    operands(Ln, b ^ 1);
    fetch_tokens(max(j - 2, 0));  // unconditional: static wait counts
    {  // dKt = -(beta dW) S^T, dQt = scale dO S^T, dKb = U dS^T: channel tile ct, one
       // k-loop with three independent chains (S read once for the first two)
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
      const float *sr_ = sm.S + (16 * ct + l16) * kLS + 4 * g4;
      const float *dsr = sm.dS + (16 * ct + l16) * kLS + 4 * g4;
      const int ao = l16 * kLB + 4 * g4;
#pragma unroll
      for (int k0 = 0; k0 < kNC; k0 += 16) {
        const f32x4 sv = ld4(sr_ + k0), dv_ = ld4(dsr + k0);
        const f32x4 xw = ld4(sm.dW + ao + k0), xo = ld4(sm.dOb + ao + k0), xu = ld4(sm.U + ao + k0);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          a0 = mfma(xw[tt], sv[tt], a0);
          a1 = mfma(xo[tt], sv[tt], a1);
          a2 = mfma(xu[tt], dv_[tt], a2);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t o = (uint32_t)((4 * g4 + i) * kD + 16 * ct + l16) * 4u;
        put<float>(part + kPdKt, o, -sm.beta[4 * g4 + i] * a0[i]);  // row factors -beta, scale
        put<float>(part + kPdQt, o, scale * a1[i]);
        put<float>(part + kPdKb, o, a2[i]);
      }
    }
    {  // dGam (before Gam) = rowsum(dS o S), channels of tile ct
      const int cc = 16 * ct + l16;
      float a = 0.f;
#pragma unroll
      for (int v4 = 0; v4 < 16; v4 += 4) {
        const f32x4 x = ld4(sm.dS + cc * kLS + 16 * g4 + v4), y = ld4(sm.S + cc * kLS + 16 * g4 + v4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a = fmaf(x[e], y[e], a);
      }
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      if (g4 == 0) put<float>(part, (uint32_t)(kPdGam + cc) * 4u, a);
    }
    // dS <- Gam dS + Kt^T (-beta dW) + Qt^T (scale dO): channel tile ct, value tiles 0..3
    // as four independent chains (this wave alone reads rows of tile ct of dS here)
    {
      f32x4 acc[4];
      float ktv[4], qtv[4], nb[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int kk = 4 * g4 + tt;
        ktv[tt] = sm.Kt[b][kk * kLT + 16 * ct + l16];
        qtv[tt] = sm.Qt[b][kk * kLT + 16 * ct + l16];
        nb[tt] = -sm.beta[kk];
      }
#pragma unroll
      for (int vtile = 0; vtile < 4; ++vtile) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cc = 16 * ct + 4 * g4 + i;
          acc[vtile][i] = sm.gam[b][cc] * sm.dS[cc * kLS + 16 * vtile + l16];
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int kk = 4 * g4 + tt;
#pragma unroll
        for (int vtile = 0; vtile < 4; ++vtile) {
          acc[vtile] = mfma(ktv[tt], nb[tt] * sm.dW[kk * kLB + 16 * vtile + l16], acc[vtile]);
          acc[vtile] = mfma(qtv[tt], scale * sm.dOb[kk * kLB + 16 * vtile + l16], acc[vtile]);
        }
      }
#pragma unroll
      for (int vtile = 0; vtile < 4; ++vtile)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.dS[(16 * ct + 4 * g4 + i) * kLS + 16 * vtile + l16] = acc[vtile][i];
    }
    block_sync();
  }
  if (p.ds0) {
    for (int e = t; e < kD * kNC; e += kBT) {
      const int cc = e / kNC, vv = e % kNC;
      p.ds0[((int64_t)chain * kD + cc) * kD + blk * kNC + vv] = sm.dS[cc * kLS + vv];
    }
  }
}

// ---------------------------------------------------------------- 3. finalize
// Workgroup of 256 threads per (sequence, head, j0, half of the key channels):
// sub-chunks j0, j0 + stride, ...  Wave w owns channel tile 4 half + w; lane
// (l16, g4) holds tokens 4 g4 + i of that tile's channel l16 (the matrix-core
// result layout).
//
// The Ab and P terms of dk, dq and dG are sums over token pairs weighted by
// e^{G_r - G_s}.  With the reference M = G at the sub-chunk's token 7 they are
// products of 16 x 16 matrices with 16 x 16 channel tiles:
//   dk_row = e^{G-M} o ((beta dA) (k e^{M-G})),   dq_row = e^{G-M} o (dP (k e^{M-G})),
//   dk_col = e^{M-G} o ((beta dA)^T (k e^{G-M}) + dP^T (q e^{G-M})),
//   dG    += k o dk_row + q o dq_row - k o dk_col,
// exact up to rounding while every |G - M| in the wave's tile stays within
// kRefSpan (each factor below e^60).  Otherwise the wave sums the pairs one by
// one, each with its own exponential.
constexpr int kFT = 256;

template <class IO>
__global__ __launch_bounds__(kFT) void bwd_finalize_kernel(BwdParams p, int stride) {
  constexpr int kFH = kD / 2;   // channels per workgroup
  constexpr int kLF = kFH + 4;  // LDS row stride
  __shared__ __attribute__((aligned(16))) float kx[kSC * kLF], qx[kSC * kLF], Gs[kSC * kLF];
  __shared__ float dA[kSC * kLM], dP[kSC * kLM], sb[kSC], tot[4 * kFH];
  int64_t unit;
  int half;
  xcd_unit(blockIdx.x, 2, unit, half);
  if (unit >= p.chains * stride) return;
  const int chain = p.seq0 * p.H + (int)(unit / stride), j0 = (int)(unit % stride);
  const int n = chain / p.H, h = chain % p.H;
  int64_t bos, len;
  seq_range(p, n, bos, len);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, l16 = lane & 15, g4 = lane >> 4;
  const int cl = t & (kFH - 1), hh = t >> 6;  // staging: channel cl, rows 4 hh .. 4 hh + 3
  const int cs = half * kFH + cl;
  const IO *q = reinterpret_cast<const IO *>(p.q), *k = reinterpret_cast<const IO *>(p.k);
  const int64_t rowstride = (int64_t)p.H * kD;
  const int nsub = (int)((len + kSC - 1) / kSC);
  for (int j = j0; j < nsub; j += stride) {
    const int64_t t0 = bos + (int64_t)j * kSC;
    const int L = sub_len(len, j);
    const int64_t slot = slot_of(p, bos, n, j);
    const float *pa = p.part + (slot * p.H + h) * kNB * (int64_t)kPart;
    // loads (unconditional: rows past L read row L - 1 and are masked at use)
    IO kv[4], qv[4];
    float gv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t off = (t0 + min(4 * hh + i, L - 1)) * rowstride + (int64_t)h * kD + cs;
      kv[i] = k[off];
      qv[i] = q[off];
      gv[i] = p.g[off];
    }
    const int e = t;  // element of dA, dP, Ab
    const float da_t = pa[kPdA + e] + pa[kPart + kPdA + e];
    const float dp_t = pa[kPdP + e] + pa[kPart + kPdP + e];
    const float bv = p.beta[(t0 + min(t & 15, L - 1)) * p.H + h];
    const float ab_t = p.rec[(slot * p.H + h) * (int64_t)kRec + kRecAb + e];
    const float db_t = pa[kPdB + (e >> 4)] + pa[kPart + kPdB + (e >> 4)];
    const int cc = 16 * w + l16, c = half * kFH + cc;  // local and global channel
    float pkt[4], pqt[4], pkb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = (4 * g4 + i) * kD + c;
      pkt[i] = pa[kPdKt + o] + pa[kPart + kPdKt + o];
      pqt[i] = pa[kPdQt + o] + pa[kPart + kPdQt + o];
      pkb[i] = pa[kPdKb + o] + pa[kPart + kPdKb + o];
    }
    const float pgam = pa[kPdGam + c] + pa[kPart + kPdGam + c];
    // stage k, q and the cumulative decay G (rows past L: zero, G constant)
    float gr[4], a = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * hh + i;
      const bool live = r < L;
      kx[r * kLF + cl] = live ? to_f32(kv[i]) : 0.f;
      qx[r * kLF + cl] = live ? to_f32(qv[i]) : 0.f;
      a += live ? gv[i] : 0.f;
      gr[i] = a;
    }
    tot[hh * kFH + cl] = a;
    dA[(e >> 4) * kLM + (e & 15)] = da_t;
    dP[(e >> 4) * kLM + (e & 15)] = dp_t;
    sb[t & 15] = (t & 15) < L ? bv : 0.f;
    {  // dbeta_rb = sum_v dW (V - KS) (both halves) + sum_{s<rb} dA_{rb s} Ab_{rb s}
      const int rb = e >> 4, s_ = e & 15;
      float x = s_ < rb ? da_t * ab_t : 0.f;
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m);
      if (half == 0 && s_ == 0 && rb < L) p.dbeta[(t0 + rb) * p.H + h] = x + db_t;
    }
    block_sync();
    {
      float base = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) base += u < hh ? tot[u * kFH + cl] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) Gs[(4 * hh + i) * kLF + cl] = base + gr[i];
    }
    block_sync();
    // per-lane operands of the pair products (shared by both tiles)
    float daA[4], dpA[4], daT[4], dpT[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int kk = 4 * g4 + tt;
      daA[tt] = dA[l16 * kLM + kk] * sb[l16];
      dpA[tt] = dP[l16 * kLM + kk];
      daT[tt] = dA[kk * kLM + l16] * sb[kk];
      dpT[tt] = dP[kk * kLM + l16];
    }
    float kr[4], qr[4], G[4], span = 0.f;
    const float M = Gs[7 * kLF + cc], Gl = Gs[(kSC - 1) * kLF + cc];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g4 + i;
      kr[i] = kx[r * kLF + cc];
      qr[i] = qx[r * kLF + cc];
      G[i] = Gs[r * kLF + cc];
      span = fmaxf(span, fabsf(G[i] - M));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) span = fmaxf(span, __shfl_xor(span, m));
    const bool fast = __builtin_amdgcn_readfirstlane(span <= kRefSpan ? 1 : 0) != 0;
    {
      float dk[4], dq[4], dG[4], tail = 0.f;
      float ekm[4];  // e^{G - M}
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float eg = __expf(G[i]), eb = __expf(Gl - G[i]);
        dk[i] = pkt[i] * eg + pkb[i] * eb;
        dq[i] = pqt[i] * eg;
        dG[i] = (pkt[i] * kr[i] + pqt[i] * qr[i]) * eg - pkb[i] * kr[i] * eb;
        tail += pkb[i] * kr[i] * eb;
        ekm[i] = __expf(G[i] - M);
      }
      if (fast) {
        f32x4 Kd, Ke, Qe;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float emk = __expf(M - G[i]);
          Kd[i] = kr[i] * emk;
          Ke[i] = kr[i] * ekm[i];
          Qe[i] = qr[i] * ekm[i];
        }
        f32x4 Rk = {0.f, 0.f, 0.f, 0.f}, Rq = Rk, Ck = Rk;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          Rk = mfma(daA[tt], Kd[tt], Rk);
          Rq = mfma(dpA[tt], Kd[tt], Rq);
          Ck = mfma(daT[tt], Ke[tt], Ck);
          Ck = mfma(dpT[tt], Qe[tt], Ck);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float row_k = ekm[i] * Rk[i], row_q = ekm[i] * Rq[i];
          const float col_k = __expf(M - G[i]) * Ck[i];
          dk[i] += row_k + col_k;
          dq[i] += row_q;
          dG[i] += kr[i] * (row_k - col_k) + qr[i] * row_q;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g4 + i;
          const float br = sb[r];
#pragma unroll 1
          for (int s_ = 0; s_ < kSC; ++s_) {
            const float Gx = Gs[s_ * kLF + cc], kxs = kx[s_ * kLF + cc];
            const float ex = __expf(s_ <= r ? G[i] - Gx : Gx - G[i]);  // <= 1 for g <= 0
            // pair (r, s_), s_ <= r
            const float da = s_ < r ? dA[r * kLM + s_] * br : 0.f;
            const float dp = s_ <= r ? dP[r * kLM + s_] : 0.f;
            // pair (s_, r), s_ >= r
            const float da2 = s_ > r ? dA[s_ * kLM + r] * sb[s_] : 0.f;
            const float dp2 = s_ >= r ? dP[s_ * kLM + r] : 0.f;
            const float row = (da * kr[i] + dp * qr[i]) * kxs;
            const float coef = da2 * kxs + dp2 * qx[s_ * kLF + cc];
            dk[i] += (da * kxs + coef) * ex;
            dq[i] += dp * kxs * ex;
            dG[i] += (row - coef * kr[i]) * ex;
          }
        }
      }
      // dg_r = sum_{s >= r} dG_s + (terms of the last row: every row's g reaches G_last)
      float suf[4];
      suf[3] = dG[3];
#pragma unroll
      for (int i = 2; i >= 0; --i) suf[i] = suf[i + 1] + dG[i];
      float above = 0.f;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const float x = __shfl(suf[0], l16 + 16 * gg);
        above += gg > g4 ? x : 0.f;
      }
      tail += __shfl_xor(tail, 16);
      tail += __shfl_xor(tail, 32);
      const float last = tail + pgam * __expf(Gl);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        if (r < L) {
          const int64_t off = (t0 + r) * rowstride + (int64_t)h * kD + c;
          p.dq[off] = dq[i];
          p.dk[off] = dk[i];
          p.dg[off] = suf[i] + above + last;
        }
      }
    }
    block_sync();
  }
}

template <class IO>
hipError_t launch_typed(const BwdParams &p, int64_t chains, int stride, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_prep_kernel<IO>, dim3((unsigned)(chains * stride)), dim3(kPT), 0, stream,
                     p, stride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_states_kernel<IO>, dim3((unsigned)xcd_grid(chains, kNB)), dim3(kBT), 0,
                     stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_serial_kernel<IO>, dim3((unsigned)xcd_grid(chains, kNB)), dim3(kBT), 0,
                     stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_finalize_kernel<IO>, dim3((unsigned)xcd_grid(chains * stride, 2)),
                     dim3(kFT), 0, stream, p, stride);
  return hipGetLastError();
}

struct WorkspaceLayout {
  size_t ck, part, rec, total;
};

WorkspaceLayout layout(int64_t total_tokens, int32_t num_seqs, int32_t heads) {
  const int64_t slots = total_tokens / kSC + num_seqs + 1;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WorkspaceLayout l;
  l.ck = 0;
  l.part = up((size_t)slots * heads * kD * kD * sizeof(float));
  l.rec = l.part + up((size_t)slots * heads * kNB * kPart * sizeof(float));
  l.total = l.rec + (size_t)slots * heads * kRec * sizeof(float);
  return l;
}

// Token range of sequence n (host side: cu_seqlens_host, or the fixed length).
struct Span {
  int64_t bos, len;
};
Span span_of(const kda_chunk_bwd_args &a, int32_t n) {
  if (a.cu_seqlens) return {a.cu_seqlens_host[n], (int64_t)a.cu_seqlens_host[n + 1] - a.cu_seqlens_host[n]};
  return {(int64_t)n * a.seq_len, a.seq_len};
}
// Workspace of sequences n0 .. n1 - 1 run in one launch: with bos0 their first
// token and T their tokens, every relative slot (bos / 16 - bos0 / 16) + (n - n0)
// + j stays below T / 16 + (n1 - n0) + 1.
size_t group_bytes(const kda_chunk_bwd_args &a, int32_t n0, int32_t n1) {
  const Span f = span_of(a, n0), l = span_of(a, n1 - 1);
  return layout(l.bos + l.len - f.bos, n1 - n0, a.num_heads).total;
}

}  // namespace

// Workspace: sub-chunk slots T_total / 16 + N + 1, each holding H states
// (64 KiB), H x 2 partial-sum records and H prep records.
size_t chunk_bwd_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t heads) {
  return layout(total_tokens, num_seqs, heads).total;
}

// The smallest workspace the backward runs in: the largest single sequence's.
size_t chunk_bwd_min_workspace_bytes(const kda_chunk_bwd_args &a) {
  size_t m = 0;
  for (int32_t n = 0; n < a.num_seqs; ++n) {
    const size_t b = group_bytes(a, n, n + 1);
    if (b > m) m = b;
  }
  return m;
}

// Sequences are independent, so a workspace smaller than the whole pack's is
// used for consecutive groups of sequences, each as large as fits, one launch
// sequence (prep, states, serial, finalize) per group.
hipError_t launch_chunk_bwd(const kda_chunk_bwd_args &a, int64_t total_tokens, int64_t max_sub,
                            hipStream_t stream) {
  (void)max_sub;
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.dO = a.dO;
  p.g = a.g;
  p.beta = a.beta;
  p.s0 = a.initial_state;
  p.dsf = a.dfinal_state;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.dg = a.dg;
  p.dbeta = a.dbeta;
  p.ds0 = a.dinitial_state;
  p.cu = a.cu_seqlens;
  p.total_tokens = total_tokens;
  p.H = a.num_heads;
  p.seq_len = a.seq_len;
  p.scale = a.scale;
  char *ws = reinterpret_cast<char *>(a.workspace);
  for (int32_t n0 = 0; n0 < a.num_seqs;) {
    int32_t n1 = n0 + 1;
    while (n1 < a.num_seqs && group_bytes(a, n0, n1 + 1) <= a.workspace_bytes) ++n1;
    const Span f = span_of(a, n0);
    const WorkspaceLayout l = layout(span_of(a, n1 - 1).bos + span_of(a, n1 - 1).len - f.bos,
                                     n1 - n0, a.num_heads);
    p.ckpt = reinterpret_cast<float *>(ws + l.ck);
    p.part = reinterpret_cast<float *>(ws + l.part);
    p.rec = reinterpret_cast<float *>(ws + l.rec);
    p.seq0 = n0;
    p.slot0 = f.bos / kSC + n0;
    p.chains = (int64_t)(n1 - n0) * a.num_heads;
    int64_t ms = 1;
    for (int32_t n = n0; n < n1; ++n) {
      const int64_t sub = (span_of(a, n).len + kSC - 1) / kSC;
      if (sub > ms) ms = sub;
    }
    const int stride = (int)(ms > 64 ? 64 : ms);
    const hipError_t e = a.io_dtype == KDA_BF16
                             ? launch_typed<bf16>(p, p.chains, stride, stream)
                             : launch_typed<float>(p, p.chains, stride, stream);
    if (e != hipSuccess) return e;
    n0 = n1;
  }
  return hipSuccess;
}

}  // namespace kda
