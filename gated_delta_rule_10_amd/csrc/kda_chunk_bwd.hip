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
// s <= r), so nothing overflows in fp32 for any decay.  The backward of one
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
//     depend on the state: Ab, P (one exponential per channel and pair) and
//     X = (I + A)^{-1} (forward substitution), kept in the workspace;
//  1. states: per (sequence, head, half of the value columns) the sub-chunk
//     forward from the initial state, writing the state at every sub-chunk
//     start to the workspace;
//  2. serial: per (sequence, head, half) the sub-chunks in reverse, the state
//     gradient carried in LDS; it writes dv and, for the terms that sum over
//     value columns, this half's partial sums to the workspace;
//  3. finalize: per (sub-chunk, head) the two halves' partials summed and dq,
//     dk, dg, dbeta formed (the e^{G_r - G_s} terms one channel per thread).
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
constexpr int kLS = kNC + 1;     // row stride of the state halves (odd: no bank conflicts)
constexpr int kLT = kD + 1;      // row stride of 16 x 128 token matrices
constexpr int kLB = kNC + 1;     // row stride of 16 x 64 token blocks
constexpr int kLM = kSC + 1;     // row stride of 16 x 16 matrices

struct BwdParams {
  const void *q, *k, *v, *dO;
  const float *g, *beta, *s0, *dsf;
  float *dq, *dk, *dv, *dg, *dbeta, *ds0;
  const int32_t *cu;
  int64_t total_tokens, chains;
  int32_t H, seq_len;
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

// Sub-chunk slot of sub-chunk j of a sequence starting at token bos: distinct
// for all (sequence n, j), below T_total / 16 + N + 1.
__device__ __forceinline__ int64_t slot_of(int64_t bos, int n, int j) {
  return bos / kSC + n + j;
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

// acc (a 16 x 16 tile; lane holds rows 4 g4 + i, column l16) += sum_{k<K} A(m, k) B(k, n)
// for K a multiple of 16, on fp32 matrix cores; a(m, k) and b(k, n) read the operands.
template <class FA, class FB>
__device__ __forceinline__ void mm(f32x4 &acc, int K, int l16, int g4, FA a, FB b) {
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kk = k0 + 4 * g4 + t;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(l16, kk), b(kk, l16), acc, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// ---------------------------------------------------------------- 0. prep
// Workgroup per (sequence, head, j0): sub-chunks j0, j0 + stride, ...
template <class IO>
__global__ __launch_bounds__(kPT) void bwd_prep_kernel(BwdParams p, int stride) {
  __shared__ float kx[kSC * kLT], qx[kSC * kLT], G[kSC * kLT], A[kSC * kLM], bt[kSC], tot[kD];
  const int chain = blockIdx.x / stride, j0 = blockIdx.x % stride;
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
    block_sync();
    float *rec = p.rec + (slot_of(bos, n, j) * p.H + h) * (int64_t)kRec;
    {  // Ab and P: thread (r, s), every channel, with e^{G_rc - G_sc} (s <= r)
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
  const IO *q = reinterpret_cast<const IO *>(p.q), *k = reinterpret_cast<const IO *>(p.k);
  const int64_t rowstride = (int64_t)p.H * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(4 * qr + i, L - 1);
    const int64_t off = (t0 + r) * rowstride + (int64_t)h * kD + c;
    x.k[i] = k[off];
    if (QT) x.q[i] = q[off];
    x.g[i] = p.g[off];
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
  const IO *b = reinterpret_cast<const IO *>(base);
  const int64_t rowstride = (int64_t)p.H * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(4 * g4 + i, L - 1);
    x[i] = b[(t0 + r) * rowstride + (int64_t)h * kD + col0 + l16];
  }
}
template <class IO>
__device__ __forceinline__ void take_tile(const IO *x, int L, int g4, float *y) {
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = 4 * g4 + i < L ? to_f32(x[i]) : 0.f;
}

struct StatesSmem {
  float S[kD * kLS];
  float Kt[kSC * kLT], Kb[kSC * kLT];
  float U[kSC * kLB];
  float X[kSC * kLM];
  float beta[kSC];
  float gam[kD];
  float tot[4 * kD];
};

// ---------------------------------------------------------------- 1. states
// Waves 0-3: KS = Kt S, W = beta (V - KS), U = X W for value tile w (registers);
// waves 4-7: the state checkpoint.  Then all eight: S <- Gam S + Kb^T U, wave w
// owning channel tile w.
template <class IO>
__global__ __launch_bounds__(kBT) void bwd_states_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) StatesSmem sm;
  int64_t unit;
  int blk;
  xcd_unit(blockIdx.x, kNB, unit, blk);
  if (unit >= p.chains) return;
  const int chain = (int)unit;
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
  // registers for the sub-chunk about to be processed (raw, masked at use)
  TokRegs<IO, false> tok;
  IO vraw[4];
  // Every thread consumes what it loads (X and beta are written to LDS by all
  // threads, copies of equal values), so no wave is left with loads it never
  // waits for.
  float braw = 0.f, xr = 0.f;
  auto fetch = [&](int j) {
    const int64_t t0 = bos + (int64_t)j * kSC;
    const int L = sub_len(len, j);
    load_tokens<IO, false>(p, t0, L, h, c, qr, tok);
    braw = p.beta[(t0 + min(t & 15, L - 1)) * p.H + h];
    xr = p.rec[(slot_of(bos, n, j) * p.H + h) * (int64_t)kRec + kRecX + (t & 255)];
  };
  auto fetch_v = [&](int j) {
    load_tile<IO>(p.v, p, bos + (int64_t)j * kSC, sub_len(len, j), h, blk * kNC + 16 * (w & 3),
                  l16, g4, vraw);
  };
  if (nsub > 0) {
    fetch(0);
    fetch_v(0);
  }
  for (int j = 0; j < nsub; ++j) {
    const int L = sub_len(len, j);
    float kr[4], gr[4];
    take_tokens<IO, false>(tok, L, qr, kr, nullptr, gr);
    // A: small matrices and the decay totals
    sm.beta[t & 15] = (t & 15) < L ? braw : 0.f;
    sm.X[((t & 255) >> 4) * kLM + (t & 15)] = xr;
#pragma unroll
    for (int i = 1; i < 4; ++i) gr[i] += gr[i - 1];
    sm.tot[qr * kD + c] = gr[3];
    block_sync();
    // B: decay-weighted operands; next sub-chunk's tokens in flight
    decay_operands<false>(kr, nullptr, gr, sm.tot, c, qr, sm.Kt, nullptr, sm.Kb, sm.gam);
    fetch(min(j + 1, nsub - 1));  // unconditional: static wait counts
    block_sync();
    // C
    if (w < 4) {
      float vt[4];
      take_tile<IO>(vraw, L, g4, vt);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mm(acc, kD, l16, g4, [&](int m, int kk) { return sm.Kt[m * kLT + kk]; },
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
      float *ck = p.ckpt + (slot_of(bos, n, j) * p.H + h) * (int64_t)(kD * kD) + blk * kNC;
      const int tw = t - 256, col = 4 * (tw & 15);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int row = (tw >> 4) + 16 * m;
        f32x4 s;
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = sm.S[row * kLS + col + e];
        *reinterpret_cast<f32x4 *>(ck + row * kD + col) = s;
      }
    }
    fetch_v(min(j + 1, nsub - 1));
    block_sync();
    // D: S <- Gam S + Kb^T U, channel tile w, value tiles 0..3
#pragma unroll 1
    for (int vtile = 0; vtile < 4; ++vtile) {
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cc = 16 * w + 4 * g4 + i;
        acc[i] = sm.gam[cc] * sm.S[cc * kLS + 16 * vtile + l16];
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int kk = 4 * g4 + tt;
        acc = mfma(sm.Kb[kk * kLT + 16 * w + l16], sm.U[kk * kLB + 16 * vtile + l16], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.S[(16 * w + 4 * g4 + i) * kLS + 16 * vtile + l16] = acc[i];
    }
    block_sync();
  }
}

struct SerialSmem {
  float S[kD * kLS];         // incoming state of the sub-chunk, this half's columns
  float dS[kD * kLS];        // state gradient
  float Kt[kSC * kLT], Qt[kSC * kLT], Kb[kSC * kLT];
  float VmKS[kSC * kLB], U[kSC * kLB], dW[kSC * kLB], dOb[kSC * kLB];
  float P[kSC * kLM], X[kSC * kLM];
  float beta[kSC];
  float gam[kD];
  float tot[4 * kD];
};

// ---------------------------------------------------------------- 2. serial
// Per sub-chunk, in reverse: A stage inputs; B decay-weighted operands;
// C waves 0-3: KS, W, U (value tile w), waves 4-7: dU = scale P^T dO + Kb dS,
// dW = X^T dU, dv (value tile w - 4); D wave w, channel tile w: dKt, dQt, dKb,
// dGam partials and dS <- Gam dS + Kt^T (-beta dW) + Qt^T (scale dO); waves 0-2
// also dA, dP and the W part of dbeta.
template <class IO>
__global__ __launch_bounds__(kBT) void bwd_serial_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) SerialSmem sm;
  int64_t unit;
  int blk;
  xcd_unit(blockIdx.x, kNB, unit, blk);
  if (unit >= p.chains) return;
  const int chain = (int)unit;
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
  const int64_t rowstride = (int64_t)p.H * kD;
  TokRegs<IO, true> tok;
  IO vraw[4];
  float braw = 0.f, pr = 0.f;  // consumed by every thread (as in the states pass)
  f32x4 sr[4];
  const int scol = 4 * (t & 15);  // state load: rows (t >> 4) + 32 m, columns scol..scol+3
  auto fetch = [&](int j) {
    const int64_t t0 = bos + (int64_t)j * kSC;
    const int L = sub_len(len, j);
    const int64_t slot = slot_of(bos, n, j);
    load_tokens<IO, true>(p, t0, L, h, c, qr, tok);
    braw = p.beta[(t0 + min(t & 15, L - 1)) * p.H + h];
    const float *ck = p.ckpt + (slot * p.H + h) * (int64_t)(kD * kD) + blk * kNC;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      sr[m] = *reinterpret_cast<const f32x4 *>(ck + ((t >> 4) + 32 * m) * kD + scol);
    pr = p.rec[(slot * p.H + h) * (int64_t)kRec + kRecP + t];  // P (t < 256), X
  };
  auto fetch_vd = [&](int j) {  // v tile (waves 0-3) or dO tile (waves 4-7)
    load_tile<IO>(w < 4 ? p.v : p.dO, p, bos + (int64_t)j * kSC, sub_len(len, j), h,
                  blk * kNC + 16 * (w & 3), l16, g4, vraw);
  };
  if (nsub > 0) {
    fetch(nsub - 1);
    fetch_vd(nsub - 1);
  }
  for (int j = nsub - 1; j >= 0; --j) {
    const int64_t t0 = bos + (int64_t)j * kSC;
    const int L = sub_len(len, j);
    const int64_t slot = slot_of(bos, n, j);
    float kr[4], qv[4], gr[4];
    take_tokens<IO, true>(tok, L, qr, kr, qv, gr);
    // A: stage the state, dO, beta, P, X and the decay totals
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = (t >> 4) + 32 * m;
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.S[row * kLS + scol + e] = sr[m][e];
    }
    sm.beta[t & 15] = (t & 15) < L ? braw : 0.f;
    (t < 256 ? sm.P : sm.X)[((t >> 4) & 15) * kLM + (t & 15)] = pr;
#pragma unroll
    for (int i = 1; i < 4; ++i) gr[i] += gr[i - 1];
    sm.tot[qr * kD + c] = gr[3];
    block_sync();
    // B
    decay_operands<true>(kr, qv, gr, sm.tot, c, qr, sm.Kt, sm.Qt, sm.Kb, sm.gam);
    fetch(max(j - 1, 0));  // unconditional: static wait counts
    block_sync();
    // C
    float vd[4];  // v tile (waves 0-3) or dO tile (waves 4-7)
    take_tile<IO>(vraw, L, g4, vd);
    if (w < 4) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mm(acc, kD, l16, g4, [&](int m, int kk) { return sm.Kt[m * kLT + kk]; },
         [&](int kk, int nn) { return sm.S[kk * kLS + 16 * w + nn]; });
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
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.dOb[(4 * g4 + i) * kLB + 16 * vt + l16] = vd[i];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc = mfma(scale * sm.P[(4 * g4 + tt) * kLM + l16], vd[tt], acc);
      mm(acc, kD, l16, g4, [&](int m, int kk) { return sm.Kb[m * kLT + kk]; },
         [&](int kk, int nn) { return sm.dS[kk * kLS + 16 * vt + nn]; });
      f32x4 dw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) dw = mfma(sm.X[(4 * g4 + tt) * kLM + l16], acc[tt], dw);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i, col = 16 * vt + l16;
        sm.dW[r * kLB + col] = dw[i];
        if (r < L)  // dV = beta dW
          p.dv[(t0 + r) * rowstride + (int64_t)h * kD + blk * kNC + col] = sm.beta[r] * dw[i];
      }
    }
    fetch_vd(max(j - 1, 0));
    block_sync();
    // D
    float *part = p.part + ((slot * p.H + h) * kNB + blk) * (int64_t)kPart;
    const int ct = w;
    if (w == 0) {  // dA = -tril(dW U^T)
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mm(acc, kNC, l16, g4, [&](int m, int kk) { return sm.dW[m * kLB + kk]; },
         [&](int kk, int nn) { return sm.U[nn * kLB + kk]; });
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        part[kPdA + r * kSC + l16] = l16 < r ? -acc[i] : 0.f;
      }
    } else if (w == 1) {  // dP = scale tril(dO U^T)
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mm(acc, kNC, l16, g4, [&](int m, int kk) { return sm.dOb[m * kLB + kk]; },
         [&](int kk, int nn) { return sm.U[nn * kLB + kk]; });
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        part[kPdP + r * kSC + l16] = l16 <= r ? scale * acc[i] : 0.f;
      }
    } else if (w == 2) {  // dbeta, W part: sum_v dW (V - KS)
      float a = 0.f;
#pragma unroll
      for (int vv = 0; vv < 16; ++vv)
        a = fmaf(sm.dW[l16 * kLB + 16 * g4 + vv], sm.VmKS[l16 * kLB + 16 * g4 + vv], a);
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      if (g4 == 0) part[kPdB + l16] = a;
    }
    {  // dKt = -(beta dW) S^T, dQt = scale dO S^T, dKb = U dS^T: channel tile ct
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
      mm(a0, kNC, l16, g4, [&](int m, int kk) { return -sm.beta[m] * sm.dW[m * kLB + kk]; },
         [&](int kk, int nn) { return sm.S[(16 * ct + nn) * kLS + kk]; });
      mm(a1, kNC, l16, g4, [&](int m, int kk) { return scale * sm.dOb[m * kLB + kk]; },
         [&](int kk, int nn) { return sm.S[(16 * ct + nn) * kLS + kk]; });
      mm(a2, kNC, l16, g4, [&](int m, int kk) { return sm.U[m * kLB + kk]; },
         [&](int kk, int nn) { return sm.dS[(16 * ct + nn) * kLS + kk]; });
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = (4 * g4 + i) * kD + 16 * ct + l16;
        part[kPdKt + o] = a0[i];
        part[kPdQt + o] = a1[i];
        part[kPdKb + o] = a2[i];
      }
    }
    {  // dGam (before Gam) = rowsum(dS o S), channels of tile ct
      const int cc = 16 * ct + l16;
      float a = 0.f;
#pragma unroll
      for (int vv = 0; vv < 16; ++vv)
        a = fmaf(sm.dS[cc * kLS + 16 * g4 + vv], sm.S[cc * kLS + 16 * g4 + vv], a);
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      if (g4 == 0) part[kPdGam + cc] = a;
    }
    // dS <- Gam dS + Kt^T (-beta dW) + Qt^T (scale dO): channel tile ct, value tiles 0..3
    // (this wave alone reads rows of tile ct of dS in this stage)
#pragma unroll 1
    for (int vtile = 0; vtile < 4; ++vtile) {
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cc = 16 * ct + 4 * g4 + i;
        acc[i] = sm.gam[cc] * sm.dS[cc * kLS + 16 * vtile + l16];
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int kk = 4 * g4 + tt;
        acc = mfma(sm.Kt[kk * kLT + 16 * ct + l16],
                   -sm.beta[kk] * sm.dW[kk * kLB + 16 * vtile + l16], acc);
        acc = mfma(sm.Qt[kk * kLT + 16 * ct + l16], scale * sm.dOb[kk * kLB + 16 * vtile + l16],
                   acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.dS[(16 * ct + 4 * g4 + i) * kLS + 16 * vtile + l16] = acc[i];
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
// Workgroup of 512 threads per (sequence, head, j0, quarter of the key
// channels): sub-chunks j0, j0 + stride, ...; thread (row r, channel c) forms
// dq, dk, dg of token r, channel c.  The Ab and P terms: row r's pairs
// (r, s <= r) and the pairs (s >= r, r) in which token r is the earlier one,
// each with its own e^{G_r - G_s} <= 1.  LDS is double-buffered by sub-chunk
// parity, so three barriers per sub-chunk suffice.
constexpr int kFC = 32;  // key channels per finalize workgroup
constexpr int kFT = kFC * kSC;

struct FinSmem {
  float dA[kSC * kSC], dP[kSC * kSC], sb[kSC];
  float kx[kSC][kFC], qx[kSC][kFC], gx[kSC][kFC], Gs[kSC][kFC], dGs[kSC][kFC], tl[kSC][kFC];
};

template <class IO>
__global__ __launch_bounds__(kFT) void bwd_finalize_kernel(BwdParams p, int stride) {
  int64_t unit;
  int quarter;
  xcd_unit(blockIdx.x, kD / kFC, unit, quarter);
  if (unit >= p.chains * stride) return;
  const int chain = (int)(unit / stride), j0 = (int)(unit % stride), c0 = quarter * kFC;
  const int n = chain / p.H, h = chain % p.H;
  int64_t bos, len;
  seq_range(p, n, bos, len);
  const int t = threadIdx.x, cl = t % kFC, r = t / kFC, c = c0 + cl;
  const IO *q = reinterpret_cast<const IO *>(p.q), *k = reinterpret_cast<const IO *>(p.k);
  const int64_t rowstride = (int64_t)p.H * kD;
  __shared__ FinSmem smb[2];
  const int nsub = (int)((len + kSC - 1) / kSC);
  // Loads of one sub-chunk, issued one sub-chunk ahead (unconditional: rows past
  // L read row L - 1 and are masked at use; every thread consumes what it loads).
  struct In {
    IO k, q;
    float g, dkt[2], dqt[2], dkb[2], da[2], dp[2], db[2], dgam[2], ab, beta;
  } in;
  const int o = r * kD + c;
  auto fetch = [&](int j) {
    const int64_t t0 = bos + (int64_t)j * kSC;
    const int L = sub_len(len, j);
    const float *pa = p.part + (slot_of(bos, n, j) * p.H + h) * kNB * (int64_t)kPart;
    const int64_t off = (t0 + min(r, L - 1)) * rowstride + (int64_t)h * kD + c;
    in.k = k[off];
    in.q = q[off];
    in.g = p.g[off];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      in.dkt[b] = pa[b * kPart + kPdKt + o];
      in.dqt[b] = pa[b * kPart + kPdQt + o];
      in.dkb[b] = pa[b * kPart + kPdKb + o];
      in.da[b] = pa[b * kPart + kPdA + (t & 255)];
      in.dp[b] = pa[b * kPart + kPdP + (t & 255)];
      in.db[b] = pa[b * kPart + kPdB + ((t >> 4) & 15)];
      in.dgam[b] = pa[b * kPart + kPdGam + c];
    }
    in.ab = p.rec[(slot_of(bos, n, j) * p.H + h) * (int64_t)kRec + kRecAb + (t & 255)];
    in.beta = p.beta[(t0 + min(t & 15, L - 1)) * p.H + h];
  };
  if (j0 < nsub) fetch(j0);
  int parity = 0;
  for (int j = j0; j < nsub; j += stride, parity ^= 1) {
    FinSmem &sm = smb[parity];
    const int64_t t0 = bos + (int64_t)j * kSC;
    const int L = sub_len(len, j);
    const bool live = r < L;
    const int64_t off = (t0 + r) * rowstride + (int64_t)h * kD + c;
    const float kr = live ? to_f32(in.k) : 0.f, qv = live ? to_f32(in.q) : 0.f;
    sm.kx[r][cl] = kr;
    sm.qx[r][cl] = qv;
    sm.gx[r][cl] = live ? in.g : 0.f;
    const float dKt = in.dkt[0] + in.dkt[1];
    const float dQt = in.dqt[0] + in.dqt[1];
    const float dKb = in.dkb[0] + in.dkb[1];
    sm.dA[t & 255] = in.da[0] + in.da[1];  // equal copies from both halves of the threads
    sm.dP[t & 255] = in.dp[0] + in.dp[1];
    sm.sb[t & 15] = (t & 15) < L ? in.beta : 0.f;
    const float ab = in.ab, db = in.db[0] + in.db[1], dgs = in.dgam[0] + in.dgam[1];
    fetch(j + stride < nsub ? j + stride : j);  // unconditional: static wait counts
    block_sync();
    float Gr = 0.f, Gl = 0.f;
#pragma unroll
    for (int s = 0; s < kSC; ++s) {
      const float x = sm.gx[s][cl];
      Gr += s <= r ? x : 0.f;
      Gl += x;
    }
    sm.Gs[r][cl] = Gr;
    {  // dbeta_rb = sum_v dW (V - KS) (both halves) + sum_{s<rb} dA_{rb s} Ab_{rb s}:
       // 16 lanes per row rb (every wave computes; the first quarter's waves 0-3 store)
      const int rb = (t >> 4) & 15, sb_ = t & 15;
      float a = sb_ < rb ? sm.dA[rb * kSC + sb_] * ab : 0.f;
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) a += __shfl_xor(a, m);
      if (c0 == 0 && t < kSC * kSC && sb_ == 0 && rb < L)
        p.dbeta[(t0 + rb) * p.H + h] = a + db;
    }
    block_sync();
    const float eg = __expf(Gr), eb = __expf(Gl - Gr);
    float dk = dKt * eg + dKb * eb, dq = dQt * eg;
    float dG = (dKt * kr + dQt * qv) * eg - dKb * kr * eb;
    const float br = sm.sb[r];
#pragma unroll
    for (int s = 0; s < kSC; ++s) {
      const float Gx = sm.Gs[s][cl], kxs = sm.kx[s][cl];
      if (s <= r) {  // pair (r, s): Ab_rs and P_rs
        const float e = __expf(Gr - Gx);
        const float da = s < r ? sm.dA[r * kSC + s] * br : 0.f, dp = sm.dP[r * kSC + s];
        dk = fmaf(da * kxs, e, dk);
        dq = fmaf(dp * kxs, e, dq);
        dG = fmaf((da * kr + dp * qv) * kxs, e, dG);
      }
      if (s >= r) {  // pair (s, r): token r is the earlier one
        const float e = __expf(Gx - Gr);
        const float da = s > r ? sm.dA[s * kSC + r] * sm.sb[s] : 0.f, dp = sm.dP[s * kSC + r];
        const float coef = (da * kxs + dp * sm.qx[s][cl]) * e;
        dk += coef;
        dG = fmaf(-coef, kr, dG);
      }
    }
    sm.dGs[r][cl] = dG;
    sm.tl[r][cl] = dKb * kr * eb;  // through G_last: belongs to the last row's dG
    block_sync();
    // dg_r = sum_{s >= r} dG_s + (terms of the last row, which every row's g reaches)
    float dg = dgs * __expf(Gl);
#pragma unroll
    for (int s = 0; s < kSC; ++s) dg += (s >= r ? sm.dGs[s][cl] : 0.f) + sm.tl[s][cl];
    if (live) {
      p.dq[off] = dq;
      p.dk[off] = dk;
      p.dg[off] = dg;
    }
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
  hipLaunchKernelGGL(bwd_finalize_kernel<IO>, dim3((unsigned)xcd_grid(chains * stride, kD / kFC)),
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

}  // namespace

// Workspace: sub-chunk slots T_total / 16 + N + 1, each holding H states
// (64 KiB), H x 2 partial-sum records and H prep records.
size_t chunk_bwd_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t heads) {
  return layout(total_tokens, num_seqs, heads).total;
}

hipError_t launch_chunk_bwd(const kda_chunk_bwd_args &a, int64_t total_tokens, int64_t max_sub,
                            hipStream_t stream) {
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
  const WorkspaceLayout l = layout(total_tokens, a.num_seqs, a.num_heads);
  char *ws = reinterpret_cast<char *>(a.workspace);
  p.ckpt = reinterpret_cast<float *>(ws + l.ck);
  p.part = reinterpret_cast<float *>(ws + l.part);
  p.rec = reinterpret_cast<float *>(ws + l.rec);
  const int64_t chains = (int64_t)a.num_seqs * a.num_heads;
  p.chains = chains;
  const int stride = (int)(max_sub < 1 ? 1 : (max_sub > 64 ? 64 : max_sub));
  if (chains == 0) return hipSuccess;
  return a.io_dtype == KDA_BF16 ? launch_typed<bf16>(p, chains, stride, stream)
                                : launch_typed<float>(p, chains, stride, stream);
}

}  // namespace kda
