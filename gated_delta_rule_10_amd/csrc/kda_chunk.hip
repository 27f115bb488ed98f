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
#include <queue>
#include <vector>
#include <type_traits>

#include "kda_chunk_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

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
  static constexpr int NRW = DV / 16;                    // waves running the recurrence
  static_assert(NRW <= kWaves, "value block too wide");
  // EARLY (bf16): the transposed operands Kbar^T and (beta V)^T get buffers of
  // their own and are written with the Gram operands, so the raw inputs are
  // dead -- and the next chunk's loads can be issued -- before the Gram
  // products start.  fp32 operands do not leave room for that; there they
  // share the region and are written after the inverse.
  static constexpr bool EARLY = sizeof(OpT) == 2;
  // Region R: phases reuse the same bytes.
  //  Gram:       Kr[64][LD_KH], Qr[64][LD_KH], Kc[160][LD_KH]                 (OpT)
  //  recurrence: nBKt[64][LD_D], Qt[64][LD_D] (+ KbT[128][LD_C], BVT[DV][LD_C] unless EARLY)
  //  output:     Ost[64][LD_O]                                               (OpT)
  static constexpr size_t kGram = (size_t)(64 + 64 + 160) * LD_KH * sizeof(OpT);
  static constexpr size_t kKV = ((size_t)128 * LD_C + (size_t)DV * LD_C) * sizeof(OpT);
  static constexpr size_t kRec = (size_t)2 * 64 * LD_D * sizeof(OpT) + (EARLY ? 0 : kKV);
  static constexpr size_t kOut = (size_t)64 * LD_O * sizeof(OpT);
  static constexpr size_t kGramOut = kGram > kOut ? kGram : kOut;
  static constexpr size_t kRegion = kGramOut > kRec ? kGramOut : kRec;
  static constexpr size_t kKVOff = EARLY ? kRegion : 2 * 64 * LD_D * sizeof(OpT);
  static constexpr size_t kAfterKV = EARLY ? kRegion + kKV : kRegion;
  // half-sub-tile totals and first values of the log-decay ([2][8][128] fp32):
  // inside the region when the recurrence view leaves room past the Gram view
  static constexpr size_t kHalf = (size_t)2 * kWaves * 128 * 4;
  static constexpr bool kHalfInRegion = kRegion - kGramOut >= kHalf;
  static constexpr size_t kHalfOff = kHalfInRegion ? kGramOut : kAfterKV;
  static constexpr size_t kAfterRegion = kHalfInRegion ? kAfterKV : kAfterKV + kHalf;
  // Lm: the unit-lower-triangular system, -A in the strictly lower 16x16 blocks
  // and the inverse of each diagonal block on the diagonal; Pm: the P matrix.
  static constexpr size_t kLm = (size_t)64 * LD_C * sizeof(OpT);
  static constexpr size_t kP = kLm;
  static constexpr size_t kSmall = (size_t)(64 + 128 + 4 * 128) * 4;
  static constexpr size_t kTotal = kAfterRegion + kLm + kP + kSmall;
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
__device__ __forceinline__ void raw_load(Raw<float> &r, __amdgpu_buffer_rsrc_t rs, uint32_t off,
                                         uint32_t soff) {
  r.f = buf_load_f32x2(rs, off, soff);
}
template <class OpT> __device__ __forceinline__ void raw_zero(Raw<OpT> &r);
template <> __device__ __forceinline__ void raw_zero(Raw<float> &r) { r.f = f32x2{0.f, 0.f}; }

// Gram jobs of waves 4..7: (kind, row tile i, column tile j), kind 0 = A, 1 = P.
// Waves 0..3 compute A of the diagonal tile (w, w) in both orientations and its
// inverse; waves 4..7 compute P of the diagonal tiles and A, P of the six
// off-diagonal tiles.
__device__ __forceinline__ void gram_job(int jw, int u, int &kind, int &i, int &j) {
  // rows: [P00 A10 P10 A20] [P11 P20 A21 P21] [P22 A30 P30 A31] [P33 P31 A32 P32]
  const int code[4][4] = {{0x100, 0x010, 0x110, 0x020},
                          {0x111, 0x120, 0x021, 0x121},
                          {0x122, 0x030, 0x130, 0x031},
                          {0x133, 0x131, 0x032, 0x132}};
  const int c = code[jw][u];
  kind = c >> 8;
  i = (c >> 4) & 15;
  j = c & 15;
}

// GATE: g holds gate logits of the lower-bounded gate, applied as a chunk's
// log-decay is summed (gate_log2).
template <class OpT, int DV, bool GATE>
__global__ __launch_bounds__(kThreads) void chunk_fwd_kernel(ChunkParams p) {
  typedef Layout<OpT, DV> L;
  constexpr int VS = kD / DV;  // value blocks per head
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::kTotal];

  unsigned char *region = smem;
  float *htot = reinterpret_cast<float *>(smem + L::kHalfOff);  // [8][128]
  float *hfirst = htot + kWaves * 128;                          // [8][128]
  OpT *Lm = reinterpret_cast<OpT *>(smem + L::kAfterRegion);
  OpT *Pm = reinterpret_cast<OpT *>(smem + L::kAfterRegion + L::kLm);
  float *sbeta = reinterpret_cast<float *>(smem + L::kAfterRegion + L::kLm + L::kP);
  float *sgam = sbeta + 64;
  float *eBt = sgam + 128;  // [4][128] e^{G_ref} per sub-tile and channel

  // Gram phase views
  OpT *Kr = reinterpret_cast<OpT *>(region);
  OpT *Qr = Kr + 64 * L::LD_KH;
  OpT *Kc = Qr + 64 * L::LD_KH;
  // recurrence phase views.  With a single Gram pass (bf16), -beta K~ and Q~ are
  // rescalings of Kr and Qr in place: nBKt aliases Kr and Qt aliases Qr.
  OpT *nBKt = reinterpret_cast<OpT *>(region);
  OpT *Qt = nBKt + 64 * L::LD_D;
  OpT *KbT = reinterpret_cast<OpT *>(smem + L::kKVOff);
  OpT *BVT = KbT + 128 * L::LD_C;
  constexpr bool kInPlace = L::NH == 1 && L::LD_D == L::LD_KH;
  // output staging
  OpT *Ost = reinterpret_cast<OpT *>(region);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int st = w >> 1;  // elementwise: 16-token sub-tile of this wave
  const int th = w & 1;   //              and its half (tokens 8 th .. 8 th + 7)

  // ---- work item: (sequence rank, head, segment item, value block)
  const ChunkItem itm = decode_item(p, VS);
  if (itm.skip) return;  // uniform: the whole workgroup
  const int vs = itm.vs, h = itm.h;
  const int64_t bos = itm.bos, len = itm.len;
  const float *s0p = itm.s0;
  float *sfp = itm.sf;
  const bool write_o = itm.write_o;
  const bool zero_v = itm.zero_v;  // M = the map of the incoming state: v = 0, S0 = I
  const int nchunks = (int)((len + kC - 1) / kC);
  const int H = p.H;
  const int64_t rowstride = (int64_t)H * kD;  // elements between consecutive tokens
  const int vblk = vs * DV;                   // first value column of this workgroup
  const int vloc = 16 * w;                    // recurrence: this wave's columns (local)
  const bool rec_wave = w < L::NRW;

  const OpT *__restrict__ qg = reinterpret_cast<const OpT *>(p.q) + (int64_t)h * kD;
  const OpT *__restrict__ kg = reinterpret_cast<const OpT *>(p.k) + (int64_t)h * kD;
  const OpT *__restrict__ vg = reinterpret_cast<const OpT *>(p.v) + (int64_t)h * kD + vblk;
  const float *__restrict__ gg = p.g + (int64_t)h * kD;
  OpT *__restrict__ og = reinterpret_cast<OpT *>(p.o) + (int64_t)h * kD + vblk;

  // One-time zero of the strictly-upper blocks (0,1) and (2,3) of P, which the
  // 32-wide k-steps of the P U product read.
  for (int e = tid; e < 2 * 256; e += kThreads) {
    const int b = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
    Pm[(32 * b + rr) * L::LD_C + skpos(32 * b + 16 + cc)] = from_f32<OpT>(0.f);
  }

  // ---- state (fp32 accumulators) of the recurrence waves:
  //      S[ct] holds S[16 ct + 4 g4 + i][vblk + vloc + l16]
  f32x4 S[8];
  {
    const float *s0 = rec_wave ? s0p : nullptr;
    const int col = vblk + vloc + l16;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * ct + 4 * g4 + i;
        S[ct][i] = s0 ? s0[row * kD + col] : (zero_v && row == col ? 1.f : 0.f);
      }
  }

  // ---- register prefetch of a chunk's raw inputs: wave w = tokens
  //      16 st + 8 th + t (t < 8); lane = channels 2 lane, 2 lane + 1 (value
  //      channels vblk + 2 lane; lanes < 32 cover the 64 columns when DV = 64).
  Raw<OpT> rq[8], rk[8], rv[8];
  f32x2 rg[8];
  float rb = 0.f;
  const int c0 = 2 * lane;
  const bool has_v = (DV == 128) || (lane < 32);  // this lane's value columns exist
  const uint32_t lane_off_qk = (uint32_t)c0 * (uint32_t)sizeof(OpT);  // byte offsets
  const uint32_t lane_off_g = (uint32_t)c0 * 4u;
  const uint32_t row_qk = (uint32_t)rowstride * (uint32_t)sizeof(OpT);  // bytes per token
  const uint32_t row_g = (uint32_t)rowstride * 4u;
  // next-chunk descriptors (scalar registers) and valid-row count
  __amdgpu_buffer_rsrc_t rq_s, rk_s, rv_s, rg_s;
  uint32_t nv = 0;
  auto prefetch_begin = [&](int j) {
    const int64_t t0 = bos + (int64_t)j * kC + 16 * st + 8 * th;  // uniform
    const int64_t rem = bos + len - t0;
    nv = rem <= 0 ? 0u : (rem >= 8 ? 8u : (uint32_t)rem);  // valid rows
    // descriptors cover exactly this wave's valid rows of its head
    rq_s = make_rsrc(qg + t0 * rowstride, nv * row_qk);
    rk_s = make_rsrc(kg + t0 * rowstride, nv * row_qk);
    rv_s = make_rsrc(vg + t0 * rowstride, (has_v && !zero_v) ? nv * row_qk : 0u);
    rg_s = make_rsrc(gg + t0 * rowstride, nv * row_g);
    rb = (lane < 8 && (uint32_t)lane < nv) ? p.beta[(t0 + lane) * H + h] : 0.f;
    if (p.beta_logits && lane < 8 && (uint32_t)lane < nv) rb = sigmoid_fast(rb);
  };
  auto prefetch_row = [&](int t) {
    if ((uint32_t)t < nv) {
      // row offsets are uniform: they go in the scalar offset of the instruction
      const uint32_t so_qk = __builtin_amdgcn_readfirstlane(t * row_qk);
      const uint32_t so_g = __builtin_amdgcn_readfirstlane(t * row_g);
      raw_load(rq[t], rq_s, lane_off_qk, so_qk);
      raw_load(rk[t], rk_s, lane_off_qk, so_qk);
      raw_load(rv[t], rv_s, lane_off_qk, so_qk);  // reads as zero outside the descriptor
      rg[t] = buf_load_f32x2(rg_s, lane_off_g, so_g);
    } else {
      raw_zero(rq[t]); raw_zero(rk[t]); raw_zero(rv[t]);
      rg[t] = f32x2{0.f, 0.f};
    }
  };
  auto prefetch = [&](int j) {
    prefetch_begin(j);
#pragma unroll
    for (int t = 0; t < 8; ++t) prefetch_row(t);
  };
  if (nchunks > 0) prefetch(0);
  // gate constants: the head's factor and the bias of this lane's two channels
  float gate_a = 0.f, gate_dt0 = 0.f, gate_dt1 = 0.f;
  if constexpr (GATE) {
    gate_a = gate_head_factor(p.A_log[h]);
    if (p.dt_bias) {
      gate_dt0 = p.dt_bias[h * kD + c0];
      gate_dt1 = p.dt_bias[h * kD + c0 + 1];
    }
  }

  for (int j = 0; j < nchunks; ++j) {
    const int Lc = (int)((len - (int64_t)j * kC) < kC ? (len - (int64_t)j * kC) : kC);

    // ===== P0: per-channel cumulative log2-decay over this wave's 8 tokens
    float Gl0[8], Gl1[8];
    {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if constexpr (GATE) {  // rows past the sequence end keep log-decay 0
          if (16 * st + 8 * th + t < Lc) {
            a0 += gate_log2(rg[t][0], gate_a, gate_dt0, p.gate_scale);
            a1 += gate_log2(rg[t][1], gate_a, gate_dt1, p.gate_scale);
          }
        } else {
          a0 += rg[t][0] * kLog2e;
          a1 += rg[t][1] * kLog2e;
        }
        Gl0[t] = a0;
        Gl1[t] = a1;
      }
      *reinterpret_cast<f32x2 *>(htot + w * 128 + c0) = f32x2{a0, a1};
      *reinterpret_cast<f32x2 *>(hfirst + w * 128 + c0) = f32x2{Gl0[0], Gl1[0]};
      if (lane < 8) sbeta[16 * st + 8 * th + lane] = rb;
    }
    block_sync();

    // chunk-relative G at each sub-tile's reference token (its token 8), G(last),
    // and this half's offset from its sub-tile start
    float gref0[4], gref1[4], glast0 = 0.f, glast1 = 0.f, gmid0 = 0.f, gmid1 = 0.f;
    float hoff0 = 0.f, hoff1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 t0v = *reinterpret_cast<const f32x2 *>(htot + (2 * i) * 128 + c0);
      const f32x2 t1v = *reinterpret_cast<const f32x2 *>(htot + (2 * i + 1) * 128 + c0);
      const f32x2 f1v = *reinterpret_cast<const f32x2 *>(hfirst + (2 * i + 1) * 128 + c0);
      const float m0 = t0v[0] + f1v[0], m1 = t0v[1] + f1v[1];  // sub-tile relative
      gref0[i] = glast0 + m0;
      gref1[i] = glast1 + m1;
      if (i == st) {
        gmid0 = m0;
        gmid1 = m1;
        hoff0 = th ? t0v[0] : 0.f;
        hoff1 = th ? t0v[1] : 0.f;
      }
      glast0 += t0v[0] + t1v[0];
      glast1 += t0v[1] + t1v[1];
    }
    // E1 = e^{G_t - G_ref} (row factor), E2 = e^{G_ref - G_t} (column factor)
    float E1a[8], E1b[8], E2a[8], E2b[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float d0 = hoff0 + Gl0[t] - gmid0, d1 = hoff1 + Gl1[t] - gmid1;
      E1a[t] = fast_exp2(d0);
      E1b[t] = fast_exp2(d1);
      E2a[t] = fast_exp2(-d0);
      E2b[t] = fast_exp2(-d1);
    }

    // Kbar^T (rows = channels) and (beta V)^T (rows = value columns), 8
    // consecutive tokens per row: Kbar = k e^{G_C - G} = k E2 e^{G_C - G_ref}
    auto write_kv = [&](const float *e2a, const float *e2b) {
      const float eK0 = fast_exp2(glast0 - gref0[st]);
      const float eK1 = fast_exp2(glast1 - gref1[st]);
      float kb0[8], kb1[8], bv0[8], bv1[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float br = sbeta[16 * st + 8 * th + t];
        kb0[t] = rk[t].lo() * e2a[t] * eK0;
        kb1[t] = rk[t].hi() * e2b[t] * eK1;
        bv0[t] = br * rv[t].lo();
        bv1[t] = br * rv[t].hi();
      }
      const int tc = 16 * st + 8 * th;
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4) {
        store4<OpT>(KbT + c0 * L::LD_C + skpos(tc + 4 * q4),
                    f32x4{kb0[4 * q4], kb0[4 * q4 + 1], kb0[4 * q4 + 2], kb0[4 * q4 + 3]});
        store4<OpT>(KbT + (c0 + 1) * L::LD_C + skpos(tc + 4 * q4),
                    f32x4{kb1[4 * q4], kb1[4 * q4 + 1], kb1[4 * q4 + 2], kb1[4 * q4 + 3]});
        if (has_v) {
          store4<OpT>(BVT + c0 * L::LD_C + tc + 4 * q4,
                      f32x4{bv0[4 * q4], bv0[4 * q4 + 1], bv0[4 * q4 + 2], bv0[4 * q4 + 3]});
          store4<OpT>(BVT + (c0 + 1) * L::LD_C + tc + 4 * q4,
                      f32x4{bv1[4 * q4], bv1[4 * q4 + 1], bv1[4 * q4 + 2], bv1[4 * q4 + 3]});
        }
      }
    };

    // ===== P1 + Gram
    f32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hc = 0; hc < L::NH; ++hc) {
      if (c0 / L::KH == hc) {
        const int cc = c0 - hc * L::KH;
        float F0[4], F1[4];  // e^{G_ref(i) - G_ref(st)} for i > st
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          F0[i] = i > st ? fast_exp2(gref0[i] - gref0[st]) : 1.f;
          F1[i] = i > st ? fast_exp2(gref1[i] - gref1[st]) : 1.f;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int r = 16 * st + 8 * th + t;
          const float k0 = rk[t].lo(), k1 = rk[t].hi();
          const float q0 = rq[t].lo(), q1 = rq[t].hi();
          // columns in split-k order (the Gram products sum over channels, so a
          // permutation shared by all three operands leaves them unchanged)
          const int pc = skpos(cc);
          store2<OpT>(Kr + r * L::LD_KH + pc, k0 * E1a[t], k1 * E1b[t]);
          store2<OpT>(Qr + r * L::LD_KH + pc, q0 * E1a[t], q1 * E1b[t]);
          const float b0 = k0 * E2a[t], b1 = k1 * E2b[t];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i >= st)
              store2<OpT>(Kc + (tri_index(i, st) * 16 + 8 * th + t) * L::LD_KH + pc, b0 * F0[i],
                          b1 * F1[i]);
        }
      }
      if (L::EARLY) {
        write_kv(E2a, E2b);
        if (th == 0)
          *reinterpret_cast<f32x2 *>(eBt + st * 128 + c0) =
              f32x2{fast_exp2(gref0[st]), fast_exp2(gref1[st])};
        if (w == 0)
          *reinterpret_cast<f32x2 *>(sgam + c0) = f32x2{fast_exp2(glast0), fast_exp2(glast1)};
        // raw registers are dead: start loading the next chunk
        if (j + 1 < nchunks) prefetch(j + 1);
      }
      block_sync();
      if (w < 4) {
        // A_ww as [r][s] (acc[0]) and [s][r] (acc[1])
        const OpT *krw = Kr + 16 * w * L::LD_KH;
        const OpT *kcw = Kc + tri_index(w, w) * 16 * L::LD_KH;
#pragma unroll
        for (int kk = 0; kk < L::KH / 32; ++kk) {
          Frag<OpT> fk, fc;
          lds_frag_ck(fk, krw, L::LD_KH, l16, 32 * kk, g4);
          lds_frag_ck(fc, kcw, L::LD_KH, l16, 32 * kk, g4);
          mma(acc[0], fk, fc);
          mma(acc[1], fc, fk);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int kind, ti, tj;
          gram_job(w - 4, u, kind, ti, tj);
          const OpT *xs = Kc + tri_index(ti, tj) * 16 * L::LD_KH;
          const OpT *ys = (kind ? Qr : Kr) + 16 * ti * L::LD_KH;
#pragma unroll
          for (int kk = 0; kk < L::KH / 32; ++kk) {
            Frag<OpT> fx, fy;
            lds_frag_ck(fx, xs, L::LD_KH, l16, 32 * kk, g4);
            lds_frag_ck(fy, ys, L::LD_KH, l16, 32 * kk, g4);
            mma(acc[u], fx, fy);  // lane holds [r = 16 ti + l16][s = 16 tj + 4 g4 + i]
          }
        }
      }
      if (L::NH > 1) block_sync();  // the next channel pass rewrites the Gram region
    }
    if (L::EARLY) block_sync();  // Gram operands read: Kr, Qr may be rescaled in place

    if (w < 4) {
      // inverse of the diagonal block (I + A_ww), in registers.  R layout: lane
      // holds M[4 g4 + i][l16].  N = strictly lower A_ww, NT = N^T.
      f32x4 N, NT;
      const float bl = sbeta[16 * w + l16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = 4 * g4 + i;
        N[i] = l16 < a ? sbeta[16 * w + a] * acc[0][i] : 0.f;
        NT[i] = a < l16 ? bl * acc[1][i] : 0.f;
      }
      // (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8), exact since N^16 = 0.
      // rr_tn(B, C) = B^T C, so products pair each power with its transpose.
      const f32x4 N2 = rr_tn(NT, N), T2 = rr_tn(N, NT);
      const f32x4 N3 = rr_tn(NT, N2), T3 = rr_tn(N, T2);
      const f32x4 N4 = rr_tn(T2, N2), T4 = rr_tn(N2, T2);
      const f32x4 N8 = rr_tn(T4, N4);
      f32x4 P1, P1T;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float id = (4 * g4 + i) == l16 ? 1.f : 0.f;
        P1[i] = id - N[i] + N2[i] - N3[i];
        P1T[i] = id - NT[i] + T2[i] - T3[i];
      }
      const f32x4 P2 = P1 + rr_tn(P1T, N4);
      const f32x4 P2T = P1T + rr_tn(N4, P1T);
      const f32x4 Xd = P2 + rr_tn(P2T, N8);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Lm[(16 * w + 4 * g4 + i) * L::LD_C + 16 * w + l16] = from_f32<OpT>(Xd[i]);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int kind, ti, tj;
        gram_job(w - 4, u, kind, ti, tj);
        const int r = 16 * ti + l16;
        if (kind == 0) {  // -beta_r A (strictly lower, off-diagonal tile)
          store4<OpT>(Lm + r * L::LD_C + 16 * tj + 4 * g4, acc[u] * (-sbeta[r]));
        } else {          // P, masked to s <= r on the diagonal
          f32x4 pv = acc[u];
          if (ti == tj) {
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[i] = (4 * g4 + i) <= l16 ? pv[i] : 0.f;
          }
          store4<OpT>(Pm + r * L::LD_C + skpos(16 * tj + 4 * g4), pv);
        }
      }
      if (L::EARLY) {
        // Q~ = Qr e^{G_ref}, -beta K~ = -beta Kr e^{G_ref}: every row, in place,
        // four stored columns (four consecutive channels) at a time
        const int lt = tid - 4 * 64;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int e = lt + 256 * k;             // granule index: 64 rows x 32
          const int r = e >> 5, pos = (e & 31) * 4;
          const f32x4 eb = *reinterpret_cast<const f32x4 *>(eBt + (r >> 4) * 128 + skcol(pos));
          const float nb = -sbeta[r];
          OpT *pq = Qt + r * L::LD_D + pos;
          OpT *pk = nBKt + r * L::LD_D + pos;
          Frag4<OpT> fq, fk;
          fq.v = *reinterpret_cast<const decltype(fq.v) *>(pq);
          fk.v = *reinterpret_cast<const decltype(fk.v) *>(pk);
          f32x4 vq, vk;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vq[i] = to_f32(fq.v[i]) * eb[i];
            vk[i] = to_f32(fk.v[i]) * eb[i] * nb;
          }
          store4<OpT>(pq, vq);
          store4<OpT>(pk, vk);
        }
      }
    }
    block_sync();  // Gram region free; Lm / Pm written

    // ===== P2 (fp32 operands): operands of the state products (region now holds
    // the recurrence views)
    if (!L::EARLY) {
      const float eB0 = fast_exp2(gref0[st]), eB1 = fast_exp2(gref1[st]);  // e^{G_ref}
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int r = 16 * st + 8 * th + t;
        const float br = sbeta[r];
        if (kInPlace) {
          // Q~ = Qr e^{G_ref}, -beta K~ = -beta Kr e^{G_ref}, element by element in place
          OpT *pq = Qt + r * L::LD_D + skpos(c0);
          OpT *pk = nBKt + r * L::LD_D + skpos(c0);
          const float q0 = to_f32(pq[0]), q1 = to_f32(pq[1]);
          const float kr0 = to_f32(pk[0]), kr1 = to_f32(pk[1]);
          store2<OpT>(pq, q0 * eB0, q1 * eB1);
          store2<OpT>(pk, -br * kr0 * eB0, -br * kr1 * eB1);
        } else {
          const float e0 = E1a[t] * eB0, e1 = E1b[t] * eB1;
          store2<OpT>(Qt + r * L::LD_D + skpos(c0), rq[t].lo() * e0, rq[t].hi() * e1);
          store2<OpT>(nBKt + r * L::LD_D + skpos(c0), -br * rk[t].lo() * e0, -br * rk[t].hi() * e1);
        }
      }
      write_kv(E2a, E2b);
      if (w == 0) *reinterpret_cast<f32x2 *>(sgam + c0) = f32x2{fast_exp2(glast0), fast_exp2(glast1)};
      // raw registers are free: start loading the next chunk
      if (j + 1 < nchunks) prefetch(j + 1);
      block_sync();
    }

    // ===== recurrence on this wave's 16 value columns
    f32x4 accOT[4];
    if (rec_wave) {
      // Y = beta V - beta K~ S        (lane holds Y[s = 16 st + 4 g4 + i][v])
      f32x4 accY[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        Frag4<OpT> b4;
        lds_frag4(b4, BVT, L::LD_C, vloc + l16, 16 * s4, g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) accY[s4][i] = to_f32(b4.v[i]);
      }
      // O^T = S^T Q~^T first, sharing the S fragments with Y
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) accOT[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        Frag<OpT> sf;
        acc_frag_sk(sf, S[2 * kk], S[2 * kk + 1]);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          Frag<OpT> xb, xq;
          lds_frag_ck(xb, nBKt, L::LD_D, 16 * s4 + l16, 32 * kk, g4);
          lds_frag_ck(xq, Qt, L::LD_D, 16 * s4 + l16, 32 * kk, g4);
          mma(accY[s4], xb, sf);
          mma(accOT[s4], sf, xq);
        }
      }
      // U = (I + A)^{-1} Y by block forward substitution:
      //   U_i = X_ii (Y_i - sum_{k<i} A_ik U_k)
      f32x4 accU[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int k = 0; k < i; ++k) {
          Frag4<OpT> la, uk;
          lds_frag4(la, Lm, L::LD_C, 16 * i + l16, 16 * k, g4);
          acc_frag4(uk, accU[k]);
          mma16(accY[i], la, uk);
        }
        Frag4<OpT> xd, yi;
        lds_frag4(xd, Lm, L::LD_C, 16 * i + l16, 16 * i, g4);
        acc_frag4(yi, accY[i]);
        accU[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        mma16(accU[i], xd, yi);
      }
      Frag<OpT> uf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) acc_frag_sk(uf[kk], accU[2 * kk], accU[2 * kk + 1]);
      // O^T += U^T P^T      (lane holds O[r = 16 rt + l16][v = .. + 4 g4 + i])
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk <= rt / 2) {
            Frag<OpT> xp;
            lds_frag_ck(xp, Pm, L::LD_C, 16 * rt + l16, 32 * kk, g4);
            mma(accOT[rt], uf[kk], xp);
          }
        }
      // S <- Gamma S + Kbar^T U
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const f32x4 gm = *reinterpret_cast<const f32x4 *>(sgam + 16 * ct + 4 * g4);
        S[ct] *= gm;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          Frag<OpT> xk;
          lds_frag_ck(xk, KbT, L::LD_C, 16 * ct + l16, 32 * kk, g4);
          mma(S[ct], xk, uf[kk]);
        }
      }
    }
    block_sync();

    // ===== output: stage O (scaled, io dtype) in LDS, then row-contiguous stores
    if (!write_o) continue;  // uniform; the next chunk's first barrier still orders LDS
    if (rec_wave) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        store4<OpT>(Ost + (16 * rt + l16) * L::LD_O + vloc + 4 * g4, accOT[rt] * p.scale);
    }
    block_sync();
    {
      constexpr int kVec = 16 / (int)sizeof(OpT);       // elements per 16-byte store
      constexpr int kPerRow = DV / kVec;                // stores per output row
      constexpr int kRowsPerPass = kThreads / kPerRow;
      const int col = (tid % kPerRow) * kVec;
      const __amdgpu_buffer_rsrc_t ors =
          make_rsrc(og + (bos + (int64_t)j * kC) * rowstride, (uint32_t)Lc * row_qk);
      for (int r = tid / kPerRow; r < Lc; r += kRowsPerPass) {
        const f32x4 val = *reinterpret_cast<const f32x4 *>(Ost + r * L::LD_O + col);
        buf_store_b128(ors, (uint32_t)r * row_qk + (uint32_t)col * (uint32_t)sizeof(OpT), val);
      }
    }
    // (the next chunk's first barrier orders these LDS reads before its writes)
  }

  if (sfp && rec_wave) {
    float *sf = sfp;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sf[(16 * ct + 4 * g4 + i) * kD + vblk + vloc + l16] = S[ct][i];
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

// Composition of segment transitions ([P3] section 4.1): for each chain, in
// order, S_in[s + 1] = M_s S_in[s] + S~_s for s = 1 .. P_n - 2 (S_in[1] is the
// final state of segment 0's run).  Columns of the states compose independently,
// so one workgroup of 256 threads takes 32 columns of one chain (four per
// chain); each thread owns a 4 x 4 block of the 128 x 32 product, fp32
// throughout.
constexpr int kCombineCols = 32;
__global__ __launch_bounds__(256) void segment_combine_kernel(ChunkParams p) {
  constexpr int kK = 16;  // reduction slice staged in LDS
  constexpr int NB = kD / kCombineCols;
  __shared__ __attribute__((aligned(16))) float Ms[kK][kD];            // M[:, k0 + kk] by row
  __shared__ __attribute__((aligned(16))) float Bs[kK][kCombineCols];  // S_in[k0 + kk, cols]
  const int crank = p.chain0 + (int)(blockIdx.x / NB);
  const int cb = (int)(blockIdx.x % NB) * kCombineCols;
  const int srank = crank / p.H;
  const int n = p.order ? p.order[srank] : srank;
  const int64_t chain = (int64_t)n * p.H + (crank - srank * p.H);
  int64_t len = p.seq_len;
  if (p.cu) {
    const int64_t a = p.cu[n], b = p.cu[n + 1];
    const int64_t lo = a < 0 ? 0 : (a > p.total_tokens ? p.total_tokens : a);
    const int64_t hi = b < lo ? lo : (b > p.total_tokens ? p.total_tokens : b);
    len = hi - lo;
  }
  const int pn = seg_count(p.seg_P, (int)((len + kC - 1) / kC));
  const int t = threadIdx.x;
  const int r0 = (t >> 3) * 4, c0 = (t & 7) * 4;  // rows r0 .. r0+3, columns cb + c0 .. +3
  for (int sg = 1; sg + 2 <= pn; ++sg) {
    const float *M = seg_state(p, chain, kM, sg);
    const float *B = seg_state(p, chain, kSin, sg);
    const float *St = seg_state(p, chain, kSt, sg);
    float *out = seg_state(p, chain, kSin, sg + 1);
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = St[(r0 + i) * kD + cb + c0 + j];
    for (int k0 = 0; k0 < kD; k0 += kK) {
      __syncthreads();
      for (int e = t; e < kK * kD; e += 256) {
        const int kk = e & (kK - 1), r = e / kK;  // M row r, column k0 + kk
        Ms[kk][r] = M[r * kD + k0 + kk];
      }
      for (int e = t; e < kK * kCombineCols; e += 256) {
        const int br = e / kCombineCols, bc = e % kCombineCols;
        Bs[br][bc] = B[(k0 + br) * kD + cb + bc];
      }
      __syncthreads();
#pragma unroll 4
      for (int kk = 0; kk < kK; ++kk) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = Ms[kk][r0 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[kk][c0 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) out[(r0 + i) * kD + cb + c0 + j] = acc[i][j];
    __syncthreads();  // this block of S_in[sg + 1] complete before the next step reads it
  }
}

// Clears the hand-over flags of the balanced schedule before its launch (a
// kernel rather than a memset, so the sequence can be captured in a graph).
__global__ void clear_flags_kernel(int32_t *flag, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) flag[i] = 0;
}

template <class OpT, int DV>
hipError_t launch_typed(const ChunkParams &p, int64_t items, hipStream_t stream) {
  if (p.gate)
    hipLaunchKernelGGL((chunk_fwd_kernel<OpT, DV, true>), dim3((unsigned)items), dim3(kThreads),
                       0, stream, p);
  else
    hipLaunchKernelGGL((chunk_fwd_kernel<OpT, DV, false>), dim3((unsigned)items),
                       dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Item lengths (chunks) of run w of the balanced schedule, in order, as the
// kernels take them (run_item_at).
static int run_lengths(int64_t C, int64_t n, int64_t L, int64_t w, int64_t *len) {
  const int W = run_workers((int)C, (int)n, (int)L);
  int m = 0;
  for (int k = 0;; ++k) {
    const RunItem it = run_item_at((int)C, (int)n, (int)L, k * W + (int)w);
    if (it.chain < 0) break;
    len[m++] = it.c1 - it.c0;
  }
  return m;
}

// Whether the balanced schedule beats whole chains: the finishing time of the
// items dispatched round by round, workgroup i to accelerator complex i mod 8
// and there to the first free unit, each item costing its chunks plus one for
// the pipeline's start, against ceil(C / U) n for whole chains.
static bool balanced_schedule_pays(int64_t C, int64_t n, int U, ChunkPlan *pl) {
  const int64_t total = C * n, L = (total + U - 1) / U, W = (total + L - 1) / L;
  const int64_t K = L / n + 2;  // items per run at most
  if (W > 4096 || K > 64 || total >= ((int64_t)1 << 30)) return false;
  std::vector<int64_t> len((size_t)(W * K), -1);
  int64_t rounds = 0;
  for (int64_t w = 0; w < W; ++w) {
    int64_t l[66];
    const int m = run_lengths(C, n, L, w, l);
    for (int k = 0; k < m; ++k) len[(size_t)(k * W + w)] = l[k];
    if (m > rounds) rounds = m;
  }
  const int xcd = U % 8 == 0 ? 8 : 1, per = U / xcd;
  int64_t finish = 0;
  for (int x = 0; x < xcd; ++x) {
    std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
    for (int u = 0; u < per; ++u) free_at.push(0);
    for (int64_t i = x; i < rounds * W; i += xcd) {
      const int64_t c = len[(size_t)i];
      if (c < 0) continue;
      const int64_t t = free_at.top() + c + 1;
      free_at.pop();
      free_at.push(t);
      if (t > finish) finish = t;
    }
  }
  const int64_t whole = ((C + U - 1) / U) * (n + 1);
  if (10 * finish > 9 * whole) return false;
  pl->ho_len = L;
  pl->ho_workers = W;
  pl->ho_rounds = rounds;
  return true;
}

// Equal chains that do not fill whole rounds of the units, two chunks or more
// each, where the schedule pays.
bool balanced_schedule_applies(int64_t C, int64_t n, int U, ChunkPlan *pl) {
  return U > 0 && C > U && C % U != 0 && n >= 2 && balanced_schedule_pays(C, n, U, pl);
}

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
  // segments per sequence: explicit, or chosen in automatic mode (bf16 only).
  // A split repeats the chunk-local work of the transition items, so it only
  // pays where chains would otherwise leave compute units idle: with C <= U
  // chains on U units, every chain is split into three segments with shares
  // 2:1:1; the first pass (the runs of segment 0 and the two transitions of
  // segment 1, 3C workgroups whose short ones finish in time for the rest) and
  // the second (segments 1 and 2) then take about 3/4 of an unsplit chain
  // (measured: 65,536 tokens x 96 heads, 5.16 -> 4.06 ms).  For U < C < 2U
  // splitting the chains past the first U measured no gain: a chain alone on
  // a less busy device already runs ~20% faster than in a full round.
  int64_t P = a.segments > 1 ? a.segments : 1;
  pl.seg_front = false;
  const int64_t chains = (int64_t)a.num_seqs * a.num_heads;
  int cus = 0;
  if (a.segments == 0 && a.io_dtype == KDA_BF16) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 0;
  }
  if (pl.max_chunks >= 8) {
    if (cus > 0 && chains <= cus) {
      P = 3;
      pl.seg_front = true;
    }
  }
  if (P > kMaxSegments) P = kMaxSegments;
  if (P > pl.max_chunks) P = pl.max_chunks < 1 ? 1 : pl.max_chunks;
  pl.segments = (int32_t)P;
  size_t off = 0;
  if (pl.varlen && a.num_seqs > 1 && a.num_seqs <= 4096) {
    pl.order_off = off;
    pl.order_bytes = (size_t)a.num_seqs * sizeof(int32_t);
    off += (pl.order_bytes + 255) & ~(size_t)255;
  }
  if (pl.segments > 1) {
    pl.seg_state_off = off;
    pl.seg_state_bytes = (size_t)a.num_seqs * a.num_heads * 3 * pl.segments * kD * kD * 4;
    off += pl.seg_state_bytes;
  }
  // Equal-length chains that do not fill whole rounds of the compute units (C
  // chains of n chunks, U units, C mod U != 0): runs of L = ceil(C n / U)
  // consecutive chunks of the chains laid end to end, a chain cut between two
  // runs handing its state over (run_shape).  Where the units, taking the
  // runs' items round by round as they free up, finish clearly before whole
  // chains would (1.5 n instead of 2 n for 384 chains on 256 units), the
  // prefill uses it.
  if (pl.segments <= 1 && !pl.varlen &&
      balanced_schedule_applies(chains, pl.max_chunks, cus, &pl)) {
    pl.ho_off = off;
    pl.ho_bytes = (size_t)pl.ho_workers * (kD * kD * 4 + 4);
    off += (pl.ho_bytes + 255) & ~(size_t)255;
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
  p.gate = a.gate.mode == KDA_GATE_LOWER_BOUND ? 1 : 0;
  p.A_log = a.gate.A_log;
  p.dt_bias = a.gate.dt_bias;
  // lower_bound log2(e), folded once for the kernels' base-2 exponentials
  p.gate_scale = (float)((double)a.gate.lower_bound * 1.4426950408889634);
  p.beta_logits = a.gate.beta_logits;
  if (plan.order_bytes) {
    int32_t *order = reinterpret_cast<int32_t *>((char *)a.workspace + plan.order_off);
    hipLaunchKernelGGL(order_longest_first_kernel, dim3(1), dim3(1024), 0, stream,
                       a.cu_seqlens, a.num_seqs, order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.order = order;
  }
  const int64_t chains = (int64_t)a.num_seqs * a.num_heads;
  const int VS = a.io_dtype == KDA_BF16 ? 1 : 2;  // value blocks per chain
  auto run = [&](int64_t items) {
    return a.io_dtype == KDA_BF16 ? launch_chunk_fwd_pipe(p, items, stream)
                                  : launch_typed<float, 64>(p, items, stream);
  };
  p.seg_P = plan.segments;
  p.seg_front = plan.seg_front ? 1 : 0;
  p.ws = nullptr;
  p.chain0 = 0;
  p.nchains = (int32_t)chains;
  p.ho_state = nullptr;
  p.ho_flag = nullptr;
  p.ho_len = 0;
  p.ho_polls = 0;
  p.status = nullptr;
  if (plan.ho_workers > 0) {
    char *base = (char *)a.workspace + plan.ho_off;
    p.ho_state = reinterpret_cast<float *>(base);
    p.ho_flag = reinterpret_cast<int32_t *>(base + (size_t)plan.ho_workers * kD * kD * 4);
    p.ho_len = plan.ho_len;
    p.ho_polls = handoff_poll_limit();
    const hipError_t es = device_status_word(&p.status);
    if (es != hipSuccess) return es;
    p.pass = kPassHandoff;
    hipLaunchKernelGGL(clear_flags_kernel, dim3((unsigned)((plan.ho_workers + 255) / 256)),
                       dim3(256), 0, stream, p.ho_flag, plan.ho_workers);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return run(plan.ho_workers * plan.ho_rounds);
  }
  if (plan.segments <= 1) {
    p.pass = 0;
    return run(chains * VS);
  }
  // segmented: first pass (segment 0 runs; transitions of segments 1 .. P-2),
  // composition, second pass (segments 1 .. P-1 from their exact incoming states)
  hipError_t e = hipSuccess;
  p.ws = reinterpret_cast<float *>((char *)a.workspace + plan.seg_state_off);
  const int P = plan.segments;
  p.pass = 1;
  e = run(p.nchains * (int64_t)(2 * P - 3) * VS);
  if (e != hipSuccess) return e;
  if (P > 2) {
    hipLaunchKernelGGL(segment_combine_kernel, dim3((unsigned)p.nchains * (kD / kCombineCols)),
                       dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  p.pass = 2;
  return run(p.nchains * (int64_t)(P - 1) * VS);
}

}  // namespace kda
