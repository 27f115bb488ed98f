// kda_chunk_pipe.hip -- chunkwise KDA prefill forward, bf16 I/O, on gfx950:
// chunk-local work and the state recurrence run concurrently in one workgroup.
//
// Pages (cited by title and section):
//  [P1] "How Kimi K3 Engineered Its Way to the Frontier": "How KDA updates its
//       state" (the recurrence; decay per key channel = per row of S) and
//       "FlashKDA steps the state once per 16 tokens" (inside a chunk, dense
//       products; the state stepped once per chunk; exponentials of cumulative
//       decays kept in range; 16x16 unit-triangular inverse by a Neumann series).
//  [P2] "Kimi K3: Open Frontier Intelligence", section 6 (the equation; the
//       gate's lower bound keeps a 16-token cumulative log-decay above -80).
//  [P3] "Kimi K3 -- Training and Infrastructure Notes", section 4.1 (overlap the
//       chunk-local work with the cross-chunk state recurrence).
//
// Algebra of one window of tokens r = 0 .. 63 (a whole 64-token chunk, or a
// 16-token quarter of one, see below), incoming state S (128 x 128, rows = key
// channels), G_r = sum_{s <= r} g_s per channel (log2 units), and a per-channel
// reference Gm inside [min G, max G]:
//   nKr = -beta k 2^{G - Gm},  Qr = q 2^{G - Gm},  Kc = k 2^{Gm - G},  S' = 2^{Gm} S
//   nKr Kc^T = -beta A (below the diagonal),  Qr Kc^T = P (on and below it)
//   U = (I + beta A)^{-1} beta (V - K~ S)   with   beta (V - K~ S) = beta V + nKr S'
//   O = Q~ S + P U = Qr S' + P U
//   S_next = 2^{G_end} S + Kbar^T U = 2^{G_end - Gm} (S' + Kc^T U).
// So the state is carried pre-scaled: the accumulator holds S' during a window
// and is multiplied by 2^{G_end - Gm} 2^{Gm(next)} when the next one starts.
// Every exponent is G_r - Gm or Gm - G_r, bounded by half the window's range of
// G.  A chunk whose range exceeds 128 (2^64 either way) is processed as four
// 16-token windows instead (under the pages' lower bound a 16-token range is at
// most 115).
//
// Workgroup of 8 waves, one (sequence, head) chain:
//  * waves 4..7 (producers): per window, the elementwise work (decay factors,
//    scaled operands to LDS), the Gram products on matrix cores, the inverse of
//    the four diagonal 16x16 blocks (Neumann product in registers); they run
//    one window ahead of
//  * waves 0..3 (consumers): 32 value columns each of the fp32 state (matrix-core
//    accumulators, never leaving registers): Y and O products, block forward
//    substitution, the state update, and o stores.
// Producer and consumer of the same SIMD overlap vector and matrix work; two
// barriers per window.  Operands are double-buffered in LDS; matrix-core
// operands whose contraction runs over tokens (Kc^T, V) are read with gfx950's
// transposing LDS load, so every operand is stored once, row-major.
#include "kda_chunk_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kLDK = 136;            // operand row stride: 128 bf16 + 16 bytes
constexpr int kLDC = 72;             // 64-wide matrices (Lm, Pm): 64 bf16 + 16 bytes
constexpr float kMaxRange = 128.f;   // largest log2 range of G over a 64-token window

struct Buf {                   // one window's operands
  bf16 nkr[64 * kLDK];         // -beta k 2^{G - Gm}      rows = tokens, columns skpos
  bf16 qr[64 * kLDK];          // q 2^{G - Gm}
  bf16 kc[64 * kLDK];          // k 2^{Gm - G}
  bf16 lm[64 * kLDC];          // -beta A below the diagonal blocks, X_ii on them
  bf16 pm[64 * kLDC];          // P (s <= r), columns skpos
  float beta[64];
  float mfac[128];             // state multiplier at the window's start
  float post[128];             // 2^{G_end - Gm}
  int info[4];                 // first row, end row, token offset of row 0, valid
};
struct Smem {
  Buf buf[2];
  bf16 v[64 * kLDK];           // v of the current chunk (rows = tokens, natural columns)
  int flag[4];                 // per producer wave: the next chunk fits one reference
};
static_assert(sizeof(Buf) % 16 == 0, "buffer alignment");
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget exceeded");

typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef shortx4_t __attribute__((address_space(3))) lds_shortx4;

// Transposing LDS load (DS_READ_B64_TR_B16).  Within each group of 16 lanes,
// lane j supplies the address of 4 consecutive bf16 (a quarter of a 16-element
// row segment; lanes 4s .. 4s+3 form segment s); lane i receives element i of
// segments 0..3.  So if lanes 4s + q point at row R_s, columns c0 + 4q .. +3,
// lane i gets column c0 + i of rows R_0 .. R_3.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16 *p) {
  const shortx4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)p);
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ float bperm(float v, int src_lane) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane << 2, __float_as_int(v)));
}

// Gram jobs of producer wave P: (kind, row tile i, column tile j).
// kind 0: -beta A tile (i > j) -> Lm;  1: P tile -> Pm;  2, 3: the diagonal tile
// (i, i) of -beta A as [r][s] and as [s][r] (for the inverse).  Each wave owns
// one diagonal block; the off-diagonal tiles are spread so a wave's tiles share
// operands.
struct Job { int kind, i, j; };
__device__ constexpr Job kJobs[4][6] = {
    {{2, 0, 0}, {3, 0, 0}, {1, 0, 0}, {0, 1, 0}, {1, 1, 0}, {0, 2, 0}},
    {{2, 3, 3}, {3, 3, 3}, {1, 3, 3}, {1, 2, 0}, {0, 3, 0}, {1, 3, 0}},
    {{2, 1, 1}, {3, 1, 1}, {1, 1, 1}, {0, 2, 1}, {1, 2, 1}, {0, 3, 1}},
    {{2, 2, 2}, {3, 2, 2}, {1, 2, 2}, {1, 3, 1}, {0, 3, 2}, {1, 3, 2}}};

// Gram products of one window and the inverse of this wave's diagonal block;
// writes Lm and Pm.
template <int P>
__device__ __forceinline__ void gram_and_inverse(Buf &B, int l16, int g4) {
  f32x4 acc[6];
#pragma unroll
  for (int u = 0; u < 6; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const Job jb = kJobs[P][u];
      Frag<bf16> fx, fy;
      if (jb.kind == 2) {         // [r][s]: rows of nKr_i against Kc_i
        lds_frag_ck(fx, B.nkr, kLDK, 16 * jb.i + l16, 32 * kk, g4);
        lds_frag_ck(fy, B.kc, kLDK, 16 * jb.i + l16, 32 * kk, g4);
      } else if (jb.kind == 3) {  // [s][r]
        lds_frag_ck(fx, B.kc, kLDK, 16 * jb.i + l16, 32 * kk, g4);
        lds_frag_ck(fy, B.nkr, kLDK, 16 * jb.i + l16, 32 * kk, g4);
      } else {                    // lane holds [r = 16 i + l16][s = 16 j + 4 g4 + e]
        lds_frag_ck(fx, B.kc, kLDK, 16 * jb.j + l16, 32 * kk, g4);
        lds_frag_ck(fy, jb.kind == 0 ? B.nkr : B.qr, kLDK, 16 * jb.i + l16, 32 * kk, g4);
      }
      mma(acc[u], fx, fy);
    }
  }
  // off-diagonal -beta A and P tiles
#pragma unroll
  for (int u = 2; u < 6; ++u) {
    const Job jb = kJobs[P][u];
    const int r = 16 * jb.i + l16;
    if (jb.kind == 0) {
      store4<bf16>(B.lm + r * kLDC + 16 * jb.j + 4 * g4, acc[u]);
    } else {
      f32x4 pv = acc[u];
      if (jb.i == jb.j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = (4 * g4 + e) <= l16 ? pv[e] : 0.f;
      }
      store4<bf16>(B.pm + r * kLDC + skpos(16 * jb.j + 4 * g4), pv);
    }
  }
  // inverse of the diagonal block (I + N), N = beta A_ii strictly lower, in the
  // result layout (lane holds M[4 g4 + e][l16]):
  //   (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8), exact since N^16 = 0.
  // rr_tn(B, C) = B^T C, so each power is paired with its transpose.
  constexpr int d = kJobs[P][0].i;
  f32x4 N, NT;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int a = 4 * g4 + e;
    N[e] = l16 < a ? -acc[0][e] : 0.f;
    NT[e] = a < l16 ? -acc[1][e] : 0.f;
  }
  const f32x4 N2 = rr_tn(NT, N), T2 = rr_tn(N, NT);
  const f32x4 N3 = rr_tn(NT, N2), T3 = rr_tn(N, T2);
  const f32x4 N4 = rr_tn(T2, N2), T4 = rr_tn(N2, T2);
  const f32x4 N8 = rr_tn(T4, N4);
  f32x4 P1, P1T;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float id = (4 * g4 + e) == l16 ? 1.f : 0.f;
    P1[e] = id - N[e] + N2[e] - N3[e];
    P1T[e] = id - NT[e] + T2[e] - T3[e];
  }
  const f32x4 P2 = P1 + rr_tn(P1T, N4);
  const f32x4 P2T = P1T + rr_tn(N4, P1T);
  const f32x4 Xd = P2 + rr_tn(P2T, N8);
#pragma unroll
  for (int e = 0; e < 4; ++e) B.lm[(16 * d + 4 * g4 + e) * kLDC + 16 * d + l16] = (bf16)Xd[e];
}

// ---------------------------------------------------------------- producers
// Lane = (token quarter tq, channel pair cp) of producer wave pw: channels
// 32 pw + 2 cp and + 1, tokens 16 tq .. 16 tq + 15 of the chunk.  A chunk's q,
// k, v, g and beta are loaded into registers one chunk ahead (g two ahead, so
// that whether a chunk fits one reference is known before its window starts).
__device__ __forceinline__ void producer_loop(const ChunkParams &p, const ChunkItem &itm,
                                              Smem &sm, const int pw, const int lane,
                                              const int nblk) {
  const int h = itm.h;
  const int64_t bos = itm.bos, len = itm.len;
  const int H = p.H;
  const int64_t rowstride = (int64_t)H * kD;          // elements between tokens
  const uint32_t row_b16 = (uint32_t)rowstride * 2u;  // bytes between bf16 rows
  const uint32_t row_f32 = (uint32_t)rowstride * 4u;  // bytes between fp32 rows
  const int tq = lane >> 4, cp = lane & 15;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int c0 = 32 * pw + 2 * cp;
  const int pc0 = skpos(c0);  // stored column of c0 (c0 + 1 follows it)

  uint32_t Rq[16], Rk[16], Rv[16];  // bf16 channel pairs
  f32x2 Rg[16];
  float G0[16], G1[16];             // chunk-relative cumulative log2-decay
  float pre0 = 0.f, pre1 = 0.f;     // its value before this lane's quarter
  float gm0 = 0.f, gm1 = 0.f, ge0 = 0.f, ge1 = 0.f;  // one-reference window of the chunk
  float post0 = 1.f, post1 = 1.f;   // previous window's 2^{G_end - Gm}
  float bl = 0.f;                   // beta of token 16 tq + cp
  int blk = 0, win = 0;
  bool slow = false;

  const bf16 *qg = reinterpret_cast<const bf16 *>(p.q) + (int64_t)h * kD;
  const bf16 *kg = reinterpret_cast<const bf16 *>(p.k) + (int64_t)h * kD;
  const bf16 *vg = reinterpret_cast<const bf16 *>(p.v) + (int64_t)h * kD;
  const float *gg = p.g + (int64_t)h * kD;
  const uint32_t voff_b16 = (uint32_t)tq * 16u * row_b16 + (uint32_t)c0 * 2u;
  const uint32_t voff_f32 = (uint32_t)tq * 16u * row_f32 + (uint32_t)c0 * 4u;
  auto rows_of = [&](int b) -> uint32_t {
    const int64_t rem = len - (int64_t)b * kC;
    return rem >= kC ? (uint32_t)kC : (uint32_t)(rem > 0 ? rem : 0);
  };
  // Loads through buffer resources that end at the chunk's last token: rows
  // past it read as zero.
  auto issue_qk = [&](int b) {  // q, k, beta of chunk b
    const int64_t t0 = bos + (int64_t)b * kC;
    const uint32_t nr = rows_of(b);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg + t0 * rowstride, nr * row_b16);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + t0 * rowstride, nr * row_b16);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t so = (uint32_t)t * row_b16;
      Rq[t] = buf_load_b32(rq, voff_b16, so);
      Rk[t] = buf_load_b32(rk, voff_b16, so);
    }
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.beta + t0 * H + h, nr * (uint32_t)H * 4u);
    bl = __uint_as_float(buf_load_b32(rb, (uint32_t)(16 * tq + cp) * (uint32_t)H * 4u));
  };
  auto issue_v = [&](int b) {
    const int64_t t0 = bos + (int64_t)b * kC;
    const uint32_t nr = itm.zero_v ? 0u : rows_of(b);  // the M tracker runs with v = 0
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + t0 * rowstride, nr * row_b16);
#pragma unroll
    for (int t = 0; t < 16; ++t) Rv[t] = buf_load_b32(rv, voff_b16, (uint32_t)t * row_b16);
  };
  auto issue_g = [&](int b) {
    const int64_t t0 = bos + (int64_t)b * kC;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gg + t0 * rowstride, rows_of(b) * row_f32);
#pragma unroll
    for (int t = 0; t < 16; ++t) Rg[t] = buf_load_f32x2(rg, voff_f32, (uint32_t)t * row_f32);
  };
  // Cumulative log2-decay of a chunk from Rg, its one-reference window (Gm =
  // middle of the range of G, G_end), and whether that range fits; the wave's
  // verdict goes to sm.flag[pw].
  auto digest_g = [&]() {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      a0 = fmaf(Rg[t][0], kLog2e, a0);
      a1 = fmaf(Rg[t][1], kLog2e, a1);
      G0[t] = a0;
      G1[t] = a1;
    }
    float q0[4], q1[4];  // quarter totals of this channel pair
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      q0[q] = bperm(a0, 16 * q + cp);
      q1[q] = bperm(a1, 16 * q + cp);
    }
    pre0 = 0.f;
    pre1 = 0.f;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      pre0 += q < tq ? q0[q] : 0.f;
      pre1 += q < tq ? q1[q] : 0.f;
    }
    ge0 = q0[0] + q0[1] + q0[2] + q0[3];
    ge1 = q1[0] + q1[1] + q1[2] + q1[3];
    float mx0 = -INFINITY, mn0 = INFINITY, mx1 = -INFINITY, mn1 = INFINITY;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      G0[t] += pre0;
      G1[t] += pre1;
      mx0 = fmaxf(mx0, G0[t]);
      mn0 = fminf(mn0, G0[t]);
      mx1 = fmaxf(mx1, G1[t]);
      mn1 = fminf(mn1, G1[t]);
    }
#pragma unroll
    for (int x = 16; x < 64; x <<= 1) {
      mx0 = fmaxf(mx0, bperm(mx0, lane ^ x));
      mn0 = fminf(mn0, bperm(mn0, lane ^ x));
      mx1 = fmaxf(mx1, bperm(mx1, lane ^ x));
      mn1 = fminf(mn1, bperm(mn1, lane ^ x));
    }
    gm0 = 0.5f * (mx0 + mn0);
    gm1 = 0.5f * (mx1 + mn1);
    const bool ok = (mx0 - mn0 <= kMaxRange) && (mx1 - mn1 <= kMaxRange);  // false on NaN
    const bool wave_ok = __builtin_amdgcn_ballot_w64(!ok) == 0;
    if (lane == 0) sm.flag[pw] = wave_ok ? 1 : 0;
  };

  if (nblk > 0) {
    issue_g(0);
    digest_g();  // waits for g of chunk 0
    issue_qk(0);
    issue_v(0);
    if (nblk > 1) issue_g(1);
  }
  block_sync();
  if (nblk > 0) slow = !(sm.flag[0] && sm.flag[1] && sm.flag[2] && sm.flag[3]);

  for (int it = 0;; ++it) {
    Buf &B = sm.buf[it & 1];
    // ====================== phase 1: operands of window it
    if (blk < nblk) {
      const int Lc = (int)rows_of(blk);
      const int nwin = slow ? (Lc + 15) / 16 : 1;
      const int row_lo = slow ? 16 * win : 0;
      const int row_hi = slow ? (16 * win + 16 < Lc ? 16 * win + 16 : Lc) : Lc;
      // the window's reference and end, per channel; a 16-token window is the
      // quarter tq == win, measured from its start
      const bool mine = !slow || tq == win;
      float off0 = 0.f, off1 = 0.f, wm0 = gm0, wm1 = gm1, we0 = ge0, we1 = ge1;
      if (slow) {
        off0 = pre0;
        off1 = pre1;
        float mx0 = -INFINITY, mn0 = INFINITY, mx1 = -INFINITY, mn1 = INFINITY;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          mx0 = fmaxf(mx0, G0[t]);
          mn0 = fminf(mn0, G0[t]);
          mx1 = fmaxf(mx1, G1[t]);
          mn1 = fminf(mn1, G1[t]);
        }
        // computed on every lane, taken from the window's lanes
        wm0 = bperm(0.5f * (mx0 + mn0) - off0, 16 * win + cp);
        wm1 = bperm(0.5f * (mx1 + mn1) - off1, 16 * win + cp);
        we0 = bperm(G0[15] - off0, 16 * win + cp);
        we1 = bperm(G1[15] - off1, 16 * win + cp);
      }
      if (tq == 0)
        *reinterpret_cast<f32x2 *>(B.mfac + c0) = f32x2{post0 * fast_exp2(wm0), post1 * fast_exp2(wm1)};
      post0 = fast_exp2(we0 - wm0);
      post1 = fast_exp2(we1 - wm1);
      if (tq == 0) *reinterpret_cast<f32x2 *>(B.post + c0) = f32x2{post0, post1};
      if (pw == 0) {
        const int r = 16 * tq + cp;
        B.beta[r] = (r >= row_lo && r < row_hi) ? bl : 0.f;
        if (lane == 0) {
          B.info[0] = row_lo;
          B.info[1] = row_hi;
          B.info[2] = blk * kC;
          B.info[3] = 1;
        }
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float nb = -bperm(bl, 16 * tq + t);
        const int r = 16 * tq + t;
        float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f, k20 = 0.f, k21 = 0.f;
        if (mine) {
          const float d0 = G0[t] - off0 - wm0, d1 = G1[t] - off1 - wm1;
          const float e10 = fast_exp2(d0), e11 = fast_exp2(d1);
          const float e20 = fast_exp2(-d0), e21 = fast_exp2(-d1);
          const float k0 = __uint_as_float(Rk[t] << 16), k1 = __uint_as_float(Rk[t] & 0xffff0000u);
          const float x0 = __uint_as_float(Rq[t] << 16), x1 = __uint_as_float(Rq[t] & 0xffff0000u);
          a0 = k0 * e10 * nb;
          a1 = k1 * e11 * nb;
          b0 = x0 * e10;
          b1 = x1 * e11;
          k20 = k0 * e20;
          k21 = k1 * e21;
        }
        store2<bf16>(B.nkr + r * kLDK + pc0, a0, a1);
        store2<bf16>(B.qr + r * kLDK + pc0, b0, b1);
        store2<bf16>(B.kc + r * kLDK + pc0, k20, k21);
      }
      // the chunk's q, k, beta are dead after its last window: load the next
      if (win == nwin - 1 && blk + 1 < nblk) issue_qk(blk + 1);
    } else if (pw == 0 && lane == 0) {
      B.info[3] = 0;  // no window: the consumers finish with the previous one
    }
    block_sync();
    // ====================== phase 2: Gram products and inverses of window it
    if (blk < nblk) {
      const int Lc = (int)rows_of(blk);
      const int nwin = slow ? (Lc + 15) / 16 : 1;
      switch (pw) {
        case 0: gram_and_inverse<0>(B, l16, g4); break;
        case 1: gram_and_inverse<1>(B, l16, g4); break;
        case 2: gram_and_inverse<2>(B, l16, g4); break;
        default: gram_and_inverse<3>(B, l16, g4); break;
      }
      if (win == 0) {
        // v of this chunk for the consumers (their reads of the previous chunk's v
        // were in the phase before the last barrier); then load the next chunk's
#pragma unroll
        for (int t = 0; t < 16; ++t)
          *reinterpret_cast<uint32_t *>(sm.v + (16 * tq + t) * kLDK + c0) = Rv[t];
        if (blk + 1 < nblk) issue_v(blk + 1);
      }
      if (win == nwin - 1) {
        if (blk + 1 < nblk) {
          digest_g();  // the next chunk; its verdict is read after the barrier
          if (blk + 2 < nblk) issue_g(blk + 2);
        }
        ++blk;
        win = 0;
      } else {
        ++win;
      }
    }
    block_sync();
    if (blk < nblk && win == 0) slow = !(sm.flag[0] && sm.flag[1] && sm.flag[2] && sm.flag[3]);
    if (!sm.buf[it & 1].info[3]) break;
  }
}

// ---------------------------------------------------------------- consumers
// Consumer wave cw owns value columns 32 cw .. 32 cw + 31 of the state.
__device__ __forceinline__ void consumer_loop(const ChunkParams &p, const ChunkItem &itm,
                                              Smem &sm, const int cw, const int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
  const int vcol = 32 * cw;
  const int64_t rowstride = (int64_t)p.H * kD;
  f32x4 acc[2][8];  // acc[c2][ct] = S'[16 ct + 4 g4 + e][vcol + 16 c2 + l16]
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * ct + 4 * g4 + e, col = vcol + 16 * c2 + l16;
        acc[c2][ct][e] = itm.s0 ? itm.s0[row * kD + col] : (itm.zero_v && row == col ? 1.f : 0.f);
      }
  block_sync();

  int it = 0;
  for (;; ++it) {
    Buf &B = sm.buf[(it + 1) & 1];  // window it - 1
    f32x4 accY[2][4], accOT[2][4];
    // ====================== phase 1: Y and O^T products
    if (it > 0) {
      // bring the state to this window's scale
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const f32x4 m = *reinterpret_cast<const f32x4 *>(B.mfac + 16 * ct + 4 * g4);
        acc[0][ct] *= m;
        acc[1][ct] *= m;
      }
      Frag<bf16> sf[2][4];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc_frag_sk(sf[c2][kk], acc[c2][2 * kk], acc[c2][2 * kk + 1]);
      // Y = beta V + nKr S'   (lane holds Y[16 s4 + 4 g4 + e][vcol + 16 c2 + l16])
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const f32x4 b4 = *reinterpret_cast<const f32x4 *>(B.beta + 16 * s4 + 4 * g4);
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const bf16x4 v4 = lds_read_tr(sm.v + (16 * s4 + 4 * g4 + (l16 >> 2)) * kLDK + vcol +
                                        16 * c2 + 4 * (l16 & 3));
#pragma unroll
          for (int e = 0; e < 4; ++e) accY[c2][s4][e] = b4[e] * (float)v4[e];
          accOT[c2][s4] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      // O^T = S'^T Qr^T, sharing the S' fragments with Y
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          Frag<bf16> xb, xq;
          lds_frag_ck(xb, B.nkr, kLDK, 16 * s4 + l16, 32 * kk, g4);
          lds_frag_ck(xq, B.qr, kLDK, 16 * s4 + l16, 32 * kk, g4);
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            mma(accY[c2][s4], xb, sf[c2][kk]);
            mma(accOT[c2][s4], sf[c2][kk], xq);
          }
        }
    }
    block_sync();
    // ====================== phase 2: U, O, state update, o stores
    if (it > 0) {
      const int row_lo = B.info[0], row_hi = B.info[1], tok0 = B.info[2];
      // U = (I + beta A)^{-1} Y by block forward substitution:
      //   U_i = X_ii (Y_i + sum_{k < i} Lm_ik U_k),  Lm_ik = -beta A_ik
      f32x4 accU[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int k = 0; k < i; ++k) {
          Frag4<bf16> la;
          lds_frag4(la, B.lm, kLDC, 16 * i + l16, 16 * k, g4);
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            Frag4<bf16> uk;
            acc_frag4(uk, accU[c2][k]);
            mma16(accY[c2][i], la, uk);
          }
        }
        Frag4<bf16> xd;
        lds_frag4(xd, B.lm, kLDC, 16 * i + l16, 16 * i, g4);
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          Frag4<bf16> yi;
          acc_frag4(yi, accY[c2][i]);
          accU[c2][i] = f32x4{0.f, 0.f, 0.f, 0.f};
          mma16(accU[c2][i], xd, yi);
        }
      }
      Frag<bf16> uf[2][2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) acc_frag_sk(uf[c2][kk], accU[c2][2 * kk], accU[c2][2 * kk + 1]);
      // O^T += U^T P^T     (lane holds O[16 rt + l16][vcol + 16 c2 + 4 g4 + e])
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk <= rt / 2) {
            Frag<bf16> xp;
            lds_frag_ck(xp, B.pm, kLDC, 16 * rt + l16, 32 * kk, g4);
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) mma(accOT[c2][rt], uf[c2][kk], xp);
          }
        }
      // S' += Kc^T U   (Kc^T fragments by transposing loads of the row-major Kc)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16 *base = B.kc + skpos(16 * ct + 4 * (l16 & 3));
          const int r0 = 32 * kk + 4 * g4 + (l16 >> 2);
          const bf16x4 lo = lds_read_tr(base + r0 * kLDK);
          const bf16x4 hi = lds_read_tr(base + (r0 + 16) * kLDK);
          Frag<bf16> a;
          a.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) mma(acc[c2][ct], a, uf[c2][kk]);
        }
      // o rows of this window
      if (itm.write_o) {
        bf16 *og = reinterpret_cast<bf16 *>(p.o) + (itm.bos + tok0) * rowstride +
                   (int64_t)itm.h * kD + vcol + 4 * g4;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int r = 16 * rt + l16;
          if (r >= row_lo && r < row_hi) {
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
              store4<bf16>(og + (int64_t)r * rowstride + 16 * c2, accOT[c2][rt] * p.scale);
          }
        }
      }
    }
    block_sync();
    if (!sm.buf[it & 1].info[3]) break;
  }

  // final state S = 2^{G_end - Gm} S' of the last window
  if (itm.sf) {
    const float *post = it > 0 ? sm.buf[(it + 1) & 1].post : nullptr;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const f32x4 m = post ? *reinterpret_cast<const f32x4 *>(post + 16 * ct + 4 * g4)
                           : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          itm.sf[(16 * ct + 4 * g4 + e) * kD + vcol + 16 * c2 + l16] = acc[c2][ct][e] * m[e];
    }
  }
}

__global__ __launch_bounds__(512) void chunk_fwd_pipe_kernel(ChunkParams p) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  const ChunkItem itm = decode_item(p, 1);
  if (itm.skip) return;  // uniform: the whole workgroup
  const int nblk = (int)((itm.len + kC - 1) / kC);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // one-time zero of the strictly-upper tiles (0,1) and (2,3) of both P buffers,
  // which the 32-wide k-steps of the P U product read
  for (int e = tid; e < 2 * 2 * 256; e += 512) {
    const int b = e >> 9, t = (e >> 8) & 1, rr = (e >> 4) & 15, cc = e & 15;
    sm.buf[b].pm[(32 * t + rr) * kLDC + skpos(32 * t + 16 + cc)] = (bf16)0.f;
  }

  // The two roles run separate loops with the same barriers (one before the
  // loop, two per iteration) and leave them at the same iteration: every wave
  // reads the same LDS flag after the same barrier.  In iteration it the
  // producers build window it into buf[it & 1] while the consumers run window
  // it - 1 from buf[(it - 1) & 1].
  if (w >= 4)
    producer_loop(p, itm, sm, w - 4, lane, nblk);
  else
    consumer_loop(p, itm, sm, w, lane);
}

}  // namespace

hipError_t launch_chunk_fwd_pipe(const ChunkParams &p, int64_t items, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_fwd_pipe_kernel, dim3((unsigned)items), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
