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
// G.  A chunk whose range exceeds 128 (2^64 either way) needs one reference per
// 16-token quarter instead (under the pages' lower bound a 16-token range is at
// most 115).  With the gate front end such a chunk stays one window in quarter
// mode: every quarter's operands use its own reference Gm_q (its token 8); the
// Gram tile of quarters (i, j), i > j, scales quarter j's Kc by
// 2^{Gm_i - Gm_j} <= 1 per channel, so it pairs both at quarter i's reference
// and holds the entries of the definition; quarter q's Y and O rows use the
// window-start state at quarter q's reference (S' times 2^{Gm_q - Gm_0}); the
// substitution and P U run over all tiles as in a one-reference window; and the
// state update takes the quarters in order, moving the state by
// 2^{Gm_q - Gm_{q-1}} before adding quarter q's Kc^T U.  Every factor is at most
// 1 (a decay), so nothing overflows; what underflows is negligible against the
// terms it is added to.  With log-decay input such a chunk runs as four 16-token
// windows instead (registers are the limit of the non-gate kernel).
//
// Workgroup of 8 waves, one (sequence, head) chain:
//  * waves 4..7 (producers): per window, the elementwise work (decay factors,
//    scaled operands to LDS) and the Gram products on matrix cores; they run
//    one window ahead of
//  * waves 0..3 (consumers): 32 value columns each of the fp32 state (matrix-core
//    accumulators, never leaving registers): Y and O products, the inverse of
//    one diagonal 16x16 block each (Neumann product in registers), block forward
//    substitution, the state update, and o stores.
// Producer and consumer of the same SIMD overlap vector and matrix work; two
// barriers per window.  Operands are double-buffered in LDS; matrix-core
// operands whose contraction runs over tokens (Kc^T, V) are read with gfx950's
// transposing LDS load, so every operand is stored once, row-major, in the
// bank-conflict-free layouts of kda_pipe_layout.h.
#include "kda_chunk_common.h"
#include "kda_internal.h"
#include "kda_pipe_layout.h"

namespace kda {
namespace {

using layout::kRow;                  // operand and v row stride: 128 bf16, no padding
constexpr int kLDC = 72;             // 64-wide matrices (Lm, Pm): 64 bf16 + 16 bytes
constexpr float kMaxHalf = 64.f;     // largest log2-decay over each 32-token half of a window

struct Buf {                   // one window's operands
  bf16 nkr[64 * kRow];         // -beta k 2^{G - Gm}      rows = tokens, at layout::opnd_at
  bf16 qr[64 * kRow];          // q 2^{G - Gm}
  bf16 kc[64 * kRow];          // k 2^{Gm - G}
  bf16 lm[64 * kLDC];          // -beta A below the diagonal blocks, X_ii on them
  bf16 pm[64 * kLDC];          // P (s <= r), columns skpos
  float beta[64];
  float mfac[128];             // state multiplier at the window's start
  float post[128];             // 2^{G_end - Gm}
  int info[4];                 // first row, end row, token offset of row 0, valid
};
struct Smem {
  Buf buf[2];
  bf16 v[64 * kRow];           // v of the current chunk (rows = tokens, at layout::v_at)
  float dt[128];               // the lower-bounded gate's dt_bias of the chain's head
  float qtot[4][128];          // next chunk: sum of log2-decay over each 16-token quarter
  float qref[4][128];          // next chunk: log2-decay from each quarter's start to its token 8
  int flag[4];                 // next chunk: no positive log-decay in quarter pw
  int handoff_arrived;         // the tail's hand-over flag was seen set
};
static_assert(sizeof(Buf) % 16 == 0, "buffer alignment");

// Quarter mode keeps per-channel factor vectors in Lm's upper tiles, which no
// mode writes otherwise: slot k = tile (0,1), (0,2), (0,3), (1,2), (1,3), (2,3);
// channel c at float (c / 8) * (kLDC / 2) + c % 8 of its slot, so four
// consecutive channels 4 m .. 4 m + 3 are one aligned 16-byte access
// (quarter_off).  With Gm_q the log2-decay at quarter q's reference (its token
// 8): slots 0..2 hold r_q = 2^{Gm_{q+1} - Gm_q}, slots 3 and 4 hold
// d_q = 2^{Gm_q - Gm_0} for q = 2, 3 (d_1 = r_0); all are at most 1.
__device__ __forceinline__ float *quarter_slot(Buf &B, int k) {
  const int i = k < 3 ? 0 : (k < 5 ? 1 : 2);
  const int j = k < 3 ? k + 1 : (k < 5 ? k - 1 : 3);
  return reinterpret_cast<float *>(B.lm + 16 * i * kLDC + 16 * j);
}
// Float offset within a slot of channels 16 ct + 4 g4 .. 16 ct + 4 g4 + 3.
__device__ __forceinline__ int quarter_off(int ct, int g4) {
  return (2 * ct + (g4 >> 1)) * (kLDC / 2) + 4 * (g4 & 1);
}
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget exceeded");

// The two 8-byte halves of a 16-byte read, exchanged where sw.
__device__ __forceinline__ f32x4 swap_halves(const f32x4 &x, bool sw) {
  return f32x4{sw ? x[2] : x[0], sw ? x[3] : x[1], sw ? x[0] : x[2], sw ? x[1] : x[3]};
}

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

// Exchanges between the four 16-lane rows of a wave on the vector unit, without
// the LDS crossbar (gfx950's V_PERMLANE16_SWAP / V_PERMLANE32_SWAP with both
// operands equal): every lane gets the value of the same lane in the even and
// the odd row of its pair (rows 0,1 or 2,3), resp. in rows 0..31 and 32..63.
__device__ __forceinline__ void rows_of_pair(float v, float &even, float &odd) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  even = __uint_as_float(r[0]);
  odd = __uint_as_float(r[1]);
}
__device__ __forceinline__ void halves(float v, float &lower, float &upper) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lower = __uint_as_float(r[0]);
  upper = __uint_as_float(r[1]);
}

// A fragment of an operand matrix (layout::opnd_at): rows 16 t + l16, lane group
// g's chunk of channels 32 kk .. 32 kk + 31, at frag_step(f0, t, kk) for the
// lane's f0 = frag_lane(l16, g).
__device__ __forceinline__ void lds_frag_ch(Frag<bf16> &f, const bf16 *base, int f0, int t, int kk) {
  f.v = *reinterpret_cast<const bf16x8 *>(base + layout::frag_step(f0, t, kk));
}
// The state fragment matching lds_frag_ch: tiles lo (channels 32 kk + 4 g + e)
// and hi (+16), in the chunk's order (hi first where sw, for g = 2, 3).
__device__ __forceinline__ void acc_frag_ch(Frag<bf16> &f, const f32x4 &lo, const f32x4 &hi, bool sw) {
  Frag<bf16> t;
  acc_frag_sk(t, lo, hi);
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t w = __builtin_bit_cast(u32x4_t, t.v);
  const u32x4_t r = {sw ? w[2] : w[0], sw ? w[3] : w[1], sw ? w[0] : w[2], sw ? w[1] : w[3]};
  f.v = __builtin_bit_cast(bf16x8, r);
}

// B^T C for 16x16 fp32 tiles in the result layout (lane holds M[4 g4 + e][l16]),
// on bf16 matrix cores with each operand split into a bf16 head and a bf16 tail
// (x = h + t): B^T C ~ Bh^T Ch + Bh^T Ct + Bt^T Ch, relative error ~2^-16.  The
// result layout is directly the operand layout of V_MFMA_F32_16X16X16_BF16 for
// a transposed left factor, so no data moves between lanes.
struct Split { Frag4<bf16> h, t; };
__device__ __forceinline__ Split split(const f32x4 &x) {
  Split s;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16 h = (bf16)x[e];
    s.h.v[e] = h;
    s.t.v[e] = (bf16)(x[e] - (float)h);
  }
  return s;
}
__device__ __forceinline__ f32x4 tn(const Split &b, const Split &c) {
  // Bh^T Ct + Bt^T Ch as one 32-deep product (the two 16-deep operand pairs
  // side by side in each lane's 8 k-slots) and Bh^T Ch as a 16-deep one, each
  // into an accumulator of its own, summed on the vector unit.  Chaining the
  // 16-deep product onto the 32-deep one's accumulator (different matrix
  // instructions back to back on the same registers) made the result depend on
  // timing: it occasionally took the chained accumulator before the first
  // product had landed.
  Frag<bf16> x, y;
  x.v = __builtin_shufflevector(b.h.v, b.t.v, 0, 1, 2, 3, 4, 5, 6, 7);
  y.v = __builtin_shufflevector(c.t.v, c.h.v, 0, 1, 2, 3, 4, 5, 6, 7);
  f32x4 tail = {0.f, 0.f, 0.f, 0.f};
  mma(tail, x, y);
  f32x4 head = {0.f, 0.f, 0.f, 0.f};
  mma16(head, b.h, c.h);
  return head + tail;
}

// Gram jobs of producer wave P: (kind, row tile i, column tile j).
// kind 0: -beta A tile (i >= j) -> Lm;  1: P tile -> Pm.  Each wave owns one
// diagonal block; the off-diagonal tiles are spread so a wave's tiles share
// operands.
struct Job { int kind, i, j; };
__device__ constexpr Job kJobs[4][5] = {
    {{0, 0, 0}, {1, 0, 0}, {0, 1, 0}, {1, 1, 0}, {0, 2, 0}},
    {{0, 3, 3}, {1, 3, 3}, {1, 2, 0}, {0, 3, 0}, {1, 3, 0}},
    {{0, 1, 1}, {1, 1, 1}, {0, 2, 1}, {1, 2, 1}, {0, 3, 1}},
    {{0, 2, 2}, {1, 2, 2}, {1, 3, 1}, {0, 3, 2}, {1, 3, 2}}};

// A Kc fragment of quarter j (channels 32 kk + 4 g4 + e of the lower and
// 32 kk + 16 + 4 g4 + e of the upper tile, in the chunk's order) times
// e_ij = r_j .. r_{i-1} = 2^{Gm_i - Gm_j} <= 1 per channel: in a quarter-mode
// window, Gram tile (i, j) below the diagonal then pairs quarter i's rows with
// quarter j's columns at quarter i's reference, and its entries are those of
// the definition (no factor exceeds 1, so nothing overflows).
__device__ __forceinline__ void scale_cross(Frag<bf16> &f, Buf &B, int i, int j, int kk, int g4) {
  const bool hi_first = (g4 >> 1) & 1;
  const int o0 = quarter_off(2 * kk + (hi_first ? 1 : 0), g4);
  const int o1 = quarter_off(2 * kk + (hi_first ? 0 : 1), g4);
  f32x4 e0 = f32x4{1.f, 1.f, 1.f, 1.f}, e1 = e0;
  for (int t = j; t < i; ++t) {
    const float *r = quarter_slot(B, t);
    e0 *= *reinterpret_cast<const f32x4 *>(r + o0);
    e1 *= *reinterpret_cast<const f32x4 *>(r + o1);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)((float)f.v[e] * (e < 4 ? e0[e] : e1[e - 4]));
}

// Gram products of one window: -beta A into Lm and P into Pm.
template <int P>
__device__ __forceinline__ void gram(Buf &B, int l16, int g4, bool quarters) {
  f32x4 acc[5];
#pragma unroll
  for (int u = 0; u < 5; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int f0 = layout::frag_lane(l16, g4);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      const Job jb = kJobs[P][u];
      // lane holds [r = 16 i + l16][s = 16 j + 4 g4 + e]
      Frag<bf16> fx, fy;
      lds_frag_ch(fx, B.kc, f0, jb.j, kk);
      lds_frag_ch(fy, jb.kind == 0 ? B.nkr : B.qr, f0, jb.i, kk);
      if (jb.i > jb.j && quarters) scale_cross(fx, B, jb.i, jb.j, kk, g4);
      mma(acc[u], fx, fy);
    }
  }
#pragma unroll
  for (int u = 0; u < 5; ++u) {
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
}

// In place on diagonal block d of Lm: -beta A_dd (its strictly lower part)
// becomes X_dd = (I + N)^{-1}, N = beta A_dd.  In the result layout (lane holds
// M[4 g4 + e][l16]):
//   (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8), exact since N^16 = 0;
// each power is paired with its transpose because the products are B^T C.
__device__ __forceinline__ void inverse(Buf &B, int d, int l16, int g4) {
  bf16 *blk = B.lm + 16 * d * kLDC + 16 * d;
  // T[4 g4 + e][l16] by a transposing load; T^T[4 g4 + e][l16] = T[l16][4 g4 + e] directly
  const bf16x4 t = lds_read_tr(blk + (4 * g4 + (l16 >> 2)) * kLDC + 4 * (l16 & 3));
  const bf16x4 tt = *reinterpret_cast<const bf16x4 *>(blk + l16 * kLDC + 4 * g4);
  f32x4 N, NT;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int a = 4 * g4 + e;
    N[e] = l16 < a ? -(float)t[e] : 0.f;
    NT[e] = a < l16 ? -(float)tt[e] : 0.f;
  }
  const Split sN = split(N), sNT = split(NT);
  const f32x4 N2 = tn(sNT, sN), T2 = tn(sN, sNT);
  const Split sN2 = split(N2), sT2 = split(T2);
  const f32x4 N3 = tn(sNT, sN2), T3 = tn(sN, sT2);
  const f32x4 N4 = tn(sT2, sN2), T4 = tn(sN2, sT2);
  const Split sN4 = split(N4), sT4 = split(T4);
  const f32x4 N8 = tn(sT4, sN4);
  f32x4 P1, P1T;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float id = (4 * g4 + e) == l16 ? 1.f : 0.f;
    P1[e] = id - N[e] + N2[e] - N3[e];
    P1T[e] = id - NT[e] + T2[e] - T3[e];
  }
  const Split sP1T = split(P1T);
  const f32x4 P2 = P1 + tn(sP1T, sN4);
  const f32x4 P2T = P1T + tn(sN4, sP1T);
  const f32x4 Xd = P2 + tn(split(P2T), split(N8));
  // every lane has read its operands before any writes (one wave, in order)
#pragma unroll
  for (int e = 0; e < 4; ++e) blk[(4 * g4 + e) * kLDC + l16] = (bf16)Xd[e];
}

// ---------------------------------------------------------------- producers
// Producer wave pw handles tokens 16 pw .. 16 pw + 15 (quarter pw) of a chunk,
// all 128 channels: lane = (ts, co) holds tokens 16 pw + 4 ts + j (j < 4) and
// channels 8 co .. 8 co + 7, so every load instruction reads four whole
// 256-byte token rows.  A chunk's q, k, v, beta are loaded one chunk ahead, its
// g two ahead: its cumulative decay and whether one reference fits it are known
// before its first window starts.
//
// One reference per 64-token window is used when, on every channel, the
// decay over tokens 0..31 and over 32..63 each stay within 2^64 and no
// log-decay is positive; then Gm = G_31 and every factor is within 2^{+-64}.
// Otherwise the chunk runs as four 16-token windows, window w with the
// reference at its token 8.
//
// GATE: g holds gate logits and the lower-bounded gate is applied as the chunk
// is digested (gate_log2); beta logits (p.beta_logits) pass through a sigmoid
// as a window's beta is first used.
template <bool GATE>
__device__ __forceinline__ void producer_loop(const ChunkParams &p, const ChunkItem &itm,
                                              Smem &sm, const int pw, const int lane,
                                              const int nblk) {
  const int h = itm.h;
  const int64_t bos = itm.bos, len = itm.len;
  const int H = p.H;
  const int64_t rowstride = (int64_t)H * kD;          // elements between tokens
  const uint32_t row_b16 = (uint32_t)rowstride * 2u;  // bytes between bf16 rows
  const uint32_t row_f32 = (uint32_t)rowstride * 4u;  // bytes between fp32 rows
  const uint32_t row_beta = (uint32_t)H * 4u;         // bytes between beta rows
  const int ts = lane >> 4, co = lane & 15;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int r0 = 16 * pw + 4 * ts;                    // this lane's first row in the chunk
  // the lane's two channel quads in row r0 (row r0 + j: layout::opnd_row_step)
  const int pA = layout::opnd_at(r0, 8 * co), pB = layout::opnd_at(r0, 8 * co + 4);
  const int pV = layout::v_at(r0, 8 * co);  // its v chunk in row r0

  u32x4 Rq[4], Rk[4], Rv[4];   // 8 bf16 channels per token
  f32x4 Rg[4][2];              // 8 fp32 channels per token
  float Rb[4];                 // beta per token
  float Gl[4][8];              // log2-decay summed from the quarter's start (inclusive)
  // without the gate: per channel the chunk-relative prefix of this quarter and
  // the one-reference window's reference and end, held from decide() to phase 1
  // (the gate variant re-reads them from sm.qtot to keep its registers free)
  float qp[8], gref[8], gend[8];
  int blk = 0, win = 0;
  bool slow = false;

  const bf16 *qg = reinterpret_cast<const bf16 *>(p.q) + (int64_t)h * kD;
  const bf16 *kg = reinterpret_cast<const bf16 *>(p.k) + (int64_t)h * kD;
  const bf16 *vg = reinterpret_cast<const bf16 *>(p.v) + (int64_t)h * kD;
  const float *gg = p.g + (int64_t)h * kD;
  // gate constants: the head's factor, and the bias of this lane's channels in
  // registers for the first chunk (later chunks read it from sm.dt, so it holds
  // no registers through the loop)
  float gate_a = 0.f, dt0[8];
  if constexpr (GATE) {
    gate_a = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                           __builtin_bit_cast(int, gate_head_factor(p.A_log[h]))));
#pragma unroll
    for (int i = 0; i < 8; ++i) dt0[i] = p.dt_bias ? p.dt_bias[h * kD + 8 * co + i] : 0.f;
    if (pw == 0 && ts == 0) {
      *reinterpret_cast<f32x4 *>(sm.dt + 8 * co) = f32x4{dt0[0], dt0[1], dt0[2], dt0[3]};
      *reinterpret_cast<f32x4 *>(sm.dt + 8 * co + 4) = f32x4{dt0[4], dt0[5], dt0[6], dt0[7]};
    }
  }
  const uint32_t voff_b16 = (uint32_t)r0 * row_b16 + 16u * co;
  const uint32_t voff_f32 = (uint32_t)r0 * row_f32 + 32u * co;
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
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.beta + t0 * H + h, nr * row_beta);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Rq[j] = buf_load_b128(rq, voff_b16, (uint32_t)j * row_b16);
      Rk[j] = buf_load_b128(rk, voff_b16, (uint32_t)j * row_b16);
      Rb[j] = __uint_as_float(buf_load_b32(rb, (uint32_t)r0 * row_beta, (uint32_t)j * row_beta));
    }
  };
  auto issue_v = [&](int b) {
    const int64_t t0 = bos + (int64_t)b * kC;
    const uint32_t nr = itm.zero_v ? 0u : rows_of(b);  // the M tracker runs with v = 0
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + t0 * rowstride, nr * row_b16);
#pragma unroll
    for (int j = 0; j < 4; ++j) Rv[j] = buf_load_b128(rv, voff_b16, (uint32_t)j * row_b16);
  };
  auto issue_g = [&](int b) {
    const int64_t t0 = bos + (int64_t)b * kC;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gg + t0 * rowstride, rows_of(b) * row_f32);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Rg[j][0] = __builtin_bit_cast(f32x4, buf_load_b128(rg, voff_f32, (uint32_t)j * row_f32));
      Rg[j][1] = __builtin_bit_cast(f32x4, buf_load_b128(rg, voff_f32 + 16u, (uint32_t)j * row_f32));
    }
  };
  // Log2-decay of a chunk from Rg: Gl (from the quarter's start), the quarter's
  // totals to sm.qtot[pw], and whether no log-decay of the quarter is positive
  // to sm.flag[pw].
  // nvalid: rows of the chunk in the sequence; dt_of(i): the gate's bias of
  // channel 8 co + i
  auto digest_g = [&](int nvalid, auto dt_of) {
    bool ok = true;
    float a[8], y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0.f;
      float dt = 0.f;
      if constexpr (GATE) dt = dt_of(i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gv = Rg[j][i >> 2][i & 3];
        if constexpr (GATE) {
          // rows past the sequence end read gate logit 0, whose gate is not 0:
          // they get log-decay 0 (a 0 / 1 factor)
          const float live = __builtin_amdgcn_fmed3f((float)(nvalid - r0 - j), 0.f, 1.f);
          const float gl = live * gate_log2(gv, gate_a, dt, p.gate_scale);
          ok = ok && gl <= 0.f;  // false on NaN
          a[i] += gl;
        } else {
          ok = ok && gv <= 0.f;  // false on NaN
          a[i] = fmaf(gv, kLog2e, a[i]);
        }
        Gl[j][i] = a[i];
      }
    }
    // exclusive scan over the four lanes (rows) that share a channel: the pair's
    // even row, then the total of rows 0,1 for rows 2,3
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float ev, od, lo, hi;
      rows_of_pair(a[i], ev, od);
      halves(ev + od, lo, hi);
      y[i] = lo + hi;  // quarter total
      const float excl = ((ts & 1) ? ev : 0.f) + (ts >= 2 ? lo : 0.f);
#pragma unroll
      for (int j = 0; j < 4; ++j) Gl[j][i] += excl;
    }
    if (ts == 0) {
      *reinterpret_cast<f32x4 *>(&sm.qtot[pw][8 * co]) = f32x4{y[0], y[1], y[2], y[3]};
      *reinterpret_cast<f32x4 *>(&sm.qtot[pw][8 * co + 4]) = f32x4{y[4], y[5], y[6], y[7]};
    }
    if constexpr (GATE) {
      if (ts == 2) {  // the quarter's token 8: its reference in quarter mode
        *reinterpret_cast<f32x4 *>(&sm.qref[pw][8 * co]) = f32x4{Gl[0][0], Gl[0][1], Gl[0][2], Gl[0][3]};
        *reinterpret_cast<f32x4 *>(&sm.qref[pw][8 * co + 4]) = f32x4{Gl[0][4], Gl[0][5], Gl[0][6], Gl[0][7]};
      }
    }
    const bool wave_ok = __builtin_amdgcn_ballot_w64(!ok) == 0;
    if (lane == 0) sm.flag[pw] = wave_ok ? 1 : 0;
  };
  // From the quarter totals of the current chunk (sm.qtot, written by
  // digest_g and read after the barrier that follows it, until the chunk's last
  // window digests the next one): per channel of the lane, the chunk-relative
  // prefix of this quarter qp, the one-reference window's reference gref
  // (token 31) and end gend -- what decide() leaves in registers, re-read by the
  // gate variant.
  auto chunk_refs = [&](float (&qp)[8], float (&gref)[8], float (&gend)[8]) {
    f32x4 t[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      t[q][0] = *reinterpret_cast<const f32x4 *>(&sm.qtot[q][8 * co]);
      t[q][1] = *reinterpret_cast<const f32x4 *>(&sm.qtot[q][8 * co + 4]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = t[0][i >> 2][i & 3], q1 = t[1][i >> 2][i & 3];
      const float q2 = t[2][i >> 2][i & 3], q3 = t[3][i >> 2][i & 3];
      qp[i] = (pw > 0 ? q0 : 0.f) + (pw > 1 ? q1 : 0.f) + (pw > 2 ? q2 : 0.f);
      gref[i] = q0 + q1;
      gend[i] = q0 + q1 + q2 + q3;
    }
  };
  // After the barrier that follows digest_g: whether one reference fits the
  // chunk (same on all waves).
  auto decide = [&]() -> bool {
    f32x4 t[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      t[q][0] = *reinterpret_cast<const f32x4 *>(&sm.qtot[q][8 * co]);
      t[q][1] = *reinterpret_cast<const f32x4 *>(&sm.qtot[q][8 * co + 4]);
    }
    bool ok = sm.flag[0] && sm.flag[1] && sm.flag[2] && sm.flag[3];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = t[0][i >> 2][i & 3], q1 = t[1][i >> 2][i & 3];
      const float q2 = t[2][i >> 2][i & 3], q3 = t[3][i >> 2][i & 3];
      qp[i] = (pw > 0 ? q0 : 0.f) + (pw > 1 ? q1 : 0.f) + (pw > 2 ? q2 : 0.f);
      gref[i] = q0 + q1;
      gend[i] = q0 + q1 + q2 + q3;
      ok = ok && (-gref[i] <= kMaxHalf) && (gref[i] - gend[i] <= kMaxHalf);
    }
    return __builtin_amdgcn_ballot_w64(!ok) == 0;
  };

  // Every iteration issues the same loads in the same order -- q, k, beta in
  // the first phase; v, then g in the second -- so the hardware's in-order load
  // counter lets each use wait for exactly its own group.  Loads of a chunk past
  // the sequence read nothing (empty buffer range); a group that is not due yet
  // (the next window is in the same chunk) reloads the chunk it already holds.
  issue_g(0);
  digest_g((int)rows_of(0), [&](int i) { return dt0[i]; });  // waits for g of chunk 0
  issue_qk(0);
  issue_v(0);
  issue_g(1);
  block_sync();
  slow = !decide();

  for (int it = 0;; ++it) {
    Buf &B = sm.buf[it & 1];
    const Buf &Bprev = sm.buf[(it + 1) & 1];
    const int Lc = (int)rows_of(blk);
    // A chunk too wide for one reference: with the gate front end, one window in
    // quarter mode (each quarter, the rows of one wave, with its own reference);
    // with log-decay input, four 16-token windows
    const bool sixteen = !GATE && slow;
    const int nwin = sixteen ? (Lc + 15) / 16 : 1;
    const bool last = win == nwin - 1;  // last window of the chunk
    // ====================== phase 1: operands of window it
    if (blk < nblk) {
      if (p.beta_logits) {
#pragma unroll
        for (int j = 0; j < 4; ++j) Rb[j] = sigmoid_fast(Rb[j]);
      }
      const int row_lo = sixteen ? 16 * win : 0;
      const int row_hi = sixteen ? (16 * win + 16 < Lc ? 16 * win + 16 : Lc) : Lc;
      // this window's reference and end per channel, relative to its start; the
      // lanes' offset to it (a 16-token window is quarter win, so only its wave
      // holds its tokens; in quarter mode every wave takes its own quarter's)
      const bool mine = !sixteen || pw == win;
      float off[8], wref[8], wend[8];
      if (!slow) {
        if constexpr (GATE) {
          float qp2[8];
          chunk_refs(qp2, wref, wend);
#pragma unroll
          for (int i = 0; i < 8; ++i) off[i] = qp2[i] - wref[i];
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            wref[i] = gref[i];
            wend[i] = gend[i];
            off[i] = qp[i] - gref[i];
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          wref[i] = bperm(Gl[0][i], 32 + co);  // token 8 of the quarter
          wend[i] = bperm(Gl[3][i], 48 + co);  // token 15
          off[i] = -wref[i];
        }
      }
      // The reference factor 2^{ref} (times the previous window's end factor) and
      // the end factor 2^{end - ref}: one wave's lanes of co.  In quarter mode
      // wave 0 writes the first, wave 3 the second, and wave q >= 1 the factors
      // r_{q-1} (previous quarter's reference to its own) and, q >= 2, d_q
      // (quarter 0's reference to its own) into Lm's upper tiles, from the
      // quarter totals and token-8 offsets of the digest
      const bool quarters = GATE && slow;
      const bool writer = ts == 0 && (quarters || (slow ? pw == win : pw == 0));
      if (writer) {
        if (!quarters || pw == 0) {
          f32x4 mf[2];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float prev = it > 0 ? Bprev.post[8 * co + i] : 1.f;
            mf[i >> 2][i & 3] = prev * fast_exp2(wref[i]);
          }
          *reinterpret_cast<f32x4 *>(B.mfac + 8 * co) = mf[0];
          *reinterpret_cast<f32x4 *>(B.mfac + 8 * co + 4) = mf[1];
        }
        if (!quarters || pw == 3) {
          f32x4 po[2];
#pragma unroll
          for (int i = 0; i < 8; ++i) po[i >> 2][i & 3] = fast_exp2(wend[i] - wref[i]);
          *reinterpret_cast<f32x4 *>(B.post + 8 * co) = po[0];
          *reinterpret_cast<f32x4 *>(B.post + 8 * co + 4) = po[1];
        }
        if (GATE && quarters && pw > 0) {
          f32x4 rr[2], dd[2];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int c = 8 * co + i;
            float before = 0.f;  // log2-decay of quarters 0 .. pw - 1
#pragma unroll
            for (int t = 0; t < 3; ++t) before += t < pw ? sm.qtot[t][c] : 0.f;
            rr[i >> 2][i & 3] = fast_exp2(sm.qtot[pw - 1][c] - sm.qref[pw - 1][c] + wref[i]);
            dd[i >> 2][i & 3] = fast_exp2(before + wref[i] - sm.qref[0][c]);
          }
          float *rd = quarter_slot(B, pw - 1) + co * (kLDC / 2);
          *reinterpret_cast<f32x4 *>(rd) = rr[0];
          *reinterpret_cast<f32x4 *>(rd + 4) = rr[1];
          if (pw >= 2) {
            float *dq = quarter_slot(B, pw + 1) + co * (kLDC / 2);
            *reinterpret_cast<f32x4 *>(dq) = dd[0];
            *reinterpret_cast<f32x4 *>(dq + 4) = dd[1];
          }
        }
      }
      if (co == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) B.beta[r0 + j] = mine ? Rb[j] : 0.f;
      }
      if (pw == 0 && lane == 0) {
        B.info[0] = row_lo;
        B.info[1] = row_hi;
        B.info[2] = blk * kC;
        B.info[3] = quarters ? 2 : 1;  // 2: quarter mode
      }
      // one window's operands; in a 16-token window the other waves write zeros
      auto operands = [&](bool keep) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float nb = -Rb[j];
          const u32x4 kr = keep ? Rk[j] : u32x4{0u, 0u, 0u, 0u};
          const u32x4 qr = keep ? Rq[j] : u32x4{0u, 0u, 0u, 0u};
          float a[8], b[8], c[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float d = keep ? Gl[j][i] + off[i] : 0.f;
            const float e1 = fast_exp2(d), e2 = fast_exp2(-d);
            const uint32_t kw = kr[i >> 1], qw = qr[i >> 1];
            const float kv = __uint_as_float((i & 1) ? (kw & 0xffff0000u) : (kw << 16));
            const float qv = __uint_as_float((i & 1) ? (qw & 0xffff0000u) : (qw << 16));
            a[i] = kv * e1 * nb;
            b[i] = qv * e1;
            c[i] = kv * e2;
          }
          const int oA = layout::opnd_row_step(pA, j), oB = layout::opnd_row_step(pB, j);
          store4<bf16>(B.nkr + oA, f32x4{a[0], a[1], a[2], a[3]});
          store4<bf16>(B.nkr + oB, f32x4{a[4], a[5], a[6], a[7]});
          store4<bf16>(B.qr + oA, f32x4{b[0], b[1], b[2], b[3]});
          store4<bf16>(B.qr + oB, f32x4{b[4], b[5], b[6], b[7]});
          store4<bf16>(B.kc + oA, f32x4{c[0], c[1], c[2], c[3]});
          store4<bf16>(B.kc + oB, f32x4{c[4], c[5], c[6], c[7]});
        }
      };
      if (!slow)
        operands(true);
      else
        operands(mine);
    } else if (pw == 0 && lane == 0) {
      B.info[3] = 0;  // no window: the consumers finish with the previous one
    }
    // q, k, beta of the next window's chunk
    issue_qk(last ? blk + 1 : blk);
    block_sync();
    // ====================== phase 2: Gram products of window it
    if (blk < nblk) {
      const bool quarters = GATE && slow;
      switch (pw) {
        case 0: gram<0>(B, l16, g4, quarters); break;
        case 1: gram<1>(B, l16, g4, quarters); break;
        case 2: gram<2>(B, l16, g4, quarters); break;
        default: gram<3>(B, l16, g4, quarters); break;
      }
      if (win == 0) {
        // v of this chunk for the consumers (their reads of the previous chunk's v
        // were in the phase before the last barrier)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<u32x4 *>(sm.v + layout::v_row_step(pV, j)) = Rv[j];
      }
    }
    // Wave priorities order the SIMD's issue between its producer and consumer
    // wave: the producer runs its operands and Gram products at 3, the
    // consumer its block substitution at 2, everything else runs at 0 (the
    // loads, digest and decision here; the consumer's products with the state
    // and o stores).  Measured on the 1M-token pack: -2.5% against no
    // priorities; the producer at 3 in its whole loop, the consumer's
    // substitution at 3, or the Gram below the substitution, gained less or
    // nothing.
    __builtin_amdgcn_s_setprio(0);
    issue_v(blk + 1);  // v of the next chunk (written at its first window)
    if (blk < nblk && last && blk + 1 < nblk)  // read after the barrier
      digest_g((int)rows_of(blk + 1),
               [&](int i) { return sm.dt[8 * co + i]; });
    issue_g(blk < nblk && last ? blk + 2 : blk + 1);
    bool fresh = false;  // a new chunk starts at the next window
    if (blk < nblk) {
      if (last) {
        ++blk;
        win = 0;
        fresh = blk < nblk;
      } else {
        ++win;
      }
    }
    block_sync();
    __builtin_amdgcn_s_setprio(3);
    if (fresh) slow = !decide();
    if (!sm.buf[it & 1].info[3]) break;
  }
}

// ---------------------------------------------------------------- consumers
// Consumer wave cw owns value columns 32 cw .. 32 cw + 31 of the state.
template <bool GATE>
__device__ __forceinline__ void consumer_loop(const ChunkParams &p, const ChunkItem &itm,
                                              Smem &sm, const int cw, const int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
  const int vcol = 32 * cw;
  const int64_t rowstride = (int64_t)p.H * kD;
  // lane offsets in the LDS layouts: operand fragments (whose chunks hold the
  // upper tile's quad first where fsw), the transposing reads of Kc and v, the
  // o staging stores and reads (quads swapped where ssw)
  const int f0 = layout::frag_lane(l16, g4);
  const bool fsw = (g4 >> 1) & 1;
  const int kt0 = layout::kc_tr_lane(l16, g4);
  const int vt0 = layout::v_tr_lane(l16, g4, vcol);
  const int sw0 = layout::stage_w_lane(l16, g4), sr0 = layout::stage_r_lane(l16, g4);
  const bool ssw = layout::stage_swapped(l16);
  f32x4 acc[2][8];  // acc[c2][ct] = S'[16 ct + 4 g4 + e][vcol + 16 c2 + l16]
  if (itm.s0) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[c2][ct][e] = itm.poison ? __builtin_nanf("")
                                      : itm.s0[(16 * ct + 4 * g4 + e) * kD + vcol + 16 * c2 + l16];
  } else {
    const float diag = itm.zero_v ? 1.f : 0.f;  // identity for the M tracker
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[c2][ct][e] = (16 * ct + 4 * g4 + e) == (vcol + 16 * c2 + l16) ? diag : 0.f;
  }
  block_sync();

  int it = 0;
  // Window it - 1 in iteration it: Y and O^T products in the first phase, the
  // substitution, state update and o stores in the second.  A quarter-mode
  // window (gate front end only) keeps one reference per 16-token quarter: its
  // Y and O^T rows of quarter q use the window-start state at quarter q's
  // reference (S' times d_q), the substitution and P U run over all tiles as
  // usual (the producers scale the cross-quarter Gram tiles), and the state
  // update walks the quarters, moving the state from one reference to the next
  // (factor r_q) before adding quarter q + 1's K^T U.
  for (;; ++it) {
    f32x4 accY[2][4], accOT[2][4];
    // ====================== phase 1: Y and O^T products, one diagonal inverse
    if (it > 0) {
      Buf &B = sm.buf[(it + 1) & 1];  // window it - 1
      const bool quarters = GATE && __builtin_amdgcn_readfirstlane(B.info[3]) == 2;  // wave-uniform
      // bring the state to this window's scale
  #pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const f32x4 m = *reinterpret_cast<const f32x4 *>(B.mfac + 16 * ct + 4 * g4);
        acc[0][ct] *= m;
        acc[1][ct] *= m;
      }
      // Y = beta V + nKr S'   (lane holds Y[16 s4 + 4 g4 + e][vcol + 16 c2 + l16])
  #pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const f32x4 b4 = *reinterpret_cast<const f32x4 *>(B.beta + 16 * s4 + 4 * g4);
  #pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const bf16x4 v4 = lds_read_tr(sm.v + layout::v_tr_step(vt0, s4, c2));
  #pragma unroll
          for (int e = 0; e < 4; ++e) accY[c2][s4][e] = b4[e] * (float)v4[e];
          accOT[c2][s4] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      if constexpr (GATE) {
        // row tile by row tile, the S' fragments formed as they are used; in a
        // quarter-mode window quarter q's rows meet d_q S' (d_1 = r_0 in slot 0,
        // d_2 and d_3 in slots 3 and 4), the state at quarter q's reference
  #pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const float *dq = quarter_slot(B, s4 == 1 ? 0 : s4 + 1);
  #pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            Frag<bf16> sq[2];
            if (quarters && s4 > 0) {
              const f32x4 dl = *reinterpret_cast<const f32x4 *>(dq + quarter_off(2 * kk, g4));
              const f32x4 dh = *reinterpret_cast<const f32x4 *>(dq + quarter_off(2 * kk + 1, g4));
  #pragma unroll
              for (int c2 = 0; c2 < 2; ++c2)
                acc_frag_ch(sq[c2], acc[c2][2 * kk] * dl, acc[c2][2 * kk + 1] * dh, fsw);
            } else {
  #pragma unroll
              for (int c2 = 0; c2 < 2; ++c2) acc_frag_ch(sq[c2], acc[c2][2 * kk], acc[c2][2 * kk + 1], fsw);
            }
            Frag<bf16> xb, xq;
            lds_frag_ch(xb, B.nkr, f0, s4, kk);
            lds_frag_ch(xq, B.qr, f0, s4, kk);
  #pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
              mma(accY[c2][s4], xb, sq[c2]);
              mma(accOT[c2][s4], sq[c2], xq);
            }
          }
        }
      } else {
        Frag<bf16> sf[2][4];
  #pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
  #pragma unroll
          for (int kk = 0; kk < 4; ++kk) acc_frag_ch(sf[c2][kk], acc[c2][2 * kk], acc[c2][2 * kk + 1], fsw);
        // O^T = S'^T Qr^T, sharing the S' fragments with Y
  #pragma unroll
        for (int kk = 0; kk < 4; ++kk)
  #pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            Frag<bf16> xb, xq;
            lds_frag_ch(xb, B.nkr, f0, s4, kk);
            lds_frag_ch(xq, B.qr, f0, s4, kk);
  #pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
              mma(accY[c2][s4], xb, sf[c2][kk]);
              mma(accOT[c2][s4], sf[c2][kk], xq);
            }
          }
      }
      // diagonal block cw of the triangular system, for the next phase
      inverse(B, cw, l16, g4);
    }
    block_sync();
    // ====================== phase 2: U, O, state update, o stores
    __builtin_amdgcn_s_setprio(2);  // the substitution chain (see producer_loop)
    if (it > 0) {
      Buf &B = sm.buf[(it + 1) & 1];  // window it - 1
      const bool quarters = GATE && __builtin_amdgcn_readfirstlane(B.info[3]) == 2;  // wave-uniform
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
      __builtin_amdgcn_s_setprio(0);
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
      if constexpr (GATE) {
        // S' += Kc_q^T U_q quarter by quarter (16-deep products); in a
        // quarter-mode window the state first moves from quarter q - 1's
        // reference to quarter q's (factor r_{q-1} in slot q - 1), ending at
        // quarter 3's
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (quarters && q > 0) {
            const float *rq = quarter_slot(B, q - 1);
  #pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
              const f32x4 m = *reinterpret_cast<const f32x4 *>(rq + quarter_off(ct, g4));
              acc[0][ct] *= m;
              acc[1][ct] *= m;
            }
          }
          Frag4<bf16> uq[2];  // U_q: half q & 1 of the packed 32-token fragment
  #pragma unroll
          for (int c2 = 0; c2 < 2; ++c2)
            uq[c2].v = (q & 1) ? __builtin_shufflevector(uf[c2][q >> 1].v, uf[c2][q >> 1].v, 4, 5, 6, 7)
                               : __builtin_shufflevector(uf[c2][q >> 1].v, uf[c2][q >> 1].v, 0, 1, 2, 3);
  #pragma unroll
          for (int ct = 0; ct < 8; ++ct) {
            Frag4<bf16> a;
            a.v = lds_read_tr(B.kc + layout::kc_tr_step(kt0, ct, q >> 1, q & 1));
  #pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) mma16(acc[c2][ct], a, uq[c2]);
          }
        }
      } else {
        // S' += Kc^T U   (Kc^T fragments by transposing loads of the row-major Kc)
  #pragma unroll
        for (int ct = 0; ct < 8; ++ct)
  #pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const bf16x4 lo = lds_read_tr(B.kc + layout::kc_tr_step(kt0, ct, kk, 0));
            const bf16x4 hi = lds_read_tr(B.kc + layout::kc_tr_step(kt0, ct, kk, 1));
            Frag<bf16> a;
            a.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  #pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) mma(acc[c2][ct], a, uf[c2][kk]);
          }
      }
      // o rows of this window: staged through this wave's own 16 rows of the
      // window's nKr (read by no one after phase 1; layout::stage_at), so each
      // store writes 64 contiguous bytes of a row
      if (itm.write_o) {
        bf16 *stage = B.nkr + 16 * kRow * cw;
  #pragma unroll
        for (int rt = 0; rt < 4; ++rt)
  #pragma unroll
          for (int c2 = 0; c2 < 2; ++c2)
            store4<bf16>(stage + layout::stage_w_step(sw0, rt, c2), accOT[c2][rt] * p.scale);
        const __amdgpu_buffer_rsrc_t ors = make_rsrc(
            reinterpret_cast<bf16 *>(p.o) + (itm.bos + tok0) * rowstride + (int64_t)itm.h * kD + vcol,
            (uint32_t)row_hi * (uint32_t)rowstride * 2u);
  #pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int r = 16 * k + l16;
          const f32x4 val =
              swap_halves(*reinterpret_cast<const f32x4 *>(stage + layout::stage_r_step(sr0, k)), ssw);
          if (r >= row_lo)
            buf_store_b128_cached(ors, (uint32_t)r * (uint32_t)rowstride * 2u + 16u * g4, val);
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

// State hand-over between the workgroups of the balanced schedule.  The head's
// final state is stored by the consumer waves; every thread's release fence at
// device scope, a barrier, then the flag.  The tail's reader polls the flag, at
// most p.ho_polls times so that every wave exits; then a barrier and an acquire
// fence in every thread before the state is read.  A tail that gives up sets
// KDA_DEVICE_HANDOFF_TIMEOUT in the GPU's status word and runs from a NaN state,
// so its o rows and the chain's final state come out NaN instead of wrong.
__device__ __forceinline__ void publish_state(int32_t *flag, int tid) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool await_state(const ChunkParams &p, const int32_t *flag, int tid,
                                            int *arrived) {
  if (tid == 0) {
    int ok = 0;
    for (int i = 0; i < p.ho_polls && !ok; ++i) {
      ok = __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != 0;
      if (!ok) __builtin_amdgcn_s_sleep(8);
    }
    if (!ok && p.status)
      __hip_atomic_fetch_or(p.status, (uint32_t)KDA_DEVICE_HANDOFF_TIMEOUT, __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
    *arrived = ok;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return *arrived != 0;
}

template <bool GATE>
__global__ __launch_bounds__(512) void chunk_fwd_pipe_kernel(ChunkParams p) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // one-time zero of the strictly-upper tiles (0,1) and (2,3) of both P buffers,
  // which the 32-wide k-steps of the P U product read
  for (int e = tid; e < 2 * 2 * 256; e += 512) {
    const int b = e >> 9, t = (e >> 8) & 1, rr = (e >> 4) & 15, cc = e & 15;
    sm.buf[b].pm[(32 * t + rr) * kLDC + skpos(32 * t + 16 + cc)] = (bf16)0.f;
  }

  ChunkItem itm = p.pass == kPassHandoff ? run_item(p) : decode_item(p, 1);
  if (itm.skip) return;  // uniform: the whole workgroup
  if (itm.wait) itm.poison = !await_state(p, itm.wait, tid, &sm.handoff_arrived);
  const int nblk = (int)((itm.len + kC - 1) / kC);

  // The two roles run separate loops with the same barriers (one before the
  // loop, two per iteration) and leave them at the same iteration: every wave
  // reads the same LDS flag after the same barrier.  In iteration it the
  // producers build window it into buf[it & 1] while the consumers run window
  // it - 1 from buf[(it - 1) & 1].
  if (w >= 4)
    producer_loop<GATE>(p, itm, sm, w - 4, lane, nblk);
  else
    consumer_loop<GATE>(p, itm, sm, w, lane);
  if (itm.signal) publish_state(itm.signal, tid);
}

}  // namespace

hipError_t launch_chunk_fwd_pipe(const ChunkParams &p, int64_t items, hipStream_t stream) {
  if (p.gate)
    hipLaunchKernelGGL(chunk_fwd_pipe_kernel<true>, dim3((unsigned)items), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL(chunk_fwd_pipe_kernel<false>, dim3((unsigned)items), dim3(512), 0, stream,
                       p);
  return hipGetLastError();
}

}  // namespace kda
