// kda_pipe_layout.h -- LDS layouts of the bf16 prefill kernel (kda_chunk_pipe.hip):
// the operand matrices nKr, Qr, Kc, the chunk's v, and the o staging area, as
// element offsets, plus the per-lane offsets the kernel steps through with one
// XOR per unrolled index.  Plain constexpr integer functions, so a host program
// (tests/lds_layout_check.cpp) checks the same definitions the kernel uses.
//
// gfx950's LDS, as measured with single-instruction access patterns: 64
// four-byte banks (a 256-byte period) for 64- and 128-bit reads and the
// transposing read, a 128-byte period for writes; a wave's access is served in
// lane groups, one per cycle -- 32 consecutive lanes for 64-bit and transposing
// reads, 16 for 64-bit writes, 8 for 128-bit writes, and for 128-bit reads the
// lanes {0-3, 12-15, 20-23, 24-27} and {4-11, 16-19, 28-31} of each half-wave.
// Two lanes of one group on one bank at different addresses cost a cycle; a
// same-address broadcast is free.  Every layout below gives each access of the
// kernel distinct banks within each group.
#pragma once

#if defined(__HIPCC__)
#define KDA_HD __host__ __device__
#else
#define KDA_HD
#endif

namespace kda {
namespace layout {

constexpr int kRow = 128;  // row stride of the operand matrices and v, in bf16 (no padding)

// Operand matrices: row r holds 128 channels in 16 chunks of 16 bytes.  Chunk
// (kk, g) -- channels 32 kk + 4 g + e of the lower and 32 kk + 16 + 4 g + e of the
// upper 16-channel tile, the 8 channels a matrix-core fragment over channels
// 32 kk .. 32 kk + 31 gives lane group g -- sits at slot (kk + 4 pi(g)) ^ (r & 15),
// pi = (0, 3, 1, 2), the upper tile's quad first for g = 2, 3 (the order may
// depend on g alone: a product sums the channels of two different rows).  Then
//  - a fragment read (16 rows, one chunk each) covers all 16 slots within each
//    128-bit read group;
//  - a producer's row store (16 lanes, one channel quad each) fills 128 bytes;
//  - the transposing reads of Kc (8 rows x the 4 quads of a 16-channel tile per
//    32 lanes) meet every bank once: rows 4 apart share a slot, and pi and the
//    quad order put them in opposite halves.
KDA_HD constexpr int gperm(int g) { return ((g & 1) << 1) | ((g ^ (g >> 1)) & 1); }
KDA_HD constexpr int opnd_at(int r, int c) {
  return kRow * r + 8 * (((c >> 5) + 4 * gperm((c >> 2) & 3)) ^ (r & 15)) +
         4 * (((c >> 4) & 1) ^ ((c >> 3) & 1)) + (c & 3);
}
// v: chunk j (channels 8 j .. 8 j + 7) of row r at slot j ^ 2 (r & 7): the
// transposing reads (8 rows x 32 bytes per 32 lanes) and the producers' row
// stores (8 lanes x 16 bytes) meet every bank once.
KDA_HD constexpr int v_at(int r, int c) { return kRow * r + 8 * ((c >> 3) ^ (2 * (r & 7))) + (c & 7); }
// o staging, one consumer wave's 64 rows x 32 columns (4 KB): quad q = c / 4 of
// row r at 8-byte slot 2 ((q / 2) ^ ((r / 2) & 3)) + ((q & 1) ^ ((r / 8) & 1)) of
// the row's 64 bytes.  The 16 rows of one quad, written at once, fill 128
// bytes; the 16-byte reads of two quads of 16 rows meet every bank once (the
// two quads come swapped in rows with bit 3 set).
KDA_HD constexpr int stage_at(int r, int c) {
  return 32 * r + 8 * (((c >> 3) & 3) ^ ((r >> 1) & 3)) + 4 * (((c >> 2) & 1) ^ ((r >> 3) & 1)) +
         (c & 3);
}

// ---------------------------------------------------------------- lane offsets
// Lane (l16, g) of a matrix-core fragment read: chunk (kk, g) of row 16 t + l16
// is at frag_step(frag_lane(l16, g), t, kk).
KDA_HD constexpr int frag_lane(int l16, int g) { return kRow * l16 + 8 * ((4 * gperm(g)) ^ l16); }
KDA_HD constexpr int frag_step(int f0, int t, int kk) { return 16 * kRow * t + (f0 ^ (8 * kk)); }
// Producer lane (ts, co) of wave pw, rows r0 + j (r0 = 16 pw + 4 ts): with
// p = opnd_at(r0, c) for its quads c = 8 co, 8 co + 4 (resp. v_at(r0, 8 co)),
// row r0 + j is at opnd_row_step(p, j) (resp. v_row_step).
KDA_HD constexpr int opnd_row_step(int p, int j) { return (p ^ (8 * j)) + kRow * j; }
KDA_HD constexpr int v_row_step(int p, int j) { return (p ^ (16 * j)) + kRow * j; }
// Transposing reads of Kc by lane (l16, g4): channels 16 ct + 4 (l16 & 3) of row
// 32 kk + 16 hh + 4 g4 + l16 / 4.
KDA_HD constexpr int kc_tr_lane(int l16, int g4) { return opnd_at(4 * g4 + (l16 >> 2), 4 * (l16 & 3)); }
KDA_HD constexpr int kc_tr_step(int k0, int ct, int kk, int hh) {
  return 32 * kRow * kk + 16 * kRow * hh + (k0 ^ (4 * ct));
}
// Transposing reads of v by lane (l16, g4) of the consumer wave owning columns
// vcol .. vcol + 31: columns vcol + 16 c2 + 4 (l16 & 3) of row 16 s4 + 4 g4 + l16 / 4.
KDA_HD constexpr int v_tr_lane(int l16, int g4, int vcol) {
  return v_at(4 * g4 + (l16 >> 2), vcol + 4 * (l16 & 3));
}
KDA_HD constexpr int v_tr_step(int v0, int s4, int c2) { return 16 * kRow * s4 + (v0 ^ (16 * c2)); }
// o staging by lane (l16, g4): stores of columns 16 c2 + 4 g4 of row 16 rt + l16;
// 16-byte reads of columns 8 g4 .. 8 g4 + 7 of row 16 k + l16 (quads swapped
// where stage_swapped).
KDA_HD constexpr int stage_w_lane(int l16, int g4) { return stage_at(l16, 4 * g4); }
KDA_HD constexpr int stage_w_step(int s0, int rt, int c2) { return 512 * rt + (s0 ^ (16 * c2)); }
KDA_HD constexpr int stage_r_lane(int l16, int g4) { return stage_at(l16, 8 * g4) & ~4; }
KDA_HD constexpr int stage_r_step(int s0, int k) { return 512 * k + s0; }
KDA_HD constexpr bool stage_swapped(int l16) { return (l16 >> 3) & 1; }

}  // namespace layout
}  // namespace kda
