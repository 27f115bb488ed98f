// Host check of the prefill kernel's LDS layouts (kda_pipe_layout.h): every
// layout is a bijection onto its buffer, the per-lane offsets the kernel steps
// through equal the layout functions, and every access the kernel makes with
// them has conflict degree 1 under gfx950's bank rules as the header states
// them (bank period and lane groups per instruction kind).  Prints "ok" and
// exits 0 on success.  Built and run by tests/test_lds_layout_host.py.
#include <algorithm>
#include <cstdio>
#include <map>
#include <set>
#include <vector>

#include "kda_pipe_layout.h"

using namespace kda::layout;

static int fails = 0;
#define CHECK(c, ...)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      if (fails < 20) {                                 \
        std::printf("FAIL line %d: ", __LINE__);        \
        std::printf(__VA_ARGS__);                       \
        std::printf("\n");                              \
      }                                                 \
      ++fails;                                          \
    }                                                   \
  } while (0)

enum Kind { READ64, READ128, WRITE64, WRITE128 };  // the transposing read is READ64

// Largest number of distinct dwords one bank serves in one lane group of a wave
// instruction; addr[lane] = byte address.
static int conflict_degree(const std::vector<long> &addr, Kind kind) {
  std::vector<std::vector<int>> groups;
  auto consecutive = [&](int n) {
    for (int g = 0; g < 64 / n; ++g) {
      std::vector<int> v;
      for (int l = 0; l < n; ++l) v.push_back(g * n + l);
      groups.push_back(v);
    }
  };
  if (kind == READ64) consecutive(32);
  if (kind == WRITE64) consecutive(16);
  if (kind == WRITE128) consecutive(8);
  if (kind == READ128) {
    for (int h = 0; h < 2; ++h) {
      std::vector<int> a, b;
      for (int l = 0; l < 32; ++l) {
        const int q = l / 4;
        ((q == 0 || q == 3 || q == 5 || q == 6) ? a : b).push_back(32 * h + l);
      }
      groups.push_back(a);
      groups.push_back(b);
    }
  }
  const int width = (kind == READ128 || kind == WRITE128) ? 16 : 8;
  const int period = (kind == WRITE64 || kind == WRITE128) ? 128 : 256;
  int worst = 1;
  for (const auto &g : groups) {
    std::map<int, std::set<long>> bank;
    for (int l : g)
      for (int b = 0; b < width; b += 4) bank[((addr[l] + b) % period) / 4].insert((addr[l] + b) / 4);
    for (const auto &kv : bank) worst = std::max(worst, (int)kv.second.size());
  }
  return worst;
}

static void bijection(const char *name, int rows, int cols, int (*at)(int, int), int quad) {
  std::set<int> seen;
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) {
      const int o = at(r, c);
      CHECK(o >= 0 && o < rows * cols, "%s(%d, %d) = %d out of range", name, r, c, o);
      CHECK(at(r, c - c % quad) + c % quad == o, "%s: group of %d not contiguous at (%d, %d)", name, quad, r, c);
      seen.insert(o);
    }
  CHECK((int)seen.size() == rows * cols, "%s is not a bijection", name);
}

int main() {
  bijection("opnd_at", 64, 128, opnd_at, 4);
  bijection("v_at", 64, 128, v_at, 8);
  bijection("stage_at", 64, 32, stage_at, 4);
  int worst = 1;
  auto note = [&](const std::vector<long> &a, Kind k, const char *what) {
    const int d = conflict_degree(a, k);
    CHECK(d == 1, "%s: conflict degree %d", what, d);
    worst = std::max(worst, d);
  };
  // producer stores: wave pw, lane (ts = lane / 16, co = lane % 16), rows r0 + j
  for (int pw = 0; pw < 4; ++pw)
    for (int j = 0; j < 4; ++j) {
      std::vector<long> qa(64), qb(64), va(64);
      for (int lane = 0; lane < 64; ++lane) {
        const int ts = lane >> 4, co = lane & 15, r0 = 16 * pw + 4 * ts;
        const int oa = opnd_row_step(opnd_at(r0, 8 * co), j), ob = opnd_row_step(opnd_at(r0, 8 * co + 4), j);
        const int ov = v_row_step(v_at(r0, 8 * co), j);
        CHECK(oa == opnd_at(r0 + j, 8 * co) && ob == opnd_at(r0 + j, 8 * co + 4), "operand store pw %d j %d", pw, j);
        CHECK(ov == v_at(r0 + j, 8 * co), "v store pw %d j %d", pw, j);
        qa[lane] = 2L * oa;
        qb[lane] = 2L * ob;
        va[lane] = 2L * ov;
      }
      note(qa, WRITE64, "operand store, first quad");
      note(qb, WRITE64, "operand store, second quad");
      note(va, WRITE128, "v store");
    }
  // fragment reads: lane (l16, g), tile t, channel block kk; chunk order by g
  for (int t = 0; t < 4; ++t)
    for (int kk = 0; kk < 4; ++kk) {
      std::vector<long> a(64);
      for (int lane = 0; lane < 64; ++lane) {
        const int l16 = lane & 15, g = lane >> 4, row = 16 * t + l16;
        const int off = frag_step(frag_lane(l16, g), t, kk);
        const bool upper_first = (g >> 1) & 1;
        const int lo = opnd_at(row, 32 * kk + 4 * g), hi = opnd_at(row, 32 * kk + 16 + 4 * g);
        CHECK(off % 8 == 0 && (upper_first ? hi : lo) == off && (upper_first ? lo : hi) == off + 4,
              "fragment t %d kk %d lane %d", t, kk, lane);
        a[lane] = 2L * off;
      }
      note(a, READ128, "fragment read");
    }
  // transposing reads of Kc
  for (int ct = 0; ct < 8; ++ct)
    for (int kk = 0; kk < 2; ++kk)
      for (int hh = 0; hh < 2; ++hh) {
        std::vector<long> a(64);
        for (int lane = 0; lane < 64; ++lane) {
          const int l16 = lane & 15, g4 = lane >> 4;
          const int off = kc_tr_step(kc_tr_lane(l16, g4), ct, kk, hh);
          CHECK(off == opnd_at(32 * kk + 16 * hh + 4 * g4 + (l16 >> 2), 16 * ct + 4 * (l16 & 3)),
                "Kc transposing read ct %d lane %d", ct, lane);
          a[lane] = 2L * off;
        }
        note(a, READ64, "Kc transposing read");
      }
  // transposing reads of v, consumer wave cw
  for (int cw = 0; cw < 4; ++cw)
    for (int s4 = 0; s4 < 4; ++s4)
      for (int c2 = 0; c2 < 2; ++c2) {
        std::vector<long> a(64);
        for (int lane = 0; lane < 64; ++lane) {
          const int l16 = lane & 15, g4 = lane >> 4, vcol = 32 * cw;
          const int off = v_tr_step(v_tr_lane(l16, g4, vcol), s4, c2);
          CHECK(off == v_at(16 * s4 + 4 * g4 + (l16 >> 2), vcol + 16 * c2 + 4 * (l16 & 3)), "v transposing read");
          a[lane] = 2L * off;
        }
        note(a, READ64, "v transposing read");
      }
  // o staging
  for (int rt = 0; rt < 4; ++rt)
    for (int c2 = 0; c2 < 2; ++c2) {
      std::vector<long> a(64);
      for (int lane = 0; lane < 64; ++lane) {
        const int l16 = lane & 15, g4 = lane >> 4;
        const int off = stage_w_step(stage_w_lane(l16, g4), rt, c2);
        CHECK(off == stage_at(16 * rt + l16, 16 * c2 + 4 * g4), "staging store");
        a[lane] = 2L * off;
      }
      note(a, WRITE64, "staging store");
    }
  for (int k = 0; k < 4; ++k) {
    std::vector<long> a(64);
    for (int lane = 0; lane < 64; ++lane) {
      const int l16 = lane & 15, g4 = lane >> 4;
      const int off = stage_r_step(stage_r_lane(l16, g4), k);
      const bool sw = stage_swapped(l16);
      const int q0 = stage_at(16 * k + l16, 8 * g4), q1 = stage_at(16 * k + l16, 8 * g4 + 4);
      CHECK(off % 8 == 0 && (sw ? q1 : q0) == off && (sw ? q0 : q1) == off + 4, "staging read lane %d", lane);
      a[lane] = 2L * off;
    }
    note(a, READ128, "staging read");
  }
  // the rules themselves, on two patterns the old padded layout had: a 272-byte
  // row stride conflicts two ways for fragment reads and 64-bit row stores
  {
    std::vector<long> a(64), b(64);
    for (int l = 0; l < 64; ++l) {
      a[l] = 272L * (l % 16) + 64 * (l / 16);
      b[l] = 144L * (l % 16) + 8 * (l / 16);
    }
    CHECK(conflict_degree(a, READ128) == 2, "rule check: padded fragment read");
    CHECK(conflict_degree(b, WRITE64) == 2, "rule check: 144-byte row store");
  }
  std::printf("worst conflict degree %d; %s\n", worst, fails ? "FAILED" : "ok");
  return fails != 0;
}
