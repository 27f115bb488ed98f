// kda_chunk_common.h -- what the prefill kernels share: launch parameters, the
// mapping of a workgroup to its (sequence, head[, segment]) work item, and the
// column permutation of the split-k operand layout.
#pragma once

#include "kda.h"
#include "kda_device.h"

namespace kda {

constexpr int kC = KDA_CHUNK;     // 64 tokens per chunk
constexpr int kD = KDA_HEAD_DIM;  // 128 channels
constexpr int kMaxSegments = 64;  // segments per sequence (segment parallelism)

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
  // segment parallelism: each sequence is split into seg_P segments of whole
  // chunks; pass 0 = no split, 1 = first pass, 2 = second pass
  int32_t seg_P;
  int32_t pass;
  float *ws;             // [N H][3 seg_P][128 x 128] fp32 segment states
  // chains of this launch: ranks chain0 .. chain0 + nchains - 1 in the
  // (sequence rank, head) order; seg_front: segment 0 takes two shares of the
  // chunks, the others one each (the first pass's runs then last as long as
  // two rounds of its transition items)
  int32_t chain0, nchains;
  int32_t seg_front;
  // gate front end: with gate != 0, g holds gate logits of the lower-bounded
  // gate (A_log [H], dt_bias [H][128] or null, gate_scale = lower_bound log2 e);
  // with beta_logits != 0, beta holds logits
  const float *A_log, *dt_bias;
  float gate_scale;
  int32_t gate, beta_logits;
  // balanced schedule of equal-length chains (pass kPassHandoff): the chains'
  // chunks laid end to end are cut into runs of ho_len chunks, one per
  // workgroup; a chain cut in two hands its state over through ho_state
  float *ho_state;       // [workgroups][128 x 128] fp32 handed-over states
  int32_t *ho_flag;      // [workgroups] set to 1 once that state is stored
  int64_t ho_len;        // chunks per workgroup
  int32_t ho_polls;      // polls of a hand-over flag before a tail gives up
  uint32_t *status;      // the GPU's status word (KDA_DEVICE_* bits), or null
};

constexpr int kPassHandoff = 3;

// Segment items ("Kimi K3 -- Training and Infrastructure Notes", section 4.1):
// a run evaluates a segment from its incoming state; the two trackers of a
// segment give its transition, M (from S0 = I with v = 0) and S~ (from S0 = 0).
enum SegMode { kRun = 0, kTrackM = 1, kTrackS = 2 };
enum SegKind { kSin = 0, kM = 1, kSt = 2 };  // workspace state kinds

// A sequence of nch chunks is split into P_n = min(P, nch) segments of whole
// chunks (equal shares, or two shares for segment 0, see seg_bounds).
__device__ __forceinline__ int seg_count(int P, int nch) {
  const int pn = P < nch ? P : nch;
  return pn < 1 ? 1 : pn;
}
__device__ __forceinline__ float *seg_state(const ChunkParams &p, int64_t chain, int kind,
                                            int seg) {
  return p.ws + ((chain * 3 + kind) * p.seg_P + seg) * (int64_t)(kD * kD);
}

// Work item of one workgroup: the token range [bos, bos + len) of head h, the
// incoming state (null = zero, or the identity when zero_v), where the final
// state goes (null = nowhere), whether o is written, and the value block.
struct ChunkItem {
  int64_t bos, len, chain;
  int h, vs;
  const float *s0;
  float *sf;
  const int32_t *wait;  // flag to see set before s0 is read (null = none)
  int32_t *signal;      // flag to set once sf is stored (null = none)
  bool write_o, zero_v, skip;
  bool poison;          // the incoming state never arrived: start from NaN
};

// Chunks [lo, hi) of segment seg of a sequence of nch chunks split into pn.
__device__ __forceinline__ void seg_bounds(const ChunkParams &p, int seg, int pn, int nch,
                                           int &lo, int &hi) {
  if (p.seg_front) {  // shares 2, 1, 1, ...
    lo = seg == 0 ? 0 : (int)((int64_t)(seg + 1) * nch / (pn + 1));
    hi = (int)((int64_t)(seg + 2) * nch / (pn + 1));
  } else {
    lo = (int)((int64_t)seg * nch / pn);
    hi = (int)((int64_t)(seg + 1) * nch / pn);
  }
}

// blockIdx.x = (segment item * nchains + chain rank - chain0) * VS + value
// block: item-major, so a pass's long runs (item 0) are dispatched first.
__device__ __forceinline__ ChunkItem decode_item(const ChunkParams &p, int VS) {
  ChunkItem r;
  const int item = blockIdx.x;
  r.vs = item % VS;
  const int cit = item / VS;
  const int it = cit / p.nchains;
  const int crank = p.chain0 + (cit - it * p.nchains);
  const int srank = crank / p.H;
  r.h = crank - srank * p.H;
  const int n = p.order ? p.order[srank] : srank;
  int64_t bos = (int64_t)n * p.seq_len, len = p.seq_len;
  if (p.cu) {  // device offsets, clamped to the validated token range
    const int64_t a = p.cu[n], b = p.cu[n + 1];
    bos = a < 0 ? 0 : (a > p.total_tokens ? p.total_tokens : a);
    const int64_t e = b < bos ? bos : (b > p.total_tokens ? p.total_tokens : b);
    len = e - bos;
  }
  r.chain = (int64_t)n * p.H + r.h;
  int seg = 0, mode = kRun;
  if (p.pass == 1 && it > 0) {
    seg = 1 + (it - 1) / 2;
    mode = (it & 1) ? kTrackM : kTrackS;
  } else if (p.pass == 2) {
    seg = 1 + it;
  }
  r.s0 = p.s0 ? p.s0 + r.chain * (kD * kD) : nullptr;
  r.sf = p.sfinal ? p.sfinal + r.chain * (kD * kD) : nullptr;
  r.skip = false;
  if (p.pass != 0) {
    const int nch_all = (int)((len + kC - 1) / kC);
    const int pn = seg_count(p.seg_P, nch_all);
    // trackers exist for the segments 1 .. P_n - 2, runs for 0 .. P_n - 1
    r.skip = mode == kRun ? seg >= pn : seg >= pn - 1;
    int c_lo, c_hi;
    seg_bounds(p, seg, pn, nch_all, c_lo, c_hi);
    const int64_t t_lo = (int64_t)c_lo * kC;
    const int64_t t_hi = (int64_t)c_hi * kC < len ? (int64_t)c_hi * kC : len;
    bos += t_lo;
    len = t_hi > t_lo ? t_hi - t_lo : 0;
    if (mode == kRun) {
      if (seg > 0) r.s0 = seg_state(p, r.chain, kSin, seg);
      r.sf = seg == pn - 1 ? r.sf : (p.pass == 1 ? seg_state(p, r.chain, kSin, 1) : nullptr);
    } else {
      r.s0 = nullptr;
      r.sf = seg_state(p, r.chain, mode == kTrackM ? kM : kSt, seg);
    }
  }
  r.bos = bos;
  r.len = len;
  r.write_o = mode == kRun;
  r.zero_v = mode == kTrackM;
  r.wait = nullptr;
  r.signal = nullptr;
  r.poison = false;
  return r;
}

// Balanced schedule of C chains of n chunks each (fixed-length batch, C above
// the number of compute units).  The chunks of chains 0 .. C-1, laid end to
// end, are cut into W runs of L = ho_len >= n chunks.  Run w starts with the
// tail of a chain cut by run w-1 (or at a chain start), holds whole chains,
// and ends with the head of a chain that run w+1 finishes (or at a chain end);
// since L >= n a chain is cut at most once.  Items are numbered round by
// round, blockIdx.x = k W + w for item k of run w, k = 0 first: the head (its
// state goes to ho_state[w] and ho_flag[w] is set), then the whole chains,
// then the tail (it waits for ho_flag[w-1]).  A tail waits for a head of a
// lower-numbered workgroup, dispatched earlier, that never waits itself.
struct RunShape {
  int c_lo, c_hi;  // first and last chain touched
  int tail0;       // first chunk of the tail of chain c_lo (0: no tail)
  int head1;       // end chunk of the head of chain c_hi (n: no head)
  int count;       // items of the run
};
// 32-bit arithmetic (the host enables the schedule for C n < 2^30 only).
__host__ __device__ inline RunShape run_shape(int nchains, int n, int L, int w) {
  const int total = nchains * n;
  const int s = w * L, e = s + L < total ? s + L : total;
  RunShape r;
  r.c_lo = s / n;
  r.c_hi = (e - 1) / n;
  r.tail0 = s - r.c_lo * n;
  r.head1 = e - r.c_hi * n;
  const int whole = (r.c_hi - (r.head1 < n)) - (r.c_lo + (r.tail0 > 0)) + 1;
  r.count = (r.head1 < n) + (whole > 0 ? whole : 0) + (r.tail0 > 0);
  if (e <= s) r.count = 0;
  return r;
}
// Workgroups of the schedule: W runs, items of round k at k W .. k W + W - 1.
__host__ __device__ inline int run_workers(int nchains, int n, int L) {
  return (nchains * n + L - 1) / L;
}
// Item of workgroup `block`: chunks [c0, c1) of chain `chain` (chain < 0: the
// run has no item in this round), role 1 = head (stores its state for run
// w + 1), 2 = tail (takes the state run w - 1 stores), 0 = whole chain.  The
// kernels and the host's schedule model both take their items from here.
struct RunItem {
  int chain, c0, c1, role, w;
};
__host__ __device__ inline RunItem run_item_at(int nchains, int n, int L, int block) {
  const int W = run_workers(nchains, n, L);
  const int k = block / W, w = block - k * W;
  const RunShape rs = run_shape(nchains, n, L, w);
  RunItem r;
  r.w = w;
  r.chain = -1;
  r.c0 = r.c1 = 0;
  r.role = 0;
  if (k >= rs.count) return r;
  const bool head = rs.head1 < n;
  r.role = head && k == 0 ? 1 : (rs.tail0 > 0 && k == rs.count - 1) ? 2 : 0;
  r.chain = r.role == 1 ? rs.c_hi : r.role == 2 ? rs.c_lo : rs.c_lo + (rs.tail0 > 0) + (k - (int)head);
  r.c0 = r.role == 2 ? rs.tail0 : 0;
  r.c1 = r.role == 1 ? rs.head1 : n;
  return r;
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ ChunkItem run_item(const ChunkParams &p) {
  const int n = (p.seq_len + kC - 1) / kC;
  const RunItem it = run_item_at(p.nchains, n, (int)p.ho_len, (int)blockIdx.x);
  ChunkItem r;
  r.wait = nullptr;
  r.signal = nullptr;
  r.poison = false;
  r.skip = uniform(it.chain) < 0;  // the run has fewer items than this round
  if (r.skip) return r;
  const int role = uniform(it.role), w = uniform(it.w);
  const int chain = uniform(it.chain);
  const int c0 = uniform(it.c0), c1 = uniform(it.c1);
  const int srank = chain / p.H;
  r.h = chain - srank * p.H;
  r.vs = 0;
  r.chain = chain;
  const int t0 = c0 * kC, t1 = c1 * kC < p.seq_len ? c1 * kC : p.seq_len;
  r.bos = (int64_t)srank * p.seq_len + t0;
  r.len = t1 - t0;
  r.s0 = p.s0 ? p.s0 + (int64_t)chain * (kD * kD) : nullptr;
  r.sf = p.sfinal ? p.sfinal + (int64_t)chain * (kD * kD) : nullptr;
  if (role == 1) {
    r.sf = p.ho_state + (int64_t)w * (kD * kD);
    r.signal = p.ho_flag + w;
  } else if (role == 2) {
    r.s0 = p.ho_state + (int64_t)(w - 1) * (kD * kD);
    r.wait = p.ho_flag + (w - 1);
  }
  r.write_o = true;
  r.zero_v = false;
  r.skip = r.len <= 0;
  return r;
}

// Column order of the matrices read as split-k fragments (k = 4g+i and
// 16+4g+i of each 32-column block): stored so that those eight k-values are
// adjacent, each fragment is one 16-byte LDS read.  Groups of four aligned
// columns stay contiguous.
__device__ __forceinline__ int skpos(int c) {
  return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}
// Column held at position p (inverse of skpos).
__device__ __forceinline__ int skcol(int p) {
  return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
}

// Host launchers of the two prefill kernels.
hipError_t launch_chunk_fwd_pipe(const ChunkParams &p, int64_t items, hipStream_t stream);

}  // namespace kda
