// kda_api.cpp -- the extern "C" entry points declared in include/kda.h:
// host-side validation (before anything is enqueued), workspace planning and
// dispatch to the HIP launchers.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "kda_chunk_common.h"
#include "kda_internal.h"

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p & (n - 1)) == 0; }
bool valid_dtype(kda_dtype d) { return d == KDA_F32 || d == KDA_BF16; }

kda_status launch_status(hipError_t e) { return e == hipSuccess ? KDA_SUCCESS : KDA_ERROR_LAUNCH; }

// The gate and beta front end: a known mode, A_log present in the gate mode,
// the bound inside the range the prefill's exponent bounds are derived for.
kda_status check_gate(const kda_gate &g, bool check_pointers) {
  if (g.mode != KDA_GATE_LOG_DECAY && g.mode != KDA_GATE_LOWER_BOUND)
    return KDA_ERROR_INVALID_VALUE;
  if (g.beta_logits != 0 && g.beta_logits != 1) return KDA_ERROR_INVALID_VALUE;
  if (g.mode == KDA_GATE_LOWER_BOUND) {
    if (!(g.lower_bound >= -5.f && g.lower_bound <= 0.f)) return KDA_ERROR_INVALID_VALUE;
    if (check_pointers) {
      if (!g.A_log || !aligned(g.A_log, 4)) return KDA_ERROR_INVALID_VALUE;
      if (g.dt_bias && !aligned(g.dt_bias, 4)) return KDA_ERROR_INVALID_VALUE;
    }
  }
  return KDA_SUCCESS;
}

// Shared checks of the prefill arguments; fills the token count on success.
// The workspace query reads sizes only, so it skips the pointer checks.
constexpr int32_t kMaxHeads = 65536;

kda_status check_chunk_args(const kda_chunk_fwd_args *a, int64_t *total_tokens,
                            bool check_pointers) {
  if (!a) return KDA_ERROR_INVALID_VALUE;
  if (a->num_seqs < 1 || a->num_heads < 1) return KDA_ERROR_INVALID_VALUE;
  if (!valid_dtype(a->io_dtype)) return KDA_ERROR_INVALID_VALUE;
  if (!isfinite(a->scale)) return KDA_ERROR_INVALID_VALUE;
  if (a->segments < 0) return KDA_ERROR_INVALID_VALUE;
  if (a->head_dim != KDA_HEAD_DIM || a->chunk_size != KDA_CHUNK) return KDA_ERROR_UNSUPPORTED;
  int64_t T = 0;
  if (a->cu_seqlens) {
    if (!a->cu_seqlens_host || ((uintptr_t)a->cu_seqlens & 3u)) return KDA_ERROR_INVALID_VALUE;
    if (a->cu_seqlens_host[0] != 0) return KDA_ERROR_INVALID_VALUE;
    for (int32_t i = 0; i < a->num_seqs; ++i)
      if (a->cu_seqlens_host[i + 1] < a->cu_seqlens_host[i]) return KDA_ERROR_INVALID_VALUE;
    T = a->cu_seqlens_host[a->num_seqs];
  } else {
    if (a->seq_len < 0) return KDA_ERROR_INVALID_VALUE;
    T = (int64_t)a->num_seqs * a->seq_len;
    if (T > INT32_MAX) return KDA_ERROR_INVALID_VALUE;
  }
  // tokens and (sequence, head) chains in int32; a 64-token chunk of one tensor
  // (64 rows of H x 128 fp32) must stay below 2^32 bytes for the kernels'
  // 32-bit buffer offsets
  if ((int64_t)a->num_seqs * a->num_heads > INT32_MAX / 2) return KDA_ERROR_INVALID_VALUE;
  if (a->num_heads > kMaxHeads) return KDA_ERROR_INVALID_VALUE;
  if (check_gate(a->gate, check_pointers && T > 0) != KDA_SUCCESS) return KDA_ERROR_INVALID_VALUE;
  if (T > 0 && check_pointers) {
    const void *req[] = {a->q, a->k, a->v, a->g, a->o};
    for (const void *p : req)
      if (!p || !aligned16(p)) return KDA_ERROR_INVALID_VALUE;
    if (!a->beta || !aligned(a->beta, 4)) return KDA_ERROR_INVALID_VALUE;
    if (a->o == a->q || a->o == a->k || a->o == a->v) return KDA_ERROR_INVALID_VALUE;
  }
  if (check_pointers) {
    if (a->initial_state && !aligned16(a->initial_state)) return KDA_ERROR_INVALID_VALUE;
    if (a->final_state && !aligned16(a->final_state)) return KDA_ERROR_INVALID_VALUE;
  }
  *total_tokens = T;
  return KDA_SUCCESS;
}

// Checks of the fused-step arguments; the token pointers (q, k, v, g, beta, o)
// are checked only when `tokens` is set.
kda_status check_fused_args(const kda_fused_step_args *a, bool tokens) {
  if (!a) return KDA_ERROR_INVALID_VALUE;
  if (a->batch < 0 || a->num_heads < 1 || a->num_slots < 0) return KDA_ERROR_INVALID_VALUE;
  if (!valid_dtype(a->io_dtype) || !isfinite(a->scale)) return KDA_ERROR_INVALID_VALUE;
  if (a->head_dim != KDA_HEAD_DIM) return KDA_ERROR_UNSUPPORTED;
  if ((int64_t)a->batch * a->num_heads > INT32_MAX) return KDA_ERROR_INVALID_VALUE;
  if (!(a->l2_eps >= 0.f) || !isfinite(a->l2_eps) || !(a->norm_eps >= 0.f) ||
      !isfinite(a->norm_eps))
    return KDA_ERROR_INVALID_VALUE;
  if (a->out_norm != 0 && a->out_norm != 1) return KDA_ERROR_INVALID_VALUE;
  if (check_gate(a->gate, a->batch > 0) != KDA_SUCCESS) return KDA_ERROR_INVALID_VALUE;
  if (!a->state_indices && a->batch > a->num_slots) return KDA_ERROR_INVALID_VALUE;
  if (a->batch > 0) {
    const uintptr_t es = a->io_dtype == KDA_F32 ? 4u : 2u;
    if (tokens) {
      const void *io[] = {a->q, a->k, a->v, a->o};
      for (const void *p : io)
        if (!p || !aligned(p, es)) return KDA_ERROR_INVALID_VALUE;
      if (!a->g || !aligned(a->g, 4) || !a->beta || !aligned(a->beta, 4))
        return KDA_ERROR_INVALID_VALUE;
    }
    if (!a->conv_cache || !aligned(a->conv_cache, es)) return KDA_ERROR_INVALID_VALUE;
    if (!a->conv_weight || !aligned16(a->conv_weight)) return KDA_ERROR_INVALID_VALUE;
    if (a->norm_weight && !aligned(a->norm_weight, 4)) return KDA_ERROR_INVALID_VALUE;
    if (!a->state || !aligned16(a->state)) return KDA_ERROR_INVALID_VALUE;
    if (a->state_indices && ((uintptr_t)a->state_indices & 3u)) return KDA_ERROR_INVALID_VALUE;
  }
  return KDA_SUCCESS;
}

// The backward's arguments: the forward's size and offset rules, then pointers.
kda_status check_bwd_args(const kda_chunk_bwd_args *a, int64_t *total_tokens, int64_t *max_sub,
                          bool check_pointers) {
  if (!a) return KDA_ERROR_INVALID_VALUE;
  kda_chunk_fwd_args f = {};
  f.num_seqs = a->num_seqs;
  f.seq_len = a->seq_len;
  f.cu_seqlens = a->cu_seqlens;
  f.cu_seqlens_host = a->cu_seqlens_host;
  f.num_heads = a->num_heads;
  f.head_dim = a->head_dim;
  f.chunk_size = KDA_CHUNK;
  f.io_dtype = a->io_dtype;
  f.scale = a->scale;
  const kda_status st = check_chunk_args(&f, total_tokens, false);
  if (st != KDA_SUCCESS) return st;
  const int64_t T = *total_tokens;
  int64_t ms = 0;
  for (int32_t n = 0; n < a->num_seqs; ++n) {
    const int64_t len = a->cu_seqlens ? (int64_t)a->cu_seqlens_host[n + 1] - a->cu_seqlens_host[n]
                                      : a->seq_len;
    const int64_t sub = (len + 15) / 16;
    if (sub > ms) ms = sub;
  }
  *max_sub = ms;
  if (T > 0 && check_pointers) {
    const void *in16[] = {a->q, a->k, a->v, a->dO, a->g, a->dq, a->dk, a->dv, a->dg};
    for (const void *p : in16)
      if (!p || !aligned16(p)) return KDA_ERROR_INVALID_VALUE;
    if (!a->beta || !aligned(a->beta, 4) || !a->dbeta || !aligned(a->dbeta, 4))
      return KDA_ERROR_INVALID_VALUE;
    const void *outs[] = {a->dq, a->dk, a->dv, a->dg, a->dbeta};
    const void *ins[] = {a->q, a->k, a->v, a->dO, a->g, a->beta};
    for (const void *o : outs)
      for (const void *i : ins)
        if (o == i) return KDA_ERROR_INVALID_VALUE;
  }
  if (check_pointers) {
    if (a->initial_state && !aligned16(a->initial_state)) return KDA_ERROR_INVALID_VALUE;
    if (a->dfinal_state && !aligned16(a->dfinal_state)) return KDA_ERROR_INVALID_VALUE;
    if (a->dinitial_state && !aligned16(a->dinitial_state)) return KDA_ERROR_INVALID_VALUE;
  }
  return KDA_SUCCESS;
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status s) {
  switch (s) {
    case KDA_SUCCESS: return "KDA_SUCCESS";
    case KDA_ERROR_INVALID_VALUE: return "KDA_ERROR_INVALID_VALUE";
    case KDA_ERROR_UNSUPPORTED: return "KDA_ERROR_UNSUPPORTED";
    case KDA_ERROR_WORKSPACE: return "KDA_ERROR_WORKSPACE";
    case KDA_ERROR_LAUNCH: return "KDA_ERROR_LAUNCH";
  }
  return "KDA_ERROR_UNKNOWN";
}

const char *kda_version(void) { return "libkda 0.2 (gfx950)"; }

size_t kda_state_bytes(int32_t num_heads, int32_t head_dim, kda_dtype dtype) {
  if (num_heads < 1 || head_dim < 1 || !valid_dtype(dtype)) return 0;
  return (size_t)num_heads * head_dim * head_dim * (dtype == KDA_F32 ? 4u : 2u);
}

kda_status kda_chunk_fwd_workspace_size(const kda_chunk_fwd_args *a, size_t *bytes) {
  if (!bytes) return KDA_ERROR_INVALID_VALUE;
  int64_t T = 0;
  const kda_status st = check_chunk_args(a, &T, false);
  if (st != KDA_SUCCESS) return st;
  kda::ChunkPlan plan;
  const kda_status ps = kda::plan_chunk_fwd(*a, &plan);
  if (ps != KDA_SUCCESS) return ps;
  *bytes = plan.total_bytes;
  return KDA_SUCCESS;
}

kda_status kda_chunk_fwd(const kda_chunk_fwd_args *a, void *stream) {
  int64_t T = 0;
  const kda_status st = check_chunk_args(a, &T, true);
  if (st != KDA_SUCCESS) return st;
  kda::ChunkPlan plan;
  const kda_status ps = kda::plan_chunk_fwd(*a, &plan);
  if (ps != KDA_SUCCESS) return ps;
  if (plan.total_bytes > 0) {
    if (!a->workspace || a->workspace_bytes < plan.total_bytes) return KDA_ERROR_WORKSPACE;
    if (((uintptr_t)a->workspace & 255u) != 0) return KDA_ERROR_INVALID_VALUE;
  }
  return launch_status(kda::launch_chunk_fwd(*a, plan, (hipStream_t)stream));
}

kda_status kda_chunk_fwd_no_alloc(const kda_chunk_fwd_args *a, void *stream) {
  int64_t T = 0;
  const kda_status st = check_chunk_args(a, &T, true);
  if (st != KDA_SUCCESS) return st;
  kda::ChunkPlan plan;
  const kda_status ps = kda::plan_chunk_fwd(*a, &plan);
  if (ps != KDA_SUCCESS) return ps;
  if (plan.total_bytes > kda::kNoAllocScratchBytes) return KDA_ERROR_WORKSPACE;
  kda_chunk_fwd_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (plan.total_bytes > 0) {
    if (kda::no_alloc_scratch(&b.workspace) != hipSuccess) return KDA_ERROR_LAUNCH;
    b.workspace_bytes = kda::kNoAllocScratchBytes;
  }
  return launch_status(kda::launch_chunk_fwd(b, plan, (hipStream_t)stream));
}

size_t kda_chunk_fwd_no_alloc_max_workspace(void) { return kda::kNoAllocScratchBytes; }

kda_status kda_device_status(void *stream, int32_t clear, uint32_t *bits) {
  if (!bits) return KDA_ERROR_INVALID_VALUE;
  uint32_t v = 0;
  const hipError_t e = kda::read_device_status((hipStream_t)stream, clear != 0, &v);
  if (e != hipSuccess) return KDA_ERROR_LAUNCH;
  *bits = v;
  return KDA_SUCCESS;
}

kda_status kda_set_handoff_poll_limit(int32_t polls) {
  if (polls < 0) return KDA_ERROR_INVALID_VALUE;
  kda::set_handoff_poll_limit(polls);
  return KDA_SUCCESS;
}

int32_t kda_handoff_poll_limit(void) { return kda::handoff_poll_limit(); }

kda_status kda_balanced_schedule(int32_t num_seqs, int32_t seq_len, int32_t num_heads,
                                 int32_t compute_units, int32_t *items, int64_t capacity,
                                 int64_t *count) {
  if (!count || num_seqs < 1 || seq_len < 0 || num_heads < 1 || compute_units < 1)
    return KDA_ERROR_INVALID_VALUE;
  const int64_t chains = (int64_t)num_seqs * num_heads;
  const int64_t n = ((int64_t)seq_len + KDA_CHUNK - 1) / KDA_CHUNK;
  if (chains >= ((int64_t)1 << 30)) return KDA_ERROR_INVALID_VALUE;
  kda::ChunkPlan plan;
  *count = 0;
  if (!kda::balanced_schedule_applies(chains, n, compute_units, &plan)) return KDA_SUCCESS;
  const int64_t blocks = plan.ho_workers * plan.ho_rounds;
  *count = blocks;
  if (!items) return KDA_SUCCESS;
  if (capacity < blocks) return KDA_ERROR_INVALID_VALUE;
  for (int64_t b = 0; b < blocks; ++b) {
    const kda::RunItem it = kda::run_item_at((int)chains, (int)n, (int)plan.ho_len, (int)b);
    int32_t *o = items + 5 * b;
    o[0] = it.chain;
    o[1] = it.c0;
    o[2] = it.c1;
    o[3] = it.chain < 0 ? 0 : it.role;
    o[4] = it.chain >= 0 && it.role == 2 ? it.w - 1 : -1;
  }
  return KDA_SUCCESS;
}

kda_status kda_chunk_bwd_workspace_size(const kda_chunk_bwd_args *a, size_t *bytes) {
  if (!bytes) return KDA_ERROR_INVALID_VALUE;
  int64_t T = 0, ms = 0;
  const kda_status st = check_bwd_args(a, &T, &ms, false);
  if (st != KDA_SUCCESS) return st;
  *bytes = kda::chunk_bwd_workspace_bytes(T, a->num_seqs, a->num_heads);
  return KDA_SUCCESS;
}

kda_status kda_chunk_bwd_min_workspace_size(const kda_chunk_bwd_args *a, size_t *bytes) {
  if (!bytes) return KDA_ERROR_INVALID_VALUE;
  int64_t T = 0, ms = 0;
  const kda_status st = check_bwd_args(a, &T, &ms, false);
  if (st != KDA_SUCCESS) return st;
  *bytes = kda::chunk_bwd_min_workspace_bytes(*a);
  return KDA_SUCCESS;
}

kda_status kda_chunk_bwd(const kda_chunk_bwd_args *a, void *stream) {
  int64_t T = 0, ms = 0;
  const kda_status st = check_bwd_args(a, &T, &ms, true);
  if (st != KDA_SUCCESS) return st;
  const size_t need = kda::chunk_bwd_min_workspace_bytes(*a);
  if (T > 0 && (!a->workspace || a->workspace_bytes < need)) return KDA_ERROR_WORKSPACE;
  if (((uintptr_t)a->workspace & 255u) != 0) return KDA_ERROR_INVALID_VALUE;
  return launch_status(kda::launch_chunk_bwd(*a, T, ms, (hipStream_t)stream));
}

kda_status kda_recurrent_step(const kda_recurrent_step_args *a, void *stream) {
  if (!a) return KDA_ERROR_INVALID_VALUE;
  if (a->batch < 0 || a->num_heads < 1 || a->num_slots < 0) return KDA_ERROR_INVALID_VALUE;
  if (!valid_dtype(a->io_dtype) || !isfinite(a->scale)) return KDA_ERROR_INVALID_VALUE;
  if (a->head_dim != KDA_HEAD_DIM) return KDA_ERROR_UNSUPPORTED;
  if ((int64_t)a->batch * a->num_heads > INT32_MAX) return KDA_ERROR_INVALID_VALUE;
  if (check_gate(a->gate, a->batch > 0) != KDA_SUCCESS) return KDA_ERROR_INVALID_VALUE;
  if (!a->state_indices && a->batch > a->num_slots) return KDA_ERROR_INVALID_VALUE;
  if (a->batch > 0) {
    // the step reads q, k, v, g, beta and writes o element by element; the state
    // is accessed in 16-byte vectors
    const uintptr_t es = a->io_dtype == KDA_F32 ? 4u : 2u;
    const void *io[] = {a->q, a->k, a->v, a->o};
    for (const void *p : io)
      if (!p || !aligned(p, es)) return KDA_ERROR_INVALID_VALUE;
    if (!a->g || !aligned(a->g, 4) || !a->beta || !aligned(a->beta, 4))
      return KDA_ERROR_INVALID_VALUE;
    if (!a->state || !aligned16(a->state)) return KDA_ERROR_INVALID_VALUE;
    if (a->state_indices && ((uintptr_t)a->state_indices & 3u)) return KDA_ERROR_INVALID_VALUE;
  }
  return launch_status(kda::launch_recurrent_step(*a, (hipStream_t)stream));
}

size_t kda_conv_cache_bytes(int32_t num_heads, int32_t head_dim, kda_dtype dtype) {
  if (num_heads < 1 || head_dim < 1 || !valid_dtype(dtype)) return 0;
  return (size_t)3 * (KDA_CONV_WIDTH - 1) * num_heads * head_dim * (dtype == KDA_F32 ? 4u : 2u);
}

kda_status kda_fused_decode_step(const kda_fused_step_args *a, void *stream) {
  const kda_status st = check_fused_args(a, true);
  if (st != KDA_SUCCESS) return st;
  return launch_status(kda::launch_fused_decode_step(*a, (hipStream_t)stream));
}

kda_status kda_spec_verify_step(const kda_spec_verify_args *v, void *stream) {
  if (!v) return KDA_ERROR_INVALID_VALUE;
  if (v->window < 0 || v->replay_window < 0) return KDA_ERROR_INVALID_VALUE;
  const kda_status st = check_fused_args(&v->step, v->window > 0);
  if (st != KDA_SUCCESS) return st;
  const kda_fused_step_args &a = v->step;
  const int64_t tmax = v->window > v->replay_window ? v->window : v->replay_window;
  if ((int64_t)a.batch * tmax * a.num_heads > INT32_MAX) return KDA_ERROR_INVALID_VALUE;
  if (a.batch > 0 && v->replay_window > 0) {
    const uintptr_t es = a.io_dtype == KDA_F32 ? 4u : 2u;
    const void *io[] = {v->replay_q, v->replay_k, v->replay_v};
    for (const void *p : io)
      if (!p || !aligned(p, es)) return KDA_ERROR_INVALID_VALUE;
    if (!v->replay_g || !aligned(v->replay_g, 4) || !v->replay_beta ||
        !aligned(v->replay_beta, 4))
      return KDA_ERROR_INVALID_VALUE;
  }
  if (v->num_replay && ((uintptr_t)v->num_replay & 3u)) return KDA_ERROR_INVALID_VALUE;
  return launch_status(kda::launch_spec_verify(*v, (hipStream_t)stream));
}

kda_status kda_state_io(kda_state_op op, const void *src, kda_dtype src_dtype,
                        int32_t src_slots, void *dst, kda_dtype dst_dtype, int32_t dst_slots,
                        const int32_t *indices, int32_t count, int32_t num_heads,
                        int32_t head_dim, void *stream) {
  if (op != KDA_STATE_ZERO && op != KDA_STATE_COPY && op != KDA_STATE_GATHER &&
      op != KDA_STATE_SCATTER)
    return KDA_ERROR_INVALID_VALUE;
  if (count < 0 || num_heads < 1 || src_slots < 0 || dst_slots < 0)
    return KDA_ERROR_INVALID_VALUE;
  if (!valid_dtype(dst_dtype) || (op != KDA_STATE_ZERO && !valid_dtype(src_dtype)))
    return KDA_ERROR_INVALID_VALUE;
  if (head_dim != KDA_HEAD_DIM) return KDA_ERROR_UNSUPPORTED;
  if ((int64_t)count * num_heads > INT32_MAX) return KDA_ERROR_INVALID_VALUE;  // one workgroup per head
  if (count == 0) return KDA_SUCCESS;
  if (!dst || !aligned16(dst)) return KDA_ERROR_INVALID_VALUE;
  if (op != KDA_STATE_ZERO && (!src || !aligned16(src))) return KDA_ERROR_INVALID_VALUE;
  if ((op == KDA_STATE_GATHER || op == KDA_STATE_SCATTER) && !indices)
    return KDA_ERROR_INVALID_VALUE;
  if (indices && ((uintptr_t)indices & 3u)) return KDA_ERROR_INVALID_VALUE;
  // the positions i themselves index a pool: they must lie inside it
  if (op == KDA_STATE_COPY && (count > src_slots || count > dst_slots))
    return KDA_ERROR_INVALID_VALUE;
  if (op == KDA_STATE_GATHER && count > dst_slots) return KDA_ERROR_INVALID_VALUE;
  if (op == KDA_STATE_SCATTER && count > src_slots) return KDA_ERROR_INVALID_VALUE;
  if (op == KDA_STATE_ZERO && !indices && count > dst_slots) return KDA_ERROR_INVALID_VALUE;
  if (op != KDA_STATE_ZERO) {
    // source and destination ranges must not overlap
    const size_t sb = kda_state_bytes(num_heads, head_dim, src_dtype) * (size_t)src_slots;
    const size_t db = kda_state_bytes(num_heads, head_dim, dst_dtype) * (size_t)dst_slots;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (s0 < d0 + db && d0 < s0 + sb) return KDA_ERROR_INVALID_VALUE;
  }
  return launch_status(kda::launch_state_io(op, src, src_dtype, src_slots, dst, dst_dtype,
                                            dst_slots, indices, count, num_heads,
                                            (hipStream_t)stream));
}

}  // extern "C"
