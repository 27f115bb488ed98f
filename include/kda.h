/*
 * kda.h -- C ABI of libkda, an MI355X (gfx950) implementation of the Kimi Delta
 * Attention (KDA) token mixer: the chunkwise-parallel prefill forward and the
 * single-token recurrent decode step, plus state-pool copies.
 *
 * Pages this interface follows (cited by title and section):
 *  [P1] "How Kimi K3 Engineered Its Way to the Frontier": section "How KDA
 *       updates its state" (recurrence order forget -> erase+write -> read;
 *       decay per key channel; state layout S[B,HV,K,V], gate g[B,T,HV,K] in
 *       natural-log space); section "What the hybrid saves" (per-layer state of
 *       96 heads x 128 x 128; FlashKDA accepts bf16 or fp32 states); section
 *       "FlashKDA steps the state once per 16 tokens" (chunkwise form, result
 *       equal to the token loop; forward-only prefill with head dim fixed at
 *       128).
 *  [P2] "Kimi K3: Open Frontier Intelligence", section 6: the KDA equation
 *       S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *       o_t = S_t^T q_t.
 *  [P3] "Kimi K3 -- Training and Infrastructure Notes": section 4.1 (segment
 *       transitions evaluated independently of the incoming state and composed
 *       exactly afterwards, inside one device); section 4.5 (decode updates the
 *       state in place; states stored head by head contiguously; checkpoints are
 *       read-only snapshots copied into a private running state).
 *  [P4] "Kimi K3: a 2.8T open model ...", subsection "FlashKDA: the equation,
 *       shipped as a kernel": query, key, value, gate and beta in, optional
 *       recurrent state in and out, variable-length batches through cumulative
 *       sequence lengths, bf16 activations with fp32 parameters.
 *
 * Conventions shared by every entry point
 *  - Layouts are row-major with the innermost index last.  Tokens of all
 *    sequences are packed: q, k, v, o are [T_total, H, 128]; g is
 *    [T_total, H, 128]; beta is [T_total, H]; states are [N, H, 128, 128] with
 *    rows indexed by key channel and columns by value channel, each head's
 *    128 x 128 block contiguous.  A fixed-length batch [B, T, ...] is the same
 *    memory with N = B and T_total = B * T.
 *  - g is the natural-log decay (alpha = exp(g), g <= 0 expected); beta is the
 *    post-sigmoid write strength in [0, 1] -- unless kda_gate says they hold
 *    gate logits or beta logits (below).  o = scale * S_t^T q_t; the pages'
 *    formula has scale = 1.
 *  - Ownership: the caller allocates and owns every buffer (device memory unless
 *    a field says host).  The library allocates no device memory, keeps no
 *    pointer after a call returns and holds no mutable global state -- except
 *    the per-GPU scratch buffer of kda_chunk_fwd_no_alloc (a static device
 *    array reserved when the library is loaded), the per-GPU device status
 *    word (kda_device_status) and the process-wide hand-over poll limit
 *    (kda_set_handoff_poll_limit).
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  Work is enqueued asynchronously; no call synchronises the host.
 *  - Errors: arguments are validated on the host before anything is enqueued.
 *    An invalid call returns a status other than KDA_SUCCESS and touches no
 *    buffer.  A launch failure reported by the HIP runtime returns
 *    KDA_ERROR_LAUNCH.  Values inside device buffers (cu_seqlens contents,
 *    slot indices) cannot be checked on the host; how each call treats bad
 *    device-side values is stated at the call.  No C++ exception crosses the ABI.
 *  - Alignment: state pools and the prefill's q, k, v, g, o must be 16-byte
 *    aligned; beta needs 4 bytes; the decode step's q, k, v, o need their
 *    element size and g 4 bytes.
 *  - Thread safety: calls are reentrant.  Two calls that write the same buffer
 *    must be ordered by the caller (same stream or events).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
  KDA_SUCCESS = 0,
  KDA_ERROR_INVALID_VALUE = 1, /* null pointer, bad size, bad alignment, bad offsets */
  KDA_ERROR_UNSUPPORTED = 2,   /* a valid request the library does not implement    */
  KDA_ERROR_WORKSPACE = 3,     /* workspace missing or smaller than required        */
  KDA_ERROR_LAUNCH = 4         /* the HIP runtime rejected a kernel launch          */
} kda_status;

typedef enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Head dimension (d_k = d_v) and chunk length the library implements. */
#define KDA_HEAD_DIM 128
#define KDA_CHUNK 64

/* ------------------------------------------------------------------------
 * Gate and beta front end, shared by the prefill and the decode step.
 *
 * KDA_GATE_LOG_DECAY: g holds the natural-log decay itself (alpha = exp(g)).
 * KDA_GATE_LOWER_BOUND: g holds raw per-channel gate logits x, and the kernels
 * compute K3's lower-bounded gate ([P1] "How KDA updates its state", the gate
 * that replaces Kimi Linear's softplus gate) on the fly:
 *     g[t, h, c] = lower_bound * sigmoid(exp(A_log[h]) * (x[t, h, c] + dt_bias[h, c]))
 * so every g lies in [lower_bound, 0].  lower_bound * log2(e) is folded into one
 * constant on the host, as [P1] "FlashKDA steps the state once per 16 tokens"
 * describes.
 * beta_logits = 1: beta holds logits and the kernels use sigmoid(beta) ([P4]
 * "FlashKDA: the equation, shipped as a kernel": beta logits pass through a
 * sigmoid); 0: beta is used as given.
 * A zero-initialised kda_gate is the plain mode (log-decay g, beta as given).
 * ---------------------------------------------------------------------- */
typedef enum kda_gate_mode {
  KDA_GATE_LOG_DECAY = 0,
  KDA_GATE_LOWER_BOUND = 1
} kda_gate_mode;

typedef struct kda_gate {
  kda_gate_mode mode;
  const float *A_log;    /* device [H] fp32; required with KDA_GATE_LOWER_BOUND     */
  const float *dt_bias;  /* device [H, 128] fp32, or NULL = no bias                   */
  float lower_bound;     /* KDA_GATE_LOWER_BOUND: in [-5, 0] (the pages use -5; the  */
                         /* prefill's exponent bounds are derived for that floor)     */
  int32_t beta_logits;   /* 0 or 1, see above                                         */
} kda_gate;

/* ------------------------------------------------------------------------
 * Chunkwise prefill forward ([P1] "FlashKDA steps the state once per 16
 * tokens"; [P2] section 6; [P4] "FlashKDA: the equation, shipped as a kernel").
 *
 * For every sequence n and head h, starting from S = initial_state[n, h] (zero
 * when initial_state is NULL) it computes, for each token t of the sequence in
 * order, the KDA recurrence
 *     S <- (I - beta_t k_t k_t^T) Diag(exp(g_t)) S + beta_t k_t v_t^T
 *     o_t = scale * S^T q_t
 * and stores the last S into final_state[n, h].  Tokens are processed in chunks
 * of `chunk_size` that start at each sequence start; the result equals the
 * token loop up to rounding.  The state is carried in fp32; products of the
 * chunk algebra run on matrix cores in bf16 (io_dtype KDA_BF16) or fp32
 * (io_dtype KDA_F32) with fp32 accumulation; o is written in io_dtype (bf16
 * rounded to nearest-even).
 *
 * Intra-device segment parallelism ([P3] section 4.1): with `segments` > 1
 * every sequence is split into that many segments of whole chunks (at most one
 * per chunk, at most 64).  The transition of each inner segment (the map M of
 * its incoming state and the state S~ it produces from zero) is evaluated in
 * parallel, the transitions are composed in order, and every segment is then
 * run from its exact incoming state.  The result is the same recurrence up to
 * rounding.  The workspace holds 3 x segments fp32 states per (sequence,
 * head).  segments = 0 lets the library choose: for bf16 I/O, sequences of
 * at least 8 chunks and no more num_seqs * num_heads chains than the current
 * device has compute units, every sequence is split into three segments whose
 * first one takes half of the chunks; otherwise no split.  Also in automatic
 * mode, a fixed-length bf16 batch with more chains than compute units, not a
 * whole multiple of them, may run as equal runs of chunks per workgroup: a
 * chain cut at a chunk boundary between two workgroups hands its state over
 * through the workspace (one 128 x 128 fp32 state and a flag per workgroup),
 * so the result is the same recurrence up to rounding at the cut.
 * ---------------------------------------------------------------------- */
typedef struct kda_chunk_fwd_args {
  int32_t num_seqs;               /* N >= 1                                              */
  int32_t seq_len;                /* tokens per sequence when cu_seqlens == NULL (>= 0)  */
  const int32_t *cu_seqlens;      /* device [N+1] packed offsets, or NULL (fixed length) */
  const int32_t *cu_seqlens_host; /* host copy of cu_seqlens; required with cu_seqlens.  */
                                  /* Must be 0-based, non-decreasing, the device copy     */
                                  /* must hold the same values (not checked).            */
  int32_t num_heads;              /* H >= 1                                              */
  int32_t head_dim;               /* must be KDA_HEAD_DIM                                */
  int32_t chunk_size;             /* must be KDA_CHUNK                                   */
  kda_dtype io_dtype;             /* dtype of q, k, v and o                              */
  float scale;                    /* output scale (1.0 = the pages' formula)             */
  const void *q;                  /* [T_total, H, 128] io_dtype                          */
  const void *k;                  /* [T_total, H, 128] io_dtype                          */
  const void *v;                  /* [T_total, H, 128] io_dtype                          */
  const float *g;                 /* [T_total, H, 128] log-decay, or gate logits         */
  const float *beta;              /* [T_total, H] beta, or beta logits                   */
  const float *initial_state;     /* [N, H, 128, 128] or NULL = zeros                    */
  float *final_state;             /* [N, H, 128, 128] or NULL = not written.  May equal  */
                                  /* initial_state (in-place update).                    */
  void *o;                        /* [T_total, H, 128] io_dtype; must not alias inputs   */
  void *workspace;                /* device scratch of >= the queried size, 256-B aligned */
  size_t workspace_bytes;
  int32_t segments;               /* 0 = automatic, 1 = never split, > 1 = split each    */
                                  /* sequence into this many segments (capped so every   */
                                  /* segment holds at least one chunk)                   */
  kda_gate gate;                  /* how g and beta are read (zero = log-decay, beta)    */
} kda_chunk_fwd_args;

/* Bytes of workspace kda_chunk_fwd needs for these arguments (pointers are not
 * read; only sizes, cu_seqlens_host and segments).  Host only: no GPU work; in
 * automatic mode it reads the current device's compute-unit count. */
kda_status kda_chunk_fwd_workspace_size(const kda_chunk_fwd_args *args, size_t *bytes);

/* Enqueue the prefill forward on `stream`.  Errors: KDA_ERROR_INVALID_VALUE for
 * null required pointers, negative sizes, misaligned pointers, cu_seqlens_host
 * that is not 0-based and non-decreasing, T_total beyond 2^31 - 1 tokens,
 * num_seqs * num_heads beyond 2^30 - 1, num_heads beyond 65,536, an unknown
 * gate mode, a missing or misaligned A_log, a misaligned dt_bias, lower_bound
 * outside [-5, 0] or beta_logits other than 0 or 1;
 * KDA_ERROR_UNSUPPORTED for head_dim != 128 or chunk_size != 64;
 * KDA_ERROR_WORKSPACE when the workspace is smaller than queried. */
kda_status kda_chunk_fwd(const kda_chunk_fwd_args *args, void *stream);

/* The prefill forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It computes exactly what kda_chunk_fwd
 * computes (same kernels, same plan, same bits) but takes its workspace from a
 * buffer the library holds: one static device array of
 * kda_chunk_fwd_no_alloc_max_workspace() bytes (64 MiB) per GPU, reserved when
 * the library is loaded and held until the process ends.  args->workspace and
 * args->workspace_bytes are ignored.  The call allocates nothing.
 * Limit: returns KDA_ERROR_WORKSPACE, touching no buffer, when the plan needs
 * more than that (kda_chunk_fwd_workspace_size tells how much a call needs;
 * e.g. 56.6 MiB for one 65,536-token sequence of 96 heads split into three
 * segments).  Other errors as kda_chunk_fwd; KDA_ERROR_LAUNCH also when the
 * buffer's device address cannot be looked up.
 * Every call on a GPU shares that GPU's buffer and leaves its contents behind:
 * all the prefill reads from it is written earlier in the same call (the
 * hand-over flags are cleared by a kernel at the start of each call), so the
 * previous contents never matter, but calls that overlap in time on one GPU race
 * on the buffer and must be ordered by the caller (one stream, or events). */
kda_status kda_chunk_fwd_no_alloc(const kda_chunk_fwd_args *args, void *stream);

/* Size in bytes of the per-GPU buffer of kda_chunk_fwd_no_alloc. */
size_t kda_chunk_fwd_no_alloc_max_workspace(void);

/* ------------------------------------------------------------------------
 * Failures detected on the device.  A kernel cannot return a status to the
 * host call that enqueued it; what it detects it ORs into a status word the
 * library keeps on each GPU, and it makes the affected outputs NaN.
 *   KDA_DEVICE_HANDOFF_TIMEOUT: in the balanced schedule of kda_chunk_fwd, a
 *     workgroup that continues a chain gave up waiting for the state of the
 *     workgroup that began it (it polls its flag a bounded number of times so
 *     that every wave exits).  That workgroup ran from a NaN state: its o rows
 *     and the chain's final state are NaN.  The wait is on a workgroup
 *     dispatched earlier that never waits itself, so it is not expected to
 *     happen; it is reported rather than left to hang or to yield a silent
 *     wrong state.
 * ---------------------------------------------------------------------- */
#define KDA_DEVICE_HANDOFF_TIMEOUT 0x1u

/* Read the current GPU's status word in stream order: waits until the work
 * enqueued on `stream` before the call has finished, then stores the bits set
 * since the last clear in *bits (0 = no device-side failure).  With clear != 0
 * the word is reset in the same atomic exchange.  Bits set by work on other
 * streams appear once that work has run.  Errors: KDA_ERROR_INVALID_VALUE for a
 * null `bits`; KDA_ERROR_LAUNCH when the runtime fails (bits untouched).
 * Synchronises the host with `stream`; not for use under graph capture. */
kda_status kda_device_status(void *stream, int32_t clear, uint32_t *bits);

/* Polls of a hand-over flag before a workgroup of the balanced schedule gives
 * up (default 4,194,304, several seconds; each poll is followed by a short
 * sleep).  Process-wide; read when a prefill is enqueued.  0 makes every
 * workgroup that continues a chain give up without polling: the failure path
 * of KDA_DEVICE_HANDOFF_TIMEOUT, for tests.  Errors: KDA_ERROR_INVALID_VALUE
 * for a negative count. */
kda_status kda_set_handoff_poll_limit(int32_t polls);
int32_t kda_handoff_poll_limit(void);

/* The balanced schedule kda_chunk_fwd would use for a fixed-length batch of
 * num_seqs sequences of seq_len tokens and num_heads heads in automatic mode
 * (segments = 0, bf16) on a GPU with `compute_units` compute units -- host only,
 * no GPU needed.  *count receives the number of workgroups of the launch (0 when
 * the prefill would run whole chains instead).  If items is not NULL and
 * capacity >= *count, items[5 i .. 5 i + 4] describe workgroup i in dispatch
 * order: chain (sequence * num_heads + head, or -1 for a workgroup with no
 * work), first chunk, end chunk (64-token chunks, end exclusive), role (0 =
 * whole chain, 1 = begins a chain that another workgroup finishes, 2 = finishes
 * a chain from the state of workgroup items[5 i + 4]), and that workgroup's
 * index (-1 for roles 0 and 1).  Errors: KDA_ERROR_INVALID_VALUE for sizes
 * below 1 (seq_len below 0), a null count, or a capacity below *count with
 * items given (then *count is still set). */
kda_status kda_balanced_schedule(int32_t num_seqs, int32_t seq_len, int32_t num_heads,
                                 int32_t compute_units, int32_t *items, int64_t capacity,
                                 int64_t *count);

/* ------------------------------------------------------------------------
 * Chunked backward ([P1] "How KDA updates its state": the recurrence;
 * "FlashKDA steps the state once per 16 tokens": the chunkwise form, forward
 * only in FlashKDA; [P3] section 4.1: the KDA kernels serve training).
 *
 * For the forward of kda_chunk_fwd (log-decay g, beta as given) and the loss
 *     L = sum_t <dO_t, o_t> + sum_{n,h} <dfinal_state[n,h], S_T[n,h]>
 * it writes dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta and dL/dinitial_state.  The
 * state is recomputed from the inputs (states at every 16-token sub-chunk start
 * kept in the workspace); all gradients are fp32.
 * ---------------------------------------------------------------------- */
typedef struct kda_chunk_bwd_args {
  int32_t num_seqs;               /* as kda_chunk_fwd_args                               */
  int32_t seq_len;
  const int32_t *cu_seqlens;
  const int32_t *cu_seqlens_host;
  int32_t num_heads;
  int32_t head_dim;               /* must be KDA_HEAD_DIM                                */
  kda_dtype io_dtype;             /* dtype of q, k, v and dO                             */
  float scale;
  const void *q, *k, *v;          /* [T_total, H, 128] io_dtype                          */
  const float *g;                 /* [T_total, H, 128] log-decay                         */
  const float *beta;              /* [T_total, H]                                        */
  const float *initial_state;     /* [N, H, 128, 128] or NULL = zeros                    */
  const void *dO;                 /* [T_total, H, 128] io_dtype: dL/do                   */
  const float *dfinal_state;      /* [N, H, 128, 128] or NULL = zeros                    */
  float *dq, *dk, *dv, *dg;       /* [T_total, H, 128] fp32 outputs                      */
  float *dbeta;                   /* [T_total, H] fp32 output                            */
  float *dinitial_state;          /* [N, H, 128, 128] fp32 output, or NULL               */
  void *workspace;                /* device scratch of >= the queried size, 256-B aligned */
  size_t workspace_bytes;
} kda_chunk_bwd_args;

/* Bytes of workspace for the whole pack in one pass: (T_total / 16 + N + 1) x
 * H x (64 KiB of state + 27,200 B of partial sums + 3,072 B of per-sub-chunk
 * matrices), each region 256-B aligned.  Host only. */
kda_status kda_chunk_bwd_workspace_size(const kda_chunk_bwd_args *args, size_t *bytes);

/* The smallest workspace kda_chunk_bwd accepts: the largest single sequence's
 * requirement (its length / 16 + 2 slots).  A workspace between this and
 * kda_chunk_bwd_workspace_size is used for consecutive groups of sequences,
 * each group as large as fits, one after another on the stream; the results
 * are the same bits.  Host only. */
kda_status kda_chunk_bwd_min_workspace_size(const kda_chunk_bwd_args *args, size_t *bytes);

/* Enqueue the backward on `stream`.  Errors as kda_chunk_fwd (sizes, offsets,
 * alignment: q, k, v, dO, g and the gradients 16 bytes, beta and dbeta 4; the
 * outputs may not alias the inputs), KDA_ERROR_WORKSPACE when the workspace is
 * smaller than kda_chunk_bwd_min_workspace_size. */
kda_status kda_chunk_bwd(const kda_chunk_bwd_args *args, void *stream);

/* ------------------------------------------------------------------------
 * Recurrent decode step ([P1] "How KDA updates its state"; [P3] section 4.5:
 * the state is updated in place at every decoding step).
 *
 * For each row b with slot s = state_indices[b] (s = b when state_indices is
 * NULL) and each head h, one token is applied in place to state[s, h]:
 *     S <- Diag(exp(g)) S;  r = S^T k;  S <- S + beta k (v - r)^T;
 *     o = scale * S^T q
 * Rows whose slot is negative or >= num_slots are skipped: their state is not
 * touched and their o rows are not written.  Two rows naming the same slot race
 * (caller error; no out-of-bounds access results).
 * ---------------------------------------------------------------------- */
typedef struct kda_recurrent_step_args {
  int32_t batch;                  /* B >= 0 rows, one token each                         */
  int32_t num_heads;              /* H >= 1                                              */
  int32_t head_dim;               /* must be KDA_HEAD_DIM                                */
  kda_dtype io_dtype;             /* dtype of q, k, v and o                              */
  float scale;
  const void *q;                  /* [B, H, 128] io_dtype                                */
  const void *k;                  /* [B, H, 128] io_dtype                                */
  const void *v;                  /* [B, H, 128] io_dtype                                */
  const float *g;                 /* [B, H, 128] log-decay, or gate logits               */
  const float *beta;              /* [B, H] beta, or beta logits                         */
  float *state;                   /* pool [num_slots, H, 128, 128] fp32, in place        */
  const int32_t *state_indices;   /* device [B] or NULL (identity, needs B <= num_slots) */
  int32_t num_slots;
  void *o;                        /* [B, H, 128] io_dtype                                */
  kda_gate gate;                  /* how g and beta are read (zero = log-decay, beta)    */
} kda_recurrent_step_args;

/* Enqueue one decode step on `stream`.  Errors: KDA_ERROR_INVALID_VALUE for
 * null or misaligned pointers, negative sizes, batch * num_heads beyond
 * 2^31 - 1, batch > num_slots without state_indices, and the gate checks of
 * kda_chunk_fwd; KDA_ERROR_UNSUPPORTED for head_dim != 128. */
kda_status kda_recurrent_step(const kda_recurrent_step_args *args, void *stream);

/* ------------------------------------------------------------------------
 * Fused decode step: the layer's front end, the recurrence and the output
 * normalisation in one kernel ([P3] section 4.5: one fused kernel covers short
 * convolution, input normalisation, gating, the KDA recurrence and output
 * normalisation; [P4] "Kimi Delta Attention": queries and keys come from a short
 * convolution followed by Swish and L2 normalisation, values from a short
 * convolution and Swish; [P1] "How KDA updates its state" and "What the hybrid
 * saves": one ShortConv cache each for the query, key and value projections,
 * kernel size 4).
 *
 * For each row b with slot s = state_indices[b] (s = b when NULL; rows whose
 * slot is negative or >= num_slots are skipped) and head h:
 *   for X = q, k, v (i = 0, 1, 2) and channel c, with the cache holding the three
 *   previous raw inputs, oldest first:
 *     y = sum_{j<4} conv_weight[i, h, c, j] * (cache[s, i, 0..2, h, c], X[b, h, c])_j
 *     cache[s, i, ., h, c] <- (cache[s, i, 1, h, c], cache[s, i, 2, h, c], X[b, h, c])
 *     X' = y * sigmoid(y)                                    (Swish)
 *   q' <- q' / sqrt(|q'|^2 + l2_eps), k' likewise            (per head)
 *   the step of kda_recurrent_step with q', k', v' (g and beta read per `gate`)
 *   o <- o / sqrt(mean_c o_c^2 + norm_eps) * norm_weight[c]  (when out_norm)
 * The cache holds raw inputs, so it round-trips exactly in io_dtype; the
 * convolution, norms and recurrence run in fp32.  Two rows naming the same slot
 * race (caller error; no out-of-bounds access results).
 * ---------------------------------------------------------------------- */
#define KDA_CONV_WIDTH 4

typedef struct kda_fused_step_args {
  int32_t batch;                  /* B >= 0 rows, one token each                         */
  int32_t num_heads;              /* H >= 1                                              */
  int32_t head_dim;               /* must be KDA_HEAD_DIM                                */
  kda_dtype io_dtype;             /* dtype of q, k, v, o and the conv cache              */
  float scale;
  const void *q;                  /* [B, H, 128] io_dtype, projected, before the conv    */
  const void *k;                  /* [B, H, 128] io_dtype                                */
  const void *v;                  /* [B, H, 128] io_dtype                                */
  const float *g;                 /* [B, H, 128] log-decay, or gate logits               */
  const float *beta;              /* [B, H] beta, or beta logits                         */
  const float *conv_weight;       /* [3, H, 128, 4] fp32 taps (q, k, v), oldest first    */
  void *conv_cache;               /* [num_slots, 3, 3, H, 128] io_dtype, in place        */
  float *state;                   /* [num_slots, H, 128, 128] fp32, in place             */
  const int32_t *state_indices;   /* device [B] or NULL (identity, needs B <= num_slots) */
                                  /* one slot indexes both the state and the conv cache  */
  int32_t num_slots;
  float l2_eps;                   /* >= 0, finite (1e-6 is the usual value)              */
  int32_t out_norm;               /* 1 = RMSNorm the output, 0 = raw o                   */
  const float *norm_weight;       /* [128] fp32 output-norm weight, or NULL = 1          */
  float norm_eps;                 /* >= 0, finite                                        */
  void *o;                        /* [B, H, 128] io_dtype                                */
  kda_gate gate;                  /* how g and beta are read (zero = log-decay, beta)    */
} kda_fused_step_args;

/* Bytes of one slot's conv cache (3 caches x 3 inputs x H x head_dim elements of
 * dtype): 216 KiB for 96 heads in bf16 ([P1] "What the hybrid saves").  0 for
 * invalid input. */
size_t kda_conv_cache_bytes(int32_t num_heads, int32_t head_dim, kda_dtype dtype);

/* Enqueue one fused decode step on `stream`.  Errors: KDA_ERROR_INVALID_VALUE for
 * null or misaligned pointers (conv_weight and the state need 16 bytes, the
 * others their element size), negative sizes, batch * num_heads beyond
 * 2^31 - 1, batch > num_slots without state_indices, negative or non-finite
 * epsilons, out_norm other than 0 or 1, and the gate checks of kda_chunk_fwd;
 * KDA_ERROR_UNSUPPORTED for head_dim != 128. */
kda_status kda_fused_decode_step(const kda_fused_step_args *args, void *stream);

/* ------------------------------------------------------------------------
 * Speculative-decode verification with replay ([P3] section 4.5, KDA decoding:
 * after verification rejects some drafted tokens the in-place state has run past
 * the last accepted one; instead of a state snapshot per draft position, only the
 * drafts' projected inputs are kept, the accepted tokens are replayed to rebuild
 * the state on chip, the state of the verified tokens is written back, and the
 * replayed tokens and the next draft window share one recurrent loop in one
 * kernel with the front end and the output normalisation).
 *
 * The caller keeps the previous call's window inputs (q, k, v, g, beta of
 * `replay_window` tokens per row) and passes them back with the number of those
 * tokens that were accepted.  For each row b with slot s (as kda_fused_decode_step)
 * and head h, in one loop:
 *   1. the first n_b = clamp(num_replay[b], 0, replay_window) replay tokens
 *      (all replay_window when num_replay is NULL) run through the fused step in
 *      order, without outputs; if n_b > 0 the state and the conv cache reached
 *      are written back to slot s (n_b = 0 leaves both untouched);
 *   2. the `window` new tokens run through the fused step from there, their
 *      outputs are written to o, and the state and conv window they reach are
 *      dropped.
 * The state is read once and written at most once per call, however many tokens
 * run.  The fields of `step` keep their meaning except that q, k, v, g, o are
 * [B, window, H, 128] and beta [B, window, H].
 * ---------------------------------------------------------------------- */
typedef struct kda_spec_verify_args {
  kda_fused_step_args step;       /* the new window and everything shared            */
  int32_t window;                 /* new tokens per row (>= 0)                           */
  const void *replay_q;           /* [B, replay_window, H, 128] io_dtype                 */
  const void *replay_k;
  const void *replay_v;
  const float *replay_g;          /* [B, replay_window, H, 128] (read per step.gate)     */
  const float *replay_beta;       /* [B, replay_window, H]                               */
  int32_t replay_window;          /* >= 0; replay pointers may be NULL when 0            */
  const int32_t *num_replay;      /* device [B] accepted tokens to replay, or NULL = all */
} kda_spec_verify_args;

/* Enqueue one verification on `stream`.  Errors: those of kda_fused_decode_step
 * (for step, whose token pointers are checked when window > 0), negative
 * window or replay_window, missing or misaligned replay pointers when
 * replay_window > 0, a misaligned num_replay, and B * max(window,
 * replay_window) * H beyond 2^31 - 1. */
kda_status kda_spec_verify_step(const kda_spec_verify_args *args, void *stream);

/* ------------------------------------------------------------------------
 * State-pool copies ([P3] section 4.5: states are stored head by head
 * contiguously; a cache hit copies a read-only snapshot into the request's
 * private running state; new checkpoints are written to fresh slots).
 * One "state" is H x 128 x 128 elements.  For i in [0, count):
 *   KDA_STATE_ZERO    dst[slot] = 0,              slot = indices ? indices[i] : i
 *   KDA_STATE_COPY    dst[i] = src[i]
 *   KDA_STATE_GATHER  dst[i] = src[indices[i]]    (restore a snapshot)
 *   KDA_STATE_SCATTER dst[indices[i]] = src[i]    (save a checkpoint)
 * converting between src_dtype and dst_dtype (fp32 -> bf16 rounds to nearest
 * even).  A negative index, or one >= the slot count of the indexed pool,
 * skips that i.  src and dst must not overlap.  Errors: an op out of range,
 * count < 0, num_heads < 1, head_dim != 128 (KDA_ERROR_UNSUPPORTED), missing or
 * misaligned (16-byte) pools, missing or misaligned indices for a gather or
 * scatter, count beyond the pool it indexes directly, overlapping pools, and
 * count x num_heads beyond 2^31 - 1 (one workgroup per head of a state).
 * ---------------------------------------------------------------------- */
typedef enum kda_state_op {
  KDA_STATE_ZERO = 0,
  KDA_STATE_COPY = 1,
  KDA_STATE_GATHER = 2,
  KDA_STATE_SCATTER = 3
} kda_state_op;

kda_status kda_state_io(kda_state_op op, const void *src, kda_dtype src_dtype,
                        int32_t src_slots, void *dst, kda_dtype dst_dtype,
                        int32_t dst_slots, const int32_t *indices, int32_t count,
                        int32_t num_heads, int32_t head_dim, void *stream);

/* Bytes of one state (H x head_dim x head_dim elements of dtype), e.g. 3 MiB
 * for 96 heads in bf16 ([P1] "What the hybrid saves").  0 for invalid input. */
size_t kda_state_bytes(int32_t num_heads, int32_t head_dim, kda_dtype dtype);

/* Human-readable name of a status code (static string). */
const char *kda_status_string(kda_status status);

/* Library version string (static). */
const char *kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
