/*
 * kda_oracle.c -- plain, slow, fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's cpu_baseline leg may load this library.  The product path
 * (the HIP library) shares no code, header, table or helper with it and never
 * calls it.
 *
 * Sources (web pages; cited by title and section):
 *  [P1] "How Kimi K3 Engineered Its Way to the Frontier", section
 *       "How KDA updates its state" (the forget / erase+write / read token loop
 *       of flash-linear-attention's naive.py, decay on the key axis, state
 *       layout S[B,HV,K,V], gates g[B,T,HV,K] in natural-log space) and section
 *       "FlashKDA steps the state once per 16 tokens" (the chunkwise form gives
 *       the same result as the token loop; only the schedule changes).
 *  [P2] "Kimi K3: Open Frontier Intelligence" (Chlience paper archive), section 6
 *       (the KDA equation S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
 *       o_t = S_t^T q_t).
 *  [P3] "Kimi K3 -- Training and Infrastructure Notes", section 4.1 "KDA
 *       algorithm-system co-design" (a segment's effect is a transition M acting
 *       on the incoming state plus a state S~ generated from zero) and section
 *       4.5 "Inference and online serving" (decode updates the state in place).
 *  [P4] "Kimi K3: a 2.8T open model ...", section "Kimi Delta Attention:
 *       constant-size memory over a million tokens" (same equation) and
 *       subsection "FlashKDA: the equation, shipped as a kernel" (optional state
 *       in and out, variable-length batches through cumulative sequence lengths;
 *       beta arrives as logits that pass through a sigmoid).
 *  [P1] section "How KDA updates its state" (the layer carries three ShortConv
 *       caches, for the query, key and value projections) and "What the
 *       hybrid saves" (kernel size 4); [P4] "Kimi Delta Attention" (queries and
 *       keys come from a short convolution followed by Swish and L2
 *       normalisation, values from a short convolution and Swish); [P3]
 *       section 4.5 (the fused decode kernel covers short convolution, input
 *       normalisation, gating, the recurrence and output normalisation).
 *  [P1] section "How KDA updates its state", the part on how the decay logit
 *       becomes a decay: K3's lower-bounded gate (flash-linear-attention's
 *       gate.py) turns a raw per-channel gate logit into a log-decay in
 *       (lower_bound, 0); lower_bound defaults to -5.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - No query scale appears in any formula; `scale` multiplies o and the pages'
 *    formula is scale = 1.
 *  - g is the natural-log decay (alpha = exp(g)), beta is already post-sigmoid.
 *  - Variable-length batches reset the state to the sequence's own initial state
 *    at every cu_seqlens boundary.
 *  - ShortConv is a causal depthwise convolution without bias whose cache holds
 *    the W - 1 previous raw inputs, oldest first; taps w[c, 0..W-1] run oldest
 *    to newest, so w[c, W-1] multiplies the current input.
 *  - L2 normalisation is x / sqrt(sum x^2 + eps); "output normalisation" is an
 *    RMSNorm over each head's V outputs, x / sqrt(mean x^2 + eps) * w.
 *
 * Layouts (row-major, innermost last), the same as the product ABI:
 *   q, k, g : [T_total, H, K]      v, o : [T_total, H, V]      beta : [T_total, H]
 *   state   : [N, H, K, V]  (rows = key channels, columns = value channels)
 * cu_seqlens: N+1 non-decreasing offsets into T_total, cu_seqlens[0] == 0.
 *
 * Parity status: every function below is pinned by the CPU tests (brute-force
 * equation form on tiny inputs, closed forms, invariants); none is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_OK 0
#define KDA_ORACLE_EINVAL 1
#define KDA_ORACLE_ENOMEM 2

static int check_cu(int N, const int64_t *cu, int64_t T_total) {
  if (N < 0 || !cu || cu[0] != 0) return 0;
  for (int n = 0; n < N; ++n)
    if (cu[n + 1] < cu[n]) return 0;
  return cu[N] == T_total;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/*
 * One token of the recurrence on one head's state S (K x V), in the order of
 * [P1] "How KDA updates its state": forget (scale row i of S by exp(g_i)),
 * erase+write (S += beta * k (v - k^T S)^T, with k^T S read from the decayed
 * state), then read o = scale * S^T q from the updated state.
 * `r` is caller-provided scratch of length V.
 */
static void token_step(int K, int V, double *S, const double *q, const double *k,
                       const double *v, const double *g, double beta, double scale,
                       double *o, double *r) {
  /* forget: decay acts on the key axis, i.e. on rows of S */
  for (int i = 0; i < K; ++i) {
    const double a = exp(g[i]);
    for (int j = 0; j < V; ++j) S[(size_t)i * V + j] *= a; /*MUT_DECAY*/
  }
  /* what the decayed state returns for key k:  r = S^T k */
  for (int j = 0; j < V; ++j) r[j] = 0.0;
  for (int i = 0; i < K; ++i)
    for (int j = 0; j < V; ++j) r[j] += k[i] * S[(size_t)i * V + j];
  /*MUT_WRITE_BEGIN*/
  /* erase + write: S += beta * k (v - r)^T */
  for (int i = 0; i < K; ++i) {
    const double bk = beta * k[i];
    for (int j = 0; j < V; ++j) S[(size_t)i * V + j] += bk * (v[j] - r[j]); /*MUT_ERASE*/
  }
  /*MUT_WRITE_END*/
  /*MUT_READ_BEGIN*/
  /* read from the updated state: o = scale * S^T q */
  if (o) {
    for (int j = 0; j < V; ++j) o[j] = 0.0;
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < V; ++j) o[j] += q[i] * S[(size_t)i * V + j];
    for (int j = 0; j < V; ++j) o[j] *= scale;
  }
  /*MUT_READ_END*/
}

/*
 * The definition: the token-by-token recurrence over a packed batch of N
 * sequences and H heads.  S0 may be NULL (zero initial state); S_final may be
 * NULL (not written).  o may be NULL (outputs not written).
 */
int kda_oracle_recurrent(int N, const int64_t *cu_seqlens, int H, int K, int V,
                         const double *q, const double *k, const double *v,
                         const double *g, const double *beta, double scale,
                         const double *S0, double *o, double *S_final, int nthreads) {
  if (H <= 0 || K <= 0 || V <= 0 || !cu_seqlens) return KDA_ORACLE_EINVAL;
  if (!check_cu(N, cu_seqlens, cu_seqlens[N])) return KDA_ORACLE_EINVAL;
  set_threads(nthreads);
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int64_t nh = 0; nh < (int64_t)N * H; ++nh) {
    const int n = (int)(nh / H), h = (int)(nh % H);
    double *S = (double *)malloc(sizeof(double) * ((size_t)K * V + V));
    if (!S) { err |= 1; continue; }
    double *r = S + (size_t)K * V;
    if (S0) memcpy(S, S0 + ((size_t)n * H + h) * K * V, sizeof(double) * K * V);
    else memset(S, 0, sizeof(double) * K * V);
    for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
      const size_t th = (size_t)t * H + h;
      token_step(K, V, S, q + th * K, k + th * K, v + th * V, g + th * K, beta[th],
                 scale, o ? o + th * V : NULL, r);
    }
    if (S_final) memcpy(S_final + ((size_t)n * H + h) * K * V, S, sizeof(double) * K * V);
    free(S);
  }
  return err ? KDA_ORACLE_ENOMEM : KDA_ORACLE_OK;
}

/*
 * Decode: one token per batch row, applied in place to a slot pool
 * state_pool[num_slots, H, K, V] ([P3] section 4.5: the state is updated in
 * place at every decoding step).  Row b uses slot slot_idx[b] (identity when
 * slot_idx is NULL); a negative slot skips the row (its o is left untouched).
 * q, k, g: [B, H, K]; v, o: [B, H, V]; beta: [B, H].
 */
int kda_oracle_decode_step(int B, int H, int K, int V, const double *q, const double *k,
                           const double *v, const double *g, const double *beta,
                           double scale, double *state_pool, const int64_t *slot_idx,
                           int64_t num_slots, double *o, int nthreads) {
  if (B < 0 || H <= 0 || K <= 0 || V <= 0 || !state_pool) return KDA_ORACLE_EINVAL;
  for (int b = 0; b < B; ++b) {
    const int64_t s = slot_idx ? slot_idx[b] : b;
    if (s >= num_slots) return KDA_ORACLE_EINVAL;
    for (int b2 = 0; b2 < b; ++b2) /* two rows may not share a slot */
      if (s >= 0 && (slot_idx ? slot_idx[b2] : b2) == s) return KDA_ORACLE_EINVAL;
  }
  set_threads(nthreads);
  int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
  for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int64_t s = slot_idx ? slot_idx[b] : b;
    if (s < 0) continue;
    double *r = (double *)malloc(sizeof(double) * V);
    if (!r) { err |= 1; continue; }
    const size_t th = (size_t)b * H + h;
    token_step(K, V, state_pool + ((size_t)s * H + h) * K * V, q + th * K, k + th * K,
               v + th * V, g + th * K, beta[th], scale, o ? o + th * V : NULL, r);
    free(r);
  }
  return err ? KDA_ORACLE_ENOMEM : KDA_ORACLE_OK;
}

/*
 * The chunkwise evaluation ([P1] "FlashKDA steps the state once per 16 tokens":
 * split the sequence into blocks of C tokens, compute inside a block with dense
 * products, step the state once per block; the result matches the token loop).
 * The pages give the shape, not the algebra; this is the block form obtained by
 * unrolling the recurrence over one block with incoming state S (K x V):
 *
 *   G_r   = sum_{s<=r} g_s                        (per key channel, within the block)
 *   A[r,s]= beta_r * sum_c k_r[c] k_s[c] exp(G_r[c]-G_s[c])     for s <  r
 *   P[r,s]=          sum_c q_r[c] k_s[c] exp(G_r[c]-G_s[c])     for s <= r
 *   u_r   = beta_r (v_r - S^T (exp(G_r) * k_r)) - sum_{s<r} A[r,s] u_s
 *           (i.e. (I + A) U = diag(beta) (V - K~ S): a unit lower-triangular
 *            system, solved here by plain forward substitution)
 *   o_r   = scale * ( S^T (exp(G_r) * q_r) + sum_{s<=r} P[r,s] u_s )
 *   S    <- exp(G_last) * S + sum_s (exp(G_last - G_s) * k_s) u_s^T
 *
 * Every exponent in A and P is G_r - G_s with s <= r, so no factor exceeds 1.
 * Independent of the token loop above: it shares nothing with token_step.
 */
int kda_oracle_chunked(int N, const int64_t *cu_seqlens, int H, int K, int V, int C,
                       const double *q, const double *k, const double *v, const double *g,
                       const double *beta, double scale, const double *S0, double *o,
                       double *S_final, int nthreads) {
  if (H <= 0 || K <= 0 || V <= 0 || C <= 0 || !cu_seqlens) return KDA_ORACLE_EINVAL;
  if (!check_cu(N, cu_seqlens, cu_seqlens[N])) return KDA_ORACLE_EINVAL;
  set_threads(nthreads);
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int64_t nh = 0; nh < (int64_t)N * H; ++nh) {
    const int n = (int)(nh / H), h = (int)(nh % H);
    const size_t kv = (size_t)K * V;
    /* S, Snew, G, A, P, U, tmp */
    const size_t need = 2 * kv + (size_t)C * K + 2 * (size_t)C * C + (size_t)C * V + (size_t)V;
    double *buf = (double *)malloc(sizeof(double) * need);
    if (!buf) { err |= 1; continue; }
    double *S = buf, *Sn = S + kv, *G = Sn + kv, *A = G + (size_t)C * K;
    double *P = A + (size_t)C * C, *U = P + (size_t)C * C, *tmp = U + (size_t)C * V;
    if (S0) memcpy(S, S0 + ((size_t)n * H + h) * kv, sizeof(double) * kv);
    else memset(S, 0, sizeof(double) * kv);

    for (int64_t c0 = cu_seqlens[n]; c0 < cu_seqlens[n + 1]; c0 += C) {
      const int L = (int)((cu_seqlens[n + 1] - c0 < C) ? (cu_seqlens[n + 1] - c0) : C);
#define ROW(ptr, r, D) ((ptr) + ((size_t)(c0 + (r)) * H + h) * (D))
      /* cumulative log-decay inside the block */
      for (int r = 0; r < L; ++r)
        for (int c = 0; c < K; ++c)
          G[(size_t)r * K + c] = ROW(g, r, K)[c] + (r ? G[(size_t)(r - 1) * K + c] : 0.0);
      /* A and P */
      for (int r = 0; r < L; ++r) {
        const double br = beta[(size_t)(c0 + r) * H + h];
        for (int s = 0; s <= r; ++s) {
          double a = 0.0, p = 0.0;
          for (int c = 0; c < K; ++c) {
            const double e = exp(G[(size_t)r * K + c] - G[(size_t)s * K + c]);
            a += ROW(k, r, K)[c] * ROW(k, s, K)[c] * e;
            p += ROW(q, r, K)[c] * ROW(k, s, K)[c] * e;
          }
          A[(size_t)r * C + s] = (s < r) ? br * a : 0.0;
          P[(size_t)r * C + s] = p;
        }
      }
      /* forward substitution for U */
      for (int r = 0; r < L; ++r) {
        const double br = beta[(size_t)(c0 + r) * H + h];
        for (int j = 0; j < V; ++j) tmp[j] = 0.0; /* S^T (exp(G_r) * k_r) */
        for (int c = 0; c < K; ++c) {
          const double kt = ROW(k, r, K)[c] * exp(G[(size_t)r * K + c]);
          for (int j = 0; j < V; ++j) tmp[j] += kt * S[(size_t)c * V + j];
        }
        for (int j = 0; j < V; ++j) {
          double u = br * (ROW(v, r, V)[j] - tmp[j]);
          for (int s = 0; s < r; ++s) u -= A[(size_t)r * C + s] * U[(size_t)s * V + j];
          U[(size_t)r * V + j] = u;
        }
      }
      /* outputs */
      if (o) {
        for (int r = 0; r < L; ++r) {
          for (int j = 0; j < V; ++j) tmp[j] = 0.0;
          for (int c = 0; c < K; ++c) {
            const double qt = ROW(q, r, K)[c] * exp(G[(size_t)r * K + c]);
            for (int j = 0; j < V; ++j) tmp[j] += qt * S[(size_t)c * V + j];
          }
          for (int s = 0; s <= r; ++s)
            for (int j = 0; j < V; ++j) tmp[j] += P[(size_t)r * C + s] * U[(size_t)s * V + j];
          double *orow = ROW(o, r, V);
          for (int j = 0; j < V; ++j) orow[j] = scale * tmp[j];
        }
      }
      /* state step */
      for (int c = 0; c < K; ++c) {
        const double gl = G[(size_t)(L - 1) * K + c];
        for (int j = 0; j < V; ++j) Sn[(size_t)c * V + j] = exp(gl) * S[(size_t)c * V + j];
        for (int s = 0; s < L; ++s) {
          const double kb = ROW(k, s, K)[c] * exp(gl - G[(size_t)s * K + c]);
          for (int j = 0; j < V; ++j) Sn[(size_t)c * V + j] += kb * U[(size_t)s * V + j];
        }
      }
      memcpy(S, Sn, sizeof(double) * kv);
#undef ROW
    }
    if (S_final) memcpy(S_final + ((size_t)n * H + h) * kv, S, sizeof(double) * kv);
    free(buf);
  }
  return err ? KDA_ORACLE_ENOMEM : KDA_ORACLE_OK;
}

/*
 * Segment transition ([P3] section 4.1, intra-device and cross-device context
 * parallelism): over tokens t = 0..T-1 of one head, the segment maps an
 * incoming state S_in to S_out = M S_in + S~, with
 *   M  = M_{T-1} ... M_1 M_0,   M_t = (I - beta_t k_t k_t^T) Diag(exp(g_t))   (K x K)
 *   S~ = the state the recurrence reaches from a zero incoming state        (K x V)
 * k, g: [T, K], v: [T, V], beta: [T] (one head, contiguous).  Either output may
 * be NULL.
 */
int kda_oracle_transition(int64_t T, int K, int V, const double *k, const double *v,
                          const double *g, const double *beta, double *M, double *S_tilde) {
  if (T < 0 || K <= 0 || V <= 0) return KDA_ORACLE_EINVAL;
  double *Mt = (double *)malloc(sizeof(double) * ((size_t)K * K + K));
  double *S = (double *)calloc((size_t)K * V + V, sizeof(double));
  if (!Mt || !S) { free(Mt); free(S); return KDA_ORACLE_ENOMEM; }
  double *w = Mt + (size_t)K * K;
  double *r = S + (size_t)K * V;
  for (int i = 0; i < K; ++i)
    for (int j = 0; j < K; ++j) Mt[(size_t)i * K + j] = (i == j) ? 1.0 : 0.0;
  for (int64_t t = 0; t < T; ++t) {
    const double *kt = k + (size_t)t * K, *gt = g + (size_t)t * K;
    /* M <- (I - b k k^T) Diag(a) M : first Diag(a) M, then subtract b k (k^T (Diag(a) M)) */
    for (int i = 0; i < K; ++i) {
      const double a = exp(gt[i]);
      for (int j = 0; j < K; ++j) Mt[(size_t)i * K + j] *= a;
    }
    for (int j = 0; j < K; ++j) {
      double s = 0.0;
      for (int i = 0; i < K; ++i) s += kt[i] * Mt[(size_t)i * K + j];
      w[j] = s;
    }
    for (int i = 0; i < K; ++i)
      for (int j = 0; j < K; ++j) Mt[(size_t)i * K + j] -= beta[t] * kt[i] * w[j];
    /* S~: the plain token recurrence from zero, outputs not needed */
    token_step(K, V, S, kt, kt, v + (size_t)t * V, gt, beta[t], 1.0, NULL, r);
  }
  if (M) memcpy(M, Mt, sizeof(double) * K * K);
  if (S_tilde) memcpy(S_tilde, S, sizeof(double) * K * V);
  free(Mt);
  free(S);
  return KDA_ORACLE_OK;
}

/*
 * Gradients of the token loop (the backward pass a training step needs; [P1]
 * "FlashKDA steps the state once per 16 tokens" notes FlashKDA is forward-only,
 * [P3] section 4.1 that KDA kernels serve training).  For the loss
 *   L = sum_t <dO_t, o_t> + sum_{n,h} <dS_final[n,h], S_T[n,h]>
 * reverse-mode through each token of kda_oracle_recurrent, in the order the
 * token was computed:
 *   S' = Diag(a) S,  a = exp(g);  r = S'^T k;  u = beta (v - r);  S+ = S' + k u^T;
 *   o = scale S+^T q
 * backwards (dS is dL/dS+ on entry):
 *   dS += scale q dO^T;     dq = scale S+ dO
 *   dk = dS u;  du = dS^T k;  dv = beta du;  dbeta = (v - r) . du;  dr = -beta du
 *   dS' = dS + k dr^T;      dk += S' dr
 *   dg_i = sum_j dS'_ij S'_ij  (= a_i sum_j dS'_ij S_ij);   dS <- Diag(a) dS'
 * The states before each token are kept (T x K x V per chain), so this is for
 * small cases.  s0 and dS_final may be NULL (zero); dS0 may be NULL.
 */
int kda_oracle_recurrent_bwd(int N, const int64_t *cu_seqlens, int H, int K, int V,
                             const double *q, const double *k, const double *v,
                             const double *g, const double *beta, double scale,
                             const double *S0, const double *dO, const double *dS_final,
                             double *dq, double *dk, double *dv, double *dg, double *dbeta,
                             double *dS0) {
  if (H <= 0 || K <= 0 || V <= 0 || !cu_seqlens || !dO) return KDA_ORACLE_EINVAL;
  if (!check_cu(N, cu_seqlens, cu_seqlens[N])) return KDA_ORACLE_EINVAL;
  const size_t KV = (size_t)K * V;
  for (int n = 0; n < N; ++n)
    for (int h = 0; h < H; ++h) {
      const int64_t t0 = cu_seqlens[n], t1 = cu_seqlens[n + 1], T = t1 - t0;
      /* states before each token (T + 1 of them), then work vectors */
      double *St = (double *)malloc(sizeof(double) * ((size_t)(T + 1) * KV + 2 * KV + 4 * V));
      if (!St) return KDA_ORACLE_ENOMEM;
      double *dS = St + (size_t)(T + 1) * KV, *Sp = dS + KV;
      double *r = Sp + KV, *u = r + V, *du = u + V, *dr = du + V;
      if (S0) memcpy(St, S0 + ((size_t)n * H + h) * KV, sizeof(double) * KV);
      else memset(St, 0, sizeof(double) * KV);
      /* forward, keeping every state */
      for (int64_t t = 0; t < T; ++t) {
        const size_t th = (size_t)(t0 + t) * H + h;
        const double *kt = k + th * K, *gt = g + th * K, *vt = v + th * V;
        double *S = St + (size_t)(t + 1) * KV;
        for (int i = 0; i < K; ++i)
          for (int j = 0; j < V; ++j) S[i * V + j] = exp(gt[i]) * St[(size_t)t * KV + i * V + j];
        for (int j = 0; j < V; ++j) {
          double acc = 0.0;
          for (int i = 0; i < K; ++i) acc += kt[i] * S[i * V + j];
          r[j] = acc;
        }
        for (int i = 0; i < K; ++i)
          for (int j = 0; j < V; ++j) S[i * V + j] += beta[th] * kt[i] * (vt[j] - r[j]);
      }
      if (dS_final) memcpy(dS, dS_final + ((size_t)n * H + h) * KV, sizeof(double) * KV);
      else memset(dS, 0, sizeof(double) * KV);
      /* backward */
      for (int64_t t = T - 1; t >= 0; --t) {
        const size_t th = (size_t)(t0 + t) * H + h;
        const double *qt = q + th * K, *kt = k + th * K, *gt = g + th * K, *vt = v + th * V;
        const double *dOt = dO + th * V;
        const double *Sprev = St + (size_t)t * KV, *Snew = St + (size_t)(t + 1) * KV;
        const double b = beta[th];
        for (int i = 0; i < K; ++i)
          for (int j = 0; j < V; ++j) Sp[i * V + j] = exp(gt[i]) * Sprev[i * V + j];
        for (int j = 0; j < V; ++j) {
          double acc = 0.0;
          for (int i = 0; i < K; ++i) acc += kt[i] * Sp[i * V + j];
          r[j] = acc;
          u[j] = b * (vt[j] - acc);
        }
        /* o = scale S+^T q */
        for (int i = 0; i < K; ++i) {
          double acc = 0.0;
          for (int j = 0; j < V; ++j) {
            dS[i * V + j] += scale * qt[i] * dOt[j];
            acc += Snew[i * V + j] * dOt[j];
          }
          if (dq) dq[th * K + i] = scale * acc;
        }
        /* S+ = S' + k u^T */
        for (int j = 0; j < V; ++j) {
          double acc = 0.0;
          for (int i = 0; i < K; ++i) acc += dS[i * V + j] * kt[i];
          du[j] = acc;
        }
        double db = 0.0;
        for (int j = 0; j < V; ++j) {
          if (dv) dv[th * V + j] = b * du[j];
          db += (vt[j] - r[j]) * du[j];
          dr[j] = -b * du[j];
        }
        if (dbeta) dbeta[th] = db;
        for (int i = 0; i < K; ++i) {
          double dki = 0.0, dgi = 0.0;
          for (int j = 0; j < V; ++j) {
            dki += dS[i * V + j] * u[j] + Sp[i * V + j] * dr[j];
            const double dSp = dS[i * V + j] + kt[i] * dr[j];  /* dL/dS' */
            dgi += dSp * Sp[i * V + j];
            dS[i * V + j] = exp(gt[i]) * dSp;                  /* dL/dS before the token */
          }
          if (dk) dk[th * K + i] = dki;
          if (dg) dg[th * K + i] = dgi;
        }
      }
      if (dS0) memcpy(dS0 + ((size_t)n * H + h) * KV, dS, sizeof(double) * KV);
      free(St);
    }
  return KDA_ORACLE_OK;
}

/*
 * K3's lower-bounded gate ([P1] section "How KDA updates its state"), elementwise over tokens t,
 * heads h and key channels c of x [T, H, K]:
 *   g[t,h,c] = lower_bound * sigmoid(exp(A_log[h]) * (x[t,h,c] + dt_bias[h,c]))
 * with sigmoid(z) = 1 / (1 + exp(-z)).  A_log: [H]; dt_bias: [H, K] or NULL
 * (no bias).  g may equal x (in place).
 */
static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

int kda_oracle_lowerbound_gate(int64_t T, int H, int K, const double *x, const double *A_log,
                               const double *dt_bias, double lower_bound, double *g) {
  if (T < 0 || H <= 0 || K <= 0 || !A_log || (T > 0 && (!x || !g))) return KDA_ORACLE_EINVAL;
  for (int64_t t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h) {
      const double a = exp(A_log[h]);
      for (int c = 0; c < K; ++c) {
        const size_t i = ((size_t)t * H + h) * K + c;
        const double z = x[i] + (dt_bias ? dt_bias[(size_t)h * K + c] : 0.0);
        g[i] = lower_bound * sigmoid(a * z);
      }
    }
  return KDA_ORACLE_OK;
}

/*
 * beta from its logits ([P4] subsection "FlashKDA: the equation, shipped as a
 * kernel": beta logits pass through a sigmoid), elementwise over n values.
 */
int kda_oracle_sigmoid(int64_t n, const double *x, double *y) {
  if (n < 0 || (n > 0 && (!x || !y))) return KDA_ORACLE_EINVAL;
  for (int64_t i = 0; i < n; ++i) y[i] = sigmoid(x[i]);
  return KDA_ORACLE_OK;
}

/*
 * ShortConv: causal depthwise convolution of width W over T tokens of C channels,
 * continuing from the cache of the W - 1 previous inputs (cache[j, c] is the input
 * at time j - (W - 1), j = 0 oldest):
 *   y[t, c] = sum_{i=0}^{W-1} w[c, i] * x[t - (W - 1) + i, c]
 * The cache is replaced by the last W - 1 inputs.  x, y: [T, C]; w: [C, W];
 * cache: [W - 1, C].  y may not alias x.
 */
int kda_oracle_short_conv(int64_t T, int C, int W, const double *x, const double *w,
                          double *cache, double *y) {
  if (T < 0 || C <= 0 || W < 1 || !w || !cache || (T > 0 && (!x || !y)))
    return KDA_ORACLE_EINVAL;
  const int64_t n = T + W - 1;  /* the cache rows, then the new inputs */
  double *ext = (double *)malloc(sizeof(double) * (size_t)n * C);
  if (!ext) return KDA_ORACLE_ENOMEM;
  memcpy(ext, cache, sizeof(double) * (size_t)(W - 1) * C);
  if (T > 0) memcpy(ext + (size_t)(W - 1) * C, x, sizeof(double) * (size_t)T * C);
  for (int64_t t = 0; t < T; ++t)
    for (int c = 0; c < C; ++c) {
      double acc = 0.0;
      for (int i = 0; i < W; ++i) acc += w[(size_t)c * W + i] * ext[(size_t)(t + i) * C + c];
      y[(size_t)t * C + c] = acc;
    }
  memcpy(cache, ext + (size_t)T * C, sizeof(double) * (size_t)(W - 1) * C);
  free(ext);
  return KDA_ORACLE_OK;
}

/* Swish (SiLU) elementwise: x * sigmoid(x). */
int kda_oracle_swish(int64_t n, const double *x, double *y) {
  if (n < 0 || (n > 0 && (!x || !y))) return KDA_ORACLE_EINVAL;
  for (int64_t i = 0; i < n; ++i) y[i] = x[i] * sigmoid(x[i]);
  return KDA_ORACLE_OK;
}

/* L2 normalisation of each of `rows` vectors of length n: x / sqrt(sum x^2 + eps). */
int kda_oracle_l2norm(int64_t rows, int n, const double *x, double eps, double *y) {
  if (rows < 0 || n <= 0 || (rows > 0 && (!x || !y))) return KDA_ORACLE_EINVAL;
  for (int64_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[(size_t)r * n + i] * x[(size_t)r * n + i];
    const double inv = 1.0 / sqrt(ss + eps);
    for (int i = 0; i < n; ++i) y[(size_t)r * n + i] = x[(size_t)r * n + i] * inv;
  }
  return KDA_ORACLE_OK;
}

/* RMSNorm of each of `rows` vectors of length n: x / sqrt(mean x^2 + eps) * w
 * (w: [n], or NULL for 1). */
int kda_oracle_rmsnorm(int64_t rows, int n, const double *x, const double *w, double eps,
                       double *y) {
  if (rows < 0 || n <= 0 || (rows > 0 && (!x || !y))) return KDA_ORACLE_EINVAL;
  for (int64_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[(size_t)r * n + i] * x[(size_t)r * n + i];
    const double inv = 1.0 / sqrt(ss / n + eps);
    for (int i = 0; i < n; ++i) y[(size_t)r * n + i] = x[(size_t)r * n + i] * inv * (w ? w[i] : 1.0);
  }
  return KDA_ORACLE_OK;
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
