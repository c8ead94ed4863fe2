/*
 * kda_oracle.c -- plain, slow, token-by-token fp64 CPU oracle for Kimi Delta
 * Attention (KDA) multi-token recurrent prefill.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only the test suite, the package smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper with
 * the HIP implementation.
 *
 * What it computes (one (sequence n, head h) pair at a time, all arithmetic in
 * fp64, inputs upcast exactly):
 *
 *   S <- S0 (or zeros)                          K x V state, row d = key channel
 *   for t = 1 .. L_n:
 *     S   <- Diag(exp(g_t)) S                   per-key-channel decay, g_t <= 0
 *     p   <- S^T k_t                            value the decayed state predicts
 *     S   <- S + beta_t k_t (v_t - p)^T         delta-rule rank-1 correction
 *     o_t <- scale * S^T q_t                    read-out of the updated state
 *     if t == ckpt_offset[n]: ckpt[n,h] <- S    state after t tokens
 *   if ckpt_offset[n] == 0: ckpt[n,h] <- S0
 *   final[n,h] <- S
 *
 * Sources.  The recurrence is Kimi Delta Attention as the Kimi Linear model
 * defines it: a fixed-size K x V recurrent state per head (FlashKDA page, item
 * description), decayed per key channel, corrected by the delta rule with
 * strength beta and read out with a caller scale.  The contract -- BF16 q/k/v,
 * K = V = 128, FP32 initial/final state, a gate lower bound in [-5, 0] --
 * is the one stated in lmdeploy PR #5050 (Modification), and in FlashInfer PR
 * #4262 "cake_kda" (Dispatch contract).  Checkpoint export "processes the full
 * supplied interval and also exports the recurrent state at the requested
 * position" (lmdeploy PR #5050, Modification); the offset is read as the
 * number of tokens of the sequence already consumed, counted from the
 * sequence start, so 0 exports the initial state and L_n the final state.
 * Offsets outside [0, L_n] export nothing (the slot is left untouched).
 * A sequence with zero tokens keeps its initial state (FlashInfer PR #4633,
 * Reviewer Notes: zero-token handling preserves the FP32 initial state).
 * Packed batches follow cu_seqlens: starts at 0, ends at T_total,
 * non-decreasing (FlashInfer PR #4633, test changes for malformed offsets).
 *
 * None of the pages writes the recurrence as a formula; the reading above is
 * the plainest one consistent with them (decay first, then the delta
 * correction on the decayed state, then the read-out of the updated state).
 *
 * Layouts (row-major, last index fastest):
 *   q, k          [T_total, H, K]  bf16 bit patterns (uint16)
 *   v             [T_total, H, V]  bf16 bit patterns
 *   g             [T_total, H, K]  fp32 natural-log decay
 *   beta          [T_total, H]     fp32
 *   cu_seqlens    [N+1] int32, or NULL: N equal sequences of T_total/N tokens
 *   initial_state [N, H, K, V] fp32, or NULL (zeros)
 *   ckpt_offsets  [N] int32, or NULL (no export)
 *   out           [T_total, H, V]  fp64
 *   final_state   [N, H, K, V]     fp64
 *   ckpt_state    [N, H, K, V]     fp64 (may be NULL iff ckpt_offsets is NULL)
 *
 * Input prologue (flags).  FlashInfer PR #4262 (Dispatch contract) lists
 * kernels that L2-normalise q and k per token and head inside the kernel and
 * take beta as a logit.  With flag 1 each q_t and k_t is divided by its
 * Euclidean norm over the K channels (a zero vector stays zero); with flag 2
 * beta_t is replaced by 1 / (1 + exp(-beta_t)).  Both in fp64, before the
 * step above.
 *
 * Parity status: pinned by tests against a dense per-step matrix form, the
 * closed-form product expansion, and invariants (no-decay/no-write identity,
 * pure decay, orthonormal overwrite, repeated-key EMA, scalar K = V = 1); the
 * prologue by a hand-worked two-token case and scale invariance.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_bits_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

typedef struct {
  int N, H, K, V;
  long T_total;
  double scale;
  const uint16_t *q, *k, *v;
  const float *g, *beta;
  const int32_t *cu_seqlens;
  const float *initial_state;
  const int32_t *ckpt_offsets;
  double *out, *final_state, *ckpt_state;
  int flags;                    /* 1: L2-normalise q and k; 2: beta is a logit */
  long next_pair;               /* work counter, guarded by lock */
  pthread_mutex_t lock;
} oracle_job;

/* One (sequence, head) pair, token by token. */
static void run_pair(const oracle_job *J, int n, int h, double *S, double *p,
                     double *kt, double *qt, double *vt) {
  const int H = J->H, K = J->K, V = J->V;
  long bos, len;
  if (J->cu_seqlens) {
    bos = J->cu_seqlens[n];
    len = (long)J->cu_seqlens[n + 1] - (long)J->cu_seqlens[n];
  } else {
    len = J->T_total / J->N;
    bos = (long)n * len;
  }
  const size_t state_off = ((size_t)n * H + h) * (size_t)K * V;

  /* S <- S0 or zeros */
  for (int d = 0; d < K; ++d)
    for (int j = 0; j < V; ++j)
      S[d * V + j] = J->initial_state ? (double)J->initial_state[state_off + (size_t)d * V + j] : 0.0;

  long ckpt_at = -1;
  if (J->ckpt_offsets) {
    long off = J->ckpt_offsets[n];
    if (off >= 0 && off <= len) ckpt_at = off;
  }
  if (ckpt_at == 0)
    for (int e = 0; e < K * V; ++e) J->ckpt_state[state_off + e] = S[e];

  for (long t = 0; t < len; ++t) {
    const size_t row = (size_t)(bos + t) * H + h;
    const float *gt = J->g + row * K;
    double bt = (double)J->beta[row];
    for (int d = 0; d < K; ++d) {
      kt[d] = bf16_bits_to_double(J->k[row * K + d]);
      qt[d] = bf16_bits_to_double(J->q[row * K + d]);
    }
    if (J->flags & 1) {
      double nk = 0.0, nq = 0.0;
      for (int d = 0; d < K; ++d) {
        nk += kt[d] * kt[d];
        nq += qt[d] * qt[d];
      }
      nk = sqrt(nk);
      nq = sqrt(nq);
      for (int d = 0; d < K; ++d) {
        if (nk > 0.0) kt[d] /= nk;
        if (nq > 0.0) qt[d] /= nq;
      }
    }
    if (J->flags & 2) bt = 1.0 / (1.0 + exp(-bt));
    for (int j = 0; j < V; ++j) vt[j] = bf16_bits_to_double(J->v[row * V + j]);

    /* decay: S <- Diag(exp(g_t)) S */
    for (int d = 0; d < K; ++d) {
      const double a = exp((double)gt[d]);
      for (int j = 0; j < V; ++j) S[d * V + j] *= a;
    }
    /* prediction p = S^T k_t */
    for (int j = 0; j < V; ++j) p[j] = 0.0;
    for (int d = 0; d < K; ++d)
      for (int j = 0; j < V; ++j) p[j] += S[d * V + j] * kt[d];
    /* delta-rule correction: S <- S + beta k (v - p)^T */
    for (int d = 0; d < K; ++d) {
      const double c = bt * kt[d];
      for (int j = 0; j < V; ++j) S[d * V + j] += c * (vt[j] - p[j]);
    }
    /* read-out: o = scale S^T q */
    double *o = J->out + row * V;
    for (int j = 0; j < V; ++j) o[j] = 0.0;
    for (int d = 0; d < K; ++d)
      for (int j = 0; j < V; ++j) o[j] += S[d * V + j] * qt[d];
    for (int j = 0; j < V; ++j) o[j] *= J->scale;

    if (ckpt_at == t + 1)
      for (int e = 0; e < K * V; ++e) J->ckpt_state[state_off + e] = S[e];
  }
  for (int e = 0; e < K * V; ++e) J->final_state[state_off + e] = S[e];
}

static void *worker(void *arg) {
  oracle_job *J = (oracle_job *)arg;
  const int K = J->K, V = J->V;
  double *S = (double *)malloc(sizeof(double) * (size_t)K * V);
  double *p = (double *)malloc(sizeof(double) * (size_t)V);
  double *kt = (double *)malloc(sizeof(double) * (size_t)K);
  double *qt = (double *)malloc(sizeof(double) * (size_t)K);
  double *vt = (double *)malloc(sizeof(double) * (size_t)V);
  const long pairs = (long)J->N * J->H;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    long i = J->next_pair++;
    pthread_mutex_unlock(&J->lock);
    if (i >= pairs) break;
    run_pair(J, (int)(i / J->H), (int)(i % J->H), S, p, kt, qt, vt);
  }
  free(S); free(p); free(kt); free(qt); free(vt);
  return NULL;
}

/*
 * Returns 0 on success, -1 on an argument error (the caller's buffers are then
 * untouched).  num_threads <= 0 means one thread.
 */
int kda_oracle_prefill_f64(int N, long T_total, int H, int K, int V, double scale,
                           const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const float *g, const float *beta,
                           const int32_t *cu_seqlens, const float *initial_state,
                           const int32_t *ckpt_offsets,
                           double *out, double *final_state, double *ckpt_state,
                           int flags, int num_threads) {
  if (N <= 0 || H <= 0 || K <= 0 || V <= 0 || T_total < 0) return -1;
  if (!q || !k || !v || !g || !beta || !out || !final_state) return -1;
  if ((ckpt_offsets == NULL) != (ckpt_state == NULL)) return -1;
  if (!cu_seqlens && (T_total % N) != 0) return -1;
  if (cu_seqlens) {
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T_total) return -1;
    for (int n = 0; n < N; ++n)
      if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  }
  oracle_job J;
  J.N = N; J.H = H; J.K = K; J.V = V; J.T_total = T_total; J.scale = scale;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta;
  J.cu_seqlens = cu_seqlens; J.initial_state = initial_state;
  J.ckpt_offsets = ckpt_offsets;
  J.out = out; J.final_state = final_state; J.ckpt_state = ckpt_state;
  J.flags = flags;
  J.next_pair = 0;
  pthread_mutex_init(&J.lock, NULL);
  if (num_threads <= 1) {
    worker(&J);
  } else {
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)num_threads);
    for (int i = 0; i < num_threads; ++i) pthread_create(&tid[i], NULL, worker, &J);
    for (int i = 0; i < num_threads; ++i) pthread_join(tid[i], NULL);
    free(tid);
  }
  pthread_mutex_destroy(&J.lock);
  return 0;
}
