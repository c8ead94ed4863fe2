/* A plain C99 caller of libkda: include/kda.h must compile as C and the
 * library must be callable from C with no C++ or HIP headers.  Host-only
 * entry points are called (no device is touched); the results are printed as
 * "key value" lines that tests/test_c_consumer.py compares with the Python
 * binding's view of the same calls and struct layouts. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

#define FIELD(T, f) printf(#T "." #f " %zu %zu\n", offsetof(T, f), sizeof(((T*)0)->f))

static kda_problem problem(int32_t n, int64_t tokens, int32_t h, int32_t variant, int32_t ckpt) {
  kda_problem p;
  memset(&p, 0, sizeof p);
  p.num_seqs = n;
  p.total_tokens = tokens;
  p.num_heads = h;
  p.head_dim_k = 128;
  p.head_dim_v = 128;
  p.scale = 0.08838834764831845f;
  p.gate_lower_bound = -5.0f;
  p.variant = variant;
  p.ckpt_per_seq = ckpt;
  return p;
}

/* fake, 16-byte aligned, disjoint addresses: kda_validate compares pointers
 * and never dereferences them */
static const void* addr(int i) { return (const void*)(uintptr_t)(((uint64_t)1 << 40) + ((uint64_t)i << 32)); }

int main(void) {
  printf("sizeof.kda_problem %zu\n", sizeof(kda_problem));
  FIELD(kda_problem, num_seqs);
  FIELD(kda_problem, total_tokens);
  FIELD(kda_problem, num_heads);
  FIELD(kda_problem, head_dim_k);
  FIELD(kda_problem, head_dim_v);
  FIELD(kda_problem, scale);
  FIELD(kda_problem, gate_lower_bound);
  FIELD(kda_problem, variant);
  FIELD(kda_problem, value_split);
  FIELD(kda_problem, stages);
  FIELD(kda_problem, ckpt_per_seq);
  FIELD(kda_problem, state_dtype);
  FIELD(kda_problem, prologue);
  FIELD(kda_problem, cu_seqlens_int64);
  FIELD(kda_problem, seq_order);
  FIELD(kda_problem, chain_parts);
  printf("sizeof.kda_decode_problem %zu\n", sizeof(kda_decode_problem));
  FIELD(kda_decode_problem, num_seqs);
  FIELD(kda_decode_problem, tokens_per_seq);
  FIELD(kda_decode_problem, num_heads);
  FIELD(kda_decode_problem, head_dim_k);
  FIELD(kda_decode_problem, head_dim_v);
  FIELD(kda_decode_problem, scale);
  FIELD(kda_decode_problem, gate_lower_bound);
  FIELD(kda_decode_problem, pool_size);
  FIELD(kda_decode_problem, prologue);
  FIELD(kda_decode_problem, state_dtype);

  /* workspace sizes: fixed B8 T8192 H12, a packed batch with 3 offsets per
   * sequence, the one-launch schedule (no workspace), B1 T8192 H12 (with the
   * chain area AUTO may use) and the same with 4 chain pieces */
  kda_problem ws[5] = {problem(8, 8 * 8192, 12, KDA_VARIANT_AUTO, 0),
                       problem(5, 1000, 3, KDA_VARIANT_DECOMP, 3),
                       problem(8, 8 * 8192, 12, KDA_VARIANT_FUSED, 0),
                       problem(1, 8192, 12, KDA_VARIANT_AUTO, 0),
                       problem(1, 8192, 12, KDA_VARIANT_DECOMP, 0)};
  ws[4].chain_parts = 4;
  for (int i = 0; i < 5; ++i) {
    size_t bytes = 0;
    const kda_status s = kda_prefill_workspace_size(&ws[i], &bytes);
    printf("workspace.%d %d %zu\n", i, (int)s, bytes);
  }

  /* kda_validate: a good fixed-layout call, then one change each */
  kda_problem p = problem(2, 512, 4, KDA_VARIANT_FUSED, 0);
  const void* q = addr(0);
  const void* k = addr(1);
  const void* v = addr(2);
  const float* g = (const float*)addr(3);
  const float* beta = (const float*)addr(4);
  const float* s0 = (const float*)addr(5);
  const void* out = addr(6);
  const float* fin = (const float*)addr(7);
  printf("validate.good %d\n", (int)kda_validate(&p, q, k, v, g, beta, NULL, s0, out, fin, NULL, NULL, NULL, 0));
  printf("validate.misaligned %d\n",
         (int)kda_validate(&p, (const char*)q + 2, k, v, g, beta, NULL, s0, out, fin, NULL, NULL, NULL, 0));
  printf("validate.alias_out_v %d\n", (int)kda_validate(&p, q, k, v, g, beta, NULL, s0, v, fin, NULL, NULL, NULL, 0));
  printf("validate.overlap_out_q %d\n",
         (int)kda_validate(&p, q, k, v, g, beta, NULL, s0, (const char*)q + 256, fin, NULL, NULL, NULL, 0));
  p.head_dim_k = 64;
  printf("validate.head_dim %d\n", (int)kda_validate(&p, q, k, v, g, beta, NULL, s0, out, fin, NULL, NULL, NULL, 0));
  p.head_dim_k = 128;
  p.gate_lower_bound = -6.0f;
  printf("validate.bound %d\n", (int)kda_validate(&p, q, k, v, g, beta, NULL, s0, out, fin, NULL, NULL, NULL, 0));
  p.gate_lower_bound = -5.0f;
  p.variant = KDA_VARIANT_DECOMP;
  printf("validate.no_workspace %d\n", (int)kda_validate(&p, q, k, v, g, beta, NULL, s0, out, fin, NULL, NULL, NULL, 0));

  /* decode validation */
  kda_decode_problem d;
  memset(&d, 0, sizeof d);
  d.num_seqs = 4;
  d.tokens_per_seq = 1;
  d.num_heads = 2;
  d.head_dim_k = 128;
  d.head_dim_v = 128;
  d.scale = 0.125f;
  d.gate_lower_bound = -5.0f;
  d.pool_size = 6;
  printf("decode.good %d\n", (int)kda_decode_validate(&d, q, k, v, g, beta, s0, (const int32_t*)addr(8), out));
  d.pool_size = 0;
  printf("decode.empty_pool %d\n", (int)kda_decode_validate(&d, q, k, v, g, beta, s0, (const int32_t*)addr(8), out));
  d.pool_size = 6;

  /* speculative verify and commit: argument errors only (a call that passes
   * every check would launch) */
  float* pool = (float*)addr(5);
  const int32_t* idx = (const int32_t*)addr(8);
  printf("verify.no_out %d\n", (int)kda_decode_verify(&d, (const uint16_t*)q, (const uint16_t*)k,
                                                       (const uint16_t*)v, g, beta, pool, idx, NULL,
                                                       (float*)addr(9), NULL));
  printf("verify.trace_on_pool %d\n", (int)kda_decode_verify(&d, (const uint16_t*)q, (const uint16_t*)k,
                                                              (const uint16_t*)v, g, beta, pool, idx,
                                                              (uint16_t*)out, pool + 4, NULL));
  printf("commit.no_accepted %d\n", (int)kda_decode_commit(&d, pool, idx, (const float*)addr(9), NULL, NULL));
  printf("commit.trace_on_pool %d\n",
         (int)kda_decode_commit(&d, pool, idx, pool + 4, (const int32_t*)addr(10), NULL));
  printf("advance.no_accepted %d\n", (int)kda_decode_advance(&d, (const uint16_t*)q, (const uint16_t*)k,
                                                               (const uint16_t*)v, g, beta, pool, idx, NULL,
                                                               NULL));

  for (int s = -8; s <= 0; ++s) printf("status.%d %s\n", s, kda_status_string(s));
  return 0;
}
