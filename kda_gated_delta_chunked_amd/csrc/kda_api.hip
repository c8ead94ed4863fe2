// kda_api.hip -- host side of libkda: argument validation, schedule choice and
// launch.  The declarations and the contract are in include/kda.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "kda.h"
#include "kda_kernels.h"

namespace {

constexpr int kHeadDim = 128;
constexpr int kMaxCkptPerSeq = 64;
constexpr int64_t kInt32Max = 2147483647LL;

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
  bool empty() const { return lo == hi; }
};

Range range_of(const void* p, uint64_t bytes) {
  Range r;
  if (p && bytes) {
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + bytes;
  }
  return r;
}

bool overlaps(const Range& a, const Range& b) {
  return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}
bool exact(const Range& a, const Range& b) { return !a.empty() && a.lo == b.lo && a.hi == b.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// checkpoint offsets per sequence (0 in the problem means 1)
int ckpt_count(const kda_problem* p) { return p->ckpt_per_seq > 1 ? p->ckpt_per_seq : 1; }

kda_status check_problem(const kda_problem* p) {
  if (!p) return KDA_ERR_INVALID_ARG;
  if (p->head_dim_k != kHeadDim || p->head_dim_v != kHeadDim) return KDA_ERR_UNSUPPORTED;
  if (p->num_seqs < 1 || p->num_heads < 1 || p->total_tokens < 0) return KDA_ERR_INVALID_ARG;
  if (!std::isfinite(p->scale)) return KDA_ERR_INVALID_ARG;
  // gate lower bound contract: [-5, 0], both ends included
  if (!std::isfinite(p->gate_lower_bound) || p->gate_lower_bound < -5.0f ||
      p->gate_lower_bound > 0.0f)
    return KDA_ERR_INVALID_ARG;
  if (p->variant != KDA_VARIANT_AUTO && p->variant != KDA_VARIANT_FUSED &&
      p->variant != KDA_VARIANT_DECOMP)
    return KDA_ERR_UNSUPPORTED;
  const int vs = p->value_split;
  if (vs != 0 && vs != 1 && vs != 2 && vs != 4 && vs != 8) return KDA_ERR_UNSUPPORTED;
  if (p->variant == KDA_VARIANT_FUSED && (vs == 1 || vs == 8)) return KDA_ERR_UNSUPPORTED;
  if (p->stages < 0 || p->stages > KDA_STAGE_RECURRENCE) return KDA_ERR_INVALID_ARG;
  if (p->stages != 0 && p->variant != KDA_VARIANT_DECOMP) return KDA_ERR_UNSUPPORTED;
  if (p->ckpt_per_seq < 0) return KDA_ERR_INVALID_ARG;
  if (p->state_dtype != KDA_STATE_F32 && p->state_dtype != KDA_STATE_BF16) return KDA_ERR_UNSUPPORTED;
  if (p->prologue & ~(KDA_PROLOGUE_QK_L2NORM | KDA_PROLOGUE_BETA_LOGIT)) return KDA_ERR_INVALID_ARG;
  if (p->ckpt_per_seq > kMaxCkptPerSeq) return KDA_ERR_UNSUPPORTED;
  // the flat output index T_total * H * 128 must fit in int32
  if (p->total_tokens * (int64_t)p->num_heads * kHeadDim > kInt32Max) return KDA_ERR_TOO_LARGE;
  if ((int64_t)p->num_seqs * p->num_heads > kInt32Max / 8) return KDA_ERR_TOO_LARGE;
  return KDA_OK;
}

// workspace size past which the slots no longer stay in MI355X's 256 MB
// Infinity Cache between the two launches (measured: a 160 MiB workspace
// still behaves as cached, a 192 MiB one does not)
constexpr size_t kDecompCacheBytes = size_t(176) << 20;

int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

size_t decomp_bytes(const kda_problem* p) {
  size_t header = 0, bytes = 0;
  int64_t slots = 0;
  kda::decomp_workspace_layout(p->num_seqs, p->total_tokens, p->num_heads, ckpt_count(p), &header,
                              &slots, &bytes);
  return bytes;
}

// Schedule choice.  FUSED: each workgroup carries one (sequence, head) pair
// and a slice of the state's columns, and repeats the chunk preparation; two
// workgroups per pair, four when there are too few pairs to occupy half the
// CUs.  DECOMP: the recurrence workgroup holds two slot buffers in LDS, so one
// runs per CU; two workgroups per pair, or four (below).  AUTO takes DECOMP
// whenever the workspace holds it (value_split 1 and 8 are DECOMP-only, 2 and 4
// exist in both).
// workgroups per pair of the one-launch schedule
int fused_vsplit(const kda_problem* p, int cus) {
  if (p->value_split) return p->value_split;
  const int64_t pairs = (int64_t)p->num_seqs * p->num_heads;
  return (cus > 0 && pairs * 2 < cus / 2) ? 4 : 2;
}

// The schedule table, keyed on the CU count and on what the host knows of the
// shape (N, H and the mean sequence length T_total / N).  The one-launch
// schedule wins when all its workgroups run at once (pairs x workgroups per
// pair <= CUs) and the sequences are short (a mean of at most two 64-token
// chunks): the per-segment chain is then too short to repay the prepare
// launch and its workspace round trip.  Measured on MI355X (256 CUs), H = 12,
// in us per call, DECOMP / FUSED: B1 T64 26.4 / 18.9, B8 T64 28.6 / 21.7,
// B8 T128 32.9 / 31.4, packed 8 x 128 30.8 / 25.5; past either bound DECOMP
// wins: B8 T192 39.2 / 40.7, B16 T128 45.3 / 53.7, B32 T64 49.9 / 52.6.
bool fused_is_faster(const kda_problem* p, int cus) {
  if (cus <= 0 || p->value_split == 1 || p->value_split == 8) return false;
  const int64_t pairs = (int64_t)p->num_seqs * p->num_heads;
  const int64_t mean_len = p->total_tokens / p->num_seqs;
  return mean_len <= 2 * 64 && pairs * fused_vsplit(p, cus) <= cus;
}

void choose(const kda_problem* p, int cus, size_t ws_bytes, int32_t* variant, int32_t* vsplit) {
  int32_t var = p->variant;
  if (var == KDA_VARIANT_AUTO) {
    var = ws_bytes >= decomp_bytes(p) ? KDA_VARIANT_DECOMP : KDA_VARIANT_FUSED;
    if (var == KDA_VARIANT_FUSED && (p->value_split == 1 || p->value_split == 8))
      var = KDA_VARIANT_DECOMP;  // rejected later by the workspace check
    if (var == KDA_VARIANT_DECOMP && fused_is_faster(p, cus)) var = KDA_VARIANT_FUSED;
  }
  *variant = var;
  if (var == KDA_VARIANT_FUSED) {
    *vsplit = fused_vsplit(p, cus);
  } else if (p->value_split) {
    *vsplit = p->value_split;
  } else {
    // measured on MI355X (256 CUs, 256 MB Infinity Cache), H = 12 unless
    // stated, ms per call, two / four workgroups per pair: while the
    // workspace stays in the Infinity Cache two are best (B1 T8192 0.251 /
    // 0.260, B1 T8192 H20 0.287 / 0.289, B4 T2048 0.103 / 0.105); once it
    // does not, four are, when they all fit at once (B2 T8192 0.335 / 0.307,
    // B1 T32768 1.070 / 0.984, B5 T8192 0.465 / 0.432, B1 T8192 H64 0.462 /
    // 0.436).  Past the CU count two (B8 T8192 0.614 / 0.751); one and eight
    // are slower everywhere.
    const int64_t pairs = (int64_t)p->num_seqs * p->num_heads;
    *vsplit = (cus > 0 && pairs * 4 <= cus && decomp_bytes(p) > kDecompCacheBytes) ? 4 : 2;
  }
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
    case KDA_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case KDA_ERR_OVERLAP: return "buffers overlap";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KDA_ERR_TOO_LARGE: return "problem exceeds the int32 flat-index bound";
    case KDA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

kda_status kda_prefill_workspace_size(const kda_problem* p, size_t* bytes) {
  if (!bytes) return KDA_ERR_INVALID_ARG;
  const kda_status st = check_problem(p);
  if (st != KDA_OK) return st;
  *bytes = p->variant == KDA_VARIANT_FUSED ? 0 : decomp_bytes(p);
  return KDA_OK;
}

kda_status kda_validate(const kda_problem* p, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const int32_t* cu_seqlens,
                        const float* initial_state, const void* out, const float* final_state,
                        const int32_t* ckpt_offsets, const float* ckpt_state,
                        const void* workspace, size_t workspace_bytes) {
  kda_status st = check_problem(p);
  if (st != KDA_OK) return st;
  const int64_t T = p->total_tokens;
  const int64_t N = p->num_seqs, H = p->num_heads;
  if (!cu_seqlens && (T % N) != 0) return KDA_ERR_INVALID_ARG;
  if (T > 0 && (!q || !k || !v || !g || !beta || !out)) return KDA_ERR_INVALID_ARG;
  if ((ckpt_offsets == nullptr) != (ckpt_state == nullptr)) return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, g, beta, cu_seqlens, initial_state, out, final_state,
                        ckpt_offsets, ckpt_state, workspace};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_ALIGNMENT;
  // DECOMP (named, or implied by a DECOMP-only value_split) needs its
  // workspace; AUTO falls back to FUSED when the workspace is smaller
  int32_t var = 0, vs = 0;
  choose(p, 0, workspace ? workspace_bytes : 0, &var, &vs);
  if (var == KDA_VARIANT_DECOMP && (!workspace || workspace_bytes < decomp_bytes(p)))
    return KDA_ERR_WORKSPACE_TOO_SMALL;

  const uint64_t tok_bf16 = (uint64_t)T * H * kHeadDim * 2;
  const uint64_t tok_f32 = (uint64_t)T * H * kHeadDim * 4;
  const uint64_t state =
      (uint64_t)N * H * kHeadDim * kHeadDim * (p->state_dtype == KDA_STATE_BF16 ? 2 : 4);
  const Range rq = range_of(q, tok_bf16), rk = range_of(k, tok_bf16), rv = range_of(v, tok_bf16);
  const Range rg = range_of(g, tok_f32), rb = range_of(beta, (uint64_t)T * H * 4);
  const Range rcu = range_of(cu_seqlens, (uint64_t)(N + 1) * 4);
  const Range rs0 = range_of(initial_state, state);
  const Range rout = range_of(out, tok_bf16), rfin = range_of(final_state, state);
  const Range roff = range_of(ckpt_offsets, (uint64_t)N * ckpt_count(p) * 4);
  const Range rck = range_of(ckpt_state, state * ckpt_count(p));
  const Range rws = range_of(workspace, workspace_bytes);

  // out: may be exactly v; must not touch any other buffer
  for (const Range& r : {rq, rk, rg, rb, rcu, rs0, rfin, roff, rck, rws})
    if (overlaps(rout, r)) return KDA_ERR_OVERLAP;
  if (overlaps(rout, rv) && !exact(rout, rv)) return KDA_ERR_OVERLAP;
  // final state: may be exactly the initial state
  for (const Range& r : {rq, rk, rv, rg, rb, rcu, roff, rck, rws})
    if (overlaps(rfin, r)) return KDA_ERR_OVERLAP;
  if (overlaps(rfin, rs0) && !exact(rfin, rs0)) return KDA_ERR_OVERLAP;
  // checkpoint buffer: no overlap with anything
  for (const Range& r : {rq, rk, rv, rg, rb, rcu, rs0, roff, rws})
    if (overlaps(rck, r)) return KDA_ERR_OVERLAP;
  // workspace: written by the call, so it overlaps no other buffer either
  for (const Range& r : {rq, rk, rv, rg, rb, rcu, rs0, roff})
    if (overlaps(rws, r)) return KDA_ERR_OVERLAP;
  return KDA_OK;
}

kda_status kda_plan(const kda_problem* p, int32_t* variant, int32_t* value_split) {
  if (!variant || !value_split) return KDA_ERR_INVALID_ARG;
  const kda_status st = check_problem(p);
  if (st != KDA_OK) return st;
  choose(p, device_cu_count(), decomp_bytes(p), variant, value_split);
  return KDA_OK;
}

kda_status kda_prefill(const kda_problem* p, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const float* g, const float* beta,
                       const int32_t* cu_seqlens, const float* initial_state, uint16_t* out,
                       float* final_state, const int32_t* ckpt_offsets, float* ckpt_state,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const kda_status st = kda_validate(p, q, k, v, g, beta, cu_seqlens, initial_state, out,
                                     final_state, ckpt_offsets, ckpt_state, workspace,
                                     workspace_bytes);
  if (st != KDA_OK) return st;
  int32_t variant = 0, vsplit = 0;
  choose(p, device_cu_count(), workspace ? workspace_bytes : 0, &variant, &vsplit);
  const hipStream_t st_ = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (variant == KDA_VARIANT_DECOMP) {
    size_t header = 0, bytes = 0;
    int64_t slots = 0;
    kda::decomp_workspace_layout(p->num_seqs, p->total_tokens, p->num_heads, ckpt_count(p), &header,
                              &slots, &bytes);
    kda::DecompArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.cu_seqlens = cu_seqlens;
    a.s0 = initial_state;
    a.out = out;
    a.final_state = final_state;
    a.ckpt_off = ckpt_offsets;
    a.ckpt = ckpt_state;
    a.ckpt_per_seq = ckpt_count(p);
    a.state_bf16 = p->state_dtype == KDA_STATE_BF16;
    a.seg_base = static_cast<int32_t*>(workspace);
    a.order = cu_seqlens ? a.seg_base + p->num_seqs + 1 : nullptr;
    a.slots = static_cast<unsigned char*>(workspace) + header;
    a.N = p->num_seqs;
    a.H = p->num_heads;
    a.T_total = p->total_tokens;
    a.prologue = p->prologue;
    a.T_fixed = cu_seqlens ? 0 : p->total_tokens / p->num_seqs;
    a.slots_per_seq = cu_seqlens ? 0 : (a.T_fixed + 63) / 64 + (ckpt_offsets ? a.ckpt_per_seq : 0);
    a.slot_bound = slots;
    a.scale = p->scale;
    const int64_t prepare_slots = cu_seqlens ? slots : (int64_t)p->num_seqs * a.slots_per_seq;
    const int stages = p->stages ? p->stages : (KDA_STAGE_PREPARE | KDA_STAGE_RECURRENCE);
    // measured on MI355X, ms per call, normal / non-temporal workspace
    // stores: B8 T8192 0.643 / 0.630, B1 T8192 0.252 / 0.272, packed 8 x 1024
    // 0.091 / 0.093 (the last two keep their workspace in the cache)
    const bool stream_ws = bytes > kDecompCacheBytes;
    err = kda::launch_decomp(a, vsplit, prepare_slots, stages, stream_ws, st_);
  } else {
    kda::FusedArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.cu_seqlens = cu_seqlens;
    a.s0 = initial_state;
    a.out = out;
    a.final_state = final_state;
    a.ckpt_off = ckpt_offsets;
    a.ckpt = ckpt_state;
    a.ckpt_per_seq = ckpt_count(p);
    a.state_bf16 = p->state_dtype == KDA_STATE_BF16;
    a.N = p->num_seqs;
    a.H = p->num_heads;
    a.num_pairs = p->num_seqs * p->num_heads;
    a.T_fixed = cu_seqlens ? 0 : p->total_tokens / p->num_seqs;
    a.scale = p->scale;
    a.prologue = p->prologue;
    err = kda::launch_fused(a, vsplit, st_);
  }
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_validate(const kda_decode_problem* p, const void* q, const void* k,
                               const void* v, const float* g, const float* beta,
                               const float* state_pool, const int32_t* state_indices,
                               const void* out) {
  if (!p) return KDA_ERR_INVALID_ARG;
  if (p->head_dim_k != kHeadDim || p->head_dim_v != kHeadDim) return KDA_ERR_UNSUPPORTED;
  if (p->num_seqs < 0 || p->tokens_per_seq < 1 || p->num_heads < 1 || p->pool_size < 1)
    return KDA_ERR_INVALID_ARG;
  if (!std::isfinite(p->scale)) return KDA_ERR_INVALID_ARG;
  if (!std::isfinite(p->gate_lower_bound) || p->gate_lower_bound < -5.0f ||
      p->gate_lower_bound > 0.0f)
    return KDA_ERR_INVALID_ARG;
  if (p->prologue & ~(KDA_PROLOGUE_QK_L2NORM | KDA_PROLOGUE_BETA_LOGIT)) return KDA_ERR_INVALID_ARG;
  const int64_t N = p->num_seqs, T = p->tokens_per_seq, H = p->num_heads;
  if (N * T * H * kHeadDim > kInt32Max) return KDA_ERR_TOO_LARGE;
  if (N > 0 && (!q || !k || !v || !g || !beta || !state_pool || !state_indices || !out))
    return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, g, beta, state_pool, state_indices, out};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_ALIGNMENT;
  const uint64_t tok_bf16 = (uint64_t)N * T * H * kHeadDim * 2;
  const Range rq = range_of(q, tok_bf16), rk = range_of(k, tok_bf16), rv = range_of(v, tok_bf16);
  const Range rg = range_of(g, tok_bf16 * 2), rb = range_of(beta, (uint64_t)N * T * H * 4);
  const Range rpool = range_of(state_pool, (uint64_t)p->pool_size * H * kHeadDim * kHeadDim * 4);
  const Range ridx = range_of(state_indices, (uint64_t)N * 4);
  const Range rout = range_of(out, tok_bf16);
  for (const Range& r : {rq, rk, rg, rb, rpool, ridx})
    if (overlaps(rout, r)) return KDA_ERR_OVERLAP;
  if (overlaps(rout, rv) && !exact(rout, rv)) return KDA_ERR_OVERLAP;
  for (const Range& r : {rq, rk, rv, rg, rb, ridx})
    if (overlaps(rpool, r)) return KDA_ERR_OVERLAP;
  return KDA_OK;
}

kda_status kda_decode(const kda_decode_problem* p, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const float* g, const float* beta, float* state_pool,
                      const int32_t* state_indices, uint16_t* out, void* stream) {
  const kda_status st = kda_decode_validate(p, q, k, v, g, beta, state_pool, state_indices, out);
  if (st != KDA_OK) return st;
  if (p->num_seqs == 0) return KDA_OK;
  kda::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.pool = state_pool;
  a.state_indices = state_indices;
  a.out = out;
  a.N = p->num_seqs;
  a.T = p->tokens_per_seq;
  a.H = p->num_heads;
  a.pool_size = p->pool_size;
  a.scale = p->scale;
  a.prologue = p->prologue;
  return kda::launch_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
