// kda_api.hip -- host side of libkda: argument validation, schedule choice and
// launch.  The declarations and the contract are in include/kda.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

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
  if (p->cu_seqlens_int64 != 0 && p->cu_seqlens_int64 != 1) return KDA_ERR_INVALID_ARG;
  if (p->ckpt_per_seq > kMaxCkptPerSeq) return KDA_ERR_UNSUPPORTED;
  if (p->chain_parts < 0 || p->chain_parts > KDA_MAX_CHAIN_PARTS) return KDA_ERR_INVALID_ARG;
  if (p->chain_parts > 1 && p->variant == KDA_VARIANT_FUSED) return KDA_ERR_UNSUPPORTED;
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

// DECOMP workspace bytes with the chain area for `pieces` (none below 2)
size_t decomp_bytes(const kda_problem* p, int pieces) {
  size_t header = 0, bytes = 0;
  int64_t slots = 0;
  kda::decomp_workspace_layout(p->num_seqs, p->total_tokens, p->num_heads, ckpt_count(p), pieces,
                              &header, &slots, &bytes);
  return bytes;
}

// Chain split.  The recurrence of a (sequence, head) pair is a chain of
// segments, one after the other; with few pairs most CUs idle while it runs.
// Cut into P pieces, the pieces after the first are run from a zero state and
// from the identity (their affine map), a scan composes the maps, and every
// piece is run again from its true incoming state.  The first split launch
// holds pairs x (P - 1) groups of 2 x vsplit workgroups.
// (pairs x pieces) the first split launch fits on a 256-CU device at one
// workgroup per pair and column group: the workspace is sized for at most this
constexpr int64_t kChainGroupBudget = 128;
// fewest 64-token chunks per piece (shorter pieces do not repay the scan)
constexpr int64_t kMinChunksPerPiece = 8;

// pieces the workspace query provides for: chain_parts when given, else the
// most that AUTO could pick from what the host knows (N, H, T_total / N)
int chain_cap(const kda_problem* p) {
  if (p->variant == KDA_VARIANT_FUSED) return 1;
  if (p->chain_parts) return p->chain_parts;
  const int64_t pairs = (int64_t)p->num_seqs * p->num_heads;
  const int64_t chunks = (p->total_tokens / p->num_seqs + 63) / 64;
  int64_t cap = 1 + kChainGroupBudget / pairs;
  cap = cap < KDA_MAX_CHAIN_PARTS ? cap : KDA_MAX_CHAIN_PARTS;
  cap = cap < chunks / kMinChunksPerPiece ? cap : chunks / kMinChunksPerPiece;
  return cap >= 3 ? (int)cap : 1;
}

size_t decomp_bytes(const kda_problem* p) { return decomp_bytes(p, chain_cap(p)); }

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
// pair <= CUs) and the sequences are short (a mean of at most one 64-token
// chunk): the per-segment chain is then too short to repay the prepare
// launch and its workspace round trip.  Measured on MI355X (256 CUs), H = 12,
// per-sequence initial states, in us per call, DECOMP / FUSED: B1 T64
// 20.9 / 16.7, B8 T64 22.9 / 19.6; past either bound DECOMP wins or ties:
// B8 T128 27.6 / 31.8, packed 8 x 128 32.6 / 32.2, B8 T192 34.0 / 43.8,
// B16 T128 40.6 / 59.5, B32 T64 45.4 / 55.0.
bool fused_is_faster(const kda_problem* p, int cus) {
  if (cus <= 0) return false;
  const int64_t pairs = (int64_t)p->num_seqs * p->num_heads;
  const int64_t mean_len = p->total_tokens / p->num_seqs;
  return mean_len <= 64 && pairs * fused_vsplit(p, cus) <= cus;
}

// Cost model of the recurrence, in segment times of the unsplit two-
// workgroup schedule, fitted to MI355X measurements (256 CUs; H = 12 unless
// stated; recurrence us unsplit -> split, vsplit, pieces):
//   B1 T8192      212 -> 96   (2, 6) / 93 (2, 11) / 92 (1, 11)
//   B2 T8192      224 -> 145  (2, 6); 167 (2, 5); 172 (2, 11)
//   B1 T32768     875 -> 305  (2, 11); 343 (2, 6)
//   B1 T2048       61 -> 51   (2, 5)
//   B1 T8192 H32  226 -> 178  (2, 3); 188 (2, 5)
//   B4 T2048       61 -> 91   (2, 3)  (the split loses: kept unsplit)
// A run of L segments costs L x seg_cost(vsplit) per round of workgroups;
// workgroups are dealt to the 8 XCDs round-robin by group and one runs per
// CU, so a launch of G groups of W workgroups takes ceil(ceil(G / 8) W /
// (CUs / 8)) rounds.  The split adds its scan (P - 2 steps) and two launches.
double seg_cost(int vsplit) { return vsplit == 1 ? 1.6 : (vsplit == 2 ? 1.0 : 1.05); }
constexpr double kScanStepCost = 0.85;  // one scan step (1.5 us), in segment times (1.74 us)
constexpr double kSplitCost = 6.0;      // the extra launches and per-run start-up

int64_t rounds(int64_t groups, int per_group, int cus) {
  const int64_t per_xcd = (groups + 7) / 8 * per_group, slots = cus / 8;
  return (per_xcd + slots - 1) / slots;
}

double split_cost(int64_t pairs, int64_t chunks, int vsplit_first, int vsplit, int P, int cus) {
  const int64_t groups = pairs * (P - 1), L = (chunks + P - 1) / P;
  return (double)L * (seg_cost(vsplit_first) * (double)rounds(groups, 2 * vsplit_first, cus) +
                      seg_cost(vsplit) * (double)rounds(groups, vsplit, cus)) +
         kScanStepCost * (P - 2) + kSplitCost;
}

// Chain pieces (and the workgroups per pair they run with) for the two-launch
// schedule: chain_parts when given; else (AUTO) the split, up to chain_cap
// pieces, whose modelled cost is below 0.9 of the unsplit run's -- over
// vsplit 1, 2 and 4 when value_split is automatic -- and whose chain area the
// workspace holds (none when no device is known).  Fewer than 3 pieces run
// nothing side by side.  The first split launch
// holds twice the workgroups of the second, so with value_split automatic it
// takes its own count (vsplit_first): at B1 T8192 H12, 11 pieces, one
// workgroup per pair and role fits the first launch in one round where two
// need two.
struct FirstPass {
  int vsplit;
  double cost;
};

int chain_pieces(const kda_problem* p, int cus, size_t ws_bytes, int32_t* vsplit, int32_t* vsplit_first) {
  *vsplit_first = *vsplit;
  if (cus < 8) return p->chain_parts ? p->chain_parts : 1;
  const int64_t pairs = (int64_t)p->num_seqs * p->num_heads;
  const int64_t chunks = (p->total_tokens / p->num_seqs + 63) / 64;
  auto first_pass = [&](int P, int vs) {
    FirstPass f{vs, split_cost(pairs, chunks, vs, vs, P, cus)};
    if (!p->value_split)
      for (int v1 : {1, 2, 4}) {
        const double c = split_cost(pairs, chunks, v1, vs, P, cus);
        if (c < f.cost) f = FirstPass{v1, c};
      }
    return f;
  };
  if (p->chain_parts) {
    if (p->chain_parts >= 2) *vsplit_first = first_pass(p->chain_parts, *vsplit).vsplit;
    return p->chain_parts;
  }
  const int cap = chain_cap(p);
  if (cap < 3) return 1;
  const double unsplit = seg_cost(*vsplit) * (double)chunks * (double)rounds(pairs, *vsplit, cus);
  double best = 0.9 * unsplit;
  int best_p = 1, best_vs = *vsplit, best_first = *vsplit;
  for (int vs : {2, 1, 4}) {
    if (p->value_split && vs != p->value_split) continue;
    for (int P = 3; P <= cap; ++P) {
      if (ws_bytes < decomp_bytes(p, P)) continue;
      const FirstPass f = first_pass(P, vs);
      if (f.cost < best) {
        best = f.cost;
        best_p = P;
        best_vs = vs;
        best_first = f.vsplit;
      }
    }
  }
  *vsplit = best_vs;
  *vsplit_first = best_first;
  return best_p;
}

void choose(const kda_problem* p, int cus, size_t ws_bytes, int32_t* variant, int32_t* vsplit,
            int32_t* pieces, int32_t* vsplit_first = nullptr) {
  int32_t var = p->variant;
  int32_t first = 0;
  *pieces = 1;
  if (var == KDA_VARIANT_AUTO) {
    // value_split 1 and 8 and a chain split exist only in DECOMP
    const bool decomp_only = p->value_split == 1 || p->value_split == 8 || p->chain_parts > 1;
    var = ws_bytes >= decomp_bytes(p, 1) ? KDA_VARIANT_DECOMP : KDA_VARIANT_FUSED;
    if (var == KDA_VARIANT_FUSED && decomp_only) var = KDA_VARIANT_DECOMP;  // rejected later by the workspace check
    if (var == KDA_VARIANT_DECOMP && !decomp_only && fused_is_faster(p, cus)) var = KDA_VARIANT_FUSED;
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
    // are slower everywhere, also where the pairs outnumber the CUs (two /
    // one: packed 32 ragged 0.553 / 0.562, 16 ragged + checkpoints 0.661 /
    // 0.707, B32 T512 0.158 / 0.158).
    const int64_t pairs = (int64_t)p->num_seqs * p->num_heads;
    *vsplit = (cus > 0 && pairs * 4 <= cus && decomp_bytes(p, 1) > kDecompCacheBytes) ? 4 : 2;
  }
  first = *vsplit;
  if (var == KDA_VARIANT_DECOMP) *pieces = chain_pieces(p, cus, ws_bytes, vsplit, &first);
  if (vsplit_first) *vsplit_first = first;
}

// ---------------------------------------------------------------------------
// The allocation-free entry point's scratch: the DECOMP workspace lives in a
// file-scope device array, one copy per GPU, held until the process ends.  In
// host code `scratch` only names the symbol: its device address (different on
// every GPU) comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is handed to kernels.
constexpr size_t kNoallocScratchBytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

// device address of this GPU's `scratch` (the current device's)
kda_status scratch_address(void** addr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KDA_ERR_HIP;
    g_scratch_addr[dev] = ptr;
  }
  *addr = g_scratch_addr[dev];
  return KDA_OK;
}

}  // namespace

namespace {

// What a decode-family call passes besides the inputs: kda_decode and the
// verify write `out`; the verify may also write a state trace; the advance
// writes no output and reads the accepted counts.
enum DecodeMode { DECODE, VERIFY, ADVANCE };

// kda_decode_validate's checks, and those of the verify and the advance
kda_status decode_check(const kda_decode_problem* p, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const float* state_pool,
                        const int32_t* state_indices, const void* out, const float* trace,
                        const int32_t* accepted, DecodeMode mode) {
  if (!p) return KDA_ERR_INVALID_ARG;
  if (p->head_dim_k != kHeadDim || p->head_dim_v != kHeadDim) return KDA_ERR_UNSUPPORTED;
  if (p->num_seqs < 0 || p->tokens_per_seq < 1 || p->num_heads < 1 || p->pool_size < 1)
    return KDA_ERR_INVALID_ARG;
  if (!std::isfinite(p->scale)) return KDA_ERR_INVALID_ARG;
  if (!std::isfinite(p->gate_lower_bound) || p->gate_lower_bound < -5.0f ||
      p->gate_lower_bound > 0.0f)
    return KDA_ERR_INVALID_ARG;
  if (p->prologue & ~(KDA_PROLOGUE_QK_L2NORM | KDA_PROLOGUE_BETA_LOGIT)) return KDA_ERR_INVALID_ARG;
  if (p->state_dtype != KDA_STATE_F32 && p->state_dtype != KDA_STATE_BF16) return KDA_ERR_INVALID_ARG;
  const uint64_t es = p->state_dtype == KDA_STATE_BF16 ? 2 : 4;  // bytes per state element
  const int64_t N = p->num_seqs, T = p->tokens_per_seq, H = p->num_heads;
  if (N * T * H * kHeadDim > kInt32Max) return KDA_ERR_TOO_LARGE;
  if (N > 0 && (!q || !k || !v || !g || !beta || !state_pool || !state_indices))
    return KDA_ERR_INVALID_ARG;
  if (N > 0 && mode != ADVANCE && !out) return KDA_ERR_INVALID_ARG;
  if (N > 0 && mode == ADVANCE && !accepted) return KDA_ERR_INVALID_ARG;
  if (mode == ADVANCE) out = nullptr;
  if (mode != VERIFY) trace = nullptr;
  if (mode != ADVANCE) accepted = nullptr;
  const void* ptrs[] = {q, k, v, g, beta, state_pool, state_indices, out, trace, accepted};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_ALIGNMENT;
  const uint64_t tok_bf16 = (uint64_t)N * T * H * kHeadDim * 2;
  const Range rq = range_of(q, tok_bf16), rk = range_of(k, tok_bf16), rv = range_of(v, tok_bf16);
  const Range rg = range_of(g, tok_bf16 * 2), rb = range_of(beta, (uint64_t)N * T * H * 4);
  const Range rpool = range_of(state_pool, (uint64_t)p->pool_size * H * kHeadDim * kHeadDim * es);
  const Range ridx = range_of(state_indices, (uint64_t)N * 4);
  const Range racc = range_of(accepted, (uint64_t)N * 4);
  const Range rout = range_of(out, tok_bf16);
  for (const Range& r : {rq, rk, rg, rb, rpool, ridx})
    if (overlaps(rout, r)) return KDA_ERR_OVERLAP;
  if (overlaps(rout, rv) && !exact(rout, rv)) return KDA_ERR_OVERLAP;
  // the pool is written (read only by a verify, checked the same way)
  for (const Range& r : {rq, rk, rv, rg, rb, ridx, racc})
    if (overlaps(rpool, r)) return KDA_ERR_OVERLAP;
  if (trace) {
    // the trace is written: it overlaps nothing else
    const Range rtr = range_of(trace, (uint64_t)N * T * H * kHeadDim * kHeadDim * es);
    for (const Range& r : {rq, rk, rv, rg, rb, rpool, ridx, rout})
      if (overlaps(rtr, r)) return KDA_ERR_OVERLAP;
  }
  return KDA_OK;
}

kda::DecodeArgs decode_args(const kda_decode_problem* p, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const float* g, const float* beta, float* state_pool,
                            const int32_t* state_indices, uint16_t* out, float* trace,
                            const int32_t* accepted, bool writeback) {
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
  a.trace = trace;
  a.accepted = accepted;
  a.writeback = writeback ? 1 : 0;
  a.state_bf16 = p->state_dtype == KDA_STATE_BF16 ? 1 : 0;
  return a;
}
}  // namespace

extern "C" {

const char* kda_status_string(int status) {
  // an int, not the enum: any value may come in, and reading an int that no
  // enumerator names through the enum type would be undefined in C++
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
    case KDA_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case KDA_ERR_OVERLAP: return "buffers overlap";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KDA_ERR_TOO_LARGE: return "problem exceeds the int32 flat-index bound";
    case KDA_ERR_HIP: return "HIP runtime error";
    case KDA_ERR_SCRATCH_TOO_SMALL:
      return "problem needs more workspace than the allocation-free entry point's static scratch";
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
                        const float* g, const float* beta, const void* cu_seqlens,
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
  // seq_order orders a packed batch's sequences
  if (p->seq_order && !cu_seqlens) return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, g, beta, cu_seqlens, initial_state, out, final_state,
                        ckpt_offsets, ckpt_state, workspace, p->seq_order};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_ALIGNMENT;
  // DECOMP (named, or implied by a DECOMP-only value_split) needs its
  // workspace; AUTO falls back to FUSED when the workspace is smaller
  // (with no device known AUTO splits no chain here; a given chain_parts
  // needs its chain area)
  int32_t var = 0, vs = 0, pieces = 1;
  choose(p, 0, workspace ? workspace_bytes : 0, &var, &vs, &pieces);
  if (var == KDA_VARIANT_DECOMP && (!workspace || workspace_bytes < decomp_bytes(p, pieces)))
    return KDA_ERR_WORKSPACE_TOO_SMALL;

  const uint64_t tok_bf16 = (uint64_t)T * H * kHeadDim * 2;
  const uint64_t tok_f32 = (uint64_t)T * H * kHeadDim * 4;
  const uint64_t state =
      (uint64_t)N * H * kHeadDim * kHeadDim * (p->state_dtype == KDA_STATE_BF16 ? 2 : 4);
  const Range rq = range_of(q, tok_bf16), rk = range_of(k, tok_bf16), rv = range_of(v, tok_bf16);
  const Range rg = range_of(g, tok_f32), rb = range_of(beta, (uint64_t)T * H * 4);
  const Range rcu = range_of(cu_seqlens, (uint64_t)(N + 1) * (p->cu_seqlens_int64 ? 8 : 4));
  const Range rord = range_of(p->seq_order, (uint64_t)N * 4);
  const Range rs0 = range_of(initial_state, state);
  const Range rout = range_of(out, tok_bf16), rfin = range_of(final_state, state);
  const Range roff = range_of(ckpt_offsets, (uint64_t)N * ckpt_count(p) * 4);
  const Range rck = range_of(ckpt_state, state * ckpt_count(p));
  const Range rws = range_of(workspace, workspace_bytes);

  // out: may be exactly v; must not touch any other buffer
  for (const Range& r : {rq, rk, rg, rb, rcu, rs0, rfin, roff, rck, rws, rord})
    if (overlaps(rout, r)) return KDA_ERR_OVERLAP;
  if (overlaps(rout, rv) && !exact(rout, rv)) return KDA_ERR_OVERLAP;
  // final state: may be exactly the initial state
  for (const Range& r : {rq, rk, rv, rg, rb, rcu, roff, rck, rws, rord})
    if (overlaps(rfin, r)) return KDA_ERR_OVERLAP;
  if (overlaps(rfin, rs0) && !exact(rfin, rs0)) return KDA_ERR_OVERLAP;
  // checkpoint buffer: no overlap with anything
  for (const Range& r : {rq, rk, rv, rg, rb, rcu, rs0, roff, rws, rord})
    if (overlaps(rck, r)) return KDA_ERR_OVERLAP;
  // workspace: written by the call, so it overlaps no other buffer either
  for (const Range& r : {rq, rk, rv, rg, rb, rcu, rs0, roff, rord})
    if (overlaps(rws, r)) return KDA_ERR_OVERLAP;
  return KDA_OK;
}

kda_status kda_plan(const kda_problem* p, int32_t* variant, int32_t* value_split,
                    int32_t* chain_parts) {
  if (!variant || !value_split) return KDA_ERR_INVALID_ARG;
  const kda_status st = check_problem(p);
  if (st != KDA_OK) return st;
  int32_t pieces = 1;
  choose(p, device_cu_count(), decomp_bytes(p), variant, value_split, &pieces);
  if (chain_parts) *chain_parts = pieces;
  return KDA_OK;
}

kda_status kda_prefill(const kda_problem* p, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const float* g, const float* beta,
                       const void* cu_seqlens, const float* initial_state, uint16_t* out,
                       float* final_state, const int32_t* ckpt_offsets, float* ckpt_state,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const kda_status st = kda_validate(p, q, k, v, g, beta, cu_seqlens, initial_state, out,
                                     final_state, ckpt_offsets, ckpt_state, workspace,
                                     workspace_bytes);
  if (st != KDA_OK) return st;
  int32_t variant = 0, vsplit = 0, pieces = 1, vsplit_first = 0;
  choose(p, device_cu_count(), workspace ? workspace_bytes : 0, &variant, &vsplit, &pieces, &vsplit_first);
  const hipStream_t st_ = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (variant == KDA_VARIANT_DECOMP) {
    size_t header = 0, bytes = 0;
    int64_t slots = 0;
    kda::decomp_workspace_layout(p->num_seqs, p->total_tokens, p->num_heads, ckpt_count(p), 1,
                                 &header, &slots, &bytes);
    kda::DecompArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.cu_seqlens = cu_seqlens;
    a.cu64 = p->cu_seqlens_int64;
    a.seq_order = p->seq_order;
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
    // the chain area follows the slots (bytes = header + slot area)
    a.pieces = pieces;
    a.pass = 0;
    a.chain = pieces >= 2 ? reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + bytes) : nullptr;
    const int64_t prepare_slots = cu_seqlens ? slots : (int64_t)p->num_seqs * a.slots_per_seq;
    // measured on MI355X, ms per call, normal / non-temporal workspace
    // stores: B8 T8192 0.643 / 0.630, B1 T8192 0.252 / 0.272, packed 8 x 1024
    // 0.091 / 0.093 (the last two keep their workspace in the cache)
    const bool stream_ws = bytes > kDecompCacheBytes;
    // a slot's heads on one XCD, also only for a workspace past the cache.
    // Measured on MI355X, outputs bit for bit the same, ms per call with
    // slot-major order / heads on one XCD: B8 T8192 0.560 / 0.552 (prepare
    // 0.289 / 0.282), 16 ragged + checkpoints 0.689 / 0.678, 32 ragged 0.579
    // / 0.570, B6 T8192 0.471 / 0.468; with the workspace in the cache no
    // gain (B8 T1024 0.075 both ways, B1 T8192 0.133 both ways) or a loss
    // (B1 T512 0.034 / 0.035: the prepare alike, the recurrence slower)
    a.prep_xcd = stream_ws;
    const int stages = p->stages ? p->stages : (KDA_STAGE_PREPARE | KDA_STAGE_RECURRENCE);
    err = kda::launch_decomp(a, vsplit, vsplit_first, prepare_slots, stages, stream_ws, st_);
  } else {
    kda::FusedArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.cu_seqlens = cu_seqlens;
    a.cu64 = p->cu_seqlens_int64;
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
    a.T_total = p->total_tokens;
    a.T_fixed = cu_seqlens ? 0 : p->total_tokens / p->num_seqs;
    a.scale = p->scale;
    a.prologue = p->prologue;
    err = kda::launch_fused(a, vsplit, st_);
  }
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_prefill_noalloc(const kda_problem* p, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const float* g, const float* beta,
                               const void* cu_seqlens, const float* initial_state, uint16_t* out,
                               float* final_state, const int32_t* ckpt_offsets, float* ckpt_state,
                               void* stream) {
  const kda_status st = check_problem(p);
  if (st != KDA_OK) return st;
  // FUSED needs no workspace; AUTO and DECOMP may take the two-launch
  // schedule, whose workspace must fit the static scratch (without the chain
  // area, unless chain_parts asks for it, AUTO then splits no chain)
  size_t need = p->variant == KDA_VARIANT_FUSED ? 0 : decomp_bytes(p);
  if (need > kNoallocScratchBytes && p->chain_parts < 2) need = decomp_bytes(p, 1);
  if (need > kNoallocScratchBytes) return KDA_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  if (need) {
    const kda_status sa = scratch_address(&ws);
    if (sa != KDA_OK) return sa;
  }
  return kda_prefill(p, q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, ckpt_offsets,
                     ckpt_state, ws, need ? kNoallocScratchBytes : 0, stream);
}

kda_status kda_decode_validate(const kda_decode_problem* p, const void* q, const void* k,
                               const void* v, const float* g, const float* beta,
                               const float* state_pool, const int32_t* state_indices,
                               const void* out) {
  return decode_check(p, q, k, v, g, beta, state_pool, state_indices, out, nullptr, nullptr, DECODE);
}



kda_status kda_decode(const kda_decode_problem* p, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const float* g, const float* beta, float* state_pool,
                      const int32_t* state_indices, uint16_t* out, void* stream) {
  const kda_status st = kda_decode_validate(p, q, k, v, g, beta, state_pool, state_indices, out);
  if (st != KDA_OK) return st;
  if (p->num_seqs == 0) return KDA_OK;
  const kda::DecodeArgs a =
      decode_args(p, q, k, v, g, beta, state_pool, state_indices, out, nullptr, nullptr, true);
  return kda::launch_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_verify(const kda_decode_problem* p, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const float* g, const float* beta,
                             const float* state_pool, const int32_t* state_indices, uint16_t* out,
                             float* state_trace, void* stream) {
  const kda_status st =
      decode_check(p, q, k, v, g, beta, state_pool, state_indices, out, state_trace, nullptr, VERIFY);
  if (st != KDA_OK) return st;
  if (p->num_seqs == 0) return KDA_OK;
  // the pool is only read: the kernel runs with its write-back off
  const kda::DecodeArgs a = decode_args(p, q, k, v, g, beta, const_cast<float*>(state_pool), state_indices,
                                        out, state_trace, nullptr, false);
  return kda::launch_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_advance(const kda_decode_problem* p, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const float* g, const float* beta, float* state_pool,
                              const int32_t* state_indices, const int32_t* accepted, void* stream) {
  const kda_status st =
      decode_check(p, q, k, v, g, beta, state_pool, state_indices, nullptr, nullptr, accepted, ADVANCE);
  if (st != KDA_OK) return st;
  if (p->num_seqs == 0) return KDA_OK;
  const kda::DecodeArgs a =
      decode_args(p, q, k, v, g, beta, state_pool, state_indices, nullptr, nullptr, accepted, true);
  return kda::launch_decode(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_commit(const kda_decode_problem* p, float* state_pool,
                             const int32_t* state_indices, const float* state_trace,
                             const int32_t* accepted, void* stream) {
  if (!p) return KDA_ERR_INVALID_ARG;
  if (p->head_dim_k != kHeadDim || p->head_dim_v != kHeadDim) return KDA_ERR_UNSUPPORTED;
  if (p->num_seqs < 0 || p->tokens_per_seq < 1 || p->num_heads < 1 || p->pool_size < 1)
    return KDA_ERR_INVALID_ARG;
  if (p->state_dtype != KDA_STATE_F32 && p->state_dtype != KDA_STATE_BF16) return KDA_ERR_INVALID_ARG;
  const uint64_t es = p->state_dtype == KDA_STATE_BF16 ? 2 : 4;
  const int64_t N = p->num_seqs, T = p->tokens_per_seq, H = p->num_heads;
  if (N * T * H * kHeadDim > kInt32Max) return KDA_ERR_TOO_LARGE;
  if (N > 0 && (!state_pool || !state_indices || !state_trace || !accepted)) return KDA_ERR_INVALID_ARG;
  const void* ptrs[] = {state_pool, state_indices, state_trace, accepted};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KDA_ERR_ALIGNMENT;
  const Range rpool = range_of(state_pool, (uint64_t)p->pool_size * H * kHeadDim * kHeadDim * es);
  const Range ridx = range_of(state_indices, (uint64_t)N * 4);
  const Range racc = range_of(accepted, (uint64_t)N * 4);
  const Range rtr = range_of(state_trace, (uint64_t)N * T * H * kHeadDim * kHeadDim * es);
  for (const Range& r : {ridx, racc, rtr})
    if (overlaps(rpool, r)) return KDA_ERR_OVERLAP;
  if (N == 0) return KDA_OK;
  kda::DecodeCommitArgs a;
  a.pool = state_pool;
  a.state_indices = state_indices;
  a.trace = state_trace;
  a.accepted = accepted;
  a.N = p->num_seqs;
  a.T = p->tokens_per_seq;
  a.H = p->num_heads;
  a.pool_size = p->pool_size;
  a.state_bf16 = p->state_dtype == KDA_STATE_BF16 ? 1 : 0;
  return kda::launch_decode_commit(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
