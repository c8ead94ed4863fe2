// kda_kernels.h -- launch interface between the C ABI layer and the HIP
// kernels of libkda (internal; not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// A workgroup barrier that orders LDS accesses only.  Its release side waits
// for the wave's own outstanding LDS operations, not for its global loads and
// stores, as a barrier on all memory (__syncthreads) does: that one waits for
// every store of the wave to be acknowledged.  For kernels whose waves share
// data through LDS only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Arguments of the one-launch schedule.  Pointers are device memory; q/k/v/out
// are bf16 bit patterns.  Layouts are those of include/kda.h.
struct FusedArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* g;
  const float* beta;
  const void* cu_seqlens;     // int32 or int64 [N + 1] (cu64); NULL: N sequences of T_fixed tokens
  int cu64;
  const float* s0;            // NULL: zero initial state
  uint16_t* out;
  float* final_state;         // may be NULL
  const int32_t* ckpt_off;    // [N, ckpt_per_seq]; NULL: no export
  float* ckpt;                // [N, ckpt_per_seq, H, 128, 128]
  int ckpt_per_seq;           // C >= 1
  int state_bf16;             // states (s0, final_state, ckpt) are bf16, not fp32
  int N;
  int H;
  int num_pairs;              // N * H
  int64_t T_total;
  int64_t T_fixed;
  float scale;
  int prologue;               // bit 0: L2-normalise q and k; bit 1: beta is a logit
};

// vsplit = workgroups per (sequence, head): 2 or 4.
hipError_t launch_fused(const FusedArgs& a, int vsplit, hipStream_t stream);

// Two-launch schedule.  The workspace holds a header of (N + 1) int32 slot
// offsets and N int32 sequence indices in recurrence order (packed layout),
// followed by one slot of kDecompSlotBytes per (segment, head).
constexpr int kDecompSlotBytes = 60416;

struct DecompArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* g;
  const float* beta;
  const void* cu_seqlens;     // int32 or int64 [N + 1] (cu64); NULL: N sequences of T_fixed tokens
  int cu64;
  const int32_t* seq_order;   // caller's recurrence order (packed layout), or NULL
  const float* s0;            // NULL: zero initial state
  uint16_t* out;
  float* final_state;         // may be NULL
  const int32_t* ckpt_off;    // [N, ckpt_per_seq]; NULL: no export
  float* ckpt;                // [N, ckpt_per_seq, H, 128, 128]
  int ckpt_per_seq;           // C >= 1
  int state_bf16;             // states (s0, final_state, ckpt) are bf16, not fp32
  int prologue;               // bit 0: L2-normalise q and k; bit 1: beta is a logit
  unsigned char* slots;       // workspace slot area
  int32_t* seg_base;          // workspace header: first slot of each sequence (packed layout)
  int32_t* order;             // workspace header: sequences by decreasing length (packed layout), or NULL
  int N;
  int H;
  int64_t T_total;
  int64_t T_fixed;
  int64_t slots_per_seq;      // fixed layout: slots owned by each sequence
  int64_t slot_bound;         // slots the workspace holds
  float scale;
  // prepare launch order.  0: block b prepares slot b / H, head b % H.  1:
  // block b prepares slot 8 (b / 8 / H) + b % 8, head (b / 8) % H.  Blocks go
  // to the 8 XCDs in turn, so with 1 the H workgroups of a slot share one XCD
  // and its L2 fetches the slot's beta rows (all heads of a token in one
  // row) once instead of on up to 8 XCDs.
  int prep_xcd;
  // chain split (pieces >= 2): each (sequence, head)'s segments are cut into
  // `pieces` consecutive ranges; `chain` holds per pair and piece three fp32
  // 128 x 128 matrices (chain_matrix).  pass 0: no split; 1 and 2: the two
  // recurrence launches of the split (set by launch_decomp)
  int pieces;
  int pass;
  float* chain;
};

// The chain split's matrices of pair n * H + h, piece p: 0 = the state
// entering the piece, 1 = the piece's end state from a zero start, 2 = the
// transpose of the piece's state transition (its end state from the
// identity with V = 0).  Element offset into the chain area.
constexpr int kChainMatrices = 3;
__host__ __device__ constexpr size_t chain_matrix(int64_t pair, int pieces, int p, int which) {
  return (((size_t)pair * pieces + p) * kChainMatrices + which) * 128 * 128;
}
inline size_t chain_bytes(int64_t pairs, int pieces) {
  return pieces >= 2 ? (size_t)pairs * pieces * kChainMatrices * 128 * 128 * 4 : 0;
}

// Workspace layout for (N, T_total, H) with `pieces` chain pieces: header
// bytes, slot capacity and total bytes (the chain area, when pieces >= 2,
// follows the slots).
inline void decomp_workspace_layout(int64_t N, int64_t T_total, int64_t H, int64_t C, int pieces,
                                    size_t* header, int64_t* slots, size_t* bytes) {
  *header = (size_t)(((2 * N + 1) * 4 + 255) / 256 * 256);
  // ceil(L/64) summed over sequences is at most floor(T/64) + N; C more per
  // sequence for the chunks cut at its C checkpoint offsets
  *slots = T_total / 64 + N + N * (C < 1 ? 1 : C);
  *bytes = *header + (size_t)(*slots) * (size_t)H * kDecompSlotBytes + chain_bytes(N * H, pieces);
}

// vsplit = workgroups per (sequence, head): 1, 2, 4 or 8.  prepare_slots =
// slots the prepare launch covers (fixed layout: N * slots_per_seq; packed:
// slot_bound), rounded up to a multiple of 8 when a.prep_xcd is set.
// stages: bit 0 = the prepare launch (and the slot plan), bit 1 = the recurrence.
// stream_ws: the prepare writes the workspace with non-temporal stores (for a
// workspace that does not stay in the Infinity Cache until the recurrence).
// With a.pieces >= 2 the recurrence runs as the chain split's two launches
// with the scan of the piece transitions between them; the first of them
// with vsplit_first workgroups per pair and role, the second with vsplit.
hipError_t launch_decomp(const DecompArgs& a, int vsplit, int vsplit_first, int64_t prepare_slots, int stages,
                         bool stream_ws, hipStream_t stream);

// State-pool decode: N requests advance by T tokens each from the pool
// states their indices name (kda_decode.hip).
struct DecodeArgs {
  const uint16_t* q;          // [N * T, H, 128] bf16
  const uint16_t* k;
  const uint16_t* v;
  const float* g;             // [N * T, H, 128]
  const float* beta;          // [N * T, H]
  float* pool;                // [pool_size, H, 128, 128] fp32 or bf16, updated in place
  const int32_t* state_indices;  // [N]; outside [0, pool_size): no state
  uint16_t* out;              // [N * T, H, 128] bf16, or NULL (no outputs)
  int N;
  int T;
  int H;
  int64_t pool_size;
  float scale;
  int prologue;               // bit 0: L2-normalise q and k; bit 1: beta is a logit
  float* trace;               // NULL, or [N, T, H, 128, 128]: the state after each token
  const int32_t* accepted;    // NULL (every request takes its T tokens), or [N]: request n
                              // takes its first accepted[n] (outside [0, T]: none)
  int writeback;              // store the advanced state back into the pool
  int state_bf16;             // pool and trace hold bf16 states (else fp32)
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Commit after a verify: pool[idx[n]] <- trace[n, accepted[n] - 1] for the
// requests with a pool index and 1 <= accepted[n] <= T.
struct DecodeCommitArgs {
  float* pool;
  const int32_t* state_indices;
  const float* trace;         // [N, T, H, 128, 128]
  const int32_t* accepted;    // [N]
  int N;
  int T;
  int H;
  int64_t pool_size;
  int state_bf16;             // pool and trace hold bf16 states (else fp32)
};

hipError_t launch_decode_commit(const DecodeCommitArgs& a, hipStream_t stream);

}  // namespace kda
