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
  const int32_t* cu_seqlens;  // NULL: N sequences of T_fixed tokens
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
  int64_t T_fixed;
  float scale;
  int prologue;               // bit 0: L2-normalise q and k; bit 1: beta is a logit
};

// vsplit = workgroups per (sequence, head): 2 or 4.
hipError_t launch_fused(const FusedArgs& a, int vsplit, hipStream_t stream);

// Two-launch schedule.  The workspace holds a header of (N + 1) int32 slot
// offsets and N int32 sequence indices in recurrence order (packed layout),
// followed by one slot of kDecompSlotBytes per (segment, head).
constexpr int kDecompSlotBytes = 64512;

struct DecompArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* g;
  const float* beta;
  const int32_t* cu_seqlens;  // NULL: N sequences of T_fixed tokens
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
};

// Workspace layout for (N, T_total, H): header bytes and slot capacity.
inline void decomp_workspace_layout(int64_t N, int64_t T_total, int64_t H, int64_t C,
                                    size_t* header, int64_t* slots, size_t* bytes) {
  *header = (size_t)(((2 * N + 1) * 4 + 255) / 256 * 256);
  // ceil(L/64) summed over sequences is at most floor(T/64) + N; C more per
  // sequence for the chunks cut at its C checkpoint offsets
  *slots = T_total / 64 + N + N * (C < 1 ? 1 : C);
  *bytes = *header + (size_t)(*slots) * (size_t)H * kDecompSlotBytes;
}

// vsplit = workgroups per (sequence, head): 1, 2, 4 or 8.  prepare_slots =
// slots the prepare launch covers (fixed layout: N * slots_per_seq; packed:
// slot_bound).
// stages: bit 0 = the prepare launch (and the slot plan), bit 1 = the recurrence.
// stream_ws: the prepare writes the workspace with non-temporal stores (for a
// workspace that does not stay in the Infinity Cache until the recurrence).
hipError_t launch_decomp(const DecompArgs& a, int vsplit, int64_t prepare_slots, int stages,
                         bool stream_ws, hipStream_t stream);

// State-pool decode: N requests advance by T tokens each from the pool
// states their indices name (kda_decode.hip).
struct DecodeArgs {
  const uint16_t* q;          // [N * T, H, 128] bf16
  const uint16_t* k;
  const uint16_t* v;
  const float* g;             // [N * T, H, 128]
  const float* beta;          // [N * T, H]
  float* pool;                // [pool_size, H, 128, 128], updated in place
  const int32_t* state_indices;  // [N]; outside [0, pool_size): no state
  uint16_t* out;              // [N * T, H, 128] bf16
  int N;
  int T;
  int H;
  int64_t pool_size;
  float scale;
  int prologue;               // bit 0: L2-normalise q and k; bit 1: beta is a logit
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace kda
