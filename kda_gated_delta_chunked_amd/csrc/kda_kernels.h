// kda_kernels.h -- launch interface between the C ABI layer and the HIP
// kernels of libkda (internal; not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

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
  const int32_t* ckpt_off;    // NULL: no export
  float* ckpt;
  int N;
  int H;
  int num_pairs;              // N * H
  int64_t T_fixed;
  float scale;
};

// vsplit = workgroups per (sequence, head): 2 or 4.
hipError_t launch_fused(const FusedArgs& a, int vsplit, hipStream_t stream);

}  // namespace kda
