// kda_ckpt.h -- checkpoint offsets and segment boundaries of one sequence,
// shared by the two prefill schedules.
//
// A sequence of L tokens is processed in segments: its 64-token chunks,
// aligned to the sequence start, with every chunk that holds a checkpoint
// offset strictly inside it cut in two at that offset, so that the state
// after p tokens is a segment boundary and is exported exactly (lmdeploy PR
// #5050, Modification: the state at the requested position is exported while
// the whole interval is processed).
//
// A sequence has C offsets, taken in order.  An offset is honoured when it
// lies in [0, L] and is not below the previous honoured one; the others
// export nothing and leave their checkpoint slot untouched (offsets are the
// caller's contract and are never checked on the host).
#ifndef KDA_CKPT_H_
#define KDA_CKPT_H_

#include <hip/hip_runtime.h>

#include <cstdint>

namespace kda {

// Token range of a sequence from its two cu_seqlens entries b = cu[n] and
// e = cu[n + 1], kept inside [0, T_total]: b is clamped into [0, T_total] and
// e into [b, T_total].  Offsets that break the contract (start at 0, end at
// T_total, non-decreasing; lmdeploy PR #5050, Modification, leaves them to the
// caller) then give a shorter or empty sequence, never an access outside the
// q/k/v/g/beta/out tensors.
__host__ __device__ inline void clamp_seq_range(int64_t b, int64_t e, int64_t T_total, int64_t* bos,
                                                int64_t* len) {
  b = b < 0 ? 0 : (b > T_total ? T_total : b);
  e = e < b ? b : (e > T_total ? T_total : e);
  *bos = b;
  *len = e - b;
}

// Entry n of cu_seqlens, held as int32 or (cu64) int64.
__host__ __device__ inline int64_t cu_at(const void* cu, int cu64, int64_t n) {
  return cu64 ? static_cast<const int64_t*>(cu)[n] : (int64_t)static_cast<const int32_t*>(cu)[n];
}

// On the device the C <= 64 offsets live one per lane of the wave (lane c
// holds offset c, read once at kernel start) and are taken out with
// readlane: the walks below then do no memory access, so they add no wait on
// the wave's memory counters.  Host code (tests) reads them through p.
struct CkptList {
  const int32_t* p;  // the sequence's C offsets (host reads)
  int lane_val;      // device: offset number `lane` of the sequence
  int C;             // 0: no offsets
  int len;           // tokens of the sequence
  __host__ __device__ int at(int c) const {
#ifdef __HIP_DEVICE_COMPILE__
    return __builtin_amdgcn_readlane(lane_val, c);
#else
    return p[c];
#endif
  }
};

// The offsets of sequence n (row n of [N, C]) as seen by this lane.
__device__ inline CkptList load_ckpt_list(const int32_t* offs, int C, int n, int len) {
  CkptList k;
  k.p = nullptr;
  k.C = offs ? C : 0;
  k.len = len;
  const int lane = threadIdx.x & 63;
  k.lane_val = (offs && lane < C) ? offs[(size_t)n * C + lane] : 0;
  return k;
}

// f(c, p) for every honoured offset, in order
template <class F>
__host__ __device__ inline void for_each_honoured(const CkptList& k, F f) {
  int last = 0;
  for (int c = 0; c < k.C; ++c) {
    const int p = k.at(c);
    if (p < last || p > k.len) continue;
    last = p;
    f(c, p);
  }
}

// f(x) for every cut point: honoured, strictly inside, off the 64-token grid,
// each value once, ascending
template <class F>
__host__ __device__ inline void for_each_cut(const CkptList& k, F f) {
  int last_cut = 0;
  for_each_honoured(k, [&](int, int p) {
    if (p > last_cut && p < k.len && (p & 63) != 0) {
      f(p);
      last_cut = p;
    }
  });
}

__host__ __device__ inline int count_cuts(const CkptList& k) {
  int n = 0;
  for_each_cut(k, [&](int) { ++n; });
  return n;
}

// Interior boundary i (0-based, ascending) of the segments.  Chunk boundary
// 64 m (m >= 1) and cut x_k merge into one ascending list; x_k sits at
// position (x_k - 1) / 64 + k, and a position no cut takes holds the chunk
// boundary 64 (i - cuts before it + 1).
__host__ __device__ inline int interior_boundary(const CkptList& k, int i) {
  int kk = 0, before = 0, found = -1;
  for_each_cut(k, [&](int x) {
    const int pos = (x - 1) / 64 + kk;
    if (pos == i) found = x;
    else if (pos < i) ++before;
    ++kk;
  });
  return found >= 0 ? found : 64 * (i - before + 1);
}

// first segment boundary after p0 (p0 < len): the next chunk boundary or an
// earlier cut, at most len
__host__ __device__ inline int next_boundary(const CkptList& k, int p0) {
  int e = (p0 / 64 + 1) * 64;
  if (e > k.len) e = k.len;
  int best = e;
  for_each_cut(k, [&](int x) {
    if (x > p0 && x < best) best = x;
  });
  return best;
}

}  // namespace kda

#endif  // KDA_CKPT_H_
