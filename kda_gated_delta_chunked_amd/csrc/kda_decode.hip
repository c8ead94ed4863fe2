// kda_decode.hip -- KDA decode / multi-token state update on a state pool for
// gfx950 (MI355X).
//
// Serving keeps one fp32 K x V state per (request, head) in a pool and, per
// step, advances each request by one token (decode) or a few (multi-token
// verify), addressed by a per-request pool index (the state pool and
// ssm_state_indices of the sglang KDA decode backend, FlashInferKDAKernel
// page; FlashInfer PR #4262 leaves decode and state-pool features on its
// other path).  The update is the token recurrence itself:
//   S <- Diag(exp(g_t)) S,  u = beta_t (v_t - S^T k_t),  S <- S + k_t u^T,
//   o_t = scale S^T q_t = scale (S_decayed^T q_t + (k_t . q_t) u)
// so each token needs two reductions over the 128 key rows of the state,
// and no chunking.
//
// One workgroup of 256 threads owns one (sequence, head) and 8 CPT of the 128
// state columns, CPT = 4 with an fp32 pool and 8 with a bf16 one; columns are
// independent, so a state runs in P = 128 / (8 CPT) workgroups.  Thread
// (rr = tid / 8, cg = tid % 8) holds rows rr + 32 i (i = 0..3) of CPT
// consecutive columns in registers, read once from the pool, kept across the
// call's tokens and written back in place.  Workgroups are handed to the 8
// XCDs in turn, so block b takes part (b / 8) % P of pair 8 (b / (8 P)) + b %
// 8: the workgroups of a pair share one XCD and its L2, which serves the token
// vectors they all read.  The path is bound by HBM: 64 KiB of fp32 state in
// and out per (sequence, head), 32 KiB with a bf16 pool (widened on load, the
// tokens in fp32, rounded to nearest even once on store).
//
// Speculative steps use the same kernel: a verify runs the T draft tokens
// with the pool only read (write-back off), optionally storing the state after
// every token to a trace; a commit launch then copies each request's traced
// state at its accepted length into the pool, or, with no trace, an advance
// runs the kernel again over each request's first accepted[n] tokens only,
// with no outputs, and writes that state back.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int DK = 128;
constexpr int QCOLS = 32;  // state columns per workgroup of the commit

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// two floats to two bf16 (round to nearest even), low half first
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 r = __builtin_convertvector((f2){x, y}, b2);
  return __builtin_bit_cast(uint32_t, r);
}

// four bf16 (two packed pairs, low half first) to four floats (exact)
__device__ __forceinline__ float4 bf16x4_to_f32(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}

// CPT state columns per thread: 4 for an fp32 pool, 8 for a bf16 one (one
// 16-byte load per row piece, half as many workgroups).  Measured on MI355X,
// 1024 requests x 1 token x 12 heads, us per call, CPT 4 / 8: fp32 298 / 312,
// bf16 200 / 161; 4 tokens bf16 445 / 410.
template <int CPT>
__global__ __launch_bounds__(256) void kda_decode_kernel(DecodeArgs a) {
  constexpr int WC = 8 * CPT;      // state columns per workgroup
  constexpr int PARTS = DK / WC;   // workgroups per (sequence, head)
  __shared__ float sk[DK], sq[DK], sd[DK];  // k, q and exp(g) of the token
  __shared__ float sv[WC];                  // v of the token, this workgroup's columns
  __shared__ float red[2][4][WC];           // per-wave partial S^T k and S^T q
  __shared__ float sbeta;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cg = tid & 7, rr = tid >> 3;
  const int64_t blk = blockIdx.x;
  const int part = (int)((blk >> 3) % PARTS);
  const int64_t pair = (blk / (8 * PARTS)) * 8 + (blk & 7);
  const int H = a.H;
  if (pair >= (int64_t)a.N * H) return;
  const int n = (int)(pair / H), h = (int)(pair - (int64_t)n * H);
  const int col = part * WC + CPT * cg;
  const int T = a.T;
  const int idx = a.state_indices[n];
  // tokens this request takes: all T, or its accepted prefix (none when the
  // count is out of range)
  int Tn = T;
  if (a.accepted) {
    const int acc = a.accepted[n];
    Tn = acc >= 0 && acc <= T ? acc : 0;
  }

  if (idx < 0 || (int64_t)idx >= a.pool_size) {
    // a request slot with no state: its outputs are zero, no state is touched
    if (rr == 0 && a.out)
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int c = 0; c < CPT; c += 4)
          *reinterpret_cast<uint2*>(a.out + (((int64_t)n * T + t) * H + h) * DK + col + c) = make_uint2(0u, 0u);
    return;
  }
  if (Tn == 0) return;  // nothing accepted: the pool keeps its state

  // element offset of this thread's first state element in the pool (fp32 or
  // bf16 elements)
  const int64_t se = ((int64_t)idx * H + h) * DK * DK + col;
  float S[4][CPT];
  if (a.state_bf16) {
    const uint16_t* sp = reinterpret_cast<const uint16_t*>(a.pool) + se;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < CPT; c += 4) {
        const float4 f = bf16x4_to_f32(*reinterpret_cast<const uint2*>(sp + (rr + 32 * i) * DK + c));
        S[i][c] = f.x; S[i][c + 1] = f.y; S[i][c + 2] = f.z; S[i][c + 3] = f.w;
      }
  } else {
    const float* sp = a.pool + se;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < CPT; c += 4) {
        const float4 f = *reinterpret_cast<const float4*>(sp + (rr + 32 * i) * DK + c);
        S[i][c] = f.x; S[i][c + 1] = f.y; S[i][c + 2] = f.z; S[i][c + 3] = f.w;
      }
  }
  // the state's four rows to `dst` at element offset e0: fp32, or bf16
  // rounded to nearest even
  auto store_state = [&](float* dst, int64_t e0) {
    if (a.state_bf16) {
      uint16_t* p16 = reinterpret_cast<uint16_t*>(dst) + e0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < CPT; c += 4)
          *reinterpret_cast<uint2*>(p16 + (rr + 32 * i) * DK + c) =
              make_uint2(pack_bf16x2(S[i][c], S[i][c + 1]), pack_bf16x2(S[i][c + 2], S[i][c + 3]));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < CPT; c += 4)
          *reinterpret_cast<float4*>(dst + e0 + (rr + 32 * i) * DK + c) =
              make_float4(S[i][c], S[i][c + 1], S[i][c + 2], S[i][c + 3]);
    }
  };

  // The per-token vectors are fetched one token ahead into registers (threads
  // 0..127: k, q, g of row tid; the next WC: v of this workgroup's columns;
  // then one for beta), so their latency overlaps the previous token's
  // arithmetic.
  uint16_t nk = 0, nq = 0;
  float nx = 0.f;
  auto fetch = [&](int t) {
    const int64_t tok = (int64_t)n * T + t;
    const int64_t vbase = (tok * H + h) * DK;
    if (tid < DK) {
      nk = a.k[vbase + tid];
      nq = a.q[vbase + tid];
      nx = a.g[vbase + tid];
    } else if (tid < DK + WC) {
      nk = a.v[vbase + part * WC + tid - DK];
    } else if (tid == DK + WC) {
      nx = a.beta[tok * H + h];
    }
  };
  fetch(0);

  for (int t = 0; t < Tn; ++t) {
    const int64_t tok = (int64_t)n * T + t;
    const int64_t vbase = (tok * H + h) * DK;
    if (tid < DK) {
      sk[tid] = bf16_to_f32(nk);
      sq[tid] = bf16_to_f32(nq);
      sd[tid] = __expf(nx);
    } else if (tid < DK + WC) {
      sv[tid - DK] = bf16_to_f32(nk);
    } else if (tid == DK + WC) {
      sbeta = (a.prologue & 2) ? 1.f / (1.f + __expf(-nx)) : nx;  // beta given as a logit
    }
    lds_barrier();
    if (t + 1 < Tn) fetch(t + 1);
    // k . q, and with the prologue the norms of k and q: every wave sums the
    // 128 staged values itself (no further barrier)
    float kq = sk[lane] * sq[lane] + sk[lane + 64] * sq[lane + 64];
    float kk = 0.f, qq = 0.f;
    if (a.prologue & 1) {
      kk = sk[lane] * sk[lane] + sk[lane + 64] * sk[lane + 64];
      qq = sq[lane] * sq[lane] + sq[lane + 64] * sq[lane + 64];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      kq += __shfl_xor(kq, o, 64);
      if (a.prologue & 1) {
        kk += __shfl_xor(kk, o, 64);
        qq += __shfl_xor(qq, o, 64);
      }
    }
    float inv_k = 1.f, inv_q = 1.f;
    if (a.prologue & 1) {
      inv_k = kk > 0.f ? 1.f / __builtin_sqrtf(kk) : 0.f;
      inv_q = qq > 0.f ? 1.f / __builtin_sqrtf(qq) : 0.f;
    }
    // decay the rows, then partial S^T k and S^T q over this thread's rows
    float pk[CPT], pq[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) pk[j] = pq[j] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rr + 32 * i;
      const float d = sd[r], kr = sk[r] * inv_k, qr = sq[r] * inv_q;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        S[i][j] *= d;
        pk[j] += kr * S[i][j];
        pq[j] += qr * S[i][j];
      }
    }
    // sum over the 8 row positions of the wave (lanes cg, cg + 8, ..., cg + 56)
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
      for (int o = 8; o < 64; o <<= 1) {
        pk[j] += __shfl_xor(pk[j], o, 64);
        pq[j] += __shfl_xor(pq[j], o, 64);
      }
    if (lane < 8) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        red[0][w][CPT * cg + j] = pk[j];
        red[1][w][CPT * cg + j] = pq[j];
      }
    }
    lds_barrier();
    float u[CPT], o[CPT];
    const float beta = sbeta;
    kq *= inv_k * inv_q;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = CPT * cg + j;
      const float p = (red[0][0][c] + red[0][1][c]) + (red[0][2][c] + red[0][3][c]);
      const float sqc = (red[1][0][c] + red[1][1][c]) + (red[1][2][c] + red[1][3][c]);
      u[j] = beta * (sv[c] - p);
      o[j] = a.scale * (sqc + kq * u[j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float kr = sk[rr + 32 * i] * inv_k;
#pragma unroll
      for (int j = 0; j < CPT; ++j) S[i][j] += kr * u[j];
    }
    if (rr == 0 && a.out)
#pragma unroll
      for (int c = 0; c < CPT; c += 4)
        *reinterpret_cast<uint2*>(a.out + vbase + col + c) =
            make_uint2(pack_bf16x2(o[c], o[c + 1]), pack_bf16x2(o[c + 2], o[c + 3]));
    if (a.trace) store_state(a.trace, (tok * H + h) * DK * DK + col);
    lds_barrier();  // the staged vectors and partial sums are rewritten next token
  }

  if (a.writeback) store_state(a.pool, se);
}

// One workgroup per (request, head, quarter of the columns), in the decode
// kernel's block order with 4 parts per pair and its CPT = 4 thread layout:
// each thread copies rows rr + 32 i of its 4 columns.
__global__ __launch_bounds__(256) void kda_decode_commit_kernel(DecodeCommitArgs a) {
  const int tid = threadIdx.x, cg = tid & 7, rr = tid >> 3;
  const int64_t blk = blockIdx.x;
  const int quarter = (int)((blk >> 3) & 3);
  const int64_t pair = (blk >> 5) * 8 + (blk & 7);
  const int H = a.H;
  if (pair >= (int64_t)a.N * H) return;
  const int n = (int)(pair / H), h = (int)(pair - (int64_t)n * H);
  const int idx = a.state_indices[n], acc = a.accepted[n];
  if (idx < 0 || (int64_t)idx >= a.pool_size || acc < 1 || acc > a.T) return;
  const int col = quarter * QCOLS + 4 * cg;
  const int64_t se = (((int64_t)n * a.T + acc - 1) * H + h) * DK * DK + col;
  const int64_t de = ((int64_t)idx * H + h) * DK * DK + col;
  if (a.state_bf16) {
    const uint16_t* src = reinterpret_cast<const uint16_t*>(a.trace) + se;
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.pool) + de;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint2*>(dst + (rr + 32 * i) * DK) = *reinterpret_cast<const uint2*>(src + (rr + 32 * i) * DK);
  } else {
    const float* src = a.trace + se;
    float* dst = a.pool + de;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<float4*>(dst + (rr + 32 * i) * DK) = *reinterpret_cast<const float4*>(src + (rr + 32 * i) * DK);
  }
}

}  // namespace

// blocks for N x H pairs: whole groups of 8 pairs, `parts` workgroups each
static int64_t decode_blocks(int64_t pairs, int parts) { return (pairs + 7) / 8 * 8 * parts; }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.N * a.H;
  if (pairs == 0 || a.T == 0) return hipSuccess;
  if (a.state_bf16)
    hipLaunchKernelGGL(kda_decode_kernel<8>, dim3((unsigned)decode_blocks(pairs, 2)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(kda_decode_kernel<4>, dim3((unsigned)decode_blocks(pairs, 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_commit(const DecodeCommitArgs& a, hipStream_t stream) {
  const int64_t blocks = decode_blocks((int64_t)a.N * a.H, 4);
  if (blocks == 0 || a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(kda_decode_commit_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
