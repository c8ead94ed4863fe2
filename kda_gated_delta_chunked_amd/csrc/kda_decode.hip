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
// One workgroup of 256 threads owns one (sequence, head) and 32 of the 128
// state columns; columns are independent, so the four quarters of a state
// run in four workgroups.  Thread (rr = tid / 8, cg = tid % 8) holds rows
// rr + 32 i (i = 0..3) of columns 4 cg .. 4 cg + 3 as four float4 registers,
// read once from the pool, kept across the call's tokens and written back in
// place.  The path is bound by HBM: 64 KiB of state in and out per (sequence,
// head).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int DK = 128;
constexpr int QCOLS = 32;  // state columns per workgroup

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// two floats to two bf16 (round to nearest even), low half first
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 r = __builtin_convertvector((f2){x, y}, b2);
  return __builtin_bit_cast(uint32_t, r);
}

__global__ __launch_bounds__(256) void kda_decode_kernel(DecodeArgs a) {
  __shared__ float sk[DK], sq[DK], sd[DK];  // k, q and exp(g) of the token
  __shared__ float sv[QCOLS];               // v of the token, this workgroup's columns
  __shared__ float red[2][4][QCOLS];        // per-wave partial S^T k and S^T q
  __shared__ float sbeta;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cg = tid & 7, rr = tid >> 3;
  const int64_t blk = blockIdx.x;
  const int quarter = (int)(blk & 3);
  const int64_t pair = blk >> 2;
  const int H = a.H;
  const int n = (int)(pair / H), h = (int)(pair - (int64_t)n * H);
  const int col = quarter * QCOLS + 4 * cg;
  const int T = a.T;
  const int idx = a.state_indices[n];

  if (idx < 0 || (int64_t)idx >= a.pool_size) {
    // a request slot with no state: its outputs are zero, no state is touched
    if (rr == 0)
      for (int t = 0; t < T; ++t)
        *reinterpret_cast<uint2*>(a.out + (((int64_t)n * T + t) * H + h) * DK + col) = make_uint2(0u, 0u);
    return;
  }

  float* sp = a.pool + ((int64_t)idx * H + h) * DK * DK + col;
  float4 S[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) S[i] = *reinterpret_cast<const float4*>(sp + (rr + 32 * i) * DK);

  // The per-token vectors are fetched one token ahead into registers (threads
  // 0..127: k, q, g of row tid; 128..159: v of this workgroup's columns; 160:
  // beta), so their latency overlaps the previous token's arithmetic.
  uint16_t nk = 0, nq = 0;
  float nx = 0.f;
  auto fetch = [&](int t) {
    const int64_t tok = (int64_t)n * T + t;
    const int64_t vbase = (tok * H + h) * DK;
    if (tid < DK) {
      nk = a.k[vbase + tid];
      nq = a.q[vbase + tid];
      nx = a.g[vbase + tid];
    } else if (tid < DK + QCOLS) {
      nk = a.v[vbase + quarter * QCOLS + tid - DK];
    } else if (tid == DK + QCOLS) {
      nx = a.beta[tok * H + h];
    }
  };
  fetch(0);

  for (int t = 0; t < T; ++t) {
    const int64_t tok = (int64_t)n * T + t;
    const int64_t vbase = (tok * H + h) * DK;
    if (tid < DK) {
      sk[tid] = bf16_to_f32(nk);
      sq[tid] = bf16_to_f32(nq);
      sd[tid] = __expf(nx);
    } else if (tid < DK + QCOLS) {
      sv[tid - DK] = bf16_to_f32(nk);
    } else if (tid == DK + QCOLS) {
      sbeta = (a.prologue & 2) ? 1.f / (1.f + __expf(-nx)) : nx;  // beta given as a logit
    }
    lds_barrier();
    if (t + 1 < T) fetch(t + 1);
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
    float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rr + 32 * i;
      const float d = sd[r], kr = sk[r] * inv_k, qr = sq[r] * inv_q;
      S[i].x *= d;
      S[i].y *= d;
      S[i].z *= d;
      S[i].w *= d;
      pk[0] += kr * S[i].x;
      pk[1] += kr * S[i].y;
      pk[2] += kr * S[i].z;
      pk[3] += kr * S[i].w;
      pq[0] += qr * S[i].x;
      pq[1] += qr * S[i].y;
      pq[2] += qr * S[i].z;
      pq[3] += qr * S[i].w;
    }
    // sum over the 8 row positions of the wave (lanes cg, cg + 8, ..., cg + 56)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int o = 8; o < 64; o <<= 1) {
        pk[j] += __shfl_xor(pk[j], o, 64);
        pq[j] += __shfl_xor(pq[j], o, 64);
      }
    if (lane < 8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        red[0][w][4 * cg + j] = pk[j];
        red[1][w][4 * cg + j] = pq[j];
      }
    }
    lds_barrier();
    float u[4], o[4];
    const float beta = sbeta;
    kq *= inv_k * inv_q;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 4 * cg + j;
      const float p = (red[0][0][c] + red[0][1][c]) + (red[0][2][c] + red[0][3][c]);
      const float sqc = (red[1][0][c] + red[1][1][c]) + (red[1][2][c] + red[1][3][c]);
      u[j] = beta * (sv[c] - p);
      o[j] = a.scale * (sqc + kq * u[j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float kr = sk[rr + 32 * i] * inv_k;
      S[i].x += kr * u[0];
      S[i].y += kr * u[1];
      S[i].z += kr * u[2];
      S[i].w += kr * u[3];
    }
    if (rr == 0)
      *reinterpret_cast<uint2*>(a.out + vbase + col) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    lds_barrier();  // the staged vectors and partial sums are rewritten next token
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<float4*>(sp + (rr + 32 * i) * DK) = S[i];
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.N * a.H * 4;
  if (blocks == 0 || a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(kda_decode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
