// kda_decomp.hip -- two-launch chunked KDA prefill for gfx950 (MI355X).
//
// The chunk-parallel / recurrent split of the prefill: a prepare launch that
// runs over every (segment, head) at once, and a recurrence launch that carries
// the state across a sequence's segments (FlashInfer PR #4633, Description:
// the "decomp" variant, two launches sharing one scratch arena).
//
// Segments are the 64-token chunks of each sequence, aligned to its start,
// with the chunk that holds a checkpoint offset cut in two at that offset.  A
// segment of c <= 64 rows sits in the last c rows of a 64-row tile; the rows
// before it are zero and contribute nothing.  With G_r = g_0 + ... + g_r per
// key channel (reset at every segment):
//   A[r,s] = sum_d k_rd k_sd exp(G_rd - G_sd)   s < r      (gated K K^T)
//   M[r,s] = sum_d q_rd k_sd exp(G_rd - G_sd)   s <= r     (gated Q K^T)
//   T = (I + diag(beta) A)^-1,  N = T - I
//   K~ = K exp(G),  Q~ = Q exp(G),  K^ = K exp(G_end - G),  Gam = exp(G_end)
// are state independent (prepare).  The recurrence then does, per segment,
//   X = V - K~ S,  Y = diag(beta) X,  U = Y + N Y
//   O = scale (Q~ S + M U),   S <- diag(Gam) S + K^^T U
// (the prepare folds the scale into Q~ and M)
// which regroups the token recurrence (decay, delta-rule correction, read-out
// of the updated state) by segments.
//
// Prepare stores its results in the caller's workspace already in the lane
// order of the v_mfma_f32_16x16x32_bf16 operands the recurrence feeds, so the
// recurrence copies a slot straight into LDS (global_load_lds) and reads each
// operand fragment with one 16-byte LDS load per lane.
//
// Fragment conventions (lane l = 16 g + q, g = 0..3, q = 0..15).  Within a
// 32-wide contraction block b, element e = 0..7 of lane l stands for index
//   kidx(b, g, e) = 32 b + 16 (e / 4) + 4 g + (e % 4).
// An A operand of row tile t holds X[16 t + q][kidx]; a B operand of column
// tile t holds Y[kidx][16 t + q]; an accumulator holds C[4 g + i][q].  With
// this order, the accumulators of row tiles 2b and 2b+1 of a matrix Z, taken
// side by side, are exactly the B operand of Z for block b (and the A operand
// of Z^T), so state and U feed the next product without any data movement.
// Token contractions (U, M, N, the token axis of K^^T) use kidx as it is.  The
// state is held with its rows permuted: row R of the accumulators holds key
// channel state_row_channel(R), chosen so that in the key-channel operands
// (K~, Q~) element e of lane l in block b is channel 32 b + 8 g + e -- eight
// consecutive channels, which the prepare reads with one 16-byte load of q
// and k per lane (8-byte pieces, two per lane, were about a fifth slower to
// fetch).
//
// Exponent range (prepare): rows form 16-row blocks i with local cumulative
// sums Gl_r = G_r - G_{16i-1} <= 0 and block sums bt_i.  With g >= -5 (the gate
// lower bound of lmdeploy PR #5050, Modification) every factor used below lies
// in [exp(-80), exp(80)] or is a product of factors <= 1:
//   block (i,i):   exp(G_r - G_s) = exp(Gl_r) * exp(-Gl_s)
//   block (i,j<i): exp(G_r - G_s) = exp(Gl_r) * exp(bt_j - Gl_s) * prod_{j<m<i} exp(bt_m)
//
// Precision.  The matrix cores take fp16 operands with fp32 accumulation
// (v_mfma_f32_16x16x32_f16) wherever the operand's range allows it: K~, Q~
// and K^ (|k|, |q| <= 1 times factors <= 1), N (|N| <= 1: an entry of T is
// the response of one write to an earlier one through contracting steps), the
// gated products left of the diagonal block (both factors <= 1), and the
// state, V, Y and U after multiplying them by a power of two 2^s kept per
// compute wave.  The diagonal 16 x 16 blocks of A and M, whose right factor
// reaches exp(80), take bf16 hi + lo operands; U is fed as fp16 hi + lo into
// the state update; the identity part of T stays fp32 (U = Y + N Y); the
// triangular solve is fp32.  fp16 keeps 11 significant bits against bf16's 8:
// at slow decay (g near 0) the corrections K~ S and N Y are as large as the
// writes themselves and their rounding no longer decays away, which with
// bf16 operands put the state's error near 1e-3.
//
// The power of two: the recurrence multiplies its fp32 state by 2^s and feeds
// 2^s V to the products, so every product of the segment is 2^s times the
// unscaled one (exact).  s is reset, when the larger of max|2^s S| and
// max|2^s V| leaves [4, 64], so that it lands in [16, 32): then |2^s X| <=
// sqrt(128) 64, |2^s Y| < 2^9.6 and |2^s U| < 64 * 2^9.6 (rows of T sum at most
// 64 terms of magnitude <= 1) stay below the fp16 limit of 65504, and the
// values that matter stay far above its subnormal range.  The read-out takes
// scale * 2^-s, and exported states 2^-s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_ckpt.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int CH = 64;    // chunk rows
constexpr int DK = 128;   // key channels = value channels

// Slot layout (bytes).  Fragments are 64 lanes x 16 bytes = 1 KiB, fp16.
constexpr int SL_KT = 0;        // K~  : row tile t (4) x key block b (4), A of K~ S
constexpr int SL_QT = 16384;    // Q~  : token tile t (4) x key block b (4), B of S^T Q~^T
constexpr int SL_KH = 32768;    // K^  : key tile m (8) x token block b (2), A of K^^T U
constexpr int SL_M = 49152;     // M  : token tile t x token block b <= t/2 (6 fragments, 5 KiB)
constexpr int SL_N = 54272;     // N  : same tiling as M
constexpr int SL_GAM = 59392;   // exp(G_end), 128 fp32
constexpr int SL_BETA = 59904;  // beta per tile row, 64 fp32 (0 on empty rows)
// segment header: int32 off (first tile row of the segment), int32 spare,
// int64 tok0 (token of tile row 0), uint64 export mask (bit c: checkpoint c
// of the sequence is the state after this segment)
constexpr int SL_HDR = 60160;
constexpr int SLOT_UNITS = 59;  // 1 KiB copy units per slot
static_assert(SLOT_UNITS * 1024 == kDecompSlotBytes, "slot size");
static_assert(SL_BETA + 256 <= SL_HDR && SL_HDR + 24 <= kDecompSlotBytes, "slot layout");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// two floats -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack2h(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}
__device__ __forceinline__ float h_lo(uint32_t p) { return (float)__builtin_bit_cast(f16x2, p)[0]; }
__device__ __forceinline__ float h_hi(uint32_t p) { return (float)__builtin_bit_cast(f16x2, p)[1]; }
// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ float lo_of(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_of(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// eight floats -> bf16x8 (hi), and optionally the rounding remainder (lo)
__device__ __forceinline__ bf16x8 to_bf16x8(const float (&x)[8]) {
  uint4 u;
  u.x = pack2(x[0], x[1]);
  u.y = pack2(x[2], x[3]);
  u.z = pack2(x[4], x[5]);
  u.w = pack2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = pack2(x[2 * e], x[2 * e + 1]);
    l[e] = pack2(x[2 * e] - lo_of(h[e]), x[2 * e + 1] - hi_of(h[e]));
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}
// two accumulators (row tiles 2b, 2b+1) -> the B operand of block b
__device__ __forceinline__ bf16x8 acc_pair(const f32x4& a, const f32x4& b) {
  uint4 u;
  u.x = pack2(a[0], a[1]);
  u.y = pack2(a[2], a[3]);
  u.z = pack2(b[0], b[1]);
  u.w = pack2(b[2], b[3]);
  return __builtin_bit_cast(bf16x8, u);
}
// the fp16 counterparts: eight floats -> f16x8, hi + lo pairs, accumulator pairs
__device__ __forceinline__ f16x8 to_f16x8(const float (&x)[8]) {
  uint4 u;
  u.x = pack2h(x[0], x[1]);
  u.y = pack2h(x[2], x[3]);
  u.z = pack2h(x[4], x[5]);
  u.w = pack2h(x[6], x[7]);
  return __builtin_bit_cast(f16x8, u);
}
__device__ __forceinline__ f16x8 acc_pair_h(const f32x4& a, const f32x4& b) {
  uint4 u;
  u.x = pack2h(a[0], a[1]);
  u.y = pack2h(a[2], a[3]);
  u.z = pack2h(b[0], b[1]);
  u.w = pack2h(b[2], b[3]);
  return __builtin_bit_cast(f16x8, u);
}
__device__ __forceinline__ void acc_pair_split_h(const f32x4& a, const f32x4& b, f16x8& hi, f16x8& lo) {
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = pack2h(x[2 * e], x[2 * e + 1]);
    l[e] = pack2h(x[2 * e] - h_lo(h[e]), x[2 * e + 1] - h_hi(h[e]));
  }
  hi = __builtin_bit_cast(f16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(f16x8, make_uint4(l[0], l[1], l[2], l[3]));
}
// Workspace stores of the prepare.  With NT they are non-temporal
// (streamed): for a workspace too large to stay in the Infinity Cache until
// the recurrence reads it, that keeps the write stream from displacing what
// the caches still serve; a workspace that does stay there is written
// normally, so that the recurrence finds it in the cache.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <bool NT, class T>
__device__ __forceinline__ void ws_put(unsigned char* p, const T& v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
  else *reinterpret_cast<T*>(p) = v;
}
template <bool NT>
__device__ __forceinline__ void ws_store(unsigned char* p, const uint4& v) {
  ws_put<NT>(p, (u32x4){v.x, v.y, v.z, v.w});
}
template <bool NT>
__device__ __forceinline__ void ws_store(unsigned char* p, const uint2& v) {
  ws_put<NT>(p, (u32x2){v.x, v.y});
}
template <bool NT>
__device__ __forceinline__ void ws_store(unsigned char* p, const bf16x8& v) {
  ws_put<NT>(p, v);
}
template <bool NT>
__device__ __forceinline__ void ws_store(unsigned char* p, float v) {
  ws_put<NT>(p, v);
}

// key channel of accumulator row R of the state: R = 32 b + 16 h + 4 g + e
// holds channel 32 b + 8 g + 4 h + e, so that kidx(b, g, e) maps to channel
// 32 b + 8 g + e
__host__ __device__ constexpr int state_row_channel(int R) {
  return (R & ~31) + 8 * ((R >> 2) & 3) + 4 * ((R >> 4) & 1) + (R & 3);
}
// M / N fragment index of (token tile t, token block b <= t / 2)
__host__ __device__ constexpr int tri_frag(int t, int b) { return t < 2 ? t : 2 * t - 2 + b; }
// Fragments (0, 0) and (2, 1) lie on the diagonal with an all-zero upper half
// (token block 2b + 1 > t): only their lower 8 bytes per lane are stored.
__host__ __device__ constexpr bool tri_half(int f) { return f == 0 || f == 3; }
// byte offset of fragment f inside the M or N region (half fragments take 512 bytes)
__host__ __device__ constexpr int tri_off(int f) {
  return f == 0 ? 0 : f == 1 ? 512 : f == 2 ? 1536 : f == 3 ? 2560 : f == 4 ? 3072 : 4096;
}

// ---------------------------------------------------------------------------
// Sequence and segment geometry (shared by both launches).

struct SeqInfo {
  int64_t bos;   // first token of the sequence
  int len;       // tokens
  int nseg;      // segments: the 64-token chunks, those holding a cut point cut in two
  CkptList ck;   // checkpoint offsets (C = 0 when none)
};

__device__ __forceinline__ SeqInfo seq_info(const DecompArgs& a, int n) {
  SeqInfo s;
  int64_t b, e;
  if (a.cu_seqlens) {
    b = cu_at(a.cu_seqlens, a.cu64, n);
    e = cu_at(a.cu_seqlens, a.cu64, n + 1);
  } else {
    b = (int64_t)n * a.T_fixed;
    e = b + a.T_fixed;
  }
  // keep every access inside [0, T_total) even for offsets that break the contract
  int64_t len;
  clamp_seq_range(b, e, a.T_total, &s.bos, &len);
  s.len = (int)len;
  s.ck = load_ckpt_list(a.ckpt_off, a.ckpt_per_seq, n, s.len);
  s.nseg = (s.len + CH - 1) / CH + count_cuts(s.ck);
  return s;
}

// token range [lo, hi) of segment j, relative to the sequence start
__device__ __forceinline__ void seg_range(const SeqInfo& s, int j, int& lo, int& hi) {
  lo = j == 0 ? 0 : interior_boundary(s.ck, j - 1);
  hi = j >= s.nseg - 1 ? s.len : interior_boundary(s.ck, j);
}

// ---------------------------------------------------------------------------
// Launch 0 (packed layout only): first slot of every sequence.  Sequence n
// owns ceil(L_n / 64) slots, plus C when C checkpoint offsets per sequence are
// requested (each may cut a chunk in two).  base[N] is the total.
//
// It also writes the order in which the recurrence takes the sequences: the
// caller's seq_order when given and a permutation of 0..N-1 (checked here,
// for N <= kSeqOrderMax), else longest first (ties by index), so that when
// there are more workgroups than the device holds at once, the long chains
// start first and short ones fill the tail.  Up to kOrderMax sequences are
// ranked; beyond that, and for a seq_order that is no permutation, the order
// is the identity.

constexpr int kOrderMax = 1024;
constexpr int kSeqOrderMax = 65536;

__global__ __launch_bounds__(1024) void kda_plan_kernel(DecompArgs a) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t nslots[kOrderMax];
  __shared__ uint32_t seen[kSeqOrderMax / 32];
  __shared__ int order_bad;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int extra = a.ckpt_off ? a.ckpt_per_seq : 0;
  int64_t carry = 0;
  for (int n0 = 0; n0 < a.N; n0 += 1024) {
    const int n = n0 + t;
    int cnt = 0;
    if (n < a.N) {
      int64_t b, len;
      clamp_seq_range(cu_at(a.cu_seqlens, a.cu64, n), cu_at(a.cu_seqlens, a.cu64, n + 1), a.T_total,
                      &b, &len);
      cnt = (int)((len + CH - 1) / CH) + extra;
    }
    int x = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      woff += i < w ? wsum[i] : 0;
      tot += wsum[i];
    }
    if (n < a.N) a.seg_base[n] = (int32_t)(carry + woff + x - cnt);
    if (a.N <= kOrderMax) nslots[t] = cnt;
    __syncthreads();
    carry += tot;
  }
  if (t == 0) a.seg_base[a.N] = (int32_t)carry;
  if (!a.order) return;
  if (a.seq_order && a.N <= kSeqOrderMax) {
    // the caller's order, if it names every sequence once: N entries in
    // [0, N), all distinct
    for (int i = t; i < (a.N + 31) / 32; i += 1024) seen[i] = 0u;
    if (t == 0) order_bad = 0;
    __syncthreads();
    for (int n = t; n < a.N; n += 1024) {
      const int x = a.seq_order[n];
      if (x < 0 || x >= a.N) {
        order_bad = 1;
      } else {
        const uint32_t bit = 1u << (x & 31);
        if (atomicOr(&seen[x >> 5], bit) & bit) order_bad = 1;
      }
    }
    __syncthreads();
    const bool ok = order_bad == 0;
    for (int n = t; n < a.N; n += 1024) a.order[n] = ok ? a.seq_order[n] : n;
    return;
  }
  if (a.N > kOrderMax) {
    for (int n = t; n < a.N; n += 1024) a.order[n] = n;
    return;
  }
  if (t < a.N) {
    // rank = sequences that come before this one
    const int mine = nslots[t];
    int rank = 0;
    for (int m = 0; m < a.N; ++m) {
      const int o = nslots[m];
      rank += (o > mine || (o == mine && m < t)) ? 1 : 0;
    }
    a.order[rank] = t;
  }
}

// ---------------------------------------------------------------------------
// Launch 1: prepare.  One workgroup of 4 waves per (slot, head).  Wave i owns
// the 16-row block i of the tile and works in the lane order of the matrix
// fragments throughout: lane l = 16 g + q holds row 16 i + q and, for key
// block b, the 8 channels 32 b + 8 g + (0..7).

constexpr int P_LP = CH + 4;    // fp32 pitch of L and T
// per-channel factor rows
constexpr int F_BT = 0;         // bt_0..3 (block sums of g)
constexpr int F_P = 4;          // P_1..3 = exp(bt_0 + ... + bt_{i-1})  (row F_P + i - 1)
constexpr int F_R = 7;          // R_0..2 = exp(bt_{i+1} + ... + bt_3)  (row F_R + i)
constexpr int F_IBD = 10;       // exp(-bt_i)
constexpr int F_ROWS = 14;
// the off-diagonal blocks' factors W, as fp16 rows (sW): exp(bt_1) for
// block (2, 0), exp(bt_2) for (3, 1), exp(bt_1 + bt_2) for (3, 0)
constexpr int W_ROWS = 3;
// k exp(bt_j - Gl_s) of row blocks 0..2 (fp32 [block][row][channel]); after
// the gated products the same space holds T (pitch P_LP)
constexpr int P_E_FLOATS = CH * P_LP + 4 * 512;
// during steps 2-3 the same space holds k exp(bt_j - Gl_s) as bf16 (12 KiB)
// and, after it, the K^^T half fragments that waves hand to their partner
// (4 waves x 4 fragments x 512 bytes)
constexpr int P_EP = DK + 8;    // bf16 pitch of those rows (16-byte shift per row: fewer bank conflicts)
constexpr int P_X_BYTES = 3 * 16 * P_EP * 2;
static_assert(P_E_FLOATS * 4 >= P_X_BYTES + 4 * 4 * 512, "prepare LDS layout");

// the 8 channels of key block b of this lane: 8 consecutive at p + off
__device__ __forceinline__ void load8_f32(const float* p, float (&x)[8], int off) {
  const float4 a = *reinterpret_cast<const float4*>(p + off);
  const float4 b = *reinterpret_cast<const float4*>(p + off + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void store8_f32(float* p, const float (&x)[8], int off) {
  *reinterpret_cast<float4*>(p + off) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + off + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void unpack8(const uint2 (&u)[2], float (&x)[8]) {
  x[0] = lo_of(u[0].x); x[1] = hi_of(u[0].x); x[2] = lo_of(u[0].y); x[3] = hi_of(u[0].y);
  x[4] = lo_of(u[1].x); x[5] = hi_of(u[1].x); x[6] = lo_of(u[1].y); x[7] = hi_of(u[1].y);
}
// value of lane q - n of this 16-lane row (0 for q < n)
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, true));
}
// largest value over the wave of non-negative x, the same in every lane: the
// 16-lane rows by DPP shifts (lane 15 of a row ends with the row's maximum),
// then the four row results through scalar registers
__device__ __forceinline__ float wave_max_nonneg(float x) {
  x = fmaxf(x, row_shr<1>(x));
  x = fmaxf(x, row_shr<2>(x));
  x = fmaxf(x, row_shr<4>(x));
  x = fmaxf(x, row_shr<8>(x));
  const int xi = __float_as_int(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(xi, 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(xi, 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(xi, 47));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(xi, 63));
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(fmaxf(fmaxf(r0, r1), fmaxf(r2, r3)))));
}

// 2^e for |e| <= 126, built from its exponent bits
__device__ __forceinline__ float pow2f(int e) { return __int_as_float((e + 127) << 23); }

// Operand scale exponent after seeing `big`, the largest of |2^s S| and
// |2^s V| over the wave (the same in every lane): s stays while big lies in
// [4, 64] or is 0 (or not finite); otherwise the new s puts big in [16, 32),
// limited to |s| <= 120.
__device__ __forceinline__ int rescale_exponent(float big, int s) {
  const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane(__float_as_int(big));
  if (b == 0u || b >= 0x7f800000u || (b >= 0x40800000u && b <= 0x42800000u)) return s;
  const int e = (int)(b >> 23) - 127;   // big in [2^e, 2^(e + 1)) (e = -127: subnormal)
  int ns = s + 4 - e;
  ns = ns < -120 ? -120 : (ns > 120 ? 120 : ns);
  return ns;
}

template <bool NT>
__global__ __launch_bounds__(256, 3) void kda_prepare_kernel(DecompArgs a) {
  __shared__ __attribute__((aligned(16))) float sF[F_ROWS * DK];
  __shared__ __attribute__((aligned(16))) _Float16 sW[W_ROWS * DK];
  __shared__ __attribute__((aligned(16))) float sE[P_E_FLOATS];
  __shared__ __attribute__((aligned(16))) float sL[CH * P_LP];        // beta_r A[r,s]
  __shared__ __attribute__((aligned(16))) float sB[CH];

  const int H = a.H;
  const int64_t bid = blockIdx.x;
  int64_t s;
  int h;
  if (a.prep_xcd) {
    const int64_t r = bid >> 3;
    s = (r / H) * 8 + (bid & 7);
    h = (int)(r - (r / H) * H);
  } else {
    s = bid / H;
    h = (int)(bid - s * H);
  }
  if (s >= a.slot_bound) return;
  if (!a.cu_seqlens && s >= (int64_t)a.N * a.slots_per_seq) return;

  // slot -> (sequence, segment)
  int n, j;
  if (a.cu_seqlens) {
    if (s >= a.seg_base[a.N]) return;
    int lo = 0, hi = a.N;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.seg_base[mid] <= s) lo = mid; else hi = mid;
    }
    n = lo;
    j = (int)(s - a.seg_base[n]);
  } else {
    n = (int)(s / a.slots_per_seq);
    j = (int)(s - (int64_t)n * a.slots_per_seq);
  }
  const SeqInfo si = seq_info(a, n);
  if (j >= si.nseg) return;
  int lo_t, hi_t;
  seg_range(si, j, lo_t, hi_t);
  const int off = CH - (hi_t - lo_t);
  const int64_t tok0 = si.bos + lo_t - off;        // token of tile row 0
  unsigned char* slot = a.slots + (size_t)(s * H + h) * kDecompSlotBytes;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, q = lane & 15;
  const int i = w;
  const int r = 16 * i + q;

  // (0) Loads.  All are unconditional: a row before the segment (r < off)
  // reads row `off` instead, which is inside it, and is zeroed where used (a
  // load under a per-lane condition makes the compiler wait before the join).
  const bool rv = r >= off;
  const size_t erow = ((size_t)(tok0 + max(r, off)) * H + h) * DK;
  // g and beta first: the gate cumsum and the block factors need only them,
  // and run while k and q are still arriving (loads complete in order)
  uint2 kA[4][2], qA[4][2];
  float4 gA[4][2];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int ch = 32 * b + 8 * g4;
    gA[b][0] = *reinterpret_cast<const float4*>(a.g + erow + ch);
    gA[b][1] = *reinterpret_cast<const float4*>(a.g + erow + ch + 4);
  }
  const float beta_ld = a.beta[(size_t)(tok0 + max(tid & (CH - 1), off)) * H + h];
  __builtin_amdgcn_sched_barrier(0);  // keep the k and q loads behind these
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int ch = 32 * b + 8 * g4;
    const uint4 kv = *reinterpret_cast<const uint4*>(a.k + erow + ch);
    const uint4 qv = *reinterpret_cast<const uint4*>(a.q + erow + ch);
    kA[b][0] = make_uint2(kv.x, kv.y);
    kA[b][1] = make_uint2(kv.z, kv.w);
    qA[b][0] = make_uint2(qv.x, qv.y);
    qA[b][1] = make_uint2(qv.z, qv.w);
  }

  // Gl: cumulative sum of g over the rows of the block, for this lane's 32
  // channels -- an inclusive scan over the 16 lanes of a DPP row (lane q = row q)
  float gl[4][8];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float4 u = gA[b][0], v = gA[b][1];
    const float x[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float y = rv ? x[e] : 0.f;
      y += row_shr<1>(y);
      y += row_shr<2>(y);
      y += row_shr<4>(y);
      y += row_shr<8>(y);
      gl[b][e] = y;
    }
  }
  // block sums (row 15 of the block) and beta to LDS
  if (q == 15) {
#pragma unroll
    for (int b = 0; b < 4; ++b) store8_f32(sF, gl[b], (F_BT + i) * DK + 32 * b + 8 * g4);
  }
  // input prologue: beta given as a logit; q and k divided by their L2 norms
  // (the row's 128 channels sit in lanes q, q + 16, q + 32, q + 48)
  if (tid < CH) sB[tid] = tid >= off ? ((a.prologue & 2) ? 1.f / (1.f + __expf(-beta_ld)) : beta_ld) : 0.f;
  float inv_k = 1.f, inv_q = 1.f;
  if (a.prologue & 1) {
    float ssk = 0.f, ssq = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      // opaque copies: this unpacking stays inside the branch rather than
      // being shared with step (2)'s, which would make every wave wait for
      // its k and q before the first barrier, prologue or not
      uint2 kk[2] = {kA[b][0], kA[b][1]}, qq[2] = {qA[b][0], qA[b][1]};
      asm volatile("" : "+v"(kk[0]), "+v"(kk[1]), "+v"(qq[0]), "+v"(qq[1]));
      float kf[8], qf[8];
      unpack8(kk, kf);
      unpack8(qq, qf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ssk += kf[e] * kf[e];
        ssq += qf[e] * qf[e];
      }
    }
    ssk += __shfl_xor(ssk, 16, 64);
    ssk += __shfl_xor(ssk, 32, 64);
    ssq += __shfl_xor(ssq, 16, 64);
    ssq += __shfl_xor(ssq, 32, 64);
    inv_k = ssk > 0.f ? 1.f / __builtin_sqrtf(ssk) : 0.f;
    inv_q = ssq > 0.f ? 1.f / __builtin_sqrtf(ssq) : 0.f;
  }
  // per-row factors of k and q: the prologue's norms, and 0 on rows before
  // the segment (one factor per row instead of a select per channel); the
  // read-out scale is applied by the recurrence
  const float kmul = rv ? inv_k : 0.f, qmul = rv ? inv_q : 0.f;
  lds_barrier();

  // (1) per-channel block factors; Gam and beta go straight to the slot
  if (tid < DK) {
    const int d = tid;
    const float b0 = sF[F_BT * DK + d], b1 = sF[(F_BT + 1) * DK + d];
    const float b2 = sF[(F_BT + 2) * DK + d], b3 = sF[(F_BT + 3) * DK + d];
    sF[(F_P + 0) * DK + d] = __expf(b0);
    sF[(F_P + 1) * DK + d] = __expf(b0 + b1);
    sF[(F_P + 2) * DK + d] = __expf(b0 + b1 + b2);
    sF[(F_R + 0) * DK + d] = __expf(b1 + b2 + b3);
    sF[(F_R + 1) * DK + d] = __expf(b2 + b3);
    sF[(F_R + 2) * DK + d] = __expf(b3);
    sF[(F_IBD + 0) * DK + d] = __expf(-b0);
    sF[(F_IBD + 1) * DK + d] = __expf(-b1);
    sF[(F_IBD + 2) * DK + d] = __expf(-b2);
    sF[(F_IBD + 3) * DK + d] = __expf(-b3);
    sW[0 * DK + d] = (_Float16)__expf(b1);
    sW[1 * DK + d] = (_Float16)__expf(b2);
    sW[2 * DK + d] = (_Float16)__expf(b1 + b2);
    // Gam in the state's row order
    const int sd = state_row_channel(d);
    ws_store<NT>(slot + SL_GAM + 4 * d,
        __expf(sF[F_BT * DK + sd] + sF[(F_BT + 1) * DK + sd] + sF[(F_BT + 2) * DK + sd] +
               sF[(F_BT + 3) * DK + sd]));
  } else if (tid < DK + CH) {
    ws_store<NT>(slot + SL_BETA + 4 * (tid - DK), sB[tid - DK]);
  } else if (tid == DK + CH) {
    // the recurrence's compute waves take the segment geometry and the
    // checkpoints it completes from here, with no scalar memory access
    unsigned long long mask = 0;
    for_each_honoured(si.ck, [&](int c, int p) {
      if (p > 0 && p == hi_t) mask |= 1ull << c;
    });
    *reinterpret_cast<int4*>(slot + SL_HDR) =
        make_int4(off, 0, (int)(uint32_t)(uint64_t)tok0, (int)(uint32_t)((uint64_t)tok0 >> 32));
    *reinterpret_cast<unsigned long long*>(slot + SL_HDR + 16) = mask;
  }
  lds_barrier();
  // nothing of step (2) (the unpacking of k and q) moves above the barrier:
  // there it would wait for k and q
  __builtin_amdgcn_sched_barrier(0);

  // (2) wave i: operands of row block i and the diagonal block (i, i).
  // Identity slices that transpose a K^ tile with one exact matrix product:
  // lane 16 g + n holds 1.0 (fp16) at element 4 h + n % 4 when n / 4 == g.
  f16x8 eye[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    uint32_t wv[4] = {0u, 0u, 0u, 0u};
    const int el = 4 * hh + (q & 3);
    const bool on = (q >> 2) == g4;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (on && el == e) wv[e >> 1] |= 0x3c00u << (16 * (e & 1));
    eye[hh] = __builtin_bit_cast(f16x8, make_uint4(wv[0], wv[1], wv[2], wv[3]));
  }
  const float beta_r = sB[r];
  // the diagonal block's products accumulate key block by key block, so its
  // bf16 hi / lo operands need not stay live; the fp16 row-block operands
  // (aK, aQ) serve the off-diagonal blocks in step (3)
  f16x8 aK[4], aQ[4];
  uint16_t* sEb = reinterpret_cast<uint16_t*>(sE);
  uint2* sX = reinterpret_cast<uint2*>(reinterpret_cast<unsigned char*>(sE) + P_X_BYTES);
  uint2 kh_keep[4];
  f32x4 adiag = {0.f, 0.f, 0.f, 0.f}, mdiag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int ch0 = 32 * b + 8 * g4;
    float kf[8], qf[8], bt[8], fac[8];
    unpack8(kA[b], kf);
    unpack8(qA[b], qf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] *= kmul;
      qf[e] *= qmul;
    }
    load8_f32(sF, bt, (F_BT + i) * DK + ch0);
    float Kf[8], Qf[8], kb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ef = __expf(gl[b][e]);             // exp(G_r - G_{16i-1}) <= 1
      kb[e] = kf[e] * __expf(bt[e] - gl[b][e]);      // k exp(G_{16i+15} - G_r), <= |k|
      Kf[e] = kf[e] * ef;
      Qf[e] = qf[e] * ef;
    }
    aK[b] = to_f16x8(Kf);
    aQ[b] = to_f16x8(Qf);
    // K~ and Q~ fragments (row tile i, key block b)
    float kt[8], qt[8];
    if (i > 0) {
      load8_f32(sF, fac, (F_P + i - 1) * DK + ch0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kt[e] = Kf[e] * fac[e];
        qt[e] = Qf[e] * fac[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kt[e] = Kf[e];
        qt[e] = Qf[e];
      }
    }
    ws_store<NT>(slot + SL_KT + ((i * 4 + b) * 64 + lane) * 16, __builtin_bit_cast(uint4, to_f16x8(kt)));
    ws_store<NT>(slot + SL_QT + ((i * 4 + b) * 64 + lane) * 16, __builtin_bit_cast(uint4, to_f16x8(qt)));
    // k exp(bt - Gl) of this block, as fp16, for the later waves' off-diagonal
    // products (those round it again after the factor W, when W is not 1)
    if (i < 3) *reinterpret_cast<f16x8*>(sEb + (i * 16 + q) * P_EP + ch0) = to_f16x8(kb);
    // diagonal block: right operand k exp(-Gl) = k exp(bt - Gl) exp(-bt) (up
    // to exp(80): bf16), all operands hi + lo
    load8_f32(sF, fac, (F_IBD + i) * DK + ch0);
    float kr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kr[e] = kb[e] * fac[e];
    bf16x8 bD, bDl, aKh, aKl, aQh, aQl;
    split8(kr, bD, bDl);
    split8(Kf, aKh, aKl);
    split8(Qf, aQh, aQl);
    adiag = mfma(bD, aKh, adiag);
    adiag = mfma(bDl, aKh, adiag);
    adiag = mfma(bD, aKl, adiag);
    mdiag = mfma(bD, aQh, mdiag);
    mdiag = mfma(bDl, aQh, mdiag);
    mdiag = mfma(bD, aQl, mdiag);
    // K^ = k exp(G_end - G_r) = k exp(bt_i - Gl) R_i; transposed into K^^T
    // fragments by products with the identity slices (exact: one nonzero
    // bf16 term per output), stored as the half of each fragment that token
    // tile i fills
    float kh[8];
    if (i < 3) {
      load8_f32(sF, fac, (F_R + i) * DK + ch0);
#pragma unroll
      for (int e = 0; e < 8; ++e) kh[e] = kb[e] * fac[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kh[e] = kb[e];
    }
    const f16x8 khi = to_f16x8(kh);
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int m = 2 * b + hh;
      const f32x4 th = mfma(khi, eye[hh], z4);
      // K^^T fragment (m, i / 2) takes 8 bytes per lane from token tile i and
      // 8 from its partner i ^ 1.  Wave i stores the whole fragments of key
      // tiles 4 (i & 1) .. + 3 after the next barrier: it keeps its halves of
      // those and hands the partner its halves of the others through LDS.
      const uint2 half = make_uint2(pack2h(th[0], th[1]), pack2h(th[2], th[3]));
      if ((m >> 2) == (i & 1)) kh_keep[m & 3] = half;
      else sX[(i * 4 + (m & 3)) * 64 + lane] = half;
    }
  }

  // diagonal block: A_ii^T and M_ii^T (hi + lo operands), lane holds row r, s = 16 i + 4 g4 + e
  f32x4 macc[4];
  {
    const f32x4 aacc = adiag;
    f32x4 m0 = mdiag;
    float4 lv;
    float* lp = &lv.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int sidx = 16 * i + 4 * g4 + e;
      lp[e] = sidx < r ? beta_r * aacc[e] : 0.f;
      m0[e] = sidx <= r ? m0[e] : 0.f;
    }
    *reinterpret_cast<float4*>(&sL[r * P_LP + 16 * i + 4 * g4]) = lv;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) macc[jj] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (jj == i) macc[jj] = m0;
  }
  lds_barrier();
  // whole K^^T fragments (m, i / 2) for m = 4 (i & 1) .. + 3: the even token
  // tile's 8 bytes first
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const int m = 4 * (i & 1) + s4;
    const uint2 other = sX[((i ^ 1) * 4 + s4) * 64 + lane];
    const uint2 lo = (i & 1) ? other : kh_keep[s4], hi = (i & 1) ? kh_keep[s4] : other;
    ws_store<NT>(slot + SL_KH + ((m * 2 + (i >> 1)) * 64 + lane) * 16, make_uint4(lo.x, lo.y, hi.x, hi.y));
  }

  // (3) off-diagonal blocks (i, jb < i): right operand k exp(bt_jb - Gl_s) W_{i,jb}
  // from LDS, W = prod_{jb<m<i} exp(bt_m)
#pragma unroll
  for (int jb = 0; jb < 3; ++jb) {
    if (jb >= i) continue;
    f32x4 aacc = {0.f, 0.f, 0.f, 0.f};
    f32x4 m1 = {0.f, 0.f, 0.f, 0.f};
    // W's fp16 row (none for the block next to the diagonal); the scaled
    // operand is rounded once more, by the packed fp16 products
    const int wsel = (jb == i - 1) ? -1 : (i == 2 ? 0 : (jb == 1 ? 1 : 2));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int ch0 = 32 * b + 8 * g4;
      f16x8 bb = *reinterpret_cast<const f16x8*>(sEb + (jb * 16 + q) * P_EP + ch0);
      if (wsel >= 0) bb = bb * *reinterpret_cast<const f16x8*>(&sW[wsel * DK + ch0]);
      aacc = mfma(bb, aK[b], aacc);
      m1 = mfma(bb, aQ[b], m1);
    }
    *reinterpret_cast<float4*>(&sL[r * P_LP + 16 * jb + 4 * g4]) =
        make_float4(beta_r * aacc[0], beta_r * aacc[1], beta_r * aacc[2], beta_r * aacc[3]);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (jj == jb) macc[jj] = m1;
  }
  // M fragments of token tile i (B operand of O^T += U^T M^T)
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    if (2 * tb > i) continue;
    const int f = tri_frag(i, tb);
    const uint4 mv = __builtin_bit_cast(uint4, acc_pair_h(macc[2 * tb], macc[2 * tb + 1]));
    if (tri_half(f))
      ws_store<NT>(slot + SL_M + tri_off(f) + lane * 8, make_uint2(mv.x, mv.y));
    else
      ws_store<NT>(slot + SL_M + tri_off(f) + lane * 16, mv);
  }
  // (4) T_bb = (I + L_bb)^-1 by forward substitution, lane = (block, column).
  // Wave 0, which has no block in step (3), solves them while the other waves
  // run it: the solve reads only the diagonal blocks of L, which step (3)
  // does not write.  The result waits in registers until the barrier, since
  // T's space still holds the operands step (3) reads.
  float* sT = sE;
  float tdg[16];
  if (w == 0) {
    const int bb = lane >> 4, col = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float acc = rr == col ? 1.f : 0.f;
      const float* lrow = &sL[(16 * bb + rr) * P_LP + 16 * bb];
#pragma unroll
      for (int ss = 0; ss < rr; ++ss) acc -= lrow[ss] * tdg[ss];
      tdg[rr] = acc;
    }
  }
  lds_barrier();
  if (w == 0) {
    const int bb = lane >> 4, col = lane & 15;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sT[(16 * bb + rr) * P_LP + 16 * bb + col] = tdg[rr];
  }
  lds_barrier();

  // (5) off-diagonal blocks of T in two levels.  First the 32 x 32 halves:
  // T_10 = -T_11 L_10 T_00 and T_32 = -T_33 L_32 T_22.  Then the lower-left
  // quarter of the block inverse, -T_hh L_hl T_ll with hh = rows 32..63 and
  // ll = columns 0..31: wave w writes block (2 + w / 2, w % 2) as
  //   T_ij = -sum_{p=2}^{i} T_ip Z_pj,   Z_pj = sum_{m=j}^{1} L_pm T_mj.
  // Each 16 x 16 x 16 block product is four fp32 matrix-core steps
  // (v_mfma_f32_16x16x4_f32, fp32 products and sums).  Step e takes the
  // contraction index 4 g + e from lane group g, which is the row an fp32
  // accumulator holds in its element e (lane 16 g + q: rows 4 g .. 4 g + 3 of
  // column q): a product's accumulator is then the right operand of the next
  // as it stands, and Z never goes through LDS.
  auto mf4 = [](float x, float y, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, c, 0, 0, 0); };
  // acc += A[block ab, kb] B[block kb, jb], both 16 x 16 blocks of pitch P_LP in LDS
  auto mm_lds = [&](const float* A, int ab, int kb, const float* B, int jb, f32x4 acc) {
    const float4 av = *reinterpret_cast<const float4*>(&A[(16 * ab + q) * P_LP + 16 * kb + 4 * g4]);
    const float* bp = &B[(16 * kb + 4 * g4) * P_LP + 16 * jb + q];
    acc = mf4(av.x, bp[0], acc);
    acc = mf4(av.y, bp[P_LP], acc);
    acc = mf4(av.z, bp[2 * P_LP], acc);
    acc = mf4(av.w, bp[3 * P_LP], acc);
    return acc;
  };
  // acc += A[block ab, kb] Z, Z an accumulator
  auto mm_acc = [&](const float* A, int ab, int kb, const f32x4& Z, f32x4 acc) {
    const float4 av = *reinterpret_cast<const float4*>(&A[(16 * ab + q) * P_LP + 16 * kb + 4 * g4]);
    acc = mf4(av.x, Z[0], acc);
    acc = mf4(av.y, Z[1], acc);
    acc = mf4(av.z, Z[2], acc);
    acc = mf4(av.w, Z[3], acc);
    return acc;
  };
  // -O into block (ib, jb) of T
  auto store_neg = [&](int ib, int jb, const f32x4& o) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sT[(16 * ib + 4 * g4 + e) * P_LP + 16 * jb + q] = -o[e];
  };
  const f32x4 z4t = {0.f, 0.f, 0.f, 0.f};
  if (w < 2) {
    const int ib = 2 * w + 1, jb = 2 * w;
    const f32x4 z = mm_lds(sL, ib, jb, sT, jb, z4t);
    store_neg(ib, jb, mm_acc(sT, ib, ib, z, z4t));
  }
  lds_barrier();
  {
    const int ib = 2 + (w >> 1), jb = w & 1;
    f32x4 o = z4t;
    for (int pb = 2; pb <= ib; ++pb) {
      f32x4 z = z4t;
      for (int m = jb; m < 2; ++m) z = mm_lds(sL, pb, m, sT, jb, z);
      o = mm_acc(sT, ib, pb, z, o);
    }
    store_neg(ib, jb, o);
  }
  lds_barrier();

  // (6) N = T - I fragments of token tile w (A operand of N Y)
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    if (2 * tb > w) continue;
    const int s0 = 32 * tb + 4 * g4;
    const float4 v0 = *reinterpret_cast<const float4*>(&sT[r * P_LP + s0]);
    const float4 v1 = *reinterpret_cast<const float4*>(&sT[r * P_LP + s0 + 16]);
    const float x[8] = {s0 + 0 < r ? v0.x : 0.f, s0 + 1 < r ? v0.y : 0.f,
                        s0 + 2 < r ? v0.z : 0.f, s0 + 3 < r ? v0.w : 0.f,
                        s0 + 16 < r ? v1.x : 0.f, s0 + 17 < r ? v1.y : 0.f,
                        s0 + 18 < r ? v1.z : 0.f, s0 + 19 < r ? v1.w : 0.f};
    const int f = tri_frag(w, tb);
    const uint4 nv = __builtin_bit_cast(uint4, to_f16x8(x));
    if (tri_half(f))
      ws_store<NT>(slot + SL_N + tri_off(f) + lane * 8, make_uint2(nv.x, nv.y));
    else
      ws_store<NT>(slot + SL_N + tri_off(f) + lane * 16, nv);
  }
}

// ---------------------------------------------------------------------------
// Launch 2: recurrence.  One workgroup per (sequence, head, column group) with
// CW compute waves and KW copy waves.  Compute wave w owns 16 columns
// of the state (all 128 rows: 8 accumulator tiles in registers).  The copy
// waves bring the next segment's slot and V block into the idle one of two
// LDS buffers with global_load_lds while the compute waves consume the other;
// a copy wave may stall on a full memory queue, while inside the segment loop
// a compute wave reads only LDS.  One barrier per segment hands the buffers
// over.

template <int CW, int KW, bool SPLIT>
__global__ __launch_bounds__(64 * (CW + KW), 1) void kda_recurrence_kernel(DecompArgs a) {
  constexpr int WAVES = CW;
  // with at most two waves per SIMD (one compute, one copy) a compute wave has
  // up to 256 registers and reads its fragments in large batches; with more
  // waves it reads them as it goes and the other compute wave on the SIMD
  // covers the latency
  constexpr bool BATCHED = CW + KW <= 8;
  constexpr int VW = 16 * CW;                     // columns per workgroup
  constexpr int VUNITS = CH * VW * 2 / 1024;      // 1 KiB units of the V block
  constexpr int UNITS = SLOT_UNITS + VUNITS;
  // K~ (the first KTU units of a slot, read first in a segment) has three
  // buffers when LDS holds them, so its copy can run two segments ahead; the
  // rest of the slot and the V block have two
  constexpr int KTU = 16;
  constexpr bool KT3 = 2 * (UNITS - KTU) + 3 * KTU <= 158;
  constexpr int KB = KT3 ? KTU * 1024 : 0;        // bytes of the slot not in the `ops` buffers
  constexpr int OPS_UNITS = UNITS - KB / 1024;
  // buffers as separate arrays, so the compiler sees that reads of one do not
  // wait for copies into another
  __shared__ __attribute__((aligned(16))) uint4 opsA[OPS_UNITS * 64];
  __shared__ __attribute__((aligned(16))) uint4 opsB[OPS_UNITS * 64];
  __shared__ __attribute__((aligned(16))) uint4 ktA[KT3 ? KTU * 64 : 1];
  __shared__ __attribute__((aligned(16))) uint4 ktB[KT3 ? KTU * 64 : 1];
  __shared__ __attribute__((aligned(16))) uint4 ktC[KT3 ? KTU * 64 : 1];
  constexpr int VG = 8 / WAVES;  // column groups (workgroups) per run
  const int H = a.H;
  // What the workgroup runs over its range of segments (all of them without
  // the chain split):
  //   MAIN  from the initial state, with outputs and checkpoints
  //   ZERO  from a zero state, no outputs: the piece's affine part
  //   EYE   from the identity with V = 0, no outputs: the piece's transition
  //   CONT  from the state the chain scan left for the piece, with outputs
  // The state update is affine in the state entering a piece (the decay and
  // the delta rule's correction are linear maps of S, V enters additively),
  // so the state leaving it is T_p S + B_p with T_p from EYE and B_p from ZERO.
  enum { MAIN, ZERO, EYE, CONT };
  // workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8): keep
  // the workgroups that read one piece's slots (its column groups, and in the
  // first split launch both ZERO and EYE) on one XCD so they share L2
  const int bx = blockIdx.x, xcd = bx & 7, rest = bx >> 3;
  int pair, cg, piece = 0, role = MAIN;
  if constexpr (!SPLIT) {
    pair = (rest / VG) * 8 + xcd;
    cg = rest % VG;
    if (pair >= a.N * H) return;
  } else {
    // pass 1: pieces 0 .. P-2 (piece 0 as MAIN, the others as ZERO and EYE);
    // pass 2: pieces 1 .. P-1 as CONT
    const int per = a.pieces - 1, W = a.pass == 1 ? 2 * VG : VG;
    const int slot = rest % W, gi = (rest / W) * 8 + xcd;
    if (gi >= a.N * H * per) return;
    pair = gi / per;
    piece = gi - pair * per;
    cg = slot % VG;
    if (a.pass == 1) {
      if (piece == 0 && slot >= VG) return;
      role = piece == 0 ? MAIN : (slot < VG ? ZERO : EYE);
    } else {
      ++piece;
      role = CONT;
    }
  }
  const int rank = pair / H, h = pair - rank * H;
  const int n = a.order ? a.order[rank] : rank;
  const int64_t spair = (int64_t)n * H + h;  // the pair's index in the state layouts
  const bool emit = !SPLIT || role == MAIN || role == CONT;
  // V's weight: EYE runs with V = 0 (the V block is still copied; finite
  // bf16 values times 0 give 0)
  const float vmul = SPLIT && role == EYE ? 0.f : 1.f;
  // the wave index as a scalar: the role branch below is then uniform, so the
  // compiler keeps the two roles' code paths (and their memory counters) apart
  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, q = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  const SeqInfo si = seq_info(a, n);
  int64_t base = a.cu_seqlens ? (int64_t)a.seg_base[n] : (int64_t)n * a.slots_per_seq;
  int nseg = si.nseg;
  if (base + nseg > a.slot_bound) nseg = base >= a.slot_bound ? 0 : (int)(a.slot_bound - base);
  // the piece's segments [j0, j1) (all of them without the split)
  const int nseg_all = nseg;
  int j0 = 0;
  if constexpr (SPLIT) {
    j0 = (int)((int64_t)piece * nseg / a.pieces);
    const int j1 = (int)((int64_t)(piece + 1) * nseg / a.pieces);
    base += j0;
    nseg = j1 - j0;
  }
  auto geometry = [&](int jseg, int& off, int64_t& tok0) {
    int lo, hi;
    seg_range(si, j0 + jseg, lo, hi);
    off = CH - (hi - lo);
    tok0 = si.bos + lo - off;
  };

  if (w >= CW) {
    // ---- copy waves: unit u of the slot (or of the V block) goes to copy wave u % KW
    const int cw = w - CW;
    // geometry (off, tok0) of the segment copied next, worked out one copy
    // ahead: its scalar reads of the checkpoint offsets then wait while the
    // previous copy is in flight, not before the V rows are requested
    // the slot from unit KB / 1024 on, and the V block, into an `ops` buffer
    auto copy = [&](int jseg, uint4* dst, int off, int64_t tok0) {
      const unsigned char* src = a.slots + ((size_t)(base + jseg) * H + h) * kDecompSlotBytes;
      for (int u = KB / 1024 + cw; u < SLOT_UNITS; u += KW)
        __builtin_amdgcn_global_load_lds(src + u * 1024 + lane * 16, dst + (u - KB / 1024) * 64, 16, 0, 0);
      // V rows 0..63 (rows before the segment read row `off`; their beta is 0)
      constexpr int LPR = VW / 8, RPI = 64 / LPR;  // lanes per row, rows per unit
      for (int k = cw; k < VUNITS; k += KW) {
        const int row = max(k * RPI + lane / LPR, off);
        const uint16_t* vsrc = a.v + ((size_t)(tok0 + row) * H + h) * DK + VW * cg + 8 * (lane % LPR);
        __builtin_amdgcn_global_load_lds(vsrc, dst + (SLOT_UNITS - KB / 1024 + k) * 64, 16, 0, 0);
      }
    };
    // the checkpoint offsets (read at kernel start) have landed: the
    // geometry walks below then add no wait to the copies in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);
    int goff = 0;
    int64_t gtok = 0;
    if (KT3) {
      // K~ of segment j + 2 is requested after the rest of segment j + 1, and
      // the wait before each barrier leaves only those newest KT_PER copies in
      // flight (loads of one kind complete in order)
      constexpr int KT_PER = KTU / KW;
      auto copy_kt = [&](int jseg) {
        uint4* dst = jseg % 3 == 0 ? ktA : (jseg % 3 == 1 ? ktB : ktC);
        const unsigned char* src = a.slots + ((size_t)(base + jseg) * H + h) * kDecompSlotBytes;
        for (int u = cw; u < KTU; u += KW)
          __builtin_amdgcn_global_load_lds(src + u * 1024 + lane * 16, dst + u * 64, 16, 0, 0);
      };
      bool kt_last = false;
      if (nseg > 0) {
        geometry(0, goff, gtok);
        copy_kt(0);
        copy(0, opsA, goff, gtok);
      }
      if (nseg > 1) {
        copy_kt(1);
        kt_last = true;
        geometry(1, goff, gtok);
      }
      for (int jseg = 0; jseg < nseg; ++jseg) {
        if (kt_last)
          __builtin_amdgcn_s_waitcnt((KT_PER & 15) | ((KT_PER >> 4) << 14) | 0x0F70);
        else
          __builtin_amdgcn_s_waitcnt(0x0F70);
        // a workgroup barrier without the workgroup-scope fence (whose wait
        // for all memory operations would also take in the K~ copies kept in
        // flight); the wavefront-scope fences keep the copies on their side
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        kt_last = false;
        if (jseg + 1 < nseg) {
          copy(jseg + 1, (jseg & 1) ? opsA : opsB, goff, gtok);
          if (jseg + 2 < nseg) geometry(jseg + 2, goff, gtok);
        }
        if (jseg + 2 < nseg) {
          copy_kt(jseg + 2);
          kt_last = true;
        }
      }
      return;
    }
    if (nseg > 0) {
      geometry(0, goff, gtok);
      copy(0, opsA, goff, gtok);
    }
    if (nseg > 1) geometry(1, goff, gtok);
    for (int jseg = 0; jseg < nseg; jseg += 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies landed
      __syncthreads();
      if (jseg + 1 < nseg) {
        copy(jseg + 1, opsB, goff, gtok);
        if (jseg + 2 < nseg) geometry(jseg + 2, goff, gtok);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (jseg + 2 < nseg) {
          copy(jseg + 2, opsA, goff, gtok);
          if (jseg + 3 < nseg) geometry(jseg + 3, goff, gtok);
        }
      }
    }
    return;
  }

  // ---- compute waves
  const int col0 = 16 * (cg * WAVES + w);
  // accumulator row 16 m + 4 g4 + e holds key channel state_row_channel of it,
  // that is 8 g4 + srow(m, e)
  const size_t sbase = (size_t)spair * DK * DK + col0 + q + (size_t)(8 * g4) * DK;
  auto srow = [](int m, int e) { return 32 * (m >> 1) + 4 * (m & 1) + e; };
  // S holds 2^sexp times the state (sexp is the wave's operand scale exponent)
  f32x4 S[8];
  int sexp = 0;
  // a sequence with no segment keeps its initial state bit for bit, also
  // through the split (the scan's hi + lo products keep 16 bits)
  const bool from_s0 = !SPLIT || role == MAIN || (role == CONT && nseg_all == 0);
  if (from_s0 && a.s0 && a.state_bf16) {
    const uint16_t* s0 = reinterpret_cast<const uint16_t*>(a.s0);
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[m][e] = bf2f(s0[sbase + (size_t)srow(m, e) * DK]);
  } else if ((from_s0 && a.s0) || (SPLIT && role == CONT && !from_s0)) {
    const float* src = from_s0 ? a.s0 + sbase
                               : a.chain + chain_matrix(spair, a.pieces, piece, 0) + (sbase - (size_t)spair * DK * DK);
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[m][e] = src[(size_t)srow(m, e) * DK];
  } else if (SPLIT && role == EYE) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[m][e] = 8 * g4 + srow(m, e) == col0 + q ? 1.f : 0.f;
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m) S[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  // state store into dst at element offset e0 (fp32, or bf16 rounded to
  // nearest even when the states are bf16); the power of two comes off
  // exactly
  auto store_state = [&](float* dst, size_t e0, bool bf16 = true) {
    // the lane's offsets are formed here from an opaque lane index, so the 32
    // store addresses are not kept live in registers across the segment loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const size_t o = e0 + (size_t)spair * DK * DK + col0 + (ln & 15) + (ln >> 4) * 8 * DK;
    const float unscale = pow2f(-sexp);
    if (bf16 && a.state_bf16) {
      uint16_t* rowp = reinterpret_cast<uint16_t*>(dst) + o;
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) rowp[srow(m, e) * DK] = (uint16_t)pack2(S[m][e] * unscale, 0.f);
    } else {
      float* rowp = dst + o;
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) rowp[srow(m, e) * DK] = S[m][e] * unscale;
    }
  };
  // checkpoint c of this sequence (layout [N, C, H, K, V]): element offset
  auto ckpt_slot = [&](int c) { return ((size_t)n * (a.ckpt_per_seq - 1) + c) * (size_t)H * DK * DK; };
  // the piece's state transition T (EYE's end state; row = key channel, as
  // the state), for the scan's matrix products: bf16 hi and lo parts
  // (T = hi + lo to 16 bits), [K][K] row-major, hi then lo
  auto store_transition = [&](float* mat) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    uint16_t* hi = reinterpret_cast<uint16_t*>(mat) + col0 + (ln & 15) + (size_t)((ln >> 4) * 8) * DK;
    uint16_t* lo = hi + DK * DK;
    const float unscale = pow2f(-sexp);
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = S[m][e] * unscale;
        const uint32_t h = pack2(x, 0.f) & 0xffffu;
        hi[srow(m, e) * DK] = (uint16_t)h;
        lo[srow(m, e) * DK] = (uint16_t)pack2(x - bf2f(h), 0.f);
      }
  };
  if (!SPLIT || role == MAIN)
    for_each_honoured(si.ck, [&](int c, int p) {
      if (p == 0) store_state(a.ckpt, ckpt_slot(c));
    });

  uint32_t opk[8];
  int poff = CH;
  int64_t ptok = 0;
  // O^T tile t of the segment (first row poff, token of row 0 ptok): lane
  // holds token 16 t + q, columns col0 + 4 g4 .. + 3 (one 8-byte store per
  // tile).  Issued at the end of the segment, behind the state update's
  // products, rather than next to the copy waves' requests at its start
  // (about 3% at B8 T8192).
  auto store_out = [&]() {
    uint16_t* ob = a.out + ((size_t)ptok * H + h) * DK + col0;
    // lane offset formed here (opaque), not kept live across the segment loop
    int ro = q * H * DK + 4 * g4;
    asm volatile("" : "+v"(ro));
    if (poff == 0) {
      // a whole segment (all but a sequence's last and those cut at a
      // checkpoint): no per-lane condition, so no branches around the stores
#pragma unroll
      for (int t = 0; t < 4; ++t)
        *reinterpret_cast<uint2*>(ob + ro + t * 16 * H * DK) = make_uint2(opk[2 * t], opk[2 * t + 1]);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (16 * t + q >= poff)
          *reinterpret_cast<uint2*>(ob + ro + t * 16 * H * DK) = make_uint2(opk[2 * t], opk[2 * t + 1]);
    }
  };

  auto step = [&](int jseg, const uint4* cur) {
    // K~ of this segment: its own buffer, or the start of `cur`
    const uint4* kcur = !KT3 ? cur : (jseg % 3 == 0 ? ktA : (jseg % 3 == 1 ? ktB : ktC));
    lds_barrier();  // the copy waves have filled `cur`
    // An opaque copy of the lane index, renewed every segment: LDS addresses
    // become one register plus an immediate offset instead of dozens of
    // precomputed addresses kept live across the loop.
    int lq = lane;
    asm volatile("" : "+v"(lq));
    const int qq = lq & 15, gg = lq >> 4;
    // slot byte offsets: K~ from `kcur`, the rest from `cur` (shifted by KB)
    auto frag = [&](int byte_off) {
      return __builtin_bit_cast(f16x8, byte_off < SL_QT ? kcur[(byte_off >> 4) + lq]
                                                        : cur[((byte_off - KB) >> 4) + lq]);
    };
    auto f4 = [&](int byte_off) {
      return *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(cur) + byte_off - KB);
    };
    // M or N fragment f (half fragments: upper 8 bytes are zero)
    auto trifrag = [&](int region, int f) {
      const char* base = reinterpret_cast<const char*>(cur) + region - KB + tri_off(f);
      if (tri_half(f)) {
        const uint2 lo = *reinterpret_cast<const uint2*>(base + lq * 8);
        return __builtin_bit_cast(f16x8, make_uint4(lo.x, lo.y, 0u, 0u));
      }
      return __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(base + lq * 16));
    };
    const uint16_t* vblk = reinterpret_cast<const uint16_t*>(cur + (SLOT_UNITS - KB / 1024) * 64);

    // The segment runs as load batches and matrix batches separated by
    // scheduling fences: fragment reads go out together and are consumed while
    // the next batch is in flight (without the fences the reads are issued one
    // at a time, each waited for before its product).
#define KDA_FENCE()                                 \
  do {                                              \
    if (BATCHED) __builtin_amdgcn_sched_barrier(0); \
  } while (0)
    f16x8 fk[16], fq[16];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        fk[t * 4 + b] = frag(SL_KT + (t * 4 + b) * 1024);
        fq[t * 4 + b] = frag(SL_QT + (t * 4 + b) * 1024);
      }
    float4 bt4[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) bt4[t] = f4(SL_BETA + (16 * t + 4 * gg) * 4);
    f16x8 Sb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) Sb[b] = acc_pair_h(S[2 * b], S[2 * b + 1]);
    // max |2^s S| for the operand scale check below, formed beside the first
    // products (it needs only the state)
    float smx = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) smx = fmaxf(smx, fabsf(S[m][e]));
    float4 gm[8];
    if constexpr (BATCHED) {
#pragma unroll
      for (int m = 0; m < 8; ++m) gm[m] = f4(SL_GAM + (16 * m + 4 * gg) * 4);
    }
    KDA_FENCE();
    // X = K~ S, key blocks 0-1; the rest of K~ is read meanwhile
    f32x4 X[4], O[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) X[t] = mfma(fk[t * 4], Sb[0], (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int b = 2; b < 4; ++b) fk[t * 4 + b] = frag(SL_KT + (t * 4 + b) * 1024);
#pragma unroll
    for (int t = 0; t < 4; ++t) X[t] = mfma(fk[t * 4 + 1], Sb[1], X[t]);
    KDA_FENCE();
#pragma unroll
    for (int b = 2; b < 4; ++b)
#pragma unroll
      for (int t = 0; t < 4; ++t) X[t] = mfma(fk[t * 4 + b], Sb[b], X[t]);
    // the decayed state diag(Gam) S, the state update's accumulator input,
    // formed while the products run (off the chain of the update; S itself
    // stays for the scale check).  Without batches (three waves per SIMD,
    // fewer registers each) it is formed at the update instead.
    f32x4 Sd[8];
    auto decay = [&]() {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        Sd[m][0] = S[m][0] * gm[m].x;
        Sd[m][1] = S[m][1] * gm[m].y;
        Sd[m][2] = S[m][2] * gm[m].z;
        Sd[m][3] = S[m][3] * gm[m].w;
      }
    };
    if constexpr (BATCHED) decay();
    KDA_FENCE();
    // the rest of Q~, the V block and N, read while O^T = S^T Q~^T runs
    const int4 hd = *reinterpret_cast<const int4*>(reinterpret_cast<const char*>(cur) + SL_HDR - KB);
    const uint2 hmask = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(cur) + SL_HDR - KB + 16);
    const int off = __builtin_amdgcn_readfirstlane(hd.x);
    const int64_t tok0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(hd.w) << 32) |
                                   (uint32_t)__builtin_amdgcn_readfirstlane(hd.z));
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int b = 2; b < 4; ++b) fq[t * 4 + b] = frag(SL_QT + (t * 4 + b) * 1024);
    uint16_t vv[16];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[4 * t + e] = vblk[(16 * t + 4 * gg + e) * VW + 16 * w + qq];
    // N: read here when the wave reads in batches; without batches (more
    // waves, fewer registers each) only after the scale check below, so that
    // its registers are free for a recomputation
    f16x8 fn[6];
    if constexpr (BATCHED) {
#pragma unroll
      for (int i = 0; i < 6; ++i) fn[i] = trifrag(SL_N, i);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) O[t] = mfma(Sb[0], fq[t * 4], (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int b = 1; b < 4; ++b)
#pragma unroll
      for (int t = 0; t < 4; ++t) O[t] = mfma(Sb[b], fq[t * 4 + b], O[t]);
    // Operand scale check, while the products above run (no fence: its VALU
    // work fills the issue slots between them): the largest of
    // |2^s S| and |2^s V| over the wave must lie in [4, 64] (or be 0).  When
    // it does not, s is reset so that it lands in [16, 32) -- the state is
    // multiplied by the change of 2^s (exact) and X, O are formed again.
    {
      const float mx = smx;
      // |V| as bf16 bits: for non-negative values their order is the values' order
      uint32_t vmax = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) vmax = max(vmax, (uint32_t)vv[i] & 0x7fffu);
      const float big = wave_max_nonneg(fmaxf(mx, bf2f(vmax) * (pow2f(sexp) * vmul)));
      const int nexp = rescale_exponent(big, sexp);
      if (nexp != sexp) {
        const int dexp = nexp - sexp;
        sexp = nexp;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            S[m][e] = __builtin_ldexpf(S[m][e], dexp);
            if constexpr (BATCHED) Sd[m][e] = __builtin_ldexpf(Sd[m][e], dexp);
          }
#pragma unroll
        for (int b = 0; b < 4; ++b) Sb[b] = acc_pair_h(S[2 * b], S[2 * b + 1]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          X[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
          O[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
        // K~ and Q~ read again (the buffers hold them until the next
        // barrier), one key block at a time
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            X[t] = mfma(frag(SL_KT + (t * 4 + b) * 1024), Sb[b], X[t]);
            O[t] = mfma(Sb[b], frag(SL_QT + (t * 4 + b) * 1024), O[t]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if constexpr (!BATCHED) {
#pragma unroll
      for (int i = 0; i < 6; ++i) fn[i] = trifrag(SL_N, i);
    }
    const float sig = pow2f(sexp) * vmul;
    // Y = beta (2^s V - X), kept in U; U = Y + N Y.  Rows before the segment
    // have beta = 0 (their V read is a copy of row `off`), so they give U = 0.
    f32x4 U[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float bv[4] = {bt4[t].x, bt4[t].y, bt4[t].z, bt4[t].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) U[t][e] = bv[e] * (bf2f(vv[4 * t + e]) * sig - X[t][e]);
    }
    const f16x8 Y0 = acc_pair_h(U[0], U[1]), Y1 = acc_pair_h(U[2], U[3]);
    U[0] = mfma(fn[tri_frag(0, 0)], Y0, U[0]);
    U[1] = mfma(fn[tri_frag(1, 0)], Y0, U[1]);
    U[2] = mfma(fn[tri_frag(2, 0)], Y0, U[2]);
    U[3] = mfma(fn[tri_frag(3, 0)], Y0, U[3]);
    U[2] = mfma(fn[tri_frag(2, 1)], Y1, U[2]);
    U[3] = mfma(fn[tri_frag(3, 1)], Y1, U[3]);
    // M and the first half of K^, read while N Y runs
    f16x8 fm[6], fh[16];
#pragma unroll
    for (int i = 0; i < 6; ++i) fm[i] = trifrag(SL_M, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) fh[i] = frag(SL_KH + i * 1024);
    KDA_FENCE();
    f16x8 Uh[2], Ul[2];
    acc_pair_split_h(U[0], U[1], Uh[0], Ul[0]);
    acc_pair_split_h(U[2], U[3], Uh[1], Ul[1]);
    // O^T += U^T M^T
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (2 * b > t) continue;
        O[t] = mfma(Uh[b], fm[tri_frag(t, b)], O[t]);
      }
    // second half of K^, read while M U runs
#pragma unroll
    for (int i = 8; i < 16; ++i) fh[i] = frag(SL_KH + i * 1024);
    KDA_FENCE();
    // read-out: scale * 2^-s
    const float osc = a.scale * pow2f(-sexp);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      opk[2 * t] = pack2(O[t][0] * osc, O[t][1] * osc);
      opk[2 * t + 1] = pack2(O[t][2] * osc, O[t][3] * osc);
    }
    // S <- diag(Gam) S + K^^T U
    if constexpr (!BATCHED) {
#pragma unroll
      for (int m = 0; m < 8; ++m) gm[m] = f4(SL_GAM + (16 * m + 4 * gg) * 4);
      decay();
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      S[m] = mfma(fh[2 * m], Uh[0], Sd[m]);
      S[m] = mfma(fh[2 * m], Ul[0], S[m]);
      S[m] = mfma(fh[2 * m + 1], Uh[1], S[m]);
      S[m] = mfma(fh[2 * m + 1], Ul[1], S[m]);
    }
#undef KDA_FENCE
    poff = off;
    ptok = tok0;
    if (emit) store_out();
    if (emit && si.ck.C > 0) {
      unsigned long long mask = ((unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane(hmask.y) << 32) |
                                (uint32_t)__builtin_amdgcn_readfirstlane(hmask.x);
      while (mask) {
        const int c = __builtin_ctzll(mask);
        mask &= mask - 1;
        store_state(a.ckpt, ckpt_slot(c));
      }
    }
  };

  for (int jseg = 0; jseg < nseg; jseg += 2) {
    step(jseg, opsA);
    if (jseg + 1 < nseg) step(jseg + 1, opsB);
  }
  // the end state: the result, or what the chain scan takes (as offsets from
  // the pair's own state offset, which store_state adds)
  if constexpr (SPLIT) {
    const size_t own = (size_t)spair * DK * DK;
    if (role == EYE) {
      store_transition(a.chain + chain_matrix(spair, a.pieces, piece, 2));
    } else if (role == ZERO) {
      store_state(a.chain, chain_matrix(spair, a.pieces, piece, 1) - own, false);
    } else if (role == MAIN) {
      store_state(a.chain, chain_matrix(spair, a.pieces, 1, 0) - own, false);
    } else if (a.final_state && piece == a.pieces - 1) {
      store_state(a.final_state, 0);
    }
  } else if (a.final_state) {
    store_state(a.final_state, 0);
  }
}

// ---------------------------------------------------------------------------
// Chain scan, between the split's two recurrence launches: the state entering
// piece p + 1 is T_p S_p + B_p for p = 1 .. P-2 (S_1 from the first launch's
// MAIN run; T_p from EYE as bf16 hi + lo, B_p from ZERO).  Columns of the
// state are independent, so one workgroup takes 16 columns of one (sequence,
// head) pair through all the steps.  T_p S_p runs on the matrix cores as
// three bf16 products, Th Sh + Th Sl + Tl Sh (16x16x32, fp32 accumulation);
// the Tl Sl term dropped is about 2^-16 of the result, far below the fp32
// state's own rounding over a piece.  Wave w owns rows 32 w .. 32 w + 31 (two
// 16-row tiles).  T_{p+1} streams into one LDS buffer (direct global-to-LDS
// loads) while step p computes from the other; the buffers are separate
// arrays and the steps alternate between them by name, so the compiler sees
// that reads of one do not wait for the copies into the other.  In LDS a row
// of T (256 bytes per part) keeps its 16-byte pieces XOR-swizzled by the row
// index, and so does S^T, so that a fragment read, 16 rows at one k, hits 16
// different bank groups.
constexpr int kScanCols = 16;
constexpr int kScanThreads = 256;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

__global__ __launch_bounds__(kScanThreads) void kda_chain_scan_kernel(DecompArgs a) {
  __shared__ __attribute__((aligned(16))) uint4 TA[DK * DK * 4 / 16];  // hi, then lo: [K][K] bf16
  __shared__ __attribute__((aligned(16))) uint4 TB[DK * DK * 4 / 16];
  __shared__ __attribute__((aligned(16))) uint4 St[kScanCols * DK * 4 / 16];  // S^T hi, lo: [16][K] bf16
  // a pair's 8 column groups on one XCD (workgroups are dealt to the 8 XCDs
  // round-robin), so that T_p is fetched into that XCD's L2 once
  static_assert(DK / kScanCols == 8, "one column group per XCD slot");
  const int bx = blockIdx.x, xcd = bx & 7, slot = bx >> 3;
  const int64_t pair = (int64_t)(slot >> 3) * 8 + xcd;
  const int c0 = (slot & 7) * kScanCols;
  if (pair >= (int64_t)a.N * a.H || a.pieces < 3) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, q = lane & 15, g4 = lane >> 4;
  constexpr int PART = DK * DK * 2;  // bytes of one bf16 part of T
  // T_p (64 KiB: hi then lo), 1 KiB units, wave w taking units w, w + 4, ...;
  // LDS byte o holds row o / 256 of its part, swizzled piece (o % 256) / 16
  auto fetch = [&](int p, uint4* dst) {
    const unsigned char* src = reinterpret_cast<const unsigned char*>(a.chain + chain_matrix(pair, a.pieces, p, 2));
#pragma unroll
    for (int i = 0; i < 2 * PART / 1024 / (kScanThreads / 64); ++i) {
      const int u = w + (kScanThreads / 64) * i;
      const int o = u * 1024 + lane * 16, part = o / PART, r = (o % PART) >> 8, pc = (o >> 4) & 15;
      __builtin_amdgcn_global_load_lds(src + part * PART + r * 256 + ((pc ^ (r & 15)) << 4), dst + u * 64, 16, 0,
                                       0);
    }
  };
  // the lane's outputs: column c0 + q, rows r0(tile) + 4 g4 + e
  auto r0 = [&](int tile) { return 32 * w + 16 * tile; };
  auto load_b = [&](int p, f32x4& b0, f32x4& b1) {
    const float* bp = a.chain + chain_matrix(pair, a.pieces, p, 1) + c0 + q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b0[e] = bp[(size_t)(r0(0) + 4 * g4 + e) * DK];
      b1[e] = bp[(size_t)(r0(1) + 4 * g4 + e) * DK];
    }
  };
  // S'^T hi and lo into St: the lane's 4 rows are 4 consecutive k of column q
  auto put_s = [&](int tile, const f32x4& v) {
    const int k = r0(tile) + 4 * g4;
    const uint32_t h0 = pack2(v[0], v[1]), h1 = pack2(v[2], v[3]);
    const uint32_t l0 = pack2(v[0] - lo_of(h0), v[1] - hi_of(h0)), l1 = pack2(v[2] - lo_of(h1), v[3] - hi_of(h1));
    unsigned char* sb = reinterpret_cast<unsigned char*>(St) + swz(q, k >> 3) + (k & 4) * 2;
    *reinterpret_cast<uint2*>(sb) = make_uint2(h0, h1);
    *reinterpret_cast<uint2*>(sb + kScanCols * DK * 2) = make_uint2(l0, l1);
  };
  auto step = [&](int p, const uint4* cur, uint4* nxt, f32x4& b0, f32x4& b1) {
    f32x4 acc[2][3];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      acc[tile][0] = tile ? b1 : b0;
      acc[tile][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
      acc[tile][2] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    if (p + 2 < a.pieces) {
      fetch(p + 1, nxt);
      load_b(p + 1, b0, b1);
    }
    const unsigned char* tb = reinterpret_cast<const unsigned char*>(cur);
    const unsigned char* sb = reinterpret_cast<const unsigned char*>(St);
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      const int ch = 4 * kb + g4;  // 16-byte piece: k = 8 ch .. 8 ch + 7
      const bf16x8 sh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(sb + swz(q, ch)));
      const bf16x8 sl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(sb + kScanCols * DK * 2 + swz(q, ch)));
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const int r = r0(tile) + q;
        const bf16x8 th = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tb + swz(r, ch)));
        const bf16x8 tl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tb + PART + swz(r, ch)));
        acc[tile][0] = mfma(th, sh, acc[tile][0]);
        acc[tile][1] = mfma(th, sl, acc[tile][1]);
        acc[tile][2] = mfma(tl, sh, acc[tile][2]);
      }
    }
    f32x4 res[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile)
#pragma unroll
      for (int e = 0; e < 4; ++e) res[tile][e] = acc[tile][0][e] + (acc[tile][1][e] + acc[tile][2][e]);
    // every wave is done reading St and `cur` (its reads have returned: the
    // products used them); the copies into `nxt` stay in flight, so no
    // workgroup-scope fence, whose release would wait for them
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    put_s(0, res[0]);
    put_s(1, res[1]);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's part of T_{p+1} landed
    lds_barrier();                       // every wave's part landed; St holds S_{p+1}
    // S_{p+1} for the second launch, stored after the wait above so that it
    // covers the copies only; the next step's wait finds these done
    float* dst = a.chain + chain_matrix(pair, a.pieces, p + 1, 0) + c0 + q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dst[(size_t)(r0(0) + 4 * g4 + e) * DK] = res[0][e];
      dst[(size_t)(r0(1) + 4 * g4 + e) * DK] = res[1][e];
    }
  };
  fetch(1, TA);
  f32x4 b0, b1;
  load_b(1, b0, b1);
  {
    // S_1's 16 columns, split: thread t takes row (k) t / 2, columns 8 (t & 1) .. + 7
    const int k = t >> 1, cb = 8 * (t & 1);
    const float4* s1 = reinterpret_cast<const float4*>(a.chain + chain_matrix(pair, a.pieces, 1, 0) + (size_t)k * DK +
                                                       c0 + cb);
    const float4 x = s1[0], y = s1[1];
    const float v[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    unsigned char* sb = reinterpret_cast<unsigned char*>(St);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t h = pack2(v[j], 0.f) & 0xffffu;
      const int off = swz(cb + j, k >> 3) + (k & 7) * 2;
      *reinterpret_cast<uint16_t*>(sb + off) = (uint16_t)h;
      *reinterpret_cast<uint16_t*>(sb + kScanCols * DK * 2 + off) = (uint16_t)pack2(v[j] - bf2f(h), 0.f);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  lds_barrier();
  for (int p = 1; p + 1 < a.pieces; p += 2) {
    step(p, TA, TB, b0, b1);
    if (p + 2 < a.pieces) step(p + 1, TB, TA, b0, b1);
  }
}

template <int CW, int KW>
hipError_t launch_recurrence(const DecompArgs& a, hipStream_t stream) {
  constexpr int VG = 8 / CW;
  const int64_t pairs = (int64_t)a.N * a.H;
  const dim3 grid((unsigned)(((pairs + 7) / 8) * 8 * VG));
  hipLaunchKernelGGL((kda_recurrence_kernel<CW, KW, false>), grid, dim3(64 * (CW + KW)), 0, stream, a);
  return hipGetLastError();
}

// one launch of the chain split: groups of (pair, piece), `roles` runs of VG
// workgroups each per group (the first launch: ZERO's and EYE's)
template <int CW, int KW>
hipError_t launch_split_pass(const DecompArgs& b, int64_t groups, int roles, hipStream_t stream) {
  constexpr int VG = 8 / CW;
  hipLaunchKernelGGL((kda_recurrence_kernel<CW, KW, true>), dim3((unsigned)(((groups + 7) / 8) * 8 * roles * VG)),
                     dim3(64 * (CW + KW)), 0, stream, b);
  return hipGetLastError();
}

hipError_t split_pass(int vsplit, const DecompArgs& b, int64_t groups, int roles, hipStream_t stream) {
  switch (vsplit) {
    case 1: return launch_split_pass<8, 4>(b, groups, roles, stream);
    case 2: return launch_split_pass<4, 4>(b, groups, roles, stream);
    case 4: return launch_split_pass<2, 2>(b, groups, roles, stream);
    case 8: return launch_split_pass<1, 1>(b, groups, roles, stream);
    default: return hipErrorInvalidValue;
  }
}

// the chain split: P - 1 groups of (pair, piece) per pair in each launch; a
// group of the first launch holds ZERO's and EYE's workgroups (piece 0's
// MAIN takes ZERO's place).  The two launches may run with different
// workgroups per pair: the first holds twice the workgroups of the second.
hipError_t launch_split(const DecompArgs& a, int vsplit_first, int vsplit, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.N * a.H;
  const int64_t groups = pairs * (a.pieces - 1);
  DecompArgs b = a;
  b.pass = 1;
  hipError_t err = split_pass(vsplit_first, b, groups, 2, stream);
  if (err != hipSuccess) return err;
  if (a.pieces > 2) {
    hipLaunchKernelGGL(kda_chain_scan_kernel, dim3((unsigned)(((pairs + 7) / 8) * 8 * (DK / kScanCols))),
                       dim3(kScanThreads), 0, stream, b);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  b.pass = 2;
  return split_pass(vsplit, b, groups, 1, stream);
}

}  // namespace

hipError_t launch_decomp(const DecompArgs& a, int vsplit, int vsplit_first, int64_t prepare_slots, int stages,
                         bool stream_ws, hipStream_t stream) {
  hipError_t err;
  if (stages & 1) {
    if (a.cu_seqlens) {
      hipLaunchKernelGGL(kda_plan_kernel, dim3(1), dim3(1024), 0, stream, a);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const int64_t blocks = (a.prep_xcd ? (prepare_slots + 7) / 8 * 8 : prepare_slots) * a.H;
    if (blocks > 0) {
      if (stream_ws)
        hipLaunchKernelGGL(kda_prepare_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL(kda_prepare_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  if (!(stages & 2)) return hipSuccess;
  if (a.pieces >= 2) return launch_split(a, vsplit_first, vsplit, stream);
  switch (vsplit) {
    case 1: return launch_recurrence<8, 4>(a, stream);
    case 2: return launch_recurrence<4, 4>(a, stream);
    case 4: return launch_recurrence<2, 2>(a, stream);
    case 8: return launch_recurrence<1, 1>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
