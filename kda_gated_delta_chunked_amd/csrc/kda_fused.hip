// kda_fused.hip -- one-launch chunked KDA prefill for gfx950 (MI355X).
//
// One workgroup of 512 threads (8 wave64s) owns one (sequence, head) pair and
// a slice of VW columns of its 128 x 128 fp32 state (VSPLIT = 128 / VW
// workgroups share a pair; the columns of the state evolve independently).
// It walks the sequence in segments of at most 64 tokens aligned to the
// sequence start; a checkpoint offset inside a chunk splits that chunk in two,
// so the exported state is the exact state after that many tokens.
//
// Per segment of c <= 64 rows (placed in the last c rows of a 64-row tile;
// the rows before them are zero and contribute nothing),
// with G_r = g_0 + ... + g_r per key channel:
//   A[r,s] = sum_d k_rd k_sd exp(G_rd - G_sd)   s < r    (gated K K^T)
//   M[r,s] = sum_d q_rd k_sd exp(G_rd - G_sd)   s <= r   (gated Q K^T)
//   T = (I + diag(beta) A)^-1,  N = T - I
//   X = V - (K exp(G)) S,  Y = diag(beta) X,  U = Y + N Y
//   O = scale ((Q exp(G)) S + M U)
//   S <- diag(exp(G_end)) S + (K exp(G_end - G))^T U
// which is the token recurrence (decay, delta-rule correction, read-out of
// the updated state) regrouped by chunks.
//
// Exponent range: exp(G_r - G_s) is split as a product of two factors around
// a reference inside the chunk.  Rows are grouped in 16-row blocks; with
// g >= -5 (the gate lower bound of the KDA prefill contract, lmdeploy PR
// #5050, Modification) no factor exceeds exp(80), which fp32 and bf16 hold.
// Per row r of block i: Ef_r = exp(G_r - G_{16i-1}) <= 1 (prefix product of
// exp(g) inside the block) and Eb_r = exp(G_{16i+15} - G_r) <= 1 (suffix
// product); bd_i = exp(sum of g over block i).
//   block (i,i):    exp(G_r - G_s) = Ef_r * (Eb_s / bd_i)
//   block (i,i-1):  exp(G_r - G_s) = Ef_r * Eb_s
//   block (i,j<i-1):exp(G_r - G_s) = Ef_r * Eb_s * prod_{j<m<i} bd_m
//
// Matrix products run on the matrix cores with fp32 accumulation.  Operands
// are fp16 (v_mfma_f32_16x16x32_f16) wherever their range allows it: K exp(G),
// Q exp(G), K exp(G_end - G) (|k|, |q| <= 1 times factors <= 1), the blocks of
// the gated products left of the diagonal block (both factors <= 1), L, T
// and N in the solve merges (|A|, |T| <= 1), and the state, V, Y and U after
// multiplying them by a power of two 2^s shared by the workgroup.  The
// diagonal 16 x 16 blocks of A and M, whose factors span exp(-80) to exp(80),
// take bf16 hi + lo operands; U is fed as fp16 hi + lo into the state update;
// the identity part of T is applied in fp32 (U = Y + N Y).  fp16 keeps 11
// significant bits against bf16's 8: at slow decay (g near 0) K exp(G) S and
// N Y are as large as the writes themselves and their rounding no longer
// decays away.
//
// The power of two: the state is held as 2^s S and V enters as 2^s V, so
// every product is 2^s times the unscaled one (exact).  After each segment
// every wave publishes the largest |2^s S| of its rows, and the staging of a
// segment's V its largest |V|; when the larger of max|2^s S| and 2^s max|V|
// leaves [4, 64], s is reset so that it lands in [16, 32) (the bounds that
// keep 2^s X, 2^s Y and 2^s U inside fp16).  The read-out takes scale 2^-s,
// exported states 2^-s.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_ckpt.h"
#include "kda_kernels.h"

namespace kda {
namespace {

constexpr int CH = 64;        // chunk rows
constexpr int DK = 128;       // key channels
constexpr int DVT = 128;      // value channels (total)
constexpr int NT = 512;       // threads per workgroup (8 wave64s)
constexpr int KP = DK + 8;    // bf16 pitch of [row][d] operand tiles
constexpr int RP = CH + 8;    // bf16 pitch of [*][r] tiles (64 wide)
constexpr int LDP = 16 + 4;   // fp32 pitch of the 16 x 16 diagonal L blocks
constexpr int TP = 32 + 8;    // bf16 pitch of 32 x 32 solve tiles
constexpr int SP = 16 + 8;    // bf16 pitch of 16 x 16 solve tiles

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ float lo_of(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_of(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
// hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack2(a, b);
  lo = pack2(a - lo_of(hi), b - hi_of(hi));
}
// two floats -> packed fp16 pair (round to nearest even), one v_cvt_pk_f16_f32
__device__ __forceinline__ uint32_t pack2h(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}
__device__ __forceinline__ float h_lo(uint32_t p) { return (float)__builtin_bit_cast(f16x2, p)[0]; }
__device__ __forceinline__ float h_hi(uint32_t p) { return (float)__builtin_bit_cast(f16x2, p)[1]; }
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// hi = fp16(x), lo = fp16(x - hi)
__device__ __forceinline__ void split2h(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack2h(a, b);
  lo = pack2h(a - h_lo(hi), b - h_hi(hi));
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ f16x8 lds8h(const uint16_t* p) {
  return *reinterpret_cast<const f16x8*>(p);
}
__device__ __forceinline__ f16x8 zero8h() {
  return __builtin_bit_cast(f16x8, make_uint4(0u, 0u, 0u, 0u));
}
// eight values stored in LDS as bf16 hi (+ lo) pairs, as one fp16 operand
// (a value too small for fp16 flushes towards 0: in the gated products that
// only happens where the whole product is below fp16's range)
__device__ __forceinline__ f16x8 lds8_bf_to_h(const uint16_t* hi_p, const uint16_t* lo_p) {
  const uint4 h = *reinterpret_cast<const uint4*>(hi_p);
  const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
  uint32_t o[4];
  if (lo_p) {
    const uint4 l = *reinterpret_cast<const uint4*>(lo_p);
    const uint32_t lw[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = pack2h(lo_of(hw[e]) + lo_of(lw[e]), hi_of(hw[e]) + hi_of(lw[e]));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack2h(lo_of(hw[e]), hi_of(hw[e]));
  }
  return __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3]));
}
// value of lane q - n of this 16-lane row (0 for q < n)
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, true));
}
// largest value over the wave of non-negative x, the same in every lane
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
// Operand scale exponent after seeing `big` (the same in every lane): s stays
// while big lies in [4, 64] or is 0 (or not finite); otherwise the new s puts
// big in [16, 32), limited to |s| <= 120.
__device__ __forceinline__ int rescale_exponent(float big, int s) {
  const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane(__float_as_int(big));
  if (b == 0u || b >= 0x7f800000u || (b >= 0x40800000u && b <= 0x42800000u)) return s;
  const int e = (int)(b >> 23) - 127;
  int ns = s + 4 - e;
  ns = ns < -120 ? -120 : (ns > 120 ? 120 : ns);
  return ns;
}

template <int VW>
struct Layout {
  static constexpr int NTILE = VW / 16;
  static constexpr int VP = VW + 8;                    // bf16 pitch of [64][VW] tiles
  // gate-operand phase (rows x KP, bf16 or fp16 as noted).  The left
  // operands serve the diagonal blocks (bf16: their factor goes down to
  // exp(-80)) and, turned into fp16 on load, the blocks left of them.
  static constexpr int G_KF = 0;                       // K exp(G - G_blockstart), bf16 hi
  static constexpr int G_KFLO = G_KF + 64 * KP * 2;    //   and lo
  static constexpr int G_QF = G_KFLO + 64 * KP * 2;    // Q exp(G - G_blockstart), bf16 hi
  static constexpr int G_QFLO = G_QF + 64 * KP * 2;    //   and lo
  static constexpr int G_KR = G_QFLO + 64 * KP * 2;    // diagonal-block right operand, bf16 hi
  static constexpr int G_KRLO = G_KR + 64 * KP * 2;    //   and lo
  static constexpr int G_KB = G_KRLO + 64 * KP * 2;   // K exp(G_blockend - G), blocks 0..2, fp16
  static constexpr int G_OPS = G_KB + 48 * KP * 2;
  // prepared operands (same region, after the gate products), fp16
  static constexpr int P_KT = 0;                       // -K exp(G)   [64][KP]
  static constexpr int P_QT = P_KT + 64 * KP * 2;      //  Q exp(G)   [64][KP]
  static constexpr int P_KHT = P_QT + 64 * KP * 2;     //  K exp(G_end - G), transposed [128][RP]
  static constexpr int P_M = P_KHT + DK * RP * 2;      //  M [64][RP]
  static constexpr int P_N = P_M + 64 * RP * 2;        //  N [64][RP]
  static constexpr int P_END = P_N + 64 * RP * 2;
  // triangular-solve scratch (after the gate products, before the recurrence), fp16
  static constexpr int S_LB = P_END;                   // L [64][RP] (off-diagonal blocks)
  static constexpr int S_TAT = S_LB + 64 * RP * 2;     // [[T00,0],[T10,T11]]^T [32][TP]
  static constexpr int S_TBR = S_TAT + 32 * TP * 2;    // [[T22,0],[T32,T33]]   [32][TP]
  static constexpr int S_T22T = S_TBR + 32 * TP * 2;   // T22^T [16][SP]
  static constexpr int S_T11R = S_T22T + 16 * SP * 2;  // T11   [16][SP]
  static constexpr int S_END = S_T11R + 16 * SP * 2;
  // recurrence scratch (after the solve; aliases the solve scratch), fp16
  static constexpr int D_UHI = P_END;                  // U^T hi [VW][RP]
  static constexpr int D_ULO = D_UHI + VW * RP * 2;    // U^T lo [VW][RP]
  static constexpr int D_Y = D_ULO + VW * RP * 2;      // Y^T [VW][RP]
  static constexpr int D_END = D_Y + VW * RP * 2;
  // half-block products of the next segment's gate factors [8][128] fp32,
  // live from its gate_factors_1 to gate_factors_2, both inside phase D (or
  // before the first segment), when only the prepared operands and the
  // recurrence scratch below it are in use (the solve scratch is dead by then)
  static constexpr int D_HALF = D_END;
  static constexpr int D_HALF_END = D_HALF + 8 * DK * 4;
  static constexpr int G_END = G_OPS > D_HALF_END ? (G_OPS > S_END ? G_OPS : S_END)
                                                  : (D_HALF_END > S_END ? D_HALF_END : S_END);
  // always-live
  static constexpr int A_V = G_END;                    // V slice bf16 [64][VP]
  static constexpr int A_BETA = A_V + 64 * VP * 2;     // [64] fp32
  static constexpr int A_GAM = A_BETA + 64 * 4;        // [128] fp32
  static constexpr int A_BD = A_GAM + DK * 4;          // [4][128] fp32
  static constexpr int A_LDT = A_BD + 4 * DK * 4;      // diag blocks of L, transposed, fp32 [4][16][LDP]
  static constexpr int A_OSTG = A_LDT + 4 * 16 * LDP * 4;  // output staging bf16 [64][VP]
  static constexpr int A_ST = A_OSTG + 64 * VP * 2;    // (2^s S)^T fp16 [VW][KP]: the state as a B operand
  static constexpr int A_MAX = A_ST + VW * KP * 2;     // [8] max |2^s S| per wave, [8] max |V| per wave
  static constexpr int TOTAL = A_MAX + 16 * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Raw inputs of one segment for one thread of the elementwise role (rows
// 16ib + 8hb .. +7, channels d0, d0+1), plus its share of the V slice and beta.
struct SegmentLoads {
  float2 g[8];
  uint32_t k[8], q[8];
  uint4 v;
  float beta;
  bool bvalid;  // this thread's beta row lies in the segment
};

template <int VW>
__global__ __launch_bounds__(NT, 1) void kda_fused_kernel(FusedArgs a) {
  using Lay = Layout<VW>;
  constexpr int VSPLIT = DVT / VW;
  constexpr int NTILE = Lay::NTILE;                  // 16-column tiles owned
  constexpr int NTW = NTILE >= 2 ? NTILE / 2 : 1;    // tiles per wave in the row-block phases
  constexpr int PER_ROW = VW / 8;                    // 16-byte pieces per V row
  __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::TOTAL];

  // ---- which (sequence, head, column slice) this workgroup owns --------------
  // Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8); keep
  // the VSPLIT workgroups of a pair on the same XCD so they share L2 for q/k/g.
  const int bx = blockIdx.x;
  const int xcd = bx & 7, rest = bx >> 3;
  const int vs = rest % VSPLIT;
  const int pair = (rest / VSPLIT) * 8 + xcd;
  if (pair >= a.num_pairs) return;
  const int n = pair / a.H, h = pair % a.H;
  const int H = a.H;

  int64_t bos, len;
  if (a.cu_seqlens) {
    // clamped into [0, T_total] even for offsets that break the contract
    clamp_seq_range(cu_at(a.cu_seqlens, a.cu64, n), cu_at(a.cu_seqlens, a.cu64, n + 1), a.T_total, &bos,
                    &len);
  } else {
    len = a.T_fixed;
    bos = (int64_t)n * len;
  }
  // checkpoint offsets of the sequence (C = 0 when none)
  const CkptList ck = load_ckpt_list(a.ckpt_off, a.ckpt_per_seq, n, (int)len);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;   // w is wave-uniform
  const int col0 = vs * VW;             // first state column owned

  uint16_t* gKf = reinterpret_cast<uint16_t*>(smem + Lay::G_KF);
  uint16_t* gKfLo = reinterpret_cast<uint16_t*>(smem + Lay::G_KFLO);
  uint16_t* gQf = reinterpret_cast<uint16_t*>(smem + Lay::G_QF);
  uint16_t* gKr = reinterpret_cast<uint16_t*>(smem + Lay::G_KR);
  uint16_t* gKrLo = reinterpret_cast<uint16_t*>(smem + Lay::G_KRLO);
  uint16_t* gQfLo = reinterpret_cast<uint16_t*>(smem + Lay::G_QFLO);
  uint16_t* gKb = reinterpret_cast<uint16_t*>(smem + Lay::G_KB);
  uint16_t* pKt = reinterpret_cast<uint16_t*>(smem + Lay::P_KT);
  uint16_t* pQt = reinterpret_cast<uint16_t*>(smem + Lay::P_QT);
  uint16_t* pKhT = reinterpret_cast<uint16_t*>(smem + Lay::P_KHT);
  uint16_t* pM = reinterpret_cast<uint16_t*>(smem + Lay::P_M);
  uint16_t* pN = reinterpret_cast<uint16_t*>(smem + Lay::P_N);
  uint16_t* sLb = reinterpret_cast<uint16_t*>(smem + Lay::S_LB);
  uint16_t* sTaT = reinterpret_cast<uint16_t*>(smem + Lay::S_TAT);
  uint16_t* sTbR = reinterpret_cast<uint16_t*>(smem + Lay::S_TBR);
  uint16_t* sT22T = reinterpret_cast<uint16_t*>(smem + Lay::S_T22T);
  uint16_t* sT11R = reinterpret_cast<uint16_t*>(smem + Lay::S_T11R);
  uint16_t* dUhi = reinterpret_cast<uint16_t*>(smem + Lay::D_UHI);
  uint16_t* dUlo = reinterpret_cast<uint16_t*>(smem + Lay::D_ULO);
  uint16_t* mY = reinterpret_cast<uint16_t*>(smem + Lay::D_Y);
  uint16_t* mV = reinterpret_cast<uint16_t*>(smem + Lay::A_V);
  float* mBeta = reinterpret_cast<float*>(smem + Lay::A_BETA);
  float* mGam = reinterpret_cast<float*>(smem + Lay::A_GAM);
  float* mBd = reinterpret_cast<float*>(smem + Lay::A_BD);
  float* mHalf = reinterpret_cast<float*>(smem + Lay::D_HALF);
  float* sLdT = reinterpret_cast<float*>(smem + Lay::A_LDT);
  uint16_t* oStg = reinterpret_cast<uint16_t*>(smem + Lay::A_OSTG);
  uint16_t* dST = reinterpret_cast<uint16_t*>(smem + Lay::A_ST);
  float* mMaxS = reinterpret_cast<float*>(smem + Lay::A_MAX);
  float* mMaxV = mMaxS + 8;

  // ---- state: wave w owns rows d in [16w, 16w+16), all VW columns ------------
  // S[nt][e] = S[16w + 4lg + e][col0 + 16nt + lr]
  f32x4 S[NTILE];
  const size_t state_base = (size_t)pair * DK * DVT;
  {
    const int lr = l & 15, lg = l >> 4;
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 16 * w + 4 * lg + e;
        const int j = col0 + 16 * nt + lr;
        const size_t i = state_base + (size_t)d * DVT + j;
        S[nt][e] = !a.s0 ? 0.f
                         : a.state_bf16 ? bf2f(reinterpret_cast<const uint16_t*>(a.s0)[i]) : a.s0[i];
      }
    // fp16 copy of the state, transposed, as the B operand of the next
    // segment (2^s S with s = 0 here; the first segment's scale check
    // rewrites it when s changes)
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt)
      *reinterpret_cast<uint2*>(dST + (16 * nt + lr) * KP + 16 * w + 4 * lg) =
          make_uint2(pack2h(S[nt][0], S[nt][1]), pack2h(S[nt][2], S[nt][3]));
  }
  int sexp = 0;   // the workgroup's operand scale exponent: S holds 2^sexp times the state
  // largest |2^s S| over this wave's rows, published for the scale check
  auto publish_state_max = [&]() {
    float mx = 0.f;
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(S[nt][e]));
    mx = wave_max_nonneg(mx);
    if (l == 0) mMaxS[w] = mx;
  };
  publish_state_max();

  // state store into dst at element offset e0 (fp32, or bf16 rounded to
  // nearest even when the states are bf16)
  auto export_state = [&](float* dst, size_t e0) {
    const int lr = l & 15, lg = l >> 4;
    const float unscale = pow2f(-sexp);
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 16 * w + 4 * lg + e;
        const int j = col0 + 16 * nt + lr;
        const size_t i = e0 + state_base + (size_t)d * DVT + j;
        if (a.state_bf16)
          reinterpret_cast<uint16_t*>(dst)[i] = (uint16_t)pack2(S[nt][e] * unscale, 0.f);
        else
          dst[i] = S[nt][e] * unscale;
      }
  };

  // checkpoint c of this sequence (layout [N, C, H, K, V]): element offset
  auto ckpt_slot = [&](int c) { return ((size_t)n * (a.ckpt_per_seq - 1) + c) * (size_t)H * DK * DVT; };
  for_each_honoured(ck, [&](int c, int p) {
    if (p == 0) export_state(a.ckpt, ckpt_slot(c));
  });

  // elementwise role: block ib, rows 16ib + 8hb .. +7, channels d0, d0+1
  const int ib = w >> 1;
  const int hb = w & 1;
  // row-block role in the recurrence: block rb, column tiles [nt0, nt0 + NTW)
  const int rb = w & 3;
  const int nt0 = NTILE >= 2 ? (w >> 2) * NTW : 0;
  const bool rb_active = NTILE >= 2 || w < 4;
  const bool v_thread = tid < 64 * PER_ROW;

  // Segment geometry: at most 64 tokens, never crossing a multiple of 64 from
  // the sequence start, split at the checkpoint offset.  The segment's c
  // tokens sit in the LAST c rows of the 64-row tile (rows before `off` are
  // zero and contribute nothing), so its final 16 tokens are always tile rows
  // 48..63, the rows whose K exp(G_end - G) carries a lo part.  Tile row r
  // holds token tok0 + r.
  auto seg_end_of = [&](int64_t p0) { return (int64_t)next_boundary(ck, (int)p0); };
  const size_t row_stride = (size_t)H * DK;   // elements between consecutive tokens
  auto load_segment = [&](int64_t p0, SegmentLoads& L) {
    const int d0 = 2 * l;
    const int vr = tid / PER_ROW, vc8 = tid % PER_ROW;
    const int off = CH - (int)(seg_end_of(p0) - p0);
    const int64_t t0 = bos + p0 - off;
    const int r0 = 16 * ib + 8 * hb;
    // rows before `off` belong to the previous segment or sequence: zero
    const size_t e0 = ((size_t)(t0 + r0) * H + h) * DK + d0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (r0 + e >= off) {
        const size_t o = e0 + (size_t)e * row_stride;
        L.g[e] = *reinterpret_cast<const float2*>(a.g + o);
        L.k[e] = *reinterpret_cast<const uint32_t*>(a.k + o);
        L.q[e] = *reinterpret_cast<const uint32_t*>(a.q + o);
      } else {
        L.g[e] = make_float2(0.f, 0.f);
        L.k[e] = 0u;
        L.q[e] = 0u;
      }
    }
    L.v = make_uint4(0, 0, 0, 0);
    if (v_thread && vr >= off)
      L.v = *reinterpret_cast<const uint4*>(a.v + ((size_t)(t0 + vr) * H + h) * DVT + col0 + 8 * vc8);
    L.bvalid = tid < 64 && tid >= off;
    L.beta = L.bvalid ? a.beta[(size_t)(t0 + tid) * H + h] : 0.f;
  };
  // Gate factors of a segment, first half: exp(g), prefix (Ef) and suffix (Eb)
  // products inside this thread's half block, the half-block product to LDS,
  // and the segment's V slice and beta to LDS.  Second half (after a barrier):
  // combine with the other half block and publish the block decays.
  float Ef[8][2], Eb[8][2];
  auto gate_factors_1 = [&](const SegmentLoads& L) {
    const int d0 = 2 * l;
    const int vr = tid / PER_ROW, vc8 = tid % PER_ROW;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      float ex[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ex[e] = __expf(ch ? L.g[e].y : L.g[e].x);
      float run = 1.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) { run *= ex[e]; Ef[e][ch] = run; }
      run = 1.f;
#pragma unroll
      for (int e = 7; e >= 0; --e) { Eb[e][ch] = run; run *= ex[e]; }
    }
    *reinterpret_cast<float2*>(mHalf + (2 * ib + hb) * DK + d0) = make_float2(Ef[7][0], Ef[7][1]);
    (void)vr; (void)vc8;
  };
  auto stage_v_beta = [&](const SegmentLoads& L) {
    const int vr = tid / PER_ROW, vc8 = tid % PER_ROW;
    if (v_thread) *reinterpret_cast<uint4*>(mV + vr * Lay::VP + 8 * vc8) = L.v;
    // largest |V| of the wave's share (bf16 bits of non-negative values order
    // as the values; rows outside the segment were loaded as zero)
    {
      const uint32_t wv[4] = {L.v.x, L.v.y, L.v.z, L.v.w};
      uint32_t vm = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) vm = max(vm, max(wv[e] & 0x7fffu, (wv[e] >> 16) & 0x7fffu));
      const float mv = wave_max_nonneg(v_thread ? __uint_as_float(vm << 16) : 0.f);
      if (l == 0) mMaxV[w] = mv;
    }
    // input prologue: beta given as a logit (rows outside the segment stay 0)
    if (tid < 64) mBeta[tid] = ((a.prologue & 2) && L.bvalid) ? 1.f / (1.f + __expf(-L.beta)) : L.beta;
  };
  auto gate_factors_2 = [&]() {
    const int d0 = 2 * l;
    const float2 other = *reinterpret_cast<const float2*>(mHalf + (2 * ib + (1 - hb)) * DK + d0);
    if (hb == 0)
      *reinterpret_cast<float2*>(mBd + ib * DK + d0) =
          make_float2(Ef[7][0] * other.x, Ef[7][1] * other.y);
    // Ef_r = exp(G_r - G_{16ib-1}), Eb_r = exp(G_{16ib+15} - G_r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (hb == 1) { Ef[e][0] *= other.x; Ef[e][1] *= other.y; }
      else { Eb[e][0] *= other.x; Eb[e][1] *= other.y; }
    }
  };
  // store the staged output tile of a finished segment (rows >= off_prev,
  // token tok0_prev + row) with 16-byte stores
  auto flush_out = [&](int off_prev, int64_t tok0_prev) {
    const int vr = tid / PER_ROW, vc8 = tid % PER_ROW;
    if (v_thread && vr >= off_prev)
      *reinterpret_cast<uint4*>(a.out + ((size_t)(tok0_prev + vr) * H + h) * DVT + col0 + 8 * vc8) =
          *reinterpret_cast<const uint4*>(oStg + vr * Lay::VP + 8 * vc8);
  };
  int pending_off = -1;        // staged output of the previous segment, if any
  int64_t pending_tok0 = 0;

  SegmentLoads ld;
  int64_t pos = 0;
  if (pos < len) {
    load_segment(pos, ld);
    gate_factors_1(ld);
    stage_v_beta(ld);
    lds_barrier();
    gate_factors_2();
    lds_barrier();
  }
  while (pos < len) {
    const int64_t seg_end = seg_end_of(pos);
    const int c = (int)(seg_end - pos);
    const int off = CH - c;
    const int64_t tok0 = bos + pos - off;
    const bool has_next = seg_end < len;
    // per-iteration copies of the lane coordinates: keeps the compiler from
    // hoisting every derived LDS address out of the segment loop
    int lane_it = l;
    asm volatile("" : "+v"(lane_it));
    const int lr = lane_it & 15, lg = lane_it >> 4, d0 = 2 * lane_it;

    // Operand scale check: the largest |2^s S| (published after the previous
    // state update) and |V| of this segment (published by its staging).  A
    // new s multiplies the state by the change (exact) and rewrites its fp16
    // copy; the barriers before phase D publish that.
    {
      float bs = 0.f, bv = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bs = fmaxf(bs, mMaxS[i]);
        bv = fmaxf(bv, mMaxV[i]);
      }
      const int nexp = rescale_exponent(fmaxf(bs, bv * pow2f(sexp)), sexp);
      if (nexp != sexp) {
        const int dexp = nexp - sexp;
        sexp = nexp;
#pragma unroll
        for (int nt = 0; nt < NTILE; ++nt) {
#pragma unroll
          for (int e = 0; e < 4; ++e) S[nt][e] = __builtin_ldexpf(S[nt][e], dexp);
          *reinterpret_cast<uint2*>(dST + (16 * nt + lr) * KP + 16 * w + 4 * lg) =
              make_uint2(pack2h(S[nt][0], S[nt][1]), pack2h(S[nt][2], S[nt][3]));
        }
      }
    }

    // ================= phase A: gate-product operands =========================
    // (this segment's Ef, Eb, block decays, V and beta were prepared during the
    // previous segment's recurrence)
    float cref[2], Pend[2], rbd[2];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      float bd[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) bd[m] = mBd[m * DK + d0 + ch];
      float cr = 1.f, pe = 1.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m < ib) cr *= bd[m];
        if (m > ib) pe *= bd[m];
      }
      cref[ch] = cr; Pend[ch] = pe;
      rbd[ch] = __builtin_amdgcn_rcpf(bd[ib]);   // ~1 ulp; feeds hi+lo operands
      if (ib == 0 && hb == 0) mGam[d0 + ch] = bd[0] * bd[1] * bd[2] * bd[3];
    }
    // kept for the prepared operands after the gate products: -K exp(G) and
    // Q exp(G) as fp16 pairs, K exp(G_end - G) in fp32
    uint32_t kfp[8], qfp[8];
    float kb[8][2];
    // input prologue: q and k of each row divided by their L2 norms over the
    // 128 channels (the row's channels sit two per lane across this wave; a
    // zero row stays zero)
    float ink[8], inq[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ink[e] = 1.f;
      inq[e] = 1.f;
    }
    if (a.prologue & 1) {
      float sk[8], sq[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float k0 = lo_of(ld.k[e]), k1 = hi_of(ld.k[e]);
        const float q0 = lo_of(ld.q[e]), q1 = hi_of(ld.q[e]);
        sk[e] = k0 * k0 + k1 * k1;
        sq[e] = q0 * q0 + q1 * q1;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sk[e] += __shfl_xor(sk[e], o, 64);
          sq[e] += __shfl_xor(sq[e], o, 64);
        }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ink[e] = sk[e] > 0.f ? 1.f / __builtin_sqrtf(sk[e]) : 0.f;
        inq[e] = sq[e] > 0.f ? 1.f / __builtin_sqrtf(sq[e]) : 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int rl = 8 * hb + e;        // row within the block
      const int r = 16 * ib + rl;
      // k, q of this segment are still in the prefetch registers (the next
      // prefetch is issued only after this phase)
      const float kk[2] = {lo_of(ld.k[e]) * ink[e], hi_of(ld.k[e]) * ink[e]};
      const float qq[2] = {lo_of(ld.q[e]) * inq[e], hi_of(ld.q[e]) * inq[e]};
      float kf[2], qf[2];
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        kf[ch] = kk[ch] * Ef[e][ch];
        qf[ch] = qq[ch] * Ef[e][ch];
        kb[e][ch] = kk[ch] * Eb[e][ch];
      }
      uint32_t hi, lo;
      split2(kf[0], kf[1], hi, lo);
      *reinterpret_cast<uint32_t*>(gKf + r * KP + d0) = hi;
      *reinterpret_cast<uint32_t*>(gKfLo + r * KP + d0) = lo;
      split2(qf[0], qf[1], hi, lo);
      *reinterpret_cast<uint32_t*>(gQf + r * KP + d0) = hi;
      *reinterpret_cast<uint32_t*>(gQfLo + r * KP + d0) = lo;
      // K exp(G) = K exp(G - G_blockstart) cref, Q likewise (<= 1)
      kfp[e] = pack2h(-kf[0] * cref[0], -kf[1] * cref[1]);
      qfp[e] = pack2h(qf[0] * cref[0], qf[1] * cref[1]);
      split2(kb[e][0] * rbd[0], kb[e][1] * rbd[1], hi, lo);
      *reinterpret_cast<uint32_t*>(gKr + r * KP + d0) = hi;
      *reinterpret_cast<uint32_t*>(gKrLo + r * KP + d0) = lo;
      if (ib <= 2) *reinterpret_cast<uint32_t*>(gKb + r * KP + d0) = pack2h(kb[e][0], kb[e][1]);
    }
    lds_barrier();  // (3) gate operands ready
    if (pending_off >= 0) flush_out(pending_off, pending_tok0);

    // ================= phase B: gated K K^T and Q K^T blocks ==================
    // Waves 0-3 take the diagonal block (w, w) and invert it right away (C1);
    // waves 4-7 take the off-diagonal blocks.
    float tcol[16];                      // column lr of T_ww = (I + L_ww)^-1 (waves 0-3)
    f32x4 accA[2], accM[2];
    int ui[2], uj[2], nunits = 0;
    if (w < 4) {
      ui[0] = w; uj[0] = w; nunits = 1;
    } else {
      // (1,0),(3,2) | (2,0),(3,1) | (2,1) | (3,0)
      const int i0 = w == 4 ? 1 : (w == 5 ? 2 : (w == 6 ? 2 : 3));
      const int j0 = w == 4 ? 0 : (w == 5 ? 0 : (w == 6 ? 1 : 0));
      ui[0] = i0; uj[0] = j0; nunits = 1;
      if (w == 4) { ui[1] = 3; uj[1] = 2; nunits = 2; }
      if (w == 5) { ui[1] = 3; uj[1] = 1; nunits = 2; }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      accA[s] = f32x4{0.f, 0.f, 0.f, 0.f};
      accM[s] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s < nunits) {
        const int i = ui[s], j = uj[s];
        const uint16_t* left_k = gKf + (16 * i + lr) * KP;
        const uint16_t* left_kl = gKfLo + (16 * i + lr) * KP;
        const uint16_t* left_q = gQf + (16 * i + lr) * KP;
        const uint16_t* left_ql = gQfLo + (16 * i + lr) * KP;
        // right operand: the diagonal block's own; left of it k exp(G_blockend(j)
        // - G_s) of block j, times W = the decays of the blocks between j and i
        // (bd_1 for (2,0), bd_2 for (3,1), bd_1 bd_2 for (3,0))
        const uint16_t* right = i == j ? gKr + (16 * i + lr) * KP : gKb + (16 * j + lr) * KP;
        const int wsel = (i == j || j == i - 1) ? 0 : (i == 2 ? 1 : (j == 1 ? 2 : 3));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int off8 = 32 * ks + 8 * lg;
          if (i == j) {
            // diagonal block: factors from exp(-80) to exp(80), bf16; A with
            // hi + lo on both sides, M (the read-out only) with hi + lo on the right
            const bf16x8 kh = lds8(left_k + off8), kl = lds8(left_kl + off8);
            const bf16x8 bk = lds8(right + off8);
            const bf16x8 bkl = lds8(gKrLo + (16 * i + lr) * KP + off8);
            accA[s] = mfma(kh, bk, accA[s]);
            accA[s] = mfma(kh, bkl, accA[s]);
            accA[s] = mfma(kl, bk, accA[s]);
            const bf16x8 qh = lds8(left_q + off8), ql = lds8(left_ql + off8);
            accM[s] = mfma(qh, bk, accM[s]);
            accM[s] = mfma(qh, bkl, accM[s]);
            accM[s] = mfma(ql, bk, accM[s]);
          } else {
            // left of the diagonal block: both factors <= 1, fp16
            f16x8 bk = lds8h(right + off8);
            if (wsel) {
              float wf[8];
              const float* b1 = mBd + DK + off8;
              const float* b2 = mBd + 2 * DK + off8;
#pragma unroll
              for (int e = 0; e < 8; ++e)
                wf[e] = wsel == 1 ? b1[e] : (wsel == 2 ? b2[e] : b1[e] * b2[e]);
              const uint4 u = __builtin_bit_cast(uint4, bk);
              const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
              uint32_t o[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                o[e] = pack2h(h_lo(uw[e]) * wf[2 * e], h_hi(uw[e]) * wf[2 * e + 1]);
              bk = __builtin_bit_cast(f16x8, make_uint4(o[0], o[1], o[2], o[3]));
            }
            accA[s] = mfma(lds8_bf_to_h(left_k + off8, left_kl + off8), bk, accA[s]);
            accM[s] = mfma(lds8_bf_to_h(left_q + off8, left_ql + off8), bk, accM[s]);
          }
        }
      }
    }
    if (w < 4) {
      // C1: L_ww = diag(beta) A_ww (strictly lower), transposed to LDS (this
      // wave's own block), then T_ww by column-wise forward substitution in
      // fp32, lane column lr (all four lane groups compute the same column)
      {
        float lv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * w + 4 * lg + e;
          lv[e] = lr < 4 * lg + e ? mBeta[r] * accA[0][e] : 0.f;
        }
        *reinterpret_cast<float4*>(sLdT + (16 * w + lr) * LDP + 4 * lg) =
            make_float4(lv[0], lv[1], lv[2], lv[3]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int r = 0; r < 16; ++r) tcol[r] = r == lr ? 1.f : 0.f;
      const float* LT = sLdT + (16 * w) * LDP;   // LT[s][r] = L[r][s]
#pragma unroll
      for (int s2 = 0; s2 < 15; ++s2) {
        float lcol[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v4 = *reinterpret_cast<const float4*>(LT + s2 * LDP + 4 * q4);
          lcol[4 * q4] = v4.x; lcol[4 * q4 + 1] = v4.y; lcol[4 * q4 + 2] = v4.z; lcol[4 * q4 + 3] = v4.w;
        }
#pragma unroll
        for (int r = s2 + 1; r < 16; ++r) tcol[r] = fmaf(-lcol[r], tcol[s2], tcol[r]);
      }
    }
    lds_barrier();  // (4) gate operands consumed; region reused below

    // L off-diagonal blocks (fp16, for the matrix-core merges) and M (fp16,
    // lower incl. diagonal)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < nunits) {
        const int i = ui[s], j = uj[s];
        const int sc = 16 * j + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * i + 4 * lg + e;
          pM[r * RP + sc] = f2h(sc <= r ? accM[s][e] : 0.f);
          if (i != j) sLb[r * RP + sc] = f2h(mBeta[r] * accA[s][e]);
        }
      }
    }
    // zero the upper blocks of M and N that the M U and N Y products read: (0,1), (2,3)
    {
      const int blk = tid >> 8, rr = (tid >> 4) & 15, cc = tid & 15;
      const int r = blk == 0 ? rr : 32 + rr, sc = blk == 0 ? 16 + cc : 48 + cc;
      pM[r * RP + sc] = 0;
      pN[r * RP + sc] = 0;
    }
    // T_ww outputs of the diagonal inversions
    if (w < 4 && lg == 0) {
      const int cc = lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) pN[(16 * w + r) * RP + 16 * w + cc] = f2h(r > cc ? tcol[r] : 0.f);
      uint32_t tp[8];
#pragma unroll
      for (int r2 = 0; r2 < 8; ++r2) tp[r2] = pack2h(tcol[2 * r2], tcol[2 * r2 + 1]);
      const uint4 t_lo = make_uint4(tp[0], tp[1], tp[2], tp[3]);
      const uint4 t_hi = make_uint4(tp[4], tp[5], tp[6], tp[7]);
      const uint4 z = make_uint4(0, 0, 0, 0);
      if (w == 0) {          // Ta^T[0:16][0:16] = T00^T
        *reinterpret_cast<uint4*>(sTaT + cc * TP) = t_lo;
        *reinterpret_cast<uint4*>(sTaT + cc * TP + 8) = t_hi;
      } else if (w == 1) {   // Ta^T[16:32][16:32] = T11^T, Ta^T[16:32][0:16] = 0; T11 row-major
        *reinterpret_cast<uint4*>(sTaT + (16 + cc) * TP + 16) = t_lo;
        *reinterpret_cast<uint4*>(sTaT + (16 + cc) * TP + 24) = t_hi;
        *reinterpret_cast<uint4*>(sTaT + (16 + cc) * TP) = z;
        *reinterpret_cast<uint4*>(sTaT + (16 + cc) * TP + 8) = z;
#pragma unroll
        for (int r = 0; r < 16; ++r) sT11R[r * SP + cc] = (uint16_t)(tp[r >> 1] >> (16 * (r & 1)));
      } else if (w == 2) {   // T22^T; Tb[0:16][0:16] = T22 row-major, Tb[0:16][16:32] = 0
        *reinterpret_cast<uint4*>(sT22T + cc * SP) = t_lo;
        *reinterpret_cast<uint4*>(sT22T + cc * SP + 8) = t_hi;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sTbR[r * TP + cc] = (uint16_t)(tp[r >> 1] >> (16 * (r & 1)));
          sTbR[r * TP + 16 + cc] = 0;
        }
      } else {               // Tb[16:32][16:32] = T33 row-major
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sTbR[(16 + r) * TP + 16 + cc] = (uint16_t)(tp[r >> 1] >> (16 * (r & 1)));
      }
    }
    // prepared operands: -K exp(G), Q exp(G), K exp(G_end - G) (transposed)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 16 * ib + 8 * hb + e;
      *reinterpret_cast<uint32_t*>(pKt + r * KP + d0) = kfp[e];
      *reinterpret_cast<uint32_t*>(pQt + r * KP + d0) = qfp[e];
    }
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      uint32_t hp[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        hp[e2] = pack2h(kb[2 * e2][ch] * Pend[ch], kb[2 * e2 + 1][ch] * Pend[ch]);
      *reinterpret_cast<uint4*>(pKhT + (d0 + ch) * RP + 16 * ib + 8 * hb) =
          make_uint4(hp[0], hp[1], hp[2], hp[3]);
    }
    // prefetch the next segment's inputs; they land during phases C and D
    if (has_next) load_segment(seg_end, ld);
    lds_barrier();  // (5) L, M, T_ii and prepared operands ready

    // ================= phase C: merges of N = (I + L)^-1 - I ==================
    // With Ta = T[0:32,0:32], Tb = T[32:64,32:64]:
    //   T10 = -T11 (L10 T00),  T32 = -T33 (L32 T22),  T[32:64,0:32] = -Tb (L[32:64,0:32] Ta).
    // A product's fp32 accumulator feeds the next product as its B operand
    // directly: lane group lg holds rows 4lg..4lg+3 of each 16-row tile, so
    // the reduction index of the second product is permuted the same way in
    // its A operand (the order of terms in a matrix product is free).
    const f16x8 z8 = zero8h();
    auto acc_to_b4 = [&](const f32x4& c4) {   // 4 rows -> k-slots 0..3, zeros 4..7
      const uint4 u = make_uint4(pack2h(c4[0], c4[1]), pack2h(c4[2], c4[3]), 0u, 0u);
      return __builtin_bit_cast(f16x8, u);
    };
    auto acc_to_b8 = [&](const f32x4& c0, const f32x4& c1) {   // two tiles -> 8 k-slots
      const uint4 u = make_uint4(pack2h(c0[0], c0[1]), pack2h(c0[2], c0[3]), pack2h(c1[0], c1[1]),
                                 pack2h(c1[2], c1[3]));
      return __builtin_bit_cast(f16x8, u);
    };
    auto lds4_z4 = [&](const uint16_t* p) {   // 4 fp16 from LDS, then 4 zeros
      const uint2 v2 = *reinterpret_cast<const uint2*>(p);
      return __builtin_bit_cast(f16x8, make_uint4(v2.x, v2.y, 0u, 0u));
    };
    auto lds4_4 = [&](const uint16_t* p, const uint16_t* q2) {   // 4 + 4 fp16 from two places
      const uint2 v0 = *reinterpret_cast<const uint2*>(p);
      const uint2 v1 = *reinterpret_cast<const uint2*>(q2);
      return __builtin_bit_cast(f16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
    };
    if (w < 2) {
      // w 0: T10 = -T11 (L10 T00);  w 1: T32 = -T33 (L32 T22)   (16-deep products:
      // lane groups 2, 3 feed zeros to the first)
      const uint16_t* A1 = w == 0 ? sLb + (16 + lr) * RP : sLb + (48 + lr) * RP + 32;
      const uint16_t* B1 = w == 0 ? sTaT + lr * TP : sT22T + lr * SP;
      f32x4 P = {0.f, 0.f, 0.f, 0.f};
      P = mfma(lg < 2 ? lds8h(A1 + 8 * lg) : z8, lg < 2 ? lds8h(B1 + 8 * lg) : z8, P);
      const uint16_t* A2 = w == 0 ? sT11R + lr * SP + 4 * lg : sTbR + (16 + lr) * TP + 16 + 4 * lg;
      f32x4 Tn = {0.f, 0.f, 0.f, 0.f};
      Tn = mfma(lds4_z4(A2), acc_to_b4(P), Tn);
      uint16_t tv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) tv[e] = f2h(-Tn[e]);
      if (w == 0) {
        // Ta^T[n][16 + m] = T10[m][n]; N block (1,0)
        *reinterpret_cast<uint2*>(sTaT + lr * TP + 16 + 4 * lg) =
            make_uint2(pack2h(-Tn[0], -Tn[1]), pack2h(-Tn[2], -Tn[3]));
#pragma unroll
        for (int e = 0; e < 4; ++e) pN[(16 + 4 * lg + e) * RP + lr] = tv[e];
      } else {
        // Tb[16 + m][n] = T32[m][n]; N block (3,2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sTbR[(16 + 4 * lg + e) * TP + lr] = tv[e];
          pN[(48 + 4 * lg + e) * RP + 32 + lr] = tv[e];
        }
      }
    }
    lds_barrier();
    if (w < 2) {
      // column block ni = w of T[32:64, 0:32]: Q = L[32:64,0:32] Ta[:, ni] (two
      // 16-row tiles), then -Tb Q
      const int ni = w;
      f32x4 Q0 = {0.f, 0.f, 0.f, 0.f}, Q1 = {0.f, 0.f, 0.f, 0.f};
      const f16x8 bta = lds8h(sTaT + (16 * ni + lr) * TP + 8 * lg);
      Q0 = mfma(lds8h(sLb + (32 + lr) * RP + 8 * lg), bta, Q0);
      Q1 = mfma(lds8h(sLb + (48 + lr) * RP + 8 * lg), bta, Q1);
      const f16x8 bq = acc_to_b8(Q0, Q1);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const uint16_t* Ar = sTbR + (16 * mi + lr) * TP;
        f32x4 Tn = {0.f, 0.f, 0.f, 0.f};
        Tn = mfma(lds4_4(Ar + 4 * lg, Ar + 16 + 4 * lg), bq, Tn);
#pragma unroll
        for (int e = 0; e < 4; ++e) pN[(32 + 16 * mi + 4 * lg + e) * RP + 16 * ni + lr] = f2h(-Tn[e]);
      }
    }
    lds_barrier();  // (C) solve done; solve scratch free

    // ================= phase D: the chunk recurrence ==========================
    // dST holds 2^s times the incoming state in fp16.  2^s X = 2^s V - K exp(G)
    // (2^s S), 2^s Y = beta 2^s X and 2^s P = Q exp(G) (2^s S) for the rows of
    // block rb.
    const float sig = pow2f(sexp);
    f32x4 Y[NTW], PO[NTW];
    if (rb_active) {
#pragma unroll
      for (int t2 = 0; t2 < NTW; ++t2) {
        const int nt = nt0 + t2;
        f32x4 acc, po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[e] = bf2f(mV[(16 * rb + 4 * lg + e) * Lay::VP + 16 * nt + lr]) * sig;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int o8 = 32 * ks + 8 * lg;
          const f16x8 bs = lds8h(dST + (16 * nt + lr) * KP + o8);
          acc = mfma(lds8h(pKt + (16 * rb + lr) * KP + o8), bs, acc);
          po = mfma(lds8h(pQt + (16 * rb + lr) * KP + o8), bs, po);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= mBeta[16 * rb + 4 * lg + e];
        Y[t2] = acc;
        PO[t2] = po;
        *reinterpret_cast<uint2*>(mY + (16 * nt + lr) * RP + 16 * rb + 4 * lg) =
            make_uint2(pack2h(acc[0], acc[1]), pack2h(acc[2], acc[3]));
      }
    }
    // next segment's gate factors, first half (its inputs were prefetched)
    if (has_next) gate_factors_1(ld);
    lds_barrier();  // (D1) Y and the next segment's half-block products ready

    // U = Y + N Y
    const int nks = rb >= 2 ? 2 : 1;   // k-steps of 32 rows covering rows < 16(rb+1)
    if (rb_active) {
#pragma unroll
      for (int t2 = 0; t2 < NTW; ++t2) {
        const int nt = nt0 + t2;
        f32x4 acc = Y[t2];
        for (int ks = 0; ks < nks; ++ks) {
          const int o8 = 32 * ks + 8 * lg;
          acc = mfma(lds8h(pN + (16 * rb + lr) * RP + o8), lds8h(mY + (16 * nt + lr) * RP + o8), acc);
        }
        uint2 ph, pl;
        split2h(acc[0], acc[1], ph.x, pl.x);
        split2h(acc[2], acc[3], ph.y, pl.y);
        *reinterpret_cast<uint2*>(dUhi + (16 * nt + lr) * RP + 16 * rb + 4 * lg) = ph;
        *reinterpret_cast<uint2*>(dUlo + (16 * nt + lr) * RP + 16 * rb + 4 * lg) = pl;
      }
    }
    // next segment: second half of the gate factors; its V slice and beta
    if (has_next) {
      gate_factors_2();
      stage_v_beta(ld);
    }
    lds_barrier();  // (D2) U ready; nobody reads dST, mV, mBeta again in this segment

    // O = scale 2^-s (2^s P + M 2^s U)   (rows of block rb), staged for 16-byte stores
    if (rb_active) {
      const float osc = a.scale * pow2f(-sexp);
#pragma unroll
      for (int t2 = 0; t2 < NTW; ++t2) {
        const int nt = nt0 + t2;
        f32x4 acc = PO[t2];
        for (int ks = 0; ks < nks; ++ks) {
          const int o8 = 32 * ks + 8 * lg;
          acc = mfma(lds8h(pM + (16 * rb + lr) * RP + o8), lds8h(dUhi + (16 * nt + lr) * RP + o8), acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          oStg[(16 * rb + 4 * lg + e) * Lay::VP + 16 * nt + lr] = f2bf(acc[e] * osc);
      }
    }

    // 2^s S <- diag(exp(G_end)) 2^s S + (K exp(G_end - G))^T 2^s U  (rows
    // 16w..16w+15, U as hi + lo), then its fp16 copy for the next segment's B
    // operand and this wave's largest |2^s S| for the next scale check
    {
      const int drow = 16 * w;
      float gam[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) gam[e] = mGam[drow + 4 * lg + e];
      f16x8 akh[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) akh[ks] = lds8h(pKhT + (drow + lr) * RP + 32 * ks + 8 * lg);
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt) {
        f32x4 acc = S[nt];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= gam[e];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int o8 = 32 * ks + 8 * lg;
          acc = mfma(akh[ks], lds8h(dUhi + (16 * nt + lr) * RP + o8), acc);
          acc = mfma(akh[ks], lds8h(dUlo + (16 * nt + lr) * RP + o8), acc);
        }
        S[nt] = acc;
        *reinterpret_cast<uint2*>(dST + (16 * nt + lr) * KP + 16 * w + 4 * lg) =
            make_uint2(pack2h(acc[0], acc[1]), pack2h(acc[2], acc[3]));
      }
      publish_state_max();
    }
    lds_barrier();  // (E) segment done: the gate-operand region is free again

    pending_off = off;
    pending_tok0 = tok0;
    for_each_honoured(ck, [&](int c, int p) {
      if (p > 0 && p == seg_end) export_state(a.ckpt, ckpt_slot(c));
    });
    pos = seg_end;
  }

  if (pending_off >= 0) flush_out(pending_off, pending_tok0);
  if (a.final_state) export_state(a.final_state, 0);
}

}  // namespace

template <int VW>
static hipError_t launch_fused_vw(const FusedArgs& a, hipStream_t stream) {
  constexpr int VSPLIT = DVT / VW;
  const int groups = (a.num_pairs + 7) / 8;
  const dim3 grid(groups * 8 * VSPLIT);
  hipLaunchKernelGGL(kda_fused_kernel<VW>, grid, dim3(NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fused(const FusedArgs& a, int vsplit, hipStream_t stream) {
  switch (vsplit) {
    case 2: return launch_fused_vw<64>(a, stream);
    case 4: return launch_fused_vw<32>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
