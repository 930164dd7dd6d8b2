// msd_device.hpp -- gfx950 device helpers shared by every MSD kernel.
//
// Method: the page "WeightQuantBatchMatmulExperiment 算子深度解析：A16W4 PerGroup
// 伪量化 MatMul 的 MSD 算法与双模板流水设计" (lpnh.cn/news/2294145), called the
// WQBMM-Exp page below.  §4.1 gives the eleven MSD formulas; §4.3 the int4
// storage (two per byte); the kernel there keeps the expansion factors as the
// fp32 literals 7.49f, 14.98f, 14.98f.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace wqbmm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Expansion factors (WQBMM-Exp page §4.1, fp32 as the page's kernel keeps them).
constexpr float kF1 = 7.49f;
constexpr float kF2 = 14.98f;

// Step-10 weights of the three levels, with the 1/16 that undoes the
// high-nibble int4 unpack (each weight enters the contraction as 16*w).
constexpr float kC1 = (float)(1.0 / (16.0 * (double)kF1));
constexpr float kC2 = (float)(1.0 / (16.0 * (double)(kF1 * kF2)));
constexpr float kC3 = (float)(1.0 / (16.0 * (double)(kF1 * kF2 * kF2)));

__device__ __forceinline__ float half_bits_to_float(uint32_t h16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)h16));
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));  // RNE
}

// Division by a group's A_max.  Step 2 divides tmp = 7.49*a by A_max with a
// correctly rounded fp32 divide.  Every element of a group shares the divisor,
// so its reciprocal is formed once: y = rcp(d) refined by one Newton step,
// y' = y + y*(1 - d*y).  Each quotient is then q0 = t*y', corrected once with
// the exact remainder: q = q0 + y'*(t - d*q0) (Markstein's final step; both
// corrections are single fused multiply-adds).  For the operands that occur
// here (d a positive fp16 value, t = rn(7.49*a) with |a| <= d an fp16 value)
// the result equals the correctly rounded t/d for every pair; a GPU test
// checks that exhaustively against the CPU oracle's division.
__device__ __forceinline__ float msd_recip(float d) {
  const float y = __builtin_amdgcn_rcpf(d);
  return __builtin_fmaf(__builtin_fmaf(-d, y, 1.0f), y, y);
}

__device__ __forceinline__ float msd_div(float t, float d, float y) {
  const float q0 = t * y;
  return __builtin_fmaf(__builtin_fmaf(-q0, d, t), y, q0);
}

// Round half to even is v_rndne_f32 (rintf).  For an integer-valued r with
// |r| < 2^22, u = r + kMagic (1.5*2^23) lands where the float spacing is 1,
// so the sum is exact and holds r in its low mantissa bits: its low byte is r
// as a two's-complement int8.
constexpr float kMagic = 12582912.0f;

// ---- WQBMM-Exp page §4.1 steps 1-8: the one decomposition every kernel uses
//
// Step 1 (A_max = rowMax(|A_group|)) is exact: the maximum is taken over the
// fp16 magnitudes' bit patterns as unsigned integers (for non-negative finite
// values the order of the patterns is the order of the values, and an integer
// max needs no NaN handling) and widened once.  A kernel takes the maximum of
// its lane-local elements with chunk_max_bits, reduces it over the lanes that
// share the group (group_max_bits, or a shuffle), and forms the divisor's
// reciprocal with msd_group_scale.  Steps 2-7 then run per element in
// msd_levels.  A zero group (A_max = 0, so every element is +-0) takes a zero
// reciprocal, which makes every quotient 0 and so every level 0, as the
// definition's guard requires.

// Largest fp16 magnitude bit pattern among the 8 values of a 16-byte chunk.
__device__ __forceinline__ uint32_t chunk_max_bits(const uint4 xv) {
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  const u16x2 m01 = __builtin_elementwise_max(__builtin_bit_cast(u16x2, xw[0] & 0x7fff7fffu),
                                              __builtin_bit_cast(u16x2, xw[1] & 0x7fff7fffu));
  const u16x2 m23 = __builtin_elementwise_max(__builtin_bit_cast(u16x2, xw[2] & 0x7fff7fffu),
                                              __builtin_bit_cast(u16x2, xw[3] & 0x7fff7fffu));
  const u16x2 mh = __builtin_elementwise_max(m01, m23);
  return max((uint32_t)mh.x, (uint32_t)mh.y);
}

// A_max (exact) and the refined reciprocal of step 2's divisor, from the
// group's largest magnitude bit pattern; rcp = 0 for a zero group.
__device__ __forceinline__ void msd_group_scale(uint32_t max_bits, float& amax, float& rcp) {
  amax = half_bits_to_float(max_bits);
  rcp = amax > 0.0f ? msd_recip(amax) : 0.0f;
}

// Steps 2-7 for one element (fp16 bit pattern h) of a group with maximum amax
// and reciprocal rcp: tmp1 = 7.49*a/A_max, A1 = round(tmp1), tmp2 =
// (tmp1-A1)*14.98, A2 = round(tmp2), tmp3 = (tmp2-A2)*14.98, A3 =
// round(tmp3).  Every operation is one IEEE fp32 rounding in this order (no
// contraction; tmp = 7.49*a is one fused multiply-add with a zero addend
// straight from the fp16 value: exact widening, one rounding of the product;
// the division is correctly rounded, see msd_div); round is half to even
// (rintf).  Out: the levels r_l = A_l as floats and the sums u_l = A_l +
// kMagic, whose low byte is A_l as int8 (a kernel uses either; the other is
// not computed).  |A_l| <= 7 follows from 7.49 < 7.5 and |residual| <= 0.5.
// (A level that rounds to zero from below is -0.0 in r_l; it has the same
// value, byte and contribution as +0.0.)
__device__ __forceinline__ void msd_levels(uint32_t h, float amax, float rcp, float (&u)[3],
                                           float (&r)[3]) {
#pragma clang fp contract(off)
  const _Float16 a = __builtin_bit_cast(_Float16, (uint16_t)h);
  const float t1 = msd_div(__builtin_fmaf((float)a, kF1, 0.0f), amax, rcp);
  r[0] = __builtin_rintf(t1);
  u[0] = r[0] + kMagic;
  const float t2 = (t1 - r[0]) * kF2;
  r[1] = __builtin_rintf(t2);
  u[1] = r[1] + kMagic;
  const float t3 = (t2 - r[1]) * kF2;
  r[2] = __builtin_rintf(t3);
  u[2] = r[2] + kMagic;
}

// Maximum over WIDTH (4, 8 or 16) consecutive, aligned lanes of non-negative
// float bit patterns, as unsigned integers, with DPP lane permutations (no
// LDS traffic): exchange within quads (xor 1, xor 2), then mirror within each
// half-row of 8 lanes, then within each row of 16.  max is exact, so the
// order does not matter.  Every lane of the wave must call it.
template <int WIDTH>
__device__ __forceinline__ uint32_t group_max_bits(uint32_t v) {
  static_assert(WIDTH == 4 || WIDTH == 8 || WIDTH == 16, "group of 4, 8 or 16 lanes");
  auto dpp = [](uint32_t x, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, decltype(ctrl)::value, 0xf, 0xf, false);
  };
  v = max(v, dpp(v, std::integral_constant<int, 0xB1>{}));    // lane ^ 1
  v = max(v, dpp(v, std::integral_constant<int, 0x4E>{}));    // lane ^ 2
  if constexpr (WIDTH >= 8) v = max(v, dpp(v, std::integral_constant<int, 0x141>{}));   // row_half_mirror
  if constexpr (WIDTH == 16) v = max(v, dpp(v, std::integral_constant<int, 0x140>{}));  // row_mirror
  return v;
}

// Low bytes of four dwords -> one dword (byte j from x_j): three v_perm_b32
// (selector 0x0c gives a zero byte).
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  const uint32_t p01 = __builtin_amdgcn_perm(x1, x0, 0x0c0c0400u);   // x0.b0 x1.b0 0 0
  const uint32_t p23 = __builtin_amdgcn_perm(x3, x2, 0x0c0c0400u);   // x2.b0 x3.b0 0 0
  return __builtin_amdgcn_perm(p23, p01, 0x05040100u);               // x0.b0 x1.b0 x2.b0 x3.b0
}

// Steps 1-8 for 8 consecutive elements of one row (one 16-byte fp16 chunk)
// whose group's GS elements are held by GS/8 consecutive, aligned lanes;
// every lane of the wave must call this (the max is a cross-lane reduction).
// Out: the 8 levels of each of A1..A3 packed as int8 bytes in two dwords
// each, and the group's A_max.
template <int GS>
__device__ __forceinline__ void msd_decompose8(const uint4 xv, uint32_t (&lv)[3][2], float& amax) {
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  float rcp;
  msd_group_scale(group_max_bits<GS / 8>(chunk_max_bits(xv)), amax, rcp);
  uint32_t u[3][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float uf[3], rf[3];
    msd_levels(i & 1 ? xw[i >> 1] >> 16 : xw[i >> 1] & 0xffffu, amax, rcp, uf, rf);
#pragma unroll
    for (int l = 0; l < 3; ++l) u[l][i] = __float_as_uint(uf[l]);
  }
#pragma unroll
  for (int l = 0; l < 3; ++l) {
    lv[l][0] = pack_low_bytes(u[l][0], u[l][1], u[l][2], u[l][3]);
    lv[l][1] = pack_low_bytes(u[l][4], u[l][5], u[l][6], u[l][7]);
  }
}

// ---- tiled int4 weights -> int8 MFMA operands ---------------------------------
//
// In the tiled weight format, byte j of a dword holds rows j (low nibble) and
// j+4 (high nibble) of one column.  lo16/hi16 isolate one nibble per byte in
// the byte's high half, i.e. the int8 value 16*w (exact; the 1/16 is folded
// into the step-10 weights kC1..kC3): lo16 gives rows 0..3, hi16 rows 4..7.

__device__ __forceinline__ uint32_t lo16(uint32_t e) { return (e << 4) & 0xF0F0F0F0u; }  // rows j, 16*w
__device__ __forceinline__ uint32_t hi16(uint32_t e) { return e & 0xF0F0F0F0u; }         // rows j+4, 16*w

// v_mfma_i32_16x16x64_i8: D[16][16] += A[16][64] . B[64][16] in int32.
// Lane l supplies row (l%16) of A and column (l%16) of B, 16 bytes each, for
// the k-block (l/16); within that block both operands use the same byte->k
// assignment, so any consistent ordering of the 64 k values is a valid
// contraction.  D: lane l holds column (l%16), rows 4*(l/16)+i in element i.
__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace wqbmm
