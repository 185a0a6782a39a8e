// Value-side quantizer steps on one 128-channel vector spread over 16 lanes
// (8 contiguous channels per lane), shared by the value kernel and the fused
// append kernel, so that both turn the same input into the same bytes.
//
// Quantizer definitions: ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity
// ...", method paragraph (clipped symmetric INT grid, RMS clip) and end-to-end
// paragraph (percentile-clipped affine grid); values are quantized as stored,
// their transform being folded into the weights (same summary, deployment
// paragraph).
#pragma once

#include <climits>

#include "device_common.h"
#include "internal.h"
#include "sort32.h"

namespace wushkv {

typedef uint32_t vu32x4 __attribute__((ext_vector_type(4)));

// The lane's 8 channels from its raw words: bf16, one 16-byte word group
// (channel 2e in the low half of word e); fp32, two.
template <bool F32IN>
__device__ __forceinline__ void unpack_vals(const vu32x4* p, float* x) {
  if constexpr (F32IN) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = __uint_as_float(p[0][e]);
      x[4 + e] = __uint_as_float(p[1][e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16lo_to_f32(p[0][e]);
      x[2 * e + 1] = bf16hi_to_f32(p[0][e]);
    }
  }
}

// The lane's part of the vector's sum of squares: the contiguous pairwise tree
// over its 8 channels.  dpp_sum16 then combines the 16 lanes' parts as the
// upper levels of the same tree.
__device__ __forceinline__ float lane_sumsq8(const float* x) {
  float q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = x[e] * x[e];
  return ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
}

// Per-vector constants of the symmetric code step from the fp16 step delta.
// 2 bits: the step itself (0: every code is 2).  3/4 bits: the step (+inf for
// a zero step) and its reciprocal (0 for a zero step, giving code L/2).
template <int BITS>
__device__ __forceinline__ float4 value_thresholds(float delta) {
  const float tp = delta == 0.0f ? __builtin_inff() : delta;  // +inf for a zero step
  float4 th;
  if constexpr (BITS == 2) {
    th.x = delta;
    th.y = th.z = th.w = 0.0f;
  } else {
    th.x = tp;
    th.y = delta == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(delta);
    th.z = th.w = 0.0f;
  }
  return th;
}

// 2-bit symmetric codes of 8 values, LSB first in the low 16 bits: code =
// [y > -step] + [y >= 0] + [y > step].  The high bit is [y >= 0], the sign bit
// inverted; the low bit is [y > step] for y >= 0 and [y > -step] for y < 0,
// the sign of m = (step - |y|) * y + 0 (one fma): for |y| != step the signs of
// (step - |y|) and y decide it, and at a tie |y| = step (and at y = +0) the
// exact product is a zero that the +0 makes +0 (bit clear: the even code).
// The bits are shifted in from the last value down (alignbit: w = 2w + bit 31
// of the operand).  y must not be -0; a zero step gives code 2 everywhere.
__device__ __forceinline__ uint32_t sym2_bits8(const float* y, float delta) {
  uint32_t w = 0;
#pragma unroll
  for (int e = 7; e >= 0; --e) {
    const float m = __builtin_fmaf(delta - __builtin_fabsf(y[e]), y[e], 0.0f);
    w = __builtin_amdgcn_alignbit(w, __float_as_uint(y[e]), 31);
    w = __builtin_amdgcn_alignbit(w, __float_as_uint(m), 31);
  }
  return delta == 0.0f ? 0xAAAAu : (w ^ 0xAAAAu);
}

// 2-bit symmetric codes of the lane's 8 channels from its raw words (delta:
// the step, th.x of value_thresholds<2>).  The values are unpacked exactly and
// a -0 becomes +0 (x + 0), so that a zero of either sign takes the even code 2.
template <bool F32IN>
__device__ __forceinline__ uint32_t value_codes2(const vu32x4* p, float delta) {
  float x[8];
  unpack_vals<F32IN>(p, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = x[e] + 0.0f;
  return sym2_bits8(x, delta);
}

// 3/4-bit symmetric codes of the lane's 8 channels, LSB first: fast path, and
// exact codes for lanes with a value within rounding error of a midpoint.
template <int BITS>
__device__ __forceinline__ uint32_t value_codes_sym(const float* x, float4 th) {
  uint32_t packed = 0;
  bool near = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) packed |= sym_code_fast<BITS>(x[e], th.y, near) << (BITS * e);
  near = near && th.y != 0.0f;
  if (__builtin_amdgcn_ballot_w64(near) != 0) {
    if (near) {
      packed = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) packed |= sym_code<BITS>(x[e], th.x, th.y) << (BITS * e);
      // keep the word 32 bits wide so code counts compile to compare + add-with-carry
      asm("" : "+v"(packed));
    }
  }
  return packed;
}

// v from the lane the DPP control CTRL names (within a row of 16 lanes).
template <int CTRL>
__device__ __forceinline__ int32_t dpp_i32(int32_t v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

// Percentile-clipped affine codes of the lane's 8 channels, group of 32
// channels = 4 consecutive lanes (a DPP quad); sh, zh are the group's fp16 step
// and zero.  GEN false: the two extremes at each end by IEEE totalOrder, merged
// by xor 1, 2 (kind 1); GEN true: each lane sorts its 8 keys, every lane of the
// quad gathers the quad's four sorted lists and merges them into the 32 sorted
// keys, and the order statistics are read off those (kind 2).
template <int BITS, bool GEN = false>
__device__ __forceinline__ uint32_t value_codes_affine(const float* x, const QuantArgs& qa, uint16_t& sh,
                                                       uint16_t& zh) {
  constexpr int L = 1 << BITS;
  float lo, hi;
  if constexpr (GEN) {
    int32_t k[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) k[e] = total_order_key(x[e]);
    bitonic_sort<8>(k);
    // quad_perm [r, r, r, r]: lane r of the quad, in every lane of the quad
    int32_t q0[8], q1[8], q2[8], q3[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      q0[e] = dpp_i32<0x00>(k[e]);
      q1[e] = dpp_i32<0x55>(k[e]);
      q2[e] = dpp_i32<0xAA>(k[e]);
      q3[e] = dpp_i32<0xFF>(k[e]);
    }
    int32_t m01[16], m23[16], srt[32];
    bitonic_merge<8>(q0, q1, m01);
    bitonic_merge<8>(q2, q3, m23);
    bitonic_merge<16>(m01, m23, srt);
    lo = percentile_sorted(srt, qa.lo_i, qa.g_lo, qa.lo_mode);
    hi = percentile_sorted(srt, qa.hi_i, qa.g_hi, qa.hi_mode);
  } else if (qa.lo_mode == 0 && qa.hi_mode == 0) {
    // Both percentiles interpolate (the 1st/99th): the extremes by float
    // minimum, maximum and median, merged over the quad by DPP (a zero of
    // either sign tied for an order statistic gives the same lo and hi, see
    // affine_runs).
    Extremes2 e = extremes2_init();
#pragma unroll
    for (int i = 0; i < 8; ++i) extremes2_add(e, x[i]);
    e = extremes2_merge(e, {dpp_f32<0xB1>(e.m1), dpp_f32<0xB1>(e.m2), dpp_f32<0xB1>(e.x1), dpp_f32<0xB1>(e.x2)});
    e = extremes2_merge(e, {dpp_f32<0x4E>(e.m1), dpp_f32<0x4E>(e.m2), dpp_f32<0x4E>(e.x1), dpp_f32<0x4E>(e.x2)});
    lo = __builtin_fmaf(qa.g_lo, e.m2 - e.m1, e.m1);
    hi = __builtin_fmaf(qa.g_hi, e.x1 - e.x2, e.x2);
  } else {
    // a percentile taken as an order statistic itself: IEEE totalOrder keys
    // (-0 below +0), as the oracle sorts
    int32_t mn1 = INT_MAX, mn2 = INT_MAX, mx1 = INT_MIN, mx2 = INT_MIN;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int32_t k = total_order_key(x[e]);
      mn2 = min(mn2, max(mn1, k));
      mn1 = min(mn1, k);
      mx2 = max(mx2, min(mx1, k));
      mx1 = max(mx1, k);
    }
#pragma unroll
    for (int off = 1; off <= 2; off <<= 1) {
      const int32_t o1 = __shfl_xor(mn1, off), o2 = __shfl_xor(mn2, off);
      const int32_t u1 = __shfl_xor(mx1, off), u2 = __shfl_xor(mx2, off);
      mn2 = min(max(mn1, o1), min(mn2, o2));
      mn1 = min(mn1, o1);
      mx2 = max(min(mx1, u1), max(mx2, u2));
      mx1 = max(mx1, u1);
    }
    const float s0 = total_order_value(mn1), s1 = total_order_value(mn2);
    const float s31 = total_order_value(mx1), s30 = total_order_value(mx2);
    lo = qa.lo_mode ? s0 : __builtin_fmaf(qa.g_lo, s1 - s0, s0);
    hi = qa.hi_mode == 0 ? __builtin_fmaf(qa.g_hi, s31 - s30, s30) : (qa.hi_mode == 1 ? s30 : s31);
  }
  const float s32 = div_small<L - 1>(hi - lo);
  sh = f16_sat_bits(s32);
  zh = f16_sat_bits(lo);
  const float s32h = f16_bits_to_f32(sh), z32h = f16_bits_to_f32(zh);
  const float rs = s32h == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s32h);
  uint32_t packed = 0;
  bool near = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) packed |= affine_code_fast<BITS>(x[e], z32h, rs, near) << (BITS * e);
  // rare: a value within rounding error of a midpoint; exact codes for those lanes
  if (__builtin_amdgcn_ballot_w64(near) != 0) {
    if (near) {
      const double sd = (double)s32h, zd = (double)z32h;
      packed = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t c = sd == 0.0 ? 0u : affine_code<BITS>(x[e], zd, sd);
        packed |= c << (BITS * e);
      }
    }
  }
  return packed;
}

}  // namespace wushkv
