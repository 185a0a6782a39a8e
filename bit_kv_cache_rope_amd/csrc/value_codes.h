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
// 2 bits: midpoint tests A = [x > -step], B = [x >= 0], C = [x > step] (ties as
// in the nearest-level rule).  bf16 input: A and C are decided on the raw word
// (bf16_gt_threshold), B as an unsigned bound (x >= 0 or x = -0); a zero step
// makes A and B always true and C never: code 2.  3/4 bits: the step (+inf for
// a zero step) and its reciprocal (0 for a zero step, giving code L/2).
template <int BITS, bool F32IN>
__device__ __forceinline__ float4 value_thresholds(float delta) {
  const float tp = delta == 0.0f ? __builtin_inff() : delta;  // +inf for a zero step
  float4 th;
  if constexpr (BITS == 2) {
    th.x = F32IN ? -tp : bf16_gt_threshold(-tp);
    th.y = F32IN ? tp : bf16_gt_threshold(tp);
    th.z = __uint_as_float(delta == 0.0f ? 0xFFFFFFFFu : (F32IN ? 0x80000000u : 0x8000FFFFu));
    th.w = 0.0f;
  } else {
    th.x = tp;
    th.y = delta == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(delta);
    th.z = th.w = 0.0f;
  }
  return th;
}

// 2-bit symmetric codes of the lane's 8 channels, LSB first (16 bits), from the
// raw words.  The masks are wave-wide ballots: every lane of the wave must run it.
template <bool F32IN>
__device__ __forceinline__ uint32_t value_codes2(const vu32x4* p, float4 th) {
  // the 8 words to test, channel order: bf16 -> low halves shifted up, high
  // halves raw; fp32 -> the values' bits
  uint32_t w[8];
  if constexpr (F32IN) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = p[0][e];
      w[4 + e] = p[1][e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[2 * e] = p[0][e] << 16;
      w[2 * e + 1] = p[0][e];
    }
  }
  const uint32_t tb = __float_as_uint(th.z);
  const uint32_t tbl = F32IN ? tb : (tb & 0xFFFF0000u);  // low halves are exact
  uint64_t m[16];
#pragma unroll
  for (int e = 7; e >= 0; --e) {
    const Sym2Masks k = sym2_masks_raw(w[e], th.x, (e & 1) ? tb : tbl, th.y);
    m[2 * (7 - e)] = k.b1;
    m[2 * (7 - e) + 1] = k.b0;
  }
  const uint32_t packed = shift_in8(0u, m);
  return shift_in8(packed, m + 8);
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
