// Key-side quantizer steps on one 32 x 32 output block of v_mfma_f32_32x32x16_bf16,
// shared by the key kernels (the tiled prefill kernel and the fused append kernel),
// so that both turn the same y into the same bytes.
//
// Layout of the block (one wave, 32 rows of T~ times 32 tokens): lane l holds the
// token column col = l % 32 and, in acc[i], row 8 (i / 4) + 4 (l / 32) + (i % 4)
// of the wave's 32 rows.  Lanes l and l ^ 32 together hold a token's 32 rows.
//
// Quantizer definitions: ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity
// ...", method paragraph (clipped symmetric INT grid, RMS clip) and end-to-end
// paragraph (percentile-clipped affine grid); the bit layout is the library's
// LSB-first record (16 * b bytes per 128-vector).
#pragma once

#include <climits>

#include "device_common.h"
#include "internal.h"
#include "sort32.h"

namespace wushkv {

// Sum of y^2 over the wave's 32 rows of the lane's token, in the contiguous
// pairwise order: runs of 4 rows in-lane, the two lanes' runs of 8 rows
// (rows 8q .. 8q + 3 in lane half 0, 8q + 4 .. 8q + 7 in half 1), then
// ((0 + 1) + (2 + 3)) over the four 8-row runs.  The same value in lanes l
// and l ^ 32.
__device__ __forceinline__ float col_sumsq32(const f32x16& acc) {
  float P8[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float q0 = acc[4 * q] * acc[4 * q];
    const float q1 = acc[4 * q + 1] * acc[4 * q + 1];
    const float q2 = acc[4 * q + 2] * acc[4 * q + 2];
    const float q3 = acc[4 * q + 3] * acc[4 * q + 3];
    const float p4 = (q0 + q1) + (q2 + q3);
    const Halves x = halves(p4);
    P8[q] = __uint_as_float(x.lo) + __uint_as_float(x.hi);
  }
  return (P8[0] + P8[1]) + (P8[2] + P8[3]);
}

// The same sums for both 32-token column blocks of a tile at once, with one
// lane exchange per 8-row run: lane l gets block l / 32's token l % 32.  The
// swap hands lane l < 32 block 0's run from lane l + 32 and lane l + 32 block
// 1's run from lane l, so every lane adds (lane half 0's run) + (lane half 1's
// run) of its own token, in the order col_sumsq32 uses.
__device__ __forceinline__ float col_sumsq32x2(const f32x16& a0, const f32x16& a1) {
  float P8[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float p4[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const f32x16& acc = nb ? a1 : a0;
      const float q0 = acc[4 * q] * acc[4 * q];
      const float q1 = acc[4 * q + 1] * acc[4 * q + 1];
      const float q2 = acc[4 * q + 2] * acc[4 * q + 2];
      const float q3 = acc[4 * q + 3] * acc[4 * q + 3];
      p4[nb] = (q0 + q1) + (q2 + q3);
    }
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p4[0]), __float_as_uint(p4[1]), false, false);
    P8[q] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return (P8[0] + P8[1]) + (P8[2] + P8[3]);
}

// 2-bit symmetric codes of the lane's 16 rows as one word: run q (4 rows) in
// byte q, LSB first.  The bits are shifted in from the last row down (alignbit:
// w = 2w + bit 31 of the operand).  Code = [y > -step] + [y >= 0] + [y > step]:
// the high bit is [y >= 0], the sign of y inverted (an MFMA result that starts
// from a +0 accumulator is never -0); the low bit is [y > step] for y >= 0 and
// [y > -step] for y < 0, which is the sign of m = (step - |y|) * y + 0 (one
// fma): for |y| != step the signs of (step - |y|) and y decide it, and at a tie
// |y| = step (and at y = +0) the exact product is a zero, which the +0 makes +0
// (bit clear, the even code).  A zero step gives code 2 everywhere.
__device__ __forceinline__ uint32_t sym2_word(const f32x16& acc, float delta) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 15; i >= 0; --i) {
    const float y = acc[i];
    const float m = __builtin_fmaf(delta - __builtin_fabsf(y), y, 0.0f);
    w = __builtin_amdgcn_alignbit(w, __float_as_uint(y), 31);
    w = __builtin_amdgcn_alignbit(w, __float_as_uint(m), 31);
  }
  return delta == 0.0f ? 0xAAAAAAAAu : w ^ 0xAAAAAAAAu;
}

// 3/4-bit symmetric codes: run[q] packs the codes of acc[4q .. 4q + 3], LSB
// first.  Fast path with a flagged exact recomputation near a midpoint.
template <int BITS>
__device__ __forceinline__ void sym_runs(const f32x16& acc, float delta, uint32_t* run) {
  // A zero step becomes +inf (threshold / step) so every code comes out L/2.
  const float tp = delta == 0.0f ? __builtin_inff() : delta;
  const float rd = delta == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(delta);
  bool near = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t rc = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) rc |= sym_code_fast<BITS>(acc[4 * q + e], rd, near) << (BITS * e);
    run[q] = rc;
  }
  near = near && rd != 0.0f;
  // rare: a value within rounding error of a midpoint; exact codes for those lanes
  if (__builtin_amdgcn_ballot_w64(near) != 0) {
    if (near) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t rc = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) rc |= sym_code<BITS>(acc[4 * q + e], tp, rd) << (BITS * e);
        asm("" : "+v"(rc));  // keep the word 32 bits wide (compare + add-with-carry codegen)
        run[q] = rc;
      }
    }
  }
}

// Percentile-clipped affine codes, group = the wave's 32 rows of the token,
// split between lanes l and l ^ 32; sh, zh are the fp16 step and zero (the same
// in both lanes).  GEN false: the two smallest and two largest values by IEEE
// totalOrder, merged across the lane pair, give the percentiles (kind 1); GEN
// true: each lane sorts its 16 keys, the pair's two lists are merged in both
// lanes, and the order statistics are read off the 32 sorted keys (kind 2).
template <int BITS, bool GEN = false>
__device__ __forceinline__ void affine_runs(const f32x16& acc, const QuantArgs& qa, uint32_t* run, uint16_t& sh,
                                            uint16_t& zh) {
  constexpr int L = 1 << BITS;
  float lo, hi;
  if constexpr (GEN) {
    int32_t k[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) k[i] = total_order_key(acc[i]);
    bitonic_sort<16>(k);
    int32_t a[16], b[16], srt[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const Halves hv = halves((uint32_t)k[i]);
      a[i] = (int32_t)hv.lo;
      b[i] = (int32_t)hv.hi;
    }
    bitonic_merge<16>(a, b, srt);
    lo = percentile_sorted(srt, qa.lo_i, qa.g_lo, qa.lo_mode);
    hi = percentile_sorted(srt, qa.hi_i, qa.g_hi, qa.hi_mode);
  } else if (qa.lo_mode == 0 && qa.hi_mode == 0) {
    // Both percentiles interpolate (the 1st/99th): the extremes by float
    // minimum, maximum and median.  Where -0 and +0 tie for an order statistic
    // their order does not reach the result: fma(g, s1 - s0, s0) with s0, s1
    // zeros of either signs is +0 in every order (and so for s30, s31).
    Extremes2 e = extremes2_init();
#pragma unroll
    for (int i = 0; i < 16; ++i) extremes2_add(e, acc[i]);
    Extremes2 o;
    {
      const Halves m1 = halves(e.m1), m2 = halves(e.m2), x1 = halves(e.x1), x2 = halves(e.x2);
      o = extremes2_merge({__uint_as_float(m1.lo), __uint_as_float(m2.lo), __uint_as_float(x1.lo), __uint_as_float(x2.lo)},
                          {__uint_as_float(m1.hi), __uint_as_float(m2.hi), __uint_as_float(x1.hi), __uint_as_float(x2.hi)});
    }
    lo = __builtin_fmaf(qa.g_lo, o.m2 - o.m1, o.m1);
    hi = __builtin_fmaf(qa.g_hi, o.x1 - o.x2, o.x2);
  } else {
    // a percentile taken as an order statistic itself: IEEE totalOrder keys
    // (-0 below +0), as the oracle sorts
    int32_t mn1 = INT_MAX, mn2 = INT_MAX, mx1 = INT_MIN, mx2 = INT_MIN;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int32_t k = total_order_key(acc[i]);
      mn2 = min(mn2, max(mn1, k));
      mn1 = min(mn1, k);
      mx2 = max(mx2, min(mx1, k));
      mx1 = max(mx1, k);
    }
    const Halves n1 = halves((uint32_t)mn1), n2 = halves((uint32_t)mn2);
    const Halves x1 = halves((uint32_t)mx1), x2 = halves((uint32_t)mx2);
    const int32_t a1 = (int32_t)n1.lo, b1 = (int32_t)n1.hi, a2 = (int32_t)n2.lo, b2 = (int32_t)n2.hi;
    const int32_t c1 = (int32_t)x1.lo, d1 = (int32_t)x1.hi, c2 = (int32_t)x2.lo, d2 = (int32_t)x2.hi;
    const float s0 = total_order_value(min(a1, b1));
    const float s1 = total_order_value(min(max(a1, b1), min(a2, b2)));
    const float s31 = total_order_value(max(c1, d1));
    const float s30 = total_order_value(max(min(c1, d1), max(c2, d2)));
    lo = qa.lo_mode ? s0 : __builtin_fmaf(qa.g_lo, s1 - s0, s0);
    hi = qa.hi_mode == 0 ? __builtin_fmaf(qa.g_hi, s31 - s30, s30) : (qa.hi_mode == 1 ? s30 : s31);
  }
  const float s32 = div_small<L - 1>(hi - lo);
  sh = f16_sat_bits(s32);
  zh = f16_sat_bits(lo);
  const float s32h = f16_bits_to_f32(sh), z32h = f16_bits_to_f32(zh);
  const float rs = s32h == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s32h);
  bool near = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t rc = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) rc |= affine_code_fast<BITS>(acc[4 * q + e], z32h, rs, near) << (BITS * e);
    run[q] = rc;
  }
  // rare: a value within rounding error of a midpoint; exact codes for those lanes
  if (__builtin_amdgcn_ballot_w64(near) != 0) {
    if (near) {
      const double sd = (double)s32h, zd = (double)z32h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t rc = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t cd = sd == 0.0 ? 0u : affine_code<BITS>(acc[4 * q + e], zd, sd);
          rc |= cd << (BITS * e);
        }
        run[q] = rc;
      }
    }
  }
}

// The lane's share of the token's record for the wave's 32 rows: lane half 0
// writes rows 0-15 (its runs 0, 1 interleaved with those of lane l + 32), half 1
// rows 16-31; BITS * 4 bytes at record byte BITS * (4 wq + 2 lh).
// 2-bit symmetric, from the sym2_word words: bytes {half 0: selectors 0-3,
// half 1: 4-7}; half 0 takes bytes 0, 1 of both, half 1 bytes 2, 3.
__device__ __forceinline__ uint32_t record_chunk2(uint32_t W2, int lh) {
  const Halves w = halves(W2);
  return __builtin_amdgcn_perm(w.hi, w.lo, lh ? 0x07030602u : 0x05010400u);
}
template <int BITS>
__device__ __forceinline__ uint64_t record_chunk(const uint32_t* rn, int lh) {
  constexpr int RB = 4 * BITS;  // bits in a run of 4 codes
  const uint32_t send = lh ? (rn[0] | (rn[1] << RB)) : (rn[2] | (rn[3] << RB));
  const Halves w = halves(send);
  const uint32_t recv = lh ? w.lo : w.hi;
  const uint64_t p0 = recv & ((1u << RB) - 1u), p1 = recv >> RB;
  return lh ? (p0 | ((uint64_t)rn[2] << RB) | (p1 << (2 * RB)) | ((uint64_t)rn[3] << (3 * RB)))
            : ((uint64_t)rn[0] | (p0 << RB) | ((uint64_t)rn[1] << (2 * RB)) | (p1 << (3 * RB)));
}

// Writes a record chunk of BITS * 4 bytes (2-byte aligned for 3 bits).
template <int BITS>
__device__ __forceinline__ void put_chunk(uint8_t* dst, uint64_t chunk) {
  if constexpr (BITS == 2) {
    *(uint32_t*)dst = (uint32_t)chunk;
  } else if constexpr (BITS == 4) {
    *(uint64_t*)dst = chunk;
  } else {
    ((uint16_t*)dst)[0] = (uint16_t)chunk;
    ((uint16_t*)dst)[1] = (uint16_t)(chunk >> 16);
    ((uint16_t*)dst)[2] = (uint16_t)(chunk >> 32);
  }
}

}  // namespace wushkv
