// In-register bitonic sorting of IEEE totalOrder keys (device_common.h's
// total_order_key), for the order statistics of the percentile-clipped affine
// quantizer at general percentiles: 32 values of a group, held 16 per lane in a
// lane pair or 8 per lane in a lane quad, end up sorted in every lane of the
// group (ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity ...",
// end-to-end paragraph: the percentile-clipped affine quantizer).
//
// Every loop bound is a compile-time constant, so the networks unroll into
// straight min/max instructions on registers.
#pragma once

#include "device_common.h"

namespace wushkv {

// (a, b) <- (min, max)
__device__ __forceinline__ void cex_up(int32_t& a, int32_t& b) {
  const int32_t lo = min(a, b);
  b = max(a, b);
  a = lo;
}

// Ascending bitonic sort of N keys (N a power of two).
template <int N>
__device__ __forceinline__ void bitonic_sort(int32_t* k) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          if ((i & size) == 0) {
            cex_up(k[i], k[j]);
          } else {
            cex_up(k[j], k[i]);
          }
        }
      }
    }
  }
}

// Two ascending lists of N keys -> one ascending list of 2N: a followed by b
// reversed is bitonic, and log2(2N) half-cleaner stages sort it.
template <int N>
__device__ __forceinline__ void bitonic_merge(const int32_t* a, const int32_t* b, int32_t* out) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    out[i] = a[i];
    out[2 * N - 1 - i] = b[i];
  }
#pragma unroll
  for (int stride = N; stride > 0; stride >>= 1) {
#pragma unroll
    for (int i = 0; i < 2 * N; ++i) {
      const int j = i ^ stride;
      if (j > i) cex_up(out[i], out[j]);
    }
  }
}

// s[idx] for an index that is the same in every lane (a kernel argument), as an
// element of a 32-wide register vector: the backend reads it with indexed
// register moves (a select tree on the index bits would be folded back into an
// indexed array in scratch memory).
typedef int32_t i32x32 __attribute__((ext_vector_type(32)));
__device__ __forceinline__ int32_t select32(const int32_t* s, int idx) {
  i32x32 v;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = s[i];
  return v[idx & 31];
}

// The percentile by the interpolation rule of the quantizer description: order
// statistics s_i and s_{i+1} of the sorted keys, weight g; mode 1 takes s_i.
__device__ __forceinline__ float percentile_sorted(const int32_t* s, int i, float g, int exact) {
  const float a = total_order_value(select32(s, i));
  if (exact) return a;
  const float b = total_order_value(select32(s, i + 1));
  return __builtin_fmaf(g, b - a, a);
}

}  // namespace wushkv
