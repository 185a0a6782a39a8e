// Exhaustive check, on the device, of the two fp32 primitives the step computation
// relies on being correctly rounded: the square root (rms = sqrt(S / 128)) and
// the division of the clip range by 2^b - 1 (div_small), as the kernels compile them.
//
// For every fp32 bit pattern x:
//   sqrt  s = __builtin_sqrtf(x).  For finite x > 0 the correctly rounded root is
//         the float s with m_lo^2 < x < m_hi^2, where m_lo, m_hi are the midpoints
//         between s and its neighbours; the midpoints and their squares are exact
//         in fp64 (25 and 50 significant bits), and x never equals one (an odd
//         50-bit square is no 24-bit float), so the comparisons decide exactly.
//         Zeros must return themselves, +inf +inf, negatives and NaN a NaN.
//   div   div_small<D>(x) for D = 3, 7, 15 against (float)((double)x / D): the fp64
//         quotient is correctly rounded, and rounding it again to fp32 cannot
//         differ from rounding x / D once (the binary expansion of a quotient by
//         3, 7 or 15 repeats with period at most 4, so it never carries the
//         28 equal bits a double rounding needs); NaN must stay NaN.
// Mismatches are counted per check into counts[0..3] with vector atomics.
#include "device_common.h"
#include "internal.h"

namespace wushkv {

namespace {

__device__ __forceinline__ bool sqrt_ok(float x) {
  const float s = __builtin_sqrtf(x);
  const uint32_t ux = __float_as_uint(x);
  if (x != x) return s != s;                                  // NaN in, NaN out
  if (ux == 0u || ux == 0x80000000u) return __float_as_uint(s) == ux;  // +-0
  if (ux & 0x80000000u) return s != s;                        // negative: NaN
  if (ux == 0x7F800000u) return __float_as_uint(s) == ux;     // +inf
  if (!(s > 0.0f) || s == __builtin_inff()) return false;
  // neighbours of a positive finite float: the adjacent bit patterns
  const double sd = (double)s;
  const double lo = 0.5 * (sd + (double)__uint_as_float(__float_as_uint(s) - 1u));
  const double hi = 0.5 * (sd + (double)__uint_as_float(__float_as_uint(s) + 1u));
  const double xd = (double)x;
  return lo * lo < xd && xd < hi * hi;
}

template <int Dv>
__device__ __forceinline__ bool div_ok(float x) {
  const float q = div_small<Dv>(x);
  const float r = (float)((double)x / (double)Dv);
  if (r != r) return q != q;
  return __float_as_uint(q) == __float_as_uint(r);
}

__global__ void __launch_bounds__(256) arith_check_kernel(uint32_t* counts) {
  uint32_t bad[4] = {0u, 0u, 0u, 0u};
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32); i += stride) {
    const float x = __uint_as_float((uint32_t)i);
    bad[0] += !sqrt_ok(x);
    bad[1] += !div_ok<3>(x);
    bad[2] += !div_ok<7>(x);
    bad[3] += !div_ok<15>(x);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (bad[k]) atomicAdd(&counts[k], bad[k]);
}

__global__ void zero4_kernel(uint32_t* counts) {
  if (threadIdx.x < 4) counts[threadIdx.x] = 0u;
}

}  // namespace

hipError_t launch_arith_check(uint32_t* counts, int cus, hipStream_t st) {
  zero4_kernel<<<1, 64, 0, st>>>(counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  arith_check_kernel<<<dim3((unsigned)(cus * 16)), 256, 0, st>>>(counts);
  return hipGetLastError();
}

}  // namespace wushkv
