// Device helpers shared by the libwushkv HIP kernels (gfx950 / CDNA4).
//
// Everything here is part of the GPU library only; the CPU oracle has its own,
// independent implementation of the same definitions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wushkv {

constexpr int kD = 128;     // head dimension
constexpr int kPairs = 64;  // RoPE pairs (i, i + 64)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2v v = {a, b};
  bf16x2v r = __builtin_convertvector(v, bf16x2v);
  return __builtin_bit_cast(uint32_t, r);
}

// bf16 bit patterns -> fp32 (exact).
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> fp16 bits, round-to-nearest-even, saturating finite values to +-65504.
__device__ __forceinline__ uint16_t f16_sat_bits(float x) {
  x = __builtin_fminf(__builtin_fmaxf(x, -65504.0f), 65504.0f);
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// Monotone map from IEEE totalOrder on floats to signed ints (an involution).
__device__ __forceinline__ int32_t total_order_key(float f) {
  int32_t i = __float_as_int(f);
  return i ^ ((i >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float total_order_value(int32_t k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}

// ---------------------------------------------------------------------------------------------
// Code assignment: index of the nearest level in exact arithmetic, ties to the even code.
//
// Symmetric grid, L = 2^BITS levels (q - (L-1)/2) * delta.  The midpoint between
// levels k and k+1 is (k + 1 - L/2) * delta: an integer multiple of delta with at
// most 4 significant bits times an 11-bit fp16 step, so it is exact in fp32 and
// every comparison below is exact.
template <int BITS>
__device__ __forceinline__ uint32_t sym_code(float y, float delta, float rdelta) {
  constexpr int L = 1 << BITS, H = L / 2;
  if (BITS == 2) {
    // midpoints -delta (k=0, tie -> 0), 0 (k=1, tie -> 2), +delta (k=2, tie -> 2)
    return (uint32_t)(y > -delta) + (uint32_t)(y >= 0.0f) + (uint32_t)(y > delta);
  } else {
    // f = floor(y / delta): estimate, clamp to the grid's reach, then correct
    // against the exact multiples f*delta and (f+1)*delta.
    float t = __builtin_fminf(__builtin_fmaxf(y * rdelta, -(float)(H + 1)), (float)H);
    float f = __builtin_floorf(t);
    float lo = f * delta;
    if (y < lo) {
      f -= 1.0f;
    } else if (y >= lo + delta) {
      f += 1.0f;
    }
    int fi = (int)f;
    // y/delta in (f, f+1): nearest level is code H + f.  y == f*delta: tie between
    // codes H+f-1 and H+f; H is even, so the even one is H+f when f is even.
    bool tie = (y == f * delta);
    int q = H + fi - ((tie && (fi & 1)) ? 1 : 0);
    q = q < 0 ? 0 : (q > L - 1 ? L - 1 : q);
    return (uint32_t)q;
  }
}

// Affine grid z + q*s, q in [0, L).  The midpoints z + (k + 1/2) s are exact in
// fp64 for fp16 z and s, so comparing the fp32 input against them in fp64 is exact.
template <int BITS>
__device__ __forceinline__ uint32_t affine_code(float x, double z, double s) {
  constexpr int L = 1 << BITS;
  double xd = (double)x;
  uint32_t q = 0;
#pragma unroll
  for (int k = 0; k < L - 1; ++k) {
    double mid = __builtin_fma((double)k + 0.5, s, z);
    q += (k & 1) ? (uint32_t)(xd >= mid) : (uint32_t)(xd > mid);
  }
  return q;
}

// ---------------------------------------------------------------------------------------------
// RoPE cos/sin of the exact angle pos * w_i, rounded once to fp32.
//
// pos = ph * 1024 + pl.  Tables (built on the host in extended precision):
//   lo[pl][i]  = (cos, sin)(pl * w_i)            as fp64, tails in lo_t
//   hi[ph][i]  = (cos, sin)(ph * 1024 * w_i)     as fp64, tails in hi_t
// Fast path: angle addition in fp64 (absolute error below 2^-51).  If every
// value within 2^-49 of that estimate rounds to the same fp32, that float is
// the answer; otherwise a slow path rounds a double-double evaluation from the
// tables and their tails (error near 2^-100 plus the tables' own ~2^-64).
constexpr double kRopeFastErr = 0x1p-49;

__device__ __forceinline__ void two_prod(double a, double b, double& p, double& e) {
  p = a * b;
  e = __builtin_fma(a, b, -p);
}
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// Adjacent floats (finite inputs): the next one up / down.
__device__ __forceinline__ float float_next_up(float f) {
  if (f == 0.0f) return __uint_as_float(1u);
  uint32_t u = __float_as_uint(f);
  return __uint_as_float(f > 0.0f ? u + 1u : u - 1u);
}
__device__ __forceinline__ float float_next_down(float f) { return -float_next_up(-f); }

// Correctly rounds v = a1*b1 + sg*a2*b2 to fp32, where each factor is given as
// an fp64 head plus tail (a1 + a1t, ...).  v is formed as a double-double
// (vh + vl, error near 2^-100 absolute), RN32(vh) is taken, and the residual
// (vh - f) + vl decides whether the neighbouring float is nearer.
__device__ __noinline__ float rope_round_slow(double a1, double a1t, double b1, double b1t,
                                              double a2, double a2t, double b2, double b2t, double sg) {
  double p1, e1, p2, e2;
  two_prod(a1, b1, p1, e1);
  two_prod(a2, b2, p2, e2);
  p2 *= sg;
  e2 *= sg;
  double t, e3;
  two_sum(p1, p2, t, e3);
  double cross = (a1 * b1t + a1t * b1) + sg * (a2 * b2t + a2t * b2);
  double rest = ((e1 + e2) + e3) + cross;
  double vh, vl;
  two_sum(t, rest, vh, vl);
  float f = (float)vh;
  double d = (vh - (double)f) + vl;  // vh - f is exact (f is the fp32 rounding of vh)
  if (d > 0.0) {
    float u = float_next_up(f);
    double halfgap = 0.5 * ((double)u - (double)f);
    if (d > halfgap || (d == halfgap && (__float_as_uint(u) & 1u) == 0u)) f = u;
  } else if (d < 0.0) {
    float w = float_next_down(f);
    double halfgap = 0.5 * ((double)f - (double)w);
    if (-d > halfgap || (-d == halfgap && (__float_as_uint(w) & 1u) == 0u)) f = w;
  }
  return f;
}

// (cos, sin)(pos * w_i) as fp32.
__device__ __forceinline__ float2 rope_cos_sin(int pos, int i, const double2* __restrict__ lo,
                                               const double2* __restrict__ hi,
                                               const double2* __restrict__ lo_t,
                                               const double2* __restrict__ hi_t) {
  const int pl = pos & 1023, ph = pos >> 10;
  const double2 B = lo[pl * kPairs + i];  // (cos, sin) of the low part
  const double2 A = hi[ph * kPairs + i];  // (cos, sin) of the high part
  // cos(A+B) = cA cB - sA sB ;  sin(A+B) = sA cB + cA sB
  const double c = __builtin_fma(A.x, B.x, -(A.y * B.y));
  const double s = __builtin_fma(A.y, B.x, A.x * B.y);
  float fc, fs;
  {
    float f1 = (float)(c - kRopeFastErr), f2 = (float)(c + kRopeFastErr);
    if (__builtin_expect(f1 == f2, 1)) {
      fc = f1;
    } else {
      const double2 Bt = lo_t[pl * kPairs + i], At = hi_t[ph * kPairs + i];
      fc = rope_round_slow(A.x, At.x, B.x, Bt.x, A.y, At.y, B.y, Bt.y, -1.0);
    }
  }
  {
    float f1 = (float)(s - kRopeFastErr), f2 = (float)(s + kRopeFastErr);
    if (__builtin_expect(f1 == f2, 1)) {
      fs = f1;
    } else {
      const double2 Bt = lo_t[pl * kPairs + i], At = hi_t[ph * kPairs + i];
      fs = rope_round_slow(A.y, At.y, B.x, Bt.x, A.x, At.x, B.y, Bt.y, 1.0);
    }
  }
  return make_float2(fc, fs);
}

}  // namespace wushkv
