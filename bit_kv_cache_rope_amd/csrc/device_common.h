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

// v_permlane32_swap of a value with itself: `lo` holds, in every lane l, the
// value of lane l % 32, and `hi` the value of lane l % 32 + 32.
struct Halves {
  uint32_t lo, hi;
};
__device__ __forceinline__ Halves halves(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return {r[0], r[1]};
}
__device__ __forceinline__ Halves halves(float x) { return halves(__float_as_uint(x)); }

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

// x / D correctly rounded (round-to-nearest-even) for D = 3, 7, 15: q0 = x * RN(1/D),
// then one residual correction r = q0 D - x (exact in an fma) and q = q0 - r RN(1/D);
// written this way round, x = -0 gives -0.  An infinite x makes r NaN; q0 is then
// the quotient (and is NaN for a NaN x).  Five VALU operations in place of the
// general division's scale/reciprocal/fixup sequence.  Agreement with x / D for
// every fp32 x (subnormals, zeros, infinities and NaN included) is checked on the
// CPU by tests/test_fast_division.py.
template <int D>
__device__ __forceinline__ float div_small(float x) {
  static_assert(D == 3 || D == 7 || D == 15, "exactness is shown for 3, 7 and 15 only");
  constexpr float y = 1.0f / (float)D;
  const float q0 = x * y;
  const float r = __builtin_fmaf(q0, (float)D, -x);
  const float q = __builtin_fmaf(-r, y, q0);
  return q == q ? q : q0;
}

// Symmetric step from the sum of squares S of a 128-vector: rms = sqrt(S / 128)
// (correctly rounded), C = alpha rms, step = RN16sat(2C / (L - 1)).
template <int L>
__device__ __forceinline__ uint16_t sym_step_f16(float S, float alpha) {
  const float ms = S * 0.0078125f;  // S / 128, exact scaling
  const float rms = __builtin_sqrtf(ms);
  const float C = alpha * rms;
  const float twoC = 2.0f * C;
  return f16_sat_bits(div_small<L - 1>(twoC));
}

// Monotone map from IEEE totalOrder on floats to signed ints (an involution).
__device__ __forceinline__ int32_t total_order_key(float f) {
  int32_t i = __float_as_int(f);
  return i ^ ((i >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float total_order_value(int32_t k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}

// Running two smallest (m1 <= m2) and two largest (x1 >= x2) of a stream of
// floats, one v_med3_f32 each: the median of (m1, m2, v) is the new second
// smallest, the median of (m1, v, -inf) the new smallest.  It orders -0 and
// +0 as equal, which the percentile-clipped quantizer may use only where both
// percentiles interpolate between order statistics (a zero of either sign
// there gives the same interpolated value, see affine_runs).
struct Extremes2 {
  float m1, m2, x1, x2;
};
__device__ __forceinline__ Extremes2 extremes2_init() {
  return {__builtin_inff(), __builtin_inff(), -__builtin_inff(), -__builtin_inff()};
}
__device__ __forceinline__ void extremes2_add(Extremes2& e, float v) {
  e.m2 = __builtin_amdgcn_fmed3f(e.m1, e.m2, v);
  e.m1 = __builtin_amdgcn_fmed3f(e.m1, v, -__builtin_inff());
  e.x2 = __builtin_amdgcn_fmed3f(e.x1, e.x2, v);
  e.x1 = __builtin_amdgcn_fmed3f(e.x1, v, __builtin_inff());
}
// The union of two such sets.
__device__ __forceinline__ Extremes2 extremes2_merge(const Extremes2& a, const Extremes2& b) {
  const float ninf = -__builtin_inff(), pinf = __builtin_inff();
  Extremes2 r;
  r.m1 = __builtin_amdgcn_fmed3f(a.m1, b.m1, ninf);
  r.m2 = __builtin_amdgcn_fmed3f(__builtin_amdgcn_fmed3f(a.m1, b.m1, pinf), __builtin_amdgcn_fmed3f(a.m2, b.m2, ninf), ninf);
  r.x1 = __builtin_amdgcn_fmed3f(a.x1, b.x1, pinf);
  r.x2 = __builtin_amdgcn_fmed3f(__builtin_amdgcn_fmed3f(a.x1, b.x1, ninf), __builtin_amdgcn_fmed3f(a.x2, b.x2, pinf), pinf);
  return r;
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

// 3/4-bit symmetric code, fast path.  The midpoints are the integer multiples
// j * step, |j| < 2^(b-1), so away from them the code is floor(y / step +
// 2^(b-1)), clamped to the grid.  w = fma(y, rdelta, 2^(b-1)) (rdelta =
// v_rcp_f32(step), within 1 ulp) is within |y / step| * 1.8e-7 + 2^-21 of
// y / step + 2^(b-1); clamped to [1/2, 2^b - 1/2] (the codes beyond are the
// extremes, and no midpoint lies between the clamp and the grid's end) that
// is below 2e-6, so when w is farther than kSymNear from every integer,
// trunc(w) is the code and y is no tie.  Otherwise `near` is set and the
// caller recomputes the code with sym_code.  A zero step (rdelta = 0) gives
// w = 2^(b-1), code 2^(b-1); callers drop `near` for it.
constexpr float kSymNear = 0x1p-17f;
template <int BITS>
__device__ __forceinline__ uint32_t sym_code_fast(float y, float rdelta, bool& near) {
  constexpr float H = (float)(1 << (BITS - 1));
  const float w = __builtin_amdgcn_fmed3f(__builtin_fmaf(y, rdelta, H), 0.5f, 2.0f * H - 0.5f);
  near |= __builtin_fabsf(w - __builtin_rintf(w)) < kSymNear;
  return (uint32_t)w;  // w > 0: truncation is floor
}

// Sum over aligned groups of 2, 4, 8 and 16 lanes by DPP moves: after step k a
// lane holds the sum of its 2^k-lane block, each step adding the two halves'
// sums (commutative, so both halves hold the same value).  Equal to xor
// butterflies with offsets 1, 2, 4, 8.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_sum16(float v) {
  v = v + dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v = v + dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v = v + dpp_f32<0x141>(v);  // row_half_mirror
  v = v + dpp_f32<0x140>(v);  // row_mirror
  return v;
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

// Affine code, fast path.  (x - zero) * rstep (rstep = v_rcp_f32(step),
// within 1 ulp; the difference rounded once) is within |v| * 2.4e-7 of the
// exact v = (x - zero) / step, and w = fma(x - zero, rstep, 1/2) within that
// plus 2^-21 of v + 1/2; clamped to [1/2, 2^b - 1/2] the bound is below
// 4.2e-6.  The midpoints sit at integer w, so when w is farther than kAffNear
// from every integer, trunc(w) is the nearest level and no tie; otherwise
// `near` is set and the caller recomputes the code with affine_code.  A zero
// step (rstep = 0) gives w = 1/2, code 0, as affine_code's callers do.
constexpr float kAffNear = 0x1p-16f;
template <int BITS>
__device__ __forceinline__ uint32_t affine_code_fast(float x, float zero, float rstep, bool& near) {
  constexpr float Lm1 = (float)((1 << BITS) - 1);
  const float w = __builtin_amdgcn_fmed3f(__builtin_fmaf(x - zero, rstep, 0.5f), 0.5f, Lm1 + 0.5f);
  near |= __builtin_fabsf(w - __builtin_rintf(w)) < kAffNear;
  return (uint32_t)w;  // w > 0: truncation is floor
}

// ---------------------------------------------------------------------------------------------
// RoPE cos/sin of the exact angle pos * w_i, rounded once to fp32.
//
// pos = p2 * 1024 + p1 * 32 + p0 with p0, p1 < 32.  Tables (built on the host in
// extended precision, heads as fp64 with their tails in separate arrays):
//   t0[p0][i] = (cos, sin)(p0 * w_i)          32 rows  (kept in LDS by the key kernel)
//   t1[p1][i] = (cos, sin)(p1 * 32 * w_i)     32 rows  (kept in LDS by the key kernel)
//   t2[p2][i] = (cos, sin)(p2 * 1024 * w_i)   ceil(max_pos / 1024) rows (global)
// Fast path: two angle additions in fp64 (absolute error below 2^-50).  If every
// value within 2^-49 of that estimate rounds to the same fp32, that float is
// the answer; otherwise a slow path redoes both additions in double-double from
// the heads and tails (error near 2^-100 plus the tables' own ~2^-64) and
// rounds that.
constexpr double kRopeFastErr = 0x1p-49;
constexpr int kRopeLoRows = 32;
constexpr int kRopeMidRows = 32;

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

// Double-double v = a1*b1 + sg*a2*b2 from head+tail factors (error ~2^-100 for
// |factors| <= 1); sg is +1 or -1.
__device__ __forceinline__ void dd_pair(double a1, double a1t, double b1, double b1t, double a2, double a2t,
                                        double b2, double b2t, double sg, double& vh, double& vl) {
  double p1, e1, p2, e2;
  two_prod(a1, b1, p1, e1);
  two_prod(a2, b2, p2, e2);
  p2 *= sg;
  e2 *= sg;
  double t, e3;
  two_sum(p1, p2, t, e3);
  const double cross = (a1 * b1t + a1t * b1) + sg * (a2 * b2t + a2t * b2);
  const double rest = ((e1 + e2) + e3) + cross;
  two_sum(t, rest, vh, vl);
}

// RN32 of the double-double vh + vl: RN32(vh), then the residual (vh - f) + vl
// decides whether a neighbouring float is nearer (ties to even).
__device__ __forceinline__ float dd_round_f32(double vh, double vl) {
  float f = (float)vh;
  const double d = (vh - (double)f) + vl;  // vh - f is exact
  if (d > 0.0) {
    const float u = float_next_up(f);
    const double halfgap = 0.5 * ((double)u - (double)f);
    if (d > halfgap || (d == halfgap && (__float_as_uint(u) & 1u) == 0u)) f = u;
  } else if (d < 0.0) {
    const float w = float_next_down(f);
    const double halfgap = 0.5 * ((double)f - (double)w);
    if (-d > halfgap || (-d == halfgap && (__float_as_uint(w) & 1u) == 0u)) f = w;
  }
  return f;
}

// Slow path: (cos, sin)(a + m + b) correctly rounded, from the three table
// entries (head, tail) of the angle parts.
__device__ __forceinline__ float2 rope_cos_sin_slow(double2 A, double2 At, double2 M, double2 Mt, double2 B,
                                                 double2 Bt) {
  double ch, cl, sh, sl;
  dd_pair(A.x, At.x, M.x, Mt.x, A.y, At.y, M.y, Mt.y, -1.0, ch, cl);  // cos(a+m)
  dd_pair(A.y, At.y, M.x, Mt.x, A.x, At.x, M.y, Mt.y, 1.0, sh, sl);   // sin(a+m)
  double c2h, c2l, s2h, s2l;
  dd_pair(ch, cl, B.x, Bt.x, sh, sl, B.y, Bt.y, -1.0, c2h, c2l);      // cos(a+m+b)
  dd_pair(sh, sl, B.x, Bt.x, ch, cl, B.y, Bt.y, 1.0, s2h, s2l);       // sin(a+m+b)
  return make_float2(dd_round_f32(c2h, c2l), dd_round_f32(s2h, s2l));
}

// Fast path from the three heads; `exact` is false when the slow path is needed.
__device__ __forceinline__ float2 rope_cos_sin_fast(double2 A, double2 M, double2 B, bool& exact) {
  const double c1 = __builtin_fma(A.x, M.x, -(A.y * M.y));
  const double s1 = __builtin_fma(A.y, M.x, A.x * M.y);
  const double c = __builtin_fma(c1, B.x, -(s1 * B.y));
  const double s = __builtin_fma(s1, B.x, c1 * B.y);
  const float fc1 = (float)(c - kRopeFastErr), fc2 = (float)(c + kRopeFastErr);
  const float fs1 = (float)(s - kRopeFastErr), fs2 = (float)(s + kRopeFastErr);
  exact = (fc1 == fc2) && (fs1 == fs2);
  return make_float2(fc1, fs1);
}

struct RopeTables {
  const double2* t0;    // [32][64]
  const double2* t1;    // [32][64]
  const double2* t2;    // [hi_rows][64]
  const double2* t0t;   // tails
  const double2* t1t;
  const double2* t2t;
};

// (cos, sin)(pos * w_i) with every table read from global memory.
__device__ __forceinline__ float2 rope_cos_sin(int pos, int i, const RopeTables& t) {
  const int p0 = pos & 31, p1 = (pos >> 5) & 31, p2 = pos >> 10;
  const double2 A = t.t2[p2 * kPairs + i], M = t.t1[p1 * kPairs + i], B = t.t0[p0 * kPairs + i];
  bool exact;
  float2 v = rope_cos_sin_fast(A, M, B, exact);
  if (__builtin_expect(!exact, 0))
    v = rope_cos_sin_slow(A, t.t2t[p2 * kPairs + i], M, t.t1t[p1 * kPairs + i], B, t.t0t[p0 * kPairs + i]);
  return v;
}

// ---------------------------------------------------------------------------------------------
// Two-level split used by the key kernel: pos = h * 32 + p0 with p0 < 32.
//   lo[p0][i] = (cos, sin)(p0 * w_i)        32 rows: the t0 table above (kept in LDS by the key
//                                           kernel)
//   hi[h][i]  = (cos, sin)(h * 32 * w_i)    ceil(max_pos / 32) rows (global), built on the device
//                                           from t1 and t2 in double-double (head, tail)
// Fast path: one angle addition in fp64, rounded to fp32.  With every head within 2^-53 (plus
// ~2^-63) of its exact value and |cos|, |sin| <= 1, each product carries at most 2 * 2^-53 from
// its factors, the rounded product 2^-53 more and the fma 2^-53: below 6.1 * 2^-53 in all, so
// the fp32 rounding differs from the exact one only for a value within that distance of an fp32
// rounding midpoint (about 2^-24 of values).  The RoPE handle marks, once, every position for
// which any of its 64 pairs differs (comparing with the double-double sum), in a bitmap of one
// bit per position: exc[pos / 32] bit pos % 32.  Marked positions take the double-double path.
__device__ __forceinline__ float2 rope2_fast(double2 H, double2 B) {
  const double c = __builtin_fma(H.x, B.x, -(H.y * B.y));
  const double s = __builtin_fma(H.y, B.x, H.x * B.y);
  return make_float2((float)c, (float)s);
}

__device__ __forceinline__ float2 rope2_slow(double2 H, double2 Ht, double2 B, double2 Bt) {
  double ch, cl, sh, sl;
  dd_pair(H.x, Ht.x, B.x, Bt.x, H.y, Ht.y, B.y, Bt.y, -1.0, ch, cl);  // cos(h + b)
  dd_pair(H.y, Ht.y, B.x, Bt.x, H.x, Ht.x, B.y, Bt.y, 1.0, sh, sl);   // sin(h + b)
  return make_float2(dd_round_f32(ch, cl), dd_round_f32(sh, sl));
}

struct Rope2Tables {
  const double2* lo;     // [32][64] heads (= t0)
  const double2* hi;     // [hi2_rows][64] heads
  const double2* lot;    // tails
  const double2* hit;
  const uint32_t* exc;   // [hi2_rows] positions whose fast sum rounds differently
};

__device__ __forceinline__ bool rope2_marked(const uint32_t* exc, int pos) {
  return (exc[pos >> 5] >> (pos & 31)) & 1u;
}

// (cos, sin)(pos * w_i) with every table read from global memory; the key kernel computes the
// same function with lo read from LDS.
__device__ __forceinline__ float2 rope2_cos_sin(int pos, int i, const Rope2Tables& t) {
  const int p0 = pos & 31, h = pos >> 5;
  const double2 H = t.hi[h * kPairs + i], B = t.lo[p0 * kPairs + i];
  if (__builtin_expect(rope2_marked(t.exc, pos), 0))
    return rope2_slow(H, t.hit[h * kPairs + i], B, t.lot[p0 * kPairs + i]);
  return rope2_fast(H, B);
}

// (cos, sin) of pairs 2c and 2c + 1 at position pos, as (c0, s0, c1, s1), from the heads
// H0, H1 of hi row pos / 32, B0, B1 of lo row pos % 32 and that hi row's bitmap word; a
// marked position reads the tails from global memory and takes the double-double sum.
__device__ __forceinline__ float4 rope2_pair_cs(int pos, int c, double2 H0, double2 H1, uint32_t exc_word,
                                                double2 B0, double2 B1, const double2* hit, const double2* lot) {
  float2 v0, v1;
  if (__builtin_expect((exc_word >> (pos & 31)) & 1u, 0)) {  // a marked position: rare
    const uint32_t hr = ((uint32_t)pos >> 5) * (uint32_t)kPairs + 2 * c;
    const uint32_t lr = (uint32_t)(pos & 31) * kPairs + 2 * c;
    v0 = rope2_slow(H0, hit[hr], B0, lot[lr]);
    v1 = rope2_slow(H1, hit[hr + 1], B1, lot[lr + 1]);
  } else {
    v0 = rope2_fast(H0, B0);
    v1 = rope2_fast(H1, B1);
  }
  return make_float4(v0.x, v0.y, v1.x, v1.y);
}

}  // namespace wushkv
