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

// 3/4-bit symmetric code, fast path.  The midpoints are the integer multiples
// j * step, |j| < 2^(b-1), so away from them the code is 2^(b-1) +
// floor(y / step), clamped.  v = y * rdelta (rdelta = v_rcp_f32(step), within
// 1 ulp) is within |y / step| * 1.8e-7 of y / step; after clamping to
// +-(2^(b-1) - 1/2) (the codes there are the extremes, and no midpoint lies
// between the clamp and the grid's end) that is below 1.5e-6, so when v is
// farther than kSymNear from every integer, floor(v) = floor(y / step) and y
// is no tie.  Otherwise `near` is set and the caller recomputes the code with
// sym_code.  A zero step (rdelta = 0) gives v = 0, code 2^(b-1); callers drop
// `near` for it.
constexpr float kSymNear = 0x1p-17f;
template <int BITS>
__device__ __forceinline__ uint32_t sym_code_fast(float y, float rdelta, bool& near) {
  constexpr float H = (float)(1 << (BITS - 1));
  const float v = __builtin_amdgcn_fmed3f(y * rdelta, -H + 0.5f, H - 0.5f);
  const float fl = __builtin_floorf(v);
  near |= __builtin_fabsf(v - __builtin_rintf(v)) < kSymNear;
  return (uint32_t)(fl + H);
}

// Lane masks of the two bits of a 2-bit symmetric code from the midpoint
// tests A = [x > -step], B = [x >= 0], C = [x > step]: bit1 = B and
// bit0 = B ? C : A, i.e. one test of x against the threshold that B selects
// (+step or -step).  A zero step uses thresholds that make every code 2.
struct Sym2Masks {
  uint64_t b1, b0;
};

// For a value tested as a raw 32-bit word (see bf16_gt_threshold): B is the
// unsigned bound word <= tb (x >= 0 or x = -0), A and C compare the word as a
// float with the bf16-rounded thresholds ta and tc.  Two vector compares and
// one select per code, no scalar mask logic.
__device__ __forceinline__ Sym2Masks sym2_masks_raw(uint32_t w, float ta, uint32_t tb, float tc) {
  const bool B = w <= tb;
  const float t = B ? tc : ta;
  return {__builtin_amdgcn_ballot_w64(B), __builtin_amdgcn_ballot_w64(__uint_as_float(w) > t)};
}

// r = 2r + bit, once per lane mask, first mask first (so it ends up most
// significant): one v_addc_co_u32 per bit with the mask as carry-in.  The
// leading s_nop gives the two wait states a vector compare's mask needs
// before an add-with-carry may read it.
__device__ __forceinline__ uint32_t shift_in8(uint32_t r, const uint64_t* m) {
  uint64_t co;
  asm("s_nop 1\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %2\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %3\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %4\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %5\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %6\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %7\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %8\n\t"
      "v_addc_co_u32_e64 %0, %1, %0, %0, %9"
      : "+v"(r), "=&s"(co)
      : "s"(m[0]), "s"(m[1]), "s"(m[2]), "s"(m[3]), "s"(m[4]), "s"(m[5]), "s"(m[6]), "s"(m[7]));
  return r;
}

// Thresholds that decide "x > t" for a bf16 value x from the raw 32-bit word
// whose high half holds x (the low half holding anything): with c the
// smallest bf16 above t, x > t iff x >= c.  For c > 0 every word with high
// half x >= c reads as a float >= c and every other one as < c, so the test
// is word > prev_fp32(c), whose bits are bits(t) | 0xFFFF.  For t < 0 the
// test is word > d with d the largest bf16 <= t (a word's float lies within
// one bf16 step below its high half, towards -inf).  Both tests also decide
// exact bf16 values (low half zero) correctly.  t = +-inf maps to itself.
__device__ __forceinline__ float bf16_gt_threshold(float t) {
  const uint32_t b = __float_as_uint(t);
  if (__builtin_isinf(t)) return t;
  if (t >= 0.0f) return __uint_as_float(b | 0xFFFFu);
  return __uint_as_float((((b & 0x7FFFFFFFu) + 0xFFFFu) & 0xFFFF0000u) | 0x80000000u);
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

// Affine code, fast path.  v = (x - zero) * rstep (rstep = v_rcp_f32(step),
// within 1 ulp; the difference rounded once) is within |v| * 2.4e-7 of the
// exact (x - zero) / step; clamped to [0, 2^b - 1] that is below 3.6e-6.  The
// midpoints sit at v = k + 1/2, so when v is farther than kAffNear from every
// half-integer, rint(v) is the nearest level and no tie; otherwise `near` is
// set and the caller recomputes the code with affine_code.  A zero step
// (rstep = 0) gives code 0, as affine_code's callers do.
constexpr float kAffNear = 0x1p-16f;
template <int BITS>
__device__ __forceinline__ uint32_t affine_code_fast(float x, float zero, float rstep, bool& near) {
  constexpr float Lm1 = (float)((1 << BITS) - 1);
  const float v = __builtin_amdgcn_fmed3f((x - zero) * rstep, 0.0f, Lm1);
  near |= __builtin_fabsf(v - __builtin_floorf(v) - 0.5f) < kAffNear;
  return (uint32_t)__builtin_rintf(v);
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

}  // namespace wushkv
