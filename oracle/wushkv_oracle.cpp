/*
 * wushkv_oracle — plain CPU oracle for the WUSH-KV KV-cache write/read path.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  The GPU library never
 * links, loads or calls it, and this file shares no code, header or table with
 * the GPU library.
 *
 * What it computes (sources are the five web pages about WUSH-KV, arXiv
 * 2609.38121; each function below names the passage it follows):
 *
 *   keys:   k --RoPE--> x --bf16--> x~ ;  y = T~ x~ (T~ = bf16(T_k)) ;
 *           y --clipped b-bit quantizer--> codes + fp16 scale(s) --> packed record
 *   values: v --clipped b-bit quantizer--> codes + scale(s) --> packed record
 *   read:   record --> unpack --> dequantize --> (keys) T~inv * y^
 *   attend: q --pairing--> q' = bf16(T~inv^T q) ; softmax(q'.y^ * scale) . v^
 *           over a sequence's rows of the packed key and value caches
 *
 * Readings taken where the pages are silent:
 *   - RoPE is the rotate-half form on channel pairs (i, i+64) with
 *     w_i = RN32(theta^(-2i/128)); cos and sin of the exact angle pos*w_i are
 *     rounded once to fp32.  Evaluated here in x87 extended precision.
 *   - The transform is y = T_k x with bf16 operands and a sum that is rounded
 *     once to fp32 (here: fp64 accumulation over ascending j).
 *   - Symmetric quantizer: clip C = alpha * RMS(y); 2^b uniform levels with end
 *     points at +-C; the fp16 scale stores the level step Delta = 2C/(2^b-1).
 *     The scale follows a fixed fp32 operation order (pairwise sum of squares).
 *   - Affine quantizer: per group of 32 channels, lo/hi = p_lo/p_hi percentiles
 *     (linear interpolation between order statistics), fp16 step and zero.
 *   - Codes: the index of the nearest level (exact arithmetic), ties to the
 *     even code; a zero step gives code 2^(b-1) (symmetric) or 0 (affine).
 *   - Packing: code j occupies bits [b*j, b*j+b) of an LSB-first bit stream of
 *     16*b bytes per (token, head).
 *   - Query pairing uses the inverse transform the read path uses: q'_j =
 *     sum_r T~inv[r][j] q_r, rounded once to fp32 and then to the bf16 operand
 *     of the score product; q'.y^ equals q.(T~inv y^), the score against the
 *     read path's keys.  Attention (one query per sequence, grouped query
 *     heads) is the exact softmax-weighted mean of the dequantized values.
 *
 * Build: g++ -O2 -std=c++17 -ffp-contract=off (no fast-math), x86-64.
 */
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr int kD = 128;        // head dimension
constexpr int kPairs = 64;     // RoPE rotates channel i with channel i + 64

enum { kF32 = 0, kBF16 = 1 };
enum { kSym = 0, kAffine = 1 };

inline uint32_t bits_of(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
inline float float_of(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

// bf16 rounding, round-to-nearest-even, finite inputs.
inline uint16_t bf16_bits(float f) {
  uint32_t u = bits_of(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
inline float bf16_value(uint16_t h) { return float_of((uint32_t)h << 16); }
inline float round_bf16(float f) { return bf16_value(bf16_bits(f)); }

// fp32 -> fp16, round-to-nearest-even, finite values beyond the fp16 range
// saturate to +-65504.  Done in exact double arithmetic: scale to an integer
// significand and round with rint (the default rounding mode is to-nearest-even).
uint16_t f32_to_f16_sat(float f) {
  uint16_t sign = (bits_of(f) >> 16) & 0x8000u;
  double a = std::fabs((double)f);
  if (!(a < 65520.0)) return sign | 0x7BFFu;  // would round to +-inf: saturate
  if (a < 0x1p-14) {                           // subnormal range, quantum 2^-24
    double m = std::rint(a * 0x1p24);          // 0..1024; 1024 is the least normal
    return sign | (uint16_t)m;
  }
  int e;
  std::frexp(a, &e);                           // a = f * 2^e, f in [0.5, 1)
  double m = std::rint(std::ldexp(a, 11 - e)); // 1024 .. 2048
  if (m == 2048.0) { m = 1024.0; e += 1; }
  int field = e - 1 + 15;
  return sign | (uint16_t)(field << 10) | (uint16_t)((int)m - 1024);
}

float f16_to_f32(uint16_t h) {
  int e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp((double)(1024 + m), e - 25);
  return (float)((h & 0x8000u) ? -v : v);
}

// Monotone map from IEEE totalOrder on floats to signed integers.
inline int32_t total_order_key(float f) {
  int32_t i = (int32_t)bits_of(f);
  return i ^ (int32_t)(((uint32_t)(i >> 31)) & 0x7FFFFFFFu);
}

// RoPE frequency w_i = RN32(theta^(-2i/128)), i = 0..63.
// Pages: the key transform runs "after RoPE" (ai4snews summary "WUSH-KV cuts
// 2-bit KV-cache perplexity...", deployment paragraph; arXiv abstract).  The
// RoPE form itself is not on the pages; rotate-half with base theta is the
// reading for Qwen3-shaped models.
float omega(float theta, int i) {
  return (float)std::pow((double)theta, -(double)(2 * i) / 128.0);
}

// cos/sin of the exact angle pos * w_i (a 24-bit by 24-bit product: exact in
// the 64-bit significand), each rounded once to fp32.
void cos_sin(int32_t pos, float w, float* c, float* s) {
  long double a = (long double)pos * (long double)w;
  *c = (float)cosl(a);
  *s = (float)sinl(a);
}

// Rotate-half RoPE in fp32 with an explicit operation order:
//   x_i      = fma(k_i, c, -(k_{i+64} * s))
//   x_{i+64} = fma(k_{i+64}, c, k_i * s)
void rope(const float* k, int32_t pos, const float* w, float* x) {
  for (int i = 0; i < kPairs; ++i) {
    float c, s;
    cos_sin(pos, w[i], &c, &s);
    float a = k[i], b = k[i + kPairs];
    float bs = b * s;
    float as = a * s;
    x[i] = std::fmaf(a, c, -bs);
    x[i + kPairs] = std::fmaf(b, c, as);
  }
}

// y_r = RN32( sum_j T~[r][j] * x~_j ), j ascending, fp64 accumulation; every
// product of two bf16 values is exact in fp64.
// Pages: a per-KV-head general invertible key transform, not restricted to
// orthogonal matrices (ai4snews summary, method paragraph), applied online
// as a matmul (cere-bro "WUSH-KV: 2-bit KV-Cache Quantization...", Gaps).
void transform(const float* Tt /* bf16-rounded [128][128] */, const float* xt, float* y) {
  for (int r = 0; r < kD; ++r) {
    double acc = 0.0;
    for (int j = 0; j < kD; ++j) acc += (double)Tt[r * kD + j] * (double)xt[j];
    y[r] = (float)acc;
  }
}

// Contiguous pairwise sum: P(a..b) = P(first half) + P(second half), fp32.
float pairwise_sum(const float* a, int n) {
  if (n == 1) return a[0];
  int h = n / 2;
  float l = pairwise_sum(a, h);
  float r = pairwise_sum(a + h, n - h);
  return l + r;
}

// Nearest of the L symmetric levels (q - m) * delta, m = (L-1)/2; ties go to
// the even code.  The midpoint between levels k and k+1 is (k + 1 - L/2)*delta,
// an exact fp64 value, so every comparison below is exact.
uint8_t nearest_sym(float y, float delta, int L) {
  if (delta == 0.0f) return (uint8_t)(L / 2);
  int q = 0;
  for (int k = 0; k < L - 1; ++k) {
    double mid = (double)(k + 1 - L / 2) * (double)delta;
    if ((double)y > mid) ++q;
    else if ((double)y == mid && (k & 1)) ++q;
  }
  return (uint8_t)q;
}

// Symmetric RMS-clipped quantizer on one 128-vector.
// Pages: clipped quantizers paired with the transforms, QuEST INT the one the
// theory covers (arXiv abstract; ai4snews theory paragraph).  The grid and the
// clip C = alpha * RMS are the workload definition (clip 2.0 x RMS).
void sym_quantize(const float* y, int bits, float alpha, uint8_t* q, uint16_t* scale) {
  const int L = 1 << bits;
  float sq[kD];
  for (int j = 0; j < kD; ++j) sq[j] = y[j] * y[j];
  float S = pairwise_sum(sq, kD);
  float ms = S / 128.0f;
  float rms = std::sqrt(ms);
  float C = alpha * rms;
  float twoC = 2.0f * C;
  float d32 = twoC / (float)(L - 1);
  uint16_t dh = f32_to_f16_sat(d32);
  float delta = f16_to_f32(dh);
  *scale = dh;
  for (int j = 0; j < kD; ++j) q[j] = nearest_sym(y[j], delta, L);
}

// Percentile of 32 sorted values by linear interpolation between order
// statistics: h = 31 p / 100, i = floor(h), g = h - i,
// value = s_i + g (s_{i+1} - s_i)   (fma, the difference rounded to fp32).
float percentile32(const float* s, float p) {
  double h = 31.0 * (double)p / 100.0;
  if (h >= 31.0) return s[31];
  double fl = std::floor(h);
  int i = (int)fl;
  float g = (float)(h - fl);
  if (g == 0.0f) return s[i];
  float d = s[i + 1] - s[i];
  return std::fmaf(g, d, s[i]);
}

// Nearest of the L affine levels z + q*s; ties to the even code.  Midpoints
// z + (k + 1/2) s are exact in fp64 for fp16 z and s.
uint8_t nearest_affine(float x, float z, float s, int L) {
  if (s == 0.0f) return 0;
  int q = 0;
  for (int k = 0; k < L - 1; ++k) {
    double mid = (double)z + ((double)k + 0.5) * (double)s;
    if ((double)x > mid) ++q;
    else if ((double)x == mid && (k & 1)) ++q;
  }
  return (uint8_t)q;
}

// Percentile-clipped affine quantizer on one group of 32 values.
// Pages: the end-to-end evaluation uses "OSCAR-style percentile-clipped affine
// quantization" (arXiv abstract; ai4snews end-to-end paragraph).  Group 32,
// percentiles 1/99 and fp16 scale+zero are the workload definition.
void affine_quantize_group(const float* x, int bits, float p_lo, float p_hi, uint8_t* q,
                           uint16_t* scale, uint16_t* zero) {
  const int L = 1 << bits;
  float s[32];
  std::memcpy(s, x, sizeof(s));
  std::sort(s, s + 32, [](float a, float b) { return total_order_key(a) < total_order_key(b); });
  float lo = percentile32(s, p_lo);
  float hi = percentile32(s, p_hi);
  float s32 = (hi - lo) / (float)(L - 1);
  uint16_t sh = f32_to_f16_sat(s32), zh = f32_to_f16_sat(lo);
  *scale = sh;
  *zero = zh;
  float sf = f16_to_f32(sh), zf = f16_to_f32(zh);
  for (int j = 0; j < 32; ++j) q[j] = nearest_affine(x[j], zf, sf, L);
}

// LSB-first bit stream: code j at stream bits [b*j, b*j+b), stream bit 8k+t is
// bit t of byte k.  16*b bytes per 128 codes.
void pack(const uint8_t* q, int bits, uint8_t* rec) {
  std::memset(rec, 0, (size_t)16 * bits);
  for (int j = 0; j < kD; ++j)
    for (int t = 0; t < bits; ++t)
      if ((q[j] >> t) & 1) {
        int b = bits * j + t;
        rec[b >> 3] |= (uint8_t)(1u << (b & 7));
      }
}

void unpack(const uint8_t* rec, int bits, uint8_t* q) {
  for (int j = 0; j < kD; ++j) {
    int v = 0;
    for (int t = 0; t < bits; ++t) {
      int b = bits * j + t;
      v |= ((rec[b >> 3] >> (b & 7)) & 1) << t;
    }
    q[j] = (uint8_t)v;
  }
}

}  // namespace

extern "C" {

// The oracle's own quantizer description (not shared with the GPU library).
typedef struct {
  int32_t kind;       // 0: symmetric RMS clip, 1: percentile affine
  float clip_alpha;   // symmetric: C = alpha * RMS
  int32_t group;      // 128 (symmetric) or 32 (affine)
  float p_lo, p_hi;   // affine percentiles in [0, 100]
} wko_quantizer;

int wko_version(void) { return 1; }

float wko_round_bf16(float f) { return round_bf16(f); }
uint16_t wko_f32_to_f16(float f) { return f32_to_f16_sat(f); }
float wko_f16_to_f32(uint16_t h) { return f16_to_f32(h); }
float wko_omega(float theta, int i) { return omega(theta, i); }

void wko_round_bf16_array(const float* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = round_bf16(in[i]);
}
void wko_f32_to_f16_array(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_f16_sat(in[i]);
}

// cs[n][64][2] = (cos, sin) of pos[n] * w_i.
void wko_cos_sin(float theta, const int32_t* pos, int64_t n, float* cs) {
  float w[kPairs];
  for (int i = 0; i < kPairs; ++i) w[i] = omega(theta, i);
  for (int64_t t = 0; t < n; ++t)
    for (int i = 0; i < kPairs; ++i) cos_sin(pos[t], w[i], &cs[(t * kPairs + i) * 2], &cs[(t * kPairs + i) * 2 + 1]);
}

// RoPE of one 128-vector (fp32 result before the bf16 operand rounding).
void wko_rope(const float* k, int32_t pos, float theta, float* x) {
  float w[kPairs];
  for (int i = 0; i < kPairs; ++i) w[i] = omega(theta, i);
  rope(k, pos, w, x);
}

float wko_pairwise_sum(const float* a, int n) { return pairwise_sum(a, n); }

void wko_sym_quantize(const float* y, int bits, float alpha, uint8_t* q, uint16_t* scale) {
  sym_quantize(y, bits, alpha, q, scale);
}
void wko_affine_quantize_group(const float* x, int bits, float p_lo, float p_hi, uint8_t* q,
                               uint16_t* scale, uint16_t* zero) {
  affine_quantize_group(x, bits, p_lo, p_hi, q, scale, zero);
}
float wko_percentile32(const float* sorted, float p) { return percentile32(sorted, p); }
void wko_pack(const uint8_t* q, int bits, uint8_t* rec) { pack(q, bits, rec); }
void wko_unpack(const uint8_t* rec, int bits, uint8_t* q) { unpack(rec, bits, q); }

// y = T~ x in fp64 (T~ = bf16(T)), no final rounding; for the q.k invariant.
void wko_transform_f64(const float* T, const double* x, double* y) {
  for (int r = 0; r < kD; ++r) {
    double acc = 0.0;
    for (int j = 0; j < kD; ++j) acc += (double)round_bf16(T[r * kD + j]) * x[j];
    y[r] = acc;
  }
}

// Query-side pairing q' = T~^{-T} q: solve T~^T q' = q by Gaussian elimination
// with partial pivoting in fp64.  Then q'.(T~ x) = q.x for every x: the key
// transform is built with the query heads that read the cached keys in view
// (ai4snews summary, method paragraph).  Returns 0, or -1 if singular.
int wko_query_pair(const float* T, const double* q, double* qp) {
  std::vector<double> A((size_t)kD * kD);
  std::vector<double> b(q, q + kD);
  for (int r = 0; r < kD; ++r)
    for (int c = 0; c < kD; ++c) A[(size_t)r * kD + c] = (double)round_bf16(T[c * kD + r]);  // A = T~^T
  for (int col = 0; col < kD; ++col) {
    int piv = col;
    for (int r = col + 1; r < kD; ++r)
      if (std::fabs(A[(size_t)r * kD + col]) > std::fabs(A[(size_t)piv * kD + col])) piv = r;
    if (A[(size_t)piv * kD + col] == 0.0) return -1;
    if (piv != col) {
      for (int c = 0; c < kD; ++c) std::swap(A[(size_t)piv * kD + c], A[(size_t)col * kD + c]);
      std::swap(b[piv], b[col]);
    }
    for (int r = col + 1; r < kD; ++r) {
      double f = A[(size_t)r * kD + col] / A[(size_t)col * kD + col];
      for (int c = col; c < kD; ++c) A[(size_t)r * kD + c] -= f * A[(size_t)col * kD + c];
      b[r] -= f * b[col];
    }
  }
  for (int r = kD - 1; r >= 0; --r) {
    double acc = b[r];
    for (int c = r + 1; c < kD; ++c) acc -= A[(size_t)r * kD + c] * qp[c];
    qp[r] = acc / A[(size_t)r * kD + r];
  }
  return 0;
}

}  // extern "C"

namespace {

int check_quantizer(const wko_quantizer* qz, int bits) {
  if (!qz || bits < 2 || bits > 4) return -1;
  if (qz->kind == kSym && qz->group != kD) return -1;
  if (qz->kind == kAffine && (qz->group != 32 || !(qz->p_lo >= 0.0f) || !(qz->p_hi <= 100.0f) ||
                              !(qz->p_lo <= qz->p_hi)))
    return -1;
  if (qz->kind != kSym && qz->kind != kAffine) return -1;
  return 0;
}

// Quantize one fp32 128-vector into its record and scale slots.
void quantize_vector(const float* y, int bits, const wko_quantizer* qz, uint8_t* rec,
                            uint16_t* scales, uint16_t* zeros) {
  uint8_t q[kD];
  if (qz->kind == kSym) {
    sym_quantize(y, bits, qz->clip_alpha, q, scales);
  } else {
    for (int g = 0; g < 4; ++g)
      affine_quantize_group(y + 32 * g, bits, qz->p_lo, qz->p_hi, q + 32 * g, scales + g, zeros + g);
  }
  pack(q, bits, rec);
}

template <class F>
void parallel_for(int64_t n, int threads, F f) {
  if (threads <= 1 || n < 2) { f(0, n); return; }
  if (threads > n) threads = (int)n;
  std::vector<std::thread> th;
  for (int t = 0; t < threads; ++t) th.emplace_back(f, n * t / threads, n * (t + 1) / threads);
  for (auto& x : th) x.join();
}

inline float load_elem(const void* p, int dtype, int64_t i) {
  return dtype == kBF16 ? bf16_value(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

}  // namespace

extern "C" {

// Keys: RoPE -> bf16 -> T~ -> quantize -> pack, for tokens n = 0..N-1.
// K element (n, h, c) is at K[n * token_stride + h * 128 + c].  Output record
// row = slots[n] (or n), codes[row][H][16 b], scales[row][H] (symmetric) or
// [row][H][4] (affine) fp16, zeros[row][H][4] (affine).  y_out, if given,
// receives the fp32 transformed vectors [N][H][128].
int wko_quantize_keys(const void* K, int k_dtype, int64_t N, int H, int64_t token_stride,
                      const int32_t* pos, const float* T, float theta, int bits,
                      const wko_quantizer* qz, uint8_t* codes, uint16_t* scales, uint16_t* zeros,
                      const int64_t* slots, float* y_out, int threads) {
  if (check_quantizer(qz, bits) || H <= 0 || N < 0 || token_stride < (int64_t)H * kD) return -1;
  if (N == 0) return 0;
  std::vector<float> Tt((size_t)H * kD * kD);
  for (size_t i = 0; i < Tt.size(); ++i) Tt[i] = round_bf16(T[i]);
  float w[kPairs];
  for (int i = 0; i < kPairs; ++i) w[i] = omega(theta, i);
  const int rec_bytes = 16 * bits;
  const int nsc = qz->kind == kSym ? 1 : 4;
  parallel_for(N, threads, [&](int64_t n0, int64_t n1) {
    float k[kD], x[kD], y[kD];
    for (int64_t n = n0; n < n1; ++n) {
      int64_t row = slots ? slots[n] : n;
      for (int h = 0; h < H; ++h) {
        for (int c = 0; c < kD; ++c) k[c] = load_elem(K, k_dtype, n * token_stride + (int64_t)h * kD + c);
        rope(k, pos[n], w, x);
        for (int c = 0; c < kD; ++c) x[c] = round_bf16(x[c]);
        transform(&Tt[(size_t)h * kD * kD], x, y);
        if (y_out) std::memcpy(y_out + (n * H + h) * kD, y, sizeof(y));
        int64_t slot = row * H + h;
        quantize_vector(y, bits, qz, codes + slot * rec_bytes, scales + slot * nsc,
                        zeros ? zeros + slot * nsc : nullptr);
      }
    }
  });
  return 0;
}

// Values: quantize -> pack (their transform is folded into the weights, so
// nothing runs online before the quantizer: ai4snews deployment paragraph;
// the value branch of the cere-bro flowchart, which costs nothing at run time).
int wko_quantize_values(const void* V, int v_dtype, int64_t N, int H, int64_t token_stride,
                        int bits, const wko_quantizer* qz, uint8_t* codes, uint16_t* scales,
                        uint16_t* zeros, const int64_t* slots, int threads) {
  if (check_quantizer(qz, bits) || H <= 0 || N < 0 || token_stride < (int64_t)H * kD) return -1;
  if (N == 0) return 0;
  const int rec_bytes = 16 * bits;
  const int nsc = qz->kind == kSym ? 1 : 4;
  parallel_for(N, threads, [&](int64_t n0, int64_t n1) {
    float v[kD];
    for (int64_t n = n0; n < n1; ++n) {
      int64_t row = slots ? slots[n] : n;
      for (int h = 0; h < H; ++h) {
        for (int c = 0; c < kD; ++c) v[c] = load_elem(V, v_dtype, n * token_stride + (int64_t)h * kD + c);
        int64_t slot = row * H + h;
        quantize_vector(v, bits, qz, codes + slot * rec_bytes, scales + slot * nsc,
                        zeros ? zeros + slot * nsc : nullptr);
      }
    }
  });
  return 0;
}

// Read path: unpack and dequantize rows (slots[n] or n) into out[N][H][128]
// fp32.  Symmetric: y^ = (q - m) * Delta (exact).  Affine: y^ = RN32(z + q*s).
// With T_inv: k^ = RN32( sum_j T~inv[r][j] * y^_j ), T~inv = bf16(T_inv).
int wko_dequantize(const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                   const int64_t* slots, int64_t N, int H, int bits, const wko_quantizer* qz,
                   const float* Tinv, float* out, int threads) {
  if (check_quantizer(qz, bits) || H <= 0 || N < 0) return -1;
  if (qz->kind == kAffine && !zeros) return -1;
  if (N == 0) return 0;
  std::vector<float> Ti;
  if (Tinv) {
    Ti.resize((size_t)H * kD * kD);
    for (size_t i = 0; i < Ti.size(); ++i) Ti[i] = round_bf16(Tinv[i]);
  }
  const int rec_bytes = 16 * bits;
  const int nsc = qz->kind == kSym ? 1 : 4;
  const int L = 1 << bits;
  parallel_for(N, threads, [&](int64_t n0, int64_t n1) {
    uint8_t q[kD];
    float yh[kD];
    for (int64_t n = n0; n < n1; ++n) {
      int64_t row = slots ? slots[n] : n;
      for (int h = 0; h < H; ++h) {
        int64_t slot = row * H + h;
        unpack(codes + slot * rec_bytes, bits, q);
        if (qz->kind == kSym) {
          double delta = (double)f16_to_f32(scales[slot]);
          double m = (double)(L - 1) / 2.0;
          for (int j = 0; j < kD; ++j) yh[j] = (float)(((double)q[j] - m) * delta);
        } else {
          for (int j = 0; j < kD; ++j) {
            int g = j / 32;
            double s = (double)f16_to_f32(scales[slot * nsc + g]);
            double z = (double)f16_to_f32(zeros[slot * nsc + g]);
            yh[j] = (float)(z + (double)q[j] * s);
          }
        }
        float* o = out + (n * H + h) * kD;
        if (Tinv) {
          const float* M = &Ti[(size_t)h * kD * kD];
          for (int r = 0; r < kD; ++r) {
            double acc = 0.0;
            for (int j = 0; j < kD; ++j) acc += (double)M[r * kD + j] * (double)yh[j];
            o[r] = (float)acc;
          }
        } else {
          std::memcpy(o, yh, sizeof(yh));
        }
      }
    }
  });
  return 0;
}

}  // extern "C"

namespace {

// (code - m) * step for a symmetric record: exact in fp64 (a code of at most 4
// bits times an fp16 step).
void dequant_sym(const uint8_t* rec, uint16_t step, int bits, double* y) {
  uint8_t q[kD];
  unpack(rec, bits, q);
  const double d = (double)f16_to_f32(step), m = (double)((1 << bits) - 1) / 2.0;
  for (int j = 0; j < kD; ++j) y[j] = ((double)q[j] - m) * d;
}

// z_g + code * s_g for a percentile-clipped affine record (group g = j / 32, four
// fp16 steps and zeros per record): exact in fp64 (an fp16 zero plus a code of at
// most 4 bits times an fp16 step).  ai4snews summary, end-to-end paragraph.
void dequant_affine(const uint8_t* rec, const uint16_t* steps, const uint16_t* zeros, int bits, double* y) {
  uint8_t q[kD];
  unpack(rec, bits, q);
  for (int j = 0; j < kD; ++j)
    y[j] = (double)f16_to_f32(zeros[j / 32]) + (double)q[j] * (double)f16_to_f32(steps[j / 32]);
}

}  // namespace

extern "C" {

// Query-side pairing: q'_j = RN32( sum_r T~inv[r][j] q_r ) in fp64 over
// ascending r (a bf16 entry times an fp32 query element is exact in fp64),
// then rounded to bf16.  Query head hq reads KV head hq / (Hq / Hkv).  The
// transform is built with the query heads that read the cached keys in view
// (ai4snews summary, method paragraph), so scoring the transformed-basis keys
// with q' scores the read path's keys T~inv y^ with q.
// Q: [N][Hq][128] (fp32 or bf16 bits) with token_stride elements per token;
// Tinv: [Hkv][128][128] fp32 (rounded to bf16 here); out: bf16 bits [N][Hq][128].
int wko_pair_queries(const void* Q, int q_dtype, int64_t N, int Hq, int64_t token_stride,
                     const float* Tinv, int Hkv, uint16_t* out) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || N < 0 || token_stride < (int64_t)Hq * kD) return -1;
  const int G = Hq / Hkv;
  for (int64_t n = 0; n < N; ++n)
    for (int hq = 0; hq < Hq; ++hq) {
      const float* M = Tinv + (size_t)(hq / G) * kD * kD;
      for (int j = 0; j < kD; ++j) {
        double acc = 0.0;
        for (int r = 0; r < kD; ++r)
          acc += (double)round_bf16(M[r * kD + j]) * (double)load_elem(Q, q_dtype, n * token_stride + (int64_t)hq * kD + r);
        out[(n * Hq + hq) * kD + j] = bf16_bits((float)acc);
      }
    }
  return 0;
}

// Decode attention over packed caches: symmetric (kzeros and vzeros NULL, one
// step per record) or percentile-clipped affine (both set; four steps and four
// zeros per record).  Sequence b's tokens are the cache rows row0[b] + n,
// n < len[b]; rows outside [0, n_rows) are absent.
// For query head hq (KV head hq / G) with paired query q' (bf16 [B][Hq][128]):
//   s_n = scale * sum_j q'_j y^_nj        (y^: dequantized keys, fp64 sum)
//   o   = sum_n exp(s_n - max s) v^_n / sum_n exp(s_n - max s)
// in fp64, written as fp32 [B][Hq][128]; a sequence without tokens gives 0.
// Keys are scored in their transformed basis and values read as stored (their
// transform is folded into the weights): ai4snews summary, deployment paragraph.
int wko_decode_attention(const uint16_t* qp, int B, int Hq, int Hkv, const uint8_t* kcodes,
                         const uint16_t* kscales, const uint16_t* kzeros, const uint8_t* vcodes,
                         const uint16_t* vscales, const uint16_t* vzeros, int64_t n_rows, int bits,
                         const int64_t* row0, const int32_t* len, float scale, float* out, int threads) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || bits < 2 || bits > 4 || n_rows < 0) return -1;
  if ((kzeros == nullptr) != (vzeros == nullptr)) return -1;
  const bool affine = kzeros != nullptr;
  const int G = Hq / Hkv;
  const int rec = 16 * bits;
  auto dequant = [&](const uint8_t* codes, const uint16_t* steps, const uint16_t* zeros, int64_t slot, double* y) {
    if (affine) {
      dequant_affine(codes + slot * rec, steps + slot * 4, zeros + slot * 4, bits, y);
    } else {
      dequant_sym(codes + slot * rec, steps[slot], bits, y);
    }
  };
  parallel_for((int64_t)B * Hq, threads, [&](int64_t u0, int64_t u1) {
    double y[kD], v[kD], q[kD], o[kD];
    std::vector<double> s;
    std::vector<int64_t> rows;
    for (int64_t u = u0; u < u1; ++u) {
      const int64_t b = u / Hq;
      const int hq = (int)(u % Hq), h = hq / G;
      for (int j = 0; j < kD; ++j) q[j] = (double)bf16_value(qp[u * kD + j]);
      s.clear();
      rows.clear();
      for (int64_t n = 0; n < (int64_t)len[b]; ++n) {
        const int64_t row = row0[b] + n;
        if (row < 0 || row >= n_rows) continue;
        const int64_t slot = row * Hkv + h;
        dequant(kcodes, kscales, kzeros, slot, y);
        double acc = 0.0;
        for (int j = 0; j < kD; ++j) acc += q[j] * y[j];
        s.push_back((double)scale * acc);
        rows.push_back(row);
      }
      for (int j = 0; j < kD; ++j) o[j] = 0.0;
      if (!s.empty()) {
        const double M = *std::max_element(s.begin(), s.end());
        double l = 0.0;
        for (size_t i = 0; i < s.size(); ++i) {
          const double p = std::exp(s[i] - M);
          const int64_t slot = rows[i] * Hkv + h;
          dequant(vcodes, vscales, vzeros, slot, v);
          for (int j = 0; j < kD; ++j) o[j] += p * v[j];
          l += p;
        }
        for (int j = 0; j < kD; ++j) o[j] /= l;
      }
      for (int j = 0; j < kD; ++j) out[u * kD + j] = (float)o[j];
    }
  });
  return 0;
}

}  // extern "C"
