// Decode attention straight from the packed cache, with the query paired
// through the inverse key transform.
//
// The keys sit in the cache in the transformed basis y = T_k x.  A query head
// that reads them is paired once, q' = T~inv^T q, so that q'.y^ = q.(T~inv y^):
// the scores against the read path's keys come out without a 128x128 product
// per cached key (ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity
// ...", method paragraph: the transform is built with the query heads that
// read the cached keys in view; deployment paragraph: keys are cached after
// the transform, the value transform is folded into the weights, so values
// are read as stored).
//
// Work decomposition (one query token per sequence, grouped query heads):
//   * pair_queries_kernel: q'_j = RN32(sum_r T~inv[r][j] q_r) in fp64 FMAs
//     over ascending r (every product is exact), then bf16.
//   * one block of four waves per (2048-token split, KV head, sequence); a
//     split writes (max, sum, unnormalized output) per query head, and
//     combine_kernel merges the splits of a sequence.
//   * attention_wave_kernel (symmetric caches of every width): each wave
//     takes 64-token rounds of the split on its own, loads its key codes
//     straight into registers and keeps its own online softmax.  3-bit
//     records are loaded as 12-byte pieces (32 channels) and widened in
//     registers to the 4-bit layout, after which they take the 4-bit path.
//       scores  S[g][n] = sum_j q'[g][j] c[n][j] on
//               v_mfma_f32_16x16x128_f8f6f4, all 128 channels in one
//               product: the query in 20-bit fixed point as four base-32
//               digits (fp8 integers in rows 4 g + i), the codes as fp4
//               (2 bits) or fp8 (3 and 4 bits) values made with one mask per
//               word, one lane per (query, token) after the digits are combined.
//       values  O[ch][g] += c[ch][n] * p[n][g] on v_mfma_f32_16x16x32_bf16:
//               rows = 16 channels, k = 32 tokens, columns = the query heads'
//               weights p * step_v split into three bf16 parts (exact to
//               fp32).  The value records go to the wave's LDS as token
//               pairs: halfword j of tokens 2i and 2i + 1 side by side in one
//               word, so that a lane turns the word into its channel's two
//               operands with one rotate and one mask.
//   * attention_affine_kernel (affine caches of every width): rounds of 256 tokens
//     staged in LDS by the whole block, scores on v_mfma_f32_16x16x32_bf16
//     with the codes as exact bf16 values 0.5 + c / SB, values on
//     v_mfma_f32_4x4x1f32 with fp32 weights (an affine record has a step and
//     zero per 32 channels).
#include "device_common.h"
#include "internal.h"

#include <mutex>
#include <type_traits>

namespace wushkv {

namespace {

constexpr int kChunk = 2048;     // tokens per split (one block)
constexpr int kSub = 256;        // tokens staged in LDS per round (attention_affine_kernel)
constexpr int kPartFloats = 132;  // per (sequence, query head, split): max, sum, 2 pad, o[128]
constexpr int kPairVecs = 4;      // query vectors per pairing block

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): loads at offsets past `bytes`
// (including offsets that wrapped below zero) return zeros.
constexpr int kRawBufferWord3 = 0x00020000;
__device__ __forceinline__ rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

// grid (ceil(N G / kPairVecs), Hkv), 256 threads.
__global__ void __launch_bounds__(256) pair_queries_kernel(const PairArgs a) {
  __shared__ __align__(16) uint16_t t_lds[kD][kD];  // T~inv[r][j] of this KV head (bf16 bits)
  __shared__ float q_lds[kPairVecs][kD];
  const int h = blockIdx.y, tid = threadIdx.x;
  const int64_t v0 = (int64_t)blockIdx.x * kPairVecs;
  const int64_t nv = a.n_tokens * a.G;
  // the handle's 16-byte chunks, read in order: chunk (mt, s, l) holds
  // T~inv[32 mt + l % 32][16 s + 8 (l / 32) .. + 7]
  const u32x4* T = (const u32x4*)a.Tinv + (int64_t)h * (kD * kD / 8);
  for (int k = tid; k < kD * kD / 8; k += 256) {
    const int l = k & 63, s = (k >> 6) & 7, mt = k >> 9;
    *(u32x4*)&t_lds[32 * mt + (l & 31)][16 * s + 8 * (l >> 5)] = T[k];
  }
  for (int i = tid; i < kPairVecs * kD; i += 256) {
    const int vi = i >> 7, c = i & 127;
    const int64_t v = v0 + vi;
    float x = 0.0f;
    if (v < nv) {
      const int64_t n = v / a.G;
      const int hq = h * a.G + (int)(v - n * a.G);
      const int64_t e = n * a.stride + (int64_t)hq * kD + c;
      x = a.f32_in ? ((const float*)a.Q)[e] : bf16lo_to_f32(((const uint16_t*)a.Q)[e]);
    }
    q_lds[vi][c] = x;
  }
  __syncthreads();
  const int j = tid & 127;
  for (int vi = tid >> 7; vi < kPairVecs; vi += 2) {
    const int64_t v = v0 + vi;
    if (v >= nv) break;
    double acc = 0.0;
#pragma unroll 8
    for (int r = 0; r < kD; ++r) acc = __builtin_fma((double)bf16lo_to_f32(t_lds[r][j]), (double)q_lds[vi][r], acc);
    const int64_t n = v / a.G;
    const int hq = h * a.G + (int)(v - n * a.G);
    const uint32_t w = pack_bf16x2((float)acc, 0.0f);
    a.out[(n * a.n_q_heads + hq) * kD + j] = (uint16_t)w;
  }
}

// Channel of element e of the score product's k step s for lane group r: the
// order in which the code operand below lays out the lane's 32 channels.
template <int BITS>
__device__ __forceinline__ int score_channel(int r, int s, int e) {
  const int u = e >> 1;
  if constexpr (BITS == 2) {
    // word s / 2 of the lane's 8 bytes, field 2 (s % 2) + u / 2, bytes 2 (u % 2) + e % 2
    return 4 * (8 * r + 4 * (s >> 1) + 2 * (u & 1) + (e & 1)) + 2 * (s & 1) + (u >> 1);
  } else if constexpr (BITS == 4) {
    // word s of the lane's 16 bytes, nibble u / 2, bytes 2 (u % 2) + e % 2
    return 32 * r + 8 * s + 2 * (2 * (u & 1) + (e & 1)) + (u >> 1);
  } else {
    return 32 * r + 8 * s + e;
  }
}

// bf16 words 0x3F00 | (code << SH) (the value 0.5 + code / SB), two per u32:
// bytes b0, b1 of q (each holding a code in bits SH.. of the byte) under the
// constant high byte 0x3F.
__device__ __forceinline__ uint32_t code_pair(uint32_t q, bool hi) {
  return __builtin_amdgcn_perm(q, 0x3F3F3F3Fu, hi ? 0x00070006u : 0x00050004u);
}

template <int BITS>
__device__ __forceinline__ void score_operands(const uint32_t* W, bf16x8* A) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t q0 = (W[w] << 5) & 0x60606060u, q1 = (W[w] << 3) & 0x60606060u;
      const uint32_t q2 = (W[w] << 1) & 0x60606060u, q3 = (W[w] >> 1) & 0x60606060u;
      const u32x4 a0 = {code_pair(q0, false), code_pair(q0, true), code_pair(q1, false), code_pair(q1, true)};
      const u32x4 a1 = {code_pair(q2, false), code_pair(q2, true), code_pair(q3, false), code_pair(q3, true)};
      A[2 * w] = __builtin_bit_cast(bf16x8, a0);
      A[2 * w + 1] = __builtin_bit_cast(bf16x8, a1);
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t q0 = (W[s] << 3) & 0x78787878u, q1 = (W[s] >> 1) & 0x78787878u;
      const u32x4 a = {code_pair(q0, false), code_pair(q0, true), code_pair(q1, false), code_pair(q1, true)};
      A[s] = __builtin_bit_cast(bf16x8, a);
    }
  } else {
    // 24 bits per k step: bits 24 s .. 24 s + 23 of the lane's 96
    const uint32_t x[4] = {W[0], __builtin_amdgcn_alignbit(W[1], W[0], 24), __builtin_amdgcn_alignbit(W[2], W[1], 16),
                           W[2] >> 8};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 a;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t c0 = (x[s] >> (6 * t)) & 7u, c1 = (x[s] >> (6 * t + 3)) & 7u;
        a[t] = 0x3F003F00u | (c0 << 4) | (c1 << 20);
      }
      A[s] = __builtin_bit_cast(bf16x8, a);
    }
  }
}

// Value side: lane (token b = lane / 4, column x = lane % 4) of wave w holds
// channel value_channel(w, x, k) of its token for product k = 0..7, as the
// fp32 value code * value_scale(x).
template <int BITS>
__device__ __forceinline__ int value_channel(int w, int x, int k) {
  if constexpr (BITS == 4) return 32 * w + 16 * (x >> 1) + 8 * (k >> 2) + 2 * (k & 3) + (x & 1);
  return 32 * w + 4 * k + x;
}
template <int BITS>
__device__ __forceinline__ float value_scale(int x) {
  if constexpr (BITS == 2) return (float)(1 << (2 * x));
  if constexpr (BITS == 4) return (x & 1) ? 16.0f : 1.0f;
  return 1.0f;
}
template <int BITS>
__device__ __forceinline__ int value_byte_offset(int w, int x) {
  if constexpr (BITS == 2) return 8 * w;
  if constexpr (BITS == 4) return 16 * w + 8 * (x >> 1);
  return 12 * w;
}
__device__ __forceinline__ float byte_f32(uint32_t v, int k) { return (float)((v >> (8 * k)) & 0xFFu); }

template <int BITS>
__device__ __forceinline__ void value_operands(const uint32_t* U, int x, float* B) {
  if constexpr (BITS == 2 || BITS == 4) {
    const uint32_t mask = BITS == 2 ? (0x03030303u << (2 * x)) : (0x0F0F0F0Fu << (4 * (x & 1)));
    const uint32_t m0 = U[0] & mask, m1 = U[1] & mask;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      B[k] = byte_f32(m0, k);
      B[4 + k] = byte_f32(m1, k);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int p = 12 * k + 3 * x;  // bit of the code in the lane's 96
      const int wi = p >> 5;
      const uint32_t lo = wi == 0 ? U[0] : (wi == 1 ? U[1] : U[2]);
      const uint32_t hi = wi == 0 ? U[1] : (wi == 1 ? U[2] : 0u);
      B[k] = (float)(__builtin_amdgcn_alignbit(hi, lo, p & 31) & 7u);
    }
  }
}

template <int NW>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t* W) {
  if constexpr (NW == 2) {
    const uint2 v = *(const uint2*)p;
    W[0] = v.x; W[1] = v.y;
  } else if constexpr (NW == 4) {
    const uint4 v = *(const uint4*)p;
    W[0] = v.x; W[1] = v.y; W[2] = v.z; W[3] = v.w;
  } else {
    const uint32_t* q = (const uint32_t*)p;
    W[0] = q[0]; W[1] = q[1]; W[2] = q[2];
  }
}

__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m, 64); }

// (x & m) | c as one v_and_or_b32: m from an SGPR, c from a VGPR (a VOP3
// instruction reads at most one scalar operand on this chip, so with both as
// constants the compiler would split it into an and and an or).
__device__ __forceinline__ uint32_t and_or_sv(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// (a & m) | (b & ~m): one v_bfi_b32
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

// 32 consecutive 3-bit codes (12 bytes of a record, LSB first) widened to the
// 4-bit record layout: nibble n of word r holds code 8 r + n in its low three
// bits; the nibble's top bit is left undefined (the operands mask it off).
// Each 24-bit run of eight codes spreads in three steps: the high six codes'
// bits move up by 4 (runs of four codes in each halfword), then codes 2, 3 of
// each halfword by 2, then the odd codes of each byte by 1.
__device__ __forceinline__ u32x4 widen3(const u32x3 d) {
  const uint32_t x[4] = {d[0], __builtin_amdgcn_alignbit(d[1], d[0], 24), __builtin_amdgcn_alignbit(d[2], d[1], 16),
                         d[2] >> 8};
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t w = bfi(0x00000FFFu, x[k], x[k] << 4);
    w = bfi(0x003F003Fu, w, w << 2);
    r[k] = bfi(0x07070707u, w, w << 1);
  }
  return r;
}

// ---- narrow-format score product (2 and 4 bits, symmetric keys) on
// v_mfma_f32_16x16x128_f8f6f4: A = the paired query in fixed point as four
// base-32 digits, each an fp8 (e4m3) integer; B = the key codes of 16 tokens,
// k = the 128 channels.  A 2-bit code zero-extended to a nibble is the fp4
// (e2m1) value c / 2, and a 4-bit code zero-extended to a byte is the fp8
// (e4m3) value c * 2^-9, so the codes become operands with one mask (and one
// shift) per word.  This product does not add its 128 terms as fp32 would:
// measured, a sum is exact when every term's bits lie within 13 binary places
// of the largest term's leading bit, and loses low bits beyond that.  A digit
// row keeps every term on one grid (|digit| <= 16, code <= 15: 8 places), so
// each row sums exactly, and the digits are combined afterwards in fp32.
// Operand layout (measured): an 8-bit operand's lane (group g = lane / 16, row
// or column lane % 16) holds k = 16 g + j in byte j < 16 and k = 64 + 16 g +
// j - 16 in byte j >= 16; a 4-bit operand's lane holds k = 32 g + j in nibble
// j.  Only the pairing of A's and B's elements matters, which the map below
// fixes.

// Position 32 g + j (lane group g, byte j of A's 32) of channel ch in the
// query operand, matched to where the code operand puts that channel's code.
template <int BITS>
__device__ __forceinline__ int qpart_pos(int ch) {
  const int g = ch >> 5, c = ch & 31;
  if constexpr (BITS == 2) {
    // code operand: lane group g takes the record's bytes 8 g .. 8 g + 7 (words
    // w0, w1) as the nibble words w0 & m, (w0 >> 2) & m, w1 & m, (w1 >> 2) & m
    // (m = 0x33333333): nibble i of word d is channel 32 g + 16 (d / 2) + 2 i + d % 2
    const int d = 2 * (c >> 4) + (c & 1), i = (c & 15) >> 1;
    const int k = 32 * g + 8 * d + i;  // its k
    return k < 64 ? 32 * (k >> 4) + (k & 15) : 32 * ((k - 64) >> 4) + 16 + ((k - 64) & 15);
  } else {
    // code operand: lane group g takes bytes 16 g .. 16 g + 15 (words W0..W3) as
    // the byte words W0 & m, (W0 >> 4) & m, W1 & m, ... (m = 0x0F0F0F0F): byte
    // i of word r is channel 32 g + 8 (r / 2) + 2 i + r % 2; both operands are
    // 8-bit, so A's byte j pairs with B's byte j
    const int r = 2 * (c >> 3) + (c & 1), i = (c & 7) >> 1;
    return 32 * g + 4 * r + i;
  }
}

// max(x, y) as one v_max_f32 (no quieting of signalling NaNs, which never occur here)
__device__ __forceinline__ float vmax(float x, float y) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}

// Affine caches of every width (a step and a zero per 32-channel group).
// grid 8 * n_splits8 * Hkv * B blocks (see the block map below), 256 threads.
// A block takes up to kChunk tokens of one sequence and KV head, in rounds of
// KS tokens, with the running max, sums and value accumulators rescaled from
// round to round (online softmax).  Scores on v_mfma_f32_16x16x32_bf16 with
// the codes as exact bf16 values 0.5 + c / SB; values on the fp32 4x4x1
// product, where wave w owns channels 32 w .. 32 w + 31 (one affine group).
template <int BITS, int QS>
__global__ void __launch_bounds__(256, (QS == 1 && BITS != 4) ? 3 : 2) attention_affine_kernel(const AttnArgs a) {
  constexpr int NQ = 4 * QS;   // query rows of the value product (G <= NQ)
  constexpr int KS = kSub;  // tokens per round (three blocks' LDS fits a CU)
  constexpr int REC = 16 * BITS;
  constexpr int SNW = BITS;    // words of key codes per lane (32 channels)
  constexpr int VNW = BITS == 3 ? 3 : 2;  // words of value codes per lane
  constexpr float SB = BITS == 2 ? 8.0f : (BITS == 3 ? 16.0f : 32.0f);
  constexpr int SROW = KS + 16;  // s_lds row (padded against bank conflicts)
  constexpr float NINF = -__builtin_inff();
  constexpr int PU = BITS == 2 ? 4 : 2;   // value steps per pass (4x4x1 product)

  __shared__ __align__(16) uint8_t kc_lds[KS * REC];  // the round's key records
  __shared__ __align__(16) uint8_t vc_lds[KS * REC];  // the round's value records
  __shared__ __align__(16) float s_lds[NQ][SROW];       // scores (log2 units), then p
  __shared__ __align__(16) float off_lds[KS];         // 0, or -inf for an absent token
  __shared__ float pr_lds[KS];                        // 1, or 0 for an absent token
  __shared__ float q_lds[NQ][kD + 1];
  __shared__ float mx_lds[4][NQ];
  __shared__ float sum_lds[4][NQ];
  // per group g and token n at [g * KS + n]: the key step and zero times
  // scale * log2(e), the value step and zero (0 for an absent token)
  __shared__ __align__(16) float ksc_lds[4 * KS];
  __shared__ __align__(16) float kzr_lds[4 * KS];
  __shared__ __align__(16) float vsc_lds[4 * KS];
  __shared__ __align__(16) float vzr_lds[4 * KS];
  __shared__ float zsum_lds[4][NQ];  // sum_n p_n z_n of wave w's group, per query

  // Block L runs on XCD L % 8 (blocks are dispatched to the XCDs round-robin).
  // The split s of sequence b goes to XCD (s + b) % 8, so that each XCD gets
  // a like share of every sequence's splits, and its KV heads to blocks L
  // eight apart (one XCD, dispatched one after the other), which then read
  // the same cache lines (a row holds every KV head's record) through one L2.
  const int L = blockIdx.x, xcd = L & 7, q = L >> 3;
  const int h = q % a.n_kv_heads, q2 = q / a.n_kv_heads;
  const int b = q2 / a.n_splits8, s8 = q2 - b * a.n_splits8;
  const int split = 8 * s8 + ((xcd - b) & 7);
  if (split >= a.n_splits) return;
  const int len = min(max(a.len[b], 0), a.max_len);
  const int n_lo = split * kChunk;
  if (n_lo >= len) return;  // uniform over the block
  const int cnt_all = min(len - n_lo, kChunk);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.G, Hkv = a.n_kv_heads;
  if (a.n_rows <= 0) {
    // no row exists: the split contributes nothing (max -inf, sums and output 0)
    for (int i = tid; i < G * kPartFloats; i += 256) {
      const int g = i / kPartFloats, e = i - g * kPartFloats;
      a.part[(((int64_t)b * a.n_q_heads + h * G + g) * a.n_splits + split) * kPartFloats + e] =
          e == 0 ? -__builtin_inff() : 0.0f;
    }
    return;
  }

  // (the loads of all four passes are issued before the first is used)
  uint16_t qv[NQ * kD / 256];
#pragma unroll
  for (int j = 0; j < NQ * kD / 256; ++j) {
    const int i = tid + 256 * j, g = i >> 7, c = i & 127;
    const uint16_t v = a.qp[((int64_t)b * a.n_q_heads + h * G + (g < G ? g : 0)) * kD + c];  // unconditional
    qv[j] = g < G ? v : (uint16_t)0;
  }
#pragma unroll
  for (int j = 0; j < NQ * kD / 256; ++j) {
    const int i = tid + 256 * j;
    q_lds[i >> 7][i & 127] = bf16lo_to_f32(qv[j]);
  }
  // the sequence's first row, read once (a load in the loop would be redone and
  // waited for in every round: the compiler cannot tell it from the stores)
  const int64_t row_base = a.row0[b] + n_lo;
  __syncthreads();

  // score operands of the paired queries: lane (column col, group grp).  The
  // score product's 16 columns are (query gq = col / 4, group
  // ga = col % 4) of each 4-query set qs: a lane's operand holds its query's
  // channels of group ga only where its k group grp is that group (lane group
  // grp holds channels 32 grp .. 32 grp + 31), so each column sums one group:
  // raw = sum_{j in ga} (0.5 + c_j / SB) q'_j SB = (SB / 2) Q + sum_{j in ga} c_j q'_j,
  // with Q = sum_{j in ga} q'_j (fp64, then fp32).
  const int col = lane & 15, grp = lane >> 4;
  bf16x8 Bqa[QS][4];
  float kqa[QS], Qa[QS];
  {
    const int gq = col >> 2, ga = col & 3;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      double sq = 0.0;
      for (int j = 32 * ga; j < 32 * ga + 32; ++j) sq += (double)q_lds[4 * qs + gq][j];
      Qa[qs] = (float)sq;
      kqa[qs] = (float)(sq * (double)(0.5f * SB));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float x0 = 0.0f, x1 = 0.0f;
          if (ga == grp) {
            x0 = q_lds[4 * qs + gq][score_channel<BITS>(grp, s, 2 * t)] * SB;
            x1 = q_lds[4 * qs + gq][score_channel<BITS>(grp, s, 2 * t + 1)] * SB;
          }
          v[t] = pack_bf16x2(x0, x1);  // exact: bf16 values times a power of two
        }
        Bqa[qs][s] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }

  const int tb = lane >> 2, x = lane & 3;  // 4x4x1 value product: token block, column
  const int voff = value_byte_offset<BITS>(w, x);
  constexpr int NACC = 8;  // acc[qs][k]: product k of the lane's channels
  f32x4 acc[QS][NACC];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs)
#pragma unroll
    for (int k = 0; k < NACC; ++k) acc[qs][k] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  // this lane's sum_n p_n z_n (wave w's group) for query 4 qs + x
  float zs[QS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) zs[qs] = 0.0f;
  float m_run[NQ], lsum[NQ];  // running max (uniform); this thread's sums
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    m_run[g] = NINF;
    lsum[g] = 0.0f;
  }

  // ---- records of a round: CPT 16-byte pieces per record, one load round.
  // Tokens [t0, t1) of a round have cache rows (rows r0 + t in [0, n_rows),
  // t < the round's count); the loads go through buffer resources over those
  // rows only, so that every other token reads zeros and moves no bytes.
  constexpr int CPT = REC / 16;
  constexpr int PR = KS * CPT / 256;  // pieces per thread and cache
  static_assert(PR * 256 == KS * CPT && PR <= 4, "one load round of at most four pieces");
  // piece c of a round: part c % CPT of token c / CPT
  auto piece_tok = [&](int c) __attribute__((always_inline)) -> int { return c / CPT; };
  auto piece_part = [&](int c) __attribute__((always_inline)) -> int { return c % CPT; };
  struct RoundSrc {
    int t0, t1;
    rsrc_t k, v, ks, vs, kz, vz;
  };
  constexpr uint32_t NSC = 4;  // fp16 steps and zeros per record
  const uint32_t row_stride = (uint32_t)Hkv * REC;  // bytes between cache rows (< 2^22)
  auto round_src = [&](int base) __attribute__((always_inline)) -> RoundSrc {
    const int cnt = min(cnt_all - base, KS);
    const int64_t r0 = row_base + base;
    const int64_t lo = r0 < 0 ? -r0 : 0, hi = a.n_rows - r0;
    RoundSrc R;
    R.t0 = (int)(lo < KS ? lo : KS);
    R.t1 = (int)(hi < cnt ? (hi > 0 ? hi : 0) : cnt);
    R.t1 = R.t1 > R.t0 ? R.t1 : R.t0;
    const uint32_t n = (uint32_t)(R.t1 - R.t0);
    const int64_t row = n ? r0 + R.t0 : 0;  // first present row
    R.k = buffer_rsrc(a.kc + (row * Hkv + h) * REC, n * row_stride);
    R.v = buffer_rsrc(a.vc + (row * Hkv + h) * REC, n * row_stride);
    R.ks = buffer_rsrc(a.ks + (row * Hkv + h) * NSC, n * (uint32_t)Hkv * 2u * NSC);
    R.vs = buffer_rsrc(a.vs + (row * Hkv + h) * NSC, n * (uint32_t)Hkv * 2u * NSC);
    R.kz = buffer_rsrc(a.kz + (row * Hkv + h) * NSC, n * (uint32_t)Hkv * 2u * NSC);
    R.vz = buffer_rsrc(a.vz + (row * Hkv + h) * NSC, n * (uint32_t)Hkv * 2u * NSC);
    return R;
  };
  u32x4 pk[PR], pv[PR];
  u32x2 aks[KS / 256], akz[KS / 256], avs[KS / 256], avz[KS / 256];
  auto load_round = [&](int base) __attribute__((always_inline)) {
    const RoundSrc R = round_src(base);
#pragma unroll
    for (int j = 0; j < PR; ++j) {
      const int c = tid + 256 * j;
      // (t - t0) wraps to a huge offset below the first present row
      // (24-bit multiply: |t - t0| <= 512 and row_stride < 2^22)
      const uint32_t off = (uint32_t)__mul24(piece_tok(c) - R.t0, (int)row_stride) + 16u * piece_part(c);
      pk[j] = __builtin_amdgcn_raw_buffer_load_b128(R.k, off, 0, 0);
      pv[j] = __builtin_amdgcn_raw_buffer_load_b128(R.v, off, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < KS / 256; ++j) {
      const uint32_t off = (uint32_t)__mul24(tid + 256 * j - R.t0, 8 * Hkv);
      aks[j] = __builtin_amdgcn_raw_buffer_load_b64(R.ks, off, 0, 0);
      akz[j] = __builtin_amdgcn_raw_buffer_load_b64(R.kz, off, 0, 0);
      avs[j] = __builtin_amdgcn_raw_buffer_load_b64(R.vs, off, 0, 0);
      avz[j] = __builtin_amdgcn_raw_buffer_load_b64(R.vz, off, 0, 0);
    }
  };
  // the registers of load_round(base) -> LDS: records, and per token the -inf
  // offset of an absent token and the groups' steps and zeros
  auto stage_round = [&](int base) __attribute__((always_inline)) {
    const RoundSrc R = round_src(base);
#pragma unroll
    for (int j = 0; j < PR; ++j) {
      const int c = tid + 256 * j, tok = piece_tok(c), part = piece_part(c);
      *(u32x4*)&kc_lds[16 * (tok * CPT + part)] = pk[j];
      *(u32x4*)&vc_lds[16 * (tok * CPT + part)] = pv[j];
    }
#pragma unroll
    for (int j = 0; j < KS / 256; ++j) {
      const int i = tid + 256 * j;
      const bool ok = i >= R.t0 && i < R.t1;
      off_lds[i] = ok ? 0.0f : NINF;
      // the weights are p (0 for an absent token); the group steps and zeros
      // go to the value product
      pr_lds[i] = ok ? 1.0f : 0.0f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t sw = aks[j][g >> 1] >> (16 * (g & 1)), zw = akz[j][g >> 1] >> (16 * (g & 1));
        const uint32_t vw = avs[j][g >> 1] >> (16 * (g & 1)), uw = avz[j][g >> 1] >> (16 * (g & 1));
        ksc_lds[g * KS + i] = ok ? f16_bits_to_f32((uint16_t)sw) * a.c0 : 0.0f;
        kzr_lds[g * KS + i] = ok ? f16_bits_to_f32((uint16_t)zw) * a.c0 : 0.0f;
        vsc_lds[g * KS + i] = ok ? f16_bits_to_f32((uint16_t)vw) : 0.0f;
        vzr_lds[g * KS + i] = ok ? f16_bits_to_f32((uint16_t)uw) : 0.0f;
      }
    }
  };
  for (int base = 0; base < cnt_all; base += KS) {
    const int cnt = min(cnt_all - base, KS);
    load_round(base);
    // every piece is written (tokens past the round's end read zeros), so that
    // the loads are waited for here and nowhere else
    stage_round(base);
    __syncthreads();

    // ---- scores: wave w takes 16-token tiles w, w + 4, ...
    {
      // per column (query gq, group ga): s_ga (raw - (SB / 2) Q) + z_ga Q, with the
      // step and zero already times scale * log2(e); the quad of a query's four
      // groups then sums them (every lane of the quad holds the score)
      float mxa[QS];
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) mxa[qs] = NINF;
      const int gq = col >> 2, ga = col & 3;
      for (int t0 = w; 16 * t0 < cnt; t0 += 4) {
        uint32_t W[SNW];
        load_words<SNW>(&kc_lds[(16 * t0 + col) * REC + 4 * BITS * grp], W);  // any bytes if absent
        bf16x8 A[4];
        score_operands<BITS>(W, A);
        const int i0 = 16 * t0 + 4 * grp;  // rows of the product: tokens i0 .. i0 + 3
        const float4 of4 = *(const float4*)&off_lds[i0];
        const float4 ks4 = *(const float4*)&ksc_lds[ga * KS + i0];
        const float4 kz4 = *(const float4*)&kzr_lds[ga * KS + i0];
        const float ofv[4] = {of4.x, of4.y, of4.z, of4.w};
        const float ksv[4] = {ks4.x, ks4.y, ks4.z, ks4.w}, kzv[4] = {kz4.x, kz4.y, kz4.z, kz4.w};
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < 4; ++s) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[s], Bqa[qs][s], sc, 0, 0, 0);
          float sv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float part = __builtin_fmaf(sc[e] - kqa[qs], ksv[e], kzv[e] * Qa[qs]);
            part += dpp_f32<0xB1>(part);  // quad_perm [1,0,3,2]
            part += dpp_f32<0x4E>(part);  // quad_perm [2,3,0,1]
            sv[e] = part + ofv[e];
            mxa[qs] = __builtin_fmaxf(mxa[qs], sv[e]);
          }
          if (ga == 0) *(float4*)&s_lds[4 * qs + gq][i0] = make_float4(sv[0], sv[1], sv[2], sv[3]);
        }
      }
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        float m = __builtin_fmaxf(mxa[qs], __shfl_xor(mxa[qs], 16, 64));
        m = __builtin_fmaxf(m, __shfl_xor(m, 32, 64));
        if (lane < 16 && ga == 0) mx_lds[w][4 * qs + gq] = m;
      }
    }
    __syncthreads();

    // ---- p = exp2(s - max) (0 past the round's tokens); the sums and
    // accumulators so far are rescaled to the new max
    const int n16 = (cnt + 15) & ~15;
    float alpha[NQ];
#pragma unroll
    for (int g = 0; g < NQ; ++g) {
      const float mr = __builtin_fmaxf(__builtin_fmaxf(mx_lds[0][g], mx_lds[1][g]),
                                       __builtin_fmaxf(mx_lds[2][g], mx_lds[3][g]));
      const float mn = __builtin_fmaxf(m_run[g], mr);
      // nothing seen yet: keep scale 1 and subtract 0 (every p is then 0)
      alpha[g] = m_run[g] == NINF ? 1.0f : __builtin_amdgcn_exp2f(m_run[g] - mn);
      const float msub = mn == NINF ? 0.0f : mn;
      m_run[g] = mn;
      float ls = 0.0f;
      // two consecutive tokens per thread
      for (int n = 2 * tid; n < KS; n += 512) {
        float pv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          pv[e] = 0.0f;
          if (n + e < n16) {
            const float p = __builtin_amdgcn_exp2f(s_lds[g][n + e] - msub);
            pv[e] = p * pr_lds[n + e];
            ls += p;
          }
        }
        s_lds[g][n] = pv[0];
        s_lds[g][n + 1] = pv[1];
      }
      lsum[g] = lsum[g] * alpha[g] + ls;
    }
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
      for (int k = 0; k < NACC; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[qs][k][e] *= alpha[4 * qs + e];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      const float al = x == 0 ? alpha[4 * qs] : (x == 1 ? alpha[4 * qs + 1] : (x == 2 ? alpha[4 * qs + 2] : alpha[4 * qs + 3]));
      zs[qs] *= al;
    }
    __syncthreads();

    // ---- values: wave w owns channels 32 w .. 32 w + 31 (the weights past
    // the round's tokens are 0)
    for (int u = 0; u < n16; u += 16 * PU) {
      uint32_t U[PU][VNW];
      float pa[PU][QS];
#pragma unroll
      for (int jj = 0; jj < PU; ++jj) {
        const int i = u + 16 * jj + tb;  // < KS
        load_words<VNW>(&vc_lds[i * REC + voff], U[jj]);  // any bytes if absent (its weight is 0)
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) pa[jj][qs] = s_lds[4 * qs + x][i];
        // v^ = z + c s of wave w's group: weights p s for the codes, p z summed aside
        const float vsg = vsc_lds[w * KS + i], vzg = vzr_lds[w * KS + i];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          zs[qs] = __builtin_fmaf(pa[jj][qs], vzg, zs[qs]);
          pa[jj][qs] *= vsg;
        }
      }
#pragma unroll
      for (int jj = 0; jj < PU; ++jj) {
        float Bv[8];
        value_operands<BITS>(U[jj], x, Bv);
#pragma unroll
        for (int k = 0; k < NACC; ++k)
#pragma unroll
          for (int qs = 0; qs < QS; ++qs)
            acc[qs][k] = __builtin_amdgcn_mfma_f32_4x4x1f32(pa[jj][qs], Bv[k], acc[qs][k], 0, 0, 0);
      }
    }
    __syncthreads();  // before the next round overwrites the LDS
  }

  // ---- sums over the block; the 16 token blocks of the value product
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    float ls = lsum[g];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) ls = xor_sum(ls, o);
    if (lane == 0) sum_lds[w][g] = ls;
  }
#pragma unroll
  for (int qs = 0; qs < QS; ++qs)
#pragma unroll
    for (int k = 0; k < NACC; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // the 16 token blocks (lanes x, x + 4, ..., x + 60)
        float v = acc[qs][k][e];
        v = v + dpp_f32<0x124>(v);  // row_ror:4
        v = v + dpp_f32<0x128>(v);  // row_ror:8
        v = xor_sum(v, 16);
        v = xor_sum(v, 32);
        acc[qs][k][e] = v;
      }
  // the 16 token blocks' zero sums (lanes x, x + 4, ..., x + 60), per query 4 qs + x
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    float v = zs[qs];
    v = v + dpp_f32<0x124>(v);  // row_ror:4
    v = v + dpp_f32<0x128>(v);  // row_ror:8
    v = xor_sum(v, 16);
    v = xor_sum(v, 32);
    if (lane < 4) zsum_lds[w][4 * qs + lane] = v;
  }
  __syncthreads();
  if (lane < 4) {
    const float inv = 1.0f / value_scale<BITS>(x);
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int g = 4 * qs + e;
        if (g < G) {
          float* o = a.part + (((int64_t)b * a.n_q_heads + h * G + g) * a.n_splits + split) * kPartFloats + 4;
          const float zt = zsum_lds[w][g];
#pragma unroll
          for (int k = 0; k < NACC; ++k) o[value_channel<BITS>(w, x, k)] = __builtin_fmaf(acc[qs][k][e], inv, zt);
        }
      }
  }
  if (w == 0 && lane < G) {
    const int g = lane;
    float* o = a.part + (((int64_t)b * a.n_q_heads + h * G + g) * a.n_splits + split) * kPartFloats;
    float m = m_run[0];
#pragma unroll
    for (int gg = 1; gg < NQ; ++gg)
      if (gg == g) m = m_run[gg];
    o[0] = m;
    o[1] = (sum_lds[0][g] + sum_lds[1][g]) + (sum_lds[2][g] + sum_lds[3][g]);
  }
}

// ---- decode attention for symmetric caches (2, 3 and 4 bits).
// Block map, split records and launch as attention_affine_kernel; 256 threads.  Wave
// w of a block takes the 64-token rounds w, w + 4, w + 8, ... of the block's
// split on its own: the key codes go straight from memory into registers
// and into the score product's operand layout (4 bits: lane (k group g, token
// col) loads its bytes 16 g ..; 2 bits: one 16-byte load covers two tiles and
// a swap of 16-lane rows hands each lane its 8 bytes of both), the softmax
// runs in registers with the wave's own running max, and the values pass through an LDS region of the wave's own (token-pair
// words and bf16 weight parts).  No barrier inside the loop; the four waves'
// (max, sum, output) merge once at the end.  The next round's loads are
// issued at the start of a round, so that they are in flight during its
// scores, softmax and value product.
template <int BITS, int QS>
__global__ void __launch_bounds__(256, QS == 2 ? 2 : (BITS == 2 ? 4 : 3)) attention_wave_kernel(const AttnArgs a) {
  constexpr int NW = 4;                     // waves per block
  constexpr int NQ = 4 * QS;
  constexpr int RT = 4;                    // 16-token tiles per round
  constexpr int RTOK = 16 * RT;            // tokens per round
  constexpr int REC = 16 * BITS;           // bytes per record in the cache
  // 3-bit records are widened in registers to the 4-bit layout as they
  // arrive (widen3), and everything after the loads runs as for 4 bits
  constexpr int OB = BITS == 3 ? 4 : BITS;  // bits per code in the operand layout
  constexpr int OREC = 16 * OB;            // bytes per record in that layout
  constexpr int CPT = OREC / 16;           // 16-byte pieces per record (in that layout)
  constexpr int PB = BITS == 3 ? 12 : 16;  // bytes of a piece in the cache
  constexpr float SB = BITS == 2 ? 8.0f : 32.0f;
  constexpr float M = (float)((1 << BITS) - 1) * 0.5f;
  constexpr int CPH = 16 / OB;             // channels per halfword of a record
  constexpr int NHW = OREC / 2;            // halfwords per record
  constexpr int VPR = RTOK / 2 + 4;        // pair words per halfword row (padded)
  constexpr int WPR = RTOK + 8;            // bf16 weights per column row (padded)
  constexpr int VPB = NHW * VPR * 4;       // bytes of pair words
  constexpr int WTB = QS * 16 * WPR * 2;   // bytes of weight parts
  constexpr int REDB = NQ * kD * 4;        // bytes of the merge
  constexpr int WB = VPB + WTB > REDB ? VPB + WTB : REDB;
  constexpr float NINF = -__builtin_inff();
  typedef int i32x8 __attribute__((ext_vector_type(8)));

  __shared__ __align__(16) uint8_t wbuf[NW][WB];  // per wave: pair words, weights; then its merge terms
  __shared__ __align__(16) uint8_t qtab[QS * 2048];
  __shared__ float q_lds[NQ][kD + 1];
  __shared__ float k1_lds[NQ], e_lds[NQ];
  __shared__ float mw_lds[NW][NQ], lw_lds[NW][NQ];

  // block map: as attention_affine_kernel
  const int L = blockIdx.x, xcd = L & 7, q = L >> 3;
  const int h = q % a.n_kv_heads, q2 = q / a.n_kv_heads;
  const int b = q2 / a.n_splits8, s8 = q2 - b * a.n_splits8;
  const int split = 8 * s8 + ((xcd - b) & 7);
  if (split >= a.n_splits) return;
  const int len = min(max(a.len[b], 0), a.max_len);
  const int n_lo = split * kChunk;
  if (n_lo >= len) return;  // uniform over the block
  const int cnt_all = min(len - n_lo, kChunk);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int G = a.G, Hkv = a.n_kv_heads;
  if (a.n_rows <= 0) {
    // no row exists: the split contributes nothing (max -inf, sums and output 0)
    for (int i = tid; i < G * kPartFloats; i += 256) {
      const int g = i / kPartFloats, e = i - g * kPartFloats;
      a.part[(((int64_t)b * a.n_q_heads + h * G + g) * a.n_splits + split) * kPartFloats + e] =
          e == 0 ? -__builtin_inff() : 0.0f;
    }
    return;
  }

  // ---- the paired queries as fixed-point digits: x =
  // rint(q' 2^E) with max |q'| 2^E in [2^18, 2^19) (exact for every element
  // down to 2^-11 of the largest, and within 2^-19 of it below: less than one
  // fp32 rounding of a sum over the same terms), x = d0 2^15 + d1 2^10 + d2 2^5
  // + d3 with d1..d3 in [-16, 15] and |d0| <= 16, in rows 4 (g % 4) + i of
  // query set g / 4's operand table (lane order)
  for (int i = tid; i < NQ * kD; i += 256) {
    const int g = i / kD, c = i % kD;
    q_lds[g][c] = g < G ? bf16lo_to_f32(a.qp[((int64_t)b * a.n_q_heads + h * G + g) * kD + c]) : 0.0f;
  }
  const int64_t row_base = a.row0[b] + n_lo;
  __syncthreads();
  if (tid < 32 * NQ) {
    const int g = tid >> 5, part = tid & 31;
    const float* qr = q_lds[g];
    double sq = ((double)qr[4 * part] + (double)qr[4 * part + 1]) + ((double)qr[4 * part + 2] + (double)qr[4 * part + 3]);
    float qm = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(qr[4 * part]), __builtin_fabsf(qr[4 * part + 1])),
                               __builtin_fmaxf(__builtin_fabsf(qr[4 * part + 2]), __builtin_fabsf(qr[4 * part + 3])));
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      sq += __shfl_xor(sq, o, 32);
      qm = __builtin_fmaxf(qm, __shfl_xor(qm, o, 32));
    }
    const int ex = (int)((__builtin_bit_cast(uint32_t, qm) >> 23) & 0xFFu) - 127;  // 0 or subnormal: -127
    const int E = ex < -108 ? 126 : 18 - ex;                                      // -109 .. 126
    const float sc = __builtin_bit_cast(float, (uint32_t)(E + 127) << 23);
    uint8_t* tab = qtab + (g >> 2) * 2048 + 4 * (g & 3) * 32;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ch = 4 * part + e;
      int r = (int)__builtin_rintf(qr[ch] * sc);
      int d[4];
#pragma unroll
      for (int i = 3; i > 0; --i) {
        d[i] = ((r + 16) & 31) - 16;
        r = (r - d[i]) / 32;  // exact
      }
      d[0] = r;
      // the four digits as fp8 (e4m3) bytes, exact: integers of at most 5 bits
      uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32((float)d[0], (float)d[1], 0, false);
      pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32((float)d[2], (float)d[3], (int)pk, true);
      const int pos = qpart_pos<OB>(ch);
      uint8_t* t = tab + (pos >> 5) * 512 + (pos & 31);
#pragma unroll
      for (int i = 0; i < 4; ++i) t[32 * i] = (uint8_t)(pk >> (8 * i));
    }
    if (part == 0) {
      // sum_j q'_j (c_j - m) = raw - m sum_j q'_j (the sum in fp64); raw = S 2^(shift - E):
      // shift 1 for the fp4 values c / 2, 9 for the fp8 c 2^-9
      k1_lds[g] = (float)(sq * (double)M);
      e_lds[g] = __builtin_bit_cast(float, (uint32_t)((BITS == 2 ? 128 : 136) - E) << 23);
    }
  }
  __syncthreads();
  i32x8 Aq[QS];
  float eq[QS], k1q[QS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    Aq[qs] = *(const i32x8*)(qtab + qs * 2048 + 32 * lane);
    eq[qs] = e_lds[4 * qs + grp];
    k1q[qs] = k1_lds[4 * qs + grp];
  }

  uint32_t* vp = (uint32_t*)wbuf[w];              // pair words [NHW][VPR]
  uint16_t* wt = (uint16_t*)(wbuf[w] + VPB);      // weight parts [QS][16][WPR]
  // columns 12..15 of each set's weights carry nothing
  for (int i = lane; i < QS * 4 * WPR / 8; i += 64) {
    const int qs = i / (4 * WPR / 8), r = i - qs * (4 * WPR / 8);
    *(u32x4*)(wt + qs * 16 * WPR + 12 * WPR + 8 * r) = (u32x4){0u, 0u, 0u, 0u};
  }
  // value operand of this lane: channel 16 mt + col, halfword row (16 mt + col) / CPH
  const int vrow0 = (col / CPH) * VPR;
  const int vrot = (OB * (col % CPH) - (BITS == 2 ? 5 : 3)) & 31;
  // (3 bits: the widened nibble's undefined top bit falls outside the mask)
  constexpr uint32_t VMASK = BITS == 2 ? 0x00600060u : (BITS == 3 ? 0x00380038u : 0x00780078u);

  f32x4 acc[QS][8];
  float m_run[QS], l_run[QS], vs_run[QS];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[qs][mt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    m_run[qs] = NINF;
    l_run[qs] = 0.0f;
    vs_run[qs] = 0.0f;
  }

  // ---- rounds
  struct RoundSrc {
    int t0, t1;
    rsrc_t k, v, ks, vs;
  };
  const uint32_t row_stride = (uint32_t)Hkv * REC;
  auto round_src = [&](int base) __attribute__((always_inline)) -> RoundSrc {
    const int cnt = min(cnt_all - base, RTOK);
    const int64_t r0 = row_base + base;
    const int64_t lo = r0 < 0 ? -r0 : 0, hi = a.n_rows - r0;
    RoundSrc R;
    R.t0 = (int)(lo < RTOK ? lo : RTOK);
    R.t1 = (int)(hi < cnt ? (hi > 0 ? hi : 0) : cnt);
    R.t1 = R.t1 > R.t0 ? R.t1 : R.t0;
    const uint32_t n = (uint32_t)(R.t1 - R.t0);
    const int64_t row = n ? r0 + R.t0 : 0;
    R.k = buffer_rsrc(a.kc + (row * Hkv + h) * REC, n * row_stride);
    R.v = buffer_rsrc(a.vc + (row * Hkv + h) * REC, n * row_stride);
    R.ks = buffer_rsrc(a.ks + row * Hkv + h, n * (uint32_t)Hkv * 2u);
    R.vs = buffer_rsrc(a.vs + row * Hkv + h, n * (uint32_t)Hkv * 2u);
    return R;
  };
  // piece c = lane + 64 j of a round's value records: pairs of tokens in
  // neighbouring lanes (piece (2 i + e, part) at c = 2 (CPT i + part) + e)
  auto piece_tok = [&](int c) __attribute__((always_inline)) -> int { return ((c >> 1) / CPT << 1) | (c & 1); };
  auto piece_part = [&](int c) __attribute__((always_inline)) -> int { return (c >> 1) % CPT; };
  // key codes: 2 bits, per pair of tiles (2 p, 2 p + 1) lane (g, col) loads
  // bytes 16 (g / 2) .. + 15 of token 16 (2 p + g % 2) + col, and a swap of
  // 16-lane rows hands each lane its 8 bytes of both tiles; 4 bits, per tile
  // lane (g, col) loads bytes 16 g .. + 15 of token 16 t + col
  typedef std::conditional_t<BITS == 3, u32x3, u32x4> Piece;  // a piece as loaded
  Piece kw4[RT];
  Piece vw[CPT];
  uint32_t ksw, vsw;  // the steps of token `lane` of the round
  // the lanes' offsets from the round's first row; a round subtracts t0 rows
  // (a scalar), so that a token below the first present row wraps to a huge
  // offset (|n - t0| <= 64 and row_stride < 2^22)
  const uint32_t kbase = BITS == 2 ? (uint32_t)(col + 16 * (grp & 1)) * row_stride + 16u * (grp >> 1)
                                   : (uint32_t)col * row_stride + (uint32_t)PB * grp;
  const uint32_t sbase = (uint32_t)lane * 2u * (uint32_t)Hkv;
  uint32_t vbase[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
    vbase[j] = (uint32_t)piece_tok(lane + 64 * j) * row_stride + (uint32_t)PB * piece_part(lane + 64 * j);
  // one piece of a record: 16 bytes, or (3 bits) 12 bytes, widened to 16 only
  // where it is used (widening at the load would wait for it there)
  auto load_piece = [&](rsrc_t rs, uint32_t off) __attribute__((always_inline)) -> Piece {
    if constexpr (BITS == 3) {
      return __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, 0);
    } else {
      return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    }
  };
  auto wide = [&](const Piece& x) __attribute__((always_inline)) -> u32x4 {
    if constexpr (BITS == 3) {
      return widen3(x);
    } else {
      return x;
    }
  };
  auto load_round = [&](int base) __attribute__((always_inline)) {
    const RoundSrc R = round_src(base);
#pragma unroll
    for (int t = 0; t < (BITS == 2 ? RT / 2 : RT); ++t) {
      const uint32_t off = kbase + (uint32_t)(((BITS == 2 ? 32 : 16) * t - R.t0) * (int)row_stride);
      kw4[t] = load_piece(R.k, off);
    }
    const uint32_t so = sbase - (uint32_t)R.t0 * 2u * (uint32_t)Hkv;
    ksw = __builtin_amdgcn_raw_buffer_load_b16(R.ks, so, 0, 0);
    vsw = __builtin_amdgcn_raw_buffer_load_b16(R.vs, so, 0, 0);
#pragma unroll
    for (int j = 0; j < CPT; ++j)
      vw[j] = load_piece(R.v, vbase[j] - (uint32_t)R.t0 * row_stride);
  };

  uint32_t vhi = 0x3F003F00u;  // the value operands' constant high bytes, held in a VGPR
  asm volatile("" : "+v"(vhi));
  int base = RTOK * w;
  if (base < cnt_all) load_round(base);
  for (; base < cnt_all; base += NW * RTOK) {
    const RoundSrc R = round_src(base);
    // value records -> token-pair words: halfword j of tokens 2 i and 2 i + 1
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = lane + 64 * j, tok = piece_tok(c), part = piece_part(c);
      const uint32_t sel = (tok & 1) ? 0x03020706u : 0x05040100u;
      const u32x4 vwj = wide(vw[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t own = vwj[e];
        const uint32_t oth = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)own, 0xB1, 0xF, 0xF, true);  // lane ^ 1
        vp[(2 * (4 * part + e) + (tok & 1)) * VPR + (tok >> 1)] = __builtin_amdgcn_perm(oth, own, sel);
      }
    }
    // key operands and steps of tokens 16 t + col (the steps from lane 16 t + col)
    i32x8 B[RT];
    float dk[RT], dv[RT], of[RT];
    const float dkl = f16_bits_to_f32((uint16_t)ksw) * a.c0, dvl = f16_bits_to_f32((uint16_t)vsw);
    u32x2 kw2[RT];
    if constexpr (BITS == 2) {
#pragma unroll
      for (int p = 0; p < RT / 2; ++p) {
        // odd rows of words 0, 1 <-> even rows of words 2, 3: then words 0, 1 hold
        // tile 2 p and words 2, 3 tile 2 p + 1
        const auto x0 = __builtin_amdgcn_permlane16_swap(kw4[p][0], kw4[p][2], false, false);
        const auto x1 = __builtin_amdgcn_permlane16_swap(kw4[p][1], kw4[p][3], false, false);
        kw2[2 * p] = (u32x2){x0[0], x1[0]};
        kw2[2 * p + 1] = (u32x2){x0[1], x1[1]};
      }
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      if constexpr (BITS == 2) {
        constexpr uint32_t m = 0x33333333u;
        const u32x2 wd = kw2[t];
        B[t] = (i32x8){(int)(wd[0] & m), (int)((wd[0] >> 2) & m), (int)(wd[1] & m), (int)((wd[1] >> 2) & m), 0, 0, 0, 0};
      } else {
        constexpr uint32_t m = BITS == 3 ? 0x07070707u : 0x0F0F0F0Fu;  // (3 bits: the widened codes)
        const u32x4 wd = wide(kw4[t]);
        B[t] = (i32x8){(int)(wd[0] & m), (int)((wd[0] >> 4) & m), (int)(wd[1] & m), (int)((wd[1] >> 4) & m),
                       (int)(wd[2] & m), (int)((wd[2] >> 4) & m), (int)(wd[3] & m), (int)((wd[3] >> 4) & m)};
      }
      const int n = 16 * t + col;
      const bool ok = n >= R.t0 && n < R.t1;
      dk[t] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * n, __builtin_bit_cast(int, dkl)));
      const float dvn = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * n, __builtin_bit_cast(int, dvl)));
      dv[t] = ok ? dvn : 0.0f;
      of[t] = ok ? 0.0f : NINF;
    }
    if (base + NW * RTOK < cnt_all) load_round(base + NW * RTOK);

    // ---- scores, softmax and weights: lane (query 4 qs + grp, token 16 t + col)
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float sv[RT];
      float rm = NINF;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        // the digit sums a0..a3 give S = ((a0 32 + a1) 32 + a2) 32 + a3, raw = S 2^(shift - E)
        const f32x4 sc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Aq[qs], B[t], (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 0,
                                                                          BITS == 2 ? 4 : 0, 0, 0, 0, 0);
        float S = __builtin_fmaf(sc[0], 32.0f, sc[1]);
        S = __builtin_fmaf(S, 32.0f, sc[2]);
        S = __builtin_fmaf(S, 32.0f, sc[3]);
        // (raw - k1) * step * scale * log2(e); -inf for an absent token
        sv[t] = __builtin_fmaf(__builtin_fmaf(S, eq[qs], -k1q[qs]), dk[t], of[t]);
        rm = vmax(rm, sv[t]);
      }
      rm = vmax(rm, dpp_f32<0xB1>(rm));   // quad_perm [1,0,3,2]
      rm = vmax(rm, dpp_f32<0x4E>(rm));   // quad_perm [2,3,0,1]
      rm = vmax(rm, dpp_f32<0x124>(rm));  // row_ror:4
      rm = vmax(rm, dpp_f32<0x128>(rm));  // row_ror:8
      const float mn = vmax(m_run[qs], rm);
      // nothing seen yet: keep scale 1 and subtract 0 (every p is then 0)
      const float alpha = m_run[qs] == NINF ? 1.0f : __builtin_amdgcn_exp2f(m_run[qs] - mn);
      const float msub = mn == NINF ? 0.0f : mn;
      m_run[qs] = mn;
      float ls = 0.0f, vsum = 0.0f, pv[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const float p = __builtin_amdgcn_exp2f(sv[t] - msub);
        pv[t] = p * dv[t];
        ls += p;
        vsum += pv[t];
      }
      l_run[qs] = __builtin_fmaf(l_run[qs], alpha, ls);
      vs_run[qs] = __builtin_fmaf(vs_run[qs], alpha, vsum);
      // weight parts hi + mid + lo (bf16, exact up to the last part's rounding),
      // column grp + 4 part of the set
      uint16_t* wq = wt + qs * 16 * WPR + grp * WPR + col;
#pragma unroll
      for (int t = 0; t < RT; t += 2) {
        const uint32_t hb = pack_bf16x2(pv[t], pv[t + 1]);
        const float r0 = pv[t] - bf16lo_to_f32(hb), r1 = pv[t + 1] - bf16hi_to_f32(hb);
        const uint32_t mb = pack_bf16x2(r0, r1);
        const uint32_t lb = pack_bf16x2(r0 - bf16lo_to_f32(mb), r1 - bf16hi_to_f32(mb));
        wq[16 * t] = (uint16_t)hb;
        wq[16 * t + 16] = (uint16_t)(hb >> 16);
        wq[4 * WPR + 16 * t] = (uint16_t)mb;
        wq[4 * WPR + 16 * t + 16] = (uint16_t)(mb >> 16);
        wq[8 * WPR + 16 * t] = (uint16_t)lb;
        wq[8 * WPR + 16 * t + 16] = (uint16_t)(lb >> 16);
      }
      // the accumulators' column col is query col % 4 of the set: its scale
      // from lane 16 (col % 4); skipped when no query's max moved
      const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 0));
      const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 16));
      const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 32));
      const float a3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 48));
      if (!(a0 == 1.0f && a1 == 1.0f && a2 == 1.0f && a3 == 1.0f)) {
        const int cq = col & 3;
        const float ac = cq == 0 ? a0 : (cq == 1 ? a1 : (cq == 2 ? a2 : a3));
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[qs][mt][e] *= ac;
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- values: O[ch][col] += c[ch][n] w[n][col], 32 tokens per product
#pragma unroll
    for (int ch2 = 0; ch2 < RTOK / 32; ++ch2) {
      bf16x8 P[QS];
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) P[qs] = *(const bf16x8*)(wt + qs * 16 * WPR + col * WPR + 32 * ch2 + 8 * grp);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const u32x4 wp = *(const u32x4*)(vp + vrow0 + mt * (16 / CPH) * VPR + 16 * ch2 + 4 * grp);
        u32x4 av;
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = and_or_sv(__builtin_amdgcn_alignbit(wp[i], wp[i], vrot), VMASK, vhi);
        const bf16x8 A = __builtin_bit_cast(bf16x8, av);
#pragma unroll
        for (int qs = 0; qs < QS; ++qs)
          acc[qs][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, P[qs], acc[qs][mt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the four waves: the block max, each wave's terms scaled to it
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const float ls = dpp_sum16(l_run[qs]);
    vs_run[qs] = dpp_sum16(vs_run[qs]);
    if (col == 0) {
      mw_lds[w][4 * qs + grp] = m_run[qs];
      lw_lds[w][4 * qs + grp] = ls;
    }
  }
  __syncthreads();
  float* red = (float*)wbuf[w];  // [NQ][128]: this wave's scaled output terms
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    // the three weight parts: columns c, c + 4, c + 8 (c + 12 is 0)
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = acc[qs][mt][e];
        v = v + dpp_f32<0x124>(v);  // row_ror:4
        v = v + dpp_f32<0x128>(v);  // row_ror:8
        acc[qs][mt][e] = v;
      }
    // this wave's scale for query g: lane col < 4 holds query 4 qs + col
    const int g = 4 * qs + (col & 3);
    const float mb = vmax(vmax(mw_lds[0][g], mw_lds[1][g]), vmax(mw_lds[2][g], mw_lds[3][g]));
    const float scl = mw_lds[w][g] == NINF ? 0.0f : __builtin_amdgcn_exp2f(mw_lds[w][g] - mb);
    // vs of query g: in lanes 16 (g % 4) + any
    const float vsg = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * 16 * (col & 3), __builtin_bit_cast(int, vs_run[qs])));
    const float cst = (0.5f * SB + M) * vsg;
    if (col < 4) {
      // lane (column col, group grp): channels 16 mt + 4 grp + e
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[g * kD + 16 * mt + 4 * grp + e] = scl * (SB * acc[qs][mt][e] - cst);
    }
  }
  __syncthreads();
  for (int i = tid; i < G * kD; i += 256) {
    const int g = i >> 7, c = i & 127;
    float* rec = a.part + (((int64_t)b * a.n_q_heads + h * G + g) * a.n_splits + split) * kPartFloats;
    rec[4 + c] = (((const float*)wbuf[0])[i] + ((const float*)wbuf[1])[i]) +
                 (((const float*)wbuf[2])[i] + ((const float*)wbuf[3])[i]);
    if (c == 0) {
      const float mb = vmax(vmax(mw_lds[0][g], mw_lds[1][g]), vmax(mw_lds[2][g], mw_lds[3][g]));
      float l = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) l += mw_lds[k][g] == NINF ? 0.0f : __builtin_amdgcn_exp2f(mw_lds[k][g] - mb) * lw_lds[k][g];
      rec[0] = mb;
      rec[1] = l;
    }
  }
}

// grid (Hq, B), 128 threads: out = sum_s 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s.
__global__ void __launch_bounds__(128) combine_kernel(const AttnArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int len = min(max(a.len[b], 0), a.max_len);
  const int ns = (len + kChunk - 1) / kChunk;
  const float* p = a.part + ((int64_t)b * a.n_q_heads + hq) * a.n_splits * kPartFloats;
  // the splits' maxima and sums through LDS (thread s loads split s), then
  // every thread's output column with four splits' loads in flight at a time
  __shared__ float ms[128], ls[128];
  float m = -__builtin_inff(), l = 0.0f, o = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += 128) {
    const int nb = min(ns - s0, 128);
    __syncthreads();
    if (c < nb) {
      ms[c] = p[(s0 + c) * kPartFloats];
      ls[c] = p[(s0 + c) * kPartFloats + 1];
    }
    __syncthreads();
    float mb = m;
    for (int s = 0; s < nb; ++s) mb = __builtin_fmaxf(mb, ms[s]);
    if (mb == -__builtin_inff()) continue;  // uniform: nothing present so far
    const float r = m == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m - mb);
    l *= r;
    o *= r;
    m = mb;
    int s = 0;
    for (; s + 4 <= nb; s += 4) {
      float v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = p[(s0 + s + k) * kPartFloats + 4 + c];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float f = __builtin_amdgcn_exp2f(ms[s + k] - m);
        l += f * ls[s + k];
        o += f * v[k];
      }
    }
    for (; s < nb; ++s) {
      const float f = __builtin_amdgcn_exp2f(ms[s] - m);
      l += f * ls[s];
      o += f * p[(s0 + s) * kPartFloats + 4 + c];
    }
  }
  a.out[((int64_t)b * a.n_q_heads + hq) * kD + c] = l > 0.0f ? o / l : 0.0f;
}

template <int BITS>
hipError_t launch_attention_bits(const AttnArgs& a, int qs, hipStream_t st) {
  const dim3 grid((unsigned)(8 * (int64_t)a.n_splits8 * a.n_kv_heads * a.n_seqs));
  if (a.kz) return qs == 1 ? launch_kernel(attention_affine_kernel<BITS, 1>, grid, dim3(256), st, a)
                           : launch_kernel(attention_affine_kernel<BITS, 2>, grid, dim3(256), st, a);
  return qs == 1 ? launch_kernel(attention_wave_kernel<BITS, 1>, grid, dim3(256), st, a)
                 : launch_kernel(attention_wave_kernel<BITS, 2>, grid, dim3(256), st, a);
}

}  // namespace

hipError_t launch_pair_queries(const PairArgs& a, hipStream_t st) {
  const int64_t nv = a.n_tokens * a.G;
  const dim3 grid((unsigned)((nv + kPairVecs - 1) / kPairVecs), (unsigned)a.n_kv_heads);
  return launch_kernel(pair_queries_kernel, grid, dim3(256), st, a);
}

hipError_t launch_attention(const AttnArgs& a, int bits, hipStream_t st) {
  const int qs = a.G > 4 ? 2 : 1;
  hipError_t e = hipErrorInvalidValue;
  if (a.n_splits > 0) {
    switch (bits) {
      case 2: e = launch_attention_bits<2>(a, qs, st); break;
      case 3: e = launch_attention_bits<3>(a, qs, st); break;
      case 4: e = launch_attention_bits<4>(a, qs, st); break;
    }
    if (e != hipSuccess) return e;
  }
  combine_kernel<<<dim3((unsigned)a.n_q_heads, (unsigned)a.n_seqs), dim3(128), 0, st>>>(a);
  return hipGetLastError();
}

// Split partials of the calls that bring no workspace: a buffer of fixed size
// that each GPU the library runs on holds until the process ends.  Host code
// never uses the array's name as an address: attention_scratch() returns the
// device address hipGetSymbolAddress reports for the current device, looked up
// once per device.
static __device__ __align__(256) float scratch[WUSHKV_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kScratchDevices = 64;
void* g_scratch[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t attention_scratch(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[device] = p;
  }
  *ptr = g_scratch[device];
  return hipSuccess;
}

size_t attention_workspace_bytes(int64_t n_seqs, int n_q_heads, int max_len) {
  const int64_t ns = ((int64_t)max_len + kChunk - 1) / kChunk;
  return (size_t)(n_seqs * n_q_heads * ns * kPartFloats * 4);
}

int attention_splits(int max_len) { return (max_len + kChunk - 1) / kChunk; }

}  // namespace wushkv
