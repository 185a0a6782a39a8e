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
//   * attention_kernel: one block of four waves per (2048-token split, KV
//     head, sequence), in rounds of 512 tokens (256 at 3 and 4 bits) whose
//     key and value records are first copied to LDS with all loads in flight
//     at once (at 2 and 4 bits, the next round's during this round's work).
//       scores  S[n][g] = sum_j code-operand[n][j] * q'[g][j] on
//               v_mfma_f32_16x16x32_bf16 (16 tokens x 16 columns, G used);
//               the key codes enter as exact bf16 values 0.5 + c / SB built
//               with one shift, mask and v_perm per pair of codes, and the
//               constant part is subtracted after the product.
//       softmax p = exp2(s - max) over the split, then p * step_v.
//       values  O[ch][g] += c[ch][n] * p[n][g] on v_mfma_f32_16x16x32_bf16
//               (2 and 4 bits): rows = 16 channels, k = 32 tokens from the
//               value records stored transposed in LDS, columns = the query
//               heads' weights p * step_v split into three bf16 parts (exact
//               to fp32).  3-bit codes straddle words: v_mfma_f32_4x4x1f32
//               with fp32 weights (16 blocks = 16 tokens, rows = queries).
//     A split writes (max, sum, unnormalized output) per query head.
//   * combine_kernel merges the splits of a sequence.
#include "device_common.h"
#include "internal.h"

namespace wushkv {

namespace {

constexpr int kChunk = 2048;     // tokens per split (one block)
constexpr int kSub = 512;        // tokens staged in LDS per round
constexpr int kPartFloats = 132;  // per (sequence, query head, split): max, sum, 2 pad, o[128]
constexpr int kPairVecs = 4;      // query vectors per pairing block

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// grid 8 * n_splits8 * Hkv * B blocks (see the block map below), 256 threads.
// A block takes up to kChunk tokens of one sequence and KV head, in rounds of
// KS tokens, with the running max, sums and value accumulators rescaled from
// round to round (online softmax).
template <int BITS, int QS>
__global__ void __launch_bounds__(256, QS == 1 ? 3 : 2) attention_kernel(const AttnArgs a) {
  constexpr int NQ = 4 * QS;   // query rows of the value product (G <= NQ)
  // tokens per round: 512, or 256 for 3- and 4-bit records (so that three
  // blocks' LDS fits a CU and a 4-bit round's records fit one load round)
  constexpr int KS = BITS == 2 ? kSub : kSub / 2;
  constexpr int REC = 16 * BITS;
  constexpr int SNW = BITS;    // words of key codes per lane (32 channels)
  constexpr int VNW = BITS == 3 ? 3 : 2;  // words of value codes per lane
  constexpr float SB = BITS == 2 ? 8.0f : (BITS == 3 ? 16.0f : 32.0f);
  constexpr float M = (float)((1 << BITS) - 1) * 0.5f;
  constexpr int SROW = KS + 16;  // s_lds row (padded against bank conflicts)
  constexpr float NINF = -__builtin_inff();
  constexpr int PU = BITS == 2 ? 4 : 2;   // value steps per pass (4x4x1 product)
  constexpr bool TWO = BITS == 2;         // score tiles two at a time
  // 2 and 4 bits: the value product runs on bf16 16x16x32 MFMA with the value
  // records stored transposed (word w of token n at vt[w][n]) and the weights
  // split into three bf16 parts (columns g + 4 part); 3 bits: fp32 4x4x1 MFMA.
  constexpr bool VT = BITS != 3;
  constexpr int NWV = REC / 4;            // words per record
  constexpr int VROW = KS + 4;          // vt row (u32)
  constexpr int PROW = KS + 8;          // weight row (bf16), 16-byte pieces spread over the banks
  constexpr int KBYTES = KS * REC > QS * 16 * PROW * 2 ? KS * REC : QS * 16 * PROW * 2;

  // the round's key records; after the scores, the bf16 weights [QS][16][PROW]
  __shared__ __align__(16) uint8_t kc_lds[KBYTES];
  __shared__ __align__(16) uint8_t vc_lds[VT ? NWV * VROW * 4 : KS * REC];  // value records
  __shared__ __align__(16) float s_lds[NQ][SROW];       // scores (log2 units), then p * step_v
  __shared__ __align__(16) float dk_lds[KS];          // key step * scale * log2(e); 0: token absent
  __shared__ __align__(16) float off_lds[KS];         // 0, or -inf for an absent token
  __shared__ float dv_lds[KS];                        // value step
  __shared__ float q_lds[NQ][kD + 1];
  __shared__ float k1_lds[NQ];
  __shared__ float mx_lds[4][NQ];
  __shared__ float sum_lds[4][NQ][2];

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
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
  if (tid < 32 * NQ) {
    // sum_j q'_j (c_j - m) = raw - (SB / 2 + m) sum_j q'_j; the sum in fp64
    const int g = tid >> 5, part = tid & 31;
    double sq = ((double)q_lds[g][4 * part] + (double)q_lds[g][4 * part + 1]) +
                ((double)q_lds[g][4 * part + 2] + (double)q_lds[g][4 * part + 3]);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) sq += __shfl_xor(sq, o, 32);
    if (part == 0) k1_lds[g] = (float)(sq * (double)(0.5f * SB + M));
  }

  // score operands of the paired queries: lane (column col, group grp)
  const int col = lane & 15, grp = lane >> 4;
  bf16x8 Bq[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 v;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x0 = 0.0f, x1 = 0.0f;
      if (col < NQ) {
        x0 = q_lds[col][score_channel<BITS>(grp, s, 2 * t)] * SB;
        x1 = q_lds[col][score_channel<BITS>(grp, s, 2 * t + 1)] * SB;
      }
      v[t] = pack_bf16x2(x0, x1);  // exact: bf16 values times a power of two
    }
    Bq[s] = __builtin_bit_cast(bf16x8, v);
  }

  const int tb = lane >> 2, x = lane & 3;  // 4x4x1 value product: token block, column
  const int voff = value_byte_offset<BITS>(w, x);
  // 4x4x1: acc[qs][k]; 16x16x32: acc[qs][mt] (mt = 16-channel tile) in acc[qs][0..1]
  constexpr int NACC = VT ? 2 : 8;
  f32x4 acc[QS][NACC];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs)
#pragma unroll
    for (int k = 0; k < NACC; ++k) acc[qs][k] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  // 16x16x32 value product: lane (row vr_ch = 16 mt + lane % 16 of the wave's
  // 32 channels, k group grp = 8 tokens); the code's word, byte and bit
  const int vch = 32 * w + (lane & 15);  // + 16 mt
  int vword[2], vrot[2];
  uint32_t vsel[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int j = vch + 16 * mt;
    const int bit = BITS * j;                   // in the record's bit stream
    vword[mt] = bit >> 5;
    const int byte = (bit & 31) >> 3, inb = bit & 7;
    vsel[mt] = (uint32_t)byte | 0x0C00u | ((uint32_t)(4 + byte) << 16) | 0x0C000000u;
    // rotate the code from bit inb of each half's low byte to bit SH (5: 2 bits, 3: 4 bits)
    vrot[mt] = (inb - (BITS == 2 ? 5 : 3)) & 31;
  }
  float m_run[NQ], lsum[NQ], vsum[NQ];  // running max (uniform); this thread's sums
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    m_run[g] = NINF;
    lsum[g] = 0.0f;
    vsum[g] = 0.0f;
  }
  float k1 = 0.0f;

  // ---- records of a round: CPT 16-byte pieces per record; rows outside the
  // cache are read from row 0 and never used (their key step marks them absent)
  constexpr int CPT = REC / 16;
  constexpr int NLD = KS * CPT / 256;  // pieces per thread and cache
  constexpr int NR = NLD > 4 ? 2 : 1;    // load rounds (at most 4 + 4 pieces in registers)
  constexpr int PR = NLD / NR;
  // one load round: the next round's records and steps are loaded into
  // registers while this round is worked on, and go to LDS at its end
  constexpr bool PF = NR == 1 && VT;
  static_assert(!PF || VT, "the prefetch path writes the transposed value layout");
  u32x4 pk[PR], pv[PR];
  uint32_t pks[KS / 256], pvs[KS / 256];
  auto prefetch = [&](int base) __attribute__((always_inline)) {
    const int cnt = min(cnt_all - base, KS);
    if (cnt <= 0) return;  // uniform
    const int64_t r0 = row_base + base;
#pragma unroll
    for (int j = 0; j < PR; ++j) {
      const int c = tid + 256 * j, tok = c / CPT, part = c - tok * CPT;
      if (tok < cnt) {
        int64_t row = r0 + tok;
        row = (row >= 0 && row < a.n_rows) ? row : 0;
        const int64_t off = (row * Hkv + h) * REC + 16 * part;
        pk[j] = *(const u32x4*)(a.kc + off);
        pv[j] = *(const u32x4*)(a.vc + off);
      }
    }
#pragma unroll
    for (int j = 0; j < KS / 256; ++j) {
      const int i = tid + 256 * j;
      if (i < cnt) {
        int64_t row = r0 + i;
        row = (row >= 0 && row < a.n_rows) ? row : 0;
        pks[j] = a.ks[row * Hkv + h];
        pvs[j] = a.vs[row * Hkv + h];
      }
    }
  };
  if constexpr (PF) prefetch(0);

  for (int base = 0; base < cnt_all; base += KS) {
    const int cnt = min(cnt_all - base, KS);
    const int64_t r0 = row_base + base;
    if constexpr (PF) {
      {
        // written for every piece, also past the round's tokens (whose
        // registers hold stale bits: those tokens are absent), so that every
        // load is waited for here and nowhere else
#pragma unroll
        for (int j = 0; j < PR; ++j) {
          const int c = tid + 256 * j;
          *(u32x4*)&kc_lds[16 * c] = pk[j];
          const int tok = c / CPT, part = c - tok * CPT;
          uint32_t* vt = (uint32_t*)vc_lds;
#pragma unroll
          for (int e = 0; e < 4; ++e) vt[(4 * part + e) * VROW + tok] = pv[j][e];
        }
#pragma unroll
        for (int j = 0; j < KS / 256; ++j) {
          const int i = tid + 256 * j;
          const int64_t row = r0 + i;
          const bool ok = i < cnt && row >= 0 && row < a.n_rows;
          dk_lds[i] = ok ? f16_bits_to_f32((uint16_t)pks[j]) * a.c0 : 0.0f;
          off_lds[i] = ok ? 0.0f : NINF;
          dv_lds[i] = ok ? f16_bits_to_f32((uint16_t)pvs[j]) : 0.0f;
        }
      }
      __syncthreads();
      prefetch(base + KS);
    } else {
    {
#pragma unroll
      for (int rd = 0; rd < NR; ++rd) {
        u32x4 kr[PR], vr[PR];
#pragma unroll
        for (int j = 0; j < PR; ++j) {
          const int c = tid + 256 * (rd * PR + j), tok = c / CPT, part = c - tok * CPT;
          if (tok < cnt) {
            int64_t row = r0 + tok;
            row = (row >= 0 && row < a.n_rows) ? row : 0;
            const int64_t off = (row * Hkv + h) * REC + 16 * part;
            kr[j] = *(const u32x4*)(a.kc + off);
            vr[j] = *(const u32x4*)(a.vc + off);
          }
        }
        if (rd == 0) {
          for (int i = tid; i < KS; i += 256) {
            float dk = 0.0f, off = NINF, dv = 0.0f;
            const int64_t row = r0 + i;
            if (i < cnt && row >= 0 && row < a.n_rows) {
              dk = f16_bits_to_f32(a.ks[row * Hkv + h]) * a.c0;
              off = 0.0f;
              dv = f16_bits_to_f32(a.vs[row * Hkv + h]);
            }
            dk_lds[i] = dk;
            off_lds[i] = off;
            dv_lds[i] = dv;
          }
        }
        // written for every piece (past the round's tokens: stale bits of
        // absent tokens), so that the loads are waited for here only
#pragma unroll
        for (int j = 0; j < PR; ++j) {
          const int c = tid + 256 * (rd * PR + j);
          *(u32x4*)&kc_lds[16 * c] = kr[j];
          if constexpr (VT) {
            const int tok = c / CPT, part = c - tok * CPT;
            uint32_t* vt = (uint32_t*)vc_lds;
#pragma unroll
            for (int e = 0; e < 4; ++e) vt[(4 * part + e) * VROW + tok] = vr[j][e];
          } else {
            *(u32x4*)&vc_lds[16 * c] = vr[j];
          }
        }
      }
    }
    __syncthreads();
    }
    if (base == 0) k1 = col < NQ ? k1_lds[col] : 0.0f;

    // ---- scores: wave w takes 16-token tiles w, w + 4, ... (two at a time)
    float mx = NINF;
    for (int t0 = w; 16 * t0 < cnt; t0 += TWO ? 8 : 4) {
      const bool two = TWO && 16 * (t0 + 4) < cnt;  // uniform over the wave
      uint32_t W[2][SNW];
      load_words<SNW>(&kc_lds[(16 * t0 + col) * REC + 4 * BITS * grp], W[0]);  // any bytes if absent
      if (two) load_words<SNW>(&kc_lds[(16 * t0 + 64 + col) * REC + 4 * BITS * grp], W[1]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (j == 1 && !two) break;
        const int t = t0 + 4 * j;
        bf16x8 A[4];
        score_operands<BITS>(W[j], A);
        f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[s], Bq[s], sc, 0, 0, 0);
        // sc[e]: token 16 t + 4 grp + e, query head col
        const int i0 = 16 * t + 4 * grp;
        const float4 dk4 = *(const float4*)&dk_lds[i0];
        const float4 of4 = *(const float4*)&off_lds[i0];
        const float dkv[4] = {dk4.x, dk4.y, dk4.z, dk4.w}, ofv[4] = {of4.x, of4.y, of4.z, of4.w};
        float sv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // (raw - k1) * step * scale * log2(e); -inf for an absent token
          sv[e] = __builtin_fmaf(sc[e] - k1, dkv[e], ofv[e]);
          mx = __builtin_fmaxf(mx, sv[e]);
        }
        if (col < NQ) *(float4*)&s_lds[col][i0] = make_float4(sv[0], sv[1], sv[2], sv[3]);
      }
    }
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (lane < NQ) mx_lds[w][lane] = mx;
    __syncthreads();

    // ---- p = exp2(s - max) and p * step_v (0 past the round's tokens); the
    // sums and accumulators so far are rescaled to the new max
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
      float ls = 0.0f, vs = 0.0f;
      // two consecutive tokens per thread (paired bf16 writes)
      for (int n = 2 * tid; n < KS; n += 512) {
        float pv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          pv[e] = 0.0f;
          if (n + e < n16) {
            const float p = __builtin_amdgcn_exp2f(s_lds[g][n + e] - msub);
            pv[e] = p * dv_lds[n + e];
            ls += p;
            vs += pv[e];
          }
        }
        if constexpr (VT) {
          // pv = hi + mid + lo in bf16 (exact up to the last part's rounding)
          uint32_t* pt = (uint32_t*)((uint16_t*)kc_lds + (g >> 2) * 16 * PROW + (g & 3) * PROW + n);
          const uint32_t hb = pack_bf16x2(pv[0], pv[1]);
          const float r10 = pv[0] - bf16lo_to_f32(hb), r11 = pv[1] - bf16hi_to_f32(hb);
          const uint32_t mb = pack_bf16x2(r10, r11);
          const float r20 = r10 - bf16lo_to_f32(mb), r21 = r11 - bf16hi_to_f32(mb);
          pt[0] = hb;
          pt[2 * PROW] = mb;
          pt[4 * PROW] = pack_bf16x2(r20, r21);
        } else {
          s_lds[g][n] = pv[0];
          s_lds[g][n + 1] = pv[1];
        }
      }
      lsum[g] = lsum[g] * alpha[g] + ls;
      vsum[g] = vsum[g] * alpha[g] + vs;
    }
    if constexpr (VT) {
      // weight columns 12..15 carry nothing (they overlay last round's key records)
      for (int i = tid; i < QS * 4 * PROW / 8; i += 256) {
        const int qs = i / (4 * PROW / 8), r = i - qs * (4 * PROW / 8);
        *(u32x4*)((uint16_t*)kc_lds + qs * 16 * PROW + 12 * PROW + 8 * r) = (u32x4){0u, 0u, 0u, 0u};
      }
      // column col = g + 4 part of the weights: query 4 qs + col % 4
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        const int cg = col & 3;
        const float al = cg == 0 ? alpha[4 * qs] : (cg == 1 ? alpha[4 * qs + 1] : (cg == 2 ? alpha[4 * qs + 2] : alpha[4 * qs + 3]));
#pragma unroll
        for (int k = 0; k < NACC; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[qs][k][e] *= al;
      }
    } else {
#pragma unroll
      for (int qs = 0; qs < QS; ++qs)
#pragma unroll
        for (int k = 0; k < NACC; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[qs][k][e] *= alpha[4 * qs + e];
    }
    __syncthreads();

    // ---- values: wave w owns channels 32 w .. 32 w + 31 (the weights past
    // the round's tokens are 0)
    if constexpr (VT) {
      const uint32_t* vt = (const uint32_t*)vc_lds;
      const uint16_t* pt = (const uint16_t*)kc_lds;
      constexpr uint32_t VMASK = BITS == 2 ? 0x00600060u : 0x00780078u;
      for (int n0 = 0; n0 < n16; n0 += 32) {
        const int nk = n0 + 8 * grp;  // this lane's 8 tokens
        bf16x8 P[QS];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) P[qs] = *(const bf16x8*)(pt + qs * 16 * PROW + col * PROW + nk);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const u32x4 wa = *(const u32x4*)(vt + vword[mt] * VROW + nk);
          const u32x4 wb = *(const u32x4*)(vt + vword[mt] * VROW + nk + 4);
          const uint32_t wv[8] = {wa[0], wa[1], wa[2], wa[3], wb[0], wb[1], wb[2], wb[3]};
          u32x4 av;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t pr = __builtin_amdgcn_perm(wv[2 * t + 1], wv[2 * t], vsel[mt]);
            av[t] = (__builtin_amdgcn_alignbit(pr, pr, vrot[mt]) & VMASK) | 0x3F003F00u;
          }
          const bf16x8 A = __builtin_bit_cast(bf16x8, av);
#pragma unroll
          for (int qs = 0; qs < QS; ++qs)
            acc[qs][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, P[qs], acc[qs][mt], 0, 0, 0);
        }
      }
    } else
    for (int u = 0; u < n16; u += 16 * PU) {
      uint32_t U[PU][VNW];
      float pa[PU][QS];
#pragma unroll
      for (int jj = 0; jj < PU; ++jj) {
        const int i = u + 16 * jj + tb;  // < KS
        load_words<VNW>(&vc_lds[i * REC + voff], U[jj]);  // any bytes if absent (its weight is 0)
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) pa[jj][qs] = s_lds[4 * qs + x][i];
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
    float ls = lsum[g], vs = vsum[g];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      ls = xor_sum(ls, o);
      vs = xor_sum(vs, o);
    }
    if (lane == 0) {
      sum_lds[w][g][0] = ls;
      sum_lds[w][g][1] = vs;
    }
  }
#pragma unroll
  for (int qs = 0; qs < QS; ++qs)
#pragma unroll
    for (int k = 0; k < NACC; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // 16x16x32: the three weight parts (columns c, c + 4, c + 8; c + 12 is 0);
        // 4x4x1: the 16 token blocks (lanes x, x + 4, ..., x + 60)
        float v = acc[qs][k][e];
        v = v + dpp_f32<0x124>(v);  // row_ror:4
        v = v + dpp_f32<0x128>(v);  // row_ror:8
        if constexpr (!VT) {
          v = xor_sum(v, 16);
          v = xor_sum(v, 32);
        }
        acc[qs][k][e] = v;
      }
  __syncthreads();
  if constexpr (VT) {
    if (col < 4) {
      // lane (column col, group grp): channels 32 w + 16 mt + 4 grp + e
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        const int g = 4 * qs + col;
        if (g < G) {
          const float vs = (sum_lds[0][g][1] + sum_lds[1][g][1]) + (sum_lds[2][g][1] + sum_lds[3][g][1]);
          const float cst = (0.5f * SB + M) * vs;
          float* o = a.part + (((int64_t)b * a.n_q_heads + h * G + g) * a.n_splits + split) * kPartFloats + 4;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[32 * w + 16 * mt + 4 * grp + e] = SB * acc[qs][mt][e] - cst;
        }
      }
    }
  } else if (lane < 4) {
    const float inv = 1.0f / value_scale<BITS>(x);
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int g = 4 * qs + e;
        if (g < G) {
          const float vs = (sum_lds[0][g][1] + sum_lds[1][g][1]) + (sum_lds[2][g][1] + sum_lds[3][g][1]);
          float* o = a.part + (((int64_t)b * a.n_q_heads + h * G + g) * a.n_splits + split) * kPartFloats + 4;
#pragma unroll
          for (int k = 0; k < NACC; ++k) o[value_channel<BITS>(w, x, k)] = acc[qs][k][e] * inv - M * vs;
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
    o[1] = (sum_lds[0][g][0] + sum_lds[1][g][0]) + (sum_lds[2][g][0] + sum_lds[3][g][0]);
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
  return qs == 1 ? launch_kernel(attention_kernel<BITS, 1>, grid, dim3(256), st, a)
                 : launch_kernel(attention_kernel<BITS, 2>, grid, dim3(256), st, a);
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

size_t attention_workspace_bytes(int64_t n_seqs, int n_q_heads, int max_len) {
  const int64_t ns = ((int64_t)max_len + kChunk - 1) / kChunk;
  return (size_t)(n_seqs * n_q_heads * ns * kPartFloats * 4);
}

int attention_splits(int max_len) { return (max_len + kChunk - 1) / kChunk; }

}  // namespace wushkv
