// Key path with the Hadamard transform T = H_128 / 8 applied as an in-register
// fast Walsh-Hadamard transform instead of the dense MFMA product: RoPE ->
// bf16 -> FWHT (7 butterfly stages, O(d log d)) -> clipped b-bit quantizer ->
// bit packing.  The Hadamard transform is the pages' fixed-rotation baseline,
// and cheaper structured transforms are the future work they name (ai4snews
// summary "WUSH-KV cuts 2-bit KV-cache perplexity ...", method and limitations
// paragraphs; cere-bro post "WUSH-KV: 2-bit KV-Cache Quantization with
// Data-Adaptive Transforms", Gaps).  The dense key kernel computes the same y
// through any 128 x 128 matrix, this one only through H_128 / 8.
//
// Work decomposition.  A block of four waves takes a tile of 16 tokens and a
// group of up to 8 heads at a time (persistent over tiles).  The tile's
// (cos, sin) / 8 of every token and pair are computed once into LDS and shared
// by the group's heads.  A 128-channel (token, head) vector spans 16 lanes, 8
// channels per lane (channels 8 l .. 8 l + 7 of lane l), as in the value
// kernel: one 16-byte load per lane, four vectors per wave instruction.
//   RoPE: the partner channel i +- 64 sits in lane l ^ 8 and arrives through
//     DPP; the products and fma are the dense kernel's, so bf16(RoPE(k)) is the
//     same value (scaled by 1/8, an exact power of two, folded into cos/sin).
//   FWHT: channel bits 0-2 are in-lane butterflies (a + b, a - b); bits 3-6 are
//     lane bits 0-3, one stage each: u = fma(partner, c, u) with c = -1 in the
//     stage's upper lanes, which leaves each lane's value negated once per
//     upper-lane stage; one fma by the accumulated sign (plus +0, so no -0
//     reaches the quantizer) restores y = H x~ / 8 in natural row order.
//   Quantizer: the value kernel's per-vector steps (value_codes.h); sums of
//     squares in the same contiguous pairwise tree as the dense key kernel.
//   Stores: a token's records of the group's heads are one contiguous run of
//     the cache row, staged in LDS and written as 16-byte chunks.
#include "device_common.h"
#include "internal.h"
#include "value_codes.h"

namespace wushkv {

namespace {

constexpr int kTileTok = 16;  // tokens per tile
constexpr int kMaxHg = 8;     // heads per group
constexpr int kFWaves = 4;
constexpr int kRawWord3 = 0x00020000;  // raw buffer resource, 32-bit data format

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t fwht_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawWord3);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// v from lane l ^ 4 of each row of 16: banks 0 and 2 (lanes with bit 2 clear)
// read four lanes up, banks 1 and 3 four lanes down.
__device__ __forceinline__ float dpp_xor4(float v) {
  const int x = __builtin_bit_cast(int, v);
  const int lo = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0x5, false);  // row_shl:4, banks 0, 2
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(lo, x, 0x114, 0xF, 0xA, false));  // row_shr:4
}

template <int BITS, int QK, bool F32IN, bool YOUT>
__global__ void __launch_bounds__(64 * kFWaves) __attribute__((amdgpu_waves_per_eu(QK == 2 ? 2 : ((F32IN || QK) ? 3 : 4))))
keys_fwht_kernel(const KeysArgs a) {
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  constexpr int NSC = QK ? 8 : 1;  // fp16 values per (token, head): step; or 4 scales + 4 zeros
  constexpr int GPW = kTileTok * kMaxHg / 4 / kFWaves;  // 4-vector groups per wave and tile, at most
  constexpr int HALF = GPW / 2;                          // groups quantized together
  constexpr uint32_t ESZ = F32IN ? 4 : 2;
  // (cos, sin) / 8 of the tile's tokens: [0] with -sin (the lanes of channels
  // i < 64, which subtract their partner's product), [1] with +sin
  __shared__ __align__(16) float2 cs_lds[2][kTileTok][kPairs];
  __shared__ __align__(16) uint8_t rec_lds[kTileTok][kMaxHg * REC];
  __shared__ __align__(16) uint16_t sc_lds[kTileTok][kMaxHg * NSC];
  __shared__ int32_t row_lds[kTileTok];
  __shared__ float ss_lds[kFWaves][HALF * 4];
  __shared__ __align__(16) float4 th_lds[kFWaves][HALF * 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane >> 4, l16 = lane & 15;
  const int H = a.n_heads;
  const int n_hg = (H + kMaxHg - 1) / kMaxHg;
  const int hgs = (H + n_hg - 1) / n_hg;  // heads per group (the last group may have fewer)
  const int64_t n_tok = a.n_tokens;
  const int64_t n_units = ((n_tok + kTileTok - 1) / kTileTok) * n_hg;
  // lane constants: the sign of this lane's products in RoPE and of each
  // cross-lane butterfly stage, and the sign the four stages leave
  const int half = l16 >> 3;  // 0: channels i < 64 of the vector, 1: their partners i + 64
  const float c1 = (l16 & 1) ? -1.0f : 1.0f, c2 = (l16 & 2) ? -1.0f : 1.0f;
  const float c4 = (l16 & 4) ? -1.0f : 1.0f, c8 = (l16 & 8) ? -1.0f : 1.0f;
  const float sgn = (__builtin_popcount(l16) & 1) ? -1.0f : 1.0f;

  for (int64_t u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int64_t tt = u / n_hg;
    const int gi = (int)(u - tt * n_hg);
    const int h0 = gi * hgs, hg = min(hgs, H - h0);
    const int64_t n0 = tt * kTileTok;
    const int ntok = (int)min((int64_t)kTileTok, n_tok - n0);
    const int nvec = ntok * hg;  // vectors of the unit, token-major
    // this wave's vectors: groups gw = w + 4 k, vector 4 gw + sub = (token t, head hl)
    const rsrc_t kr = fwht_rsrc((const char*)a.K + (n0 * a.stride + h0 * kD) * ESZ,
                                (uint32_t)(((int64_t)(ntok - 1) * a.stride + hg * kD) * ESZ));
    u32x4 raw[GPW][F32IN ? 2 : 1];
#pragma unroll
    for (int k = 0; k < GPW; ++k) {
      const int vi = 4 * (w + kFWaves * k) + sub;
      const int t = vi / hg, hl = vi - t * hg;  // (vectors past nvec read past the resource: zeros)
      const uint32_t off = vi < nvec ? (uint32_t)(((int64_t)t * a.stride + hl * kD + 8 * l16) * ESZ) : 0xFFFFFFC0u;
#pragma unroll
      for (int q = 0; q < (F32IN ? 2 : 1); ++q) raw[k][q] = __builtin_amdgcn_raw_buffer_load_b128(kr, off + 16 * q, 0, 2);
    }
    // the tile's (cos, sin): thread (token tid / 16, pairs 2c, 2c + 1 and 2c + 32, 2c + 33), c = tid % 16
    {
      const int t = tid >> 4, c = tid & 15;
      const int64_t n = n0 + t;
      const int p = n < n_tok ? min(max(a.pos[n], 0), a.max_pos - 1) : 0;
      const uint32_t hr = ((uint32_t)p >> 5) * (uint32_t)kPairs, lr = (uint32_t)(p & 31) * kPairs;
      const uint32_t exc = a.rope_exc[p >> 5];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cc = c + 16 * j;
        const float4 v = rope2_pair_cs(p, cc, a.rope_hi[hr + 2 * cc], a.rope_hi[hr + 2 * cc + 1], exc,
                                       a.rope_lo[lr + 2 * cc], a.rope_lo[lr + 2 * cc + 1], a.rope_hit, a.rope_lot);
        const float4 s = make_float4(0.125f * v.x, 0.125f * v.y, 0.125f * v.z, 0.125f * v.w);
        *(float4*)&cs_lds[1][t][2 * cc] = s;
        *(float4*)&cs_lds[0][t][2 * cc] = make_float4(s.x, -s.y, s.z, -s.w);
      }
      if constexpr (!YOUT) {
        if (tid < kTileTok) {
          const int64_t nt = n0 + tid;
          int32_t row = -1;
          if (nt < n_tok) {
            const int64_t r = a.slots ? a.slots[nt] : nt;
            row = (r >= 0 && r < a.n_rows) ? (int32_t)r : -1;
          }
          row_lds[tid] = row;
        }
      }
    }
    __syncthreads();

#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float y[HALF][8];
#pragma unroll
      for (int kk = 0; kk < HALF; ++kk) {
        const int k = hh * HALF + kk;
        const int vi = 4 * (w + kFWaves * k) + sub;
        const int t = min(vi / hg, kTileTok - 1);
        float x[8];
        unpack_vals<F32IN>(raw[k], x);
        // RoPE: channel i (lanes 0-7 of the vector) x_i c - x_{i+64} s; channel
        // i + 64 (lanes 8-15) x_{i+64} c + x_i s; pair index 8 (l % 8) + e
        const float4* csp = (const float4*)&cs_lds[half][t][8 * (l16 & 7)];
        float r[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 cs = csp[q];
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const int e = 2 * q + e2;
            const float c = e2 ? cs.z : cs.x, s = e2 ? cs.w : cs.y;
            const float pt = dpp_mov<0x128>(x[e]) * s;  // row_ror:8: the partner lane l ^ 8
            r[e] = __builtin_fmaf(x[e], c, pt);
          }
        }
        // bf16 rounding (the transform's input is bf16, as on the MFMA path)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t b = pack_bf16x2(r[e], r[e + 1]);
          r[e] = bf16lo_to_f32(b);
          r[e + 1] = bf16hi_to_f32(b);
        }
        // in-lane butterflies over channel bits 0, 1, 2
#pragma unroll
        for (int m = 1; m < 8; m <<= 1)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!(e & m)) {
              const float p0 = r[e], p1 = r[e + m];
              r[e] = p0 + p1;
              r[e + m] = p0 - p1;
            }
        // cross-lane butterflies over channel bits 3..6 (lane bits 0..3)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v = r[e];
          v = __builtin_fmaf(dpp_mov<0xB1>(v), c1, v);  // quad_perm [1,0,3,2]: lane ^ 1
          v = __builtin_fmaf(dpp_mov<0x4E>(v), c2, v);  // quad_perm [2,3,0,1]: lane ^ 2
          v = __builtin_fmaf(dpp_xor4(v), c4, v);       // lane ^ 4
          v = __builtin_fmaf(dpp_mov<0x128>(v), c8, v); // row_ror:8: lane ^ 8
          y[kk][e] = __builtin_fmaf(v, sgn, 0.0f);
        }
        if constexpr (YOUT) {
          if (vi < nvec) {
            const int hl = vi - (vi / hg) * hg;
            float* dst = a.y_out + (((n0 + vi / hg) * H + h0 + hl) * kD + 8 * l16);
            *(float4*)dst = make_float4(y[kk][0], y[kk][1], y[kk][2], y[kk][3]);
            *(float4*)(dst + 4) = make_float4(y[kk][4], y[kk][5], y[kk][6], y[kk][7]);
          }
        } else if constexpr (QK == 0) {
          const float P = dpp_sum16(lane_sumsq8(y[kk]));
          if (l16 == 0) ss_lds[w][4 * kk + sub] = P;
        }
      }
      if constexpr (!YOUT) {
        if constexpr (QK == 0) {
          // one lane per vector: the step (of y = H x~ / 8), its fp16 bits and thresholds
          if (lane < 4 * HALF) {
            const int kk = lane >> 2, sb = lane & 3;
            const int vi = 4 * (w + kFWaves * (hh * HALF + kk)) + sb;
            const uint16_t sc = sym_step_f16<L>(ss_lds[w][lane], a.q.alpha);
            if (vi < nvec) {
              const int t = vi / hg;
              sc_lds[t][vi - t * hg] = sc;
            }
            const float delta = f16_bits_to_f32(sc);
            if constexpr (BITS == 2) {
              th_lds[w][lane] = make_float4(delta, 0.0f, 0.0f, 0.0f);
            } else {
              th_lds[w][lane] = value_thresholds<BITS>(delta);
            }
          }
        }
#pragma unroll
        for (int kk = 0; kk < HALF; ++kk) {
          const int vi = 4 * (w + kFWaves * (hh * HALF + kk)) + sub;
          const int t = vi / hg, hl = vi - t * hg;
          uint32_t packed;
          if constexpr (QK == 0) {
            const float4 th = th_lds[w][4 * kk + sub];
            if constexpr (BITS == 2) {
              packed = sym2_bits8(y[kk], th.x);  // th.x: the step (0: every code is 2); y is never -0 here
            } else {
              packed = value_codes_sym<BITS>(y[kk], th);
            }
          } else {
            uint16_t sh, zh;
            packed = value_codes_affine<BITS, QK == 2>(y[kk], a.q, sh, zh);
            if ((l16 & 3) == 0 && vi < nvec) {
              sc_lds[t][hl * 8 + (l16 >> 2)] = sh;
              sc_lds[t][hl * 8 + 4 + (l16 >> 2)] = zh;
            }
          }
          if (vi < nvec) {
            uint8_t* dst = &rec_lds[t][hl * REC + BITS * l16];
            if constexpr (BITS == 2) {
              *(uint16_t*)dst = (uint16_t)packed;
            } else if constexpr (BITS == 4) {
              *(uint32_t*)dst = packed;
            } else {
              dst[0] = (uint8_t)packed;
              dst[1] = (uint8_t)(packed >> 8);
              dst[2] = (uint8_t)(packed >> 16);
            }
          }
        }
      }
    }
    __syncthreads();
    if constexpr (!YOUT) {
      // the unit's records: token t's run of the group's heads, 16-byte chunks
      const int cpt = hg * BITS;  // chunks per token
      const uint32_t row_rec = (uint32_t)H * REC;
      for (int c = tid; c < ntok * cpt; c += 64 * kFWaves) {
        const int t = c / cpt, k = c - t * cpt;
        const int32_t row = row_lds[t];
        if (row >= 0) {
          const u32x4 v = *(const u32x4*)&rec_lds[t][16 * k];
          __builtin_nontemporal_store(v, (u32x4*)(a.codes + (uint64_t)(uint32_t)row * row_rec + h0 * REC + 16 * k));
        }
      }
      if (tid < ntok * hg) {
        const int t = tid / hg, hl = tid - t * hg;
        const int32_t row = row_lds[t];
        if (row >= 0) {
          const uint64_t slot = (uint64_t)(uint32_t)row * H + h0 + hl;
          if constexpr (QK == 0) {
            a.scales[slot] = sc_lds[t][hl];
          } else {
            *(uint2*)(a.scales + slot * 4) = *(const uint2*)&sc_lds[t][hl * 8];
            *(uint2*)(a.zeros + slot * 4) = *(const uint2*)&sc_lds[t][hl * 8 + 4];
          }
        }
      }
    }
    __syncthreads();  // the LDS of this unit is read before the next unit writes it
  }
}

// As many blocks as fit on the chip at once, then as few as give every block
// the same number of units.
template <int BITS, int QK, bool F32IN, bool YOUT>
hipError_t launch_fwht_one(const KeysArgs& a, int cus, hipStream_t st) {
  constexpr auto k = keys_fwht_kernel<BITS, QK, F32IN, YOUT>;
  static int occ = 0;
  if (!occ) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, 64 * kFWaves, 0) != hipSuccess || n < 1) n = 1;
    occ = n;
  }
  const int n_hg = (a.n_heads + kMaxHg - 1) / kMaxHg;
  const int64_t units = (a.n_tokens + kTileTok - 1) / kTileTok * n_hg;
  if (units <= 0) return hipSuccess;
  const int64_t cap = (int64_t)cus * occ;
  const int64_t per_block = (units + cap - 1) / cap;
  const int64_t blocks = (units + per_block - 1) / per_block;
  return launch_kernel(k, dim3((unsigned)blocks), dim3(64 * kFWaves), st, a);
}

template <int BITS, int QK>
hipError_t launch_fwht_bits(const KeysArgs& a, int f32_in, int cus, hipStream_t st) {
  return f32_in ? launch_fwht_one<BITS, QK, true, false>(a, cus, st)
                : launch_fwht_one<BITS, QK, false, false>(a, cus, st);
}

}  // namespace

hipError_t launch_keys_fwht(const KeysArgs& a, int bits, int f32_in, int y_out, int cus, hipStream_t st) {
  if (y_out) return f32_in ? launch_fwht_one<2, 0, true, true>(a, cus, st) : launch_fwht_one<2, 0, false, true>(a, cus, st);
  const int kind = a.q.kind;
  switch (bits) {
    case 2: return kind == 0 ? launch_fwht_bits<2, 0>(a, f32_in, cus, st)
                             : (kind == 1 ? launch_fwht_bits<2, 1>(a, f32_in, cus, st) : launch_fwht_bits<2, 2>(a, f32_in, cus, st));
    case 3: return kind == 0 ? launch_fwht_bits<3, 0>(a, f32_in, cus, st)
                             : (kind == 1 ? launch_fwht_bits<3, 1>(a, f32_in, cus, st) : launch_fwht_bits<3, 2>(a, f32_in, cus, st));
    case 4: return kind == 0 ? launch_fwht_bits<4, 0>(a, f32_in, cus, st)
                             : (kind == 1 ? launch_fwht_bits<4, 1>(a, f32_in, cus, st) : launch_fwht_bits<4, 2>(a, f32_in, cus, st));
  }
  return hipErrorInvalidValue;
}

}  // namespace wushkv
