// Read path for gfx950: unpack -> dequantize, optionally through T_k^-1.
//
// Symmetric records decode exactly to (q - (2^b-1)/2) * step; affine records
// to RN32(zero + q * step).  For keys read back through T_k^-1 the scale is
// factored out of the contraction so that the MFMA operands are exact small
// integers in bf16:
//   sym:    k^ = (step/2) * (T~inv w),          w_j = 2 q_j - (2^b - 1)
//   affine: k^_r = sum_g step_g * (T~inv|g q)_r + zero_g * G_g[r],
//           G_g[r] = sum_{j in group g} T~inv[r][j]   (precomputed per head)
// The work decomposition of the MFMA kernel mirrors the key kernel: two waves
// per head, each holding half of T~inv's rows as A operands, 32-token tiles.
#include "device_common.h"
#include "internal.h"

namespace wushkv {

namespace {

constexpr int kWaves = 4;
constexpr int kPerWave = 16;
constexpr int kVecs = kWaves * kPerWave;
constexpr int kTile = 32;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 codes of channels 8*k .. 8*k+7 from a record held as dwords.
template <int BITS>
__device__ __forceinline__ uint32_t codes8(const uint32_t* w, int k) {
  if constexpr (BITS == 2) {
    return (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
  } else if constexpr (BITS == 4) {
    return w[k];
  } else {
    const int bit = 24 * k, d = bit >> 5, sh = bit & 31;
    const uint64_t lo = w[d];
    const uint64_t hi = (d + 1 < 12) ? (uint64_t)w[d + 1] : 0ull;
    return (uint32_t)(((hi << 32) | lo) >> sh) & 0xFFFFFFu;
  }
}

template <int BITS, int QK, bool BF16OUT>
__global__ void __launch_bounds__(64 * kWaves) dequant_plain_kernel(const DequantArgs a) {
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = lane >> 4, l16 = lane & 15;
  const int64_t nv = a.n_tokens * a.n_heads;
  const int64_t n_iter = (nv + kVecs - 1) / kVecs;
  for (int64_t it = blockIdx.x; it < n_iter; it += gridDim.x) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t v = it * kVecs + wave * kPerWave + 4 * u + sub;
      if (v >= nv) continue;
      const int64_t n = v / a.n_heads;
      const int h = (int)(v - n * a.n_heads);
      const int64_t row = a.slots ? a.slots[n] : n;
      float y[8];
      if (row >= 0 && row < a.n_rows) {
        const int64_t slot = row * a.n_heads + h;
        const uint8_t* rec = a.codes + slot * REC + BITS * l16;
        uint32_t c;
        if constexpr (BITS == 2) c = *(const uint16_t*)rec;
        else if constexpr (BITS == 4) c = *(const uint32_t*)rec;
        else c = (uint32_t)rec[0] | ((uint32_t)rec[1] << 8) | ((uint32_t)rec[2] << 16);
        if constexpr (QK == 0) {
          const float hs = 0.5f * f16_bits_to_f32(a.scales[slot]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int q = (c >> (BITS * e)) & (L - 1);
            y[e] = (float)(2 * q - (L - 1)) * hs;
          }
        } else {
          const int g = l16 >> 2;
          const float s = f16_bits_to_f32(a.scales[slot * 4 + g]);
          const float z = f16_bits_to_f32(a.zeros[slot * 4 + g]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int q = (c >> (BITS * e)) & (L - 1);
            y[e] = __builtin_fmaf((float)q, s, z);
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = 0.0f;
      }
      if constexpr (BF16OUT) {
        uint16_t* o = (uint16_t*)a.out + v * kD + 8 * l16;
        *(uint4*)o = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                                pack_bf16x2(y[6], y[7]));
      } else {
        float* o = (float*)a.out + v * kD + 8 * l16;
        *(float4*)o = make_float4(y[0], y[1], y[2], y[3]);
        *(float4*)(o + 4) = make_float4(y[4], y[5], y[6], y[7]);
      }
    }
  }
}

template <int BITS, int QK, bool BF16OUT, int HG>
__global__ void __launch_bounds__(128 * HG) dequant_tinv_kernel(const DequantArgs a) {
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  constexpr int RW = REC / 4;  // record dwords
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = wave >> 1, half = wave & 1, lh = lane >> 5, col = lane & 31;
  const int grp = blockIdx.x % a.n_groups;
  const int h = grp * HG + hh;
  const int64_t n_tiles = (a.n_tokens + kTile - 1) / kTile;

  bf16x8 A[2][8];
  {
    const bf16x8* Tp = (const bf16x8*)a.Tinv;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        A[m][s] = Tp[(((int64_t)h * 4 + 2 * half + m) * 8 + s) * 64 + lane];
  }

  for (int64_t tile = blockIdx.x / a.n_groups; tile < n_tiles; tile += a.blocks_per_group) {
    const int64_t t = tile * kTile + col;
    int64_t row = -1;
    if (t < a.n_tokens) row = a.slots ? a.slots[t] : t;
    const bool valid = row >= 0 && row < a.n_rows;
    const int64_t slot = valid ? row * a.n_heads + h : 0;
    uint32_t w[RW];
    if (valid) {
      const uint4* rp = (const uint4*)(a.codes + slot * REC);
#pragma unroll
      for (int k = 0; k < BITS; ++k) {
        const uint4 x = rp[k];
        w[4 * k] = x.x; w[4 * k + 1] = x.y; w[4 * k + 2] = x.z; w[4 * k + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < RW; ++k) w[k] = 0;
    }
    // B operand: channels 16s + 8lh + e
    bf16x8 B[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t c = codes8<BITS>(w, 2 * s + lh);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = (c >> (BITS * e)) & (L - 1);
        v[e] = QK == 0 ? (float)(2 * q - (L - 1)) : (float)q;
      }
      u32x4 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                  pack_bf16x2(v[6], v[7])};
      B[s] = __builtin_bit_cast(bf16x8, pk);
    }

#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int mt = 2 * half + m;
      float res[16];
      if constexpr (QK == 0) {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[m][s], B[s], acc, 0, 0, 0);
        const float hs = valid ? 0.5f * f16_bits_to_f32(a.scales[slot]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) res[i] = acc[i] * hs;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) res[i] = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x16 acc = {};
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[m][2 * g], B[2 * g], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[m][2 * g + 1], B[2 * g + 1], acc, 0, 0, 0);
          const float sg = valid ? f16_bits_to_f32(a.scales[slot * 4 + g]) : 0.0f;
          const float zg = valid ? f16_bits_to_f32(a.zeros[slot * 4 + g]) : 0.0f;
          const float* G = a.gsum + ((int64_t)h * 4 + g) * kD + 32 * mt + 4 * lh;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float4 gv = *(const float4*)(G + 8 * j);
            const float gg[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              res[4 * j + e] = __builtin_fmaf(sg, acc[4 * j + e], res[4 * j + e]);
              res[4 * j + e] = __builtin_fmaf(zg, gg[e], res[4 * j + e]);
            }
          }
        }
      }
      if (t < a.n_tokens) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 32 * mt + 8 * j + 4 * lh;
          const int64_t o = (t * a.n_heads + h) * kD + r;
          if constexpr (BF16OUT) {
            *(uint2*)((uint16_t*)a.out + o) =
                make_uint2(pack_bf16x2(res[4 * j], res[4 * j + 1]), pack_bf16x2(res[4 * j + 2], res[4 * j + 3]));
          } else {
            *(float4*)((float*)a.out + o) = make_float4(res[4 * j], res[4 * j + 1], res[4 * j + 2], res[4 * j + 3]);
          }
        }
      }
    }
  }
}

template <int BITS, int QK, bool BF16OUT>
hipError_t launch_dq(const DequantArgs& a, int hg, int max_blocks, hipStream_t st) {
  if (a.Tinv) {
    const dim3 grid((unsigned)a.n_groups * (unsigned)a.blocks_per_group);
    switch (hg) {
      case 1: dequant_tinv_kernel<BITS, QK, BF16OUT, 1><<<grid, 128, 0, st>>>(a); break;
      case 2: dequant_tinv_kernel<BITS, QK, BF16OUT, 2><<<grid, 256, 0, st>>>(a); break;
      case 4: dequant_tinv_kernel<BITS, QK, BF16OUT, 4><<<grid, 512, 0, st>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    const int64_t nv = a.n_tokens * a.n_heads;
    const int64_t n_iter = (nv + kVecs - 1) / kVecs;
    const int blocks = (int)(n_iter < max_blocks ? n_iter : max_blocks);
    if (blocks <= 0) return hipSuccess;
    dequant_plain_kernel<BITS, QK, BF16OUT><<<blocks, 64 * kWaves, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <int BITS, int QK>
hipError_t launch_dq_out(const DequantArgs& a, int hg, int max_blocks, hipStream_t st) {
  return a.out_bf16 ? launch_dq<BITS, QK, true>(a, hg, max_blocks, st)
                    : launch_dq<BITS, QK, false>(a, hg, max_blocks, st);
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& a, int bits, int hg, int max_blocks, hipStream_t st) {
  if (a.kind == 0) {
    switch (bits) {
      case 2: return launch_dq_out<2, 0>(a, hg, max_blocks, st);
      case 3: return launch_dq_out<3, 0>(a, hg, max_blocks, st);
      case 4: return launch_dq_out<4, 0>(a, hg, max_blocks, st);
    }
  } else {
    switch (bits) {
      case 2: return launch_dq_out<2, 1>(a, hg, max_blocks, st);
      case 3: return launch_dq_out<3, 1>(a, hg, max_blocks, st);
      case 4: return launch_dq_out<4, 1>(a, hg, max_blocks, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace wushkv
