// Fused key path for gfx950: RoPE -> bf16 -> per-head 128x128 transform on
// MFMA (bf16 in, fp32 accumulate) -> clipped b-bit quantizer -> bit packing.
//
// The key transform is a general invertible per-KV-head matrix applied online
// after RoPE (ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity ...",
// method and deployment paragraphs; cere-bro post "WUSH-KV: 2-bit KV-Cache
// Quantization with Data-Adaptive Transforms", Gaps).
//
// Work decomposition.  A block owns HG heads and walks 32-token tiles
// (persistent: tile = first, first + blocks_per_group, ...).  Two waves serve
// each head; wave `half` keeps rows [64*half, 64*half+64) of T~ (64 VGPRs of
// A operands, loaded once) and computes those output rows for the tile with
// 16 v_mfma_f32_32x32x16_bf16.  The B operand is the tile's keys: lane l holds
// token l%32 and, for k step s, channels 16s + 8(l/32) + 0..7 -- so RoPE pairs
// (i, i+64) sit in the same lane (k steps s and s+4) and rotate in registers.
// cos/sin for the tile are computed once per block into LDS (double-buffered,
// one tile ahead) and shared by all waves.
//
// Per-tile pipeline: next tile's keys are loaded into registers and its cos/sin
// are produced while the current tile is rotated, multiplied, quantized and
// packed; packed records and scales are staged in LDS and written as whole
// 16-byte chunks (a head group's records of a token are contiguous).
#include "device_common.h"
#include "internal.h"

#include <climits>

namespace wushkv {

namespace {

constexpr int kTile = 32;
constexpr int kCsStride = 66;  // float2 per token row of the cos/sin tile (64 + 2 pad)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
             pack_bf16x2(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, w);
}

template <bool F32IN>
struct RawKeys;
template <>
struct RawKeys<false> {  // bf16: 8 channels per 16-byte load
  uint4 v[8];
};
template <>
struct RawKeys<true> {   // fp32: 8 channels = two 16-byte loads
  float4 v[16];
};

template <bool F32IN>
__device__ __forceinline__ void load_keys(RawKeys<F32IN>& r, const KeysArgs& a, int64_t tok, int h,
                                          int lh) {
  if (tok < a.n_tokens) {
    if constexpr (F32IN) {
      const float* base = (const float*)a.K + tok * a.stride + (int64_t)h * kD + 8 * lh;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        r.v[2 * s] = *(const float4*)(base + 16 * s);
        r.v[2 * s + 1] = *(const float4*)(base + 16 * s + 4);
      }
    } else {
      const uint16_t* base = (const uint16_t*)a.K + tok * a.stride + (int64_t)h * kD + 8 * lh;
#pragma unroll
      for (int s = 0; s < 8; ++s) r.v[s] = *(const uint4*)(base + 16 * s);
    }
  } else {
#pragma unroll
    for (int s = 0; s < (F32IN ? 16 : 8); ++s) r.v[s] = {};
  }
}

template <bool F32IN>
__device__ __forceinline__ void unpack8(const RawKeys<F32IN>& r, int s, float* x) {
  if constexpr (F32IN) {
    const float4 p = r.v[2 * s], q = r.v[2 * s + 1];
    x[0] = p.x; x[1] = p.y; x[2] = p.z; x[3] = p.w;
    x[4] = q.x; x[5] = q.y; x[6] = q.z; x[7] = q.w;
  } else {
    const uint4 p = r.v[s];
    x[0] = bf16lo_to_f32(p.x); x[1] = bf16hi_to_f32(p.x);
    x[2] = bf16lo_to_f32(p.y); x[3] = bf16hi_to_f32(p.y);
    x[4] = bf16lo_to_f32(p.z); x[5] = bf16hi_to_f32(p.z);
    x[6] = bf16lo_to_f32(p.w); x[7] = bf16hi_to_f32(p.w);
  }
}

template <int BITS, int QK, bool F32IN, int HG, bool YOUT>
__global__ void __launch_bounds__(128 * HG) keys_kernel(const KeysArgs a) {
  constexpr int NT = 128 * HG;
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  constexpr int RECROW = HG * REC + 16;  // LDS row of one token's records (+16 B pad)
  constexpr int NSC = QK ? 8 : 1;        // fp16 values per (token, head): sym 1; affine 4 + 4
  constexpr int RB = 4 * BITS;           // bits in a run of 4 codes

  __shared__ __align__(16) float2 cs_lds[2][kTile][kCsStride];
  __shared__ float red_lds[HG][2][kTile];
  __shared__ __align__(16) uint8_t rec_lds[kTile][RECROW];
  __shared__ uint16_t sc_lds[kTile][HG * NSC];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hh = wave >> 1, half = wave & 1, lh = lane >> 5, col = lane & 31;
  const int grp = blockIdx.x % a.n_groups;
  const int64_t first_tile = blockIdx.x / a.n_groups;
  const int h = grp * HG + hh;
  const int64_t n_tiles = (a.n_tokens + kTile - 1) / kTile;
  if (first_tile >= n_tiles) return;  // uniform over the block
  const int64_t tile_step = a.blocks_per_group;

  // This wave's half of T~ as MFMA A operands: rows 32*(2*half+m) + (lane % 32).
  bf16x8 A[2][8];
  {
    const bf16x8* Tp = (const bf16x8*)a.T;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        A[m][s] = Tp[(((int64_t)h * 4 + 2 * half + m) * 8 + s) * 64 + lane];
  }

  auto fill_cs = [&](int64_t tile, int buf) {
    for (int idx = tid; idx < kTile * kPairs; idx += NT) {
      const int n = idx >> 6, i = idx & 63;
      const int64_t tok = tile * kTile + n;
      float2 v = make_float2(1.0f, 0.0f);
      if (tok < a.n_tokens) {
        int p = a.pos[tok];
        p = p < 0 ? 0 : (p >= a.max_pos ? a.max_pos - 1 : p);
        v = rope_cos_sin(p, i, a.rope_lo, a.rope_hi, a.rope_lo_t, a.rope_hi_t);
      }
      cs_lds[buf][n][i] = v;
    }
  };

  RawKeys<F32IN> cur, nxt;
  int64_t tile = first_tile;
  int buf = 0;
  load_keys<F32IN>(cur, a, tile * kTile + col, h, lh);
  fill_cs(tile, 0);
  __syncthreads();

  while (true) {
    const int64_t next = tile + tile_step;
    const bool has_next = next < n_tiles;
    if (has_next) {
      load_keys<F32IN>(nxt, a, next * kTile + col, h, lh);
      fill_cs(next, buf ^ 1);
    }

    // ---- RoPE (rotate-half, pairs (i, i+64)) and bf16 operands
    bf16x8 Bop[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float ka[8], kb[8];
      unpack8<F32IN>(cur, s, ka);
      unpack8<F32IN>(cur, s + 4, kb);
      const float4* csp = (const float4*)&cs_lds[buf][col][16 * s + 8 * lh];
      float c[8], sn[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 v = csp[e];
        c[2 * e] = v.x; sn[2 * e] = v.y; c[2 * e + 1] = v.z; sn[2 * e + 1] = v.w;
      }
      float xa[8], xb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float bs = kb[e] * sn[e];
        const float as = ka[e] * sn[e];
        xa[e] = __builtin_fmaf(ka[e], c[e], -bs);
        xb[e] = __builtin_fmaf(kb[e], c[e], as);
      }
      Bop[s] = pack8(xa);
      Bop[s + 4] = pack8(xb);
    }

    // ---- y = T~ x~ for this wave's 64 rows (fp32 accumulate)
    f32x16 acc[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) acc[m] = (f32x16){};
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int m = 0; m < 2; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[m][s], Bop[s], acc[m], 0, 0, 0);

    const int64_t tok = tile * kTile + col;

    if constexpr (YOUT) {
      if (tok < a.n_tokens) {
        float* yo = a.y_out + (tok * a.n_heads + h) * kD;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 32 * (2 * half + m) + 8 * j + 4 * lh;
            *(float4*)(yo + r) = make_float4(acc[m][4 * j], acc[m][4 * j + 1], acc[m][4 * j + 2],
                                             acc[m][4 * j + 3]);
          }
      }
      __syncthreads();
    } else {
      // Output element acc[m][i] is row 32*(2*half+m) + 8*(i/4) + 4*lh + (i%4) of token `col`.
      // run[m][j] packs the codes of acc[m][4j .. 4j+3] (4 consecutive rows), LSB first.
      uint32_t run[2][4];
      if constexpr (QK == 0) {
        // Sum of squares as the contiguous pairwise tree over rows 0..127:
        // runs of 4 in-lane, pairs of runs across lanes l and l^32, then up.
        float P8[2][4];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float q0 = acc[m][4 * j] * acc[m][4 * j];
            const float q1 = acc[m][4 * j + 1] * acc[m][4 * j + 1];
            const float q2 = acc[m][4 * j + 2] * acc[m][4 * j + 2];
            const float q3 = acc[m][4 * j + 3] * acc[m][4 * j + 3];
            const float p4 = (q0 + q1) + (q2 + q3);
            P8[m][j] = p4 + __shfl_xor(p4, 32);
          }
        const float P32a = (P8[0][0] + P8[0][1]) + (P8[0][2] + P8[0][3]);
        const float P32b = (P8[1][0] + P8[1][1]) + (P8[1][2] + P8[1][3]);
        const float P64 = P32a + P32b;
        if (lh == 0) red_lds[hh][half][col] = P64;
        __syncthreads();
        const float S = red_lds[hh][0][col] + red_lds[hh][1][col];
        const float ms = S * 0.0078125f;  // S / 128, exact scaling
        const float rms = __builtin_sqrtf(ms);
        const float C = a.q.alpha * rms;
        const float twoC = 2.0f * C;
        const float d32 = twoC / (float)(L - 1);
        const uint16_t dh = f16_sat_bits(d32);
        const float delta = f16_bits_to_f32(dh);
        const float rdelta = __builtin_amdgcn_rcpf(delta);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t r = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t q = delta == 0.0f ? (uint32_t)(L / 2) : sym_code<BITS>(acc[m][4 * j + e], delta, rdelta);
              r |= q << (BITS * e);
            }
            run[m][j] = r;
          }
        if (half == 0 && lh == 0) sc_lds[col][hh] = dh;
      } else {
        // Percentile-clipped affine quantizer, group = one 32-row tile = rows
        // split between lanes l and l^32: two smallest and two largest values by
        // IEEE totalOrder, merged across the lane pair.
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          int32_t mn1 = INT_MAX, mn2 = INT_MAX, mx1 = INT_MIN, mx2 = INT_MIN;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int32_t k = total_order_key(acc[m][i]);
            mn2 = min(mn2, max(mn1, k));
            mn1 = min(mn1, k);
            mx2 = max(mx2, min(mx1, k));
            mx1 = max(mx1, k);
          }
          const int32_t o1 = __shfl_xor(mn1, 32), o2 = __shfl_xor(mn2, 32);
          const int32_t u1 = __shfl_xor(mx1, 32), u2 = __shfl_xor(mx2, 32);
          const float s0 = total_order_value(min(mn1, o1));
          const float s1 = total_order_value(min(max(mn1, o1), min(mn2, o2)));
          const float s31 = total_order_value(max(mx1, u1));
          const float s30 = total_order_value(max(min(mx1, u1), max(mx2, u2)));
          const float lo = a.q.lo_mode ? s0 : __builtin_fmaf(a.q.g_lo, s1 - s0, s0);
          const float hi = a.q.hi_mode == 0 ? __builtin_fmaf(a.q.g_hi, s31 - s30, s30)
                                            : (a.q.hi_mode == 1 ? s30 : s31);
          const float s32 = (hi - lo) / (float)(L - 1);
          const uint16_t sh = f16_sat_bits(s32), zh = f16_sat_bits(lo);
          const double sd = (double)f16_bits_to_f32(sh), zd = (double)f16_bits_to_f32(zh);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t r = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t q = sd == 0.0 ? 0u : affine_code<BITS>(acc[m][4 * j + e], zd, sd);
              r |= q << (BITS * e);
            }
            run[m][j] = r;
          }
          if (lh == 0) {
            sc_lds[col][hh * 8 + 2 * half + m] = sh;
            sc_lds[col][hh * 8 + 4 + 2 * half + m] = zh;
          }
        }
      }

      // ---- pack: runs of 4 codes -> 16 contiguous rows per lane -> LDS record row
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t* rn = run[m];
        const uint32_t send = lh ? (rn[0] | (rn[1] << RB)) : (rn[2] | (rn[3] << RB));
        const uint32_t recv = __shfl_xor(send, 32);
        const uint64_t p0 = recv & ((1u << RB) - 1u), p1 = recv >> RB;
        const uint64_t chunk =
            lh ? (p0 | ((uint64_t)rn[2] << RB) | (p1 << (2 * RB)) | ((uint64_t)rn[3] << (3 * RB)))
               : ((uint64_t)rn[0] | (p0 << RB) | ((uint64_t)rn[1] << (2 * RB)) | (p1 << (3 * RB)));
        const int mt = 2 * half + m;
        uint8_t* dst = &rec_lds[col][hh * REC + BITS * (4 * mt + 2 * lh)];
        if constexpr (BITS == 2) {
          *(uint32_t*)dst = (uint32_t)chunk;
        } else if constexpr (BITS == 4) {
          *(uint64_t*)dst = chunk;
        } else {
          ((uint16_t*)dst)[0] = (uint16_t)chunk;
          ((uint16_t*)dst)[1] = (uint16_t)(chunk >> 16);
          ((uint16_t*)dst)[2] = (uint16_t)(chunk >> 32);
        }
      }
      __syncthreads();

      // ---- stores: each token's HG records are contiguous in the cache row
      const int64_t tbase = tile * kTile;
      constexpr int CPT = HG * BITS;  // 16-byte chunks per token
      for (int c = tid; c < kTile * CPT; c += NT) {
        const int n = c / CPT, k = c - n * CPT;
        const int64_t t = tbase + n;
        if (t < a.n_tokens) {
          const int64_t row = a.slots ? a.slots[t] : t;
          if (row >= 0 && row < a.n_rows) {
            const uint4 v = *(const uint4*)&rec_lds[n][16 * k];
            *(uint4*)(a.codes + (row * a.n_heads + grp * HG) * REC + 16 * k) = v;
          }
        }
      }
      for (int c = tid; c < kTile * HG; c += NT) {
        const int n = c / HG, j = c - n * HG;
        const int64_t t = tbase + n;
        if (t < a.n_tokens) {
          const int64_t row = a.slots ? a.slots[t] : t;
          if (row >= 0 && row < a.n_rows) {
            const int64_t slot = row * a.n_heads + grp * HG + j;
            if constexpr (QK == 0) {
              a.scales[slot] = sc_lds[n][j];
            } else {
              const uint16_t* s = &sc_lds[n][j * 8];
              *(uint2*)(a.scales + slot * 4) =
                  make_uint2(s[0] | ((uint32_t)s[1] << 16), s[2] | ((uint32_t)s[3] << 16));
              *(uint2*)(a.zeros + slot * 4) =
                  make_uint2(s[4] | ((uint32_t)s[5] << 16), s[6] | ((uint32_t)s[7] << 16));
            }
          }
        }
      }
    }
    __syncthreads();
    if (!has_next) break;
    tile = next;
    buf ^= 1;
    cur = nxt;
  }
}

__global__ void rope_cos_sin_kernel(const double2* lo, const double2* hi, const double2* lo_t,
                                    const double2* hi_t, int32_t max_pos, const int32_t* pos,
                                    int64_t n, float* cs) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * kPairs) return;
  const int64_t t = idx / kPairs;
  const int i = (int)(idx - t * kPairs);
  int p = pos[t];
  p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
  const float2 v = rope_cos_sin(p, i, lo, hi, lo_t, hi_t);
  cs[2 * idx] = v.x;
  cs[2 * idx + 1] = v.y;
}

template <int BITS, int QK, bool F32IN, bool YOUT>
hipError_t launch_hg(const KeysArgs& a, int hg, dim3 grid, hipStream_t st) {
  switch (hg) {
    case 1: keys_kernel<BITS, QK, F32IN, 1, YOUT><<<grid, 128, 0, st>>>(a); break;
    case 2: keys_kernel<BITS, QK, F32IN, 2, YOUT><<<grid, 256, 0, st>>>(a); break;
    case 4: keys_kernel<BITS, QK, F32IN, 4, YOUT><<<grid, 512, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BITS, int QK>
hipError_t launch_bits(const KeysArgs& a, int f32_in, int hg, int y_out, dim3 grid, hipStream_t st) {
  if (y_out) return f32_in ? launch_hg<BITS, QK, true, true>(a, hg, grid, st)
                           : launch_hg<BITS, QK, false, true>(a, hg, grid, st);
  return f32_in ? launch_hg<BITS, QK, true, false>(a, hg, grid, st)
                : launch_hg<BITS, QK, false, false>(a, hg, grid, st);
}

}  // namespace

hipError_t launch_keys(const KeysArgs& a, int bits, int f32_in, int hg, int y_out, hipStream_t st) {
  const dim3 grid((unsigned)a.n_groups * (unsigned)a.blocks_per_group);
  if (y_out) return launch_bits<2, 0>(a, f32_in, hg, 1, grid, st);  // transform only
  if (a.q.kind == 0) {
    switch (bits) {
      case 2: return launch_bits<2, 0>(a, f32_in, hg, 0, grid, st);
      case 3: return launch_bits<3, 0>(a, f32_in, hg, 0, grid, st);
      case 4: return launch_bits<4, 0>(a, f32_in, hg, 0, grid, st);
    }
  } else {
    switch (bits) {
      case 2: return launch_bits<2, 1>(a, f32_in, hg, 0, grid, st);
      case 3: return launch_bits<3, 1>(a, f32_in, hg, 0, grid, st);
      case 4: return launch_bits<4, 1>(a, f32_in, hg, 0, grid, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rope_cos_sin(const wushkv_rope* r, const int32_t* pos, int64_t n, float* cs,
                               hipStream_t st) {
  const int64_t total = n * kPairs;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  rope_cos_sin_kernel<<<dim3((unsigned)blocks), threads, 0, st>>>(r->d_lo, r->d_hi, r->d_lo_t, r->d_hi_t,
                                                                  r->max_pos, pos, n, cs);
  return hipGetLastError();
}

}  // namespace wushkv
