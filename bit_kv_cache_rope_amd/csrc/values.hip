// Value path for gfx950: clipped b-bit quantizer -> bit packing.  Values take
// no online transform: theirs is folded into the weights (ai4snews summary
// "WUSH-KV cuts 2-bit KV-cache perplexity ...", deployment paragraph; cere-bro
// post "WUSH-KV: 2-bit KV-Cache Quantization with Data-Adaptive Transforms",
// flowchart).
//
// Layout: a 128-channel (token, head) vector is spread over 16 lanes, 8
// contiguous channels per lane, so one wave load instruction covers 4 vectors
// (1 KiB contiguous for a dense tensor).  Each wave handles 16 vectors per
// iteration (4 loads per lane, the next iteration's loads in flight while the
// current one is quantized).  Reductions are xor butterflies inside the 16-lane
// group, which realise the contiguous pairwise tree exactly (offsets 1, 2, 4, 8
// combine 16-, 32-, 64-, 128-channel halves).  Records are staged in LDS and
// written back as 16-byte chunks.
#include "device_common.h"
#include "internal.h"

#include <climits>

namespace wushkv {

namespace {

constexpr int kWaves = 4;
constexpr int kPerWave = 16;              // vectors per wave per iteration
constexpr int kVecs = kWaves * kPerWave;  // vectors per block per iteration

template <bool F32IN>
struct RawVals;
template <>
struct RawVals<false> {
  uint4 v[4];
};
template <>
struct RawVals<true> {
  float4 v[8];
};

template <bool F32IN>
__device__ __forceinline__ void load_vals(RawVals<F32IN>& r, const ValuesArgs& a, int64_t vbase, int l16) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t v = vbase + 4 * u;
    const int64_t nv = a.n_tokens * a.n_heads;
    if (v < nv) {
      const int64_t n = v / a.n_heads;
      const int h = (int)(v - n * a.n_heads);
      if constexpr (F32IN) {
        const float* p = (const float*)a.V + n * a.stride + (int64_t)h * kD + 8 * l16;
        r.v[2 * u] = *(const float4*)p;
        r.v[2 * u + 1] = *(const float4*)(p + 4);
      } else {
        const uint16_t* p = (const uint16_t*)a.V + n * a.stride + (int64_t)h * kD + 8 * l16;
        r.v[u] = *(const uint4*)p;
      }
    } else {
      if constexpr (F32IN) {
        r.v[2 * u] = {};
        r.v[2 * u + 1] = {};
      } else {
        r.v[u] = {};
      }
    }
  }
}

template <int BITS, int QK, bool F32IN>
__global__ void __launch_bounds__(64 * kWaves) values_kernel(const ValuesArgs a) {
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  __shared__ __align__(16) uint8_t rec_lds[kVecs * REC];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = lane >> 4, l16 = lane & 15;
  const int64_t nv = a.n_tokens * a.n_heads;
  const int64_t n_iter = (nv + kVecs - 1) / kVecs;
  int64_t it = blockIdx.x;
  if (it >= n_iter) return;

  RawVals<F32IN> cur, nxt;
  load_vals<F32IN>(cur, a, it * kVecs + wave * kPerWave + sub, l16);

  while (true) {
    const int64_t it_next = it + gridDim.x;
    const bool has_next = it_next < n_iter;
    if (has_next) load_vals<F32IN>(nxt, a, it_next * kVecs + wave * kPerWave + sub, l16);

#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int vloc = wave * kPerWave + 4 * u + sub;  // vector index within the block iteration
      const int64_t v = it * kVecs + vloc;
      float x[8];
      if constexpr (F32IN) {
        const float4 p = cur.v[2 * u], q = cur.v[2 * u + 1];
        x[0] = p.x; x[1] = p.y; x[2] = p.z; x[3] = p.w; x[4] = q.x; x[5] = q.y; x[6] = q.z; x[7] = q.w;
      } else {
        const uint4 p = cur.v[u];
        x[0] = bf16lo_to_f32(p.x); x[1] = bf16hi_to_f32(p.x);
        x[2] = bf16lo_to_f32(p.y); x[3] = bf16hi_to_f32(p.y);
        x[4] = bf16lo_to_f32(p.z); x[5] = bf16hi_to_f32(p.z);
        x[6] = bf16lo_to_f32(p.w); x[7] = bf16hi_to_f32(p.w);
      }
      uint32_t packed = 0;
      uint16_t sc = 0, sh = 0, zh = 0;
      if constexpr (QK == 0) {
        float q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = x[e] * x[e];
        float P = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
        P = P + __shfl_xor(P, 1);
        P = P + __shfl_xor(P, 2);
        P = P + __shfl_xor(P, 4);
        P = P + __shfl_xor(P, 8);
        const float ms = P * 0.0078125f;
        const float rms = __builtin_sqrtf(ms);
        const float C = a.q.alpha * rms;
        const float twoC = 2.0f * C;
        const float d32 = twoC / (float)(L - 1);
        sc = f16_sat_bits(d32);
        const float delta = f16_bits_to_f32(sc);
        const float rdelta = __builtin_amdgcn_rcpf(delta);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t c = delta == 0.0f ? (uint32_t)(L / 2) : sym_code<BITS>(x[e], delta, rdelta);
          packed |= c << (BITS * e);
        }
      } else {
        // group of 32 channels = 4 lanes: two extremes at each end, merged by xor 1, 2
        int32_t mn1 = INT_MAX, mn2 = INT_MAX, mx1 = INT_MIN, mx2 = INT_MIN;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int32_t k = total_order_key(x[e]);
          mn2 = min(mn2, max(mn1, k));
          mn1 = min(mn1, k);
          mx2 = max(mx2, min(mx1, k));
          mx1 = max(mx1, k);
        }
#pragma unroll
        for (int off = 1; off <= 2; off <<= 1) {
          const int32_t o1 = __shfl_xor(mn1, off), o2 = __shfl_xor(mn2, off);
          const int32_t u1 = __shfl_xor(mx1, off), u2 = __shfl_xor(mx2, off);
          mn2 = min(max(mn1, o1), min(mn2, o2));
          mn1 = min(mn1, o1);
          mx2 = max(min(mx1, u1), max(mx2, u2));
          mx1 = max(mx1, u1);
        }
        const float s0 = total_order_value(mn1), s1 = total_order_value(mn2);
        const float s31 = total_order_value(mx1), s30 = total_order_value(mx2);
        const float lo = a.q.lo_mode ? s0 : __builtin_fmaf(a.q.g_lo, s1 - s0, s0);
        const float hi = a.q.hi_mode == 0 ? __builtin_fmaf(a.q.g_hi, s31 - s30, s30)
                                          : (a.q.hi_mode == 1 ? s30 : s31);
        const float s32 = (hi - lo) / (float)(L - 1);
        sh = f16_sat_bits(s32);
        zh = f16_sat_bits(lo);
        const double sd = (double)f16_bits_to_f32(sh), zd = (double)f16_bits_to_f32(zh);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t c = sd == 0.0 ? 0u : affine_code<BITS>(x[e], zd, sd);
          packed |= c << (BITS * e);
        }
      }
      // this lane's 8 codes: BITS bytes at record offset BITS * l16
      uint8_t* dst = &rec_lds[vloc * REC + BITS * l16];
      if constexpr (BITS == 2) {
        *(uint16_t*)dst = (uint16_t)packed;
      } else if constexpr (BITS == 4) {
        *(uint32_t*)dst = packed;
      } else {
        dst[0] = (uint8_t)packed;
        dst[1] = (uint8_t)(packed >> 8);
        dst[2] = (uint8_t)(packed >> 16);
      }
      if (v < nv) {
        const int64_t n = v / a.n_heads;
        const int h = (int)(v - n * a.n_heads);
        const int64_t row = a.slots ? a.slots[n] : n;
        if (row >= 0 && row < a.n_rows) {
          const int64_t slot = row * a.n_heads + h;
          if constexpr (QK == 0) {
            if (l16 == 0) a.scales[slot] = sc;
          } else {
            if ((l16 & 3) == 0) {
              a.scales[slot * 4 + (l16 >> 2)] = sh;
              a.zeros[slot * 4 + (l16 >> 2)] = zh;
            }
          }
        }
      }
    }
    __syncthreads();
    // write back the block's records as 16-byte chunks
    for (int c = tid; c < kVecs * BITS; c += 64 * kWaves) {
      const int vloc = c / BITS, k = c - vloc * BITS;
      const int64_t v = it * kVecs + vloc;
      if (v < nv) {
        const int64_t n = v / a.n_heads;
        const int h = (int)(v - n * a.n_heads);
        const int64_t row = a.slots ? a.slots[n] : n;
        if (row >= 0 && row < a.n_rows)
          *(uint4*)(a.codes + (row * a.n_heads + h) * REC + 16 * k) = *(const uint4*)&rec_lds[vloc * REC + 16 * k];
      }
    }
    __syncthreads();
    if (!has_next) break;
    it = it_next;
    cur = nxt;
  }
}

template <int BITS, int QK>
hipError_t launch_v(const ValuesArgs& a, int f32_in, int blocks, hipStream_t st) {
  if (f32_in) values_kernel<BITS, QK, true><<<blocks, 64 * kWaves, 0, st>>>(a);
  else values_kernel<BITS, QK, false><<<blocks, 64 * kWaves, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_values(const ValuesArgs& a, int bits, int f32_in, int max_blocks, hipStream_t st) {
  const int64_t nv = a.n_tokens * a.n_heads;
  const int64_t n_iter = (nv + kVecs - 1) / kVecs;
  const int blocks = (int)(n_iter < max_blocks ? n_iter : max_blocks);
  if (blocks <= 0) return hipSuccess;
  if (a.q.kind == 0) {
    switch (bits) {
      case 2: return launch_v<2, 0>(a, f32_in, blocks, st);
      case 3: return launch_v<3, 0>(a, f32_in, blocks, st);
      case 4: return launch_v<4, 0>(a, f32_in, blocks, st);
    }
  } else {
    switch (bits) {
      case 2: return launch_v<2, 1>(a, f32_in, blocks, st);
      case 3: return launch_v<3, 1>(a, f32_in, blocks, st);
      case 4: return launch_v<4, 1>(a, f32_in, blocks, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace wushkv
