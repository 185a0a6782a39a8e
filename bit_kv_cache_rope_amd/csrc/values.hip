// Value path for gfx950: clipped b-bit quantizer -> bit packing.  Values take
// no online transform: theirs is folded into the weights (ai4snews summary
// "WUSH-KV cuts 2-bit KV-cache perplexity ...", deployment paragraph; cere-bro
// post "WUSH-KV: 2-bit KV-Cache Quantization with Data-Adaptive Transforms",
// flowchart).
//
// Layout: a 128-channel (token, head) vector is spread over 16 lanes, 8
// contiguous channels per lane, so one wave load instruction covers 4 vectors
// (1 KiB contiguous for a dense tensor).  A wave handles 16 vectors per
// iteration (4 loads of 16 bytes per lane, kU).  Reductions are xor butterflies
// inside the 16-lane group, which realise the contiguous pairwise tree exactly
// (offsets 1, 2, 4, 8 combine 16-, 32-, 64-, 128-channel halves).  One lane
// per vector turns its sum of squares into the step and the code thresholds,
// which reach the vector's 16 lanes through LDS.  Records and scales are
// staged in LDS (two buffers, alternating by iteration) and written back as
// 16-byte chunks.
//
// Loads go through a raw buffer resource sized to the iteration's vectors:
// vectors past the end read zeros and are never stored.  The next
// iteration's loads are in flight while the current one is quantized (two
// register sets); under 128 VGPRs four waves are resident per SIMD.
#include "device_common.h"
#include "internal.h"
#include "value_codes.h"

namespace wushkv {

namespace {

constexpr int kWaves = 4;
constexpr int kU = 4;                     // loads per lane per iteration
constexpr int kPerWave = 4 * kU;          // vectors per wave per iteration
constexpr int kVecs = kWaves * kPerWave;  // vectors per block per iteration
constexpr int kRawBufferWord3 = 0x00020000;  // raw buffer resource, 32-bit data format
constexpr int kNT = 2;  // cache policy of the streaming loads: non-temporal (read once)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

// 16 bytes from LDS to global memory with a non-temporal store (the packed
// cache is written once here and not read back by this kernel).
__device__ __forceinline__ void store_nt16(void* dst, const void* lds_src) {
  __builtin_nontemporal_store(*(const u32x4*)lds_src, (u32x4*)dst);
}

template <bool F32IN>
struct RawVals {
  u32x4 v[F32IN ? 2 * kU : kU];
};

// (token, head) of a flattened vector index v < 2^31: n = v / H by a multiply-high.
__device__ __forceinline__ uint32_t div_heads(uint32_t v, const ValuesArgs& a) {
  return (__umulhi(v, a.div_m) + v) >> a.div_l;
}

// Loads of block-iteration `it` (vectors it * kVecs ...): this wave's vector
// base + 4u (u < kU), 16 bytes per lane (32 for fp32).  `rows` receives the
// cache row of each (strided layouts only).  Vectors past the end read zeros.
template <bool F32IN, bool DENSE>
__device__ __forceinline__ void load_vals(RawVals<F32IN>& r, int64_t* rows, const ValuesArgs& a, uint32_t it,
                                          int wave, int sub, int l16) {
  constexpr uint32_t ESZ = F32IN ? 4 : 2;
  const uint32_t nv = (uint32_t)(a.n_tokens * a.n_heads);
  const uint32_t v0 = it * kVecs;  // first vector of the iteration (< nv)
  const uint32_t nvalid = nv - v0 < (uint32_t)kVecs ? nv - v0 : (uint32_t)kVecs;
  if constexpr (DENSE) {
    const rsrc_t rs = buffer_rsrc((const char*)a.V + (uint64_t)v0 * kD * ESZ, nvalid * kD * ESZ);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t off = (uint32_t)(wave * kPerWave + 4 * u + sub) * (kD * ESZ) + 8 * ESZ * l16;
      if constexpr (F32IN) {
        r.v[2 * u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT);
        r.v[2 * u + 1] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, kNT);
      } else {
        r.v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT);
      }
    }
  } else {
    // tokens n0 .. n_last of the iteration; bytes up to the end of n_last's heads
    const uint32_t n0 = div_heads(v0, a), n_last = div_heads(v0 + nvalid - 1, a);
    const uint64_t row_bytes = (uint64_t)a.stride * ESZ;
    const rsrc_t rs = buffer_rsrc((const char*)a.V + n0 * row_bytes,
                                  (uint32_t)((n_last - n0) * row_bytes + (uint64_t)a.n_heads * kD * ESZ));
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t v = v0 + wave * kPerWave + 4 * u + sub;
      const uint32_t n = div_heads(v, a);
      const uint32_t h = v - n * (uint32_t)a.n_heads;
      // a vector past the end maps past n_last: offset >= the resource size
      const uint32_t off = (uint32_t)((n - n0) * row_bytes) + h * (kD * ESZ) + 8 * ESZ * l16;
      if (rows) rows[u] = v < nv ? (a.slots ? a.slots[n] : (int64_t)n) : -1;
      if constexpr (F32IN) {
        r.v[2 * u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT);
        r.v[2 * u + 1] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, kNT);
      } else {
        r.v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT);
      }
    }
  }
}

template <int BITS, int QK, bool F32IN, bool DENSE>
__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(QK == 2 ? 2 : (F32IN && QK ? 3 : 4))))
values_kernel(const ValuesArgs a) {
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  constexpr int NSC = QK ? 4 : 1;
  __shared__ __align__(16) uint8_t rec_lds[2][kVecs * REC];
  __shared__ __align__(16) uint16_t sc_lds[2][kVecs * NSC];
  __shared__ __align__(16) uint16_t zr_lds[2][QK ? kVecs * 4 : 8];
  __shared__ int64_t row_lds[2][DENSE ? 1 : kVecs];
  __shared__ float ss_lds[kWaves][kPerWave];              // sum of squares per vector
  __shared__ __align__(16) float4 th_lds[kWaves][kPerWave];  // per vector: thresholds / step

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x, lane = tid & 63;
  const int sub = lane >> 4, l16 = lane & 15;
  const int64_t nv = a.n_tokens * a.n_heads;
  const uint32_t n_iter = (uint32_t)((nv + kVecs - 1) / kVecs);
  uint32_t it = blockIdx.x;
  if (it >= n_iter) return;

  auto step = [&](RawVals<F32IN>& cur, int64_t* rcur, RawVals<F32IN>& nxt, int64_t* rnxt, int par)
      __attribute__((always_inline)) -> bool {
    const uint32_t it_next = it + gridDim.x;
    const bool has_next = it_next < n_iter;
    if (has_next) load_vals<F32IN, DENSE>(nxt, rnxt, a, it_next, wave, sub, l16);

    // the raw words of vector slot u (one 16-byte group for bf16, two for fp32)
    auto words = [&](int u) __attribute__((always_inline)) -> const u32x4* { return &cur.v[F32IN ? 2 * u : u]; };
    auto unpack = [&](int u, float* x) __attribute__((always_inline)) { unpack_vals<F32IN>(words(u), x); };
    auto store_codes = [&](int vloc, uint32_t packed) __attribute__((always_inline)) {
      // this lane's 8 codes: BITS bytes at record offset BITS * l16
      uint8_t* dst = &rec_lds[par][vloc * REC + BITS * l16];
      if constexpr (BITS == 2) {
        *(uint16_t*)dst = (uint16_t)packed;
      } else if constexpr (BITS == 4) {
        *(uint32_t*)dst = packed;
      } else {
        dst[0] = (uint8_t)packed;
        dst[1] = (uint8_t)(packed >> 8);
        dst[2] = (uint8_t)(packed >> 16);
      }
    };
    if constexpr (!DENSE) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (l16 == 0) row_lds[par][wave * kPerWave + 4 * u + sub] = rcur[u];
    }

    if constexpr (QK == 0) {
      // (1) sum of squares of each vector: in-lane pairwise over 8 channels, then
      //     across the 16 lanes of the vector.
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float x[8];
        unpack(u, x);
        const float P = dpp_sum16(lane_sumsq8(x));
        if (l16 == 0) ss_lds[wave][4 * u + sub] = P;
      }
      // (2) one lane per vector: step, fp16 scale and thresholds
      if (lane < kPerWave) {
        const float P = ss_lds[wave][lane];
        const uint16_t sc = sym_step_f16<L>(P, a.q.alpha);
        const float delta = f16_bits_to_f32(sc);
        sc_lds[par][wave * kPerWave + lane] = sc;
        const float4 th = value_thresholds<BITS>(delta);
        th_lds[wave][lane] = th;
      }
      // (3) codes
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float4 th = th_lds[wave][4 * u + sub];
        if constexpr (BITS == 2) {
          store_codes(wave * kPerWave + 4 * u + sub, value_codes2<F32IN>(words(u), th.x));
        } else {
          float x[8];
          unpack(u, x);
          store_codes(wave * kPerWave + 4 * u + sub, value_codes_sym<BITS>(x, th));
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int vloc = wave * kPerWave + 4 * u + sub;
        float x[8];
        unpack(u, x);
        uint16_t sh, zh;
        const uint32_t packed = value_codes_affine<BITS, QK == 2>(x, a.q, sh, zh);
        if ((l16 & 3) == 0) {
          sc_lds[par][vloc * 4 + (l16 >> 2)] = sh;
          zr_lds[par][vloc * 4 + (l16 >> 2)] = zh;
        }
        store_codes(vloc, packed);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the prefetch has landed
    __syncthreads();

    // write back: records (BITS 16-byte chunks each) and scales (+ zeros).  The
    // staging buffers alternate, so the next iteration may fill the other one
    // while these stores still read this one.
    const int64_t vb = (int64_t)it * kVecs;
    if constexpr (DENSE) {
      const int64_t nvalid = nv - vb < kVecs ? nv - vb : kVecs;
      for (int c = tid; c < kVecs * BITS; c += 64 * kWaves)
        if (c < nvalid * BITS) store_nt16(a.codes + vb * REC + 16 * c, &rec_lds[par][16 * c]);
      constexpr int SCB = kVecs * NSC * 2 / 16;  // 16-byte chunks of scales
      for (int c = tid; c < SCB; c += 64 * kWaves) {
        const int64_t first = (int64_t)c * 8 / NSC;  // first vector of the chunk
        if (first + 8 / NSC <= nvalid) {
          store_nt16(a.scales + vb * NSC + 8 * c, &sc_lds[par][8 * c]);
          if constexpr (QK != 0) store_nt16(a.zeros + vb * NSC + 8 * c, &zr_lds[par][8 * c]);
        } else {
          for (int k = 0; k < 8; ++k)
            if ((int64_t)(8 * c + k) < nvalid * NSC) {
              a.scales[vb * NSC + 8 * c + k] = sc_lds[par][8 * c + k];
              if constexpr (QK != 0) a.zeros[vb * NSC + 8 * c + k] = zr_lds[par][8 * c + k];
            }
        }
      }
    } else {
      for (int c = tid; c < kVecs * BITS; c += 64 * kWaves) {
        const int vloc = c / BITS, k = c - vloc * BITS;
        const int64_t v = vb + vloc;
        const int64_t row = row_lds[par][vloc];
        if (v < nv && row >= 0 && row < a.n_rows) {
          const uint32_t n = div_heads((uint32_t)v, a);
          const int h = (int)((uint32_t)v - n * (uint32_t)a.n_heads);
          store_nt16(a.codes + (row * a.n_heads + h) * REC + 16 * k, &rec_lds[par][vloc * REC + 16 * k]);
        }
      }
      for (int vloc = tid; vloc < kVecs; vloc += 64 * kWaves) {
        const int64_t v = vb + vloc;
        const int64_t row = row_lds[par][vloc];
        if (v < nv && row >= 0 && row < a.n_rows) {
          const uint32_t n = div_heads((uint32_t)v, a);
          const int h = (int)((uint32_t)v - n * (uint32_t)a.n_heads);
          const int64_t slot = row * a.n_heads + h;
          if constexpr (QK == 0) {
            a.scales[slot] = sc_lds[par][vloc];
          } else {
            const uint16_t* sp = &sc_lds[par][vloc * 4];
            const uint16_t* zp = &zr_lds[par][vloc * 4];
            *(uint2*)(a.scales + slot * 4) = make_uint2(sp[0] | ((uint32_t)sp[1] << 16), sp[2] | ((uint32_t)sp[3] << 16));
            *(uint2*)(a.zeros + slot * 4) = make_uint2(zp[0] | ((uint32_t)zp[1] << 16), zp[2] | ((uint32_t)zp[3] << 16));
          }
        }
      }
    }
    if (has_next) it = it_next;
    return has_next;
  };

  RawVals<F32IN> ra, rb;
  int64_t rowa[DENSE ? 1 : kU], rowb[DENSE ? 1 : kU];
  load_vals<F32IN, DENSE>(ra, DENSE ? nullptr : rowa, a, it, wave, sub, l16);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing in flight when the loop starts
  while (true) {
    if (!step(ra, rowa, rb, rowb, 0)) break;
    if (!step(rb, rowb, ra, rowa, 1)) break;
  }
}

template <int BITS, int QK, bool F32IN, bool DENSE>
hipError_t launch_v(const ValuesArgs& a, int cus, hipStream_t st) {
  auto k = values_kernel<BITS, QK, F32IN, DENSE>;
  static int occ = 0;  // resident blocks per CU, one value per instantiation
  if (!occ) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, 64 * kWaves, 0) != hipSuccess || n < 1) n = 1;
    occ = n;
  }
  const int64_t nv = a.n_tokens * a.n_heads;
  const int64_t n_iter = (nv + kVecs - 1) / kVecs;
  // as many blocks as fit at once, then as few as give every block the same
  // number of iterations (a last round run by a fraction of the blocks would
  // leave most of the chip idle)
  if (n_iter <= 0) return hipSuccess;
  const int64_t cap = (int64_t)cus * occ;
  const int64_t per_block = (n_iter + cap - 1) / cap;
  const int blocks = (int)((n_iter + per_block - 1) / per_block);
  return launch_kernel(k, dim3(blocks), dim3(64 * kWaves), st, a);
}

template <int BITS, int QK>
hipError_t launch_vd(const ValuesArgs& a, int f32_in, int cus, hipStream_t st) {
  const bool dense = a.slots == nullptr && a.stride == (int64_t)a.n_heads * kD;
  if (f32_in) return dense ? launch_v<BITS, QK, true, true>(a, cus, st) : launch_v<BITS, QK, true, false>(a, cus, st);
  return dense ? launch_v<BITS, QK, false, true>(a, cus, st) : launch_v<BITS, QK, false, false>(a, cus, st);
}

}  // namespace

hipError_t launch_values(const ValuesArgs& a, int bits, int f32_in, int cus, hipStream_t st) {
  if (a.q.kind == 0) {
    switch (bits) {
      case 2: return launch_vd<2, 0>(a, f32_in, cus, st);
      case 3: return launch_vd<3, 0>(a, f32_in, cus, st);
      case 4: return launch_vd<4, 0>(a, f32_in, cus, st);
    }
  } else if (a.q.kind == 1) {
    switch (bits) {
      case 2: return launch_vd<2, 1>(a, f32_in, cus, st);
      case 3: return launch_vd<3, 1>(a, f32_in, cus, st);
      case 4: return launch_vd<4, 1>(a, f32_in, cus, st);
    }
  } else {
    switch (bits) {
      case 2: return launch_vd<2, 2>(a, f32_in, cus, st);
      case 3: return launch_vd<3, 2>(a, f32_in, cus, st);
      case 4: return launch_vd<4, 2>(a, f32_in, cus, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace wushkv
