// Fused append path for gfx950: the keys and the values of the same tokens in one
// dispatch, built for the latency of small appends: a decode step's one token
// per sequence, or the 16-token chunks of chunked prefill (ai4snews summary
// "WUSH-KV cuts 2-bit KV-cache perplexity ...", experiments paragraph, and its
// deployment paragraph on paged caches).  Keys take RoPE, the per-head key
// transform on MFMA and the clipped quantizer; values only the quantizer (the
// same summary's method and deployment paragraphs).
//
// Work unit: one head's 8 consecutive tokens, keys and values; one block of four
// waves per unit, so a 64-token, 8-head decode call runs as 64 blocks.  Units
// are numbered token-group-major with the head fastest, so the units of one head
// share an XCD (block b runs on XCD b % 8) and read that head's T~ through the
// same L2.
//
// Each thread issues all its loads before it waits on any: the position of its
// RoPE token, the cache rows, a value vector's 16 bytes (used by waves 0, 1), its
// two key channel pairs, and (per wave) 32 rows of T~ as MFMA A operands; then,
// once the position is in, the RoPE table rows for it.  Waves 0, 1 quantize the
// values while those are in flight.  A thread computes the exact (cos, sin) of its own two
// pairs (the same function as the tiled key kernel) and rotates them in fp32;
// the bf16 operands meet in LDS, and wave w computes rows 32 w .. 32 w + 31 of
// y = T~ x~ for the unit's tokens with the same v_mfma_f32_32x32x16_bf16
// sequence as the tiled key kernel (the unit's tokens in columns 0..7), so the
// two paths produce identical y and identical bytes.  The statistic, the codes
// and the record layout come from the shared key_codes.h and value_codes.h.
#include "device_common.h"
#include "internal.h"
#include "key_codes.h"
#include "value_codes.h"

namespace wushkv {

namespace {

constexpr int kUT = 8;         // tokens per unit
constexpr int kThreads = 256;  // four waves
constexpr int kRawBufferWord3 = 0x00020000;  // raw buffer resource, 32-bit data format
constexpr int kNT = 2;         // cache policy of the streaming K and V loads: non-temporal

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): loads past `bytes` return zeros.
__device__ __forceinline__ rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

template <int BITS, int QK, bool F32IN>
__global__ void __launch_bounds__(kThreads) kv_append_kernel(const AppendArgs a) {
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  constexpr uint32_t ESZ = F32IN ? 4 : 2;
  // B operands: k step s, lane l = token l % 32 (columns 0..7 used), channels
  // 16 s + 8 (l / 32) + 0..7
  __shared__ __align__(16) bf16x8 xb_lds[8][64];
  __shared__ float red_lds[4][32];  // per wave and token: the sum of squares of its 32 rows

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lh = lane >> 5, col = lane & 31;
  const int jr = threadIdx.x >> 5;                         // RoPE role: token of the unit
  const int jv = 4 * wave + (lane >> 4), l16 = lane & 15;  // value role (waves 0, 1): token, lane of its vector
  const int H = a.n_heads;
  const int n_tok = (int)a.n_tokens;
  const int n_units = ((n_tok + kUT - 1) / kUT) * H;  // < 2^31 (n_tokens * n_heads < 2^31)
  const uint32_t krow = (uint32_t)(a.k_stride * ESZ), vrow = (uint32_t)(a.v_stride * ESZ);

  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int h = u % H, n0 = (u / H) * kUT;
    const int nv = min(kUT, n_tok - n0);  // tokens of the unit that exist

    // ---- loads, straight-line and oldest first (tokens past the end, and the
    // slots of a cache without them, read zeros through the buffer resources),
    // so that each first use waits only for the loads it needs
    const int p_raw =
        (int)__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(a.pos + n0, 4u * (uint32_t)nv), 4 * jr, 0, 0);
    const u32x2 k_sw = __builtin_amdgcn_raw_buffer_load_b64(
        buffer_rsrc(a.k_slots ? a.k_slots + n0 : nullptr, a.k_slots ? 8u * (uint32_t)nv : 0u), 8 * col, 0, 0);
    const u32x2 v_sw = __builtin_amdgcn_raw_buffer_load_b64(
        buffer_rsrc(a.v_slots ? a.v_slots + n0 : nullptr, a.v_slots ? 8u * (uint32_t)nv : 0u), 8 * (jv & 7), 0, 0);
    // a value vector per 16 lanes: tokens jv < 8 in waves 0, 1 (waves 2, 3 address
    // tokens 8 .. 15, past the resource: zeros, unused)
    vu32x4 vw[F32IN ? 2 : 1];
    {
      const rsrc_t vs = buffer_rsrc((const char*)a.V + ((int64_t)n0 * a.v_stride + (int64_t)h * kD) * ESZ,
                                    (uint32_t)(nv - 1) * vrow + kD * ESZ);
      const uint32_t off = (uint32_t)jv * vrow + 8 * ESZ * l16;
      vw[0] = __builtin_amdgcn_raw_buffer_load_b128(vs, off, 0, kNT);
      if constexpr (F32IN) vw[1] = __builtin_amdgcn_raw_buffer_load_b128(vs, off + 16, 0, kNT);
    }
    // channels 2 col, 2 col + 1 of token jr and their partners 64 higher
    const rsrc_t ks = buffer_rsrc((const char*)a.K + ((int64_t)n0 * a.k_stride + (int64_t)h * kD) * ESZ,
                                  (uint32_t)(nv - 1) * krow + kD * ESZ);
    const uint32_t koff = (uint32_t)jr * krow + 2 * ESZ * col;
    uint32_t kw[F32IN ? 4 : 2];
    if constexpr (F32IN) {
      const u32x2 wa = __builtin_amdgcn_raw_buffer_load_b64(ks, koff, 0, kNT);
      const u32x2 wb = __builtin_amdgcn_raw_buffer_load_b64(ks, koff + 64 * ESZ, 0, kNT);
      kw[0] = wa[0]; kw[1] = wa[1]; kw[2] = wb[0]; kw[3] = wb[1];
    } else {
      kw[0] = __builtin_amdgcn_raw_buffer_load_b32(ks, koff, 0, kNT);
      kw[1] = __builtin_amdgcn_raw_buffer_load_b32(ks, koff + 64 * ESZ, 0, kNT);
    }
    // this wave's 32 rows of T~ as MFMA A operands
    bf16x8 A[8];
    {
      const bf16x8* Tp = (const bf16x8*)a.T + (((int64_t)h * 4 + wave) * 8) * 64 + lane;
#pragma unroll
      for (int s = 0; s < 8; ++s) A[s] = Tp[s * 64];
    }
    // every load above is issued before anything waits for the position
    __builtin_amdgcn_sched_barrier(0);
    // the RoPE table rows of the token's position: heads of hi row p / 32 and
    // lo row p % 32 for pairs 2 col, 2 col + 1, and the hi row's bitmap word
    const int p = min(max(p_raw, 0), a.max_pos - 1);
    const uint32_t hr = ((uint32_t)p >> 5) * (uint32_t)kPairs + 2 * col;
    const uint32_t lr = (uint32_t)(p & 31) * kPairs + 2 * col;
    const double2 H0 = a.rope_hi[hr], H1 = a.rope_hi[hr + 1];
    const double2 B0 = a.rope_lo[lr], B1 = a.rope_lo[lr + 1];
    const uint32_t exc = a.rope_exc[(uint32_t)p >> 5];
    __builtin_amdgcn_sched_barrier(0);
    // cache rows: token col (keys), token jv (values); -1 for no store
    auto row_of = [&](u32x2 w, const int64_t* slots, int64_t n_rows, int j) __attribute__((always_inline)) {
      const int64_t r = slots ? (int64_t)(((uint64_t)w[1] << 32) | w[0]) : (int64_t)(n0 + j);
      return (j < nv && r >= 0 && r < n_rows) ? r : (int64_t)-1;
    };

    // ---- values, while the table rows are in flight (wave-uniform branch: the
    // 2-bit codes take wave-wide ballots)
    if (wave < 2) {
      float x[8];
      unpack_vals<F32IN>(vw, x);
      uint32_t packed;
      uint16_t sh = 0, zh = 0;
      if constexpr (QK == 0) {
        // every lane of the vector holds the whole sum after the butterflies
        sh = sym_step_f16<L>(dpp_sum16(lane_sumsq8(x)), a.q.alpha);
        const float4 th = value_thresholds<BITS>(f16_bits_to_f32(sh));
        if constexpr (BITS == 2) {
          packed = value_codes2<F32IN>(vw, th.x);
        } else {
          packed = value_codes_sym<BITS>(x, th);
        }
      } else {
        packed = value_codes_affine<BITS, QK == 2>(x, a.q, sh, zh);
      }
      const int64_t v_row = row_of(v_sw, a.v_slots, a.v_rows, jv);
      if (v_row >= 0) {
        const int64_t slot = v_row * H + h;
        uint8_t* dst = a.v_codes + slot * REC + BITS * l16;
        if constexpr (BITS == 2) {
          *(uint16_t*)dst = (uint16_t)packed;
        } else if constexpr (BITS == 4) {
          *(uint32_t*)dst = packed;
        } else {
          dst[0] = (uint8_t)packed;
          dst[1] = (uint8_t)(packed >> 8);
          dst[2] = (uint8_t)(packed >> 16);
        }
        if constexpr (QK == 0) {
          if (l16 == 0) a.v_scales[slot] = sh;
        } else {
          if ((l16 & 3) == 0) {
            a.v_scales[slot * 4 + (l16 >> 2)] = sh;
            a.v_zeros[slot * 4 + (l16 >> 2)] = zh;
          }
        }
      }
    }

    // ---- RoPE (rotate-half, pairs (i, i + 64)) -> bf16 operands in LDS
    {
      float ka[2], kb[2];
      if constexpr (F32IN) {
        ka[0] = __uint_as_float(kw[0]); ka[1] = __uint_as_float(kw[1]);
        kb[0] = __uint_as_float(kw[2]); kb[1] = __uint_as_float(kw[3]);
      } else {
        ka[0] = bf16lo_to_f32(kw[0]); ka[1] = bf16hi_to_f32(kw[0]);
        kb[0] = bf16lo_to_f32(kw[1]); kb[1] = bf16hi_to_f32(kw[1]);
      }
      const float4 cs = rope2_pair_cs(p, col, H0, H1, exc, B0, B1, a.rope_hit, a.rope_lot);
      const float cc[2] = {cs.x, cs.z}, sn[2] = {cs.y, cs.w};
      float xa[2], xb[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float bs = kb[e] * sn[e];
        const float as = ka[e] * sn[e];
        xa[e] = __builtin_fmaf(ka[e], cc[e], -bs);
        xb[e] = __builtin_fmaf(kb[e], cc[e], as);
      }
      // channel 2 col: k step col / 8, lane half (col / 4) % 2, word col % 4 of the 16 bytes
      const int s = col >> 3, ls = jr + 32 * ((col >> 2) & 1), wd = col & 3;
      ((uint32_t*)&xb_lds[s][ls])[wd] = pack_bf16x2(xa[0], xa[1]);
      ((uint32_t*)&xb_lds[s + 4][ls])[wd] = pack_bf16x2(xb[0], xb[1]);
    }
    __syncthreads();

    // ---- y = T~ x~: this wave's 32 rows for the unit's tokens (columns 0..7)
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], xb_lds[s][lane], acc, 0, 0, 0);

    // ---- key statistic, codes and record chunk of token col
    uint64_t chunk;
    uint16_t ksh = 0, kzh = 0;
    if constexpr (QK == 0) {
      red_lds[wave][col] = col_sumsq32(acc);  // lanes l and l ^ 32 write the same value
      __syncthreads();
      const float S = (red_lds[0][col] + red_lds[1][col]) + (red_lds[2][col] + red_lds[3][col]);
      ksh = sym_step_f16<L>(S, a.q.alpha);
      const float delta = f16_bits_to_f32(ksh);
      if constexpr (BITS == 2) {
        chunk = record_chunk2(sym2_word(acc, delta), lh);
      } else {
        uint32_t run[4];
        sym_runs<BITS>(acc, delta, run);
        chunk = record_chunk<BITS>(run, lh);
      }
    } else {
      uint32_t run[4];
      affine_runs<BITS, QK == 2>(acc, a.q, run, ksh, kzh);
      chunk = record_chunk<BITS>(run, lh);
      __syncthreads();  // every wave has read xb_lds before the next unit's RoPE writes it
    }
    const int64_t k_row = row_of(k_sw, a.k_slots, a.k_rows, col);
    if (k_row >= 0) {
      const int64_t slot = k_row * H + h;
      put_chunk<BITS>(a.k_codes + slot * REC + BITS * (4 * wave + 2 * lh), chunk);
      if constexpr (QK == 0) {
        if (wave == 0 && lh == 0) a.k_scales[slot] = ksh;
      } else {
        if (lh == 0) {
          a.k_scales[slot * 4 + wave] = ksh;
          a.k_zeros[slot * 4 + wave] = kzh;
        }
      }
    }
  }
}

template <int BITS, int QK, bool F32IN>
hipError_t launch_a(const AppendArgs& a, int cus, hipStream_t st) {
  const int64_t n_units = ((a.n_tokens + kUT - 1) / kUT) * a.n_heads;
  const int64_t cap = (int64_t)cus * 8;
  const int blocks = (int)(n_units < cap ? n_units : cap);
  if (blocks <= 0) return hipSuccess;
  return launch_kernel(kv_append_kernel<BITS, QK, F32IN>, dim3(blocks), dim3(kThreads), st, a);
}

template <int BITS, int QK>
hipError_t launch_af(const AppendArgs& a, int f32_in, int cus, hipStream_t st) {
  return f32_in ? launch_a<BITS, QK, true>(a, cus, st) : launch_a<BITS, QK, false>(a, cus, st);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int bits, int f32_in, int cus, hipStream_t st) {
  if (a.q.kind == 0) {
    switch (bits) {
      case 2: return launch_af<2, 0>(a, f32_in, cus, st);
      case 3: return launch_af<3, 0>(a, f32_in, cus, st);
      case 4: return launch_af<4, 0>(a, f32_in, cus, st);
    }
  } else if (a.q.kind == 1) {
    switch (bits) {
      case 2: return launch_af<2, 1>(a, f32_in, cus, st);
      case 3: return launch_af<3, 1>(a, f32_in, cus, st);
      case 4: return launch_af<4, 1>(a, f32_in, cus, st);
    }
  } else {
    switch (bits) {
      case 2: return launch_af<2, 2>(a, f32_in, cus, st);
      case 3: return launch_af<3, 2>(a, f32_in, cus, st);
      case 4: return launch_af<4, 2>(a, f32_in, cus, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace wushkv
