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
constexpr int kTile = 32;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 codes of channels 16 s + 8 lh .. + 7 from a record held as dwords.  The
// dword indices depend on s only (a compile-time constant where it is called);
// the lane half lh picks a shift or a register, so that the record stays in
// registers (an index that varies by lane would put it in scratch memory).
template <int BITS>
__device__ __forceinline__ uint32_t codes8(const uint32_t* w, int s, int lh) {
  if constexpr (BITS == 2) {
    return (w[s] >> (16 * lh)) & 0xFFFFu;
  } else if constexpr (BITS == 4) {
    return lh ? w[2 * s + 1] : w[2 * s];
  } else {
    // bits o .. o + 23, o = 48 s + 24 lh: both candidates from constant dwords
    // (a 64-bit value assembled from the array would be loaded from memory)
    auto at = [&](int o) __attribute__((always_inline)) -> uint32_t {
      const int d = o >> 5, sh = o & 31;
      const uint32_t v = sh + 24 <= 32 ? w[d] >> sh : __builtin_amdgcn_alignbit(w[d + 1], w[d], sh);
      return v & 0xFFFFFFu;
    };
    return lh ? at(48 * s + 24) : at(48 * s);
  }
}

// Zero bytes that a lane reads instead of a record or scale it has no row for,
// so that every iteration issues the same loads (the wait before decoding then
// covers only the older iteration's loads).
__device__ __align__(16) uint8_t g_zero_record[64] = {};

// Plain read path.  Wave w of block b owns vectors 256 b + 64 w .. + 63.
// Lane j first loads vector j's whole record and scale(s) (a few wide loads per
// lane, contiguous across lanes in the dense case) and puts them in the wave's
// LDS area; then lane (s, c) = (l / 16, l % 16) decodes channels 8c .. 8c+7 of
// vectors 4u + s, u = 0..15, and writes each as one 16-byte (bf16) or 32-byte
// (fp32) chunk: every store instruction covers four whole vectors.  The LDS
// area is the wave's own, so no block barrier is needed (LDS operations of one
// wave complete in order).
constexpr int kPlainRounds = 16;
constexpr int kPlainVecs = kWaves * 64;  // vectors per block

template <int BITS, int QK, bool BF16OUT, bool SLOTS>
__global__ void __launch_bounds__(64 * kWaves) dequant_plain_kernel(const DequantArgs a) {
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  constexpr int NSC = QK ? 8 : 2;  // fp16 values per vector in LDS: sym step (+ pad); affine 4 steps, 4 zeros
  __shared__ __align__(16) uint8_t rec_lds[kWaves][64 * REC];
  __shared__ __align__(16) uint16_t sc_lds[kWaves][64 * NSC];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = lane >> 4, l16 = lane & 15;
  const int64_t nv = a.n_tokens * a.n_heads;
  const int64_t vw = (int64_t)blockIdx.x * kPlainVecs + 64 * wave;
  {
    const int64_t v = vw + lane;
    bool ok;
    int64_t slot;
    if constexpr (SLOTS) {
      const int64_t n = v >= nv ? 0
                                : (nv <= (int64_t)UINT32_MAX ? (int64_t)((uint32_t)v / (uint32_t)a.n_heads)
                                                             : v / a.n_heads);
      const int64_t row = *(v < nv ? a.slots + n : (const int64_t*)g_zero_record);
      ok = v < nv && row >= 0 && row < a.n_rows;
      slot = ok ? row * a.n_heads + (v - n * a.n_heads) : 0;
    } else {
      ok = v < nv && v < a.n_rows * a.n_heads;
      slot = ok ? v : 0;
    }
    const uint4* rp = (const uint4*)(ok ? a.codes + slot * REC : g_zero_record);
    uint4 r[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) r[k] = rp[k];
    if constexpr (QK == 0) {
      const uint16_t sc = *(ok ? a.scales + slot : (const uint16_t*)g_zero_record);
      *(uint32_t*)&sc_lds[wave][NSC * lane] = sc;
    } else {
      const uint2 sv = *(const uint2*)(ok ? (const uint8_t*)(a.scales + slot * 4) : g_zero_record);
      const uint2 zv = *(const uint2*)(ok ? (const uint8_t*)(a.zeros + slot * 4) : g_zero_record);
      *(uint4*)&sc_lds[wave][NSC * lane] = make_uint4(sv.x, sv.y, zv.x, zv.y);
    }
#pragma unroll
    for (int k = 0; k < BITS; ++k) *(uint4*)&rec_lds[wave][REC * lane + 16 * k] = r[k];
  }
#pragma unroll
  for (int u = 0; u < kPlainRounds; ++u) {
    const int j = 4 * u + sub;
    const int64_t v = vw + j;
    const int o = REC * j + BITS * l16;  // byte offset of this lane's codes
    uint32_t c;
    if constexpr (BITS == 2) {
      c = *(const uint16_t*)&rec_lds[wave][o];
    } else if constexpr (BITS == 4) {
      c = *(const uint32_t*)&rec_lds[wave][o];
    } else {
      const uint32_t* d = (const uint32_t*)&rec_lds[wave][o & ~3];
      c = __builtin_amdgcn_alignbit(d[1], d[0], 8 * (o & 3)) & 0xFFFFFFu;
    }
    if constexpr (QK == 0 && BITS == 2 && BF16OUT) {
      // Four possible outputs per vector: their bf16 values form an 8-byte
      // table, and one v_perm_b32 per pair of codes picks two of them.  The
      // selector of codes (q0, q1) is bytes {2q0, 2q0+1, 2q1, 2q1+1}.  (An
      // invalid vector has a zero step: +0 everywhere, the + 0 turning -0 into +0.)
      const float hs = 0.5f * f16_bits_to_f32(sc_lds[wave][NSC * j]);
      const uint32_t t01 = pack_bf16x2(-3.0f * hs + 0.0f, -hs + 0.0f);
      const uint32_t t23 = pack_bf16x2(hs + 0.0f, 3.0f * hs + 0.0f);
      uint32_t o4[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t x = c >> (4 * pr);
        const uint32_t t = (x & 3u) | ((x & 0xCu) << 14);  // q0 in byte 0, q1 in byte 2
        o4[pr] = __builtin_amdgcn_perm(t23, t01, t * 0x0202u + 0x01000100u);
      }
      if (v < nv) *(uint4*)((uint16_t*)a.out + v * kD + 8 * l16) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
      continue;
    }
    float y[8];
    if constexpr (QK == 0) {
      // an invalid vector has a zero step: +0 everywhere (the + 0 turns -0 into +0)
      const float hs = 0.5f * f16_bits_to_f32(sc_lds[wave][NSC * j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = (c >> (BITS * e)) & (L - 1);
        y[e] = (float)(2 * q - (L - 1)) * hs + 0.0f;
      }
    } else {
      const float st = f16_bits_to_f32(sc_lds[wave][NSC * j + (l16 >> 2)]);
      const float z = f16_bits_to_f32(sc_lds[wave][NSC * j + 4 + (l16 >> 2)]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = (c >> (BITS * e)) & (L - 1);
        y[e] = __builtin_fmaf((float)q, st, z);
      }
    }
    if (v < nv) {
      if constexpr (BF16OUT) {
        uint16_t* out = (uint16_t*)a.out + v * kD + 8 * l16;
        *(uint4*)out = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                                  pack_bf16x2(y[6], y[7]));
      } else {
        float* out = (float*)a.out + v * kD + 8 * l16;
        *(float4*)out = make_float4(y[0], y[1], y[2], y[3]);
        *(float4*)(out + 4) = make_float4(y[4], y[5], y[6], y[7]);
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

  // B-operand lookup: for 2-bit records, entry b (words 2b, 2b + 1) holds the
  // four bf16 operands of the codes in byte b; for 4-bit, entry b (word b) the
  // two of its codes; for 3-bit, entry b < 64 (word b) the two of a 6-bit pair
  // of codes, each entry in its own LDS bank.  Operand of code q: 2q - (2^b - 1)
  // (symmetric) or q (affine), exact in bf16.
  __shared__ __align__(16) uint32_t lut[512];
  // Output staging: each wave's 32 tokens x 64 rows, padded rows of OROW bytes.
  constexpr int OESZ = BF16OUT ? 2 : 4;
  constexpr int OROW = 64 * OESZ + 16;
  __shared__ __align__(16) uint8_t out_lds[2 * HG][kTile * OROW];
  for (int b = tid; b < 256; b += 128 * HG) {
    constexpr int PER = BITS == 2 ? 4 : 2;  // codes per index (8 bits; 3 bits: 6)
    uint16_t v[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = (b >> (BITS * i)) & (L - 1);
      const float f = QK == 0 ? (float)(2 * q - (L - 1)) : (float)q;
      v[i] = (uint16_t)(__float_as_uint(f) >> 16);  // exact: a small integer
    }
    if constexpr (BITS != 2) {
      if (BITS == 4 || b < 64) lut[b] = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
    } else {
      *(uint2*)&lut[2 * b] = make_uint2((uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16));
    }
  }
  __syncthreads();

  // A tile's inputs for this lane's token: its record, its scale(s) (invalid
  // or past the end: the zero record), loaded one tile ahead.
  struct TileIn {
    uint32_t w[RW];
    uint16_t sc[QK ? 4 : 1], zr[QK ? 4 : 1];
    bool valid;
  };
  auto load_tile = [&](int64_t tile, TileIn& p) __attribute__((always_inline)) {
    const int64_t t = tile * kTile + col;
    const bool in = t < a.n_tokens;
    int64_t row = t;
    if (a.slots) row = *(in ? a.slots + t : (const int64_t*)g_zero_record);
    p.valid = in && row >= 0 && row < a.n_rows;
    const int64_t slot = p.valid ? row * a.n_heads + h : 0;
    const uint4* rp = (const uint4*)(p.valid ? a.codes + slot * REC : g_zero_record);
#pragma unroll
    for (int k = 0; k < BITS; ++k) {
      const uint4 x = rp[k];
      p.w[4 * k] = x.x; p.w[4 * k + 1] = x.y; p.w[4 * k + 2] = x.z; p.w[4 * k + 3] = x.w;
    }
    if constexpr (QK == 0) {
      p.sc[0] = *(p.valid ? a.scales + slot : (const uint16_t*)g_zero_record);
    } else {
      const uint2 sv = *(const uint2*)(p.valid ? (const uint8_t*)(a.scales + slot * 4) : g_zero_record);
      const uint2 zv = *(const uint2*)(p.valid ? (const uint8_t*)(a.zeros + slot * 4) : g_zero_record);
      p.sc[0] = sv.x & 0xFFFF; p.sc[1] = sv.x >> 16; p.sc[2] = sv.y & 0xFFFF; p.sc[3] = sv.y >> 16;
      p.zr[0] = zv.x & 0xFFFF; p.zr[1] = zv.x >> 16; p.zr[2] = zv.y & 0xFFFF; p.zr[3] = zv.y >> 16;
    }
  };

  auto compute = [&](int64_t tile, const TileIn& p) __attribute__((always_inline)) {
    const bool valid = p.valid;
    const uint32_t* w = p.w;
    // B operand: channels 16s + 8lh + e
    bf16x8 B[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t c = codes8<BITS>(w, s, lh);
      u32x4 pk;
      if constexpr (BITS == 2) {
        const uint2 lo = *(const uint2*)&lut[2 * (c & 0xFF)], hi = *(const uint2*)&lut[2 * ((c >> 8) & 0xFF)];
        pk = (u32x4){lo.x, lo.y, hi.x, hi.y};
      } else if constexpr (BITS == 4) {
        pk = (u32x4){lut[c & 0xFF], lut[(c >> 8) & 0xFF], lut[(c >> 16) & 0xFF], lut[c >> 24]};
      } else {
        pk = (u32x4){lut[c & 63], lut[(c >> 6) & 63], lut[(c >> 12) & 63], lut[c >> 18]};
      }
      B[s] = __builtin_bit_cast(bf16x8, pk);
    }

    // symmetric: both row blocks' accumulation chains interleaved
    f32x16 accs[2] = {};
    if constexpr (QK == 0) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
#pragma unroll
        for (int m = 0; m < 2; ++m) accs[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[m][s], B[s], accs[m], 0, 0, 0);
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int mt = 2 * half + m;
      float res[16];
      if constexpr (QK == 0) {
        const float hs = valid ? 0.5f * f16_bits_to_f32(p.sc[0]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) res[i] = accs[m][i] * hs + 0.0f;  // + 0: a missing row reads +0, not -0
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) res[i] = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x16 acc = {};
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[m][2 * g], B[2 * g], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[m][2 * g + 1], B[2 * g + 1], acc, 0, 0, 0);
          const float sg = valid ? f16_bits_to_f32(p.sc[g]) : 0.0f;
          const float zg = valid ? f16_bits_to_f32(p.zr[g]) : 0.0f;
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
      // rows 32 m + 8 j + 4 lh .. + 3 of the wave's half, token col -> LDS
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint8_t* d = &out_lds[wave][col * OROW + (32 * m + 8 * j + 4 * lh) * OESZ];
        if constexpr (BF16OUT) {
          *(uint2*)d = make_uint2(pack_bf16x2(res[4 * j], res[4 * j + 1]), pack_bf16x2(res[4 * j + 2], res[4 * j + 3]));
        } else {
          *(float4*)d = make_float4(res[4 * j], res[4 * j + 1], res[4 * j + 2], res[4 * j + 3]);
        }
      }
    }
    // LDS -> global in whole 16-byte chunks: CPT lanes cover a token's half
    // vector (64 rows), so a store instruction writes 64 / CPT tokens' halves,
    // each contiguous.  (The wave reads back only what it wrote; LDS operations
    // of one wave complete in order.)
    constexpr int CPT = 64 * OESZ / 16;
    constexpr int TPI = 64 / CPT;
#pragma unroll
    for (int k = 0; k < kTile / TPI; ++k) {
      const int tq = TPI * k + lane / CPT, ch = lane % CPT;
      const u32x4 v = *(const u32x4*)&out_lds[wave][tq * OROW + 16 * ch];
      const int64_t tt = tile * kTile + tq;
      if (tt < a.n_tokens) {
        uint8_t* dst = (uint8_t*)a.out + ((tt * a.n_heads + h) * kD + 64 * half) * OESZ + 16 * ch;
        *(u32x4*)dst = v;
      }
    }
  };

  int64_t tile = blockIdx.x / a.n_groups;
  if (tile >= n_tiles) return;
  const int64_t tile_step = a.blocks_per_group;
  // Input sets used in turn (no register copies, which would wait for their
  // loads): while a tile is computed and stored, the loads of the next DEPTH
  // tiles are in flight.  DEPTH 3 for symmetric records; affine kernels keep
  // one, their registers being taken by the per-group scales and zeros.
  constexpr int DEPTH = QK == 0 ? 3 : 1;
  auto step = [&](TileIn& cur, TileIn& fut) __attribute__((always_inline)) -> bool {
    load_tile(tile + DEPTH * tile_step, fut);
    compute(tile, cur);
    tile += tile_step;
    return tile < n_tiles;
  };
  if constexpr (DEPTH == 3) {
    TileIn t0, t1, t2, t3;
    load_tile(tile, t0);
    load_tile(tile + tile_step, t1);
    load_tile(tile + 2 * tile_step, t2);
    while (step(t0, t3) && step(t1, t0) && step(t2, t1) && step(t3, t2)) {
    }
  } else {
    TileIn t0, t1;
    load_tile(tile, t0);
    while (step(t0, t1) && step(t1, t0)) {
    }
  }
}

// Resident blocks per CU of kernel K at the given block size (cached per
// kernel: K is the kernel itself, not its type, which all instantiations share).
template <auto K>
int occupancy(int threads) {
  static int cached = 0;
  if (!cached) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, K, threads, 0) != hipSuccess || n < 1) n = 1;
    cached = n;
  }
  return cached;
}

// Persistent grids: as many blocks as fit on the chip at once (per head group
// for the MFMA kernel), never more than there is work for.
template <int BITS, int QK, bool BF16OUT, int HG>
hipError_t launch_tinv(DequantArgs a, int cus, hipStream_t st) {
  constexpr auto k = dequant_tinv_kernel<BITS, QK, BF16OUT, HG>;
  const int64_t n_tiles = (a.n_tokens + kTile - 1) / kTile;
  int64_t b = (int64_t)cus * occupancy<k>(128 * HG) / a.n_groups;
  b = b < 1 ? 1 : (b > n_tiles ? n_tiles : b);
  a.blocks_per_group = (int)b;
  return launch_kernel(k, dim3((unsigned)(a.n_groups * b)), dim3(128 * HG), st, a);
}

template <int BITS, int QK, bool BF16OUT>
hipError_t launch_dq(const DequantArgs& a, int hg, int cus, hipStream_t st) {
  if (a.Tinv) {
    switch (hg) {
      case 1: return launch_tinv<BITS, QK, BF16OUT, 1>(a, cus, st);
      case 2: return launch_tinv<BITS, QK, BF16OUT, 2>(a, cus, st);
      case 4: return launch_tinv<BITS, QK, BF16OUT, 4>(a, cus, st);
      default: return hipErrorInvalidValue;
    }
  }
  const int64_t nv = a.n_tokens * a.n_heads;
  const int64_t blocks = (nv + kPlainVecs - 1) / kPlainVecs;
  if (blocks <= 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  return launch_kernel(a.slots ? dequant_plain_kernel<BITS, QK, BF16OUT, true> : dequant_plain_kernel<BITS, QK, BF16OUT, false>,
                       dim3((unsigned)blocks), dim3(64 * kWaves), st, a);
}

template <int BITS, int QK>
hipError_t launch_dq_out(const DequantArgs& a, int hg, int cus, hipStream_t st) {
  return a.out_bf16 ? launch_dq<BITS, QK, true>(a, hg, cus, st) : launch_dq<BITS, QK, false>(a, hg, cus, st);
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& a, int bits, int hg, int cus, hipStream_t st) {
  if (a.kind == 0) {
    switch (bits) {
      case 2: return launch_dq_out<2, 0>(a, hg, cus, st);
      case 3: return launch_dq_out<3, 0>(a, hg, cus, st);
      case 4: return launch_dq_out<4, 0>(a, hg, cus, st);
    }
  } else {
    switch (bits) {
      case 2: return launch_dq_out<2, 1>(a, hg, cus, st);
      case 3: return launch_dq_out<3, 1>(a, hg, cus, st);
      case 4: return launch_dq_out<4, 1>(a, hg, cus, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace wushkv
