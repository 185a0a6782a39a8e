// Fused key path for gfx950: RoPE -> bf16 -> per-head 128x128 transform on
// MFMA (bf16 in, fp32 accumulate) -> clipped b-bit quantizer -> bit packing.
//
// The key transform is a general invertible per-KV-head matrix applied online
// after RoPE (ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity ...",
// method and deployment paragraphs; cere-bro post "WUSH-KV: 2-bit KV-Cache
// Quantization with Data-Adaptive Transforms", Gaps).
//
// Work decomposition.  A block owns HG heads and walks 64-token tiles
// (persistent: tile = first, first + blocks_per_group, ...).  Four waves serve
// each head; wave wq keeps rows [32 wq, 32 wq + 32) of T~ (32 VGPRs of A
// operands, loaded once) and computes those output rows for the tile's two
// 32-token column blocks with 16 v_mfma_f32_32x32x16_bf16 (two independent
// accumulation chains).  The B operand is the rotated keys: lane l holds
// token l%32 of a column block and, for k step s, channels 16s + 8(l/32) +
// 0..7.  Wave wq loads and rotates 16 of the tile's tokens, token-major (each
// load instruction covers eight tokens' whole 128-byte lines; the RoPE
// partners (i, i+64) sit in one lane), and the four waves of a head exchange
// their bf16 operands through LDS.  At under 128 VGPRs four waves are
// resident per SIMD.
//
// cos/sin come from the RoPE handle's table (one 512-byte fp32 row per
// position, exact): each wave loads a few of the next tile's rows into
// registers and writes them to one of two LDS tile buffers before that tile's
// RoPE phase (see the pipeline below).
//
// Per-tile pipeline, three barriers: [loads of the next tile's cos/sin rows
// and cache rows, of the positions of the tile after; RoPE -> LDS; the next
// tile's keys into the registers RoPE freed] B1 [MFMA; sums of squares ->
// LDS; cos/sin rows -> LDS] B2 [scale(s), codes, records -> LDS; wait for the
// loads older than the keys] B3 [stores] (one head per block: the cos/sin rows
// are loaded in the MFMA phase and written after the codes, behind a wait for
// every load).
// Packed records and scales are staged in LDS and written as whole 16-byte
// chunks (a head group's records of a token are contiguous in the cache row).
#include "device_common.h"
#include "internal.h"

#include <climits>

namespace wushkv {

namespace {

constexpr int kTile = 64;      // tokens per tile
constexpr int kNB = 2;         // 32-token MFMA column blocks per tile
constexpr int kCsStride = 66;  // float2 per token row of the cos/sin tile (64 + 2 pad)
constexpr int kXcds = 8;       // accelerator complex dies of an MI355X (blocks spread round-robin)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw (unswizzled, stride 0) buffer resource over [base, base + bytes).  A
// load through it returns zeros at offsets past `bytes`; the key path uses
// that instead of clamping indices of tokens past the end (their results are
// never stored).  Word 3 selects the 32-bit data format for untyped access.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kNT = 2;  // cache policy of the key loads: non-temporal (each byte is read once)
__device__ __forceinline__ rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

// v_permlane32_swap of a value with itself: `lo` holds, in every lane l, the
// value of lane l % 32, and `hi` the value of lane l % 32 + 32.
struct Halves {
  uint32_t lo, hi;
};
__device__ __forceinline__ Halves halves(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return {r[0], r[1]};
}
__device__ __forceinline__ Halves halves(float x) { return halves(__float_as_uint(x)); }

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
             pack_bf16x2(x[6], x[7])};
  return __builtin_bit_cast(bf16x8, w);
}

// The keys a wave loads and rotates for one tile: for each token group g
// (tokens 16 wq + 8 g + l / 8), a chunk of 8 channels i < 64 and the partner
// chunk i + 64.
template <bool F32IN>
struct RawKeys;
template <>
struct RawKeys<false> {  // bf16: 8 channels per 16-byte load; [g][partner]
  u32x4 v[2 * kNB];
};
template <>
struct RawKeys<true> {   // fp32: 8 channels = two 16-byte loads
  u32x4 v[4 * kNB];
};

// `rs` covers the tile's rows of this head (zeros past the last token);
// `off` is the lane's byte offset in token group 0, `g_step` the offset of
// token group 1.
template <bool F32IN>
__device__ __forceinline__ void load_keys(RawKeys<F32IN>& r, rsrc_t rs, uint32_t off, uint32_t g_step) {
  constexpr uint32_t kPartner = 64 * (F32IN ? 4 : 2);  // bytes from channel i to channel i + 64
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const uint32_t o = off + nb * g_step;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (F32IN) {
        r.v[4 * nb + 2 * j] = __builtin_amdgcn_raw_buffer_load_b128(rs, o + j * kPartner, 0, kNT);
        r.v[4 * nb + 2 * j + 1] = __builtin_amdgcn_raw_buffer_load_b128(rs, o + j * kPartner + 16, 0, kNT);
      } else {
        r.v[2 * nb + j] = __builtin_amdgcn_raw_buffer_load_b128(rs, o + j * kPartner, 0, kNT);
      }
    }
  }
}

// Block barrier that orders LDS only: waits for this wave's own LDS
// instructions and never for its global loads in flight.  The "memory"
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool F32IN>
__device__ __forceinline__ void unpack8(const RawKeys<F32IN>& r, int nb, int j, float* x) {
  if constexpr (F32IN) {
    const u32x4 p = r.v[4 * nb + 2 * j], q = r.v[4 * nb + 2 * j + 1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = __uint_as_float(p[e]);
      x[4 + e] = __uint_as_float(q[e]);
    }
  } else {
    const u32x4 p = r.v[2 * nb + j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16lo_to_f32(p[e]);
      x[2 * e + 1] = bf16hi_to_f32(p[e]);
    }
  }
}

template <int BITS, int QK, bool F32IN, int HG, bool YOUT>
__global__ void __launch_bounds__(256 * HG) keys_kernel(const KeysArgs a) {
  // Head groups: with two or four heads per block the block runs two groups
  // (of HG / 2 heads, four waves each per head), one phase apart (see the
  // schedule below).
  constexpr int NG = HG >= 2 ? 2 : 1;
  constexpr int HGG = HG / NG;      // heads per group
  constexpr int WG = 4 * HGG;       // waves per group
  constexpr int RPG = kTile / NG;   // cos/sin rows each group loads per tile
  constexpr int TPW = RPG / WG;     // ... each of its waves
  constexpr int NCS = TPW / 2;      // ... two rows per load
  constexpr int NKL = F32IN ? 8 : 4;  // key loads per lane per tile
  static_assert(NG == 1 || NCS + NKL < 16, "vmcnt immediate");
  constexpr int CSB = NG;           // cos/sin tile buffers (by tile parity when two groups)
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  constexpr int RECROW = HGG * REC + 16;  // LDS row of one token's records in a group (+16 B pad)
  constexpr int NSC = QK ? 8 : 1;         // fp16 values per (token, head): sym 1; affine 4 + 4
  constexpr int RB = 4 * BITS;            // bits in a run of 4 codes
  constexpr int ESZ = F32IN ? 4 : 2;

  __shared__ __align__(16) float2 cs_lds[CSB][kTile][kCsStride];  // cos/sin rows of a tile
  __shared__ __align__(16) bf16x8 xb_lds[HG][kNB][8][64];        // rotated operands shared by a head's waves
  __shared__ int32_t slot_lds[2][kTile];  // cache row per token, -1: no store; tile j in slot j & 1
  __shared__ float red_lds[HG][4][kTile];
  __shared__ __align__(16) uint8_t rec_lds[NG][kTile][RECROW];
  __shared__ __align__(16) uint16_t sc_lds[NG][kTile][HGG * NSC];

  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The lane index is re-derived at every interval (see the top of the
  // loop), so the per-lane offsets are recomputed there rather than held in
  // registers across it.
  int lane = threadIdx.x & 63, lh = lane >> 5, col = lane & 31;
  // Four waves per head: wave wq holds rows 32 wq .. 32 wq + 31 of T~.
  const int hh = wave_u >> 2, wq = wave_u & 3;
  const int g = hh / HGG, hg = hh - g * HGG;  // head group and head within it
  const int gw = wave_u - g * WG;             // wave within the group
  // Blocks are dispatched to the chip's XCDs round-robin (block b on XCD
  // b % 8).  When blocks_per_group is a multiple of 8, the head groups of one
  // tile run on the same XCD, so the tile's cos/sin rows are fetched into
  // that XCD's L2 once for all its head groups.
  int grp, first_tile;
  if (a.blocks_per_group % kXcds == 0) {
    const int x = blockIdx.x % kXcds, q = blockIdx.x / kXcds;
    grp = q % a.n_groups;
    first_tile = (q / a.n_groups) * kXcds + x;
  } else {
    grp = blockIdx.x % a.n_groups;
    first_tile = blockIdx.x / a.n_groups;
  }
  const int h = grp * HG + hh;
  // Token and tile indices fit 32 bits (n_tokens < 2^31 - 2^7).
  const int n_tok = (int)a.n_tokens;
  const int n_tiles = (n_tok + kTile - 1) / kTile;
  if (first_tile >= n_tiles) return;  // uniform over the block
  const int tile_step = a.blocks_per_group;
  const int count = (n_tiles - first_tile + tile_step - 1) / tile_step;  // tiles of this block
  auto tile_of = [&](int j) __attribute__((always_inline)) -> int { return first_tile + j * tile_step; };
  const uint32_t row_bytes = (uint32_t)(a.stride * ESZ);  // bytes between tokens (<= 2^24)
  // Tokens of tile t that exist (0 past the end).
  // (readfirstlane keeps the value in an SGPR: a buffer resource built from a
  // VGPR would be treated as divergent.)
  auto tile_len = [&](int t) __attribute__((always_inline)) -> uint32_t {
    const int left = n_tok - t * kTile;
    return __builtin_amdgcn_readfirstlane(left <= 0 ? 0 : (left < kTile ? left : kTile));
  };
  // This head's keys of tile t.
  auto keys_rsrc = [&](int t) __attribute__((always_inline)) -> rsrc_t {
    const char* base = (const char*)a.K + ((int64_t)(t * kTile) * a.stride + h * kD) * ESZ;
    return buffer_rsrc(base, tile_len(t) * row_bytes);
  };
  // RoPE layout (token-major, so that every key load covers whole 128-byte
  // lines): wave wq rotates tokens 16 wq + 8 j + (l / 8), j = 0, 1, of the
  // tile; lane l holds channels 8 (l % 8) .. + 7 and their partners 64 higher.
  auto keys_off = [&]() __attribute__((always_inline)) -> uint32_t {
    return (16 * wq + (lane >> 3)) * row_bytes + 8 * (lane & 7) * ESZ;
  };
  // cos/sin rows: wave w of group g fills rows RPG*g + TPW*w .. + TPW - 1 of a
  // tile buffer, two per 16-byte-per-lane load (lanes 0-31 one row, lanes
  // 32-63 the next).  posv[i] is the position of row RPG*g + TPW*w + 2i + (l / 32)
  // of a tile (0 past the end), csv[i] the matching half-row of the table.
  auto load_pos = [&](int t, int* pv) __attribute__((always_inline)) {
    const rsrc_t rs = buffer_rsrc(a.pos + t * kTile, tile_len(t) * 4u);
#pragma unroll
    for (int i = 0; i < NCS; ++i)
      pv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (RPG * g + TPW * gw + 2 * i + lh), 0, 0);
  };
  auto load_cs = [&](const int* pv, u32x4* cv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCS; ++i) {
      const uint32_t p = (uint32_t)min(max(pv[i], 0), a.max_pos - 1);  // clamp to the table
      cv[i] = *(const u32x4*)((const uint8_t*)(a.cs + 2 * col) + ((uint64_t)p << 9));  // 512-byte rows
    }
  };
  auto store_cs = [&](const u32x4* cv, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCS; ++i) *(u32x4*)&cs_lds[buf][RPG * g + TPW * gw + 2 * i + lh][2 * col] = cv[i];
  };
  // Cache rows of tile t's tokens, loaded by wave 0 (lane = token): the raw
  // slot words, turned into a row or -1 by row_of once they have arrived.
  auto load_rows = [&](int t) __attribute__((always_inline)) -> u32x2 {
    const rsrc_t rs = buffer_rsrc(a.slots + t * kTile, tile_len(t) * 8u);
    return __builtin_amdgcn_raw_buffer_load_b64(rs, 8 * lane, 0, 0);
  };
  auto row_of = [&](u32x2 w, int t) __attribute__((always_inline)) -> int32_t {
    const int tok = t * kTile + lane;
    const int64_t row = a.slots ? (int64_t)(((uint64_t)w[1] << 32) | w[0]) : tok;
    return (tok < n_tok && row >= 0 && row < a.n_rows) ? (int32_t)row : -1;
  };

  RawKeys<F32IN> r;  // a tile's keys until RoPE has read them, then the next tile's
  // Prologue: the first tile's keys, rows, positions and cos/sin; T~.
  load_keys<F32IN>(r, keys_rsrc(first_tile), keys_off(), 8 * row_bytes);
  u32x2 row_w = {0u, 0u};  // read only when a.slots is set
  int posv[NCS], posv_n[NCS];  // positions of the next tile's rows, then of the one after
  u32x4 csv[NCS];
  if (a.slots && wave_u == 0) row_w = load_rows(first_tile);
  load_pos(first_tile, posv);
  // This wave's quarter of T~ as MFMA A operands: rows 32 wq + (lane % 32).
  bf16x8 A[8];
  {
    const bf16x8* Tp = (const bf16x8*)a.T;
#pragma unroll
    for (int s = 0; s < 8; ++s) A[s] = Tp[(((int64_t)h * 4 + wq) * 8 + s) * 64 + lane];
  }
  load_cs(posv, csv);
  load_pos(tile_of(1), posv);
  // Nothing may be in flight when the loop starts: its first wait would
  // otherwise also cover the previous tile's stores on later iterations.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  store_cs(csv, 0);
  if (wave_u == 0) slot_lds[0][lane] = row_of(row_w, first_tile);
  __syncthreads();

  f32x16 acc[kNB];
  int tid = threadIdx.x;

  // ---- phase 0 of the group's j-th tile: the stores of tile j - 1, then (for
  // j < count) the loads for later tiles, RoPE and the next tile's keys.
  auto phase0 = [&](int j) __attribute__((always_inline)) {
    // Only this tile's keys can still be in flight (two groups: the phase-2
    // wait leaves them); wait here, before the stores and loads below are
    // issued, so that RoPE does not also wait for those.
    if constexpr (NG == 2) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if constexpr (!YOUT) {
      if (j >= 1) {
        const int sb = (j - 1) & 1;
        // each token's group records are contiguous in the cache row
        // (16-byte chunks, at most one per thread), then its scales (and zeros)
        constexpr int CPT = HGG * BITS;  // 16-byte chunks per token
        constexpr int NCH = kTile * CPT;  // <= 64 * WG
        const uint32_t tg = (uint32_t)(tid - 64 * WG * g);  // thread within the group
        const uint32_t row_rec = (uint32_t)a.n_heads * REC;  // bytes per cache row
        if (NCH == 64 * WG || tg < (uint32_t)NCH) {
          const uint32_t n = tg / CPT, k = tg - n * CPT;
          const int32_t row = slot_lds[sb][n];
          if (row >= 0) {
            // (24-bit multiply: a full 32-bit one issues at a quarter of the rate)
            const u32x4 v = *(const u32x4*)((const uint8_t*)rec_lds[g] + __umul24(n, RECROW) + 16 * k);
            uint8_t* dst = a.codes + (uint64_t)(uint32_t)row * row_rec + ((grp * HG + g * HGG) * REC + 16 * k);
            __builtin_nontemporal_store(v, (u32x4*)dst);  // written once, not read back here
          }
        }
        if constexpr (QK == 0) {
          // one store of the group's HGG fp16 steps per token, by its last wave
          const int n = (int)tg - (64 * WG - 64);
          if (n >= 0) {
            const int32_t row = slot_lds[sb][n];
            if (row >= 0) {
              uint16_t* dst = a.scales + (uint64_t)(uint32_t)row * a.n_heads + grp * HG + g * HGG;
              if constexpr (HGG == 2) {
                *(uint32_t*)dst = *(const uint32_t*)&sc_lds[g][n][0];
              } else {
                *dst = sc_lds[g][n][0];
              }
            }
          }
        } else {
          // per (token, head): 4 scales and 4 zeros, 8 bytes each
          const int c = (int)tg - (64 * WG - 64 * HGG);
          if (c >= 0) {
            const int n = c / HGG, jh = c - n * HGG;
            const int32_t row = slot_lds[sb][n];
            if (row >= 0) {
              const uint64_t slot = (uint64_t)(uint32_t)row * a.n_heads + grp * HG + g * HGG + jh;
              *(uint2*)(a.scales + slot * 4) = *(const uint2*)&sc_lds[g][n][jh * 8];
              *(uint2*)(a.zeros + slot * 4) = *(const uint2*)&sc_lds[g][n][jh * 8 + 4];
            }
          }
        }
      }
    }
    if (j >= count) return;
    const int next = tile_of(j + 1);
    // With two groups, each loads its half of the next tile's cos/sin rows
    // here (its stores above are older, the loads below younger) and writes
    // them to LDS at the end of its phase 1.
    if (NG == 2) load_cs(posv, csv);
    // the next tile's cache rows and the positions of the tile after (zeros
    // past the end)
    if (a.slots && wave_u == 0) row_w = load_rows(next);
    load_pos(tile_of(j + 2), posv_n);
    // RoPE (rotate-half, pairs (i, i+64)) -> bf16 operands in LDS.
    // Chunk c = l % 8 of token t is channels 8c .. 8c+7 (k step c / 2, lane
    // half c % 2 of the B operand) and its partner chunk (k step 4 + c / 2).
    // B-operand rows are stored with lane index lane' ^ (4 (s % 4) + 2 (lane' / 32)),
    // which for this chunk is lane' ^ 2c: the eight chunks of a token land in
    // eight different bank groups, and each row stays a permutation of itself.
    const int cb = j & (CSB - 1);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int c8 = lane & 7, gt = lane >> 3;
      const int t = 16 * wq + 8 * jj + gt;  // token within the tile
      float ka[8], kb[8];
      unpack8<F32IN>(r, jj, 0, ka);
      unpack8<F32IN>(r, jj, 1, kb);
      const float4* csp = (const float4*)&cs_lds[cb][t][8 * c8];
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
      const int nb = t >> 5, s0 = c8 >> 1;
      const int ls = ((t & 31) + 32 * (c8 & 1)) ^ (2 * c8);
      xb_lds[hh][nb][s0][ls] = pack8(xa);
      xb_lds[hh][nb][s0 + 4][ls] = pack8(xb);
    }
    // the next tile's keys, into the registers RoPE has just consumed
    load_keys<F32IN>(r, keys_rsrc(next), keys_off(), 8 * row_bytes);
  };

  // ---- phase 1: y = T~ x~ for this wave's 32 rows and both column blocks,
  // then (symmetric) the sums of squares.
  auto phase1 = [&](int j) __attribute__((always_inline)) {
    // one group: the next tile's cos/sin rows, into registers until phase 2
    // ends (loaded here rather than in phase 0 so they are not live during RoPE)
    if (NG == 1) load_cs(posv, csv);
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) acc[nb] = (f32x16){};
    // B operands one k step ahead of the MFMAs that use them; the scheduling
    // barriers keep the compiler from hoisting all sixteen reads (64 VGPRs).
    {
      // lane index of k step s in the stored row: lane ^ (4 (s % 4) + 2 lh)
      const int lsw = lane ^ (2 * lh);
      bf16x8 bc[kNB], bn[kNB];
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) bc[nb] = xb_lds[hh][nb][0][lsw];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s < 7) {
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) bn[nb] = xb_lds[hh][nb][s + 1][lsw ^ (4 * ((s + 1) & 3))];
        }
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], bc[nb], acc[nb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) bc[nb] = bn[nb];
      }
    }
    if constexpr (YOUT) {
      const int t = tile_of(j);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int64_t tok = (int64_t)t * kTile + 32 * nb + col;
        if (tok < a.n_tokens) {
          float* yo = a.y_out + (tok * a.n_heads + h) * kD;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int rr = 32 * wq + 8 * q + 4 * lh;
            *(float4*)(yo + rr) = make_float4(acc[nb][4 * q], acc[nb][4 * q + 1], acc[nb][4 * q + 2],
                                              acc[nb][4 * q + 3]);
          }
        }
      }
    } else if constexpr (QK == 0) {
      // Sum of squares as the contiguous pairwise tree over rows 0..127:
      // runs of 4 in-lane, pairs of runs across lanes l and l^32, the 32
      // rows of this wave, then the four waves' sums ((0 + 1) + (2 + 3)).
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        float P8[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float q0 = acc[nb][4 * q] * acc[nb][4 * q];
          const float q1 = acc[nb][4 * q + 1] * acc[nb][4 * q + 1];
          const float q2 = acc[nb][4 * q + 2] * acc[nb][4 * q + 2];
          const float q3 = acc[nb][4 * q + 3] * acc[nb][4 * q + 3];
          const float p4 = (q0 + q1) + (q2 + q3);
          const Halves x = halves(p4);
          P8[q] = __uint_as_float(x.lo) + __uint_as_float(x.hi);
        }
        const float P32 = (P8[0] + P8[1]) + (P8[2] + P8[3]);
        if (lh == nb) red_lds[hh][wq][32 * nb + col] = P32;
      }
    }
    if (NG == 2) {
      // the cos/sin rows loaded in phase 0 have landed: only the younger
      // cache-row, position and key loads (and, for the y output, its stores)
      // may still be in flight
      if constexpr (YOUT) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70 | (NCS + NKL));  // vmcnt(NCS + NKL)
      }
      store_cs(csv, (j + 1) & 1);
    }
  };

  // ---- phase 2: scales, codes and records of tile j -> LDS; then every load
  // has landed and (group 0) the next tile's cos/sin rows and cache rows go to LDS.
  auto phase2 = [&](int j) __attribute__((always_inline)) {
    if constexpr (!YOUT) {
      // Output element acc[nb][i] is row 32*wq + 8*(i/4) + 4*lh + (i%4) of
      // token 32*nb + col.  run[nb][q] packs the codes of acc[nb][4q .. 4q+3]
      // (4 consecutive rows), LSB first.
      uint32_t run[kNB][4];
      uint32_t W2[kNB] = {};  // 2-bit symmetric: whole words of codes
      if constexpr (QK == 0) {
        // One step per lane for token tt = 32 lh + col (the lane pair l, l^32
        // covers both column blocks): column block nb's step is then the
        // value of lane half nb.
        const int tt = 32 * lh + col;
        const float S = (red_lds[hh][0][tt] + red_lds[hh][1][tt]) + (red_lds[hh][2][tt] + red_lds[hh][3][tt]);
        const float ms = S * 0.0078125f;  // S / 128, exact scaling
        const float rms = __builtin_sqrtf(ms);
        const float C = a.q.alpha * rms;
        const float twoC = 2.0f * C;
        const float d32 = twoC / (float)(L - 1);
        const uint16_t dh = f16_sat_bits(d32);
        if (wq == 0) sc_lds[g][tt][hg] = dh;
        const Halves dd = halves(f16_bits_to_f32(dh));
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const float delta = __uint_as_float(nb ? dd.hi : dd.lo);
          // A zero step becomes +inf (threshold / step) so every code comes out L/2.
          const float tp = delta == 0.0f ? __builtin_inff() : delta;
          if constexpr (BITS == 2) {
            // W2[nb]: the lane's 16 codes of the block, run q (4 rows) in byte
            // q, shifted in from the last row down (alignbit: w = 2w + bit 31
            // of the operand).  Code = [y > -step] + [y >= 0] + [y > step]:
            // the high bit is [y >= 0], the sign of y inverted (an MFMA result
            // that starts from a +0 accumulator is never -0); the low bit is
            // [y > t] with t = +-step carrying y's sign, i.e. the sign of
            // t - y, which is +0 (bit clear) exactly at a tie.  A zero step
            // gives code 2 everywhere.
            const uint32_t db = __float_as_uint(delta);
            uint32_t w = 0;
#pragma unroll
            for (int i = 15; i >= 0; --i) {
              const float y = acc[nb][i];
              const float t = __uint_as_float((__float_as_uint(y) & 0x80000000u) | db);
              w = __builtin_amdgcn_alignbit(w, __float_as_uint(y), 31);
              w = __builtin_amdgcn_alignbit(w, __float_as_uint(t - y), 31);
            }
            W2[nb] = delta == 0.0f ? 0xAAAAAAAAu : w ^ 0xAAAAAAAAu;
          } else {
            const float rd = delta == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(delta);
            bool near = false;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint32_t rc = 0;
#pragma unroll
              for (int e = 0; e < 4; ++e) rc |= sym_code_fast<BITS>(acc[nb][4 * q + e], rd, near) << (BITS * e);
              run[nb][q] = rc;
            }
            near = near && rd != 0.0f;
            // rare: a value within rounding error of a midpoint; exact codes for those lanes
            if (__builtin_amdgcn_ballot_w64(near) != 0) {
              if (near) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  uint32_t rc = 0;
#pragma unroll
                  for (int e = 0; e < 4; ++e) rc |= sym_code<BITS>(acc[nb][4 * q + e], tp, rd) << (BITS * e);
                  asm("" : "+v"(rc));  // keep the word 32 bits wide (compare + add-with-carry codegen)
                  run[nb][q] = rc;
                }
              }
            }
          }
        }
      } else {
        // Percentile-clipped affine quantizer, group = this wave's 32 rows of
        // a token, split between lanes l and l^32: two smallest and two
        // largest values by IEEE totalOrder, merged across the lane pair.
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          int32_t mn1 = INT_MAX, mn2 = INT_MAX, mx1 = INT_MIN, mx2 = INT_MIN;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int32_t k = total_order_key(acc[nb][i]);
            mn2 = min(mn2, max(mn1, k));
            mn1 = min(mn1, k);
            mx2 = max(mx2, min(mx1, k));
            mx1 = max(mx1, k);
          }
          const Halves n1 = halves((uint32_t)mn1), n2 = halves((uint32_t)mn2);
          const Halves x1 = halves((uint32_t)mx1), x2 = halves((uint32_t)mx2);
          const int32_t a1 = (int32_t)n1.lo, b1 = (int32_t)n1.hi, a2 = (int32_t)n2.lo, b2 = (int32_t)n2.hi;
          const int32_t c1 = (int32_t)x1.lo, d1 = (int32_t)x1.hi, c2 = (int32_t)x2.lo, d2 = (int32_t)x2.hi;
          const float s0 = total_order_value(min(a1, b1));
          const float s1 = total_order_value(min(max(a1, b1), min(a2, b2)));
          const float s31 = total_order_value(max(c1, d1));
          const float s30 = total_order_value(max(min(c1, d1), max(c2, d2)));
          const float lo = a.q.lo_mode ? s0 : __builtin_fmaf(a.q.g_lo, s1 - s0, s0);
          const float hi = a.q.hi_mode == 0 ? __builtin_fmaf(a.q.g_hi, s31 - s30, s30)
                                            : (a.q.hi_mode == 1 ? s30 : s31);
          const float s32 = (hi - lo) / (float)(L - 1);
          const uint16_t sh = f16_sat_bits(s32), zh = f16_sat_bits(lo);
          const float s32h = f16_bits_to_f32(sh), z32h = f16_bits_to_f32(zh);
          const float rs = s32h == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s32h);
          bool near = false;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t rc = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) rc |= affine_code_fast<BITS>(acc[nb][4 * q + e], z32h, rs, near) << (BITS * e);
            run[nb][q] = rc;
          }
          // rare: a value within rounding error of a midpoint; exact codes for those lanes
          if (__builtin_amdgcn_ballot_w64(near) != 0) {
            if (near) {
              const double sd = (double)s32h, zd = (double)z32h;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                uint32_t rc = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const uint32_t cd = sd == 0.0 ? 0u : affine_code<BITS>(acc[nb][4 * q + e], zd, sd);
                  rc |= cd << (BITS * e);
                }
                run[nb][q] = rc;
              }
            }
          }
          if (lh == 0) {
            sc_lds[g][32 * nb + col][hg * 8 + wq] = sh;
            sc_lds[g][32 * nb + col][hg * 8 + 4 + wq] = zh;
          }
        }
      }

      // pack: runs of 4 codes -> 16 contiguous rows per lane -> LDS record row.
      // Lane l (lh = 0) writes rows 0-15 of the block: its runs 0, 1
      // interleaved with those of lane l + 32; lane l + 32 writes rows 16-31.
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        uint8_t* dst = &rec_lds[g][32 * nb + col][hg * REC + BITS * (4 * wq + 2 * lh)];
        if constexpr (QK == 0 && BITS == 2) {
          // bytes {lane half 0: selectors 0-3, lane half 1: 4-7}: lh = 0 takes
          // bytes 0, 1 of both, lh = 1 bytes 2, 3
          const Halves w = halves(W2[nb]);
          *(uint32_t*)dst = __builtin_amdgcn_perm(w.hi, w.lo, lh ? 0x07030602u : 0x05010400u);
        } else {
          const uint32_t* rn = run[nb];
          const uint32_t send = lh ? (rn[0] | (rn[1] << RB)) : (rn[2] | (rn[3] << RB));
          const Halves w = halves(send);
          const uint32_t recv = lh ? w.lo : w.hi;
          const uint64_t p0 = recv & ((1u << RB) - 1u), p1 = recv >> RB;
          const uint64_t chunk =
              lh ? (p0 | ((uint64_t)rn[2] << RB) | (p1 << (2 * RB)) | ((uint64_t)rn[3] << (3 * RB)))
                 : ((uint64_t)rn[0] | (p0 << RB) | ((uint64_t)rn[1] << (2 * RB)) | (p1 << (3 * RB)));
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
      }
    }
    // The cache rows and positions have landed.  With two groups the next
    // tile's keys (the youngest loads) stay in flight until RoPE needs them;
    // one group also waits for its cos/sin rows, loaded after the keys.
    if constexpr (NG == 2 && !YOUT) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | NKL);  // vmcnt(NKL), expcnt and lgkmcnt untouched
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    if (g == 0) {
      const int next = tile_of(j + 1);
      if (wave_u == 0) slot_lds[(j + 1) & 1][lane] = row_of(row_w, next);
      if (NG == 1) store_cs(csv, 0);
    }
#pragma unroll
    for (int i = 0; i < NCS; ++i) posv[i] = posv_n[i];
  };

  // Schedule.  Each group runs phase 0, 1, 2 of its tiles in turn with a
  // block barrier after every phase; group 1 starts one barrier later (and
  // group 0 ends one later), so group 1 trails group 0 by one phase: while one
  // group's waves run their MFMA phase the other group's waves, on the same
  // SIMDs, run VALU work.  Both groups pass the same number of barriers
  // (3 count + 2), and every barrier orders the LDS hand-offs within and
  // between the groups: cos/sin tile j lives in buffer j % CSB from the end of
  // each group's phase 1 of tile j - 1 until group 1's phase 0 of tile j (one
  // group: from its phase 2 of tile j - 1 until its phase 0 of tile j), and the cache
  // rows of tile j in slot_lds[j % 2] until group 1's stores of tile j.
  auto next_phase = [&]() __attribute__((always_inline)) {
    __syncthreads();
    asm volatile("" : "+v"(lane));
    lh = lane >> 5;
    col = lane & 31;
    tid = 64 * wave_u + lane;
  };
  if (NG == 2 && g == 1) next_phase();
  for (int j = 0; j < count; ++j) {
    phase0(j);
    next_phase();
    phase1(j);
    next_phase();
    phase2(j);
    next_phase();
  }
  phase0(count);  // the last tile's stores
  next_phase();
  if (NG == 2 && g == 0) next_phase();
}

// (cos, sin) of every position p < max_pos, pair i: entry p * 64 + i.
__global__ void build_cs_table_kernel(RopeTables t, int64_t n, float2* cs) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  cs[idx] = rope_cos_sin((int)(idx / kPairs), (int)(idx % kPairs), t);
}

__global__ void gather_cs_kernel(const float2* table, int32_t max_pos, const int32_t* pos, int64_t n,
                                 float2* out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * kPairs) return;
  const int64_t k = idx / kPairs;
  int p = pos[k];
  p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
  out[idx] = table[(int64_t)p * kPairs + (idx - k * kPairs)];
}

// Persistent grid: as many blocks per head group as fit on the chip at once.
// The cache is per kernel instantiation (K is the kernel itself, not its type,
// which all instantiations share).
template <auto K>
int resident_blocks(int threads) {
  static int cached = 0;
  if (!cached) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, K, threads, 0) != hipSuccess || n < 1) n = 1;
    cached = n;
  }
  return cached;
}

template <int BITS, int QK, bool F32IN, int HG, bool YOUT>
hipError_t launch_one(KeysArgs a, int cus, hipStream_t st) {
  constexpr auto k = keys_kernel<BITS, QK, F32IN, HG, YOUT>;
  const int64_t n_tiles = (a.n_tokens + kTile - 1) / kTile;
  int64_t b = (int64_t)cus * resident_blocks<k>(256 * HG) / a.n_groups;
  b = b < 1 ? 1 : (b > n_tiles ? n_tiles : b);
  if (b >= kXcds) b -= b % kXcds;  // multiple of 8: XCD-aware tile mapping
  a.blocks_per_group = (int)b;
  return launch_kernel(k, dim3((unsigned)(a.n_groups * b)), dim3(256 * HG), st, a);
}

template <int BITS, int QK, bool F32IN, bool YOUT>
hipError_t launch_hg(const KeysArgs& a, int hg, int cus, hipStream_t st) {
  switch (hg) {
    case 1: return launch_one<BITS, QK, F32IN, 1, YOUT>(a, cus, st);
    case 2: return launch_one<BITS, QK, F32IN, 2, YOUT>(a, cus, st);
    case 4:
      if constexpr (!F32IN) return launch_one<BITS, QK, F32IN, 4, YOUT>(a, cus, st);
      break;
  }
  return hipErrorInvalidValue;
}

template <int BITS, int QK>
hipError_t launch_bits(const KeysArgs& a, int f32_in, int hg, int y_out, int cus, hipStream_t st) {
  if (y_out) return f32_in ? launch_hg<BITS, QK, true, true>(a, hg, cus, st)
                           : launch_hg<BITS, QK, false, true>(a, hg, cus, st);
  return f32_in ? launch_hg<BITS, QK, true, false>(a, hg, cus, st)
                : launch_hg<BITS, QK, false, false>(a, hg, cus, st);
}

}  // namespace

hipError_t launch_keys(const KeysArgs& a, int bits, int f32_in, int hg, int y_out, int cus, hipStream_t st) {
  if (y_out) return launch_bits<2, 0>(a, f32_in, hg, 1, cus, st);  // transform only
  if (a.q.kind == 0) {
    switch (bits) {
      case 2: return launch_bits<2, 0>(a, f32_in, hg, 0, cus, st);
      case 3: return launch_bits<3, 0>(a, f32_in, hg, 0, cus, st);
      case 4: return launch_bits<4, 0>(a, f32_in, hg, 0, cus, st);
    }
  } else {
    switch (bits) {
      case 2: return launch_bits<2, 1>(a, f32_in, hg, 0, cus, st);
      case 3: return launch_bits<3, 1>(a, f32_in, hg, 0, cus, st);
      case 4: return launch_bits<4, 1>(a, f32_in, hg, 0, cus, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_build_cs_table(const wushkv_rope* r, hipStream_t st) {
  const int64_t total = (int64_t)r->max_pos * kPairs;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  const RopeTables t{r->t0, r->t1, r->t2, r->t0t, r->t1t, r->t2t};
  build_cs_table_kernel<<<dim3((unsigned)blocks), threads, 0, st>>>(t, total, r->cs);
  return hipGetLastError();
}

hipError_t launch_gather_cs(const wushkv_rope* r, const int32_t* pos, int64_t n, float* cs_out,
                            hipStream_t st) {
  const int64_t total = n * kPairs;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  gather_cs_kernel<<<dim3((unsigned)blocks), threads, 0, st>>>(r->cs, r->max_pos, pos, n, (float2*)cs_out);
  return hipGetLastError();
}

}  // namespace wushkv
