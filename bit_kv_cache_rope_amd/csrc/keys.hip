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
// 16 v_mfma_f32_32x32x16_bf16.  The B operand is the tile's rotated keys: lane
// l holds token l%32 and, for k step s, channels 16s + 8(l/32) + 0..7, so the
// RoPE partners (i, i+64) sit in one lane (k steps s and s+4).  Each wave of a
// head loads and rotates half of the pairs (k steps 2*half, 2*half+1 and their
// partners) and the two waves swap their bf16 operands through LDS.
//
// cos/sin for a tile are computed once per block into LDS (double-buffered);
// the two small angle tables live in LDS for the whole launch, and the
// high-angle table entries (and slot rows) are loaded two tiles ahead, the
// positions three tiles ahead, so that no computation waits on a fresh load.
//
// Per-tile pipeline.  Vector-memory loads retire in order, so each iteration
// issues the loads for later tiles first (table entries, positions), then the
// next tile's keys, and the work that consumes only older data runs while they
// are in flight.  Every iteration ends with one explicit wait before its
// stores, and the loop is unrolled by two over two register sets, so the
// compiler's own waits never cover the key prefetch.  Packed records and
// scales are staged in LDS and written as whole 16-byte chunks (a head
// group's records of a token are contiguous in the cache row).
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

// The four k steps a wave loads and rotates: 2h, 2h+1 and their partners +4.
__device__ __forceinline__ int own_step(int j, int half) { return (j & 1) + 2 * half + 4 * (j >> 1); }

template <bool F32IN>
struct RawKeys;
template <>
struct RawKeys<false> {  // bf16: 8 channels per 16-byte load, 4 k steps
  uint4 v[4];
};
template <>
struct RawKeys<true> {   // fp32: 8 channels = two 16-byte loads
  float4 v[8];
};

// Loads are unconditional: a token past the end reads the last token's row (its
// results are never stored), so the compiler never has to cover a
// conditionally issued load with its waits.
template <bool F32IN>
__device__ __forceinline__ void load_keys(RawKeys<F32IN>& r, const KeysArgs& a, int64_t tok, int h, int lh,
                                          int half) {
  tok = tok < a.n_tokens ? tok : a.n_tokens - 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = own_step(j, half);
    if constexpr (F32IN) {
      const float* base = (const float*)a.K + tok * a.stride + (int64_t)h * kD + 16 * s + 8 * lh;
      r.v[2 * j] = *(const float4*)base;
      r.v[2 * j + 1] = *(const float4*)(base + 4);
    } else {
      r.v[j] = *(const uint4*)((const uint16_t*)a.K + tok * a.stride + (int64_t)h * kD + 16 * s + 8 * lh);
    }
  }
}

template <bool F32IN>
__device__ __forceinline__ void unpack8(const RawKeys<F32IN>& r, int j, float* x) {
  if constexpr (F32IN) {
    const float4 p = r.v[2 * j], q = r.v[2 * j + 1];
    x[0] = p.x; x[1] = p.y; x[2] = p.z; x[3] = p.w;
    x[4] = q.x; x[5] = q.y; x[6] = q.z; x[7] = q.w;
  } else {
    const uint4 p = r.v[j];
    x[0] = bf16lo_to_f32(p.x); x[1] = bf16hi_to_f32(p.x);
    x[2] = bf16lo_to_f32(p.y); x[3] = bf16hi_to_f32(p.y);
    x[4] = bf16lo_to_f32(p.z); x[5] = bf16hi_to_f32(p.z);
    x[6] = bf16lo_to_f32(p.w); x[7] = bf16hi_to_f32(p.w);
  }
}

// High-angle table entries and slot rows of one future tile.
template <int PPT>
struct CsStage {
  double2 hi[PPT];
  int64_t slot;
};

template <int BITS, int QK, bool F32IN, int HG, bool YOUT>
__global__ void __launch_bounds__(128 * HG) keys_kernel(const KeysArgs a) {
  constexpr int NT = 128 * HG;
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  constexpr int RECROW = HG * REC + 16;  // LDS row of one token's records (+16 B pad)
  constexpr int NSC = QK ? 8 : 1;        // fp16 values per (token, head): sym 1; affine 4 + 4
  constexpr int RB = 4 * BITS;           // bits in a run of 4 codes
  constexpr int PPT = kTile * kPairs / NT;  // cos/sin pairs per thread per tile

  __shared__ __align__(16) double2 tab_lds[2][32][kPairs];  // heads of the p0 and p1 angle tables
  __shared__ __align__(16) float2 cs_lds[2][kTile][kCsStride];
  __shared__ __align__(16) bf16x8 xb_lds[HG][8][64];        // rotated operands swapped between a head's waves
  __shared__ int64_t slot_lds[2][kTile];
  __shared__ int pos_lds[4][kTile];
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

  // Angle tables t0 (p0) and t1 (p1) into LDS for the whole launch.
  for (int e = tid; e < 2 * 32 * kPairs; e += NT) {
    const int t = e / (32 * kPairs), r = e - t * 32 * kPairs;
    tab_lds[t][r / kPairs][r % kPairs] = (t == 0 ? a.t0 : a.t1)[r];
  }

  // Tiles are visited as j = 0, 1, 2, ...: tile(j) = first_tile + j * tile_step.
  // Thread (wave w, lane i) computes cos/sin pair i of tokens w + (NT/64) k,
  // k < PPT, so every position it reads is wave-uniform.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int64_t last_tok = a.n_tokens - 1;
  int pos_r = 0;
  auto load_pos = [&](int64_t tile) __attribute__((always_inline)) {
    const int64_t tok = tile * kTile + (tid & (kTile - 1));
    pos_r = a.pos[tok < last_tok ? tok : last_tok];
  };
  auto store_pos = [&](int pb) __attribute__((always_inline)) {
    if (tid < kTile) {
      const int p = pos_r;
      pos_lds[pb][tid] = p < 0 ? 0 : (p >= a.max_pos ? a.max_pos - 1 : p);
    }
  };
  // Position of token n of the tile in pos_lds slot pb (uniform over the wave).
  auto pos_of = [&](int pb, int n) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(pos_lds[pb][n]);
  };
  auto issue_cs = [&](CsStage<PPT>& st, int64_t tile, int pb) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) st.hi[k] = a.t2[(pos_of(pb, wave_u + (NT / 64) * k) >> 10) * kPairs + lane];
    if (a.slots) {
      const int64_t tok = tile * kTile + (tid & (kTile - 1));
      st.slot = a.slots[tok < last_tok ? tok : last_tok];
    }
  };
  // Fast path for every pair; the rare pairs whose fp32 rounding it cannot
  // certify are redone in double-double in a loop that is not unrolled (its
  // loads are issued only when such a pair occurs).
  auto finish_cs = [&](const CsStage<PPT>& st, int64_t tile, int pb, int buf) __attribute__((always_inline)) {
    uint32_t bad = 0;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int n = wave_u + (NT / 64) * k;
      const int p = pos_of(pb, n);
      const double2 M = tab_lds[1][(p >> 5) & 31][lane], B = tab_lds[0][p & 31][lane];
      bool exact;
      cs_lds[buf][n][lane] = rope_cos_sin_fast(st.hi[k], M, B, exact);
      bad |= (uint32_t)!exact << k;
    }
    if (__builtin_expect(bad != 0, 0)) {
#pragma unroll 1
      for (int k = 0; k < PPT; ++k) {
        if ((bad >> k) & 1) {
          const int n = wave_u + (NT / 64) * k;
          const int p = pos_lds[pb][n];
          const int p2 = p >> 10, p1 = (p >> 5) & 31, p0 = p & 31;
          cs_lds[buf][n][lane] =
              rope_cos_sin_slow(a.t2[p2 * kPairs + lane], a.t2t[p2 * kPairs + lane], tab_lds[1][p1][lane],
                                a.t1t[p1 * kPairs + lane], tab_lds[0][p0][lane], a.t0t[p0 * kPairs + lane]);
        }
      }
    }
    if (tid < kTile) slot_lds[buf][tid] = a.slots ? st.slot : tile * kTile + tid;
  };

  RawKeys<F32IN> ra, rb;
  CsStage<PPT> sa, sb;
  int64_t tile = first_tile;
  int buf = 0, j = 0;
  load_pos(tile);
  store_pos(0);
  for (int d = 1; d < 3; ++d)
    if (tile + d * tile_step < n_tiles) {
      load_pos(tile + d * tile_step);
      store_pos(d);
    }
  __syncthreads();  // angle tables and the first three tiles' positions
  issue_cs(sa, tile, 0);
  load_keys<F32IN>(ra, a, tile * kTile + col, h, lh, half);
  finish_cs(sa, tile, 0, 0);
  if (tile + tile_step < n_tiles) issue_cs(sb, tile + tile_step, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the loop starts with nothing in flight
  __syncthreads();

  // One tile per call: `cur` holds this tile's keys, `nxt` receives the next
  // tile's; `rdy` holds the next tile's table entries (consumed first, so its
  // registers are free again), `fut` receives those of the tile after.
  // Unrolled by two with the sets swapped.
  auto step = [&](RawKeys<F32IN>& cur, RawKeys<F32IN>& nxt, CsStage<PPT>& rdy, CsStage<PPT>& fut)
      __attribute__((always_inline)) -> bool {
    const int64_t next = tile + tile_step, next2 = next + tile_step, next3 = next2 + tile_step;
    const bool has_next = next < n_tiles, has_next2 = next2 < n_tiles, has_next3 = next3 < n_tiles;
    if (has_next) finish_cs(rdy, next, (j + 1) & 3, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    if (has_next2) issue_cs(fut, next2, (j + 2) & 3);
    if (has_next3) load_pos(next3);
    __builtin_amdgcn_sched_barrier(0);
    if (has_next) load_keys<F32IN>(nxt, a, next * kTile + col, h, lh, half);
    __builtin_amdgcn_sched_barrier(0);

    // ---- RoPE (rotate-half, pairs (i, i+64)) of this wave's pairs -> bf16 operands
    bf16x8 Bop[8];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int s = 2 * half + jj;  // k step of channels i; the partners are in k step s + 4
      float ka[8], kb[8];
      unpack8<F32IN>(cur, jj, ka);
      unpack8<F32IN>(cur, jj + 2, kb);
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
      xb_lds[hh][s][lane] = pack8(xa);
      xb_lds[hh][s + 4][lane] = pack8(xb);
    }
    __syncthreads();
    // All eight operands come back from LDS: indexing registers by the
    // wave's half would turn into select chains.
#pragma unroll
    for (int s = 0; s < 8; ++s) Bop[s] = xb_lds[hh][s][lane];

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
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 32 * (2 * half + m) + 8 * jj + 4 * lh;
            *(float4*)(yo + r) = make_float4(acc[m][4 * jj], acc[m][4 * jj + 1], acc[m][4 * jj + 2],
                                             acc[m][4 * jj + 3]);
          }
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
    } else {
      // Output element acc[m][i] is row 32*(2*half+m) + 8*(i/4) + 4*lh + (i%4) of token `col`.
      // run[m][q] packs the codes of acc[m][4q .. 4q+3] (4 consecutive rows), LSB first.
      uint32_t run[2][4];
      uint32_t W2[2];  // 2-bit symmetric: whole words of codes
      if constexpr (QK == 0) {
        // Sum of squares as the contiguous pairwise tree over rows 0..127:
        // runs of 4 in-lane, pairs of runs across lanes l and l^32, then up.
        float P8[2][4];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float q0 = acc[m][4 * q] * acc[m][4 * q];
            const float q1 = acc[m][4 * q + 1] * acc[m][4 * q + 1];
            const float q2 = acc[m][4 * q + 2] * acc[m][4 * q + 2];
            const float q3 = acc[m][4 * q + 3] * acc[m][4 * q + 3];
            const float p4 = (q0 + q1) + (q2 + q3);
            P8[m][q] = p4 + __shfl_xor(p4, 32);
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
        // A zero step becomes +inf (threshold / step) so every code comes out L/2.
        const float tp = delta == 0.0f ? __builtin_inff() : delta;
        const float tz = delta == 0.0f ? -__builtin_inff() : 0.0f;
        const float rd = delta == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(delta);
        if constexpr (BITS == 2) {
          // W[m]: the lane's 16 codes of m-tile m, run q (4 rows) in byte q,
          // shifted in from the last row down.  Midpoint tests A = [y > -step],
          // B = [y >= 0], C = [y > step]; code bits B and C | (A & !B).
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            uint32_t w = 0;
#pragma unroll
            for (int g = 3; g >= 0; --g) {  // 4 rows per add-with-carry block
              uint64_t mk[8];
#pragma unroll
              for (int e = 3; e >= 0; --e) {
                const float y = acc[m][4 * g + e];
                const Sym2Masks k = sym2_masks(y > -tp, y >= tz, y > tp);
                mk[2 * (3 - e)] = k.b1;
                mk[2 * (3 - e) + 1] = k.b0;
              }
              w = shift_in8(w, mk);
            }
            W2[m] = w;
          }
        } else {
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              uint32_t r = 0;
#pragma unroll
              for (int e = 0; e < 4; ++e) r |= sym_code<BITS>(acc[m][4 * q + e], tp, rd) << (BITS * e);
              asm("" : "+v"(r));  // keep the word 32 bits wide (compare + add-with-carry codegen)
              run[m][q] = r;
            }
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
          for (int q = 0; q < 4; ++q) {
            uint32_t r = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t c = sd == 0.0 ? 0u : affine_code<BITS>(acc[m][4 * q + e], zd, sd);
              r |= c << (BITS * e);
            }
            run[m][q] = r;
          }
          if (lh == 0) {
            sc_lds[col][hh * 8 + 2 * half + m] = sh;
            sc_lds[col][hh * 8 + 4 + 2 * half + m] = zh;
          }
        }
      }

      // ---- pack: runs of 4 codes -> 16 contiguous rows per lane -> LDS record row.
      // Lane l (lh = 0) writes rows 0-15 of the m-tile: its runs 0, 1 interleaved
      // with those of lane l + 32; lane l + 32 writes rows 16-31 likewise.
      if constexpr (QK == 0 && BITS == 2) {
        // bytes of {partner (selectors 4-7), own (0-3)}
        const uint32_t sel = lh ? 0x03070206u : 0x05010400u;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint32_t chunk = __builtin_amdgcn_perm(__shfl_xor(W2[m], 32), W2[m], sel);
          *(uint32_t*)&rec_lds[col][hh * REC + 2 * (4 * (2 * half + m) + 2 * lh)] = chunk;
        }
      } else
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
      // The loads for later tiles have been in flight during this tile's work;
      // wait for them here (vmcnt = 0, expcnt and lgkmcnt untouched) so that
      // every iteration starts with no vector-memory loads outstanding.
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();

      // ---- stores: each token's HG records are contiguous in the cache row
      const int64_t tbase = tile * kTile;
      constexpr int CPT = HG * BITS;  // 16-byte chunks per token
      for (int c = tid; c < kTile * CPT; c += NT) {
        const int n = c / CPT, k = c - n * CPT;
        const int64_t t = tbase + n;
        if (t < a.n_tokens) {
          const int64_t row = slot_lds[buf][n];
          if (row >= 0 && row < a.n_rows) {
            const uint4 v = *(const uint4*)&rec_lds[n][16 * k];
            *(uint4*)(a.codes + (row * a.n_heads + grp * HG) * REC + 16 * k) = v;
          }
        }
      }
      for (int c = tid; c < kTile * HG; c += NT) {
        const int n = c / HG, jh = c - n * HG;
        const int64_t t = tbase + n;
        if (t < a.n_tokens) {
          const int64_t row = slot_lds[buf][n];
          if (row >= 0 && row < a.n_rows) {
            const int64_t slot = row * a.n_heads + grp * HG + jh;
            if constexpr (QK == 0) {
              a.scales[slot] = sc_lds[n][jh];
            } else {
              const uint16_t* s = &sc_lds[n][jh * 8];
              *(uint2*)(a.scales + slot * 4) =
                  make_uint2(s[0] | ((uint32_t)s[1] << 16), s[2] | ((uint32_t)s[3] << 16));
              *(uint2*)(a.zeros + slot * 4) =
                  make_uint2(s[4] | ((uint32_t)s[5] << 16), s[6] | ((uint32_t)s[7] << 16));
            }
          }
        }
      }
    }
    if (has_next3) store_pos((j + 3) & 3);  // its load has completed: every path above waits for vmcnt 0
    __syncthreads();
    if (has_next) {
      tile = next;
      buf ^= 1;
      ++j;
    }
    return has_next;
  };
  while (true) {
    if (!step(ra, rb, sb, sa)) break;
    if (!step(rb, ra, sa, sb)) break;
  }
}

__global__ void rope_cos_sin_kernel(RopeTables t, int32_t max_pos, const int32_t* pos, int64_t n, float* cs) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * kPairs) return;
  const int64_t k = idx / kPairs;
  const int i = (int)(idx - k * kPairs);
  int p = pos[k];
  p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
  const float2 v = rope_cos_sin(p, i, t);
  cs[2 * idx] = v.x;
  cs[2 * idx + 1] = v.y;
}

// Persistent grid: as many blocks per head group as fit on the chip at once.
template <typename Kernel>
int resident_blocks(Kernel k, int threads) {
  static int cached = 0;  // one value per kernel instantiation
  if (!cached) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, threads, 0) != hipSuccess || n < 1) n = 1;
    cached = n;
  }
  return cached;
}

template <int BITS, int QK, bool F32IN, int HG, bool YOUT>
hipError_t launch_one(KeysArgs a, int cus, hipStream_t st) {
  auto k = keys_kernel<BITS, QK, F32IN, HG, YOUT>;
  const int64_t n_tiles = (a.n_tokens + kTile - 1) / kTile;
  int64_t b = (int64_t)cus * resident_blocks(k, 128 * HG) / a.n_groups;
  b = b < 1 ? 1 : (b > n_tiles ? n_tiles : b);
  a.blocks_per_group = (int)b;
  k<<<dim3((unsigned)(a.n_groups * b)), 128 * HG, 0, st>>>(a);
  return hipGetLastError();
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

hipError_t launch_rope_cos_sin(const wushkv_rope* r, const int32_t* pos, int64_t n, float* cs,
                               hipStream_t st) {
  const int64_t total = n * kPairs;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  const RopeTables t{r->t0, r->t1, r->t2, r->t0t, r->t1t, r->t2t};
  rope_cos_sin_kernel<<<dim3((unsigned)blocks), threads, 0, st>>>(t, r->max_pos, pos, n, cs);
  return hipGetLastError();
}

}  // namespace wushkv
