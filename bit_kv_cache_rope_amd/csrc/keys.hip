// Fused key path for gfx950: RoPE -> bf16 -> per-head 128x128 transform on
// MFMA (bf16 in, fp32 accumulate) -> clipped b-bit quantizer -> bit packing.
//
// The key transform is a general invertible per-KV-head matrix applied online
// after RoPE (ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity ...",
// method and deployment paragraphs; cere-bro post "WUSH-KV: 2-bit KV-Cache
// Quantization with Data-Adaptive Transforms", Gaps).
//
// Work decomposition.  A block owns HG heads and walks 32-token tiles
// (persistent: tile = first, first + blocks_per_group, ...).  Four waves serve
// each head; wave wq keeps rows [32 wq, 32 wq + 32) of T~ (32 VGPRs of A
// operands, loaded once) and computes those output rows for the tile with 8
// v_mfma_f32_32x32x16_bf16.  The B operand is the tile's rotated keys: lane l
// holds token l%32 and, for k step s, channels 16s + 8(l/32) + 0..7, so the
// RoPE partners (i, i+64) sit in one lane (k steps s and s+4).  Wave wq loads
// and rotates k step wq and its partner, and the four waves share their bf16
// operands through LDS.  At under 128 VGPRs, four waves per SIMD are resident.
//
// cos/sin for a tile are computed once per block into LDS; the two small
// angle tables live in LDS for the whole launch, and the high-angle table
// entries (and slot rows) are loaded a tile ahead of their use, the positions
// three tiles ahead, so that no computation waits on a fresh load.
//
// Per-tile pipeline.  Vector-memory loads retire in order, so each iteration
// issues the next tile's position and keys first and its table entries last,
// and ends with one explicit wait for all but those table entries before its
// stores; the loop is unrolled by two over two key register sets, so the
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

// The two k steps a wave loads and rotates: wq (channels i < 64) and its
// partner wq + 4 (channels i + 64).
template <bool F32IN>
struct RawKeys;
template <>
struct RawKeys<false> {  // bf16: 8 channels per 16-byte load, 2 k steps
  uint4 v[2];
};
template <>
struct RawKeys<true> {   // fp32: 8 channels = two 16-byte loads
  float4 v[4];
};

// Loads are unconditional: a token past the end reads the last token's row (its
// results are never stored), so the compiler never has to cover a
// conditionally issued load with its waits.
template <bool F32IN>
__device__ __forceinline__ void load_keys(RawKeys<F32IN>& r, const KeysArgs& a, int64_t tok, int h, int lh,
                                          int wq) {
  tok = tok < a.n_tokens ? tok : a.n_tokens - 1;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int s = wq + 4 * j;
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
__global__ void __launch_bounds__(256 * HG) keys_kernel(const KeysArgs a) {
  constexpr int NT = 256 * HG;
  constexpr int NW = NT / 64;
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  constexpr int RECROW = HG * REC + 16;  // LDS row of one token's records (+16 B pad)
  constexpr int NSC = QK ? 8 : 1;        // fp16 values per (token, head): sym 1; affine 4 + 4
  constexpr int RB = 4 * BITS;           // bits in a run of 4 codes
  constexpr int PPT = kTile * kPairs / NT;  // cos/sin pairs per thread per tile

  __shared__ __align__(16) double2 tab_lds[2][32][kPairs];  // heads of the p0 and p1 angle tables
  __shared__ __align__(16) float2 cs_lds[2][kTile][kCsStride];
  __shared__ __align__(16) bf16x8 xb_lds[HG][8][64];        // rotated operands shared by a head's four waves
  __shared__ int64_t slot_lds[3][kTile];  // cache row per token, tile j in slot j % 3
  __shared__ int pos_lds[4][kTile];
  __shared__ float red_lds[HG][4][kTile];
  __shared__ __align__(16) uint8_t rec_lds[kTile][RECROW];
  __shared__ uint16_t sc_lds[kTile][HG * NSC];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // Four waves per head: wave wq holds rows 32 wq .. 32 wq + 31 of T~ and
  // rotates the RoPE pairs of k step wq (channels 16 wq + 8 (l / 32) + 0..7
  // and their partners 64 higher).
  const int hh = wave >> 2, wq = wave & 3, lh = lane >> 5, col = lane & 31;
  const int grp = blockIdx.x % a.n_groups;
  const int64_t first_tile = blockIdx.x / a.n_groups;
  const int h = grp * HG + hh;
  const int64_t n_tiles = (a.n_tokens + kTile - 1) / kTile;
  if (first_tile >= n_tiles) return;  // uniform over the block
  const int64_t tile_step = a.blocks_per_group;

  // Tiles are visited as j = 0, 1, 2, ...: tile(j) = first_tile + j * tile_step.
  // Thread (wave w, lane i) computes cos/sin pair i of tokens w + NW k,
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
    for (int k = 0; k < PPT; ++k) st.hi[k] = a.t2[(pos_of(pb, wave_u + NW * k) >> 10) * kPairs + lane];
    // Issued whether or not there are slots (a dummy 8-byte read of T~
    // otherwise), so every iteration issues the same loads in the same order.
    const int64_t tok = tile * kTile + (tid & (kTile - 1));
    st.slot = a.slots ? a.slots[tok < last_tok ? tok : last_tok] : *(const int64_t*)a.T;
  };
  // cos/sin of the next tile into cs_lds[buf]: the fast path for every pair
  // (returns the pairs it cannot certify), the rare rest redone in
  // double-double in a loop that is not unrolled (its loads are issued only
  // when such a pair occurs).
  auto finish_cs_fast = [&](const CsStage<PPT>& st, int pb, int buf) __attribute__((always_inline)) -> uint32_t {
    uint32_t bad = 0;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int n = wave_u + NW * k;
      const int p = pos_of(pb, n);
      const double2 M = tab_lds[1][(p >> 5) & 31][lane], B = tab_lds[0][p & 31][lane];
      bool exact;
      cs_lds[buf][n][lane] = rope_cos_sin_fast(st.hi[k], M, B, exact);
      bad |= (uint32_t)!exact << k;
    }
    return bad;
  };
  auto finish_cs_slow = [&](uint32_t bad, int pb, int buf) __attribute__((always_inline)) {
    if (__builtin_expect(bad != 0, 0)) {
#pragma unroll 1
      for (int k = 0; k < PPT; ++k) {
        if ((bad >> k) & 1) {
          const int n = wave_u + NW * k;
          const int p = pos_lds[pb][n];
          const int p2 = p >> 10, p1 = (p >> 5) & 31, p0 = p & 31;
          cs_lds[buf][n][lane] =
              rope_cos_sin_slow(a.t2[p2 * kPairs + lane], a.t2t[p2 * kPairs + lane], tab_lds[1][p1][lane],
                                a.t1t[p1 * kPairs + lane], tab_lds[0][p0][lane], a.t0t[p0 * kPairs + lane]);
        }
      }
    }
  };
  auto put_slot = [&](const CsStage<PPT>& st, int64_t tile, int sb) __attribute__((always_inline)) {
    if (tid < kTile) slot_lds[sb][tid] = a.slots ? st.slot : tile * kTile + tid;
  };

  RawKeys<F32IN> ra, rb;
  CsStage<PPT> st;
  int64_t tile = first_tile;
  int buf = 0, j = 0;
  // Prologue: every load that depends on nothing is issued up front (the
  // first two tiles' keys, three tiles' positions, T~, the angle tables), so
  // their latencies overlap; only positions -> table entries -> cos/sin is a
  // chain.  Clamped reads past the end keep every address valid.
  load_keys<F32IN>(ra, a, tile * kTile + col, h, lh, wq);
  int pos_d[3];
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    load_pos(tile + d * tile_step);
    pos_d[d] = pos_r;
  }
  // This wave's quarter of T~ as MFMA A operands: rows 32 wq + (lane % 32).
  bf16x8 A[8];
  {
    const bf16x8* Tp = (const bf16x8*)a.T;
#pragma unroll
    for (int s = 0; s < 8; ++s) A[s] = Tp[(((int64_t)h * 4 + wq) * 8 + s) * 64 + lane];
  }

  // Angle tables t0 (p0) and t1 (p1) into LDS for the whole launch.
  for (int e = tid; e < 2 * 32 * kPairs; e += NT) {
    const int t = e / (32 * kPairs), r = e - t * 32 * kPairs;
    tab_lds[t][r / kPairs][r % kPairs] = (t == 0 ? a.t0 : a.t1)[r];
  }

#pragma unroll
  for (int d = 0; d < 3; ++d) {
    pos_r = pos_d[d];
    store_pos(d);
  }
  if (tid < kTile) pos_lds[3][tid] = 0;  // a valid position in the fourth slot
  __syncthreads();  // angle tables and the first three tiles' positions
  issue_cs(st, tile, 0);
  finish_cs_slow(finish_cs_fast(st, 0, 0), 0, 0);
  put_slot(st, tile, 0);
  issue_cs(st, tile + tile_step, 1);  // consumed in the first iteration
  __builtin_amdgcn_s_waitcnt(0x0F70 | (PPT + 1));  // all but those table entries
  __syncthreads();

  // One tile per call (tile j; ss = j % 3).  `cur` holds this tile's keys and
  // `nxt` receives the next tile's.  `st` holds the next tile's table
  // entries; they are consumed after this tile's quantizer, and `st` then
  // receives the entries of the tile after next.  Loads for later tiles are
  // issued unconditionally (clamped addresses past the end), so every
  // iteration issues the same loads in the same order: position, keys, table
  // entries + slot row.  Waiting for all but the table loads before the
  // stores leaves exactly those in flight.  Three barriers per tile.
  // Unrolled by two over the two key sets.
  constexpr int kWaitTail = 0x0F70 | (PPT + 1);
  auto step = [&](RawKeys<F32IN>& cur, RawKeys<F32IN>& nxt, int ss)
      __attribute__((always_inline)) -> bool {
    const int64_t next = tile + tile_step, next2 = next + tile_step, next3 = next2 + tile_step;
    const bool has_next = next < n_tiles;
    load_pos(next3);
    __builtin_amdgcn_sched_barrier(0);
    load_keys<F32IN>(nxt, a, next * kTile + col, h, lh, wq);
    __builtin_amdgcn_sched_barrier(0);

    // ---- RoPE (rotate-half, pairs (i, i+64)) of this wave's pairs -> bf16 operands
    bf16x8 Bop[8];
    {
      const int s = wq;  // k step of channels i; the partners are in k step s + 4
      float ka[8], kb[8];
      unpack8<F32IN>(cur, 0, ka);
      unpack8<F32IN>(cur, 1, kb);
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
    // All eight operands come from LDS (each wave of the head wrote two).
#pragma unroll
    for (int s = 0; s < 8; ++s) Bop[s] = xb_lds[hh][s][lane];

    // ---- y = T~ x~ for this wave's 32 rows (fp32 accumulate)
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], Bop[s], acc, 0, 0, 0);

    // The next tile's cos/sin (computed for a tile past the end too: harmless,
    // into the buffer nobody reads), then the table entries of the tile after.
    auto next_cs = [&]() __attribute__((always_inline)) {
      const uint32_t bad = finish_cs_fast(st, (j + 1) & 3, buf ^ 1);
      finish_cs_slow(bad, (j + 1) & 3, buf ^ 1);
      put_slot(st, next, ss == 2 ? 0 : ss + 1);
      __builtin_amdgcn_sched_barrier(0);
      issue_cs(st, next2, (j + 2) & 3);
      __builtin_amdgcn_sched_barrier(0);
    };
    const int64_t tok = tile * kTile + col;

    if constexpr (YOUT) {
      next_cs();
      if (tok < a.n_tokens) {
        float* yo = a.y_out + (tok * a.n_heads + h) * kD;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 32 * wq + 8 * jj + 4 * lh;
          *(float4*)(yo + r) = make_float4(acc[4 * jj], acc[4 * jj + 1], acc[4 * jj + 2], acc[4 * jj + 3]);
        }
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);
      store_pos((j + 3) & 3);
      __syncthreads();
    } else {
      // Output element acc[i] is row 32*wq + 8*(i/4) + 4*lh + (i%4) of token `col`.
      // run[q] packs the codes of acc[4q .. 4q+3] (4 consecutive rows), LSB first.
      uint32_t run[4];
      uint32_t W2 = 0;  // 2-bit symmetric: the whole word of codes
      if constexpr (QK == 0) {
        // Sum of squares as the contiguous pairwise tree over rows 0..127:
        // runs of 4 in-lane, pairs of runs across lanes l and l^32, the 32
        // rows of this wave, then the four waves' sums ((0 + 1) + (2 + 3)).
        float P8[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float q0 = acc[4 * q] * acc[4 * q];
          const float q1 = acc[4 * q + 1] * acc[4 * q + 1];
          const float q2 = acc[4 * q + 2] * acc[4 * q + 2];
          const float q3 = acc[4 * q + 3] * acc[4 * q + 3];
          const float p4 = (q0 + q1) + (q2 + q3);
          P8[q] = p4 + __shfl_xor(p4, 32);
        }
        const float P32 = (P8[0] + P8[1]) + (P8[2] + P8[3]);
        if (lh == 0) red_lds[hh][wq][col] = P32;
        __syncthreads();
        const float S = (red_lds[hh][0][col] + red_lds[hh][1][col]) + (red_lds[hh][2][col] + red_lds[hh][3][col]);
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
          for (int g = 3; g >= 0; --g) {  // 4 rows per add-with-carry block
            uint64_t mk[8];
#pragma unroll
            for (int e = 3; e >= 0; --e) {
              const float y = acc[4 * g + e];
              const Sym2Masks k = sym2_masks(y, -tp, tz, tp);
              mk[2 * (3 - e)] = k.b1;
              mk[2 * (3 - e) + 1] = k.b0;
            }
            W2 = shift_in8(W2, mk);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t r = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) r |= sym_code<BITS>(acc[4 * q + e], tp, rd) << (BITS * e);
            asm("" : "+v"(r));  // keep the word 32 bits wide (compare + add-with-carry codegen)
            run[q] = r;
          }
        }
        if (wq == 0 && lh == 0) sc_lds[col][hh] = dh;
      } else {
        // Percentile-clipped affine quantizer, group = one 32-row tile = rows
        // split between lanes l and l^32: two smallest and two largest values by
        // IEEE totalOrder, merged across the lane pair.
        {
          int32_t mn1 = INT_MAX, mn2 = INT_MAX, mx1 = INT_MIN, mx2 = INT_MIN;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int32_t k = total_order_key(acc[i]);
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
              const uint32_t c = sd == 0.0 ? 0u : affine_code<BITS>(acc[4 * q + e], zd, sd);
              r |= c << (BITS * e);
            }
            run[q] = r;
          }
          if (lh == 0) {
            sc_lds[col][hh * 8 + wq] = sh;
            sc_lds[col][hh * 8 + 4 + wq] = zh;
          }
        }
      }

      // ---- pack: runs of 4 codes -> 16 contiguous rows per lane -> LDS record row.
      // Lane l (lh = 0) writes rows 0-15 of the m-tile: its runs 0, 1 interleaved
      // with those of lane l + 32; lane l + 32 writes rows 16-31 likewise.
      if constexpr (QK == 0 && BITS == 2) {
        // bytes of {partner (selectors 4-7), own (0-3)}
        const uint32_t sel = lh ? 0x03070206u : 0x05010400u;
        const uint32_t chunk = __builtin_amdgcn_perm(__shfl_xor(W2, 32), W2, sel);
        *(uint32_t*)&rec_lds[col][hh * REC + 2 * (4 * wq + 2 * lh)] = chunk;
      } else {
        const uint32_t* rn = run;
        const uint32_t send = lh ? (rn[0] | (rn[1] << RB)) : (rn[2] | (rn[3] << RB));
        const uint32_t recv = __shfl_xor(send, 32);
        const uint64_t p0 = recv & ((1u << RB) - 1u), p1 = recv >> RB;
        const uint64_t chunk =
            lh ? (p0 | ((uint64_t)rn[2] << RB) | (p1 << (2 * RB)) | ((uint64_t)rn[3] << (3 * RB)))
               : ((uint64_t)rn[0] | (p0 << RB) | ((uint64_t)rn[1] << (2 * RB)) | (p1 << (3 * RB)));
        uint8_t* dst = &rec_lds[col][hh * REC + BITS * (4 * wq + 2 * lh)];
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
      next_cs();
      // The loads for later tiles have been in flight during this tile's work.
      // Wait here for all but the newest keys and table entries (expcnt and
      // lgkmcnt untouched), so the stores below never queue behind them.
      __builtin_amdgcn_s_waitcnt(kWaitTail);
      store_pos((j + 3) & 3);  // its load was issued before the newest keys and table entries
      __syncthreads();

      // ---- stores: each token's HG records are contiguous in the cache row
      const int64_t tbase = tile * kTile;
      constexpr int CPT = HG * BITS;  // 16-byte chunks per token
      for (int c = tid; c < kTile * CPT; c += NT) {
        const int n = c / CPT, k = c - n * CPT;
        const int64_t t = tbase + n;
        if (t < a.n_tokens) {
          const int64_t row = slot_lds[ss][n];
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
          const int64_t row = slot_lds[ss][n];
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
    if (has_next) {
      tile = next;
      buf ^= 1;
      ++j;
    }
    return has_next;
  };
  while (true) {
    if (!step(ra, rb, j % 3)) break;
    if (!step(rb, ra, j % 3)) break;
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
  int64_t b = (int64_t)cus * resident_blocks(k, 256 * HG) / a.n_groups;
  b = b < 1 ? 1 : (b > n_tiles ? n_tiles : b);
  a.blocks_per_group = (int)b;
  k<<<dim3((unsigned)(a.n_groups * b)), 256 * HG, 0, st>>>(a);
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
