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
// cos/sin are computed in the kernel, exactly (fp32 roundings of cos and sin
// of the exact angle): pos = 32 h + p0, the (cos, sin) of p0 * w_i come from a
// 32-row fp64 table the block keeps in LDS, those of 32 h * w_i from an fp64
// table row in global memory (L2-resident: one row serves 32 positions), and
// one fp64 angle addition rounded to fp32 gives the pair, except at the rare
// positions the RoPE handle has marked, which take a double-double sum.  The
// block computes a tile's 64 x 64 pairs once for all its heads into one LDS
// tile buffer.
//
// Per-tile pipeline, three barriers: [stores of the previous tile; cache rows
// and the positions of the tile after next; the high table entries for the
// next tile; RoPE -> LDS; the next tile's keys into the registers RoPE freed]
// B1 [(cos, sin) of the next tile; MFMA; sums of squares -> LDS] B2
// [scale(s), codes, records -> LDS; wait for the loads older than the keys]
// B3.  The next tile's (cos, sin) reach the tile buffer in the interval after
// both groups have read the current tile's (see the schedule at the end).
// Packed records and scales are staged in LDS and written as whole 16-byte
// chunks (a head group's records of a token are contiguous in the cache row).
#include "device_common.h"
#include "internal.h"
#include "key_codes.h"

namespace wushkv {

namespace {

constexpr int kTile = 64;      // tokens per tile
constexpr int kNB = 2;         // 32-token MFMA column blocks per tile
constexpr int kCsStride = 66;  // float2 per token row of the cos/sin tile (64 + 2 pad)
constexpr int kRopeLo = 32;    // positions covered by the LDS (cos, sin) table
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
  constexpr int RPG = kTile / NG;   // cos/sin rows each group computes per tile
  constexpr int TPW = RPG / WG;     // ... each of its waves
  constexpr int NCS = TPW / 2;      // ... in slots of two rows (lane halves) x two pairs
  // slots whose high entries are loaded before RoPE (the 4-bit affine kernel keeps one: its
  // registers are the scarcest)
  constexpr int NPRE = NCS < 2 ? NCS : ((QK && BITS == 4) ? 1 : 2);
  constexpr int NKL = F32IN ? 8 : 4;  // key loads per lane per tile
  constexpr int L = 1 << BITS;
  constexpr int REC = 16 * BITS;
  constexpr int RECROW = HGG * REC + 16;  // LDS row of one token's records in a group (+16 B pad)
  constexpr int NSC = QK ? 8 : 1;         // fp16 values per (token, head): sym 1; affine 4 + 4
  constexpr int ESZ = F32IN ? 4 : 2;

  // (cos, sin) of a tile: token row t, 16-byte chunk q (pairs 2q, 2q + 1) at chunk
  // q ^ ((q >> 3) & 2), so that the eight chunk-loads of a row that one RoPE
  // read instruction issues (chunks 4c + e, c < 8) fall in eight bank groups.
  __shared__ __align__(16) float2 cs_lds[kTile][kCsStride];
  // (cos, sin)(p0 * w_i) in fp64, pair j of row p0 at (j & 1) * 32 + j / 2: a lane's two
  // pairs 2c, 2c + 1 sit at c and 32 + c, contiguous across the lanes.
  __shared__ __align__(16) double2 lo_lds[kRopeLo][kPairs];
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
  // (cos, sin) slots: wave w of group g computes rows RPG*g + TPW*w .. + TPW - 1 of a
  // tile; slot i is row RPG*g + TPW*w + 2i + (l / 32) and pairs 2 (l % 32), 2 (l % 32) + 1
  // (one float4 of the row).  posv[i] is the position of slot i's row (0 past the end).
  auto load_pos = [&](int t, int* pv) __attribute__((always_inline)) {
    const rsrc_t rs = buffer_rsrc(a.pos + t * kTile, tile_len(t) * 4u);
#pragma unroll
    for (int i = 0; i < NCS; ++i)
      pv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (RPG * g + TPW * gw + 2 * i + lh), 0, 0);
  };
  auto clamp_pos = [&](int p) __attribute__((always_inline)) -> int { return min(max(p, 0), a.max_pos - 1); };
  // A slot's high-table heads (32 contiguous bytes of row p / 32) and the word
  // of the handle's bitmap that marks the positions of that row which take the
  // double-double path.
  struct HiSlot {
    double2 h[2];
    uint32_t exc;
  };
  auto hi_load = [&](int p, HiSlot& hv) __attribute__((always_inline)) {
    const uint32_t row = (uint32_t)p >> 5;
    const double2* src = a.rope_hi + row * (uint32_t)kPairs + 2 * col;
    hv.h[0] = src[0];
    hv.h[1] = src[1];
    hv.exc = a.rope_exc[row];
  };
  // (cos, sin) of a slot: the high heads plus the angle of p % 32 from LDS
  auto cs_slot = [&](int p, const HiSlot& hv) __attribute__((always_inline)) -> float4 {
    return rope2_pair_cs(p, col, hv.h[0], hv.h[1], hv.exc, lo_lds[p & 31][col], lo_lds[p & 31][32 + col],
                         a.rope_hit, a.rope_lot);
  };
  auto cs_store = [&](int i, float4 v) __attribute__((always_inline)) {
    *(float4*)&cs_lds[RPG * g + TPW * gw + 2 * i + lh][2 * (col ^ ((col >> 3) & 2))] = v;
  };
  // Cache rows of tile t's tokens, loaded by the first wave of the last group
  // (lane = token): the raw slot words, turned into a row or -1 by row_of once
  // they have arrived.
  const bool row_wave = wave_u == (NG - 1) * WG;
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
  // Prologue: the positions of the first two tiles (first: the one dependent chain,
  // position -> high-table entries, starts from them, and the second tile's are in by
  // the time the loop starts); the (cos, sin) table of p0 < 32 into LDS; the first
  // tile's keys and rows; T~; the first tile's (cos, sin).
  int posv[NCS], posv_n[NCS];  // positions of the next tile's slot rows, then of the one after
  load_pos(first_tile, posv);
  load_pos(tile_of(1), posv_n);
  constexpr int NLO = kRopeLo * kPairs / (256 * HG);  // lo-table entries per thread
  double2 lov[NLO];
#pragma unroll
  for (int k = 0; k < NLO; ++k) lov[k] = a.rope_lo[threadIdx.x + 256 * HG * k];
  // (the second group's first keys are loaded once the prologue is done: that
  // group starts one phase later, and the first group's keys arrive sooner
  // without them in the queue)
  if (NG == 1 || g == 0) load_keys<F32IN>(r, keys_rsrc(first_tile), keys_off(), 8 * row_bytes);
  u32x2 row_w = {0u, 0u};  // read only when a.slots is set
  HiSlot hv[NPRE];             // high-table entries of the next tile's first NPRE slots
  float4 csr[NCS];             // the next tile's (cos, sin) slots, held by group 0 until phase 2
  if (a.slots && row_wave) row_w = load_rows(first_tile);
  // This wave's quarter of T~ as MFMA A operands: rows 32 wq + (lane % 32).
  bf16x8 A[8];
  {
    const bf16x8* Tp = (const bf16x8*)a.T;
#pragma unroll
    for (int s = 0; s < 8; ++s) A[s] = Tp[(((int64_t)h * 4 + wq) * 8 + s) * 64 + lane];
  }
  {
    HiSlot h0[NCS];
#pragma unroll
    for (int i = 0; i < NCS; ++i) hi_load(clamp_pos(posv[i]), h0[i]);
#pragma unroll
    for (int k = 0; k < NLO; ++k) {
      const int e = threadIdx.x + 256 * HG * k, j = e & 63;  // entry (e / 64, j) of the table
      lo_lds[e >> 6][(j & 1) * 32 + (j >> 1)] = lov[k];
    }
    __syncthreads();  // lo_lds
#pragma unroll
    for (int i = 0; i < NCS; ++i) cs_store(i, cs_slot(clamp_pos(posv[i]), h0[i]));
  }
#pragma unroll
  for (int i = 0; i < NCS; ++i) posv[i] = posv_n[i];
  // Nothing may be in flight when the loop starts: its first wait would
  // otherwise also cover the previous tile's stores on later iterations.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if (row_wave) slot_lds[0][lane] = row_of(row_w, first_tile);
  __syncthreads();

  f32x16 acc[kNB];
  int tid = threadIdx.x;

  // ---- phase 0 of the group's j-th tile: the stores of tile j - 1, then (for
  // j < count) the loads for later tiles, RoPE and the next tile's keys.
  auto phase0 = [&](int j) __attribute__((always_inline)) {
    // Only this tile's keys can still be in flight (the phase-2 wait leaves
    // them); wait here, before the stores and loads below are issued, so that
    // RoPE does not also wait for those.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if constexpr (!YOUT) {
      // The later group (the only one with one group) stores both groups'
      // records and steps of tile j - 1: a token's records of the block's
      // heads are one contiguous run of the cache row (a whole 128-byte line
      // for four 2-bit heads), written at once rather than in two halves one
      // phase apart.  The earlier group's rows stay in LDS until its next
      // phase 2, which comes after this phase.
      if (j >= 1 && g == NG - 1) {
        const int sb = (j - 1) & 1;
        constexpr int CPG = HGG * BITS;      // 16-byte chunks per token and group
        constexpr int CPB = NG * CPG;        // ... and block
        constexpr int NCH = kTile * CPB;
        const uint32_t tg = (uint32_t)(tid - 64 * WG * g);  // thread within the group
        const uint32_t row_rec = (uint32_t)a.n_heads * REC;  // bytes per cache row
#pragma unroll
        for (uint32_t c = tg; c < (uint32_t)NCH; c += 64 * WG) {
          const uint32_t n = c / CPB, k = c - n * CPB, gg = k / CPG, kk = k - gg * CPG;
          const int32_t row = slot_lds[sb][n];
          if (row >= 0) {
            // (24-bit multiply: a full 32-bit one issues at a quarter of the rate)
            const u32x4 v = *(const u32x4*)((const uint8_t*)rec_lds[gg] + __umul24(n, RECROW) + 16 * kk);
            uint8_t* dst = a.codes + (uint64_t)(uint32_t)row * row_rec + (grp * HG * REC + 16 * k);
            __builtin_nontemporal_store(v, (u32x4*)dst);  // written once, not read back here
          }
        }
        // the block's HG heads' steps (and zeros) of a token, by the group's last wave
        const int n = (int)tg - (64 * WG - 64);
        if (n >= 0) {
          const int32_t row = slot_lds[sb][n];
          if (row >= 0) {
            const uint64_t slot = (uint64_t)(uint32_t)row * a.n_heads + grp * HG;
            if constexpr (QK == 0) {
              uint16_t sv[HG];
#pragma unroll
              for (int gg = 0; gg < NG; ++gg)
#pragma unroll
                for (int hg2 = 0; hg2 < HGG; ++hg2) sv[gg * HGG + hg2] = sc_lds[gg][n][hg2];
              if constexpr (HG == 4) {
                *(uint2*)(a.scales + slot) = make_uint2(sv[0] | ((uint32_t)sv[1] << 16), sv[2] | ((uint32_t)sv[3] << 16));
              } else if constexpr (HG == 2) {
                *(uint32_t*)(a.scales + slot) = sv[0] | ((uint32_t)sv[1] << 16);
              } else {
                a.scales[slot] = sv[0];
              }
            } else {
              // per head: 4 scales and 4 zeros, 8 bytes each
#pragma unroll
              for (int gg = 0; gg < NG; ++gg)
#pragma unroll
                for (int hg2 = 0; hg2 < HGG; ++hg2) {
                  const uint64_t sl = slot + gg * HGG + hg2;
                  *(uint2*)(a.scales + sl * 4) = *(const uint2*)&sc_lds[gg][n][hg2 * 8];
                  *(uint2*)(a.zeros + sl * 4) = *(const uint2*)&sc_lds[gg][n][hg2 * 8 + 4];
                }
            }
          }
        }
      }
    }
    if (j >= count) return;
    const int next = tile_of(j + 1);
    // the next tile's cache rows and the positions of the tile after (zeros
    // past the end); the high-table entries of the next tile's first slots,
    // issued before the next tile's keys so that waiting for them in phase 1
    // leaves the keys in flight
    if (a.slots && row_wave) row_w = load_rows(next);
    load_pos(tile_of(j + 2), posv_n);
#pragma unroll
    for (int i = 0; i < NPRE; ++i) hi_load(clamp_pos(posv[i]), hv[i]);
    // RoPE (rotate-half, pairs (i, i+64)) -> bf16 operands in LDS.
    // Chunk c = l % 8 of token t is channels 8c .. 8c+7 (k step c / 2, lane
    // half c % 2 of the B operand) and its partner chunk (k step 4 + c / 2).
    // B-operand rows are stored with lane index lane' ^ (4 (s % 4) + 2 (lane' / 32)),
    // which for this chunk is lane' ^ 2c: the eight chunks of a token land in
    // eight different bank groups, and each row stays a permutation of itself.
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int c8 = lane & 7, gt = lane >> 3;
      const int t = 16 * wq + 8 * jj + gt;  // token within the tile
      float ka[8], kb[8];
      unpack8<F32IN>(r, jj, 0, ka);
      unpack8<F32IN>(r, jj, 1, kb);
      const float4* csp = (const float4*)&cs_lds[t][8 * c8];
      const int sw = (c8 >> 1) & 2;  // the row's chunk swizzle for chunks 4 c8 .. 4 c8 + 3
      float c[8], sn[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 v = csp[e ^ sw];
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
    // (cos, sin) of the next tile's slots.  Their high entries were loaded in
    // phase 0 before the next tile's keys, so this wait leaves the keys in
    // flight (slots beyond NPRE, with fewer than four waves per group, load
    // theirs here).  Group 1 (and a single group) writes them to the tile
    // buffer now, since every wave has read the current tile's in its phase 0;
    // group 0 at the start of its phase 2, when group 1 has passed its phase 0.
    __builtin_amdgcn_s_waitcnt(0x0F70 | NKL);  // vmcnt(NKL)
#pragma unroll
    for (int i = 0; i < NCS; ++i) {
      const int p = clamp_pos(posv[i]);
      float4 v;
      if (i < NPRE) {
        v = cs_slot(p, hv[i < NPRE ? i : 0]);
      } else {
        HiSlot h2;
        hi_load(p, h2);
        v = cs_slot(p, h2);
      }
      if (NG == 1 || g == 1) {
        cs_store(i, v);
      } else {
        csr[i] = v;
      }
    }
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
      // rows of this wave (lane l: token l of the tile), then the four
      // waves' sums ((0 + 1) + (2 + 3)).
      red_lds[hh][wq][lane] = col_sumsq32x2(acc[0], acc[1]);
    }
    if constexpr (YOUT) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the y stores
    } else if (row_wave) {
      // the next tile's cache rows: group 1's phase 1 (or a single group's)
      // runs after every store that read this slot buffer's previous tile
      slot_lds[(j + 1) & 1][lane] = row_of(row_w, tile_of(j + 1));
    }
  };

  // ---- phase 2: scales, codes and records of tile j -> LDS; then every load
  // has landed and (group 0) the next tile's cos/sin rows and cache rows go to LDS.
  auto phase2 = [&](int j) __attribute__((always_inline)) {
    if (NG == 2 && g == 0) {
#pragma unroll
      for (int i = 0; i < NCS; ++i) cs_store(i, csr[i]);
    }
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
        const uint16_t dh = sym_step_f16<L>(S, a.q.alpha);
        if (wq == 0) sc_lds[g][tt][hg] = dh;
        const Halves dd = halves(f16_bits_to_f32(dh));
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          const float delta = __uint_as_float(nb ? dd.hi : dd.lo);
          if constexpr (BITS == 2) {
            W2[nb] = sym2_word(acc[nb], delta);
          } else {
            sym_runs<BITS>(acc[nb], delta, run[nb]);
          }
        }
      } else {
        // Percentile-clipped affine quantizer, group = this wave's 32 rows of
        // a token (see affine_runs).
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
          uint16_t sh, zh;
          affine_runs<BITS, QK == 2>(acc[nb], a.q, run[nb], sh, zh);
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
          put_chunk<2>(dst, record_chunk2(W2[nb], lh));
        } else {
          put_chunk<BITS>(dst, record_chunk<BITS>(run[nb], lh));
        }
      }
    }
    // The positions have landed; the next tile's keys (the youngest loads)
    // stay in flight until RoPE needs them.
    if constexpr (!YOUT) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | NKL);  // vmcnt(NKL), expcnt and lgkmcnt untouched
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
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
  // between the groups.  The intervals between barriers run (group 0, group 1)
  // = (P0 j, P2 j-1), (P1 j, P0 j), (P2 j, P1 j), (P0 j+1, P2 j), ...: the
  // (cos, sin) of tile j + 1 are written in the (P2 j, P1 j) interval, after
  // both groups' phase 0 of tile j has read tile j's and before group 0's
  // phase 0 of tile j + 1 reads them (one group: written in its phase 1 of
  // tile j).  The cache rows of tile j + 1 go to slot_lds[(j + 1) % 2] in the
  // same interval (group 1's phase 1 of tile j), after both groups' stores of
  // tile j - 1 have read that buffer, and stay there until group 1's stores of
  // tile j + 1.
  auto next_phase = [&]() __attribute__((always_inline)) {
    __syncthreads();
    asm volatile("" : "+v"(lane));
    lh = lane >> 5;
    col = lane & 31;
    tid = 64 * wave_u + lane;
  };
  if (NG == 2 && g == 1) {
    load_keys<F32IN>(r, keys_rsrc(first_tile), keys_off(), 8 * row_bytes);
    next_phase();
  }
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

// (cos, sin)(h * 32 * w_i) for h < n / 64 as double-double (head, tail): the
// angle sum of t2[h / 32] and t1[h % 32].  Entry h * 64 + i.
__global__ void build_rope_hi_kernel(RopeTables t, int64_t n, double2* hi, double2* hit) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int h = (int)(idx / kPairs), i = (int)(idx % kPairs);
  const int a2 = (h >> 5) * kPairs + i, a1 = (h & 31) * kPairs + i;
  const double2 A = t.t2[a2], At = t.t2t[a2], M = t.t1[a1], Mt = t.t1t[a1];
  double ch, cl, sh, sl;
  dd_pair(A.x, At.x, M.x, Mt.x, A.y, At.y, M.y, Mt.y, -1.0, ch, cl);  // cos(a + m)
  dd_pair(A.y, At.y, M.x, Mt.x, A.x, At.x, M.y, Mt.y, 1.0, sh, sl);   // sin(a + m)
  hi[idx] = make_double2(ch, sh);
  hit[idx] = make_double2(cl, sl);
}

// Bit pos % 32 of exc[pos / 32]: does the fp64 fast sum of any pair of position
// pos round differently from the double-double sum?  One thread per position,
// 64-thread blocks (one wave: two bitmap words).
__global__ void __launch_bounds__(64) build_rope_exc_kernel(Rope2Tables t, int32_t max_pos, uint32_t* exc) {
  const int pos = blockIdx.x * 64 + threadIdx.x;
  bool marked = false;
  if (pos < max_pos) {
    const int p0 = pos & 31, h = pos >> 5;
    for (int i = 0; i < kPairs; ++i) {
      const double2 H = t.hi[h * kPairs + i], B = t.lo[p0 * kPairs + i];
      const float2 f = rope2_fast(H, B);
      const float2 x = rope2_slow(H, t.hit[h * kPairs + i], B, t.lot[p0 * kPairs + i]);
      marked |= __float_as_uint(f.x) != __float_as_uint(x.x) || __float_as_uint(f.y) != __float_as_uint(x.y);
    }
  }
  const uint64_t m = __builtin_amdgcn_ballot_w64(marked);
  if (pos < max_pos && (threadIdx.x & 31) == 0) exc[pos >> 5] = (uint32_t)(m >> (threadIdx.x & 32));
}

__global__ void gather_cs_kernel(Rope2Tables t, int32_t max_pos, const int32_t* pos, int64_t n, float2* out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * kPairs) return;
  const int64_t k = idx / kPairs;
  int p = pos[k];
  p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
  out[idx] = rope2_cos_sin(p, (int)(idx - k * kPairs), t);
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
      // (general percentiles sort in registers: at most two heads per block)
      if constexpr (!F32IN && QK != 2) return launch_one<BITS, QK, F32IN, 4, YOUT>(a, cus, st);
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
  } else if (a.q.kind == 1) {
    switch (bits) {
      case 2: return launch_bits<2, 1>(a, f32_in, hg, 0, cus, st);
      case 3: return launch_bits<3, 1>(a, f32_in, hg, 0, cus, st);
      case 4: return launch_bits<4, 1>(a, f32_in, hg, 0, cus, st);
    }
  } else {
    switch (bits) {
      case 2: return launch_bits<2, 2>(a, f32_in, hg, 0, cus, st);
      case 3: return launch_bits<3, 2>(a, f32_in, hg, 0, cus, st);
      case 4: return launch_bits<4, 2>(a, f32_in, hg, 0, cus, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_build_rope_hi(const wushkv_rope* r, hipStream_t st) {
  const int64_t total = (int64_t)r->hi2_rows * kPairs;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  const RopeTables t{r->t0, r->t1, r->t2, r->t0t, r->t1t, r->t2t};
  build_rope_hi_kernel<<<dim3((unsigned)blocks), threads, 0, st>>>(t, total, r->hi, r->hit);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const Rope2Tables t2{r->t0, r->hi, r->t0t, r->hit, r->exc};
  build_rope_exc_kernel<<<dim3((unsigned)((r->max_pos + 63) / 64)), 64, 0, st>>>(t2, r->max_pos, r->exc);
  return hipGetLastError();
}

hipError_t launch_gather_cs(const wushkv_rope* r, const int32_t* pos, int64_t n, float* cs_out,
                            hipStream_t st) {
  const int64_t total = n * kPairs;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  const Rope2Tables t{r->t0, r->hi, r->t0t, r->hit, r->exc};
  gather_cs_kernel<<<dim3((unsigned)blocks), threads, 0, st>>>(t, r->max_pos, pos, n, (float2*)cs_out);
  return hipGetLastError();
}

}  // namespace wushkv
