// Internal interfaces of libwushkv: handle layouts and kernel launch arguments.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wushkv.h"

// Key-transform handle: T~ = bf16(T) in the order the MFMA A operand is read.
// Chunk (h, mt, s) holds, for lane l, the 8 bf16 values
//   T~[h][32*mt + (l % 32)][16*s + 8*(l / 32) + e], e = 0..7,
// so each wave reads one contiguous 1 KiB chunk per (row tile, k step).
struct wushkv_transform {
  int n_heads;
  int device;
  int hadamard;    // 1: T = H_128 / 8 for every head, and the key path takes the FWHT kernel
  void* d_swz;     // bf16 [H][4][8][64][8]
  float* d_gsum;   // [H][4][128]: sum over j in group g of T~[h][r][j], for affine reads
};

// RoPE handle: cos/sin split tables (see rope_cos_sin and rope2_cos_sin in device_common.h).
struct wushkv_rope {
  float theta;
  int32_t max_pos;
  int device;
  int hi_rows;            // ceil(max_pos / 1024)
  int hi2_rows;           // ceil(max_pos / 32)
  void* d_block;          // one allocation holding the six host-built tables
  const double2* t0;      // [32][64]       (cos, sin)(p0 * w)
  const double2* t1;      // [32][64]       (cos, sin)(p1 * 32 * w)
  const double2* t2;      // [hi_rows][64]  (cos, sin)(p2 * 1024 * w)
  const double2* t0t;     // tails of the three
  const double2* t1t;
  const double2* t2t;
  double2* hi;            // [hi2_rows][64] (cos, sin)(h * 32 * w): head ...
  double2* hit;           // ... and tail, built on the device from t1 and t2
  uint32_t* exc;          // [hi2_rows] bitmap of the positions the fast path rounds differently
};

namespace wushkv {

struct QuantArgs {
  int kind;       // 0 sym; 1 affine, percentiles from the extreme order statistics; 2 affine, general
  float alpha;    // sym clip factor
  // affine, kind 1: the low percentile from order statistics 0, 1, the high one from 30, 31
  //   lo_mode 0: fma(g_lo, s1 - s0, s0); 1: s0
  //   hi_mode 0: fma(g_hi, s31 - s30, s30); 1: s30; 2: s31
  // affine, kind 2: order statistics lo_i, lo_i + 1 and hi_i, hi_i + 1 of the sorted group
  //   mode 0: fma(g, s_{i+1} - s_i, s_i); 1: s_i
  float g_lo;
  int lo_mode;
  float g_hi;
  int hi_mode;
  int lo_i, hi_i;
};

struct KeysArgs {
  const void* K;
  int64_t n_tokens;
  int n_heads;
  int64_t stride;  // elements between tokens
  const int32_t* pos;
  int32_t max_pos;
  const void* T;   // swizzled bf16
  const double2* rope_lo;   // [32][64] (cos, sin)(p0 * w): heads, then tails at rope_lot
  const double2* rope_lot;
  const double2* rope_hi;   // [ceil(max_pos / 32)][64] (cos, sin)(h * 32 * w): heads and tails
  const double2* rope_hit;
  const uint32_t* rope_exc;  // [ceil(max_pos / 32)] positions that take the double-double path
  uint8_t* codes;
  uint16_t* scales;
  uint16_t* zeros;
  const int64_t* slots;
  int64_t n_rows;
  QuantArgs q;
  float* y_out;    // debug: fp32 transformed keys instead of codes
  int n_groups;    // head groups (heads per group = the kernel's HG)
  int blocks_per_group;  // set by the launcher
};

struct ValuesArgs {
  const void* V;
  int64_t n_tokens;
  int n_heads;
  int64_t stride;
  uint32_t div_m;  // v / n_heads == (umulhi(v, div_m) + v) >> div_l for v < 2^31
  uint32_t div_l;
  uint8_t* codes;
  uint16_t* scales;
  uint16_t* zeros;
  const int64_t* slots;
  int64_t n_rows;
  QuantArgs q;
};

// Keys and values of the same tokens in one dispatch (wushkv_quantize_kv).
struct AppendArgs {
  const void* K;
  const void* V;
  int64_t n_tokens;
  int n_heads;
  int64_t k_stride, v_stride;  // elements between tokens
  const int32_t* pos;
  int32_t max_pos;
  const void* T;               // swizzled bf16
  const double2* rope_lo;      // as in KeysArgs
  const double2* rope_lot;
  const double2* rope_hi;
  const double2* rope_hit;
  const uint32_t* rope_exc;
  uint8_t* k_codes;
  uint16_t* k_scales;
  uint16_t* k_zeros;
  const int64_t* k_slots;
  int64_t k_rows;
  uint8_t* v_codes;
  uint16_t* v_scales;
  uint16_t* v_zeros;
  const int64_t* v_slots;
  int64_t v_rows;
  QuantArgs q;
};

struct DequantArgs {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* zeros;
  const int64_t* slots;
  int64_t n_rows;
  int64_t n_tokens;
  int n_heads;
  int kind;
  const void* Tinv;       // swizzled bf16 (NULL: no transform)
  const float* gsum;      // [H][4][128] (affine with Tinv)
  void* out;
  int out_bf16;
  int n_groups;
  int blocks_per_group;  // set by the launcher
};

struct PairArgs {
  const void* Q;          // [n_tokens][n_q_heads][128] with `stride` elements per token
  int f32_in;
  int64_t n_tokens;
  int64_t stride;
  int n_q_heads, n_kv_heads, G;
  const void* Tinv;       // swizzled bf16 of the inverse transform
  uint16_t* out;          // bf16 [n_tokens][n_q_heads][128]
};

struct AttnArgs {
  const uint16_t* qp;     // paired queries, bf16 [n_seqs][n_q_heads][128]
  const uint8_t* kc;
  const uint16_t* ks;
  const uint8_t* vc;
  const uint16_t* vs;
  const uint16_t* kz;     // affine caches: [rows][Hkv][4] zeros beside [rows][Hkv][4] steps; NULL: symmetric
  const uint16_t* vz;
  int64_t n_rows;
  const int64_t* row0;    // first cache row of each sequence
  const int32_t* len;     // tokens of each sequence
  int n_seqs, n_q_heads, n_kv_heads, G;
  int max_len, n_splits;
  int n_splits8;          // ceil(n_splits / 8)
  float c0;               // softmax scale * log2(e)
  float* part;            // workspace: per (sequence, query head, split) max, sum, o[128]
  float* out;             // fp32 [n_seqs][n_q_heads][128]
};

int device_cu_count(int device);

// Events that the next hot-path launch on this host thread records at its
// kernel's start and end (set by wushkv_debug_time_next_launch; consumed by
// that launch).  Timing support only.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents take_launch_events();

// Launch kernel k with its single argument struct, recording the pending
// launch events, if any, around the kernel itself.
template <typename Args>
hipError_t launch_kernel(void (*k)(Args), dim3 grid, dim3 block, hipStream_t st, const Args& a) {
  const LaunchEvents ev = take_launch_events();
  if (ev.start || ev.stop) {
    void* args[] = {const_cast<Args*>(&a)};
    return hipExtLaunchKernel((const void*)k, grid, block, args, 0, st, ev.start, ev.stop, 0);
  }
  k<<<grid, block, 0, st>>>(a);
  return hipGetLastError();
}

// Launchers size their persistent grids from the device's CU count and the
// kernel's occupancy.
hipError_t launch_keys(const KeysArgs& a, int bits, int f32_in, int heads_per_group, int y_out, int cus,
                       hipStream_t stream);
// Keys through T = H_128 / 8 as an in-register fast Walsh-Hadamard transform
// (handles made by wushkv_transform_create_hadamard); a.T is not read.
hipError_t launch_keys_fwht(const KeysArgs& a, int bits, int f32_in, int y_out, int cus, hipStream_t st);
hipError_t launch_values(const ValuesArgs& a, int bits, int f32_in, int cus, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, int bits, int f32_in, int cus, hipStream_t stream);
// Exhaustive device check of the correctly rounded sqrt and div_small: mismatch counts
// for sqrt, / 3, / 7, / 15 into counts[0..3] (device memory).
hipError_t launch_arith_check(uint32_t* counts, int cus, hipStream_t stream);
hipError_t launch_dequant(const DequantArgs& a, int bits, int heads_per_group, int cus, hipStream_t stream);
hipError_t launch_pair_queries(const PairArgs& a, hipStream_t stream);
hipError_t launch_attention(const AttnArgs& a, int bits, hipStream_t stream);
size_t attention_workspace_bytes(int64_t n_seqs, int n_q_heads, int max_len);
// Device address of the library's fixed attention scratch buffer
// (WUSHKV_NOALLOC_SCRATCH_BYTES) on `device`, which must be the current device;
// looked up once per device.
hipError_t attention_scratch(int device, void** ptr);
int attention_splits(int max_len);
// Fills r->hi and r->hit (the (cos, sin) of h * 32 * w_i for h < r->hi2_rows as
// double-double (head, tail) angle sums of the t2 and t1 entries), then the bitmap
// r->exc of the positions whose fp64 fast sum rounds differently from the
// double-double one for some pair.
hipError_t launch_build_rope_hi(const wushkv_rope* r, hipStream_t stream);
// cs_out[n][64][2] = the (cos, sin) the key kernel computes for clamp(pos[n]).
hipError_t launch_gather_cs(const wushkv_rope* r, const int32_t* pos, int64_t n, float* cs_out,
                            hipStream_t stream);

}  // namespace wushkv
