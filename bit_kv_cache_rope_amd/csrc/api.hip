// libwushkv C ABI: argument validation, handles and launch dispatch.
//
// Every entry point validates on the host before anything is launched and
// reports failures as status codes with a thread-local detail string.  Handle
// creation allocates device memory; the quantize / dequantize calls do not.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_err;
thread_local wushkv::LaunchEvents g_launch_events;  // see wushkv_debug_time_next_launch

wushkv_status fail(wushkv_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

wushkv_status hip_fail(hipError_t e, const char* what) {
  return fail(WUSHKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// bf16 bit pattern of an fp32 value, round-to-nearest-even (finite inputs).
uint16_t host_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
float host_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

wushkv_status current_device(int* dev) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return fail(WUSHKV_ERR_NO_DEVICE, "no HIP device visible");
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  return WUSHKV_OK;
}

// Quantizer description -> kernel arguments.  The percentile interpolation
// follows h = 31 p / 100, i = floor(h), g = RN32(h - i); the kernels provide
// order statistics 0, 1 (low end) and 30, 31 (high end).
wushkv_status make_quant(const wushkv_quantizer* q, wushkv::QuantArgs* out) {
  if (!q) return fail(WUSHKV_ERR_INVALID_ARG, "quantizer is NULL");
  std::memset(out, 0, sizeof(*out));
  if (q->kind == WUSHKV_Q_SYM_RMS) {
    if (q->group != WUSHKV_HEAD_DIM) return fail(WUSHKV_ERR_UNSUPPORTED, "symmetric quantizer needs group 128");
    if (!(q->clip_alpha > 0.0f) || !std::isfinite(q->clip_alpha))
      return fail(WUSHKV_ERR_INVALID_ARG, "clip_alpha must be finite and > 0");
    out->kind = 0;
    out->alpha = q->clip_alpha;
    return WUSHKV_OK;
  }
  if (q->kind == WUSHKV_Q_AFFINE_PCT) {
    if (q->group != 32) return fail(WUSHKV_ERR_UNSUPPORTED, "affine quantizer needs group 32");
    if (!(q->p_lo >= 0.0f) || !(q->p_hi <= 100.0f) || !(q->p_lo <= q->p_hi))
      return fail(WUSHKV_ERR_INVALID_ARG, "need 0 <= p_lo <= p_hi <= 100");
    // order statistic i and weight g of each percentile (h >= 31: the largest, exactly)
    auto split = [](float p, int* i, float* g, int* exact) {
      const double h = 31.0 * (double)p / 100.0;
      if (h >= 31.0) {
        *i = 31;
        *g = 0.0f;
        *exact = 1;
        return;
      }
      const double fl = std::floor(h);
      *i = (int)fl;
      *g = (float)(h - fl);
      *exact = *g == 0.0f ? 1 : 0;
    };
    int il, ih, el, eh;
    float gl, gh;
    split(q->p_lo, &il, &gl, &el);
    split(q->p_hi, &ih, &gh, &eh);
    if (il == 0 && (ih == 30 || ih == 31)) {
      // the extreme order statistics (the 1st/99th percentiles among them): kind 1
      out->kind = 1;
      out->g_lo = gl;
      out->lo_mode = el;
      out->g_hi = gh;
      out->hi_mode = ih == 31 ? 2 : eh;
    } else {
      out->kind = 2;
      out->g_lo = gl;
      out->lo_mode = el;
      out->g_hi = gh;
      out->hi_mode = eh;
    }
    out->lo_i = il;
    out->hi_i = ih;
    return WUSHKV_OK;
  }
  return fail(WUSHKV_ERR_INVALID_ARG, "unknown quantizer kind");
}

wushkv_status check_packed(const wushkv_packed* p, int kind, int64_t n_tokens, bool writer) {
  if (!p) return fail(WUSHKV_ERR_INVALID_ARG, "packed cache view is NULL");
  if (p->n_rows < 0) return fail(WUSHKV_ERR_INVALID_ARG, "n_rows < 0");
  if (p->n_rows > 0) {  // a cache of no rows is never dereferenced: its pointers may be NULL
    if (!p->codes || !p->scales) return fail(WUSHKV_ERR_INVALID_ARG, "codes and scales must be set");
    if (kind != 0 && !p->zeros) return fail(WUSHKV_ERR_INVALID_ARG, "affine quantizer needs zeros");
  }
  if (!aligned(p->codes, 16)) return fail(WUSHKV_ERR_ALIGNMENT, "codes must be 16-byte aligned");
  if (!aligned(p->scales, 16)) return fail(WUSHKV_ERR_ALIGNMENT, "scales must be 16-byte aligned");
  if (kind != 0 && !aligned(p->zeros, 16)) return fail(WUSHKV_ERR_ALIGNMENT, "zeros must be 16-byte aligned");
  if (p->n_rows > INT32_MAX) return fail(WUSHKV_ERR_UNSUPPORTED, "n_rows must be below 2^31");
  if (!p->slots && p->n_rows < n_tokens)
    return fail(WUSHKV_ERR_INVALID_ARG, writer ? "cache has fewer rows than tokens" : "cache has fewer rows than requested");
  return WUSHKV_OK;
}

wushkv_status check_tensor(const void* X, wushkv_dtype dt, int64_t n_tokens, int n_heads, int64_t stride) {
  if (dt != WUSHKV_F32 && dt != WUSHKV_BF16) return fail(WUSHKV_ERR_INVALID_ARG, "dtype must be F32 or BF16");
  if (n_heads < 1 || n_heads > 4096) return fail(WUSHKV_ERR_INVALID_ARG, "n_heads out of range");
  if (n_tokens < 0) return fail(WUSHKV_ERR_INVALID_ARG, "n_tokens < 0");
  if (n_tokens > INT32_MAX - 128) return fail(WUSHKV_ERR_UNSUPPORTED, "n_tokens must be below 2^31 - 128");
  if (stride < (int64_t)n_heads * WUSHKV_HEAD_DIM) return fail(WUSHKV_ERR_INVALID_ARG, "token_stride < n_heads*128");
  const int64_t esz = dt == WUSHKV_F32 ? 4 : 2;
  if ((stride * esz) % 16) return fail(WUSHKV_ERR_ALIGNMENT, "token_stride must span a multiple of 16 bytes");
  if (stride * esz > (1 << 24)) return fail(WUSHKV_ERR_UNSUPPORTED, "token_stride spans more than 2^24 bytes");
  if (n_tokens > 0) {
    if (!X) return fail(WUSHKV_ERR_INVALID_ARG, "input tensor is NULL");
    if (!aligned(X, 16)) return fail(WUSHKV_ERR_ALIGNMENT, "input tensor must be 16-byte aligned");
  }
  return WUSHKV_OK;
}

// Round-up multiplier for division by d (Granlund and Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, v / d == (umulhi(v, m) + v) >> l for v < 2^31.
void div_magic(uint32_t d, uint32_t* m, uint32_t* l) {
  uint32_t k = 0;
  while ((1ull << k) < d) ++k;
  *l = k;
  *m = (uint32_t)(((1ull << 32) * ((1ull << k) - d)) / d + 1);
}

int choose_hg(int64_t n_tiles, int n_heads, int cus, int max_hg) {
  int hg = (n_tiles * n_heads >= 2LL * cus) ? 4 : 1;
  if (hg > max_hg) hg = max_hg;
  while (hg > 1 && n_heads % hg) hg /= 2;
  return hg;
}

constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices];
std::mutex g_cus_mu;

}  // namespace

namespace wushkv {

LaunchEvents take_launch_events() {
  const LaunchEvents e = g_launch_events;
  g_launch_events = LaunchEvents{};
  return e;
}

int device_cu_count(int device) {
  if (device < 0 || device >= kMaxDevices) return 256;
  std::lock_guard<std::mutex> lk(g_cus_mu);
  if (!g_cus[device]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0) n = 256;
    g_cus[device] = n;
  }
  return g_cus[device];
}

}  // namespace wushkv

extern "C" {

int wushkv_version(void) { return 1; }

const char* wushkv_last_error(void) { return g_err.c_str(); }

const char* wushkv_status_string(wushkv_status s) {
  switch (s) {
    case WUSHKV_OK: return "ok";
    case WUSHKV_ERR_INVALID_ARG: return "invalid argument";
    case WUSHKV_ERR_UNSUPPORTED: return "unsupported";
    case WUSHKV_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case WUSHKV_ERR_NO_DEVICE: return "no HIP device";
    case WUSHKV_ERR_HIP: return "HIP runtime error";
    case WUSHKV_ERR_OOM: return "out of device memory";
  }
  return "unknown status";
}

wushkv_status wushkv_rope_frequencies(float theta, float* omega_out) {
  if (!omega_out) return fail(WUSHKV_ERR_INVALID_ARG, "omega_out is NULL");
  if (!(theta > 1.0f) || !std::isfinite(theta)) return fail(WUSHKV_ERR_INVALID_ARG, "theta must be finite and > 1");
  for (int i = 0; i < 64; ++i) omega_out[i] = (float)std::pow((double)theta, -(double)(2 * i) / 128.0);
  return WUSHKV_OK;
}

static wushkv_status transform_create(const float* T, int n_heads, int hadamard, wushkv_transform** out) {
  int dev;
  wushkv_status st = current_device(&dev);
  if (st) return st;
  const size_t H = (size_t)n_heads, D = WUSHKV_HEAD_DIM;
  for (size_t i = 0; i < H * D * D; ++i)
    if (!std::isfinite(T[i])) return fail(WUSHKV_ERR_INVALID_ARG, "T has a non-finite entry");
  // A-operand order: chunk (h, mt, s), lane l, element e <- T~[h][32 mt + l%32][16 s + 8 (l/32) + e]
  std::vector<uint16_t> swz(H * D * D);
  for (size_t h = 0; h < H; ++h)
    for (int mt = 0; mt < 4; ++mt)
      for (int s = 0; s < 8; ++s)
        for (int l = 0; l < 64; ++l)
          for (int e = 0; e < 8; ++e) {
            const size_t r = 32 * mt + (l % 32), c = 16 * s + 8 * (l / 32) + e;
            swz[((((h * 4 + mt) * 8 + s) * 64 + l) * 8) + e] = host_bf16(T[(h * D + r) * D + c]);
          }
  std::vector<float> gsum(H * 4 * D);
  for (size_t h = 0; h < H; ++h)
    for (int g = 0; g < 4; ++g)
      for (size_t r = 0; r < D; ++r) {
        double acc = 0.0;
        for (int j = 32 * g; j < 32 * g + 32; ++j) acc += (double)host_bf16_value(host_bf16(T[(h * D + r) * D + j]));
        gsum[(h * 4 + g) * D + r] = (float)acc;
      }
  auto* t = new (std::nothrow) wushkv_transform();
  if (!t) return fail(WUSHKV_ERR_OOM, "host allocation failed");
  t->n_heads = n_heads;
  t->device = dev;
  t->hadamard = hadamard;
  hipError_t e = hipMalloc(&t->d_swz, swz.size() * 2);
  if (e != hipSuccess) { delete t; return fail(WUSHKV_ERR_OOM, "hipMalloc for the transform failed"); }
  e = hipMalloc((void**)&t->d_gsum, gsum.size() * 4);
  if (e != hipSuccess) { (void)hipFree(t->d_swz); delete t; return fail(WUSHKV_ERR_OOM, "hipMalloc for the transform failed"); }
  e = hipMemcpy(t->d_swz, swz.data(), swz.size() * 2, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(t->d_gsum, gsum.data(), gsum.size() * 4, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(t->d_swz); (void)hipFree(t->d_gsum); delete t;
    return hip_fail(e, "hipMemcpy (transform)");
  }
  *out = t;
  return WUSHKV_OK;
}

wushkv_status wushkv_transform_create(const float* T, int n_heads, wushkv_transform** out) {
  if (!out) return fail(WUSHKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!T) return fail(WUSHKV_ERR_INVALID_ARG, "T is NULL");
  if (n_heads < 1 || n_heads > 4096) return fail(WUSHKV_ERR_INVALID_ARG, "n_heads out of range");
  return transform_create(T, n_heads, 0, out);
}

wushkv_status wushkv_transform_create_hadamard(int n_heads, wushkv_transform** out) {
  if (!out) return fail(WUSHKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (n_heads < 1 || n_heads > 4096) return fail(WUSHKV_ERR_INVALID_ARG, "n_heads out of range");
  // the dense matrix as well (H[r][c] = (-1)^popcount(r & c) / 8), for the calls
  // that read it: the fused append kernel and the debug transform of dense handles
  const size_t D = WUSHKV_HEAD_DIM;
  std::vector<float> T((size_t)n_heads * D * D);
  for (size_t h = 0; h < (size_t)n_heads; ++h)
    for (size_t r = 0; r < D; ++r)
      for (size_t c = 0; c < D; ++c) T[(h * D + r) * D + c] = (__builtin_popcountll(r & c) & 1) ? -0.125f : 0.125f;
  return transform_create(T.data(), n_heads, 1, out);
}

wushkv_status wushkv_transform_destroy(wushkv_transform* t) {
  if (!t) return WUSHKV_OK;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(t->device);
  (void)hipFree(t->d_swz);
  (void)hipFree(t->d_gsum);
  if (prev >= 0) (void)hipSetDevice(prev);
  delete t;
  return WUSHKV_OK;
}

wushkv_status wushkv_rope_create(float theta, int32_t max_pos, wushkv_rope** out) {
  if (!out) return fail(WUSHKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (max_pos < 1 || max_pos > WUSHKV_MAX_POS) return fail(WUSHKV_ERR_INVALID_ARG, "max_pos must be in [1, 2^24]");
  float om[64];
  wushkv_status st = wushkv_rope_frequencies(theta, om);
  if (st) return st;
  int dev;
  st = current_device(&dev);
  if (st) return st;
  const int hi_rows = (max_pos + 1023) / 1024;
  const size_t n0 = (size_t)32 * 64, n2 = (size_t)hi_rows * 64;
  // [t0 | t1 | t2 | t0t | t1t | t2t], each entry (cos, sin) as two doubles
  const size_t heads = 2 * n0 + n2;
  std::vector<double> buf(4 * heads);
  double* head = buf.data();
  double* tail = head + 2 * heads;
  // entry e of a table starting at entry offset `off`: angle = mult * w_i
  auto fill = [&](size_t off, size_t row, double mult, int i) {
    const double ang = mult * (double)om[i];  // exact: < 2^24 times a 24-bit significand
    const long double c = cosl((long double)ang), s = sinl((long double)ang);
    const double ch = (double)c, sh = (double)s;
    const size_t k = 2 * (off + row * 64 + i);
    head[k] = ch;
    head[k + 1] = sh;
    tail[k] = (double)(c - (long double)ch);
    tail[k + 1] = (double)(s - (long double)sh);
  };
  for (size_t r = 0; r < 32; ++r)
    for (int i = 0; i < 64; ++i) {
      fill(0, r, (double)r, i);
      fill(n0, r, (double)(r * 32), i);
    }
  for (size_t r = 0; r < (size_t)hi_rows; ++r)
    for (int i = 0; i < 64; ++i) fill(2 * n0, r, (double)(r * 1024), i);
  auto* rp = new (std::nothrow) wushkv_rope();
  if (!rp) return fail(WUSHKV_ERR_OOM, "host allocation failed");
  rp->theta = theta;
  rp->max_pos = max_pos;
  rp->device = dev;
  rp->hi_rows = hi_rows;
  hipError_t e = hipMalloc(&rp->d_block, buf.size() * sizeof(double));
  if (e != hipSuccess) { delete rp; return fail(WUSHKV_ERR_OOM, "hipMalloc for the RoPE tables failed"); }
  e = hipMemcpy(rp->d_block, buf.data(), buf.size() * sizeof(double), hipMemcpyHostToDevice);
  if (e != hipSuccess) { (void)hipFree(rp->d_block); delete rp; return hip_fail(e, "hipMemcpy (RoPE tables)"); }
  const double2* base = (const double2*)rp->d_block;
  rp->t0 = base;
  rp->t1 = base + n0;
  rp->t2 = base + 2 * n0;
  rp->t0t = base + heads;
  rp->t1t = base + heads + n0;
  rp->t2t = base + heads + 2 * n0;
  // The (cos, sin) of every multiple of 32 positions (head and tail, 32 bytes per
  // pair): the key kernel adds the angle of pos % 32 to them.
  rp->hi2_rows = (max_pos + 31) / 32;
  const size_t hi_bytes = (size_t)rp->hi2_rows * 64 * 2 * sizeof(double2);
  e = hipMalloc((void**)&rp->hi, hi_bytes + (size_t)rp->hi2_rows * sizeof(uint32_t));
  if (e != hipSuccess) {
    (void)hipFree(rp->d_block);
    delete rp;
    return fail(WUSHKV_ERR_OOM, "hipMalloc for the RoPE tables failed");
  }
  rp->hit = rp->hi + (size_t)rp->hi2_rows * 64;
  rp->exc = (uint32_t*)((char*)rp->hi + hi_bytes);
  e = wushkv::launch_build_rope_hi(rp, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(rp->hi);
    (void)hipFree(rp->d_block);
    delete rp;
    return hip_fail(e, "RoPE table build");
  }
  *out = rp;
  return WUSHKV_OK;
}

wushkv_status wushkv_rope_destroy(wushkv_rope* r) {
  if (!r) return WUSHKV_OK;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(r->device);
  (void)hipFree(r->hi);
  (void)hipFree(r->d_block);
  if (prev >= 0) (void)hipSetDevice(prev);
  delete r;
  return WUSHKV_OK;
}

static wushkv_status keys_common(const void* K, wushkv_dtype k_dtype, int64_t n_tokens, int n_heads,
                                 int64_t token_stride, const int32_t* pos, const wushkv_rope* rope,
                                 const wushkv_transform* T_k, int bits, const wushkv_quantizer* quantizer,
                                 const wushkv_packed* out, float* y_out, void* stream) {
  wushkv_status st = check_tensor(K, k_dtype, n_tokens, n_heads, token_stride);
  if (st) return st;
  if (!rope) return fail(WUSHKV_ERR_INVALID_ARG, "rope handle is NULL");
  if (!T_k) return fail(WUSHKV_ERR_INVALID_ARG, "transform handle is NULL");
  if (T_k->n_heads != n_heads) return fail(WUSHKV_ERR_INVALID_ARG, "transform has a different head count");
  wushkv::QuantArgs qa{};
  if (!y_out) {
    if (bits < 2 || bits > 4) return fail(WUSHKV_ERR_INVALID_ARG, "bits must be 2, 3 or 4");
    st = make_quant(quantizer, &qa);
    if (st) return st;
    st = check_packed(out, qa.kind, n_tokens, true);
    if (st) return st;
  } else if (!aligned(y_out, 16)) {
    return fail(WUSHKV_ERR_ALIGNMENT, "y_out must be 16-byte aligned");
  }
  if (n_tokens == 0) return WUSHKV_OK;
  if (!pos) return fail(WUSHKV_ERR_INVALID_ARG, "pos is NULL");
  int dev;
  st = current_device(&dev);
  if (st) return st;
  if (dev != T_k->device || dev != rope->device)
    return fail(WUSHKV_ERR_INVALID_ARG, "handles belong to another device than the current one");
  const int cus = wushkv::device_cu_count(dev);
  const int64_t n_tiles = (n_tokens + 63) / 64;
  // fp32 keys and general percentiles (a 32-key sort per group in registers) run at up to
  // two heads per block, where a wave has twice the registers
  const int hg = choose_hg(n_tiles, n_heads, cus, (k_dtype == WUSHKV_F32 || qa.kind == 2) ? 2 : 4);
  wushkv::KeysArgs a{};
  a.K = K;
  a.n_tokens = n_tokens;
  a.n_heads = n_heads;
  a.stride = token_stride;
  a.pos = pos;
  a.max_pos = rope->max_pos;
  a.T = T_k->d_swz;
  a.rope_lo = rope->t0;
  a.rope_lot = rope->t0t;
  a.rope_hi = rope->hi;
  a.rope_hit = rope->hit;
  a.rope_exc = rope->exc;
  if (out && !y_out) {
    a.codes = (uint8_t*)out->codes;
    a.scales = (uint16_t*)out->scales;
    a.zeros = (uint16_t*)out->zeros;
    a.slots = out->slots;
    a.n_rows = out->n_rows;
  }
  a.q = qa;
  a.y_out = y_out;
  a.n_groups = n_heads / hg;
  hipError_t e = T_k->hadamard
                     ? wushkv::launch_keys_fwht(a, bits, k_dtype == WUSHKV_F32, y_out != nullptr, cus, (hipStream_t)stream)
                     : wushkv::launch_keys(a, bits, k_dtype == WUSHKV_F32, hg, y_out != nullptr, cus, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "key kernel launch");
  return WUSHKV_OK;
}

wushkv_status wushkv_quantize_keys(const void* K, wushkv_dtype k_dtype, int64_t n_tokens, int n_heads,
                                   int64_t token_stride, const int32_t* pos, const wushkv_rope* rope,
                                   const wushkv_transform* T_k, int bits, const wushkv_quantizer* quantizer,
                                   const wushkv_packed* out, void* stream) {
  return keys_common(K, k_dtype, n_tokens, n_heads, token_stride, pos, rope, T_k, bits, quantizer, out,
                     nullptr, stream);
}

wushkv_status wushkv_debug_rope_transform(const void* K, wushkv_dtype k_dtype, int64_t n_tokens, int n_heads,
                                          int64_t token_stride, const int32_t* pos, const wushkv_rope* rope,
                                          const wushkv_transform* T_k, float* y_out, void* stream) {
  if (!y_out) return fail(WUSHKV_ERR_INVALID_ARG, "y_out is NULL");
  return keys_common(K, k_dtype, n_tokens, n_heads, token_stride, pos, rope, T_k, 2, nullptr, nullptr, y_out,
                     stream);
}

wushkv_status wushkv_quantize_values(const void* V, wushkv_dtype v_dtype, int64_t n_tokens, int n_heads,
                                     int64_t token_stride, int bits, const wushkv_quantizer* quantizer,
                                     const wushkv_packed* out, void* stream) {
  wushkv_status st = check_tensor(V, v_dtype, n_tokens, n_heads, token_stride);
  if (st) return st;
  if (bits < 2 || bits > 4) return fail(WUSHKV_ERR_INVALID_ARG, "bits must be 2, 3 or 4");
  wushkv::QuantArgs qa{};
  st = make_quant(quantizer, &qa);
  if (st) return st;
  st = check_packed(out, qa.kind, n_tokens, true);
  if (st) return st;
  if (n_tokens == 0) return WUSHKV_OK;
  int dev;
  st = current_device(&dev);
  if (st) return st;
  if (n_tokens * n_heads >= (1LL << 31))
    return fail(WUSHKV_ERR_UNSUPPORTED, "values need n_tokens * n_heads < 2^31");
  wushkv::ValuesArgs a{};
  a.V = V;
  a.n_tokens = n_tokens;
  a.n_heads = n_heads;
  a.stride = token_stride;
  div_magic((uint32_t)n_heads, &a.div_m, &a.div_l);
  a.codes = (uint8_t*)out->codes;
  a.scales = (uint16_t*)out->scales;
  a.zeros = (uint16_t*)out->zeros;
  a.slots = out->slots;
  a.n_rows = out->n_rows;
  a.q = qa;
  hipError_t e = wushkv::launch_values(a, bits, v_dtype == WUSHKV_F32, wushkv::device_cu_count(dev),
                                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "value kernel launch");
  return WUSHKV_OK;
}

wushkv_status wushkv_quantize_kv(const void* K, const void* V, wushkv_dtype dtype, int64_t n_tokens, int n_heads,
                                 int64_t k_stride, int64_t v_stride, const int32_t* pos, const wushkv_rope* rope,
                                 const wushkv_transform* T_k, int bits, const wushkv_quantizer* quantizer,
                                 const wushkv_packed* k_out, const wushkv_packed* v_out, void* stream) {
  wushkv_status st = check_tensor(K, dtype, n_tokens, n_heads, k_stride);
  if (st) return st;
  st = check_tensor(V, dtype, n_tokens, n_heads, v_stride);
  if (st) return st;
  if (!rope) return fail(WUSHKV_ERR_INVALID_ARG, "rope handle is NULL");
  if (!T_k) return fail(WUSHKV_ERR_INVALID_ARG, "transform handle is NULL");
  if (T_k->n_heads != n_heads) return fail(WUSHKV_ERR_INVALID_ARG, "transform has a different head count");
  if (bits < 2 || bits > 4) return fail(WUSHKV_ERR_INVALID_ARG, "bits must be 2, 3 or 4");
  wushkv::QuantArgs qa{};
  st = make_quant(quantizer, &qa);
  if (st) return st;
  st = check_packed(k_out, qa.kind, n_tokens, true);
  if (st) return st;
  st = check_packed(v_out, qa.kind, n_tokens, true);
  if (st) return st;
  if (n_tokens == 0) return WUSHKV_OK;
  if (!pos) return fail(WUSHKV_ERR_INVALID_ARG, "pos is NULL");
  if (n_tokens * n_heads >= (1LL << 31))
    return fail(WUSHKV_ERR_UNSUPPORTED, "the fused call needs n_tokens * n_heads < 2^31");
  int dev;
  st = current_device(&dev);
  if (st) return st;
  if (dev != T_k->device || dev != rope->device)
    return fail(WUSHKV_ERR_INVALID_ARG, "handles belong to another device than the current one");
  wushkv::AppendArgs a{};
  a.K = K;
  a.V = V;
  a.n_tokens = n_tokens;
  a.n_heads = n_heads;
  a.k_stride = k_stride;
  a.v_stride = v_stride;
  a.pos = pos;
  a.max_pos = rope->max_pos;
  a.T = T_k->d_swz;
  a.rope_lo = rope->t0;
  a.rope_lot = rope->t0t;
  a.rope_hi = rope->hi;
  a.rope_hit = rope->hit;
  a.rope_exc = rope->exc;
  a.k_codes = (uint8_t*)k_out->codes;
  a.k_scales = (uint16_t*)k_out->scales;
  a.k_zeros = (uint16_t*)k_out->zeros;
  a.k_slots = k_out->slots;
  a.k_rows = k_out->n_rows;
  a.v_codes = (uint8_t*)v_out->codes;
  a.v_scales = (uint16_t*)v_out->scales;
  a.v_zeros = (uint16_t*)v_out->zeros;
  a.v_slots = v_out->slots;
  a.v_rows = v_out->n_rows;
  a.q = qa;
  hipError_t e = wushkv::launch_append(a, bits, dtype == WUSHKV_F32, wushkv::device_cu_count(dev),
                                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fused key/value kernel launch");
  return WUSHKV_OK;
}

wushkv_status wushkv_dequantize(const wushkv_packed* in, int64_t n_tokens, int n_heads, int bits,
                                const wushkv_quantizer* quantizer, const wushkv_transform* T_k_inv, void* out,
                                wushkv_dtype out_dtype, void* stream) {
  if (bits < 2 || bits > 4) return fail(WUSHKV_ERR_INVALID_ARG, "bits must be 2, 3 or 4");
  if (n_heads < 1 || n_heads > 4096) return fail(WUSHKV_ERR_INVALID_ARG, "n_heads out of range");
  if (n_tokens < 0) return fail(WUSHKV_ERR_INVALID_ARG, "n_tokens < 0");
  if (out_dtype != WUSHKV_F32 && out_dtype != WUSHKV_BF16) return fail(WUSHKV_ERR_INVALID_ARG, "bad out_dtype");
  wushkv::QuantArgs qa{};
  wushkv_status st = make_quant(quantizer, &qa);
  if (st) return st;
  st = check_packed(in, qa.kind, n_tokens, false);
  if (st) return st;
  if (T_k_inv && T_k_inv->n_heads != n_heads) return fail(WUSHKV_ERR_INVALID_ARG, "T_k_inv has a different head count");
  if (n_tokens == 0) return WUSHKV_OK;
  if (!out) return fail(WUSHKV_ERR_INVALID_ARG, "out is NULL");
  if (!aligned(out, 16)) return fail(WUSHKV_ERR_ALIGNMENT, "out must be 16-byte aligned");
  // without T_k_inv one thread per (token, head) vector, in one dispatch
  if (!T_k_inv && n_tokens * n_heads > ((int64_t)1 << 32) - 256)
    return fail(WUSHKV_ERR_UNSUPPORTED, "n_tokens * n_heads must be at most 2^32 - 256 without T_k_inv");
  int dev;
  st = current_device(&dev);
  if (st) return st;
  if (T_k_inv && T_k_inv->device != dev) return fail(WUSHKV_ERR_INVALID_ARG, "T_k_inv belongs to another device");
  const int cus = wushkv::device_cu_count(dev);
  wushkv::DequantArgs a{};
  a.codes = (const uint8_t*)in->codes;
  a.scales = (const uint16_t*)in->scales;
  a.zeros = (const uint16_t*)in->zeros;
  a.slots = in->slots;
  a.n_rows = in->n_rows;
  a.n_tokens = n_tokens;
  a.n_heads = n_heads;
  a.kind = qa.kind == 0 ? 0 : 1;  // both affine kinds read z + q s
  a.out = out;
  a.out_bf16 = out_dtype == WUSHKV_BF16;
  int hg = 1;
  if (T_k_inv) {
    a.Tinv = T_k_inv->d_swz;
    a.gsum = T_k_inv->d_gsum;
    const int64_t n_tiles = (n_tokens + 31) / 32;
    hg = choose_hg(n_tiles, n_heads, cus, 4);
    a.n_groups = n_heads / hg;
  }
  hipError_t e = wushkv::launch_dequant(a, bits, hg, cus, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "dequantize kernel launch");
  return WUSHKV_OK;
}

wushkv_status wushkv_debug_check_arith(uint32_t* counts, void* stream) {
  if (!counts) return fail(WUSHKV_ERR_INVALID_ARG, "counts is NULL");
  if (!aligned(counts, 4)) return fail(WUSHKV_ERR_ALIGNMENT, "counts must be 4-byte aligned");
  int dev;
  wushkv_status st = current_device(&dev);
  if (st) return st;
  hipError_t e = wushkv::launch_arith_check(counts, wushkv::device_cu_count(dev), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "arithmetic check launch");
  return WUSHKV_OK;
}

wushkv_status wushkv_debug_time_next_launch(void* start, void* stop) {
  g_launch_events.start = (hipEvent_t)start;
  g_launch_events.stop = (hipEvent_t)stop;
  return WUSHKV_OK;
}

wushkv_status wushkv_debug_rope_cos_sin(const wushkv_rope* rope, const int32_t* pos, int64_t n, float* cs_out,
                                        void* stream) {
  if (n < 0) return fail(WUSHKV_ERR_INVALID_ARG, "n < 0");
  if (n > ((int64_t)1 << 26))  // one thread per (position, pair) in one dispatch
    return fail(WUSHKV_ERR_UNSUPPORTED, "n must be at most 2^26");
  if (!rope) return fail(WUSHKV_ERR_INVALID_ARG, "rope handle is NULL");
  if (n == 0) return WUSHKV_OK;
  if (!pos || !cs_out) return fail(WUSHKV_ERR_INVALID_ARG, "pos and cs_out must be set");
  hipError_t e = wushkv::launch_gather_cs(rope, pos, n, cs_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cos/sin gather launch");
  return WUSHKV_OK;
}

static constexpr int64_t kMaxPairVecs = ((int64_t)1 << 26) - 4;

wushkv_status wushkv_pair_queries(const void* Q, wushkv_dtype q_dtype, int64_t n_tokens, int n_q_heads,
                                  int64_t token_stride, const wushkv_transform* T_k_inv, void* q_out,
                                  void* stream) {
  wushkv_status st = check_tensor(Q, q_dtype, n_tokens, n_q_heads, token_stride);
  if (st) return st;
  if (n_tokens > kMaxPairVecs)  // at least one query vector per token and KV head
    return fail(WUSHKV_ERR_UNSUPPORTED, "more than 2^26 - 4 query vectors per KV head in one call");
  if (!T_k_inv) return fail(WUSHKV_ERR_INVALID_ARG, "transform handle is NULL");
  if (n_q_heads % T_k_inv->n_heads)
    return fail(WUSHKV_ERR_INVALID_ARG, "n_q_heads must be a multiple of the transform's head count");
  if (n_tokens == 0) return WUSHKV_OK;
  if (!q_out) return fail(WUSHKV_ERR_INVALID_ARG, "q_out is NULL");
  if (!aligned(q_out, 2)) return fail(WUSHKV_ERR_ALIGNMENT, "q_out must be 2-byte aligned");
  // 256-thread blocks of 4 query vectors: fewer than 2^24 blocks per KV head
  if (n_tokens * (n_q_heads / T_k_inv->n_heads) > kMaxPairVecs)
    return fail(WUSHKV_ERR_UNSUPPORTED, "more than 2^26 - 4 query vectors per KV head in one call");
  int dev;
  st = current_device(&dev);
  if (st) return st;
  if (dev != T_k_inv->device) return fail(WUSHKV_ERR_INVALID_ARG, "transform belongs to another device");
  wushkv::PairArgs a{};
  a.Q = Q;
  a.f32_in = q_dtype == WUSHKV_F32;
  a.n_tokens = n_tokens;
  a.stride = token_stride;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = T_k_inv->n_heads;
  a.G = n_q_heads / T_k_inv->n_heads;
  a.Tinv = T_k_inv->d_swz;
  a.out = (uint16_t*)q_out;
  hipError_t e = wushkv::launch_pair_queries(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "query pairing launch");
  return WUSHKV_OK;
}

static wushkv_status attention_shape(int n_seqs, int n_q_heads, int n_kv_heads, int max_seq_len) {
  if (n_seqs < 0 || n_seqs > 65535) return fail(WUSHKV_ERR_INVALID_ARG, "n_seqs must be in [0, 65535]");
  if (n_kv_heads < 1 || n_kv_heads > 65535) return fail(WUSHKV_ERR_INVALID_ARG, "n_kv_heads must be in [1, 65535]");
  if (n_q_heads < 1 || n_q_heads % n_kv_heads)
    return fail(WUSHKV_ERR_INVALID_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
  if (n_q_heads / n_kv_heads > 8) return fail(WUSHKV_ERR_UNSUPPORTED, "more than 8 query heads per KV head");
  if (n_q_heads > 65535) return fail(WUSHKV_ERR_INVALID_ARG, "n_q_heads above 65535");
  if (max_seq_len < 0 || max_seq_len > (1 << 30)) return fail(WUSHKV_ERR_INVALID_ARG, "max_seq_len must be in [0, 2^30]");
  // one 256-thread block per (sequence, KV head, split), splits rounded up to
  // a multiple of 8: a dispatch holds fewer than 2^32 work-items
  const int64_t splits8 = ((int64_t)wushkv::attention_splits(max_seq_len) + 7) / 8;
  if (8 * splits8 * n_kv_heads * (int64_t)n_seqs >= ((int64_t)1 << 24))
    return fail(WUSHKV_ERR_UNSUPPORTED, "a call needs 8 * ceil(ceil(max_seq_len / 2048) / 8) * n_kv_heads * n_seqs "
                                        "below 2^24 (one 256-thread block each)");
  return WUSHKV_OK;
}

wushkv_status wushkv_decode_attention_workspace(int n_seqs, int n_q_heads, int n_kv_heads, int max_seq_len,
                                                size_t* bytes) {
  if (!bytes) return fail(WUSHKV_ERR_INVALID_ARG, "bytes is NULL");
  wushkv_status st = attention_shape(n_seqs, n_q_heads, n_kv_heads, max_seq_len);
  if (st) return st;
  *bytes = wushkv::attention_workspace_bytes(n_seqs, n_q_heads, max_seq_len);
  return WUSHKV_OK;
}

static wushkv_status attention_common(const void* q_paired, int n_seqs, int n_q_heads,
                                      const wushkv_packed* k_cache, const wushkv_packed* v_cache, int n_kv_heads,
                                      int bits, const wushkv_quantizer* quantizer, const int64_t* seq_row0,
                                      const int32_t* seq_len, int max_seq_len, float scale, bool own_scratch,
                                      void* workspace, size_t workspace_bytes, float* out, void* stream) {
  wushkv_status st = attention_shape(n_seqs, n_q_heads, n_kv_heads, max_seq_len);
  if (st) return st;
  if (bits < 2 || bits > 4) return fail(WUSHKV_ERR_INVALID_ARG, "bits must be 2, 3 or 4");
  wushkv::QuantArgs qa{};
  st = make_quant(quantizer, &qa);
  if (st) return st;
  // symmetric (one step per record) or affine (four steps and zeros) caches, both
  // written with this quantizer
  st = check_packed(k_cache, qa.kind, 0, false);
  if (st) return st;
  st = check_packed(v_cache, qa.kind, 0, false);
  if (st) return st;
  if (k_cache->n_rows != v_cache->n_rows) return fail(WUSHKV_ERR_INVALID_ARG, "key and value caches differ in rows");
  if (!std::isfinite(scale)) return fail(WUSHKV_ERR_INVALID_ARG, "scale must be finite");
  if (n_seqs == 0) return WUSHKV_OK;
  if (!q_paired || !seq_row0 || !seq_len || !out)
    return fail(WUSHKV_ERR_INVALID_ARG, "q_paired, seq_row0, seq_len and out must be set");
  if (!aligned(q_paired, 2) || !aligned(seq_row0, 8) || !aligned(seq_len, 4) || !aligned(out, 4))
    return fail(WUSHKV_ERR_ALIGNMENT, "misaligned q_paired, seq_row0, seq_len or out");
  const size_t need = wushkv::attention_workspace_bytes(n_seqs, n_q_heads, max_seq_len);
  if (own_scratch) {
    if (need > WUSHKV_NOALLOC_SCRATCH_BYTES)
      return fail(WUSHKV_ERR_UNSUPPORTED, "split partials of " + std::to_string(need) +
                                              " bytes exceed the library's scratch buffer of " +
                                              std::to_string((size_t)WUSHKV_NOALLOC_SCRATCH_BYTES) + " bytes");
    int dev;
    st = current_device(&dev);
    if (st) return st;
    const hipError_t e = wushkv::attention_scratch(dev, &workspace);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (attention scratch)");
  } else {
    if (workspace_bytes < need)
      return fail(WUSHKV_ERR_INVALID_ARG, "workspace smaller than wushkv_decode_attention_workspace");
    if (need > 0 && (!workspace || !aligned(workspace, 16)))
      return fail(workspace ? WUSHKV_ERR_ALIGNMENT : WUSHKV_ERR_INVALID_ARG, "workspace must be set and 16-byte aligned");
  }
  wushkv::AttnArgs a{};
  a.qp = (const uint16_t*)q_paired;
  a.kc = (const uint8_t*)k_cache->codes;
  a.ks = (const uint16_t*)k_cache->scales;
  a.vc = (const uint8_t*)v_cache->codes;
  a.vs = (const uint16_t*)v_cache->scales;
  a.kz = qa.kind ? (const uint16_t*)k_cache->zeros : nullptr;
  a.vz = qa.kind ? (const uint16_t*)v_cache->zeros : nullptr;
  a.n_rows = k_cache->n_rows;
  a.row0 = seq_row0;
  a.len = seq_len;
  a.n_seqs = n_seqs;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.G = n_q_heads / n_kv_heads;
  a.max_len = max_seq_len;
  a.n_splits = wushkv::attention_splits(max_seq_len);
  a.n_splits8 = (a.n_splits + 7) / 8;
  a.c0 = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)
  a.part = (float*)workspace;
  a.out = out;
  hipError_t e = wushkv::launch_attention(a, bits, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return WUSHKV_OK;
}

wushkv_status wushkv_decode_attention(const void* q_paired, int n_seqs, int n_q_heads,
                                      const wushkv_packed* k_cache, const wushkv_packed* v_cache,
                                      int n_kv_heads, int bits, const wushkv_quantizer* quantizer,
                                      const int64_t* seq_row0, const int32_t* seq_len, int max_seq_len,
                                      float scale, void* workspace, size_t workspace_bytes, float* out,
                                      void* stream) {
  return attention_common(q_paired, n_seqs, n_q_heads, k_cache, v_cache, n_kv_heads, bits, quantizer, seq_row0,
                          seq_len, max_seq_len, scale, false, workspace, workspace_bytes, out, stream);
}

wushkv_status wushkv_decode_attention_noalloc(const void* q_paired, int n_seqs, int n_q_heads,
                                              const wushkv_packed* k_cache, const wushkv_packed* v_cache,
                                              int n_kv_heads, int bits, const wushkv_quantizer* quantizer,
                                              const int64_t* seq_row0, const int32_t* seq_len, int max_seq_len,
                                              float scale, float* out, void* stream) {
  return attention_common(q_paired, n_seqs, n_q_heads, k_cache, v_cache, n_kv_heads, bits, quantizer, seq_row0,
                          seq_len, max_seq_len, scale, true, nullptr, 0, out, stream);
}

}  // extern "C"
