/*
 * Seeded synthetic inputs for the WUSH-KV write/read path.
 *
 * This module produces the tensors that both the CPU oracle and the GPU
 * library consume: pre-RoPE keys, values, positions, decode slots and the
 * per-head key transforms T_k = Q * diag(s) with their closed-form inverses.
 * It holds none of the method's arithmetic (no RoPE, no transform, no
 * quantizer); it only draws numbers.
 *
 * Generator: every draw is the idx-th output of a SplitMix64 stream
 * (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014): state = key + idx * 0x9E3779B97F4A7C15, output = the SplitMix64
 * finalizer of that state.  The stream key is derived from (seed, stream id), so
 * any slice (layer, token range) regenerates identically and in any order.
 *
 *   uniform(key, i)  = ((draw >> 11) + 0.5) * 2^-53            in (0, 1)
 *   normal(key, i)   = Box-Muller on the uniform pair (2*(i>>1), 2*(i>>1)+1):
 *                      r = sqrt(-2 ln u1), t = 2 pi u2; even i -> r cos t, odd i -> r sin t
 *   t3(key, i)       = z0 / sqrt((z1^2 + z2^2 + z3^2) / 3), z_k = normal(key, 4i+k)
 *   lognormal(mu,sg) = exp(mu + sg * normal)
 *
 * Values are produced in fp64, rounded once to fp32 and, for bf16 output, then
 * rounded to bf16 with round-to-nearest-even.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define D 128

enum { DIST_GAUSS_OUTLIER = 0, DIST_HEAVY_T3 = 1, DIST_LOGNORMAL_GAUSS = 2 };
enum {
  TAG_K = 0, TAG_V = 1, TAG_Q = 2, TAG_S = 3, TAG_SIGMA_K = 4, TAG_SIGMA_V = 5,
  TAG_OUT_K = 6, TAG_OUT_V = 7, TAG_POS = 8
};

static inline uint64_t sm64_final(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}
static inline uint64_t draw(uint64_t key, uint64_t idx) {
  return sm64_final(key + (idx + 1) * 0x9E3779B97F4A7C15ULL);
}
static uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return draw(draw(seed, 0) ^ (stream * 0xD2B74407B1CE6E93ULL), 0);
}
static inline double uniform01(uint64_t key, uint64_t idx) {
  return ((double)(draw(key, idx) >> 11) + 0.5) * 0x1p-53;
}
static inline double normal(uint64_t key, uint64_t idx) {
  uint64_t p = idx >> 1;
  double u1 = uniform01(key, 2 * p), u2 = uniform01(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  return (idx & 1) ? r * sin(t) : r * cos(t);
}
static inline double student_t3(uint64_t key, uint64_t idx) {
  double z0 = normal(key, 4 * idx), z1 = normal(key, 4 * idx + 1);
  double z2 = normal(key, 4 * idx + 2), z3 = normal(key, 4 * idx + 3);
  return z0 / sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0);
}
static uint64_t layer_stream(int layer, int tag) { return ((uint64_t)layer << 8) | (uint64_t)tag; }

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Outlier channels of (layer, head, tensor): a partial Fisher-Yates shuffle of
 * 0..127 driven by the stream, first n_out entries. */
static void outlier_channels(uint64_t seed, int layer, int tensor, int head, int n_out, int* out) {
  int perm[D];
  for (int i = 0; i < D; ++i) perm[i] = i;
  uint64_t key = stream_key(seed, layer_stream(layer, tensor == 0 ? TAG_OUT_K : TAG_OUT_V));
  for (int t = 0; t < n_out; ++t) {
    int j = t + (int)(draw(key, (uint64_t)head * 16 + t) % (uint64_t)(D - t));
    int tmp = perm[t]; perm[t] = perm[j]; perm[j] = tmp;
  }
  for (int t = 0; t < n_out; ++t) out[t] = perm[t];
}

typedef struct {
  uint64_t seed; int dist; int layer; int tensor; int64_t n0, n1; int H;
  int out_bf16; void* out; double outlier_scale; int n_outliers;
  const double* sigma; /* [H][128] or NULL */
  const unsigned char* is_out; /* [H][128] or NULL */
} kv_job;

static void* kv_worker(void* arg) {
  kv_job* j = (kv_job*)arg;
  uint64_t key = stream_key(j->seed, layer_stream(j->layer, j->tensor == 0 ? TAG_K : TAG_V));
  for (int64_t n = j->n0; n < j->n1; ++n) {
    for (int h = 0; h < j->H; ++h) {
      for (int c = 0; c < D; ++c) {
        uint64_t idx = ((uint64_t)n * (uint64_t)j->H + (uint64_t)h) * D + (uint64_t)c;
        double v;
        if (j->dist == DIST_GAUSS_OUTLIER) {
          v = normal(key, idx);
          if (j->is_out[h * D + c]) v *= j->outlier_scale;
        } else if (j->dist == DIST_HEAVY_T3) {
          v = j->sigma[h * D + c] * student_t3(key, idx);
        } else {
          v = j->sigma[h * D + c] * normal(key, idx);
        }
        float f = (float)v;
        /* j->out already points at this worker's first token */
        int64_t o = ((n - j->n0) * j->H + h) * D + c;
        if (j->out_bf16) ((uint16_t*)j->out)[o] = f32_to_bf16_rne(f);
        else ((float*)j->out)[o] = f;
      }
    }
  }
  return NULL;
}

/* Channel scales sigma[h][c] ~ LogNormal(0, 1), one set per (layer, tensor). */
void synth_channel_sigma(uint64_t seed, int layer, int tensor, int H, double* sigma) {
  uint64_t key = stream_key(seed, layer_stream(layer, tensor == 0 ? TAG_SIGMA_K : TAG_SIGMA_V));
  for (int i = 0; i < H * D; ++i) sigma[i] = exp(normal(key, (uint64_t)i));
}

/* Fill out[n][H][128] for tokens n0 .. n0+n-1 of (layer, tensor). */
int synth_kv(uint64_t seed, int dist, int layer, int tensor, int64_t n0, int64_t n, int H,
             int out_bf16, void* out, int nthreads) {
  if (H <= 0 || n < 0 || (dist < 0 || dist > 2)) return -1;
  double* sigma = (double*)malloc(sizeof(double) * (size_t)H * D);
  unsigned char* is_out = (unsigned char*)calloc((size_t)H * D, 1);
  if (!sigma || !is_out) { free(sigma); free(is_out); return -2; }
  synth_channel_sigma(seed, layer, tensor, H, sigma);
  for (int h = 0; h < H; ++h) {
    int oc[4];
    outlier_channels(seed, layer, tensor, h, 4, oc);
    for (int t = 0; t < 4; ++t) is_out[h * D + oc[t]] = 1;
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if ((int64_t)nthreads > n) nthreads = n > 0 ? (int)n : 1;
  pthread_t th[64];
  kv_job jobs[64];
  for (int t = 0; t < nthreads; ++t) {
    kv_job* j = &jobs[t];
    j->seed = seed; j->dist = dist; j->layer = layer; j->tensor = tensor; j->H = H;
    j->out_bf16 = out_bf16; j->outlier_scale = 20.0; j->n_outliers = 4;
    j->sigma = sigma; j->is_out = is_out;
    j->n0 = n0 + n * t / nthreads; j->n1 = n0 + n * (t + 1) / nthreads;
    /* each worker writes relative to its own start; shift the output pointer */
    size_t esz = out_bf16 ? 2 : 4;
    j->out = (char*)out + (size_t)(j->n0 - n0) * (size_t)H * D * esz;
  }
  if (nthreads == 1) {
    kv_worker(&jobs[0]);
  } else {
    for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, kv_worker, &jobs[t]);
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  }
  free(sigma); free(is_out);
  return 0;
}

/* Outlier channel indices for (layer, tensor, head): 4 ints. */
void synth_outliers(uint64_t seed, int layer, int tensor, int head, int* out4) {
  outlier_channels(seed, layer, tensor, head, 4, out4);
}

/* Per-head key transform T = Q diag(s) and T^-1 = diag(1/s) Q^T, stored
 * row-major [H][128][128] fp32.  Q: Gram-Schmidt (two passes) on the columns
 * of a Gaussian matrix, which yields the Q of a QR factorisation with
 * positive diagonal R; s ~ LogNormal(0, 0.5). */
int synth_transform(uint64_t seed, int layer, int H, float* T, float* Tinv) {
  double* G = (double*)malloc(sizeof(double) * D * D);
  double* Q = (double*)malloc(sizeof(double) * D * D);
  if (!G || !Q) { free(G); free(Q); return -2; }
  uint64_t kq = stream_key(seed, layer_stream(layer, TAG_Q));
  uint64_t ks = stream_key(seed, layer_stream(layer, TAG_S));
  for (int h = 0; h < H; ++h) {
    for (int i = 0; i < D * D; ++i) G[i] = normal(kq, (uint64_t)h * D * D + (uint64_t)i);
    /* column j of G is G[r*D + j] */
    for (int j = 0; j < D; ++j) {
      double v[D];
      for (int r = 0; r < D; ++r) v[r] = G[r * D + j];
      for (int pass = 0; pass < 2; ++pass) {
        for (int i = 0; i < j; ++i) {
          double dot = 0.0;
          for (int r = 0; r < D; ++r) dot += Q[r * D + i] * v[r];
          for (int r = 0; r < D; ++r) v[r] -= dot * Q[r * D + i];
        }
      }
      double nrm = 0.0;
      for (int r = 0; r < D; ++r) nrm += v[r] * v[r];
      nrm = sqrt(nrm);
      for (int r = 0; r < D; ++r) Q[r * D + j] = v[r] / nrm;
    }
    double s[D];
    for (int c = 0; c < D; ++c) s[c] = exp(0.5 * normal(ks, (uint64_t)h * D + (uint64_t)c));
    for (int r = 0; r < D; ++r)
      for (int c = 0; c < D; ++c) {
        if (T) T[((size_t)h * D + r) * D + c] = (float)(Q[r * D + c] * s[c]);
        if (Tinv) Tinv[((size_t)h * D + r) * D + c] = (float)(Q[c * D + r] / s[r]);
      }
  }
  free(G); free(Q);
  return 0;
}

/* Uniform integers in [0, bound): draw % bound over the position stream. */
void synth_uniform_ints(uint64_t seed, int64_t n, int64_t bound, int32_t* out) {
  uint64_t key = stream_key(seed, layer_stream(0, TAG_POS));
  for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)(draw(key, (uint64_t)i) % (uint64_t)bound);
}

/* Raw stream access, for tests of the generator itself. */
uint64_t synth_draw(uint64_t seed, uint64_t stream, uint64_t idx) {
  return draw(stream_key(seed, stream), idx);
}
double synth_normal(uint64_t seed, uint64_t stream, uint64_t idx) {
  return normal(stream_key(seed, stream), idx);
}
double synth_t3(uint64_t seed, uint64_t stream, uint64_t idx) {
  return student_t3(stream_key(seed, stream), idx);
}
