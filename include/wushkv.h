/*
 * libwushkv — WUSH-KV KV-cache write/read path on AMD Instinct MI355X (gfx950).
 *
 * What the library computes, and where the pages about WUSH-KV (arXiv
 * 2609.38121) state it:
 *   - Keys are rotated with RoPE, then multiplied by their KV head's key
 *     transform T_k, a general invertible 128x128 matrix (not only an
 *     orthogonal one), online, because the transform is applied after RoPE
 *     (ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity ...", method and
 *     deployment paragraphs; arXiv abstract; cere-bro post "WUSH-KV: 2-bit
 *     KV-Cache Quantization with Data-Adaptive Transforms", Gaps, which counts the
 *     extra matrix product per decode step as the method's online cost).
 *   - Values need no online transform (it is folded into the weights) and are
 *     only quantized (same sources; the value branch of the cere-bro flowchart).
 *   - Both go through a clipped b-bit scalar quantizer: an RMS-clipped
 *     symmetric INT grid (the QuEST-style quantizer of the theory) or a
 *     percentile-clipped affine grid (the OSCAR-style quantizer of the
 *     end-to-end evaluation), per token, and are bit-packed into a paged /
 *     slot-addressed cache (ai4snews deployment and end-to-end paragraphs).
 *   - A read path unpacks and dequantizes, for keys optionally through T_k^-1.
 *
 * Numerical contract (what the GPU kernels reproduce):
 *   RoPE     rotate-half on channel pairs (i, i+64); w_i = RN32(theta^(-2i/128));
 *            c, s = cos, sin of the exact angle pos*w_i, each rounded once to
 *            fp32; x_i = fma(k_i, c, -(k_{i+64} s)), x_{i+64} = fma(k_{i+64}, c, k_i s).
 *   operands x~ = bf16(x) and T~ = bf16(T_k) (round-to-nearest-even);
 *            y = T~ x~ accumulated in fp32 (MFMA).
 *   sym      S = contiguous pairwise fp32 sum of y_j^2; rms = sqrt(S/128)
 *            (correctly rounded); C = alpha*rms; step = RN16sat(2C/(2^b-1));
 *            levels (q - (2^b-1)/2)*step.
 *   affine   per 32-channel group: lo, hi = p_lo / p_hi percentiles by linear
 *            interpolation between order statistics (IEEE totalOrder);
 *            step = RN16sat((hi-lo)/(2^b-1)), zero = RN16sat(lo); levels zero + q*step.
 *   codes    index of the nearest level in exact arithmetic, ties to the even
 *            code; step 0 gives code 2^(b-1) (sym) or 0 (affine).
 *   packing  code j of a 128-vector at bits [b*j, b*j+b) of an LSB-first bit
 *            stream (stream bit 8k+t = bit t of byte k): 16*b bytes per record.
 *
 * Memory layout (all device memory, caller-owned; the library never allocates
 * on the hot path):
 *   K, V     [n_tokens][n_heads][128], element (n,h,c) at base + n*token_stride
 *            + h*128 + c; bf16 or fp32; 16-byte aligned rows; a token row
 *            (token_stride elements) spans at most 2^24 bytes; n_tokens is
 *            below 2^31 - 128.
 *   codes    [n_rows][n_heads][16*bits] bytes.
 *   scales   fp16; sym: [n_rows][n_heads]; affine: [n_rows][n_heads][4].
 *   zeros    fp16, affine only: [n_rows][n_heads][4].
 *   row      slots[n] when slots != NULL, else n.
 *
 * Every call validates its arguments on the host before any launch and
 * returns a status; nothing is thrown.  Launches are asynchronous on the
 * given HIP stream (a hipStream_t passed as void*; NULL = the null stream).
 * Non-finite inputs are not supported (results unspecified, memory-safe).
 */
#ifndef WUSHKV_H_
#define WUSHKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WUSHKV_HEAD_DIM 128
#define WUSHKV_MAX_POS (1 << 24)

typedef enum {
  WUSHKV_OK = 0,
  WUSHKV_ERR_INVALID_ARG = 1,  /* NULL pointer, bad size, bad enum value        */
  WUSHKV_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. more than 8 query heads per KV head) */
  WUSHKV_ERR_ALIGNMENT = 3,    /* pointer or stride not aligned as required    */
  WUSHKV_ERR_NO_DEVICE = 4,    /* no HIP device visible                        */
  WUSHKV_ERR_HIP = 5,          /* a HIP runtime call failed                    */
  WUSHKV_ERR_OOM = 6           /* device allocation failed (handles only)      */
} wushkv_status;

typedef enum { WUSHKV_F32 = 0, WUSHKV_BF16 = 1 } wushkv_dtype;

typedef enum {
  WUSHKV_Q_SYM_RMS = 0,    /* symmetric grid, clip = clip_alpha * RMS over the 128-vector */
  WUSHKV_Q_AFFINE_PCT = 1  /* affine grid per 32-channel group, percentile clip          */
} wushkv_qkind;

/* Scalar quantizer description.
 *   WUSHKV_Q_SYM_RMS:    group must be 128; clip_alpha > 0 (2.0 in the workloads).
 *   WUSHKV_Q_AFFINE_PCT: group must be 32; 0 <= p_lo <= p_hi <= 100.  Each
 *     percentile interpolates linearly between order statistics i = floor(h)
 *     and i + 1 of the group, h = 31 p / 100 (see the numerical contract).
 *     When p_lo < 100/31 and p_hi >= 3000/31 (the 1st/99th percentiles among
 *     them) the kernels select the two extreme values at each end; other
 *     percentiles sort each group's 32 values in registers (bitonic network),
 *     which costs several times the vector instructions. */
typedef struct {
  int32_t kind;       /* wushkv_qkind */
  float clip_alpha;
  int32_t group;
  float p_lo, p_hi;
} wushkv_quantizer;

/* Packed cache view (device pointers, caller-owned).
 *   codes:  [n_rows][n_heads][16*bits] bytes, 16-byte aligned.
 *   scales: fp16 bits, 16-byte aligned.
 *   zeros:  fp16 bits for affine (16-byte aligned), NULL for symmetric.
 *   slots:  int64 row per token, or NULL (row = token index).  Rows outside
 *           [0, n_rows) are skipped by writers; the reader returns +0 for
 *           every channel of such a token.
 *   n_rows: capacity of the cache in rows, below 2^31.  With n_rows = 0 the
 *           pointers may be NULL (nothing is read or written through them). */
typedef struct {
  void* codes;
  void* scales;
  void* zeros;
  const int64_t* slots;
  int64_t n_rows;
} wushkv_packed;

typedef struct wushkv_transform wushkv_transform; /* opaque, library-owned */
typedef struct wushkv_rope wushkv_rope;           /* opaque, library-owned */

/* Key transform handle: rounds T (host, fp32, [n_heads][128][128] row-major,
 * y = T x) to bf16 once and stores it on the current device in the MFMA
 * operand order the kernels read.  The same call prepares T_k^-1 for reads.
 * Allocates device memory (not a hot-path call). */
wushkv_status wushkv_transform_create(const float* T_host, int n_heads, wushkv_transform** out);

/* Structured key transform: T = H_128 / 8 for every head, H the Sylvester
 * Hadamard matrix (H[r][c] = (-1)^popcount(r & c)), the pages' fixed-rotation
 * baseline (ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity ...",
 * method paragraph; cheaper structured transforms: limitations paragraph).
 * wushkv_quantize_keys and wushkv_debug_rope_transform take such a handle
 * through an in-register fast Walsh-Hadamard transform (7 butterfly stages in
 * fp32, no matrix product); the same T given to wushkv_transform_create runs
 * through the dense MFMA product.  Both compute y = T bf16(RoPE(k)) with fp32
 * accumulation and differ only in the order of the roundings.  The handle
 * holds the dense bf16 matrix too, which wushkv_quantize_kv uses.  Allocates
 * device memory (not a hot-path call). */
wushkv_status wushkv_transform_create_hadamard(int n_heads, wushkv_transform** out);
wushkv_status wushkv_transform_destroy(wushkv_transform* t);

/* RoPE handle for base theta and positions [0, max_pos), max_pos <= 2^24.
 * Holds fp64 (cos, sin) tables with extended-precision tails: those of
 * p0 * w_i for p0 < 32, and those of 32 h * w_i for every h < max_pos / 32
 * (64 bytes per position: 8 MiB at 2^17 positions, 1 GiB at 2^24), and a
 * bitmap of the positions whose fp64 angle sum rounds to fp32 differently from
 * the exact value for some pair (found once, at creation, against a
 * double-double sum).  The key kernel computes each token's exact fp32
 * (cos, sin) from them: one fp64 angle addition, double-double at the marked
 * positions.  Allocates device memory and synchronizes the device (not a
 * hot-path call). */
wushkv_status wushkv_rope_create(float theta, int32_t max_pos, wushkv_rope** out);
wushkv_status wushkv_rope_destroy(wushkv_rope* r);

/* Host-only: the 64 RoPE frequencies w_i = RN32(theta^(-2i/128)) the library
 * uses.  Touches no device. */
wushkv_status wushkv_rope_frequencies(float theta, float* omega_out /* [64] */);

/* Keys: RoPE -> bf16 -> T_k -> quantize -> pack into `out`.
 *   K: device, bf16 or fp32, layout above; token_stride in elements (>= n_heads*128,
 *      a multiple of 8 for bf16 and 4 for fp32).
 *   pos: device int32 [n_tokens]; positions are clamped to [0, max_pos).
 *   T_k: handle with n_heads heads; rope: handle for theta.
 *   bits: 2, 3 or 4.  n_tokens == 0 is a no-op. */
wushkv_status wushkv_quantize_keys(const void* K, wushkv_dtype k_dtype, int64_t n_tokens,
                                   int n_heads, int64_t token_stride, const int32_t* pos,
                                   const wushkv_rope* rope, const wushkv_transform* T_k, int bits,
                                   const wushkv_quantizer* quantizer, const wushkv_packed* out,
                                   void* stream);

/* Values: quantize -> pack (no RoPE, no transform).  Same layouts as keys.
 * n_tokens*n_heads must stay below 2^31 (WUSHKV_ERR_UNSUPPORTED otherwise). */
wushkv_status wushkv_quantize_values(const void* V, wushkv_dtype v_dtype, int64_t n_tokens,
                                     int n_heads, int64_t token_stride, int bits,
                                     const wushkv_quantizer* quantizer, const wushkv_packed* out,
                                     void* stream);

/* Keys and values of the same tokens in one dispatch: the append path of a
 * paged cache, built for small calls (one decode step's tokens, one per
 * sequence, or a 16-token chunk: ai4snews summary "WUSH-KV cuts 2-bit KV-cache
 * perplexity ...", experiments paragraph on 16-token chunks and deployment
 * paragraph on paged caches).  Computes exactly what wushkv_quantize_keys on K
 * and wushkv_quantize_values on V compute (the same bytes in both caches), with
 * one kernel instead of two; for long prefills those two calls are faster.
 *   K, V: device, both of `dtype`, layouts as for the single calls, with their
 *      own token strides.
 *   pos, rope, T_k, bits, quantizer: as for wushkv_quantize_keys; the one
 *      quantizer applies to keys and values.
 *   k_out, v_out: the key and value caches (each with its own slots and
 *      n_rows); their memory must not overlap.
 *   n_tokens * n_heads must stay below 2^31 (WUSHKV_ERR_UNSUPPORTED otherwise);
 *   n_tokens == 0 is a no-op. */
wushkv_status wushkv_quantize_kv(const void* K, const void* V, wushkv_dtype dtype, int64_t n_tokens, int n_heads,
                                 int64_t k_stride, int64_t v_stride, const int32_t* pos, const wushkv_rope* rope,
                                 const wushkv_transform* T_k, int bits, const wushkv_quantizer* quantizer,
                                 const wushkv_packed* k_out, const wushkv_packed* v_out, void* stream);

/* Read path: rows in->slots[n] (or n) for n < n_tokens are unpacked and
 * dequantized into out[n_tokens][n_heads][128] (fp32 or bf16, contiguous,
 * 16-byte aligned).  T_k_inv: NULL for values (or for keys kept in the
 * transformed basis); otherwise a transform handle holding T_k^-1, applied as
 * k^ = T~inv y^ with bf16 T~inv and fp32 accumulation.  Without T_k_inv the
 * call is one thread per vector in one dispatch: n_tokens * n_heads at most
 * 2^32 - 256, else WUSHKV_ERR_UNSUPPORTED. */
wushkv_status wushkv_dequantize(const wushkv_packed* in, int64_t n_tokens, int n_heads, int bits,
                                const wushkv_quantizer* quantizer,
                                const wushkv_transform* T_k_inv, void* out,
                                wushkv_dtype out_dtype, void* stream);

/* Query-side pairing for attention on the transformed-basis key cache: the
 * keys are cached as y = T_k x, and a query head q that reads them is paired
 * once as q' = T~inv^T q, so that q'.y^ = q.(T~inv y^), the score against the
 * read path's keys (ai4snews summary "WUSH-KV cuts 2-bit KV-cache perplexity
 * ...", method paragraph: the key transform is built with the query heads that
 * consume the cached keys in view).
 *   Q: device, bf16 or fp32, [n_tokens][n_q_heads][128] with token_stride
 *      elements per token (same rules as K); query head hq reads KV head
 *      hq / (n_q_heads / T_k_inv's head count).  At most 2^26 - 4 query
 *      vectors per KV head (n_tokens * n_q_heads / heads) per call (one
 *      256-thread block per four, and a dispatch holds fewer than 2^32
 *      work-items), else WUSHKV_ERR_UNSUPPORTED.
 *   T_k_inv: transform handle holding T_k^-1 (the read path's), bf16 T~inv.
 *   q_out: device bf16 [n_tokens][n_q_heads][128], contiguous, caller-owned:
 *      q'_j = bf16(RN32(sum_r T~inv[r][j] q_r)), the sum exact before the fp32
 *      rounding (fp64 accumulation of exact products in ascending r).
 * n_tokens == 0 is a no-op. */
wushkv_status wushkv_pair_queries(const void* Q, wushkv_dtype q_dtype, int64_t n_tokens, int n_q_heads,
                                  int64_t token_stride, const wushkv_transform* T_k_inv, void* q_out,
                                  void* stream);

/* Bytes of workspace wushkv_decode_attention needs for these sizes (host
 * only).  The workspace holds one partial result per (sequence, query head,
 * 2048-token split of max_seq_len). */
wushkv_status wushkv_decode_attention_workspace(int n_seqs, int n_q_heads, int n_kv_heads, int max_seq_len,
                                                size_t* bytes);

/* Decode attention of one query token per sequence over packed key and value
 * caches, symmetric or percentile-clipped affine, without dequantizing the cache
 * to memory.  Keys are scored
 * in their transformed basis with the paired query; values are read as stored
 * (their transform is folded into the weights: ai4snews summary, deployment
 * paragraph).  For sequence b and query head hq (KV head hq / G, G =
 * n_q_heads / n_kv_heads, at most 8):
 *   s_n = scale * q'.y^_n,  o = sum_n exp(s_n - max) v^_n / sum_n exp(s_n - max)
 * over the cache rows seq_row0[b] + n, n < min(seq_len[b], max_seq_len); rows
 * outside [0, n_rows) are absent; a sequence with no row present gives 0.
 *   q_paired: device bf16 [n_seqs][n_q_heads][128] (wushkv_pair_queries).
 *   k_cache, v_cache: caches written by wushkv_quantize_keys /
 *      wushkv_quantize_values with the same bits, quantizer and n_rows (their
 *      slots are not used here).  Affine caches (zeros set) are read as
 *      z_g + q s_g per 32-channel group (ai4snews summary, end-to-end
 *      paragraph): the score product sums each group's codes in its own
 *      column and the value product runs in fp32 with the weights times the
 *      group's step, the weighted zeros summed beside it.
 *   seq_row0: device int64 [n_seqs]; seq_len: device int32 [n_seqs].
 *   workspace: device, 16-byte aligned, at least the bytes reported by
 *      wushkv_decode_attention_workspace; caller-owned scratch that the call
 *      overwrites (two calls sharing one workspace must be ordered).
 *   out: device fp32 [n_seqs][n_q_heads][128].
 * Precision: codes and steps exact; q' bf16; scores accumulated in fp32 on
 * MFMA; exp2 and the weighted sum of values in fp32 (no bf16 rounding of the
 * weights).  Calls with 8 * ceil(ceil(max_seq_len / 2048) / 8) * n_kv_heads *
 * n_seqs at or above 2^24 (one 256-thread block each; a dispatch holds fewer
 * than 2^32 work-items) return WUSHKV_ERR_UNSUPPORTED, also from
 * wushkv_decode_attention_workspace.  n_seqs == 0 is a no-op. */
wushkv_status wushkv_decode_attention(const void* q_paired, int n_seqs, int n_q_heads,
                                      const wushkv_packed* k_cache, const wushkv_packed* v_cache,
                                      int n_kv_heads, int bits, const wushkv_quantizer* quantizer,
                                      const int64_t* seq_row0, const int32_t* seq_len, int max_seq_len,
                                      float scale, void* workspace, size_t workspace_bytes, float* out,
                                      void* stream);

/* Size of the library's own attention scratch buffer, per GPU. */
#define WUSHKV_NOALLOC_SCRATCH_BYTES (24u << 20)

/* Decode attention that allocates nothing, for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops and harnesses that forbid
 * hipMalloc.  Arguments, results and precision are those of
 * wushkv_decode_attention, minus the workspace: the split partials go to a
 * buffer of WUSHKV_NOALLOC_SCRATCH_BYTES that the library holds in static
 * device memory on every GPU it runs on, until the process ends.  Calls whose
 * partials need more (wushkv_decode_attention_workspace reports the bytes)
 * return WUSHKV_ERR_UNSUPPORTED before launching anything.  Every call on one
 * GPU shares that GPU's buffer, whose contents persist from the last call
 * (each call writes every partial it reads, so nothing is cleared): calls that
 * may overlap on one GPU (unordered streams) race and must be ordered by the
 * caller.  The call issues no hipMalloc, hipFree or other allocation. */
wushkv_status wushkv_decode_attention_noalloc(const void* q_paired, int n_seqs, int n_q_heads,
                                              const wushkv_packed* k_cache, const wushkv_packed* v_cache,
                                              int n_kv_heads, int bits, const wushkv_quantizer* quantizer,
                                              const int64_t* seq_row0, const int32_t* seq_len, int max_seq_len,
                                              float scale, float* out, void* stream);

/* Test support: the fp32 transformed keys y = T~ bf16(RoPE(K)) as the key
 * kernel computes them, written to y_out [n_tokens][n_heads][128] (device). */
wushkv_status wushkv_debug_rope_transform(const void* K, wushkv_dtype k_dtype, int64_t n_tokens,
                                          int n_heads, int64_t token_stride, const int32_t* pos,
                                          const wushkv_rope* rope, const wushkv_transform* T_k,
                                          float* y_out, void* stream);

/* Test support: the (cos, sin) pairs the key kernel uses, cs_out[n][64][2]
 * fp32 (device), for device positions pos[n] (clamped to [0, max_pos)),
 * computed by the same device function.  n at most 2^26 (one thread per
 * position and pair), else WUSHKV_ERR_UNSUPPORTED. */
wushkv_status wushkv_debug_rope_cos_sin(const wushkv_rope* rope, const int32_t* pos,
                                        int64_t n, float* cs_out, void* stream);

/* Self-check of the device arithmetic the step computation relies on: the fp16 step
 * comes from rms = sqrt(S / 128) and a division of the clip range by 2^b - 1, both of
 * which the numerical contract above takes as correctly rounded.
 * Runs, on the current device, sqrt and the division by 3, 7 and 15 exactly as the
 * kernels compile them over all 2^32 fp32 bit patterns, checking each result exactly
 * (sqrt against the squares of the neighbouring fp32 midpoints in fp64; the divisions
 * against the fp32 rounding of the fp64 quotient).  counts: device uint32[4],
 * overwritten with the mismatch counts for sqrt, / 3, / 7 and / 15 (all zero on a
 * conforming device).  Asynchronous on `stream`; tens of milliseconds. */
wushkv_status wushkv_debug_check_arith(uint32_t* counts, void* stream);

/* Timing support: the next wushkv_quantize_keys, wushkv_quantize_values, wushkv_quantize_kv,
 * wushkv_dequantize, wushkv_pair_queries or wushkv_decode_attention call
 * (its first kernel) on this host thread records `start` (a hipEvent_t)
 * when its kernel starts and `stop` when it ends (hipExtLaunchKernel), so
 * that hipEventElapsedTime(start, stop) is the kernel's own duration without
 * its dispatch latency.  Either may be NULL.  The events must exist (created,
 * for instance by one ordinary hipEventRecord) and belong to the device of
 * that call; the library neither creates nor destroys them.  The setting is
 * used once, by the next kernel launch of those calls on this thread; a call
 * that fails or returns without launching (zero tokens) leaves it pending.
 * Not for use while a stream is being captured into a graph. */
wushkv_status wushkv_debug_time_next_launch(void* start, void* stop);

const char* wushkv_status_string(wushkv_status s);
/* Detail message of the last failed call on this thread ("" if none). */
const char* wushkv_last_error(void);
int wushkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WUSHKV_H_ */
