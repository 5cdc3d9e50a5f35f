/*
 * libkvq -- rotation-based KV-cache quantization and decode attention computed
 * directly on the compressed cache, for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is either host memory (named *_host) or
 * device memory owned by the caller; the library never allocates, never frees
 * and keeps no global mutable state other than a thread-local error string.
 * Every call that launches work is asynchronous on the caller's HIP stream and
 * returns after host-side validation and the launch; results are valid after
 * the stream is synchronised.  No C++ exception crosses this boundary.
 *
 * Method (sources are web pages; cited by title and section):
 *  - "Shrinking the LLM KV Cache by 8x on CPU: The Engineering Behind AdapTQ",
 *    "The Math Fix": a random sign flip followed by a fast Walsh-Hadamard
 *    transform spreads outlier channels before scalar quantization;
 *    "Engineering the Hot Path": the query is rotated once and keys are scored
 *    from their codes through a small table, never dequantized in the loop.
 *  - "I Ported a Google Research Paper to Apple Silicon" (VeloxQuant-MLX),
 *    "The Core Idea" / "Stage 2": Lloyd-Max codebook for a Gaussian, computed
 *    once; each rotated vector is normalised, its norm kept in fp16, and each
 *    coordinate replaced by the index of its nearest centroid;
 *    "The Bit-Packing Problem": b-bit indices packed LSB-first into bytes.
 *  - "FoveatedKV", "Making it fast": one fused split-K decode dispatch, query
 *    pre-scaled by 1/sqrt(D), online softmax with one exp per score, split
 *    merge; "The VR headset thing": a near tier of exact fp16 tokens plus a far
 *    tier with fp8-E4M3 keys and 4-bit values, sharing one softmax.
 *
 * Definitions used throughout:
 *   d      head dimension (64, 128 or 256)
 *   s      sign vector in {-1,+1}^d (int8), shared by keys, values and queries
 *   H      d x d Sylvester Hadamard matrix, H[i][j] = (-1)^popcount(i & j)
 *   R      = H diag(s) / sqrt(d)   (orthonormal rotation)
 *   c      Lloyd-Max centroid table for N(0, 1/d): 2^b float32 values, ascending
 *   row    packed codes of one vector: d*b/8 bytes, code j in stream bits
 *          [b*j, b*j+b), least significant bit first (even j = low nibble at 4 bits)
 *
 * Lloyd-Max codec of a vector x (keys and values):
 *   z = H (s * x);   norm = RNE_fp16(||x||);
 *   code_j = #{ i : z_j >= m_i * sqrt(d) * ||x|| },  m_i = (c_i + c_{i+1})/2
 *   (ties to the upper cell; a zero vector gets norm 0 and code 2^(b-1));
 *   reconstruction in the rotated domain: norm * c[code_j].
 * fp8 key codec (far tier): e_j = E4M3FN(RNE, saturating at +-448)((R x)_j),
 *   no scale, no norm.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_EINVAL = 1,        /* null pointer, bad size, misaligned buffer, bad enum */
  KVQ_EUNSUPPORTED = 2,  /* valid but not built: head_dim / format / GQA group combination */
  KVQ_ERANGE = 3,        /* token positions outside the cache capacity */
  KVQ_EHIP = 4           /* the HIP runtime reported an error at launch */
} kvq_status;

typedef enum { KVQ_F32 = 0, KVQ_F16 = 1 } kvq_dtype;

/* Code formats.  KVQ_LM2/3/4: b-bit Lloyd-Max codes + fp16 norm per vector.
 * KVQ_FP8_E4M3: rotated coordinates in OCP E4M3FN, one byte each, no norm
 * (far-tier keys only). */
typedef enum { KVQ_LM2 = 2, KVQ_LM3 = 3, KVQ_LM4 = 4, KVQ_FP8_E4M3 = 8 } kvq_format;

/* A compressed cache for one layer.  All pointers are device memory owned by
 * the caller and must stay valid while work using them is in flight.
 * Layouts (row-major, innermost last):
 *   k_codes  [batch][kv_heads][capacity][kvq_row_bytes(k_format, head_dim)]
 *   k_norms  [batch][kv_heads][capacity]   fp16 bits (unused, may be NULL, for FP8)
 *   v_codes, v_norms: same with v_format (v_format must be a Lloyd-Max format)
 *   signs    [head_dim] int8, each +1 or -1
 *   k_centroids, v_centroids [2^bits] float32 (the table kvq_lloyd_max fills);
 *            k_centroids is unused (may be NULL) for FP8 keys
 *   near_k, near_v  two-tier caches only: [batch][kv_heads][near_len][head_dim]
 *            fp16 bits in the original (unrotated) domain; NULL with near_len 0
 *   outlier stream of the keys ("Outlier Two-Stream Cache"), Lloyd-Max keys
 *   only, outlier_count 0 (off) or 8:
 *     outlier_idx    [batch][kv_heads][8] int32 channel indices, ascending
 *                    (kvq_calibrate_outliers fills them)
 *     outlier_codes  [batch][kv_heads][capacity][8] int8
 *     outlier_scales [batch][kv_heads][capacity] float32
 *   With the stream on, kvq_quantize_append zeroes those channels of every
 *   key before the rotation codec and stores them as int8 codes with the
 *   per-token scale RN_fp32(max |x_o| / 127) (code = nearest integer of
 *   x_o / scale, ties to even, zero scale gives zero codes); attention adds
 *   q[idx] . (code * scale) / sqrt(d) to every far-tier score.
 *   QJL residual sketch of the keys ("Stage 3: QJL Residual Correction",
 *   "Memory Layout"), Lloyd-Max keys only, not together with the outlier
 *   stream; qjl_dim 0 (off) or head_dim (m sketch rows, m = head_dim):
 *     qjl_proj   [head_dim][m] float32, the projection S transposed:
 *                element (j, i) is S[i][j]; caller-drawn (Gaussian entries
 *                make the estimate below unbiased), read-only
 *     qjl_signs  [batch][kv_heads][capacity][m/8] bytes: bit i (LSB-first
 *                stream) is 1 iff S_i . r >= 0, r = R k - n * c[code] the key
 *                codec's rotated-domain residual (float64 on the device)
 *     qjl_norms  [batch][kv_heads][capacity] fp16 bits of ||r||
 *   With the sketch on, attention adds
 *   ||r||_16 sqrt(pi/2)/m sum_i (2 z_i - 1) (S_i . R q) / sqrt(d) to every
 *   far-tier score, an estimate of the query's product with the residual
 *   that is unbiased over Gaussian S.  A key whose fp16 norm overflows
 *   (||k|| >= 65520) has no defined residual; its sketch bits and residual
 *   norm are unspecified.
 * Code, norm and sign buffers must be 16-byte aligned and capacity a multiple of 16. */
typedef struct kvq_cache {
  int32_t batch;
  int32_t kv_heads;
  int32_t head_dim;
  int32_t capacity;
  int32_t k_format;          /* kvq_format */
  int32_t v_format;          /* kvq_format */
  void *k_codes;
  uint16_t *k_norms;
  void *v_codes;
  uint16_t *v_norms;
  const int8_t *signs;
  const float *k_centroids;
  const float *v_centroids;
  const uint16_t *near_k;
  const uint16_t *near_v;
  int32_t near_len;
  int32_t outlier_count;     /* 0 or 8 */
  const int32_t *outlier_idx;
  int8_t *outlier_codes;
  float *outlier_scales;
  int32_t qjl_dim;           /* 0 or head_dim */
  const float *qjl_proj;
  uint8_t *qjl_signs;
  uint16_t *qjl_norms;
} kvq_cache;

/* Bytes of one packed row ("The Bit-Packing Problem"): head_dim*bits/8 for
 * Lloyd-Max formats, head_dim for FP8.  Returns 0 for an invalid format or a
 * head_dim that is not 64, 128 or 256. */
size_t kvq_row_bytes(int32_t format, int32_t head_dim);

/* Lloyd-Max centroids for N(0, 1/head_dim) with 2^bits levels ("The Core
 * Idea": boundaries at centroid midpoints, each centroid the conditional mean
 * of its cell; computed once).  Solves the fixed point for N(0,1) in double
 * precision, divides by sqrt(head_dim) and rounds to float32 (nearest-even).
 * centroids_host: host array of 2^bits floats, filled ascending.
 * bits in {1,2,3,4}; KVQ_EINVAL otherwise or on NULL. */
kvq_status kvq_lloyd_max(int32_t bits, int32_t head_dim, float *centroids_host);

/* Seeded Rademacher signs ("Stage 1: Random Rotation": r is a random +-1
 * vector; the builder takes a seed).  Generator: SplitMix64 (Steele, Lea and
 * Flood, 2014) started at `seed`; s_j = +1 if the top bit of the j-th output
 * is 0, else -1.  signs_host: host array of head_dim int8. */
kvq_status kvq_make_signs(uint64_t seed, int32_t head_dim, int8_t *signs_host);

/* Quantize-on-append ("The Math Fix", "Stage 2", "The Bit-Packing Problem"):
 * encodes n_new new key and value vectors per (batch, kv head) and writes them
 * at token positions [start_pos, start_pos + n_new) of the cache.
 *   k, v   device [batch][kv_heads][n_new][head_dim] in `dtype` (KVQ_F32/F16)
 * Keys use cache->k_format (Lloyd-Max or FP8), values cache->v_format.
 * Errors: KVQ_EINVAL (NULL, bad dtype/format, n_new < 0), KVQ_ERANGE
 * (start_pos < 0 or start_pos + n_new > capacity), KVQ_EUNSUPPORTED,
 * KVQ_EHIP.  n_new == 0 launches nothing and returns KVQ_OK. */
kvq_status kvq_quantize_append(const kvq_cache *cache, const void *k, const void *v,
                               int32_t dtype, int32_t start_pos, int32_t n_new,
                               hipStream_t stream);

/* Fused split-K GQA decode attention on the compressed cache ("Engineering
 * the Hot Path"; "Making it fast").  For each batch entry b and query head h
 * (KV head h / (q_heads / kv_heads)):
 *   far splits:  tokens [0, seq_len) of the code buffers, cut into num_splits
 *                contiguous chunks of C = ceil(seq_len / num_splits) tokens
 *                rounded up to a multiple of 32 (split s covers
 *                [s*C, min((s+1)*C, seq_len)); trailing splits may be empty);
 *                scores s_t = (R q) . khat_t / sqrt(d) with khat the rotated
 *                reconstruction; values accumulated in the rotated domain.
 *   near splits: tokens [0, near_len) of near_k/near_v cut the same way into
 *                num_near_splits chunks, scored in the original domain.
 * Each split writes its softmax state:
 *   part_ml [batch][q_heads][num_near_splits + num_splits][2] float32:
 *           m = max score of the chunk (natural-log units, -inf if empty),
 *           l = sum_t exp(s_t - m)
 *   part_o  [batch][q_heads][num_near_splits + num_splits][head_dim] float32:
 *           sum_t exp(s_t - m) * vhat_t / l   (0 if empty); near splits first,
 *           original domain; far splits rotated domain.
 *   q       device [batch][q_heads][head_dim] in q_dtype (KVQ_F32/F16),
 *           original domain, 16-byte aligned.
 * part_o and part_ml must be 16-byte aligned.
 * The softmax scale 1/sqrt(d) is applied inside.  num_near_splits must be 0
 * unless the cache has a near tier.  Errors: KVQ_EINVAL, KVQ_ERANGE
 * (seq_len > capacity), KVQ_EUNSUPPORTED (GQA group or format combination not
 * built), KVQ_EHIP. */
kvq_status kvq_decode_attention(const kvq_cache *cache, const void *q, int32_t q_dtype,
                                int32_t q_heads, int32_t seq_len, int32_t num_splits,
                                int32_t num_near_splits, float *part_o, float *part_ml,
                                hipStream_t stream);

/* kvq_decode_attention with the far tier's score gate and spike flags
 * ("FoveatedKV", "Making it fast": value loading skipped for a token whose
 * score falls below e^-16 of the reference; far-tier tokens that outscore the
 * near tier detected during the softmax).  Same arguments, layout and
 * partial outputs as kvq_decode_attention, plus:
 *   gate_ref    device float [batch][q_heads] or NULL: far token t adds
 *               nothing to head h's values when s_t < gate_ref[b][h] - 16
 *               (natural-log score units, those of part_ml's m; a previous
 *               step's log-sum-exp is a natural reference); its weight still
 *               counts in l.  Near-tier tokens are never gated.
 *   spike_ref   device float [batch][q_heads] or NULL: bit t % 32 of
 *               spike_bits[b][h][t / 32] is or-ed to 1 when far token
 *               t < seq_len scores s_t > spike_ref[b][h];
 *   spike_bits  device uint32 [batch][q_heads][ceil(seq_len / 32)], zeroed by
 *               the caller before the call (bits are or-ed in); required
 *               exactly when spike_ref is given.
 * The results do not depend on how rows are fetched; for speed, each wave
 * requests value rows together with the keys until a block of its tokens
 * has one gated for every head, and from then on skips the value rows of
 * such tokens, so a pass that gates nothing costs about an ungated one.
 * At least one of gate_ref and spike_ref must be given.  All three are
 * caller-owned and 4-byte aligned.  Caches with an outlier stream or a QJL
 * sketch are not served (KVQ_EUNSUPPORTED).  Served by the VALU kernel for every
 * format (query groups G = 1, 2, 4; 3-bit codes at G = 1).  Errors as
 * kvq_decode_attention, and KVQ_EINVAL for a missing or unpaired reference. */
kvq_status kvq_decode_attention_gated(const kvq_cache *cache, const void *q, int32_t q_dtype,
                                      int32_t q_heads, int32_t seq_len, int32_t num_splits,
                                      int32_t num_near_splits, const float *gate_ref,
                                      const float *spike_ref, uint32_t *spike_bits, float *part_o,
                                      float *part_ml, hipStream_t stream);

/* Outlier-channel calibration for the key outlier stream ("I Ported a Google
 * Research Paper to Apple Silicon", "Outlier Two-Stream Cache": calibration on
 * the first tokens, then detection).  For every (b, KV head), the 8 channels
 * with the largest population variance over keys[.., 0..n_tokens, ..]
 * (float64: the mean first, then the mean squared deviation; ties to the
 * lower channel) are written ascending to idx_out.
 *   keys     device [batch][kv_heads][n_tokens][head_dim] in dtype
 *            (KVQ_F32/F16), 16-byte aligned: the context's first tokens;
 *   idx_out  device int32 [batch][kv_heads][8], 16-byte aligned (normally
 *            the cache's outlier_idx).
 * The cache supplies the shape only.  Errors: KVQ_EINVAL (NULL, misaligned,
 * n_tokens < 1, bad dtype or cache), KVQ_EUNSUPPORTED, KVQ_EHIP. */
kvq_status kvq_calibrate_outliers(const kvq_cache *cache, const void *keys, int32_t dtype,
                                  int32_t n_tokens, int32_t *idx_out, hipStream_t stream);

/* Name of the attention kernel kvq_decode_attention launches for this cache,
 * query-head count and split counts (for profiles and reports): a static
 * string, or NULL if the arguments are invalid (num_splits < 1 among them)
 * or the call would return KVQ_EUNSUPPORTED (kvq_last_error then says why).
 * A near tier beside 4-bit codes at head_dim 128 shares the pair-table
 * launch when the near splits are at most the far splits and the far splits
 * fit one work-group per compute unit ("attend_pair_kernel"); a near tier
 * beside other codes that a pair-table kernel covers is served by two
 * launches on the stream (near splits, then far splits), named
 * "<far kernel>+attend_kernel". */
const char *kvq_decode_attention_kernel(const kvq_cache *cache, int32_t q_heads, int32_t num_splits,
                                        int32_t num_near_splits);

/* Split merge and the single inverse rotation ("Making it fast": split-K
 * partial softmax states merged; rotated-domain values mapped back once):
 *   M = max_s m_s,  w_s = l_s exp(m_s - M),  W = sum_s w_s,
 *   out = ( sum_{near s} w_s o_s + R^T sum_{far s} w_s o_s ) / W
 *   out [batch][q_heads][head_dim] float32 (original domain);
 *   lse [batch][q_heads] float32 = M + log W, or NULL to skip.
 * Partials as written by kvq_decode_attention with the same split counts
 * (part_o 16-byte aligned).
 * Errors: KVQ_EINVAL, KVQ_EHIP. */
kvq_status kvq_merge(const kvq_cache *cache, const float *part_o, const float *part_ml,
                     int32_t q_heads, int32_t num_splits, int32_t num_near_splits,
                     float *out, float *lse, hipStream_t stream);

/* Decode attention and split merge in one call ("FoveatedKV", "Making it
 * fast": the fused split-K pass over both tiers, then the merge of the split
 * states with the single inverse rotation): kvq_decode_attention into split
 * partials held in `workspace`, then kvq_merge into out/lse, two launches on
 * `stream`.  Arguments, layouts and results as those two calls;
 *   workspace        caller-owned device memory, 16-byte aligned, at least
 *                    kvq_decode_workspace_bytes(batch, q_heads, num_splits,
 *                    num_near_splits, head_dim) bytes; scratch only (its
 *                    contents after the call are unspecified), so it must not
 *                    be used by other work in flight on other streams.
 * Errors: those of the two calls, and KVQ_EINVAL for a NULL, misaligned or
 * too small workspace. */
kvq_status kvq_decode(const kvq_cache *cache, const void *q, int32_t q_dtype, int32_t q_heads, int32_t seq_len,
                      int32_t num_splits, int32_t num_near_splits, void *workspace, size_t workspace_bytes,
                      float *out, float *lse, hipStream_t stream);

/* Bytes of the workspace kvq_decode needs (0 for an invalid shape). */
size_t kvq_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t num_splits, int32_t num_near_splits,
                                  int32_t head_dim);

/* kvq_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the split partials go to a fixed device scratch
 * array the library holds, one per GPU it runs on, until the process ends
 * (16 MiB: for example batch 16, 64 query heads, 32 splits at head_dim 128).
 * The call itself allocates nothing; the first call on a device resolves that
 * device's array once.  Calls that overlap on one GPU (several streams,
 * threads) share the array and race: serialise them.  Calls whose partials
 * need more than the array, kvq_decode_workspace_bytes(...) > 16 MiB, return
 * KVQ_ERANGE.  Other arguments and errors as kvq_decode. */
kvq_status kvq_decode_noalloc(const kvq_cache *cache, const void *q, int32_t q_dtype, int32_t q_heads,
                              int32_t seq_len, int32_t num_splits, int32_t num_near_splits, float *out, float *lse,
                              hipStream_t stream);

/* Floats in part_o for the given shape (part_ml needs 2/head_dim of that). */
size_t kvq_partials_floats(int32_t batch, int32_t q_heads, int32_t total_splits,
                           int32_t head_dim);

/* Static text for a status code. */
const char *kvq_status_string(kvq_status status);

/* Human-readable reason for the last non-OK status returned on this thread
 * (empty string if none). */
const char *kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
