// extern "C" entry points of libkvq: host-side validation, then one launch on
// the caller's stream.  Nothing here allocates or synchronises.
#include <stdint.h>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool is_lm(int32_t f) { return f == KVQ_LM2 || f == KVQ_LM3 || f == KVQ_LM4; }

kvq_status check_cache(const kvq_cache *c, const char *fn) {
  using kvq::fail;
  if (!c) return fail(KVQ_EINVAL, "%s: cache is NULL", fn);
  if (c->batch < 1 || c->kv_heads < 1 || c->capacity < 0)
    return fail(KVQ_EINVAL, "%s: bad cache shape batch=%d kv_heads=%d capacity=%d", fn, c->batch, c->kv_heads,
                c->capacity);
  if (!kvq::valid_head_dim(c->head_dim))
    return fail(KVQ_EUNSUPPORTED, "%s: head_dim=%d (built: 64, 128, 256)", fn, c->head_dim);
  if (!kvq::format_bits(c->k_format)) return fail(KVQ_EINVAL, "%s: bad k_format %d", fn, c->k_format);
  if (!is_lm(c->v_format)) return fail(KVQ_EINVAL, "%s: v_format %d is not a Lloyd-Max format", fn, c->v_format);
  if (!c->k_codes || !c->v_codes || !c->v_norms || !c->signs || !c->v_centroids)
    return fail(KVQ_EINVAL, "%s: NULL cache buffer", fn);
  if (is_lm(c->k_format) && (!c->k_norms || !c->k_centroids))
    return fail(KVQ_EINVAL, "%s: Lloyd-Max keys need k_norms and k_centroids", fn);
  if (!aligned(c->k_codes, 16) || !aligned(c->v_codes, 16))
    return fail(KVQ_EINVAL, "%s: code buffers must be 16-byte aligned", fn);
  if (!aligned(c->k_norms, 16) || !aligned(c->v_norms, 16) || !aligned(c->signs, 16))
    return fail(KVQ_EINVAL, "%s: norms and signs must be 16-byte aligned", fn);
  if (c->capacity % 16) return fail(KVQ_EINVAL, "%s: capacity %d is not a multiple of 16", fn, c->capacity);
  if (c->near_len < 0 || (c->near_len > 0 && (!c->near_k || !c->near_v)))
    return fail(KVQ_EINVAL, "%s: near tier needs near_k and near_v", fn);
  if (c->near_len > 0 && (!aligned(c->near_k, 16) || !aligned(c->near_v, 16)))
    return fail(KVQ_EINVAL, "%s: near tier buffers must be 16-byte aligned", fn);
  if (c->outlier_count != 0 && c->outlier_count != kvq::kOutlierCount)
    return fail(KVQ_EUNSUPPORTED, "%s: outlier_count %d (built: 0, %d)", fn, c->outlier_count, kvq::kOutlierCount);
  if (c->outlier_count) {
    if (!is_lm(c->k_format)) return fail(KVQ_EUNSUPPORTED, "%s: the outlier stream needs Lloyd-Max keys", fn);
    if (!c->outlier_idx || !c->outlier_codes || !c->outlier_scales)
      return fail(KVQ_EINVAL, "%s: outlier stream buffers are NULL", fn);
    if (!aligned(c->outlier_idx, 16) || !aligned(c->outlier_codes, 16) || !aligned(c->outlier_scales, 16))
      return fail(KVQ_EINVAL, "%s: outlier stream buffers must be 16-byte aligned", fn);
  }
  if (c->qjl_dim != 0 && c->qjl_dim != c->head_dim)
    return fail(KVQ_EUNSUPPORTED, "%s: qjl_dim %d (built: 0, head_dim)", fn, c->qjl_dim);
  if (c->qjl_dim) {
    if (!is_lm(c->k_format)) return fail(KVQ_EUNSUPPORTED, "%s: the QJL sketch needs Lloyd-Max keys", fn);
    if (c->outlier_count) return fail(KVQ_EUNSUPPORTED, "%s: QJL sketch and outlier stream together", fn);
    if (!c->qjl_proj || !c->qjl_signs || !c->qjl_norms) return fail(KVQ_EINVAL, "%s: QJL buffers are NULL", fn);
    if (!aligned(c->qjl_proj, 16) || !aligned(c->qjl_signs, 16) || !aligned(c->qjl_norms, 16))
      return fail(KVQ_EINVAL, "%s: QJL buffers must be 16-byte aligned", fn);
  }
  return KVQ_OK;
}

kvq_status hip_status(hipError_t e, const char *fn) {
  if (e != hipSuccess) return kvq::fail(KVQ_EHIP, "%s: %s", fn, hipGetErrorString(e));
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_quantize_append(const kvq_cache *cache, const void *k, const void *v, int32_t dtype,
                               int32_t start_pos, int32_t n_new, hipStream_t stream) {
  const char *fn = "kvq_quantize_append";
  kvq::clear_error();
  kvq_status st = check_cache(cache, fn);
  if (st != KVQ_OK) return st;
  if (dtype != KVQ_F32 && dtype != KVQ_F16) return kvq::fail(KVQ_EINVAL, "%s: dtype %d", fn, dtype);
  if (n_new < 0) return kvq::fail(KVQ_EINVAL, "%s: n_new=%d", fn, n_new);
  if (start_pos < 0 || (int64_t)start_pos + n_new > cache->capacity)
    return kvq::fail(KVQ_ERANGE, "%s: positions [%d, %lld) outside capacity %d", fn, start_pos,
                     (long long)start_pos + n_new, cache->capacity);
  if (n_new == 0) return KVQ_OK;
  if (!k || !v) return kvq::fail(KVQ_EINVAL, "%s: k or v is NULL", fn);
  if (!aligned(k, 16) || !aligned(v, 16)) return kvq::fail(KVQ_EINVAL, "%s: k and v must be 16-byte aligned", fn);
  if ((int64_t)cache->batch * cache->kv_heads * n_new > (1ll << 31) / 64)
    return kvq::fail(KVQ_EINVAL, "%s: too many vectors in one call", fn);
  kvq::AppendArgs a{k, v, dtype == KVQ_F16, cache->batch, cache->kv_heads, cache->head_dim, cache->capacity,
                    start_pos, n_new, cache->k_format, cache->v_format,
                    static_cast<uint8_t *>(cache->k_codes), static_cast<uint8_t *>(cache->v_codes),
                    cache->k_norms, cache->v_norms, cache->signs, cache->k_centroids, cache->v_centroids,
                    cache->outlier_count ? cache->outlier_idx : nullptr, cache->outlier_codes, cache->outlier_scales};
  if (cache->qjl_dim) {
    a.qjl_proj = cache->qjl_proj;
    a.qjl_signs = cache->qjl_signs;
    a.qjl_norms = cache->qjl_norms;
  }
  bool ok = true;
  hipError_t e = kvq::launch_append(a, stream, &ok);
  if (!ok) return kvq::fail(KVQ_EUNSUPPORTED, "%s: format combination not built", fn);
  return hip_status(e, fn);
}

namespace {

// Validation shared by the decode-attention calls; fills the launch arguments.
kvq_status attend_args(const char *fn, const kvq_cache *cache, const void *q, int32_t q_dtype, int32_t q_heads,
                       int32_t seq_len, int32_t num_splits, int32_t num_near_splits, float *part_o, float *part_ml,
                       kvq::AttendArgs *out) {
  kvq_status st = check_cache(cache, fn);
  if (st != KVQ_OK) return st;
  if (!q || !part_o || !part_ml) return kvq::fail(KVQ_EINVAL, "%s: NULL q or partial buffer", fn);
  if (!aligned(q, 16)) return kvq::fail(KVQ_EINVAL, "%s: q must be 16-byte aligned", fn);
  if (!aligned(part_o, 16) || !aligned(part_ml, 16))
    return kvq::fail(KVQ_EINVAL, "%s: partial buffers must be 16-byte aligned", fn);
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_F16) return kvq::fail(KVQ_EINVAL, "%s: q_dtype %d", fn, q_dtype);
  if (q_heads < 1 || q_heads % cache->kv_heads)
    return kvq::fail(KVQ_EINVAL, "%s: q_heads=%d not a multiple of kv_heads=%d", fn, q_heads, cache->kv_heads);
  if (seq_len < 0) return kvq::fail(KVQ_EINVAL, "%s: seq_len=%d", fn, seq_len);
  if (seq_len > cache->capacity)
    return kvq::fail(KVQ_ERANGE, "%s: seq_len=%d > capacity=%d", fn, seq_len, cache->capacity);
  if (num_splits < 1 || num_splits > 65535 || num_near_splits < 0 || num_near_splits > 65535)
    return kvq::fail(KVQ_EINVAL, "%s: splits far=%d near=%d", fn, num_splits, num_near_splits);
  if (num_near_splits > 0 && cache->near_len == 0)
    return kvq::fail(KVQ_EINVAL, "%s: near splits requested but the cache has no near tier", fn);
  if (num_near_splits == 0 && cache->near_len > 0)
    return kvq::fail(KVQ_EINVAL, "%s: the cache has a near tier; give it at least one split", fn);
  if ((int64_t)cache->batch * cache->kv_heads > 65535)
    return kvq::fail(KVQ_EINVAL, "%s: batch*kv_heads above 65535", fn);
  *out = kvq::AttendArgs{q, q_dtype == KVQ_F16, cache->batch, cache->kv_heads, q_heads, cache->head_dim,
                         cache->capacity, seq_len, num_splits, num_near_splits, cache->near_len, cache->k_format,
                         cache->v_format, static_cast<const uint8_t *>(cache->k_codes),
                         static_cast<const uint8_t *>(cache->v_codes), cache->k_norms, cache->v_norms, cache->signs,
                         cache->k_centroids, cache->v_centroids, cache->near_k, cache->near_v, part_o, part_ml};
  if (cache->outlier_count) {
    out->outlier_idx = cache->outlier_idx;
    out->outlier_codes = cache->outlier_codes;
    out->outlier_scales = cache->outlier_scales;
  }
  if (cache->qjl_dim) {
    out->qjl_proj = cache->qjl_proj;
    out->qjl_signs = cache->qjl_signs;
    out->qjl_norms = cache->qjl_norms;
  }
  return KVQ_OK;
}

kvq_status attend_status(const char *fn, const kvq_cache *cache, int32_t q_heads, bool ok, hipError_t e) {
  if (!ok)
    return kvq::fail(KVQ_EUNSUPPORTED, "%s: group %d with formats (%d,%d) at head_dim %d not built", fn,
                     q_heads / cache->kv_heads, cache->k_format, cache->v_format, cache->head_dim);
  return hip_status(e, fn);
}

}  // namespace

kvq_status kvq_decode_attention(const kvq_cache *cache, const void *q, int32_t q_dtype, int32_t q_heads,
                                int32_t seq_len, int32_t num_splits, int32_t num_near_splits, float *part_o,
                                float *part_ml, hipStream_t stream) {
  const char *fn = "kvq_decode_attention";
  kvq::clear_error();
  kvq::AttendArgs a;
  const kvq_status st = attend_args(fn, cache, q, q_dtype, q_heads, seq_len, num_splits, num_near_splits, part_o,
                                    part_ml, &a);
  if (st != KVQ_OK) return st;
  bool ok = true;
  const hipError_t e = kvq::launch_attend(a, stream, &ok);
  return attend_status(fn, cache, q_heads, ok, e);
}

kvq_status kvq_decode_attention_gated(const kvq_cache *cache, const void *q, int32_t q_dtype, int32_t q_heads,
                                      int32_t seq_len, int32_t num_splits, int32_t num_near_splits,
                                      const float *gate_ref, const float *spike_ref, uint32_t *spike_bits,
                                      float *part_o, float *part_ml, hipStream_t stream) {
  const char *fn = "kvq_decode_attention_gated";
  kvq::clear_error();
  kvq::AttendArgs a;
  const kvq_status st = attend_args(fn, cache, q, q_dtype, q_heads, seq_len, num_splits, num_near_splits, part_o,
                                    part_ml, &a);
  if (st != KVQ_OK) return st;
  if (!gate_ref && !spike_ref) return kvq::fail(KVQ_EINVAL, "%s: neither gate_ref nor spike_ref given", fn);
  if (cache->outlier_count || cache->qjl_dim)
    return kvq::fail(KVQ_EUNSUPPORTED, "%s: the gated pass is not built for an outlier stream or QJL sketch", fn);
  if ((spike_ref == nullptr) != (spike_bits == nullptr))
    return kvq::fail(KVQ_EINVAL, "%s: spike_ref and spike_bits go together", fn);
  if (!aligned(gate_ref, 4) || !aligned(spike_ref, 4) || !aligned(spike_bits, 4))
    return kvq::fail(KVQ_EINVAL, "%s: references and flag words must be 4-byte aligned", fn);
  a.gate_ref = gate_ref;
  a.spike_ref = spike_ref;
  a.spike_bits = spike_bits;
  bool ok = true;
  const hipError_t e = kvq::launch_attend_gated(a, stream, &ok);
  return attend_status(fn, cache, q_heads, ok, e);
}

kvq_status kvq_calibrate_outliers(const kvq_cache *cache, const void *keys, int32_t dtype, int32_t n_tokens,
                                  int32_t *idx_out, hipStream_t stream) {
  const char *fn = "kvq_calibrate_outliers";
  kvq::clear_error();
  const kvq_status st = check_cache(cache, fn);
  if (st != KVQ_OK) return st;
  if (!keys || !idx_out) return kvq::fail(KVQ_EINVAL, "%s: NULL keys or idx_out", fn);
  if (dtype != KVQ_F32 && dtype != KVQ_F16) return kvq::fail(KVQ_EINVAL, "%s: dtype %d", fn, dtype);
  if (n_tokens < 1) return kvq::fail(KVQ_EINVAL, "%s: n_tokens=%d", fn, n_tokens);
  if (!aligned(keys, 16) || !aligned(idx_out, 16))
    return kvq::fail(KVQ_EINVAL, "%s: keys and idx_out must be 16-byte aligned", fn);
  if ((int64_t)cache->batch * cache->kv_heads > (1ll << 31) - 1) return kvq::fail(KVQ_EINVAL, "%s: grid too large", fn);
  return hip_status(kvq::launch_calibrate(keys, dtype == KVQ_F16, cache->batch, cache->kv_heads, cache->head_dim,
                                          n_tokens, idx_out, stream), fn);
}

const char *kvq_decode_attention_kernel(const kvq_cache *cache, int32_t q_heads, int32_t num_splits,
                                        int32_t num_near_splits) {
  kvq::clear_error();
  if (check_cache(cache, "kvq_decode_attention_kernel") != KVQ_OK) return nullptr;
  if (q_heads < 1 || q_heads % cache->kv_heads) return nullptr;
  if (num_splits < 1 || num_near_splits < 0) {
    kvq::fail(KVQ_EINVAL, "kvq_decode_attention_kernel: num_splits %d, num_near_splits %d", num_splits, num_near_splits);
    return nullptr;
  }
  kvq::AttendArgs a{nullptr, 0, cache->batch, cache->kv_heads, q_heads, cache->head_dim, cache->capacity, 0, num_splits,
                    num_near_splits, cache->near_len, cache->k_format, cache->v_format,
                    static_cast<const uint8_t *>(cache->k_codes), static_cast<const uint8_t *>(cache->v_codes),
                    cache->k_norms, cache->v_norms, cache->signs, cache->k_centroids, cache->v_centroids,
                    cache->near_k, cache->near_v, nullptr, nullptr};
  if (cache->outlier_count) a.outlier_idx = cache->outlier_idx;
  if (cache->qjl_dim) a.qjl_proj = cache->qjl_proj;
  const char *name = kvq::attend_kernel_name(a);
  if (!name)
    kvq::fail(KVQ_EUNSUPPORTED, "kvq_decode_attention_kernel: group %d with formats (%d,%d) at head_dim %d not built",
              q_heads / cache->kv_heads, cache->k_format, cache->v_format, cache->head_dim);
  return name;
}

}  // extern "C"

namespace {

// Byte layout of a decode workspace: part_o, then part_ml at the next
// 16-byte boundary.
size_t ws_part_o_bytes(int32_t batch, int32_t q_heads, int32_t total_splits, int32_t head_dim) {
  return ((size_t)batch * q_heads * total_splits * head_dim * 4 + 15) / 16 * 16;
}

size_t ws_bytes(int32_t batch, int32_t q_heads, int32_t total_splits, int32_t head_dim) {
  return ws_part_o_bytes(batch, q_heads, total_splits, head_dim) + (size_t)batch * q_heads * total_splits * 2 * 4;
}

kvq_status merge_launch(const char *fn, const kvq_cache *cache, const float *part_o, const float *part_ml,
                        int32_t q_heads, int32_t num_splits, int32_t num_near_splits, float *out, float *lse,
                        hipStream_t stream);

// Attention into the partials at `ws`, then the merge into out/lse.
kvq_status decode_into(const char *fn, const kvq_cache *cache, const void *q, int32_t q_dtype, int32_t q_heads,
                       int32_t seq_len, int32_t num_splits, int32_t num_near_splits, uint8_t *ws, float *out,
                       float *lse, hipStream_t stream) {
  float *part_o = reinterpret_cast<float *>(ws);
  float *part_ml = reinterpret_cast<float *>(
      ws + ws_part_o_bytes(cache->batch, q_heads, num_splits + num_near_splits, cache->head_dim));
  kvq::AttendArgs a;
  kvq_status st = attend_args(fn, cache, q, q_dtype, q_heads, seq_len, num_splits, num_near_splits, part_o, part_ml,
                              &a);
  if (st != KVQ_OK) return st;
  if (!out) return kvq::fail(KVQ_EINVAL, "%s: out is NULL", fn);
  bool ok = true;
  const hipError_t e = kvq::launch_attend(a, stream, &ok);
  st = attend_status(fn, cache, q_heads, ok, e);
  if (st != KVQ_OK) return st;
  return merge_launch(fn, cache, part_o, part_ml, q_heads, num_splits, num_near_splits, out, lse, stream);
}

}  // namespace

extern "C" {

size_t kvq_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t num_splits, int32_t num_near_splits,
                                  int32_t head_dim) {
  if (batch < 1 || q_heads < 1 || num_splits < 1 || num_near_splits < 0 || !kvq::valid_head_dim(head_dim)) return 0;
  return ws_bytes(batch, q_heads, num_splits + num_near_splits, head_dim);
}

kvq_status kvq_decode(const kvq_cache *cache, const void *q, int32_t q_dtype, int32_t q_heads, int32_t seq_len,
                      int32_t num_splits, int32_t num_near_splits, void *workspace, size_t workspace_bytes,
                      float *out, float *lse, hipStream_t stream) {
  const char *fn = "kvq_decode";
  kvq::clear_error();
  kvq_status st = check_cache(cache, fn);
  if (st != KVQ_OK) return st;
  if (q_heads < 1 || num_splits < 1 || num_near_splits < 0)
    return kvq::fail(KVQ_EINVAL, "%s: q_heads=%d splits far=%d near=%d", fn, q_heads, num_splits, num_near_splits);
  if (!workspace || !aligned(workspace, 16)) return kvq::fail(KVQ_EINVAL, "%s: workspace NULL or not 16-byte aligned", fn);
  const size_t need = ws_bytes(cache->batch, q_heads, num_splits + num_near_splits, cache->head_dim);
  if (workspace_bytes < need)
    return kvq::fail(KVQ_EINVAL, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
  return decode_into(fn, cache, q, q_dtype, q_heads, seq_len, num_splits, num_near_splits,
                     static_cast<uint8_t *>(workspace), out, lse, stream);
}

kvq_status kvq_decode_noalloc(const kvq_cache *cache, const void *q, int32_t q_dtype, int32_t q_heads,
                              int32_t seq_len, int32_t num_splits, int32_t num_near_splits, float *out, float *lse,
                              hipStream_t stream) {
  const char *fn = "kvq_decode_noalloc";
  kvq::clear_error();
  kvq_status st = check_cache(cache, fn);
  if (st != KVQ_OK) return st;
  if (q_heads < 1 || num_splits < 1 || num_near_splits < 0)
    return kvq::fail(KVQ_EINVAL, "%s: q_heads=%d splits far=%d near=%d", fn, q_heads, num_splits, num_near_splits);
  const size_t need = ws_bytes(cache->batch, q_heads, num_splits + num_near_splits, cache->head_dim);
  if (need > kvq::kNoAllocScratchBytes)
    return kvq::fail(KVQ_ERANGE, "%s: the split partials need %zu bytes; the fixed scratch holds %zu", fn, need,
                     (size_t)kvq::kNoAllocScratchBytes);
  void *ws = nullptr;
  const hipError_t e = kvq::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, fn);
  return decode_into(fn, cache, q, q_dtype, q_heads, seq_len, num_splits, num_near_splits, static_cast<uint8_t *>(ws),
                     out, lse, stream);
}

kvq_status kvq_merge(const kvq_cache *cache, const float *part_o, const float *part_ml, int32_t q_heads,
                     int32_t num_splits, int32_t num_near_splits, float *out, float *lse, hipStream_t stream) {
  kvq::clear_error();
  return merge_launch("kvq_merge", cache, part_o, part_ml, q_heads, num_splits, num_near_splits, out, lse, stream);
}

}  // extern "C"

namespace {

kvq_status merge_launch(const char *fn, const kvq_cache *cache, const float *part_o, const float *part_ml,
                        int32_t q_heads, int32_t num_splits, int32_t num_near_splits, float *out, float *lse,
                        hipStream_t stream) {
  if (!cache) return kvq::fail(KVQ_EINVAL, "%s: cache is NULL", fn);
  if (!kvq::valid_head_dim(cache->head_dim))
    return kvq::fail(KVQ_EUNSUPPORTED, "%s: head_dim=%d", fn, cache->head_dim);
  if (!part_o || !part_ml || !out || !cache->signs) return kvq::fail(KVQ_EINVAL, "%s: NULL buffer", fn);
  if (!aligned(part_o, 16)) return kvq::fail(KVQ_EINVAL, "%s: part_o must be 16-byte aligned", fn);
  if (cache->batch < 1 || q_heads < 1 || num_splits < 0 || num_near_splits < 0 || num_splits + num_near_splits < 1)
    return kvq::fail(KVQ_EINVAL, "%s: bad shape", fn);
  if ((int64_t)cache->batch * q_heads > (1ll << 31) - 1) return kvq::fail(KVQ_EINVAL, "%s: grid too large", fn);
  kvq::MergeArgs a{part_o, part_ml, cache->batch, q_heads, cache->head_dim, num_splits, num_near_splits,
                   cache->signs, out, lse};
  bool ok = true;
  hipError_t e = kvq::launch_merge(a, stream, &ok);
  if (!ok) return kvq::fail(KVQ_EUNSUPPORTED, "%s: head_dim not built", fn);
  return hip_status(e, fn);
}

}  // namespace
