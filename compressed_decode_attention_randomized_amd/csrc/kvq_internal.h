// Internal declarations shared by the libkvq translation units.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "kvq.h"

namespace kvq {

constexpr int kOutlierCount = 8;   // channels of the key outlier stream
constexpr size_t kNoAllocScratchBytes = 16u << 20;   // fixed device scratch of kvq_decode_noalloc

// This device's copy of the fixed scratch (resolved once per device).
hipError_t noalloc_scratch(void **ptr);

kvq_status fail(kvq_status st, const char *fmt, ...);
void clear_error();
bool valid_head_dim(int32_t d);
int format_bits(int32_t f);

// Quantize-on-append launch (validated arguments).
struct AppendArgs {
  const void *k, *v;        // [B][Hkv][n_new][d]
  int32_t in_f16;           // 1: fp16 input, 0: fp32
  int32_t batch, kv_heads, head_dim, capacity, start_pos, n_new;
  int32_t k_format, v_format;
  uint8_t *k_codes, *v_codes;
  uint16_t *k_norms, *v_norms;
  const int8_t *signs;
  const float *k_centroids, *v_centroids;
  // key outlier stream (NULL idx: off): channels [B][Hkv][8], codes
  // [B][Hkv][capacity][8], scales [B][Hkv][capacity]
  const int32_t *outlier_idx = nullptr;
  int8_t *outlier_codes = nullptr;
  float *outlier_scales = nullptr;
  // QJL residual sketch of the keys (NULL proj: off; m = head_dim): S^T
  // [d][m] float32, sign bits [B][Hkv][capacity][m/8], fp16 norms [B][Hkv][capacity]
  const float *qjl_proj = nullptr;
  uint8_t *qjl_signs = nullptr;
  uint16_t *qjl_norms = nullptr;
};
hipError_t launch_append(const AppendArgs &a, hipStream_t stream, bool *supported);
// Bulk-throughput variant (Lloyd-Max keys and values, head_dim 64/128/256).
bool fast_append_supported(const AppendArgs &a);
hipError_t launch_append_fast(const AppendArgs &a, hipStream_t stream);
// Bulk variant with one lane per vector (fp16 input, Lloyd-Max or fp8 keys,
// Lloyd-Max values, head_dim 64/128/256, no key side streams).
bool bulk_append_supported(const AppendArgs &a);
hipError_t launch_append_bulk(const AppendArgs &a, hipStream_t stream);

// Decode-attention launch (validated arguments).
struct AttendArgs {
  const void *q;            // [B][Hq][d]
  int32_t q_f16;
  int32_t batch, kv_heads, q_heads, head_dim, capacity, seq_len;
  int32_t num_splits, num_near_splits, near_len;
  int32_t k_format, v_format;
  const uint8_t *k_codes, *v_codes;
  const uint16_t *k_norms, *v_norms;
  const int8_t *signs;
  const float *k_centroids, *v_centroids;
  const uint16_t *near_k, *near_v;
  float *part_o, *part_ml;
  int32_t near_only = 0;    // launch only the near-tier splits (the far ones go to another kernel)
  int32_t gated = 0;        // score gate / spike flags (VALU kernel only)
  const float *gate_ref = nullptr, *spike_ref = nullptr;
  uint32_t *spike_bits = nullptr;
  // key outlier stream (NULL idx: off)
  const int32_t *outlier_idx = nullptr;
  const int8_t *outlier_codes = nullptr;
  const float *outlier_scales = nullptr;
  // QJL residual sketch of the keys (NULL proj: off)
  const float *qjl_proj = nullptr;
  const uint8_t *qjl_signs = nullptr;
  const uint16_t *qjl_norms = nullptr;
};
hipError_t launch_attend(const AttendArgs &a, hipStream_t stream, bool *supported);
// Score-gated attention with spike flags (a.gate_ref / a.spike_ref / a.spike_bits):
// always the VALU kernel.
hipError_t launch_attend_gated(const AttendArgs &a, hipStream_t stream, bool *supported);
// Name of the kernel launch_attend picks for these arguments (for a cache
// with a near tier whose far splits go to a pair-table kernel, the far
// kernel's name followed by "+attend_kernel").
const char *attend_kernel_name(const AttendArgs &a);
// Matrix-core variant (Lloyd-Max 2/4-bit keys and values, no near tier, G <= 8).
bool mfma_attend_supported(const AttendArgs &a);
hipError_t launch_attend_mfma(const AttendArgs &a, hipStream_t stream, bool *supported);
// Pair-table variant (4-bit keys and values, head_dim 128, G <= 8).
// pair_attend_supported: no near tier.  pair_near_supported: with an fp16
// near tier in the same launch (at most as many near splits as far splits,
// one work-group per far split).  For a launch without near splits,
// part_base: far split 0 goes to partial row index part_base of rows that
// hold part_base + num_splits splits (the near-tier splits come first); with
// near splits the rows are laid out that way with part_base = near splits.
bool pair_attend_supported(const AttendArgs &a);
bool pair_near_supported(const AttendArgs &a);
hipError_t launch_attend_pair(const AttendArgs &a, hipStream_t stream, int part_base = 0);
// Two-wave-per-SIMD pair-table variant: head_dim 256 (4-, 2-bit keys and
// values at G <= 8, 3-bit at 2 <= G <= 8), or head_dim 128 with 4-bit codes
// and the key outlier stream, or 3-bit keys beside 4-bit values at
// 2 <= G <= 8 (with or without the QJL sketch); no near tier.
bool wide_attend_supported(const AttendArgs &a);
hipError_t launch_attend_wide(const AttendArgs &a, hipStream_t stream, int part_base = 0);

// Outlier-channel calibration (validated arguments): keys [B][Hkv][n][head_dim].
hipError_t launch_calibrate(const void *keys, int in_f16, int batch, int kv_heads, int head_dim, int n,
                            int32_t *idx, hipStream_t stream);

// Split-merge launch (validated arguments).
struct MergeArgs {
  const float *part_o, *part_ml;
  int32_t batch, q_heads, head_dim, num_splits, num_near_splits;
  const int8_t *signs;
  float *out, *lse;
};
hipError_t launch_merge(const MergeArgs &a, hipStream_t stream, bool *supported);

}  // namespace kvq
