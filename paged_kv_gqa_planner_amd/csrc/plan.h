// Host planner and kernel argument blocks. Plain C++: no HIP headers, so the
// planner builds and runs on a machine without a GPU.
#pragma once

#include <stdint.h>

#include "verify_attention.h"

namespace vat {

// Threads per partial-kernel workgroup: four wave64s.
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Row-tiled kernel: keys each wave consumes per step (two 16-key MFMA tiles).
constexpr int kStepKeys = 32;
// Streaming kernel: eight waves; keys per LDS stage (four 16-key MFMA tiles),
// most 16-row tiles per KV head it takes (one or two per wave), LDS its stage
// ring may fill.
constexpr int kStreamThreads = 512;
constexpr int kStageKeys = 64;
// Keys per streaming stage: 64 when a key row is 256 bytes (bf16, D = 128),
// else 128, so a stage is 32 KB either way.
constexpr int stream_stage_keys(int kv_dtype, int head_dim) {
  return (kv_dtype == VAT_BF16 && head_dim == 128) ? 64 : 128;
}
// Two-pass stages: bf16 D = 128 plans with two row tiles per wave (prefill
// blocks, wide trees), or with query RoPE, one tile per wave, all eight
// waves issuing loads and several row blocks, stream 128-key stages (two of
// 64 KB), each taken in two 64-key passes: half as many stage barriers. Their
// keys come mostly from L2 (each group's row blocks share them), so one stage
// of look-ahead suffices.
constexpr bool stream_two_pass(int kv_dtype, int head_dim, int rt, int dma_waves, int rope,
                               int mask_mode, long long row_blocks) {
  return kv_dtype == VAT_BF16 && head_dim == 128 &&
         (rt == 2 || (rope && rt == 1 && dma_waves == kStreamThreads / 64 && mask_mode != 2 &&
                      row_blocks > 1));
}
constexpr int kStreamMaxTiles = 16;
constexpr int kStreamLdsBudget = 128 * 1024;
// Page ids the streaming kernel keeps in LDS at a time.
constexpr int kStreamPageWindow = 2048;
// Query rows merged per merge-kernel workgroup: one wave per row, or four
// rows per wave.
constexpr int kMergeRows = 4;
constexpr int kMergeRows4 = 16;
constexpr int kMergeThreads = 256;
// Chunk lengths the planner picks are multiples of kChunkQuantum, at least
// kMinChunkKeys (and for the row-tiled kernel at most kMaxChunkKeys).
constexpr int kChunkQuantum = 16;
constexpr int kMinChunkKeys = 128;
constexpr int kMaxChunkKeys = 2048;
// Batches up to this size are scheduled as balanced slices of the page-index
// space (a wave holds one request per lane).
constexpr int kSliceMaxBatch = 64;
// Largest draft count per request a bit-packed mask may carry (one 64-bit
// register holds a row).
constexpr int kMaxMaskedLen = 64;

// Arguments of both partial kernels; every field is a plain pointer or integer.
struct PartialArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* last_page_len;
  const int32_t* qo_indptr;
  const uint8_t* mask;
  const int32_t* mask_indptr;
  void* out;
  float* lse;
  float* part_o;
  float* part_lse;
  float c_log2;   // sm_scale * k_scale * log2(e): raw logit -> base-2 exponent
  float v_scale;
  int32_t batch, hq, hkv, group, tokens;
  int32_t page_shift, num_pages, num_kv_indices, num_mask_bytes;
  int32_t rows_per_block, row_blocks, waves_rows, waves_keys;
  int32_t chunk_keys, num_ids, has_mask;
  int32_t slices;  // > 0: balanced page slices per KV head (streaming kernel, B <= 64)
  int32_t block_order;  // 1: one-dimensional grid, row blocks of a group on one XCD
  const float* q_cos_sin;  // [T, D] RoPE cos/sin row per query token, or null
};

// Arguments of the merge kernel.
struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* kv_indptr;
  const int32_t* last_page_len;
  const int32_t* qo_indptr;
  void* out;
  float* lse;
  float v_scale;
  int32_t batch, hq, hkv, group, tokens;
  int32_t page_shift, num_kv_indices;
  int32_t rows_per_block, row_blocks, chunk_keys, num_ids, row_groups;
  int32_t slices;  // > 0: partials come from balanced page slices, slot = slice + request
};

// Arguments of the draft key/value write (cache append) kernel.
struct AppendArgs {
  const void* k_new;  // [T, Hkv, D] in the source dtype
  const void* v_new;
  void* k_cache;      // [num_pages, page_size, Hkv, D] in the cache dtype
  void* v_cache;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* last_page_len;
  const int32_t* qo_indptr;
  const float* k_cos_sin;  // [T, D] RoPE cos/sin row per draft token, or null
  float k_scale, v_scale;
  float k_inv, v_inv;  // exact 1 / scale when both scales are powers of two
  int32_t head_dim;
  int32_t batch;
  int32_t row_units;  // Hkv * D / 8: 8-element units in one token row
  int32_t page_shift;
  int32_t num_pages;
  int32_t num_kv_indices;
  int32_t tokens;
};

constexpr int kAppendThreads = 256;

// Shape validation (host-detectable errors only).
vat_status_t validate_problem(const vat_problem_t* p);

// Validation of the fields the cache append reads (batch, num_kv_heads,
// head_dim, page_size, num_pages, num_kv_indices, num_qo_tokens, max_qo_len,
// kv_dtype, num_cus) and of the source dtype.
vat_status_t validate_append(const vat_problem_t* p, int32_t src_dtype);

// Shape-only plan for `num_cus` compute units. Calls validate_problem.
vat_status_t make_plan(const vat_problem_t* p, int32_t num_cus, vat_plan_t* plan);

// Byte offset of the partial-lse array inside the workspace.
int64_t workspace_lse_offset(const vat_plan_t& plan, int32_t head_dim, int32_t num_kv_heads);

}  // namespace vat
