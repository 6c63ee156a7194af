// Shape-only planner: reads sizes, never device memory, so a call can be
// captured into a HIP graph. Its job follows the split planner of the
// flashmap page "sglang/verify_attention.py" (SplitKVVerify.splits and
// row_blocks): pick row blocks that hold all G*L query rows of one KV head,
// and split the prefix so that the batch fills every compute unit.
#include "plan.h"

#include <string.h>

namespace vat {

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int64_t x) {
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

vat_status_t validate_problem(const vat_problem_t* p) {
  if (!p) return VAT_ERR_NULL;
  if (p->batch < 0 || p->num_qo_heads < 1 || p->num_kv_heads < 1 || p->num_pages < 0 ||
      p->num_kv_indices < 0 || p->num_qo_tokens < 0 || p->max_qo_len < 0 ||
      p->num_mask_bytes < 0 || p->num_cus < 0)
    return VAT_ERR_SHAPE;
  if (p->num_qo_heads % p->num_kv_heads) return VAT_ERR_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return VAT_ERR_UNSUPPORTED;
  if (!is_pow2(p->page_size) || p->page_size > 256) return VAT_ERR_UNSUPPORTED;
  const bool pair_ok = (p->q_dtype == VAT_F32 && p->kv_dtype == VAT_F32) ||
                       (p->q_dtype == VAT_BF16 && p->kv_dtype == VAT_BF16) ||
                       (p->q_dtype == VAT_BF16 && p->kv_dtype == VAT_FP8_E4M3FN);
  if (!pair_ok) return VAT_ERR_UNSUPPORTED;
  if (p->has_mask != 0 && p->has_mask != 1) return VAT_ERR_SHAPE;
  if (p->has_mask && p->max_qo_len > kMaxMaskedLen) return VAT_ERR_UNSUPPORTED;
  if (p->chunk_keys < -1 || (p->chunk_keys > 0 && p->chunk_keys % kChunkQuantum))
    return VAT_ERR_SHAPE;
  if (p->batch > 0 && p->num_qo_tokens > 0 && p->num_pages < 1) return VAT_ERR_SHAPE;
  // Keys addressable through the page table must fit the int32 key counters.
  if (int64_t(p->num_kv_indices) * p->page_size > int64_t(INT32_MAX) / 2) return VAT_ERR_SHAPE;
  if (int64_t(p->num_qo_tokens) * p->num_qo_heads > int64_t(INT32_MAX)) return VAT_ERR_SHAPE;
  return VAT_OK;
}

vat_status_t make_plan(const vat_problem_t* p, int32_t num_cus, vat_plan_t* plan) {
  if (!plan) return VAT_ERR_NULL;
  vat_status_t st = validate_problem(p);
  if (st != VAT_OK) return st;
  memset(plan, 0, sizeof(*plan));
  if (num_cus < 1) return VAT_ERR_SHAPE;
  const int64_t G = p->num_qo_heads / p->num_kv_heads;
  const int64_t R = G * p->max_qo_len;
  plan->group = int32_t(G);
  plan->num_cus = num_cus;
  plan->threads = kThreads;
  plan->merge_threads = kMergeThreads;
  if (R == 0 || p->batch == 0 || p->num_qo_tokens == 0) {
    // Nothing to compute: an empty plan enqueues nothing.
    plan->direct = 1;
    plan->row_tiles_per_wave = 1;
    plan->waves_rows = 1;
    plan->waves_keys = kWaves;
    plan->rows_per_block = 16;
    return VAT_OK;
  }
  if (R > int64_t(INT32_MAX) / 2) return VAT_ERR_SHAPE;
  plan->rows = int32_t(R);

  // Row tiling. A wave holds RT 16-row MFMA tiles of the row block; waves
  // split the rows (waves_rows) and, when rows are few, the keys (waves_keys),
  // so the workgroup's four waves stay busy at any G*L.
  const int64_t tiles = cdiv(R, 16);
  int rt, wr;
  if (tiles <= 3) {
    rt = int(tiles);
    wr = 1;
  } else if (tiles == 4) {
    rt = 2;
    wr = 2;
  } else if (tiles <= 6) {
    rt = 3;
    wr = 2;
  } else {
    rt = 2;
    wr = 4;
  }
  const int wk = kWaves / wr;
  const int64_t M = int64_t(wr) * rt * 16;
  const int64_t RB = cdiv(R, M);
  plan->row_tiles_per_wave = rt;
  plan->waves_rows = wr;
  plan->waves_keys = wk;
  plan->rows_per_block = int32_t(M);
  plan->row_blocks = int32_t(RB);
  if (int64_t(p->num_kv_heads) * RB > 65535) return VAT_ERR_UNSUPPORTED;

  // Split or not. Without a split each (request, KV head, row block) is one
  // workgroup that writes the output itself; that is enough work items when
  // they already cover the chip several times over. Otherwise the prefix is
  // cut into fixed-length chunks (plus one item per request for the draft
  // block), sized from the page-table capacity so the chunk count fills the
  // compute units; a later merge combines them.
  const int64_t base_items = int64_t(p->batch) * p->num_kv_heads * RB;
  bool direct;
  int64_t ck = 0;
  if (p->chunk_keys == 0) {
    direct = true;
  } else if (p->chunk_keys > 0) {
    direct = false;
    ck = p->chunk_keys;
  } else {
    direct = base_items >= 4 * int64_t(num_cus);
    if (!direct) {
      const int64_t total_keys = int64_t(p->num_kv_indices) * p->page_size;
      const int64_t target = 4 * int64_t(num_cus);
      int64_t slots = target - 2 * base_items;
      if (slots < num_cus) slots = num_cus;
      ck = cdiv(total_keys * p->num_kv_heads * RB, slots);
      ck = cdiv(ck, kChunkQuantum) * kChunkQuantum;
      if (ck < kMinChunkKeys) ck = kMinChunkKeys;
    }
  }
  plan->direct = direct ? 1 : 0;
  const int64_t ndt = p->head_dim / 16;
  // LDS: per-wave staging of one step's V tile (bf16 after any fp8 decode),
  // and the slots the key-splitting waves use to combine their partials.
  int64_t lds_v = (p->kv_dtype == VAT_F32) ? 0 : int64_t(kWaves) * kStepKeys * p->head_dim * 2;
  int64_t lds_c = 0;
  if (wk > 1) lds_c = int64_t(wk / 2) * wr * (int64_t(rt) * ndt * 256 + int64_t(rt) * 32) * 4;
  plan->lds_bytes = int32_t(lds_v > lds_c ? lds_v : lds_c);
  if (plan->lds_bytes > 160 * 1024) return VAT_ERR_UNSUPPORTED;

  if (direct) {
    plan->chunk_keys = 0;
    plan->num_chunk_ids = 0;
    plan->grid_x = p->batch;
    plan->grid_y = int32_t(p->num_kv_heads * RB);
    plan->merge_grid = 0;
    plan->workspace_bytes = 0;
    return VAT_OK;
  }
  const int64_t total_keys = int64_t(p->num_kv_indices) * p->page_size;
  const int64_t ids = total_keys / ck + 2 * int64_t(p->batch);
  if (ids > int64_t(INT32_MAX)) return VAT_ERR_UNSUPPORTED;
  plan->chunk_keys = int32_t(ck);
  plan->num_chunk_ids = int32_t(ids);
  plan->grid_x = int32_t(ids);
  plan->grid_y = int32_t(p->num_kv_heads * RB);
  const int64_t row_groups = cdiv(M, kMergeRows);
  const int64_t mg = base_items * row_groups;
  if (mg > int64_t(INT32_MAX)) return VAT_ERR_UNSUPPORTED;
  plan->merge_grid = int32_t(mg);
  const int64_t parts = ids * p->num_kv_heads * RB;
  const int64_t o_bytes = parts * M * p->head_dim * 4;
  const int64_t lse_off = cdiv(o_bytes, 256) * 256;
  plan->workspace_bytes = lse_off + cdiv(parts * M * 4, 256) * 256;
  return VAT_OK;
}

int64_t workspace_lse_offset(const vat_plan_t& plan, int32_t head_dim, int32_t num_kv_heads) {
  const int64_t parts = int64_t(plan.num_chunk_ids) * num_kv_heads * plan.row_blocks;
  const int64_t o_bytes = parts * plan.rows_per_block * head_dim * 4;
  return cdiv(o_bytes, 256) * 256;
}

}  // namespace vat
