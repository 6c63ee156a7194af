// Shape-only planner: reads sizes, never device memory, so a call can be
// captured into a HIP graph. It follows the split planner of the flashmap
// page "sglang/verify_attention.py" (SplitKVVerify.splits and row_blocks):
// hold all G*L query rows of a KV head together so each key is read once per
// KV head, and split the keys so the batch fills every compute unit -- here
// with chunks of a fixed length sized from the page-table capacity, so long
// and short requests get work items of the same size.
#include "plan.h"

#include <string.h>

namespace vat {

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t elem_bytes(int32_t dtype) { return dtype == VAT_F32 ? 4 : (dtype == VAT_BF16 ? 2 : 1); }

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
  if (p->has_mask < 0 || p->has_mask > 2) return VAT_ERR_SHAPE;
  if (p->has_mask && p->max_qo_len > kMaxMaskedLen) return VAT_ERR_UNSUPPORTED;
  if (p->has_mask && p->num_mask_bytes < 1) return VAT_ERR_SHAPE;
  if (p->rope != 0 && p->rope != 1) return VAT_ERR_SHAPE;
  // Query RoPE runs in the streaming kernel: not for fp32 caches (the
  // row-tiled kernel) nor for fp8 with D = 64, whose query layout puts the
  // two dimensions of a rotated pair (i, i + D/2) in different lanes.
  if (p->rope && (p->kv_dtype == VAT_F32 || (p->kv_dtype == VAT_FP8_E4M3FN && p->head_dim == 64)))
    return VAT_ERR_UNSUPPORTED;
  if (p->chunk_keys < -1 || (p->chunk_keys > 0 && p->chunk_keys % kChunkQuantum))
    return VAT_ERR_SHAPE;
  if (p->batch > 0 && p->num_qo_tokens > 0 && p->num_pages < 1) return VAT_ERR_SHAPE;
  // Keys addressable through the page table must fit the int32 key counters.
  if (int64_t(p->num_kv_indices) * p->page_size > int64_t(INT32_MAX) / 2) return VAT_ERR_SHAPE;
  if (int64_t(p->num_qo_tokens) * p->num_qo_heads > int64_t(INT32_MAX)) return VAT_ERR_SHAPE;
  return VAT_OK;
}

vat_status_t validate_append(const vat_problem_t* p, int32_t src_dtype) {
  if (!p) return VAT_ERR_NULL;
  if (p->batch < 0 || p->num_kv_heads < 1 || p->num_pages < 0 || p->num_kv_indices < 0 ||
      p->num_qo_tokens < 0 || p->max_qo_len < 0 || p->num_cus < 0)
    return VAT_ERR_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return VAT_ERR_UNSUPPORTED;
  if (!is_pow2(p->page_size) || p->page_size > 256) return VAT_ERR_UNSUPPORTED;
  if (src_dtype != VAT_F32 && src_dtype != VAT_BF16) return VAT_ERR_UNSUPPORTED;
  if (p->kv_dtype != VAT_F32 && p->kv_dtype != VAT_BF16 && p->kv_dtype != VAT_FP8_E4M3FN)
    return VAT_ERR_UNSUPPORTED;
  if (p->batch > 0 && p->num_qo_tokens > 0 && p->num_pages < 1) return VAT_ERR_SHAPE;
  if (int64_t(p->num_kv_indices) * p->page_size > int64_t(INT32_MAX) / 2) return VAT_ERR_SHAPE;
  // Key positions and token rows are int32 inside the kernel.
  if (int64_t(p->max_qo_len) * p->num_kv_heads * p->head_dim > int64_t(INT32_MAX))
    return VAT_ERR_SHAPE;
  return VAT_OK;
}

// Query rows per merge workgroup: four per wave (16 lanes a row) when a
// request's partials fit one round of that kernel's loads, else one per wave.
static int32_t merge_rows_for(int64_t partials, int64_t head_dim) {
  const int64_t per_round = head_dim == 128 ? 8 : 16;
  return partials <= per_round ? kMergeRows4 : kMergeRows;
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
  const int64_t tiles = cdiv(R, 16);
  const int64_t D = p->head_dim;
  const int64_t eb = elem_bytes(p->kv_dtype);

  // Several KV heads per workgroup: fp8 caches with D = 128 (128-byte head
  // rows) and a head count divisible by the group, every head's rows in at
  // most two tiles, a batch the balanced slices serve and no byte-row masks.
  // A key's DMA then reads the group's rows as one run (512 bytes for four
  // heads, 256 for two) instead of 128-byte runs, each fetched by another
  // workgroup at another time.
  //  * Four heads (head count divisible by 4, no RoPE): one computing wave
  //    per head holding all of its row tiles, so each key and value is
  //    decoded once per head; 32-key stages of 32 KB.
  //  * Two heads (other even head counts, and RoPE, whose rotated query
  //    leaves the registers for one row tile per wave): one tile per
  //    computing wave, the tiles of head h, then those of h + 1; 64-key
  //    stages of 32 KB.
  // Four DMA waves either way.
  const bool fp8 = p->kv_dtype == VAT_FP8_E4M3FN;
  if (fp8 && D == 128 && p->num_kv_heads % 2 == 0 && tiles <= 2 && p->has_mask != 2 &&
      p->chunk_keys == -1 && p->batch <= kSliceMaxBatch) {
    const int64_t M = tiles * 16;
    const int64_t hp = p->num_kv_heads % 4 == 0 && !p->rope ? 4 : 2;
    const int64_t groups = p->num_kv_heads / hp;
    plan->kernel = 1;
    plan->heads_per_group = int32_t(hp);
    plan->threads = kStreamThreads;
    plan->row_tiles_per_wave = hp == 4 ? int32_t(tiles) : 1;
    plan->waves_rows = hp == 4 ? 4 : int32_t(2 * tiles);
    plan->waves_keys = 1;
    plan->dma_waves = 4;
    plan->rows_per_block = int32_t(M);
    plan->row_blocks = 1;
    plan->stages = 4;
    plan->lds_bytes = 4 * 32 * 1024 + kStreamPageWindow * 4;
    int64_t nx = int64_t(num_cus) / groups;
    if (nx < 1) nx = 1;
    plan->slices = int32_t(nx);
    plan->direct = nx == 1 ? 1 : 0;
    plan->chunk_keys = 0;
    plan->num_chunk_ids = int32_t(nx + p->batch);  // partial slots: slice + request
    plan->grid_x = int32_t(nx);
    plan->grid_y = int32_t(groups);
    if (plan->direct) return VAT_OK;
    plan->merge_rows = merge_rows_for(nx / p->batch + 1, D);
    const int64_t row_groups = cdiv(M, plan->merge_rows);
    plan->merge_grid = int32_t(int64_t(p->batch) * p->num_kv_heads * row_groups);
    const int64_t parts = (nx + p->batch) * p->num_kv_heads;
    const int64_t lse_off = cdiv(parts * M * D * 4, 256) * 256;
    plan->workspace_bytes = lse_off + cdiv(parts * M * 4, 256) * 256;
    return VAT_OK;
  }
  plan->heads_per_group = 1;

  // Kernel and row tiling.
  //  * Streaming kernel (bf16 / fp8 caches): wave w of eight computes row
  //    tiles [w rt, w rt + rt) of a row block over all of the block's keys
  //    (rt = 1 up to eight tiles, else 2: blocks of 128 or 256 rows), so each
  //    key is read from HBM once per row block and no two waves share a row's
  //    softmax state. Verify shapes fit one block; a prefill takes several.
  //  * Row-tiled kernel (fp32 caches, fp8 with D = 64): a wave holds RT
  //    tiles; waves split the rows and, when rows are few, the keys.
  int rt, wr, wk;
  // fp8 caches with D = 64 have too few 1 KB loads per stage for eight waves;
  // with fp8 the decode registers leave room for one row tile per wave.
  const bool stream = (p->kv_dtype != VAT_F32) && !(fp8 && p->head_dim == 64);
  int dw = 0;
  if (stream) {
    // fp8, full byte-row masks and query RoPE keep one row tile per wave
    // (registers).
    const int64_t max_tiles =
        (fp8 || p->has_mask == 2 || p->rope) ? kStreamThreads / 64 : kStreamMaxTiles;
    const int64_t bt = tiles <= max_tiles ? tiles : max_tiles;  // tiles per row block
    rt = bt <= kStreamThreads / 64 ? 1 : 2;
    wr = int(cdiv(bt, rt));
    // One or two row tiles: two waves per tile split every stage's keys
    // (their softmax states meet in LDS at the end of each segment), so four
    // SIMDs share the math.
    wk = bt <= 2 ? 2 : 1;
    // Up to six computing waves leave the last four (or two) to issue the DMA
    // alone, so a computing wave never stalls behind the memory queue.
    dw = wr * wk <= 4 ? 4 : (rt == 1 && wr * wk <= 6 ? 2 : kStreamThreads / 64);
    // One row tile (decode) keeps this pair too. A single computing wave
    // with all eight waves issuing was faster while the K/V loads kept the
    // default cache policy (B64 decode 224.5 -> 215.3 us); with non-temporal
    // loads the pair with four DMA waves is (210-214 -> 194-195 us).
  } else if (tiles <= 3) {
    rt = int(tiles);
    wr = 1;
    wk = kWaves;
  } else if (tiles == 4) {
    rt = 2;
    wr = 2;
    wk = 2;
  } else if (tiles <= 6) {
    rt = 3;
    wr = 2;
    wk = 2;
  } else {
    rt = 2;
    wr = 4;
    wk = 1;
  }
  const int64_t M = int64_t(wr) * rt * 16;
  const int64_t RB = cdiv(R, M);
  plan->kernel = stream ? 1 : 0;
  plan->threads = stream ? kStreamThreads : kThreads;
  plan->row_tiles_per_wave = rt;
  plan->waves_rows = wr;
  plan->waves_keys = wk;
  plan->dma_waves = dw;
  plan->rows_per_block = int32_t(M);
  plan->row_blocks = int32_t(RB);
  if (int64_t(p->num_kv_heads) * RB > 65535) return VAT_ERR_UNSUPPORTED;

  // LDS. Streaming: a ring of stages (K and V of 64 keys at bf16 D 128 with
  // one row tile per wave, else 128 keys), as many as fit the budget (2..8),
  // plus the work item's page ids. Row-tiled: a
  // per-wave 32-key V staging tile (bf16 after any fp8 decode) and the slots
  // of the key-splitting waves' combine.
  const int64_t ndt = D / 16;
  if (stream) {
    const bool two_pass = stream_two_pass(p->kv_dtype, int(D), rt, dw, p->rope, p->has_mask, RB);
    const int64_t stage = 2 * int64_t(two_pass ? 128 : stream_stage_keys(p->kv_dtype, p->head_dim)) * D * eb;
    int64_t ns = kStreamLdsBudget / stage;
    if (ns > 8) ns = 8;
    if (ns < 2) ns = 2;
    plan->stages = int32_t(ns);
    // ring, page-id window and, for tile pairs, one softmax-state slot per tile
    const int64_t pair_slot = (int64_t(rt) * ndt * 256 + int64_t(rt) * 32) * 4;
    plan->lds_bytes = int32_t(ns * stage + kStreamPageWindow * 4 + (wk - 1) * int64_t(wr) * pair_slot);
  } else {
    const int64_t lds_v = (p->kv_dtype == VAT_F32) ? 0 : int64_t(kWaves) * kStepKeys * D * 2;
    int64_t lds_c = 0;
    if (wk > 1) lds_c = int64_t(wk / 2) * wr * (int64_t(rt) * ndt * 256 + int64_t(rt) * 32) * 4;
    plan->lds_bytes = int32_t(lds_v > lds_c ? lds_v : lds_c);
  }
  if (plan->lds_bytes > 160 * 1024) return VAT_ERR_UNSUPPORTED;

  // Chunk length. Each request's keys [0, kv_len) form ceil(kv_len / C)
  // work items (the draft block is masked inside the last one); a request
  // with one item writes its output directly, the others go through the
  // log-sum-exp merge. The planner sizes C from the page-table capacity so
  // that the items about fill the compute units once (the streaming kernel
  // holds one workgroup per CU), at least kMinChunkKeys (the row-tiled
  // kernel's also at most kMaxChunkKeys); a
  // row-tiled plan whose (request, KV head, row block) items already cover
  // the chip four times over is not split at all.
  const int64_t total_keys = int64_t(p->num_kv_indices) * p->page_size;
  const int64_t whole = cdiv(total_keys > 0 ? total_keys : 1, kChunkQuantum) * kChunkQuantum;
  const int64_t base_items = int64_t(p->batch) * p->num_kv_heads * RB;
  int64_t ck;
  if (p->chunk_keys == 0) {
    ck = whole;
  } else if (p->chunk_keys > 0) {
    ck = p->chunk_keys;
  } else if (base_items >= 4 * int64_t(num_cus) || (stream && RB > 1 && base_items >= int64_t(num_cus))) {
    // Enough (request, KV head, row block) items to fill the chip.
    ck = whole;
  } else if (stream) {
    // Split the average request evenly into as many chunks as leave one
    // workgroup per CU: with equal request lengths every chunk then has the
    // same length and the items fill the CUs exactly once. No upper bound:
    // capping the length would leave a short remainder chunk per request,
    // whose workgroups take CUs in the first round and push full-length ones
    // into a second (a long chunk only moves the page window).
    const int64_t per_req = cdiv(total_keys, p->batch);
    int64_t nchunk = int64_t(num_cus) / (int64_t(p->batch) * p->num_kv_heads * RB);
    if (nchunk < 1) nchunk = 1;
    ck = cdiv(cdiv(per_req, nchunk), kChunkQuantum) * kChunkQuantum;
    if (ck < kMinChunkKeys) ck = kMinChunkKeys;
  } else {
    ck = cdiv(total_keys * p->num_kv_heads * RB, 4 * int64_t(num_cus));
    ck = cdiv(ck, kChunkQuantum) * kChunkQuantum;
    if (ck < kMinChunkKeys) ck = kMinChunkKeys;
    if (ck > kMaxChunkKeys) ck = kMaxChunkKeys;
  }
  if (ck > int64_t(INT32_MAX) / 2) return VAT_ERR_UNSUPPORTED;
  // Balanced key slices (streaming kernel, planner's choice, small batches):
  // one workgroup per CU share of each KV head, whatever the length mix.
  if (stream && RB == 1 && p->chunk_keys == -1 && p->batch <= kSliceMaxBatch) {
    int64_t nx = int64_t(num_cus) / p->num_kv_heads;
    if (nx < 1) nx = 1;
    plan->slices = int32_t(nx);
    plan->direct = nx == 1 ? 1 : 0;
    plan->chunk_keys = 0;
    plan->num_chunk_ids = int32_t(nx + p->batch);  // partial slots: slice + request
    plan->grid_x = int32_t(nx);
    plan->grid_y = int32_t(p->num_kv_heads * RB);
    if (plan->direct) return VAT_OK;
    // A request's pages span about nx / B + 1 slices.
    plan->merge_rows = merge_rows_for(nx / p->batch + 1, D);
    const int64_t row_groups = cdiv(M, plan->merge_rows);
    plan->merge_grid = int32_t(base_items * row_groups);
    const int64_t parts = (nx + p->batch) * p->num_kv_heads * RB;
    const int64_t lse_off = cdiv(parts * M * D * 4, 256) * 256;
    plan->workspace_bytes = lse_off + cdiv(parts * M * 4, 256) * 256;
    return VAT_OK;
  }
  const bool direct = ck >= total_keys;
  const int64_t ids = total_keys / ck + p->batch;
  if (ids > int64_t(INT32_MAX)) return VAT_ERR_UNSUPPORTED;
  plan->direct = direct ? 1 : 0;
  plan->chunk_keys = int32_t(ck);
  plan->num_chunk_ids = int32_t(ids);
  plan->grid_x = int32_t(ids);
  plan->grid_y = int32_t(p->num_kv_heads * RB);
  if (stream && RB > 1) {
    // Row blocks re-read their group's keys: keep each group's blocks on one
    // XCD (one L2), eight groups per round (one-dimensional grid). With eight
    // or more row blocks per CU, pair them (block order 2): a workgroup runs
    // its group's blocks RB - 1 - k and k back to back, so half as many
    // workgroups pay the start-up and the causal work per workgroup evens
    // out. Both blocks restart at the item's first key, so the item's pages
    // must fit the page window.
    const int64_t groups = ids * p->num_kv_heads;
    const bool pair = groups * RB >= 8 * int64_t(num_cus) &&
                      cdiv(ck, p->page_size) + 1 <= kStreamPageWindow;
    const int64_t w = pair ? cdiv(RB, 2) : RB;
    const int64_t g1 = 8 * w * cdiv(groups, 8);
    if (g1 > int64_t(INT32_MAX)) return VAT_ERR_UNSUPPORTED;
    plan->block_order = pair ? 2 : 1;
    plan->grid_x = int32_t(g1);
    plan->grid_y = 1;
  }
  if (direct) {
    plan->merge_grid = 0;
    plan->workspace_bytes = 0;
    return VAT_OK;
  }
  // A request of average length has about total_keys / (B C) + 1 chunks.
  plan->merge_rows = merge_rows_for(total_keys / (int64_t(p->batch) * ck) + 1, D);
  const int64_t row_groups = cdiv(M, plan->merge_rows);
  const int64_t mg = base_items * row_groups;
  if (mg > int64_t(INT32_MAX)) return VAT_ERR_UNSUPPORTED;
  plan->merge_grid = int32_t(mg);
  const int64_t parts = ids * p->num_kv_heads * RB;
  const int64_t o_bytes = parts * M * D * 4;
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
