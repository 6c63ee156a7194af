/*
 * verify_attention.h -- C ABI of the MI355X (gfx950) library for multi-query
 * verification attention over a paged KV cache.
 *
 * What one call computes. Each request b has L_b query ("draft") tokens --
 * a chain or a tree plus its root -- whose keys and values are already the
 * last L_b entries of the request's paged cache (the vLLM page "[WIP] Support
 * for cached multi-query attention towards speculative decoding": all draft
 * keys and values are cached before attention). Query token t of query head
 * hq attends, with KV head hq / G (G = Hq / Hkv, consecutive query heads
 * share a KV head: vLLM page "[Performance] Support MQA/GQA in prefill stage
 * by using FlashAttention"), to
 *   - every prefix key n < prefix_b = kv_len_b - L_b, and
 *   - draft key j (key prefix_b + j) iff j <= t (causal, no mask) or iff
 *     entry (t, j) of the request's mask allows it (a tree mask in place of
 *     the causal one: FlashInfer page "How to implement a tree attention with
 *     flashinfer"),
 * and returns out = softmax(sm_scale * k_scale * q.K^T) . (v_scale * V) and
 * lse = natural log of the sum of exp of those scaled logits. The prefix is
 * split across workgroups and the partial results are merged by their
 * log-sum-exp (flashmap page "sglang/verify_attention.py",
 * _verify_partial_kernel / _verify_merge_kernel). A row that sees no key
 * gets out = 0 and lse = -inf.
 *
 * Layouts (dense, row-major, caller-owned DEVICE memory unless noted):
 *   q, out       [T, Hq, D]        T = qo_indptr[B]; out has q's dtype
 *   k_cache,
 *   v_cache      [num_pages, page_size, Hkv, D]   ("NHD" pages)
 *   kv_indptr    int32 [B + 1]     pages of request b are
 *   kv_indices   int32 [>= kv_indptr[B]]  kv_indices[kv_indptr[b] .. kv_indptr[b+1])
 *   last_page_len int32 [B]        entries in request b's last page, 1..page_size
 *   qo_indptr    int32 [B + 1]     query tokens of request b are rows
 *                                  qo_indptr[b] .. qo_indptr[b+1] of q
 *   mask         uint8 [num_mask_bytes] or NULL (NULL = causal)
 *   mask_indptr  int32 [B + 1] or NULL: byte offset of request b's block
 *   lse          float32 [T, Hq]
 * The paged format is the one documented on the FlashInfer page "feat:
 * Separate Q and KV dtypes for decode" (begin_forward docstring):
 * kv_len_b = (pages_b - 1) * page_size + last_page_len[b].
 *
 * Mask layouts (has_mask selects one; both cover the drafts only, the prefix
 * being always visible):
 *   1 = packed blocks (this library's layout): request b's L_b x L_b block,
 *       row-major flat index i = t * L_b + j, bit (i % 8), least significant
 *       first, of byte mask[mask_indptr[b] + i / 8]; 1 = allowed. Each
 *       segment must hold at least ceil(L_b * L_b / 8) bytes.
 *   2 = full byte rows (sglang's layout, as the flashmap page
 *       "sglang/verify_attention.py" reads it): request b holds L_b rows of
 *       prefix_b + L_b bytes from byte mask_indptr[b], one byte per key;
 *       entry (t, j) is byte mask_indptr[b] + t * (prefix_b + L_b) + prefix_b
 *       + j, nonzero = allowed. The prefix bytes are not read. Each segment
 *       must hold L_b * (prefix_b + L_b) bytes.
 *
 * Device-content contract (not checked on the host, which never reads device
 * memory): kv_indptr non-decreasing from 0 with kv_indptr[B] <=
 * num_kv_indices; 0 <= kv_indices[..] < num_pages; 1 <= last_page_len <=
 * page_size for requests with pages; qo_indptr non-decreasing from 0 to T;
 * 0 <= L_b <= min(max_qo_len, kv_len_b); mask segments as above. Kernels
 * clamp every index they derive from these arrays, so a violation gives
 * unspecified values but never an out-of-bounds access. vat_check_inputs
 * checks the contract on the device and reports which rule a call breaks.
 *
 * Calls never allocate, free, synchronise or read device memory on the
 * host. They enqueue at most two kernels on `stream` (a hipStream_t; NULL =
 * the default stream) and may be captured into a HIP graph; the workspace
 * must then outlive the graph. Calls on different streams need different
 * workspaces. The library keeps only a per-device cache of the compute-unit
 * count, filled on first use.
 */
#ifndef PAGED_KV_VERIFY_ATTENTION_H
#define PAGED_KV_VERIFY_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VAT_F32 = 0,        /* IEEE binary32 */
  VAT_BF16 = 1,       /* bfloat16 */
  VAT_FP8_E4M3FN = 2  /* OCP FP8 E4M3 (finite-only, max 448): KV cache only */
} vat_dtype_t;

typedef enum {
  VAT_OK = 0,
  VAT_ERR_NULL = 1,        /* a required pointer is NULL */
  VAT_ERR_SHAPE = 2,       /* inconsistent or negative sizes, Hq % Hkv != 0, bad scales */
  VAT_ERR_UNSUPPORTED = 3, /* head_dim, page_size, dtype pair or mask length not built */
  VAT_ERR_ALIGN = 4,       /* q, caches or out not 16-byte aligned */
  VAT_ERR_WORKSPACE = 5,   /* workspace smaller than vat_workspace_size() */
  VAT_ERR_HIP = 6          /* the HIP runtime reported an error (device query or launch) */
} vat_status_t;

/* Shapes and options of one call. Every field is a host integer. */
typedef struct {
  int32_t batch;          /* B >= 0 */
  int32_t num_qo_heads;   /* Hq >= 1 */
  int32_t num_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;       /* D: 64 or 128 */
  int32_t page_size;      /* power of two, 1 .. 256 */
  int32_t num_pages;      /* first dimension of each cache, >= 1 */
  int32_t num_kv_indices; /* capacity of kv_indices (>= kv_indptr[B]) */
  int32_t num_qo_tokens;  /* T = rows of q = qo_indptr[B] */
  int32_t max_qo_len;     /* host bound on every L_b; <= 64 when has_mask */
  int32_t q_dtype;        /* vat_dtype_t: F32 or BF16; out has this dtype */
  int32_t kv_dtype;       /* F32 (with F32 q), BF16 or FP8_E4M3FN (with BF16 q) */
  int32_t has_mask;       /* 0: causal drafts (mask ignored); 1: packed L x L bit
                             blocks; 2: full byte rows (see the mask layouts) */
  int32_t num_mask_bytes; /* size of mask when has_mask (>= 1) */
  int32_t num_cus;        /* compute units to plan for; 0 = query the current device */
  int32_t chunk_keys;     /* -1: planner; 0: no split (one work item per request,
                             KV head and row block writes out directly);
                             > 0: chunk length in keys, multiple of 16 */
  int32_t rope;           /* 0; 1: verify_attention_rope rotates the queries by
                             RoPE (bf16 caches, or fp8 with D 128; either mask
                             layout) */
} vat_problem_t;

/* What the planner decided; filled by vat_plan. Shape-only: the same problem
 * always gives the same plan. */
typedef struct {
  int32_t direct;           /* 1: every request fits one chunk: no merge kernel,
                               the partial kernel writes out/lse itself */
  int32_t kernel;           /* 1: LDS-ring streaming kernel (bf16 KV, and fp8 KV
                               with D 128; rows in blocks of up to 256 (bf16) or
                               128 (fp8, or full byte-row masks) per KV head);
                               0: row-tiled kernel (fp32 KV, fp8 KV with D 64) */
  int32_t stages;           /* streaming kernel: stages in the LDS ring. 32 KB
                               stages (64 keys at bf16 D 128, else 128 keys),
                               or, for bf16 D 128 plans whose waves hold two
                               row tiles (and query-RoPE plans of one tile
                               per wave, all eight waves loading and several
                               row blocks), two 64 KB stages of 128 keys
                               each, computed in two 64-key passes */
  int32_t slices;           /* > 0: balanced scheduling. Per KV head, the page-index
                               space [0, num_kv_indices) is cut into `slices` equal
                               ranges, one workgroup each, which processes the
                               requests' pages inside it; 0: each request is cut
                               into chunk_keys-long chunks */
  int32_t group;            /* G = Hq / Hkv */
  int32_t rows;             /* G * max_qo_len query rows per (request, KV head) */
  int32_t row_tiles_per_wave; /* 16-row MFMA tiles each wave holds */
  int32_t waves_rows;       /* waves splitting a row block's rows */
  int32_t waves_keys;       /* waves splitting each key range (streaming kernel:
                               waves per row tile set, each taking a share of
                               every stage's keys) */
  int32_t dma_waves;        /* streaming kernel: waves issuing the K/V loads (the
                               last dma_waves of eight) */
  int32_t rows_per_block;   /* M = waves_rows * row_tiles_per_wave * 16 */
  int32_t row_blocks;       /* RB = ceil(rows / M) */
  int32_t chunk_keys;       /* keys per chunk: request b's keys [0, kv_len_b) form
                               ceil(kv_len_b / chunk_keys) work items */
  int32_t num_chunk_ids;    /* partial-kernel grid x */
  int32_t grid_x, grid_y;   /* partial kernel grid */
  int32_t threads;          /* partial kernel workgroup size */
  int32_t lds_bytes;        /* partial kernel dynamic LDS */
  int32_t merge_grid;       /* merge kernel workgroups (0 when direct) */
  int32_t merge_threads;
  int32_t num_cus;          /* compute units planned for */
  int64_t workspace_bytes;  /* bytes of workspace the call needs (0 when direct) */
  int32_t block_order;      /* 0: partial grid (num_chunk_ids, Hkv * row_blocks);
                               1 (streaming kernel, more than one row block):
                               one-dimensional grid in which the row blocks of
                               each (work item, KV head) run on one XCD, one
                               workgroup per row block;
                               2: as 1, but each workgroup runs two row blocks
                               of its (work item, KV head), RB - 1 - k and k,
                               ceil(row_blocks / 2) workgroups per group */
  int32_t merge_rows;       /* query rows per merge workgroup: 4 (one wave per
                               row, for requests with many partials) or 16
                               (four rows per wave); 0 when direct */
  int32_t heads_per_group;  /* streaming kernel: KV heads one workgroup takes
                               (1, or 2 or 4 adjacent heads read as one run
                               per key: fp8 caches with D 128); grid_y
                               counts head groups (times row blocks) */
} vat_plan_t;

/* Plan a call: validates the shapes and fills *plan. Host only; touches the
 * GPU only to read the compute-unit count when problem->num_cus == 0.
 * Planning is separate from running, as in the FlashInfer page "feat:
 * Separate Q and KV dtypes for decode" (begin_forward docstring: a planning
 * call builds the auxiliary structures before the forward calls reuse them),
 * but here the plan depends on shapes alone -- never on device contents -- so
 * verify_attention replans on every call for free and stays capturable.
 * Errors: VAT_ERR_NULL for a NULL argument, otherwise those of
 * verify_attention's host checks; *plan is then unspecified. */
vat_status_t vat_plan(const vat_problem_t* problem, vat_plan_t* plan);

/* Workspace bytes verify_attention needs for this problem (host only; see
 * vat_plan for the device query). The workspace is the caller-owned scratch
 * buffer that the same FlashInfer page's begin_forward takes as its first
 * argument; here it holds the per-split partial outputs and log-sum-exps
 * (and nothing that must survive between calls). 0 for a direct plan.
 * Errors: as vat_plan; *bytes is then unchanged. */
vat_status_t vat_workspace_size(const vat_problem_t* problem, size_t* bytes);

/* The whole path: partial kernel, then (unless the plan is direct) the
 * log-sum-exp merge kernel, both on `stream`. sm_scale > 0, k_scale > 0 and
 * v_scale must be finite. workspace: device memory of at least
 * vat_workspace_size() bytes, 256-byte aligned (may be NULL when that size
 * is 0). Host-detectable problems return an error before anything is
 * enqueued. */
vat_status_t verify_attention(const vat_problem_t* problem, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* kv_indptr,
                              const int32_t* kv_indices, const int32_t* last_page_len,
                              const int32_t* qo_indptr, const uint8_t* mask,
                              const int32_t* mask_indptr, float sm_scale, float k_scale,
                              float v_scale, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream);

/* verify_attention with rotary position embedding applied to the queries
 * inside the partial kernel (FlashInfer page "feat: Separate Q and KV dtypes
 * for decode": RoPE applied on the fly in the attention kernels; a draft tree
 * needs it at each token's own position, FlashInfer page "How to implement a
 * tree attention with flashinfer"). q_cos_sin: device float32 [T, D], 16-byte
 * aligned; row r holds cos(th_0) .. cos(th_{D/2-1}), sin(th_0) ..
 * sin(th_{D/2-1}) of query token r's position. Query row r is rotated LLaMA
 * style -- dimension i pairs with i + D/2: q'_i = q_i c_i - q_{i+D/2} s_i,
 * q'_{i+D/2} = q_{i+D/2} c_i + q_i s_i -- in float32 with fused
 * multiply-adds; the rotated row enters the products as the sum of two bf16
 * rows (its bf16 rounding, then the bf16 rounding of what remains), about 16
 * significant bits. Cached keys are used as stored: a cache written with
 * vat_append_kv_rope holds rotated keys. problem->rope must be 1. */
vat_status_t verify_attention_rope(const vat_problem_t* problem, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* kv_indptr, const int32_t* kv_indices,
                                   const int32_t* last_page_len, const int32_t* qo_indptr,
                                   const uint8_t* mask, const int32_t* mask_indptr,
                                   const float* q_cos_sin, float sm_scale, float k_scale,
                                   float v_scale, void* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Largest workspace verify_attention_noalloc can serve (64 MiB). */
#define VAT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* verify_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same plan and kernels, with the workspace taken from a
 * static device array of VAT_NOALLOC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on until the process ends (its device address is
 * looked up on the first call on each device). Arguments and results as
 * verify_attention, without workspace and workspace_bytes. Returns
 * VAT_ERR_WORKSPACE, enqueueing nothing, when vat_workspace_size() of the
 * problem exceeds VAT_NOALLOC_SCRATCH_BYTES. Calls no hipMalloc, hipFree or
 * allocating routine. Every call on a GPU shares that GPU's one array, which
 * keeps the last call's contents: calls that overlap on one GPU (on
 * different streams, or graphs replayed concurrently) race and give
 * unspecified results; calls in one stream's order are safe. */
vat_status_t verify_attention_noalloc(const vat_problem_t* problem, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* kv_indptr, const int32_t* kv_indices,
                                      const int32_t* last_page_len, const int32_t* qo_indptr,
                                      const uint8_t* mask, const int32_t* mask_indptr,
                                      float sm_scale, float k_scale, float v_scale, void* out,
                                      float* lse, void* stream);

/* The two halves of verify_attention, for timing each kernel on its own
 * stream position. vat_launch_partial enqueues the partial kernel only (in a
 * direct plan it writes out and lse); vat_launch_merge enqueues the merge
 * only (a no-op returning VAT_OK for a direct plan) and must follow a
 * vat_launch_partial with identical arguments on the same stream. */
vat_status_t vat_launch_partial(const vat_problem_t* problem, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* kv_indptr,
                                const int32_t* kv_indices, const int32_t* last_page_len,
                                const int32_t* qo_indptr, const uint8_t* mask,
                                const int32_t* mask_indptr, float sm_scale, float k_scale,
                                float v_scale, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);
/* vat_launch_partial for verify_attention_rope (same q_cos_sin rows). */
vat_status_t vat_launch_partial_rope(const vat_problem_t* problem, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* kv_indptr, const int32_t* kv_indices,
                                     const int32_t* last_page_len, const int32_t* qo_indptr,
                                     const uint8_t* mask, const int32_t* mask_indptr,
                                     const float* q_cos_sin, float sm_scale, float k_scale,
                                     float v_scale, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);
vat_status_t vat_launch_merge(const vat_problem_t* problem, const int32_t* kv_indptr,
                              const int32_t* last_page_len, const int32_t* qo_indptr,
                              float v_scale, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Write the drafts' keys and values into the paged caches, rounded to the
 * cache dtype: the step before verification attention, which expects every
 * draft's key and value to be cached already (vLLM page "[WIP] Support for
 * cached multi-query attention towards speculative decoding").
 *
 * Row qo_indptr[b] + t of k_new / v_new ([T, Hkv, D], dense, in src_dtype:
 * VAT_F32 or VAT_BF16) is written to key position n = kv_len_b - L_b + t of
 * request b: slot n % page_size of page kv_indices[kv_indptr[b] + n /
 * page_size] (the paged format documented above), for t = 0 .. L_b - 1. The
 * stored element is x / scale (k_scale for keys, v_scale for values), the
 * inverse of the attention's read of scale * stored (flashmap page
 * "sglang/verify_attention.py", k_scale / v_scale folding): one IEEE binary32
 * division, then round-to-nearest-even into problem->kv_dtype -- fp32 as is,
 * bf16 (overflow to infinity as IEEE), e4m3fn after clamping to [-448, 448]
 * (saturating: the format has no infinity). A NaN input stores the canonical
 * quiet NaN of the cache dtype (0x7FC00000, 0x7FC0, 0x7F) with the input's
 * sign. Nothing else in the caches changes.
 *
 * Reads batch, num_kv_heads, head_dim (64 or 128), page_size, num_pages,
 * num_kv_indices, num_qo_tokens, max_qo_len (sizes the launch; rows beyond
 * it are still written), kv_dtype and num_cus (0 = query the current device)
 * of *problem; the other fields are ignored. k_scale and v_scale must be finite and > 0. k_new, v_new and the
 * caches must be 16-byte aligned. The same device-content contract as
 * verify_attention holds; index violations give unspecified cache contents
 * inside the caches, never an access outside them. Enqueues one kernel on
 * `stream`; allocates nothing; capturable. */
vat_status_t vat_append_kv(const vat_problem_t* problem, int32_t src_dtype, const void* k_new,
                           const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* kv_indptr, const int32_t* kv_indices,
                           const int32_t* last_page_len, const int32_t* qo_indptr, float k_scale,
                           float v_scale, void* stream);

/* vat_append_kv with the keys rotated by RoPE before they are scaled and
 * rounded (values are written as given). k_cos_sin: device float32 [T, D],
 * 16-byte aligned, row r = (cos th_i .., sin th_i ..) of draft row r's
 * position, the layout of verify_attention_rope. The rotation is evaluated in
 * binary32 with each product and each sum rounded on its own (no fused
 * multiply-add): k'_i = RN(RN(k_i c_i) - RN(k_{i+D/2} s_i)), k'_{i+D/2} =
 * RN(RN(k_{i+D/2} c_i) + RN(k_i s_i)); a NaN result (from a NaN input, or
 * infinity times zero) is the canonical positive quiet NaN. The stored code
 * of k' then follows the rules of vat_append_kv exactly. */
vat_status_t vat_append_kv_rope(const vat_problem_t* problem, int32_t src_dtype,
                                const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, const int32_t* kv_indptr,
                                const int32_t* kv_indices, const int32_t* last_page_len,
                                const int32_t* qo_indptr, const float* k_cos_sin, float k_scale,
                                float v_scale, void* stream);

/* Status bits of vat_check_inputs: which rule of the device-content contract
 * the arrays break (several may be set). */
#define VAT_CHECK_KV_INDPTR 1   /* kv_indptr[0] != 0, decreasing, or > num_kv_indices */
#define VAT_CHECK_KV_INDICES 2  /* a used page id outside [0, num_pages) */
#define VAT_CHECK_LAST_PAGE 4   /* last_page_len outside [1, page_size] (requests with pages) */
#define VAT_CHECK_QO_INDPTR 8   /* qo_indptr[0] != 0, decreasing, > T, or qo_indptr[B] != T */
#define VAT_CHECK_QO_LEN 16     /* L_b > max_qo_len or L_b > kv_len_b */
#define VAT_CHECK_MASK 32       /* a mask segment negative or past num_mask_bytes */

/* Debugging aid, not a step of the path: check the device-content contract
 * stated at the top of this header for the index arrays and mask offsets of
 * a call, and write to *status (device int32, caller-owned) the OR of the
 * VAT_CHECK_* bits of the rules they break, 0 when they keep all of them.
 * The paged-format rules are the FlashInfer page "feat: Separate Q and KV
 * dtypes for decode" (begin_forward docstring); the query and mask rules
 * are this header's layouts. Arguments as verify_attention (mask_indptr is
 * read only when has_mask; kv_indices only up to kv_indptr[B], cut to
 * num_kv_indices); every read stays inside the sizes *problem declares,
 * whatever the arrays hold. Enqueues two kernels on `stream` (clear, then
 * check), allocates nothing and is capturable; read *status after the
 * stream has reached them. Host errors (VAT_ERR_NULL, VAT_ERR_ALIGN for
 * int32 arrays not 4-byte aligned, and those of vat_plan's shape checks)
 * return before anything is enqueued. */
vat_status_t vat_check_inputs(const vat_problem_t* problem, const int32_t* kv_indptr,
                              const int32_t* kv_indices, const int32_t* last_page_len,
                              const int32_t* qo_indptr, const int32_t* mask_indptr,
                              int32_t* status, void* stream);

/* Measurement aid, not a step of the path: read `bytes` of device memory at
 * `buf` once, start to end, with 16-byte non-temporal loads spread over
 * every compute unit (eight workgroups per CU), and enqueue nothing else.
 * The time it takes gives the HBM read rate reachable with the plainest
 * access pattern, reported beside the chip's published peak when the
 * attention kernels' bandwidth is judged. buf: 16-byte aligned, bytes a
 * multiple of 16 (VAT_ERR_ALIGN / VAT_ERR_SHAPE otherwise); sink: one
 * device uint32 that the kernel almost never writes (it exists so that the
 * loads cannot be optimised away). bytes == 0 enqueues nothing. */
vat_status_t vat_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Static description of a status code. */
const char* vat_status_string(vat_status_t status);

/* ABI version of this header (bumped on any incompatible change). */
int32_t vat_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_VERIFY_ATTENTION_H */
