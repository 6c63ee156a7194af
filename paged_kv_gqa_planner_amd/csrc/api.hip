// C ABI: host validation, shape-only planning and kernel launches on the
// caller's stream. Never allocates, frees, synchronises or reads device
// memory, so calls can be captured into a HIP graph.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "plan.h"
#include "verify_attention.h"

namespace vat {
const void* tile_kernel(int kv_dtype, int head_dim, int rt);
const void* stream_kernel(int kv_dtype, int head_dim, int rt, int dma_waves, int pair,
                          int mask_mode, int rope, int heads_per_group, int stages);
const void* merge_kernel(int q_is_f32, int head_dim, int rows_per_workgroup, int one_slice_request);
const void* append_kernel(int src_dtype, int cache_dtype, int pow2_scales, int units);
const void* append_rope_kernel(int src_dtype, int cache_dtype, int pow2_scales);
const void* read_probe_kernel();
}  // namespace vat

namespace {

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];  // 0 = not yet queried

// Workspace of verify_attention_noalloc: one static array in each device's
// copy of the code object, zero at load and held until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory; its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is used.
constexpr size_t kScratchBytes = VAT_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch keeps the workspace's 256-byte alignment");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_scratch_mu;

vat_status_t device_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VAT_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return VAT_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return VAT_OK;
}

vat_status_t device_cus(int32_t* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return VAT_ERR_HIP;
  if (dev < kMaxDevices && g_cu_count[dev] > 0) {
    *cus = g_cu_count[dev];
    return VAT_OK;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return VAT_ERR_HIP;
  if (dev < kMaxDevices) g_cu_count[dev] = n;
  *cus = n;
  return VAT_OK;
}

vat_status_t plan_for(const vat_problem_t* p, vat_plan_t* plan) {
  vat_status_t st = vat::validate_problem(p);
  if (st != VAT_OK) return st;
  int32_t cus = p->num_cus;
  if (cus == 0) {
    st = device_cus(&cus);
    if (st != VAT_OK) return st;
  }
  return vat::make_plan(p, cus, plan);
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

bool plan_is_empty(const vat_plan_t& plan) { return plan.grid_x == 0 || plan.grid_y == 0; }

bool pow2_normal(float s) {
  uint32_t u;
  memcpy(&u, &s, sizeof(u));
  const uint32_t e = (u >> 23) & 0xffu;
  return (u >> 31) == 0 && (u & 0x7fffffu) == 0 && e >= 1 && e <= 253;
}

int page_shift(int32_t page_size) {
  int s = 0;
  while ((1 << s) < page_size) ++s;
  return s;
}

// Everything verify_attention checks before enqueueing, shared by the
// split launch entry points.
vat_status_t prepare(const vat_problem_t* p, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* kv_indptr, const int32_t* kv_indices,
                     const int32_t* last_page_len, const int32_t* qo_indptr, const uint8_t* mask,
                     const int32_t* mask_indptr, const float* q_cos_sin, float sm_scale,
                     float k_scale, float v_scale, void* out, float* lse, void* workspace,
                     size_t workspace_bytes, vat_plan_t* plan) {
  vat_status_t st = plan_for(p, plan);
  if (st != VAT_OK) return st;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale) || !(k_scale > 0.f) || !isfinite(k_scale) ||
      !isfinite(v_scale))
    return VAT_ERR_SHAPE;
  if (plan_is_empty(*plan)) return VAT_OK;
  if (!q || !k_cache || !v_cache || !kv_indptr || !kv_indices || !last_page_len || !qo_indptr ||
      !out || !lse)
    return VAT_ERR_NULL;
  if (p->has_mask && (!mask || !mask_indptr)) return VAT_ERR_NULL;
  if (p->rope && !q_cos_sin) return VAT_ERR_NULL;
  if (p->rope && !aligned(q_cos_sin, 16)) return VAT_ERR_ALIGN;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(lse, 4) || !aligned(kv_indptr, 4) || !aligned(kv_indices, 4) ||
      !aligned(last_page_len, 4) || !aligned(qo_indptr, 4) ||
      (mask_indptr && !aligned(mask_indptr, 4)))
    return VAT_ERR_ALIGN;
  if (plan->workspace_bytes > 0) {
    if (!workspace) return VAT_ERR_NULL;
    if (workspace_bytes < (size_t)plan->workspace_bytes) return VAT_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return VAT_ERR_ALIGN;
  }
  return VAT_OK;
}

vat_status_t launch_partial(const vat_problem_t* p, const vat_plan_t& plan, const void* q,
                            const void* k_cache, const void* v_cache, const int32_t* kv_indptr,
                            const int32_t* kv_indices, const int32_t* last_page_len,
                            const int32_t* qo_indptr, const uint8_t* mask,
                            const int32_t* mask_indptr, const float* q_cos_sin,
                            float sm_scale, float k_scale, float v_scale, void* out, float* lse,
                            void* workspace, hipStream_t stream) {
  vat::PartialArgs a;
  a.q_cos_sin = p->rope ? q_cos_sin : nullptr;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.last_page_len = last_page_len;
  a.qo_indptr = qo_indptr;
  a.mask = p->has_mask ? mask : nullptr;
  a.mask_indptr = p->has_mask ? mask_indptr : nullptr;
  a.out = out;
  a.lse = lse;
  a.part_o = plan.direct ? nullptr : (float*)workspace;
  a.part_lse = plan.direct ? nullptr
                           : (float*)((char*)workspace +
                                      vat::workspace_lse_offset(plan, p->head_dim, p->num_kv_heads));
  a.c_log2 = (float)((double)sm_scale * (double)k_scale * 1.4426950408889634);
  a.v_scale = v_scale;
  a.batch = p->batch;
  a.hq = p->num_qo_heads;
  a.hkv = p->num_kv_heads;
  a.group = plan.group;
  a.tokens = p->num_qo_tokens;
  a.page_shift = page_shift(p->page_size);
  a.num_pages = p->num_pages;
  a.num_kv_indices = p->num_kv_indices;
  a.num_mask_bytes = p->has_mask ? p->num_mask_bytes : 0;
  a.rows_per_block = plan.rows_per_block;
  a.row_blocks = plan.row_blocks;
  a.waves_rows = plan.waves_rows;
  a.waves_keys = plan.waves_keys;
  a.chunk_keys = plan.chunk_keys;
  a.num_ids = plan.num_chunk_ids;
  a.has_mask = p->has_mask;
  a.slices = plan.slices;
  a.block_order = plan.block_order;
  const void* fn = plan.kernel == 1 ? vat::stream_kernel(p->kv_dtype, p->head_dim,
                                                          plan.row_tiles_per_wave, plan.dma_waves,
                                                          plan.waves_keys, p->has_mask, p->rope,
                                                          plan.heads_per_group, plan.stages)
                                     : vat::tile_kernel(p->kv_dtype, p->head_dim,
                                                        plan.row_tiles_per_wave);
  if (plan.lds_bytes > 65536) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, plan.lds_bytes) !=
        hipSuccess)
      return VAT_ERR_HIP;
  }
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(fn, dim3(plan.grid_x, plan.grid_y, 1), dim3(plan.threads, 1, 1),
                                 args, (size_t)plan.lds_bytes, stream);
  return e == hipSuccess ? VAT_OK : VAT_ERR_HIP;
}

vat_status_t launch_merge(const vat_problem_t* p, const vat_plan_t& plan,
                          const int32_t* kv_indptr, const int32_t* last_page_len,
                          const int32_t* qo_indptr, float v_scale, void* out, float* lse,
                          void* workspace, hipStream_t stream) {
  if (plan.direct || plan.merge_grid == 0) return VAT_OK;
  vat::MergeArgs a;
  a.part_o = (const float*)workspace;
  a.part_lse =
      (const float*)((char*)workspace + vat::workspace_lse_offset(plan, p->head_dim, p->num_kv_heads));
  a.kv_indptr = kv_indptr;
  a.last_page_len = last_page_len;
  a.qo_indptr = qo_indptr;
  a.out = out;
  a.lse = lse;
  a.v_scale = v_scale;
  a.batch = p->batch;
  a.hq = p->num_qo_heads;
  a.hkv = p->num_kv_heads;
  a.group = plan.group;
  a.tokens = p->num_qo_tokens;
  a.page_shift = page_shift(p->page_size);
  a.num_kv_indices = p->num_kv_indices;
  a.rows_per_block = plan.rows_per_block;
  a.row_blocks = plan.row_blocks;
  a.chunk_keys = plan.chunk_keys;
  a.num_ids = plan.num_chunk_ids;
  a.row_groups = (plan.rows_per_block + plan.merge_rows - 1) / plan.merge_rows;
  a.slices = plan.slices;
  const void* fn = vat::merge_kernel(p->q_dtype == VAT_F32, p->head_dim, plan.merge_rows,
                                     plan.slices > 0 && p->batch == 1);
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(fn, dim3(plan.merge_grid, 1, 1), dim3(plan.merge_threads, 1, 1),
                                 args, 0, stream);
  return e == hipSuccess ? VAT_OK : VAT_ERR_HIP;
}

// The cache write; `rope` asks for keys rotated by the per-token cos/sin
// rows `k_cos_sin` first.
vat_status_t append_kv(const vat_problem_t* problem, int32_t src_dtype, const void* k_new,
                       const void* v_new, void* k_cache, void* v_cache, const int32_t* kv_indptr,
                       const int32_t* kv_indices, const int32_t* last_page_len,
                       const int32_t* qo_indptr, const float* k_cos_sin, bool rope,
                       float k_scale, float v_scale, hipStream_t stream) {
  vat_status_t st = vat::validate_append(problem, src_dtype);
  if (st != VAT_OK) return st;
  if (!(k_scale > 0.f) || !isfinite(k_scale) || !(v_scale > 0.f) || !isfinite(v_scale))
    return VAT_ERR_SHAPE;
  const vat_problem_t& p = *problem;
  if (p.batch == 0 || p.num_qo_tokens == 0 || p.max_qo_len == 0) return VAT_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !kv_indptr || !kv_indices || !last_page_len ||
      !qo_indptr || (rope && !k_cos_sin))
    return VAT_ERR_NULL;
  if (rope && !aligned(k_cos_sin, 16)) return VAT_ERR_ALIGN;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(kv_indptr, 4) || !aligned(kv_indices, 4) ||
      !aligned(last_page_len, 4) || !aligned(qo_indptr, 4))
    return VAT_ERR_ALIGN;
  vat::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.last_page_len = last_page_len;
  a.qo_indptr = qo_indptr;
  a.k_cos_sin = rope ? k_cos_sin : nullptr;
  a.head_dim = p.head_dim;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  // A normal power of two has an exact reciprocal (2^-126 .. 2^126, the
  // smallest as a subnormal), so x * (1 / s) rounds x / s exactly.
  const bool pow2 = pow2_normal(k_scale) && pow2_normal(v_scale);
  a.k_inv = pow2 ? 1.0f / k_scale : 0.f;
  a.v_inv = pow2 ? 1.0f / v_scale : 0.f;
  a.batch = p.batch;
  a.row_units = p.num_kv_heads * p.head_dim / 8;
  a.page_shift = page_shift(p.page_size);
  a.num_pages = p.num_pages;
  a.num_kv_indices = p.num_kv_indices;
  a.tokens = p.num_qo_tokens;
  // Two 8-element units per thread when the write covers every CU's 2048
  // threads at least four times over (measured: 3 % to 12 % faster there);
  // one otherwise, which halves the per-thread latency chain of small writes.
  int32_t cus = p.num_cus;
  if (cus == 0) {
    st = device_cus(&cus);
    if (st != VAT_OK) return st;
  }
  const int64_t total_units = 2 * int64_t(p.num_qo_tokens) * a.row_units;
  const int units_per_thread = total_units >= int64_t(4) * cus * 2048 ? 2 : 1;
  // Grid y covers max_qo_len tokens of K and V per request; the kernel loops
  // over any remainder, so the bound only sizes the launch.
  const int64_t units = 2 * int64_t(p.max_qo_len) * a.row_units;
  const int64_t per_block = int64_t(vat::kAppendThreads) * (rope ? 1 : units_per_thread);
  const int64_t gy = (units + per_block - 1) / per_block;
  const void* fn = rope ? vat::append_rope_kernel(src_dtype, p.kv_dtype, pow2 ? 1 : 0)
                        : vat::append_kernel(src_dtype, p.kv_dtype, pow2 ? 1 : 0, units_per_thread);
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)p.batch, (unsigned)(gy < 65535 ? gy : 65535), 1),
                                 dim3(vat::kAppendThreads, 1, 1), args, 0, stream);
  return e == hipSuccess ? VAT_OK : VAT_ERR_HIP;
}

}  // namespace

extern "C" {

vat_status_t vat_plan(const vat_problem_t* problem, vat_plan_t* plan) {
  if (!problem || !plan) return VAT_ERR_NULL;
  return plan_for(problem, plan);
}

vat_status_t vat_workspace_size(const vat_problem_t* problem, size_t* bytes) {
  if (!problem || !bytes) return VAT_ERR_NULL;
  vat_plan_t plan;
  vat_status_t st = plan_for(problem, &plan);
  if (st != VAT_OK) return st;
  *bytes = (size_t)plan.workspace_bytes;
  return VAT_OK;
}

vat_status_t vat_launch_partial(const vat_problem_t* problem, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* kv_indptr,
                                const int32_t* kv_indices, const int32_t* last_page_len,
                                const int32_t* qo_indptr, const uint8_t* mask,
                                const int32_t* mask_indptr, float sm_scale, float k_scale,
                                float v_scale, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream) {
  vat_plan_t plan;
  vat_status_t st = prepare(problem, q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                            qo_indptr, mask, mask_indptr, nullptr, sm_scale, k_scale, v_scale,
                            out, lse, workspace, workspace_bytes, &plan);
  if (st != VAT_OK || plan_is_empty(plan)) return st;
  return launch_partial(problem, plan, q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                        qo_indptr, mask, mask_indptr, nullptr, sm_scale, k_scale, v_scale, out,
                        lse, workspace, (hipStream_t)stream);
}

vat_status_t vat_launch_partial_rope(const vat_problem_t* problem, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* kv_indptr, const int32_t* kv_indices,
                                     const int32_t* last_page_len, const int32_t* qo_indptr,
                                     const uint8_t* mask, const int32_t* mask_indptr,
                                     const float* q_cos_sin, float sm_scale, float k_scale,
                                     float v_scale, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  vat_plan_t plan;
  vat_status_t st = prepare(problem, q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                            qo_indptr, mask, mask_indptr, q_cos_sin, sm_scale, k_scale, v_scale,
                            out, lse, workspace, workspace_bytes, &plan);
  if (st != VAT_OK || plan_is_empty(plan)) return st;
  return launch_partial(problem, plan, q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                        qo_indptr, mask, mask_indptr, q_cos_sin, sm_scale, k_scale, v_scale, out,
                        lse, workspace, (hipStream_t)stream);
}

vat_status_t vat_launch_merge(const vat_problem_t* problem, const int32_t* kv_indptr,
                              const int32_t* last_page_len, const int32_t* qo_indptr,
                              float v_scale, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream) {
  vat_plan_t plan;
  vat_status_t st = plan_for(problem, &plan);
  if (st != VAT_OK) return st;
  if (!isfinite(v_scale)) return VAT_ERR_SHAPE;
  if (plan_is_empty(plan) || plan.direct) return VAT_OK;
  if (!kv_indptr || !last_page_len || !qo_indptr || !out || !lse || !workspace) return VAT_ERR_NULL;
  if (workspace_bytes < (size_t)plan.workspace_bytes) return VAT_ERR_WORKSPACE;
  if (!aligned(workspace, 256) || !aligned(out, 16) || !aligned(lse, 4)) return VAT_ERR_ALIGN;
  return launch_merge(problem, plan, kv_indptr, last_page_len, qo_indptr, v_scale, out, lse,
                      workspace, (hipStream_t)stream);
}

vat_status_t verify_attention(const vat_problem_t* problem, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* kv_indptr,
                              const int32_t* kv_indices, const int32_t* last_page_len,
                              const int32_t* qo_indptr, const uint8_t* mask,
                              const int32_t* mask_indptr, float sm_scale, float k_scale,
                              float v_scale, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return verify_attention_rope(problem, q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                               qo_indptr, mask, mask_indptr, nullptr, sm_scale, k_scale, v_scale,
                               out, lse, workspace, workspace_bytes, stream);
}

vat_status_t verify_attention_rope(const vat_problem_t* problem, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* kv_indptr, const int32_t* kv_indices,
                                   const int32_t* last_page_len, const int32_t* qo_indptr,
                                   const uint8_t* mask, const int32_t* mask_indptr,
                                   const float* q_cos_sin, float sm_scale, float k_scale,
                                   float v_scale, void* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  vat_plan_t plan;
  vat_status_t st = prepare(problem, q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                            qo_indptr, mask, mask_indptr, q_cos_sin, sm_scale, k_scale, v_scale,
                            out, lse, workspace, workspace_bytes, &plan);
  if (st != VAT_OK || plan_is_empty(plan)) return st;
  st = launch_partial(problem, plan, q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                      qo_indptr, mask, mask_indptr, q_cos_sin, sm_scale, k_scale, v_scale, out,
                      lse, workspace, (hipStream_t)stream);
  if (st != VAT_OK) return st;
  return launch_merge(problem, plan, kv_indptr, last_page_len, qo_indptr, v_scale, out, lse,
                      workspace, (hipStream_t)stream);
}

vat_status_t verify_attention_noalloc(const vat_problem_t* problem, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* kv_indptr, const int32_t* kv_indices,
                                      const int32_t* last_page_len, const int32_t* qo_indptr,
                                      const uint8_t* mask, const int32_t* mask_indptr,
                                      float sm_scale, float k_scale, float v_scale, void* out,
                                      float* lse, void* stream) {
  vat_plan_t plan;
  vat_status_t st = plan_for(problem, &plan);
  if (st != VAT_OK) return st;
  if ((uint64_t)plan.workspace_bytes > (uint64_t)kScratchBytes) return VAT_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.workspace_bytes > 0 && !plan_is_empty(plan)) {
    st = device_scratch(&ws);
    if (st != VAT_OK) return st;
  }
  st = prepare(problem, q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len, qo_indptr,
               mask, mask_indptr, nullptr, sm_scale, k_scale, v_scale, out, lse, ws,
               ws ? kScratchBytes : 0, &plan);
  if (st != VAT_OK || plan_is_empty(plan)) return st;
  st = launch_partial(problem, plan, q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                      qo_indptr, mask, mask_indptr, nullptr, sm_scale, k_scale, v_scale, out,
                      lse, ws, (hipStream_t)stream);
  if (st != VAT_OK) return st;
  return launch_merge(problem, plan, kv_indptr, last_page_len, qo_indptr, v_scale, out, lse, ws,
                      (hipStream_t)stream);
}

vat_status_t vat_append_kv(const vat_problem_t* problem, int32_t src_dtype, const void* k_new,
                           const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* kv_indptr, const int32_t* kv_indices,
                           const int32_t* last_page_len, const int32_t* qo_indptr, float k_scale,
                           float v_scale, void* stream) {
  return append_kv(problem, src_dtype, k_new, v_new, k_cache, v_cache, kv_indptr, kv_indices,
                   last_page_len, qo_indptr, nullptr, false, k_scale, v_scale,
                   (hipStream_t)stream);
}

vat_status_t vat_append_kv_rope(const vat_problem_t* problem, int32_t src_dtype,
                                const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, const int32_t* kv_indptr,
                                const int32_t* kv_indices, const int32_t* last_page_len,
                                const int32_t* qo_indptr, const float* k_cos_sin, float k_scale,
                                float v_scale, void* stream) {
  return append_kv(problem, src_dtype, k_new, v_new, k_cache, v_cache, kv_indptr, kv_indices,
                   last_page_len, qo_indptr, k_cos_sin, true, k_scale, v_scale,
                   (hipStream_t)stream);
}

vat_status_t vat_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return VAT_OK;
  if (!buf || !sink) return VAT_ERR_NULL;
  if (bytes % 16 || bytes / 16 > (size_t)INT64_MAX) return VAT_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return VAT_ERR_ALIGN;
  int32_t cus = 0;
  vat_status_t st = device_cus(&cus);
  if (st != VAT_OK) return st;
  // Eight workgroups of four waves per CU; each lane keeps four 16-byte loads
  // in flight per round.
  const long long n16 = (long long)(bytes / 16);
  const long long per_round = 256LL * 4;
  long long grid = (n16 + per_round - 1) / per_round;
  if (grid > 8LL * cus) grid = 8LL * cus;
  long long n = n16;
  void* args[] = {&buf, &n, &sink};
  hipError_t e = hipLaunchKernel(vat::read_probe_kernel(), dim3((unsigned)grid, 1, 1), dim3(256, 1, 1),
                                 args, 0, (hipStream_t)stream);
  return e == hipSuccess ? VAT_OK : VAT_ERR_HIP;
}

const char* vat_status_string(vat_status_t status) {
  switch (status) {
    case VAT_OK: return "ok";
    case VAT_ERR_NULL: return "a required pointer is NULL";
    case VAT_ERR_SHAPE: return "inconsistent shapes or invalid scales";
    case VAT_ERR_UNSUPPORTED: return "head_dim, page_size, dtype pair or mask length not supported";
    case VAT_ERR_ALIGN: return "q, caches, out or workspace misaligned";
    case VAT_ERR_WORKSPACE: return "workspace too small";
    case VAT_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t vat_abi_version(void) { return 5; }

}  // extern "C"
