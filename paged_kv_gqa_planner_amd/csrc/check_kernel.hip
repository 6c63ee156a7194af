// Device-content check of a call's index arrays and mask segments: a
// debugging aid, not a step of the path. The attention kernels never read
// an index without clamping it, so contents that break the contract give
// wrong numbers rather than faults; this kernel names the broken rule.
//
// The rules are those of the paged format (FlashInfer page "feat: Separate
// Q and KV dtypes for decode", begin_forward docstring: kv_indptr /
// kv_indices / last_page_len, kv_len = (pages - 1) * page_size +
// last_page_len) and of the query and mask segments the header documents.
// Every read stays inside the array sizes the problem declares, whatever the
// arrays hold.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"
#include "verify_attention.h"

namespace vat {
namespace {

struct CheckArgs {
  const int32_t* kv_indptr;    // [batch + 1]
  const int32_t* kv_indices;   // [num_kv_indices]
  const int32_t* last_page_len;  // [batch]
  const int32_t* qo_indptr;    // [batch + 1]
  const int32_t* mask_indptr;  // [batch] (has_mask only)
  int32_t* status;
  int batch, num_kv_indices, num_pages, page_size, tokens, max_qo_len;
  int has_mask, num_mask_bytes;
};

// Status bits (the header's VAT_CHECK_* values).
constexpr int kCheckKvIndptr = 1, kCheckKvIndices = 2, kCheckLastPage = 4, kCheckQoIndptr = 8,
              kCheckQoLen = 16, kCheckMask = 32;

// One thread clears the status word before the check runs (a kernel, not a
// memset, so the pair can be captured into a graph). The address depends on
// the lane, so the store is a vector store.
__global__ void vat_check_clear(int32_t* status) {
  if (threadIdx.x == 0) status[threadIdx.x] = 0;
}

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void vat_check(CheckArgs a) {
  const int nth = (int)(gridDim.x * blockDim.x);
  const int tid = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  int bits = 0;
  if (tid == 0) {
    if (a.kv_indptr[0] != 0) bits |= kCheckKvIndptr;
    if (a.qo_indptr[0] != 0 || a.qo_indptr[a.batch] != a.tokens) bits |= kCheckQoIndptr;
  }
  for (long long b = tid; b < a.batch; b += nth) {
    const long long kv0 = a.kv_indptr[b], kv1 = a.kv_indptr[b + 1];
    const long long q0 = a.qo_indptr[b], q1 = a.qo_indptr[b + 1];
    if (kv1 < kv0 || kv1 > a.num_kv_indices) bits |= kCheckKvIndptr;
    if (q1 < q0 || q1 > a.tokens) bits |= kCheckQoIndptr;
    const long long pages = kv1 > kv0 ? kv1 - kv0 : 0;
    const long long L = q1 > q0 ? q1 - q0 : 0;
    const int lp = a.last_page_len[b];
    if (pages > 0 && (lp < 1 || lp > a.page_size)) bits |= kCheckLastPage;
    const long long kv_len = pages > 0 ? (pages - 1) * a.page_size + lp : 0;
    if (L > a.max_qo_len || L > kv_len) bits |= kCheckQoLen;
    if (a.has_mask && L > 0) {
      // The segment needs ceil(L * L / 8) bytes (packed blocks) or L rows of
      // kv_len bytes (full byte rows: prefix plus drafts). Arbitrary contents
      // can overflow those products, so each is compared by division:
      // x * y > r  <=>  y > floor(r / x) for positive x, y and r >= 0.
      const long long m0 = a.mask_indptr[b];
      const long long room = (long long)a.num_mask_bytes - m0;
      const bool over = a.has_mask == 1 ? L > (8 * room) / L : kv_len > room / L;
      if (m0 < 0 || room < 0 || over) bits |= kCheckMask;
    }
  }
  // Page ids the requests use: kv_indices[0 .. kv_indptr[B]), cut to the
  // declared capacity.
  long long used = a.kv_indptr[a.batch];
  used = used < 0 ? 0 : (used > a.num_kv_indices ? a.num_kv_indices : used);
  for (long long i = tid; i < used; i += nth) {
    const int pg = a.kv_indices[i];
    if (pg < 0 || pg >= a.num_pages) bits |= kCheckKvIndices;
  }
  if (bits) atomicOr(a.status, bits);
}

}  // namespace

}  // namespace vat

extern "C" vat_status_t vat_check_inputs(const vat_problem_t* problem, const int32_t* kv_indptr,
                                         const int32_t* kv_indices, const int32_t* last_page_len,
                                         const int32_t* qo_indptr, const int32_t* mask_indptr,
                                         int32_t* status, void* stream) {
  const vat_status_t st = vat::validate_problem(problem);
  if (st != VAT_OK) return st;
  const vat_problem_t& p = *problem;
  if (!status || !kv_indptr || !qo_indptr) return VAT_ERR_NULL;
  if (p.batch > 0 && !last_page_len) return VAT_ERR_NULL;
  if (p.num_kv_indices > 0 && !kv_indices) return VAT_ERR_NULL;
  if (p.has_mask && p.batch > 0 && !mask_indptr) return VAT_ERR_NULL;
  const auto misaligned = [](const void* ptr) { return reinterpret_cast<uintptr_t>(ptr) % 4 != 0; };
  if (misaligned(status) || misaligned(kv_indptr) || misaligned(kv_indices) ||
      misaligned(last_page_len) || misaligned(qo_indptr) || misaligned(mask_indptr))
    return VAT_ERR_ALIGN;
  const vat::CheckArgs a{kv_indptr,   kv_indices,     last_page_len, qo_indptr,
                         mask_indptr, status,         p.batch,       p.num_kv_indices,
                         p.num_pages, p.page_size,    p.num_qo_tokens, p.max_qo_len,
                         p.has_mask,  p.num_mask_bytes};
  const hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(vat::vat_check_clear, dim3(1), dim3(64), 0, s, status);
  if (hipGetLastError() != hipSuccess) return VAT_ERR_HIP;
  const long long work = p.batch > p.num_kv_indices ? p.batch : p.num_kv_indices;
  long long blocks = (work + vat::kCheckThreads - 1) / vat::kCheckThreads;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  hipLaunchKernelGGL(vat::vat_check, dim3((unsigned)blocks), dim3(vat::kCheckThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? VAT_OK : VAT_ERR_HIP;
}
