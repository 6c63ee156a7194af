// Log-sum-exp merge of a request's chunk partials (flashmap page
// "sglang/verify_attention.py", _verify_merge_kernel): each chunk's
// normalised output is weighted by its share of the softmax mass,
// w_i = 2^(lse_i - max lse), and the merged lse is max + log2(sum w).
//
// One wave per query row (each lane owns D / 64 head dims), four rows per
// workgroup, partials combined online eight at a time. A request's partials
// are its chunks (ids from chunk_start) or, with balanced slices of the
// page-index space, the slices x_lo .. x_hi its pages fall in (slot x + b). Requests that fit one chunk or
// slice were written directly by the partial kernel and are skipped.
#include "device_common.h"

namespace vat {

template <int QF32, int D>
__global__ __launch_bounds__(kMergeThreads) void vat_merge(MergeArgs a) {
  constexpr int PER = D / 64;  // head dims per lane
  const int lane = threadIdx.x & 63;
  const int lr = threadIdx.x >> 6;  // row within the group
  int x = blockIdx.x;
  const int rg = x % a.row_groups;
  x /= a.row_groups;
  const int rb = x % a.row_blocks;
  x /= a.row_blocks;
  const int h = x % a.hkv;
  const int b = x / a.hkv;
  Req r;
  int n, first;  // partials of request b: slots first + i, i < n
  if (a.slices > 0) {
    // Slices of the page-index space, `per` pages each: request b's pages
    // [kv_indptr[b], kv_indptr[b + 1]) fall in slices x_lo .. x_hi.
    r = make_req(a.kv_indptr[b], a.kv_indptr[b + 1], a.last_page_len[b], a.qo_indptr[b],
                 a.qo_indptr[b + 1], 0, a.page_shift, a.num_kv_indices, a.tokens);
    if (r.L == 0 || r.pages == 0) return;
    const int per = (a.num_kv_indices + a.slices - 1) / a.slices;
    const int x_lo = r.kv_start / per;
    const int x_hi = (r.kv_start + r.pages - 1) / per;
    n = x_hi - x_lo + 1;
    first = x_lo + b;
  } else {
    r = make_req(a.kv_indptr[b], a.kv_indptr[b + 1], a.last_page_len[b], a.qo_indptr[b],
                 a.qo_indptr[b + 1], 0, a.page_shift, a.num_kv_indices, a.tokens);
    n = chunk_count(r.kv_len, a.chunk_keys);
    first = chunk_start(r.kv_start, a.page_shift, a.chunk_keys, b);
  }
  if (n <= 1) return;  // written directly by the partial kernel
  const int local = rg * kMergeRows + lr;
  const int row = rb * a.rows_per_block + local;
  if (local >= a.rows_per_block || row >= a.group * r.L) return;
  const int t = row / a.group, g = row % a.group;
  auto slot = [&](int i) -> long long {
    const int cid = min(first + i, a.num_ids - 1);
    return (((long long)cid * a.hkv + h) * a.row_blocks + rb) * a.rows_per_block + local;
  };

  // Online combination, eight chunks per round: their lse and output rows
  // are all requested before any is used, so a request with up to eight
  // chunks costs one round of loads.
  constexpr int U = 8;
  float m = kNegInf, den = 0.f;
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  for (int base = 0; base < n; base += U) {
    float ls[U];
    float v[U][PER];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = base + u < n;
      const long long sl = slot(in ? base + u : 0);
      ls[u] = in ? a.part_lse[sl] : kNegInf;
      const float* po = a.part_o + sl * D + lane * PER;
      if constexpr (PER == 2) {
        const float2 x2 = in ? *(const float2*)po : float2{0.f, 0.f};
        v[u][0] = x2.x;
        v[u][1] = x2.y;
      } else {
        v[u][0] = in ? po[0] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float m_new = fmaxf(m, ls[u]);
      const float mb = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m - mb);  // 0 while m is -inf
      const float w = fast_exp2(ls[u] - mb);  // 0 for an empty chunk
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] = o[k] * alpha + v[u][k] * w;
      den = den * alpha + w;
      m = m_new;
    }
  }
  const float mb = (m == kNegInf) ? 0.f : m;
  const long long orow = (long long)(r.q_start + t) * a.hq + h * a.group + g;
  const float sc = den > 0.f ? a.v_scale / den : 0.f;
  if constexpr (QF32) {
    float* op = (float*)a.out + orow * D + lane * PER;
#pragma unroll
    for (int k = 0; k < PER; ++k) op[k] = o[k] * sc;
  } else {
    unsigned short* op = (unsigned short*)a.out + orow * D + lane * PER;
    if constexpr (PER == 2) *(unsigned*)op = pack_bf16x2(o[0] * sc, o[1] * sc);
    else op[0] = (unsigned short)f32_to_bf16_bits(o[0] * sc);
  }
  if (lane == 0) a.lse[orow] = den > 0.f ? (mb + fast_log2(den)) * kLn2 : kNegInf;
}

const void* merge_kernel(int q_is_f32, int head_dim) {
  if (q_is_f32) return (const void*)(head_dim == 64 ? vat_merge<1, 64> : vat_merge<1, 128>);
  return (const void*)(head_dim == 64 ? vat_merge<0, 64> : vat_merge<0, 128>);
}

}  // namespace vat
