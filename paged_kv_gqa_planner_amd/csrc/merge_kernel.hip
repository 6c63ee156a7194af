// Log-sum-exp merge of a request's chunk partials (flashmap page
// "sglang/verify_attention.py", _verify_merge_kernel): each chunk's
// normalised output is weighted by its share of the softmax mass,
// w_i = 2^(lse_i - max lse), and the merged lse is max + log2(sum w).
//
// One wave per query row (each lane owns D / 64 head dims), four rows per
// workgroup: the partials' lse give their max and weights, then the weighted
// sum of their rows is formed. A request's partials
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

  // The first U partial rows are requested together with every partial's
  // base-2 lse (lane i holds partials i, i + 64, ...), so a request with up
  // to U partials costs one round of loads after its geometry.
  constexpr int U = 16;
  auto load_row = [&](int i, float (&v)[PER]) {
    const float* po = a.part_o + slot(i) * D + lane * PER;
    if constexpr (PER == 2) {
      const float2 x2 = *(const float2*)po;
      v[0] = x2.x;
      v[1] = x2.y;
    } else {
      v[0] = po[0];
    }
  };
  // Only rows that exist are requested (n is wave-uniform).
  float v0[U][PER];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u < n) load_row(u, v0[u]);
  const float ls0 = lane < n ? a.part_lse[slot(lane)] : kNegInf;
  float m = ls0;
  for (int i = lane + 64; i < n; i += 64) m = fmaxf(m, a.part_lse[slot(i)]);
  m = wave_max(m);
  const float mb = (m == kNegInf) ? 0.f : m;
  // Weights w_i = 2^(lse_i - max) (0 for an empty partial) and the weighted
  // sum of the rows; rows past the first U are requested U at a time.
  float den = 0.f;
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const float lsi = base == 0 ? ls0 : (i < n ? a.part_lse[slot(i)] : kNegInf);
    const float w = fast_exp2(lsi - mb);
    den += w;
    const int cnt = min(64, n - base);
    for (int j0 = 0; j0 < cnt; j0 += U) {
      float v[U][PER], wj[U];
      const bool first = base == 0 && j0 == 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (j0 + u >= cnt) break;
        wj[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j0 + u));
        if (first) {
#pragma unroll
          for (int k = 0; k < PER; ++k) v[u][k] = v0[u][k];
        } else {
          load_row(base + j0 + u, v[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (j0 + u >= cnt) break;
#pragma unroll
        for (int k = 0; k < PER; ++k) o[k] += wj[u] * v[u][k];
      }
    }
  }
  den = wave_sum(den);
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
