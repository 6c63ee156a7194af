// Log-sum-exp merge of a request's chunk partials (flashmap page
// "sglang/verify_attention.py", _verify_merge_kernel): each chunk's
// normalised output is weighted by its share of the softmax mass,
// w_i = 2^(lse_i - max lse), and the merged lse is max + log2(sum w).
//
// A request's partials are its chunks (ids from chunk_start) or, with
// balanced slices of the page-index space, the slices x_lo .. x_hi its pages
// fall in (slot x + b). Requests that fit one chunk or slice were written
// directly by the partial kernel and are skipped.
#include "device_common.h"

namespace vat {

// Sixteen lanes own one row's D head dims, D / 16 consecutive dims each, so
// one partial row is two (D 128) or one 16-byte load per lane. Without SPLIT
// a wave merges four rows (requests with few partials); with SPLIT it merges
// one row and its four 16-lane groups take every fourth partial, so up to 4 U
// partials arrive in one round of loads, and the groups combine at the end.
// Every lane reads the lse values of its own partials (the 16 lanes of a
// group share each address), so the weights need no cross-lane traffic; a
// row with more partials than one round holds takes several rounds, combined
// with a running max that rescales what came before.
//
// PRE (one request over balanced slices): the request's pages start at index
// 0, so its partials are slots 0 .. n - 1 whatever the page table holds. The
// first round of their loads is issued before the request-table reads, and
// what lies at or past n is dropped once those land: one dependent round of
// loads instead of two.
template <int QF32, int D, bool SPLIT, bool PRE = false>
__global__ __launch_bounds__(kMergeThreads) void vat_merge(MergeArgs a) {
  constexpr int PER = D / 16;  // head dims per lane: 8 or 4
  constexpr int U = 64 / PER;  // partials per lane per round: 8 or 16
  constexpr int STEP = SPLIT ? 4 : 1;
  constexpr int ROWS = SPLIT ? kMergeThreads / 64 : kMergeThreads / 16;  // rows per workgroup
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4, l16 = lane & 15;
  int x = blockIdx.x;
  // The pointer line of the argument block joins the opening round of
  // argument loads (the block index below waits on it), instead of arriving
  // in a second round after the index arithmetic.
  {
    const void* p0 = a.part_o;
    asm volatile("" : "+s"(x) : "s"(p0));
  }
  const int rg = x % a.row_groups;
  x /= a.row_groups;
  const int rb = x % a.row_blocks;
  x /= a.row_blocks;
  const int h = x % a.hkv;
  const int b = x / a.hkv;
  float pre_ls[U];
  f32x4 pre_v[U][PER / 4];
  if constexpr (PRE) {
    const int plocal = rg * ROWS + (SPLIT ? (int)(threadIdx.x >> 6) : (int)(threadIdx.x >> 4));
    const int pph = SPLIT ? sub : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = pph + u * STEP;
      pre_ls[u] = kNegInf;
      if (i < a.slices && plocal < a.rows_per_block) {
        const long long sl =
            (((long long)i * a.hkv + h) * a.row_blocks + rb) * a.rows_per_block + plocal;
        pre_ls[u] = a.part_lse[sl];
        const f32x4* po = (const f32x4*)(a.part_o + sl * D + l16 * PER);
#pragma unroll
        for (int k = 0; k < PER / 4; ++k) pre_v[u][k] = po[k];
      }
    }
  }
  const Req r = make_req(a.kv_indptr[b], a.kv_indptr[b + 1], a.last_page_len[b], a.qo_indptr[b],
                         a.qo_indptr[b + 1], 0, a.page_shift, a.num_kv_indices, a.tokens);
  int n, first;  // partials of request b: slots first + i, i < n
  if (a.slices > 0) {
    // Slices of `per` pages: request b's pages [kv_indptr[b], kv_indptr[b + 1])
    // fall in slices x_lo .. x_hi.
    if (r.L == 0 || r.pages == 0) return;
    const int per = (a.num_kv_indices + a.slices - 1) / a.slices;
    const int x_lo = r.kv_start / per;
    n = (r.kv_start + r.pages - 1) / per - x_lo + 1;
    first = x_lo + b;
  } else {
    n = chunk_count(r.kv_len, a.chunk_keys);
    first = chunk_start(r.kv_start, a.page_shift, a.chunk_keys, b);
  }
  if (n <= 1) return;  // written directly by the partial kernel
  const int local = rg * ROWS + (SPLIT ? (int)(threadIdx.x >> 6) : (int)(threadIdx.x >> 4));
  const int row = rb * a.rows_per_block + local;
  const bool ok = local < a.rows_per_block && row < a.group * r.L;
  if (!__ballot(ok)) return;
  const int ph = SPLIT ? sub : 0;  // this lane group's first partial
  auto slot = [&](int i) -> long long {
    const int cid = min(first + i, a.num_ids - 1);
    return (((long long)cid * a.hkv + h) * a.row_blocks + rb) * a.rows_per_block + local;
  };
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  float m = kNegInf, den = 0.f;
  for (int i0 = 0; i0 < n; i0 += U * STEP) {
    float ls[U];
    f32x4 v[U][PER / 4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + ph + u * STEP;
      ls[u] = kNegInf;
      if constexpr (PRE) {
        if (i0 == 0 && first == 0) {  // the round loaded ahead (slot i, i < n <= slices)
          if (i < n && ok) {
            ls[u] = pre_ls[u];
#pragma unroll
            for (int k = 0; k < PER / 4; ++k) v[u][k] = pre_v[u][k];
          }
          continue;
        }
      }
      if (i < n && ok) {
        const long long sl = slot(i);
        ls[u] = a.part_lse[sl];
        const f32x4* po = (const f32x4*)(a.part_o + sl * D + l16 * PER);
#pragma unroll
        for (int k = 0; k < PER / 4; ++k) v[u][k] = po[k];
      }
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mn = fmaxf(mn, ls[u]);
    const float base = (mn == kNegInf) ? 0.f : mn;
    const float sc = fast_exp2(m - base);
    den *= sc;
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ls[u] == kNegInf) continue;  // absent, or an empty partial: adds nothing
      const float w = fast_exp2(ls[u] - base);
      den += w;
#pragma unroll
      for (int k = 0; k < PER / 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[4 * k + e] += w * v[u][k][e];
    }
    m = mn;
  }
  if constexpr (SPLIT) {
    // The four lane groups hold disjoint partials of the same row.
    float mall = fmaxf(m, __shfl_xor(m, 16));
    mall = fmaxf(mall, __shfl_xor(mall, 32));
    const float base = (mall == kNegInf) ? 0.f : mall;
    const float sc = fast_exp2(m - base);
    den *= sc;
    den += __shfl_xor(den, 16);
    den += __shfl_xor(den, 32);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      o[k] *= sc;
      o[k] += __shfl_xor(o[k], 16);
      o[k] += __shfl_xor(o[k], 32);
    }
    m = mall;
    if (sub != 0) return;
  }
  if (!ok) return;
  const int t = row / a.group, g = row % a.group;
  const long long orow = (long long)(r.q_start + t) * a.hq + h * a.group + g;
  const float sc = den > 0.f ? a.v_scale / den : 0.f;
  if constexpr (QF32) {
    f32x4* op = (f32x4*)((float*)a.out + orow * D + l16 * PER);
#pragma unroll
    for (int k = 0; k < PER / 4; ++k)
      op[k] = f32x4{o[4 * k] * sc, o[4 * k + 1] * sc, o[4 * k + 2] * sc, o[4 * k + 3] * sc};
  } else {
    unsigned short* op = (unsigned short*)a.out + orow * D + l16 * PER;
    if constexpr (PER == 8) {
      *(u32x4*)op = u32x4{pack_bf16x2(o[0] * sc, o[1] * sc), pack_bf16x2(o[2] * sc, o[3] * sc),
                          pack_bf16x2(o[4] * sc, o[5] * sc), pack_bf16x2(o[6] * sc, o[7] * sc)};
    } else {
      *(u32x2*)op = u32x2{pack_bf16x2(o[0] * sc, o[1] * sc), pack_bf16x2(o[2] * sc, o[3] * sc)};
    }
  }
  if (l16 == 0) a.lse[orow] = den > 0.f ? (m + fast_log2(den)) * kLn2 : kNegInf;
}

template <bool PRE>
const void* merge_variant(int q_is_f32, int head_dim, int rows_per_workgroup) {
  if (rows_per_workgroup == kMergeRows4) {
    if (q_is_f32)
      return (const void*)(head_dim == 64 ? vat_merge<1, 64, false, PRE> : vat_merge<1, 128, false, PRE>);
    return (const void*)(head_dim == 64 ? vat_merge<0, 64, false, PRE> : vat_merge<0, 128, false, PRE>);
  }
  if (q_is_f32)
    return (const void*)(head_dim == 64 ? vat_merge<1, 64, true, PRE> : vat_merge<1, 128, true, PRE>);
  return (const void*)(head_dim == 64 ? vat_merge<0, 64, true, PRE> : vat_merge<0, 128, true, PRE>);
}

// rows_per_workgroup: kMergeRows (one row per wave, SPLIT) or kMergeRows4;
// one_slice_request: balanced slices with a batch of one request (PRE).
const void* merge_kernel(int q_is_f32, int head_dim, int rows_per_workgroup, int one_slice_request) {
  return one_slice_request ? merge_variant<true>(q_is_f32, head_dim, rows_per_workgroup)
                           : merge_variant<false>(q_is_f32, head_dim, rows_per_workgroup);
}

}  // namespace vat
