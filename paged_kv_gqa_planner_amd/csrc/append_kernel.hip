// Write of the draft tokens' keys and values into the paged cache, rounded to
// the cache dtype on the way.
//
// Verification attention expects every draft's key and value to be cached
// before it runs (vLLM page "[WIP] Support for cached multi-query attention
// towards speculative decoding"): token t of request b becomes key position
// n = kv_len_b - L_b + t, which lives at slot n % page_size of page
// kv_indices[kv_indptr[b] + n / page_size] (paged format of the FlashInfer
// page "feat: Separate Q and KV dtypes for decode"). The attention reads a
// stored element as scale * stored (flashmap page "sglang/verify_attention.py",
// k_scale / v_scale folding), so the value written is x / scale: one IEEE
// binary32 division, then round-to-nearest-even into the cache dtype
// (e4m3fn: clamped to +-448 first, the format having no infinity). A NaN
// input stores the dtype's canonical quiet NaN with the input's sign.
//
// The work is a gather-free scatter of whole 16-byte groups, bound by HBM:
// one thread moves 8 elements (16 or 32 source bytes, 8 to 32 cache bytes),
// consecutive threads take consecutive elements of one token row, so a wave
// reads and writes contiguous runs. Workgroup (b, y) handles request b's
// units y * 256 + tid, y * 256 + tid + gridDim.y * 256, ...
#include "device_common.h"

namespace vat {
namespace {

// 8 source elements as binary32 (bf16 widens exactly by a 16-bit shift).
template <int SRC>
__device__ __forceinline__ void load8(const void* base, long long elem, float (&x)[8]) {
  if constexpr (SRC == KV_BF16) {
    const u32x4 w = *reinterpret_cast<const u32x4*>((const uint16_t*)base + elem);
    const unsigned ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __builtin_bit_cast(float, ws[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, ws[i] & 0xffff0000u);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>((const float*)base + elem);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
}

// |y| -> e4m3fn magnitude code (0x00 .. 0x7E), y not NaN, nearest with ties
// to even after clamping to 448.
__device__ __forceinline__ unsigned e4m3_mag_code(float y) {
  const unsigned a = __builtin_bit_cast(unsigned, y) & 0x7fffffffu;
  if (a >= 0x43e00000u) return 0x7eu;  // >= 448 (and +inf): saturate
  if (a < 0x3c800000u) {
    // Below the smallest normal 2^-6 the codes are m * 2^-9, m = 0..8 (8 is
    // 2^-6 itself, code 0x08). Scaling by 2^9 is exact; rint rounds half to
    // even.
    return (unsigned)__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
  }
  // Normal: keep 3 of the 23 significand bits, rounding half to even (a
  // carry moves into the exponent field); rebias the exponent 127 -> 7.
  const unsigned r = a + 0x7ffffu + ((a >> 20) & 1u);
  return (r >> 20) - (120u << 3);
}

template <int DST>
struct Store8;

template <>
struct Store8<KV_F32> {
  __device__ static void run(void* base, long long elem, const float (&y)[8], const float (&x)[8]) {
    unsigned u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned s = __builtin_bit_cast(unsigned, x[i]) & 0x80000000u;
      u[i] = (x[i] != x[i]) ? (0x7fc00000u | s) : __builtin_bit_cast(unsigned, y[i]);
    }
    u32x4* p = reinterpret_cast<u32x4*>((float*)base + elem);
    p[0] = u32x4{u[0], u[1], u[2], u[3]};
    p[1] = u32x4{u[4], u[5], u[6], u[7]};
  }
};

template <>
struct Store8<KV_BF16> {
  __device__ static void run(void* base, long long elem, const float (&y)[8], const float (&x)[8]) {
    unsigned h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned s = (__builtin_bit_cast(unsigned, x[i]) >> 16) & 0x8000u;
      h[i] = (x[i] != x[i]) ? (0x7fc0u | s) : f32_to_bf16_bits(y[i]);
    }
    *reinterpret_cast<u32x4*>((uint16_t*)base + elem) =
        u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
};

template <>
struct Store8<KV_E4M3> {
  __device__ static void run(void* base, long long elem, const float (&y)[8], const float (&x)[8]) {
    unsigned c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned s = (__builtin_bit_cast(unsigned, x[i]) >> 24) & 0x80u;
      c[i] = s | ((x[i] != x[i]) ? 0x7fu : e4m3_mag_code(y[i]));
    }
    *reinterpret_cast<u32x2*>((uint8_t*)base + elem) =
        u32x2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
              c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
  }
};

template <int SRC, int DST>
__global__ __launch_bounds__(kAppendThreads) void vat_append(AppendArgs a) {
  const int b = blockIdx.x;
  const Req r = make_req(a.kv_indptr[b], a.kv_indptr[b + 1], a.last_page_len[b], a.qo_indptr[b],
                         a.qo_indptr[b + 1], 0, a.page_shift, a.num_kv_indices, a.tokens);
  const int ru = a.row_units;
  const long long per_tensor = (long long)r.L * ru;
  const long long units = 2 * per_tensor;
  const long long row_elems = (long long)ru * 8;
  for (long long u = (long long)blockIdx.y * kAppendThreads + threadIdx.x; u < units;
       u += (long long)gridDim.y * kAppendThreads) {
    const bool is_v = u >= per_tensor;
    const long long uu = is_v ? u - per_tensor : u;
    const int t = (int)(uu / ru);
    const int w = (int)(uu - (long long)t * ru);
    const int n = r.prefix + t;  // key position, < kv_len
    const int page = a.kv_indices[r.kv_start + (n >> a.page_shift)];
    float x[8];
    load8<SRC>(is_v ? a.v_new : a.k_new, (r.q_start + t) * row_elems + (long long)w * 8, x);
    if (page < 0 || page >= a.num_pages) continue;
    const float s = is_v ? a.v_scale : a.k_scale;
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i] / s;
    const long long slot_row = ((long long)page << a.page_shift) + (n & ((1 << a.page_shift) - 1));
    Store8<DST>::run(is_v ? a.v_cache : a.k_cache, slot_row * row_elems + (long long)w * 8, y, x);
  }
}

}  // namespace

const void* append_kernel(int src_dtype, int cache_dtype) {
  if (src_dtype == KV_BF16) {
    if (cache_dtype == KV_BF16) return (const void*)vat_append<KV_BF16, KV_BF16>;
    if (cache_dtype == KV_E4M3) return (const void*)vat_append<KV_BF16, KV_E4M3>;
    if (cache_dtype == KV_F32) return (const void*)vat_append<KV_BF16, KV_F32>;
  } else if (src_dtype == KV_F32) {
    if (cache_dtype == KV_BF16) return (const void*)vat_append<KV_F32, KV_BF16>;
    if (cache_dtype == KV_E4M3) return (const void*)vat_append<KV_F32, KV_E4M3>;
    if (cache_dtype == KV_F32) return (const void*)vat_append<KV_F32, KV_F32>;
  }
  return nullptr;
}

}  // namespace vat
