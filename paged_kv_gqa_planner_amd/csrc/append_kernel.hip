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
// units [y * S, y * S + S), S = 256 * U, then the same span gridDim.y * S
// further on, and so on; each thread takes U of every S, 256 apart. U = 2
// keeps two requests in flight per thread for writes that fill the chip
// several times over; smaller writes take U = 1, for more threads.
#include "device_common.h"

namespace vat {
namespace {

// 8 source elements: the loaded 32-bit words (bf16: four, fp32: eight),
// read as binary32 (bf16 widens exactly by a 16-bit shift). The words are
// kept as scalars: extracting elements of a vector that went through an
// inline-asm operand is mis-compiled (every element reads element 0).
template <int SRC>
struct Src8 {
  static constexpr int kWords = SRC == KV_BF16 ? 4 : 8;
  unsigned v[kWords];

  __device__ __forceinline__ void load(const void* base, long long elem) {
    const u32x4* p = SRC == KV_BF16
                         ? reinterpret_cast<const u32x4*>((const uint16_t*)base + elem)
                         : reinterpret_cast<const u32x4*>((const float*)base + elem);
#pragma unroll
    for (int k = 0; k < kWords / 4; ++k) {
      const u32x4 q = p[k];
      v[4 * k] = q.x;
      v[4 * k + 1] = q.y;
      v[4 * k + 2] = q.z;
      v[4 * k + 3] = q.w;
    }
  }
  // Ties the loaded registers to this point: the compiler may otherwise move
  // a unit's loads into the conditional store below them, one at a time.
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int k = 0; k < kWords; ++k) asm volatile("" : "+v"(v[k]));
  }
  __device__ __forceinline__ float get(int i) const {
    if constexpr (SRC == KV_BF16) {
      const unsigned w = v[i / 2];
      return __builtin_bit_cast(float, (i & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
      return __builtin_bit_cast(float, v[i]);
    }
  }
};

__device__ __forceinline__ unsigned bits(float f) { return __builtin_bit_cast(unsigned, f); }

// x / s, correctly rounded. When s is a power of two its reciprocal is exact
// and one multiplication rounds the same real number, so the host passes
// inv = 1 / s and the (ten-instruction) division is skipped.
template <bool POW2>
__device__ __forceinline__ float quotient(float x, float s, float inv) {
  if constexpr (POW2) return x * inv;
  else return x / s;
}

// Cache patterns of y = x / s (x is NaN exactly when y is: s is finite and
// positive). Every branch is a select, so the division is never skipped and
// no lane diverges.
template <int DST>
struct Store8;

template <>
struct Store8<KV_F32> {
  template <bool POW2, class S>
  __device__ static void run(void* base, long long elem, const S& x, float s, float inv) {
    unsigned u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = quotient<POW2>(x.get(i), s, inv);
      u[i] = (y != y) ? (0x7fc00000u | (bits(x.get(i)) & 0x80000000u)) : bits(y);
    }
    u32x4* p = reinterpret_cast<u32x4*>((float*)base + elem);
    p[0] = u32x4{u[0], u[1], u[2], u[3]};
    p[1] = u32x4{u[4], u[5], u[6], u[7]};
  }
};

template <>
struct Store8<KV_BF16> {
  template <bool POW2, class S>
  __device__ static void run(void* base, long long elem, const S& x, float s, float inv) {
    unsigned h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = quotient<POW2>(x.get(i), s, inv);
      const unsigned u = bits(y);
      // Round to nearest even on the 16 dropped bits (a carry may reach the
      // exponent, and past the largest finite value gives infinity).
      const unsigned r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
      h[i] = (y != y) ? (0x7fc0u | ((bits(x.get(i)) >> 16) & 0x8000u)) : r;
    }
    *reinterpret_cast<u32x4*>((uint16_t*)base + elem) =
        u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
};

template <>
struct Store8<KV_E4M3> {
  template <bool POW2, class S>
  __device__ static void run(void* base, long long elem, const S& x, float s, float inv) {
    unsigned c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = quotient<POW2>(x.get(i), s, inv);
      const unsigned a = bits(y) & 0x7fffffffu;
      // Below the smallest normal 2^-6 the codes are m * 2^-9, m = 0..8 (8
      // is 2^-6 itself, code 0x08): scaling by 2^9 is exact and rint rounds
      // half to even.
      const unsigned sub = (unsigned)__builtin_rintf(__builtin_fabsf(y) * 512.0f);
      // Normal: keep 3 of the 23 significand bits, half to even (a carry
      // moves into the exponent field), and rebias the exponent 127 -> 7.
      const unsigned nor = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
      // |y| >= 448 (infinity included) saturates to 448 = 0x7E.
      unsigned m = a >= 0x43e00000u ? 0x7eu : (a < 0x3c800000u ? sub : nor);
      m = (y != y) ? 0x7fu : m;
      c[i] = m | ((bits(x.get(i)) >> 24) & 0x80u);
    }
    *reinterpret_cast<u32x2*>((uint8_t*)base + elem) =
        u32x2{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
              c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
  }
};

template <int SRC, int DST, bool POW2, int U>
__global__ __launch_bounds__(kAppendThreads) void vat_append(AppendArgs a) {
  const int b = blockIdx.x;
  const Req r = make_req(a.kv_indptr[b], a.kv_indptr[b + 1], a.last_page_len[b], a.qo_indptr[b],
                         a.qo_indptr[b + 1], 0, a.page_shift, a.num_kv_indices, a.tokens);
  // Unit u < per_tensor is key unit u, else value unit u - per_tensor; key
  // unit (t, w) moves elements [8 w, 8 w + 8) of draft token t's row. The
  // host bounds max_qo_len * Hkv * D by 2^31, so unit counts fit 32 bits.
  const unsigned ru = (unsigned)a.row_units;
  const unsigned per_tensor = (unsigned)r.L * ru;
  const unsigned units = 2u * per_tensor;
  const long long row_elems = (long long)ru * 8;
  const int slot_mask = (1 << a.page_shift) - 1;
  constexpr unsigned kStep = kAppendThreads * U;
  for (unsigned base = blockIdx.y * kStep; base < units; base += gridDim.y * kStep) {
    // All loads of the U units first (page ids and sources), so each thread
    // keeps U 16-byte requests in flight; then the stores.
    Src8<SRC> x[U];
    int page[U], n[U], w[U];
    bool is_v[U], ok[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const unsigned u0 = base + j * kAppendThreads + threadIdx.x;
      ok[j] = u0 < units;
      const unsigned u = ok[j] ? u0 : 0u;  // out-of-range lanes load unit 0 (exists)
      is_v[j] = u >= per_tensor;
      const unsigned uu = is_v[j] ? u - per_tensor : u;
      const unsigned t = uu / ru;
      w[j] = (int)(uu - t * ru);
      n[j] = r.prefix + (int)t;  // key position, < kv_len
      page[j] = a.kv_indices[r.kv_start + (n[j] >> a.page_shift)];
      x[j].load(is_v[j] ? a.v_new : a.k_new,
                (long long)(r.q_start + (int)t) * row_elems + w[j] * 8);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      x[j].pin();
      asm volatile("" : "+v"(page[j]));
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (!ok[j] || page[j] < 0 || page[j] >= a.num_pages) continue;
      const long long slot_row = ((long long)page[j] << a.page_shift) + (n[j] & slot_mask);
      Store8<DST>::template run<POW2>(is_v[j] ? a.v_cache : a.k_cache,
                                      slot_row * row_elems + w[j] * 8, x[j],
                                      is_v[j] ? a.v_scale : a.k_scale,
                                      is_v[j] ? a.v_inv : a.k_inv);
    }
  }
}

// Eight rotated key elements, fed to Store8 like a source chunk.
struct F8 {
  float v[8];
  __device__ __forceinline__ float get(int i) const { return v[i]; }
};

// The write with the keys rotated by RoPE first (LLaMA style: dimension i
// pairs with i + D/2, i < D/2, by the token's cos/sin row: x'_i = x_i c_i -
// x_{i+D/2} s_i, x'_{i+D/2} = x_{i+D/2} c_i + x_i s_i), in binary32 with every
// product and sum rounded on its own, then scaled and rounded as above. Key
// unit (t, h, j) moves elements [8 j, 8 j + 8) of head h and their partners
// D/2 further; value units are the plain ones. One unit per thread.
template <int SRC, int DST, bool POW2>
__global__ __launch_bounds__(kAppendThreads) void vat_append_rope(AppendArgs a) {
  const int b = blockIdx.x;
  const Req r = make_req(a.kv_indptr[b], a.kv_indptr[b + 1], a.last_page_len[b], a.qo_indptr[b],
                         a.qo_indptr[b + 1], 0, a.page_shift, a.num_kv_indices, a.tokens);
  const int D = a.head_dim;
  const unsigned ru = (unsigned)a.row_units;  // 8-element units per token row
  const unsigned rk = ru / 2;                 // key units (element pairs of 8) per row
  const unsigned jd = (unsigned)(D / 16);     // key units per head
  const unsigned per_k = (unsigned)r.L * rk;
  const unsigned units = per_k + (unsigned)r.L * ru;
  const long long row_elems = (long long)ru * 8;
  const int slot_mask = (1 << a.page_shift) - 1;
  for (unsigned u = blockIdx.y * kAppendThreads + threadIdx.x; u < units;
       u += gridDim.y * kAppendThreads) {
    if (u < per_k) {
      const unsigned t = u / rk;
      const unsigned w = u - t * rk;
      const unsigned h = w / jd, j = w - h * jd;
      const int lo = (int)(h * D + 8 * j), hi = lo + D / 2;
      const int n = r.prefix + (int)t;
      const int page = a.kv_indices[r.kv_start + (n >> a.page_shift)];
      const long long row = (long long)(r.q_start + (int)t);
      Src8<SRC> xl, xh;
      xl.load(a.k_new, row * row_elems + lo);
      xh.load(a.k_new, row * row_elems + hi);
      const f32x4* cs = reinterpret_cast<const f32x4*>(a.k_cos_sin + row * D + 8 * j);
      const f32x4 c0 = cs[0], c1 = cs[1];
      const f32x4 s0 = cs[D / 8], s1 = cs[D / 8 + 1];
      if (page < 0 || page >= a.num_pages) continue;
      const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
      const float sn[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      F8 yl, yh;
      {
#pragma clang fp contract(off)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pl = xl.get(e) * c[e], ph = xh.get(e) * sn[e];
          const float ql = xh.get(e) * c[e], qh = xl.get(e) * sn[e];
          yl.v[e] = pl - ph;
          yh.v[e] = ql + qh;
        }
      }
      // A NaN from the rotation (a NaN input, or infinity times zero) takes
      // the canonical positive NaN: its sign would otherwise depend on how
      // the hardware forms invalid results.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        yl.v[e] = yl.v[e] != yl.v[e] ? __builtin_bit_cast(float, 0x7fc00000u) : yl.v[e];
        yh.v[e] = yh.v[e] != yh.v[e] ? __builtin_bit_cast(float, 0x7fc00000u) : yh.v[e];
      }
      const long long slot_row = ((long long)page << a.page_shift) + (n & slot_mask);
      Store8<DST>::template run<POW2>(a.k_cache, slot_row * row_elems + lo, yl, a.k_scale, a.k_inv);
      Store8<DST>::template run<POW2>(a.k_cache, slot_row * row_elems + hi, yh, a.k_scale, a.k_inv);
    } else {
      const unsigned uu = u - per_k;
      const unsigned t = uu / ru;
      const int w = (int)(uu - t * ru);
      const int n = r.prefix + (int)t;
      const int page = a.kv_indices[r.kv_start + (n >> a.page_shift)];
      Src8<SRC> x;
      x.load(a.v_new, (long long)(r.q_start + (int)t) * row_elems + w * 8);
      if (page < 0 || page >= a.num_pages) continue;
      const long long slot_row = ((long long)page << a.page_shift) + (n & slot_mask);
      Store8<DST>::template run<POW2>(a.v_cache, slot_row * row_elems + w * 8, x, a.v_scale, a.v_inv);
    }
  }
}

}  // namespace

template <int SRC, int DST>
const void* pick(bool pow2, int units) {
  if (units == 2)
    return pow2 ? (const void*)vat_append<SRC, DST, true, 2> : (const void*)vat_append<SRC, DST, false, 2>;
  return pow2 ? (const void*)vat_append<SRC, DST, true, 1> : (const void*)vat_append<SRC, DST, false, 1>;
}

template <int SRC, int DST>
const void* pick_rope(bool pow2) {
  return pow2 ? (const void*)vat_append_rope<SRC, DST, true> : (const void*)vat_append_rope<SRC, DST, false>;
}

const void* append_rope_kernel(int src_dtype, int cache_dtype, int pow2_scales) {
  const bool p = pow2_scales != 0;
  if (src_dtype == KV_BF16) {
    if (cache_dtype == KV_BF16) return pick_rope<KV_BF16, KV_BF16>(p);
    if (cache_dtype == KV_E4M3) return pick_rope<KV_BF16, KV_E4M3>(p);
    if (cache_dtype == KV_F32) return pick_rope<KV_BF16, KV_F32>(p);
  } else if (src_dtype == KV_F32) {
    if (cache_dtype == KV_BF16) return pick_rope<KV_F32, KV_BF16>(p);
    if (cache_dtype == KV_E4M3) return pick_rope<KV_F32, KV_E4M3>(p);
    if (cache_dtype == KV_F32) return pick_rope<KV_F32, KV_F32>(p);
  }
  return nullptr;
}

const void* append_kernel(int src_dtype, int cache_dtype, int pow2_scales, int units) {
  const bool p = pow2_scales != 0;
  const int u = units;
  if (src_dtype == KV_BF16) {
    if (cache_dtype == KV_BF16) return pick<KV_BF16, KV_BF16>(p, u);
    if (cache_dtype == KV_E4M3) return pick<KV_BF16, KV_E4M3>(p, u);
    if (cache_dtype == KV_F32) return pick<KV_BF16, KV_F32>(p, u);
  } else if (src_dtype == KV_F32) {
    if (cache_dtype == KV_BF16) return pick<KV_F32, KV_BF16>(p, u);
    if (cache_dtype == KV_E4M3) return pick<KV_F32, KV_E4M3>(p, u);
    if (cache_dtype == KV_F32) return pick<KV_F32, KV_F32>(p, u);
  }
  return nullptr;
}

}  // namespace vat
