// Device-side helpers shared by the gfx950 kernels: vector types, element
// conversions, wave reductions, request geometry and the chunk-id mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace vat {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

enum { KV_F32 = 0, KV_BF16 = 1, KV_E4M3 = 2 };

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }
__device__ __forceinline__ long long clampll(long long x, long long lo, long long hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Transposing LDS read (ds_read_b64_tr_b16) written as inline asm. The
// compiler cannot tell which LDS bytes the still-running DMA loads of later
// stages will write, so for the builtin form it waits for every outstanding
// vector memory load (vmcnt(0)) first, which serialises the stage ring. The
// caller orders this read after its own wait for the stage and must call
// lds_wait_tied before using the result.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  s16x4 v;
  const unsigned addr = (unsigned)(uintptr_t)(const lds_void_t*)p;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
// The same read at LDS byte address `addr + OFF`, OFF in the instruction's
// immediate offset field (no address arithmetic per read).
template <int OFF>
__device__ __forceinline__ s16x4 lds_read_tr16_at(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  s16x4 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}

// Wait until at most N LDS/scalar-memory operations are outstanding (LDS
// operations complete in order, so the reads issued before the last N have
// landed) and tie the wait to `v`, so its consumers cannot be scheduled above.
template <int N>
__device__ __forceinline__ void lds_wait_tied(s16x4& v) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}
// ds_read_b64_tr_b8, inline asm for the same reason. Within each 16-lane
// group, output lane j receives byte j % 8 of the 8-byte chunks that source
// lanes j / 8 + 2 k (k = 0..7) point at, as byte k.
__device__ __forceinline__ u32x2 lds_read_tr8(const void* p) {
  u32x2 v;
  const unsigned addr = (unsigned)(uintptr_t)(const lds_void_t*)p;
  asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr8_at(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
  u32x2 v;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}

template <int N>
__device__ __forceinline__ void lds_wait_tied(u32x2& v) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait_tied2(s16x4& v, s16x4& w) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(v), "+v"(w) : "n"(N));
}

// Max / sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Max / sum over the four lanes l, l^16, l^32, l^48 that hold one query row.
__device__ __forceinline__ float row_max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float row_sum4(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Two OCP e4m3fn codes -> two bf16 (exact). `hi` selects bytes 2,3 instead of
// 0,1. The packed result is taken as one 32-bit word: element extraction of
// this builtin's vector result is mis-lowered by the compiler.
__device__ __forceinline__ unsigned e4m3x2_to_bf16x2(unsigned w, bool hi) {
  bf16x2 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true)
                : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  return __builtin_bit_cast(unsigned, r);
}
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(unsigned a, unsigned b) {
  u32x4 r;
  r.x = e4m3x2_to_bf16x2(a, false);
  r.y = e4m3x2_to_bf16x2(a, true);
  r.z = e4m3x2_to_bf16x2(b, false);
  r.w = e4m3x2_to_bf16x2(b, true);
  return r;
}

// float -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ unsigned f32_to_bf16_bits(float f) {
  unsigned u = __builtin_bit_cast(unsigned, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Request geometry, every value clamped into range.
struct Req {
  int kv_start;  // first index into kv_indices
  int pages;
  int kv_len;
  int L;         // query tokens
  int prefix;    // kv_len - L
  int q_start;   // first query row
  int mask_off;  // byte offset of the request's mask block
};

__device__ __forceinline__ Req make_req(int ip0, int ip1, int lp, int q0, int q1, int moff,
                                        int page_shift, int num_kv_indices, int tokens) {
  Req r;
  ip0 = clampi(ip0, 0, num_kv_indices);
  ip1 = clampi(ip1, ip0, num_kv_indices);
  r.kv_start = ip0;
  r.pages = ip1 - ip0;
  lp = clampi(lp, 1, 1 << page_shift);
  r.kv_len = r.pages > 0 ? ((r.pages - 1) << page_shift) + lp : 0;
  q0 = clampi(q0, 0, tokens);
  q1 = clampi(q1, q0, tokens);
  r.L = min(q1 - q0, r.kv_len);
  r.q_start = q0;
  r.prefix = r.kv_len - r.L;
  r.mask_off = moff;
  return r;
}

// Chunk ids: request b's keys [0, kv_len_b) are cut into ceil(kv_len_b / C)
// chunks with ids start_b .. start_b + n_b - 1, start_b =
// floor(kv_indptr[b] * page_size / C) + b. Because n_b <=
// ceil(pages_b * page_size / C), consecutive requests' id ranges are disjoint
// and every id is below floor(num_kv_indices * page_size / C) + B.
__device__ __forceinline__ int chunk_start(int ip0, int page_shift, int chunk, int b) {
  return (int)(((long long)ip0 << page_shift) / chunk) + b;
}
__device__ __forceinline__ int chunk_count(int kv_len, int chunk) { return (kv_len + chunk - 1) / chunk; }

struct ReqArrays {
  const int32_t* kv_indptr;
  const int32_t* last_page_len;
  const int32_t* qo_indptr;
  const int32_t* mask_indptr;  // may be null
  int batch, page_shift, chunk, num_kv_indices, tokens;
};

// Request owning chunk id c (wave-uniform result; -1 if none) and its
// geometry. For B <= 64 one round of loads serves both the search and the
// geometry: lane i fetches request i's entries and the owner's are shuffled
// out. Larger batches search 64-way, then load the owner's entries.
__device__ __forceinline__ int find_request(const ReqArrays& ra, int c, int lane, Req& r) {
  if (ra.batch <= 64) {
    const bool in = lane < ra.batch;
    const int i = in ? lane : 0;
    const int ip0 = ra.kv_indptr[i];
    const int ip1 = ra.kv_indptr[i + 1];
    const int lp = in ? ra.last_page_len[i] : 1;
    const int q0 = ra.qo_indptr[i];
    const int q1 = ra.qo_indptr[i + 1];
    const int mo = ra.mask_indptr ? ra.mask_indptr[i] : 0;
    const int cl = clampi(ip0, 0, ra.num_kv_indices);
    const bool ok = in && chunk_start(cl, ra.page_shift, ra.chunk, i) <= c;
    const int cnt = __popcll(__ballot(ok));
    if (cnt == 0) return -1;
    const int b = cnt - 1;
    // readlane keeps the owner's entries in scalar registers: everything
    // derived from them (key range, loop bounds, addresses) stays wave-uniform.
    r = make_req(__builtin_amdgcn_readlane(ip0, b), __builtin_amdgcn_readlane(ip1, b),
                 __builtin_amdgcn_readlane(lp, b), __builtin_amdgcn_readlane(q0, b),
                 __builtin_amdgcn_readlane(q1, b), __builtin_amdgcn_readlane(mo, b),
                 ra.page_shift, ra.num_kv_indices, ra.tokens);
    return b;
  }
  int lo = 0, hi = ra.batch;
  while (hi - lo > 1) {
    const int span = hi - lo;
    const int step = (span + 63) / 64;
    const int bb = lo + lane * step;
    bool ok = false;
    if (bb < hi) {
      const int ip = clampi(ra.kv_indptr[bb], 0, ra.num_kv_indices);
      ok = chunk_start(ip, ra.page_shift, ra.chunk, bb) <= c;
    }
    const int cnt = __popcll(__ballot(ok));
    if (cnt == 0) return -1;
    lo = lo + (cnt - 1) * step;
    hi = min(hi, lo + step);
  }
  const int b = __builtin_amdgcn_readfirstlane(lo);
  r = make_req(ra.kv_indptr[b], ra.kv_indptr[b + 1], ra.last_page_len[b], ra.qo_indptr[b],
               ra.qo_indptr[b + 1], ra.mask_indptr ? ra.mask_indptr[b] : 0, ra.page_shift,
               ra.num_kv_indices, ra.tokens);
  return b;
}

// Work item `c` of the partial kernels: for batches of at most 64 requests
// the ids are compact -- request b's chunks are ids pre_b .. pre_b + n_b - 1,
// pre_b = sum over earlier requests of n = ceil(kv_len / C) (0 for requests
// without query tokens) -- so every active workgroup comes before every idle
// one in dispatch order. Larger batches use the closed-form ids of
// chunk_start(). Either way the result names request b, chunk j and the
// partial slot start_b + j (closed form, which the merge recomputes).
struct Item {
  int b, j, slot;
};

__device__ __forceinline__ bool find_item(const ReqArrays& ra, int c, int lane, Req& r, Item& it) {
  if (ra.batch <= 64) {
    const bool in = lane < ra.batch;
    const int i = in ? lane : 0;
    const int ip0 = ra.kv_indptr[i];
    const int ip1 = ra.kv_indptr[i + 1];
    const int lp = in ? ra.last_page_len[i] : 1;
    const int q0 = ra.qo_indptr[i];
    const int q1 = ra.qo_indptr[i + 1];
    const int mo = ra.mask_indptr ? ra.mask_indptr[i] : 0;
    const Req mine = make_req(ip0, ip1, lp, q0, q1, mo, ra.page_shift, ra.num_kv_indices, ra.tokens);
    const int n = (in && mine.L > 0) ? chunk_count(mine.kv_len, ra.chunk) : 0;
    // Inclusive prefix sum of n over the lanes.
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int up = __shfl_up(incl, o);
      if (lane >= o) incl += up;
    }
    const int pre = incl - n;
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (c >= total) return false;
    const int cnt = __popcll(__ballot(in && pre <= c));
    const int b = cnt - 1;
    r = make_req(__builtin_amdgcn_readlane(ip0, b), __builtin_amdgcn_readlane(ip1, b),
                 __builtin_amdgcn_readlane(lp, b), __builtin_amdgcn_readlane(q0, b),
                 __builtin_amdgcn_readlane(q1, b), __builtin_amdgcn_readlane(mo, b),
                 ra.page_shift, ra.num_kv_indices, ra.tokens);
    it.b = b;
    it.j = c - __builtin_amdgcn_readlane(pre, b);
    it.slot = chunk_start(r.kv_start, ra.page_shift, ra.chunk, b) + it.j;
    return true;
  }
  const int b = find_request(ra, c, lane, r);
  if (b < 0) return false;
  it.b = b;
  it.j = c - chunk_start(r.kv_start, ra.page_shift, ra.chunk, b);
  it.slot = c;
  return it.j >= 0 && it.j < chunk_count(r.kv_len, ra.chunk) && r.L > 0;
}

// Bits j = 0..L-1 of row t of the request's packed L x L mask block.
__device__ __forceinline__ unsigned long long load_mask_row(const uint8_t* mask, int num_mask_bytes,
                                                            int seg, int t, int L) {
  const int bit0 = t * L;
  const int nbytes = ((bit0 & 7) + L + 7) >> 3;
  const int last = max(num_mask_bytes - 1, 0);
  unsigned long long acc = 0;
  for (int i = min(nbytes, 8) - 1; i >= 0; --i)
    acc = (acc << 8) | (unsigned long long)mask[clampi(seg + (bit0 >> 3) + i, 0, last)];
  unsigned long long bits = acc >> (bit0 & 7);
  if (nbytes > 8)  // ninth byte (only when L + (bit0 & 7) > 64, so the shift is < 64)
    bits |= (unsigned long long)mask[clampi(seg + (bit0 >> 3) + 8, 0, last)] << (64 - (bit0 & 7));
  if (L < 64) bits &= (1ull << L) - 1ull;
  return bits;
}

// Bits j = 0..L-1 of row t of the request's full byte rows (prefix + L
// bytes per row from byte `seg`; the draft bytes are the last L; nonzero =
// allowed).
__device__ __forceinline__ unsigned long long load_mask_row_bytes(const uint8_t* mask,
                                                                  int num_mask_bytes, int seg,
                                                                  int t, int L, int prefix) {
  const long long last = max(num_mask_bytes - 1, 0);
  const long long byte0 = seg + (long long)t * (prefix + L) + prefix;
  unsigned long long bits = 0;
  for (int j = 0; j < L && j < 64; ++j)
    bits |= (unsigned long long)(mask[clampll(byte0 + j, 0, last)] != 0) << j;
  return bits;
}

}  // namespace vat
