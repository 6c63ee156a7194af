// Row-tiled partial kernel: fp32 caches and wide row sets (prefill).
//
// One workgroup (four wave64s) per (chunk of a request's keys, KV head, row
// block). A row block holds query rows r = t * G + g (token-major) of the
// request's G * L_b rows that share KV head h, so every key and value of the
// chunk is fetched once per KV head and row block rather than once per query
// head (flashmap page "sglang/verify_attention.py", module docstring and
// _verify_partial_kernel). The draft block at the end of the request is
// masked in place (causal or bit-packed tree mask); rows of a causal row
// block stop at their last token's key.
//
// Inner step (32 keys per wave): keys are gathered through the page table
// straight into MFMA operand registers with 16-byte loads; logits are
// computed transposed, S^T = K . Q^T (v_mfma_f32_16x16x32_bf16, or
// v_mfma_f32_16x16x4f32 for fp32), so that each lane owns one query row and
// its exponentiated logits are already laid out as the B operand of
// O^T = V^T . P^T. For bf16/fp8 caches V goes through a per-wave LDS tile
// (XOR-swizzled 16-byte chunks) to be read back transposed. The online
// softmax keeps a running max and sum per row in base 2 (the scale
// sm_scale * k_scale * log2 e is folded into one FMA before v_exp_f32).
#include "device_common.h"

namespace vat {

// ---------------------------------------------------------------------------
// Page-id window: lane i of a wave holds the page id of request page
// (base + i) in w0 and (base + 64 + i) in w1; lookups are lane shuffles.
struct PageWindow {
  int base;
  int w0, w1;
};

__device__ __forceinline__ int load_page_id(const PartialArgs& a, const Req& r, int rel_page) {
  const int idx = clampi(r.kv_start + clampi(rel_page, 0, max(r.pages - 1, 0)), 0,
                         max(a.num_kv_indices - 1, 0));
  return clampi(a.kv_indices[idx], 0, a.num_pages - 1);
}

__device__ __forceinline__ void window_init(PageWindow& w, const PartialArgs& a, const Req& r,
                                            int first_page, int lane) {
  w.base = first_page;
  w.w0 = load_page_id(a, r, first_page + lane);
  w.w1 = load_page_id(a, r, first_page + 64 + lane);
}

// Make sure pages [p0, p0 + 31] are inside the window (p0 never decreases).
__device__ __forceinline__ void window_advance(PageWindow& w, const PartialArgs& a, const Req& r,
                                               int p0, int lane) {
  if (p0 >= w.base + 128) {
    window_init(w, a, r, p0, lane);
    return;
  }
  while (p0 >= w.base + 64) {
    w.w0 = w.w1;
    w.base += 64;
    w.w1 = load_page_id(a, r, w.base + 64 + lane);
  }
}

__device__ __forceinline__ int window_lookup(const PageWindow& w, int page) {
  const int idx = page - w.base;  // 0 .. 127
  const int x0 = __shfl(w.w0, idx & 63);
  const int x1 = __shfl(w.w1, idx & 63);
  return idx < 64 ? x0 : x1;
}

// Element offset of key n (request-relative) of KV head h in a cache.
__device__ __forceinline__ long long key_offset(const PartialArgs& a, const PageWindow& w, int n,
                                                int h, int D) {
  const int page = window_lookup(w, n >> a.page_shift);
  const int slot = n & ((1 << a.page_shift) - 1);
  return ((((long long)page << a.page_shift) + slot) * a.hkv + h) * (long long)D;
}

// ---------------------------------------------------------------------------
// Operand layouts (v_mfma_f32_16x16x32_bf16, lane l, element e):
//   A[i][k]: i = l % 16, k = 8 (l / 16) + e      B[k][j]: k = 8 (l / 16) + e, j = l % 16
//   C[i][j]: i = 4 (l / 16) + e (e < 4), j = l % 16
// For S^T = K . Q^T, A = K (i = key), B = Q^T (j = query row); contraction
// index k maps to head-dim d by qk_d0() (any bijection works if A and B agree).
template <int KV>
__device__ __forceinline__ int qk_d0(int ks, int j4) {
  if constexpr (KV == KV_E4M3) return 64 * (ks >> 1) + 16 * j4 + 8 * (ks & 1);
  else return 32 * ks + 8 * j4;
}

// Register tile of one 32-key step.
template <int KV, int D>
struct StepRegs {
  // K operand: [key tile kt][d step ks] (bf16 family) ; fp32: [kt][D/4] floats
  static constexpr int NKS = (KV == KV_F32) ? D / 4 : D / 32;
  static constexpr int KW = (KV == KV_F32) ? (D / 4) : (KV == KV_E4M3 ? (D / 32) * 2 : (D / 32) * 4);
  // dwords of K per lane per kt
  unsigned k[2][KW];
  // V: bf16: 16-byte chunks this lane stages ((32 keys * D * 2 B) / 64 lanes / 16 B)
  //    e4m3: 16-byte chunks of codes ; fp32: floats [kt][e][D/16]
  static constexpr int VW = (KV == KV_F32) ? (2 * 4 * (D / 16))
                                           : (KV == KV_E4M3 ? (kStepKeys * D) / 64 / 4
                                                            : (kStepKeys * D * 2) / 64 / 4);
  unsigned v[VW];
};

template <int KV, int D>
__device__ __forceinline__ void load_step(StepRegs<KV, D>& s, const PartialArgs& a, const Req& r,
                                          PageWindow& w, int n0, int last, int h, int lane) {
  const int l16 = lane & 15;
  const int j4 = lane >> 4;
  window_advance(w, a, r, n0 >> a.page_shift, lane);
  if constexpr (KV == KV_F32) {
    const float* kc = (const float*)a.k_cache;
    const float* vc = (const float*)a.v_cache;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int n = min(n0 + 16 * kt + l16, last);
      const float* p = kc + key_offset(a, w, n, h, D) + (D / 4) * j4;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        u32x4 x = *(const u32x4*)(p + 4 * i);
        s.k[kt][4 * i + 0] = x.x;
        s.k[kt][4 * i + 1] = x.y;
        s.k[kt][4 * i + 2] = x.z;
        s.k[kt][4 * i + 3] = x.w;
      }
    }
    // V^T operand of v_mfma_f32_16x16x4f32: lane (d = l % 16, j = l / 16)
    // needs V[key 16 kt + 4 j + e][16 dt + d].
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = min(n0 + 16 * kt + 4 * j4 + e, last);
        const float* p = vc + key_offset(a, w, n, h, D) + l16;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
          s.v[(kt * 4 + e) * (D / 16) + dt] = __builtin_bit_cast(unsigned, p[16 * dt]);
      }
    }
  } else {
    constexpr int EB = (KV == KV_E4M3) ? 1 : 2;  // bytes per cache element
    const unsigned char* kc = (const unsigned char*)a.k_cache;
    const unsigned char* vc = (const unsigned char*)a.v_cache;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int n = min(n0 + 16 * kt + l16, last);
      const unsigned char* p = kc + key_offset(a, w, n, h, D) * EB;
      if constexpr (KV == KV_E4M3) {
#pragma unroll
        for (int pp = 0; pp < D / 64; ++pp) {
          u32x4 x = *(const u32x4*)(p + 64 * pp + 16 * j4);
          s.k[kt][4 * pp + 0] = x.x;
          s.k[kt][4 * pp + 1] = x.y;
          s.k[kt][4 * pp + 2] = x.z;
          s.k[kt][4 * pp + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          u32x4 x = *(const u32x4*)(p + 2 * qk_d0<KV>(ks, j4));
          s.k[kt][4 * ks + 0] = x.x;
          s.k[kt][4 * ks + 1] = x.y;
          s.k[kt][4 * ks + 2] = x.z;
          s.k[kt][4 * ks + 3] = x.w;
        }
      }
    }
    // V: 16-byte chunks, CPK per key row, KPI keys per wave instruction.
    constexpr int CPK = D * EB / 16;
    constexpr int KPI = 64 / CPK;
    constexpr int NI = kStepKeys / KPI;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = min(n0 + i * KPI + lane / CPK, last);
      const unsigned char* p = vc + key_offset(a, w, n, h, D) * EB + 16 * (lane % CPK);
      u32x4 x = *(const u32x4*)p;
      s.v[4 * i + 0] = x.x;
      s.v[4 * i + 1] = x.y;
      s.v[4 * i + 2] = x.z;
      s.v[4 * i + 3] = x.w;
    }
  }
}

// LDS V tile (bf16, [32 keys][D], 16-byte chunk c of key n stored at chunk
// c ^ 2 ((n >> 2) & 3)): the transposed reads below then hit 32 distinct banks.
template <int D>
__device__ __forceinline__ int vtile_off(int n, int chunk) {
  return n * (D * 2) + ((chunk ^ (2 * ((n >> 2) & 3))) << 4);
}

template <int KV, int D>
__device__ __forceinline__ void stage_v(const StepRegs<KV, D>& s, unsigned char* vt, int lane) {
  if constexpr (KV == KV_BF16) {
    constexpr int CPK = D * 2 / 16;
    constexpr int KPI = 64 / CPK;
#pragma unroll
    for (int i = 0; i < kStepKeys / KPI; ++i) {
      const int n = i * KPI + lane / CPK;
      u32x4 x = {s.v[4 * i], s.v[4 * i + 1], s.v[4 * i + 2], s.v[4 * i + 3]};
      *(u32x4*)(vt + vtile_off<D>(n, lane % CPK)) = x;
    }
  } else if constexpr (KV == KV_E4M3) {
    constexpr int CPK = D / 16;  // 16 codes per chunk -> two bf16 chunks
    constexpr int KPI = 64 / CPK;
#pragma unroll
    for (int i = 0; i < kStepKeys / KPI; ++i) {
      const int n = i * KPI + lane / CPK;
      const int c = 2 * (lane % CPK);
      u32x4 lo = e4m3x8_to_bf16(s.v[4 * i], s.v[4 * i + 1]);
      u32x4 hi = e4m3x8_to_bf16(s.v[4 * i + 2], s.v[4 * i + 3]);
      *(u32x4*)(vt + vtile_off<D>(n, c)) = lo;
      *(u32x4*)(vt + vtile_off<D>(n, c + 1)) = hi;
    }
  }
}

// V^T operand for head-dim tile dt: lane (d = l % 16, j = l / 16) element e
// holds V[kappa(j, e)][16 dt + d] with kappa(j, e) = 4 j + e (e < 4) or
// 16 + 4 j + e - 4 (e >= 4): the keys whose P values sit in this lane's row
// of the two S^T tiles.
template <int D>
__device__ __forceinline__ bf16x8 read_vt(const unsigned char* vt, int dt, int lane) {
  const int l16 = lane & 15;
  const int j4 = lane >> 4;
  const int d = 16 * dt + l16;
  const int chunk = d >> 3;
  const int within = (d & 7) * 2;
  unsigned w[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    const int ea = 2 * e2, eb = 2 * e2 + 1;
    const int na = ea < 4 ? 4 * j4 + ea : 16 + 4 * j4 + ea - 4;
    const int nb = eb < 4 ? 4 * j4 + eb : 16 + 4 * j4 + eb - 4;
    const unsigned lo = *(const unsigned short*)(vt + vtile_off<D>(na, chunk) + within);
    const unsigned hi = *(const unsigned short*)(vt + vtile_off<D>(nb, chunk) + within);
    w[e2] = lo | (hi << 16);
  }
  u32x4 x = {w[0], w[1], w[2], w[3]};
  return __builtin_bit_cast(bf16x8, x);
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
template <int KV, int D, int RT>
struct Acc {
  f32x4 o[RT][D / 16];  // O^T tiles: lane (row l % 16, j) holds d = 16 dt + 4 j + e
  float m[RT];          // running max of scaled logits (base 2), uniform over the row's lanes
  float l[RT];          // this lane's share of the running sum
};

// Row-visibility description for one work item.
struct Vis {
  int hi;           // keys >= hi are outside the item
  int masked_from;  // keys >= masked_from are drafts: apply causal / mask
  int has_mask;
};

template <int KV, int D, int RT>
__device__ __forceinline__ void compute_step(Acc<KV, D, RT>& acc, const StepRegs<KV, D>& s,
                                             const unsigned (&qf)[RT][StepRegs<KV, D>::NKS *
                                                                      ((KV == KV_F32) ? 1 : 4)],
                                             const int (&row_t)[RT],
                                             const unsigned long long (&row_bits)[RT],
                                             const Vis& vis, int n0, float c, unsigned char* vt,
                                             int lane) {
  const int j4 = lane >> 4;
  // ---- logits S^T[key][row]
  f32x4 st[2][RT];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) st[kt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (KV == KV_F32) {
#pragma unroll
    for (int ks = 0; ks < D / 4; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          st[kt][rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
              __builtin_bit_cast(float, s.k[kt][ks]), __builtin_bit_cast(float, qf[rt][ks]),
              st[kt][rt], 0, 0, 0);
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        u32x4 kw;
        if constexpr (KV == KV_E4M3) {
          const int pp = ks >> 1, half = ks & 1;
          kw = e4m3x8_to_bf16(s.k[kt][4 * pp + 2 * half], s.k[kt][4 * pp + 2 * half + 1]);
        } else {
          kw = u32x4{s.k[kt][4 * ks], s.k[kt][4 * ks + 1], s.k[kt][4 * ks + 2], s.k[kt][4 * ks + 3]};
        }
        const bf16x8 ka = __builtin_bit_cast(bf16x8, kw);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          u32x4 qw = {qf[rt][4 * ks], qf[rt][4 * ks + 1], qf[rt][4 * ks + 2], qf[rt][4 * ks + 3]};
          st[kt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              ka, __builtin_bit_cast(bf16x8, qw), st[kt][rt], 0, 0, 0);
        }
      }
    }
  }
  // ---- visibility: keys past the item, drafts under causal / mask
  const bool edge = (n0 + kStepKeys > vis.hi) || (n0 + kStepKeys > vis.masked_from);
  if (edge) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = n0 + 16 * kt + 4 * j4 + e;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          bool ok = n < vis.hi;
          if (n >= vis.masked_from) {
            const int jd = n - vis.masked_from;
            if (vis.has_mask) ok = ok && jd < 64 && ((row_bits[rt] >> jd) & 1ull);
            else ok = ok && jd <= row_t[rt];
          }
          if (!ok) st[kt][rt][e] = kNegInf;
        }
      }
  }
  // ---- online softmax (base 2); p overwrites the logits
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, st[kt][rt][e]);
    mx = row_max4(mx) * c;
    const float m_new = fmaxf(acc.m[rt], mx);
    // A row that has seen nothing yet keeps m = -inf; use 0 as the base so
    // that exp2 gives alpha = 1 and p = 0 without NaN.
    const float base = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(acc.m[rt] - base);
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = fast_exp2(__builtin_fmaf(st[kt][rt][e], c, -base));
        st[kt][rt][e] = p;
        sum += p;
      }
    acc.l[rt] = acc.l[rt] * alpha + sum;
    acc.m[rt] = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc.o[rt][dt] *= alpha;
  }
  // ---- O^T += V^T . P^T
  if constexpr (KV == KV_F32) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const float va = __builtin_bit_cast(float, s.v[(kt * 4 + e) * (D / 16) + dt]);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            acc.o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va, st[kt][rt][e], acc.o[rt][dt],
                                                                  0, 0, 0);
        }
  } else {
    stage_v<KV, D>(s, vt, lane);
    wave_lds_fence();
    bf16x8 pb[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      u32x4 pw = {pack_bf16x2(st[0][rt][0], st[0][rt][1]), pack_bf16x2(st[0][rt][2], st[0][rt][3]),
                  pack_bf16x2(st[1][rt][0], st[1][rt][1]), pack_bf16x2(st[1][rt][2], st[1][rt][3])};
      pb[rt] = __builtin_bit_cast(bf16x8, pw);
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const bf16x8 va = read_vt<D>(vt, dt, lane);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc.o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rt], acc.o[rt][dt], 0, 0, 0);
    }
    wave_lds_fence();
  }
}

// ---------------------------------------------------------------------------
template <int KV, int D, int RT>
__global__ __launch_bounds__(kThreads) void vat_partial(PartialArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave % a.waves_rows;
  const int wk = wave / a.waves_rows;
  const int l16 = lane & 15;
  const int j4 = lane >> 4;

  const int y = blockIdx.y;
  const int h = y % a.hkv;
  const int rb = a.row_blocks - 1 - y / a.hkv;  // heaviest (latest tokens) first
  const int cid = blockIdx.x;
  ReqArrays ra{a.kv_indptr, a.last_page_len, a.qo_indptr, a.has_mask ? a.mask_indptr : nullptr,
               a.batch, a.page_shift, a.chunk_keys, a.num_kv_indices, a.tokens};
  Req r;
  Item it;
  if (!find_item(ra, cid, lane, r, it)) return;
  const int n_items = chunk_count(r.kv_len, a.chunk_keys);
  const int j = it.j;
  const int R = a.group * r.L;
  const int row0 = rb * a.rows_per_block;
  if (row0 >= R) return;
  const int t_hi = (min(row0 + a.rows_per_block, R) - 1) / a.group;

  // Key range of this work item: chunk j of the request's keys; a causal row
  // block needs nothing past its last token's own key.
  const int lo = j * a.chunk_keys;
  int hi = min(lo + a.chunk_keys, r.kv_len);
  if (!a.has_mask) hi = min(hi, r.prefix + t_hi + 1);
  Vis vis;
  vis.has_mask = a.has_mask;
  vis.masked_from = r.prefix;
  vis.hi = hi;
  const int last = max(hi - 1, 0);

  // Rows of this wave: tile rt covers rows row0 + (wr * RT + rt) * 16 + l16.
  int row_t[RT];
  int row_g[RT];
  bool row_ok[RT];
  unsigned long long row_bits[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row0 + (wr * RT + rt) * 16 + l16;
    row_t[rt] = row / a.group;
    row_g[rt] = row % a.group;
    row_ok[rt] = row < R;
    row_bits[rt] = 0;
    if (a.has_mask == 1 && row_ok[rt])
      row_bits[rt] = load_mask_row(a.mask, a.num_mask_bytes, r.mask_off, row_t[rt], r.L);
    else if (a.has_mask == 2 && row_ok[rt])
      row_bits[rt] = load_mask_row_bytes(a.mask, a.num_mask_bytes, r.mask_off, row_t[rt], r.L,
                                         r.prefix);
  }

  // Q^T operand fragments.
  constexpr int NKS = StepRegs<KV, D>::NKS;
  constexpr int QW = (KV == KV_F32) ? NKS : NKS * 4;
  unsigned qf[RT][QW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const long long qrow =
        ((long long)(r.q_start + min(row_t[rt], max(r.L - 1, 0))) * a.hq + h * a.group + row_g[rt]) *
        D;
    if constexpr (KV == KV_F32) {
      const float* qp = (const float*)a.q + qrow + (D / 4) * j4;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        u32x4 x = row_ok[rt] ? *(const u32x4*)(qp + 4 * i) : u32x4{0, 0, 0, 0};
        qf[rt][4 * i] = x.x;
        qf[rt][4 * i + 1] = x.y;
        qf[rt][4 * i + 2] = x.z;
        qf[rt][4 * i + 3] = x.w;
      }
    } else {
      const unsigned short* qp = (const unsigned short*)a.q + qrow;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 x = row_ok[rt] ? *(const u32x4*)(qp + qk_d0<KV>(ks, j4)) : u32x4{0, 0, 0, 0};
        qf[rt][4 * ks] = x.x;
        qf[rt][4 * ks + 1] = x.y;
        qf[rt][4 * ks + 2] = x.z;
        qf[rt][4 * ks + 3] = x.w;
      }
    }
  }

  Acc<KV, D, RT> acc;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    acc.m[rt] = kNegInf;
    acc.l[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc.o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  unsigned char* vt = smem + wave * (kStepKeys * D * 2);
  const int stride = a.waves_keys * kStepKeys;
  int n = lo + wk * kStepKeys;
  if (n < hi) {
    PageWindow win;
    window_init(win, a, r, n >> a.page_shift, lane);
    StepRegs<KV, D> sa, sb;
    load_step<KV, D>(sa, a, r, win, n, last, h, lane);
    while (true) {
      const int n2 = n + stride;
      if (n2 < hi) load_step<KV, D>(sb, a, r, win, n2, last, h, lane);
      compute_step<KV, D, RT>(acc, sa, qf, row_t, row_bits, vis, n, a.c_log2, vt, lane);
      n = n2;
      if (n >= hi) break;
      const int n3 = n + stride;
      if (n3 < hi) load_step<KV, D>(sa, a, r, win, n3, last, h, lane);
      compute_step<KV, D, RT>(acc, sb, qf, row_t, row_bits, vis, n, a.c_log2, vt, lane);
      n = n3;
      if (n >= hi) break;
    }
  }
  // Full row sums.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc.l[rt] = row_sum4(acc.l[rt]);

  // Combine the key-splitting waves (same rows, disjoint keys) through LDS.
  if (a.waves_keys > 1) {
    constexpr int NDT = D / 16;
    constexpr int SLOT = RT * NDT * 256 + RT * 32;  // floats
    float* slots = (float*)smem;
    for (int half = a.waves_keys / 2; half >= 1; half /= 2) {
      __syncthreads();
      if (wk >= half && wk < 2 * half) {
        float* sl = slots + ((wk - half) * a.waves_rows + wr) * SLOT;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) *(f32x4*)(sl + ((rt * NDT + dt) * 64 + lane) * 4) = acc.o[rt][dt];
          if (j4 == 0) {
            sl[RT * NDT * 256 + rt * 32 + l16] = acc.m[rt];
            sl[RT * NDT * 256 + rt * 32 + 16 + l16] = acc.l[rt];
          }
        }
      }
      __syncthreads();
      if (wk < half) {
        const float* sl = slots + (wk * a.waves_rows + wr) * SLOT;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float mb = sl[RT * NDT * 256 + rt * 32 + l16];
          const float lb = sl[RT * NDT * 256 + rt * 32 + 16 + l16];
          const float m = fmaxf(acc.m[rt], mb);
          const float base = (m == kNegInf) ? 0.f : m;
          const float wa = fast_exp2(acc.m[rt] - base);
          const float wb = fast_exp2(mb - base);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const f32x4 ob = *(const f32x4*)(sl + ((rt * NDT + dt) * 64 + lane) * 4);
            acc.o[rt][dt] = acc.o[rt][dt] * wa + ob * wb;
          }
          acc.l[rt] = acc.l[rt] * wa + lb * wb;
          acc.m[rt] = m;
        }
      }
    }
  }
  if (wk != 0) return;

  // Write: direct -> out (q dtype) and natural-log lse; split -> fp32 partial
  // (normalised, v_scale not yet applied) and base-2 lse.
  const bool final_write = n_items == 1;
  const long long pid = ((long long)it.slot * a.hkv + h) * a.row_blocks + rb;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (!row_ok[rt]) continue;
    const float lsum = acc.l[rt];
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float lse2 = lsum > 0.f ? acc.m[rt] + fast_log2(lsum) : kNegInf;
    const int local = (wr * RT + rt) * 16 + l16;
    if (final_write) {
      const long long orow =
          ((long long)(r.q_start + row_t[rt]) * a.hq + h * a.group + row_g[rt]) * D;
      const float sc = inv * a.v_scale;
      if constexpr (KV == KV_F32) {
        float* op = (float*)a.out + orow;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) *(f32x4*)(op + 16 * dt + 4 * j4) = acc.o[rt][dt] * sc;
      } else {
        unsigned short* op = (unsigned short*)a.out + orow;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const f32x4 v = acc.o[rt][dt] * sc;
          u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(u32x2*)(op + 16 * dt + 4 * j4) = pk;
        }
      }
      if (j4 == 0)
        a.lse[(long long)(r.q_start + row_t[rt]) * a.hq + h * a.group + row_g[rt]] =
            lsum > 0.f ? lse2 * kLn2 : kNegInf;
    } else {
      float* op = a.part_o + ((long long)pid * a.rows_per_block + local) * D;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *(f32x4*)(op + 16 * dt + 4 * j4) = acc.o[rt][dt] * inv;
      if (j4 == 0) a.part_lse[(long long)pid * a.rows_per_block + local] = lse2;
    }
  }
}

// ---------------------------------------------------------------------------
typedef void (*PartialFn)(PartialArgs);

template <int KV, int D>
static PartialFn pick_rt(int rt) {
  switch (rt) {
    case 1: return vat_partial<KV, D, 1>;
    case 2: return vat_partial<KV, D, 2>;
    default: return vat_partial<KV, D, 3>;
  }
}

const void* tile_kernel(int kv_dtype, int head_dim, int rt) {
  if (kv_dtype == KV_F32) return (const void*)(head_dim == 64 ? pick_rt<KV_F32, 64>(rt) : pick_rt<KV_F32, 128>(rt));
  if (kv_dtype == KV_BF16) return (const void*)(head_dim == 64 ? pick_rt<KV_BF16, 64>(rt) : pick_rt<KV_BF16, 128>(rt));
  return (const void*)(head_dim == 64 ? pick_rt<KV_E4M3, 64>(rt) : pick_rt<KV_E4M3, 128>(rt));
}

}  // namespace vat
