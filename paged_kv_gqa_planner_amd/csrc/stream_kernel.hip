// Streaming partial kernel for verify shapes (bf16 or fp8 e4m3 caches, at
// most 96 query rows per KV head).
//
// One workgroup (eight wave64s, two per SIMD) per (chunk of a request's keys,
// KV head). It holds all G * L_b query rows of the KV head (row r = t * G + g),
// so every key and value of the chunk is read from HBM once per KV head
// (flashmap page "sglang/verify_attention.py", module docstring: all G query
// heads of a KV head in one program). The chunk is streamed through a ring of
// 64-key LDS stages filled by gfx950's direct global->LDS 16-byte loads
// (global_load_lds_dwordx4), gathered page by page through the page table
// (FlashInfer page "feat: Separate Q and KV dtypes for decode", paged layout);
// the ring keeps several stages in flight without holding them in registers.
//
// The eight waves form two groups of four. In a group, wave k owns the k-th
// 16-key tile of a stage. With two or more 16-row tiles the groups split the
// row tiles; with a single tile they take alternate stages. Per wave and tile:
//   S^T = K . Q^T      v_mfma_f32_16x16x32_bf16 (A = K from LDS, B = Q^T in VGPRs)
//   online softmax     base 2, one running max per row, raised lazily
//   O^T += V^T . P^T   v_mfma_f32_16x16x16_bf16 (A = V^T read with the LDS
//                      transpose load ds_read_b64_tr_b16 for bf16 caches,
//                      B = P^T: the exponentiated S^T tile, already in place)
// fp8 keys and values are decoded to bf16 in registers (exactly) right after
// the LDS reads. The draft block at the end of the request is masked in place:
// draft j is visible to token t iff j <= t (causal) or mask bit (t, j) is set.
// The waves' partial results are combined through LDS; a chunk that is its
// request's only one writes out and lse, otherwise a normalised fp32 partial
// and its base-2 log-sum-exp go to the workspace for the merge.
#include <utility>

#include "device_common.h"

namespace vat {

constexpr int kSWaves = kStreamThreads / 64;  // 8
constexpr int kGroupWaves = 4;

template <int KV, int D>
struct StreamGeom {
  static constexpr int EB = (KV == KV_E4M3) ? 1 : 2;  // bytes per cache element
  static constexpr int ROW = D * EB;                   // bytes per key row
  static constexpr int CPK = ROW / 16;                 // 16-byte chunks per key row
  static constexpr int KPI = 64 / CPK;                 // keys per 1 KB DMA instruction
  static constexpr int NINST = kStageKeys / KPI;       // DMA instructions per K (or V) block
  static constexpr int IPW = NINST / kSWaves;          // per wave per block
  static constexpr int NPW = 2 * IPW;                  // per wave per stage (K and V)
  static constexpr int BLK = kStageKeys * ROW;         // bytes of one K (or V) block
  static constexpr int STAGE = 2 * BLK;
  static_assert(IPW >= 1 && NINST % kSWaves == 0, "stage must split over the waves");
};

// LDS position of 16-byte chunk c of stage-local key kl: chunks are XOR
// swizzled by the key so that the operand reads below (sixteen keys at one
// chunk, or four keys at two chunks) fall in distinct banks.
template <int CPK>
__device__ __forceinline__ int swz(int kl, int c) { return c ^ (kl & (CPK - 1)); }

// Max / sum over the four lanes l, l^16, l^32, l^48 of one query row, on the
// VALU: permlane16/32_swap hand each lane its partner's value.
__device__ __forceinline__ float rowmax4_v(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (int)b[0]), __builtin_bit_cast(float, (int)b[1]));
}
__device__ __forceinline__ float rowsum4_v(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  x = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return __builtin_bit_cast(float, (int)b[0]) + __builtin_bit_cast(float, (int)b[1]);
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

// ---------------------------------------------------------------------------
// The chunk's page ids are staged in LDS (kStreamPageWindow entries from
// request page `base` on), so the DMA issue reads them with LDS loads and never
// waits on the vector-memory counter that paces the stage ring.
__device__ __forceinline__ int page_id(const PartialArgs& a, const Req& r, int rel_page) {
  const int idx = clampi(r.kv_start + clampi(rel_page, 0, max(r.pages - 1, 0)), 0,
                         max(a.num_kv_indices - 1, 0));
  return clampi(a.kv_indices[idx], 0, a.num_pages - 1);
}

__device__ __forceinline__ void fill_page_window(int* win, const PartialArgs& a, const Req& r,
                                                 int base, int last_page) {
  const int n = min(kStreamPageWindow, last_page - base + 1);
  for (int i = threadIdx.x; i < n; i += kStreamThreads) win[i] = page_id(a, r, base + i);
}

// Issue this wave's share of the DMA loads of one stage: keys n0 .. n0 + 63,
// each clamped to `last` (the item's last key) so every address is a real
// cached entry; keys past the item are masked out of the softmax later.
template <int KV, int D>
__device__ __forceinline__ void issue_stage(const PartialArgs& a, const int* win, int win_base,
                                            int last_rel, int h, int n0, int last,
                                            unsigned char* stage, int wave, int lane,
                                            bool uniform_pages) {
  using G = StreamGeom<KV, D>;
  const int ps_mask = (1 << a.page_shift) - 1;
  const long long page_bytes = (long long)G::ROW * a.hkv << a.page_shift;
  int pg[G::IPW];
#pragma unroll
  for (int ii = 0; ii < G::IPW; ++ii) {
    const int i = wave * G::IPW + ii;
    const int n = min(n0 + i * G::KPI + lane / G::CPK, last);
    const int first = min(n0 + i * G::KPI, last);
    const int rel = uniform_pages ? (first >> a.page_shift) - win_base : (n >> a.page_shift) - win_base;
    pg[ii] = win[clampi(rel, 0, last_rel)];
  }
#pragma unroll
  for (int ii = 0; ii < G::IPW; ++ii) {
    const int i = wave * G::IPW + ii;
    const int kl = i * G::KPI + lane / G::CPK;
    const int c = swz<G::CPK>(kl, lane % G::CPK);
    const int n = min(n0 + kl, last);
    const unsigned off = (unsigned)(((n & ps_mask) * a.hkv + h) * G::ROW + c * 16);
    const unsigned char* kb;
    const unsigned char* vb;
    if (uniform_pages) {
      // One page per instruction: a scalar page base plus 32-bit lane offsets.
      const long long base = (long long)__builtin_amdgcn_readfirstlane(pg[ii]) * page_bytes;
      kb = (const unsigned char*)a.k_cache + base;
      vb = (const unsigned char*)a.v_cache + base;
    } else {
      const long long base = (long long)pg[ii] * page_bytes;
      kb = (const unsigned char*)a.k_cache + base;
      vb = (const unsigned char*)a.v_cache + base;
    }
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(kb + off), (lds_void_t*)(stage + i * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(vb + off), (lds_void_t*)(stage + G::BLK + i * 1024),
                                     16, 0, 0);
  }
}

// Wait until this wave's loads of the oldest in-flight stage have landed,
// with `newer` younger stages still allowed in flight.
template <int NPW, int NS>
__device__ __forceinline__ void wait_stage(int newer) {
  static_assert(NPW * (NS - 1) < 64, "vmcnt range");
  switch (newer) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<NPW * 1>(); break;
    case 2: if constexpr (NS > 2) wait_vmcnt<NPW * 2>(); break;
    case 3: if constexpr (NS > 3) wait_vmcnt<NPW * 3>(); break;
    case 4: if constexpr (NS > 4) wait_vmcnt<NPW * 4>(); break;
    case 5: if constexpr (NS > 5) wait_vmcnt<NPW * 5>(); break;
    case 6: if constexpr (NS > 6) wait_vmcnt<NPW * 6>(); break;
    default: if constexpr (NS > 7) wait_vmcnt<NPW * 7>(); break;
  }
}

// ---------------------------------------------------------------------------
template <int D, int RT>
struct StreamAcc {
  f32x4 o[RT][D / 16];  // O^T tiles: lane (row l % 16, j = l / 16) holds d = 16 dt + 4 j + e
  float m[RT];          // running max of base-2 scaled logits (uniform over the row's lanes)
  float l[RT];          // this lane's share of the running sum
};

// Largest base-2 amount by which a tile's max may exceed the running max
// before the accumulators are rescaled.
constexpr float kRescaleSlack = 8.0f;

struct Vis {
  int hi;           // keys >= hi are outside the item
  int masked_from;  // keys >= masked_from are drafts: causal or mask
  int has_mask;
};

template <int KV, int D, int RT>
__device__ __forceinline__ void compute_stage(StreamAcc<D, RT>& acc, const unsigned (&qf)[RT][D / 8],
                                              const int (&row_t)[RT],
                                              const unsigned long long (&row_bits)[RT],
                                              const Vis& vis, const unsigned char* stage, int n0,
                                              float c, int kw, int lane) {
  using G = StreamGeom<KV, D>;
  const int l16 = lane & 15;
  const int j4 = lane >> 4;
  // ---- S^T tile of this wave's 16 keys against its row tiles
  f32x4 st[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) st[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int klk = 16 * kw + l16;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    u32x4 kw4;
    if constexpr (KV == KV_E4M3) {
      const int ch = 4 * (ks >> 1) + j4;
      const u32x2 raw = *(const u32x2*)(stage + klk * G::ROW + (swz<G::CPK>(klk, ch) << 4) + 8 * (ks & 1));
      kw4 = e4m3x8_to_bf16(raw.x, raw.y);
    } else {
      const int ch = 4 * ks + j4;
      kw4 = *(const u32x4*)(stage + klk * G::ROW + (swz<G::CPK>(klk, ch) << 4));
    }
    const bf16x8 ka = __builtin_bit_cast(bf16x8, kw4);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const u32x4 qw = {qf[rt][4 * ks], qf[rt][4 * ks + 1], qf[rt][4 * ks + 2], qf[rt][4 * ks + 3]};
      st[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, __builtin_bit_cast(bf16x8, qw), st[rt], 0, 0, 0);
    }
  }
  // ---- keys past the item, drafts under causal / mask
  const int nw = n0 + 16 * kw + 4 * j4;  // this lane's first key
  if (n0 + kStageKeys > vis.hi || n0 + kStageKeys > vis.masked_from) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int n = nw + e;
      const int jd = n - vis.masked_from;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        bool ok = n < vis.hi;
        if (jd >= 0) {
          if (vis.has_mask) ok = ok && jd < 64 && ((row_bits[rt] >> jd) & 1ull);
          else ok = ok && jd <= row_t[rt];
        }
        if (!ok) st[rt][e] = kNegInf;
      }
    }
  }
  // ---- online softmax (base 2); p replaces the logits. The running max is
  // raised only when a tile's max exceeds it by more than kRescaleSlack, so
  // the accumulators are rescaled rarely; p = 2^(s c - m) then stays below
  // 2^kRescaleSlack, and out and lse use the same m, so the result is exact.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float mx = fmaxf(fmaxf(st[rt][0], st[rt][1]), fmaxf(st[rt][2], st[rt][3]));
    mx = rowmax4_v(mx) * c;
    const bool grow = mx > acc.m[rt] + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : acc.m[rt];
      const float alpha = grow ? fast_exp2(acc.m[rt] - m_new) : 1.f;  // 0 when m was -inf
      acc.l[rt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc.o[rt][dt] *= alpha;
      acc.m[rt] = m_new;
    }
    // Rows that have seen nothing keep m = -inf; base 0 gives p = 0 for them.
    const float base = (acc.m[rt] == kNegInf) ? 0.f : acc.m[rt];
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = fast_exp2(__builtin_fmaf(st[rt][e], c, -base));
      st[rt][e] = p;
      sum += p;
    }
    acc.l[rt] += sum;
  }
  // ---- O^T += V^T . P^T
  s16x4 pb[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
    pb[rt] = __builtin_bit_cast(s16x4, u32x2{cvt_pk_bf16(st[rt][0], st[rt][1]),
                                             cvt_pk_bf16(st[rt][2], st[rt][3])});
  const unsigned char* vb = stage + G::BLK;
  constexpr int NDT = D / 16;
  if constexpr (KV == KV_E4M3) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      // Lane (d = l % 16, j = l / 16): codes of keys 16 kw + 4 j + e at d.
      const int kl0 = 16 * kw + 4 * j4;
      const int byte = 16 * dt + l16;
      const int ch = byte >> 4, within = byte & 15;
      unsigned b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        b[e] = vb[(kl0 + e) * G::ROW + (swz<G::CPK>(kl0 + e, ch) << 4) + within];
      const unsigned packed = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
      const s16x4 va = __builtin_bit_cast(
          s16x4, u32x2{e4m3x2_to_bf16x2(packed, false), e4m3x2_to_bf16x2(packed, true)});
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc.o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb[rt], acc.o[rt][dt], 0, 0, 0);
    }
  } else {
    // Transpose loads: source lane s of each 16-lane group points at the 8
    // bytes V[key 16 kw + 4 j + s / 4][d = 16 dt + 4 (s % 4) ..]; lane (d, j)
    // then receives V[16 kw + 4 j + e][16 dt + d], e = 0..3. All NDT reads
    // are issued first; tile dt waits only for its own.
    const int kl = 16 * kw + 4 * j4 + (l16 >> 2);
    s16x4 va[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int d0 = 16 * dt + 4 * (l16 & 3);
      const int ch = d0 >> 3;
      va[dt] = lds_read_tr16(vb + kl * G::ROW + (swz<G::CPK>(kl, ch) << 4) + (d0 & 7) * 2);
    }
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((lds_wait_tied<NDT - 1 - I>(va[I]),
        [&] {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            acc.o[rt][I] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[I], pb[rt], acc.o[rt][I], 0, 0, 0);
        }()),
       ...);
    }(std::make_integer_sequence<int, NDT>{});
  }
}

// Combine the partial (m, l, o) of waves that hold the same rows: waves
// [0, n) of the set fold into wave 0 through LDS slots, halving each round.
template <int D, int RT>
__device__ __forceinline__ void combine_waves(StreamAcc<D, RT>& acc, float* slots, int set,
                                              int idx, int n, int lane) {
  constexpr int NDT = D / 16;
  constexpr int SLOT = RT * NDT * 256 + RT * 32;  // floats
  const int l16 = lane & 15, j4 = lane >> 4;
  for (int half = n / 2; half >= 1; half /= 2) {
    __syncthreads();
    if (idx >= half && idx < 2 * half) {
      float* sl = slots + (set * (n / 2) + (idx - half)) * SLOT;
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
    if (idx < half) {
      const float* sl = slots + (set * (n / 2) + idx) * SLOT;
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

// ---------------------------------------------------------------------------
// One segment of work: keys [lo, hi) of request b for KV head h, all of its
// query rows. `final_write`: the segment is the whole request, so out and lse
// are written; otherwise partial slot `slot` is.
// RT: 16-row tiles per wave. ALT: one row tile, the two wave groups take
// alternate stages; otherwise group g holds row tiles [g RT, g RT + RT).
template <int KV, int D, int RT, int NS, bool ALT>
__device__ __forceinline__ void process_segment(const PartialArgs& a, const Req& r, int lo, int hi,
                                                bool final_write, int slot, int h,
                                                unsigned char* smem, int wave, int lane) {
  using G = StreamGeom<KV, D>;
  const int grp = wave / kGroupWaves;
  const int kw = wave % kGroupWaves;
  const int l16 = lane & 15;
  const int j4 = lane >> 4;
  const int R = a.group * r.L;
  Vis vis{hi, r.prefix, a.has_mask};
  const int last = max(hi - 1, 0);
  const int nst = hi > lo ? (hi - lo + kStageKeys - 1) / kStageKeys : 0;

  // ---- rows: tile rt of this wave, lane row row0 + rt * 16 + l16
  const int row0 = ALT ? 0 : grp * RT * 16;
  int row_t[RT], row_g[RT];
  bool row_ok[RT];
  unsigned long long row_bits[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row0 + rt * 16 + l16;
    row_t[rt] = row / a.group;
    row_g[rt] = row % a.group;
    row_ok[rt] = row < R;
    row_bits[rt] = 0;
    if (a.has_mask && row_ok[rt])
      row_bits[rt] = load_mask_row(a.mask, a.num_mask_bytes, r.mask_off, row_t[rt], r.L);
  }
  // Q^T operand: lane (row, j) holds d = qk_d(ks, j) .. +7 for each 32-wide step ks.
  unsigned qf[RT][D / 8];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const long long qrow =
        ((long long)(r.q_start + min(row_t[rt], r.L - 1)) * a.hq + h * a.group + row_g[rt]) * D;
    const unsigned short* qp = (const unsigned short*)a.q + qrow;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const int d0 = (KV == KV_E4M3) ? 64 * (ks >> 1) + 16 * j4 + 8 * (ks & 1) : 32 * ks + 8 * j4;
      const u32x4 x = row_ok[rt] ? *(const u32x4*)(qp + d0) : u32x4{0, 0, 0, 0};
      qf[rt][4 * ks] = x.x;
      qf[rt][4 * ks + 1] = x.y;
      qf[rt][4 * ks + 2] = x.z;
      qf[rt][4 * ks + 3] = x.w;
    }
  }
  // ---- page ids of the segment into LDS. The Q and mask loads above are in
  // flight meanwhile; all of them have landed once this returns, so the ring
  // below starts with no register load outstanding (a load still pending
  // there would make every stage wait for all of its queued DMA).
  int* win = (int*)(smem + NS * G::STAGE);
  const int last_page = last >> a.page_shift;
  int win_base = lo >> a.page_shift;
  if (nst > 0) fill_page_window(win, a, r, win_base, last_page);
  wait_vmcnt<0>();

  // A group whose tiles hold no row skips the math (it still issues loads).
  const bool has_rows = row0 < R;

  StreamAcc<D, RT> acc;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    acc.m[rt] = kNegInf;
    acc.l[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc.o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- the stage ring
  // Iteration s: wait for this wave's stage-s loads, barrier (everyone's
  // stage-s loads have landed and every wave is done with stage s - 1),
  // refill the buffer of stage s - 1 with stage s + NS - 1, compute stage s.
  // The barrier after the page-window fill also keeps a previous segment's
  // combine slots (which alias the stage buffers) safe from the new loads.
  __syncthreads();
  if (nst > 0) {
    const bool uniform_pages = (1 << a.page_shift) >= G::KPI;
    auto issue = [&](int s) {
      const int n0 = lo + s * kStageKeys;
      const int p_hi = min(n0 + kStageKeys - 1, last) >> a.page_shift;
      if (p_hi - win_base >= kStreamPageWindow) {
        // Long segment: move the window (drains the ring; once per window).
        wait_vmcnt<0>();
        __syncthreads();
        win_base = min(n0, last) >> a.page_shift;
        fill_page_window(win, a, r, win_base, last_page);
        __syncthreads();
      }
      issue_stage<KV, D>(a, win, win_base, min(last_page - win_base, kStreamPageWindow - 1), h, n0,
                         last, smem + (s % NS) * G::STAGE, wave, lane, uniform_pages);
    };
    for (int s = 0; s < NS - 1; ++s)
      if (s < nst) issue(s);
    for (int s = 0; s < nst; ++s) {
      wait_stage<G::NPW, NS>(min(NS - 2, nst - 1 - s));
      __builtin_amdgcn_s_barrier();
      if (s + NS - 1 < nst) issue(s + NS - 1);
      if (has_rows && (!ALT || (s & 1) == grp))
        compute_stage<KV, D, RT>(acc, qf, row_t, row_bits, vis, smem + (s % NS) * G::STAGE,
                                 lo + s * kStageKeys, a.c_log2, kw, lane);
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc.l[rt] = rowsum4_v(acc.l[rt]);

  // ---- combine waves that hold the same rows
  float* slots = (float*)smem;
  if (ALT) combine_waves<D, RT>(acc, slots, 0, wave, kSWaves, lane);
  else combine_waves<D, RT>(acc, slots, grp, kw, kGroupWaves, lane);
  if (ALT ? wave != 0 : (kw != 0 || !has_rows)) return;

  // ---- write: out (q dtype) and natural-log lse for a whole request;
  // otherwise a normalised fp32 partial (v_scale not yet applied) and its
  // base-2 log-sum-exp.
  constexpr int NDT = D / 16;
  const long long pid = (long long)slot * a.hkv + h;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (!row_ok[rt]) continue;
    const float lsum = acc.l[rt];
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float lse2 = lsum > 0.f ? acc.m[rt] + fast_log2(lsum) : kNegInf;
    const int local = row0 + rt * 16 + l16;
    if (final_write) {
      const long long orow = (long long)(r.q_start + row_t[rt]) * a.hq + h * a.group + row_g[rt];
      unsigned short* op = (unsigned short*)a.out + orow * D;
      const float sc = inv * a.v_scale;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const f32x4 v = acc.o[rt][dt] * sc;
        *(u32x2*)(op + 16 * dt + 4 * j4) = u32x2{cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3])};
      }
      if (j4 == 0) a.lse[orow] = lsum > 0.f ? lse2 * kLn2 : kNegInf;
    } else {
      float* op = a.part_o + (pid * a.rows_per_block + local) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) *(f32x4*)(op + 16 * dt + 4 * j4) = acc.o[rt][dt] * inv;
      if (j4 == 0) a.part_lse[pid * a.rows_per_block + local] = lse2;
    }
  }
}

template <int KV, int D, int RT, int NS, bool ALT>
__global__ __launch_bounds__(kStreamThreads, 1) void vat_stream(PartialArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  ReqArrays ra{a.kv_indptr, a.last_page_len, a.qo_indptr, a.has_mask ? a.mask_indptr : nullptr,
               a.batch, a.page_shift, a.chunk_keys, a.num_kv_indices, a.tokens};
  Req r;
  int lo, hi, slot;
  bool whole;
  if (a.slices == 0) {
    // Chunks: work item blockIdx.x is chunk j of some request.
    Item it;
    if (!find_item(ra, blockIdx.x, lane, r, it) || r.L == 0) return;
    lo = it.j * a.chunk_keys;
    hi = min(lo + a.chunk_keys, r.kv_len);
    whole = chunk_count(r.kv_len, a.chunk_keys) == 1;
    slot = it.slot;
    process_segment<KV, D, RT, NS, ALT>(a, r, lo, hi, whole, slot, h, smem, wave, lane);
    return;
  }
  // Balanced slices: workgroup x takes [x per, (x + 1) per) of the
  // concatenated key range, request segment by request segment. Every wave
  // scans the lengths; wave 0 leaves the table in LDS (past the page window)
  // so nothing per-request stays in registers across segments (field k of
  // request i at tab[64 k + i]).
  int* tab = (int*)(smem + NS * StreamGeom<KV, D>::STAGE + kStreamPageWindow * 4);
  int b, x0, x1;
  {
    SliceLanes sl;
    slice_lanes(ra, a.slices, lane, sl);
    x0 = blockIdx.x * sl.per;
    x1 = min(x0 + sl.per, sl.total);
    b = __popcll(__ballot(lane < a.batch && sl.cum + sl.n <= x0));
    if (wave == 0) {
      tab[0 * 64 + lane] = sl.ip0;
      tab[1 * 64 + lane] = sl.ip1;
      tab[2 * 64 + lane] = sl.lp;
      tab[3 * 64 + lane] = sl.q0;
      tab[4 * 64 + lane] = sl.q1;
      tab[5 * 64 + lane] = sl.mo;
      tab[6 * 64 + lane] = sl.cum;
      tab[7 * 64 + lane] = sl.n;
    }
  }
  if (x0 >= x1) return;
  __syncthreads();
  for (; b < a.batch; ++b) {
    const int cb = __builtin_amdgcn_readfirstlane(tab[6 * 64 + b]);
    if (cb >= x1) break;
    if (__builtin_amdgcn_readfirstlane(tab[7 * 64 + b]) == 0) continue;
    r = make_req(__builtin_amdgcn_readfirstlane(tab[b]), __builtin_amdgcn_readfirstlane(tab[64 + b]),
                 __builtin_amdgcn_readfirstlane(tab[128 + b]),
                 __builtin_amdgcn_readfirstlane(tab[192 + b]),
                 __builtin_amdgcn_readfirstlane(tab[256 + b]),
                 __builtin_amdgcn_readfirstlane(tab[320 + b]), a.page_shift, a.num_kv_indices,
                 a.tokens);
    lo = max(x0 - cb, 0);
    hi = min(x1 - cb, r.kv_len);
    if (lo >= hi) continue;
    // Opaque copies of the lane coordinates: what the segment derives from
    // them is recomputed per segment instead of being hoisted out of this
    // loop and held in registers across it.
    int lane_s = lane, wave_s = wave, h_s = h;
    asm volatile("" : "+v"(lane_s), "+v"(wave_s), "+s"(h_s));
    process_segment<KV, D, RT, NS, ALT>(a, r, lo, hi, lo == 0 && hi == r.kv_len, blockIdx.x + b, h_s,
                                        smem, wave_s, lane_s);
  }
}

// ---------------------------------------------------------------------------
typedef void (*PartialFn)(PartialArgs);

template <int KV, int D, int NS>
static PartialFn stream_rt(int tiles) {
  switch (tiles) {
    case 1: return vat_stream<KV, D, 1, NS, true>;
    case 2: return vat_stream<KV, D, 1, NS, false>;
    case 3:
    case 4: return vat_stream<KV, D, 2, NS, false>;
    default: return vat_stream<KV, D, 3, NS, false>;
  }
}

// `tiles`: 16-row tiles of the row block (1..6). Stage counts match the
// planner: 128 KB of LDS / (2 * 64 * D * elem bytes), at most 8.
const void* stream_kernel(int kv_dtype, int head_dim, int tiles) {
  if (kv_dtype == KV_BF16)
    return (const void*)(head_dim == 128 ? stream_rt<KV_BF16, 128, 4>(tiles) : stream_rt<KV_BF16, 64, 8>(tiles));
  return (const void*)stream_rt<KV_E4M3, 128, 8>(tiles);
}

}  // namespace vat
