// Streaming partial kernel for verify shapes (bf16 or fp8 e4m3 caches, at
// most 256 query rows per KV head).
//
// One workgroup (eight wave64s, two per SIMD) per (work item, KV head), or
// per (work item, group of two or four adjacent KV heads) for fp8 caches of
// head size 128. It holds all G * L_b query rows of each of its KV heads
// (row r = t * G + g), so every key and value is read from HBM once per KV
// head (flashmap page "sglang/verify_attention.py", module docstring: all G
// query heads of a KV head in one program). A work item is either a balanced
// slice of the page-index space, holding the segments of the requests whose
// pages fall in it, or one chunk of one request. Its keys stream through a
// ring of 32 KB LDS stages filled by gfx950's direct global->LDS 16-byte loads
// (global_load_lds_dwordx4), gathered page by page through the page table
// (FlashInfer page "feat: Separate Q and KV dtypes for decode", paged layout);
// the ring runs on across segment boundaries, so a slice pays the start-up
// latency once however many requests it touches.
//
// Wave w computes row tiles [w RT, w RT + RT) over every key of a segment, so
// its softmax state never has to be combined with another wave's:
//   S^T = K . Q^T      v_mfma_f32_16x16x32_bf16 (A = K from LDS, B = Q^T in VGPRs)
//   online softmax     base 2, one running max per row, raised lazily
//   O^T += V^T . P^T   v_mfma_f32_16x16x32_bf16 over 32 keys, two 16-key
//                      tiles side by side in k (A = V^T read with the LDS
//                      transpose loads ds_read_b64_tr_b16 for bf16 caches or
//                      ds_read_b64_tr_b8 for fp8, B = P^T: the exponentiated
//                      S^T tiles, already in place)
// fp8 keys and values are decoded to bf16 in registers (exactly) right after
// the LDS reads. The draft block at the end of the request is masked in place:
// draft j is visible to token t iff j <= t (causal) or mask bit (t, j) is set.
// A segment that is a whole request writes out and lse; otherwise a
// normalised fp32 partial and its base-2 log-sum-exp go to the workspace for
// the merge.
#include <utility>

#include "device_common.h"

namespace vat {

constexpr int kSWaves = kStreamThreads / 64;  // 8

// DW: waves issuing the DMA (2 or 4: the last ones of eight; 8: all of them);
// SK: keys per stage.
// HP: KV heads per workgroup (1, or 2 or 4 adjacent heads whose rows lie
// side by side in each slot, so a key row in LDS is all of their rows).
template <int KV, int D, int DW = kSWaves, int SK = kStageKeys, int HP = 1>
struct StreamGeom {
  static constexpr int EB = (KV == KV_E4M3) ? 1 : 2;  // bytes per cache element
  static constexpr int HROW = D * EB;                  // bytes of one head's key row
  static constexpr int ROW = HP * HROW;                // bytes per key row in LDS
  static constexpr int CPK = ROW / 16;                 // 16-byte chunks per key row
  static constexpr int KPI = 64 / CPK;                 // keys per 1 KB DMA instruction
  static constexpr int NINST = SK / KPI;               // DMA instructions per K (or V) block
  static constexpr int IPW = NINST / DW;               // per DMA wave per block
  static constexpr int NPW = 2 * IPW;                  // per DMA wave per stage (K and V)
  static constexpr int BLK = SK * ROW;                 // bytes of one K (or V) block
  static constexpr int STAGE = 2 * BLK;
  static_assert(IPW >= 1 && NINST % DW == 0, "stage must split over the DMA waves");
};

// LDS position of 16-byte chunk c of stage-local key kl: chunks are XOR
// swizzled by the key so that the operand reads below (sixteen keys at one
// chunk, or four keys at two chunks) fall in distinct banks. Rows of more
// than sixteen chunks (several heads side by side) swizzle within aligned
// groups of sixteen: that already spreads sixteen keys over every bank.
template <int CPK>
__device__ __forceinline__ int swz(int kl, int c) { return c ^ (kl & ((CPK < 16 ? CPK : 16) - 1)); }

// Where compute_stage finds 16-byte chunk `ch` of key `kl`'s row (of the
// wave's KV head) within a stage's K block, and where the V block starts.
// Per-head stages (vat_stream) hold one KV head's rows, one after another,
// chunks swizzled by swz().
// With several heads per workgroup a key row holds every one of their rows;
// `hc` is the wave's head's first chunk in it.
template <int KV, int D, int SK, int HP = 1>
struct HeadLayout {
  static constexpr int ROW = StreamGeom<KV, D, kStreamThreads / 64, SK, HP>::ROW;
  static constexpr int CPK = ROW / 16;
  static constexpr int VBLK = SK * ROW;
  // Key kl + 16 m sits 16 m rows after key kl at the same swizzled chunk
  // (the swizzle reads at most kl % 16), so the per-lane part of an address
  // is the same for every 16-key tile.
  static constexpr int KT_STRIDE = 16 * ROW;
  static_assert(CPK <= 16 || CPK % 16 == 0, "tile-invariant swizzle");
  int hc = 0;
  __device__ __forceinline__ int off(int kl, int ch) const {
    return kl * ROW + (swz<CPK>(kl, hc + ch) << 4);
  }
};

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

// Cache policy of the K/V loads: non-temporal. Each key is read once per
// KV head (or once per group of row blocks, which meet it in L2 within a
// stage or two), so its lines are not worth keeping in L2 ahead of other
// traffic. Same box, against default-policy loads: the fp8 batch-64 verify
// 121.5-122.1 -> 116.4-119.0 us, decode 215-217 -> 210 us, the chain verify
// 20.5 -> 19.1 us; prefill (row blocks sharing keys) unchanged.
constexpr int kCachePolicyNT = 2;

// ---------------------------------------------------------------------------
// Page ids of the work item live in an LDS window (kStreamPageWindow entries),
// so the DMA issue reads them with LDS loads and never waits on the
// vector-memory counter that paces the stage ring.
// Issue this wave's share of the DMA loads of one stage: keys n0 .. n0 + 63,
// each clamped to `last` (the item's last key) so every address is a real
// cached entry; keys past the item are masked out of the softmax later.
template <int KV, int D, int DW, int SK, int HP>
__device__ __forceinline__ void issue_stage(const PartialArgs& a, const int* win, int win_base,
                                            int last_rel, int h, int n0, int last,
                                            unsigned char* stage, int dw, int lane,
                                            bool uniform_pages) {
  using G = StreamGeom<KV, D, DW, SK, HP>;
  const int ps_mask = (1 << a.page_shift) - 1;
  const long long page_bytes = (long long)G::HROW * a.hkv << a.page_shift;
  int pg[G::IPW];
#pragma unroll
  for (int ii = 0; ii < G::IPW; ++ii) {
    const int i = dw * G::IPW + ii;
    const int n = min(n0 + i * G::KPI + lane / G::CPK, last);
    const int first = min(n0 + i * G::KPI, last);
    const int rel = uniform_pages ? (first >> a.page_shift) - win_base : (n >> a.page_shift) - win_base;
    pg[ii] = win[clampi(rel, 0, last_rel)];
  }
#pragma unroll
  for (int ii = 0; ii < G::IPW; ++ii) {
    const int i = dw * G::IPW + ii;
    const int kl = i * G::KPI + lane / G::CPK;
    const int c = swz<G::CPK>(kl, lane % G::CPK);
    const int n = min(n0 + kl, last);
    // Heads h .. h + HP - 1 of the key's slot, side by side.
    const unsigned off = (unsigned)(((n & ps_mask) * a.hkv + h) * G::HROW + c * 16);
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
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(kb + off), (lds_void_t*)(stage + i * 1024), 16, 0,
                                     kCachePolicyNT);
    __builtin_amdgcn_global_load_lds((gbl_void_t*)(vb + off), (lds_void_t*)(stage + G::BLK + i * 1024),
                                     16, 0, kCachePolicyNT);
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
  int t_min;        // smallest query token among this wave's rows
};

// An empty volatile asm statement: the rare branch it sits in (masking of the
// boundary stages, rescaling) stays a branch instead of being flattened into
// selects that would run on every stage.
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Visibility of keys c = 0..63 of a stage to one query row, as a bit mask:
// key c has draft index d + c (negative: a prefix key, always visible; 0..63:
// bit d + c of the row's draft bits; beyond: no draft) and must satisfy
// c <= lim (inside the item).
__device__ __forceinline__ unsigned long long visible_bits(unsigned long long bits, int d, int lim) {
  unsigned long long w;
  if (d >= 64) w = 0ull;
  else if (d >= 0) w = bits >> d;
  else if (d > -64) w = (bits << (-d)) | ((1ull << (-d)) - 1ull);
  else w = ~0ull;
  const unsigned long long in = lim >= 63 ? ~0ull : (lim < 0 ? 0ull : (2ull << lim) - 1ull);
  return w & in;
}

// One 64-key stage against this wave's RT row tiles. The four 16-key tiles
// are processed together: their S^T MFMAs interleave, the softmax takes one
// row max over all 64 keys, and the V^T reads of tile kt + 1 are in flight
// while tile kt's PV MFMAs run.
// KT: 16-key tiles this wave takes, tiles kt0 .. kt0 + KT - 1 of an SK-key
// stage.
// QLO: the queries are carried as two bf16 terms (qf + qlo, a rotated query
// that bf16 alone would round), and S^T takes one MFMA per term.
// VT (bf16 caches): form each V^T read's address per key tile instead of
// one base per d tile plus the tile's immediate offset. The latter takes
// fewer integer ops per stage and is faster where two row tiles share the
// reads; a lone computing wave that also issues DMA (decode) runs faster
// with the former (its schedule keeps eight fewer base registers live).
template <int KV, int D, int RT, int KT, int SK, bool QLO, class LAY, bool VT = false>
__device__ __forceinline__ void compute_stage(StreamAcc<D, RT>& acc, const unsigned (&qf)[RT][D / 8],
                                              const unsigned (&qlo)[RT][QLO ? D / 8 : 1],
                                              const int (&row_t)[RT],
                                              const unsigned long long (&row_bits)[RT],
                                              const Vis& vis, const unsigned char* stage, int n0,
                                              float c, int lane, int kt0, const LAY& lay) {
  static_assert(KT == 2 || KT == 4 || KT == 8, "one to four 32-key blocks");
  // Two row tiles per wave: the scheduler interleaves the stage's LDS reads
  // with its MFMAs (one-tile variants run faster with the default schedule).
  if constexpr (RT == 2) __builtin_amdgcn_iglp_opt(0);
  constexpr int NDT = D / 16;
  const int l16 = lane & 15;
  const int j4 = lane >> 4;
  constexpr int NB = KT / 2;  // 32-key blocks
  // fp8: the first 32-key block's V^T reads go out before the S^T products,
  // so their latency hides under QK and the softmax.
  unsigned vbase[NDT];
  u32x2 raw[2][KV == KV_E4M3 ? NDT : 1];
  if constexpr (KV == KV_E4M3) {
    const int e = l16 >> 1;
    const int klx = 16 * (e >> 2) + 4 * j4 + (e & 3);
    const unsigned sb = (unsigned)(uintptr_t)(const lds_void_t*)stage + kt0 * LAY::KT_STRIDE;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vbase[dt] = sb + lay.off(klx, dt) + 8 * (l16 & 1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) raw[0][dt] = lds_read_tr8_at<LAY::VBLK>(vbase[dt]);
  }
  // ---- S^T tiles: lane (key 16 kt + l % 16 as A row, query row l % 16 as
  // B column) accumulates over 32-wide d steps.
  f32x4 st[KT][RT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) st[kt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    bf16x8 ka[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int klk = 16 * (kt0 + kt) + l16;
      u32x4 kw4;
      if constexpr (KV == KV_E4M3) {
        const int ch = 4 * (ks >> 1) + j4;
        const u32x2 raw = *(const u32x2*)(stage + lay.off(klk, ch) + 8 * (ks & 1));
        kw4 = e4m3x8_to_bf16(raw.x, raw.y);
      } else {
        const int ch = 4 * ks + j4;
        kw4 = *(const u32x4*)(stage + lay.off(klk, ch));
      }
      ka[kt] = __builtin_bit_cast(bf16x8, kw4);
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const u32x4 qw = {qf[rt][4 * ks], qf[rt][4 * ks + 1], qf[rt][4 * ks + 2], qf[rt][4 * ks + 3]};
        st[kt][rt] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kt], __builtin_bit_cast(bf16x8, qw), st[kt][rt], 0, 0, 0);
        if constexpr (QLO) {
          const u32x4 ql = {qlo[rt][4 * ks], qlo[rt][4 * ks + 1], qlo[rt][4 * ks + 2], qlo[rt][4 * ks + 3]};
          st[kt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kt], __builtin_bit_cast(bf16x8, ql),
                                                               st[kt][rt], 0, 0, 0);
        }
      }
  }
  // ---- keys past the item, drafts under causal / mask. Lane (row, j) holds
  // keys 16 kt + 4 j + e.
  // Only stages that reach past the item, or hold drafts some row of this
  // wave may not see, test keys one by one (a causal stage whose drafts all
  // precede every row's token is fully visible).
  const int n_last = n0 + SK - 1;
  if (n_last >= vis.hi ||
      (n_last >= vis.masked_from && (vis.has_mask || n_last - vis.masked_from > vis.t_min))) {
    keep_branch();
    // One compare (causal) or one bit test (mask) and one select per logit,
    // no control flow. This lane's logit (kt, e) is key nb + c, c = 16 kt + e.
    const int nb = n0 + 16 * kt0 + 4 * j4;
    const int lim_in = vis.hi - 1 - nb;   // c <= lim_in: inside the item
    const int d0 = nb - vis.masked_from;  // draft index of c = 0 (negative: a prefix key)
    if (vis.has_mask) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const unsigned long long w0 = visible_bits(row_bits[rt], d0, lim_in);
        const unsigned long long w1 = KT > 4 ? visible_bits(row_bits[rt], d0 + 64, lim_in - 64) : 0ull;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = 16 * kt + e;
            const bool ok = (((c < 64 ? w0 : w1) >> (c & 63)) & 1ull) != 0ull;
            st[kt][rt][e] = ok ? st[kt][rt][e] : kNegInf;
          }
      }
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        // jd <= t  <=>  c <= t - d0 (row tokens are >= 0, so prefix keys pass)
        const int lim = min(lim_in, row_t[rt] - d0);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st[kt][rt][e] = (16 * kt + e <= lim) ? st[kt][rt][e] : kNegInf;
      }
    }
  }
  // ---- online softmax (base 2); p replaces the logits. The running max is
  // raised only when the stage's max exceeds it by more than kRescaleSlack,
  // so the accumulators are rescaled rarely; p = 2^(s c - m) then stays below
  // 2^kRescaleSlack, and out and lse use the same m, so the result is exact.
  s16x4 pb[KT][RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
      mx = fmaxf(mx, fmaxf(fmaxf(st[kt][rt][0], st[kt][rt][1]), fmaxf(st[kt][rt][2], st[kt][rt][3])));
    mx = rowmax4_v(mx) * c;
    const bool grow = mx > acc.m[rt] + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      keep_branch();
      const float m_new = grow ? mx : acc.m[rt];
      const float alpha = grow ? fast_exp2(acc.m[rt] - m_new) : 1.f;  // 0 when m was -inf
      acc.l[rt] *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc.o[rt][dt] *= alpha;
      acc.m[rt] = m_new;
    }
    // Rows that have seen nothing keep m = -inf; base 0 gives p = 0 for them.
    const float base = (acc.m[rt] == kNegInf) ? 0.f : acc.m[rt];
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(__builtin_fmaf(st[kt][rt][e], c, -base));
        sum += p[e];
      }
      pb[kt][rt] = __builtin_bit_cast(s16x4, u32x2{cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])});
    }
    acc.l[rt] += sum;
  }
  // ---- O^T += V^T . P^T, 32 keys per v_mfma_f32_16x16x32_bf16. Its k index
  // 8 j + e (lane group j) stands for key 4 j + e of tile 2 kb (e < 4) or key
  // 4 j + e - 4 of tile 2 kb + 1: the same order in both operands, so the
  // S^T tiles serve as P^T without moving, and V^T takes one 4-key read per
  // tile (the contraction does not depend on the order of k).
  auto mfma32 = [](s16x4 v_lo, s16x4 v_hi, s16x4 p_lo, s16x4 p_hi, f32x4 c) {
    const u32x2 a0 = __builtin_bit_cast(u32x2, v_lo), a1 = __builtin_bit_cast(u32x2, v_hi);
    const u32x2 b0 = __builtin_bit_cast(u32x2, p_lo), b1 = __builtin_bit_cast(u32x2, p_hi);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y}),
                                                   __builtin_bit_cast(bf16x8, u32x4{b0.x, b0.y, b1.x, b1.y}),
                                                   c, 0, 0, 0);
  };
  if constexpr (KV == KV_E4M3) {
    // One 8-bit transpose read per (32-key block, d tile): source lane s of
    // the 16-lane group j points at the 8 codes of k index 8 j + s / 2 at
    // d = 16 dt + 8 (s % 2) ..; lane (d, j) then receives the codes of k
    // indices 8 j .. 8 j + 7 at d, decoded exactly to bf16 in registers.
    // Block kb + 1's reads are in flight while block kb's MFMAs run.
    // Per-lane address of d tile dt in 32-key block 0; block kb adds the
    // immediate 2 kb KT_STRIDE.
    [&]<int... K>(std::integer_sequence<int, K...>) {
      (
          [&] {
            constexpr int kb = K;
            constexpr bool more = kb + 1 < NB;
            if constexpr (more) {
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt)
                raw[(kb + 1) & 1][dt] = lds_read_tr8_at<LAY::VBLK + 2 * (kb + 1) * LAY::KT_STRIDE>(vbase[dt]);
            }
            [&]<int... I>(std::integer_sequence<int, I...>) {
              ((lds_wait_tied<(more ? NDT : 0) + NDT - 1 - I>(raw[kb & 1][I]),
                [&] {
                  const bf16x8 va = __builtin_bit_cast(bf16x8, e4m3x8_to_bf16(raw[kb & 1][I].x, raw[kb & 1][I].y));
#pragma unroll
                  for (int rt = 0; rt < RT; ++rt) {
                    const u32x2 b0 = __builtin_bit_cast(u32x2, pb[2 * kb][rt]);
                    const u32x2 b1 = __builtin_bit_cast(u32x2, pb[2 * kb + 1][rt]);
                    acc.o[rt][I] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        va, __builtin_bit_cast(bf16x8, u32x4{b0.x, b0.y, b1.x, b1.y}), acc.o[rt][I], 0, 0, 0);
                  }
                }()),
               ...);
            }(std::make_integer_sequence<int, NDT>{});
          }(),
          ...);
    }(std::make_integer_sequence<int, NB>{});
  } else {
    // Transpose loads: source lane s of each 16-lane group points at the 8
    // bytes V[key 16 kt + 4 j + s / 4][d = 16 dt + 4 (s % 4) ..]; lane (d, j)
    // then receives V[16 kt + 4 j + e][16 dt + d], e = 0..3. Block kb's
    // second tile, and with one row tile block kb + 1's first, are requested
    // before block kb's MFMAs; each MFMA waits only for its own reads (LDS
    // reads complete in order).
    // Per-lane address of d tile dt in key tile 0; tile kt adds the
    // immediate kt KT_STRIDE.
    const int klb = 4 * j4 + (l16 >> 2);
    {
      const unsigned sb = (unsigned)(uintptr_t)(const lds_void_t*)stage + kt0 * LAY::KT_STRIDE;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d0 = 16 * dt + 4 * (l16 & 3);
        vbase[dt] = sb + lay.off(klb, d0 >> 3) + (d0 & 7) * 2;
      }
    }
    // V^T read of key tile kt (of this wave's), d tile dt.
    auto vread = [&]<int KTI>(int dt) {
      if constexpr (VT) {
        const int d0 = 16 * dt + 4 * (l16 & 3);
        return lds_read_tr16(stage + LAY::VBLK + lay.off(16 * (kt0 + KTI) + klb, d0 >> 3) + (d0 & 7) * 2);
      } else {
        return lds_read_tr16_at<LAY::VBLK + KTI * LAY::KT_STRIDE>(vbase[dt]);
      }
    };
    constexpr bool kAhead = RT == 1;  // registers for a third tile of reads
    constexpr int NBUF = kAhead ? 2 : 1;
    s16x4 va[NBUF][NDT], vv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) va[0][dt] = vread.template operator()<0>(dt);
    [&]<int... K>(std::integer_sequence<int, K...>) {
      (
          [&] {
            constexpr int kb = K;
            constexpr bool ahead = kAhead && kb + 1 < NB;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
              vv[dt] = vread.template operator()<2 * kb + 1>(dt);
            if constexpr (ahead) {
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt)
                va[(kb + 1) % NBUF][dt] = vread.template operator()<2 * kb + 2>(dt);
            }
            [&]<int... I>(std::integer_sequence<int, I...>) {
              ((lds_wait_tied2<(ahead ? NDT : 0) + NDT - 1 - I>(va[kb % NBUF][I], vv[I]),
                [&] {
#pragma unroll
                  for (int rt = 0; rt < RT; ++rt)
                    acc.o[rt][I] = mfma32(va[kb % NBUF][I], vv[I], pb[2 * kb][rt], pb[2 * kb + 1][rt], acc.o[rt][I]);
                }()),
               ...);
            }(std::make_integer_sequence<int, NDT>{});
            if constexpr (!kAhead && kb + 1 < NB) {
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt)
                va[(kb + 1) % NBUF][dt] = vread.template operator()<2 * kb + 2>(dt);
            }
          }(),
          ...);
    }(std::make_integer_sequence<int, NB>{});
  }
}

// ---------------------------------------------------------------------------
// The workgroup's segments, one per lane: segment i is keys [lo, hi) of one
// request. Its stages are numbered end to end across segments: segment i owns
// global stages [incl - nst, incl). `woff` is the page-window index of the
// request's page 0 (window index = position in kv_indices minus the window's
// first position).
struct SegLane {
  int lo = 0, hi = 0, nst = 0, incl = 0;
  int woff = 0, q_start = 0, L = 0, prefix = 0, mask_off = 0, slot = 0, whole = 0;
  int rb = 0;  // row block of the segment's rows
};

__device__ __forceinline__ int lane_val(int v, int i) { return __builtin_amdgcn_readlane(v, i); }

// Window page ids: entries [base, base + n) of the window range starting at
// kv_indices position w0, clamped to real pages.
__device__ __forceinline__ void fill_window(int* win, const PartialArgs& a, int w0, int base, int count) {
  const int n = min(kStreamPageWindow, count - base);
  for (int i = threadIdx.x; i < n; i += kStreamThreads)
    win[i] = clampi(a.kv_indices[w0 + base + i], 0, a.num_pages - 1);
}

// One wave's rows of a segment: Q^T operand fragments and mask rows. The
// loads are issued by fetch() and used only after the caller's wait, so no
// load is left for the compiler to wait on where the stages are computed:
// the mask bytes stay raw until finish(). The four lanes l, l ^ 16, l ^ 32,
// l ^ 48 hold one row and split its mask bytes: packed blocks (mask mode 1)
// take at most nine bytes from the row's first, three per lane; full byte
// rows (mode 2, ROWS) one byte per draft, sixteen per lane -- registers that
// only the ROWS instantiations (one row tile per wave) carry.
template <int KV, int D, int RT, bool ROWS, bool ROPE = false>
struct RowSet {
  static constexpr int kRaw = ROWS ? 16 : 3;
  // RoPE: cos then sin of the lane's rotated dimension pairs, 16 per 32-wide
  // d step of the first half (ROPE instantiations only).
  static constexpr int kCs = ROPE ? (D / 32 / 2) * 16 : 1;
  int row_t[RT], row_g[RT];
  bool row_ok[RT];
  unsigned long long row_bits[RT];
  unsigned qf[RT][D / 8];
  unsigned raw[RT][kRaw];  // this lane's share of the row's mask bytes
  unsigned csr[RT][kCs];   // RoPE cos/sin of the row's token (ROPE)
  unsigned qlo[RT][ROPE ? D / 8 : 1];  // ROPE: bf16 remainder of the rotated query

  __device__ __forceinline__ void fetch(const PartialArgs& a, int q_start, int L, int prefix,
                                        int mask_off, int row0, int h, int lane) {
    const int l16 = lane & 15, j4 = lane >> 4;
    const int R = a.group * L;
    const long long last = max(a.num_mask_bytes - 1, 0);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = row0 + rt * 16 + l16;
      row_t[rt] = row / a.group;
      row_g[rt] = row % a.group;
      row_ok[rt] = row < R;
      // Q^T operand: lane (row, j) holds d = qk_d(ks, j) .. +7 for each 32-wide step ks.
      const long long qrow =
          ((long long)(q_start + min(row_t[rt], L - 1)) * a.hq + h * a.group + row_g[rt]) * D;
      const unsigned short* qp = (const unsigned short*)a.q + qrow;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const int d0 = (KV == KV_E4M3) ? 64 * (ks >> 1) + 16 * j4 + 8 * (ks & 1) : 32 * ks + 8 * j4;
        const u32x4 x = *(const u32x4*)(qp + d0);
        qf[rt][4 * ks] = x.x;
        qf[rt][4 * ks + 1] = x.y;
        qf[rt][4 * ks + 2] = x.z;
        qf[rt][4 * ks + 3] = x.w;
      }
      const int t = min(row_t[rt], L - 1);
      if constexpr (ROPE) {
        // The 32-wide d steps ks < D / 64 hold the first halves of the rotated
        // pairs, and step ks + D / 64 of the same lane their partners: the
        // lane needs cos/sin of its 8 dimensions at each of the former.
        const float* cs = a.q_cos_sin + (long long)(q_start + t) * D;
#pragma unroll
        for (int ks = 0; ks < D / 64; ++ks) {
          const int d0 = (KV == KV_E4M3) ? 64 * (ks >> 1) + 16 * j4 + 8 * (ks & 1) : 32 * ks + 8 * j4;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              const u32x4 w = *(const u32x4*)(cs + half * (D / 2) + d0 + 4 * k);
              unsigned* dst = &csr[rt][ks * 16 + half * 8 + 4 * k];
              dst[0] = w.x;
              dst[1] = w.y;
              dst[2] = w.z;
              dst[3] = w.w;
            }
          }
        }
      }
      if constexpr (ROWS) {
        // Draft j of row t: byte mask_off + t (prefix + L) + prefix + j.
        const long long byte0 = mask_off + (long long)t * (prefix + L) + prefix + 16 * j4;
#pragma unroll
        for (int i = 0; i < 16; ++i) raw[rt][i] = a.mask[clampll(byte0 + i, 0, last)];
      } else if (a.has_mask) {
        // Row t of the packed L x L block starts at bit t L; L <= 64 bits
        // span at most nine bytes (indices clamped to the mask buffer).
        const long long byte0 = mask_off + ((t * L) >> 3) + 3 * j4;
#pragma unroll
        for (int i = 0; i < 3; ++i) raw[rt][i] = a.mask[j4 < 3 ? clampll(byte0 + i, 0, last) : 0];
      }
    }
  }

  __device__ __forceinline__ void finish(int L, int mask_mode, int lane) {
    const int j4 = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if constexpr (ROPE) {
        // x' = x c - y s, y' = y c + x s for the pair (x at step ks, y at step
        // ks + D / 64, same element), two elements (one word) at a time; the
        // result is kept as bf16 hi plus bf16 lo (about 2^-17 relative; hi
        // alone would be 2^-9), both rounded to nearest even by the packed
        // conversion.
#pragma unroll
        for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            unsigned& wx = qf[rt][4 * ks + k];
            unsigned& wy = qf[rt][4 * (ks + D / 64) + k];
            const float x0 = __builtin_bit_cast(float, wx << 16);
            const float x1 = __builtin_bit_cast(float, wx & 0xffff0000u);
            const float y0 = __builtin_bit_cast(float, wy << 16);
            const float y1 = __builtin_bit_cast(float, wy & 0xffff0000u);
            const float c0 = __builtin_bit_cast(float, csr[rt][ks * 16 + 2 * k]);
            const float c1 = __builtin_bit_cast(float, csr[rt][ks * 16 + 2 * k + 1]);
            const float s0 = __builtin_bit_cast(float, csr[rt][ks * 16 + 8 + 2 * k]);
            const float s1 = __builtin_bit_cast(float, csr[rt][ks * 16 + 8 + 2 * k + 1]);
            const float rx0 = __builtin_fmaf(x0, c0, -y0 * s0), rx1 = __builtin_fmaf(x1, c1, -y1 * s1);
            const float ry0 = __builtin_fmaf(y0, c0, x0 * s0), ry1 = __builtin_fmaf(y1, c1, x1 * s1);
            const unsigned hx = cvt_pk_bf16(rx0, rx1), hy = cvt_pk_bf16(ry0, ry1);
            qlo[rt][4 * ks + k] = cvt_pk_bf16(rx0 - __builtin_bit_cast(float, hx << 16),
                                              rx1 - __builtin_bit_cast(float, hx & 0xffff0000u));
            qlo[rt][4 * (ks + D / 64) + k] = cvt_pk_bf16(ry0 - __builtin_bit_cast(float, hy << 16),
                                                         ry1 - __builtin_bit_cast(float, hy & 0xffff0000u));
            wx = hx;
            wy = hy;
          }
      }
      if (!row_ok[rt]) {
#pragma unroll
        for (int k = 0; k < D / 8; ++k) qf[rt][k] = 0u;
        if constexpr (ROPE) {
#pragma unroll
          for (int k = 0; k < D / 8; ++k) qlo[rt][k] = 0u;
        }
      }
      // This lane's bits of the row, then the OR over its four lanes.
      unsigned long long part = 0;
      if constexpr (ROWS) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          part |= (unsigned long long)((raw[rt][i] & 0xffu) != 0u) << (16 * j4 + i);
      } else if (mask_mode) {
        const int sh = (min(row_t[rt], L - 1) * L) & 7;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          const int kb = 3 * j4 + i;  // byte of the row's span
          const int pos = 8 * kb - sh;
          const unsigned long long b = j4 < 3 ? (unsigned long long)(raw[rt][i] & 0xffu) : 0ull;
          part |= pos < 0 ? (b >> sh) : (pos < 64 ? (b << pos) : 0ull);
        }
      }
      if (mask_mode != 0) {
        unsigned lo = (unsigned)part, hi = (unsigned)(part >> 32);
        lo |= __shfl_xor(lo, 16);
        hi |= __shfl_xor(hi, 16);
        lo |= __shfl_xor(lo, 32);
        hi |= __shfl_xor(hi, 32);
        part = ((unsigned long long)hi << 32) | lo;
        if (L < 64) part &= (1ull << L) - 1ull;
      }
      row_bits[rt] = row_ok[rt] ? part : 0ull;
    }
  }
};

// Write a finished segment's rows of this wave (`lrow`: the rows' full sums):
// out (bf16) and natural-log lse for a whole request, otherwise a normalised
// fp32 partial (v_scale not yet applied) and its base-2 log-sum-exp in slot
// `slot`. The segment's rows are rbase .. rbase + 16 RT - 1 of the request's
// G L rows (row r = t G + g).
// `rb`: row block; `row0`: this wave's first row within the block.
// OPAQUE: the lane index passes through an empty asm first, so the
// compiler cannot hoist the lane-dependent part of these addresses out of
// the stage loop (where, in the two-tile two-pass variant, the hoisted
// values would not fit the registers and spill).
// Raw buffer resources (gfx9 family): word 3 of the descriptor for plain
// byte-addressed 32-bit data, with the hardware dropping out-of-range
// stores; the cache-policy operand's SC1 bit asks for device scope.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kCachePolicySC1 = 16;

// A pointer the compiler can keep in scalar registers (buffer descriptors
// must be); the caller guarantees it is the same in every lane.
__device__ __forceinline__ void* wave_uniform(const void* p) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(v >> 32));
  return (void*)(((unsigned long long)hi << 32) | lo);
}

template <int D, int RT, bool OPAQUE = false>
__device__ __forceinline__ void write_rows(const StreamAcc<D, RT>& acc, const float (&lrow)[RT],
                                           const PartialArgs& a, int q_start, int L, int rbase,
                                           bool whole, int slot, int rb, int row0, int h, int lane) {
  constexpr int NDT = D / 16;
  if constexpr (OPAQUE) asm volatile("" : "+v"(lane));
  const int l16 = lane & 15, j4 = lane >> 4;
  const long long pid = ((long long)slot * a.hkv + h) * a.row_blocks + rb;
  // Partials go out as device-scope buffer stores (cache policy SC1): written
  // through this XCD's L2 to the memory side, where the merge kernel reads
  // them, instead of staying dirty in L2 until the kernel's end flushes it.
  // Buffer bases must be wave-uniform; the segment's row block is.
  const __amdgpu_buffer_rsrc_t rpo = __builtin_amdgcn_make_buffer_rsrc(
      wave_uniform(a.part_o + pid * a.rows_per_block * D), 0,
      __builtin_amdgcn_readfirstlane(a.rows_per_block * D * 4), kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rpl = __builtin_amdgcn_make_buffer_rsrc(
      wave_uniform(a.part_lse + pid * a.rows_per_block), 0,
      __builtin_amdgcn_readfirstlane(a.rows_per_block * 4), kRawBufferWord3);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float lsum = lrow[rt];
    const int row = rbase + rt * 16 + l16;
    if (row >= a.group * L) continue;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float lse2 = lsum > 0.f ? acc.m[rt] + fast_log2(lsum) : kNegInf;
    const int local = row0 + rt * 16 + l16;
    if (whole) {
      const long long orow = (long long)(q_start + row / a.group) * a.hq + h * a.group + row % a.group;
      unsigned short* op = (unsigned short*)a.out + orow * D;
      const float sc = inv * a.v_scale;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const f32x4 v = acc.o[rt][dt] * sc;
        *(u32x2*)(op + 16 * dt + 4 * j4) = u32x2{cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3])};
      }
      if (j4 == 0) a.lse[orow] = lsum > 0.f ? lse2 * kLn2 : kNegInf;
    } else {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc.o[rt][dt] * inv), rpo,
                                               (local * D + 16 * dt + 4 * j4) * 4, 0, kCachePolicySC1);
      if (j4 == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse2), rpl, local * 4, 0,
                                              kCachePolicySC1);
    }
  }
}

// Softmax state of a row set in LDS, handed from the second wave of a tile
// pair to the first: O^T tiles as the lanes hold them, then the rows' running
// max and full sum.
template <int D, int RT>
struct PairSlot {
  static constexpr int NDT = D / 16;
  static constexpr int FLOATS = RT * NDT * 256 + RT * 32;
};

__device__ __forceinline__ void wait_lds_writes() {
  // s_waitcnt lgkmcnt(0), vector-memory and export counts left alone
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Workgroup barrier for hand-offs through LDS: the caller's LDS writes are
// complete first, while its global loads and stores (and the DMA waves' stage
// loads) stay in flight -- __syncthreads would wait for those too, draining
// the stage ring. The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  wait_lds_writes();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, int RT>
__device__ __forceinline__ void store_pair_state(const StreamAcc<D, RT>& acc, float* slot, int lane) {
  constexpr int NDT = D / 16;
  const int l16 = lane & 15, j4 = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float lrow = rowsum4_v(acc.l[rt]);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *(f32x4*)(slot + ((rt * NDT + dt) * 64 + lane) * 4) = acc.o[rt][dt];
    if (j4 == 0) {
      slot[RT * NDT * 256 + rt * 16 + l16] = acc.m[rt];
      slot[RT * NDT * 256 + RT * 16 + rt * 16 + l16] = lrow;
    }
  }
  wait_lds_writes();
}

// Fold the partner's state into acc; lrow receives the combined row sums.
template <int D, int RT>
__device__ __forceinline__ void merge_pair_state(StreamAcc<D, RT>& acc, float (&lrow)[RT],
                                                 const float* slot, bool partner, int lane) {
  constexpr int NDT = D / 16;
  const int l16 = lane & 15;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    lrow[rt] = rowsum4_v(acc.l[rt]);
    if (!partner) continue;
    const float mb = slot[RT * NDT * 256 + rt * 16 + l16];
    const float lb = slot[RT * NDT * 256 + RT * 16 + rt * 16 + l16];
    const float m = fmaxf(acc.m[rt], mb);
    const float base = (m == kNegInf) ? 0.f : m;
    const float wa = fast_exp2(acc.m[rt] - base);
    const float wb = fast_exp2(mb - base);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      acc.o[rt][dt] = acc.o[rt][dt] * wa + *(const f32x4*)(slot + ((rt * NDT + dt) * 64 + lane) * 4) * wb;
    lrow[rt] = lrow[rt] * wa + lb * wb;
    acc.m[rt] = m;
  }
}

// One workgroup per (work item, KV head). A work item is a balanced slice of
// the page-index space (batches of at most 64 requests) or one chunk of one
// request; either way a list of request segments whose 64-key stages flow
// through one ring of LDS buffers filled by DMA. Wave w < waves_rows owns row
// tiles [w RT, w RT + RT) of every segment and runs all of its keys, so no
// two waves ever hold parts of the same row; all eight waves issue the DMA.
// HP = 2 or 4: the workgroup takes HP adjacent KV heads, h .. h + HP - 1,
// whose rows sit side by side in every slot, so each key's DMA reads one run
// of all their rows; computing waves take the row tiles of h, then those of
// h + 1, and so on.
template <int KV, int D, int RT, int NS, int DW, int P, int SK, bool ROWS, bool ROPE, int HP = 1>
__global__ __launch_bounds__(kStreamThreads, 1) void vat_stream(PartialArgs a) {
  using G = StreamGeom<KV, D, DW, SK, HP>;
  // The argument block spans three 64-byte lines. Needing the first one
  // (the pointers) here puts it in the opening round of argument loads; left
  // alone, the compiler fetches it only after the block-index arithmetic, a
  // second dependent round of about half a microsecond before any request
  // table load can start.
  {
    const void* p0 = a.q;
    asm volatile("" ::"s"(p0));
  }
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  int* win = (int*)(smem + NS * G::STAGE);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // Row blocks of one KV head are dispatched longest first (under a causal
  // limit a later block reaches more keys). In block orders 1 and 2 the grid
  // is one-dimensional: workgroup L runs on XCD L % 8, and the W workgroups
  // of group q = (work item, KV head) are (q % 8) + 8 (W (q / 8) + k), so
  // they share that XCD's L2 and start within one round of eight groups.
  // Order 1: W = RB, workgroup k takes block RB - 1 - k. Order 2 (many
  // blocks): W = ceil(RB / 2), workgroup k takes blocks RB - 1 - k and k as
  // two segments of one ring -- half the workgroups pay the start-up, and the
  // longest causal block shares a workgroup with the shortest.
  int item, h, rb, rb2 = -1;
  if (a.block_order) {
    const int L = (int)blockIdx.x;
    const int W = a.block_order == 2 ? (a.row_blocks + 1) / 2 : a.row_blocks;
    const int q = (L & 7) + 8 * (L / (8 * W));
    if (q >= a.num_ids * a.hkv) return;
    item = q % a.num_ids;
    h = q / a.num_ids;
    const int k = (L >> 3) % W;
    rb = a.row_blocks - 1 - k;
    if (a.block_order == 2 && k < rb) rb2 = k;
  } else {
    item = (int)blockIdx.x;
    h = HP * (int)(blockIdx.y / a.row_blocks);  // first KV head of the workgroup
    rb = a.row_blocks - 1 - (int)(blockIdx.y % a.row_blocks);
  }
  const int shift = a.page_shift;

  // ---- the segment lanes and the page window: one round of loads for a slice
  SegLane sg;
  int w0, wcount;  // window range: kv_indices positions [w0, w0 + wcount)
  if (a.slices > 0) {
    const int per = (a.num_kv_indices + a.slices - 1) / a.slices;
    w0 = item * per;
    wcount = min(per, a.num_kv_indices - w0);
    if (wcount <= 0) return;
    // Page ids of the slice, requested with the request table below.
    constexpr int PT = kStreamPageWindow / kStreamThreads;
    int pid[PT];
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      const int i = threadIdx.x + k * kStreamThreads;
      pid[k] = i < min(wcount, kStreamPageWindow) ? a.kv_indices[w0 + i] : 0;
    }
    const bool in = lane < a.batch;
    const int i = in ? lane : 0;
    const Req r = make_req(a.kv_indptr[i], a.kv_indptr[i + 1], in ? a.last_page_len[i] : 1,
                           a.qo_indptr[i], a.qo_indptr[i + 1],
                           (a.has_mask && in) ? a.mask_indptr[i] : 0, shift, a.num_kv_indices,
                           a.tokens);
    const int p0 = max(r.kv_start, w0), p1 = min(r.kv_start + r.pages, w0 + wcount);
    if (in && r.L > 0 && p0 < p1) {
      sg.lo = (p0 - r.kv_start) << shift;
      sg.hi = min((p1 - r.kv_start) << shift, r.kv_len);
      sg.nst = (sg.hi - sg.lo + SK - 1) / SK;
      sg.woff = r.kv_start - w0;
      sg.q_start = r.q_start;
      sg.L = r.L;
      sg.prefix = r.prefix;
      sg.mask_off = r.mask_off;
      sg.slot = item + lane;
      sg.whole = sg.lo == 0 && sg.hi == r.kv_len;
      sg.rb = rb;
    }
#pragma unroll
    for (int k = 0; k < PT; ++k) {
      const int i2 = threadIdx.x + k * kStreamThreads;
      if (i2 < min(wcount, kStreamPageWindow)) win[i2] = clampi(pid[k], 0, a.num_pages - 1);
    }
  } else {
    // Chunk j of the request owning work item `item`: one segment (lane 0).
    ReqArrays ra{a.kv_indptr, a.last_page_len, a.qo_indptr, a.has_mask ? a.mask_indptr : nullptr,
                 a.batch, shift, a.chunk_keys, a.num_kv_indices, a.tokens};
    Req r;
    Item it;
    if (!find_item(ra, item, lane, r, it) || r.L == 0) return;
    const int lo = it.j * a.chunk_keys;
    const int hi_item = min(lo + a.chunk_keys, r.kv_len);
    const bool whole_item = chunk_count(r.kv_len, a.chunk_keys) == 1;
    // Keys [lo, hi) of row block b; an empty range when no row of the block
    // exists. Causal: no row of a block sees a key past its last row's token.
    auto block_hi = [&](int b) {
      if (b < 0 || b * a.rows_per_block >= a.group * r.L) return lo;
      if (!whole_item || a.has_mask) return hi_item;
      const int t_hi = min(r.L - 1, (b * a.rows_per_block + a.rows_per_block - 1) / a.group);
      return min(hi_item, r.prefix + t_hi + 1);
    };
    // Either block may hold no row of this request (shorter requests have
    // fewer blocks); an empty one is simply no segment.
    const int hi_a = block_hi(rb), hi_b = block_hi(rb2);
    const int hi_max = max(hi_a, hi_b);
    if (lo >= hi_max) return;
    w0 = r.kv_start + (lo >> shift);
    wcount = ((hi_max - 1) >> shift) - (lo >> shift) + 1;
    // Lane 0: block rb; lane 1: block rb2 (block order 2). Both restart at
    // key lo inside the same page window (the planner pairs only items that
    // fit the window).
    const int my_hi = lane == 0 ? hi_a : hi_b;
    if (lane < 2 && my_hi > lo) {
      sg.lo = lo;
      sg.hi = my_hi;
      sg.nst = (my_hi - lo + SK - 1) / SK;
      sg.woff = r.kv_start - w0;
      sg.q_start = r.q_start;
      sg.L = r.L;
      sg.prefix = r.prefix;
      sg.mask_off = r.mask_off;
      sg.slot = it.slot;
      sg.whole = whole_item;
      sg.rb = lane == 0 ? rb : rb2;
    }
  }
  // Global stage numbering: inclusive prefix sum of the stage counts.
  {
    int incl = sg.nst;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int up = __shfl_up(incl, o);
      if (lane >= o) incl += up;
    }
    sg.incl = incl;
  }
  const int nst_all = lane_val(sg.incl, 63);
  // Segment holding global stage g (wave-uniform).
  auto seg_of = [&](int g) { return (int)__popcll(__ballot(sg.incl <= g)); };

  // Computing wave w: row tile set w % waves_rows; with P = 2 the two waves
  // of a tile set take the first and the second half of every stage's keys,
  // and the second hands its softmax state to the first through LDS when a
  // segment ends.
  const int ncomp = a.waves_rows * P;
  const bool computes = wave < ncomp;
  const int tset = wave % a.waves_rows;
  const int phase = wave / a.waves_rows;
  const int tph = a.waves_rows / HP;          // tile sets per KV head
  const int hw = h + tset / tph;              // the wave's KV head
  const int row0 = (tset % tph) * RT * 16;    // within the row block
  int rbase = row0;                   // in the request's rows (set per segment)
  float* pair_slot = (float*)(smem + NS * G::STAGE + kStreamPageWindow * 4) + tset * PairSlot<D, RT>::FLOATS;
  RowSet<KV, D, RT, ROWS, ROPE> rs;
  StreamAcc<D, RT> acc;
  Vis vis{0, 0, a.has_mask, 0};
  bool has_rows = false;
  int seg_L = 0;
  auto start_segment = [&](int s) {
    rbase = lane_val(sg.rb, s) * a.rows_per_block + row0;
    seg_L = lane_val(sg.L, s);
    has_rows = rbase < a.group * seg_L;
    rs.fetch(a, lane_val(sg.q_start, s), seg_L, lane_val(sg.prefix, s), lane_val(sg.mask_off, s),
             rbase, hw, lane);
    vis.hi = lane_val(sg.hi, s);
    vis.masked_from = lane_val(sg.prefix, s);
    vis.t_min = rbase / a.group;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      acc.m[rt] = kNegInf;
      acc.l[rt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc.o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };


  // The first segment's rows are requested now, in flight together with a
  // chunk's page ids.
  if (computes && nst_all > 0) start_segment(seg_of(0));
  if (a.slices == 0) fill_window(win, a, w0, 0, wcount);
  lds_barrier();  // page window written; the first segment's query rows stay in flight
  if (nst_all == 0) return;

  // ---- DMA issue of global stage g into ring buffer `buf`. Every wave runs
  // this (a window move needs all of them); the DMA waves issue the loads.
  const bool dma = DW == kSWaves || wave >= kSWaves - DW;
  const int dw = DW == kSWaves ? wave : wave - (kSWaves - DW);
  const bool uniform_pages = (1 << shift) >= G::KPI;
  int wbase = 0;  // window index held in win[0]
  auto issue = [&](int g, int buf) {
    const int s = seg_of(g);
    const int lo = lane_val(sg.lo, s), last = lane_val(sg.hi, s) - 1;
    const int woff = lane_val(sg.woff, s);
    const int n0 = lo + (g - (lane_val(sg.incl, s) - lane_val(sg.nst, s))) * SK;
    if (woff + (min(n0 + SK - 1, last) >> shift) - wbase >= kStreamPageWindow) {
      // Long work item: move the window (drains the ring; once per window).
      wait_vmcnt<0>();
      __syncthreads();
      wbase = woff + (min(n0, last) >> shift);
      fill_window(win, a, w0, wbase, wcount);
      __syncthreads();
    }
    if (dma)
      issue_stage<KV, D, DW, SK, HP>(a, win, wbase - woff, min(wcount - 1 - wbase, kStreamPageWindow - 1), h,
                             n0, last, smem + buf * G::STAGE, dw, lane, uniform_pages);
  };

  // ---- start-up: NS - 1 stages (a short item repeats its last stage, so
  // every DMA wave always issues the same number of loads here). The first
  // segment's rows are older than every stage: waiting for all but the
  // stages' loads leaves only the ring in flight.
  for (int g = 0; g < NS - 1; ++g) issue(min(g, nst_all - 1), g);
  if constexpr (DW == kSWaves) {
    wait_vmcnt<(NS - 1) * G::NPW>();
  } else {
    if (computes) wait_vmcnt<0>();
  }
  if (computes) rs.finish(seg_L, a.has_mask, lane);

  // ---- the ring. Iteration g: DMA waves wait for their stage-g loads; the
  // barrier (everyone's have landed and every wave is done with stage g - 1);
  // the buffer of stage g - 1 is refilled with stage g + NS - 1; the
  // computing waves take stage g (with P = 2 each wave of a pair takes half
  // of its keys).
  for (int g = 0; g < nst_all; ++g) {
    if (dma) wait_stage<G::NPW, NS>(min(NS - 2, nst_all - 1 - g));
    __builtin_amdgcn_s_barrier();
    const int s = seg_of(g);
    const int first = lane_val(sg.incl, s) - lane_val(sg.nst, s);
    if (computes && g == first && g > 0) {
      // A later segment: its rows are loaded here (before this iteration's
      // DMA when the wave issues any) and waited for.
      start_segment(s);
      wait_vmcnt<0>();
      rs.finish(seg_L, a.has_mask, lane);
    }
    if (g + NS - 1 < nst_all) issue(g + NS - 1, (g + NS - 1) % NS);
    if (computes && has_rows) {
      const int n0 = lane_val(sg.lo, s) + (g - first) * SK;
      const unsigned char* stage = smem + (g % NS) * G::STAGE;
      // 128-key bf16 D = 128 stages are taken in two 64-key passes (the
      // registers of one pass's scores); the second is skipped when the
      // segment ends in the first. There one wave owns each tile set, so the
      // first key tile of each pass is a constant and its addresses fold
      // into immediates.
      constexpr bool kTwoPass = KV == KV_BF16 && D == 128 && SK == 128;
      static_assert(!kTwoPass || P == 1, "two-pass stages take one wave per tile set");
      using LAY = HeadLayout<KV, D, SK, HP>;
      const LAY lay{(hw - h) * (G::HROW / 16)};
      if constexpr (kTwoPass) {
        constexpr int KTW = SK / 16 / P / 2;
        constexpr bool VT = DW == kSWaves && RT == 1;  // one tile: V^T addresses per key tile
        compute_stage<KV, D, RT, KTW, SK, ROPE, LAY, VT>(acc, rs.qf, rs.qlo, rs.row_t, rs.row_bits, vis,
                                                          stage, n0, a.c_log2, lane, 0, lay);
        if (n0 + SK / 2 < vis.hi)
          compute_stage<KV, D, RT, KTW, SK, ROPE, LAY, VT>(acc, rs.qf, rs.qlo, rs.row_t, rs.row_bits,
                                                            vis, stage, n0, a.c_log2, lane, KTW, lay);
      } else {
        compute_stage<KV, D, RT, SK / 16 / P, SK, ROPE, LAY, DW == kSWaves && RT == 1 && P == 1>(
            acc, rs.qf, rs.qlo, rs.row_t, rs.row_bits, vis, stage, n0, a.c_log2, lane, phase * (SK / 16 / P),
            lay);
      }
    }
    if (g == lane_val(sg.incl, s) - 1) {
      // The segment's last stage (every wave sees it).
      float lrow[RT];
      if constexpr (P == 2) {
        if (computes && has_rows && phase == 1) store_pair_state<D, RT>(acc, pair_slot, lane);
        lds_barrier();  // not __syncthreads: the DMA waves keep their stages in flight
        if (computes && has_rows && phase == 0) merge_pair_state<D, RT>(acc, lrow, pair_slot, true, lane);
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) lrow[rt] = rowsum4_v(acc.l[rt]);
      }
      if (computes && has_rows && phase == 0)
        write_rows<D, RT, KV == KV_BF16 && D == 128 && SK == 128 && RT == 2>(
            acc, lrow, a, lane_val(sg.q_start, s), seg_L, rbase, lane_val(sg.whole, s) != 0,
            lane_val(sg.slot, s), lane_val(sg.rb, s), row0, hw, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// `rt`: 16-row tiles per computing wave (1 or 2); `dma_waves`: 2 or 4 (the
// last waves issue the loads, the first ones compute) or 8 (all issue); `pair`: 2 waves
// per row tile set (each takes half of every stage's keys) or 1. Stages hold
// 32 KB (64 bf16 keys of D = 128, else 128 keys); four of them fill the
// 128 KB the planner gives the ring -- except the planner's two-pass plans
// for bf16 D = 128 (two row tiles per wave, or RoPE with eight issuing waves
// and several row blocks; `two_pass`), whose ring holds two 64 KB stages of
// 128 keys.
template <int KV, int D, int NS, int SK>
static const void* stream_variant(int rt, int dma_waves, int pair, bool rows, bool rope, bool two_pass) {
  if (rope && rows) {
    // RoPE with full byte-row masks: one row tile per wave.
    if (dma_waves == kSWaves) return (const void*)vat_stream<KV, D, 1, NS, kSWaves, 1, SK, true, true>;
    if (dma_waves == 2) return (const void*)vat_stream<KV, D, 1, NS, 2, 1, SK, true, true>;
    return pair == 2 ? (const void*)vat_stream<KV, D, 1, NS, 4, 2, SK, true, true>
                     : (const void*)vat_stream<KV, D, 1, NS, 4, 1, SK, true, true>;
  }
  if (rope) {
    // Queries rotated by RoPE at the row fetch: one row tile per wave.
    if (dma_waves == kSWaves) {
      // Several row blocks (the planner's two-pass stages): two 64 KB
      // stages of 128 keys.
      if constexpr (KV == KV_BF16 && D == 128)
        if (two_pass) return (const void*)vat_stream<KV, D, 1, 2, kSWaves, 1, 2 * SK, false, true>;
      return (const void*)vat_stream<KV, D, 1, NS, kSWaves, 1, SK, false, true>;
    }
    if (dma_waves == 2) return (const void*)vat_stream<KV, D, 1, NS, 2, 1, SK, false, true>;
    return pair == 2 ? (const void*)vat_stream<KV, D, 1, NS, 4, 2, SK, false, true>
                     : (const void*)vat_stream<KV, D, 1, NS, 4, 1, SK, false, true>;
  }
  if (rows) {
    // Full byte-row masks: one row tile per wave (the planner's choice).
    if (dma_waves == kSWaves) return (const void*)vat_stream<KV, D, 1, NS, kSWaves, 1, SK, true, false>;
    if (dma_waves == 2) return (const void*)vat_stream<KV, D, 1, NS, 2, 1, SK, true, false>;
    return pair == 2 ? (const void*)vat_stream<KV, D, 1, NS, 4, 2, SK, true, false>
                     : (const void*)vat_stream<KV, D, 1, NS, 4, 1, SK, true, false>;
  }
  if constexpr (KV != KV_E4M3)
    if (rt == 2) {
      // bf16 D = 128: two 64 KB stages of 128 keys (the planner makes every
      // two-tile plan of this shape two-pass).
      if constexpr (D == 128) return (const void*)vat_stream<KV, D, 2, 2, kSWaves, 1, 2 * SK, false, false>;
      else return (const void*)vat_stream<KV, D, 2, NS, kSWaves, 1, SK, false, false>;
    }
  if (dma_waves == kSWaves) return (const void*)vat_stream<KV, D, 1, NS, kSWaves, 1, SK, false, false>;
  if (dma_waves == 2) return (const void*)vat_stream<KV, D, 1, NS, 2, 1, SK, false, false>;
  return pair == 2 ? (const void*)vat_stream<KV, D, 1, NS, 4, 2, SK, false, false>
                   : (const void*)vat_stream<KV, D, 1, NS, 4, 1, SK, false, false>;
}

const void* stream_kernel(int kv_dtype, int head_dim, int rt, int dma_waves, int pair,
                          int mask_mode, int rope, int heads_per_group, int stages) {
  // Two fp8 heads of D 128 per workgroup: 256-byte key rows, 64-key stages,
  // one row tile per computing wave, four DMA waves.
  if (heads_per_group == 2)
    return rope ? (const void*)vat_stream<KV_E4M3, 128, 1, 4, 4, 1, 64, false, true, 2>
                : (const void*)vat_stream<KV_E4M3, 128, 1, 4, 4, 1, 64, false, false, 2>;
  // Four fp8 heads of D 128: 512-byte key rows, 32-key stages, one computing
  // wave per head holding all of its row tiles (so each key and value is
  // decoded once per head), four DMA waves.
  if (heads_per_group == 4)
    return rt == 2 ? (const void*)vat_stream<KV_E4M3, 128, 2, 4, 4, 1, 32, false, false, 4>
                   : (const void*)vat_stream<KV_E4M3, 128, 1, 4, 4, 1, 32, false, false, 4>;
  static_assert(stream_stage_keys(KV_BF16, 128) == 64 && stream_stage_keys(KV_BF16, 64) == 128 &&
                    stream_stage_keys(KV_E4M3, 128) == 128 && stream_two_pass(KV_BF16, 128, 2, 8, 0, 0, 1),
                "stage sizes match the planner");
  const bool rows = mask_mode == 2, ro = rope != 0;
  if (kv_dtype == KV_BF16)
    return head_dim == 128 ? stream_variant<KV_BF16, 128, 4, 64>(rt, dma_waves, pair, rows, ro, stages == 2)
                           : stream_variant<KV_BF16, 64, 4, 128>(rt, dma_waves, pair, rows, ro, false);
  // The planner keeps fp8 at one row tile per wave.
  return stream_variant<KV_E4M3, 128, 4, 128>(1, dma_waves, pair, rows, ro, false);
}

}  // namespace vat
