"""Seeded input recipes for paged-KV verification attention.

Everything here is drawn on the CPU with ``torch.Generator().manual_seed(seed)``
in one fixed order -- lengths, page-pool permutation, draft-tree parents, Q, K,
V -- and returned as raw storage arrays (float32 values, bfloat16 bit patterns
as uint16, OCP e4m3fn codes as uint8), which is exactly what both the GPU
library and the oracle read.

The layouts follow the paged format of the FlashInfer page "feat: Separate Q
and KV dtypes for decode" (``begin_forward`` docstring): ``kv_indptr`` counts
pages per request, ``kv_indices`` lists page ids, ``last_page_len`` is the
number of filled slots in each request's last page. Query tokens are packed
varlen by ``qo_indptr`` as in the vLLM page "[Performance] Support MQA/GQA in
prefill stage by using FlashAttention" (``BlockDiagonalCausalMask.from_seqlens``).
The draft tokens' own K/V already sit in the cache as each request's last
``L_b`` positions (vLLM page "[WIP] Support for cached multi-query attention
towards speculative decoding": all draft keys and values are cached first).

Bit-packed tree masks: request b's ``L_b x L_b`` block, row-major flat index
``i = t * L_b + j``, bit ``i % 8`` (least significant first) of byte
``mask_indptr[b] + i // 8``; 1 = token t may attend to draft j. The pages only
show byte masks (flashmap page ``sglang/verify_attention.py``,
``_verify_partial_kernel``, the ``USE_MASK`` branch); this packing is the
build's own layout. The same blocks can also be laid out as sglang's
full-row byte masks (``mask_layout="rows"``: per request ``L_b`` rows of
``prefix_b + L_b`` bytes, one per key, nonzero = allowed, the prefix bytes
set as sglang writes them), the layout the flashmap page's kernel reads.
"""

from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

DTYPES_Q = ("f32", "bf16")
DTYPES_KV = ("f32", "bf16", "e4m3")
ELEM_BYTES = {"f32": 4, "bf16": 2, "e4m3": 1}
E4M3_MAX = 448.0
NAN_F32 = np.float32("nan")
NAN_BF16 = np.uint16(0x7FC0)
NAN_E4M3 = np.uint8(0x7F)

CONFIG_NAMES = {
    1: "tiny MQA verify fp32 (B2 Hq4 Hkv1 D64, prefix 37/100, L4 causal)",
    2: "GQA chain verify bf16 (B8 Hq32 Hkv8 D128, prefix 2048, L5 causal)",
    3: "tree verify bf16 at batch 1 (Hq32 Hkv8 D128, L17 tree, prefix {p})",
    4: "GQA causal prefill bf16 (B10x1024, Hq64 Hkv8 D128)",
    5: "mixed-dtype dynamic-draft verify (B64 Hq32 Hkv8 D128, bf16 Q, e4m3 KV, prefix U[512,8192], L U{{1..8}})",
    6: "GQA decode bf16 (B64 Hq32 Hkv8 D128, prefix U[512,8192], L1)",
    7: "wide tree verify bf16 (B4 Hq64 Hkv8 D128, L64 tree, prefix 8192: 512 rows per KV head)",
}


@dataclass
class Problem:
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    last_page_len: np.ndarray
    qo_indptr: np.ndarray
    mask: Optional[np.ndarray]
    mask_indptr: Optional[np.ndarray]
    sm_scale: float
    k_scale: float
    v_scale: float
    q_dtype: str
    kv_dtype: str
    max_qo_len: int
    page_size: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    name: str = ""
    seed: int = 0
    info: dict = field(default_factory=dict)
    mask_layout: str = "bits"  # "bits": packed L x L blocks; "rows": full byte rows

    @property
    def batch(self) -> int:
        return int(self.kv_indptr.shape[0]) - 1

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])


# ---------------------------------------------------------------- draft trees


def chain_parents(length: int) -> np.ndarray:
    """A draft chain: node i's parent is i - 1 (root 0 has none)."""
    return np.arange(-1, length - 1, dtype=np.int64)


def random_tree_parents(length: int, gen: torch.Generator) -> np.ndarray:
    """Root 0 plus ``length - 1`` nodes; node i's parent uniform in {0..i-1}."""
    parents = np.full(length, -1, dtype=np.int64)
    for i in range(1, length):
        parents[i] = int(torch.randint(0, i, (1,), generator=gen).item())
    return parents


def tree_mask_rows(parents: Sequence[int]) -> np.ndarray:
    """Ancestor-or-self relation of a tree given by parent links: ``[L, L]`` bool."""
    n = len(parents)
    rows = np.zeros((n, n), dtype=bool)
    for t in range(n):
        node = t
        while node >= 0:
            rows[t, node] = True
            node = int(parents[node])
    return rows


def pack_mask_rows(blocks: Sequence[np.ndarray], pad_bytes: int = 0):
    """Pack per-request ``[L_b, L_b]`` bool blocks into bytes + ``mask_indptr``.

    Row-major, least-significant bit first, each request's segment starting on
    a byte boundary; ``pad_bytes`` extra zero bytes follow every segment.
    """
    segments = []
    indptr = [0]
    for blk in blocks:
        blk = np.asarray(blk, dtype=bool)
        flat = blk.reshape(-1)
        nbytes = (flat.size + 7) // 8
        seg = np.zeros(nbytes + pad_bytes, dtype=np.uint8)
        for i, bit in enumerate(flat):
            if bit:
                seg[i // 8] |= np.uint8(1 << (i % 8))
        segments.append(seg)
        indptr.append(indptr[-1] + seg.size)
    data = np.concatenate(segments) if segments else np.zeros(0, dtype=np.uint8)
    if data.size == 0:
        data = np.zeros(1, dtype=np.uint8)
    return data, np.asarray(indptr, dtype=np.int32)


def pack_mask_full_rows(blocks: Sequence[np.ndarray], prefixes: Sequence[int],
                        prefix_fill="ones", true_values="ones", pad_bytes: int = 0,
                        gen: Optional[torch.Generator] = None):
    """Lay per-request ``[L_b, L_b]`` bool blocks out as full byte rows.

    Request b's segment holds ``L_b`` rows of ``prefix_b + L_b`` bytes, row t
    at byte ``t * (prefix_b + L_b)`` of the segment. The draft columns hold the
    block (``true_values`` "ones": allowed = 1; "random": a random nonzero
    byte); the prefix columns hold ``prefix_fill``: "ones" (all visible, as
    sglang writes them), "zeros" or "random" bytes. ``pad_bytes`` zero bytes
    follow every segment.
    """
    g = gen if gen is not None else torch.Generator().manual_seed(0)
    segments = []
    indptr = [0]
    for blk, prefix in zip(blocks, prefixes):
        blk = np.asarray(blk, dtype=bool)
        L = blk.shape[0]
        width = int(prefix) + L
        seg = np.zeros(L * width + pad_bytes, dtype=np.uint8)
        rows = seg[:L * width].reshape(L, width) if L else seg[:0].reshape(0, width)
        if prefix_fill == "ones":
            rows[:, :prefix] = 1
        elif prefix_fill == "random":
            rows[:, :prefix] = torch.randint(0, 256, (L, int(prefix)), generator=g).numpy()
        elif prefix_fill != "zeros":
            raise ValueError(prefix_fill)
        if true_values == "ones":
            vals = np.ones((L, L), dtype=np.uint8)
        elif true_values == "random":
            vals = torch.randint(1, 256, (L, L), generator=g).numpy().astype(np.uint8)
        else:
            raise ValueError(true_values)
        rows[:, prefix:] = np.where(blk, vals, 0)
        segments.append(seg)
        indptr.append(indptr[-1] + seg.size)
    data = np.concatenate(segments) if segments else np.zeros(0, dtype=np.uint8)
    if data.size == 0:
        data = np.zeros(1, dtype=np.uint8)
    return data, np.asarray(indptr, dtype=np.int32)


# ---------------------------------------------------------------- storage casts


def _to_storage(x: torch.Tensor, dtype: str) -> np.ndarray:
    """Float32 tensor -> raw storage array in ``dtype`` (RNE casts by torch)."""
    if dtype == "f32":
        return x.to(torch.float32).numpy().copy()
    if dtype == "bf16":
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if dtype == "e4m3":
        x = x.clamp(-E4M3_MAX, E4M3_MAX)
        return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    raise ValueError(dtype)


def _nan_code(dtype: str):
    return {"f32": NAN_F32, "bf16": NAN_BF16, "e4m3": NAN_E4M3}[dtype]


def poison_unused(cache: np.ndarray, dtype: str, kv_indptr, kv_indices, last_page_len) -> None:
    """NaN-fill every slot no request owns: spare pages and last-page tails."""
    used = np.zeros(cache.shape[0], dtype=bool)
    nan = _nan_code(dtype)
    for b in range(len(last_page_len)):
        pages = kv_indices[kv_indptr[b]:kv_indptr[b + 1]]
        used[pages] = True
        if len(pages):
            cache[pages[-1], int(last_page_len[b]):] = nan
    cache[~used] = nan


# ---------------------------------------------------------------- generic case


def make_case(
    seed: int,
    *,
    prefix_lens: Sequence[int],
    qo_lens: Sequence[int],
    num_qo_heads: int,
    num_kv_heads: int,
    head_dim: int,
    page_size: int = 16,
    q_dtype: str = "bf16",
    kv_dtype: str = "bf16",
    mask_kind: str = "causal",
    parents: Optional[Sequence[Sequence[int]]] = None,
    mask_density: float = 0.5,
    mask_pad_bytes: int = 0,
    pool_pages: Optional[int] = None,
    extra_indices: int = 0,
    sm_scale: Optional[float] = None,
    k_scale: float = 1.0,
    v_scale: float = 1.0,
    fp8_absmax_scales: bool = False,
    max_qo_len: Optional[int] = None,
    poison: bool = True,
    name: str = "",
    gen: Optional[torch.Generator] = None,
    mask_layout: str = "bits",
    rows_prefix_fill: str = "ones",
    rows_true_values: str = "ones",
) -> Problem:
    """Build one seeded problem.

    ``mask_kind``: "causal" (no mask array), "chain" (packed chain mask, equal
    to causal), "tree" (random tree per request unless ``parents`` is given,
    ancestor-or-self), "random" (independent bits with ``mask_density``; rows
    may be fully masked), "full" (every bit set). ``mask_layout`` "bits"
    packs the blocks; "rows" lays them out as full byte rows
    (``pack_mask_full_rows`` with ``rows_prefix_fill`` / ``rows_true_values``),
    drawn after every other input so the rest of the problem is the same.
    """
    if q_dtype not in DTYPES_Q or kv_dtype not in DTYPES_KV:
        raise ValueError((q_dtype, kv_dtype))
    if num_qo_heads % num_kv_heads:
        raise ValueError("Hq must be a multiple of Hkv")
    g = gen if gen is not None else torch.Generator().manual_seed(int(seed))
    batch = len(prefix_lens)
    assert len(qo_lens) == batch
    prefix_lens = [int(x) for x in prefix_lens]
    qo_lens = [int(x) for x in qo_lens]
    kv_lens = [p + l for p, l in zip(prefix_lens, qo_lens)]
    pages_per = [0 if n == 0 else (n + page_size - 1) // page_size for n in kv_lens]
    last_page_len = np.asarray(
        [0 if n == 0 else n - (pg - 1) * page_size for n, pg in zip(kv_lens, pages_per)],
        dtype=np.int32,
    )
    needed = int(sum(pages_per))
    if pool_pages is None:
        pool_pages = needed + max(8, (needed + 7) // 8)
    assert pool_pages >= needed
    perm = torch.randperm(pool_pages, generator=g).numpy().astype(np.int32)
    kv_indptr = np.zeros(batch + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(pages_per)
    kv_indices = np.full(needed + extra_indices, np.int32(0x7FFFFFFF), dtype=np.int32)
    kv_indices[:needed] = perm[:needed]
    qo_indptr = np.zeros(batch + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_lens)

    mask = mask_indptr = None
    tree_parents = None
    if mask_kind != "causal":
        blocks = []
        tree_parents = []
        for b in range(batch):
            L = qo_lens[b]
            if mask_kind == "chain":
                par = chain_parents(L)
                tree_parents.append(par)
                blocks.append(tree_mask_rows(par))
            elif mask_kind == "tree":
                par = (np.asarray(parents[b], dtype=np.int64) if parents is not None
                       else random_tree_parents(L, g))
                tree_parents.append(par)
                blocks.append(tree_mask_rows(par))
            elif mask_kind == "random":
                bits = torch.rand((L, L), generator=g).numpy() < mask_density
                blocks.append(bits)
            elif mask_kind == "full":
                blocks.append(np.ones((L, L), dtype=bool))
            else:
                raise ValueError(mask_kind)
        if mask_layout == "bits":
            mask, mask_indptr = pack_mask_rows(blocks, pad_bytes=mask_pad_bytes)
        elif mask_layout != "rows":
            raise ValueError(mask_layout)

    T = int(qo_indptr[-1])
    q32 = torch.randn((T, num_qo_heads, head_dim), generator=g, dtype=torch.float32)
    shape = (pool_pages, page_size, num_kv_heads, head_dim)
    k32 = torch.randn(shape, generator=g, dtype=torch.float32)
    v32 = torch.randn(shape, generator=g, dtype=torch.float32)

    if fp8_absmax_scales:
        assert kv_dtype == "e4m3"
        used = torch.from_numpy(kv_indices[:needed].astype(np.int64))
        kmax = float(k32[used].abs().max()) if needed else 1.0
        vmax = float(v32[used].abs().max()) if needed else 1.0
        k_scale = float(np.float32(kmax / E4M3_MAX))
        v_scale = float(np.float32(vmax / E4M3_MAX))
        k32 = k32 / k_scale
        v32 = v32 / v_scale

    q = _to_storage(q32, q_dtype)
    k_cache = _to_storage(k32, kv_dtype)
    v_cache = _to_storage(v32, kv_dtype)
    del q32, k32, v32
    if poison:
        poison_unused(k_cache, kv_dtype, kv_indptr, kv_indices, last_page_len)
        poison_unused(v_cache, kv_dtype, kv_indptr, kv_indices, last_page_len)
    if mask_kind != "causal" and mask_layout == "rows":
        mask, mask_indptr = pack_mask_full_rows(blocks, prefix_lens, rows_prefix_fill,
                                                rows_true_values, mask_pad_bytes, g)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    if max_qo_len is None:
        max_qo_len = max(qo_lens) if qo_lens else 0
    return Problem(
        q=q, k_cache=k_cache, v_cache=v_cache,
        kv_indptr=kv_indptr, kv_indices=kv_indices, last_page_len=last_page_len,
        qo_indptr=qo_indptr, mask=mask, mask_indptr=mask_indptr,
        sm_scale=float(np.float32(sm_scale)), k_scale=float(np.float32(k_scale)),
        v_scale=float(np.float32(v_scale)),
        q_dtype=q_dtype, kv_dtype=kv_dtype, max_qo_len=int(max_qo_len),
        page_size=page_size, num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, name=name, seed=int(seed),
        info={"prefix_lens": prefix_lens, "qo_lens": qo_lens, "kv_lens": kv_lens,
              "parents": tree_parents, "mask_kind": mask_kind},
        mask_layout=mask_layout if mask is not None else "bits",
    )


# ---------------------------------------------------------------- the five workloads


def make_config(cid: int, seed: Optional[int] = None, prefix: int = 4096, **overrides) -> Problem:
    """The five seeded workloads (default seed = config number).

    1: tiny MQA verify, fp32, B 2, Hq 4, Hkv 1, D 64, prefix 37/100, L 4
       causal, page 16 in a permuted 32-page pool, sm_scale 1/8.
    2: GQA chain verify, bf16, B 8, Hq 32, Hkv 8, D 128, prefix 2048, L 5 causal.
    3: tree verify at batch 1, bf16, Hq 32, Hkv 8, D 128, L 17 (root + 16
       nodes, parent uniform among earlier nodes), ancestor-or-self mask,
       ``prefix`` in {4096, 16384, 32768}.
    4: GQA causal prefill, bf16, 10 packed sequences of 1024 tokens, Hq 64,
       Hkv 8, D 128, prefix 0, K/V in the paged cache.
    5: bf16 Q with e4m3fn K/V (per-tensor absmax/448 scales), B 64, Hq 32,
       Hkv 8, D 128, prefix U[512, 8192], L U{1..8} causal, max_qo_len 8.
    6: pure decode, bf16, B 64, Hq 32, Hkv 8, D 128, prefix U[512, 8192]
       (config 5's length mix), one query token per request.
    7: wide trees, bf16, B 4, Hq 64, Hkv 8, D 128, L 64 (random tree,
       ancestor-or-self mask), prefix 8192: G L = 512 query rows per
       (request, KV head), more than one row block.
    """
    seed = cid if seed is None else seed
    if cid == 1:
        kw = dict(prefix_lens=[37, 100], qo_lens=[4, 4], num_qo_heads=4, num_kv_heads=1,
                  head_dim=64, q_dtype="f32", kv_dtype="f32", pool_pages=32,
                  sm_scale=1.0 / 8.0)
    elif cid == 2:
        kw = dict(prefix_lens=[2048] * 8, qo_lens=[5] * 8, num_qo_heads=32, num_kv_heads=8,
                  head_dim=128)
    elif cid == 3:
        kw = dict(prefix_lens=[int(prefix)], qo_lens=[17], num_qo_heads=32, num_kv_heads=8,
                  head_dim=128, mask_kind="tree")
    elif cid == 4:
        kw = dict(prefix_lens=[0] * 10, qo_lens=[1024] * 10, num_qo_heads=64,
                  num_kv_heads=8, head_dim=128)
    elif cid == 5:
        g = torch.Generator().manual_seed(int(seed))
        prefixes = torch.randint(512, 8193, (64,), generator=g).tolist()
        lens = torch.randint(1, 9, (64,), generator=g).tolist()
        kw = dict(prefix_lens=prefixes, qo_lens=lens, num_qo_heads=32, num_kv_heads=8,
                  head_dim=128, q_dtype="bf16", kv_dtype="e4m3", fp8_absmax_scales=True,
                  max_qo_len=8, gen=g)
    elif cid == 6:
        g = torch.Generator().manual_seed(int(seed))
        prefixes = torch.randint(512, 8193, (64,), generator=g).tolist()
        kw = dict(prefix_lens=prefixes, qo_lens=[1] * 64, num_qo_heads=32, num_kv_heads=8,
                  head_dim=128, gen=g)
    elif cid == 7:
        kw = dict(prefix_lens=[8192] * 4, qo_lens=[64] * 4, num_qo_heads=64, num_kv_heads=8,
                  head_dim=128, mask_kind="tree")
    else:
        raise ValueError(cid)
    kw.update(overrides)
    name = CONFIG_NAMES[cid].format(p=prefix)
    return make_case(seed, name=name, **kw)


# ---------------------------------------------------------------- bookkeeping


def problem_sha256(p: Problem) -> str:
    h = hashlib.sha256()
    for arr in (p.q, p.k_cache, p.v_cache, p.kv_indptr, p.kv_indices, p.last_page_len,
                p.qo_indptr):
        h.update(np.ascontiguousarray(arr).tobytes())
    if p.mask is not None:
        h.update(p.mask.tobytes())
        h.update(p.mask_indptr.tobytes())
    h.update(np.asarray([p.sm_scale, p.k_scale, p.v_scale], dtype=np.float64).tobytes())
    return h.hexdigest()


def kv_bytes(p: Problem) -> int:
    """Algorithmic KV bytes: every cached entry of every request, K and V, once per KV head."""
    kv_lens = np.zeros(p.batch, dtype=np.int64)
    for b in range(p.batch):
        pages = int(p.kv_indptr[b + 1] - p.kv_indptr[b])
        kv_lens[b] = 0 if pages == 0 else (pages - 1) * p.page_size + int(p.last_page_len[b])
    return int(kv_lens.sum()) * p.num_kv_heads * p.head_dim * 2 * ELEM_BYTES[p.kv_dtype]


# ---------------------------------------------------------------- new draft keys/values


def make_append_inputs(p: Problem, src_dtype: str, seed: int, spread: float = 1.0,
                       special: str = "none"):
    """New keys and values ``[T, Hkv, D]`` for the drafts of ``p`` in ``src_dtype``.

    ``spread`` scales N(0,1) draws (values beyond the cache's range exercise
    saturation). ``special`` replaces the draws with bit patterns:
    "all_bf16" cycles through all 65536 bfloat16 patterns (K takes the first
    half of the cycle, V the second); "f32_bits" draws uniform random 32-bit
    patterns (every class: NaN, infinities, subnormals, zeros).
    """
    g = torch.Generator().manual_seed(int(seed))
    T = int(p.qo_indptr[-1])
    shape = (T, p.num_kv_heads, p.head_dim)
    n = T * p.num_kv_heads * p.head_dim
    if special == "all_bf16":
        if src_dtype != "bf16":
            raise ValueError("all_bf16 needs a bf16 source")
        pats = np.arange(2 * n, dtype=np.int64) % 65536
        k = pats[:n].astype(np.uint16).reshape(shape)
        v = pats[n:].astype(np.uint16).reshape(shape)
        return k, v
    if special == "f32_bits":
        if src_dtype != "f32":
            raise ValueError("f32_bits needs an f32 source")
        bits = torch.randint(0, 1 << 32, (2, n), generator=g, dtype=torch.int64).numpy()
        bits = bits.astype(np.uint32)
        return bits[0].view(np.float32).reshape(shape), bits[1].view(np.float32).reshape(shape)
    if special != "none":
        raise ValueError(special)
    k32 = torch.randn(shape, generator=g, dtype=torch.float32) * float(spread)
    v32 = torch.randn(shape, generator=g, dtype=torch.float32) * float(spread)
    if src_dtype == "f32":
        return k32.numpy().copy(), v32.numpy().copy()
    if src_dtype == "bf16":
        return (k32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy(),
                v32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy())
    raise ValueError(src_dtype)


# ---------------------------------------------------------------- rotary positions


def tree_depths(parents: Sequence[int]) -> np.ndarray:
    """Depth of each node of a draft tree (root 0), parents before children."""
    d = np.zeros(len(parents), dtype=np.int64)
    for i in range(1, len(parents)):
        d[i] = d[int(parents[i])] + 1
    return d


def rope_positions(p: Problem) -> np.ndarray:
    """Position of every query/draft token row: ``prefix_b`` plus its depth in
    the request's tree (a chain, a random mask or no mask: its index t)."""
    pos = np.zeros(p.num_tokens, dtype=np.int64)
    parents = p.info.get("parents")
    for b in range(p.batch):
        r0, r1 = int(p.qo_indptr[b]), int(p.qo_indptr[b + 1])
        L = r1 - r0
        prefix = p.info["kv_lens"][b] - L
        if parents is not None and b < len(parents) and len(parents[b]) == L:
            pos[r0:r1] = prefix + tree_depths(parents[b])
        else:
            pos[r0:r1] = prefix + np.arange(L)
    return pos


def rope_cos_sin(positions, head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """``[len(positions), D]`` float32 rows ``(cos th_0.., sin th_0..)`` with
    ``th_i = position * theta ** (-2 i / D)`` (LLaMA-style RoPE), evaluated in
    float64 and rounded once."""
    pos = np.asarray(positions, dtype=np.float64)[:, None]
    inv = theta ** (-2.0 * np.arange(head_dim // 2, dtype=np.float64) / head_dim)
    th = pos * inv[None, :]
    return np.concatenate([np.cos(th), np.sin(th)], axis=1).astype(np.float32)
