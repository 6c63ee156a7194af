"""Plain, slow, float64 definition of verification attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

What is computed (the plain definition; the GPU method reaches the same value
up to rounding order):

For request b with ``L_b`` query (draft) tokens and ``kv_len_b`` cached keys,
query token t of query head ``hq`` attends to every key n of KV head
``hq // G`` (G = Hq / Hkv) that it is allowed to see:

* keys before the drafts (``n < prefix_b = kv_len_b - L_b``) are always
  visible -- the prefix is fully visible (flashmap page
  "sglang/verify_attention.py", module docstring and the prefix branch of
  ``_verify_partial_kernel``);
* draft key ``j = n - prefix_b`` is visible iff ``j <= t`` without a mask
  (causal, bottom-right aligned: the vLLM page "[WIP] Support for cached
  multi-query attention towards speculative decoding" raises each draft's
  sequence length from the context length by one per draft), or iff bit
  ``(t, j)`` of the request's packed mask is set (FlashInfer page "How to
  implement a tree attention with flashinfer": a tree mask replaces the
  causal one);

and gets ``out = sum_n softmax_n(s) * V[n]`` with
``s_n = sm_scale * k_scale * <q, K_stored[n]>``, ``V[n] = v_scale *
V_stored[n]`` (flashmap page, ``k_scale``/``v_scale`` folding in
``_verify_partial_kernel``), and ``lse = ln sum_n exp(s_n)``. A row with no
visible key returns ``out = 0``, ``lse = -inf`` (the flashmap merge kernel
divides by a zero denominator guard and its lse is ``-inf`` when the sum is 0).

Keys are gathered through the page table of the FlashInfer page "feat:
Separate Q and KV dtypes for decode" (``begin_forward`` docstring): request b
owns page ids ``kv_indices[kv_indptr[b]:kv_indptr[b+1]]``; its last page holds
``last_page_len[b]`` entries; key n lives in page ``n // page_size`` of that
list at slot ``n % page_size``. Caches are ``[pages, page_size, Hkv, D]``.
"""

from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

# ------------------------------------------------------------------ decoding


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64.

    bfloat16 is the top half of an IEEE binary32, so the value is the float32
    whose high 16 bits are ``bits`` and whose low 16 bits are zero.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    as32 = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return as32.view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    """One OCP FP8 E4M3 (``fn``: finite, no infinities) code -> its real value.

    Layout: sign bit, 4 exponent bits with bias 7, 3 mantissa bits. Exponent
    field 0 encodes subnormals ``m * 2**-9``; ``S.1111.111`` is NaN; there is no
    infinity, so ``S.1111.110`` = 448 is the largest finite magnitude.
    """
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn codes (uint8) -> exact float64 via the 256-entry table."""
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_storage(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage array in ``dtype`` ("f32", "bf16", "e4m3") -> float64."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(raw)
    if dtype == "e4m3":
        return decode_e4m3fn(raw)
    raise ValueError(dtype)


# ------------------------------------------------------------------ paged layout


def request_lengths(kv_indptr, last_page_len, qo_indptr, page_size: int, b: int):
    """(pages, kv_len, L, prefix) of request b.

    ``kv_len = (pages - 1) * page_size + last_page_len`` (FlashInfer page,
    ``begin_forward`` docstring: ``last_page_len`` counts the entries of the
    last page); a request without pages has ``kv_len = 0``. ``L`` is the
    request's number of query tokens in the packed ``qo_indptr`` layout and
    ``prefix = kv_len - L`` because the drafts' own K/V are the last ``L``
    cache entries.
    """
    pages = int(kv_indptr[b + 1]) - int(kv_indptr[b])
    if pages < 0:
        raise ValueError("kv_indptr must be non-decreasing")
    if pages == 0:
        kv_len = 0
    else:
        lp = int(last_page_len[b])
        if not 1 <= lp <= page_size:
            raise ValueError("last_page_len out of [1, page_size]")
        kv_len = (pages - 1) * page_size + lp
    L = int(qo_indptr[b + 1]) - int(qo_indptr[b])
    if L < 0 or L > kv_len:
        raise ValueError("need 0 <= L_b <= kv_len_b")
    return pages, kv_len, L, kv_len - L


def gather_request_kv(cache: np.ndarray, kv_indices, start: int, kv_len: int,
                      page_size: int) -> np.ndarray:
    """Key/value rows ``[kv_len, Hkv, D]`` of one request, in key order.

    Key n is slot ``n % page_size`` of page ``kv_indices[start + n // page_size]``.
    """
    num_pages = cache.shape[0]
    rows = []
    for n in range(kv_len):
        page = int(kv_indices[start + n // page_size])
        if not 0 <= page < num_pages:
            raise ValueError("page id out of range")
        rows.append(cache[page, n % page_size])
    if not rows:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.stack(rows, axis=0)


def unpack_mask_block(mask: np.ndarray, offset: int, L: int) -> np.ndarray:
    """Request's ``[L, L]`` bool block from the bit-packed mask.

    Entry (t, j) is bit ``i % 8`` (least significant first) of byte
    ``offset + i // 8`` with ``i = t * L + j``; 1 means allowed.
    """
    block = np.zeros((L, L), dtype=bool)
    for t in range(L):
        for j in range(L):
            i = t * L + j
            byte = int(mask[offset + i // 8])
            block[t, j] = (byte >> (i % 8)) & 1 == 1
    return block


def unpack_mask_rows(mask: np.ndarray, offset: int, prefix: int, L: int) -> np.ndarray:
    """Request's ``[L, L]`` bool draft block from sglang's full-row byte mask.

    In that layout (flashmap page "sglang/verify_attention.py": module
    docstring and the non-``QLEN_MASK`` branch of ``_verify_partial_kernel``)
    request b's mask starts at byte ``offset = mask_indptr[b]`` and holds one
    row of ``prefix + L`` bytes per query token, one byte per key, nonzero =
    allowed. The prefix is all visible, so only the last ``L`` bytes of each
    row are read: entry (t, j) is byte ``offset + t * (prefix + L) + prefix +
    j``.
    """
    block = np.zeros((L, L), dtype=bool)
    for t in range(L):
        for j in range(L):
            block[t, j] = int(mask[offset + t * (prefix + L) + prefix + j]) != 0
    return block


def mask_block_of(mask, mask_indptr, layout: str, b: int, prefix: int, L: int):
    """The draft block of request b under ``layout`` ("bits" or "rows"), or
    None without a mask (causal)."""
    if mask is None:
        return None
    if layout == "bits":
        return unpack_mask_block(mask, int(mask_indptr[b]), L)
    if layout == "rows":
        return unpack_mask_rows(mask, int(mask_indptr[b]), prefix, L)
    raise ValueError(layout)


def allowed_keys(L: int, prefix: int, kv_len: int, mask_block: Optional[np.ndarray]) -> np.ndarray:
    """``[L, kv_len]`` bool: which keys each of the request's query tokens sees."""
    allowed = np.zeros((L, kv_len), dtype=bool)
    for t in range(L):
        allowed[t, :prefix] = True
        for j in range(L):
            if mask_block is None:
                ok = j <= t
            else:
                ok = bool(mask_block[t, j])
            allowed[t, prefix + j] = ok
    return allowed


# ------------------------------------------------------------------ attention


def attend_rows(q_rows: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                allowed: np.ndarray, logit_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Masked softmax attention of ``q_rows [R, D]`` over ``k_rows/v_rows [N, D]``.

    ``allowed [R, N]`` selects the visible keys. Returns ``out [R, Dv]`` and the
    natural-log ``lse [R]`` of the scaled logits; a row with no visible key
    gives ``out = 0`` and ``lse = -inf``. Everything in float64.
    """
    R = q_rows.shape[0]
    out = np.zeros((R, v_rows.shape[1]), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    for r in range(R):
        vis = np.nonzero(allowed[r])[0]
        if vis.size == 0:
            continue
        s = logit_scale * (k_rows[vis] @ q_rows[r])
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        out[r] = (e @ v_rows[vis]) / z
        lse[r] = m + math.log(z)
    return out, lse


def _check_shapes(q, k_cache, v_cache, kv_indptr, last_page_len, qo_indptr, num_kv_heads):
    T, Hq, D = q.shape
    if k_cache.shape != v_cache.shape or k_cache.ndim != 4:
        raise ValueError("caches must be [pages, page_size, Hkv, D]")
    if k_cache.shape[2] != num_kv_heads or k_cache.shape[3] != D:
        raise ValueError("cache head shape mismatch")
    if Hq % num_kv_heads:
        raise ValueError("Hq must be a multiple of Hkv")
    B = len(kv_indptr) - 1
    if len(last_page_len) != B or len(qo_indptr) != B + 1:
        raise ValueError("index array lengths")
    if int(qo_indptr[0]) != 0 or int(qo_indptr[B]) != T:
        raise ValueError("qo_indptr must run 0..T")
    return T, Hq, D, B


def verify_attention(q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len, qo_indptr,
                     mask=None, mask_indptr=None, *, sm_scale: float, k_scale: float = 1.0,
                     v_scale: float = 1.0, q_dtype: str, kv_dtype: str,
                     requests: Optional[Sequence[int]] = None, mask_layout: str = "bits",
                     q_cos_sin: Optional[np.ndarray] = None):
    """The whole path on raw storage arrays; returns float64 ``out [T, Hq, D]``, ``lse [T, Hq]``.

    ``mask=None`` means causal over the drafts. Otherwise, with
    ``mask_layout="bits"``, ``mask`` is the bit-packed byte array and
    ``mask_indptr[b]`` the byte offset of request b's ``L_b x L_b`` block;
    with ``"rows"`` it is sglang's full-row byte mask (``unpack_mask_rows``).
    ``q_cos_sin [T, D]``: rotate query row t by RoPE with its cos/sin row
    (``oracle.rope.rotate``, float64) before attending; the cached keys are
    used as stored (a writer that applies RoPE stores rotated keys). ``requests`` limits the work to some requests
    (rows of other requests stay 0 / -inf), for sampled checks at full size.
    Query head ``hq`` reads KV head ``hq // G`` (vLLM page "[Performance]
    Support MQA/GQA in prefill stage by using FlashAttention": K/V expanded
    per group of G consecutive query heads).
    """
    num_kv_heads = k_cache.shape[2]
    T, Hq, D, B = _check_shapes(q, k_cache, v_cache, kv_indptr, last_page_len, qo_indptr,
                                num_kv_heads)
    if mask is not None and mask_indptr is None:
        raise ValueError("a mask needs mask_indptr")
    G = Hq // num_kv_heads
    page_size = k_cache.shape[1]
    qf = decode_storage(q, q_dtype)
    if q_cos_sin is not None:
        from .rope import rotate

        qf = rotate(qf, np.asarray(q_cos_sin)[:, None, :])
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.full((T, Hq), -np.inf, dtype=np.float64)
    logit_scale = float(sm_scale) * float(k_scale)
    todo = range(B) if requests is None else requests
    for b in todo:
        pages, kv_len, L, prefix = request_lengths(kv_indptr, last_page_len, qo_indptr,
                                                   page_size, b)
        if L == 0:
            continue
        start = int(kv_indptr[b])
        k_raw = gather_request_kv(k_cache, kv_indices, start, kv_len, page_size)
        v_raw = gather_request_kv(v_cache, kv_indices, start, kv_len, page_size)
        k_req = decode_storage(k_raw, kv_dtype)
        v_req = decode_storage(v_raw, kv_dtype) * float(v_scale)
        block = mask_block_of(mask, mask_indptr, mask_layout, b, prefix, L)
        allowed = allowed_keys(L, prefix, kv_len, block)
        t0 = int(qo_indptr[b])
        for hq in range(Hq):
            h = hq // G
            o, l = attend_rows(qf[t0:t0 + L, hq, :], k_req[:, h, :], v_req[:, h, :], allowed,
                               logit_scale)
            out[t0:t0 + L, hq, :] = o
            lse[t0:t0 + L, hq] = l
    return out, lse


# ------------------------------------------------------------------ split / merge


def verify_attention_partials(q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                              qo_indptr, mask=None, mask_indptr=None, *, key_splits,
                              sm_scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                              q_dtype: str, kv_dtype: str, mask_layout: str = "bits"):
    """Attention restricted to key ranges: one ``(out, lse)`` pair per range.

    ``key_splits(b, kv_len) -> list of (lo, hi)`` key ranges; each partial is
    the plain definition with keys outside ``[lo, hi)`` hidden (an empty range
    gives 0 / -inf). Used to check that merging partials by their
    log-sum-exp (flashmap page, ``_verify_merge_kernel``) equals the direct
    result.
    """
    num_kv_heads = k_cache.shape[2]
    T, Hq, D, B = _check_shapes(q, k_cache, v_cache, kv_indptr, last_page_len, qo_indptr,
                                num_kv_heads)
    G = Hq // num_kv_heads
    page_size = k_cache.shape[1]
    qf = decode_storage(q, q_dtype)
    logit_scale = float(sm_scale) * float(k_scale)
    results: List[List[Tuple[np.ndarray, np.ndarray]]] = []
    for b in range(B):
        pages, kv_len, L, prefix = request_lengths(kv_indptr, last_page_len, qo_indptr,
                                                   page_size, b)
        start = int(kv_indptr[b])
        k_req = decode_storage(gather_request_kv(k_cache, kv_indices, start, kv_len, page_size),
                               kv_dtype)
        v_req = decode_storage(gather_request_kv(v_cache, kv_indices, start, kv_len, page_size),
                               kv_dtype) * float(v_scale)
        block = mask_block_of(mask, mask_indptr, mask_layout, b, prefix, L)
        allowed = allowed_keys(L, prefix, kv_len, block)
        t0 = int(qo_indptr[b])
        parts = []
        for lo, hi in key_splits(b, kv_len):
            sub = np.zeros_like(allowed)
            sub[:, lo:hi] = allowed[:, lo:hi]
            o = np.zeros((L, Hq, D))
            ls = np.full((L, Hq), -np.inf)
            for hq in range(Hq):
                h = hq // G
                o[:, hq, :], ls[:, hq] = attend_rows(qf[t0:t0 + L, hq, :], k_req[:, h, :],
                                                     v_req[:, h, :], sub, logit_scale)
            parts.append((o, ls))
        results.append(parts)
    return results


def merge_partials(parts: Sequence[Tuple[np.ndarray, np.ndarray]]):
    """Combine partial results over disjoint key sets by their log-sum-exp.

    Each partial carries its normalised output and the lse of its own keys.
    With ``M = max lse`` and weights ``w = exp(lse - M)``, the merged output
    is ``sum w * out / sum w`` and the merged lse ``M + ln sum w``; partials
    with ``lse = -inf`` weigh nothing; if all are ``-inf`` the result is 0 /
    -inf (flashmap page, ``_verify_merge_kernel``).
    """
    outs = np.stack([p[0] for p in parts], axis=0)
    lses = np.stack([p[1] for p in parts], axis=0)
    M = lses.max(axis=0)
    finite = np.isfinite(M)
    base = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - base[None]), 0.0)
    den = w.sum(axis=0)
    num = (w[..., None] * np.where(np.isfinite(lses)[..., None], outs, 0.0)).sum(axis=0)
    out = np.where(den[..., None] > 0, num / np.where(den > 0, den, 1.0)[..., None], 0.0)
    lse = np.where(den > 0, base + np.log(np.where(den > 0, den, 1.0)), -np.inf)
    return out, lse
