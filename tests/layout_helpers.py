"""Test-side construction of paged problems from logical per-request tensors.

The oracle reads keys through the page table (a gather); these helpers go the
other way: they start from each request's logical key/value rows and scatter
them into a page pool under a chosen page size and page permutation. A
mistake in either direction makes the oracle disagree with a library
reference evaluated on the logical tensors.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np
import torch

from workloads.gen import Problem, pack_mask_rows


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Float values rounded to bfloat16 (as float64)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(
        torch.float64).numpy()


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "e4m3":
        return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(
            torch.uint8).numpy()
    raise ValueError(dtype)


def nan_code(dtype: str):
    return {"f32": np.float32("nan"), "bf16": np.uint16(0x7FC0), "e4m3": np.uint8(0x7F)}[dtype]


def scatter_problem(q_log: Sequence[np.ndarray], k_log: Sequence[np.ndarray],
                    v_log: Sequence[np.ndarray], *, page_size: int, q_dtype: str, kv_dtype: str,
                    mask_blocks: Optional[Sequence[np.ndarray]] = None, sm_scale: float = 1.0,
                    k_scale: float = 1.0, v_scale: float = 1.0, perm_seed: Optional[int] = 0,
                    spare_pages: int = 3, poison: bool = True, mask_pad_bytes: int = 0) -> Problem:
    """Lay out logical tensors as a paged problem.

    q_log[b]: ``[L_b, Hq, D]``; k_log[b], v_log[b]: ``[kv_len_b, Hkv, D]``
    (already representable in ``kv_dtype``). Pages are filled in key order,
    ``page_size`` keys each; physical page ids follow a seeded permutation of
    the pool (identity if ``perm_seed`` is None).
    """
    B = len(q_log)
    Hq, D = q_log[0].shape[1], q_log[0].shape[2]
    Hkv = k_log[0].shape[1]
    pages_per = [(k.shape[0] + page_size - 1) // page_size for k in k_log]
    needed = sum(pages_per)
    pool = needed + spare_pages
    if perm_seed is None:
        perm = np.arange(pool)
    else:
        perm = np.random.default_rng(perm_seed).permutation(pool)
    kc = np.full((pool, page_size, Hkv, D), nan_code(kv_dtype) if poison else 0,
                 dtype=store(np.zeros(1), kv_dtype).dtype)
    vc = kc.copy()
    indices = []
    last = []
    cursor = 0
    for b in range(B):
        n = k_log[b].shape[0]
        ks = store(k_log[b], kv_dtype)
        vs = store(v_log[b], kv_dtype)
        for p in range(pages_per[b]):
            phys = int(perm[cursor])
            cursor += 1
            indices.append(phys)
            lo, hi = p * page_size, min(n, (p + 1) * page_size)
            kc[phys, : hi - lo] = ks[lo:hi]
            vc[phys, : hi - lo] = vs[lo:hi]
        last.append(n - (pages_per[b] - 1) * page_size if pages_per[b] else 0)
    kv_indptr = np.concatenate([[0], np.cumsum(pages_per)]).astype(np.int32)
    qo_lens = [x.shape[0] for x in q_log]
    qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int32)
    q = store(np.concatenate(q_log, axis=0), q_dtype)
    mask = mask_indptr = None
    if mask_blocks is not None:
        mask, mask_indptr = pack_mask_rows(mask_blocks, pad_bytes=mask_pad_bytes)
    return Problem(q=q, k_cache=kc, v_cache=vc, kv_indptr=kv_indptr,
                   kv_indices=np.asarray(indices, dtype=np.int32),
                   last_page_len=np.asarray(last, dtype=np.int32), qo_indptr=qo_indptr,
                   mask=mask, mask_indptr=mask_indptr, sm_scale=sm_scale, k_scale=k_scale,
                   v_scale=v_scale, q_dtype=q_dtype, kv_dtype=kv_dtype,
                   max_qo_len=max(qo_lens) if qo_lens else 0, page_size=page_size,
                   num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D)


def random_logical(rng: np.random.Generator, prefixes: Sequence[int], lens: Sequence[int],
                   Hq: int, Hkv: int, D: int, kv_dtype: str = "f32", q_dtype: str = "f32"):
    """Random logical q/k/v per request, rounded to be representable in the dtypes."""
    def rep(x, dt):
        if dt == "f32":
            return x.astype(np.float32).astype(np.float64)
        if dt == "bf16":
            return bf16_round(x)
        if dt == "e4m3":
            t = torch.from_numpy(x.astype(np.float32)).clamp(-448, 448)
            return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()
        raise ValueError(dt)

    q_log, k_log, v_log = [], [], []
    for p, L in zip(prefixes, lens):
        q_log.append(rep(rng.standard_normal((L, Hq, D)), q_dtype))
        k_log.append(rep(rng.standard_normal((p + L, Hkv, D)), kv_dtype))
        v_log.append(rep(rng.standard_normal((p + L, Hkv, D)), kv_dtype))
    return q_log, k_log, v_log


def run_oracle(p: Problem, **kw):
    from oracle import verify_attention

    return verify_attention(p.q, p.k_cache, p.v_cache, p.kv_indptr, p.kv_indices,
                            p.last_page_len, p.qo_indptr, p.mask, p.mask_indptr,
                            sm_scale=p.sm_scale, k_scale=p.k_scale, v_scale=p.v_scale,
                            q_dtype=p.q_dtype, kv_dtype=p.kv_dtype,
                            mask_layout=p.mask_layout, **kw)


def sdpa_reference(q_log, k_log, v_log, allowed_blocks, *, scale: float, v_scale: float = 1.0):
    """Library reference: torch SDPA (float64, CPU) + torch.logsumexp per request.

    ``allowed_blocks[b]``: ``[L_b, kv_len_b]`` bool. GQA by repeating each KV
    head over its group of consecutive query heads. Rows with no visible key
    are returned as NaN (SDPA's own result there) for the caller to skip.
    """
    outs, lses = [], []
    for q, k, v, allowed in zip(q_log, k_log, v_log, allowed_blocks):
        Hq, Hkv = q.shape[1], k.shape[1]
        G = Hq // Hkv
        qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2))).to(torch.float64)
        kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).to(torch.float64)
        vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).to(torch.float64)
        kt = kt.repeat_interleave(G, dim=0)
        vt = vt.repeat_interleave(G, dim=0) * v_scale
        am = torch.from_numpy(np.asarray(allowed, dtype=bool))
        o = torch.nn.functional.scaled_dot_product_attention(
            qt.unsqueeze(0), kt.unsqueeze(0), vt.unsqueeze(0), attn_mask=am, scale=scale)[0]
        logits = torch.matmul(qt, kt.transpose(1, 2).contiguous()) * scale
        logits = logits.masked_fill(~am, float("-inf"))
        l = torch.logsumexp(logits, dim=-1)
        outs.append(o.permute(1, 0, 2).numpy())
        lses.append(l.permute(1, 0).numpy())
    return outs, lses


def causal_allowed(prefix: int, L: int) -> np.ndarray:
    """Bottom-right causal visibility, built from per-token sequence lengths.

    Token t sees the first ``prefix + t + 1`` keys: the single-query decode
    view of the vLLM page "[WIP] Support for cached multi-query attention
    towards speculative decoding" (seq_len raised by one per draft).
    """
    allowed = np.zeros((L, prefix + L), dtype=bool)
    for t in range(L):
        allowed[t, : prefix + t + 1] = True
    return allowed
