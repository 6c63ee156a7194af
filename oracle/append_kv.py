"""Plain definition of appending the draft tokens' keys and values to a paged cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

What is computed. Before verification attention runs, the keys and values of
the L_b draft tokens of request b are written into the request's paged cache
(the vLLM page "[WIP] Support for cached multi-query attention towards
speculative decoding" caches every draft's key and value first, then
attends). They become the last L_b entries of the request, so token t of
request b (row ``qo_indptr[b] + t`` of the new-key array) goes to key
position ``n = kv_len_b - L_b + t``: page ``kv_indices[kv_indptr[b] + n //
page_size]``, slot ``n % page_size`` (paged format of the FlashInfer page
"feat: Separate Q and KV dtypes for decode", ``begin_forward`` docstring).

What is stored. The attention reads a stored key as ``k_scale * K_stored``
and a stored value as ``v_scale * V_stored`` (flashmap page
"sglang/verify_attention.py": ``k_scale`` multiplies the logits, ``v_scale``
the accumulated output), so writing a real key ``x`` stores the cache-dtype
number nearest to ``x / k_scale``:

* the quotient is the IEEE binary32 quotient of the binary32 input and the
  binary32 scale (one correctly rounded division);
* fp32 caches store it as is;
* bf16 caches store the nearest bfloat16, ties to the even significand
  (IEEE round-to-nearest-even; beyond the largest finite bfloat16 this
  reaches infinity, as IEEE overflow does);
* e4m3fn caches first clamp the quotient to [-448, 448] (the format has no
  infinity; 448 is its largest finite value) and then store the nearest
  e4m3fn value, ties to the even code; the sign of zero is kept.

A NaN input stores the canonical quiet NaN of the cache dtype with the
input's sign: fp32 ``0x7FC00000``, bf16 ``0x7FC0``, e4m3fn ``0x7F`` (the
format's only NaN codes are ``S.1111.111``).

Everything else in the cache is left untouched.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .verify_attention import E4M3FN_TABLE, request_lengths

_SIGN32 = np.uint32(0x80000000)

# Magnitudes of the non-negative finite e4m3fn codes 0x00 .. 0x7E, ascending
# (the code order is the magnitude order within one sign).
_E4M3_MAGS = E4M3FN_TABLE[:0x7F]


def _f32_bits(y: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(y, dtype=np.float32).view(np.uint32)


def round_to_f32(y: np.ndarray) -> np.ndarray:
    """Binary32 values -> stored fp32 bit patterns (uint32); NaN canonical."""
    bits = _f32_bits(y).copy()
    nan = np.isnan(np.asarray(y, dtype=np.float32))
    bits[nan] = np.uint32(0x7FC00000) | (bits[nan] & _SIGN32)
    return bits


def round_to_bf16(y: np.ndarray) -> np.ndarray:
    """Binary32 values -> nearest bfloat16 bit patterns (uint16), ties to even.

    The bfloat16 numbers are the binary32 numbers whose low 16 bits are zero.
    For each input the two candidates are the one just below in magnitude
    (low bits cleared) and the next one up (one bfloat16 unit further from
    zero; past the largest finite value that is infinity, which IEEE rounding
    treats as the next step, 2**128). The distances are compared exactly in
    float64.
    """
    y = np.ascontiguousarray(y, dtype=np.float32)
    bits = y.view(np.uint32)
    sign = bits & _SIGN32
    mag_bits = bits & np.uint32(0x7FFFFFFF)
    lo = mag_bits & np.uint32(0xFFFF0000)
    hi = lo + np.uint32(0x10000)
    with np.errstate(invalid="ignore"):  # NaN lanes are overwritten below
        lo_val = lo.view(np.float32).astype(np.float64)
        hi_val = np.where(hi >= np.uint32(0x7F800000), 2.0 ** 128,
                          hi.view(np.float32).astype(np.float64))
        a = mag_bits.view(np.float32).astype(np.float64)
        d_lo = a - lo_val
        d_hi = hi_val - a
    lo_even = ((lo >> np.uint32(16)) & np.uint32(1)) == 0
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    out = np.where(take_hi, hi, lo)
    out = np.where(mag_bits >= np.uint32(0x7F800000), mag_bits & np.uint32(0xFFFF0000), out)
    code = ((sign | out) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(y)
    code[nan] = np.uint16(0x7FC0) | (sign[nan] >> np.uint32(16)).astype(np.uint16)
    return code


def round_to_e4m3fn_sat(y: np.ndarray) -> np.ndarray:
    """Binary32 values -> nearest e4m3fn codes (uint8) after clamping to +-448.

    Ties go to the even code (an even code has an even significand, both for
    normal and subnormal values). The sign bit is the input's sign, also when
    the magnitude rounds to zero.
    """
    y = np.ascontiguousarray(y, dtype=np.float32)
    sign = ((y.view(np.uint32) >> np.uint32(24)) & np.uint32(0x80)).astype(np.uint8)
    a = np.minimum(np.abs(y.astype(np.float64)), 448.0)
    nan = np.isnan(y)
    a[nan] = 0.0
    # Index of the first magnitude >= a; the nearest code is that one or the
    # one just below.
    up = np.searchsorted(_E4M3_MAGS, a, side="left")
    up = np.minimum(up, len(_E4M3_MAGS) - 1)
    down = np.maximum(up - 1, 0)
    d_up = _E4M3_MAGS[up] - a
    d_down = a - _E4M3_MAGS[down]
    take_up = (d_up < d_down) | ((d_up == d_down) & (up % 2 == 0))
    code = np.where(take_up, up, down).astype(np.uint8)
    code |= sign
    code[nan] = np.uint8(0x7F) | sign[nan]
    return code


def quantise(x: np.ndarray, scale: float, cache_dtype: str) -> np.ndarray:
    """Real binary32 values ``x`` -> stored cache patterns of ``x / scale``."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    s = np.float32(scale)
    if not (np.isfinite(s) and s > 0):
        raise ValueError("scale must be finite and > 0")
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        y = x / s
    # A NaN keeps the sign of the input, whatever the division did to it.
    y_bits = y.view(np.uint32).copy()
    nan = np.isnan(x)
    y_bits[nan] = np.uint32(0x7FC00000) | (x.view(np.uint32)[nan] & _SIGN32)
    y = y_bits.view(np.float32)
    if cache_dtype == "f32":
        return round_to_f32(y).view(np.float32)
    if cache_dtype == "bf16":
        return round_to_bf16(y)
    if cache_dtype == "e4m3":
        return round_to_e4m3fn_sat(y)
    raise ValueError(cache_dtype)


def source_values(raw: np.ndarray, src_dtype: str) -> np.ndarray:
    """New keys/values in their source dtype ("f32" or "bf16") -> binary32."""
    if src_dtype == "f32":
        return np.asarray(raw, dtype=np.float32)
    if src_dtype == "bf16":
        # bfloat16 is the high half of a binary32: widen by a shift (exact,
        # NaN payload and sign kept).
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32)
    raise ValueError(src_dtype)


def append_kv(k_new, v_new, src_dtype: str, k_cache, v_cache, cache_dtype: str,
              kv_indptr, kv_indices, last_page_len, qo_indptr, page_size: int,
              k_scale: float = 1.0, v_scale: float = 1.0,
              k_cos_sin: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Caches after writing each request's draft keys/values; inputs unchanged.

    ``k_new``/``v_new``: ``[T, Hkv, D]`` raw arrays in ``src_dtype``, rows in the
    packed ``qo_indptr`` order; caches ``[pages, page_size, Hkv, D]`` raw arrays
    in ``cache_dtype``. ``k_cos_sin [T, D]``: rotate key row t by RoPE in
    binary32 (``oracle.rope.rotate_f32``) before it is scaled and rounded;
    values are written as given.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    kx = source_values(k_new, src_dtype)
    vx = source_values(v_new, src_dtype)
    if k_cos_sin is not None:
        from .rope import rotate_f32

        kx = rotate_f32(kx, np.asarray(k_cos_sin, dtype=np.float32)[:, None, :])
    num_pages = k_out.shape[0]
    for b in range(len(qo_indptr) - 1):
        pages, kv_len, L, prefix = request_lengths(kv_indptr, last_page_len, qo_indptr,
                                                   page_size, b)
        row0 = int(qo_indptr[b])
        start = int(kv_indptr[b])
        for t in range(L):
            n = prefix + t
            page = int(kv_indices[start + n // page_size])
            if not 0 <= page < num_pages:
                raise ValueError("page id out of range")
            slot = n % page_size
            k_out[page, slot] = quantise(kx[row0 + t], k_scale, cache_dtype)
            v_out[page, slot] = quantise(vx[row0 + t], v_scale, cache_dtype)
    return k_out, v_out
