"""Plain definition of rotary position embedding (RoPE) at tree positions.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.

What is computed. FlashInfer's attention kernels can apply LLaMA-style
rotary embeddings on the fly (FlashInfer page "feat: Separate Q and KV
dtypes for decode", ``begin_forward`` docstring: ``pos_encoding_mode``
``ROPE_LLAMA``), and a draft tree needs them at each token's own position
rather than at its index, through the cos/sin values of the rotation
(FlashInfer page "How to implement a tree attention with flashinfer": the
RoPE cos/sin matrix and the mask are the two changes trees need). Here the
caller passes, per token row, the cos/sin row of that token's position:
``cos_sin[r] = (cos th_0 .. cos th_{D/2-1}, sin th_0 .. sin th_{D/2-1})``.

LLaMA style pairs dimension ``i`` with ``i + D/2`` (i < D/2):

    x'_i       = x_i * c_i - x_{i+D/2} * s_i
    x'_{i+D/2} = x_{i+D/2} * c_i + x_i * s_i

``rotate`` evaluates this in float64 (the attention oracle). ``rotate_f32``
evaluates it in IEEE binary32 with every product and sum rounded on its own
(no fused multiply-add): that is how the cache write defines the rotated key
it then rounds to the cache dtype, so the stored codes are reproducible; a
NaN it produces is the canonical positive quiet NaN.
The cos/sin rows themselves are inputs (drawn by the input recipe from the
tokens' positions).
"""

from __future__ import annotations

import numpy as np


def _halves(cos_sin: np.ndarray, D: int):
    cs = np.asarray(cos_sin)
    if cs.shape[-1] != D or D % 2:
        raise ValueError("cos_sin rows must have D entries, D even")
    return cs[..., : D // 2], cs[..., D // 2:]


def rotate(x: np.ndarray, cos_sin: np.ndarray) -> np.ndarray:
    """float64 RoPE of ``x [..., D]`` with per-row ``cos_sin [..., D]`` (broadcast
    over any head axis the caller inserts)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    c, s = _halves(np.asarray(cos_sin, dtype=np.float64), D)
    lo, hi = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rotate_f32(x: np.ndarray, cos_sin: np.ndarray) -> np.ndarray:
    """binary32 RoPE, each product and each sum rounded separately."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    c, s = _halves(np.asarray(cos_sin, dtype=np.float32), D)
    lo, hi = x[..., : D // 2], x[..., D // 2:]
    with np.errstate(over="ignore", invalid="ignore"):
        new_lo = (lo * c).astype(np.float32) - (hi * s).astype(np.float32)
        new_hi = (hi * c).astype(np.float32) + (lo * s).astype(np.float32)
    out = np.concatenate([new_lo.astype(np.float32), new_hi.astype(np.float32)], axis=-1)
    # Any NaN result (a NaN input, or infinity times zero) is the canonical
    # positive quiet NaN: the sign of an invalid result is platform-defined.
    bits = out.view(np.uint32)
    bits[np.isnan(out)] = np.uint32(0x7FC00000)
    return out
