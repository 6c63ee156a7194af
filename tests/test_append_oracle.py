"""Pins of the CPU oracle for the draft key/value write (quantise on write).

Each check compares the oracle with something that does not come from it:
torch's own casts and float32 division, codes worked out by hand from the
OCP e4m3fn and bfloat16 definitions, round trips through the oracle's
independent decoders, and the page-table placement written out per case.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import (
    append_kv,
    decode_bf16,
    decode_e4m3fn,
    gather_request_kv,
    quantise,
    round_to_bf16,
    round_to_e4m3fn_sat,
    source_values,
)
from workloads import make_append_inputs, make_case, make_config


def torch_e4m3_sat(y: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_bf16(y: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def all_bf16_as_f32() -> np.ndarray:
    return (np.arange(65536, dtype=np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------ e4m3fn


@pytest.mark.parametrize("scale", [1.0, 0.0123, 3.75, 2.0 ** -5])
def test_e4m3_equals_torch_clamped_cast_on_every_bf16_value(scale):
    """Every bfloat16 value (NaNs, infinities, subnormals included) divided by
    the scale: the oracle's code equals torch's float8_e4m3fn cast of the
    float32 quotient clamped to +-448."""
    x = all_bf16_as_f32()
    s = np.float32(scale)
    with np.errstate(all="ignore"):
        y = (torch.from_numpy(x) / torch.tensor(s)).numpy()
    got = quantise(x, float(s), "e4m3")
    want = torch_e4m3_sat(y)
    np.testing.assert_array_equal(got, want)


def test_e4m3_equals_torch_on_random_f32_bits():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    np.testing.assert_array_equal(round_to_e4m3fn_sat(x), torch_e4m3_sat(x))


def test_e4m3_ties_between_neighbours_go_to_even_codes():
    """The exact midpoint of two neighbouring e4m3fn values rounds to the one
    with the even code (checked against torch, and against the even rule)."""
    mags = decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (mags[:-1] + mags[1:]) / 2)  # exact in fp32
    got = round_to_e4m3fn_sat(mids)
    np.testing.assert_array_equal(got, torch_e4m3_sat(mids))
    lower = np.arange(0x7E, dtype=np.uint8)
    expect = np.where(lower % 2 == 0, lower, lower + 1).astype(np.uint8)
    np.testing.assert_array_equal(got, expect)
    np.testing.assert_array_equal(round_to_e4m3fn_sat(-mids), expect | 0x80)


# (value, code) worked by hand: e4m3fn = sign, 4 exponent bits (bias 7),
# 3 significand bits; exponent 0 holds m * 2**-9; 448 = 1.75 * 2**8 is the
# largest finite value; S.1111.111 is NaN.
HAND_E4M3 = [
    (0.0, 0x00), (-0.0, 0x80), (1.0, 0x38), (-1.0, 0xB8),
    (1.0625, 0x38),            # halfway between 1.0 (0x38) and 1.125 (0x39): even
    (1.1875, 0x3A),            # halfway between 1.125 (0x39) and 1.25 (0x3A): even
    (0.1, 0x1D),               # 1.6 * 2**-4 -> significand 4.8/8 -> 5: 1.625 * 2**-4
    (240.0, 0x77),             # 1.875 * 2**7
    (448.0, 0x7E), (464.0, 0x7E), (1.0e6, 0x7E), (-1.0e6, 0xFE),
    (float("inf"), 0x7E), (float("-inf"), 0xFE),
    (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (-(2.0 ** -10), 0x80),
    (3 * 2.0 ** -10, 0x02),    # 1.5 * 2**-9: halfway between codes 1 and 2
    (15 * 2.0 ** -10, 0x08),   # 7.5 * 2**-9: halfway to the smallest normal 2**-6
    (2.0 ** -6, 0x08), (7 * 2.0 ** -9, 0x07),
    (float("nan"), 0x7F),
]


@pytest.mark.parametrize("value,code", HAND_E4M3)
def test_e4m3_hand_worked_codes(value, code):
    assert int(quantise(np.array([value], dtype=np.float32), 1.0, "e4m3")[0]) == code


def test_e4m3_negative_nan_keeps_its_sign():
    neg_nan = np.array([0xFFC00000, 0xFF800001], dtype=np.uint32).view(np.float32)
    np.testing.assert_array_equal(quantise(neg_nan, 1.0, "e4m3"), [0xFF, 0xFF])


def test_e4m3_round_trip_of_every_code():
    """Writing back the decoded value of any finite code (scale 1) gives the
    code itself."""
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = decode_e4m3fn(codes).astype(np.float32)
    vals[codes == 0x80] = np.float32(-0.0)
    np.testing.assert_array_equal(quantise(vals, 1.0, "e4m3"), codes)


# ------------------------------------------------------------------ bfloat16


def test_bf16_equals_torch_cast_on_random_f32_bits():
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 1 << 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    finite_or_inf = ~np.isnan(x)
    np.testing.assert_array_equal(round_to_bf16(x)[finite_or_inf], torch_bf16(x)[finite_or_inf])


def test_bf16_ties_and_edges_against_torch():
    """Inputs exactly halfway between two bfloat16 values (low 16 bits 0x8000)
    for both parities of the lower neighbour, one unit either side of them,
    the largest finite float32 (rounds to infinity) and the infinities."""
    rng = np.random.default_rng(13)
    hi = rng.integers(0, 0x7F80, size=20_000).astype(np.uint32)
    sign = (rng.integers(0, 2, size=20_000).astype(np.uint32) << np.uint32(31))
    base = sign | (hi << np.uint32(16))
    cases = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001,
                            np.array([0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000,
                                      0x7F7F8000, 0x00008000, 0x80018000],
                                     dtype=np.uint32)])
    x = cases.view(np.float32)
    np.testing.assert_array_equal(round_to_bf16(x), torch_bf16(x))


HAND_BF16 = [
    (0x3F808000, 0x3F80),  # 1 + 2**-8: halfway between 1.0 (even) and 1 + 2**-7
    (0x3F818000, 0x3F82),  # halfway between 0x3F81 (odd) and 0x3F82
    (0x3F808001, 0x3F81),  # just above halfway
    (0x7F7FFFFF, 0x7F80),  # largest float32 -> infinity
    (0x00000001, 0x0000),  # smallest subnormal -> +0
    (0x80000001, 0x8000),  # -smallest subnormal -> -0
    (0x7FC00001, 0x7FC0),  # NaN -> canonical quiet NaN
    (0xFF800001, 0xFFC0),  # negative signalling NaN -> canonical, sign kept
]


@pytest.mark.parametrize("bits,code", HAND_BF16)
def test_bf16_hand_worked_codes(bits, code):
    x = np.array([bits], dtype=np.uint32).view(np.float32)
    assert int(quantise(x, 1.0, "bf16")[0]) == code


def test_bf16_round_trip_of_every_code():
    codes = np.arange(65536, dtype=np.uint32)
    x = (codes << np.uint32(16)).view(np.float32)
    keep = ~np.isnan(x)
    np.testing.assert_array_equal(quantise(x, 1.0, "bf16")[keep], codes[keep].astype(np.uint16))


# ------------------------------------------------------------------ division, fp32


def test_f32_store_is_torch_float32_division():
    rng = np.random.default_rng(14)
    x = (rng.standard_normal(200_000) * 10.0 ** rng.integers(-30, 30, 200_000)).astype(np.float32)
    for s in (0.37, 1.0 / 3.0, 1e-20, 7.0e19):
        s32 = np.float32(s)
        with np.errstate(all="ignore"):
            want = (torch.from_numpy(x) / torch.tensor(s32)).numpy()
        np.testing.assert_array_equal(quantise(x, float(s32), "f32").view(np.uint32),
                                      want.view(np.uint32))


def test_power_of_two_scale_is_an_exact_shift():
    """x / 2**k is exact, so the fp32 store is x * 2**-k and an e4m3 store of
    x * 2**k with scale 2**k equals the store of x with scale 1."""
    rng = np.random.default_rng(15)
    x = rng.standard_normal(50_000).astype(np.float32)
    np.testing.assert_array_equal(quantise(x, 8.0, "f32"), x * np.float32(0.125))
    np.testing.assert_array_equal(quantise(x * np.float32(8.0), 8.0, "e4m3"),
                                  quantise(x, 1.0, "e4m3"))


def test_nan_store_keeps_the_input_sign_for_every_cache_dtype():
    x = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFA00000], dtype=np.uint32).view(np.float32)
    np.testing.assert_array_equal(quantise(x, 0.5, "f32").view(np.uint32),
                                  [0x7FC00000, 0xFFC00000, 0x7FC00000, 0xFFC00000])
    np.testing.assert_array_equal(quantise(x, 0.5, "bf16"), [0x7FC0, 0xFFC0, 0x7FC0, 0xFFC0])
    np.testing.assert_array_equal(quantise(x, 0.5, "e4m3"), [0x7F, 0xFF, 0x7F, 0xFF])


@pytest.mark.parametrize("bad", [0.0, -1.0, float("inf"), float("nan")])
def test_bad_scales_are_refused(bad):
    with pytest.raises(ValueError):
        quantise(np.ones(4, dtype=np.float32), bad, "e4m3")


# ------------------------------------------------------------------ placement


def test_append_places_tokens_by_hand():
    """Two requests, page size 4. Request 0: pages [5, 2], kv_len 6, L 3 ->
    tokens at keys 3, 4, 5 = (page 5, slot 3), (page 2, slot 0), (page 2, slot
    1). Request 1: pages [0], kv_len 2, L 2 -> (page 0, slots 0 and 1).
    Every other cache byte stays as it was."""
    num_pages, ps, hkv, d = 6, 4, 2, 8
    rng = np.random.default_rng(16)
    k_cache = rng.integers(0, 256, size=(num_pages, ps, hkv, d), dtype=np.uint8)
    v_cache = rng.integers(0, 256, size=(num_pages, ps, hkv, d), dtype=np.uint8)
    kv_indptr = np.array([0, 2, 3], dtype=np.int32)
    kv_indices = np.array([5, 2, 0], dtype=np.int32)
    last_page_len = np.array([2, 2], dtype=np.int32)
    qo_indptr = np.array([0, 3, 5], dtype=np.int32)
    # Token r, head h, element e holds r + 1 + h / 4 + e / 64 and V its
    # negative; the values themselves go through quantise (pinned above),
    # what this checks is where they land.
    k_new = np.zeros((5, hkv, d), dtype=np.float32)
    for r in range(5):
        for h in range(hkv):
            k_new[r, h] = r + 1 + h / 4.0 + np.arange(d) / 64.0
    v_new = -k_new
    k_out, v_out = append_kv(k_new, v_new, "f32", k_cache, v_cache, "e4m3", kv_indptr,
                             kv_indices, last_page_len, qo_indptr, ps, k_scale=0.5, v_scale=2.0)
    places = {0: (5, 3), 1: (2, 0), 2: (2, 1), 3: (0, 0), 4: (0, 1)}
    k_want = k_cache.copy()
    v_want = v_cache.copy()
    for r, (page, slot) in places.items():
        k_want[page, slot] = quantise(k_new[r], 0.5, "e4m3")
        v_want[page, slot] = quantise(v_new[r], 2.0, "e4m3")
    np.testing.assert_array_equal(k_out, k_want)
    np.testing.assert_array_equal(v_out, v_want)
    # Inputs are not modified.
    assert not np.array_equal(k_out, k_cache)


@pytest.mark.parametrize("cache_dtype,src_dtype", [("bf16", "bf16"), ("e4m3", "bf16"),
                                                   ("f32", "f32"), ("e4m3", "f32")])
def test_append_then_gather_reads_back_the_drafts(cache_dtype, src_dtype):
    """Paged = contiguous: after the write, the last L_b keys of each request
    gathered through the page table are the quantised drafts, in order; the
    prefix keys are unchanged. Includes a request whose drafts straddle a page
    boundary, one with no drafts and one made only of drafts."""
    p = make_case(21, prefix_lens=[13, 0, 30, 7], qo_lens=[5, 3, 0, 9], num_qo_heads=4,
                  num_kv_heads=2, head_dim=64, page_size=4,
                  q_dtype="f32" if cache_dtype == "f32" else "bf16", kv_dtype=cache_dtype)
    k_new, v_new = make_append_inputs(p, src_dtype, seed=5, spread=3.0)
    k_out, v_out = append_kv(k_new, v_new, src_dtype, p.k_cache, p.v_cache, cache_dtype,
                             p.kv_indptr, p.kv_indices, p.last_page_len, p.qo_indptr,
                             p.page_size, k_scale=0.25, v_scale=0.75)
    kx, vx = source_values(k_new, src_dtype), source_values(v_new, src_dtype)
    for b in range(p.batch):
        start = int(p.kv_indptr[b])
        L = int(p.qo_indptr[b + 1] - p.qo_indptr[b])
        kv_len = p.info["kv_lens"][b]
        prefix = kv_len - L
        for cache, out, new, s in ((p.k_cache, k_out, kx, 0.25), (p.v_cache, v_out, vx, 0.75)):
            before = gather_request_kv(cache, p.kv_indices, start, kv_len, p.page_size)
            after = gather_request_kv(out, p.kv_indices, start, kv_len, p.page_size)
            np.testing.assert_array_equal(after[:prefix], before[:prefix])
            r0 = int(p.qo_indptr[b])
            for t in range(L):
                np.testing.assert_array_equal(after[prefix + t],
                                              quantise(new[r0 + t], s, cache_dtype))


def test_append_of_the_generators_own_values_reproduces_its_cache():
    """The generator stores a bf16 cache as torch's RNE cast of its float32
    draws. Writing the decoded draft rows back (scale 1) leaves every byte of
    the cache as it was."""
    p = make_config(2)
    T = int(p.qo_indptr[-1])
    k_new = np.zeros((T, p.num_kv_heads, p.head_dim), dtype=np.uint16)
    v_new = np.zeros_like(k_new)
    for b in range(p.batch):
        start = int(p.kv_indptr[b])
        kv_len = p.info["kv_lens"][b]
        L = int(p.qo_indptr[b + 1] - p.qo_indptr[b])
        k_rows = gather_request_kv(p.k_cache, p.kv_indices, start, kv_len, p.page_size)
        v_rows = gather_request_kv(p.v_cache, p.kv_indices, start, kv_len, p.page_size)
        r0 = int(p.qo_indptr[b])
        k_new[r0:r0 + L] = k_rows[kv_len - L:]
        v_new[r0:r0 + L] = v_rows[kv_len - L:]
    k_out, v_out = append_kv(k_new, v_new, "bf16", p.k_cache, p.v_cache, "bf16", p.kv_indptr,
                             p.kv_indices, p.last_page_len, p.qo_indptr, p.page_size)
    np.testing.assert_array_equal(k_out, p.k_cache)
    np.testing.assert_array_equal(v_out, p.v_cache)


def test_all_bf16_patterns_generator_covers_each_pattern_once():
    p = make_case(3, prefix_lens=[3, 9], qo_lens=[32, 32], num_qo_heads=4, num_kv_heads=4,
                  head_dim=128, page_size=16)
    k, v = make_append_inputs(p, "bf16", seed=0, special="all_bf16")
    pats = np.concatenate([k.reshape(-1), v.reshape(-1)])
    np.testing.assert_array_equal(np.sort(pats), np.arange(65536, dtype=np.uint16))
    vals = decode_bf16(pats)
    assert int(np.isnan(vals).sum()) == 2 * 127  # exponent all ones, significand != 0
