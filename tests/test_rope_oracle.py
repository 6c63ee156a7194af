"""Pins of the oracle's rotary position embedding (RoPE) and its use.

Checked against facts that do not come from the oracle: a hand-worked
rotation, the identity at angle zero, length preservation of each rotated
pair, the dependence of rotated dot products on the position difference only
(cos/sin evaluated here from the closed form), torch's own float32
arithmetic for the binary32 form, and, through the attention and cache-write
oracles, invariances that RoPE implies.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import append_kv, gather_request_kv, quantise, rope_rotate, rope_rotate_f32
from oracle import verify_attention as oracle_va
from workloads import make_append_inputs, make_case, rope_cos_sin, rope_positions


def closed_form_rows(positions, D, theta=10000.0):
    th = np.outer(np.asarray(positions, dtype=np.float64),
                  np.power(theta, -np.arange(0, D, 2, dtype=np.float64) / D))
    return np.concatenate([np.cos(th), np.sin(th)], axis=1)


def test_hand_worked_quarter_turn():
    # D = 4: pairs (0, 2) and (1, 3); every angle pi/2 (cos 0, sin 1):
    # x' = (x0*0 - x2, x1*0 - x3, x2*0 + x0, x3*0 + x1) = (-3, -4, 1, 2).
    x = np.array([1.0, 2.0, 3.0, 4.0])
    cs = np.array([0.0, 0.0, 1.0, 1.0])
    assert np.array_equal(rope_rotate(x, cs), [-3.0, -4.0, 1.0, 2.0])
    assert np.array_equal(rope_rotate_f32(x, cs), np.float32([-3.0, -4.0, 1.0, 2.0]))


def test_zero_angle_is_the_identity_bitwise():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 128)).astype(np.float32)
    cs = np.concatenate([np.ones((5, 1, 64)), np.zeros((5, 1, 64))], axis=-1)
    assert np.array_equal(rope_rotate_f32(x, cs), x)
    assert np.array_equal(rope_rotate(x, cs), x.astype(np.float64))


def test_each_pair_keeps_its_length():
    rng = np.random.default_rng(2)
    D = 64
    x = rng.standard_normal((7, D))
    cs = closed_form_rows(rng.integers(0, 100000, 7), D)
    y = rope_rotate(x, cs)
    np.testing.assert_allclose(x[:, :32] ** 2 + x[:, 32:] ** 2, y[:, :32] ** 2 + y[:, 32:] ** 2,
                               rtol=1e-12)


def test_dot_products_depend_on_the_position_difference_only():
    rng = np.random.default_rng(3)
    D = 128
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for pq, pk, shift in [(7, 3, 1000), (4100, 4096, -4000), (0, 9, 123456)]:
        a = rope_rotate(q, closed_form_rows([pq], D)[0]) @ rope_rotate(k, closed_form_rows([pk], D)[0])
        b = (rope_rotate(q, closed_form_rows([pq + shift], D)[0])
             @ rope_rotate(k, closed_form_rows([pk + shift], D)[0]))
        assert abs(a - b) <= 1e-9 * max(1.0, abs(a))


def test_binary32_form_equals_torch_float32_arithmetic():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 8, 128)).astype(np.float32) * 3
    cs = rope_cos_sin(rng.integers(0, 60000, 50), 128)[:, None, :]
    xt, ct = torch.from_numpy(x), torch.from_numpy(np.broadcast_to(cs, (50, 8, 128)).copy())
    lo, hi, c, s = xt[..., :64], xt[..., 64:], ct[..., :64], ct[..., 64:]
    want = torch.cat([lo * c - hi * s, hi * c + lo * s], dim=-1).numpy()
    assert np.array_equal(rope_rotate_f32(x, cs).view(np.uint32), want.view(np.uint32))


def _f32_bits(*vals):
    return np.array(vals, dtype=np.uint32)


def test_binary32_invalid_results_are_the_canonical_positive_quiet_nan():
    # D = 4: pairs (0, 2) and (1, 3). Worked by hand from the rotation
    # x'_i = x_i c - x_{i+2} s, x'_{i+2} = x_{i+2} c + x_i s, every product
    # and sum rounded on its own. An invalid operation (inf * 0, inf - inf)
    # or a NaN operand gives NaN, stored as 0x7FC00000 whatever sign or
    # payload the hardware would carry; finite and infinite lanes keep
    # their exact values.
    inf = np.float32(np.inf)
    nan_neg = _f32_bits(0xFFC00000).view(np.float32)[0]      # negative quiet NaN
    nan_sig = _f32_bits(0x7F800001).view(np.float32)[0]      # signalling NaN, payload 1
    nan_pay = _f32_bits(0xFFC12345).view(np.float32)[0]      # negative NaN with a payload
    qnan = 0x7FC00000
    cases = [
        # pair 0 at a quarter turn (c 0, s 1): inf*0 - 0*1 is NaN, 0*0 + inf*1 = inf;
        # pair 1 at angle zero (c 1, s 0): 1*1 - 2*0 = 1, 2*1 + 1*0 = 2.
        ([inf, 1.0, 0.0, 2.0], [0.0, 1.0, 1.0, 0.0], [qnan, 0x3F800000, 0x7F800000, 0x40000000]),
        # pair 0 at c = s = 1: inf*1 - inf*1 = inf - inf is NaN (x86 makes it
        # the negative "indefinite" NaN); inf*1 + inf*1 = inf. Pair 1: c 1, s 0.
        ([inf, 3.0, inf, -1.0], [1.0, 1.0, 1.0, 0.0], [qnan, 0x40400000, 0x7F800000, 0xBF800000]),
        # NaN operands of either sign and any payload; pair 1's -0 * 1 - 0 * 0 = -0 - 0 = -0.
        ([nan_neg, -0.0, 1.0, 0.0], [1.0, 1.0, 0.0, 0.0], [qnan, 0x80000000, qnan, 0x00000000]),
        # pair 0 at c = s = 1/2: 1*0.5 - 2*0.5 = -0.5, 2*0.5 + 1*0.5 = 1.5.
        ([1.0, nan_sig, 2.0, nan_pay], [0.5, 1.0, 0.5, 0.0], [0xBF000000, qnan, 0x3FC00000, qnan]),
    ]
    for x, cs, want in cases:
        got = rope_rotate_f32(np.array(x, dtype=np.float32), np.array(cs, dtype=np.float32))
        assert got.dtype == np.float32
        assert got.view(np.uint32).tolist() == want, (x, cs, [hex(v) for v in got.view(np.uint32)])


def test_cos_sin_rows_follow_the_closed_form():
    pos = np.array([0, 1, 17, 4096, 65535])
    np.testing.assert_allclose(rope_cos_sin(pos, 128), closed_form_rows(pos, 128), atol=1e-7)


def test_tree_positions_are_prefix_plus_depth():
    p = make_case(5, prefix_lens=[10, 0], qo_lens=[5, 3], num_qo_heads=2, num_kv_heads=1,
                  head_dim=64, mask_kind="tree", parents=[[-1, 0, 0, 1, 3], [-1, 0, 1]])
    assert list(rope_positions(p)) == [10, 11, 11, 12, 13, 0, 1, 2]


def _problem(seed, **kw):
    base = dict(prefix_lens=[9, 30], qo_lens=[4, 6], num_qo_heads=4, num_kv_heads=2, head_dim=64,
                page_size=4, q_dtype="f32", kv_dtype="f32", mask_kind="tree")
    base.update(kw)
    return make_case(seed, **base)


def _run(p, **kw):
    return oracle_va(p.q, p.k_cache, p.v_cache, p.kv_indptr, p.kv_indices, p.last_page_len,
                     p.qo_indptr, p.mask, p.mask_indptr, sm_scale=p.sm_scale, k_scale=p.k_scale,
                     v_scale=p.v_scale, q_dtype=p.q_dtype, kv_dtype=p.kv_dtype, **kw)


def _rotate_cache(p, angle_rows):
    """f32 caches with every stored key rotated by its row of ``angle_rows``
    (indexed by page, slot)."""
    k = rope_rotate(p.k_cache.astype(np.float64), angle_rows[:, :, None, :]).astype(np.float32)
    return k


def test_identity_rotation_leaves_attention_unchanged_bitwise():
    p = _problem(6)
    cs = np.concatenate([np.ones((p.num_tokens, 32)), np.zeros((p.num_tokens, 32))], axis=1)
    o0, l0 = _run(p)
    o1, l1 = _run(p, q_cos_sin=cs)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_one_common_angle_for_queries_and_keys_changes_nothing():
    """RoPE rotates every pair by an orthogonal map: rotating all queries and
    all cached keys by the same angles keeps every score."""
    p = _problem(7)
    cs_tok = closed_form_rows([1234] * p.num_tokens, p.head_dim)
    cs_slot = np.broadcast_to(closed_form_rows([1234], p.head_dim)[0],
                              p.k_cache.shape[:2] + (p.head_dim,))
    o0, l0 = _run(p)
    p.k_cache = _rotate_cache(p, cs_slot)
    o1, l1 = _run(p, q_cos_sin=cs_tok)
    np.testing.assert_allclose(o1, o0, atol=1e-5)
    np.testing.assert_allclose(l1, l0, atol=1e-5)


def test_shifting_every_position_changes_nothing():
    """Keys stored rotated at their positions and queries rotated at theirs:
    adding one offset to every position keeps the attention (relative
    positions only)."""
    p = _problem(8)
    outs = []
    for shift in (0, 5000):
        q_pos = rope_positions(p) + shift
        slot_pos = np.zeros(p.k_cache.shape[:2], dtype=np.int64)
        for b in range(p.batch):
            for n in range(p.info["kv_lens"][b]):
                pg = int(p.kv_indices[int(p.kv_indptr[b]) + n // p.page_size])
                slot_pos[pg, n % p.page_size] = n + shift
        pk = _problem(8)
        pk.k_cache = _rotate_cache(pk, closed_form_rows(slot_pos.reshape(-1), p.head_dim)
                                   .reshape(slot_pos.shape + (p.head_dim,)))
        outs.append(_run(pk, q_cos_sin=closed_form_rows(q_pos, p.head_dim)))
    np.testing.assert_allclose(outs[1][0], outs[0][0], atol=1e-5)
    np.testing.assert_allclose(outs[1][1], outs[0][1], atol=1e-5)


@pytest.mark.parametrize("cache_dtype,src", [("bf16", "bf16"), ("e4m3", "bf16"), ("f32", "f32")])
def test_cache_write_rotates_keys_only(cache_dtype, src):
    """A quarter turn of every pair (cos 0, sin 1) maps a key row (lo, hi) to
    (-hi, lo) exactly, so the written key is quantise((-hi, lo)); values are
    written unrotated."""
    p = make_case(9, prefix_lens=[13, 2], qo_lens=[5, 3], num_qo_heads=4, num_kv_heads=2,
                  head_dim=64, page_size=4, q_dtype="f32" if cache_dtype == "f32" else "bf16",
                  kv_dtype=cache_dtype)
    k_new, v_new = make_append_inputs(p, src, seed=3, spread=2.0)
    cs = np.concatenate([np.zeros((p.num_tokens, 32)), np.ones((p.num_tokens, 32))], axis=1)
    ko, vo = append_kv(k_new, v_new, src, p.k_cache, p.v_cache, cache_dtype, p.kv_indptr,
                       p.kv_indices, p.last_page_len, p.qo_indptr, p.page_size, 0.5, 0.25,
                       k_cos_sin=cs)
    ko0, vo0 = append_kv(k_new, v_new, src, p.k_cache, p.v_cache, cache_dtype, p.kv_indptr,
                         p.kv_indices, p.last_page_len, p.qo_indptr, p.page_size, 0.5, 0.25)
    assert np.array_equal(vo.view(np.uint8), vo0.view(np.uint8))  # NaN-poisoned slots too
    from oracle import source_values

    kx = source_values(k_new, src)
    turned = np.concatenate([-kx[..., 32:], kx[..., :32]], axis=-1)
    for b in range(p.batch):
        kv_len = p.info["kv_lens"][b]
        L = int(p.qo_indptr[b + 1] - p.qo_indptr[b])
        rows = gather_request_kv(ko, p.kv_indices, int(p.kv_indptr[b]), kv_len, p.page_size)
        for t in range(L):
            want = quantise(turned[int(p.qo_indptr[b]) + t], 0.5, cache_dtype)
            assert np.array_equal(np.ascontiguousarray(rows[kv_len - L + t]).view(np.uint8),
                                  np.ascontiguousarray(want).view(np.uint8))
