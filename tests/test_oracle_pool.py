"""The process pool that spreads the oracle over (request, KV head) items
gives bitwise the result of one direct oracle call: every mask layout, fp8
caches, RoPE rows, requests without query rows, page sizes 1 and 16; and the
in-process form gives the same bits."""

import numpy as np
import pytest

from oracle import verify_attention as oracle_va
from tests.oracle_pool import InProcessOracle, OraclePool, default_workers
from workloads import make_case, rope_cos_sin, rope_positions


@pytest.fixture(scope="module")
def pool():
    with OraclePool(workers=min(4, default_workers())) as p:
        yield p


CASES = {
    "causal_bf16": dict(prefix_lens=[33, 0, 70], qo_lens=[3, 5, 1], num_qo_heads=6, num_kv_heads=2,
                        head_dim=64, page_size=16),
    "tree_bits_fp8": dict(prefix_lens=[20, 41], qo_lens=[7, 4], num_qo_heads=8, num_kv_heads=2,
                          head_dim=128, page_size=4, kv_dtype="e4m3", mask_kind="tree",
                          fp8_absmax_scales=True),
    "random_rows": dict(prefix_lens=[12, 5, 30], qo_lens=[4, 6, 2], num_qo_heads=4,
                        num_kv_heads=4, head_dim=64, page_size=1, mask_kind="random",
                        mask_layout="rows"),
    "f32_gqa": dict(prefix_lens=[9, 17], qo_lens=[4, 4], num_qo_heads=12, num_kv_heads=3,
                    head_dim=64, page_size=16, q_dtype="f32", kv_dtype="f32"),
    "empty_request": dict(prefix_lens=[5, 10, 3], qo_lens=[2, 0, 3], num_qo_heads=4,
                          num_kv_heads=2, head_dim=64, page_size=2),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("rope", [False, True])
def test_pool_equals_direct_oracle_bitwise(pool, name, rope):
    p = make_case(17, **CASES[name])
    cs = rope_cos_sin(rope_positions(p), p.head_dim) if rope else None
    want = oracle_va(p.q, p.k_cache, p.v_cache, p.kv_indptr, p.kv_indices, p.last_page_len,
                     p.qo_indptr, p.mask, p.mask_indptr, sm_scale=p.sm_scale, k_scale=p.k_scale,
                     v_scale=p.v_scale, q_dtype=p.q_dtype, kv_dtype=p.kv_dtype,
                     mask_layout=p.mask_layout, q_cos_sin=cs)
    got = pool.run(p, q_cos_sin=cs)
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1], want[1])


def test_pool_restricted_to_some_requests(pool):
    p = make_case(18, **CASES["causal_bf16"])
    o, l = pool.run(p, requests=[2])
    t0 = int(p.qo_indptr[2])
    assert np.isneginf(l[:t0]).all() and not o[:t0].any()
    want = oracle_va(p.q, p.k_cache, p.v_cache, p.kv_indptr, p.kv_indices, p.last_page_len,
                     p.qo_indptr, None, None, sm_scale=p.sm_scale, q_dtype=p.q_dtype,
                     kv_dtype=p.kv_dtype, requests=[2])
    assert np.array_equal(o, want[0]) and np.array_equal(l, want[1])


@pytest.mark.parametrize("name", ["tree_bits_fp8", "random_rows"])
def test_in_process_form_equals_the_pool_bitwise(pool, name):
    # The form the bench uses under a profiler (no worker processes).
    p = make_case(19, **CASES[name])
    cs = rope_cos_sin(rope_positions(p), p.head_dim)
    want = pool.run(p, q_cos_sin=cs)
    got = InProcessOracle().run(p, q_cos_sin=cs)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    got = InProcessOracle().run(p, requests=[1], q_cos_sin=cs)
    want = pool.run(p, requests=[1], q_cos_sin=cs)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
