"""GPU parity of the draft key/value write (cache append with quantise-on-write).

The HIP kernel, called through the C ABI, against the CPU oracle on the same
seeded inputs. The bar is bit-exact: every byte of both caches after the
write (written slots, untouched slots and the NaN-poisoned spare pages)
equals the oracle's.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import append_kv as oracle_append
from oracle import verify_attention as oracle_attention
from tests.gpu_helpers import compare, rows_of, say, to_device, to_f64
from workloads import make_append_inputs, make_case, make_config

pytestmark = pytest.mark.gpu


def _src_tensor(arr: np.ndarray, dt: str) -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if dt == "f32":
        return torch.from_numpy(a).cuda()
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    raise ValueError(dt)


def _raw(t: torch.Tensor) -> np.ndarray:
    """Device cache -> host array of its raw storage words."""
    if t.dtype == torch.float32:
        return t.cpu().numpy().view(np.uint32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.uint8).cpu().numpy()


def _words(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _run(lib, p, k_new, v_new, src, ks, vs, max_qo_len=None, tensors=None, num_cus=0):
    t = tensors if tensors is not None else to_device(p)
    lib.append_kv(_src_tensor(k_new, src), _src_tensor(v_new, src), t["k_cache"], t["v_cache"],
                  t["kv_indptr"], t["kv_indices"], t["last_page_len"], t["qo_indptr"],
                  k_scale=ks, v_scale=vs, max_qo_len=max_qo_len, num_cus=num_cus)
    torch.cuda.synchronize()
    return t


def _check(lib, p, k_new, v_new, src, ks, vs, what, max_qo_len=None, num_cus=0):
    say(f"[append {what}] {p.name or 'case'} src={src} cache={p.kv_dtype} "
        f"T={int(p.qo_indptr[-1])} scales=({ks:.6g}, {vs:.6g}) max_qo_len={max_qo_len} "
        f"num_cus={num_cus}")
    t = _run(lib, p, k_new, v_new, src, ks, vs, max_qo_len=max_qo_len, num_cus=num_cus)
    got_k, got_v = _raw(t["k_cache"]), _raw(t["v_cache"])
    want_k, want_v = oracle_append(k_new, v_new, src, p.k_cache, p.v_cache, p.kv_dtype,
                                   p.kv_indptr, p.kv_indices, p.last_page_len, p.qo_indptr,
                                   p.page_size, k_scale=ks, v_scale=vs)
    for name, got, want in (("k_cache", got_k, want_k), ("v_cache", got_v, want_v)):
        want = _words(want)
        assert got.shape == want.shape and got.dtype == want.dtype, (name, got.dtype, want.dtype)
        bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
        if bad.size:
            i = int(bad[0])
            pytest.fail(f"{what}: {name} differs in {bad.size} words; first at flat {i} "
                        f"(index {np.unravel_index(i, got.shape)}): got {got.reshape(-1)[i]:#x} "
                        f"want {want.reshape(-1)[i]:#x}")
    say("  bit-exact")
    return t


# ---------------------------------------------------------------- the workloads' drafts


APPEND_CONFIGS = [
    # (config, source dtype, spread of the new values, scales: None = the config's)
    (1, "f32", 1.0, (1.0, 1.0)),
    (1, "f32", 1.0, (0.37, 3.0)),
    (2, "bf16", 1.0, None),
    (2, "f32", 1.0, (0.25, 0.75)),
    (3, "bf16", 1.0, (0.5, 2.0)),
    (4, "bf16", 1.0, None),
    (5, "bf16", 2.0, None),
    (5, "f32", 2.0, None),
]


@pytest.mark.parametrize("cid,src,spread,scales", APPEND_CONFIGS, ids=lambda x: str(x))
def test_append_parity_on_the_workloads(gpu_lib, cid, src, spread, scales):
    """Each workload's drafts rewritten with fresh values; config 5 writes
    e4m3fn with its absmax/448 scales and values spread beyond the cache's
    range, so some saturate."""
    p = make_config(cid)
    ks, vs = scales if scales is not None else (p.k_scale, p.v_scale)
    k_new, v_new = make_append_inputs(p, src, seed=100 + cid, spread=spread)
    _check(gpu_lib, p, k_new, v_new, src, ks, vs, f"config {cid}")


# ---------------------------------------------------------------- every value class


def _pattern_case(cache_dtype, page_size=16, head_dim=128):
    # 64 draft tokens x 4 KV heads x 128 = 32768 elements per tensor: K and V
    # together hold each of the 65536 bfloat16 patterns once. Requests with
    # no drafts, drafts that straddle pages and a request made only of drafts.
    return make_case(31, prefix_lens=[13, 0, 30, 7, 100], qo_lens=[5, 3, 0, 9, 47],
                     num_qo_heads=8, num_kv_heads=4, head_dim=head_dim, page_size=page_size,
                     q_dtype="f32" if cache_dtype == "f32" else "bf16", kv_dtype=cache_dtype,
                     name=f"patterns-{cache_dtype}-ps{page_size}-d{head_dim}")


# The write takes two units per thread when it covers every CU several times
# over; planning for one CU makes these small cases take that variant too.
NUM_CUS = [0, 1]


@pytest.mark.parametrize("num_cus", NUM_CUS)
@pytest.mark.parametrize("cache_dtype", ["bf16", "e4m3", "f32"])
@pytest.mark.parametrize("scale", [1.0, 0.0123, 3.75])
def test_every_bf16_pattern(gpu_lib, cache_dtype, scale, num_cus):
    """All 65536 bfloat16 inputs (NaNs, infinities, subnormals, both zeros)
    divided by the scale and stored (scale 1 takes the exact-reciprocal
    path: both scales are powers of two)."""
    p = _pattern_case(cache_dtype)
    k_new, v_new = make_append_inputs(p, "bf16", seed=0, special="all_bf16")
    _check(gpu_lib, p, k_new, v_new, "bf16", scale, float(np.float32(scale * 0.5)),
           f"all bf16 patterns scale {scale}", num_cus=num_cus)


@pytest.mark.parametrize("num_cus", NUM_CUS)
@pytest.mark.parametrize("cache_dtype", ["bf16", "e4m3", "f32"])
@pytest.mark.parametrize("seed,scale", [(1, 1.0), (2, 3.75), (3, 1e-3), (4, 2.0 ** -20),
                                        (5, 2.0 ** 100)])
def test_random_f32_bit_patterns(gpu_lib, cache_dtype, seed, scale, num_cus):
    """Uniformly random 32-bit inputs: every class of binary32 value, and
    quotients that underflow to subnormals or overflow (checks both the
    division and the exact-reciprocal multiply keep IEEE results)."""
    p = _pattern_case(cache_dtype)
    k_new, v_new = make_append_inputs(p, "f32", seed=seed, special="f32_bits")
    _check(gpu_lib, p, k_new, v_new, "f32", scale, scale, f"random f32 bits seed {seed}",
           num_cus=num_cus)


@pytest.mark.parametrize("scales", [(1.0, 0.75), (0.0123, 0.5), (2.0 ** -126, 2.0 ** 126),
                                    (2.0 ** 127, 1.0), (2.0 ** -130, 1.0)])
def test_mixed_and_extreme_scales(gpu_lib, scales):
    """Only both scales being normal powers of two with normal reciprocals
    takes the multiply; the extreme ones (2^127, a subnormal 2^-130) divide."""
    p = _pattern_case("e4m3")
    k_new, v_new = make_append_inputs(p, "f32", seed=6, special="f32_bits")
    ks, vs = (float(np.float32(x)) for x in scales)
    _check(gpu_lib, p, k_new, v_new, "f32", ks, vs, f"scales {scales}")


# ---------------------------------------------------------------- layout edges


@pytest.mark.parametrize("page_size,head_dim", [(1, 128), (4, 64), (16, 64), (256, 128)])
def test_page_sizes_and_head_dims(gpu_lib, page_size, head_dim):
    p = _pattern_case("e4m3", page_size=page_size, head_dim=head_dim)
    k_new, v_new = make_append_inputs(p, "bf16", seed=7, spread=300.0)
    _check(gpu_lib, p, k_new, v_new, "bf16", 0.75, 0.5, f"page {page_size} D {head_dim}")


def test_launch_bound_below_the_real_draft_count(gpu_lib):
    """max_qo_len only sizes the launch: with a bound of 1 every request's
    rows are still written (workgroups loop over the rest)."""
    p = _pattern_case("bf16")
    k_new, v_new = make_append_inputs(p, "f32", seed=8, spread=4.0)
    _check(gpu_lib, p, k_new, v_new, "f32", 1.0, 1.0, "max_qo_len 1", max_qo_len=1)


def test_long_requests_use_many_workgroups(gpu_lib):
    """Requests of 3000 drafts on 8 KV heads: 3000 workgroups per request."""
    p = make_case(33, prefix_lens=[5, 1000], qo_lens=[3000, 2999], num_qo_heads=8,
                  num_kv_heads=8, head_dim=128, page_size=16, kv_dtype="e4m3",
                  name="long-drafts")
    k_new, v_new = make_append_inputs(p, "bf16", seed=9, spread=1.5)
    _check(gpu_lib, p, k_new, v_new, "bf16", 0.0123, 0.0071, "long requests")
    _check(gpu_lib, p, k_new, v_new, "bf16", 0.0123, 0.0071, "long requests, 1 CU", num_cus=1)


def test_no_drafts_changes_nothing(gpu_lib):
    p = make_case(34, prefix_lens=[10, 20], qo_lens=[0, 0], num_qo_heads=4, num_kv_heads=2,
                  head_dim=64, page_size=16, name="no drafts")
    k_new = np.zeros((0, 2, 64), dtype=np.uint16)
    _check(gpu_lib, p, k_new, k_new.copy(), "bf16", 1.0, 1.0, "no drafts")


@pytest.mark.parametrize("cache_dtype", ["bf16", "e4m3", "f32"])
def test_writes_past_4_gib_of_the_pool_land_exactly(gpu_lib, cache_dtype):
    """The same pages placed beyond byte offset 4.5 GiB of a larger pool (in
    reverse order) receive bitwise the same drafts, and the poisoned slots
    below them stay untouched: slot addresses are 64-bit."""
    src = "f32" if cache_dtype == "f32" else "bf16"
    p = make_case(58, prefix_lens=[300, 40, 900], qo_lens=[5, 3, 8], num_qo_heads=32,
                  num_kv_heads=8, head_dim=128, q_dtype=src, kv_dtype=cache_dtype, name="big pool")
    k_new, v_new = make_append_inputs(p, src, seed=11, spread=1.0)
    fresh = to_device(p)
    t = _run(gpu_lib, p, k_new, v_new, src, p.k_scale, p.v_scale)
    page_bytes = fresh["k_cache"][0].numel() * fresh["k_cache"].element_size()
    high = -(-(9 << 29) // page_bytes)  # first slot at or past 4.5 GiB
    n = p.num_pages
    say(f"[append big pool] {high + n} pages of {page_bytes} B, cache={cache_dtype}")
    dst = high + torch.arange(n - 1, -1, -1, device="cuda")
    poison = 0x5A
    big = dict(fresh)
    pools = {}
    for name in ("k_cache", "v_cache"):
        raw = fresh[name].view(torch.uint8)
        pool = torch.full((high + n,) + tuple(raw.shape[1:]), poison, dtype=torch.uint8, device="cuda")
        pool[dst] = raw
        pools[name] = pool
        big[name] = pool.view(fresh[name].dtype)
    big["kv_indices"] = dst[fresh["kv_indices"].long()].to(torch.int32)
    _run(gpu_lib, p, k_new, v_new, src, p.k_scale, p.v_scale, tensors=big)
    for name in ("k_cache", "v_cache"):
        pool = pools[name]
        assert torch.equal(pool[dst], t[name].view(torch.uint8)), name
        assert not bool((pool[:high] != poison).any()), name
    del big, pools, pool
    torch.cuda.empty_cache()


def test_repeat_writes_are_identical(gpu_lib):
    p = make_config(5)
    k_new, v_new = make_append_inputs(p, "bf16", seed=10, spread=2.0)
    t = _run(gpu_lib, p, k_new, v_new, "bf16", p.k_scale, p.v_scale)
    first = _raw(t["k_cache"]).copy(), _raw(t["v_cache"]).copy()
    _run(gpu_lib, p, k_new, v_new, "bf16", p.k_scale, p.v_scale, tensors=t)
    assert np.array_equal(first[0], _raw(t["k_cache"]))
    assert np.array_equal(first[1], _raw(t["v_cache"]))


# ---------------------------------------------------------------- write, then attend


@pytest.mark.parametrize("cid", [2, 5])
def test_write_then_attend_matches_the_oracle_chain(gpu_lib, cid):
    """The two steps in order on the GPU (append, then verify attention on
    the same caches) against the oracle's append followed by its attention."""
    p = make_config(cid)
    k_new, v_new = make_append_inputs(p, "bf16", seed=200 + cid, spread=1.0)
    ks, vs = p.k_scale, p.v_scale
    t = _run(gpu_lib, p, k_new, v_new, "bf16", ks, vs)
    out, lse = gpu_lib.verify_attention(
        t["q"], t["k_cache"], t["v_cache"], t["kv_indptr"], t["kv_indices"], t["last_page_len"],
        t["qo_indptr"], t["mask"], t["mask_indptr"], sm_scale=p.sm_scale, k_scale=ks,
        v_scale=vs, max_qo_len=p.max_qo_len)
    torch.cuda.synchronize()
    got_o, got_l = to_f64(out, lse)
    k2, v2 = oracle_append(k_new, v_new, "bf16", p.k_cache, p.v_cache, p.kv_dtype, p.kv_indptr,
                           p.kv_indices, p.last_page_len, p.qo_indptr, p.page_size, ks, vs)
    requests = None if cid == 2 else [0, 17, 63]
    ref_o, ref_l = oracle_attention(p.q, k2, v2, p.kv_indptr, p.kv_indices, p.last_page_len,
                                    p.qo_indptr, p.mask, p.mask_indptr, sm_scale=p.sm_scale,
                                    k_scale=ks, v_scale=vs, q_dtype=p.q_dtype,
                                    kv_dtype=p.kv_dtype, requests=requests)
    rows = None if requests is None else rows_of(p, requests)
    eo, el = compare(p, got_o, got_l, ref_o, ref_l, rows=rows,
                     what=f"append+attend config {cid}")
    say(f"  append+attend config {cid}: max|out err| {eo:.3e} max|lse err| {el:.3e}")
