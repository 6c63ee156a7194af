"""GPU parity of RoPE at tree positions: queries rotated inside the partial
kernel (verify_attention_rope) and keys rotated by the cache write
(vat_append_kv_rope), both through the C ABI, against the oracle.

Attention is compared at the parity tolerances; the cache write bit for bit
over whole caches.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import append_kv as oracle_append
from oracle import verify_attention as oracle_attention
from tests.gpu_helpers import compare, oracle_of, run_gpu, say, to_device, to_f64
from workloads import make_append_inputs, make_case, make_config, rope_cos_sin, rope_positions

pytestmark = pytest.mark.gpu


def _rope_run(lib, p, cs, tensors=None, **kw):
    t = tensors if tensors is not None else to_device(p)
    out, lse = lib.verify_attention(
        t["q"], t["k_cache"], t["v_cache"], t["kv_indptr"], t["kv_indices"], t["last_page_len"],
        t["qo_indptr"], t["mask"], t["mask_indptr"], sm_scale=p.sm_scale, k_scale=p.k_scale,
        v_scale=p.v_scale, max_qo_len=p.max_qo_len, mask_layout=p.mask_layout,
        q_cos_sin=torch.from_numpy(np.ascontiguousarray(cs)).cuda(), **kw)
    torch.cuda.synchronize()
    return out, lse


def _oracle(p, cs, requests=None):
    return oracle_attention(p.q, p.k_cache, p.v_cache, p.kv_indptr, p.kv_indices,
                            p.last_page_len, p.qo_indptr, p.mask, p.mask_indptr,
                            sm_scale=p.sm_scale, k_scale=p.k_scale, v_scale=p.v_scale,
                            q_dtype=p.q_dtype, kv_dtype=p.kv_dtype, requests=requests,
                            mask_layout=p.mask_layout, q_cos_sin=cs)


@pytest.mark.parametrize("cid", [2, 3, 4, 5, 6, 7])
def test_query_rope_on_the_workloads(gpu_lib, oracle_pool, cid):
    """Every request against the oracle with rotation (spread over host cores)."""
    p = make_config(cid)
    cs = rope_cos_sin(rope_positions(p), p.head_dim)
    say(f"[rope config {cid}] {p.name}")
    got = _rope_run(gpu_lib, p, cs)
    ref = oracle_pool.run(p, q_cos_sin=cs)
    eo, el = compare(p, *to_f64(*got), *ref, what=f"rope config {cid}")
    say(f"  max|out err| {eo:.3e} max|lse err| {el:.3e}")


@pytest.mark.parametrize("seed", list(range(12)))
def test_query_rope_fuzz(gpu_lib, seed):
    rng = np.random.default_rng(700 + seed)
    pairs = [("bf16", "bf16"), ("bf16", "e4m3")]
    q_dt, kv_dt = pairs[seed % 2]
    D = 128 if kv_dt == "e4m3" else [64, 128][(seed // 2) % 2]
    B = int(rng.integers(1, 5))
    G = int(rng.choice([1, 4, 8]))
    lens = [int(x) for x in rng.integers(1, 18, size=B)]
    p = make_case(seed, prefix_lens=[int(x) for x in rng.integers(0, 500, size=B)], qo_lens=lens,
                  num_qo_heads=2 * G, num_kv_heads=2, head_dim=D, page_size=int(rng.choice([1, 16])),
                  q_dtype=q_dt, kv_dtype=kv_dt, mask_kind=["tree", "causal", "random"][seed % 3],
                  fp8_absmax_scales=(kv_dt == "e4m3"))
    pos = rope_positions(p) + int(rng.integers(0, 100000))
    cs = rope_cos_sin(pos, D, theta=float(rng.choice([10000.0, 500000.0])))
    chunk = int(rng.choice([-1, 0, 64]))
    say(f"[rope fuzz {seed}] {q_dt}/{kv_dt} D={D} G={G} L={lens} chunk={chunk}")
    got = _rope_run(gpu_lib, p, cs, chunk_keys=chunk)
    compare(p, *to_f64(*got), *_oracle(p, cs), what=f"rope fuzz {seed}")


@pytest.mark.parametrize("kv_dtype,head_dim", [("bf16", 128), ("bf16", 64), ("e4m3", 128)])
@pytest.mark.parametrize("group,page_size,max_len", [(3, 4, 64), (16, 256, 9), (5, 64, 33)])
def test_query_rope_groups_page_sizes_and_long_drafts(gpu_lib, kv_dtype, head_dim, group, page_size,
                                                      max_len):
    p = make_case(91, prefix_lens=[300, 0, 1100], qo_lens=[max_len, 1, max(1, max_len // 2)],
                  num_qo_heads=2 * group, num_kv_heads=2, head_dim=head_dim, page_size=page_size,
                  q_dtype="bf16", kv_dtype=kv_dtype, mask_kind="tree",
                  fp8_absmax_scales=(kv_dtype == "e4m3"))
    cs = rope_cos_sin(rope_positions(p) + 1234, head_dim, theta=10000.0)
    say(f"[rope] {kv_dtype} D{head_dim} G={group} page {page_size} L<={max_len}")
    got = _rope_run(gpu_lib, p, cs)
    compare(p, *to_f64(*got), *_oracle(p, cs),
            what=f"rope {kv_dtype} D{head_dim} G{group} page {page_size}")


def test_identity_rotation_equals_the_plain_call_bitwise(gpu_lib):
    p = make_config(3)
    cs = np.concatenate([np.ones((p.num_tokens, 64)), np.zeros((p.num_tokens, 64))],
                        axis=1).astype(np.float32)
    t = to_device(p)
    plain = run_gpu(gpu_lib, p, tensors=t)
    rotated = _rope_run(gpu_lib, p, cs, tensors=t)
    assert torch.equal(plain[0].view(torch.int16), rotated[0].view(torch.int16))
    assert torch.equal(plain[1], rotated[1])


def _raw(t):
    if t.dtype == torch.float32:
        return t.cpu().numpy().view(np.uint32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.uint8).cpu().numpy()


def _src(arr, dt):
    a = np.ascontiguousarray(arr)
    if dt == "f32":
        return torch.from_numpy(a).cuda()
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("cache_dtype,src", [("bf16", "bf16"), ("e4m3", "bf16"), ("f32", "f32"),
                                             ("e4m3", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.0123, 0.37)])
@pytest.mark.parametrize("special", ["none", "bits"])
def test_cache_write_with_rope_is_bit_exact(gpu_lib, cache_dtype, src, scales, special):
    p = make_case(41, prefix_lens=[13, 0, 100, 7], qo_lens=[5, 3, 17, 9], num_qo_heads=8,
                  num_kv_heads=4, head_dim=128, page_size=16,
                  q_dtype="f32" if cache_dtype == "f32" else "bf16", kv_dtype=cache_dtype,
                  mask_kind="tree")
    if special == "bits" and src == "f32":
        k_new, v_new = make_append_inputs(p, src, seed=7, special="f32_bits")
    elif special == "bits":
        k_new, v_new = make_append_inputs(p, src, seed=7, special="all_bf16")
    else:
        k_new, v_new = make_append_inputs(p, src, seed=7, spread=3.0)
    cs = rope_cos_sin(rope_positions(p) + 3000, p.head_dim)
    ks, vs = scales
    say(f"[rope write {cache_dtype} <- {src} scales {scales} {special}]")
    t = to_device(p)
    gpu_lib.append_kv(_src(k_new, src), _src(v_new, src), t["k_cache"], t["v_cache"],
                      t["kv_indptr"], t["kv_indices"], t["last_page_len"], t["qo_indptr"],
                      k_scale=ks, v_scale=vs, k_cos_sin=torch.from_numpy(cs).cuda())
    torch.cuda.synchronize()
    want_k, want_v = oracle_append(k_new, v_new, src, p.k_cache, p.v_cache, cache_dtype,
                                   p.kv_indptr, p.kv_indices, p.last_page_len, p.qo_indptr,
                                   p.page_size, ks, vs, k_cos_sin=cs)
    for name, got, want in (("k", _raw(t["k_cache"]), want_k), ("v", _raw(t["v_cache"]), want_v)):
        want = want.view(np.uint32) if want.dtype == np.float32 else want
        bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
        assert bad.size == 0, (f"{name}: {bad.size} words differ; first flat {int(bad[0])}: "
                               f"got {got.reshape(-1)[bad[0]]:#x} want {want.reshape(-1)[bad[0]]:#x}")


@pytest.mark.parametrize("cache_dtype,src", [("bf16", "bf16"), ("e4m3", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("page_size", [1, 4, 64, 256])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_cache_write_with_rope_at_every_page_size(gpu_lib, cache_dtype, src, page_size, head_dim):
    p = make_case(43, prefix_lens=[13, 0, 300, 7], qo_lens=[5, 3, 17, 9], num_qo_heads=8,
                  num_kv_heads=4, head_dim=head_dim, page_size=page_size,
                  q_dtype="f32" if cache_dtype == "f32" else "bf16", kv_dtype=cache_dtype,
                  mask_kind="tree")
    k_new, v_new = make_append_inputs(p, src, seed=8, spread=2.0)
    cs = rope_cos_sin(rope_positions(p) + 777, head_dim)
    ks, vs = (0.37, 1.5) if cache_dtype == "e4m3" else (1.0, 1.0)
    say(f"[rope write {cache_dtype} <- {src} page {page_size} D{head_dim}]")
    t = to_device(p)
    gpu_lib.append_kv(_src(k_new, src), _src(v_new, src), t["k_cache"], t["v_cache"],
                      t["kv_indptr"], t["kv_indices"], t["last_page_len"], t["qo_indptr"],
                      k_scale=ks, v_scale=vs, k_cos_sin=torch.from_numpy(cs).cuda())
    torch.cuda.synchronize()
    want_k, want_v = oracle_append(k_new, v_new, src, p.k_cache, p.v_cache, cache_dtype,
                                   p.kv_indptr, p.kv_indices, p.last_page_len, p.qo_indptr,
                                   p.page_size, ks, vs, k_cos_sin=cs)
    for name, got, want in (("k", _raw(t["k_cache"]), want_k), ("v", _raw(t["v_cache"]), want_v)):
        want = want.view(np.uint32) if want.dtype == np.float32 else want
        bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
        assert bad.size == 0, (f"{name}: {bad.size} words differ; first flat {int(bad[0])}: "
                               f"got {got.reshape(-1)[bad[0]]:#x} want {want.reshape(-1)[bad[0]]:#x}")


@pytest.mark.parametrize("cid", [3, 5])
def test_write_then_attend_with_rope(gpu_lib, cid):
    """Keys rotated at the cache write, queries in the kernel, same positions:
    the GPU chain against the oracle chain."""
    p = make_config(cid)
    cs = rope_cos_sin(rope_positions(p), p.head_dim)
    k_new, v_new = make_append_inputs(p, "bf16", seed=300 + cid, spread=1.0)
    t = to_device(p)
    gpu_lib.append_kv(_src(k_new, "bf16"), _src(v_new, "bf16"), t["k_cache"], t["v_cache"],
                      t["kv_indptr"], t["kv_indices"], t["last_page_len"], t["qo_indptr"],
                      k_scale=p.k_scale, v_scale=p.v_scale, k_cos_sin=torch.from_numpy(cs).cuda())
    got = _rope_run(gpu_lib, p, cs, tensors=t)
    k2, v2 = oracle_append(k_new, v_new, "bf16", p.k_cache, p.v_cache, p.kv_dtype, p.kv_indptr,
                           p.kv_indices, p.last_page_len, p.qo_indptr, p.page_size, p.k_scale,
                           p.v_scale, k_cos_sin=cs)
    p.k_cache, p.v_cache = k2, v2
    compare(p, *to_f64(*got), *_oracle(p, cs), what=f"rope chain {cid}")


# ---------------------------------------------------------------- RoPE with full byte-row masks


@pytest.mark.parametrize("prefix", [4096, 32768])
def test_query_rope_with_full_row_masks_on_the_tree_workload(gpu_lib, oracle_pool, prefix):
    """The batch-1 tree workload with sglang's byte rows and rotated queries:
    against the oracle, and bitwise equal to the packed-bit layout (RoPE keeps
    one row tile per wave for both layouts, so the plans are the same)."""
    p = make_config(3, prefix=prefix, mask_layout="rows")
    q = make_config(3, prefix=prefix)
    cs = rope_cos_sin(rope_positions(q), p.head_dim)
    say(f"[rope rows config 3 prefix {prefix}]")
    got = _rope_run(gpu_lib, p, cs)
    compare(p, *to_f64(*got), *oracle_pool.run(p, q_cos_sin=cs), what=f"rope rows {prefix}")
    bits = _rope_run(gpu_lib, q, cs)
    assert torch.equal(got[0].view(torch.int16), bits[0].view(torch.int16))
    assert torch.equal(got[1], bits[1])


@pytest.mark.parametrize("seed", list(range(8)))
def test_query_rope_with_full_row_masks_fuzz(gpu_lib, seed):
    rng = np.random.default_rng(900 + seed)
    kv_dt, D = [("bf16", 128), ("bf16", 64), ("e4m3", 128)][seed % 3]
    B = int(rng.integers(1, 5))
    G = int(rng.choice([1, 4, 8]))
    lens = [int(x) for x in rng.integers(1, 40, size=B)]
    p = make_case(seed, prefix_lens=[int(x) for x in rng.integers(0, 400, size=B)], qo_lens=lens,
                  num_qo_heads=2 * G, num_kv_heads=2, head_dim=D,
                  page_size=int(rng.choice([1, 4, 16, 64])), q_dtype="bf16", kv_dtype=kv_dt,
                  mask_kind=["tree", "random", "chain", "full"][seed % 4],
                  fp8_absmax_scales=(kv_dt == "e4m3"), mask_layout="rows",
                  rows_prefix_fill=["ones", "zeros", "random"][seed % 3],
                  rows_true_values=["ones", "random"][seed % 2])
    cs = rope_cos_sin(rope_positions(p) + int(rng.integers(0, 100000)), D)
    chunk = int(rng.choice([-1, 0, 64]))
    say(f"[rope rows fuzz {seed}] {kv_dt} D={D} G={G} L={lens} chunk={chunk}")
    got = _rope_run(gpu_lib, p, cs, chunk_keys=chunk)
    compare(p, *to_f64(*got), *_oracle(p, cs), what=f"rope rows fuzz {seed}")
