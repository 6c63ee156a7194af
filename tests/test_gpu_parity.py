"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerances: out within 1e-5 (fp32 inputs) or 2e-2 (bf16 / fp8 inputs, bf16
output) absolute, lse within 1e-3, -inf exactly where the oracle has -inf,
no NaN. Page-index and mask handling must be bit-exact: results are bitwise
equal under a page-pool permutation, for a chain mask versus causal, and
from run to run.
"""

import numpy as np
import pytest
import torch

from tests.gpu_helpers import compare, oracle_of, run_gpu, say, to_device, to_f64
from workloads import make_case, make_config

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- the five workloads


CONFIG_CASES = [(1, None), (2, None), (3, 4096), (3, 16384), (3, 32768), (4, None), (5, None),
                (6, None), (7, None)]


@pytest.mark.parametrize("cid,prefix", CONFIG_CASES, ids=lambda x: str(x))
def test_config_parity(gpu_lib, oracle_pool, cid, prefix):
    """Every request of every workload against the oracle (spread over host
    cores by (request, KV head))."""
    p = make_config(cid, prefix=prefix or 4096)
    say(f"[config {cid} prefix={prefix}] {p.name}")
    plan = gpu_lib.vat_plan(_problem(gpu_lib, p)).as_dict()
    say(f"  plan {plan}")
    out, lse = run_gpu(gpu_lib, p)
    got_o, got_l = to_f64(out, lse)
    ref_o, ref_l = oracle_pool.run(p)
    eo, el = compare(p, got_o, got_l, ref_o, ref_l, what=f"config {cid}")
    say(f"  max|out err| {eo:.3e}  max|lse err| {el:.3e} ({oracle_pool.workers} oracle workers)")


def test_default_max_qo_len_and_sm_scale_for_one_request(gpu_lib):
    """The binding's defaults: one request's bound is T, sm_scale is D^-0.5."""
    p = make_config(3, prefix=4096)
    assert p.batch == 1 and abs(p.sm_scale - p.head_dim ** -0.5) < 1e-7  # float32 rounding
    t = to_device(p)
    out, lse = gpu_lib.verify_attention(t["q"], t["k_cache"], t["v_cache"], t["kv_indptr"],
                                        t["kv_indices"], t["last_page_len"], t["qo_indptr"],
                                        t["mask"], t["mask_indptr"])
    torch.cuda.synchronize()
    compare(p, *to_f64(out, lse), *oracle_of(p), what="defaults")
    with pytest.raises(ValueError, match="max_qo_len"):
        q = make_config(2)
        tq = to_device(q)
        gpu_lib.verify_attention(tq["q"], tq["k_cache"], tq["v_cache"], tq["kv_indptr"],
                                 tq["kv_indices"], tq["last_page_len"], tq["qo_indptr"])


def _problem(lib, p, **kw):
    t = to_device(p)
    return lib.problem_from_tensors(t["q"], t["k_cache"], t["kv_indptr"], t["kv_indices"],
                                    t["mask"], p.max_qo_len, mask_layout=p.mask_layout, **kw)


# ---------------------------------------------------------------- seeded small-shape fuzz


def _fuzz_case(seed):
    rng = np.random.default_rng(1000 + seed)
    pairs = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "e4m3")]
    q_dt, kv_dt = pairs[seed % 3]
    D = [64, 128][(seed // 3) % 2]
    B = int(rng.integers(1, 5))
    Hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 3, 4, 8]))
    ps = int(rng.choice([1, 4, 16, 64]))
    mask_kind = ["causal", "tree", "random", "chain"][seed % 4]
    Lmax = 20 if mask_kind != "causal" else 40
    lens = [int(x) for x in rng.integers(1, Lmax + 1, size=B)]
    prefixes = [int(x) for x in rng.integers(0, 301, size=B)]
    chunk = int(rng.choice([-1, 0, 48, 64, 128]))
    p = make_case(seed, prefix_lens=prefixes, qo_lens=lens, num_qo_heads=G * Hkv,
                  num_kv_heads=Hkv, head_dim=D, page_size=ps, q_dtype=q_dt, kv_dtype=kv_dt,
                  mask_kind=mask_kind, fp8_absmax_scales=(kv_dt == "e4m3"), mask_density=0.4,
                  mask_pad_bytes=int(seed % 3), extra_indices=int(seed % 5))
    return p, chunk


@pytest.mark.parametrize("seed", list(range(36)))
def test_fuzz_small_shapes(gpu_lib, seed):
    p, chunk = _fuzz_case(seed)
    say(f"[fuzz {seed}] B={p.batch} Hq={p.num_qo_heads} Hkv={p.num_kv_heads} D={p.head_dim} "
        f"ps={p.page_size} {p.q_dtype}/{p.kv_dtype} mask={p.info['mask_kind']} "
        f"L={p.info['qo_lens']} prefix={p.info['prefix_lens']} chunk={chunk}")
    out, lse = run_gpu(gpu_lib, p, chunk_keys=chunk)
    compare(p, *to_f64(out, lse), *oracle_of(p), what=f"fuzz {seed}")


# ---------------------------------------------------------------- edge cases


EDGE = {
    "prefix0_L1": dict(prefix_lens=[0], qo_lens=[1]),
    "kv_len_multiple_of_page": dict(prefix_lens=[27, 11], qo_lens=[5, 5]),
    "last_page_len_1": dict(prefix_lens=[16, 32], qo_lens=[1, 1]),
    "verify_straddles_page": dict(prefix_lens=[14, 30], qo_lens=[7, 9]),
    "empty_request_between": dict(prefix_lens=[40, 9, 70], qo_lens=[3, 0, 4]),
    "decode_many_requests": dict(prefix_lens=list(range(0, 640, 10)), qo_lens=[1] * 64),
    "long_prefill_causal": dict(prefix_lens=[0, 35], qo_lens=[300, 129]),
}


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("chunk", [-1, 0, 64])
def test_edge_cases(gpu_lib, name, chunk):
    kw = EDGE[name]
    p = make_case(77, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16, **kw)
    say(f"[edge {name} chunk={chunk}]")
    out, lse = run_gpu(gpu_lib, p, chunk_keys=chunk)
    compare(p, *to_f64(out, lse), *oracle_of(p), what=name)


@pytest.mark.parametrize("kv_dtype,head_dim", [("f32", 64), ("bf16", 128), ("bf16", 64),
                                               ("e4m3", 128), ("e4m3", 64)])
@pytest.mark.parametrize("mask_kind", ["tree", "random"])
@pytest.mark.parametrize("chunk", [-1, 64])
def test_masks_at_the_64_draft_maximum(gpu_lib, kv_dtype, head_dim, mask_kind, chunk):
    q_dtype = "f32" if kv_dtype == "f32" else "bf16"
    p = make_case(88, prefix_lens=[100, 0, 37], qo_lens=[64, 64, 1], num_qo_heads=8, num_kv_heads=2,
                  head_dim=head_dim, q_dtype=q_dtype, kv_dtype=kv_dtype, mask_kind=mask_kind,
                  fp8_absmax_scales=(kv_dtype == "e4m3"), mask_density=0.4)
    assert p.max_qo_len == 64
    say(f"[64 drafts] {kv_dtype} D{head_dim} mask={mask_kind} chunk={chunk}")
    out, lse = run_gpu(gpu_lib, p, chunk_keys=chunk)
    compare(p, *to_f64(out, lse), *oracle_of(p), what=f"64 drafts {kv_dtype} D{head_dim} {mask_kind}")


@pytest.mark.parametrize("kv_dtype,head_dim", [("bf16", 128), ("e4m3", 128), ("f32", 64), ("e4m3", 64)])
@pytest.mark.parametrize("page_size", [2, 8, 32, 128, 256])
@pytest.mark.parametrize("chunk", [-1, 0])
def test_every_page_size(gpu_lib, kv_dtype, head_dim, page_size, chunk):
    q_dtype = "f32" if kv_dtype == "f32" else "bf16"
    p = make_case(89, prefix_lens=[700, 3, 1300], qo_lens=[6, 2, 9], num_qo_heads=16, num_kv_heads=4,
                  head_dim=head_dim, page_size=page_size, q_dtype=q_dtype, kv_dtype=kv_dtype,
                  mask_kind="tree", fp8_absmax_scales=(kv_dtype == "e4m3"))
    say(f"[page size {page_size}] {kv_dtype} D{head_dim} chunk={chunk}")
    out, lse = run_gpu(gpu_lib, p, chunk_keys=chunk)
    compare(p, *to_f64(out, lse), *oracle_of(p), what=f"page size {page_size} {kv_dtype} D{head_dim}")


@pytest.mark.parametrize("kv_dtype,head_dim", [("bf16", 128), ("e4m3", 128), ("f32", 64), ("bf16", 64)])
@pytest.mark.parametrize("group", [2, 3, 5, 16, 64])
@pytest.mark.parametrize("mask_kind", ["causal", "tree"])
def test_query_head_groups(gpu_lib, kv_dtype, head_dim, group, mask_kind):
    q_dtype = "f32" if kv_dtype == "f32" else "bf16"
    hkv = 1 if group == 64 else 2
    p = make_case(90, prefix_lens=[260, 0, 900], qo_lens=[5, 1, 12], num_qo_heads=group * hkv,
                  num_kv_heads=hkv, head_dim=head_dim, q_dtype=q_dtype, kv_dtype=kv_dtype,
                  mask_kind=mask_kind, fp8_absmax_scales=(kv_dtype == "e4m3"))
    say(f"[group {group}] Hkv={hkv} {kv_dtype} D{head_dim} mask={mask_kind}")
    out, lse = run_gpu(gpu_lib, p)
    compare(p, *to_f64(out, lse), *oracle_of(p), what=f"group {group} {kv_dtype} D{head_dim} {mask_kind}")


def test_fully_masked_rows_give_zero_and_minus_inf(gpu_lib):
    p = make_case(5, prefix_lens=[0, 0], qo_lens=[6, 9], num_qo_heads=4, num_kv_heads=1,
                  head_dim=64, page_size=4, q_dtype="f32", kv_dtype="f32", mask_kind="random",
                  mask_density=0.2)
    ref_o, ref_l = oracle_of(p)
    assert np.isneginf(ref_l).any(), "seed should produce a fully masked row"
    for chunk in (-1, 0, 64):
        say(f"[fully masked chunk={chunk}]")
        out, lse = run_gpu(gpu_lib, p, chunk_keys=chunk)
        got_o, got_l = to_f64(out, lse)
        compare(p, got_o, got_l, ref_o, ref_l, what="fully masked")
        assert np.all(got_o[np.isneginf(ref_l)] == 0.0)


def test_empty_batch_and_no_tokens(gpu_lib):
    import torch

    dev = "cuda"
    q = torch.zeros(0, 4, 64, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(2, 16, 1, 64, dtype=torch.bfloat16, device=dev)
    for B in (0, 2):
        kv_indptr = torch.zeros(B + 1, dtype=torch.int32, device=dev)
        idx = torch.zeros(1, dtype=torch.int32, device=dev)
        lpl = torch.ones(B, dtype=torch.int32, device=dev)
        qo = torch.zeros(B + 1, dtype=torch.int32, device=dev)
        out, lse = gpu_lib.verify_attention(q, kc, kc.clone(), kv_indptr, idx, lpl, qo)
        torch.cuda.synchronize()
        assert out.shape == (0, 4, 64) and lse.shape == (0, 4)


# ---------------------------------------------------------------- bit-exactness


def test_page_permutation_is_bitwise_invariant(gpu_lib):
    base = make_case(31, prefix_lens=[500, 77, 1200], qo_lens=[5, 3, 8], num_qo_heads=16,
                     num_kv_heads=4, head_dim=128, mask_kind="tree")
    t = to_device(base)
    out0, lse0 = run_gpu(gpu_lib, base, tensors=t)
    # Move every page to a new physical slot and remap the table.
    rng = np.random.default_rng(3)
    perm = rng.permutation(base.num_pages)
    k2 = np.empty_like(base.k_cache)
    v2 = np.empty_like(base.v_cache)
    k2[perm] = base.k_cache
    v2[perm] = base.v_cache
    idx2 = perm[base.kv_indices].astype(np.int32)
    moved = make_case(31, prefix_lens=[500, 77, 1200], qo_lens=[5, 3, 8], num_qo_heads=16,
                      num_kv_heads=4, head_dim=128, mask_kind="tree")
    moved.k_cache, moved.v_cache, moved.kv_indices = k2, v2, idx2
    out1, lse1 = run_gpu(gpu_lib, moved)
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0, lse1)


@pytest.mark.parametrize("kv_dtype", ["bf16", "e4m3", "f32"])
def test_pages_past_4_gib_of_the_pool_are_addressed_exactly(gpu_lib, kv_dtype):
    """The same pages placed beyond byte offset 4.5 GiB of a larger pool (in
    reverse order) give bitwise the same result: page bases are 64-bit."""
    q_dtype = "f32" if kv_dtype == "f32" else "bf16"
    kw = dict(prefix_lens=[700, 90, 1500], qo_lens=[5, 2, 9], num_qo_heads=32, num_kv_heads=8,
              head_dim=128, q_dtype=q_dtype, kv_dtype=kv_dtype, mask_kind="tree")
    base = make_case(57, **kw)
    t = to_device(base)
    out0, lse0 = run_gpu(gpu_lib, base, tensors=t)
    out0, lse0 = out0.clone(), lse0.clone()
    page_bytes = t["k_cache"][0].numel() * t["k_cache"].element_size()
    high = -(-(9 << 29) // page_bytes)  # first slot at or past 4.5 GiB
    n = base.num_pages
    say(f"pool of {high + n} pages of {page_bytes} B ({kv_dtype})")
    dst = high + torch.arange(n - 1, -1, -1, device="cuda")
    big = {}
    for name in ("k_cache", "v_cache"):
        src = t[name].view(torch.uint8)
        pool = torch.empty((high + n,) + tuple(src.shape[1:]), dtype=torch.uint8, device="cuda")
        pool[dst] = src
        big[name] = pool.view(t[name].dtype)
    t2 = dict(t, k_cache=big["k_cache"], v_cache=big["v_cache"],
              kv_indices=dst[t["kv_indices"].long()].to(torch.int32))
    out1, lse1 = run_gpu(gpu_lib, base, tensors=t2)
    same = torch.equal(out0.view(torch.int16), out1.view(torch.int16)) if out0.dtype == torch.bfloat16 \
        else torch.equal(out0.view(torch.int32), out1.view(torch.int32))
    assert same
    assert torch.equal(lse0, lse1)
    del big, t2, out1, lse1
    torch.cuda.empty_cache()


@pytest.mark.parametrize("chunk", [-1, 0])
def test_chain_mask_bitwise_equals_causal(gpu_lib, chunk):
    kw = dict(prefix_lens=[100, 3, 640], qo_lens=[6, 4, 17], num_qo_heads=8, num_kv_heads=2,
              head_dim=128)
    pc = make_case(41, mask_kind="causal", **kw)
    pm = make_case(41, mask_kind="chain", **kw)
    assert np.array_equal(pc.k_cache.view(np.uint16), pm.k_cache.view(np.uint16))
    oc, lc = run_gpu(gpu_lib, pc, chunk_keys=chunk)
    om, lm = run_gpu(gpu_lib, pm, chunk_keys=chunk)
    assert torch.equal(oc.view(torch.int16), om.view(torch.int16))
    assert torch.equal(lc, lm)


def test_repeat_runs_are_bitwise_identical(gpu_lib):
    p = make_config(2)
    t = to_device(p)
    o1, l1 = run_gpu(gpu_lib, p, tensors=t)
    o1, l1 = o1.clone(), l1.clone()
    for _ in range(3):
        o2, l2 = run_gpu(gpu_lib, p, tensors=t)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("chunk", [0, 16, 64, 112, 256, 528, 2048])
def test_any_split_matches_oracle(gpu_lib, chunk):
    p = make_config(3, prefix=4096)
    say(f"[split chunk={chunk}]")
    out, lse = run_gpu(gpu_lib, p, chunk_keys=chunk)
    compare(p, *to_f64(out, lse), *oracle_of(p), what=f"chunk {chunk}")


# ---------------------------------------------------------------- balanced slices


SLICE_CASES = {
    # mixed lengths (and requests without drafts) over many slices
    "mixed_bf16": dict(prefix_lens=[3000, 0, 17, 900, 5000, 64, 1, 2500], qo_lens=[4, 2, 0, 8, 1, 3, 5, 6],
                       num_qo_heads=32, num_kv_heads=8, head_dim=128, mask_kind="tree"),
    "mixed_e4m3": dict(prefix_lens=[700, 4100, 33, 2222], qo_lens=[8, 1, 5, 3], num_qo_heads=16,
                       num_kv_heads=2, head_dim=128, kv_dtype="e4m3", fp8_absmax_scales=True,
                       mask_kind="causal"),
    "d64_ps4": dict(prefix_lens=[1000, 250, 3100], qo_lens=[2, 7, 4], num_qo_heads=8, num_kv_heads=4,
                    head_dim=64, page_size=4, mask_kind="random", mask_density=0.5),
    # One request (the merge loads its first round of partials ahead of the
    # request table), with spare page-index capacity so that it covers only
    # some of the slices, and up to 256 slices per head (several rounds).
    "one_bf16": dict(prefix_lens=[5000], qo_lens=[9], num_qo_heads=32, num_kv_heads=8, head_dim=128,
                     mask_kind="tree", extra_indices=40),
    "one_d64_ps4": dict(prefix_lens=[3000], qo_lens=[17], num_qo_heads=16, num_kv_heads=2,
                        head_dim=64, page_size=4, extra_indices=3),
    "one_e4m3": dict(prefix_lens=[6000], qo_lens=[5], num_qo_heads=16, num_kv_heads=4, head_dim=128,
                     kv_dtype="e4m3", fp8_absmax_scales=True, extra_indices=7),
}


@pytest.mark.parametrize("name", sorted(SLICE_CASES))
@pytest.mark.parametrize("num_cus", [1, 8, 40, 256, 2048])
def test_balanced_slices_match_oracle(gpu_lib, name, num_cus):
    # The slice count follows the CU count the plan is made for, so these cover
    # one slice (direct), a few long slices spanning several requests, and more
    # slices than pages (empty slices).
    p = make_case(91, **SLICE_CASES[name])
    plan = gpu_lib.vat_plan(_problem(gpu_lib, p, num_cus=num_cus))
    say(f"[slices {name} num_cus={num_cus}] slices={plan.slices} direct={plan.direct}")
    assert plan.slices >= 1
    out, lse = run_gpu(gpu_lib, p, num_cus=num_cus)
    compare(p, *to_f64(out, lse), *oracle_of(p), what=f"{name} cus {num_cus}")


def test_long_request_moves_the_page_window(gpu_lib):
    # One request longer than the in-LDS page window (2048 pages of 16 keys)
    # processed whole by one workgroup.
    p = make_case(92, prefix_lens=[36000], qo_lens=[5], num_qo_heads=8, num_kv_heads=1,
                  head_dim=128, mask_kind="tree")
    for num_cus, chunk in ((1, -1), (256, 0)):
        say(f"[long request num_cus={num_cus} chunk={chunk}]")
        out, lse = run_gpu(gpu_lib, p, num_cus=num_cus, chunk_keys=chunk)
        compare(p, *to_f64(out, lse), *oracle_of(p), what="long request")


# ---------------------------------------------------------------- paired row blocks

# Plans with many row blocks per CU pair them: one workgroup runs blocks
# RB - 1 - k and k of its (item, KV head) as two segments of one ring. A small
# planned CU count forces that here. Shorter requests have fewer blocks, so the
# longer block of a pair can be empty while the shorter one is not.
PAIR_CASES = {
    "causal_mixed_L": dict(prefix_lens=[0, 35, 200], qo_lens=[300, 129, 40], num_qo_heads=16,
                           num_kv_heads=2, head_dim=128),
    "fp8": dict(prefix_lens=[64, 0], qo_lens=[90, 200], num_qo_heads=16, num_kv_heads=2,
                head_dim=128, kv_dtype="e4m3", fp8_absmax_scales=True),
    "d64": dict(prefix_lens=[10, 300], qo_lens=[150, 70], num_qo_heads=24, num_kv_heads=3,
                head_dim=64),
    "tree_mask": dict(prefix_lens=[500, 100], qo_lens=[48, 33], num_qo_heads=64, num_kv_heads=8,
                      head_dim=128, mask_kind="tree"),
}


@pytest.mark.parametrize("name", sorted(PAIR_CASES))
@pytest.mark.parametrize("chunk", [-1, 64])
def test_paired_row_blocks_match_oracle(gpu_lib, name, chunk):
    p = make_case(94, **PAIR_CASES[name])
    plan = gpu_lib.vat_plan(_problem(gpu_lib, p, num_cus=4, chunk_keys=chunk))
    say(f"[paired blocks {name} chunk={chunk}] row_blocks={plan.row_blocks} "
        f"block_order={plan.block_order} direct={plan.direct} grid={plan.grid_x}")
    assert plan.block_order == 2 and plan.row_blocks > 1
    out, lse = run_gpu(gpu_lib, p, num_cus=4, chunk_keys=chunk)
    compare(p, *to_f64(out, lse), *oracle_of(p), what=f"paired {name} chunk {chunk}")


# ---------------------------------------------------------------- graph capture


def test_hip_graph_capture_and_replay(gpu_lib):
    p = make_config(2)
    t = to_device(p)
    # Warm up (loads the library, plans, allocates the workspace) outside capture.
    ws_size = gpu_lib.vat_workspace_size(_problem(gpu_lib, p))
    ws = torch.empty(ws_size, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[0], t["q"].shape[1], dtype=torch.float32, device="cuda")
    call = dict(mask=t["mask"], mask_indptr=t["mask_indptr"], sm_scale=p.sm_scale,
                k_scale=p.k_scale, v_scale=p.v_scale, max_qo_len=p.max_qo_len, out=out, lse=lse,
                workspace=ws)
    args = (t["q"], t["k_cache"], t["v_cache"], t["kv_indptr"], t["kv_indices"],
            t["last_page_len"], t["qo_indptr"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gpu_lib.verify_attention(*args, **call)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_lib.verify_attention(*args, **call)
    # New inputs in the same buffers, then replay several times with eager work between.
    p2 = make_config(2, seed=99)
    t2 = to_device(p2)
    for name in ("q", "k_cache", "v_cache", "kv_indices"):
        t[name].copy_(t2[name])
    ref_o, ref_l = oracle_of(p2)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        compare(p2, *to_f64(out, lse), ref_o, ref_l, what=f"graph replay {rep}")
        eager_o, eager_l = gpu_lib.verify_attention(*args, **{**call, "out": None, "lse": None,
                                                               "workspace": None})
        torch.cuda.synchronize()
        assert torch.equal(eager_o.view(torch.int16), out.view(torch.int16))
