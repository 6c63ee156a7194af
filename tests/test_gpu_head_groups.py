"""GPU parity of the streaming kernel with several KV heads per workgroup:
fp8 e4m3 caches of D 128 where one workgroup reads the rows of two adjacent
KV heads (256-byte runs per key) or, when the head count is divisible by
four, of four (512-byte runs; twelve waves when each head has two row tiles).

Against the oracle at the parity tolerances: both head groupings, query-head
groups 1, 2 and 4 (one or two row tiles per head), draft lengths up to 32
rows per head, every power-of-two page size from 1 to 256, causal, tree and
random packed masks, requests without drafts, batches up to 64, slice counts
from one (every request written directly) to more slices than pages, and
slices longer than the page-id window; with RoPE (two heads per workgroup,
as RoPE plans take). Bit-exact: a page-pool permutation, and a HIP graph
replayed between eager calls.
"""

import numpy as np
import pytest
import torch

from tests.gpu_helpers import compare, oracle_of, run_gpu, say, to_device, to_f64
from oracle import verify_attention as oracle_va
from workloads import make_case, make_config, rope_cos_sin, rope_positions

pytestmark = pytest.mark.gpu


def _case(seed, B, G, Lmax, ps, mask_kind, prefix_hi=600, empty=False, kv="e4m3", hkv=8, **kw):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(1, Lmax + 1, size=B)]
    if empty and B > 2:
        lens[1] = 0
    prefixes = [int(x) for x in rng.integers(0, prefix_hi + 1, size=B)]
    return make_case(seed, prefix_lens=prefixes, qo_lens=lens, num_qo_heads=hkv * G,
                     num_kv_heads=hkv, head_dim=128, page_size=ps, q_dtype="bf16",
                     kv_dtype=kv, mask_kind=mask_kind, fp8_absmax_scales=(kv == "e4m3"),
                     max_qo_len=Lmax, **kw)


CASES = [
    # seed, batch, group, max L, page size, mask, num_cus, KV heads
    (1, 3, 4, 8, 16, "causal", 0, 8),
    (2, 5, 4, 8, 1, "tree", 0, 8),
    (3, 7, 2, 16, 4, "random", 0, 8),
    (4, 2, 1, 32, 64, "tree", 0, 8),
    (5, 4, 4, 8, 256, "causal", 0, 8),
    (6, 64, 4, 8, 16, "causal", 0, 8),
    (7, 6, 2, 5, 8, "chain", 0, 8),
    (8, 3, 4, 4, 2, "full", 0, 8),
    (9, 5, 4, 8, 16, "tree", 1, 8),
    (10, 5, 4, 8, 16, "tree", 3, 8),
    (11, 9, 1, 16, 32, "random", 7, 8),
    (12, 2, 4, 1, 16, "causal", 0, 8),
    (13, 12, 2, 8, 128, "tree", 40, 8),
    (14, 64, 4, 8, 16, "causal", 0, 4),
    (15, 5, 4, 8, 1, "tree", 0, 6),
    (16, 7, 2, 16, 4, "random", 0, 2),
    (17, 6, 4, 4, 16, "causal", 0, 6),
    (18, 9, 1, 16, 32, "random", 5, 6),
    (19, 40, 4, 8, 64, "tree", 0, 12),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c[0]}")
def test_head_group_kernel_matches_oracle(gpu_lib, case):
    seed, B, G, Lmax, ps, mask, cus, hkv = case
    p = _case(seed, B, G, Lmax, ps, mask, empty=seed % 2 == 0, hkv=hkv)
    t = to_device(p)
    prob = gpu_lib.problem_from_tensors(t["q"], t["k_cache"], t["kv_indptr"], t["kv_indices"],
                                        t["mask"], p.max_qo_len, num_cus=cus)
    plan = gpu_lib.vat_plan(prob)
    say(f"[head groups seed {seed}] B={B} Hkv={hkv} G={G} L<={Lmax} ps={ps} {mask} "
        f"cus={cus or 'device'} heads/wg={plan.heads_per_group} threads={plan.threads} "
        f"slices={plan.slices} direct={plan.direct}")
    assert plan.kernel == 1 and plan.heads_per_group == (4 if hkv % 4 == 0 else 2)
    out, lse = run_gpu(gpu_lib, p, tensors=t, num_cus=cus)
    compare(p, *to_f64(out, lse), *oracle_of(p), what=f"head groups seed {seed}")


@pytest.mark.parametrize("hkv", [8, 6])
def test_head_group_slices_longer_than_the_page_window(gpu_lib, oracle_pool, hkv):
    # Two slices of about 2,600 pages each (CU count = 2 x head groups):
    # more page ids than the 2,048-entry window, so each workgroup moves its
    # window once.
    hp = 4 if hkv % 4 == 0 else 2
    cus = 2 * hkv // hp
    p = make_case(21, prefix_lens=[41000, 42000], qo_lens=[8, 5], num_qo_heads=4 * hkv,
                  num_kv_heads=hkv, head_dim=128, page_size=16, kv_dtype="e4m3", mask_kind="tree",
                  fp8_absmax_scales=True, max_qo_len=8)
    t = to_device(p)
    plan = gpu_lib.vat_plan(gpu_lib.problem_from_tensors(t["q"], t["k_cache"], t["kv_indptr"],
                                                         t["kv_indices"], t["mask"], 8, num_cus=cus))
    say(f"[head groups, window moves] Hkv={hkv} pages={int(p.kv_indptr[-1])} slices={plan.slices}")
    assert plan.heads_per_group == hp and int(p.kv_indptr[-1]) / plan.slices > 2048
    out, lse = run_gpu(gpu_lib, p, tensors=t, num_cus=cus)
    compare(p, *to_f64(out, lse), *oracle_pool.run(p), what=f"head groups window moves Hkv {hkv}")


@pytest.mark.parametrize("hkv", [8, 6])
def test_head_group_page_permutation_is_bitwise_invariant(gpu_lib, hkv):
    p = _case(31, 6, 4, 8, 16, "tree", hkv=hkv)
    t = to_device(p)
    o0, l0 = run_gpu(gpu_lib, p, tensors=t)
    perm = np.random.default_rng(5).permutation(p.num_pages)
    k2, v2 = np.empty_like(p.k_cache), np.empty_like(p.v_cache)
    k2[perm], v2[perm] = p.k_cache, p.v_cache
    idx = p.kv_indices.copy()
    used = int(p.kv_indptr[-1])
    idx[:used] = perm[p.kv_indices[:used]]
    p.k_cache, p.v_cache, p.kv_indices = k2, v2, idx
    o1, l1 = run_gpu(gpu_lib, p)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)


def test_head_group_graph_replay_is_bitwise_eager(gpu_lib):
    p = make_config(5)
    t = to_device(p)
    kw = dict(mask=t["mask"], mask_indptr=t["mask_indptr"], sm_scale=p.sm_scale,
              k_scale=p.k_scale, v_scale=p.v_scale, max_qo_len=p.max_qo_len)
    args = (t["q"], t["k_cache"], t["v_cache"], t["kv_indptr"], t["kv_indices"],
            t["last_page_len"], t["qo_indptr"])
    ws = torch.empty(gpu_lib.vat_workspace_size(gpu_lib.problem_from_tensors(
        t["q"], t["k_cache"], t["kv_indptr"], t["kv_indices"], None, p.max_qo_len)),
        dtype=torch.uint8, device="cuda")
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gpu_lib.verify_attention(*args, **kw, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_lib.verify_attention(*args, **kw, out=out, lse=lse, workspace=ws)
    eager_o, eager_l = gpu_lib.verify_attention(*args, **kw)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_o.view(torch.int16)), rep
        assert torch.equal(lse, eager_l), rep
        eager_o, eager_l = gpu_lib.verify_attention(*args, **kw)
        torch.cuda.synchronize()


ROPE_CASES = [
    # seed, batch, group, max L, page size, mask, KV heads
    (41, 5, 4, 8, 16, "tree", 8),
    (42, 7, 2, 16, 4, "causal", 6),
    (43, 12, 4, 8, 64, "random", 8),
    (44, 3, 1, 32, 1, "chain", 4),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=lambda c: f"seed{c[0]}")
def test_head_group_kernel_with_rope_matches_oracle(gpu_lib, case):
    # RoPE plans take two heads per workgroup (one row tile per wave).
    seed, B, G, Lmax, ps, mask, hkv = case
    p = _case(seed, B, G, Lmax, ps, mask, hkv=hkv)
    cs = rope_cos_sin(rope_positions(p), p.head_dim)
    t = to_device(p)
    prob = gpu_lib.problem_from_tensors(t["q"], t["k_cache"], t["kv_indptr"], t["kv_indices"],
                                        t["mask"], p.max_qo_len, rope=True)
    plan = gpu_lib.vat_plan(prob)
    say(f"[head groups, rope seed {seed}] B={B} Hkv={hkv} G={G} L<={Lmax} ps={ps} {mask} "
        f"heads/wg={plan.heads_per_group}")
    assert plan.kernel == 1 and plan.heads_per_group == 2
    out, lse = gpu_lib.verify_attention(
        t["q"], t["k_cache"], t["v_cache"], t["kv_indptr"], t["kv_indices"], t["last_page_len"],
        t["qo_indptr"], t["mask"], t["mask_indptr"], sm_scale=p.sm_scale, k_scale=p.k_scale,
        v_scale=p.v_scale, max_qo_len=p.max_qo_len,
        q_cos_sin=torch.from_numpy(np.ascontiguousarray(cs)).cuda())
    torch.cuda.synchronize()
    want = oracle_va(p.q, p.k_cache, p.v_cache, p.kv_indptr, p.kv_indices, p.last_page_len,
                     p.qo_indptr, p.mask, p.mask_indptr, sm_scale=p.sm_scale, k_scale=p.k_scale,
                     v_scale=p.v_scale, q_dtype=p.q_dtype, kv_dtype=p.kv_dtype, q_cos_sin=cs)
    compare(p, *to_f64(out, lse), *want, what=f"head groups rope seed {seed}")
