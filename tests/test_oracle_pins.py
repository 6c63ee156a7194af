"""Pins for the CPU oracle: facts that do not come from the oracle itself.

Each test names the passage or the mathematics it rests on: hand-worked tiny
cases, library routines (torch SDPA in float64, torch.logsumexp, torch's
bfloat16 / float8_e4m3fn casts), closed forms, and the invariants the pages
state. A plausible slip in the oracle -- a dropped scale, a wrong head map,
a transposed mask, an off-by-one in the page arithmetic, causal aligned
top-left instead of bottom-right, a bad merge weight -- fails at least one.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (E4M3FN_TABLE, decode_bf16, merge_partials, unpack_mask_block,
                    verify_attention_partials)
from tests.layout_helpers import (causal_allowed, random_logical, run_oracle, scatter_problem,
                                  sdpa_reference)
from workloads import make_case, make_config, pack_mask_rows, tree_mask_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- element decoding


def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_fixed_points_from_the_format():
    # OCP FP8 E4M3: bias 7, 3 mantissa bits, subnormals at exponent 0, S.1111.111 NaN.
    assert E4M3FN_TABLE[0x38] == 1.0
    assert E4M3FN_TABLE[0x7E] == 448.0
    assert E4M3FN_TABLE[0x08] == 2.0 ** -6
    assert E4M3FN_TABLE[0x01] == 2.0 ** -9
    assert E4M3FN_TABLE[0x07] == 7 * 2.0 ** -9
    assert E4M3FN_TABLE[0x80] == 0.0 and math.copysign(1.0, E4M3FN_TABLE[0x80]) == -1.0
    assert np.isnan(E4M3FN_TABLE[0x7F]) and np.isnan(E4M3FN_TABLE[0xFF])
    assert E4M3FN_TABLE[0xFE] == -448.0


def test_e4m3fn_all_codes_match_torch_cast():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(E4M3FN_TABLE), nan)
    assert np.array_equal(E4M3FN_TABLE[~nan], ref[~nan])


# ---------------------------------------------------------------- mask packing golden


def _golden_cases():
    cases = []
    with open(os.path.join(GOLDEN, "mask_bits.txt")) as f:
        for line in f:
            if not line.startswith("case"):
                continue
            fields = [x.strip() for x in line.split("|")]
            L = int(fields[1].split()[1])
            parents = [int(x) for x in fields[2].split()[1:]]
            data = bytes(int(x, 16) for x in fields[3].split()[1:])
            cases.append((fields[0].split()[1], L, parents, data))
    return cases


@pytest.mark.parametrize("name,L,parents,data", _golden_cases())
def test_mask_packing_matches_hand_worked_bytes(name, L, parents, data):
    rows = tree_mask_rows(parents)
    packed, indptr = pack_mask_rows([rows])
    assert bytes(packed[: indptr[1]]) == data, name
    back = unpack_mask_block(np.frombuffer(data, dtype=np.uint8), 0, L)
    assert np.array_equal(back, rows), name


# ---------------------------------------------------------------- tiny cases by hand


def test_tiny_causal_by_hand():
    # One request, one head, D = 1, page size 1; one prefix key then two drafts.
    # q = [1, 0.5]; keys k = [1, 2, 3]; values v = [10, 20, 30]; sm_scale = 1.
    # Draft 0 sees keys {0, 1}; draft 1 sees keys {0, 1, 2} (bottom-right causal).
    q_log = [np.array([[[1.0]], [[0.5]]])]
    k_log = [np.array([[[1.0]], [[2.0]], [[3.0]]])]
    v_log = [np.array([[[10.0]], [[20.0]], [[30.0]]])]
    p = scatter_problem(q_log, k_log, v_log, page_size=1, q_dtype="f32", kv_dtype="f32",
                        sm_scale=1.0, perm_seed=5)
    out, lse = run_oracle(p)
    e = math.e
    z0 = e ** 1 + e ** 2
    z1 = e ** 0.5 + e ** 1.0 + e ** 1.5
    assert out[0, 0, 0] == pytest.approx((10 * e + 20 * e ** 2) / z0, rel=1e-14)
    assert lse[0, 0] == pytest.approx(math.log(z0), rel=1e-14)
    assert out[1, 0, 0] == pytest.approx((10 * e ** 0.5 + 20 * e + 30 * e ** 1.5) / z1, rel=1e-14)
    assert lse[1, 0] == pytest.approx(math.log(z1), rel=1e-14)


def test_tiny_tree_gqa_scales_pages_by_hand():
    # Two query heads on one KV head (G = 2), D = 2, page size 2, pages permuted.
    # prefix = 2 keys, then drafts with tree parents [-1, 0, 0]:
    #   draft 0 sees keys {0, 1, 2}; draft 1 sees {0, 1, 2, 3}; draft 2 sees {0, 1, 2, 4}.
    # sm_scale 0.5 * k_scale 2 = logit scale 1; v_scale 3 multiplies the output.
    k = np.array([[1, 0], [0, 1], [1, 1], [-1, 0], [0, -1]], dtype=float)
    v = np.array([[1, 2], [3, 4], [5, 6], [7, 8], [9, 10]], dtype=float)
    q = np.array([[[1, 0], [0, 1]], [[1, 1], [0, 0]], [[-1, 2], [2, -1]]], dtype=float)
    visible = {0: [0, 1, 2], 1: [0, 1, 2, 3], 2: [0, 1, 2, 4]}
    p = scatter_problem([q], [k[:, None, :]], [v[:, None, :]], page_size=2, q_dtype="f32",
                        kv_dtype="f32", mask_blocks=[tree_mask_rows([-1, 0, 0])],
                        sm_scale=0.5, k_scale=2.0, v_scale=3.0, perm_seed=11)
    out, lse = run_oracle(p)
    for t in range(3):
        for hq in range(2):
            keys = visible[t]
            w = [math.exp(float(q[t, hq] @ k[n])) for n in keys]
            z = sum(w)
            want = [3.0 * sum(wi * v[n, d] for wi, n in zip(w, keys)) / z for d in range(2)]
            assert out[t, hq] == pytest.approx(want, rel=1e-13), (t, hq)
            assert lse[t, hq] == pytest.approx(math.log(z), rel=1e-13), (t, hq)


def test_fully_masked_row_gives_zero_and_minus_inf():
    # A custom mask row with no bit set and no prefix: nothing to attend to.
    rng = np.random.default_rng(0)
    q_log, k_log, v_log = random_logical(rng, [0], [3], 1, 1, 4)
    block = np.array([[1, 0, 0], [0, 0, 0], [1, 1, 1]], dtype=bool)
    p = scatter_problem(q_log, k_log, v_log, page_size=2, q_dtype="f32", kv_dtype="f32",
                        mask_blocks=[block])
    out, lse = run_oracle(p)
    assert np.all(out[1] == 0.0) and lse[1, 0] == -np.inf
    assert np.isfinite(lse[0, 0]) and np.isfinite(lse[2, 0])


# ---------------------------------------------------------------- library cross-check


@pytest.mark.parametrize("seed,kv_dtype,q_dtype,mask_kind", [
    (1, "f32", "f32", "causal"),
    (2, "bf16", "bf16", "causal"),
    (3, "bf16", "bf16", "tree"),
    (4, "e4m3", "bf16", "causal"),
    (5, "e4m3", "bf16", "random"),
    (6, "f32", "f32", "tree"),
])
def test_matches_torch_sdpa_float64(seed, kv_dtype, q_dtype, mask_kind):
    rng = np.random.default_rng(seed)
    prefixes = [int(x) for x in rng.integers(0, 40, size=3)]
    lens = [int(x) for x in rng.integers(1, 7, size=3)]
    Hq, Hkv, D = 6, 2, 8
    q_log, k_log, v_log = random_logical(rng, prefixes, lens, Hq, Hkv, D, kv_dtype, q_dtype)
    blocks = None
    allowed = []
    if mask_kind == "tree":
        blocks = []
        for L in lens:
            par = [-1] + [int(rng.integers(0, i)) for i in range(1, L)]
            blocks.append(tree_mask_rows(par))
    elif mask_kind == "random":
        blocks = [rng.random((L, L)) < 0.6 for L in lens]
    for b, (pfx, L) in enumerate(zip(prefixes, lens)):
        if blocks is None:
            allowed.append(causal_allowed(pfx, L))
        else:
            a = np.zeros((L, pfx + L), dtype=bool)
            a[:, :pfx] = True
            a[:, pfx:] = blocks[b]
            allowed.append(a)
    sm, ks, vs = 0.37, 1.25, 0.75
    p = scatter_problem(q_log, k_log, v_log, page_size=4, q_dtype=q_dtype, kv_dtype=kv_dtype,
                        mask_blocks=blocks, sm_scale=sm, k_scale=ks, v_scale=vs, perm_seed=seed)
    out, lse = run_oracle(p)
    ref_o, ref_l = sdpa_reference(q_log, k_log, v_log, allowed, scale=sm * ks, v_scale=vs)
    t0 = 0
    for b, L in enumerate(lens):
        ro, rl = ref_o[b], ref_l[b]
        empty = ~allowed[b].any(axis=1)
        for t in range(L):
            if empty[t]:
                assert np.all(out[t0 + t] == 0) and np.all(lse[t0 + t] == -np.inf)
                continue
            np.testing.assert_allclose(out[t0 + t], ro[t], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(lse[t0 + t], rl[t], rtol=1e-12, atol=1e-12)
        t0 += L


# ---------------------------------------------------------------- invariants the pages state


def test_chain_mask_equals_causal_bitwise():
    # A chain-shaped tree mask is the causal mask (FlashInfer tree-attention page:
    # a triu(-inf) mask is equivalent to causal=True).
    rng = np.random.default_rng(7)
    q_log, k_log, v_log = random_logical(rng, [5, 0, 19], [4, 3, 6], 4, 2, 8)
    chain = [tree_mask_rows(list(range(-1, L - 1))) for L in (4, 3, 6)]
    pc = scatter_problem(q_log, k_log, v_log, page_size=4, q_dtype="f32", kv_dtype="f32")
    pm = scatter_problem(q_log, k_log, v_log, page_size=4, q_dtype="f32", kv_dtype="f32",
                         mask_blocks=chain, mask_pad_bytes=3)
    oc, lc = run_oracle(pc)
    om, lm = run_oracle(pm)
    assert np.array_equal(oc, om) and np.array_equal(lc, lm)


def test_tree_row_equals_chain_over_its_path():
    # Turning one draft path into its own request (FlashInfer tree-attention page:
    # one draft sequence per batch entry) gives the tree row of the path's leaf.
    rng = np.random.default_rng(8)
    parents = [-1, 0, 0, 1, 3, 2, 0]
    L = len(parents)
    prefix = 9
    q_log, k_log, v_log = random_logical(rng, [prefix], [L], 2, 1, 8)
    pt = scatter_problem(q_log, k_log, v_log, page_size=4, q_dtype="f32", kv_dtype="f32",
                         mask_blocks=[tree_mask_rows(parents)])
    ot, lt = run_oracle(pt)
    for t in range(L):
        path = []
        node = t
        while node >= 0:
            path.append(node)
            node = parents[node]
        path = path[::-1]
        keys = list(range(prefix)) + [prefix + j for j in path]
        qc = [q_log[0][path]]
        kc = [k_log[0][keys]]
        vc = [v_log[0][keys]]
        pc = scatter_problem(qc, kc, vc, page_size=3, q_dtype="f32", kv_dtype="f32")
        oc, lc = run_oracle(pc)
        assert np.array_equal(oc[-1], ot[t]) and np.array_equal(lc[-1], lt[t]), t


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "e4m3"])
def test_paged_layout_equals_contiguous_bitwise(kv_dtype):
    # The page table only relocates keys (FlashInfer page, begin_forward docstring).
    rng = np.random.default_rng(9)
    prefixes, lens = [13, 40, 0], [3, 5, 2]
    q_log, k_log, v_log = random_logical(rng, prefixes, lens, 4, 2, 8, kv_dtype, "f32")
    ref = None
    for ps, seed in [(1, None), (4, 3), (16, 4), (64, 5), (8, None)]:
        p = scatter_problem(q_log, k_log, v_log, page_size=ps, q_dtype="f32", kv_dtype=kv_dtype,
                            perm_seed=seed)
        res = run_oracle(p)
        if ref is None:
            ref = res
        else:
            assert np.array_equal(res[0], ref[0]) and np.array_equal(res[1], ref[1]), ps


def test_gqa_equals_expanded_heads_bitwise():
    # GQA = MHA with each KV head repeated over its group of consecutive query
    # heads (vLLM page "[Performance] Support MQA/GQA in prefill stage by using
    # FlashAttention": key/value expanded per group).
    rng = np.random.default_rng(10)
    q_log, k_log, v_log = random_logical(rng, [11, 4], [3, 2], 8, 2, 8)
    pg = scatter_problem(q_log, k_log, v_log, page_size=4, q_dtype="f32", kv_dtype="f32")
    k_exp = [np.repeat(k, 4, axis=1) for k in k_log]
    v_exp = [np.repeat(v, 4, axis=1) for v in v_log]
    pe = scatter_problem(q_log, k_exp, v_exp, page_size=4, q_dtype="f32", kv_dtype="f32")
    og, lg = run_oracle(pg)
    oe, le = run_oracle(pe)
    assert np.array_equal(og, oe) and np.array_equal(lg, le)


def test_single_query_is_decode():
    # L = 1: plain single-query decode over all kv_len keys (library SDPA).
    rng = np.random.default_rng(12)
    q_log, k_log, v_log = random_logical(rng, [30, 1], [1, 1], 4, 4, 16)
    p = scatter_problem(q_log, k_log, v_log, page_size=8, q_dtype="f32", kv_dtype="f32",
                        sm_scale=0.25)
    out, lse = run_oracle(p)
    for b in range(2):
        n = k_log[b].shape[0]
        ro, rl = sdpa_reference([q_log[b]], [k_log[b]], [v_log[b]],
                                [np.ones((1, n), dtype=bool)], scale=0.25)
        np.testing.assert_allclose(out[b], ro[0][0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b], rl[0][0], rtol=1e-13)


def test_causal_verify_equals_decodes_with_interpolated_lengths():
    # vLLM "[WIP] Support for cached multi-query attention towards speculative
    # decoding": draft t is a single-query decode whose sequence length runs
    # from the context length up by one per draft.
    rng = np.random.default_rng(13)
    prefix, L = 17, 5
    q_log, k_log, v_log = random_logical(rng, [prefix], [L], 4, 2, 8)
    pv = scatter_problem(q_log, k_log, v_log, page_size=4, q_dtype="f32", kv_dtype="f32")
    ov, lv = run_oracle(pv)
    for t in range(L):
        n = prefix + t + 1
        pd = scatter_problem([q_log[0][t:t + 1]], [k_log[0][:n]], [v_log[0][:n]], page_size=4,
                             q_dtype="f32", kv_dtype="f32")
        od, ld = run_oracle(pd)
        assert np.array_equal(od[0], ov[t]) and np.array_equal(ld[0], lv[t]), t


def test_any_split_merged_by_lse_equals_direct():
    # flashmap page, _verify_merge_kernel: partials weighted by their share of
    # the softmax mass reproduce the unsplit result, empty parts included.
    rng = np.random.default_rng(14)
    prefixes, lens = [50, 3, 0], [4, 2, 3]
    q_log, k_log, v_log = random_logical(rng, prefixes, lens, 4, 2, 8)
    blocks = [tree_mask_rows([-1, 0, 1, 0]), tree_mask_rows([-1, 0]),
              np.array([[1, 0, 0], [0, 0, 0], [1, 0, 1]], dtype=bool)]
    p = scatter_problem(q_log, k_log, v_log, page_size=4, q_dtype="f32", kv_dtype="f32",
                        mask_blocks=blocks)
    out, lse = run_oracle(p)

    def splits(b, kv_len):
        cuts = sorted(set([0, kv_len] + [int(x) for x in rng.integers(0, kv_len + 1, size=4)]))
        ranges = [(lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:])]
        return ranges + [(kv_len, kv_len), (0, 0)]

    parts = verify_attention_partials(p.q, p.k_cache, p.v_cache, p.kv_indptr, p.kv_indices,
                                      p.last_page_len, p.qo_indptr, p.mask, p.mask_indptr,
                                      key_splits=splits, sm_scale=p.sm_scale, q_dtype="f32",
                                      kv_dtype="f32")
    t0 = 0
    for b, L in enumerate(lens):
        mo, ml = merge_partials(parts[b])
        np.testing.assert_allclose(mo, out[t0:t0 + L], rtol=1e-12, atol=1e-13)
        fin = np.isfinite(lse[t0:t0 + L])
        assert np.array_equal(np.isfinite(ml), fin)
        np.testing.assert_allclose(ml[fin], lse[t0:t0 + L][fin], rtol=1e-13, atol=1e-13)
        t0 += L


@pytest.mark.parametrize("masked_value", [float("-inf"), -5e4])
def test_additive_float_masks_equal_boolean_mask(masked_value):
    # FlashInfer tree-attention page: -inf or -5e4 at masked entries and 0 elsewhere
    # is a correct custom mask; triu(-inf) equals causal.
    rng = np.random.default_rng(15)
    L, prefix, Hq, D = 6, 0, 2, 8
    q_log, k_log, v_log = random_logical(rng, [prefix], [L], Hq, Hq, D)
    add = torch.triu(torch.full((L, L), masked_value, dtype=torch.float64), diagonal=1)
    qt = torch.from_numpy(q_log[0].transpose(1, 0, 2).copy())
    kt = torch.from_numpy(k_log[0].transpose(1, 0, 2).copy())
    vt = torch.from_numpy(v_log[0].transpose(1, 0, 2).copy())
    ref = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None],
                                                           attn_mask=add, scale=0.5)[0]
    p = scatter_problem(q_log, k_log, v_log, page_size=4, q_dtype="f32", kv_dtype="f32",
                        sm_scale=0.5)
    out, _ = run_oracle(p)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- closed forms


def test_zero_query_gives_mean_of_visible_values_and_log_count():
    rng = np.random.default_rng(16)
    prefixes, lens = [7, 0], [3, 4]
    q_log, k_log, v_log = random_logical(rng, prefixes, lens, 2, 1, 4)
    q_log = [np.zeros_like(x) for x in q_log]
    parents = [[-1, 0, 0], [-1, 0, 1, 1]]
    blocks = [tree_mask_rows(p) for p in parents]
    p = scatter_problem(q_log, k_log, v_log, page_size=4, q_dtype="f32", kv_dtype="f32",
                        mask_blocks=blocks)
    out, lse = run_oracle(p)
    t0 = 0
    for b in range(2):
        for t in range(lens[b]):
            keys = list(range(prefixes[b])) + [prefixes[b] + j for j in range(lens[b])
                                               if blocks[b][t, j]]
            want = v_log[b][keys, 0, :].mean(axis=0)
            for hq in range(2):
                np.testing.assert_allclose(out[t0 + t, hq], want, rtol=1e-13, atol=1e-14)
                assert lse[t0 + t, hq] == pytest.approx(math.log(len(keys)), rel=1e-14)
        t0 += lens[b]


def test_single_visible_key_returns_its_value_and_logit():
    rng = np.random.default_rng(17)
    q_log, k_log, v_log = random_logical(rng, [0], [3], 1, 1, 4)
    block = np.array([[1, 0, 0], [0, 1, 0], [0, 0, 1]], dtype=bool)
    p = scatter_problem(q_log, k_log, v_log, page_size=2, q_dtype="f32", kv_dtype="f32",
                        mask_blocks=[block], sm_scale=0.3, k_scale=2.0, v_scale=1.5)
    out, lse = run_oracle(p)
    for t in range(3):
        np.testing.assert_allclose(out[t, 0], 1.5 * v_log[0][t, 0], rtol=1e-15)
        assert lse[t, 0] == pytest.approx(0.6 * float(q_log[0][t, 0] @ k_log[0][t, 0]), rel=1e-14)


def test_constant_values_and_scales():
    rng = np.random.default_rng(18)
    q_log, k_log, v_log = random_logical(rng, [21], [4], 4, 2, 8)
    vconst = [np.full_like(v_log[0], 0.625)]
    p = scatter_problem(q_log, k_log, vconst, page_size=4, q_dtype="f32", kv_dtype="f32")
    out, _ = run_oracle(p)
    np.testing.assert_allclose(out, 0.625, rtol=1e-14)
    base = scatter_problem(q_log, k_log, v_log, page_size=4, q_dtype="f32", kv_dtype="f32",
                           sm_scale=0.5, k_scale=2.0, v_scale=1.0)
    swap = scatter_problem(q_log, k_log, v_log, page_size=4, q_dtype="f32", kv_dtype="f32",
                           sm_scale=1.0, k_scale=1.0, v_scale=2.0)
    ob, lb = run_oracle(base)
    os_, ls = run_oracle(swap)
    assert np.array_equal(2.0 * ob, os_)  # only sm_scale*k_scale matters; v_scale scales out
    assert np.array_equal(lb, ls)


def test_poisoned_unused_slots_never_change_the_result():
    p1 = make_case(21, prefix_lens=[30, 3], qo_lens=[3, 2], num_qo_heads=4, num_kv_heads=2,
                   head_dim=8, q_dtype="f32", kv_dtype="f32", mask_kind="tree", poison=True)
    p2 = make_case(21, prefix_lens=[30, 3], qo_lens=[3, 2], num_qo_heads=4, num_kv_heads=2,
                   head_dim=8, q_dtype="f32", kv_dtype="f32", mask_kind="tree", poison=False)
    assert np.isnan(p1.k_cache).any() and not np.isnan(p2.k_cache).any()
    o1, l1 = run_oracle(p1)
    o2, l2 = run_oracle(p2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.isfinite(o1).all()


# ---------------------------------------------------------------- workload recipes


def test_config1_layout_matches_its_statement():
    p = make_config(1)
    assert p.num_pages == 32 and p.page_size == 16
    assert list(p.kv_indptr) == [0, 3, 10] and list(p.last_page_len) == [9, 8]
    assert list(p.qo_indptr) == [0, 4, 8] and p.mask is None
    assert p.sm_scale == 0.125 and p.q.dtype == np.float32
    assert len(set(p.kv_indices.tolist())) == 10


def test_generator_is_deterministic():
    from workloads import problem_sha256

    a = make_case(3, prefix_lens=[9, 20], qo_lens=[3, 5], num_qo_heads=4, num_kv_heads=1,
                  head_dim=16, mask_kind="tree")
    b = make_case(3, prefix_lens=[9, 20], qo_lens=[3, 5], num_qo_heads=4, num_kv_heads=1,
                  head_dim=16, mask_kind="tree")
    assert problem_sha256(a) == problem_sha256(b)
    c = make_case(4, prefix_lens=[9, 20], qo_lens=[3, 5], num_qo_heads=4, num_kv_heads=1,
                  head_dim=16, mask_kind="tree")
    assert problem_sha256(a) != problem_sha256(c)
