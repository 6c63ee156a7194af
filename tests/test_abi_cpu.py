"""The C ABI without a GPU: symbols, host validation and the shape-only planner.

Every call here fails (or plans) before anything reaches the HIP runtime, so
the library is loaded and exercised on a machine with no GPU. Problems pass
num_cus > 0 so the planner never queries a device.
"""

import ctypes
import math
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

from paged_kv_gqa_planner_amd import binding as B
from workloads import make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "verify_attention.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libvat.so not built (run __graft_entry__.build())")
    return B.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:vat_status_t|const char\*|int32_t)\s+(\w+)\s*\(", text,
                                 flags=re.M)))


def test_library_exports_every_header_function(lib):
    names = header_functions()
    assert {"verify_attention", "vat_plan", "vat_workspace_size", "vat_launch_partial",
            "vat_launch_merge", "vat_append_kv", "vat_status_string",
            "vat_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.vat_abi_version() == 5


def test_status_strings(lib):
    for code in range(7):
        assert lib.vat_status_string(code).decode()
    assert lib.vat_status_string(99).decode() == "unknown status"


def problem_of(p, **kw):
    fields = dict(batch=p.batch, num_qo_heads=p.num_qo_heads, num_kv_heads=p.num_kv_heads,
                  head_dim=p.head_dim, page_size=p.page_size, num_pages=p.num_pages,
                  num_kv_indices=len(p.kv_indices), num_qo_tokens=p.num_tokens,
                  max_qo_len=p.max_qo_len, q_dtype={"f32": 0, "bf16": 1}[p.q_dtype],
                  kv_dtype={"f32": 0, "bf16": 1, "e4m3": 2}[p.kv_dtype],
                  has_mask=p.mask is not None,
                  num_mask_bytes=0 if p.mask is None else len(p.mask), num_cus=256)
    fields.update(kw)
    return B.make_problem(**fields)


def base_problem(**kw):
    f = dict(batch=2, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=16, num_pages=64,
             num_kv_indices=40, num_qo_tokens=10, max_qo_len=5, q_dtype=1, kv_dtype=1, has_mask=0,
             num_mask_bytes=0, num_cus=256, chunk_keys=-1)
    f.update(kw)
    return B.make_problem(**f)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5, 6, 7])
def test_plans_for_the_workloads(lib, cid):
    p = make_config(cid, prefix=32768 if cid == 3 else 4096)
    plan = B.vat_plan(problem_of(p))
    G = p.num_qo_heads // p.num_kv_heads
    assert plan.group == G and plan.rows == G * p.max_qo_len
    assert plan.rows_per_block * plan.row_blocks >= plan.rows
    if plan.block_order:
        groups = plan.num_chunk_ids * p.num_kv_heads
        w = -(-plan.row_blocks // 2) if plan.block_order == 2 else plan.row_blocks
        assert plan.grid_y == 1
        assert plan.grid_x == 8 * w * -(-groups // 8)
    else:
        hp = plan.heads_per_group
        assert plan.grid_y == p.num_kv_heads // hp * plan.row_blocks
    if plan.slices:
        # Balanced slices: one workgroup per (slice, KV head group), CU-filling.
        hp = plan.heads_per_group
        assert plan.kernel == 1 and plan.chunk_keys == 0
        assert plan.slices == max(1, 256 // (p.num_kv_heads // hp)) == plan.grid_x
        assert plan.num_chunk_ids == plan.slices + p.batch
    else:
        assert plan.chunk_keys % 16 == 0 and plan.chunk_keys > 0
        total_keys = len(p.kv_indices) * p.page_size
        assert plan.num_chunk_ids == total_keys // plan.chunk_keys + p.batch
    assert plan.lds_bytes <= 160 * 1024
    if cid == 1:
        assert plan.kernel == 0 and plan.slices == 0  # fp32 caches take the row-tiled kernel
    elif cid == 4:
        # Prefill: the streaming kernel in row blocks of 256 rows, whole requests.
        assert plan.kernel == 1 and plan.direct == 1 and plan.workspace_bytes == 0
        assert plan.rows_per_block == 256 and plan.row_blocks == 32 and plan.slices == 0
        # Two row tiles per wave: two 64 KB stages of 128 keys.
        assert plan.row_tiles_per_wave == 2 and plan.stages == 2
        assert plan.lds_bytes == 2 * 64 * 1024 + 2048 * 4
    elif cid == 7:
        # Wide trees: 512 rows per KV head in two blocks, chunked prefixes.
        assert plan.kernel == 1 and plan.rows_per_block == 256 and plan.row_blocks == 2
        assert plan.slices == 0 and plan.block_order == 1
        assert plan.row_tiles_per_wave == 2 and plan.stages == 2
    elif cid == 5:
        # fp8 of D 128, 32 rows per KV head, eight KV heads: four heads per
        # workgroup, one computing wave per head with both row tiles, four
        # DMA waves.
        assert plan.kernel == 1 and plan.heads_per_group == 4 and plan.row_tiles_per_wave == 2
        assert plan.rows_per_block == 32 and plan.waves_rows == 4 and plan.dma_waves == 4
        assert plan.slices == 128 and plan.grid_y == 2
    else:
        assert plan.kernel == 1 and plan.threads == 512 and plan.slices > 0
    if not plan.direct:
        parts = plan.num_chunk_ids * p.num_kv_heads * plan.row_blocks
        assert plan.workspace_bytes >= parts * plan.rows_per_block * (p.head_dim + 1) * 4
        assert plan.merge_grid > 0
        # Few partials per request: four rows per merge wave.
        assert plan.merge_rows == (4 if cid == 3 else 16)
        groups = plan.merge_grid // (p.batch * p.num_kv_heads * plan.row_blocks)
        assert groups == -(-plan.rows_per_block // plan.merge_rows)
    else:
        assert plan.merge_rows == 0


def test_plan_is_shape_only_and_deterministic(lib):
    a = B.vat_plan(base_problem()).as_dict()
    b = B.vat_plan(base_problem()).as_dict()
    assert a == b
    # Doubling the CU count never shortens the chunk the planner picks.
    c = B.vat_plan(base_problem(num_kv_indices=4000, num_cus=512)).as_dict()
    d = B.vat_plan(base_problem(num_kv_indices=4000, num_cus=256)).as_dict()
    assert c["chunk_keys"] <= d["chunk_keys"]


def test_full_row_masks_keep_one_row_tile_per_wave(lib):
    """Byte-row masks (layout 2) plan row blocks of at most 128 rows: the
    kernels that read them hold one 16-row tile per wave."""
    for G, L in [(4, 64), (8, 40), (2, 17)]:
        bits = B.vat_plan(base_problem(num_qo_heads=2 * G, max_qo_len=L, num_qo_tokens=2 * L,
                                       has_mask=1, num_mask_bytes=1024))
        rows = B.vat_plan(base_problem(num_qo_heads=2 * G, max_qo_len=L, num_qo_tokens=2 * L,
                                       has_mask=2, num_mask_bytes=100000))
        assert rows.row_tiles_per_wave == 1 and rows.rows_per_block <= 128
        assert rows.rows_per_block * rows.row_blocks >= G * L
        if G * L <= 128:
            assert rows.as_dict() == bits.as_dict()


def test_forced_chunk_and_direct(lib):
    assert B.vat_plan(base_problem(chunk_keys=0)).direct == 1
    p = B.vat_plan(base_problem(chunk_keys=48))
    assert p.chunk_keys == 48 and p.direct == 0
    assert B.vat_workspace_size(base_problem(chunk_keys=0)) == 0
    assert B.vat_workspace_size(base_problem(chunk_keys=48)) == p.workspace_bytes > 0


def _decode_block(L, row_blocks, num_ids, hkv, order=1):
    """Host restatement of the streaming kernel's one-dimensional block orders:
    the (work item, KV head, row block) triples workgroup L runs, in order
    (block order 2 pairs blocks RB - 1 - k and k), or None for padding."""
    w = (row_blocks + 1) // 2 if order == 2 else row_blocks
    q = (L & 7) + 8 * (L // (8 * w))
    if q >= num_ids * hkv:
        return None
    k = (L >> 3) % w
    blocks = [row_blocks - 1 - k]
    if order == 2 and k < row_blocks - 1 - k:
        blocks.append(k)
    return [(q % num_ids, q // num_ids, rb) for rb in blocks]


@pytest.mark.parametrize("cid,order", [(4, 2), (7, 1)])
def test_row_blocks_of_a_group_share_an_xcd(lib, cid, order):
    """Workgroup L runs on XCD L % 8. Every (item, head, row block) is run
    once, the row blocks of one (item, head) sit on one XCD and are launched
    within one round of workgroups, the XCDs get equal shares of groups (to
    one), and a group's longest row block comes first. Prefill (config 4) has
    enough blocks to pair them (order 2: longest with shortest); the wide tree
    (config 7) keeps one block per workgroup."""
    p = make_config(cid)
    plan = B.vat_plan(problem_of(p))
    assert plan.block_order == order and plan.row_blocks > 1
    w = (plan.row_blocks + 1) // 2 if order == 2 else plan.row_blocks
    seen = {}
    for L in range(plan.grid_x):
        d = _decode_block(L, plan.row_blocks, plan.num_chunk_ids, p.num_kv_heads, order)
        if d is None:
            continue
        if order == 2:
            # The pair's blocks add up to RB - 1: every workgroup gets an equal
            # share of a causal group's work.
            assert len(d) == 1 or d[0][2] + d[1][2] == plan.row_blocks - 1
        for t in d:
            assert t not in seen
            seen[t] = L
    assert len(seen) == plan.num_chunk_ids * p.num_kv_heads * plan.row_blocks
    per_xcd = [0] * 8
    for item in range(plan.num_chunk_ids):
        for h in range(p.num_kv_heads):
            Ls = [seen[(item, h, rb)] for rb in range(plan.row_blocks)]
            assert len({L % 8 for L in Ls}) == 1
            assert max(Ls) // (8 * w) == min(Ls) // (8 * w)
            assert seen[(item, h, plan.row_blocks - 1)] == min(Ls)
            per_xcd[Ls[0] % 8] += 1
    assert max(per_xcd) - min(per_xcd) <= 1


@pytest.mark.parametrize("batch,Hkv,G,L,prefix", [(4, 8, 8, 64, 8192), (2, 8, 8, 40, 30000),
                                                   (8, 4, 8, 48, 5000), (3, 8, 16, 20, 12345)])
def test_equal_requests_split_into_equal_cu_filling_chunks(lib, batch, Hkv, G, L, prefix):
    """Streaming chunk plans cut the average request into floor(CUs / (B Hkv RB))
    chunks of equal length (no remainder chunk), so equal requests fill the
    CUs at most once: a short remainder chunk would take a CU in the first
    round and push a full-length chunk into a second."""
    kv_len = prefix + L
    pages = -(-kv_len // 16)
    prob = B.make_problem(
        batch=batch, num_qo_heads=G * Hkv, num_kv_heads=Hkv, head_dim=128, page_size=16,
        num_pages=batch * pages, num_kv_indices=batch * pages, num_qo_tokens=batch * L,
        max_qo_len=L, q_dtype=1, kv_dtype=1, has_mask=0, num_cus=256)
    plan = B.vat_plan(prob)
    assert plan.kernel == 1 and plan.slices == 0 and plan.row_blocks > 1
    RB = plan.row_blocks
    want = max(1, 256 // (batch * Hkv * RB))
    chunks = -(-kv_len // plan.chunk_keys)
    assert chunks == want
    # The last chunk is not a short remainder: it holds more than half a chunk.
    assert kv_len - (chunks - 1) * plan.chunk_keys > plan.chunk_keys // 2
    assert batch * Hkv * RB * chunks <= 256


def test_chunk_ids_of_consecutive_requests_are_disjoint():
    # Host-side check of the id layout the kernels use: request b's chunks are
    # start_b .. start_b + ceil(kv_len_b / C) - 1 with
    # start_b = floor(kv_indptr[b] * page_size / C) + b.
    rng = np.random.default_rng(0)
    for _ in range(300):
        ps = int(rng.choice([1, 4, 16, 64]))
        C = int(rng.choice([16, 48, 64, 528, 2048]))
        pages = rng.integers(0, 40, size=int(rng.integers(1, 20)))
        indptr = np.concatenate([[0], np.cumsum(pages)])
        cap = int(indptr[-1]) + int(rng.integers(0, 5))
        used = set()
        for b in range(len(pages)):
            kv_len = 0 if pages[b] == 0 else (pages[b] - 1) * ps + int(rng.integers(1, ps + 1))
            start = (int(indptr[b]) * ps) // C + b
            for j in range(math.ceil(kv_len / C)):
                cid = start + j
                assert cid not in used and cid < (cap * ps) // C + len(pages)
                used.add(cid)


def slice_segments(indptr, kv_lens, qo_lens, num_indices, slices, ps):
    """Host restatement of the balanced-slice layout in page-index space: slice
    x holds kv_indices positions [x per, (x + 1) per), per = ceil(num_indices /
    slices); request b contributes keys [lo, hi) of the pages it has there.
    Returns the (slice, request, lo, hi, slot) segments the streaming kernel
    processes and, per request, the slots the merge reads (x_lo .. x_hi,
    slot x + b)."""
    per = -(-num_indices // slices)
    segs, merged = [], {}
    for b in range(len(kv_lens)):
        p_start, p_end = int(indptr[b]), int(indptr[b + 1])
        if qo_lens[b] == 0 or p_end == p_start:
            continue
        x_lo, x_hi = p_start // per, (p_end - 1) // per
        merged[b] = [x + b for x in range(x_lo, x_hi + 1)]
        for x in range(slices):
            p0, p1 = max(p_start, x * per), min(p_end, min((x + 1) * per, num_indices))
            if p0 < p1:
                lo = (p0 - p_start) * ps
                hi = min((p1 - p_start) * ps, kv_lens[b])
                segs.append((x, b, lo, hi, x + b))
    return segs, merged


def test_slice_segments_cover_each_request_once():
    rng = np.random.default_rng(1)
    for _ in range(400):
        B = int(rng.integers(1, 65))
        ps = int(rng.choice([1, 4, 16, 64]))
        pages = rng.integers(0, 200, size=B)
        indptr = np.concatenate([[0], np.cumsum(pages)])
        num_indices = int(indptr[-1]) + int(rng.integers(0, 4))
        kv = [0 if n == 0 else (n - 1) * ps + int(rng.integers(1, ps + 1)) for n in pages]
        q = [min(int(rng.integers(0, 9)), k) for k in kv]
        slices = int(rng.integers(1, 300))
        if num_indices == 0:
            continue
        segs, merged = slice_segments(indptr, kv, q, num_indices, slices, ps)
        slots = [s[4] for s in segs]
        assert len(set(slots)) == len(slots) and all(s < slices + B for s in slots)
        for b in range(B):
            mine = sorted((lo, hi, slot) for (_, bb, lo, hi, slot) in segs if bb == b)
            if q[b] == 0 or kv[b] == 0:
                assert not mine and b not in merged
                continue
            assert mine[0][0] == 0 and mine[-1][1] == kv[b]
            assert all(lo < hi and lo % ps == 0 for lo, hi, _ in mine)
            assert all(mine[i][1] == mine[i + 1][0] for i in range(len(mine) - 1))
            # The merge reads exactly the slots written as partials; a request
            # inside one slice is written directly.
            assert merged[b] == [m[2] for m in mine]


def test_two_pass_stages(lib):
    """bf16 D 128 plans that read their keys mostly from L2 -- two row tiles
    per wave, or query RoPE with one tile per wave, all eight waves issuing
    and several row blocks -- stream 128-key stages, two of 64 KB; the rest
    keep four 32 KB stages."""
    def plan(cid, **kw):
        return B.vat_plan(problem_of(make_config(cid), **kw))
    for cid in (4, 7):
        pl = plan(cid)
        assert pl.row_tiles_per_wave == 2 and pl.stages == 2, cid
        pl = plan(cid, rope=1)
        assert pl.row_tiles_per_wave == 1 and pl.dma_waves == 8 and pl.row_blocks > 1, cid
        assert pl.stages == 2 and pl.lds_bytes == 2 * 64 * 1024 + 2048 * 4, cid
    for cid in (2, 3, 5, 6):
        assert plan(cid).stages == 4 and plan(cid, rope=1).stages == 4, cid
    # RoPE over eight row tiles in one row block (keys from HBM): four stages.
    pl = B.vat_plan(base_problem(batch=1, num_qo_heads=32, num_kv_heads=8, max_qo_len=32,
                                 num_qo_tokens=32, num_kv_indices=512, num_pages=512, rope=1))
    assert pl.row_tiles_per_wave == 1 and pl.dma_waves == 8 and pl.row_blocks == 1 and pl.stages == 4


def test_head_groups_only_where_the_shape_fits(lib):
    """fp8 caches of D 128 with an even KV-head count, at most 32 rows per KV
    head, planner-chosen slices, no byte-row masks: four heads per workgroup
    when the head count is divisible by four and there is no RoPE (one
    computing wave a head, holding all of its row tiles), else two (one row
    tile a wave); everything else one."""
    fp8 = dict(kv_dtype=2, num_kv_heads=8, num_qo_heads=32, max_qo_len=8, num_qo_tokens=16)
    plan = B.vat_plan(base_problem(**fp8))
    assert plan.heads_per_group == 4 and plan.waves_rows == 4 and plan.row_tiles_per_wave == 2
    assert plan.grid_y == 2 and plan.lds_bytes == 4 * 32 * 1024 + 2048 * 4
    plan = B.vat_plan(base_problem(**{**fp8, "max_qo_len": 4}))
    assert plan.heads_per_group == 4 and plan.waves_rows == 4 and plan.row_tiles_per_wave == 1
    plan = B.vat_plan(base_problem(**{**fp8, "num_kv_heads": 2, "num_qo_heads": 8}))
    assert plan.heads_per_group == 2 and plan.waves_rows == 4 and plan.row_tiles_per_wave == 1
    plan = B.vat_plan(base_problem(**{**fp8, "num_kv_heads": 6, "num_qo_heads": 24, "max_qo_len": 4}))
    assert plan.heads_per_group == 2 and plan.waves_rows == 2 and plan.grid_y == 3
    assert B.vat_plan(base_problem(**{**fp8, "has_mask": 1, "num_mask_bytes": 16})).heads_per_group == 4
    # RoPE: two heads per workgroup, one row tile per wave.
    plan = B.vat_plan(base_problem(**{**fp8, "rope": 1}))
    assert plan.heads_per_group == 2 and plan.waves_rows == 4 and plan.row_tiles_per_wave == 1
    for change in (dict(max_qo_len=9, num_qo_tokens=18), dict(num_kv_heads=1, num_qo_heads=4),
                   dict(num_kv_heads=3, num_qo_heads=12), dict(head_dim=64), dict(kv_dtype=1),
                   dict(chunk_keys=64), dict(has_mask=2, num_mask_bytes=64),
                   dict(batch=65, num_qo_tokens=65, max_qo_len=1, num_kv_indices=65)):
        assert B.vat_plan(base_problem(**{**fp8, **change})).heads_per_group == 1, change
    plan = B.vat_plan(base_problem(**{**fp8, "num_cus": 2}))
    assert plan.heads_per_group == 4 and plan.direct == 1 and plan.workspace_bytes == 0



@pytest.mark.parametrize("kw,code", [
    (dict(num_qo_heads=6, num_kv_heads=4), 2),
    (dict(head_dim=96), 3),
    (dict(page_size=12), 3),
    (dict(page_size=512), 3),
    (dict(q_dtype=0, kv_dtype=1), 3),
    (dict(q_dtype=1, kv_dtype=0), 3),
    (dict(has_mask=1, max_qo_len=65, num_mask_bytes=600), 3),
    (dict(has_mask=2, max_qo_len=65, num_mask_bytes=600), 3),
    (dict(has_mask=3, num_mask_bytes=8), 2),
    (dict(has_mask=1, num_mask_bytes=0), 2),
    (dict(chunk_keys=40), 2),
    (dict(chunk_keys=-2), 2),
    (dict(batch=-1), 2),
    (dict(num_pages=0), 2),
])
def test_invalid_problems_are_rejected_on_the_host(lib, kw, code):
    plan = B.VatPlan()
    assert lib.vat_plan(ctypes.byref(base_problem(**kw)), ctypes.byref(plan)) == code


def _call(lib, prob, ptrs=None, scales=(0.1, 1.0, 1.0), ws=0, ws_bytes=0):
    fake = 0x10000
    p = dict(q=fake, k=fake, v=fake, indptr=fake, indices=fake, lpl=fake, qo=fake, mask=0,
             mask_indptr=0, out=fake, lse=fake)
    if ptrs:
        p.update(ptrs)
    return lib.verify_attention(ctypes.byref(prob), p["q"], p["k"], p["v"], p["indptr"],
                                p["indices"], p["lpl"], p["qo"], p["mask"], p["mask_indptr"],
                                scales[0], scales[1], scales[2], p["out"], p["lse"], ws, ws_bytes,
                                None)


def test_host_checks_before_any_launch(lib):
    prob = base_problem(chunk_keys=0)  # direct: no workspace
    assert _call(lib, prob, ptrs=dict(q=0)) == 1
    assert _call(lib, prob, ptrs=dict(lse=0)) == 1
    assert _call(lib, prob, ptrs=dict(q=0x10002)) == 4
    assert _call(lib, prob, ptrs=dict(out=0x10008)) == 4
    assert _call(lib, prob, scales=(0.0, 1.0, 1.0)) == 2
    assert _call(lib, prob, scales=(float("nan"), 1.0, 1.0)) == 2
    assert _call(lib, prob, scales=(0.1, -1.0, 1.0)) == 2
    assert _call(lib, prob, scales=(0.1, 1.0, float("inf"))) == 2
    masked = base_problem(chunk_keys=0, has_mask=1, num_mask_bytes=8)
    assert _call(lib, masked, ptrs=dict(mask=0x20000, mask_indptr=0)) == 1
    split = base_problem(chunk_keys=48)
    need = B.vat_workspace_size(split)
    assert _call(lib, split, ws=0, ws_bytes=0) == 1
    assert _call(lib, split, ws=0x40000, ws_bytes=need - 1) == 5
    assert _call(lib, split, ws=0x40010, ws_bytes=need) == 4


def test_empty_work_returns_ok_without_a_gpu(lib):
    assert _call(lib, base_problem(num_qo_tokens=0), ptrs=dict(q=0, out=0, lse=0)) == 0
    assert _call(lib, base_problem(batch=0, num_qo_tokens=0)) == 0
    assert _call(lib, base_problem(max_qo_len=0)) == 0


def _append(lib, prob, src=1, ptrs=None, scales=(1.0, 1.0)):
    fake = 0x10000
    p = dict(kn=fake, vn=fake, kc=fake, vc=fake, indptr=fake, indices=fake, lpl=fake, qo=fake)
    if ptrs:
        p.update(ptrs)
    return lib.vat_append_kv(ctypes.byref(prob), src, p["kn"], p["vn"], p["kc"], p["vc"],
                             p["indptr"], p["indices"], p["lpl"], p["qo"], scales[0], scales[1],
                             None)


@pytest.mark.parametrize("kw,src,code", [
    (dict(head_dim=96), 1, 3),
    (dict(page_size=12), 1, 3),
    (dict(kv_dtype=3), 1, 3),
    ({}, 2, 3),            # an e4m3 source is not accepted
    ({}, 7, 3),
    (dict(batch=-1), 1, 2),
    (dict(num_pages=0), 1, 2),
    (dict(num_kv_heads=0), 1, 2),
    (dict(max_qo_len=-1), 1, 2),
    (dict(num_cus=-1), 1, 2),
])
def test_append_rejects_invalid_problems(lib, kw, src, code):
    assert _append(lib, base_problem(**kw), src=src) == code


def test_append_host_checks_before_any_launch(lib):
    prob = base_problem(kv_dtype=2)
    assert _append(lib, prob, ptrs=dict(kn=0)) == 1
    assert _append(lib, prob, ptrs=dict(vc=0)) == 1
    assert _append(lib, prob, ptrs=dict(qo=0)) == 1
    assert _append(lib, prob, ptrs=dict(kn=0x10008)) == 4
    assert _append(lib, prob, ptrs=dict(kc=0x10001)) == 4
    assert _append(lib, prob, ptrs=dict(indices=0x10002)) == 4
    for sc in [(0.0, 1.0), (-1.0, 1.0), (1.0, float("inf")), (float("nan"), 1.0)]:
        assert _append(lib, prob, scales=sc) == 2
    # The fields the append does not read are not checked.
    assert _append(lib, base_problem(num_qo_heads=3, num_kv_heads=2, q_dtype=0, kv_dtype=2,
                                     chunk_keys=-7), ptrs=dict(kn=0)) == 1


def test_rope_host_checks(lib):
    fake = 0x10000
    prob = base_problem(chunk_keys=0, rope=1)

    def call(cs, problem=prob):
        return lib.verify_attention_rope(ctypes.byref(problem), fake, fake, fake, fake, fake, fake,
                                         fake, 0, 0, cs, 0.1, 1.0, 1.0, fake, fake, 0, 0, None)

    assert call(0) == 1                      # rope without cos/sin rows
    assert call(fake + 4) == 4               # rows not 16-byte aligned
    # The plain entry point passes no rows: a rope problem is refused there.
    assert _call(lib, prob) == 1
    for kw, code in [(dict(q_dtype=0, kv_dtype=0), 3), (dict(kv_dtype=2, head_dim=64), 3),
                     (dict(rope=2), 2)]:
        bad = base_problem(chunk_keys=0, rope=kw.pop("rope", 1), **kw)
        assert call(fake, bad) == code, kw
    # Byte-row masks take RoPE (one row tile per wave); fp32 caches plan
    # normally without it.
    plan = B.vat_plan(base_problem(has_mask=2, num_mask_bytes=100, rope=1))
    assert plan.kernel == 1 and plan.row_tiles_per_wave == 1
    assert B.vat_plan(base_problem(has_mask=2, num_mask_bytes=100)).kernel == 1
    plan = B.vat_plan(base_problem(rope=1, num_qo_heads=32, max_qo_len=64, num_qo_tokens=128))
    assert plan.row_tiles_per_wave == 1 and plan.rows_per_block <= 128
    ap = base_problem(kv_dtype=2)
    args = [ctypes.byref(ap), 1] + [fake] * 8
    assert lib.vat_append_kv_rope(*args, 0, 1.0, 1.0, None) == 1
    assert lib.vat_append_kv_rope(*args, fake + 8, 1.0, 1.0, None) == 4


def test_append_of_nothing_returns_ok_without_a_gpu(lib):
    assert _append(lib, base_problem(num_qo_tokens=0), ptrs=dict(kn=0, vn=0)) == 0
    assert _append(lib, base_problem(batch=0, num_qo_tokens=0)) == 0
    assert _append(lib, base_problem(max_qo_len=0)) == 0


def test_planner_under_address_and_ub_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    driver = tmp_path / "plan_fuzz.cpp"
    driver.write_text(r'''
#include <stdio.h>
#include <stdlib.h>
#include "plan.h"
int main() {
  srand(7);
  const int dims[] = {32, 64, 96, 128}, pss[] = {1, 2, 16, 12, 256, 512};
  long ok = 0;
  for (int it = 0; it < 200000; ++it) {
    vat_problem_t p;
    p.batch = rand() % 300 - 2;
    p.num_kv_heads = 1 + rand() % 16;
    p.num_qo_heads = p.num_kv_heads * (1 + rand() % 16) + (rand() % 10 == 0);
    p.head_dim = dims[rand() % 4];
    p.page_size = pss[rand() % 6];
    p.num_pages = rand() % 100000;
    p.num_kv_indices = rand() % 2000000;
    p.num_qo_tokens = rand() % 100000;
    p.max_qo_len = rand() % 2000;
    p.q_dtype = rand() % 3; p.kv_dtype = rand() % 3;
    p.has_mask = rand() % 3;
    p.num_mask_bytes = rand() % 100000;
    p.num_cus = 1 + rand() % 512;
    p.chunk_keys = (rand() % 4 == 0) ? (rand() % 3) * 16 - 16 : -1;
    vat_plan_t plan;
    if (vat::make_plan(&p, p.num_cus, &plan) == VAT_OK) {
      ++ok;
      if (plan.lds_bytes > 160 * 1024 || plan.workspace_bytes < 0) { printf("bad plan\n"); return 1; }
    }
  }
  printf("planned %ld\n", ok);
  return ok > 0 ? 0 : 1;
}
''')
    exe = tmp_path / "plan_fuzz"
    csrc = os.path.join(ROOT, "paged_kv_gqa_planner_amd", "csrc")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", csrc, "-I", os.path.join(ROOT, "include"),
           str(driver), os.path.join(csrc, "plan.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "planned" in r.stdout


def test_binding_requires_max_qo_len_for_batches_of_several_requests():
    """The binding's only shape-derived bound is for one request (L = T); a
    batch of several must state the largest draft count, since T - (B - 1)
    would overstate it (and pass the 64-draft mask limit)."""
    import torch

    q = torch.zeros(136, 4, 128, dtype=torch.bfloat16)
    kc = torch.zeros(40, 16, 1, 128, dtype=torch.bfloat16)
    one = torch.tensor([0, 3], dtype=torch.int32)
    eight = torch.arange(0, 9 * 3, 3, dtype=torch.int32)
    idx = torch.arange(40, dtype=torch.int32)
    assert B.problem_from_tensors(q, kc, one, idx).max_qo_len == 136
    assert B.problem_from_tensors(q[:0], kc, torch.zeros(1, dtype=torch.int32), idx).max_qo_len == 0
    assert B.problem_from_tensors(q[:0], kc, eight, idx).max_qo_len == 0  # no tokens at all
    with pytest.raises(ValueError, match="max_qo_len"):
        B.problem_from_tensors(q, kc, eight, idx)
    with pytest.raises(ValueError, match="max_qo_len"):
        B.problem_from_tensors(q, kc, eight, idx, mask=torch.zeros(300, dtype=torch.uint8))
    assert B.problem_from_tensors(q, kc, eight, idx, max_qo_len=17).max_qo_len == 17


def test_read_probe_host_checks(lib):
    """The HBM read probe rejects bad arguments before touching a device."""
    vp = ctypes.c_void_p
    assert lib.vat_read_probe(None, 0, None, None) == 0            # nothing to read
    assert lib.vat_read_probe(None, 64, vp(4096), None) == 1       # NULL buffer
    assert lib.vat_read_probe(vp(4096), 64, None, None) == 1       # NULL sink
    assert lib.vat_read_probe(vp(4096), 72, vp(8192), None) == 2   # not a multiple of 16
    assert lib.vat_read_probe(vp(4104), 64, vp(8192), None) == 4   # buffer misaligned
    assert lib.vat_read_probe(vp(4096), 64, vp(8194), None) == 4   # sink misaligned


def test_check_inputs_host_checks(lib):
    """The device-content check rejects missing or misaligned arrays and
    invalid shapes before anything is enqueued."""
    vp = ctypes.c_void_p
    prob = base_problem(chunk_keys=0)
    a = [vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000), None, vp(0x5000)]
    assert lib.vat_check_inputs(None, *a, None) == 1
    assert lib.vat_check_inputs(ctypes.byref(prob), *a[:5], None, None) == 1      # status
    assert lib.vat_check_inputs(ctypes.byref(prob), None, *a[1:], None) == 1      # kv_indptr
    assert lib.vat_check_inputs(ctypes.byref(prob), a[0], None, *a[2:], None) == 1
    assert lib.vat_check_inputs(ctypes.byref(prob), *a[:2], None, *a[3:], None) == 1
    assert lib.vat_check_inputs(ctypes.byref(prob), *a[:3], None, *a[4:], None) == 1
    assert lib.vat_check_inputs(ctypes.byref(prob), *a[:5], vp(0x5002), None) == 4
    assert lib.vat_check_inputs(ctypes.byref(prob), vp(0x1001), *a[1:], None) == 4
    masked = base_problem(chunk_keys=0, has_mask=1, num_mask_bytes=8)
    assert lib.vat_check_inputs(ctypes.byref(masked), *a, None) == 1              # mask_indptr
    assert lib.vat_check_inputs(ctypes.byref(masked), *a[:4], vp(0x6002), a[5], None) == 4
    bad = base_problem(chunk_keys=0, num_kv_heads=3)                                # Hq % Hkv
    assert lib.vat_check_inputs(ctypes.byref(bad), *a, None) == 2


def test_noalloc_refuses_an_oversized_workspace_on_the_host(lib):
    """verify_attention_noalloc checks the planned workspace against its static
    array before anything else touches the device."""
    prob = B.make_problem(batch=1, num_qo_heads=64, num_kv_heads=1, head_dim=128, page_size=16,
                          num_pages=1 << 16, num_kv_indices=1 << 16, num_qo_tokens=64,
                          max_qo_len=64, q_dtype=1, kv_dtype=1, has_mask=0, num_cus=4096)
    assert B.vat_workspace_size(prob) > B.NOALLOC_SCRATCH_BYTES
    st = lib.verify_attention_noalloc(ctypes.byref(prob), *([None] * 9), 0.1, 1.0, 1.0, None,
                                      None, None)
    assert st == 5


@pytest.mark.parametrize("kv,hkv,G,L", [(1, 8, 4, 1), (1, 8, 4, 4), (1, 2, 16, 1), (2, 8, 4, 8),
                                         (2, 4, 4, 2), (1, 8, 4, 5), (1, 8, 8, 17), (2, 1, 4, 8)])
@pytest.mark.parametrize("batch", [1, 2, 5, 13, 64, 65, 300])
def test_merge_grid_covers_every_row_of_every_request(lib, kv, hkv, G, L, batch):
    """Whatever the plan, the merge launches one workgroup per (request, KV head,
    row block, group of merge_rows rows), so every row that has partials is merged."""
    prob = base_problem(batch=batch, num_qo_heads=hkv * G, num_kv_heads=hkv, kv_dtype=kv,
                        max_qo_len=L, num_qo_tokens=batch * L, num_pages=8000,
                        num_kv_indices=7000)
    plan = B.vat_plan(prob)
    if plan.direct:
        assert plan.merge_grid == 0
        return
    assert plan.merge_rows in (4, 16)
    per_item = -(-plan.rows_per_block // plan.merge_rows)
    assert plan.merge_grid == batch * hkv * plan.row_blocks * per_item
