"""GPU parity of the two-pass stages.

bf16 D 128 plans with two row tiles per wave (prefill blocks, wide trees),
and query-RoPE plans with one tile per wave, all eight waves issuing loads
and several row blocks, stream 128-key stages through a two-deep ring and
take each stage in two 64-key passes, the second skipped when the segment
ends in the first. These cases put segment ends on both sides of the pass
boundary (ragged lengths, requests of one token beside long ones), cover page
sizes 1 to 256, packed tree and random masks at the 64-draft maximum, items
split across workgroups (the merge), paired row blocks, and the RoPE
variant. Each case first checks that its plan is a two-pass one, then
compares every request with the oracle.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_helpers import compare, run_gpu, say, to_device, to_f64
from workloads import make_case, rope_cos_sin, rope_positions

pytestmark = pytest.mark.gpu

# G = 8 query heads per KV head, so a request of L tokens has 8 L rows per
# KV head; a plan is two-tile once the longest request has 17 or more.
CASES = {
    "ragged_ps16": dict(prefix_lens=[0, 500, 33, 2000, 7], qo_lens=[300, 77, 129, 65, 1], page_size=16),
    "ragged_ps1": dict(prefix_lens=[0, 70, 9], qo_lens=[150, 40, 97], page_size=1),
    "ragged_ps4": dict(prefix_lens=[3, 260, 0], qo_lens=[211, 18, 64], page_size=4),
    "ragged_ps64": dict(prefix_lens=[1000, 0, 129], qo_lens=[33, 257, 2], page_size=64),
    "ragged_ps256": dict(prefix_lens=[700, 4100], qo_lens=[190, 31], page_size=256),
    "tree64": dict(prefix_lens=[100, 3000, 0], qo_lens=[64, 64, 40], page_size=16, mask_kind="tree"),
    "random64": dict(prefix_lens=[513, 64], qo_lens=[64, 57], page_size=32, mask_kind="random"),
}

# The device's CU count; eight, where a long item's row blocks are paired in
# one workgroup; 2048, where items are split into chunks and merged.
NUM_CUS = [0, 8, 2048]


def _case(name, seed=0):
    kw = dict(CASES[name])
    mask_kind = kw.pop("mask_kind", "causal")
    return make_case(100 + seed + len(name), num_qo_heads=16, num_kv_heads=2, head_dim=128,
                     mask_kind=mask_kind, max_qo_len=max(kw["qo_lens"]), **kw)


def _plan(lib, p, t, num_cus, rope):
    return lib.vat_plan(lib.problem_from_tensors(t["q"], t["k_cache"], t["kv_indptr"], t["kv_indices"],
                                                 t["mask"], p.max_qo_len, num_cus=num_cus, rope=rope))


@pytest.mark.parametrize("num_cus", NUM_CUS)
@pytest.mark.parametrize("name", sorted(CASES))
def test_two_tile_two_pass_matches_oracle(gpu_lib, oracle_pool, name, num_cus):
    p = _case(name)
    t = to_device(p)
    plan = _plan(gpu_lib, p, t, num_cus, False)
    say(f"[two-pass {name} cus={num_cus or 'device'}] rt={plan.row_tiles_per_wave} stages={plan.stages} "
        f"blocks={plan.row_blocks} order={plan.block_order} chunk={plan.chunk_keys} direct={plan.direct}")
    assert plan.kernel == 1 and plan.row_tiles_per_wave == 2 and plan.stages == 2
    out, lse = run_gpu(gpu_lib, p, tensors=t, num_cus=num_cus)
    compare(p, *to_f64(out, lse), *oracle_pool.run(p), what=f"two-pass {name} cus {num_cus}")


@pytest.mark.parametrize("num_cus", NUM_CUS)
@pytest.mark.parametrize("name", ["ragged_ps16", "ragged_ps4", "tree64"])
def test_rope_two_pass_matches_oracle(gpu_lib, oracle_pool, name, num_cus):
    p = _case(name)
    t = to_device(p)
    plan = _plan(gpu_lib, p, t, num_cus, True)
    say(f"[rope two-pass {name} cus={num_cus or 'device'}] rt={plan.row_tiles_per_wave} "
        f"dma={plan.dma_waves} stages={plan.stages} blocks={plan.row_blocks} chunk={plan.chunk_keys}")
    assert plan.kernel == 1 and plan.row_tiles_per_wave == 1 and plan.dma_waves == 8
    assert plan.row_blocks > 1 and plan.stages == 2
    cs = rope_cos_sin(rope_positions(p), p.head_dim)
    out, lse = run_gpu(gpu_lib, p, tensors=t, num_cus=num_cus,
                       q_cos_sin=torch.from_numpy(np.ascontiguousarray(cs)).cuda())
    compare(p, *to_f64(out, lse), *oracle_pool.run(p, q_cos_sin=cs), what=f"rope two-pass {name} cus {num_cus}")


def test_two_pass_is_bitwise_repeatable_and_page_order_free(gpu_lib):
    """Two runs give the same bits, and so does the same cache with its pages
    permuted in the pool (the gather follows the page table)."""
    p = _case("ragged_ps16")
    t = to_device(p)
    a = run_gpu(gpu_lib, p, tensors=t)
    b = run_gpu(gpu_lib, p, tensors=t)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    gen = torch.Generator().manual_seed(7)
    perm = torch.randperm(p.num_pages, generator=gen).to("cuda")
    t2 = dict(t)
    t2["k_cache"] = torch.empty_like(t["k_cache"])
    t2["v_cache"] = torch.empty_like(t["v_cache"])
    t2["k_cache"][perm] = t["k_cache"]
    t2["v_cache"][perm] = t["v_cache"]
    idx = t["kv_indices"].clone()
    used = int(p.kv_indptr[-1])
    idx[:used] = perm[t["kv_indices"][:used].long()].to(torch.int32)
    t2["kv_indices"] = idx
    c = run_gpu(gpu_lib, p, tensors=t2)
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])
