"""verify_attention_noalloc: the entry point that takes its workspace from the
library's static per-device scratch array instead of the caller.

Two calls in a row through the C ABI, the second with a smaller input, each
bitwise equal to verify_attention on the same inputs (same plan, same
kernels) and within the parity tolerances of the oracle; a problem whose
workspace exceeds the array is refused with VAT_ERR_WORKSPACE before
anything is enqueued.
"""

import pytest
import torch

from tests.gpu_helpers import compare, oracle_of, say, to_device, to_f64
from workloads import make_case, make_config

pytestmark = pytest.mark.gpu


def _call(lib, p, t, fn):
    kw = dict(sm_scale=p.sm_scale, k_scale=p.k_scale, v_scale=p.v_scale, max_qo_len=p.max_qo_len,
              mask_layout=p.mask_layout)
    args = (t["q"], t["k_cache"], t["v_cache"], t["kv_indptr"], t["kv_indices"],
            t["last_page_len"], t["qo_indptr"], t["mask"], t["mask_indptr"])
    out, lse = fn(*args, **kw)
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_matches_verify_attention_twice_larger_then_smaller(gpu_lib):
    # First the fp8 batch-64 workload (a 12 MiB workspace), then a smaller
    # masked bf16 tree batch (a few hundred KiB): the second call reuses the
    # array that still holds the first call's partials. Then one request over
    # balanced slices, whose merge loads slots ahead of the request table:
    # the slots past its own hold the earlier calls' partials and must be
    # dropped.
    cases = [make_config(5),
             make_case(41, prefix_lens=[300, 45, 900], qo_lens=[9, 4, 13], num_qo_heads=8,
                       num_kv_heads=2, head_dim=128, page_size=16, mask_kind="tree"),
             make_case(43, prefix_lens=[2500], qo_lens=[9], num_qo_heads=16, num_kv_heads=4,
                       head_dim=128, page_size=16, mask_kind="tree", extra_indices=5)]
    sizes = []
    for i, p in enumerate(cases):
        t = to_device(p)
        prob = gpu_lib.problem_from_tensors(t["q"], t["k_cache"], t["kv_indptr"], t["kv_indices"],
                                            t["mask"], p.max_qo_len, mask_layout=p.mask_layout)
        ws = gpu_lib.vat_workspace_size(prob)
        sizes.append(ws)
        say(f"[noalloc call {i}] {p.name or 'tree batch'} workspace {ws} B")
        assert 0 < ws <= gpu_lib.NOALLOC_SCRATCH_BYTES
        got_o, got_l = _call(gpu_lib, p, t, gpu_lib.verify_attention_noalloc)
        ref_o, ref_l = _call(gpu_lib, p, t, gpu_lib.verify_attention)
        assert torch.equal(got_o.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(got_l, ref_l)
        compare(p, *to_f64(got_o, got_l), *oracle_of(p), what=f"noalloc call {i}")
    assert sizes[1] < sizes[0] and sizes[2] < sizes[0]


def test_noalloc_refuses_a_workspace_beyond_the_array(gpu_lib):
    # A batch-1 request of 2^20 keys, 4096 query rows per KV head, planned for
    # 4096 CUs: 257 chunks x 16 row blocks of 256 fp32 partial rows, 518 MiB.
    # Only host planning runs.
    prob = gpu_lib.make_problem(batch=1, num_qo_heads=64, num_kv_heads=1, head_dim=128,
                                page_size=16, num_pages=1 << 16, num_kv_indices=1 << 16,
                                num_qo_tokens=64, max_qo_len=64, q_dtype=1, kv_dtype=1,
                                has_mask=0, num_cus=4096)
    assert gpu_lib.vat_workspace_size(prob) > gpu_lib.NOALLOC_SCRATCH_BYTES
    lib = gpu_lib.load()
    import ctypes

    st = lib.verify_attention_noalloc(ctypes.byref(prob), *([None] * 9), 0.1, 1.0, 1.0, None,
                                      None, None)
    assert st == 5  # VAT_ERR_WORKSPACE, nothing enqueued
