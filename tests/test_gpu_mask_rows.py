"""GPU parity for sglang's full-row byte masks (mask layout 2).

Every case runs the HIP path through the C ABI and compares it with the
oracle at the parity tolerances; where the same draft blocks are also given
in the packed layout, the two GPU outputs must agree bit for bit (the layout
only changes where the visibility bits come from).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.gpu_helpers import compare, oracle_of, run_gpu, say, to_f64
from workloads import make_case, make_config

pytestmark = pytest.mark.gpu


def _bitwise_same(a, b):
    return torch.equal(a[0].view(torch.int16) if a[0].dtype == torch.bfloat16 else a[0],
                       b[0].view(torch.int16) if b[0].dtype == torch.bfloat16 else b[0]) \
        and torch.equal(a[1], b[1])


@pytest.mark.parametrize("prefix", [4096, 16384, 32768])
def test_tree_verify_config_in_full_rows(gpu_lib, prefix):
    rows = make_config(3, prefix=prefix, mask_layout="rows")
    bits = make_config(3, prefix=prefix)
    say(f"[rows config 3 prefix={prefix}] mask bytes {rows.mask.size} vs packed {bits.mask.size}")
    got_rows = run_gpu(gpu_lib, rows)
    got_bits = run_gpu(gpu_lib, bits)
    compare(rows, *to_f64(*got_rows), *oracle_of(rows), what=f"rows prefix {prefix}")
    assert _bitwise_same(got_rows, got_bits), "full-row and packed layouts differ"


def _case(seed):
    rng = np.random.default_rng(500 + seed)
    pairs = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "e4m3")]
    q_dt, kv_dt = pairs[seed % 3]
    D = [64, 128][(seed // 3) % 2]
    B = int(rng.integers(1, 6))
    Hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4, 8]))
    ps = int(rng.choice([1, 4, 16]))
    kind = ["tree", "random", "chain", "full"][seed % 4]
    Lmax = [20, 64, 33, 9][(seed // 2) % 4]
    lens = [int(x) for x in rng.integers(1, Lmax + 1, size=B)]
    prefixes = [int(x) for x in rng.integers(0, 400, size=B)]
    chunk = int(rng.choice([-1, 0, 48, 128]))
    fill = ["ones", "zeros", "random"][seed % 3]
    vals = ["ones", "random"][seed % 2]
    kw = dict(prefix_lens=prefixes, qo_lens=lens, num_qo_heads=G * Hkv, num_kv_heads=Hkv,
              head_dim=D, page_size=ps, q_dtype=q_dt, kv_dtype=kv_dt, mask_kind=kind,
              fp8_absmax_scales=(kv_dt == "e4m3"), mask_density=0.5,
              mask_pad_bytes=int(seed % 3), extra_indices=int(seed % 4))
    rows = make_case(seed, mask_layout="rows", rows_prefix_fill=fill, rows_true_values=vals, **kw)
    bits = make_case(seed, **kw)
    return rows, bits, chunk


@pytest.mark.parametrize("seed", list(range(24)))
def test_fuzz_full_rows(gpu_lib, seed):
    rows, bits, chunk = _case(seed)
    say(f"[rows fuzz {seed}] B={rows.batch} Hq={rows.num_qo_heads} Hkv={rows.num_kv_heads} "
        f"D={rows.head_dim} ps={rows.page_size} {rows.q_dtype}/{rows.kv_dtype} "
        f"mask={rows.info['mask_kind']} L={rows.info['qo_lens']} "
        f"prefix={rows.info['prefix_lens']} chunk={chunk}")
    got_rows = run_gpu(gpu_lib, rows, chunk_keys=chunk)
    compare(rows, *to_f64(*got_rows), *oracle_of(rows), what=f"rows fuzz {seed}")
    got_bits = run_gpu(gpu_lib, bits, chunk_keys=chunk)
    assert _bitwise_same(got_rows, got_bits), f"rows fuzz {seed}: layouts differ"


@pytest.mark.parametrize("num_cus", [1, 8, 256])
def test_full_rows_under_balanced_slices(gpu_lib, num_cus):
    """Many requests per workgroup (page-space slices): each segment fetches
    its own rows' bytes."""
    p = make_case(41, prefix_lens=[int(x) for x in np.arange(40) * 37 % 900],
                  qo_lens=[int(x) for x in np.arange(40) % 17 + 1], num_qo_heads=16,
                  num_kv_heads=4, head_dim=128, mask_kind="tree", mask_layout="rows",
                  rows_prefix_fill="random", rows_true_values="random")
    say(f"[rows slices num_cus={num_cus}]")
    got = run_gpu(gpu_lib, p, num_cus=num_cus)
    compare(p, *to_f64(*got), *oracle_of(p), what=f"rows slices {num_cus}")


@pytest.mark.parametrize("kv_dtype,head_dim", [("f32", 64), ("bf16", 128), ("e4m3", 128), ("e4m3", 64)])
@pytest.mark.parametrize("group,page_size", [(3, 64), (16, 256), (64, 2)])
def test_full_rows_with_uncommon_groups_and_page_sizes(gpu_lib, kv_dtype, head_dim, group, page_size):
    hkv = 1 if group == 64 else 2
    kw = dict(prefix_lens=[120, 0, 700], qo_lens=[40, 1, 64], num_qo_heads=group * hkv,
              num_kv_heads=hkv, head_dim=head_dim, page_size=page_size,
              q_dtype="f32" if kv_dtype == "f32" else "bf16", kv_dtype=kv_dtype, mask_kind="tree",
              fp8_absmax_scales=(kv_dtype == "e4m3"))
    rows = make_case(92, mask_layout="rows", rows_prefix_fill="random", rows_true_values="random", **kw)
    bits = make_case(92, **kw)
    plans = [_plan_of(gpu_lib, x, layout) for x, layout in ((rows, 2), (bits, 1))]
    say(f"[rows G={group} page {page_size}] {kv_dtype} D{head_dim} same plan: {plans[0] == plans[1]}")
    got_rows = run_gpu(gpu_lib, rows)
    compare(rows, *to_f64(*got_rows), *oracle_of(rows), what=f"rows G{group} page {page_size}")
    got_bits = run_gpu(gpu_lib, bits)
    compare(bits, *to_f64(*got_bits), *oracle_of(bits), what=f"bits G{group} page {page_size}")
    # A different split or tiling changes only the rounding order, so the two
    # layouts agree bit for bit exactly when they get the same plan (bf16 D 128
    # has no two-tile variant for full-row masks).
    if plans[0] == plans[1]:
        assert _bitwise_same(got_rows, got_bits), "full-row and packed layouts differ"


def _plan_of(lib, p, has_mask):
    prob = lib.make_problem(
        batch=p.batch, num_qo_heads=p.num_qo_heads, num_kv_heads=p.num_kv_heads,
        head_dim=p.head_dim, page_size=p.page_size, num_pages=p.num_pages,
        num_kv_indices=len(p.kv_indices), num_qo_tokens=int(p.qo_indptr[-1]),
        max_qo_len=p.max_qo_len, q_dtype={"f32": 0, "bf16": 1}[p.q_dtype],
        kv_dtype={"f32": 0, "bf16": 1, "e4m3": 2}[p.kv_dtype], has_mask=has_mask,
        num_mask_bytes=len(p.mask), num_cus=256)
    d = lib.vat_plan(prob).as_dict()
    d.pop("lds_bytes", None)
    d.pop("workspace_bytes", None)
    return d
