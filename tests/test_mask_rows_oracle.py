"""Pins of the oracle's reading of sglang's full-row byte masks.

The hand-worked layout fixture fixes the byte addressing; the rest checks
that the layout changes nothing else: the same draft blocks give bitwise
the same oracle result as the packed L x L layout (itself pinned against
float64 SDPA), whatever the prefix bytes hold and whatever nonzero value
marks an allowed entry.
"""

from __future__ import annotations

import os

import numpy as np
import pytest

from oracle import unpack_mask_rows
from tests.layout_helpers import run_oracle
from workloads import make_case, tree_mask_rows
from workloads.gen import pack_mask_full_rows

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "mask_rows.txt")


def _golden():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            if not line.startswith("batch"):
                continue
            fields = [x.strip() for x in line.split("|")]
            prefixes = [int(x) for x in fields[1].split()[1:]]
            parents = [[int(x) for x in grp.split()] for grp in fields[2][len("parents"):].split(";")]
            indptr = [int(x) for x in fields[3].split()[1:]]
            data = bytes(int(x, 16) for x in fields[4].split()[1:])
            out.append((fields[0].split()[1], prefixes, parents, indptr, data))
    return out


@pytest.mark.parametrize("name,prefixes,parents,indptr,data", _golden())
def test_rows_layout_matches_hand_worked_bytes(name, prefixes, parents, indptr, data):
    blocks = [tree_mask_rows(p) for p in parents]
    packed, ip = pack_mask_full_rows(blocks, prefixes)
    assert bytes(packed) == data, name
    assert list(ip) == indptr, name
    arr = np.frombuffer(data, dtype=np.uint8)
    for b, (blk, pfx) in enumerate(zip(blocks, prefixes)):
        assert np.array_equal(unpack_mask_rows(arr, indptr[b], pfx, blk.shape[0]), blk), name
    # The two entries the fixture spells out.
    assert unpack_mask_rows(arr, 8, 1, 3)[2, 2] and not unpack_mask_rows(arr, 8, 1, 3)[2, 1]


def _pair(seed, mask_kind, **kw):
    base = dict(prefix_lens=[0, 5, 37, 64], qo_lens=[3, 1, 9, 17], num_qo_heads=6,
                num_kv_heads=2, head_dim=16, page_size=4, mask_kind=mask_kind, **kw)
    return make_case(seed, **base), make_case(seed, mask_layout="rows", **base)


@pytest.mark.parametrize("seed,mask_kind", [(1, "tree"), (2, "random"), (3, "chain"), (4, "full")])
def test_rows_layout_equals_packed_layout_bitwise(seed, mask_kind):
    bits, rows = _pair(seed, mask_kind, kv_dtype="bf16", q_dtype="bf16")
    assert np.array_equal(bits.k_cache, rows.k_cache) and np.array_equal(bits.q, rows.q)
    ob, lb = run_oracle(bits)
    orw, lr = run_oracle(rows)
    assert np.array_equal(ob, orw) and np.array_equal(lb, lr)


@pytest.mark.parametrize("prefix_fill,true_values", [("zeros", "ones"), ("random", "random"),
                                                     ("ones", "random")])
def test_prefix_bytes_are_not_read_and_any_nonzero_allows(prefix_fill, true_values):
    _, rows = _pair(5, "random", kv_dtype="f32", q_dtype="f32")
    _, other = _pair(5, "random", kv_dtype="f32", q_dtype="f32", rows_prefix_fill=prefix_fill,
                     rows_true_values=true_values)
    assert not np.array_equal(rows.mask, other.mask)
    o1, l1 = run_oracle(rows)
    o2, l2 = run_oracle(other)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
