"""GPU tests of the device-content check (vat_check_inputs).

The check is a debugging aid: it reads a call's index arrays and mask offsets
and reports which rule of the contract they break (the paged format of the
FlashInfer page "feat: Separate Q and KV dtypes for decode", begin_forward
docstring, plus the query and mask segment rules of the C header). Valid
inputs from the workload generator must give 0; each planted violation must
give exactly its own bit; and seeded random corruptions must give the bits
that a plain host walk over the same rules gives. The attention kernels are
never run on the corrupted arrays.
"""

from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

from paged_kv_gqa_planner_amd import binding as B
from tests.gpu_helpers import say, to_device
from workloads import make_case, make_config

pytestmark = pytest.mark.gpu

KV_INDPTR, KV_INDICES, LAST_PAGE, QO_INDPTR, QO_LEN, MASK = 1, 2, 4, 8, 16, 32


def host_bits(kv_indptr, kv_indices, lpl, qo_indptr, mask_indptr, *, num_kv_indices, num_pages,
              page_size, tokens, max_qo_len, has_mask, num_mask_bytes):
    """The contract's rules, walked request by request on the host."""
    batch = len(kv_indptr) - 1
    bits = 0
    if kv_indptr[0] != 0:
        bits |= KV_INDPTR
    if qo_indptr[0] != 0 or qo_indptr[batch] != tokens:
        bits |= QO_INDPTR
    for b in range(batch):
        kv0, kv1 = int(kv_indptr[b]), int(kv_indptr[b + 1])
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        if kv1 < kv0 or kv1 > num_kv_indices:
            bits |= KV_INDPTR
        if q1 < q0 or q1 > tokens:
            bits |= QO_INDPTR
        pages = max(kv1 - kv0, 0)
        L = max(q1 - q0, 0)
        if pages > 0 and not 1 <= int(lpl[b]) <= page_size:
            bits |= LAST_PAGE
        kv_len = (pages - 1) * page_size + int(lpl[b]) if pages > 0 else 0
        if L > max_qo_len or L > kv_len:
            bits |= QO_LEN
        if has_mask and L > 0:
            need = (L * L + 7) // 8 if has_mask == 1 else L * kv_len
            m0 = int(mask_indptr[b])
            if m0 < 0 or m0 > num_mask_bytes or m0 + max(need, 0) > num_mask_bytes:
                bits |= MASK
    used = min(max(int(kv_indptr[batch]), 0), num_kv_indices)
    if used and (np.any(kv_indices[:used] < 0) or np.any(kv_indices[:used] >= num_pages)):
        bits |= KV_INDICES
    return bits


class Arrays:
    """Host copies of one call's index arrays plus the shapes the check reads.
    ``q`` and ``k_cache`` only carry shapes and dtypes (expanded views)."""

    def __init__(self, *, kv_indptr, kv_indices, last_page_len, qo_indptr, mask_indptr=None,
                 num_mask_bytes=0, mask_layout="bits", num_pages, page_size, max_qo_len,
                 num_qo_heads=8, num_kv_heads=2, head_dim=128):
        self.kv_indptr = np.array(kv_indptr, dtype=np.int32)
        self.kv_indices = np.array(kv_indices, dtype=np.int32)
        self.last_page_len = np.array(last_page_len, dtype=np.int32)
        self.qo_indptr = np.array(qo_indptr, dtype=np.int32)
        self.mask_indptr = None if mask_indptr is None else np.array(mask_indptr, dtype=np.int32)
        self.num_mask_bytes = num_mask_bytes
        self.mask_layout = mask_layout
        self.num_pages, self.page_size, self.max_qo_len = num_pages, page_size, max_qo_len
        self.hq, self.hkv, self.d = num_qo_heads, num_kv_heads, head_dim
        self.tokens = int(self.qo_indptr[-1])

    @classmethod
    def of_problem(cls, p):
        return cls(kv_indptr=p.kv_indptr, kv_indices=p.kv_indices, last_page_len=p.last_page_len,
                   qo_indptr=p.qo_indptr, mask_indptr=p.mask_indptr,
                   num_mask_bytes=0 if p.mask is None else p.mask.size, mask_layout=p.mask_layout,
                   num_pages=p.num_pages, page_size=p.page_size, max_qo_len=p.max_qo_len,
                   num_qo_heads=p.num_qo_heads, num_kv_heads=p.num_kv_heads, head_dim=p.head_dim)

    def copy(self):
        c = object.__new__(Arrays)
        c.__dict__.update({k: (v.copy() if isinstance(v, np.ndarray) else v)
                           for k, v in self.__dict__.items()})
        return c

    def expected(self):
        has_mask = 0 if self.mask_indptr is None else B.MASK_LAYOUTS[self.mask_layout]
        return host_bits(self.kv_indptr, self.kv_indices, self.last_page_len, self.qo_indptr,
                         self.mask_indptr, num_kv_indices=self.kv_indices.size,
                         num_pages=self.num_pages, page_size=self.page_size, tokens=self.tokens,
                         max_qo_len=self.max_qo_len, has_mask=has_mask,
                         num_mask_bytes=self.num_mask_bytes)

    def run(self, status=None):
        dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
        q = torch.empty(1, dtype=torch.bfloat16, device="cuda").expand(self.tokens, self.hq, self.d)
        kc = torch.empty(1, dtype=torch.bfloat16, device="cuda").expand(
            self.num_pages, self.page_size, self.hkv, self.d)
        mask = None
        if self.mask_indptr is not None:
            mask = torch.empty(1, dtype=torch.uint8, device="cuda").expand(self.num_mask_bytes)
        return B.check_inputs(q, kc, dev(self.kv_indptr), dev(self.kv_indices),
                              dev(self.last_page_len), dev(self.qo_indptr), mask,
                              dev(self.mask_indptr), max_qo_len=self.max_qo_len,
                              mask_layout=self.mask_layout, status=status)


# Valid inputs: the generator's cases, with empty requests, unused index
# slots (poisoned with 0x7FFFFFFF), both mask layouts and page sizes 1 to 256.
VALID_CASES = {
    "config1": lambda: make_config(1),
    "config2": lambda: make_config(2),
    "config3": lambda: make_config(3),
    "config7": lambda: make_config(7),
    "ragged_bits": lambda: make_case(11, prefix_lens=[0, 500, 33, 0, 7], qo_lens=[30, 7, 64, 0, 1],
                                     num_qo_heads=8, num_kv_heads=2, head_dim=128,
                                     mask_kind="tree", max_qo_len=64, extra_indices=9,
                                     mask_pad_bytes=5),
    "ragged_rows": lambda: make_case(12, prefix_lens=[40, 0, 300], qo_lens=[5, 17, 1],
                                     num_qo_heads=8, num_kv_heads=2, head_dim=64,
                                     mask_kind="tree", max_qo_len=17, page_size=1,
                                     mask_layout="rows"),
    "ps256": lambda: make_case(13, prefix_lens=[700, 4100], qo_lens=[19, 31], num_qo_heads=8,
                               num_kv_heads=2, head_dim=128, page_size=256, max_qo_len=31,
                               extra_indices=3),
}


@functools.lru_cache(maxsize=None)
def valid(name):
    return VALID_CASES[name]()


@pytest.mark.parametrize("name", sorted(VALID_CASES))
def test_valid_inputs_pass(gpu_lib, name):
    a = Arrays.of_problem(valid(name))
    assert a.expected() == 0
    status = torch.full((1,), 123, dtype=torch.int32, device="cuda")  # cleared by the call
    got = a.run(status)
    say(f"[check {name}] status={got}")
    assert got == 0


def test_binding_takes_the_tensors_of_a_call(gpu_lib):
    p = valid("ragged_bits")
    t = to_device(p)
    got = B.check_inputs(t["q"], t["k_cache"], t["kv_indptr"], t["kv_indices"], t["last_page_len"],
                         t["qo_indptr"], t["mask"], t["mask_indptr"], max_qo_len=p.max_qo_len)
    assert got == 0


def _planted():
    """One violation per case, with the bits it must give (and only those)."""
    base = Arrays.of_problem(valid("ragged_bits"))  # requests: L 30/7/64/0/1, prefix 0/500/33/0/7
    used = int(base.kv_indptr[-1])
    out = []

    def plant(name, bits, f):
        a = base.copy()
        f(a)
        out.append((name, bits, a))

    plant("kv_indptr_start", KV_INDPTR, lambda a: a.kv_indptr.__setitem__(0, -1))
    # The used range then runs to the capacity, over the poisoned spare slots.
    plant("kv_indptr_past_capacity", KV_INDPTR | KV_INDICES,
          lambda a: a.kv_indptr.__setitem__(-1, a.kv_indices.size + 1))
    plant("kv_indptr_decreasing", KV_INDPTR | QO_LEN,
          lambda a: a.kv_indptr.__setitem__(2, a.kv_indptr[1] - 1))
    plant("page_id_too_large", KV_INDICES, lambda a: a.kv_indices.__setitem__(used - 1, a.num_pages))
    plant("page_id_negative", KV_INDICES, lambda a: a.kv_indices.__setitem__(0, -5))
    plant("unused_slot_ignored", 0, lambda a: a.kv_indices.__setitem__(used, -1))
    plant("last_page_zero", LAST_PAGE, lambda a: a.last_page_len.__setitem__(1, 0))
    plant("last_page_past_page", LAST_PAGE, lambda a: a.last_page_len.__setitem__(1, a.page_size + 1))
    plant("empty_request_last_page_free", 0, lambda a: a.last_page_len.__setitem__(3, 77))
    plant("qo_indptr_start", QO_INDPTR, lambda a: a.qo_indptr.__setitem__(0, 1))
    plant("qo_indptr_end", QO_INDPTR, lambda a: a.qo_indptr.__setitem__(-1, a.tokens - 1))
    plant("qo_indptr_decreasing", QO_INDPTR, lambda a: a.qo_indptr.__setitem__(4, a.qo_indptr[3] - 1))
    plant("qo_len_over_bound", QO_LEN, lambda a: setattr(a, "max_qo_len", 63))
    # Request 0 has no prefix: its 30 drafts fill its pages exactly, so a
    # shorter last page leaves fewer keys than drafts.
    plant("qo_len_over_keys", QO_LEN, lambda a: a.last_page_len.__setitem__(0, a.last_page_len[0] - 1))
    plant("mask_past_end", MASK, lambda a: a.mask_indptr.__setitem__(2, a.num_mask_bytes - 8))
    plant("mask_negative", MASK, lambda a: a.mask_indptr.__setitem__(1, -1))
    plant("everything", KV_INDPTR | KV_INDICES | LAST_PAGE | QO_INDPTR | QO_LEN | MASK,
          lambda a: (a.kv_indptr.__setitem__(0, -1), a.kv_indices.__setitem__(3, -2),
                     a.last_page_len.__setitem__(2, 0), a.qo_indptr.__setitem__(0, 2),
                     a.mask_indptr.__setitem__(4, 1 << 30), setattr(a, "max_qo_len", 10)))
    return out


PLANTED = _planted()


@pytest.mark.parametrize("name,bits,a", PLANTED, ids=[n for n, _, _ in PLANTED])
def test_planted_violation_gives_its_bit(gpu_lib, name, bits, a):
    assert a.expected() == bits, "the planted case must break exactly the rules named"
    got = a.run()
    say(f"[check planted {name}] want={bits} got={got}")
    assert got == bits


def test_rows_layout_segment_covers_prefix_and_drafts(gpu_lib):
    """Full byte rows need L * kv_len bytes per request: the last request's
    segment one byte short is reported."""
    a = Arrays.of_problem(valid("ragged_rows"))
    L = int(a.qo_indptr[-1] - a.qo_indptr[-2])
    kv_len = int((a.kv_indptr[-1] - a.kv_indptr[-2] - 1) * a.page_size + a.last_page_len[-1])
    assert int(a.mask_indptr[-2]) + L * kv_len <= a.num_mask_bytes
    a.mask_indptr[-2] = a.num_mask_bytes - L * kv_len + 1
    assert a.expected() == MASK
    assert a.run() == MASK


def test_many_requests_and_pages_use_the_whole_grid(gpu_lib):
    """More requests and page ids than one pass of the launch covers (the
    grid is capped at 1024 workgroups of 256): a violation in the last
    request and at the last used page id is still seen."""
    g = np.random.default_rng(5)
    batch = 300_000
    pages_per = g.integers(1, 3, batch)
    kv_indptr = np.concatenate([[0], np.cumsum(pages_per)]).astype(np.int32)
    used = int(kv_indptr[-1])
    num_pages = used + 100
    kv_indices = g.permutation(num_pages)[:used].astype(np.int32)
    lpl = g.integers(1, 17, batch).astype(np.int32)
    qo_lens = np.minimum(g.integers(0, 3, batch), lpl)
    qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int32)
    a = Arrays(kv_indptr=kv_indptr, kv_indices=kv_indices, last_page_len=lpl, qo_indptr=qo_indptr,
               num_pages=num_pages, page_size=16, max_qo_len=2)
    assert a.expected() == 0 and a.run() == 0
    b = a.copy()
    b.kv_indices[used - 1] = num_pages
    b.last_page_len[batch - 1] = 17
    assert b.expected() == KV_INDICES | LAST_PAGE
    assert b.run() == KV_INDICES | LAST_PAGE


def test_random_corruptions_match_the_host_walk(gpu_lib):
    """Seeded random edits of every array (one to three per case): the device
    bits equal the host walk's."""
    g = np.random.default_rng(17)
    bases = [Arrays.of_problem(valid(n)) for n in ("ragged_bits", "ragged_rows", "config3", "ps256")]
    seen = 0
    for case in range(60):
        a = bases[case % len(bases)].copy()
        for _ in range(int(g.integers(1, 4))):
            which = int(g.integers(0, 5 if a.mask_indptr is not None else 4))
            arr = [a.kv_indptr, a.kv_indices, a.last_page_len, a.qo_indptr, a.mask_indptr][which]
            i = int(g.integers(0, arr.size))
            v = int(arr[i]) + int(g.choice([-300, -2, -1, 1, 2, 300, 1 << 20]))
            arr[i] = min(max(v, -(1 << 31)), (1 << 31) - 1)
        want = a.expected()
        got = a.run()
        seen |= want
        assert got == want, (case, want, got)
    assert seen == KV_INDPTR | KV_INDICES | LAST_PAGE | QO_INDPTR | QO_LEN | MASK


def test_check_in_a_hip_graph(gpu_lib):
    """The clear and check kernels capture into a graph: replays after the
    arrays change in place report the new contents, a replay after a failing
    one starts from a cleared word, and eager calls run between replays."""
    import ctypes

    a = Arrays.of_problem(valid("ragged_bits"))
    used = int(a.kv_indptr[-1])
    dev = {k: torch.from_numpy(np.ascontiguousarray(getattr(a, k))).cuda()
           for k in ("kv_indptr", "kv_indices", "last_page_len", "qo_indptr", "mask_indptr")}
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    problem = B.make_problem(batch=len(a.kv_indptr) - 1, num_qo_heads=a.hq, num_kv_heads=a.hkv,
                             head_dim=a.d, page_size=a.page_size, num_pages=a.num_pages,
                             num_kv_indices=a.kv_indices.size, num_qo_tokens=a.tokens,
                             max_qo_len=a.max_qo_len, q_dtype=B.VAT_BF16, kv_dtype=B.VAT_BF16,
                             has_mask=1, num_mask_bytes=a.num_mask_bytes, num_cus=1)
    lib = B.load()

    def enqueue():
        st = lib.vat_check_inputs(ctypes.byref(problem), dev["kv_indptr"].data_ptr(),
                                  dev["kv_indices"].data_ptr(), dev["last_page_len"].data_ptr(),
                                  dev["qo_indptr"].data_ptr(), dev["mask_indptr"].data_ptr(),
                                  status.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == 0

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        enqueue()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enqueue()
    steps = [
        (lambda: dev["kv_indices"].__setitem__(used - 1, a.num_pages), KV_INDICES),
        (lambda: dev["kv_indices"].__setitem__(used - 1, int(a.kv_indices[used - 1])), 0),
        (lambda: dev["last_page_len"].__setitem__(1, 0), LAST_PAGE),
        (lambda: dev["mask_indptr"].__setitem__(2, -4), LAST_PAGE | MASK),
        (lambda: (dev["last_page_len"].__setitem__(1, int(a.last_page_len[1])),
                  dev["mask_indptr"].__setitem__(2, int(a.mask_indptr[2]))), 0),
    ]
    for rep, (change, want) in enumerate(steps):
        change()
        status.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        got = int(status.item())
        say(f"[check graph replay {rep}] want={want} got={got}")
        assert got == want
        # Eager work between replays: a check of the unchanged valid arrays.
        assert Arrays.of_problem(valid("ragged_bits")).run() == 0


def test_verify_attention_check_option(gpu_lib):
    """verify_attention(check=True): valid arrays give bitwise the plain
    call's result; a page id out of range raises VatContentError with its bit
    before the attention kernels are enqueued (out keeps its contents)."""
    p = valid("ragged_bits")
    t = to_device(p)
    kw = dict(mask=t["mask"], mask_indptr=t["mask_indptr"], sm_scale=p.sm_scale,
              max_qo_len=p.max_qo_len)
    args = lambda tt: (tt["q"], tt["k_cache"], tt["v_cache"], tt["kv_indptr"], tt["kv_indices"],
                       tt["last_page_len"], tt["qo_indptr"])
    o0, l0 = B.verify_attention(*args(t), **kw)
    o1, l1 = B.verify_attention(*args(t), check=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)
    bad = dict(t)
    bad["kv_indices"] = t["kv_indices"].clone()
    bad["kv_indices"][int(p.kv_indptr[-1]) - 1] = p.num_pages
    out = torch.full_like(t["q"], 7.0)
    with pytest.raises(B.VatContentError) as err:
        B.verify_attention(*args(bad), check=True, out=out, **kw)
    say(f"[check option] {err.value}")
    assert err.value.bits == KV_INDICES
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
