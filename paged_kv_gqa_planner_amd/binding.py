"""Thin ctypes binding of ``libvat.so`` with the C ABI's names.

Argument marshalling only: torch tensors become device pointers, the current
HIP stream is passed through, status codes become exceptions. All compute
runs in the library's kernels; if the library is missing this module raises
instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvat.so")

VAT_F32, VAT_BF16, VAT_FP8_E4M3FN = 0, 1, 2
STATUS = {
    0: "VAT_OK", 1: "VAT_ERR_NULL", 2: "VAT_ERR_SHAPE", 3: "VAT_ERR_UNSUPPORTED",
    4: "VAT_ERR_ALIGN", 5: "VAT_ERR_WORKSPACE", 6: "VAT_ERR_HIP",
}
_VALUE_ERRORS = {1, 2, 3, 4, 5}


class VatProblem(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "num_qo_heads", "num_kv_heads", "head_dim", "page_size", "num_pages",
        "num_kv_indices", "num_qo_tokens", "max_qo_len", "q_dtype", "kv_dtype", "has_mask",
        "num_mask_bytes", "num_cus", "chunk_keys", "rope")]


class VatPlan(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "direct", "kernel", "stages", "slices", "group", "rows", "row_tiles_per_wave", "waves_rows", "waves_keys", "dma_waves",
        "rows_per_block", "row_blocks", "chunk_keys", "num_chunk_ids", "grid_x", "grid_y",
        "threads", "lds_bytes", "merge_grid", "merge_threads", "num_cus")] + [
        ("workspace_bytes", ctypes.c_int64), ("block_order", ctypes.c_int32),
        ("merge_rows", ctypes.c_int32), ("heads_per_group", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class VatError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_lib_status_string(status)})")


class VatValueError(VatError, ValueError):
    pass


_lib = None


def load(path: Optional[str] = None):
    """Load the shared library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    f = ctypes.c_float
    lib.vat_plan.argtypes = [P(VatProblem), P(VatPlan)]
    lib.vat_plan.restype = ctypes.c_int
    lib.vat_workspace_size.argtypes = [P(VatProblem), P(ctypes.c_size_t)]
    lib.vat_workspace_size.restype = ctypes.c_int
    full = [P(VatProblem), vp, vp, vp, vp, vp, vp, vp, vp, vp, f, f, f, vp, vp, vp, ctypes.c_size_t, vp]
    lib.verify_attention.argtypes = full
    lib.verify_attention.restype = ctypes.c_int
    lib.vat_launch_partial.argtypes = full
    lib.vat_launch_partial.restype = ctypes.c_int
    lib.vat_launch_merge.argtypes = [P(VatProblem), vp, vp, vp, f, vp, vp, vp, ctypes.c_size_t, vp]
    lib.verify_attention_rope.argtypes = full[:10] + [vp] + full[10:]
    lib.verify_attention_rope.restype = ctypes.c_int
    lib.vat_launch_partial_rope.argtypes = full[:10] + [vp] + full[10:]
    lib.vat_launch_partial_rope.restype = ctypes.c_int
    lib.vat_append_kv_rope.argtypes = [P(VatProblem), ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp, f, f, vp]
    lib.vat_append_kv_rope.restype = ctypes.c_int
    lib.vat_launch_merge.restype = ctypes.c_int
    lib.vat_append_kv.argtypes = [P(VatProblem), ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp,
                                  f, f, vp]
    lib.vat_append_kv.restype = ctypes.c_int
    lib.verify_attention_noalloc.argtypes = full[:15] + [vp]
    lib.verify_attention_noalloc.restype = ctypes.c_int
    lib.vat_check_inputs.argtypes = [P(VatProblem), vp, vp, vp, vp, vp, vp, vp]
    lib.vat_check_inputs.restype = ctypes.c_int
    lib.vat_read_probe.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.vat_read_probe.restype = ctypes.c_int
    lib.vat_status_string.argtypes = [ctypes.c_int]
    lib.vat_status_string.restype = ctypes.c_char_p
    lib.vat_abi_version.argtypes = []
    lib.vat_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def _lib_status_string(status: int) -> str:
    if _lib is None:
        return ""
    return _lib.vat_status_string(status).decode()


def _check(status: int, where: str):
    if status == 0:
        return
    if status in _VALUE_ERRORS:
        raise VatValueError(status, where)
    raise VatError(status, where)


# ------------------------------------------------------------------ problem description


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return VAT_F32
    if t.dtype == torch.bfloat16:
        return VAT_BF16
    if t.dtype == torch.float8_e4m3fn:
        return VAT_FP8_E4M3FN
    raise ValueError(f"unsupported dtype {t.dtype}")


def make_problem(*, batch, num_qo_heads, num_kv_heads, head_dim, page_size, num_pages,
                 num_kv_indices, num_qo_tokens, max_qo_len, q_dtype, kv_dtype, has_mask,
                 num_mask_bytes=0, num_cus=0, chunk_keys=-1, rope=0) -> VatProblem:
    return VatProblem(batch, num_qo_heads, num_kv_heads, head_dim, page_size, num_pages,
                      num_kv_indices, num_qo_tokens, max_qo_len, q_dtype, kv_dtype,
                      int(has_mask), num_mask_bytes, num_cus, chunk_keys, int(rope))


MASK_LAYOUTS = {"bits": 1, "rows": 2}


def problem_from_tensors(q, k_cache, kv_indptr, kv_indices, mask=None, max_qo_len=None,
                         num_cus=0, chunk_keys=-1, mask_layout="bits", rope=False) -> VatProblem:
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [T, Hq, D] and caches [pages, page_size, Hkv, D]")
    batch = kv_indptr.numel() - 1
    T = q.shape[0]
    if max_qo_len is None:
        # One request holds every query row. With more requests the bound
        # cannot come from shapes alone without overstating it (T - (B - 1)
        # may pass the 64-draft mask limit, and a loose bound inflates the
        # planned rows per KV head), and reading qo_indptr would synchronise:
        # the caller states it.
        if batch > 1 and T > 0:
            raise ValueError("max_qo_len is required when the batch holds more than one "
                             "request (the largest qo_indptr[b+1] - qo_indptr[b])")
        max_qo_len = T if batch > 0 else 0
    return make_problem(
        batch=batch, num_qo_heads=q.shape[1], num_kv_heads=k_cache.shape[2], head_dim=q.shape[2],
        page_size=k_cache.shape[1], num_pages=k_cache.shape[0], num_kv_indices=kv_indices.numel(),
        num_qo_tokens=T, max_qo_len=int(max_qo_len), q_dtype=_dtype_code(q),
        kv_dtype=_dtype_code(k_cache), has_mask=0 if mask is None else MASK_LAYOUTS[mask_layout],
        num_mask_bytes=0 if mask is None else mask.numel(), num_cus=num_cus,
        chunk_keys=chunk_keys, rope=rope)


def vat_plan(problem: VatProblem) -> VatPlan:
    lib = load()
    plan = VatPlan()
    _check(lib.vat_plan(ctypes.byref(problem), ctypes.byref(plan)), "vat_plan")
    return plan


def vat_workspace_size(problem: VatProblem) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    _check(lib.vat_workspace_size(ctypes.byref(problem), ctypes.byref(n)), "vat_workspace_size")
    return int(n.value)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream_handle(stream) -> int:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _check_tensors(q, k_cache, v_cache, idx):
    for name, t in [("q", q), ("k_cache", k_cache), ("v_cache", v_cache)] + idx:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must have one shape and dtype")


def _prepare(q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len, qo_indptr, mask,
             mask_indptr, sm_scale, max_qo_len, out, lse, workspace, chunk_keys, num_cus,
             mask_layout="bits", q_cos_sin=None):
    import torch

    idx = [("kv_indptr", kv_indptr), ("kv_indices", kv_indices), ("last_page_len", last_page_len),
           ("qo_indptr", qo_indptr), ("mask", mask), ("mask_indptr", mask_indptr)]
    _check_tensors(q, k_cache, v_cache, idx)
    for name, t in idx:
        if t is None:
            continue
        want = torch.uint8 if name == "mask" else torch.int32
        if t.dtype != want:
            raise ValueError(f"{name} must be {want}")
    if q_cos_sin is not None:
        if not q_cos_sin.is_cuda or not q_cos_sin.is_contiguous() or q_cos_sin.dtype != torch.float32:
            raise ValueError("q_cos_sin must be a contiguous float32 device tensor")
        if tuple(q_cos_sin.shape) != (q.shape[0], q.shape[2]):
            raise ValueError("q_cos_sin must be [T, D]")
    problem = problem_from_tensors(q, k_cache, kv_indptr, kv_indices, mask, max_qo_len,
                                   num_cus=num_cus, chunk_keys=chunk_keys,
                                   mask_layout=mask_layout, rope=q_cos_sin is not None)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[2])
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    need = vat_workspace_size(problem)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return problem, float(sm_scale), out, lse, workspace, ws_bytes


def verify_attention(q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len, qo_indptr,
                     mask=None, mask_indptr=None, sm_scale: Optional[float] = None,
                     k_scale: float = 1.0, v_scale: float = 1.0, max_qo_len: Optional[int] = None,
                     out=None, lse=None, workspace=None, chunk_keys: int = -1, num_cus: int = 0,
                     stream=None, mask_layout: str = "bits",
                     q_cos_sin=None, check: bool = False) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Multi-query verification attention over a paged KV cache; returns (out, lse).

    ``sm_scale`` defaults to ``head_dim ** -0.5``; ``max_qo_len`` (the largest
    request's query-token count) may be omitted only for a batch of one
    request, where it is T, or when there are no query tokens; ``chunk_keys`` -1 lets the planner
    choose the prefix split, 0 forces one work item per request (direct
    output), a positive multiple of 16 forces that chunk length.
    ``mask_layout``: "bits" (packed L x L blocks) or "rows" (sglang's full
    byte rows). ``q_cos_sin`` ([T, D] float32 cos/sin rows of the query
    tokens' positions) rotates the queries by RoPE inside the kernel.
    ``check`` (a debugging aid) first runs the device-content check
    (``vat_check_inputs``) on the same stream, waits for it and raises
    ``VatContentError`` naming the broken rules before anything else is
    enqueued.
    """
    lib = load()
    problem, sm, out, lse, workspace, ws_bytes = _prepare(
        q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len, qo_indptr, mask, mask_indptr,
        sm_scale, max_qo_len, out, lse, workspace, chunk_keys, num_cus, mask_layout, q_cos_sin)
    if check:
        bits = _run_check(problem, kv_indptr, kv_indices, last_page_len, qo_indptr, mask,
                          mask_indptr, None, stream)
        if bits:
            raise VatContentError(bits)
    head = (ctypes.byref(problem), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_indptr),
            _ptr(kv_indices), _ptr(last_page_len), _ptr(qo_indptr), _ptr(mask), _ptr(mask_indptr))
    tail = (sm, float(k_scale), float(v_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
            _stream_handle(stream))
    if q_cos_sin is None:
        _check(lib.verify_attention(*head, *tail), "verify_attention")
    else:
        _check(lib.verify_attention_rope(*head, _ptr(q_cos_sin), *tail), "verify_attention_rope")
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20


def verify_attention_noalloc(q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                             qo_indptr, mask=None, mask_indptr=None,
                             sm_scale: Optional[float] = None, k_scale: float = 1.0,
                             v_scale: float = 1.0, max_qo_len: Optional[int] = None, out=None,
                             lse=None, num_cus: int = 0, stream=None, mask_layout: str = "bits"):
    """``verify_attention`` through the C entry point that allocates nothing:
    its workspace is the library's static per-device scratch array. ``out``
    and ``lse`` are allocated here when not given."""
    import torch

    lib = load()
    idx = [("kv_indptr", kv_indptr), ("kv_indices", kv_indices), ("last_page_len", last_page_len),
           ("qo_indptr", qo_indptr), ("mask", mask), ("mask_indptr", mask_indptr)]
    _check_tensors(q, k_cache, v_cache, idx)
    problem = problem_from_tensors(q, k_cache, kv_indptr, kv_indices, mask, max_qo_len,
                                   num_cus=num_cus, mask_layout=mask_layout)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[2])
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    st = lib.verify_attention_noalloc(
        ctypes.byref(problem), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_indptr),
        _ptr(kv_indices), _ptr(last_page_len), _ptr(qo_indptr), _ptr(mask), _ptr(mask_indptr),
        float(sm_scale), float(k_scale), float(v_scale), _ptr(out), _ptr(lse),
        _stream_handle(stream))
    _check(st, "verify_attention_noalloc")
    return out, lse


def append_problem(k_new, k_cache, kv_indptr, kv_indices, max_qo_len=None,
                   num_cus=0) -> VatProblem:
    """Problem record for vat_append_kv from the tensors' shapes."""
    if k_new.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("k_new must be [T, Hkv, D] and caches [pages, page_size, Hkv, D]")
    batch = kv_indptr.numel() - 1
    T = k_new.shape[0]
    if max_qo_len is None:
        max_qo_len = T - (batch - 1) if batch > 0 else 0
    hkv, d = k_cache.shape[2], k_cache.shape[3]
    return make_problem(batch=batch, num_qo_heads=hkv, num_kv_heads=hkv, head_dim=d,
                        page_size=k_cache.shape[1], num_pages=k_cache.shape[0],
                        num_kv_indices=kv_indices.numel(), num_qo_tokens=T,
                        max_qo_len=max(int(max_qo_len), 0), q_dtype=_dtype_code(k_new),
                        kv_dtype=_dtype_code(k_cache), has_mask=0, num_cus=num_cus)


def _append_args(k_new, v_new, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                 qo_indptr, k_scale, v_scale, max_qo_len, stream, num_cus=0, k_cos_sin=None):
    import torch

    idx = [("kv_indptr", kv_indptr), ("kv_indices", kv_indices),
           ("last_page_len", last_page_len), ("qo_indptr", qo_indptr)]
    _check_tensors(k_new, k_cache, v_cache, idx + [("v_new", v_new)])
    for name, t in idx:
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be torch.int32")
    if v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise ValueError("k_new and v_new must have one shape and dtype")
    if k_new.shape[1:] != k_cache.shape[2:]:
        raise ValueError("k_new rows must be [Hkv, D] of the cache")
    problem = append_problem(k_new, k_cache, kv_indptr, kv_indices, max_qo_len, num_cus)
    head = (ctypes.byref(problem), _dtype_code(k_new), _ptr(k_new), _ptr(v_new),
            _ptr(k_cache), _ptr(v_cache), _ptr(kv_indptr), _ptr(kv_indices),
            _ptr(last_page_len), _ptr(qo_indptr))
    tail = (float(k_scale), float(v_scale), _stream_handle(stream))
    if k_cos_sin is None:
        return problem, head + tail, False
    if not k_cos_sin.is_cuda or not k_cos_sin.is_contiguous() or k_cos_sin.dtype != torch.float32:
        raise ValueError("k_cos_sin must be a contiguous float32 device tensor")
    if tuple(k_cos_sin.shape) != (k_new.shape[0], k_new.shape[2]):
        raise ValueError("k_cos_sin must be [T, D]")
    return problem, head + (_ptr(k_cos_sin),) + tail, True


def append_kv(k_new, v_new, k_cache, v_cache, kv_indptr, kv_indices, last_page_len, qo_indptr,
              k_scale: float = 1.0, v_scale: float = 1.0, max_qo_len: Optional[int] = None,
              stream=None, num_cus: int = 0, k_cos_sin=None):
    """Write the drafts' keys/values ``[T, Hkv, D]`` (fp32 or bf16) into the
    paged caches in place, stored as ``x / scale`` rounded to the cache dtype.
    ``max_qo_len`` defaults to the shape-only bound ``T - (B - 1)``;
    ``num_cus`` 0 sizes the launch for the current device; ``k_cos_sin``
    ([T, D] float32 cos/sin rows of the drafts' positions) rotates the keys by
    RoPE first."""
    lib = load()
    problem, args, rope = _append_args(k_new, v_new, k_cache, v_cache, kv_indptr, kv_indices,
                                       last_page_len, qo_indptr, k_scale, v_scale, max_qo_len,
                                       stream, num_cus, k_cos_sin)
    fn = lib.vat_append_kv_rope if rope else lib.vat_append_kv
    _check(fn(*args), "vat_append_kv")
    return k_cache, v_cache


class PreparedAppend:
    """vat_append_kv with every argument fixed (checked once), for timing."""

    def __init__(self, k_new, v_new, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                 qo_indptr, k_scale=1.0, v_scale=1.0, max_qo_len=None, stream=None, num_cus=0,
                 k_cos_sin=None):
        self.lib = load()
        self.keep = (k_new, v_new, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                     qo_indptr, k_cos_sin)
        self.problem, self.args, rope = _append_args(k_new, v_new, k_cache, v_cache, kv_indptr,
                                                     kv_indices, last_page_len, qo_indptr,
                                                     k_scale, v_scale, max_qo_len, stream,
                                                     num_cus, k_cos_sin)
        self.fn = self.lib.vat_append_kv_rope if rope else self.lib.vat_append_kv

    def __call__(self):
        _check(self.fn(*self.args), "vat_append_kv")


class PreparedCall:
    """A call with every pointer fixed, launched without Python-side checks.

    Used for timing: ``partial()`` and ``merge()`` enqueue the two kernels
    separately, ``__call__`` the whole path.
    """

    def __init__(self, q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len, qo_indptr,
                 mask=None, mask_indptr=None, sm_scale=None, k_scale=1.0, v_scale=1.0,
                 max_qo_len=None, out=None, lse=None, workspace=None, chunk_keys=-1, num_cus=0,
                 stream=None, mask_layout="bits", q_cos_sin=None):
        self.lib = load()
        (self.problem, self.sm, self.out, self.lse, self.workspace,
         self.ws_bytes) = _prepare(q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len,
                                   qo_indptr, mask, mask_indptr, sm_scale, max_qo_len, out, lse,
                                   workspace, chunk_keys, num_cus, mask_layout, q_cos_sin)
        self.keep = (q, k_cache, v_cache, kv_indptr, kv_indices, last_page_len, qo_indptr, mask,
                     mask_indptr, q_cos_sin)
        self.rope = q_cos_sin is not None
        self.k_scale = float(k_scale)
        self.v_scale = float(v_scale)
        self.stream = _stream_handle(stream)
        self.plan = vat_plan(self.problem)
        self.args = (ctypes.byref(self.problem), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                     _ptr(kv_indptr), _ptr(kv_indices), _ptr(last_page_len), _ptr(qo_indptr),
                     _ptr(mask), _ptr(mask_indptr), self.sm, self.k_scale, self.v_scale,
                     _ptr(self.out), _ptr(self.lse), _ptr(self.workspace), self.ws_bytes,
                     self.stream)
        self.rope_args = self.args[:10] + (_ptr(q_cos_sin),) + self.args[10:]
        self.merge_args = (ctypes.byref(self.problem), _ptr(kv_indptr), _ptr(last_page_len),
                           _ptr(qo_indptr), self.v_scale, _ptr(self.out), _ptr(self.lse),
                           _ptr(self.workspace), self.ws_bytes, self.stream)

    def __call__(self):
        if self.rope:
            _check(self.lib.verify_attention_rope(*self.rope_args), "verify_attention_rope")
        else:
            _check(self.lib.verify_attention(*self.args), "verify_attention")
        return self.out, self.lse

    def call_on(self, stream):
        """The whole call enqueued on ``stream`` (e.g. a graph-capture stream)."""
        h = _stream_handle(stream)
        if self.rope:
            _check(self.lib.verify_attention_rope(*self.rope_args[:-1], h), "verify_attention_rope")
        else:
            _check(self.lib.verify_attention(*self.args[:-1], h), "verify_attention")
        return self.out, self.lse

    def partial(self):
        if self.rope:
            _check(self.lib.vat_launch_partial_rope(*self.rope_args), "vat_launch_partial_rope")
        else:
            _check(self.lib.vat_launch_partial(*self.args), "vat_launch_partial")

    def merge(self):
        _check(self.lib.vat_launch_merge(*self.merge_args), "vat_launch_merge")


CHECK_BITS = {1: "kv_indptr", 2: "kv_indices", 4: "last_page_len", 8: "qo_indptr", 16: "qo_len",
              32: "mask"}


class VatContentError(ValueError):
    """Device contents break the contract; ``bits`` is the VAT_CHECK_* OR."""

    def __init__(self, bits: int):
        self.bits = bits
        names = [n for b, n in CHECK_BITS.items() if bits & b]
        super().__init__(f"device contents break the contract: {', '.join(names)} (bits {bits})")


def _run_check(problem, kv_indptr, kv_indices, last_page_len, qo_indptr, mask, mask_indptr,
               status, stream) -> int:
    import torch

    idx = [("kv_indptr", kv_indptr), ("kv_indices", kv_indices), ("last_page_len", last_page_len),
           ("qo_indptr", qo_indptr), ("mask_indptr", mask_indptr)]
    for name, t in idx:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.int32:
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    batch = kv_indptr.numel() - 1
    if qo_indptr.numel() != batch + 1 or last_page_len.numel() != batch:
        raise ValueError("qo_indptr must have batch + 1 entries and last_page_len batch")
    if mask is not None and (mask_indptr is None or mask_indptr.numel() < batch):
        raise ValueError("a mask needs mask_indptr with an offset per request")
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=kv_indptr.device)
    lib = load()
    _check(lib.vat_check_inputs(ctypes.byref(problem), _ptr(kv_indptr), _ptr(kv_indices),
                                _ptr(last_page_len), _ptr(qo_indptr), _ptr(mask_indptr),
                                _ptr(status), _stream_handle(stream)), "vat_check_inputs")
    s = stream if stream is not None else torch.cuda.current_stream()
    s.synchronize()
    return int(status.item())


def check_inputs(q, k_cache, kv_indptr, kv_indices, last_page_len, qo_indptr, mask=None,
                 mask_indptr=None, max_qo_len=None, mask_layout="bits", status=None,
                 stream=None) -> int:
    """Check the device-content contract of a call's index arrays and mask
    offsets on the device (a debugging aid) and return the OR of the
    VAT_CHECK_* bits of the rules they break (0: none; ``CHECK_BITS`` names
    each bit). Shapes come from the tensors as in ``verify_attention``;
    ``status`` is an optional one-element int32 device tensor to write into.
    Synchronises the stream to read the result."""
    problem = problem_from_tensors(q, k_cache, kv_indptr, kv_indices, mask, max_qo_len,
                                   num_cus=1, mask_layout=mask_layout)
    return _run_check(problem, kv_indptr, kv_indices, last_page_len, qo_indptr, mask, mask_indptr,
                      status, stream)


def read_probe(buf, sink, stream=None):
    """Enqueue one streaming read of the whole device tensor ``buf`` (a
    measurement aid: the plainest HBM read, for the roofline); ``sink`` is a
    one-element int32 device tensor."""
    lib = load()
    n = buf.numel() * buf.element_size()
    _check(lib.vat_read_probe(_ptr(buf), n, _ptr(sink), _stream_handle(stream)), "vat_read_probe")
