"""The oracle spread over (request, KV head) work items in worker processes.

Test and measurement infrastructure only. Each work item is one request and
one KV head. Its sub-problem holds

* the request's query rows of that KV head's G query heads,
* the request's pages of that KV head, in the request's key order,
* the request's mask segment and RoPE rows.

Each worker runs the unchanged oracle (``oracle.verify_attention``) on the
sub-problem with one BLAS thread. The parent places each item's rows and
heads in the full result.

The split rests on two invariants the oracle's own tests pin bit for bit:
a request's result does not depend on where its pages sit in the pool, and
KV heads (with their query-head groups) are independent. So the result
equals one direct oracle call bitwise.

Workers are started with "spawn": they never inherit a parent that has
initialised the GPU, and they import only NumPy and the oracle.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import time
from typing import Iterator, Optional, Sequence, Tuple

import numpy as np

# One GPU's share of the host's cores on the GPU machines.
MAX_WORKERS = 16


def default_workers() -> int:
    """Cores this process may run on, capped at one GPU's share."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_WORKERS))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _init_worker():
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except ImportError:
        pass


def _run_item(item):
    from oracle import verify_attention as oracle_va

    b, h, sub = item
    out, lse = oracle_va(sub["q"], sub["k"], sub["v"], sub["kv_indptr"], sub["kv_indices"],
                         sub["last_page_len"], sub["qo_indptr"], sub["mask"], sub["mask_indptr"],
                         sm_scale=sub["sm_scale"], k_scale=sub["k_scale"],
                         v_scale=sub["v_scale"], q_dtype=sub["q_dtype"],
                         kv_dtype=sub["kv_dtype"], mask_layout=sub["mask_layout"],
                         q_cos_sin=sub["q_cos_sin"])
    return b, h, out, lse


def sub_problem(p, b: int, h: int, q_cos_sin=None) -> Optional[dict]:
    """Request b's work for KV head h as a one-request, one-KV-head problem,
    or None when the request has no query rows."""
    t0, t1 = int(p.qo_indptr[b]), int(p.qo_indptr[b + 1])
    if t1 <= t0:
        return None
    G = p.num_qo_heads // p.num_kv_heads
    pages = np.asarray(p.kv_indices[int(p.kv_indptr[b]):int(p.kv_indptr[b + 1])], dtype=np.int64)
    mask = mask_indptr = None
    if p.mask is not None:
        off = int(p.mask_indptr[b])
        mask = np.ascontiguousarray(p.mask[off:])
        mask_indptr = np.array([0, mask.shape[0]], dtype=np.int32)
    return dict(
        q=np.ascontiguousarray(p.q[t0:t1, h * G:(h + 1) * G]),
        k=np.ascontiguousarray(p.k_cache[pages][:, :, h:h + 1]),
        v=np.ascontiguousarray(p.v_cache[pages][:, :, h:h + 1]),
        kv_indptr=np.array([0, pages.shape[0]], dtype=np.int32),
        kv_indices=np.arange(pages.shape[0], dtype=np.int32),
        last_page_len=np.array([int(p.last_page_len[b])], dtype=np.int32),
        qo_indptr=np.array([0, t1 - t0], dtype=np.int32),
        mask=mask, mask_indptr=mask_indptr, mask_layout=p.mask_layout,
        sm_scale=p.sm_scale, k_scale=p.k_scale, v_scale=p.v_scale,
        q_dtype=p.q_dtype, kv_dtype=p.kv_dtype,
        q_cos_sin=None if q_cos_sin is None else np.ascontiguousarray(q_cos_sin[t0:t1]))


def _items(p, requests, q_cos_sin) -> Iterator[Tuple[int, int, dict]]:
    for b in requests:
        for h in range(p.num_kv_heads):
            sub = sub_problem(p, b, h, q_cos_sin)
            if sub is not None:
                yield b, h, sub


class OraclePool:
    """A pool of oracle workers, started once and reused across calls."""

    def __init__(self, workers: Optional[int] = None):
        self.workers = workers or default_workers()
        self._pool = mp.get_context("spawn").Pool(self.workers, initializer=_init_worker)

    def close(self):
        self._pool.close()
        self._pool.join()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def run(self, p, requests: Optional[Sequence[int]] = None, q_cos_sin=None):
        """float64 ``out [T, Hq, D]`` and ``lse [T, Hq]`` of the oracle; rows of
        requests not listed stay 0 / -inf."""
        T, Hq, D = p.q.shape
        G = p.num_qo_heads // p.num_kv_heads
        out = np.zeros((T, Hq, D), dtype=np.float64)
        lse = np.full((T, Hq), -np.inf, dtype=np.float64)
        todo = range(p.batch) if requests is None else requests
        for b, h, o, l in self._pool.imap_unordered(_run_item, _items(p, todo, q_cos_sin)):
            t0, t1 = int(p.qo_indptr[b]), int(p.qo_indptr[b + 1])
            out[t0:t1, h * G:(h + 1) * G] = o
            lse[t0:t1, h * G:(h + 1) * G] = l
        return out, lse

    def timed(self, p, min_seconds: float, requests=None, q_cos_sin=None):
        """Run the whole oracle until ``min_seconds`` have passed (at least
        once); returns the last result, the seconds taken and the repeats."""
        reps = 0
        t0 = time.perf_counter()
        while True:
            res = self.run(p, requests, q_cos_sin)
            reps += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
        return res, time.perf_counter() - t0, reps


class InProcessOracle:
    """The same interface without worker processes: the oracle runs in this
    process with one BLAS thread. For runs where starting processes is not
    allowed (a profiler that has initialised the GPU before the program
    starts must not see this process fork and exec)."""

    workers = 1

    def close(self):
        pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def run(self, p, requests: Optional[Sequence[int]] = None, q_cos_sin=None):
        from threadpoolctl import threadpool_limits

        from oracle import verify_attention as oracle_va

        with threadpool_limits(1):
            return oracle_va(p.q, p.k_cache, p.v_cache, p.kv_indptr, p.kv_indices, p.last_page_len,
                             p.qo_indptr, p.mask, p.mask_indptr, sm_scale=p.sm_scale,
                             k_scale=p.k_scale, v_scale=p.v_scale, q_dtype=p.q_dtype,
                             kv_dtype=p.kv_dtype, requests=requests, mask_layout=p.mask_layout,
                             q_cos_sin=q_cos_sin)

    timed = OraclePool.timed
