"""Throughput of multi-query verification attention over a paged KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5] [--prefix 4096]

The default workload is config 5 -- bf16 queries over an fp8 e4m3 KV cache,
batch 64, prefixes U[512, 8192], dynamic draft lengths -- the largest of the
KV-bound verify workloads; ``--config`` picks any other.

One step is one ``verify_attention`` call -- partial kernel plus log-sum-exp
merge -- over one batch of seeded synthetic inputs already resident in HBM.
Successive steps read different batches: ``--copies`` physically permuted
copies of the page pool (each with its own page table), together larger than
the 256 MB Infinity Cache, so every step streams its KV cache from HBM.

Before timing, the output of every copy is checked: copy 0 against the CPU
oracle at the parity tolerances (every request), the others bitwise against
copy 0. Timings:

* ``ms_per_step`` / ``value``: K steps back to back on one stream, averaged;
  the stream is first held by a short GPU sleep so that the host has queued
  all K steps before the first one starts and HIP events measure GPU time
  only.
* ``roofline``: K partial kernels alone, timed the same way, give that
  kernel's average duration, from which the roofline fraction is computed
  with the algorithmic bytes (KV-bound workloads) or FLOPs (prefill shapes).
* ``per_call``: one call captured in a HIP graph (one graph per pool copy)
  and replayed K times with a cache flush (1 GiB written, then read) before
  each replay: median, p10 and p90 of the per-call GPU times, plus the
  median of K warm replays without a flush.
* ``hbm_read_probe``: the library's plain streaming-read kernel over 2 GiB,
  the HBM read rate reachable on this chip, beside the published peak.

The oracle (NumPy float64) runs on the host's cores, spread over (request,
KV head) items in worker processes with one BLAS thread each, on the whole
workload: its wall time is the ``cpu_baseline`` leg, with the worker count
and CPU model stated.

``--op append`` times the step before the path instead: ``vat_append_kv``
writing the workload's draft keys and values (fresh seeded values, bf16, or
fp32 for the fp32 workload) into its paged caches, rounded to the cache
dtype. Copies of the sources and of the page table (a permutation of the
pool per copy) rotate over the steps so successive steps write different
pages. Every copy's result is checked bit for bit (copy 0 against the
oracle, the others against copy 0 through their own page tables).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
METRIC = "verified query-tokens/s + achieved KV-read HBM GB/s (% of peak), 1 MI355X"
WORKLOAD_NAMES = {
    1: "tiny MQA verify fp32: B2 Hq4 Hkv1 D64, prefix 37/100, L4 causal, page 16 (32-page pool)",
    2: "GQA chain verify bf16: B8 Hq32 Hkv8 D128, prefix 2048, L5 causal, page 16",
    3: "tree verify bf16 at batch 1: Hq32 Hkv8 D128, L17 random tree, prefix {p}, page 16",
    4: "GQA causal prefill bf16: B10 x 1024 packed, Hq64 Hkv8 D128, page 16",
    5: "bf16 Q + fp8 e4m3 KV dynamic-draft verify: B64 Hq32 Hkv8 D128, prefix U[512,8192], L U{{1..8}}, page 16",
    6: "GQA decode bf16: B64 Hq32 Hkv8 D128, prefix U[512,8192], L1, page 16",
    7: "wide tree verify bf16: B4 Hq64 Hkv8 D128, L64 random tree (512 rows per KV head), prefix 8192, page 16",
}
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def _code_hash(names) -> str:
    """sha256 (first 16 hex) of the code of these csrc files with comments
    and blank space removed, so a comment edit keeps recorded profiles valid
    while any change to the code invalidates them."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "paged_kv_gqa_planner_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    return _code_hash(("device_common.h", "stream_kernel.hip", "tile_kernel.hip",
                       "merge_kernel.hip", "plan.cpp", "plan.h", "api.hip"))


def algorithmic_work(p):
    """KV bytes (every cached entry of every request, K and V, once per KV
    head) and the FLOPs of QK^T and PV over the visible (query, key) pairs."""
    from workloads import kv_bytes

    kvb = kv_bytes(p)
    pairs = 0
    for b in range(p.batch):
        L = int(p.qo_indptr[b + 1] - p.qo_indptr[b])
        pages = int(p.kv_indptr[b + 1] - p.kv_indptr[b])
        kv_len = 0 if pages == 0 else (pages - 1) * p.page_size + int(p.last_page_len[b])
        prefix = kv_len - L
        if p.mask is None:
            pairs += L * prefix + L * (L + 1) // 2
        else:
            seg = p.mask[int(p.mask_indptr[b]):]
            bits = sum(int((seg[i // 8] >> (i % 8)) & 1) for i in range(L * L))
            pairs += L * prefix + bits
    flops = 4 * p.head_dim * p.num_qo_heads * pairs
    return kvb, flops


def profiled_traffic(key: str, src_hash: str):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) recorded in
    profiles/traffic.json for this workload, or None when the record is
    missing or was taken on different kernel sources."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    with open(PROFILE_TRAFFIC) as f:
        entry = json.load(f).get(key)
    if entry and entry.get("source_hash") == src_hash:
        return entry.get("bytes_per_launch")
    return None


def append_source_hash() -> str:
    return _code_hash(("device_common.h", "append_kernel.hip", "plan.h", "api.hip"))


def hold_stream_timer(torch, K, launches, host_per_launch):
    """Average GPU ms per launch of K back-to-back launches (``launches(i)``
    enqueues launch i); the stream is held by a GPU sleep while the host
    queues them, so the events time GPU work only."""
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    torch.cuda._sleep(1_000_000)
    c1.record()
    torch.cuda.synchronize()
    cycles_per_ms = 1_000_000 / max(c0.elapsed_time(c1), 1e-3)
    hold_ms = 20.0 + 2.0 * K * host_per_launch * 1e3
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(hold_ms * cycles_per_ms))
    start.record()
    t_enq = time.perf_counter()
    for i in range(K):
        launches(i)
    end.record()
    enqueue_ms = (time.perf_counter() - t_enq) * 1e3
    torch.cuda.synchronize()
    return start.elapsed_time(end) / K, enqueue_ms < hold_ms


def bench_append(args, p, dev):
    """--op append: the draft key/value write into the paged cache."""
    import torch

    from oracle import append_kv as oracle_append
    from paged_kv_gqa_planner_amd import binding
    from tests.gpu_helpers import to_device
    from workloads import make_append_inputs

    src = "f32" if p.kv_dtype == "f32" else "bf16"
    spread = 2.0 if p.kv_dtype == "e4m3" else 1.0
    ks, vs = p.k_scale, p.v_scale
    T = p.num_tokens
    k_rows = None
    if args.rope:
        from workloads import rope_cos_sin, rope_positions

        k_rows = rope_cos_sin(rope_positions(p), p.head_dim)
    k_new, v_new = make_append_inputs(p, src, seed=1000 + args.config, spread=spread)
    base = to_device(p, dev)
    se = 4 if src == "f32" else 2
    ce = {"f32": 4, "bf16": 2, "e4m3": 1}[p.kv_dtype]
    elems = 2 * T * p.num_kv_heads * p.head_dim
    alg_bytes = elems * (se + ce) + 4 * T  # sources read, cache rows written, page ids
    touched = elems * (se + ce)
    copies = args.copies or max(2, math.ceil((1 << 30) / max(touched, 1)))
    copies = min(copies, 64)

    def dev_src(a):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if src == "bf16" else np.float32))
        return (t.view(torch.bfloat16) if src == "bf16" else t).to(dev)

    gen = torch.Generator(device="cpu").manual_seed(4321)
    used = int(p.kv_indptr[-1])
    calls, tables = [], []
    for i in range(copies):
        if i == 0:
            idx = base["kv_indices"]
        else:
            perm = torch.randperm(p.num_pages, generator=gen).to(dev)
            idx = base["kv_indices"].clone()
            idx[:used] = perm[base["kv_indices"][:used].long()].to(torch.int32)
        kn, vn = dev_src(k_new), dev_src(v_new)
        tables.append(idx)
        calls.append(binding.PreparedAppend(kn, vn, base["k_cache"], base["v_cache"],
                                            base["kv_indptr"], idx, base["last_page_len"],
                                            base["qo_indptr"], k_scale=ks, v_scale=vs,
                                            max_qo_len=p.max_qo_len,
                                            k_cos_sin=None if k_rows is None
                                            else torch.from_numpy(k_rows).to(dev)))
    torch.cuda.synchronize()

    def raw(t):
        return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else (
            t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32))

    # ---- verification. Copy 0 on a fresh cache against the oracle (every
    # byte); each other copy's written rows, read back through its own page
    # table, against copy 0's.
    calls[0]()
    torch.cuda.synchronize()
    got_k = raw(base["k_cache"]).cpu().numpy()
    got_v = raw(base["v_cache"]).cpu().numpy()
    t_cpu = time.perf_counter()
    reps = 0
    from threadpoolctl import threadpool_limits

    with threadpool_limits(1):
        while True:
            want_k, want_v = oracle_append(k_new, v_new, src, p.k_cache, p.v_cache, p.kv_dtype,
                                           p.kv_indptr, p.kv_indices, p.last_page_len,
                                           p.qo_indptr, p.page_size, k_scale=ks, v_scale=vs,
                                           k_cos_sin=k_rows)
            reps += 1
            if args.no_cpu_baseline or time.perf_counter() - t_cpu >= args.cpu_seconds:
                break
    cpu_s = time.perf_counter() - t_cpu

    def words(a):
        return a.view(np.uint8) if a.dtype == np.uint8 else (
            a.view(np.int16) if a.dtype == np.uint16 else a.view(np.int32))

    verified = bool(np.array_equal(got_k, words(want_k)) and np.array_equal(got_v, words(want_v)))
    rows_page, rows_slot = [], []
    for b in range(p.batch):
        L = int(p.qo_indptr[b + 1] - p.qo_indptr[b])
        pages = int(p.kv_indptr[b + 1] - p.kv_indptr[b])
        kv_len = 0 if pages == 0 else (pages - 1) * p.page_size + int(p.last_page_len[b])
        for t in range(L):
            n = kv_len - L + t
            rows_page.append(int(p.kv_indptr[b]) + n // p.page_size)
            rows_slot.append(n % p.page_size)
    rp = torch.tensor(rows_page, dtype=torch.long, device=dev)
    rs = torch.tensor(rows_slot, dtype=torch.long, device=dev)

    def written(idx):
        pg = idx[rp].long()
        return raw(base["k_cache"])[pg, rs].clone(), raw(base["v_cache"])[pg, rs].clone()

    ref_rows = written(tables[0])
    for i in range(1, copies):
        calls[i]()
        torch.cuda.synchronize()
        k_rows, v_rows = written(tables[i])
        verified = verified and torch.equal(k_rows, ref_rows[0]) and torch.equal(v_rows, ref_rows[1])

    # ---- warmup and timed region (K launches back to back)
    for i in range(args.warmup):
        calls[i % copies]()
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    for i in range(3):
        calls[i % copies]()
    host_per = (time.perf_counter() - t_host) / 3
    torch.cuda.synchronize()
    K = args.steps
    ms, ahead = hold_stream_timer(torch, K, lambda i: calls[i % copies](), host_per)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "appended draft tokens/s (K and V rounded into the paged cache), 1 MI355X",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{src}->{p.kv_dtype}",
        "data": "synthetic",
        "config": {"workload": "draft K/V write of: " +
                   WORKLOAD_NAMES[args.config].format(p=args.prefix) +
                   (", keys rotated by RoPE at their tree positions" if args.rope else ""),
                   "tokens": T, "kv_heads": p.num_kv_heads, "head_dim": p.head_dim,
                   "source_copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": profiled_traffic(f"append:{args.config}" + (":rope" if args.rope else ""),
                                                 append_source_hash()),
                     "kernel": "vat_append",
                     "algorithmic_bytes_per_launch": alg_bytes},
        "verified": verified,
        "gpu_ran_ahead_of_host": bool(ahead),
        "kernel_source": append_source_hash(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = {
            "value": round(T * reps / cpu_s, 1), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"whole workload, repeated {reps}x, {cpu_s:.1f} s, NumPy, one thread"}
    print(json.dumps(line), flush=True)
    if not verified:
        sys.exit(3)


def graph_call_stats(torch, binding, batches, K, flush_bytes):
    """Per-call GPU times (ms) of one ``verify_attention`` call replayed from a
    HIP graph: ``flushed`` with a cache flush before every call (a 1 GiB
    write, then a read of the same buffer, so the 256 MB Infinity Cache and
    the L2s hold nothing of the call's inputs and nothing dirty), and
    ``warm`` with the same call replayed back to back. One graph per pool
    copy; flushed calls rotate over the copies. The stream is held by a GPU
    sleep while the host queues all calls, so each event pair brackets only
    the graph's own GPU work."""
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for call in batches:
            call.call_on(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for call in batches:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call.call_on(torch.cuda.current_stream())
        graphs.append(g)
    torch.cuda.synchronize()
    flush_buf = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def flush(i):
        flush_buf.fill_(i & 0xFF)
        binding.read_probe(flush_buf, sink)

    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    torch.cuda._sleep(1_000_000)
    c1.record()
    torch.cuda.synchronize()
    cycles_per_ms = 1_000_000 / max(c0.elapsed_time(c1), 1e-3)

    def run(with_flush):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        t_host = time.perf_counter()
        for i in range(3):
            if with_flush:
                flush(i)
            graphs[i % len(graphs)].replay()
        host_per = (time.perf_counter() - t_host) / 3
        torch.cuda.synchronize()
        torch.cuda._sleep(int((20.0 + 2.0 * K * host_per * 1e3) * cycles_per_ms))
        for i in range(K):
            if with_flush:
                flush(i)
            ev[i][0].record()
            graphs[i % len(graphs) if with_flush else 0].replay()
            ev[i][1].record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])

    flushed = run(True)
    warm = run(False)
    del graphs
    return flushed, warm


def read_probe_gbps(torch, binding, nbytes, reps=10):
    """HBM read rate of the library's streaming-read probe over ``nbytes``
    (GB/s per launch: median and best of ``reps``)."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        binding.read_probe(buf, sink)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        binding.read_probe(buf, sink)
        b.record()
    torch.cuda.synchronize()
    rates = np.array([nbytes / (a.elapsed_time(b) * 1e-3) / 1e9 for a, b in ev])
    del buf
    return float(np.median(rates)), float(rates.max())


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--op", default="verify", choices=["verify", "append"],
                    help="verify: the attention path; append: the draft K/V cache write")
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5, 6, 7],
                    help="workload (default 5: bf16 Q over an fp8 e4m3 KV cache, batch 64, "
                         "the largest of the KV-bound verify workloads)")
    ap.add_argument("--prefix", type=int, default=4096, help="prefix length for config 3")
    ap.add_argument("--rope", action="store_true",
                    help="rotate the queries by RoPE at their tree positions inside the kernel "
                         "(verify) / the keys at the cache write (append)")
    ap.add_argument("--mask-layout", default="bits", choices=["bits", "rows"],
                    help="tree-mask layout for config 3: packed L x L bits or sglang's full "
                         "byte rows")
    ap.add_argument("--copies", type=int, default=0,
                    help="page-pool copies rotated over the steps (0: enough for >= 1 GiB)")
    ap.add_argument("--chunk-keys", type=int, default=-1, help="planner override (-1: planner)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum host time spent timing the oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph-stats", action="store_true",
                    help="skip the per-call graph-replay timings and the HBM read probe")
    ap.add_argument("--oracle-workers", type=int, default=-1,
                    help="oracle worker processes (-1: the host's cores, at most 16; 0: run the "
                         "oracle in this process and start no process -- required under a "
                         "profiler that initialises the GPU before the program starts)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run K device-to-device copies of MIB MiB (for scaling HBM "
                         "byte counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the kernels run on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    # The oracle's worker processes start before this process touches the GPU.
    pool = None
    if not args.copy_calibration and args.op == "verify":
        from tests.oracle_pool import InProcessOracle, OraclePool

        pool = InProcessOracle() if args.oracle_workers == 0 else OraclePool(
            args.oracle_workers if args.oracle_workers > 0 else None)
    try:
        run_bench(args, pool)
    finally:
        if pool is not None:
            pool.close()


def run_bench(args, pool):
    import torch

    from paged_kv_gqa_planner_amd import binding
    from tests.gpu_helpers import TOL_LSE, TOL_OUT, to_device
    from workloads import make_config

    binding.load()  # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # A plain copy of known size: reads and writes exactly n bytes each.
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": args.steps}), flush=True)
        return

    extra = {"mask_layout": args.mask_layout} if args.config == 3 else {}
    p = make_config(args.config, prefix=args.prefix, **extra)
    if args.op == "append":
        bench_append(args, p, dev)
        return
    kvb, flops = algorithmic_work(p)
    tokens = p.num_tokens
    base = to_device(p, dev)
    pool_bytes = 2 * base["k_cache"].numel() * base["k_cache"].element_size()
    copies = args.copies or max(2, math.ceil((1 << 30) / pool_bytes))

    q_cs = rope_rows = None
    if args.rope:
        from workloads import rope_cos_sin, rope_positions

        rope_rows = rope_cos_sin(rope_positions(p), p.head_dim)
        q_cs = torch.from_numpy(rope_rows).to(dev)
    # Physically permuted copies of the page pool, each with its own table.
    gen = torch.Generator(device="cpu").manual_seed(1234)
    batches = []
    for i in range(copies):
        if i == 0:
            kc, vc, idx = base["k_cache"], base["v_cache"], base["kv_indices"]
        else:
            perm = torch.randperm(p.num_pages, generator=gen).to(dev)
            kc = torch.empty_like(base["k_cache"])
            vc = torch.empty_like(base["v_cache"])
            kc[perm] = base["k_cache"]
            vc[perm] = base["v_cache"]
            idx = base["kv_indices"].clone()
            used = int(p.kv_indptr[-1])
            idx[:used] = perm[base["kv_indices"][:used].long()].to(torch.int32)
        call = binding.PreparedCall(
            base["q"], kc, vc, base["kv_indptr"], idx, base["last_page_len"], base["qo_indptr"],
            base["mask"], base["mask_indptr"], sm_scale=p.sm_scale, k_scale=p.k_scale,
            v_scale=p.v_scale, max_qo_len=p.max_qo_len, chunk_keys=args.chunk_keys,
            mask_layout=p.mask_layout, q_cos_sin=q_cs)
        batches.append(call)
    torch.cuda.synchronize()

    # ---- verification: copy 0 against the oracle (every request), the others
    # bitwise against copy 0. The oracle's own wall time on the host's cores
    # is the CPU baseline.
    ref, cpu_s, cpu_reps = pool.timed(p, 0.0 if args.no_cpu_baseline else args.cpu_seconds,
                                      q_cos_sin=rope_rows)
    o0, l0 = batches[0]()
    torch.cuda.synchronize()
    o0 = o0.clone()
    l0 = l0.clone()
    go = o0.float().cpu().double().numpy()
    gl = l0.cpu().double().numpy()
    ref_o, ref_l = ref
    ninf_ok = bool(np.array_equal(np.isneginf(ref_l), np.isneginf(gl)))
    fin = ~np.isneginf(ref_l)
    err_o = float(np.abs(go - ref_o).max())
    err_l = float(np.abs(gl[fin] - ref_l[fin]).max()) if fin.any() else 0.0
    verified = (ninf_ok and not np.isnan(go).any() and err_o <= TOL_OUT[p.q_dtype]
                and err_l <= TOL_LSE)
    for call in batches[1:]:
        o, l = call()
        torch.cuda.synchronize()
        verified = verified and torch.equal(o.view(torch.int16), o0.view(torch.int16)) \
            and torch.equal(l, l0)

    # ---- warmup
    for i in range(args.warmup):
        batches[i % copies]()
    torch.cuda.synchronize()

    # ---- timed region: K whole steps back to back, then (for the roofline)
    # K partial-kernel launches back to back, each bracketed by two events.
    # Before each run the stream is held by a GPU sleep long enough for the
    # host to queue every launch, so the events time GPU work only.
    K = args.steps
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    torch.cuda._sleep(1_000_000)
    c1.record()
    torch.cuda.synchronize()
    cycles_per_ms = 1_000_000 / max(c0.elapsed_time(c1), 1e-3)
    t_host = time.perf_counter()
    for i in range(3):
        batches[i % copies].partial()
        batches[i % copies].merge()
    host_per_step = (time.perf_counter() - t_host) / 3
    torch.cuda.synchronize()
    hold_ms = 20.0 + 2.0 * K * host_per_step * 1e3

    def timed(launch):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(hold_ms * cycles_per_ms))
        start.record()
        t_enq = time.perf_counter()
        for i in range(K):
            launch(batches[i % copies])
        end.record()
        enqueue_ms = (time.perf_counter() - t_enq) * 1e3
        torch.cuda.synchronize()
        return start.elapsed_time(end), enqueue_ms < hold_ms

    def step(call):
        call.partial()
        call.merge()

    total_ms, ahead_steps = timed(step)
    partial_total_ms, ahead_partial = timed(lambda call: call.partial())
    gpu_ran_ahead = ahead_steps and ahead_partial
    ms_per_step = total_ms / K
    value = tokens * K / (total_ms * 1e-3)
    part_avg = partial_total_ms / K
    plan = batches[0].plan.as_dict()
    # The bound the workload's arithmetic intensity selects: above the ridge
    # (bf16 MFMA peak / HBM peak, about 312 FLOP per KV byte) the MFMA units
    # bound the kernel (the prefill and the wide trees), below it HBM does.
    mfma_bound = flops / kvb > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if mfma_bound:
        achieved = flops / (part_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    else:
        achieved = kvb / (part_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4)}
    src_hash = kernel_source_hash()
    key = str(args.config) if args.config != 3 else f"3@{args.prefix}"
    key += ":rows" if p.mask_layout == "rows" else ""
    key += ":rope" if args.rope else ""
    roof["traffic"] = profiled_traffic(key, src_hash)
    roof["kernel"] = "vat_stream" if plan["kernel"] == 1 else "vat_tile"
    roof["algorithmic_bytes_per_launch"] = kvb
    roof["algorithmic_flops_per_launch"] = flops

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16"}[p.q_dtype] + ("+e4m3kv" if p.kv_dtype == "e4m3" else ""),
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.config].format(p=args.prefix) +
                   (", sglang full-row byte mask" if p.mask_layout == "rows" else "") +
                   (", queries rotated by RoPE at their tree positions" if args.rope else ""),
                   "batch": p.batch, "query_tokens": tokens, "kv_bytes": kvb,
                   "parallelism": "single GPU", "page_pool_copies": copies},
        "kv_read_gbps_step": round(kvb / (ms_per_step * 1e-3) / 1e9, 1),
        "kv_frac_of_peak_step": round(kvb / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": roof,
        "partial_kernel_ms": round(part_avg, 5),
        "verified": bool(verified),
        "parity": {"max_out_err": err_o, "max_lse_err": err_l,
                   "tol_out": TOL_OUT[p.q_dtype], "tol_lse": TOL_LSE, "sample": "all requests"},
        "plan": plan,
        "gpu_ran_ahead_of_host": bool(gpu_ran_ahead),
        "kernel_source": src_hash,
    }
    if not args.no_graph_stats:
        flushed, warm = graph_call_stats(torch, binding, batches, K, 1 << 30)
        med = float(np.median(flushed))
        line["per_call"] = {
            "what": "one verify_attention call replayed from a HIP graph, GPU time by HIP events",
            "flushed_ms": {"median": round(med, 5),
                           "p10": round(float(np.percentile(flushed, 10)), 5),
                           "p90": round(float(np.percentile(flushed, 90)), 5)},
            "flush": "1 GiB written, then read, between calls",
            "warm_median_ms": round(float(np.median(warm)), 5),
            "calls": K,
            "query_tokens_per_s_flushed_median": round(tokens / (med * 1e-3), 1),
        }
        if mfma_bound:
            line["per_call"]["mfma_frac_flushed_median"] = round(
                flops / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
        else:
            line["per_call"]["kv_frac_of_peak_flushed_median"] = round(
                kvb / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        probe_med, probe_best = read_probe_gbps(torch, binding, 2 << 30)
        line["hbm_read_probe"] = {"bytes": 2 << 30, "gbps_median": round(probe_med, 1),
                                  "gbps_best": round(probe_best, 1),
                                  "frac_of_peak_median": round(probe_med / HBM_PEAK_GBPS, 4),
                                  "kernel": "vat_read_probe (16-byte non-temporal loads, "
                                            "8 workgroups per CU)"}
    if not args.no_cpu_baseline:
        from tests.oracle_pool import OraclePool, cpu_model

        line["cpu_baseline"] = {
            "value": round(tokens * cpu_reps / cpu_s, 3), "unit": "query-tokens/s",
            "cores": pool.workers, "kind": "oracle",
            "sample": (f"whole workload, {p.batch * p.num_kv_heads} (request, KV head) items over "
                       f"{pool.workers} worker processes with one BLAS thread each"
                       if pool.workers > 1 or isinstance(pool, OraclePool) else
                       "whole workload, in this process with one BLAS thread") +
                      f", repeated {cpu_reps}x, {cpu_s:.1f} s, NumPy float64; host CPU: {cpu_model()}"}
    print(json.dumps(line), flush=True)
    if not verified:
        sys.exit(3)


if __name__ == "__main__":
    main()
