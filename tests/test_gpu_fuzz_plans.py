"""Seeded mid-size fuzz over the planner's paths, against the oracle.

The small-shape fuzz keeps one or two KV heads and a handful of requests.
These cases draw the shapes that select the other plans: KV head counts of 2,
4, 8 and 12 (fp8 D 128 then takes two- or four-head workgroups), groups up to
16, batches on both sides of the balanced slices' 64-request limit, drafts up
to 64 long, both mask layouts, page sizes 1 to 256, forced chunk lengths and
compute-unit counts from 8 to 1024 (one slice, a few long slices, more
slices than pages). Each case is capped so the oracle finishes in seconds;
every request of every case is compared.
"""

from __future__ import annotations

import numpy as np
import pytest

from tests.gpu_helpers import compare, run_gpu, say, to_f64
from workloads import make_case

pytestmark = pytest.mark.gpu

# Oracle work per case (multiply-adds over visible pairs and head dims) and
# cached elements per cache.
MAX_WORK = 6e8
MAX_CACHE = 3e7


def _dtypes(seed, rng):
    q_dt, kv_dt = [("bf16", "bf16"), ("bf16", "e4m3"), ("bf16", "e4m3"), ("f32", "f32")][seed % 4]
    D = 128 if kv_dt == "e4m3" and seed % 3 else int(rng.choice([64, 128]))
    return q_dt, kv_dt, D


def _fuzz_case(seed):
    rng = np.random.default_rng(5000 + seed)
    q_dt, kv_dt, D = _dtypes(seed, rng)
    hkv = int(rng.choice([2, 4, 8, 12]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    B = int(rng.choice([1, 3, 17, 64, 65, 70]))
    kind, layout = [("causal", "bits"), ("tree", "bits"), ("random", "bits"), ("tree", "rows"),
                    ("chain", "bits"), ("causal", "bits")][seed % 6]
    # Every fifth case keeps drafts short (config 5's mix), where fp8 D 128
    # with an even head count takes the head-group workgroups.
    lmax = 8 if seed % 5 == 0 else (64 if kind != "causal" else 80)
    lens = [int(x) for x in rng.integers(1, lmax + 1, size=B)]
    lens = [0 if rng.random() < 0.05 else x for x in lens]
    prefixes = [int(x) for x in rng.integers(0, 4001, size=B)]
    # Shrink the prefixes (then the drafts) until the case fits the caps.
    def work():
        return sum(hkv * G * L * (pre + L) * D for L, pre in zip(lens, prefixes))

    def cache():
        return sum(pre + L for L, pre in zip(lens, prefixes)) * hkv * D
    while work() > MAX_WORK or cache() > MAX_CACHE:
        prefixes = [p // 2 for p in prefixes]
        if all(p == 0 for p in prefixes):
            lens = [max(1, L // 2) if L else 0 for L in lens]
    ps = int(rng.choice([1, 2, 8, 16, 32, 128, 256]))
    chunk = int(rng.choice([-1, -1, -1, 0, 64, 272]))
    cus = int(rng.choice([0, 0, 8, 64, 300, 1024]))
    p = make_case(seed + 700, prefix_lens=prefixes, qo_lens=lens, num_qo_heads=G * hkv,
                  num_kv_heads=hkv, head_dim=D, page_size=ps, q_dtype=q_dt, kv_dtype=kv_dt,
                  mask_kind=kind, mask_layout=layout, fp8_absmax_scales=(kv_dt == "e4m3"),
                  mask_density=0.5, max_qo_len=max(max(lens), 1), extra_indices=int(seed % 4))
    return p, chunk, cus


@pytest.mark.parametrize("seed", list(range(80)))
def test_fuzz_plans(gpu_lib, oracle_pool, seed):
    p, chunk, cus = _fuzz_case(seed)
    info = (f"[plan fuzz {seed}] B={p.batch} Hq={p.num_qo_heads} Hkv={p.num_kv_heads} "
            f"D={p.head_dim} ps={p.page_size} {p.q_dtype}/{p.kv_dtype} mask={p.info['mask_kind']}/"
            f"{p.mask_layout} maxL={p.max_qo_len} chunk={chunk} cus={cus or 'device'}")
    say(info)
    out, lse = run_gpu(gpu_lib, p, chunk_keys=chunk, num_cus=cus)
    compare(p, *to_f64(out, lse), *oracle_pool.run(p), what=info)


def _rope_supported(seed) -> bool:
    # Query RoPE runs in the streaming kernel: bf16 caches, or fp8 with D 128.
    _, kv_dt, D = _dtypes(seed, np.random.default_rng(5000 + seed))
    return kv_dt == "bf16" or (kv_dt == "e4m3" and D == 128)


@pytest.mark.parametrize("seed", [s for s in range(80) if _rope_supported(s)])
def test_fuzz_plans_rope(gpu_lib, oracle_pool, seed):
    """The same seeded shapes with the queries rotated by RoPE at their tree
    positions, for the cache dtypes RoPE serves."""
    import torch

    from workloads import rope_cos_sin, rope_positions

    p, chunk, cus = _fuzz_case(seed)
    info = (f"[plan fuzz rope {seed}] B={p.batch} Hq={p.num_qo_heads} Hkv={p.num_kv_heads} "
            f"D={p.head_dim} ps={p.page_size} {p.kv_dtype} mask={p.info['mask_kind']}/"
            f"{p.mask_layout} maxL={p.max_qo_len} chunk={chunk} cus={cus or 'device'}")
    say(info)
    cs = rope_cos_sin(rope_positions(p), p.head_dim)
    out, lse = run_gpu(gpu_lib, p, chunk_keys=chunk, num_cus=cus,
                       q_cos_sin=torch.from_numpy(np.ascontiguousarray(cs)).cuda())
    compare(p, *to_f64(out, lse), *oracle_pool.run(p, q_cos_sin=cs), what=info)
