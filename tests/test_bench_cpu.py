"""Host-side checks of bench.py: the one-GPU refusal, and the algorithmic work
that the roofline divides by, against closed forms of the workloads."""

import json
import os
import subprocess
import sys

import bench
from workloads import make_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2
    assert "one GPU" in line["error"]


def test_chain_verify_work_matches_its_closed_form():
    # 8 requests, prefix 2048, 5 causal drafts, Hq 32, Hkv 8, D 128, bf16 K and V.
    kvb, flops = bench.algorithmic_work(make_config(2))
    batch, prefix, drafts, hq, hkv, d = 8, 2048, 5, 32, 8, 128
    assert kvb == batch * (prefix + drafts) * hkv * d * 2 * 2
    # Draft t sees the prefix and drafts 0 .. t; QK and PV take 2 D FLOPs per pair each.
    pairs = batch * (drafts * prefix + drafts * (drafts + 1) // 2)
    assert flops == 4 * d * hq * pairs


def test_causal_prefill_work_matches_its_closed_form():
    # 10 sequences of 1024 tokens, Hq 64, Hkv 8, D 128, bf16 K and V.
    kvb, flops = bench.algorithmic_work(make_config(4))
    batch, tokens, hq, hkv, d = 10, 1024, 64, 8, 128
    assert kvb == batch * tokens * hkv * d * 2 * 2
    assert flops == 4 * d * hq * batch * tokens * (tokens + 1) // 2
