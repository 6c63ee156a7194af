"""Moving seeded problems onto the GPU and comparing with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

from workloads.gen import Problem

TOL_OUT = {"f32": 1e-5, "bf16": 2e-2}
TOL_LSE = 1e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(p: Problem, device="cuda"):
    def storage(arr, dt):
        if dt == "f32":
            return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(
                torch.bfloat16).to(device)
        if dt == "e4m3":
            return torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn).to(device)
        raise ValueError(dt)

    d = dict(
        q=storage(p.q, p.q_dtype),
        k_cache=storage(p.k_cache, p.kv_dtype),
        v_cache=storage(p.v_cache, p.kv_dtype),
        kv_indptr=torch.from_numpy(p.kv_indptr).to(device),
        kv_indices=torch.from_numpy(p.kv_indices).to(device),
        last_page_len=torch.from_numpy(p.last_page_len).to(device),
        qo_indptr=torch.from_numpy(p.qo_indptr).to(device),
        mask=None if p.mask is None else torch.from_numpy(p.mask).to(device),
        mask_indptr=None if p.mask_indptr is None else torch.from_numpy(p.mask_indptr).to(device),
    )
    return d


def run_gpu(lib, p: Problem, tensors=None, **kw):
    t = tensors if tensors is not None else to_device(p)
    out, lse = lib.verify_attention(
        t["q"], t["k_cache"], t["v_cache"], t["kv_indptr"], t["kv_indices"], t["last_page_len"],
        t["qo_indptr"], t["mask"], t["mask_indptr"], sm_scale=p.sm_scale, k_scale=p.k_scale,
        v_scale=p.v_scale, max_qo_len=p.max_qo_len, mask_layout=p.mask_layout, **kw)
    torch.cuda.synchronize()
    return out, lse


def to_f64(out, lse):
    return out.float().cpu().double().numpy(), lse.cpu().double().numpy()


def oracle_of(p: Problem, requests=None):
    from oracle import verify_attention

    return verify_attention(p.q, p.k_cache, p.v_cache, p.kv_indptr, p.kv_indices,
                            p.last_page_len, p.qo_indptr, p.mask, p.mask_indptr,
                            sm_scale=p.sm_scale, k_scale=p.k_scale, v_scale=p.v_scale,
                            q_dtype=p.q_dtype, kv_dtype=p.kv_dtype, requests=requests,
                            mask_layout=p.mask_layout)


def rows_of(p: Problem, requests):
    rows = []
    for b in requests:
        rows.extend(range(int(p.qo_indptr[b]), int(p.qo_indptr[b + 1])))
    return np.asarray(rows, dtype=np.int64)


def compare(p: Problem, got_out, got_lse, ref_out, ref_lse, rows=None, what=""):
    """Assert parity at the stated tolerances; returns (max out err, max lse err)."""
    if rows is not None:
        got_out, got_lse = got_out[rows], got_lse[rows]
        ref_out, ref_lse = ref_out[rows], ref_lse[rows]
    assert not np.isnan(got_out).any(), f"{what}: NaN in out"
    assert not np.isnan(got_lse).any(), f"{what}: NaN in lse"
    ninf_ref = np.isneginf(ref_lse)
    ninf_got = np.isneginf(got_lse)
    assert np.array_equal(ninf_ref, ninf_got), f"{what}: -inf lse pattern differs"
    tol = TOL_OUT[p.q_dtype]
    err_o = float(np.abs(got_out - ref_out).max()) if got_out.size else 0.0
    fin = ~ninf_ref
    err_l = float(np.abs(got_lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    assert err_o <= tol, f"{what}: max |out err| {err_o:.3e} > {tol}"
    assert err_l <= TOL_LSE, f"{what}: max |lse err| {err_l:.3e} > {TOL_LSE}"
    return err_o, err_l
