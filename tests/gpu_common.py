"""Shared helpers of the GPU parity tests: upload a workload, run the HIP path
through the C-ABI binding, run the oracle on the same host arrays, compare."""
from __future__ import annotations

import numpy as np

# Acceptance bar: max |err| <= 2e-3 + 1e-2 |ref| for fp16/bf16 KV, <= 3e-2
# absolute for e4m3 KV (against the dequantised oracle), |d lse| <= 1e-3.
TOL_ABS, TOL_REL, TOL_FP8, TOL_LSE = 2e-3, 1e-2, 3e-2, 1e-3


def torch_mod():
    import torch
    return torch


def to_dev(a, dtype=None):
    torch = torch_mod()
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
        if dtype is not None:
            t = t.view(dtype)
    else:
        t = torch.from_numpy(a)
    return t.to("cuda")


def qdtype(w):
    torch = torch_mod()
    return torch.float16 if w.q_dtype == "f16" else torch.bfloat16


class Dev:
    """Device copies of a workload's arrays."""

    def __init__(self, w):
        self.q = to_dev(w.q, qdtype(w))
        self.k = to_dev(w.k_pages)
        self.v = to_dev(w.v_pages)
        self.indptr = to_dev(w.kv_indptr)
        # ragged layout: the kernels get no index or last-page tables
        self.indices = None if is_ragged(w) else to_dev(w.kv_indices)
        self.last = to_dev(w.last_page_len)
        self.k_scale = to_dev(w.k_scale)
        self.v_scale = to_dev(w.v_scale)
        if w.prefix_kv_indptr is not None:
            self.p_indptr = to_dev(w.prefix_kv_indptr)
            self.p_indices = None if is_ragged(w) else to_dev(w.prefix_kv_indices)
            self.p_last = to_dev(w.prefix_last_page_len)


def is_ragged(w):
    return bool(w.meta.get("ragged"))


def is_hnd(w):
    return bool(w.meta.get("hnd"))


def make_plan(w, chunk_tokens=0, cascade=None, rope=None, tuning=None):
    """rope = None or (theta, scale): a plan with LLaMA-style RoPE.  tuning:
    optional dict of fi_tuning fields."""
    import paged_kv_decode_fi_amd as fi
    cascade = (w.prefix_kv_indptr is not None) if cascade is None else cascade
    prefix = ((w.prefix_qo_indptr, w.prefix_kv_indptr, w.prefix_last_page_len)
              if cascade else None)
    return fi.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                   num_kv_heads=w.num_kv_heads, page_size=w.page_size,
                   head_dim=w.head_dim, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                   prefix=prefix, chunk_tokens=chunk_tokens,
                   pos_encoding="none" if rope is None else "rope_llama",
                   rope_theta=0.0 if rope is None else rope[0],
                   rope_scale=0.0 if rope is None else rope[1],
                   kv_layout="ragged" if is_ragged(w) else
                   "paged_hnd" if is_hnd(w) else "paged", tuning=tuning)


def run_gpu(w, d=None, plan=None, chunk_tokens=0, rope=None, tuning=None):
    """Runs the HIP path; returns (o float64 numpy, lse float64 numpy, plan)."""
    torch = torch_mod()
    d = d or Dev(w)
    plan = plan or make_plan(w, chunk_tokens, rope=rope, tuning=tuning)
    if plan.cascade:
        o, lse = plan.cascade_run(d.q, d.k, d.v, d.p_indptr, d.p_indices, d.p_last,
                                  d.indptr, d.indices, d.last, d.k_scale, d.v_scale,
                                  sm_scale=w.sm_scale)
    else:
        o, lse = plan.run(d.q, d.k, d.v, d.indptr, d.indices, d.last, d.k_scale,
                          d.v_scale, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy(), plan


def run_oracle(w, unit_mask=None, rope=None):
    import oracle
    ragged = is_ragged(w)
    kw = dict(rope=rope, kv_layout="HND" if is_hnd(w) else "NHD", num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
              head_dim=w.head_dim, page_size=w.page_size, q_dtype=w.q_dtype,
              kv_dtype=w.kv_dtype, sm_scale=w.sm_scale, k_scale=w.k_scale,
              v_scale=w.v_scale, unit_mask=unit_mask)
    if w.prefix_kv_indptr is not None:
        return oracle.cascade(w.q, w.k_pages, w.v_pages, w.prefix_qo_indptr,
                              w.prefix_kv_indptr, None if ragged else w.prefix_kv_indices,
                              w.prefix_last_page_len, w.kv_indptr,
                              None if ragged else w.kv_indices, w.last_page_len, **kw)
    return oracle.decode(w.q, w.k_pages, w.v_pages, w.kv_indptr,
                         None if ragged else w.kv_indices, w.last_page_len, **kw)


def rows_of_units(w, unit_mask):
    """Boolean [B, Hq] of the q rows the selected (request, kv head) units cover."""
    um = np.asarray(unit_mask, bool).reshape(w.batch, w.num_kv_heads)
    return np.repeat(um, w.group_size, axis=1)


def assert_parity(w, o, lse, ro, rl, rows=None, label=""):
    """Element-wise comparison at the acceptance bar."""
    if rows is None:
        rows = np.ones((w.batch, w.num_qo_heads), bool)
    o, ro = o[rows], ro[rows]
    lse, rl = lse[rows], rl[rows]
    assert np.all(np.isfinite(ro)), "oracle produced non-finite values"
    err = np.abs(o - ro)
    if w.kv_dtype == "e4m3":
        bad = err > TOL_FP8
    else:
        bad = err > TOL_ABS + TOL_REL * np.abs(ro)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), f"{label}: empty-request lse mismatch"
    dl = np.abs(lse[~empty] - rl[~empty])
    msg = (f"{label}: max|err| {err.max() if err.size else 0:.3e} "
           f"(bad {int(bad.sum())}/{bad.size}), max|dlse| {dl.max() if dl.size else 0:.3e}")
    if bad.any():
        # where: (selected row, dim) of the worst excess over the bound, with
        # the reference value there
        ex = err - (TOL_FP8 if w.kv_dtype == "e4m3" else TOL_ABS + TOL_REL * np.abs(ro))
        k = np.unravel_index(int(np.argmax(ex)), ex.shape)
        sel = np.argwhere(rows)[k[0]]
        msg += (f"; worst at (row {int(sel[0])}, head {int(sel[1])}, dim {int(k[1])}): "
                f"got {o[k]:.5f} want {ro[k]:.5f}")
    print(msg)
    assert not bad.any(), msg
    assert dl.size == 0 or dl.max() <= TOL_LSE, msg
    return err.max() if err.size else 0.0, dl.max() if dl.size else 0.0
