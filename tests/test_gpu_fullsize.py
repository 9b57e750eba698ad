"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default plan: device CU count, automatic chunking).

The oracle cannot afford every (request, kv head) unit of a full workload in
a test, so it computes a sample of whole units one by one; the sample always
holds the units most likely to expose a mistake (the longest and shortest
requests, the first and last request, requests split into many tiles) plus
random units.  Every output row of a sampled unit is compared element by
element at the acceptance bar.  Every other row is checked for what holds at
any size: the outputs start as NaN, so each row must have been written, with
finite values (every request of these workloads has keys).
"""
import zlib

import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu

_CACHE = {}


def _workload(name):
    if name not in _CACHE:
        _CACHE.clear()                       # keep one full workload resident at a time
        _CACHE[name] = W.make(name)
    return _CACHE[name]


def _sample_units(w, n_random, seed):
    """Unit mask [B * Hkv] (uint8): every kv head of the edge requests, plus
    n_random random units."""
    B, H = w.batch, w.num_kv_heads
    lens = w.kv_lens
    reqs = {0, B - 1, int(np.argmax(lens)), int(np.argmin(lens))}
    # a second longest request (skewed: another 32K request; cascade: another long suffix)
    order = np.argsort(lens, kind="stable")
    reqs.add(int(order[-2]) if B > 1 else 0)
    mask = np.zeros((B, H), np.uint8)
    for r in reqs:
        mask[r, :] = 1
    rng = np.random.default_rng(seed)
    flat = mask.reshape(-1)
    free = np.flatnonzero(flat == 0)
    if free.size:
        flat[rng.choice(free, size=min(n_random, free.size), replace=False)] = 1
    return flat


def _run_nan_filled(w, rope=None):
    """The benchmark's launch: default plan, outputs pre-filled with NaN."""
    import torch
    d = C.Dev(w)
    plan = C.make_plan(w, rope=rope)
    o = torch.full((w.batch, w.num_qo_heads, w.head_dim), float("nan"),
                   dtype=C.qdtype(w), device="cuda")
    lse = torch.full((w.batch, w.num_qo_heads), float("nan"), dtype=torch.float32,
                     device="cuda")
    if plan.cascade:
        plan.cascade_run(d.q, d.k, d.v, d.p_indptr, d.p_indices, d.p_last, d.indptr,
                         d.indices, d.last, d.k_scale, d.v_scale, sm_scale=w.sm_scale,
                         o=o, lse=lse)
    else:
        plan.run(d.q, d.k, d.v, d.indptr, d.indices, d.last, d.k_scale, d.v_scale,
                 sm_scale=w.sm_scale, o=o, lse=lse)
    torch.cuda.synchronize()
    del d
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy(), plan


def _every_row_written(w, o, lse):
    assert w.prefix_lens is not None or np.all(w.kv_lens > 0)
    assert np.all(np.isfinite(o)), "an output row was not written (or is not finite)"
    assert np.all(np.isfinite(lse)), "an lse entry was not written (or is not finite)"


def _check(w, name, n_random=24, rope=None):
    o, lse, plan = _run_nan_filled(w, rope)
    st = plan.stats
    print(f"{w.name}: tiles {st['num_tiles']} prefix tiles {st['num_prefix_tiles']} "
          f"merge units {st['num_merge_units']} chunk {st['chunk_tokens']}", flush=True)
    _every_row_written(w, o, lse)
    mask = _sample_units(w, n_random, seed=zlib.crc32(name.encode()))
    ro, rl = C.run_oracle(w, unit_mask=mask, rope=rope)
    rows = C.rows_of_units(w, mask)
    C.assert_parity(w, o, lse, ro, rl, rows=rows,
                    label=f"{w.name} full size, {int(mask.sum())} sampled units"
                          + ("" if rope is None else f", RoPE {rope}"))
    plan.destroy()
    return o, lse


@pytest.mark.parametrize("name", ["single_L2048_h32", "batch64_gqa4", "skewed128",
                                  "cascade256"])
def test_full_size_sampled_parity(fi_lib, name):
    w = _workload(name)
    _check(w, name)


@pytest.mark.parametrize("ps", [16, 1])
def test_full_size_long_fp8_sampled_parity(fi_lib, ps):
    ws = _workload("long32_fp8")
    _check(ws[ps], f"long32_fp8_ps{ps}", n_random=8)


@pytest.mark.parametrize("name", ["batch64_gqa4", "skewed128", "cascade256"])
def test_full_size_rope_sampled_parity(fi_lib, name):
    """The same launches with LLaMA-style RoPE on the fly (skewed128 reaches
    position 32767 and splits those requests over many tiles; cascade256
    turns the shared prefix's keys and the query rows by their positions on
    the multi-row kernel)."""
    _check(_workload(name), name + "_rope", n_random=12, rope=(1e4, 1.0))


def test_full_size_rope_fp8_sampled_parity(fi_lib):
    _check(_workload("long32_fp8")[16], "long32_fp8_ps16_rope", n_random=4,
           rope=(5e5, 1.0))


def test_full_size_split_rows_cover_every_chunk(fi_lib):
    """skewed128 at full size: each 32768-token request is split into many
    chunks; one of them is sampled whole above.  Here the same request is
    checked against a planted dominant key in its LAST chunk, so a dropped
    tail chunk cannot hide under the tolerance."""
    w = _workload("skewed128")
    r = int(np.argmax(w.kv_lens))
    L = int(w.kv_lens[r])
    ps = w.page_size
    t_star = L - 3
    page = int(w.kv_indices[w.kv_indptr[r] + t_star // ps])
    G = w.group_size
    h = 5
    q = w.q.view(np.float16).astype(np.float32)
    saved_k = w.k_pages[page, t_star % ps, h].copy()
    saved_q = w.q[r].copy()
    try:
        w.k_pages[page, t_star % ps, h] = (q[r, h * G] * 4.0).astype(np.float16).view(np.uint16)
        for j in range(h * G, (h + 1) * G):
            w.q[r, j] = w.q[r, h * G]
        o, lse, plan = _run_nan_filled(w)
        assert plan.stats["num_merge_units"] > 0
        v_star = w.v_pages[page, t_star % ps, h].view(np.float16).astype(np.float64)
        for j in range(h * G, (h + 1) * G):
            assert np.abs(o[r, j] - v_star).max() < 2e-3 + 1e-2 * np.abs(v_star).max()
        plan.destroy()
    finally:
        w.k_pages[page, t_star % ps, h] = saved_k
        w.q[r] = saved_q


@pytest.fixture(scope="module")
def fi_lib():
    import paged_kv_decode_fi_amd as m
    yield m
    _CACHE.clear()


@pytest.mark.parametrize("head_dim", [64, 256])
@pytest.mark.parametrize("name", ["batch64_gqa4", "cascade256"])
def test_full_size_head_dim_sampled_parity(fi_lib, name, head_dim):
    """The same workloads (seed, lengths, heads, dtypes) at head_dim 64 and
    256, in the benchmark's launch configuration."""
    _CACHE.clear()
    w = W.make(name, head_dim=head_dim)
    _check(w, f"{name}_d{head_dim}", n_random=12)


@pytest.mark.parametrize("head_dim", [64, 256])
def test_full_size_rope_head_dim_sampled_parity(fi_lib, head_dim):
    _CACHE.clear()
    w = W.make("batch64_gqa4", head_dim=head_dim)
    _check(w, f"rope_batch64_gqa4_d{head_dim}", n_random=12, rope=(1e4, 1.0))
