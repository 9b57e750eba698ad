"""The kernels' own page walks, bit for bit.

The decode kernel and the multi-row (cascade prefix / append) kernel each
walk the page table their own way: the decode kernel shuffles a step's page
indices across lanes and clamps its tail to the tile, the multi-row kernel
stages a chunk's page indices in LDS.  fi_debug_record_walk runs each kernel
as the planned run launches it, in an instance whose loader also stores the
K-pool byte offset of every 16-byte K vector it loads.  Every (token, kv
head, chunk) of every key list must be loaded, at exactly the offset that a
plain reading of the page table gives (the oracle's gather map: logical token
t of list i in page kv_indices[kv_indptr[i] + t / page_size], slot
t % page_size; NHD / HND strides; ragged rows kv_indptr[i] + t)."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fi():
    import paged_kv_decode_fi_amd as m
    return m


def _expected(w, indptr, indices, last, lens):
    """int64 [sum(lens), Hkv, VR] K-pool byte offsets from the page table."""
    import oracle
    Hkv, rowb = w.num_kv_heads, w.row_bytes
    ps = w.page_size
    if C.is_ragged(w):
        rows = np.concatenate([np.arange(indptr[i], indptr[i] + lens[i], dtype=np.int64)
                               for i in range(len(lens))] or [np.zeros(0, np.int64)])
        page, slot = rows, np.zeros_like(rows)
    else:
        phys = oracle.gather_map(ps, indptr, indices, last)
        page, slot = phys // ps, phys % ps
    page_bytes = ps * Hkv * rowb
    slot_stride, head_stride = (rowb, ps * rowb) if C.is_hnd(w) else (Hkv * rowb, rowb)
    h = np.arange(Hkv, dtype=np.int64)
    c = np.arange(rowb // 16, dtype=np.int64)
    return (page[:, None, None] * page_bytes + slot[:, None, None] * slot_stride
            + h[None, :, None] * head_stride + 16 * c[None, None, :])


def _walk(fi, w, plan, stage, d=None):
    import torch
    d = d or C.Dev(w)
    if stage == 1 and w.prefix_kv_indptr is not None and w.qo_indptr is None:
        lens = w.prefix_lens
        tabs = (w.prefix_kv_indptr, w.prefix_kv_indices, w.prefix_last_page_len)
    else:
        lens = w.kv_lens
        tabs = (w.kv_indptr, w.kv_indices, w.last_page_len)
    base = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    vr = w.row_bytes // 16
    rec = torch.full((max(int(base[-1]), 1) * w.num_kv_heads * vr,), -1, dtype=torch.int64,
                     device="cuda")
    kw = {}
    if w.prefix_kv_indptr is not None:
        kw = dict(prefix_kv_indptr=d.p_indptr, prefix_kv_indices=d.p_indices,
                  prefix_last_page_len=d.p_last)
    plan.record_walk(stage, rec, C.to_dev(base), d.q, d.k, d.v, d.indptr, d.indices, d.last,
                     k_scale=d.k_scale, v_scale=d.v_scale, sm_scale=w.sm_scale, **kw)
    torch.cuda.synchronize()
    got = rec.cpu().numpy()[:int(base[-1]) * w.num_kv_heads * vr]
    got = got.reshape(int(base[-1]), w.num_kv_heads, vr)
    last = tabs[2]
    if last is None:   # ragged: one row per page
        last = np.ones(len(lens), np.int32)
    want = _expected(w, tabs[0], tabs[1], last, lens)
    missed = np.argwhere(got < 0)
    assert len(missed) == 0, f"{len(missed)} K vectors never loaded, first {missed[:3]}"
    bad = np.argwhere(got != want)
    assert len(bad) == 0, (f"{len(bad)} loads at the wrong offset, first (token, head, "
                           f"chunk) {bad[0]}: got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}")


def _lens(seed, n=13, hi=700):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, hi, size=n)
    lens[2] = 0
    lens[5] = 1
    return lens


@pytest.mark.parametrize("ps", [1, 3, 7, 16, 32])
@pytest.mark.parametrize("chunk,hpt", [(0, 0), (48, 8), (32, 2), (16, 1)])
def test_decode_walk_nhd(fi, ps, chunk, hpt):
    w = W.build("walk", _lens(ps), Hq=32, Hkv=8, ps=ps, seed=ps)
    plan = C.make_plan(w, chunk_tokens=chunk, tuning=dict(heads_per_tile=hpt))
    _walk(fi, w, plan, 0)
    plan.destroy()


@pytest.mark.parametrize("depth", [1, 2])
@pytest.mark.parametrize("layout", ["nhd", "hnd", "ragged"])
@pytest.mark.parametrize("ps", [7, 16])
def test_decode_walk_layouts(fi, depth, layout, ps):
    w = W.build("walk", _lens(100 + ps), Hq=16, Hkv=4, ps=ps, seed=3 + ps)
    w = {"nhd": w, "hnd": W.to_hnd(w), "ragged": W.to_ragged(w)}[layout]
    plan = C.make_plan(w, chunk_tokens=64, tuning=dict(decode_depth=depth))
    _walk(fi, w, plan, 0)
    plan.destroy()


@pytest.mark.parametrize("ps", [1, 16])
def test_decode_walk_e4m3(fi, ps):
    w = W.build("walk_fp8", _lens(7 + ps, n=9, hi=900), Hq=64, Hkv=8, ps=16, q_dtype="bf16",
                kv_dtype="e4m3", seed=9, extra_page_sizes=(1,))[ps]
    for chunk in (0, 80):
        plan = C.make_plan(w, chunk_tokens=chunk)
        _walk(fi, w, plan, 0)
        plan.destroy()


@pytest.mark.parametrize("layout", ["nhd", "hnd", "ragged"])
@pytest.mark.parametrize("ps", [1, 5, 16])
def test_cascade_prefix_walk(fi, layout, ps):
    """The multi-row kernel over shared prefixes (chunked, several groups,
    an empty one) and the suffix decode tiles of the same plan."""
    if layout == "ragged" and ps != 1:
        pytest.skip("the ragged layout has page size 1")
    lens = _lens(40 + ps, n=12, hi=300)
    w = W.build("walk_cascade", lens, Hq=32, Hkv=4, ps=ps, seed=11 + ps,
                prefix_groups=[(5, 700), (3, 0), (4, 1100)])
    w = {"nhd": w, "hnd": W.to_hnd(w), "ragged": W.to_ragged(w)}[layout]
    plan = C.make_plan(w, tuning=dict(prefix_chunk_min=256, prefix_tiles_per_cu=8))
    assert plan.stats["num_prefix_tiles"] > 3
    d = C.Dev(w)
    _walk(fi, w, plan, 1, d)
    _walk(fi, w, plan, 0, d)
    plan.destroy()


def test_cascade_prefix_walk_e4m3(fi):
    lens = _lens(77, n=10, hi=200)
    w = W.build("walk_cascade_fp8", lens, Hq=64, Hkv=8, ps=16, q_dtype="bf16",
                kv_dtype="e4m3", seed=12, prefix_groups=[(10, 1500)])
    plan = C.make_plan(w, tuning=dict(prefix_tiles_per_cu=4, decode_depth=1))
    _walk(fi, w, plan, 1)
    _walk(fi, w, plan, 0)
    plan.destroy()


@pytest.mark.parametrize("ps", [1, 16])
@pytest.mark.parametrize("causal", [True, False])
def test_append_walk(fi, ps, causal):
    import paged_kv_decode_fi_amd as m
    lens = np.array([300, 1, 0, 520, 77, 1000])
    qn = np.minimum(lens, [40, 1, 0, 130, 77, 3])
    w = W.build_append("walk_append", lens, qn, Hq=32, Hkv=8, ps=ps, seed=5, causal=causal)
    plan = m.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=32, num_kv_heads=8,
                  page_size=ps, qo_indptr=w.qo_indptr, causal=causal,
                  tuning=dict(prefix_waves=8, append_chunk_min=64))
    _walk(fi, w, plan, 1)
    plan.destroy()


def test_record_hook_refuses_what_is_not_built(fi):
    w = W.build("walk_bf16", [40, 50], Hq=8, Hkv=8, ps=16, q_dtype="bf16", kv_dtype="bf16",
                seed=1)
    plan = C.make_plan(w)
    with pytest.raises(fi.FiError) as e:
        _walk(fi, w, plan, 0)
    assert e.value.status == 2
    plan.destroy()


@pytest.mark.parametrize("ps", [1, 7, 16])
@pytest.mark.parametrize("chunk,hpt", [(0, 0), (32, 1), (48, 8), (1024, 2)])
def test_decode_walk_one_request(fi, ps, chunk, hpt):
    """One request split into chunks (the single-request decode shape): the
    loads cover every key exactly as the page table says, at every chunk and
    heads-per-tile cut."""
    w = W.build("walk_one", [1337], Hq=32, Hkv=8, ps=ps, seed=70 + ps)
    plan = C.make_plan(w, chunk_tokens=chunk, tuning=dict(heads_per_tile=hpt))
    _walk(fi, w, plan, 0)
    plan.destroy()
