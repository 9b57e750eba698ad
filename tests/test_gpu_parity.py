"""GPU parity of the HIP decode path (through the C ABI) against the fp64
oracle, on seeded synthetic inputs shaped like the named workloads."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fi():
    import paged_kv_decode_fi_amd as m
    return m


def _variants(w):
    return list(w.values()) if isinstance(w, dict) else [w]


# ---------------------------------------------------------------- page walk

@pytest.mark.parametrize("ps", [1, 7, 16])
def test_gather_is_bit_exact(fi, ps):
    import oracle
    import torch
    rng = np.random.default_rng(ps)
    lens = rng.integers(0, 300, size=9)
    n = (lens + ps - 1) // ps
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    indices = rng.permutation(int(n.sum()) + 11)[:int(n.sum())].astype(np.int32)
    last = np.where(n > 0, lens - (n - 1) * ps, 0).astype(np.int32)
    tok = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    got = fi.debug_gather(ps, C.to_dev(indptr), C.to_dev(indices), C.to_dev(last),
                          C.to_dev(tok)).cpu().numpy()
    want = oracle.gather_map(ps, indptr, indices, last)
    assert np.array_equal(got, want)


# ------------------------------------------------------- small named shapes

@pytest.mark.parametrize("name", W.WORKLOADS)
def test_small_workload_parity(fi, name):
    for w in _variants(W.make(name, small=True)):
        o, lse, plan = C.run_gpu(w)
        ro, rl = C.run_oracle(w)
        C.assert_parity(w, o, lse, ro, rl, label=f"{w.name} {plan.stats}")


@pytest.mark.parametrize("name", ["batch64_gqa4", "skewed128", "cascade256", "long32_fp8"])
@pytest.mark.parametrize("chunk", [32, 96])
def test_forced_split_parity(fi, name, chunk):
    """Small chunks force split-KV tiles and the (o, lse) merge (for cascade,
    the merge kernel or the fold of prefix states into a one-chunk suffix)."""
    for w in _variants(W.make(name, small=True)):
        o, lse, plan = C.run_gpu(w, chunk_tokens=chunk)
        assert plan.stats["num_merge_units"] + plan.stats["num_folded"] > 0
        ro, rl = C.run_oracle(w)
        C.assert_parity(w, o, lse, ro, rl, label=f"{w.name} chunk {chunk}")


def test_page_size_1_and_16_agree_bitwise(fi):
    """Same logical e4m3 data as page size 1 and 16: the kernel sums in logical
    token order with the same plan, so the outputs are identical."""
    ws = W.make("long32_fp8", small=True)
    o1, l1, _ = C.run_gpu(ws[1])
    o16, l16, _ = C.run_gpu(ws[16])
    assert np.array_equal(o1, o16) and np.array_equal(l1, l16)


def test_run_to_run_determinism_and_page_permutation(fi):
    w = W.make("batch64_gqa4", small=True)
    o1, l1, plan = C.run_gpu(w, chunk_tokens=64)
    o2, l2, _ = C.run_gpu(w, plan=plan)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # move every page to a new place in a bigger pool: same result bit for bit
    rng = np.random.default_rng(5)
    P = w.k_pages.shape[0]
    newpos = rng.permutation(P + 7)[:P]
    kp = np.full((P + 7,) + w.k_pages.shape[1:], W.NAN_BITS["f16"], w.k_pages.dtype)
    vp = kp.copy()
    kp[newpos] = w.k_pages
    vp[newpos] = w.v_pages
    import copy
    w2 = copy.copy(w)
    w2.k_pages, w2.v_pages = kp, vp
    w2.kv_indices = newpos[w.kv_indices].astype(np.int32)
    o3, l3, _ = C.run_gpu(w2, plan=plan)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


# ----------------------------------------------------------------- fuzz

def _fuzz_case(seed):
    rng = np.random.default_rng(1000 + seed)
    ps = int(rng.choice([1, 2, 3, 7, 16]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 10))
    choices = [0, 1, max(ps - 1, 1), ps, ps + 1, int(rng.integers(2, 700))]
    lens = [int(rng.choice(choices)) for _ in range(B)]
    q_dtype = str(rng.choice(["f16", "bf16"]))
    kv_dtype = str(rng.choice([q_dtype, "e4m3"]))
    return W.build(f"fuzz{seed}", lens, Hq=Hkv * G, Hkv=Hkv, ps=ps, q_dtype=q_dtype,
                   kv_dtype=kv_dtype, seed=seed)


@pytest.mark.parametrize("seed", range(24))
def test_fuzz_parity(fi, seed):
    w = _fuzz_case(seed)
    chunk = [0, 32, 64][seed % 3]
    o, lse, plan = C.run_gpu(w, chunk_tokens=chunk)
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl,
                    label=f"fuzz{seed} B{w.batch} G{w.group_size} Hkv{w.num_kv_heads} "
                          f"ps{w.page_size} {w.q_dtype}/{w.kv_dtype} lens {list(w.kv_lens)}")


def _cascade_fuzz_case(seed):
    """Random cascade: 1-3 prefix groups (some with an empty prefix), page
    sizes including non-powers of two, group sizes 1-16, 16-bit or e4m3 KV."""
    rng = np.random.default_rng(5000 + seed)
    ps = int(rng.choice([1, 3, 8, 16]))
    G = int(rng.choice([1, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 4]))
    q_dtype = str(rng.choice(["f16", "bf16"]))
    kv_dtype = str(rng.choice([q_dtype, "e4m3"]))
    groups = []
    for _ in range(int(rng.integers(1, 4))):
        groups.append((int(rng.integers(1, 5)), int(rng.choice([0, 1, ps, 300, 1000]))))
    B = sum(g[0] for g in groups)
    lens = [int(rng.choice([0, 1, ps + 1, int(rng.integers(2, 400))])) for _ in range(B)]
    return W.build(f"cfuzz{seed}", lens, Hq=Hkv * G, Hkv=Hkv, ps=ps, q_dtype=q_dtype,
                   kv_dtype=kv_dtype, seed=seed, prefix_groups=groups)


@pytest.mark.parametrize("seed", range(10))
def test_cascade_fuzz_parity(fi, seed):
    w = _cascade_fuzz_case(seed)
    chunk = [0, 32, 64][seed % 3]
    o, lse, plan = C.run_gpu(w, chunk_tokens=chunk)
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl,
                    label=f"cfuzz{seed} B{w.batch} G{w.group_size} Hkv{w.num_kv_heads} "
                          f"ps{w.page_size} {w.q_dtype}/{w.kv_dtype} groups "
                          f"{list(zip(np.diff(w.prefix_qo_indptr), w.prefix_lens))} "
                          f"lens {list(w.kv_lens)} {plan.stats}")


# ------------------------------------------------------------ spike test

def test_planted_dominant_key(fi):
    """A key planted at a random position dominates: o must equal its V row
    (catches a dropped or misplaced token that the tolerance alone cannot)."""
    w = W.make("skewed128", small=True)
    rng = np.random.default_rng(77)
    r = int(np.argmax(w.kv_lens))
    L = int(w.kv_lens[r])
    t_star = int(rng.integers(0, L))
    ps = w.page_size
    page = w.kv_indices[w.kv_indptr[r] + t_star // ps]
    q = w.q.view(np.float16).astype(np.float32)
    h = 3
    G = w.group_size
    # K row := 4 * q of head h*G (scores ~ 4|q|^2/sqrt(D) >> others), same for all G heads
    krow = (q[r, h * G] * 4.0).astype(np.float16)
    w.k_pages[page, t_star % ps, h] = krow.view(np.uint16)
    for j in range(h * G, (h + 1) * G):
        w.q[r, j] = w.q[r, h * G]
    o, lse, _ = C.run_gpu(w, chunk_tokens=64)
    ro, rl = C.run_oracle(w)
    v_star = w.v_pages[page, t_star % ps, h].view(np.float16).astype(np.float64)
    for j in range(h * G, (h + 1) * G):
        assert np.abs(ro[r, j] - v_star).max() < 1e-3
        assert np.abs(o[r, j] - v_star).max() < 2e-3 + 1e-2 * np.abs(v_star).max()
    C.assert_parity(w, o, lse, ro, rl, label="spike")


# ----------------------------------------------------------- cascade / merge

def test_cascade_matches_flat_decode(fi):
    """fi_cascade_decode vs fi_decode_run over each request's concatenated
    (prefix ++ own) page table."""
    w = W.make("cascade256", small=True)
    oc, lc, _ = C.run_gpu(w)
    import copy
    flat = copy.copy(w)
    B = w.batch
    indptr = [0]
    idx = []
    last = []
    for r in range(B):
        g = int(np.searchsorted(w.prefix_qo_indptr, r, side="right") - 1)
        pp = w.prefix_kv_indices[w.prefix_kv_indptr[g]:w.prefix_kv_indptr[g + 1]]
        own = w.kv_indices[w.kv_indptr[r]:w.kv_indptr[r + 1]]
        assert w.prefix_last_page_len[g] == w.page_size   # prefix fills whole pages
        idx.extend(pp.tolist() + own.tolist())
        indptr.append(len(idx))
        last.append(w.last_page_len[r] if len(own) else w.page_size)
    flat.kv_indptr = np.array(indptr, np.int32)
    flat.kv_indices = np.array(idx, np.int32)
    flat.last_page_len = np.array(last, np.int32)
    flat.prefix_kv_indptr = None
    flat.prefix_lens = None
    flat.kv_lens = w.kv_lens + w.prefix_lens[0]
    of, lf, _ = C.run_gpu(flat, chunk_tokens=0)
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, oc, lc, ro, rl, label="cascade vs oracle")
    C.assert_parity(flat, of, lf, ro, rl, label="flat vs oracle")


def test_split_merge_reuses_plan_with_new_data(fi):
    """One plan serves runs over different data (the plan depends on lengths
    only): each run must match the oracle on ITS data, so a merge that read a
    partial state left by the previous run fails."""
    import copy
    w1 = W.make("batch64_gqa4", small=True)
    w2 = copy.copy(w1)
    rng = np.random.default_rng(99)
    w2.q = W.cast_bits(rng.standard_normal(w1.q.shape).astype(np.float32), "f16")
    k2 = W.cast_bits(rng.standard_normal(w1.k_pages.shape).astype(np.float32), "f16")
    v2 = W.cast_bits(rng.standard_normal(w1.v_pages.shape).astype(np.float32), "f16")
    w2.k_pages = np.where(w1.k_pages != W.NAN_BITS["f16"], k2, w1.k_pages)
    w2.v_pages = np.where(w1.v_pages != W.NAN_BITS["f16"], v2, w1.v_pages)
    plan = C.make_plan(w1, chunk_tokens=32)
    assert plan.stats["num_merge_units"] > 0
    for w in (w1, w2, w1, w2):
        o, lse, _ = C.run_gpu(w, plan=plan)
        ro, rl = C.run_oracle(w)
        C.assert_parity(w, o, lse, ro, rl, label=f"plan reuse {plan.stats}")


def test_merge_of_many_states_single_request(fi):
    """One request, 32 kv heads, chunk 16: each row merges 19 states, and
    the full-length case (2048 tokens) 128 states, more than one batch of
    the merge kernel's 64; repeated runs are bitwise identical."""
    for small in (True, False):
        w = W.make("single_L2048_h32", small=small)
        plan = C.make_plan(w, chunk_tokens=16)
        o1, l1, _ = C.run_gpu(w, plan=plan)
        ro, rl = C.run_oracle(w)
        C.assert_parity(w, o1, l1, ro, rl, label=f"single chunk 16 small={small}")
        o2, l2, _ = C.run_gpu(w, plan=plan)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        plan.destroy()


@pytest.mark.parametrize("kv", ["bf16", "e4m3"])
@pytest.mark.parametrize("fold", ["1", "0"])
def test_cascade_fold_and_merge_paths(fi, kv, fold):
    """Three prefix groups (one with an empty prefix) and suffixes shorter and
    longer than the chunk: one-chunk suffixes fold their prefix states in the
    decode tile (fold on), the rest go through the merge kernel; with the
    fold off every request is merged.  e4m3 KV exercises the v_scale of the
    folded prefix states."""
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 200, size=11)
    lens[3] = 0
    w = W.build("cascade_mix", lens, Hq=32, Hkv=4, ps=16, q_dtype="bf16", kv_dtype=kv,
                seed=21, prefix_groups=[(4, 700), (3, 0), (4, 333)])
    o, lse, plan = C.run_gpu(w, chunk_tokens=64,
                             tuning=dict(cascade_fold=1 if fold == "1" else -1))
    st = plan.stats
    if fold == "1":
        assert st["num_folded"] > 0 and st["num_merge_units"] > 0
    else:
        assert st["num_folded"] == 0
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl, label=f"cascade mix {kv} fold={fold} {st}")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_merge_states_matches_oracle(fi, dt):
    import oracle
    import torch
    rng = np.random.default_rng(3)
    n_states, rows, D = 5, 37, 128
    vs = rng.standard_normal((n_states, rows, D)).astype(np.float32)
    ss = (rng.standard_normal((n_states, rows)) * 4).astype(np.float32)
    ss[1, :5] = -np.inf
    ss[:, 7] = -np.inf                       # an all-empty row
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]
    vt = [torch.from_numpy(vs[i]).to(tdt).cuda() for i in range(n_states)]
    st = [torch.from_numpy(ss[i]).cuda() for i in range(n_states)]
    vo, so = fi.merge_states(vt, st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    vin = np.stack([v.float().cpu().numpy() for v in vt]).astype(np.float64)
    ro, rl = oracle.merge(vin, ss.astype(np.float64))
    vo = vo.cpu().numpy().astype(np.float64)
    so = so.cpu().numpy().astype(np.float64)
    assert np.all(vo[7] == 0) and np.isneginf(so[7])
    ok = ~np.isneginf(rl)
    assert np.abs(vo - ro).max() <= 1e-5 + 1e-5 * np.abs(ro).max()
    assert np.abs(so[ok] - rl[ok]).max() <= 1e-5


def test_graph_capture_replays(fi):
    """The run stage only enqueues kernels: capture it and replay it several
    times with eager work in between; every replay equals the eager result."""
    import torch
    w = W.make("skewed128", small=True)
    d = C.Dev(w)
    plan = C.make_plan(w, chunk_tokens=64)
    o_e, l_e = plan.run(d.q, d.k, d.v, d.indptr, d.indices, d.last, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    o_e, l_e = o_e.clone(), l_e.clone()
    o = torch.empty_like(o_e)
    lse = torch.empty_like(l_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plan.run(d.q, d.k, d.v, d.indptr, d.indices, d.last, sm_scale=w.sm_scale, o=o, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(d.q, d.k, d.v, d.indptr, d.indices, d.last, sm_scale=w.sm_scale, o=o, lse=lse)
    for i in range(3):
        o.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(lse, l_e), f"replay {i}"


@pytest.mark.gpu
def test_cascade_graph_capture_replays(fi):
    """The cascade run (prefix, folded suffix, merge launches) only enqueues
    kernels: capture it from a side stream into a graph and check that every
    replay equals the eager result."""
    import torch
    w = W.make("cascade256", small=True)
    d = C.Dev(w)
    plan = C.make_plan(w)
    args = (d.q, d.k, d.v, d.p_indptr, d.p_indices, d.p_last, d.indptr, d.indices, d.last)
    o_e, l_e = plan.cascade_run(*args, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    o_e, l_e = o_e.clone(), l_e.clone()
    o = torch.empty_like(o_e)
    lse = torch.empty_like(l_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        plan.cascade_run(*args, sm_scale=w.sm_scale, o=o, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(o, o_e) and torch.equal(lse, l_e), "side-stream run"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.cascade_run(*args, sm_scale=w.sm_scale, o=o, lse=lse)
    for i in range(3):
        o.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(lse, l_e), f"replay {i}"


@pytest.mark.gpu
def test_run_stage_decode_equals_full_run_when_unsplit(fi):
    """fi_debug_run_stage(0) launches the decode kernel exactly as the full
    run does: with every request in one tile per head (no merge), its
    outputs are bitwise those of fi_decode_run."""
    import torch
    w = W.make("batch64_gqa4", small=True)
    d = C.Dev(w)
    plan = C.make_plan(w, chunk_tokens=4096)
    assert plan.stats["num_merge_units"] == 0
    o_r, l_r = plan.run(d.q, d.k, d.v, d.indptr, d.indices, d.last, sm_scale=w.sm_scale)
    o_s, l_s = plan.run_stage(0, d.q, d.k, d.v, d.indptr, d.indices, d.last,
                              sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o_r, o_s) and torch.equal(l_r, l_s)


@pytest.mark.parametrize("name", ["batch64_gqa4", "cascade256"])
def test_run_stages_in_order_equal_the_run(fi, name):
    """Stages 1 (prefix), 0 (decode), 2 (merge) enqueued one by one are the
    full run, bit for bit (the benchmark times its dominant kernel this
    way); split states are merged by stage 2."""
    import torch
    w = W.make(name, small=True)
    d = C.Dev(w)
    plan = C.make_plan(w, chunk_tokens=32)
    st = plan.stats
    assert st["num_merge_units"] > 0
    o_r, l_r, _ = C.run_gpu(w, d=d, plan=plan)
    o = torch.zeros_like(d.q)
    lse = torch.zeros((w.batch, w.num_qo_heads), dtype=torch.float32, device="cuda")
    args = (d.q, d.k, d.v, d.indptr, d.indices, d.last)
    pre = ((d.p_indptr, d.p_indices, d.p_last) if plan.cascade else (None, None, None))
    for sg in ((1, 0, 2) if plan.cascade else (0, 2)):
        plan.run_stage(sg, *args, *pre, d.k_scale, d.v_scale, sm_scale=w.sm_scale, o=o,
                       lse=lse)
    torch.cuda.synchronize()
    assert np.array_equal(o.float().cpu().double().numpy(), o_r)
    assert np.array_equal(lse.cpu().double().numpy(), l_r)


@pytest.mark.gpu
def test_run_stage_prefix_alone(fi):
    """Stage 1 = the cascade prefix kernel.  With no suffix pages and the
    prefix in one chunk, each row's only state comes from the prefix kernel,
    which then writes o / lse itself: equal to the full cascade run and to
    the oracle over the prefix tokens."""
    import torch
    w = W.make("cascade256", small=True)
    B = w.batch
    w.kv_indptr = np.zeros(B + 1, np.int32)
    w.kv_indices = np.zeros(1, np.int32)
    w.last_page_len = np.zeros(B, np.int32)
    d = C.Dev(w)
    # a plan for 8 compute units keeps the 512-token prefix in one chunk
    plan = fi.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                   num_kv_heads=w.num_kv_heads, page_size=w.page_size, head_dim=w.head_dim,
                   q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                   prefix=(w.prefix_qo_indptr, w.prefix_kv_indptr, w.prefix_last_page_len),
                   num_cus=8)
    st = plan.stats
    assert st["num_tiles"] == 0 and st["num_merge_units"] == 0 and st["num_prefix_tiles"] > 0
    o_c, l_c = plan.cascade_run(d.q, d.k, d.v, d.p_indptr, d.p_indices, d.p_last, d.indptr,
                                d.indices, d.last, sm_scale=w.sm_scale)
    o_s, l_s = plan.run_stage(1, d.q, d.k, d.v, d.indptr, d.indices, d.last,
                              d.p_indptr, d.p_indices, d.p_last, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_s) and torch.equal(l_c, l_s)
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o_s.float().cpu().double().numpy(), l_s.cpu().double().numpy(), ro, rl,
                    label="prefix stage vs oracle")
    # a plan without prefix tiles rejects stage 1 in the library
    w2 = W.make("batch64_gqa4", small=True)
    d2 = C.Dev(w2)
    with pytest.raises(fi.FiError):
        C.make_plan(w2).run_stage(1, d2.q, d2.k, d2.v, d2.indptr, d2.indices, d2.last,
                                  sm_scale=w2.sm_scale)


@pytest.mark.parametrize("q_dtype", ["f16", "bf16"])
def test_many_split_requests_take_the_wide_merge(fi, q_dtype):
    """>= 128 split requests go through the merge kernel's wide form (one
    workgroup per request and 32 q heads); same bar as every other path."""
    rng = np.random.default_rng(3)
    lens = rng.integers(40, 200, size=150)
    w = W.build("wide_merge", lens, Hq=16, Hkv=4, ps=16, q_dtype=q_dtype, kv_dtype=q_dtype,
                seed=4)
    o, lse, plan = C.run_gpu(w, chunk_tokens=32)
    assert plan.stats["num_merge_units"] >= 128
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl, label=f"wide merge {q_dtype} {plan.stats}")


@pytest.mark.gpu
@pytest.mark.parametrize("rope", [False, True])
def test_all_requests_empty(fi, rope):
    """A batch whose every key list is empty reads no K/V and no page index:
    the index table and the pools may be empty (NULL); every row is o = 0,
    lse = -inf."""
    import torch
    plan = fi.Plan(np.zeros(4, np.int32), np.zeros(3, np.int32), num_qo_heads=8,
                   num_kv_heads=2, page_size=16,
                   pos_encoding="rope_llama" if rope else "none")
    q = torch.randn(3, 8, 128, device="cuda").half()
    empty = torch.empty(0, device="cuda", dtype=torch.int32)
    k = torch.empty(0, 16, 2, 128, device="cuda", dtype=torch.float16)
    o, lse = plan.run(q, k, k, torch.zeros(4, dtype=torch.int32, device="cuda"), empty,
                      torch.zeros(3, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("L", [0, 1, 15, 16, 17, 300, 2048])
@pytest.mark.parametrize("chunk", [0, 16, 48, 512])
def test_one_request_plans(fi, L, chunk):
    """Plans of one request at every length / chunk edge (empty, one key,
    page and chunk boundaries, a single chunk) against the oracle."""
    w = W.build("one_req", [L], Hq=32, Hkv=8, ps=16, seed=L + 3)
    o, lse, plan = C.run_gpu(w, chunk_tokens=chunk)
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl, label=f"one request L={L} chunk={chunk} {plan.stats}")
    plan.destroy()


def test_replan_loop_reuses_pinned_staging(fi):
    """Re-planning every step (lengths change between decode steps) takes
    its pinned upload buffer from the library's pool: after the first plans
    the pool stops growing (at most 4 buffers per GPU), and every plan's
    work list is the one its lengths ask for."""
    import torch
    base = W.make("batch64_gqa4", small=True)
    counts = []
    for i in range(40):
        lens = base.kv_lens + (i % 7)
        w = W.build("replan", lens, Hq=32, Hkv=8, ps=16, seed=1, tables_only=(i % 10 != 0))
        plan = fi.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=32, num_kv_heads=8,
                       page_size=16, chunk_tokens=[0, 32, 64][i % 3])
        counts.append(plan.stats["staging_buffers"])
        if i % 10 == 0:
            o, lse, _ = C.run_gpu(w, plan=plan)
            ro, rl = C.run_oracle(w)
            C.assert_parity(w, o, lse, ro, rl, label=f"replan {i}")
        torch.cuda.synchronize()
        plan.destroy()
    assert max(counts) <= 4, counts
    assert len(set(counts[5:])) == 1, counts
