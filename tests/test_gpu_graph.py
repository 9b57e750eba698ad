"""Graph capture of every run entry point beyond plain decode and the
single-level cascade (those two are covered with the parity suite): append,
RoPE decode, RoPE cascade and append, cascades of several levels, head_dim 64
and 256, the ragged layout.  The run stage only enqueues kernels (FlashInfer README core
features, graph-capturable run stage), so each call is captured once and
replayed several times with eager work and synchronisations in between;
every replay must equal the eager result bit for bit."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fi():
    import paged_kv_decode_fi_amd as m
    return m


def _check_graph(run):
    """run(o, lse) enqueues one call writing into o / lse (None: allocate)."""
    import torch
    o_e, l_e = run(None, None)
    torch.cuda.synchronize()
    o_e, l_e = o_e.clone(), l_e.clone()
    o, lse = torch.empty_like(o_e), torch.empty_like(l_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(o, lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(o, o_e) and torch.equal(lse, l_e), "side-stream run"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(o, lse)
    scratch = torch.zeros(1 << 20, device="cuda")
    for i in range(3):
        o.fill_(0)
        lse.fill_(0)
        scratch.add_(1.0)                 # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(lse, l_e), f"replay {i}"
    return o_e, l_e


@pytest.mark.parametrize("chunk", [0, 64])
def test_append_graph(fi, chunk):
    w = W.make_append("append_batch16_q128", small=True)
    d = C.Dev(w)
    plan = fi.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                   num_kv_heads=w.num_kv_heads, page_size=w.page_size, q_dtype=w.q_dtype,
                   kv_dtype=w.kv_dtype, qo_indptr=w.qo_indptr, causal=w.causal,
                   chunk_tokens=chunk)
    _check_graph(lambda o, lse: plan.append_run(d.q, d.k, d.v, d.indptr, d.indices, d.last,
                                                sm_scale=w.sm_scale, o=o, lse=lse))
    if chunk:
        assert plan.stats["num_merge_units"] > 0


def test_rope_decode_graph(fi):
    w = W.make("batch64_gqa4", small=True)
    d = C.Dev(w)
    plan = C.make_plan(w, chunk_tokens=32, rope=(1e4, 1.0))
    o, lse = _check_graph(lambda o, lse: plan.run(d.q, d.k, d.v, d.indptr, d.indices, d.last,
                                                  sm_scale=w.sm_scale, o=o, lse=lse))
    ro, rl = C.run_oracle(w, rope=(1e4, 1.0))
    C.assert_parity(w, o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl,
                    label="RoPE decode, graph")


def test_rope_cascade_and_append_graph(fi):
    """RoPE on the multi-row kernel (cascade prefix tiles with their query
    positions, then the RoPE suffix decode and the merge; an append plan)."""
    rope = (1e4, 1.0)
    w = W.make("cascade256", small=True)
    d = C.Dev(w)
    plan = C.make_plan(w, rope=rope)
    o, lse = _check_graph(lambda o, lse: plan.cascade_run(
        d.q, d.k, d.v, d.p_indptr, d.p_indices, d.p_last, d.indptr, d.indices, d.last,
        sm_scale=w.sm_scale, o=o, lse=lse))
    ro, rl = C.run_oracle(w, rope=rope)
    C.assert_parity(w, o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl,
                    label="RoPE cascade, graph")
    wa = W.make_append("append_batch16_q128", small=True)
    da = C.Dev(wa)
    pa = fi.Plan(wa.kv_indptr, wa.last_page_len, num_qo_heads=wa.num_qo_heads,
                 num_kv_heads=wa.num_kv_heads, page_size=wa.page_size, q_dtype=wa.q_dtype,
                 kv_dtype=wa.kv_dtype, qo_indptr=wa.qo_indptr, causal=wa.causal,
                 pos_encoding="rope_llama", rope_theta=rope[0], rope_scale=rope[1])
    _check_graph(lambda o, lse: pa.append_run(da.q, da.k, da.v, da.indptr, da.indices,
                                              da.last, sm_scale=wa.sm_scale, o=o, lse=lse))


def test_cascade_levels_graph(fi):
    w = W.build_multilevel("lvg", [9, 0, 130, 1, 64, 300], [[(6, 100)], [(3, 0), (3, 77)]],
                           Hq=16, Hkv=2, ps=16, q_dtype="bf16", kv_dtype="bf16", seed=21)
    lv = w.meta["levels"]
    d = C.Dev(w)
    plan = fi.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                   num_kv_heads=w.num_kv_heads, page_size=w.page_size, q_dtype=w.q_dtype,
                   kv_dtype=w.kv_dtype, chunk_tokens=32,
                   levels=[(qo, ip, la) for (qo, ip, ix, la, _) in lv])
    tabs = [(C.to_dev(ip), C.to_dev(ix), C.to_dev(la)) for (qo, ip, ix, la, _) in lv]
    _check_graph(lambda o, lse: plan.cascade_run_levels(d.q, d.k, d.v, tabs, d.indptr,
                                                        d.indices, d.last, sm_scale=w.sm_scale,
                                                        o=o, lse=lse))


@pytest.mark.parametrize("D", [64, 256])
def test_head_dim_graph(fi, D):
    rng = np.random.default_rng(D)
    w = W.build(f"g{D}", list(rng.integers(1, 700, size=7)), Hq=32, Hkv=8, D=D, ps=16,
                q_dtype="f16", kv_dtype="e4m3", seed=D)
    d = C.Dev(w)
    plan = C.make_plan(w, chunk_tokens=64)
    _check_graph(lambda o, lse: plan.run(d.q, d.k, d.v, d.indptr, d.indices, d.last,
                                         d.k_scale, d.v_scale, sm_scale=w.sm_scale, o=o,
                                         lse=lse))


def test_ragged_graph(fi):
    w = W.to_ragged(W.make("skewed128", small=True))
    d = C.Dev(w)
    plan = C.make_plan(w, chunk_tokens=32)
    _check_graph(lambda o, lse: plan.run(d.q, d.k, d.v, d.indptr, d.indices, d.last,
                                         sm_scale=w.sm_scale, o=o, lse=lse))
