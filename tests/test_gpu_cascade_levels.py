"""GPU parity of cascade decoding with several shared levels (README "core
features" item 3: cascade attention over a hierarchical KV cache): each
request attends over its group's prefix at every level, outermost first,
then its own pages; one prefix kernel launch per level writes the states,
which the suffix tile folds in or the merge pass combines."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fi():
    import paged_kv_decode_fi_amd as m
    return m


def _run(w, chunk_tokens=0, levels_api=True, rope=None):
    import paged_kv_decode_fi_amd as m
    import torch
    lv = w.meta["levels"]
    d = C.Dev(w)
    plan = m.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                  num_kv_heads=w.num_kv_heads, page_size=w.page_size, q_dtype=w.q_dtype,
                  kv_dtype=w.kv_dtype, chunk_tokens=chunk_tokens,
                  levels=[(qo, ip, la) for (qo, ip, ix, la, _) in lv] if levels_api else None,
                  prefix=None if levels_api else (lv[0][0], lv[0][1], lv[0][3]),
                  pos_encoding="none" if rope is None else "rope_llama",
                  rope_theta=0.0 if rope is None else rope[0],
                  rope_scale=0.0 if rope is None else rope[1])
    tabs = [(C.to_dev(ip), C.to_dev(ix), C.to_dev(la)) for (qo, ip, ix, la, _) in lv]
    if levels_api:
        o, lse = plan.cascade_run_levels(d.q, d.k, d.v, tabs, d.indptr, d.indices, d.last,
                                         d.k_scale, d.v_scale, sm_scale=w.sm_scale)
    else:
        o, lse = plan.cascade_run(d.q, d.k, d.v, *tabs[0], d.indptr, d.indices, d.last,
                                  d.k_scale, d.v_scale, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy(), plan


def _oracle(w, rope=None):
    import oracle
    lv = [(qo, ip, ix, la) for (qo, ip, ix, la, _) in w.meta["levels"]]
    return oracle.cascade_levels(w.q, w.k_pages, w.v_pages, lv, w.kv_indptr, w.kv_indices,
                                 w.last_page_len, num_qo_heads=w.num_qo_heads,
                                 num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                                 page_size=w.page_size, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                                 sm_scale=w.sm_scale, k_scale=w.k_scale, v_scale=w.v_scale,
                                 rope=rope)


LEVEL_SPECS = [
    [[(6, 500)], [(2, 40), (4, 300)]],
    [[(6, 100)], [(3, 0), (3, 77)], [(1, 5), (2, 33), (3, 600)]],
    [[(2, 17), (4, 1)], [(6, 260)]],
]


@pytest.mark.parametrize("spec", range(len(LEVEL_SPECS)))
@pytest.mark.parametrize("dt", [("f16", "f16"), ("bf16", "bf16"), ("bf16", "e4m3")])
@pytest.mark.parametrize("chunk", [0, 32])
def test_multilevel_cascade_parity(fi, spec, dt, chunk):
    w = W.build_multilevel(f"ml{spec}", [9, 0, 130, 1, 64, 300], LEVEL_SPECS[spec], Hq=16,
                           Hkv=2, ps=16, q_dtype=dt[0], kv_dtype=dt[1], seed=spec)
    o, lse, plan = _run(w, chunk_tokens=chunk)
    ro, rl = _oracle(w)
    C.assert_parity(w, o, lse, ro, rl, label=f"levels {LEVEL_SPECS[spec]} {dt} chunk {chunk} "
                                              f"{plan.stats}")


def test_one_level_through_both_entry_points_is_bitwise_equal(fi):
    w = W.build_multilevel("ml1", [9, 0, 130, 1], [[(1, 40), (3, 500)]], Hq=8, Hkv=2, ps=16,
                           seed=9)
    o1, l1, _ = _run(w, levels_api=True)
    o2, l2, _ = _run(w, levels_api=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("spec", range(len(LEVEL_SPECS)))
@pytest.mark.parametrize("dt", [("f16", "f16"), ("bf16", "bf16"), ("bf16", "e4m3")])
def test_multilevel_cascade_rope_parity(fi, spec, dt):
    """RoPE over several levels: a request's keys sit at their index in the
    concatenation of its groups' prefixes (outermost first) and its own
    pages; each level's tiles turn the query by its position relative to
    that level's first key."""
    rope = (1e4, 1.0)
    w = W.build_multilevel(f"mlr{spec}", [9, 0, 130, 1, 64, 300], LEVEL_SPECS[spec], Hq=16,
                           Hkv=2, ps=16, q_dtype=dt[0], kv_dtype=dt[1], seed=40 + spec)
    o, lse, plan = _run(w, rope=rope)
    ro, rl = _oracle(w, rope=rope)
    C.assert_parity(w, o, lse, ro, rl, label=f"rope levels {LEVEL_SPECS[spec]} {dt} "
                                              f"{plan.stats}")
