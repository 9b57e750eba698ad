"""Randomised GPU parity sweep across every path at once: plain and RoPE
decode, a cascade level, several levels, append; NHD / HND / ragged layouts;
head_dim 64 / 128 / 256; page sizes 1, 3, 16, 32; every dtype pair; forced
chunk sizes.  Each seed draws one case (lengths with empty, one-token,
page-boundary and long requests) and compares every output element with the
fp64 oracle at the acceptance bar."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu

DT = [("f16", "f16"), ("bf16", "bf16"), ("f16", "e4m3"), ("bf16", "e4m3")]


def _partition(rng, B):
    """Random sizes of contiguous request groups covering a batch of B."""
    sizes, left = [], B
    while left:
        k = int(rng.integers(1, left + 1))
        sizes.append(k)
        left -= k
    return sizes


@pytest.fixture(scope="module")
def fi():
    import paged_kv_decode_fi_amd as m
    return m


@pytest.mark.parametrize("seed", range(60000, 60048))
def test_random_case_parity(fi, seed):
    import oracle
    import torch
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128, 128, 256]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 9))
    ps = int(rng.choice([1, 3, 16, 16, 32]))
    qd, kd = DT[int(rng.integers(0, 4))]
    kind = str(rng.choice(["decode", "rope", "cascade", "append", "levels"]))
    layout = str(rng.choice(["paged", "paged", "hnd", "ragged"]))
    chunk = int(rng.choice([0, 0, 32, 64, 128]))
    lens = [int(rng.choice([0, 1, 15, 16, 17, int(rng.integers(2, 1200))])) for _ in range(B)]
    label = (f"seed {seed} {kind} D{D} G{G} Hkv{Hkv} B{B} ps{ps} {qd}/{kd} {layout} "
             f"chunk {chunk} lens {lens}")
    if kind in ("decode", "rope", "cascade"):
        groups = None
        if kind == "cascade":
            groups = [(k, int(rng.choice([0, 1, 40, int(rng.integers(2, 2000))])))
                      for k in _partition(rng, B)]
        w = W.build("fz", lens, Hq=Hkv * G, Hkv=Hkv, D=D, ps=ps, q_dtype=qd, kv_dtype=kd,
                    seed=seed, prefix_groups=groups)
        if layout == "hnd":
            w = W.to_hnd(w)
        elif layout == "ragged":
            w = W.to_ragged(w)
        rope = None
        if kind == "rope":
            rope = (float(rng.choice([1e4, 5e5])), float(rng.choice([1.0, 4.0])))
        o, lse, plan = C.run_gpu(w, chunk_tokens=chunk, rope=rope)
        ro, rl = C.run_oracle(w, rope=rope)
        C.assert_parity(w, o, lse, ro, rl, label=label)
        plan.destroy()
    elif kind == "levels":
        levels = [[(k, int(rng.choice([0, 1, 33, int(rng.integers(2, 700))])))
                   for k in _partition(rng, B)] for _ in range(int(rng.integers(1, 4)))]
        w = W.build_multilevel("lv", lens, levels, Hq=Hkv * G, Hkv=Hkv, D=D, ps=ps,
                               q_dtype=qd, kv_dtype=kd, seed=seed)
        lv = w.meta["levels"]
        d = C.Dev(w)
        plan = fi.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                       num_kv_heads=w.num_kv_heads, page_size=w.page_size, head_dim=D,
                       q_dtype=qd, kv_dtype=kd, chunk_tokens=chunk,
                       levels=[(qo, ip, la) for (qo, ip, ix, la, _) in lv])
        tabs = [(C.to_dev(ip), C.to_dev(ix), C.to_dev(la)) for (qo, ip, ix, la, _) in lv]
        o, lse = plan.cascade_run_levels(d.q, d.k, d.v, tabs, d.indptr, d.indices, d.last,
                                         d.k_scale, d.v_scale, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        ro, rl = oracle.cascade_levels(w.q, w.k_pages, w.v_pages,
                                       [(qo, ip, ix, la) for (qo, ip, ix, la, _) in lv],
                                       w.kv_indptr, w.kv_indices, w.last_page_len,
                                       num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                                       head_dim=D, page_size=ps, q_dtype=qd, kv_dtype=kd,
                                       sm_scale=w.sm_scale, k_scale=w.k_scale, v_scale=w.v_scale)
        C.assert_parity(w, o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro,
                        rl, label=label)
        plan.destroy()
    else:
        L = np.array([max(x, 1) for x in lens])
        q_lens = np.array([int(rng.choice([0, 1, int(n), int(rng.integers(1, n + 1))]))
                           for n in L])
        causal = bool(rng.integers(0, 4) != 0)
        w = W.build_append("ap", L, q_lens, Hq=Hkv * G, Hkv=Hkv, D=D, ps=ps, q_dtype=qd,
                           kv_dtype=kd, seed=seed, causal=causal)
        d = C.Dev(w)
        plan = fi.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                       num_kv_heads=w.num_kv_heads, page_size=ps, head_dim=D, q_dtype=qd,
                       kv_dtype=kd, qo_indptr=w.qo_indptr, causal=causal, chunk_tokens=chunk)
        o, lse = plan.append_run(d.q, d.k, d.v, d.indptr, d.indices, d.last, d.k_scale,
                                 d.v_scale, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        ro, rl = oracle.append(w.q, w.k_pages, w.v_pages, w.qo_indptr, w.kv_indptr, w.kv_indices,
                               w.last_page_len, num_qo_heads=w.num_qo_heads,
                               num_kv_heads=w.num_kv_heads, head_dim=D, page_size=ps,
                               q_dtype=qd, kv_dtype=kd, sm_scale=w.sm_scale, causal=causal,
                               k_scale=w.k_scale, v_scale=w.v_scale)
        if w.num_rows:
            C.assert_parity(w, o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro,
                            rl, rows=np.ones((w.num_rows, w.num_qo_heads), bool),
                            label=f"{label} causal {causal} q {list(q_lens)}")
        plan.destroy()
