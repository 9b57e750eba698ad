"""GPU parity of head-major (HND) pages, [num_pages][Hkv][page_size][D] --
the other kv_layout value beside NHD in the registry quickstart's paged
call.  Rows of one (page, kv head) are contiguous; the kernels take a row at
page * page_bytes + slot * row + head * page_size * row."""
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


@pytest.mark.parametrize("name", W.WORKLOADS)
def test_small_workload_hnd_parity_and_equals_nhd(fi, name):
    """Parity with the oracle reading HND pages, and the same outputs bit
    for bit as the NHD run of the same data (one plan shape, one order of
    every sum)."""
    for w in _variants(W.make(name, small=True)):
        h = W.to_hnd(w)
        o, lse, plan = C.run_gpu(h, chunk_tokens=32)
        ro, rl = C.run_oracle(h)
        C.assert_parity(h, o, lse, ro, rl, label=f"{h.name} {plan.stats}")
        o2, l2, _ = C.run_gpu(w, chunk_tokens=32)
        assert np.array_equal(o, o2) and np.array_equal(lse, l2)


@pytest.mark.parametrize("seed", range(6))
def test_hnd_fuzz_parity(fi, seed):
    rng = np.random.default_rng(12000 + seed)
    ps = int(rng.choice([2, 3, 16, 32]))
    G = int(rng.choice([1, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 7))
    lens = [int(rng.choice([0, 1, ps + 1, int(rng.integers(2, 700))])) for _ in range(B)]
    q_dtype = str(rng.choice(["f16", "bf16"]))
    kv_dtype = str(rng.choice([q_dtype, "e4m3"]))
    groups = [(B, int(rng.choice([0, 7, 200])))] if seed % 2 else None
    w = W.to_hnd(W.build(f"hfuzz{seed}", lens, Hq=Hkv * G, Hkv=Hkv, ps=ps, q_dtype=q_dtype,
                         kv_dtype=kv_dtype, seed=seed, prefix_groups=groups))
    o, lse, plan = C.run_gpu(w, chunk_tokens=[0, 32, 64][seed % 3])
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl, label=f"hnd fuzz{seed} ps{ps} G{G} Hkv{Hkv} "
                                              f"{q_dtype}/{kv_dtype} lens {lens} {groups}")


def test_hnd_append_parity(fi):
    import oracle
    import paged_kv_decode_fi_amd as m
    import torch
    w = W.to_hnd(W.make_append("append_batch16_q128", small=True))
    plan = m.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                  num_kv_heads=w.num_kv_heads, page_size=w.page_size, q_dtype=w.q_dtype,
                  kv_dtype=w.kv_dtype, qo_indptr=w.qo_indptr, kv_layout="paged_hnd")
    d = C.Dev(w)
    o, lse = plan.append_run(d.q, d.k, d.v, d.indptr, d.indices, d.last, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.append(w.q, w.k_pages, w.v_pages, w.qo_indptr, w.kv_indptr, w.kv_indices,
                           w.last_page_len, num_qo_heads=w.num_qo_heads,
                           num_kv_heads=w.num_kv_heads, head_dim=128, page_size=w.page_size,
                           q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, sm_scale=w.sm_scale,
                           kv_layout="HND")
    C.assert_parity(w, o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl,
                    rows=np.ones((w.num_rows, w.num_qo_heads), bool), label="hnd append")
