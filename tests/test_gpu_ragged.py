"""GPU parity of the ragged KV layout (FlashInfer README "core features"
item 1: paged and ragged KV cache): every key list contiguous in K / V
[total, Hkv, D], the indptr tables counting rows, no page indices.  The
kernels take token t of a request at row kv_indptr[r] + t; the oracle reads
the same layout (its ragged mode is pinned against page-size-1 identity
tables on the CPU)."""
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
@pytest.mark.parametrize("chunk", [0, 32])
def test_small_workload_ragged_parity(fi, name, chunk):
    for w in _variants(W.make(name, small=True)):
        r = W.to_ragged(w)
        o, lse, plan = C.run_gpu(r, chunk_tokens=chunk)
        ro, rl = C.run_oracle(r)
        C.assert_parity(r, o, lse, ro, rl, label=f"{r.name} chunk {chunk} {plan.stats}")


def test_ragged_equals_paged_page_size_1_bitwise(fi):
    """long32_fp8 at page size 1 (random page permutation) and the same
    data ragged (contiguous rows): one plan shape, the same logical order of
    every sum, so identical outputs."""
    w = W.make("long32_fp8", small=True)[1]
    r = W.to_ragged(w)
    o1, l1, _ = C.run_gpu(w)
    o2, l2, _ = C.run_gpu(r)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("seed", range(6))
def test_ragged_fuzz_parity(fi, seed):
    rng = np.random.default_rng(11000 + seed)
    G = int(rng.choice([1, 4, 8]))
    Hkv = int(rng.choice([1, 2, 8]))
    B = int(rng.integers(1, 8))
    lens = [int(rng.choice([0, 1, 17, int(rng.integers(2, 900))])) for _ in range(B)]
    q_dtype = str(rng.choice(["f16", "bf16"]))
    kv_dtype = str(rng.choice([q_dtype, "e4m3"]))
    groups = None
    if seed % 2:
        groups = [(B, int(rng.choice([0, 5, 300])))]
    w = W.build(f"rfuzz{seed}", lens, Hq=Hkv * G, Hkv=Hkv, ps=int(rng.choice([1, 16])),
                q_dtype=q_dtype, kv_dtype=kv_dtype, seed=seed, prefix_groups=groups)
    r = W.to_ragged(w)
    o, lse, plan = C.run_gpu(r, chunk_tokens=[0, 32, 64][seed % 3])
    ro, rl = C.run_oracle(r)
    C.assert_parity(r, o, lse, ro, rl,
                    label=f"ragged fuzz{seed} G{G} Hkv{Hkv} {q_dtype}/{kv_dtype} lens {lens} "
                          f"groups {groups}")


def test_ragged_append_parity(fi):
    import oracle
    import paged_kv_decode_fi_amd as m
    import torch
    w = W.make_append("append_batch16_q128", small=True)
    r = W.to_ragged(w)
    plan = m.Plan(r.kv_indptr, None, num_qo_heads=r.num_qo_heads, num_kv_heads=r.num_kv_heads,
                  page_size=1, q_dtype=r.q_dtype, kv_dtype=r.kv_dtype, qo_indptr=r.qo_indptr,
                  kv_layout="ragged")
    d = C.Dev(r)
    o, lse = plan.append_run(d.q, d.k, d.v, d.indptr, None, None, sm_scale=r.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.append(r.q, r.k_pages, r.v_pages, r.qo_indptr, r.kv_indptr, None, None,
                           num_qo_heads=r.num_qo_heads, num_kv_heads=r.num_kv_heads,
                           head_dim=128, page_size=1, q_dtype=r.q_dtype, kv_dtype=r.kv_dtype,
                           sm_scale=r.sm_scale)
    C.assert_parity(r, o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl,
                    rows=np.ones((r.num_rows, r.num_qo_heads), bool), label="ragged append")
