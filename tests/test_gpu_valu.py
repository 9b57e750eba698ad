"""The VALU decode instance (tuning score_path = 2: scores as packed 16-bit
dot products with fp32 accumulation, P.V as fp32 FMAs, no MFMA) against the
fp64 oracle, for 1, 2 and 4 q heads per kv head, every K/V dtype, page sizes
1 and 16, with and without split-KV partial states.  It computes the same
function as the MFMA instance, so the same acceptance bar applies."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fi():
    import paged_kv_decode_fi_amd as m
    return m


@pytest.mark.parametrize("G", [1, 2, 4])
@pytest.mark.parametrize("dt", [("f16", "f16"), ("bf16", "bf16"), ("f16", "e4m3"),
                                ("bf16", "e4m3")])
@pytest.mark.parametrize("ps,chunk", [(16, 0), (1, 48), (7, 32)])
def test_valu_decode_parity(fi, G, dt, ps, chunk):
    rng = np.random.default_rng(G * 100 + ps)
    lens = rng.integers(0, 900, size=7)
    lens[1], lens[3] = 1, 17
    Hkv = 8 // G if G < 8 else 1
    w = W.build(f"valu_G{G}", lens, Hq=G * Hkv * 2, Hkv=Hkv * 2, ps=ps, q_dtype=dt[0],
                kv_dtype=dt[1], seed=11 + G + ps)
    o, lse, plan = C.run_gpu(w, chunk_tokens=chunk, tuning=dict(score_path=2))
    assert plan.stats["valu_heads"] == G, plan.stats
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl, label=f"valu G{G} {dt} ps{ps} chunk{chunk} {plan.stats}")
    plan.destroy()


@pytest.mark.parametrize("name", ["single_L2048_h32", "batch64_gqa4", "skewed128"])
def test_valu_small_workloads(fi, name):
    w = W.make(name, small=True)
    o, lse, plan = C.run_gpu(w, tuning=dict(score_path=2))
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl, label=f"valu {name}")
    plan.destroy()


def test_valu_refuses_what_is_not_built(fi):
    w = W.build("valu_g8", [100], Hq=8, Hkv=1, ps=16, seed=1)
    with pytest.raises(fi.FiError):
        C.make_plan(w, tuning=dict(score_path=2))
