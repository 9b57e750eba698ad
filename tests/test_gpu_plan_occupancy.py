"""The decode wave target of fi_plan on a GPU: the chunk search aims at one
round of the waves the device keeps resident of the decode kernel the run
will launch (hipOccupancyMaxActiveBlocksPerMultiprocessor on that
instance), capped at 16 per CU -- the load-balanced plan stage of the
FlashInfer README ("core features" item 2) sized for this chip's registers.
The register-heavier instances (LLaMA-style RoPE, head_dim 256) keep fewer
waves resident than plain decode at head_dim 128, so their plans cut longer
chunks; what each computes is unchanged (parity below)."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fi():
    import paged_kv_decode_fi_amd as m
    return m


def _plan(fi, lens, D=128, **kw):
    lens = np.asarray(lens)
    n = (lens + 15) // 16
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = np.where(n > 0, lens - (n - 1) * 16, 0).astype(np.int32)
    return fi.Plan(indptr, last, num_qo_heads=32, num_kv_heads=8, page_size=16, head_dim=D,
                   **kw).stats


def test_wave_target_follows_the_launched_kernel(fi):
    lens = np.random.default_rng(7).integers(512, 4097, size=64)
    plain = _plan(fi, lens)
    rope = _plan(fi, lens, pos_encoding="rope_llama")
    d256 = _plan(fi, lens, D=256)
    forced = _plan(fi, lens, pos_encoding="rope_llama", tuning={"waves_per_cu": 16})
    for st in (plain, rope, d256):
        assert st["heads_per_tile"] <= st["decode_waves_per_cu"] <= 16, st
        # uniform lengths: one round of resident waves
        assert st["num_tiles"] * st["heads_per_tile"] <= \
            st["num_cus"] * st["decode_waves_per_cu"], st
    assert rope["decode_waves_per_cu"] < plain["decode_waves_per_cu"], (rope, plain)
    assert d256["decode_waves_per_cu"] < plain["decode_waves_per_cu"], (d256, plain)
    assert forced["decode_waves_per_cu"] == 16
    assert rope["chunk_tokens"] > forced["chunk_tokens"], (rope, forced)


@pytest.mark.parametrize("rope", [False, True])
def test_occupancy_sized_plans_match_the_oracle(fi, rope):
    lens = np.random.default_rng(11).integers(512, 4097, size=12)
    w = W.build("occupancy_plan", lens, Hq=32, Hkv=8, D=128, ps=16, q_dtype="f16",
                kv_dtype="f16", seed=77)
    r = (1e4, 1.0) if rope else None
    o, lse, plan = C.run_gpu(w, rope=r)
    ro, rl = C.run_oracle(w, rope=r)
    C.assert_parity(w, o, lse, ro, rl, label=f"occupancy plan rope={rope} {plan.stats}")


def test_device_plans_choose_tile_width_by_load(fi):
    """On the device (occupancy-sized wave targets) the skewed mix gets
    four-head tiles and the uniform batch of 64 and the 32K batch keep
    eight."""
    want = {"skewed128": 4, "batch64_gqa4": 8, "long32_fp8": 8}
    for name, hpt in want.items():
        w = W.make(name, tables_only=True)
        w = w[16] if isinstance(w, dict) else w
        plan = fi.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                       num_kv_heads=w.num_kv_heads, page_size=w.page_size,
                       q_dtype=w.q_dtype, kv_dtype=w.kv_dtype)
        st = plan.stats
        assert st["heads_per_tile"] == hpt, (name, st)
        plan.destroy()
