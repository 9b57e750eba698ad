"""bf16 cascade decode over short shared prefixes (a few keys, empty or
one-key suffixes): the rows whose whole key set is a handful of prefix keys
are the case where rounding p to bf16 before P.V would move o past the
accuracy bar, so the plan must select the prefix launch that passes p with a
bf16 residual.  Compared element by element with the fp64 oracle."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fi():
    import paged_kv_decode_fi_amd as m
    return m


@pytest.mark.parametrize("ps", [1, 16])
@pytest.mark.parametrize("plen", [2, 3, 4, 8])
@pytest.mark.parametrize("suffix", [0, 1])
def test_bf16_short_prefix(fi, ps, plen, suffix):
    # 4 groups of 64 requests, each group's prefix `plen` keys (one group
    # longer, 300 keys, so one launch mixes short and long prefixes); G = 8
    # q heads per kv head as in the cascade workload
    groups = [(64, plen), (64, plen), (64, 300), (64, plen)]
    lens = np.full(256, suffix, np.int64)
    w = W.build(f"short_prefix_{plen}", lens, Hq=64, Hkv=8, ps=ps, q_dtype="bf16",
                kv_dtype="bf16", seed=7000 + 10 * plen + suffix + ps, prefix_groups=groups)
    o, lse, plan = C.run_gpu(w)
    assert plan.stats["prefix_split_p"] & 1, plan.stats
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl, label=f"bf16 prefix {plen} keys ps {ps} "
                                              f"suffix {suffix} {plan.stats}")
    plan.destroy()


def test_long_prefix_keeps_single_p(fi):
    """A level whose prefixes are all long keeps the single-p instance (the
    cascade workload's 8,192-key prefix); forcing either choice through the
    tuning computes the same function within the bar."""
    w = W.make("cascade256", small=True)
    assert w.prefix_lens.min() >= 256
    ro, rl = C.run_oracle(w)
    for force, bit in ((0, 0), (1, 1), (-1, 0)):
        o, lse, plan = C.run_gpu(w, tuning=dict(prefix_split_p=force))
        assert (plan.stats["prefix_split_p"] & 1) == bit, (force, plan.stats)
        C.assert_parity(w, o, lse, ro, rl, label=f"cascade256 small split_p={force}")
        plan.destroy()
