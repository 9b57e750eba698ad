"""The reading behind the converted-q decode instance (bf16 q over e4m3 K/V
computed in fp16): scaling a group of bf16 values by 2^e, with e chosen so
that the group's largest magnitude m lands in [2^14, 2^15), makes every value
an exact fp16 value unless it lies more than 2^28 below m (an fp16 subnormal),
and the score taken back by 2^-e equals the unscaled dot product up to the
fp32 accumulation.  CPU only: numpy's float16 is IEEE binary16 (round to
nearest even), the bf16 values are float32 with the low 16 bits clear."""
import math

import numpy as np
import pytest


def _bf16(rng, n, lo, hi):
    x = (rng.standard_normal(n) * np.exp2(rng.uniform(lo, hi, n))).astype(np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def _scale_exp(m):
    # 2^e m in [2^14, 2^15): m = f 2^E with f in [0.5, 1)  ->  e = 15 - E
    return min(15 - math.frexp(float(m))[1], 64) if m > 0 else 0


@pytest.mark.parametrize("seed", range(8))
def test_bf16_group_scaled_into_fp16_is_exact_above_the_subnormal_floor(seed):
    rng = np.random.default_rng(seed)
    lo, hi = [(-3, 3), (-40, -20), (20, 60), (-30, 10), (-1, 1), (-60, 60), (0, 0), (-100, -90)][seed]
    x = _bf16(rng, 4096, lo, hi)
    m = float(np.abs(x).max())
    e = _scale_exp(m)
    y = np.ldexp(x.astype(np.float64), e)
    assert 2.0 ** 14 <= np.abs(y).max() < 2.0 ** 15 or e == 64
    h = y.astype(np.float16).astype(np.float64)
    normal = np.abs(y) >= 2.0 ** -14
    assert np.array_equal(h[normal], y[normal])           # exact where fp16 is normal
    # below the floor: off by at most half an fp16 subnormal step (2^-25),
    # i.e. < 2^-39 of the group's maximum -- or, when e is capped at 64 (a
    # group below 2^-49), by < 2^-89 in the unscaled values
    assert np.all(np.abs(h - y) <= 2.0 ** -25)
    if e < 64:
        assert np.all(np.abs(h - y) <= 2.0 ** -39 * np.abs(y).max())
    else:
        assert m < 2.0 ** -49
        assert np.all(np.abs(np.ldexp(h, -e) - x) <= 2.0 ** -89)


def test_scaled_score_equals_the_unscaled_one():
    rng = np.random.default_rng(11)
    q = _bf16(rng, 128, -2, 2)
    k = rng.integers(-448, 449, 128).astype(np.float64)   # e4m3-range key values
    e = _scale_exp(float(np.abs(q).max()))
    qh = np.ldexp(q.astype(np.float64), e).astype(np.float16).astype(np.float64)
    s_scaled = math.ldexp(float(np.dot(qh, k)), -e)
    assert s_scaled == pytest.approx(float(np.dot(q.astype(np.float64), k)), rel=0, abs=1e-12)
