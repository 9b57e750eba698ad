"""GPU parity of decode with LLaMA-style RoPE applied on the fly (FlashInfer
README decode example, pos_encoding_mode ROPE_LLAMA) against the fp64 oracle
with the same rotation: rotate-half pairs (x_i, x_{i+D/2}) turned by
pos / scale * theta^(-2 i / D), key t of a request at position t, the query
at kv_len - 1.

The kernel turns each key back by its distance from the query (relative
form: q enters the score MFMAs as stored) in fp32 with an fp32 (cos, sin)
table, and passes the turned key as a 16-bit high part plus a 16-bit
residual; the oracle rotates q and every key by their positions in fp64.
The same acceptance bar as plain decode applies."""
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


@pytest.mark.parametrize("name", ["single_L2048_h32", "batch64_gqa4", "skewed128",
                                  "long32_fp8"])
@pytest.mark.parametrize("chunk", [0, 32])
def test_small_workload_rope_parity(fi, name, chunk):
    rope = (1e4, 1.0)
    for w in _variants(W.make(name, small=True)):
        o, lse, plan = C.run_gpu(w, chunk_tokens=chunk, rope=rope)
        ro, rl = C.run_oracle(w, rope=rope)
        C.assert_parity(w, o, lse, ro, rl, label=f"{w.name} rope chunk {chunk} {plan.stats}")
        # the rotation must matter: plain decode of the same data differs
        po, _ = C.run_oracle(w)
        assert np.abs(po - ro).max() > 10 * (C.TOL_ABS + C.TOL_REL), "RoPE had no effect"


def _rope_fuzz_case(seed):
    rng = np.random.default_rng(7000 + seed)
    ps = int(rng.choice([1, 3, 16]))
    G = int(rng.choice([1, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 8))
    choices = [0, 1, ps, ps + 1, int(rng.integers(2, 900))]
    lens = [int(rng.choice(choices)) for _ in range(B)]
    q_dtype = str(rng.choice(["f16", "bf16"]))
    kv_dtype = str(rng.choice([q_dtype, "e4m3"]))
    theta = float(rng.choice([1e4, 5e5]))
    scale = float(rng.choice([1.0, 8.0, 0.5]))
    w = W.build(f"rope_fuzz{seed}", lens, Hq=Hkv * G, Hkv=Hkv, ps=ps, q_dtype=q_dtype,
                kv_dtype=kv_dtype, seed=seed)
    return w, (theta, scale)


@pytest.mark.parametrize("seed", range(12))
def test_rope_fuzz_parity(fi, seed):
    w, rope = _rope_fuzz_case(seed)
    chunk = [0, 32, 48][seed % 3]
    o, lse, plan = C.run_gpu(w, chunk_tokens=chunk, rope=rope)
    ro, rl = C.run_oracle(w, rope=rope)
    C.assert_parity(w, o, lse, ro, rl,
                    label=f"rope fuzz{seed} {rope} B{w.batch} G{w.group_size} "
                          f"Hkv{w.num_kv_heads} ps{w.page_size} {w.q_dtype}/{w.kv_dtype} "
                          f"lens {list(w.kv_lens)}")


def test_rope_split_equals_unsplit(fi):
    """Positions are absolute token indices, so chunking the same request
    differently changes only the summation order."""
    w = W.build("rope_split", [700, 1], Hq=8, Hkv=2, ps=16, q_dtype="f16",
                kv_dtype="f16", seed=3)
    rope = (1e4, 1.0)
    o0, l0, _ = C.run_gpu(w, rope=rope)
    o1, l1, _ = C.run_gpu(w, chunk_tokens=32, rope=rope)
    assert np.abs(o0 - o1).max() < 2e-3 and np.abs(l0 - l1).max() < 1e-4


def test_rope_cascade_plan_is_rejected(fi):
    w = W.make("cascade256", small=True)
    with pytest.raises(RuntimeError, match="RoPE"):
        C.make_plan(w, rope=(1e4, 1.0))


@pytest.mark.parametrize("case", range(8))
def test_rope_single_rounded_fp16_key(fi, case):
    """fp16 q with every request at least 64 keys long: the plan passes each
    turned key to the score as one fp16 value (turned in packed fp16 against
    an fp16 (cos, sin) table, no residual), whose rounding stays well inside
    the lse bar over that many keys; tiles of fewer than head_dim / 32 kv
    heads keep the residual form."""
    rng = np.random.default_rng(900 + case)
    G = [1, 4, 8, 4, 16, 2, 8, 4][case]
    Hkv = [8, 8, 4, 2, 1, 4, 8, 8][case]
    ps = [16, 1, 16, 7, 16, 32, 16, 1][case]
    D = [128, 128, 128, 128, 128, 64, 256, 128][case]
    kv = "e4m3" if case in (3, 7) else "f16"
    lens = rng.integers(64, 3000, size=int(rng.integers(1, 9)))
    w = W.build(f"rope_single{case}", lens, Hq=G * Hkv, Hkv=Hkv, D=D, ps=ps, q_dtype="f16",
                kv_dtype=kv, seed=50 + case)
    rope = (float(rng.choice([1e4, 5e5])), 1.0)
    o, lse, plan = C.run_gpu(w, chunk_tokens=[0, 64][case % 2], rope=rope)
    # (the fp16 table rows of a step are copied one 16-byte vector per
    # thread, which needs head_dim / 32 kv heads per tile)
    want = int(plan.stats["heads_per_tile"] * 32 >= D)
    assert plan.stats["rope_single"] == want, plan.stats
    ro, rl = C.run_oracle(w, rope=rope)
    C.assert_parity(w, o, lse, ro, rl, label=f"rope single {case} lens {list(lens)}")


def test_rope_residual_kept_where_needed(fi):
    """A request shorter than 64 keys, bf16 q, or tiles of fewer than
    head_dim / 32 kv heads keep the turned key's residual; forcing either
    form on a long-request plan computes the same function."""
    short = W.build("rope_short", [700, 20], Hq=8, Hkv=2, ps=16, q_dtype="f16",
                    kv_dtype="f16", seed=4)
    bf = W.build("rope_bf16", [700, 200], Hq=8, Hkv=2, ps=16, q_dtype="bf16",
                 kv_dtype="bf16", seed=4)
    rope = (1e4, 1.0)
    for w in (short, bf, W.build("rope_narrow", [700, 300], Hq=8, Hkv=2, ps=16,
                                  q_dtype="f16", kv_dtype="f16", seed=4)):
        o, lse, plan = C.run_gpu(w, rope=rope, tuning=dict(rope_split_k=-1)
                                 if w.name == "rope_narrow" else None)
        assert plan.stats["rope_single"] == 0
        ro, rl = C.run_oracle(w, rope=rope)
        C.assert_parity(w, o, lse, ro, rl, label=f"{w.name} residual kept")
    lng = W.build("rope_long", [700, 300], Hq=16, Hkv=4, ps=16, q_dtype="f16",
                  kv_dtype="f16", seed=4)
    ro, rl = C.run_oracle(lng, rope=rope)
    for force, want in ((1, 0), (0, 1), (-1, 1)):
        o, lse, plan = C.run_gpu(lng, rope=rope,
                                 tuning=dict(rope_split_k=force, heads_per_tile=4))
        assert plan.stats["rope_single"] == want, (force, plan.stats)
        C.assert_parity(lng, o, lse, ro, rl, label=f"rope_split_k={force}")
