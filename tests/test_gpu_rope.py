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


# ---- RoPE on the multi-row kernel: cascade levels and batch append ---------
# The oracle rotates q and every key by their positions in the request's
# whole key list (cascade: the group's prefix tokens first, then the own
# tokens; append: query token i of n at L - n + i).  The prefix / append
# tiles turn each query row by its position relative to the start of the
# tile's key list and each key by its index there, in fp32, and carry both
# as a 16-bit high part plus residual through three score MFMAs.


@pytest.mark.parametrize("chunk", [0, 32])
def test_small_cascade_rope_parity(fi, chunk):
    rope = (1e4, 1.0)
    w = W.make("cascade256", small=True)
    o, lse, plan = C.run_gpu(w, chunk_tokens=chunk, rope=rope)
    assert plan.stats["num_prefix_tiles"] > 0 and plan.stats["num_folded"] == 0
    ro, rl = C.run_oracle(w, rope=rope)
    C.assert_parity(w, o, lse, ro, rl, label=f"cascade rope chunk {chunk} {plan.stats}")
    po, _ = C.run_oracle(w)
    assert np.abs(po - ro).max() > 10 * (C.TOL_ABS + C.TOL_REL), "RoPE had no effect"


def _cascade_rope_case(seed):
    rng = np.random.default_rng(7300 + seed)
    ps = int(rng.choice([1, 3, 16]))
    G = int(rng.choice([1, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    D = [64, 128, 256][seed % 3]
    groups, B = [], 0
    for _ in range(int(rng.integers(1, 4))):
        nr = int(rng.integers(1, 5))
        plen = int(rng.choice([1, 2, 5, ps + 1, 40, int(rng.integers(60, 700))]))
        groups.append((nr, plen))
        B += nr
    lens = [int(rng.choice([0, 1, 3, ps + 1, int(rng.integers(2, 400))])) for _ in range(B)]
    q_dtype = str(rng.choice(["f16", "bf16"]))
    kv_dtype = str(rng.choice([q_dtype, "e4m3"]))
    rope = (float(rng.choice([1e4, 5e5])), float(rng.choice([1.0, 8.0, 0.5])))
    w = W.build(f"rope_cascade{seed}", lens, Hq=Hkv * G, Hkv=Hkv, D=D, ps=ps, q_dtype=q_dtype,
                kv_dtype=kv_dtype, seed=seed, prefix_groups=groups)
    return w, rope, groups


@pytest.mark.parametrize("seed", range(12))
def test_cascade_rope_fuzz_parity(fi, seed):
    w, rope, groups = _cascade_rope_case(seed)
    chunk = [0, 32, 48][seed % 3]
    o, lse, plan = C.run_gpu(w, chunk_tokens=chunk, rope=rope)
    ro, rl = C.run_oracle(w, rope=rope)
    C.assert_parity(w, o, lse, ro, rl,
                    label=f"cascade rope fuzz{seed} {rope} D{w.head_dim} G{w.group_size} "
                          f"Hkv{w.num_kv_heads} ps{w.page_size} {w.q_dtype}/{w.kv_dtype} "
                          f"groups {groups} lens {list(w.kv_lens)} {plan.stats}")


def test_cascade_rope_equals_flat_rope(fi):
    """A cascade with RoPE computes what flat RoPE decode of the concatenated
    key lists does (prefix at positions 0.., the own tokens after it)."""
    rope = (1e4, 1.0)
    w = W.make("cascade256", small=True)
    flat = W.flatten_cascade(w)
    o1, l1, _ = C.run_gpu(w, rope=rope)
    o2, l2, _ = C.run_gpu(flat, rope=rope)
    assert np.abs(o1 - o2).max() < C.TOL_ABS and np.abs(l1 - l2).max() < C.TOL_LSE


def _append_rope_run(w, rope, chunk_tokens=0):
    import paged_kv_decode_fi_amd as m
    import torch
    d = C.Dev(w)
    plan = m.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                  num_kv_heads=w.num_kv_heads, page_size=w.page_size, head_dim=w.head_dim,
                  q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, chunk_tokens=chunk_tokens,
                  qo_indptr=w.qo_indptr, causal=w.causal, pos_encoding="rope_llama",
                  rope_theta=rope[0], rope_scale=rope[1])
    o = torch.full((w.num_rows, w.num_qo_heads, w.head_dim), float("nan"), dtype=C.qdtype(w),
                   device="cuda")
    lse = torch.full((w.num_rows, w.num_qo_heads), float("nan"), dtype=torch.float32,
                     device="cuda")
    plan.append_run(d.q, d.k, d.v, d.indptr, d.indices, d.last, d.k_scale, d.v_scale,
                    sm_scale=w.sm_scale, o=o, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy(), plan


def _append_rope_oracle(w, rope):
    import oracle
    return oracle.append(w.q, w.k_pages, w.v_pages, w.qo_indptr, w.kv_indptr, w.kv_indices,
                         w.last_page_len, num_qo_heads=w.num_qo_heads,
                         num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                         page_size=w.page_size, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                         sm_scale=w.sm_scale, causal=w.causal, k_scale=w.k_scale,
                         v_scale=w.v_scale, rope=rope)


@pytest.mark.parametrize("name", W.APPEND_WORKLOADS)
def test_small_append_rope_parity(fi, name):
    rope = (1e4, 1.0)
    w = W.make_append(name, small=True)
    o, lse, plan = _append_rope_run(w, rope)
    ro, rl = _append_rope_oracle(w, rope)
    rows = np.ones((w.num_rows, w.num_qo_heads), bool)
    C.assert_parity(w, o, lse, ro, rl, rows=rows, label=f"{w.name} rope {plan.stats}")


@pytest.mark.parametrize("seed", range(12))
def test_append_rope_fuzz_parity(fi, seed):
    rng = np.random.default_rng(7600 + seed)
    ps = int(rng.choice([1, 3, 16]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    D = [64, 128, 256][seed % 3]
    B = int(rng.integers(1, 6))
    lens = rng.integers(1, 500, size=B)
    kind = rng.integers(0, 4, size=B)
    q_lens = np.where(kind == 0, 1, np.where(kind == 1, lens,
                      np.where(kind == 2, rng.integers(1, lens + 1), 0)))
    q_dtype = str(rng.choice(["f16", "bf16"]))
    kv_dtype = str(rng.choice([q_dtype, "e4m3"]))
    causal = bool(rng.integers(0, 4) != 0)
    rope = (float(rng.choice([1e4, 5e5])), float(rng.choice([1.0, 8.0, 0.5])))
    w = W.build_append(f"append_rope{seed}", lens, q_lens, Hq=Hkv * G, Hkv=Hkv, D=D, ps=ps,
                       q_dtype=q_dtype, kv_dtype=kv_dtype, seed=seed, causal=causal)
    chunk = [0, 32, 96][seed % 3]
    o, lse, plan = _append_rope_run(w, rope, chunk_tokens=chunk)
    ro, rl = _append_rope_oracle(w, rope)
    rows = np.ones((w.num_rows, w.num_qo_heads), bool)
    C.assert_parity(w, o, lse, ro, rl, rows=rows,
                    label=f"append rope fuzz{seed} {rope} causal={causal} D{D} G{G} Hkv{Hkv} "
                          f"ps{ps} {q_dtype}/{kv_dtype} lens {list(lens)} q {list(q_lens)}")


def test_one_token_rope_append_equals_rope_decode(fi):
    """A one-token causal append with RoPE is RoPE decode (the query at the
    last position): the multi-row kernel's absolute turns and the decode
    kernel's relative turns agree within the bar."""
    rope = (1e4, 1.0)
    w = W.make("batch64_gqa4", small=True)
    wa = W.build_append("rope_append_as_decode", w.kv_lens, np.ones(w.batch, np.int64),
                        Hq=32, Hkv=8, ps=16, seed=1001)
    wa.q = w.q.copy()
    wa.k_pages, wa.v_pages = w.k_pages, w.v_pages
    wa.kv_indptr, wa.kv_indices, wa.last_page_len = w.kv_indptr, w.kv_indices, w.last_page_len
    o, lse, _ = _append_rope_run(wa, rope)
    od, ld, _ = C.run_gpu(w, rope=rope)
    ro, rl = C.run_oracle(w, rope=rope)
    C.assert_parity(w, o, lse, ro, rl, label="one-token rope append")
    C.assert_parity(w, od, ld, ro, rl, label="rope decode")


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


def _bf16_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _f32_to_bf16_exact(x):
    """float32 values that are already bf16 values (scaled by powers of two)
    back to their bf16 bits (exact: the low 16 bits are zero)."""
    b = np.asarray(x, np.float32).view(np.uint32)
    assert not np.any(b & 0xFFFF)
    return (b >> 16).astype(np.uint16)


@pytest.mark.parametrize("case", range(6))
def test_rope_single_bf16_q_over_e4m3(fi, case):
    """bf16 q over e4m3 K/V, every request at least 64 keys long: the decode
    kernel computes in fp16 -- q scaled into fp16 by a power of two per kv
    head, the turned key as one fp16 value, o written as bf16 -- and matches
    the oracle, as does the residual form forced on the same problem.
    Case 4 spreads the q heads of every kv head over magnitudes 2^-20 .. 2^3
    (the small ones become fp16 subnormals after the wave's scaling); case 5
    multiplies kv head 0's q by 2^16 and its k_scale by 2^-16 (same scores,
    the power of two taken out of q instead of put in)."""
    rng = np.random.default_rng(1900 + case)
    G = [4, 8, 1, 16, 4, 8][case]
    Hkv = [8, 4, 8, 1, 8, 2][case]
    ps = [16, 1, 16, 7, 16, 1][case]
    D = [128, 128, 64, 128, 256, 128][case]
    lens = rng.integers(64, 3000, size=int(rng.integers(1, 9)))
    w = W.build(f"rope_bf16q_e4m3_{case}", lens, Hq=G * Hkv, Hkv=Hkv, D=D, ps=ps,
                q_dtype="bf16", kv_dtype="e4m3", seed=70 + case)
    if case == 4:
        qf = _bf16_to_f32(w.q).reshape(w.batch, w.num_qo_heads, D)
        e = (np.arange(w.num_qo_heads) * 7) % 24 - 20
        w.q = _f32_to_bf16_exact(qf * np.exp2(e)[None, :, None].astype(np.float32))
    if case == 5:
        qf = _bf16_to_f32(w.q).reshape(w.batch, w.num_qo_heads, D).copy()
        qf[:, :G] *= np.float32(2.0 ** 16)
        w.q = _f32_to_bf16_exact(qf)
        w.k_scale = w.k_scale.copy()
        w.k_scale[0] *= np.float32(2.0 ** -16)
    rope = (float(rng.choice([1e4, 5e5])), 1.0)
    ro, rl = C.run_oracle(w, rope=rope)
    o, lse, plan = C.run_gpu(w, chunk_tokens=[0, 64][case % 2], rope=rope)
    want = int(plan.stats["heads_per_tile"] * 32 >= D)
    assert plan.stats["rope_single"] == want, plan.stats
    C.assert_parity(w, o, lse, ro, rl, label=f"bf16 q / e4m3 rope single {case}")
    o2, lse2, plan2 = C.run_gpu(w, rope=rope, tuning=dict(rope_split_k=1))
    assert plan2.stats["rope_single"] == 0
    C.assert_parity(w, o2, lse2, ro, rl, label=f"bf16 q / e4m3 rope residual {case}")
    # the two forms compute the same function: closer to each other than to the bar
    assert np.abs(o - o2).max() < 1e-2 and np.abs(lse - lse2).max() < 1e-3


def test_rope_residual_kept_where_needed(fi):
    """A request shorter than 64 keys, bf16 q over bf16 K/V, or tiles of fewer than
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
