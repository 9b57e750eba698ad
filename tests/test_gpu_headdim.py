"""GPU parity at head_dim 64 and 256 (FlashInfer README, basic usage: head_dim
is a parameter of the decode call, 128 in its example; q is [num_qo_heads,
head_dim], k and v [kv_len, num_kv_heads, head_dim]).

Both run every path the library builds for 128: plain and chunked decode,
RoPE decode (a table row of head_dim / 2 frequencies), a cascade level with
fold and merge, several levels, append (at 256 the multi-row kernel has one
16-row column tile per wave).  Every case is compared element by element
with the fp64 oracle, which takes head_dim as a parameter."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu

DTYPES = [("f16", "f16"), ("bf16", "bf16"), ("f16", "e4m3"), ("bf16", "e4m3")]


@pytest.fixture(scope="module")
def fi():
    import paged_kv_decode_fi_amd as m
    return m


def _lens(rng, B, hi):
    return [int(rng.choice([0, 1, 15, 16, 17, int(rng.integers(2, hi))])) for _ in range(B)]


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("dt", DTYPES, ids=lambda t: f"{t[0]}-{t[1]}")
@pytest.mark.parametrize("chunk", [0, 32])
def test_decode_parity(fi, D, dt, chunk):
    rng = np.random.default_rng(D * 10 + DTYPES.index(dt))
    lens = [700, 1, 33, 0, 250, 16] + list(rng.integers(1, 400, size=3))
    w = W.build(f"d{D}", lens, Hq=32, Hkv=8, D=D, ps=16, q_dtype=dt[0], kv_dtype=dt[1],
                seed=D + DTYPES.index(dt))
    o, lse, plan = C.run_gpu(w, chunk_tokens=chunk)
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl, label=f"D{D} {dt} chunk {chunk} {plan.stats}")
    if chunk:
        assert plan.stats["num_merge_units"] > 0


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("dt", DTYPES, ids=lambda t: f"{t[0]}-{t[1]}")
@pytest.mark.parametrize("chunk", [0, 32])
def test_rope_decode_parity(fi, D, dt, chunk):
    rng = np.random.default_rng(3 * D + DTYPES.index(dt))
    lens = [900, 1, 33, 0, 250, 16] + list(rng.integers(1, 400, size=3))
    w = W.build(f"r{D}", lens, Hq=32, Hkv=8, D=D, ps=16, q_dtype=dt[0], kv_dtype=dt[1],
                seed=7 * D + DTYPES.index(dt))
    rope = (1e4, 1.0)
    o, lse, plan = C.run_gpu(w, chunk_tokens=chunk, rope=rope)
    ro, rl = C.run_oracle(w, rope=rope)
    C.assert_parity(w, o, lse, ro, rl, label=f"RoPE D{D} {dt} chunk {chunk} {plan.stats}")
    po, _ = C.run_oracle(w)
    assert np.abs(po - ro).max() > 10 * (C.TOL_ABS + C.TOL_REL), "RoPE had no effect"


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("seed", range(6))
def test_rope_fuzz_parity(fi, D, seed):
    rng = np.random.default_rng(17000 + 5 * D + seed)
    G = int(rng.choice([1, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 7))
    ps = int(rng.choice([1, 3, 16]))
    q_dtype, kv_dtype = DTYPES[seed % 4]
    rope = (float(rng.choice([1e4, 5e5])), float(rng.choice([1.0, 8.0, 0.5])))
    w = W.build(f"rfz{D}_{seed}", _lens(rng, B, 900), Hq=Hkv * G, Hkv=Hkv, D=D, ps=ps,
                q_dtype=q_dtype, kv_dtype=kv_dtype, seed=seed)
    if seed % 3 == 1:
        w = W.to_hnd(w)
    elif seed % 3 == 2:
        w = W.to_ragged(w)
    chunk = [0, 32][seed % 2]
    o, lse, plan = C.run_gpu(w, chunk_tokens=chunk, rope=rope)
    ro, rl = C.run_oracle(w, rope=rope)
    C.assert_parity(w, o, lse, ro, rl,
                    label=f"RoPE D{D} fuzz{seed} G{G} Hkv{Hkv} ps{ps} {q_dtype}/{kv_dtype} "
                          f"rope {rope} lens {list(w.kv_lens)} chunk {chunk}")


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("kind", ["many_states", "many_units"])
def test_merge_paths(fi, D, kind):
    """The one-wave merge past 64 states (a 2600-token request in 32-token
    chunks: 82 states, two rounds of lse reads) and the workgroup merge
    (160 requests of 4 chunks each: >= 128 units with <= 8 states)."""
    if kind == "many_states":
        lens = [2600, 5, 300]
    else:
        lens = list(np.random.default_rng(D).integers(97, 129, size=160))
    w = W.build(f"m{D}{kind}", lens, Hq=16, Hkv=4, D=D, ps=16, q_dtype="bf16", kv_dtype="bf16",
                seed=D + len(kind))
    o, lse, plan = C.run_gpu(w, chunk_tokens=32)
    ro, rl = C.run_oracle(w)
    st = plan.stats
    C.assert_parity(w, o, lse, ro, rl, label=f"D{D} {kind} {st}")
    assert st["num_merge_units"] == (2 if kind == "many_states" else 160)


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("seed", range(6))
def test_decode_fuzz_parity(fi, D, seed):
    """Group sizes 1..16, 1..8 kv heads, page sizes 1, 3 (not a power of
    two) and 16, every dtype pair, NHD / HND / ragged layouts."""
    rng = np.random.default_rng(13000 + 7 * D + seed)
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 7))
    q_dtype, kv_dtype = DTYPES[seed % 4]
    ps = int(rng.choice([1, 3, 16]))
    w = W.build(f"fz{D}_{seed}", _lens(rng, B, 900), Hq=Hkv * G, Hkv=Hkv, D=D, ps=ps,
                q_dtype=q_dtype, kv_dtype=kv_dtype, seed=seed)
    layout = ["paged", "hnd", "ragged"][seed % 3]
    if layout == "hnd":
        w = W.to_hnd(w)
    elif layout == "ragged":
        w = W.to_ragged(w)
    chunk = [0, 32, 64][(seed // 3) % 3]
    o, lse, plan = C.run_gpu(w, chunk_tokens=chunk)
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl,
                    label=f"D{D} fuzz{seed} G{G} Hkv{Hkv} ps{ps} {q_dtype}/{kv_dtype} "
                          f"{layout} lens {list(w.kv_lens)} chunk {chunk}")


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("dt", DTYPES, ids=lambda t: f"{t[0]}-{t[1]}")
def test_cascade_parity(fi, D, dt):
    """One shared-prefix level: the default plan folds the prefix states
    into the suffix tiles; chunk 32 merges them instead."""
    rng = np.random.default_rng(500 + DTYPES.index(dt))
    lens = list(rng.integers(1, 120, size=8))
    w = W.build(f"casc{D}", lens, Hq=32, Hkv=8, D=D, ps=16, q_dtype=dt[0], kv_dtype=dt[1],
                seed=3, prefix_len=300)
    ro, rl = C.run_oracle(w)
    for chunk in (0, 32):
        o, lse, plan = C.run_gpu(w, chunk_tokens=chunk)
        C.assert_parity(w, o, lse, ro, rl, label=f"cascade D{D} {dt} chunk {chunk} {plan.stats}")


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("chunk", [0, 32])
def test_cascade_levels_parity(fi, D, chunk):
    import oracle
    import torch
    w = W.build_multilevel(f"lv{D}", [9, 0, 130, 1, 64, 300], [[(6, 100)], [(3, 0), (3, 77)]],
                           Hq=16, Hkv=2, D=D, ps=16, q_dtype="bf16", kv_dtype="bf16", seed=5)
    lv = w.meta["levels"]
    d = C.Dev(w)
    plan = fi.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                   num_kv_heads=w.num_kv_heads, page_size=w.page_size, head_dim=D,
                   q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, chunk_tokens=chunk,
                   levels=[(qo, ip, la) for (qo, ip, ix, la, _) in lv])
    tabs = [(C.to_dev(ip), C.to_dev(ix), C.to_dev(la)) for (qo, ip, ix, la, _) in lv]
    o, lse = plan.cascade_run_levels(d.q, d.k, d.v, tabs, d.indptr, d.indices, d.last,
                                     sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.cascade_levels(w.q, w.k_pages, w.v_pages,
                                   [(qo, ip, ix, la) for (qo, ip, ix, la, _) in lv],
                                   w.kv_indptr, w.kv_indices, w.last_page_len,
                                   num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                                   head_dim=D, page_size=w.page_size, q_dtype=w.q_dtype,
                                   kv_dtype=w.kv_dtype, sm_scale=w.sm_scale)
    C.assert_parity(w, o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl,
                    label=f"two levels D{D} chunk {chunk} {plan.stats}")


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("dt", DTYPES, ids=lambda t: f"{t[0]}-{t[1]}")
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("chunk", [0, 64])
def test_append_parity(fi, D, dt, causal, chunk):
    import oracle
    import torch
    rng = np.random.default_rng(900 + DTYPES.index(dt) + 10 * causal)
    lens = rng.integers(1, 400, size=4)
    q_lens = np.minimum(lens, [1, 60, 200, int(lens[3])])
    w = W.build_append(f"app{D}", lens, q_lens, Hq=16, Hkv=4, D=D, ps=16, q_dtype=dt[0],
                       kv_dtype=dt[1], seed=9, causal=causal)
    d = C.Dev(w)
    plan = fi.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                   num_kv_heads=w.num_kv_heads, page_size=w.page_size, head_dim=D,
                   q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, qo_indptr=w.qo_indptr,
                   causal=w.causal, chunk_tokens=chunk)
    o, lse = plan.append_run(d.q, d.k, d.v, d.indptr, d.indices, d.last, d.k_scale, d.v_scale,
                             sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.append(w.q, w.k_pages, w.v_pages, w.qo_indptr, w.kv_indptr, w.kv_indices,
                           w.last_page_len, num_qo_heads=w.num_qo_heads,
                           num_kv_heads=w.num_kv_heads, head_dim=D, page_size=w.page_size,
                           q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, sm_scale=w.sm_scale,
                           causal=w.causal, k_scale=w.k_scale, v_scale=w.v_scale)
    C.assert_parity(w, o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl,
                    rows=np.ones((w.num_rows, w.num_qo_heads), bool),
                    label=f"append D{D} {dt} causal {causal} chunk {chunk} {plan.stats}")


@pytest.mark.parametrize("D", [64, 256])
def test_batch64_shape_sampled_parity(fi, D):
    """The batch64_gqa4 shape (64 requests, kv_len U{512..4096}, 32/8 heads,
    fp16, page size 16) at head_dim D, in the default plan: sampled (request,
    kv head) units against the oracle, every row written."""
    rng = np.random.default_rng(1001)
    lens = rng.integers(512, 4097, size=64)
    w = W.build(f"batch64_gqa4_d{D}", lens, Hq=32, Hkv=8, D=D, ps=16, seed=1001)
    o, lse, plan = C.run_gpu(w)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "a row was not written"
    mask = np.zeros((w.batch, w.num_kv_heads), np.uint8)
    mask[[0, 63, int(np.argmax(lens)), int(np.argmin(lens))], :] = 1
    mask.reshape(-1)[rng.choice(np.flatnonzero(mask.reshape(-1) == 0), 8, replace=False)] = 1
    ro, rl = C.run_oracle(w, unit_mask=mask.reshape(-1))
    C.assert_parity(w, o, lse, ro, rl, rows=C.rows_of_units(w, mask.reshape(-1)),
                    label=f"batch64 shape D{D} {plan.stats}")
