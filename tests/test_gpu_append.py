"""GPU parity of batch append attention (FlashInfer README append example:
the last n tokens of a request's KV cache are its queries, causal mask) on
the multi-row MFMA kernel, through the C ABI, against the fp64 oracle.

Small sizes compare every output element; the full-size workloads compare
sampled (request, kv head) units and check that every row was written."""
import zlib

import numpy as np
import pytest

import workloads as W
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fi():
    import paged_kv_decode_fi_amd as m
    return m


def _plan(w, chunk_tokens=0, num_cus=0, rope=None):
    import paged_kv_decode_fi_amd as fi
    return fi.Plan(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                   num_kv_heads=w.num_kv_heads, page_size=w.page_size, head_dim=w.head_dim,
                   q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, chunk_tokens=chunk_tokens,
                   num_cus=num_cus, qo_indptr=w.qo_indptr, causal=w.causal,
                   pos_encoding="none" if rope is None else "rope_llama",
                   rope_theta=0.0 if rope is None else rope[0],
                   rope_scale=0.0 if rope is None else rope[1])


def _run(w, plan=None, chunk_tokens=0, num_cus=0, rope=None):
    """Outputs pre-filled with NaN, so an unwritten row shows."""
    import torch
    d = C.Dev(w)
    plan = plan or _plan(w, chunk_tokens, num_cus, rope)
    o = torch.full((w.num_rows, w.num_qo_heads, w.head_dim), float("nan"), dtype=C.qdtype(w),
                   device="cuda")
    lse = torch.full((w.num_rows, w.num_qo_heads), float("nan"), dtype=torch.float32,
                     device="cuda")
    plan.append_run(d.q, d.k, d.v, d.indptr, d.indices, d.last, d.k_scale, d.v_scale,
                    sm_scale=w.sm_scale, o=o, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy(), plan


def _oracle(w, unit_mask=None, rope=None):
    import oracle
    return oracle.append(w.q, w.k_pages, w.v_pages, w.qo_indptr, w.kv_indptr, w.kv_indices,
                         w.last_page_len, num_qo_heads=w.num_qo_heads,
                         num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                         page_size=w.page_size, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                         sm_scale=w.sm_scale, causal=w.causal, k_scale=w.k_scale,
                         v_scale=w.v_scale, unit_mask=unit_mask, rope=rope)


def _compare(w, o, lse, ro, rl, rows=None, label=""):
    if rows is None:
        rows = np.ones((w.num_rows, w.num_qo_heads), bool)
    # the row-major comparison helper takes [rows, heads] masks like decode's
    C.assert_parity(w, o, lse, ro, rl, rows=rows, label=label)


@pytest.mark.parametrize("name", W.APPEND_WORKLOADS)
@pytest.mark.parametrize("chunk", [0, 64])
def test_small_append_parity(fi, name, chunk):
    w = W.make_append(name, small=True)
    o, lse, plan = _run(w, chunk_tokens=chunk)
    ro, rl = _oracle(w)
    _compare(w, o, lse, ro, rl, label=f"{w.name} chunk {chunk} {plan.stats}")
    if chunk:
        assert plan.stats["num_merge_units"] > 0


def _append_fuzz_case(seed):
    rng = np.random.default_rng(9000 + seed)
    ps = int(rng.choice([1, 3, 16]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 6))
    lens = rng.integers(1, 500, size=B)
    kind = rng.integers(0, 4, size=B)
    # one-token appends, whole-request prefills, partial appends, empty
    q_lens = np.where(kind == 0, 1, np.where(kind == 1, lens,
                      np.where(kind == 2, rng.integers(1, lens + 1), 0)))
    q_dtype = str(rng.choice(["f16", "bf16"]))
    kv_dtype = str(rng.choice([q_dtype, "e4m3"]))
    causal = bool(rng.integers(0, 4) != 0)
    return W.build_append(f"append_fuzz{seed}", lens, q_lens, Hq=Hkv * G, Hkv=Hkv, ps=ps,
                          q_dtype=q_dtype, kv_dtype=kv_dtype, seed=seed, causal=causal)


@pytest.mark.parametrize("seed", range(14))
def test_append_fuzz_parity(fi, seed):
    w = _append_fuzz_case(seed)
    chunk = [0, 32, 96][seed % 3]
    o, lse, plan = _run(w, chunk_tokens=chunk, num_cus=[0, 8][seed % 2])
    ro, rl = _oracle(w)
    _compare(w, o, lse, ro, rl,
             label=f"append fuzz{seed} causal={w.causal} G{w.group_size} Hkv{w.num_kv_heads} "
                   f"ps{w.page_size} {w.q_dtype}/{w.kv_dtype} lens {list(w.kv_lens)} "
                   f"q {list(np.diff(w.qo_indptr))} chunk {chunk}")


def test_append_one_token_equals_decode(fi):
    """A one-token causal append of every request is decode: the same rows
    as the decode kernel's, to the acceptance bar on both sides."""
    w = W.make("batch64_gqa4", small=True)
    wa = W.build_append("append_as_decode", w.kv_lens, np.ones(w.batch, np.int64), Hq=32,
                        Hkv=8, ps=16, seed=1001)
    wa.q = w.q.copy()
    wa.k_pages, wa.v_pages = w.k_pages, w.v_pages
    wa.kv_indptr, wa.kv_indices, wa.last_page_len = w.kv_indptr, w.kv_indices, w.last_page_len
    o, lse, _ = _run(wa)
    od, ld, _ = C.run_gpu(w)
    ro, rl = C.run_oracle(w)
    C.assert_parity(w, o, lse, ro, rl, label="one-token append")
    C.assert_parity(w, od, ld, ro, rl, label="decode")


def test_append_planted_key_under_the_mask(fi):
    """A key that would dominate every row is planted just after query 0's
    position: rows that may see it return its value, row 0 may not."""
    w = W.build_append("append_planted", [200], [20], Hq=4, Hkv=1, ps=16, seed=77)
    q = w.q.view(np.float16).astype(np.float32)
    L, n = 200, 20
    t_star = L - n + 1                       # visible to queries 1.. only
    page = int(w.kv_indices[t_star // 16])
    w.q[:] = w.q[0, 0]                        # every row the same query
    w.k_pages[page, t_star % 16, 0] = (q[0, 0] * 6.0).astype(np.float16).view(np.uint16)
    o, lse, _ = _run(w)
    ro, rl = _oracle(w)
    _compare(w, o, lse, ro, rl, label="planted")
    v_star = w.v_pages[page, t_star % 16, 0].view(np.float16).astype(np.float64)
    assert np.abs(o[1:] - v_star).max() < 2e-2
    assert np.abs(o[0] - v_star).max() > 0.1


@pytest.mark.parametrize("head_dim", [128, 64, 256])
@pytest.mark.parametrize("name", W.APPEND_WORKLOADS)
def test_full_size_append_sampled_parity(fi, name, head_dim, rope=None):
    w = W.make_append(name, head_dim=head_dim)
    o, lse, plan = _run(w, rope=rope)
    st = plan.stats
    print(f"{w.name}: tiles {st['num_prefix_tiles']} merge units {st['num_merge_units']} "
          f"chunk {st['prefix_chunk_tokens']}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "a row was not written"
    B, H = w.batch, w.num_kv_heads
    mask = np.zeros((B, H), np.uint8)
    lens = w.kv_lens
    for r in {0, B - 1, int(np.argmax(lens)), int(np.argmin(lens))}:
        mask[r, :] = 1
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    flat = mask.reshape(-1)
    free = np.flatnonzero(flat == 0)
    if free.size:
        flat[rng.choice(free, size=min(8, free.size), replace=False)] = 1
    ro, rl = _oracle(w, unit_mask=flat, rope=rope)
    G = w.group_size
    rows = np.zeros((w.num_rows, w.num_qo_heads), bool)
    for r in range(B):
        for h in range(H):
            if mask[r, h]:
                rows[w.qo_indptr[r]:w.qo_indptr[r + 1], h * G:(h + 1) * G] = True
    _compare(w, o, lse, ro, rl, rows=rows, label=f"{w.name} full size, sampled units")
    plan.destroy()


@pytest.mark.parametrize("name", W.APPEND_WORKLOADS)
def test_full_size_append_rope_sampled_parity(fi, name):
    """The append workloads at full size with LLaMA-style RoPE (query token i
    of n at L - n + i), in the benchmark's launch configuration."""
    test_full_size_append_sampled_parity(fi, name, 128, rope=(1e4, 1.0))
