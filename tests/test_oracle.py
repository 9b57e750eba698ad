"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

Each test pins the oracle to something other than itself: format
definitions, closed forms, an independent dense brute force, invariants of
the definition of attention (page permutation, page size, split + merge),
and planted structure (GQA head map, a dominant key, NaN-poisoned tails).
"""
import json
import math
import os

import numpy as np
import pytest

from tests.helpers import f16_values, paginate, to_f16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- decoders

def test_f16_decoder_all_codes(oracle_lib):
    codes = np.arange(65536, dtype=np.uint32)
    ref = codes.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.decode_scalar(int(c), "f16") for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_bf16_decoder_all_codes(oracle_lib):
    import torch
    codes = np.arange(65536, dtype=np.int32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle_lib.decode_scalar(int(c), "bf16") for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_e4m3_decoder_all_codes(oracle_lib):
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle_lib.decode_scalar(int(c), "e4m3") for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_e4m3_spec_points(oracle_lib):
    pts = json.load(open(os.path.join(GOLDEN, "e4m3_points.json")))["points"]
    for p in pts:
        v = oracle_lib.decode_scalar(p["code"], "e4m3")
        if p["value"] == "nan":
            assert math.isnan(v), p
        else:
            assert v == p["value"] and math.copysign(1, v) == math.copysign(1, p["value"]), p


# ------------------------------------------------------ closed-form cases

def _run_dense_as_paged(oracle_lib, q, k, v, sm_scale, ps=1, seed=0):
    """q [Hq, D], k/v [L, Hkv, D] float values exactly representable in fp16."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Hq, D = q.shape
    Hkv = k.shape[1]
    rng = np.random.default_rng(seed)
    kp, indptr, idx, last = paginate([to_f16_bits(k)], ps, Hkv, D, rng)
    vp, _, _, _ = paginate([to_f16_bits(v)], ps, Hkv, D, np.random.default_rng(seed))
    return oracle_lib.decode(to_f16_bits(q)[None], kp, vp, indptr, idx, last,
                             num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                             page_size=ps, q_dtype="f16", kv_dtype="f16",
                             sm_scale=sm_scale)


@pytest.mark.parametrize("ps", [1, 2, 16])
def test_hand_cases(oracle_lib, ps):
    cases = json.load(open(os.path.join(GOLDEN, "hand_cases.json")))["cases"]
    for c in cases:
        o, lse = _run_dense_as_paged(oracle_lib, c["q"], c["k"], c["v"], c["sm_scale"], ps=ps)
        np.testing.assert_allclose(o[0], np.array(c["o"]), rtol=1e-14, atol=1e-14,
                                   err_msg=c["name"])
        np.testing.assert_allclose(lse[0], np.array(c["lse"]), rtol=1e-14, atol=1e-14,
                                   err_msg=c["name"])


def test_zero_query_gives_mean_and_log_len(oracle_lib):
    rng = np.random.default_rng(3)
    L, Hkv, D = 37, 2, 8
    k = f16_values(rng.standard_normal((L, Hkv, D)))
    v = f16_values(rng.standard_normal((L, Hkv, D)))
    q = np.zeros((4, D))
    o, lse = _run_dense_as_paged(oracle_lib, q, k, v, 0.3, ps=4)
    for j in range(4):
        np.testing.assert_allclose(o[0, j], v[:, j // 2, :].mean(0), rtol=1e-13, atol=1e-15)
        assert abs(lse[0, j] - math.log(L)) < 1e-14


def test_identical_keys_give_mean_and_shifted_lse(oracle_lib):
    rng = np.random.default_rng(4)
    L, D = 20, 8
    krow = f16_values(rng.standard_normal(D))
    k = np.tile(krow, (L, 1, 1))
    v = f16_values(rng.standard_normal((L, 1, D)))
    q = f16_values(rng.standard_normal((1, D)))
    o, lse = _run_dense_as_paged(oracle_lib, q, k, v, 0.25, ps=16)
    x = 0.25 * float(np.dot(q[0], krow))
    np.testing.assert_allclose(o[0, 0], v[:, 0].mean(0), rtol=1e-13, atol=1e-15)
    assert abs(lse[0, 0] - (x + math.log(L))) < 1e-13


def test_empty_request(oracle_lib):
    rng = np.random.default_rng(5)
    D, Hkv = 8, 1
    dense = [to_f16_bits(rng.standard_normal((5, Hkv, D))), np.zeros((0, Hkv, D), np.uint16)]
    kp, indptr, idx, last = paginate(dense, 4, Hkv, D, rng)
    q = to_f16_bits(rng.standard_normal((2, 2, D)))
    o, lse = oracle_lib.decode(q, kp, kp, indptr, idx, last, num_qo_heads=2,
                               num_kv_heads=1, head_dim=D, page_size=4,
                               q_dtype="f16", kv_dtype="f16", sm_scale=0.5)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(o[0])) and np.all(np.isfinite(lse[0]))


# ------------------------------------------------- dense brute force pin

def _random_problem(rng, B, Hq, Hkv, D, lens, ps, scale=0.1):
    qf = rng.standard_normal((B, Hq, D)) * scale
    ks = [rng.standard_normal((L, Hkv, D)) for L in lens]
    vs = [rng.standard_normal((L, Hkv, D)) for L in lens]
    return qf, ks, vs


@pytest.mark.parametrize("ps", [1, 3, 16])
def test_matches_dense_brute_force(oracle_lib, ps):
    from oracle.dense import ref_dense
    rng = np.random.default_rng(10 + ps)
    B, Hq, Hkv, D = 4, 8, 2, 16
    lens = [1, 13, 0, 40]
    qf, ks, vs = _random_problem(rng, B, Hq, Hkv, D, lens, ps)
    kb = [to_f16_bits(k) for k in ks]
    vb = [to_f16_bits(v) for v in vs]
    kp, indptr, idx, last = paginate(kb, ps, Hkv, D, np.random.default_rng(1))
    vp, _, _, _ = paginate(vb, ps, Hkv, D, np.random.default_rng(1))
    sm = 0.37
    o, lse = oracle_lib.decode(to_f16_bits(qf), kp, vp, indptr, idx, last,
                               num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                               page_size=ps, q_dtype="f16", kv_dtype="f16",
                               sm_scale=sm)
    for r in range(B):
        ro, rl = ref_dense(f16_values(qf[r]), f16_values(ks[r]), f16_values(vs[r]), sm)
        np.testing.assert_allclose(o[r], ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[r], rl, rtol=1e-12, atol=1e-13)


def test_bf16_and_e4m3_match_dense(oracle_lib):
    """Same brute force with bf16 q / e4m3 K,V and per-head scales."""
    import torch
    from oracle.dense import bf16_bits_to_f64, ref_dense
    rng = np.random.default_rng(21)
    Hq, Hkv, D, L, ps = 4, 2, 32, 29, 4
    qf = rng.standard_normal((1, Hq, D)).astype(np.float32) * 0.2
    qb = torch.from_numpy(qf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kf = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    vf = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    ksc = np.array([0.01, 0.02], np.float32)
    vsc = np.array([0.5, 0.125], np.float32)
    kc = torch.from_numpy(kf / ksc[None, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn)
    vc = torch.from_numpy(vf / vsc[None, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn)
    kp, indptr, idx, last = paginate([kc.view(torch.uint8).numpy()], ps, Hkv, D,
                                     np.random.default_rng(2), fill_bits=0x7F, dtype=np.uint8)
    vp, _, _, _ = paginate([vc.view(torch.uint8).numpy()], ps, Hkv, D,
                           np.random.default_rng(2), fill_bits=0x7F, dtype=np.uint8)
    o, lse = oracle_lib.decode(qb, kp, vp, indptr, idx, last, num_qo_heads=Hq,
                               num_kv_heads=Hkv, head_dim=D, page_size=ps,
                               q_dtype="bf16", kv_dtype="e4m3", sm_scale=0.125,
                               k_scale=ksc, v_scale=vsc)
    kd = kc.double().numpy() * ksc.astype(np.float64)[None, :, None]
    vd = vc.double().numpy() * vsc.astype(np.float64)[None, :, None]
    ro, rl = ref_dense(bf16_bits_to_f64(qb[0]), kd, vd, 0.125)
    np.testing.assert_allclose(o[0], ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0], rl, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- invariants

def test_page_permutation_and_page_size_invariance(oracle_lib):
    """The oracle sums in logical token order, so the physical layout cannot
    change a single bit of the result."""
    rng = np.random.default_rng(7)
    Hq, Hkv, D = 8, 4, 32
    lens = [50, 1, 17]
    qf, ks, vs = _random_problem(rng, 3, Hq, Hkv, D, lens, 1, scale=1.0)
    kb = [to_f16_bits(k) for k in ks]
    vb = [to_f16_bits(v) for v in vs]
    outs = []
    for ps, seed in [(1, 0), (16, 0), (16, 99), (5, 3)]:
        kp, indptr, idx, last = paginate(kb, ps, Hkv, D, np.random.default_rng(seed))
        vp, _, _, _ = paginate(vb, ps, Hkv, D, np.random.default_rng(seed))
        outs.append(oracle_lib.decode(to_f16_bits(qf), kp, vp, indptr, idx, last,
                                      num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                      page_size=ps, q_dtype="f16", kv_dtype="f16",
                                      sm_scale=0.2))
    for o, lse in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(lse, outs[0][1])


def test_gqa_head_map(oracle_lib):
    """V of kv head h is the constant h: q head j must return (j // G)."""
    rng = np.random.default_rng(8)
    Hq, Hkv, D, L = 16, 4, 8, 9
    k = to_f16_bits(rng.standard_normal((L, Hkv, D)))
    v = to_f16_bits(np.broadcast_to(np.arange(Hkv, dtype=np.float64)[None, :, None], (L, Hkv, D)))
    kp, indptr, idx, last = paginate([k], 4, Hkv, D, np.random.default_rng(11))
    vp, _, _, _ = paginate([v], 4, Hkv, D, np.random.default_rng(11))
    q = to_f16_bits(rng.standard_normal((1, Hq, D)))
    o, _ = oracle_lib.decode(q, kp, vp, indptr, idx, last, num_qo_heads=Hq,
                             num_kv_heads=Hkv, head_dim=D, page_size=4,
                             q_dtype="f16", kv_dtype="f16", sm_scale=0.3)
    for j in range(Hq):
        np.testing.assert_allclose(o[0, j], j // (Hq // Hkv), rtol=1e-14)


def test_dominant_key_returns_its_value(oracle_lib):
    rng = np.random.default_rng(9)
    Hkv, D, L, t_star = 1, 16, 333, 217
    k = rng.standard_normal((L, Hkv, D)) * 0.01
    q = np.zeros((1, D))
    q[0, 3] = 8.0
    k[t_star, 0, 3] = 8.0          # score 64*sm vs |others| < 1
    v = rng.standard_normal((L, Hkv, D))
    o, lse = _run_dense_as_paged(oracle_lib, q, f16_values(k), f16_values(v), 1.0, ps=16)
    np.testing.assert_allclose(o[0, 0], f16_values(v)[t_star, 0], atol=1e-20)


def test_nan_poisoned_tails_never_read(oracle_lib):
    """Pool pages and tail slots hold NaN; a correct walk stays finite."""
    rng = np.random.default_rng(12)
    Hq, Hkv, D = 4, 2, 16
    lens = [17, 33, 1, 16]
    qf, ks, vs = _random_problem(rng, 4, Hq, Hkv, D, lens, 16)
    kp, indptr, idx, last = paginate([to_f16_bits(k) for k in ks], 16, Hkv, D,
                                     np.random.default_rng(5), pool_extra=10)
    vp, _, _, _ = paginate([to_f16_bits(v) for v in vs], 16, Hkv, D,
                           np.random.default_rng(5), pool_extra=10)
    assert np.isnan(kp.view(np.float16)).any()
    o, lse = oracle_lib.decode(to_f16_bits(qf), kp, vp, indptr, idx, last,
                               num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                               page_size=16, q_dtype="f16", kv_dtype="f16",
                               sm_scale=0.1)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


def test_scales_are_exact_factors(oracle_lib):
    """k_scale = 2 equals sm_scale x 2 bit for bit; v_scale = 2 doubles o."""
    rng = np.random.default_rng(13)
    Hq, Hkv, D, L = 4, 2, 16, 30
    qf, ks, vs = _random_problem(rng, 1, Hq, Hkv, D, [L], 1, scale=1.0)
    import torch
    kc = torch.from_numpy(ks[0].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    vc = torch.from_numpy(vs[0].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    kp, indptr, idx, last = paginate([kc], 4, Hkv, D, np.random.default_rng(3), fill_bits=0x7F, dtype=np.uint8)
    vp, _, _, _ = paginate([vc], 4, Hkv, D, np.random.default_rng(3), fill_bits=0x7F, dtype=np.uint8)
    common = dict(num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=4,
                  q_dtype="f16", kv_dtype="e4m3")
    one = np.ones(Hkv, np.float32)
    two = np.full(Hkv, 2.0, np.float32)
    qb = to_f16_bits(qf)
    o1, l1 = oracle_lib.decode(qb, kp, vp, indptr, idx, last, sm_scale=0.5,
                               k_scale=two, v_scale=one, **common)
    o2, l2 = oracle_lib.decode(qb, kp, vp, indptr, idx, last, sm_scale=1.0,
                               k_scale=one, v_scale=one, **common)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = oracle_lib.decode(qb, kp, vp, indptr, idx, last, sm_scale=1.0,
                               k_scale=one, v_scale=two, **common)
    assert np.array_equal(o3, 2 * o2) and np.array_equal(l3, l2)


# ------------------------------------------------------------------ merge

def test_split_then_merge_equals_unsplit(oracle_lib):
    """Attention over A ++ B equals the merge of the states over A and B."""
    rng = np.random.default_rng(14)
    Hq, Hkv, D, L = 8, 2, 16, 101
    qf, ks, vs = _random_problem(rng, 1, Hq, Hkv, D, [L], 1, scale=1.0)
    kb, vb = to_f16_bits(ks[0]), to_f16_bits(vs[0])
    qb = to_f16_bits(qf)
    common = dict(num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=1,
                  q_dtype="f16", kv_dtype="f16", sm_scale=0.3)

    def run(lo, hi):
        kp, ip, ix, la = paginate([kb[lo:hi]], 1, Hkv, D, np.random.default_rng(0))
        vp, _, _, _ = paginate([vb[lo:hi]], 1, Hkv, D, np.random.default_rng(0))
        return oracle_lib.decode(qb, kp, vp, ip, ix, la, **common)

    full_o, full_l = run(0, L)
    cuts = [0, 10, 11, 64, L]
    parts = [run(a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    os_ = np.stack([p[0][0] for p in parts])
    ls_ = np.stack([p[1][0] for p in parts])
    mo, ml = oracle_lib.merge(os_, ls_)
    np.testing.assert_allclose(mo, full_o[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ml, full_l[0], rtol=1e-13, atol=1e-14)


def test_merge_identities(oracle_lib):
    rng = np.random.default_rng(15)
    o = rng.standard_normal((1, 5, 8))
    lse = rng.standard_normal((1, 5))
    # with an empty state (o = 0, lse = -inf): identity
    o2 = np.concatenate([o, np.zeros_like(o)])
    l2 = np.concatenate([lse, np.full_like(lse, -np.inf)])
    mo, ml = oracle_lib.merge(o2, l2)
    np.testing.assert_array_equal(mo, o[0])
    np.testing.assert_array_equal(ml, lse[0])
    # two equal states: o unchanged, lse + ln 2
    mo, ml = oracle_lib.merge(np.concatenate([o, o]), np.concatenate([lse, lse]))
    np.testing.assert_allclose(mo, o[0], rtol=1e-15)
    np.testing.assert_allclose(ml, lse[0] + math.log(2), rtol=1e-15)
    # all empty: o = 0, lse = -inf
    mo, ml = oracle_lib.merge(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(mo == 0) and np.all(np.isneginf(ml))
    # order independence within rounding
    a = rng.standard_normal((4, 3, 8))
    al = rng.standard_normal((4, 3)) * 5
    m1 = oracle_lib.merge(a, al)
    m2 = oracle_lib.merge(a[::-1], al[::-1])
    np.testing.assert_allclose(m1[0], m2[0], rtol=1e-13)
    np.testing.assert_allclose(m1[1], m2[1], rtol=1e-14)


# ---------------------------------------------------------------- cascade

def test_cascade_equals_flat_concatenation(oracle_lib):
    rng = np.random.default_rng(16)
    Hq, Hkv, D, ps = 8, 2, 16, 4
    groups = [(2, 9), (3, 0), (1, 20)]      # (n requests, prefix length)
    B = sum(g[0] for g in groups)
    suf = [5, 0, 7, 1, 12, 3]
    pre_dense = [to_f16_bits(rng.standard_normal((L, Hkv, D))) for _, L in groups]
    pre_vd = [to_f16_bits(rng.standard_normal((L, Hkv, D))) for _, L in groups]
    suf_k = [to_f16_bits(rng.standard_normal((L, Hkv, D))) for L in suf]
    suf_v = [to_f16_bits(rng.standard_normal((L, Hkv, D))) for L in suf]
    # one pool holding prefixes then suffixes
    kp, ip, ix, la = paginate(pre_dense + suf_k, ps, Hkv, D, np.random.default_rng(4))
    vp, _, _, _ = paginate(pre_vd + suf_v, ps, Hkv, D, np.random.default_rng(4))
    G = len(groups)
    p_indptr = ip[:G + 1].copy()
    p_indices = ix[:p_indptr[-1]]
    p_last = la[:G]
    s_indptr = (ip[G:] - ip[G]).astype(np.int32)
    s_indices = ix[ip[G]:]
    s_last = la[G:]
    qo = np.concatenate([[0], np.cumsum([g[0] for g in groups])]).astype(np.int32)
    q = to_f16_bits(rng.standard_normal((B, Hq, D)) * 0.5)
    common = dict(num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                  q_dtype="f16", kv_dtype="f16", sm_scale=0.25)
    co, cl = oracle_lib.cascade(q, kp, vp, qo, p_indptr, p_indices, p_last,
                                s_indptr, s_indices, s_last, **common)
    # flat: each request's table = its group's prefix pages ++ its own pages,
    # laid out with page size 1 so the concatenation is exact token by token
    r = 0
    for g, (n, _) in enumerate(groups):
        for _ in range(n):
            kd = np.concatenate([pre_dense[g], suf_k[r]])
            vd = np.concatenate([pre_vd[g], suf_v[r]])
            kp1, ip1, ix1, la1 = paginate([kd], 1, Hkv, D, np.random.default_rng(r))
            vp1, _, _, _ = paginate([vd], 1, Hkv, D, np.random.default_rng(r))
            fo, fl = oracle_lib.decode(q[r:r + 1], kp1, vp1, ip1, ix1, la1,
                                       **{**common, "page_size": 1})
            assert np.array_equal(fo[0], co[r]) and np.array_equal(fl[0], cl[r])
            r += 1


def test_gather_map_matches_brute_force(oracle_lib):
    rng = np.random.default_rng(17)
    for ps in (1, 4, 16):
        lens = rng.integers(0, 50, size=7)
        n = (lens + ps - 1) // ps
        indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        indices = rng.permutation(int(n.sum()) + 5)[:int(n.sum())].astype(np.int32)
        last = np.where(n > 0, lens - (n - 1) * ps, 0).astype(np.int32)
        got = oracle_lib.gather_map(ps, indptr, indices, last)
        want = []
        for r in range(len(lens)):
            pages = indices[indptr[r]:indptr[r + 1]]
            for p_i, p in enumerate(pages):
                cnt = ps if p_i < len(pages) - 1 else last[r]
                want.extend(int(p) * ps + s for s in range(cnt))
        assert np.array_equal(got, np.array(want, np.int64))


# ------------------------------------------------------------- RoPE pins
# The pages name LLaMA-style RoPE on-the-fly but give no formula; the
# oracle's reading (rotate-half, angle_i = pos / scale * theta^(-2i/D)) is
# pinned here by identities and by a complex-number restatement written
# independently of the oracle's real-valued rotation.

def _rope_complex(x, pos, theta=1e4, scale=1.0):
    """Rotate-half RoPE as a complex multiplication: the pair (x_i, x_{i+D/2})
    is the complex number x_i + i x_{i+D/2}, turned by e^{i angle_i}."""
    x = np.asarray(x, np.float64)
    h = len(x) // 2
    ang = (pos / scale) * theta ** (-2.0 * np.arange(h) / len(x))
    z = (x[:h] + 1j * x[h:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag])


@pytest.mark.parametrize("D", [64, 128, 256])
def test_rope_rotation_pins(oracle_lib, D):
    rng = np.random.default_rng(31)
    x = rng.standard_normal(D)
    y = rng.standard_normal(D)
    # position 0 is the identity
    assert np.array_equal(oracle_lib.rope_rotate(x, 0), x)
    for pos, theta, scale in [(1, 1e4, 1.0), (37, 1e4, 1.0), (4095, 5e5, 1.0),
                              (32767, 1e4, 1.0), (1000, 1e4, 4.0)]:
        r = oracle_lib.rope_rotate(x, pos, theta, scale)
        # the angle reaches pos radians: one ulp of it is ~pos * 1.1e-16
        np.testing.assert_allclose(r, _rope_complex(x, pos, theta, scale), rtol=0,
                                   atol=1e-13 + 4e-16 * pos * np.abs(x).max())
        assert abs(np.linalg.norm(r) - np.linalg.norm(x)) < 1e-12   # a rotation
    # the scale divides the position
    np.testing.assert_allclose(oracle_lib.rope_rotate(x, 1000, 1e4, 4.0),
                               oracle_lib.rope_rotate(x, 250, 1e4, 1.0), rtol=0, atol=1e-13)
    # scores depend only on the position difference
    for p1, p2, c in [(5, 9, 100), (4000, 17, 3), (0, 2047, 2048)]:
        a = np.dot(oracle_lib.rope_rotate(x, p1), oracle_lib.rope_rotate(y, p2))
        b = np.dot(oracle_lib.rope_rotate(x, p1 + c), oracle_lib.rope_rotate(y, p2 + c))
        assert abs(a - b) < 1e-11
    # a planted sign or pairing mistake does not pass the complex restatement
    wrong = x.copy()
    h = D // 2
    ang = 37 * 1e4 ** (-2.0 * np.arange(h) / D)
    wrong[:h] = x[:h] * np.cos(ang) + x[h:] * np.sin(ang)
    wrong[h:] = x[h:] * np.cos(ang) - x[:h] * np.sin(ang)
    assert np.abs(wrong - _rope_complex(x, 37)).max() > 1e-3


@pytest.mark.parametrize("D", [64, 128, 256])
def test_rope_decode_equals_plain_decode_of_prerotated_data(oracle_lib, D):
    """Decode with RoPE = plain decode (no RoPE) over keys pre-rotated at
    their logical index and queries at kv_len - 1, the rotations done here
    with the complex restatement and stored as fp64 -- pins the position each
    key and query gets and that V is not rotated."""
    rng = np.random.default_rng(32)
    Hq, Hkv, ps = 4, 2, 3
    lens = [1, 7, 40]
    kd = [f16_values(rng.standard_normal((L, Hkv, D))) for L in lens]
    vd = [f16_values(rng.standard_normal((L, Hkv, D))) for L in lens]
    q = f16_values(rng.standard_normal((len(lens), Hq, D)))
    kp, indptr, idx, last = paginate([to_f16_bits(k) for k in kd], ps, Hkv, D,
                                     np.random.default_rng(1))
    vp, _, _, _ = paginate([to_f16_bits(v) for v in vd], ps, Hkv, D, np.random.default_rng(1))
    kw = dict(num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps, sm_scale=0.09)
    o_r, l_r = oracle_lib.decode(to_f16_bits(q), kp, vp, indptr, idx, last, q_dtype="f16",
                                 kv_dtype="f16", rope=(1e4, 1.0), **kw)
    kr = [np.stack([[_rope_complex(k[t, h], t) for h in range(Hkv)] for t in range(len(k))])
          for k in kd]
    qr = np.stack([[_rope_complex(q[r, j], lens[r] - 1) for j in range(Hq)]
                   for r in range(len(lens))])
    kp2, indptr2, idx2, last2 = paginate(kr, ps, Hkv, D, np.random.default_rng(1),
                                         fill_bits=np.nan, dtype=np.float64)
    vp2, _, _, _ = paginate(vd, ps, Hkv, D, np.random.default_rng(1), fill_bits=np.nan,
                            dtype=np.float64)
    o_p, l_p = oracle_lib.decode(qr, kp2, vp2, indptr2, idx2, last2, q_dtype="f64",
                                 kv_dtype="f64", **kw)
    np.testing.assert_allclose(o_r, o_p, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_r, l_p, rtol=0, atol=1e-12)
    # a single key at position 0 with the query at position 0: RoPE is the identity
    o_0, l_0 = oracle_lib.decode(to_f16_bits(q), kp, vp, indptr, idx, last, q_dtype="f16",
                                 kv_dtype="f16", **kw)
    assert np.array_equal(o_r[0], o_0[0]) and np.array_equal(l_r[0], l_0[0])


def test_rope_cascade_is_flat_over_concatenated_keys(oracle_lib):
    """With RoPE the group's prefix tokens take positions 0 .. P-1 and the
    request's own tokens follow: cascade = flat decode over the concatenated
    table, bit for bit."""
    rng = np.random.default_rng(33)
    Hq, Hkv, D, ps = 2, 1, 128, 4
    P, lens = 10, [3, 0, 9]
    pre = to_f16_bits(rng.standard_normal((P, Hkv, D)))
    own = [to_f16_bits(rng.standard_normal((L, Hkv, D))) for L in lens]
    q = to_f16_bits(rng.standard_normal((len(lens), Hq, D)))
    pool, indptr, idx, last = paginate([pre] + own, ps, Hkv, D, np.random.default_rng(2))
    n_pre = (P + ps - 1) // ps
    kw = dict(num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps, q_dtype="f16",
              kv_dtype="f16", sm_scale=0.1, rope=(1e4, 1.0))
    p_indptr = np.array([0, n_pre], np.int32)
    own_indptr = (indptr[1:] - n_pre).astype(np.int32)
    o_c, l_c = oracle_lib.cascade(q, pool, pool, np.array([0, len(lens)], np.int32), p_indptr,
                                  idx[:n_pre], last[:1], own_indptr, idx[n_pre:], last[1:], **kw)
    # flat tables: the prefix pages then the request's own pages
    assert P % ps != 0     # the prefix's last page is partial: flat needs whole pages
    flat_dense = [np.concatenate([pre, o]) for o in own]
    fpool, findptr, fidx, flast = paginate(flat_dense, ps, Hkv, D, np.random.default_rng(3))
    o_f, l_f = oracle_lib.decode(q, fpool, fpool, findptr, fidx, flast, **kw)
    assert np.array_equal(o_c, o_f) and np.array_equal(l_c, l_f)


# ------------------------------------------------------------- append
# FlashInfer README example: append attention = single_prefill_with_kv_cache
# with causal=True where the last qo_len tokens of the KV cache are the new
# tokens; the batch form takes qo_indptr over the requests' query tokens.

def _append_problem(rng, lens, nq, Hq, Hkv, D, ps, scale=0.1):
    ks = [rng.standard_normal((L, Hkv, D)) for L in lens]
    vs = [rng.standard_normal((L, Hkv, D)) for L in lens]
    qo = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    qf = rng.standard_normal((int(qo[-1]), Hq, D)) * scale
    kp, indptr, idx, last = paginate([to_f16_bits(k) for k in ks], ps, Hkv, D,
                                     np.random.default_rng(7))
    vp, _, _, _ = paginate([to_f16_bits(v) for v in vs], ps, Hkv, D, np.random.default_rng(7))
    return qf, ks, vs, qo, kp, vp, indptr, idx, last


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("ps", [1, 5, 16])
def test_append_matches_dense_brute_force(oracle_lib, causal, ps):
    """Against the NumPy brute force with an explicit bottom-right-aligned
    lower-triangular mask (oracle/dense.py)."""
    from oracle.dense import ref_dense_append
    rng = np.random.default_rng(50 + ps)
    Hq, Hkv, D = 4, 2, 16
    lens, nq = [9, 20, 5, 33], [3, 20, 0, 7]
    qf, ks, vs, qo, kp, vp, indptr, idx, last = _append_problem(rng, lens, nq, Hq, Hkv, D, ps)
    sm = 0.41
    o, lse = oracle_lib.append(to_f16_bits(qf), kp, vp, qo, indptr, idx, last,
                               num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps,
                               q_dtype="f16", kv_dtype="f16", sm_scale=sm, causal=causal)
    for r in range(len(lens)):
        a, b = qo[r], qo[r + 1]
        if a == b:
            continue
        ro, rl = ref_dense_append(f16_values(qf[a:b]), f16_values(ks[r]), f16_values(vs[r]),
                                  sm, causal=causal)
        np.testing.assert_allclose(o[a:b], ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[a:b], rl, rtol=1e-12, atol=1e-13)


def test_append_closed_forms(oracle_lib):
    """Causal prefill of a whole request (qo_len = kv_len): row 0 sees only
    key 0, so o = v_0 and lse = sm_scale q.k_0 exactly; a one-token append
    is plain decode, bit for bit; without the mask every row is plain
    decode of that row over all keys, bit for bit."""
    rng = np.random.default_rng(60)
    Hq, Hkv, D, ps = 2, 1, 128, 4
    lens = [6, 11]
    qf, ks, vs, qo, kp, vp, indptr, idx, last = _append_problem(rng, lens, lens, Hq, Hkv, D, ps)
    kw = dict(num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps, q_dtype="f16",
              kv_dtype="f16", sm_scale=0.2)
    qb = to_f16_bits(qf)
    o, lse = oracle_lib.append(qb, kp, vp, qo, indptr, idx, last, **kw)
    for r in range(2):
        row0 = qo[r]
        for j in range(Hq):
            np.testing.assert_array_equal(o[row0, j], f16_values(vs[r][0, 0]))
            x0 = 0.2 * float(np.dot(f16_values(qf[row0, j]), f16_values(ks[r][0, 0])))
            assert abs(lse[row0, j] - x0) < 1e-12
    # the last row of a causal prefill sees every key: plain decode
    last_rows = qb[qo[1:] - 1]
    od, ld = oracle_lib.decode(last_rows, kp, vp, indptr, idx, last, **kw)
    assert np.array_equal(o[qo[1:] - 1], od) and np.array_equal(lse[qo[1:] - 1], ld)
    # one-token append = decode
    one = np.array([0, 1, 2], np.int32)
    o1, l1 = oracle_lib.append(last_rows, kp, vp, one, indptr, idx, last, **kw)
    assert np.array_equal(o1, od) and np.array_equal(l1, ld)
    # non-causal: each row is decode of that row over all the request's keys
    onc, lnc = oracle_lib.append(qb, kp, vp, qo, indptr, idx, last, causal=False, **kw)
    for r in range(2):
        rows = qb[qo[r]:qo[r + 1]]
        sub_ip = np.repeat(indptr[r:r + 2][None], len(rows), 0)
        for i in range(len(rows)):
            od_i, ld_i = oracle_lib.decode(rows[i][None], kp, vp, sub_ip[i], idx, last[r:r + 1],
                                           **kw)
            assert np.array_equal(onc[qo[r] + i], od_i[0])
            assert np.array_equal(lnc[qo[r] + i], ld_i[0])


def test_append_causal_row_equals_decode_of_truncated_request(oracle_lib):
    """Causal query i of n sits at position L - n + i: it equals plain
    decode of the request cut to its first L - n + i + 1 tokens (same pages,
    shorter last page), bit for bit -- also with RoPE, whose query position
    is then that of the cut request's last token."""
    rng = np.random.default_rng(61)
    Hq, Hkv, D, ps = 4, 2, 128, 3
    L, n = 17, 6
    qf, ks, vs, qo, kp, vp, indptr, idx, last = _append_problem(rng, [L], [n], Hq, Hkv, D, ps)
    qb = to_f16_bits(qf)
    for rope in (None, (1e4, 1.0)):
        kw = dict(num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps, q_dtype="f16",
                  kv_dtype="f16", sm_scale=0.15, rope=rope)
        o, lse = oracle_lib.append(qb, kp, vp, qo, indptr, idx, last, **kw)
        for i in range(n):
            keys = L - n + i + 1
            npg = (keys + ps - 1) // ps
            ip = np.array([0, npg], np.int32)
            la = np.array([keys - (npg - 1) * ps], np.int32)
            od, ld = oracle_lib.decode(qb[i][None], kp, vp, ip, idx[:npg], la, **kw)
            assert np.array_equal(o[i], od[0]) and np.array_equal(lse[i], ld[0]), (rope, i)


def test_append_mask_hides_later_keys(oracle_lib):
    """Changing the keys and values after query i's position leaves row i
    bit-identical under the causal mask and changes it without the mask."""
    rng = np.random.default_rng(62)
    Hq, Hkv, D, ps = 2, 2, 32, 4
    L, n = 12, 5
    qf, ks, vs, qo, kp, vp, indptr, idx, last = _append_problem(rng, [L], [n], Hq, Hkv, D, ps)
    kw = dict(num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps, q_dtype="f16",
              kv_dtype="f16", sm_scale=0.3)
    qb = to_f16_bits(qf)
    o1, l1 = oracle_lib.append(qb, kp, vp, qo, indptr, idx, last, **kw)
    n1, _ = oracle_lib.append(qb, kp, vp, qo, indptr, idx, last, causal=False, **kw)
    kp2, vp2 = kp.copy(), vp.copy()
    t = L - n + 2                      # first key hidden from rows 0 and 1
    for tt in range(t, L):
        pg, sl = idx[tt // ps], tt % ps
        kp2[pg, sl] = to_f16_bits(rng.standard_normal((Hkv, D)))
        vp2[pg, sl] = to_f16_bits(rng.standard_normal((Hkv, D)))
    o2, l2 = oracle_lib.append(qb, kp2, vp2, qo, indptr, idx, last, **kw)
    n2, _ = oracle_lib.append(qb, kp2, vp2, qo, indptr, idx, last, causal=False, **kw)
    assert np.array_equal(o1[:2], o2[:2]) and np.array_equal(l1[:2], l2[:2])
    assert not np.array_equal(o1[2:], o2[2:])
    assert not np.array_equal(n1[:2], n2[:2])


def test_append_rejects_more_queries_than_keys(oracle_lib):
    rng = np.random.default_rng(63)
    qf, ks, vs, qo, kp, vp, indptr, idx, last = _append_problem(rng, [3], [3], 2, 1, 8, 2)
    qo = np.array([0, 4], np.int32)
    with pytest.raises(ValueError):
        oracle_lib.append(to_f16_bits(np.zeros((4, 2, 8))), kp, vp, qo, indptr, idx, last,
                          num_qo_heads=2, num_kv_heads=1, head_dim=8, page_size=2,
                          q_dtype="f16", kv_dtype="f16", sm_scale=0.1)


# ------------------------------------------------------------- ragged KV
# FlashInfer README "core features" item 1 names a ragged KV cache beside
# the paged one: every request's tokens contiguous in one [total, Hkv, D]
# array, kv_indptr counting tokens, no page indices.

def _ragged_from_dense(dense_list):
    indptr = np.concatenate([[0], np.cumsum([len(d) for d in dense_list])]).astype(np.int32)
    pool = np.concatenate(dense_list)[:, None] if len(dense_list) else None
    return pool, indptr


def test_ragged_equals_paged_page_size_1_identity(oracle_lib):
    """A ragged table is the page-size-1 table whose indices are the rows
    themselves: decode, cascade and append agree bit for bit."""
    rng = np.random.default_rng(90)
    Hq, Hkv, D = 8, 2, 64
    lens = [5, 0, 33, 17]
    ks = [to_f16_bits(rng.standard_normal((L, Hkv, D))) for L in lens]
    vs = [to_f16_bits(rng.standard_normal((L, Hkv, D))) for L in lens]
    kp, ip = _ragged_from_dense(ks)
    vp, _ = _ragged_from_dense(vs)
    ident = np.arange(int(ip[-1]), dtype=np.int32)
    ones = np.ones(len(lens), np.int32)
    q = to_f16_bits(rng.standard_normal((len(lens), Hq, D)))
    kw = dict(num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=1, q_dtype="f16",
              kv_dtype="f16", sm_scale=0.13)
    o_r, l_r = oracle_lib.decode(q, kp, vp, ip, None, None, **kw)
    o_p, l_p = oracle_lib.decode(q, kp, vp, ip, ident, ones, **kw)
    assert np.array_equal(o_r, o_p) and np.array_equal(l_r, l_p)
    # cascade: a ragged prefix (the first 9 rows of request 2's data as a
    # shared prefix of requests 0..3) over ragged own rows
    pre = to_f16_bits(rng.standard_normal((9, Hkv, D)))
    kp2, ip2 = _ragged_from_dense([pre] + ks)
    vp2, _ = _ragged_from_dense([pre] + vs)
    own_ip = (ip2[1:] - ip2[1]).astype(np.int32) + ip2[1]
    own_ip = np.concatenate([[ip2[1]], own_ip[1:]]).astype(np.int32)
    qo_g = np.array([0, len(lens)], np.int32)
    p_ip = np.array([0, 9], np.int32)
    o_c, l_c = oracle_lib.cascade(q, kp2, vp2, qo_g, p_ip, None, None, own_ip, None, None, **kw)
    ident2 = np.arange(int(ip2[-1]), dtype=np.int32)
    o_cp, l_cp = oracle_lib.cascade(q, kp2, vp2, qo_g, p_ip, ident2, np.ones(1, np.int32), own_ip,
                                    ident2, ones, **kw)
    assert np.array_equal(o_c, o_cp) and np.array_equal(l_c, l_cp)
    # append
    qo = np.array([0, 2, 2, 10, 27], np.int32)
    qa = to_f16_bits(rng.standard_normal((27, Hq, D)))
    o_a, l_a = oracle_lib.append(qa, kp, vp, qo, ip, None, None, **kw)
    o_ap, l_ap = oracle_lib.append(qa, kp, vp, qo, ip, ident, ones, **kw)
    assert np.array_equal(o_a, o_ap) and np.array_equal(l_a, l_ap)


def test_ragged_matches_dense_brute_force(oracle_lib):
    from oracle.dense import ref_dense
    rng = np.random.default_rng(91)
    Hq, Hkv, D = 4, 2, 16
    lens = [7, 1, 40]
    ks = [rng.standard_normal((L, Hkv, D)) for L in lens]
    vs = [rng.standard_normal((L, Hkv, D)) for L in lens]
    qf = rng.standard_normal((len(lens), Hq, D)) * 0.1
    kp, ip = _ragged_from_dense([to_f16_bits(k) for k in ks])
    vp, _ = _ragged_from_dense([to_f16_bits(v) for v in vs])
    o, lse = oracle_lib.decode(to_f16_bits(qf), kp, vp, ip, None, None, num_qo_heads=Hq,
                               num_kv_heads=Hkv, head_dim=D, page_size=1, q_dtype="f16",
                               kv_dtype="f16", sm_scale=0.3)
    for r in range(len(lens)):
        ro, rl = ref_dense(f16_values(qf[r]), f16_values(ks[r]), f16_values(vs[r]), 0.3)
        np.testing.assert_allclose(o[r], ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[r], rl, rtol=1e-12, atol=1e-13)


def test_mixed_paged_and_ragged_tables_are_rejected(oracle_lib):
    kp = np.zeros((4, 1, 1, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle_lib.decode(np.zeros((1, 1, 8), np.uint16), kp, kp, np.array([0, 2], np.int32),
                          None, np.array([1], np.int32), num_qo_heads=1, num_kv_heads=1,
                          head_dim=8, page_size=1, q_dtype="f16", kv_dtype="f16",
                          sm_scale=0.1)


# ------------------------------------------------------------- HND pages
# The registry quickstart passes kv_layout with the cache; the other layout
# to NHD stores a page head-major: [num_pages][Hkv][page_size][D].

def test_hnd_pages_equal_nhd_pages_transposed(oracle_lib):
    """The same logical data with every page transposed to head-major gives
    bit-identical decode, cascade and append results."""
    rng = np.random.default_rng(95)
    Hq, Hkv, D, ps = 8, 4, 32, 5
    lens = [12, 0, 31, 5]
    ks = [to_f16_bits(rng.standard_normal((L, Hkv, D))) for L in lens]
    vs = [to_f16_bits(rng.standard_normal((L, Hkv, D))) for L in lens]
    kp, ip, idx, last = paginate(ks, ps, Hkv, D, np.random.default_rng(4))
    vp, _, _, _ = paginate(vs, ps, Hkv, D, np.random.default_rng(4))
    kh = np.ascontiguousarray(kp.transpose(0, 2, 1, 3))
    vh = np.ascontiguousarray(vp.transpose(0, 2, 1, 3))
    q = to_f16_bits(rng.standard_normal((len(lens), Hq, D)))
    kw = dict(num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps, q_dtype="f16",
              kv_dtype="f16", sm_scale=0.21)
    a = oracle_lib.decode(q, kp, vp, ip, idx, last, **kw)
    b = oracle_lib.decode(q, kh, vh, ip, idx, last, kv_layout="HND", **kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # a different layout really reads different rows
    c = oracle_lib.decode(q, kp, vp, ip, idx, last, kv_layout="HND", **kw)
    assert not np.array_equal(a[0], c[0])
    qo = np.array([0, 3, 3, 10, 15], np.int32)
    qa = to_f16_bits(rng.standard_normal((15, Hq, D)))
    a = oracle_lib.append(qa, kp, vp, qo, ip, idx, last, **kw)
    b = oracle_lib.append(qa, kh, vh, qo, ip, idx, last, kv_layout="HND", **kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # cascade: request 2's pages as the prefix of every request
    n2 = ip[3] - ip[2]
    p_ip = np.array([0, n2], np.int32)
    qo_g = np.array([0, len(lens)], np.int32)
    a = oracle_lib.cascade(q, kp, vp, qo_g, p_ip, idx[ip[2]:ip[3]], last[2:3], ip, idx, last, **kw)
    b = oracle_lib.cascade(q, kh, vh, qo_g, p_ip, idx[ip[2]:ip[3]], last[2:3], ip, idx, last,
                           kv_layout="HND", **kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------ multi-level cascade
# README "core features" item 3: cascade attention over a hierarchical KV
# cache; here with several shared levels (outermost first), each splitting
# the requests into contiguous groups that share a prefix.

def test_multilevel_cascade_is_flat_over_concatenated_keys(oracle_lib):
    rng = np.random.default_rng(97)
    Hq, Hkv, D, ps = 4, 2, 32, 4
    own_lens = [3, 0, 9, 5, 1]
    B = len(own_lens)
    # level 0: one group of all requests; level 1: groups {0,1}, {2,3,4}
    # (not nested in anything but level 0); level 2: {0}, {1,2}, {3,4}
    levels_groups = [[(0, 5)], [(0, 2), (2, 5)], [(0, 1), (1, 3), (3, 5)]]
    prefix_lens = [[6], [4, 0], [2, 7, 3]]
    dense = []
    level_dense = []
    for lg, pl in zip(levels_groups, prefix_lens):
        level_dense.append([to_f16_bits(rng.standard_normal((L, Hkv, D))) for L in pl])
    own = [to_f16_bits(rng.standard_normal((L, Hkv, D))) for L in own_lens]
    q = to_f16_bits(rng.standard_normal((B, Hq, D)))
    # one pool holding every list: level prefixes, then own lists
    lists = [x for ld in level_dense for x in ld] + own
    pool, ip_all, idx_all, last_all = paginate(lists, ps, Hkv, D, np.random.default_rng(5))
    levels = []
    k = 0
    for lg, ld in zip(levels_groups, level_dense):
        n = len(ld)
        sub = slice(k, k + n)
        ip = (ip_all[k:k + n + 1] - ip_all[k]).astype(np.int32)
        ix = idx_all[ip_all[k]:ip_all[k + n]]
        qo = np.array([lg[0][0]] + [g[1] for g in lg], np.int32)
        levels.append((qo, ip, ix, last_all[sub]))
        k += n
    own_ip = (ip_all[k:] - ip_all[k]).astype(np.int32)
    own_ix = idx_all[ip_all[k]:]
    kw = dict(num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps, q_dtype="f16",
              kv_dtype="f16", sm_scale=0.17)
    o_m, l_m = oracle_lib.cascade_levels(q, pool, pool, levels, own_ip, own_ix, last_all[k:], **kw)
    # flat: each request's concatenated list
    flat = []
    for r in range(B):
        parts = []
        for li, lg in enumerate(levels_groups):
            g = [gi for gi, (a, b) in enumerate(lg) if a <= r < b][0]
            parts.append(level_dense[li][g])
        parts.append(own[r])
        flat.append(np.concatenate(parts))
    fpool, fip, fix, flast = paginate(flat, ps, Hkv, D, np.random.default_rng(6))
    o_f, l_f = oracle_lib.decode(q, fpool, fpool, fip, fix, flast, **kw)
    assert np.array_equal(o_m, o_f) and np.array_equal(l_m, l_f)
    # one level through the multi-level entry = the single-level cascade
    lv = levels[1]
    o1, l1 = oracle_lib.cascade_levels(q, pool, pool, [lv], own_ip, own_ix, last_all[k:], **kw)
    o2, l2 = oracle_lib.cascade(q, pool, pool, lv[0], lv[1], lv[2], lv[3], own_ip, own_ix,
                                last_all[k:], **kw)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # no shared level = plain decode
    o0, l0 = oracle_lib.cascade_levels(q, pool, pool, [], own_ip, own_ix, last_all[k:], **kw)
    od, ld = oracle_lib.decode(q, pool, pool, own_ip, own_ix, last_all[k:], **kw)
    assert np.array_equal(o0, od) and np.array_equal(l0, ld)
