"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, validates arguments on the host, and the plan scheduler's work list
covers every (request, kv head, token) exactly once.  No GPU is touched."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fi():
    lib_path = os.path.join(ROOT, "paged_kv_decode_fi_amd", "libfi_decode.so")
    if not os.path.exists(lib_path):
        from paged_kv_decode_fi_amd import build as b
        b.build()
    import paged_kv_decode_fi_amd as m
    return m


def test_header_symbols_are_exported(fi):
    hdr = open(os.path.join(ROOT, "include", "fi_decode.h")).read()
    declared = set(re.findall(r"^(?:fi_status|const char\*)\s+(fi_\w+)\(", hdr, re.M))
    assert {"fi_plan", "fi_decode_run", "fi_merge_states", "fi_cascade_decode"} <= declared
    for name in declared:
        assert hasattr(fi.lib, name), name
    assert set(fi.EXPORTS) == declared


def _problem(fi, indptr, last, **kw):
    args = dict(num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                q_dtype="f16", kv_dtype="f16", prefix=None, chunk=0,
                pos_encoding="none", rope_theta=0.0, rope_scale=0.0)
    args.update(kw)
    indptr = np.asarray(indptr, np.int32)
    last = np.asarray(last, np.int32)
    return fi._problem(len(indptr) - 1, args["num_qo_heads"], args["num_kv_heads"],
                       args["head_dim"], args["page_size"], args["q_dtype"],
                       args["kv_dtype"], indptr, last, args["prefix"], args["chunk"],
                       args["pos_encoding"], args["rope_theta"], args["rope_scale"])


def _status(fi, indptr, last, **kw):
    pr, keep = _problem(fi, indptr, last, **kw)
    n = ctypes.c_int64(0)
    return fi.lib.fi_debug_plan_tiles(ctypes.byref(pr), 256, None, 0, ctypes.byref(n))


def test_host_validation_errors(fi):
    ok = _status(fi, [0, 2, 5], [3, 16])
    assert ok == 0
    assert _status(fi, [0, 5, 2], [3, 16]) == 1                 # indptr decreases
    assert _status(fi, [1, 2, 5], [3, 16]) == 1                 # indptr[0] != 0
    assert _status(fi, [0, 2, 5], [0, 16]) == 1                 # last_page_len 0
    assert _status(fi, [0, 2, 5], [3, 17]) == 1                 # last_page_len > ps
    assert _status(fi, [0, 2, 5], [3, 16], num_qo_heads=30) == 1  # Hq % Hkv
    assert _status(fi, [0, 2, 5], [3, 16], head_dim=96) == 2    # not built
    assert _status(fi, [0, 2, 5], [3, 16], num_qo_heads=256) == 2  # G = 32 > 16
    assert _status(fi, [0, 2, 5], [3, 16], kv_dtype="bf16") == 2   # mixed dtype
    assert _status(fi, [0, 2, 5], [3, 16], q_dtype="e4m3", kv_dtype="e4m3") == 2
    assert _status(fi, [0, 2, 5], [3, 16], page_size=0) == 1
    assert _status(fi, [0, 2, 5], [3, 16], chunk=40) == 1       # not a step multiple
    msg = fi.lib.fi_last_error().decode()
    assert "chunk_tokens" in msg


def test_head_dim_rules(fi):
    """head_dim 64, 128 and 256 are built for decode (with or without RoPE),
    a cascade level and append."""
    indptr, last = [0, 2, 5], [3, 16]
    prefix = (np.array([0, 2], np.int32), np.array([0, 1], np.int32),
              np.array([16], np.int32))
    for D in (64, 128, 256):
        assert _status(fi, indptr, last, head_dim=D) == 0
    for D in (32, 96, 512):
        assert _status(fi, indptr, last, head_dim=D) == 2
        assert "head_dim" in fi.lib.fi_last_error().decode()
    for D in (64, 256):
        assert _status(fi, indptr, last, head_dim=D, prefix=prefix) == 0
    for D in (64, 256):
        assert _status(fi, indptr, last, head_dim=D, pos_encoding="rope_llama") == 0
    for D, want in ((64, 0), (256, 0)):
        pr, keep = _problem(fi, indptr, last, head_dim=D)
        qo = np.array([0, 1, 3], np.int32)
        pr.qo_indptr, pr.causal = qo.ctypes.data, 1
        n = ctypes.c_int64(0)
        assert fi.lib.fi_debug_plan_tiles(ctypes.byref(pr), 256, None, 0, ctypes.byref(n)) == want


def test_rope_table_rows_scale_with_head_dim(fi):
    """The RoPE table holds head_dim / 2 (cos, sin) fp32 pairs per distance:
    its rows are 4 * head_dim bytes."""
    indptr, last = [0, 63], [16]                   # one request of 1,008 tokens
    for D in (64, 128, 256):
        st0, ws0 = _workspace(fi, indptr, last, head_dim=D)
        st1, ws1 = _workspace(fi, indptr, last, head_dim=D, pos_encoding="rope_llama")
        assert st0 == st1 == 0
        assert ws1 - ws0 >= 1008 * 4 * D and ws1 - ws0 < 1008 * 4 * D + 4096


def test_head_dim_workspace_scales(fi):
    """The partial states hold head_dim floats per row: a split plan's
    workspace grows with head_dim."""
    indptr, last = [0, 40], [16]                  # one request of 640 tokens
    sizes = [_workspace(fi, indptr, last, head_dim=D, chunk=64) for D in (64, 128, 256)]
    assert all(st == 0 for st, _ in sizes)
    assert sizes[0][1] < sizes[1][1] < sizes[2][1]


def _workspace(fi, indptr, last, **kw):
    pr, keep = _problem(fi, indptr, last, **kw)
    need = ctypes.c_size_t(0)
    st = fi.lib.fi_plan(ctypes.byref(pr), 256, None, 0, ctypes.byref(need), None, None)
    return st, need.value


def test_rope_plan_rules(fi):
    """RoPE plans: the mode is validated, non-finite parameters are refused,
    and the workspace grows by one (cos, sin) table row of 64 fp32 pairs per
    position 0 .. longest key list - 1 (at least 16 rows: every decode tile
    stages rows 0..15); a cascade plan's table covers the prefix and the
    suffix together, plus one query position per (level, request)."""
    indptr, last = [0, 2, 5], [3, 16]           # lengths 19 and 48
    assert _status(fi, indptr, last, pos_encoding="rope_llama") == 0
    pr, keep = _problem(fi, indptr, last)
    pr.pos_encoding = 2
    n = ctypes.c_int64(0)
    assert fi.lib.fi_debug_plan_tiles(ctypes.byref(pr), 256, None, 0, ctypes.byref(n)) == 1
    assert "pos_encoding" in fi.lib.fi_last_error().decode()
    prefix = (np.array([0, 2], np.int32), np.array([0, 1], np.int32),
              np.array([16], np.int32))
    assert _status(fi, indptr, last, pos_encoding="rope_llama", prefix=prefix) == 0
    st0, ws0 = _workspace(fi, indptr, last, prefix=prefix)
    st1, ws1 = _workspace(fi, indptr, last, pos_encoding="rope_llama", prefix=prefix)
    assert st0 == 0 and st1 == 0
    # (16 + 48 keys) x 512 B of table, the positions (256-B aligned), and
    # the partial states the fold no longer saves (RoPE plans merge)
    assert 64 * 512 + 256 <= ws1 - ws0
    assert _status(fi, indptr, last, pos_encoding="rope_llama", rope_theta=float("nan")) == 1
    assert _status(fi, indptr, last, pos_encoding="rope_llama", rope_scale=float("inf")) == 1
    st0, ws0 = _workspace(fi, indptr, last)
    st1, ws1 = _workspace(fi, indptr, last, pos_encoding="rope_llama")
    assert st0 == 0 and st1 == 0
    assert 48 * 512 <= ws1 - ws0 <= 48 * 512 + 256
    st0, ws0 = _workspace(fi, [0, 1], [3])
    st1, ws1 = _workspace(fi, [0, 1], [3], pos_encoding="rope_llama")
    assert st0 == 0 and st1 == 0 and 16 * 512 <= ws1 - ws0 <= 16 * 512 + 256
    # a large batch: RoPE tiles span 4 kv heads (8 without), and both work
    # lists cover every (request, kv head, token) once
    lens = np.full(64, 2048)
    ip = np.concatenate([[0], np.cumsum(lens // 16)]).astype(np.int32)
    la = np.full(64, 16, np.int32)
    for enc, want in (("none", 8), ("rope_llama", 4)):
        t = fi.debug_plan_tiles(ip, la, num_qo_heads=32, num_kv_heads=8, page_size=16,
                                pos_encoding=enc)
        hpt = _heads_per_tile(t, 8)
        assert hpt == want, (enc, hpt)
        _check_cover(t, lens, 8, hpt)


def test_run_calls_reject_bad_arguments_before_touching_the_device(fi):
    P = ctypes.c_void_p
    assert fi.lib.fi_decode_run(None, *([None] * 8), 0.0, None, None, None) == 1
    assert fi.lib.fi_cascade_decode(None, *([None] * 11), 0.0, None, None, None) == 1
    assert fi.lib.fi_merge_states(0, None, None, 4, 128, 0, None, None, 0, None) == 1
    assert fi.lib.fi_merge_states(65, None, None, 4, 128, 0, None, None, 0, None) == 1
    assert fi.lib.fi_merge_states(2, None, None, 4, 128, 2, None, None, 0, None) == 2
    assert fi.lib.fi_status_string(3) == b"FI_ERR_WORKSPACE_TOO_SMALL"


def test_workspace_size_query_is_host_only(fi):
    pr, keep = _problem(fi, [0, 2, 5], [3, 16])
    need = ctypes.c_size_t(0)
    st = fi.lib.fi_plan(ctypes.byref(pr), 256, None, 0, ctypes.byref(need), None, None)
    assert st == 0 and need.value > 0


def _lens(indptr, last, ps):
    n = np.diff(indptr)
    return np.where(n > 0, (n - 1) * ps + last, 0)


def _heads_per_tile(tiles, Hkv):
    """kv heads one decode tile spans, read off the work list's head offsets."""
    starts = {int(t[1]) for t in tiles if t[5] == 0} - {0}
    hpt = min(starts) if starts else Hkv
    assert Hkv % hpt == 0 and all(s % hpt == 0 for s in starts)
    return hpt


def _check_cover(tiles, lens, Hkv, hpt, has_other_states=None):
    seen = {}
    empty = set()
    for req, h0, t0, t1, slot, kind, r0, r1 in tiles:
        if kind != 0:
            continue
        assert 0 <= t0 <= t1 <= lens[req]
        if t0 == t1:
            empty.add(req)
        for h in range(h0, min(h0 + hpt, Hkv)):
            for t in range(t0, t1):
                key = (req, h, t)
                assert key not in seen, key
                seen[key] = slot
    total = int(sum(lens)) * Hkv
    assert len(seen) == total
    for r, L in enumerate(lens):
        if L == 0 and not (has_other_states is not None and has_other_states[r]):
            assert r in empty      # empty requests still get their (0, -inf) written


@pytest.mark.parametrize("head_dim", [128, 64, 256])
@pytest.mark.parametrize("seed", range(6))
def test_plan_covers_every_token_once(fi, seed, head_dim):
    rng = np.random.default_rng(seed)
    ps = [1, 16, 7, 16, 32, 2][seed]
    Hkv = [8, 8, 4, 32, 2, 1][seed]
    G = [4, 1, 8, 1, 16, 4][seed]
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, 3000, size=B)
    lens[rng.integers(0, B)] = 0
    n = (lens + ps - 1) // ps
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = np.where(n > 0, lens - (n - 1) * ps, 0).astype(np.int32)
    tiles = fi.debug_plan_tiles(indptr, last, num_qo_heads=Hkv * G, num_kv_heads=Hkv,
                                page_size=ps, num_cus=[256, 32, 8, 256, 4, 1][seed],
                                head_dim=head_dim)
    _check_cover(tiles, _lens(indptr, last, ps), Hkv, _heads_per_tile(tiles, Hkv))
    _check_dispatch_order([t[3] - t[2] for t in tiles if t[5] == 0],
                          [256, 32, 8, 256, 4, 1][seed])
    # split requests: every (req, chunk, head) has its own slot; unsplit: -1
    slots = [t[4] for t in tiles if t[4] >= 0]
    assert len(slots) == len(set(slots))
    # a decode tile carries its request's page-table base (word 6)
    for t in tiles:
        if t[5] == 0:
            assert t[6] == indptr[t[0]]
    _check_even_split(tiles, _lens(indptr, last, ps))


def _check_dispatch_order(d, num_cus):
    """Decode tiles placed for in-order dispatch (tile i on CU i mod
    num_cus): the first round holds the longest tiles, each CU's tiles run
    longest first, and the most loaded CU carries no more than under plain
    longest-first order."""
    d = [int(x) for x in d]
    n = len(d)
    k = min(n, num_cus)
    assert sorted(d[:k], reverse=True) == sorted(d, reverse=True)[:k]
    cols = [d[c::num_cus] for c in range(num_cus)]
    for col in cols:
        assert col == sorted(col, reverse=True)
    srt = sorted(d, reverse=True)
    assert max(sum(col) for col in cols) <= max(sum(srt[c::num_cus]) for c in range(num_cus))


def _check_even_split(tiles, lens, chunk=None):
    """A split request's chunks share its 16-token steps out evenly: chunk
    starts on step boundaries, step counts differ by at most one (the longer
    ones first), and none exceeds the plan's chunk length."""
    by_req = {}
    for t in tiles:
        if t[5] == 0:
            by_req.setdefault(int(t[0]), set()).add((int(t[2]), int(t[3])))
    for r, spans in by_req.items():
        spans = sorted(spans)
        steps = [(-(-(b - a) // 16)) for a, b in spans]
        assert all(a % 16 == 0 for a, _ in spans), (r, spans)
        assert max(steps) - min(steps) <= 1, (r, spans)
        assert steps == sorted(steps, reverse=True), (r, spans)
        if chunk is not None:
            assert max(b - a for a, b in spans) <= chunk, (r, spans, chunk)


@pytest.mark.parametrize("chunk", [32, 48, 304])
def test_forced_chunk_splits_evenly(fi, chunk):
    """chunk_tokens given: every request is cut into ceil(len / chunk)
    chunks of near-equal whole steps, none longer than chunk."""
    lens = np.array([0, 1, 15, 16, 17, 31, 33, 100, 303, 304, 305, 1000, 4097])
    n = (lens + 15) // 16
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = np.where(n > 0, lens - (n - 1) * 16, 0).astype(np.int32)
    tiles = fi.debug_plan_tiles(indptr, last, num_qo_heads=8, num_kv_heads=2, page_size=16,
                                chunk_tokens=chunk)
    _check_cover(tiles, lens, 2, _heads_per_tile(tiles, 2))
    _check_even_split(tiles, lens, chunk)
    for r, L in enumerate(lens):
        if L > 0:
            assert len({t[2] for t in tiles if t[0] == r and t[5] == 0}) == -(-L // chunk)


def test_plan_is_deterministic_and_depends_only_on_lengths(fi):
    lens = np.array([100, 5000, 0, 17, 32768])
    n = (lens + 15) // 16
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = np.where(n > 0, lens - (n - 1) * 16, 0).astype(np.int32)
    a = fi.debug_plan_tiles(indptr, last, num_qo_heads=32, num_kv_heads=8, page_size=16)
    b = fi.debug_plan_tiles(indptr, last, num_qo_heads=32, num_kv_heads=8, page_size=16)
    assert np.array_equal(a, b)


def test_plan_splits_long_requests(fi):
    """The skewed mix: 8 long requests must be cut into many chunks."""
    lens = np.array([500] * 120 + [32768] * 8)
    n = (lens + 15) // 16
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = np.where(n > 0, lens - (n - 1) * 16, 0).astype(np.int32)
    t = fi.debug_plan_tiles(indptr, last, num_qo_heads=32, num_kv_heads=8, page_size=16)
    long_tiles = [x for x in t if lens[x[0]] == 32768]
    assert len(long_tiles) >= 8 * 2 * 16
    assert max(x[3] - x[2] for x in t) <= 2048


@pytest.mark.parametrize("head_dim", [128, 256])
def test_cascade_plan_covers_prefix_rows_once(fi, head_dim):
    G, Hkv, ps = 8, 8, 16
    groups = [(5, 300), (3, 0), (2, 1000)]
    B = sum(g[0] for g in groups)
    lens = np.array([10, 0, 200, 3, 40, 7, 7, 7, 500, 1])
    n = (lens + ps - 1) // ps
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = np.where(n > 0, lens - (n - 1) * ps, 0).astype(np.int32)
    qo = np.concatenate([[0], np.cumsum([g[0] for g in groups])]).astype(np.int32)
    plens = np.array([g[1] for g in groups])
    pn = (plens + ps - 1) // ps
    pip = np.concatenate([[0], np.cumsum(pn)]).astype(np.int32)
    plast = np.where(pn > 0, plens - (pn - 1) * ps, 0).astype(np.int32)
    tiles = fi.debug_plan_tiles(indptr, last, num_qo_heads=G * Hkv, num_kv_heads=Hkv,
                                page_size=ps, prefix=(qo, pip, plast), num_cus=16,
                                head_dim=head_dim)
    req_prefix = np.repeat(plens, [g[0] for g in groups]) > 0
    _check_cover(tiles, lens, Hkv, _heads_per_tile(tiles, Hkv), has_other_states=req_prefix)
    seen = set()
    for grp, h, t0, t1, pc, kind, r0, r1 in tiles:
        if kind != 1:
            continue
        assert 0 <= t0 < t1 <= plens[grp]
        for row in range(r0, r1):
            assert row < (qo[grp + 1] - qo[grp]) * G
            for t in range(t0, t1):
                key = (grp, h, row, t)
                assert key not in seen
                seen.add(key)
    want = sum(g[0] * G * Hkv * g[1] for g in groups)
    assert len(seen) == want
    # row tiles: 8 waves x 32 rows, 16 rows per wave at head_dim 256
    assert max(r1 - r0 for *_, kind, r0, r1 in tiles if kind == 1) <= (
        128 if head_dim == 256 else 256)


def test_cascade_single_chunk_suffix_folds_prefix_states(fi):
    """A cascade request whose own suffix is one decode chunk gets a decode
    tile that writes the final output (slot -1) after folding in its prefix
    chunks' states (word 7 = their count); longer suffixes are split and go
    through the merge (word 7 = 0)."""
    G, Hkv, ps = 8, 8, 16
    lens = np.array([10, 0, 200, 3000, 40])
    B = len(lens)
    n = (lens + ps - 1) // ps
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = np.where(n > 0, lens - (n - 1) * ps, 0).astype(np.int32)
    qo = np.array([0, B], np.int32)
    plen = 4096
    pip = np.array([0, plen // ps], np.int32)
    plast = np.array([ps], np.int32)
    tiles = fi.debug_plan_tiles(indptr, last, num_qo_heads=G * Hkv, num_kv_heads=Hkv,
                                page_size=ps, prefix=(qo, pip, plast), num_cus=64,
                                chunk_tokens=256)
    n_pchunks = len({t[2] for t in tiles if t[5] == 1})
    assert n_pchunks >= 2
    for req, h0, t0, t1, slot, kind, r0, r1 in tiles:
        if kind != 0:
            continue
        if lens[req] <= 256:          # one chunk: folded, final output
            assert slot == -1 and r1 == n_pchunks, (req, slot, r1)
        else:                         # split: partial states, merged afterwards
            assert slot >= 0 and r1 == 0, (req, slot, r1)
    assert not any(t[0] == 1 for t in tiles if t[5] == 0)   # empty suffix: prefix only


def test_binding_rejects_host_and_mistyped_tensors(fi):
    """The binding passes device pointers only: a host tensor (its address
    would reach the kernels) or a mistyped table is refused before any call."""
    import torch
    with pytest.raises(ValueError, match="GPU tensor"):
        fi._ptr(torch.zeros(4), "q")
    with pytest.raises(ValueError, match="GPU tensor"):
        fi._tables(torch.zeros(3, dtype=torch.int32), None, None)
    assert fi._ptr(None) is None


def _append_cover(tiles, lens, nq, G, Hkv, causal):
    """Every (query token, q head, key below its limit) is covered by exactly
    one append tile; tiles reach no key that none of their rows may see."""
    qo = np.concatenate([[0], np.cumsum(nq)])
    seen = {}
    for req, h, t0, t1, slot, kind, r0, r1 in tiles:
        assert kind == 2
        n, L = nq[req], lens[req]
        assert 0 <= r0 < r1 <= n * G and 0 <= t0 < t1 <= L
        last_lim = L - n + (r1 - 1) // G + 1 if causal else L
        assert t1 <= last_lim
        for row in range(r0, r1):
            i, gg = divmod(row, G)
            lim = L - n + i + 1 if causal else L
            for t in range(t0, min(t1, lim)):
                key = (qo[req] + i, h * G + gg, t)
                assert key not in seen, key
                seen[key] = slot
    want = sum((L - n + i + 1 if causal else L) * G * Hkv
               for L, n in zip(lens, nq) for i in range(n))
    assert len(seen) == want


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("chunk", [0, 32, 64])
@pytest.mark.parametrize("head_dim", [128, 256])
def test_append_plan_covers_every_visible_key_once(fi, causal, chunk, head_dim):
    rng = np.random.default_rng(80 + chunk)
    ps, Hkv, G = 16, 2, 4
    lens = np.array([300, 5, 129, 64, 0, 77])
    nq = np.array([70, 5, 1, 64, 0, 0])
    n = (lens + ps - 1) // ps
    ip = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    la = np.where(n > 0, lens - (n - 1) * ps, 0).astype(np.int32)
    qo = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    t = fi.debug_plan_tiles(ip, la, num_qo_heads=Hkv * G, num_kv_heads=Hkv, page_size=ps,
                            qo_indptr=qo, causal=causal, chunk_tokens=chunk, num_cus=8,
                            head_dim=head_dim)
    _append_cover(t, lens, nq, G, Hkv, causal)
    if chunk:
        assert np.all(t[:, 3] - t[:, 2] <= chunk)
    # rows per tile: 8 waves x 32 rows, 16 at head_dim 256 (4-wave tiles
    # when every request has few rows, at head_dim <= 128 only)
    assert np.all(t[:, 7] - t[:, 6] <= (128 if head_dim == 256 else 256))
    del rng


def test_append_plan_rules(fi):
    ip = np.array([0, 2, 5], np.int32)
    la = np.array([3, 16], np.int32)                 # lengths 19 and 48
    ok = np.array([0, 19, 20], np.int32)
    assert _status(fi, ip, la) == 0
    pr, keep = _problem(fi, ip, la)
    q_ok = ok.copy()
    pr.qo_indptr, pr.causal = q_ok.ctypes.data, 1
    n = ctypes.c_int64(0)
    assert fi.lib.fi_debug_plan_tiles(ctypes.byref(pr), 256, None, 0, ctypes.byref(n)) == 0
    for bad in ([0, 20, 21], [1, 2, 3], [0, 5, 4]):   # 20 > 19 keys; [0] != 0; decreasing
        q_bad = np.array(bad, np.int32)
        pr.qo_indptr = q_bad.ctypes.data
        assert fi.lib.fi_debug_plan_tiles(ctypes.byref(pr), 256, None, 0, ctypes.byref(n)) == 1
    pr.qo_indptr = q_ok.ctypes.data
    pr.pos_encoding = 1                               # RoPE append: 8-wave, 128-row tiles
    assert fi.lib.fi_debug_plan_tiles(ctypes.byref(pr), 256, None, 0, ctypes.byref(n)) == 0
    pr.pos_encoding = 0
    prefix = (np.array([0, 2], np.int32), np.array([0, 1], np.int32), np.array([16], np.int32))
    pr2, keep2 = _problem(fi, ip, la, prefix=prefix)
    pr2.qo_indptr, pr2.causal = q_ok.ctypes.data, 1
    assert fi.lib.fi_debug_plan_tiles(ctypes.byref(pr2), 256, None, 0, ctypes.byref(n)) == 2
    # a one-token append of every request: one 4-row tile per (request, kv
    # head); 128-row (4-wave) tiles, two per CU: 512 tiles already give
    # 1.25 tiles per resident workgroup's worth (640) within one chunk's
    # split, so each covers all 512 keys
    lens = np.full(64, 512)
    ip3 = np.concatenate([[0], np.cumsum(lens // 16)]).astype(np.int32)
    t = fi.debug_plan_tiles(ip3, np.full(64, 16, np.int32), num_qo_heads=32, num_kv_heads=8,
                            page_size=16, qo_indptr=np.arange(65, dtype=np.int32))
    assert len(t) == 64 * 8 and set(t[:, 3] - t[:, 2]) == {512}
    assert np.all(t[:, 6] == 0) and np.all(t[:, 7] == 4)
    _append_cover(t, lens, np.ones(64, np.int64), 4, 8, True)


def test_multilevel_cascade_plan(fi):
    """Several shared levels: every (level, group, kv head, prefix token) is
    covered once by that level's prefix tiles, every row of the group's
    requests by each tile's rows; both level forms at once, and more than 8
    levels, are refused."""
    ps, Hkv, G = 16, 2, 4
    own = np.array([5, 0, 40, 17])
    n = (own + ps - 1) // ps
    ip = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    la = np.where(n > 0, own - (n - 1) * ps, 0).astype(np.int32)

    def level(groups):
        qo = np.concatenate([[0], np.cumsum([g[0] for g in groups])]).astype(np.int32)
        pl = np.array([g[1] for g in groups])
        pn = (pl + ps - 1) // ps
        pip = np.concatenate([[0], np.cumsum(pn)]).astype(np.int32)
        pla = np.where(pn > 0, pl - (pn - 1) * ps, 0).astype(np.int32)
        return (qo, pip, pla), pl

    specs = [[(4, 700)], [(2, 30), (2, 0)], [(1, 3), (3, 50)]]
    levels, plens = zip(*[level(s) for s in specs])
    t = fi.debug_plan_tiles(ip, la, num_qo_heads=Hkv * G, num_kv_heads=Hkv, page_size=ps,
                            levels=list(levels), chunk_tokens=32)
    pre = t[t[:, 5] == 1]
    # prefix tiles come level by level; within a level, cover each (group,
    # head, token) once over all row tiles
    k = 0
    for li, (qo, pip, pla) in enumerate(levels):
        ng = len(qo) - 1
        want = {(g, h, tt, row) for g in range(ng) for h in range(Hkv)
                for tt in range(int(plens[li][g])) for row in range((qo[g + 1] - qo[g]) * G)}
        got = set()
        while k < len(pre) and len(got) < len(want):
            req, h, t0, t1, slot, kind, r0, r1 = pre[k]
            for tt in range(t0, t1):
                for row in range(r0, r1):
                    key = (req, h, tt, row)
                    assert key not in got, (li, key)
                    got.add(key)
            k += 1
        assert got == want, li
    assert k == len(pre)
    pr, keep = _problem(fi, ip, la, prefix=(levels[0][0], levels[0][1], levels[0][2]))
    arr = (fi.CascadeLevel * 1)()
    arr[0].num_groups = 1
    arr[0].qo_indptr = levels[0][0].ctypes.data
    arr[0].kv_indptr = levels[0][1].ctypes.data
    arr[0].last_page_len = levels[0][2].ctypes.data
    pr.num_cascade_levels, pr.cascade_levels = 1, ctypes.cast(arr, ctypes.c_void_p)
    nn = ctypes.c_int64(0)
    assert fi.lib.fi_debug_plan_tiles(ctypes.byref(pr), 256, None, 0, ctypes.byref(nn)) == 1
    with pytest.raises(fi.FiError):
        fi.debug_plan_tiles(ip, la, num_qo_heads=Hkv * G, num_kv_heads=Hkv, page_size=ps,
                            levels=[levels[0]] * 9)


def test_tuning_is_explicit_and_environment_is_ignored(fi, monkeypatch):
    """Plans depend on fi_problem.tuning only: the library reads no
    environment variable, a zero field is the default, and a forced value
    changes the cut of the work (never its coverage)."""
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 3000, size=24)
    npg = (lens + 15) // 16
    indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    last = (lens - (npg - 1) * 16).astype(np.int32)
    kw = dict(num_qo_heads=32, num_kv_heads=8, page_size=16)
    base = fi.debug_plan_tiles(indptr, last, **kw)
    for name in ("FI_HEADS_PER_TILE", "FI_WAVES_PER_CU", "FI_CHUNK_MIN", "FI_DECODE_DEPTH",
                 "FI_CASCADE_FOLD", "FI_PREFIX_WAVES"):
        monkeypatch.setenv(name, "1")
    assert np.array_equal(fi.debug_plan_tiles(indptr, last, **kw), base)
    zero = fi.debug_plan_tiles(indptr, last, tuning={f: 0 for f in fi.TUNING_FIELDS}, **kw)
    assert np.array_equal(zero, base)
    two = fi.debug_plan_tiles(indptr, last, tuning=dict(heads_per_tile=2), **kw)
    assert set(np.unique(two[:, 1] % 2)) == {0} and len(two) > len(base)
    # every (request, kv head, token) is still covered exactly once
    cover = {}
    for r, h0, t0, t1 in two[:, :4]:
        for h in range(h0, h0 + 2):
            cover[(r, h)] = cover.get((r, h), 0) + (t1 - t0)
    assert all(cover[(r, h)] == lens[r] for r in range(24) for h in range(8))
    with pytest.raises(fi.FiError):
        fi.debug_plan_tiles(indptr, last, tuning=dict(decode_depth=3), **kw)
    with pytest.raises(fi.FiError):
        fi.debug_plan_tiles(indptr, last, tuning=dict(chunk_min=-16), **kw)
    with pytest.raises(fi.FiError):
        fi.debug_plan_tiles(indptr, last, tuning=dict(cascade_fold=2), **kw)
    with pytest.raises(ValueError):
        fi.debug_plan_tiles(indptr, last, tuning=dict(no_such_knob=1), **kw)


def _table(lens, ps=16):
    lens = np.asarray(lens)
    n = (lens + ps - 1) // ps
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    last = np.where(n > 0, lens - (n - 1) * ps, 0).astype(np.int32)
    return indptr, last


def test_plan_sizes_skewed_batches_for_two_rounds(fi):
    """Many short requests and a few very long ones: one round of 16 waves
    per CU (512 eight-head tiles on 256 CUs) leaves room for only 32 tiles of
    the 8 long requests (8192-token chunks, each running alone long after
    the short tiles end), over 1.25x the mean tokens per workgroup slot, so
    the chunk is sized for two rounds (1024 tiles: 8 x ceil(32768 / c) <= 544,
    c = 496).  With the wave target given explicitly the rule is off."""
    lens = np.array([64] * 480 + [32768] * 8)
    indptr, last = _table(lens)
    t = fi.debug_plan_tiles(indptr, last, num_qo_heads=32, num_kv_heads=8, page_size=16)
    chunk = max(int(x[3] - x[2]) for x in t if x[5] == 0)
    assert chunk == 496, chunk
    _check_cover(t, lens, 8, _heads_per_tile(t, 8))
    t = fi.debug_plan_tiles(indptr, last, num_qo_heads=32, num_kv_heads=8, page_size=16,
                            tuning={"waves_per_cu": 16})
    chunk = max(int(x[3] - x[2]) for x in t if x[5] == 0)
    assert chunk == 8192, chunk
    # uniform lengths keep the one-round chunk: 64 x 2048 keys, 512 slots,
    # mean 256 tokens per slot, chunk 256
    indptr, last = _table(np.full(64, 2048))
    t = fi.debug_plan_tiles(indptr, last, num_qo_heads=32, num_kv_heads=8, page_size=16)
    assert max(int(x[3] - x[2]) for x in t if x[5] == 0) == 256


def _roundrobin_imbalance(tiles, num_cus, hpt):
    """Most-loaded CU over the mean when tile i runs on CU i mod num_cus,
    load = 16-token steps x kv heads of the tile."""
    d = [t for t in tiles if t[5] == 0]
    load = np.zeros(num_cus)
    for i, t in enumerate(d):
        load[i % num_cus] += -(-(int(t[3]) - int(t[2])) // 16) * hpt
    return load.max() / load.mean()


def test_plan_narrows_tiles_for_uneven_work(fi):
    """Four-head decode tiles when they even out the per-CU load by more than
    their ~4 % per-byte cost: the skewed mix (a few 32K-token requests among
    short ones) gets them, the uniform batch of 64 and the 32K batch keep
    eight-head tiles, and a forced width or chunk is left alone."""
    import workloads as W
    want = {"skewed128": 4, "batch64_gqa4": 8, "long32_fp8": 8}
    for name, hpt_want in want.items():
        w = W.make(name, tables_only=True)
        w = w[16] if isinstance(w, dict) else w
        kw = dict(num_qo_heads=w.num_qo_heads, num_kv_heads=w.num_kv_heads,
                  page_size=w.page_size, num_cus=256)
        t = fi.debug_plan_tiles(w.kv_indptr, w.last_page_len, **kw)
        hpt = _heads_per_tile(t, w.num_kv_heads)
        assert hpt == hpt_want, (name, hpt)
        _check_cover(t, _lens(w.kv_indptr, w.last_page_len, w.page_size), w.num_kv_heads, hpt)
        t8 = fi.debug_plan_tiles(w.kv_indptr, w.last_page_len, tuning=dict(heads_per_tile=8), **kw)
        assert _heads_per_tile(t8, w.num_kv_heads) == 8
        i8, i4 = _roundrobin_imbalance(t8, 256, 8), _roundrobin_imbalance(
            fi.debug_plan_tiles(w.kv_indptr, w.last_page_len, tuning=dict(heads_per_tile=4), **kw),
            256, 4)
        assert (i4 * 1.04 < i8) == (hpt_want == 4), (name, i8, i4)
    w = W.make("skewed128", tables_only=True)
    t = fi.debug_plan_tiles(w.kv_indptr, w.last_page_len, num_qo_heads=32, num_kv_heads=8,
                            page_size=16, chunk_tokens=736)
    assert _heads_per_tile(t, 8) == 8


def test_cascade_suffix_tiles_are_dispatch_ordered(fi):
    """The folded suffix tiles of the cascade workload (1,024 tiles of
    uniform 128-512-key suffixes on 256 CUs) are placed for in-order
    dispatch: longest first per CU column, the first round the longest
    tiles, and the most loaded column well below plain longest-first order."""
    import workloads as W
    w = W.make("cascade256", tables_only=True)
    t = fi.debug_plan_tiles(w.kv_indptr, w.last_page_len, num_qo_heads=w.num_qo_heads,
                            num_kv_heads=w.num_kv_heads, page_size=w.page_size,
                            q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, num_cus=256,
                            prefix=(w.prefix_qo_indptr, w.prefix_kv_indptr,
                                    w.prefix_last_page_len))
    d = [int(x[3] - x[2]) for x in t if x[5] == 0]
    assert len(d) == 1024
    _check_dispatch_order(d, 256)
    cols = [sum(d[c::256]) for c in range(256)]
    srt = sorted(d, reverse=True)
    rr = [sum(srt[c::256]) for c in range(256)]
    mean = sum(d) / 256
    assert max(cols) / mean < 1.03 < max(rr) / mean
