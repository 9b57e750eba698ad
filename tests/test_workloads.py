"""CPU tests of the seeded input generator (workloads/): each named workload
has the structure its configuration states, draws are deterministic in the
seed, and the e4m3 encoder it uses rounds as the OCP E4M3 format requires.
The generator only places data; these tests pin what it places."""
import math

import numpy as np
import pytest

import workloads as W


def _check_tables(w, lens, ps):
    """Page table of request r covers ceil(L_r / ps) distinct pages of the
    pool, last_page_len = L_r - (n_r - 1) ps, no page used twice."""
    n = (np.asarray(lens) + ps - 1) // ps
    assert np.array_equal(np.diff(w.kv_indptr), n)
    want_last = np.where(n > 0, np.asarray(lens) - (n - 1) * ps, 0)
    assert np.array_equal(w.last_page_len[n > 0], want_last[n > 0])
    assert np.all((w.last_page_len[n > 0] >= 1) & (w.last_page_len[n > 0] <= ps))
    used = w.kv_indices
    if w.prefix_kv_indices is not None:
        used = np.concatenate([w.prefix_kv_indices, used])
    assert len(np.unique(used)) == len(used)
    assert used.min() >= 0 and used.max() < w.meta["pool_pages"]


def test_single_request_shape():
    w = W.make("single_L2048_h32", tables_only=True)
    assert (w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size) == \
        (1, 32, 32, 128, 16)
    assert w.kv_lens.tolist() == [2048] and w.meta["pool_pages"] == 256
    assert len(w.kv_indices) == 128 and w.q_dtype == w.kv_dtype == "f16"
    _check_tables(w, w.kv_lens, 16)
    assert w.sm_scale == np.float32(1 / math.sqrt(128))


def test_batch64_lengths_and_last_page_rule():
    w = W.make("batch64_gqa4", tables_only=True)
    assert (w.batch, w.num_qo_heads, w.num_kv_heads) == (64, 32, 8)
    assert w.kv_lens.min() >= 512 and w.kv_lens.max() <= 4096
    # last_page_len = kv_len mod 16, 16 when that is 0
    m = w.kv_lens % 16
    assert np.array_equal(w.last_page_len, np.where(m == 0, 16, m))
    used = int(np.ceil(w.kv_lens / 16).sum())
    assert w.meta["pool_pages"] == math.ceil(used * 1.25)
    _check_tables(w, w.kv_lens, 16)


def test_skewed128_lognormal_mix():
    w = W.make("skewed128", tables_only=True)
    assert w.batch == 128
    long_ = w.kv_lens == 32768
    assert long_.sum() == 8
    short = w.kv_lens[~long_]
    assert len(short) == 120 and short.min() >= 64 and short.max() <= 2048
    # the underlying normal is N(ln 512, 0.5^2): the log-lengths' median and
    # spread (clipping leaves the middle alone)
    ls = np.log(short)
    assert abs(np.median(ls) - math.log(512)) < 0.15
    assert 0.35 < np.std(ls) < 0.65
    # the long requests sit at seeded positions, not at the end
    assert not np.all(np.flatnonzero(long_) >= 120)
    _check_tables(w, w.kv_lens, 16)


def test_cascade256_prefix_and_suffixes():
    w = W.make("cascade256", tables_only=True)
    assert (w.batch, w.num_qo_heads, w.num_kv_heads) == (256, 64, 8)
    assert w.q_dtype == w.kv_dtype == "bf16"
    assert w.prefix_lens.tolist() == [8192] and len(w.prefix_kv_indices) == 512
    assert w.prefix_qo_indptr.tolist() == [0, 256]
    assert w.kv_lens.min() >= 128 and w.kv_lens.max() <= 512
    _check_tables(w, w.kv_lens, 16)
    f = W.flatten_cascade(w)
    assert np.array_equal(f.kv_lens, w.kv_lens + 8192)
    assert f.prefix_kv_indptr is None
    for r in (0, 100, 255):
        row = f.kv_indices[f.kv_indptr[r]:f.kv_indptr[r + 1]]
        assert np.array_equal(row[:512], w.prefix_kv_indices)


def test_long32_fp8_both_page_sizes():
    v = W.make("long32_fp8", tables_only=True)
    assert set(v) == {1, 16}
    for ps, w in v.items():
        assert (w.batch, w.num_qo_heads, w.num_kv_heads, w.page_size) == (32, 64, 8, ps)
        assert w.kv_dtype == "e4m3" and w.q_dtype == "bf16"
        assert np.all(w.kv_lens == 32768)
        _check_tables(w, w.kv_lens, ps)
    assert len(v[1].kv_indices) == 32 * 32768


def test_small_fp8_scales_and_identical_logical_data():
    """Per-kv-head scale = amax / 448 over the head's logical values, and the
    page-size-1 and page-size-16 variants hold the same logical rows."""
    import oracle
    v = W.make("long32_fp8", small=True)
    w16, w1 = v[16], v[1]
    assert np.array_equal(w16.k_scale, w1.k_scale) and w16.k_scale.dtype == np.float32
    g16 = oracle.gather_map(16, w16.kv_indptr, w16.kv_indices, w16.last_page_len)
    g1 = oracle.gather_map(1, w1.kv_indptr, w1.kv_indices, w1.last_page_len)
    k16 = w16.k_pages.reshape(-1, w16.num_kv_heads, w16.head_dim)[g16]
    k1 = w1.k_pages.reshape(-1, w1.num_kv_heads, w1.head_dim)[g1]
    assert np.array_equal(k16, k1)
    # the largest code magnitude of each head is (close to) 448: amax / scale
    dec = np.vectorize(lambda c: oracle.decode_scalar(int(c), "e4m3"))(k16[:, :, :8])
    assert np.all(np.abs(dec).max(axis=(0, 2)) <= 448)


def test_seed_determinism():
    for name in ("single_L2048_h32", "batch64_gqa4", "cascade256"):
        a, b = W.make(name, small=True), W.make(name, small=True)
        for f in ("q", "k_pages", "v_pages", "kv_indptr", "kv_indices", "last_page_len"):
            assert np.array_equal(getattr(a, f), getattr(b, f)), (name, f)
        c = W.make(name, small=True, seed=12345)
        assert not np.array_equal(a.q, c.q)
    # the tables do not depend on drawing the values
    full = W.make("batch64_gqa4", small=True)
    tab = W.make("batch64_gqa4", small=True, tables_only=True)
    assert np.array_equal(full.kv_indices, tab.kv_indices)


def test_nan_poisoned_tails_and_unused_pages():
    w = W.make("batch64_gqa4", small=True)
    k = w.k_pages.view(np.uint16)
    used = np.zeros(w.meta["pool_pages"], bool)
    used[w.kv_indices] = True
    assert np.all(k[~used] == 0x7E00)
    for r in range(w.batch):
        last_page = w.kv_indices[w.kv_indptr[r + 1] - 1]
        assert np.all(k[last_page, w.last_page_len[r]:] == 0x7E00)


@pytest.mark.parametrize("x,want", [(0.1, 0.1015625), (447.9, 448.0), (-1e-3, -0.001953125),
                                    (500.0, 448.0), (-1e6, -448.0), (0.0, 0.0)])
def test_e4m3_encoder_spot_values(x, want):
    """Round to nearest even into OCP E4M3 after clamping to +-448 (the
    format's largest finite value; the cast itself does not saturate)."""
    import oracle
    code = int(W.cast_bits(np.array([x], np.float32), "e4m3")[0])
    assert oracle.decode_scalar(code, "e4m3") == want


def test_e4m3_encode_of_decode_is_identity():
    import oracle
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = np.array([oracle.decode_scalar(int(c), "e4m3") for c in codes], np.float64)
    back = W.cast_bits(vals.astype(np.float32), "e4m3")
    assert np.array_equal(back, codes)
