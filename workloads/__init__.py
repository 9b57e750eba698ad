"""Seeded synthetic inputs for paged-KV decode attention.

This module only PLACES random data: it draws request lengths, a shuffled
page pool, q and K/V values, casts them to their storage dtype and writes K/V
rows into pages through the page table.  It holds none of the attention
arithmetic; both the oracle (tests) and the GPU path (tests, bench) consume
what it returns.

Workloads (names used everywhere else):

=================== =====================================================
single_L2048_h32    1 request, 32 q heads = 32 kv heads, D 128, kv_len 2048,
                    fp16, page_size 16, 128 pages shuffled in a 256-page pool
                    (the README's single-request decode example shape)
batch64_gqa4        64 requests, 32 q / 8 kv heads, kv_len ~ U{512..4096},
                    fp16, page_size 16, pool = 1.25 x pages used
skewed128           128 requests, 32/8: 120 lengths round(lognormal(ln 512,
                    0.5)) clipped to [64, 2048] + 8 of 32768 at random
                    positions, fp16, page_size 16
cascade256          256 requests, 64/8, bf16: one shared 8192-token prefix
                    (512 pages) + own suffix ~ U{128..512}, page_size 16
long32_fp8_ps{1,16} 32 requests, 64/8, kv_len 32768, K/V e4m3 with a per
                    kv-head fp32 scale (amax/448), q bf16, page_size 1 or 16
=================== =====================================================

Value recipe: numpy PCG64 ``default_rng(seed)``; q, K, V ~ N(0, 1) drawn in
fp32, rounded to nearest-even into fp16 (numpy) or bf16 (torch CPU); e4m3 via
torch's float8_e4m3fn after clamping to +-448.  Pool pages no request owns and
the slots after ``last_page_len`` in a request's last page hold NaN, so any
read of them shows up in the outputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0, "e4m3": 0x7F}
STORAGE = {"f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8}
ESIZE = {"f16": 2, "bf16": 2, "e4m3": 1}


def cast_bits(x: np.ndarray, dtype: str, scale: Optional[np.ndarray] = None):
    """fp32 values -> raw storage bits of ``dtype`` (RNE)."""
    x = np.asarray(x, np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "e4m3":
        if scale is not None:
            t = t / torch.from_numpy(np.asarray(scale, np.float32))
        # torch's cast does not saturate (it gives NaN above 448): clamp first
        t = t.clamp(-448.0, 448.0)
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError(dtype)


@dataclass
class Paged:
    """One paged decode problem, all arrays on the host."""
    name: str
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    q_dtype: str
    kv_dtype: str
    q: np.ndarray                   # [B, Hq, D] raw bits
    k_pages: np.ndarray             # [num_pages, ps, Hkv, D] raw bits
    v_pages: np.ndarray
    kv_indptr: np.ndarray           # int32 [B+1]
    kv_indices: np.ndarray          # int32 [nnz pages]
    last_page_len: np.ndarray       # int32 [B]
    kv_lens: np.ndarray             # int64 [B] (per-request own tokens)
    sm_scale: float
    k_scale: Optional[np.ndarray] = None   # float32 [Hkv] (e4m3 only)
    v_scale: Optional[np.ndarray] = None
    # cascade level (None when absent)
    prefix_qo_indptr: Optional[np.ndarray] = None
    prefix_kv_indptr: Optional[np.ndarray] = None
    prefix_kv_indices: Optional[np.ndarray] = None
    prefix_last_page_len: Optional[np.ndarray] = None
    prefix_lens: Optional[np.ndarray] = None
    # append problems: request r's query tokens qo_indptr[r] .. qo_indptr[r+1]-1
    # (q is then [total_q, Hq, D]), the last ones of its keys
    qo_indptr: Optional[np.ndarray] = None
    causal: bool = True
    meta: dict = field(default_factory=dict)

    @property
    def group_size(self) -> int:
        return self.num_qo_heads // self.num_kv_heads

    @property
    def row_bytes(self) -> int:
        return self.head_dim * ESIZE[self.kv_dtype]

    def kv_bytes(self, cascade: bool = True) -> int:
        """Algorithmic K+V bytes: valid tokens once per (token, kv head); a
        shared prefix counts once when ``cascade`` (else once per request)."""
        toks = int(self.kv_lens.sum())
        if self.prefix_lens is not None:
            if cascade:
                toks += int(self.prefix_lens.sum())
            else:
                per_req = np.repeat(self.prefix_lens, np.diff(self.prefix_qo_indptr))
                toks += int(per_req.sum())
        return 2 * toks * self.num_kv_heads * self.row_bytes

    @property
    def num_rows(self) -> int:
        """Rows of q / o / lse: query tokens (append) or requests."""
        return int(self.qo_indptr[-1]) if self.qo_indptr is not None else self.batch

    def visible_keys(self) -> int:
        """Sum over query tokens of the keys each attends (append problems)."""
        n = np.diff(self.qo_indptr).astype(np.int64)
        L = self.kv_lens.astype(np.int64)
        if not self.causal:
            return int((n * L).sum())
        # query i of n sees L - n + i + 1 keys
        return int((n * (L - n) + n * (n + 1) // 2).sum())

    def append_flops(self) -> int:
        """4 D flops per (query token, q head, visible key): q.k and p.v."""
        return 4 * self.head_dim * self.num_qo_heads * self.visible_keys()

    def other_bytes(self) -> int:
        """q + o + lse + page indices + scales."""
        qo = 2 * self.num_rows * self.num_qo_heads * self.head_dim * ESIZE[self.q_dtype]
        lse = 4 * self.num_rows * self.num_qo_heads
        if self.meta.get("ragged"):   # row offsets only
            idx = 4 * len(self.kv_indptr)
            if self.prefix_kv_indptr is not None:
                idx += 4 * (len(self.prefix_kv_indptr) + len(self.prefix_qo_indptr))
        else:
            idx = 4 * (len(self.kv_indices) + len(self.kv_indptr) + len(self.last_page_len))
            if self.prefix_kv_indices is not None:
                idx += 4 * (len(self.prefix_kv_indices) + len(self.prefix_kv_indptr)
                            + len(self.prefix_last_page_len) + len(self.prefix_qo_indptr))
        sc = 0 if self.k_scale is None else 8 * self.num_kv_heads
        return qo + lse + idx + sc


def _pages_for(lens, ps):
    n = (np.asarray(lens, np.int64) + ps - 1) // ps
    last = np.where(n > 0, np.asarray(lens, np.int64) - (n - 1) * ps, 0)
    # an empty request owns no page; its last_page_len is unused (0)
    return n, last.astype(np.int32)


def _scatter(pool, pages_of_req, L, ps, data):
    """Write logical rows data[t] of one request into its pages."""
    if L == 0:
        return
    t = np.arange(L)
    pool[pages_of_req[t // ps], t % ps] = data


def build(name, kv_lens, *, Hq, Hkv, D=128, ps=16, q_dtype="f16", kv_dtype="f16",
          seed=0, pool_pages=None, pool_factor=1.25, prefix_len=None,
          prefix_groups=None, extra_page_sizes=(), poison=True, tables_only=False):
    """General generator.

    kv_lens: per-request own token counts.  prefix_len: if given, one shared
    prefix (or ``prefix_groups`` = list of (n_requests, prefix_len) for several
    groups of contiguous requests).  extra_page_sizes: also return the SAME
    logical data laid out with these page sizes (dict in .meta['variants']).
    Returns a Paged (or a dict of Paged by page size when extra sizes given).
    tables_only: the same lengths and page tables without drawing any value
    (q, k_pages, v_pages and the e4m3 scales are None; meta['pool_pages']
    holds the pool size) -- for checking a workload's structure cheaply.
    """
    rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, np.int64)
    B = len(kv_lens)
    groups = []
    if prefix_groups is not None:
        groups = list(prefix_groups)
    elif prefix_len is not None:
        groups = [(B, int(prefix_len))]
    assert sum(g[0] for g in groups) in (0, B)
    seeds = np.random.SeedSequence(seed).spawn(4 + 2 * (B + len(groups)))
    q_bits = None
    if not tables_only:
        q_rng = np.random.default_rng(seeds[0])
        qf = q_rng.standard_normal((B, Hq, D), dtype=np.float32)
        q_bits = cast_bits(qf, q_dtype)

    # logical rows of each key list: groups' prefixes first, then requests
    lists = [("p", g, int(glen)) for g, (_, glen) in enumerate(groups)]
    lists += [("r", r, int(kv_lens[r])) for r in range(B)]
    list_seeds = {lst[:2]: (seeds[4 + 2 * i], seeds[5 + 2 * i])
                  for i, lst in enumerate(lists)}

    def logical(lst, which):
        sk, sv = list_seeds[lst[:2]]
        r = np.random.default_rng(sk if which == "k" else sv)
        return r.standard_normal((lst[2], Hkv, D), dtype=np.float32)

    k_scale = v_scale = None
    if kv_dtype == "e4m3" and not tables_only:
        amax_k = np.zeros(Hkv, np.float32)
        amax_v = np.zeros(Hkv, np.float32)
        for lst in lists:
            if lst[2] == 0:
                continue
            amax_k = np.maximum(amax_k, np.abs(logical(lst, "k")).max(axis=(0, 2)))
            amax_v = np.maximum(amax_v, np.abs(logical(lst, "v")).max(axis=(0, 2)))
        k_scale = (amax_k / np.float32(448.0)).astype(np.float32)
        v_scale = (amax_v / np.float32(448.0)).astype(np.float32)

    variants = {}
    glens = np.array([g[1] for g in groups], np.int64)
    for vi, ps_i in enumerate((ps,) + tuple(extra_page_sizes)):
        n_req, last_req = _pages_for(kv_lens, ps_i)
        if groups:
            n_pre, last_pre = _pages_for(glens, ps_i)
        else:
            n_pre, last_pre = np.zeros(0, np.int64), np.zeros(0, np.int32)
        used = int(n_req.sum() + n_pre.sum())
        if pool_pages is not None and vi == 0:
            P = int(pool_pages)
        else:
            P = int(math.ceil(used * pool_factor))
        P = max(P, used, 1)
        perm = np.random.default_rng([seed, 7919, ps_i]).permutation(P).astype(np.int32)
        pre_pages, req_pages, off = [], [], 0
        for g in range(len(groups)):
            pre_pages.append(perm[off:off + n_pre[g]])
            off += int(n_pre[g])
        for r in range(B):
            req_pages.append(perm[off:off + n_req[r]])
            off += int(n_req[r])
        st = STORAGE[kv_dtype]
        fill = NAN_BITS[kv_dtype] if poison else 0
        variants[ps_i] = dict(
            n_req=n_req, last_req=last_req, n_pre=n_pre, last_pre=last_pre,
            pre_pages=pre_pages, req_pages=req_pages, P=P,
            kp=None if tables_only else np.full((P, ps_i, Hkv, D), fill, st),
            vp=None if tables_only else np.full((P, ps_i, Hkv, D), fill, st))
    # one pass over the logical key lists, scattered into every variant's pool
    for lst in lists:
        kind, idx, L = lst
        if L == 0 or tables_only:
            continue
        kd, vd = logical(lst, "k"), logical(lst, "v")
        if kv_dtype == "e4m3":
            kb = cast_bits(kd, "e4m3", k_scale[None, :, None])
            vb = cast_bits(vd, "e4m3", v_scale[None, :, None])
        else:
            kb, vb = cast_bits(kd, kv_dtype), cast_bits(vd, kv_dtype)
        del kd, vd
        for ps_i, V in variants.items():
            pages = V["pre_pages"][idx] if kind == "p" else V["req_pages"][idx]
            _scatter(V["kp"], pages, L, ps_i, kb)
            _scatter(V["vp"], pages, L, ps_i, vb)
    out = {}
    for ps_i, V in variants.items():
        kv_indptr = np.zeros(B + 1, np.int32)
        kv_indptr[1:] = np.cumsum(V["n_req"])
        kv_indices = (np.concatenate(V["req_pages"]) if B
                      else np.zeros(0, np.int32)).astype(np.int32)
        w = Paged(name=name if ps_i == ps else f"{name}_ps{ps_i}", batch=B,
                  num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=ps_i,
                  q_dtype=q_dtype, kv_dtype=kv_dtype, q=q_bits, k_pages=V["kp"],
                  v_pages=V["vp"], kv_indptr=kv_indptr, kv_indices=kv_indices,
                  last_page_len=V["last_req"], kv_lens=kv_lens.copy(),
                  sm_scale=float(np.float32(1.0 / math.sqrt(D))),
                  k_scale=k_scale, v_scale=v_scale)
        if groups:
            w.prefix_qo_indptr = np.concatenate(
                [[0], np.cumsum([g[0] for g in groups])]).astype(np.int32)
            w.prefix_kv_indptr = np.concatenate([[0], np.cumsum(V["n_pre"])]).astype(np.int32)
            w.prefix_kv_indices = (np.concatenate(V["pre_pages"]) if V["pre_pages"]
                                   else np.zeros(0, np.int32)).astype(np.int32)
            w.prefix_last_page_len = V["last_pre"].astype(np.int32)
            w.prefix_lens = glens
        w.meta["pool_pages"] = V["P"]
        out[ps_i] = w
    if extra_page_sizes:
        return out
    return out[ps]


def build_append(name, kv_lens, q_lens, *, Hq, Hkv, D=128, ps=16, q_dtype="f16",
                 kv_dtype="f16", seed=0, causal=True, **kw):
    """Append problem: the paged K/V of ``build`` (kv_lens include the new
    tokens) and q [sum(q_lens), Hq, D] drawn from its own seeded stream."""
    q_lens = np.asarray(q_lens, np.int64)
    assert np.all(q_lens <= np.asarray(kv_lens)) and np.all(q_lens >= 0)
    w = build(name, kv_lens, Hq=Hq, Hkv=Hkv, D=D, ps=ps, q_dtype=q_dtype,
              kv_dtype=kv_dtype, seed=seed, **kw)
    qo = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q_rng = np.random.default_rng(np.random.SeedSequence([seed, 4231]))
    qf = q_rng.standard_normal((int(qo[-1]), Hq, D), dtype=np.float32)
    ws = w.values() if isinstance(w, dict) else [w]
    for v in ws:
        v.q = cast_bits(qf, q_dtype)
        v.qo_indptr = qo
        v.causal = bool(causal)
    return w


# ---- the named workloads ---------------------------------------------------

WORKLOADS = ("single_L2048_h32", "batch64_gqa4", "skewed128", "cascade256",
             "long32_fp8")


def make(name: str, seed: Optional[int] = None, small: bool = False, head_dim: int = 128,
         tables_only: bool = False):
    """Named workload at full size, or a SMALL variant with the same structure
    (same heads, dtypes, page sizes, length mix shape; several tiles and a
    ragged tail) that the oracle finishes in seconds.  head_dim other than
    128 keeps every other parameter and the seeded length draw.

    long32_fp8 returns a dict {1: Paged, 16: Paged} with identical logical data.
    """
    idx = WORKLOADS.index(name)
    seed = 1000 + idx if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "single_L2048_h32":
        L = 300 if small else 2048
        return build(name, [L], Hq=32, Hkv=32, D=head_dim, ps=16, seed=seed,
                     pool_pages=(40 if small else 256), tables_only=tables_only)
    if name == "batch64_gqa4":
        B, lo, hi = (6, 1, 600) if small else (64, 512, 4096)
        lens = rng.integers(lo, hi + 1, size=B)
        return build(name, lens, Hq=32, Hkv=8, D=head_dim, ps=16, seed=seed,
                     tables_only=tables_only)
    if name == "skewed128":
        nshort, nlong, cl, ch, mu, Llong = ((10, 2, 8, 256, math.log(64), 2048) if small
                                            else (120, 8, 64, 2048, math.log(512), 32768))
        short = np.clip(np.round(rng.lognormal(mu, 0.5, size=nshort)), cl, ch).astype(np.int64)
        lens = np.concatenate([short, np.full(nlong, Llong, np.int64)])
        lens = lens[rng.permutation(len(lens))]
        return build(name, lens, Hq=32, Hkv=8, D=head_dim, ps=16, seed=seed,
                     tables_only=tables_only)
    if name == "cascade256":
        B, lo, hi, P = (8, 1, 100, 512) if small else (256, 128, 512, 8192)
        lens = rng.integers(lo, hi + 1, size=B)
        return build(name, lens, Hq=64, Hkv=8, D=head_dim, ps=16, q_dtype="bf16",
                     kv_dtype="bf16", seed=seed, prefix_len=P, tables_only=tables_only)
    if name == "long32_fp8":
        B, L = (3, 700) if small else (32, 32768)
        return build(name, np.full(B, L, np.int64), Hq=64, Hkv=8, D=head_dim, ps=16,
                     q_dtype="bf16", kv_dtype="e4m3", seed=seed,
                     extra_page_sizes=(1,), tables_only=tables_only)
    raise KeyError(name)


# Append workloads (FlashInfer README append example: kv_len 2048, 32 q and
# 32 kv heads, head_dim 128, fp16, the last 128 cache tokens are the query,
# causal mask; and a batch of 16 such requests with GQA 32/8 and the length
# mix of batch64_gqa4).
APPEND_WORKLOADS = ("append_single_q128", "append_batch16_q128")


def make_append(name: str, seed: Optional[int] = None, small: bool = False,
                head_dim: int = 128):
    idx = APPEND_WORKLOADS.index(name)
    seed = 2000 + idx if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "append_single_q128":
        L, n = (300, 40) if small else (2048, 128)
        return build_append(name, [L], [n], Hq=32, Hkv=32, D=head_dim, ps=16, seed=seed)
    if name == "append_batch16_q128":
        B, lo, hi, n = (4, 1, 600, 48) if small else (16, 512, 4096, 128)
        lens = rng.integers(lo, hi + 1, size=B)
        return build_append(name, lens, np.minimum(lens, n), Hq=32, Hkv=8, D=head_dim,
                            ps=16, seed=seed)
    raise KeyError(name)


def to_ragged(w: Paged) -> Paged:
    """The same logical problem in the ragged KV layout: every key list
    (cascade prefixes first, then the requests) contiguous in K / V
    [total, 1, Hkv, D] (page size 1), the indptr tables counting rows;
    kv_indices / prefix_kv_indices hold the identity rows (for the oracle's
    page-size-1 reading; the ragged kernels do not read them) and the
    last-page tables are None."""
    import copy
    Hkv, D, ps = w.num_kv_heads, w.head_dim, w.page_size
    kp = w.k_pages.reshape(-1, Hkv, D)
    vp = w.v_pages.reshape(-1, Hkv, D)

    def rows(indptr, indices, last, i):
        n = int(indptr[i + 1] - indptr[i])
        L = 0 if n == 0 else (n - 1) * ps + int(last[i])
        t = np.arange(L)
        return indices[indptr[i] + t // ps].astype(np.int64) * ps + t % ps

    parts = []
    ng = 0 if w.prefix_kv_indptr is None else len(w.prefix_kv_indptr) - 1
    for g in range(ng):
        parts.append(rows(w.prefix_kv_indptr, w.prefix_kv_indices, w.prefix_last_page_len, g))
    for r in range(w.batch):
        parts.append(rows(w.kv_indptr, w.kv_indices, w.last_page_len, r))
    sizes = [len(x) for x in parts]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    allrows = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    r = copy.copy(w)
    r.name = w.name + "_ragged"
    r.page_size = 1
    r.k_pages = np.ascontiguousarray(kp[allrows][:, None])
    r.v_pages = np.ascontiguousarray(vp[allrows][:, None])
    r.kv_indptr = offs[ng:].copy()
    r.kv_indices = np.arange(int(offs[-1]), dtype=np.int32)
    r.last_page_len = None
    if ng:
        r.prefix_kv_indptr = offs[:ng + 1].copy()
        r.prefix_kv_indices = r.kv_indices
        r.prefix_last_page_len = None
    r.meta = dict(w.meta, ragged=True)
    return r


def to_hnd(w: Paged) -> Paged:
    """The same problem with head-major (HND) pages [num_pages][Hkv][ps][D]."""
    import copy
    r = copy.copy(w)
    r.name = w.name + "_hnd"
    r.k_pages = np.ascontiguousarray(w.k_pages.transpose(0, 2, 1, 3))
    r.v_pages = np.ascontiguousarray(w.v_pages.transpose(0, 2, 1, 3))
    r.meta = dict(w.meta, hnd=True)
    return r


def build_multilevel(name, kv_lens, levels, *, Hq, Hkv, D=128, ps=16, q_dtype="f16",
                     kv_dtype="f16", seed=0):
    """Cascade with several shared levels, outermost first: levels[l] is a
    list of (n_requests, prefix_len) groups of contiguous requests covering
    the batch.  Returns a Paged whose meta["levels"] holds, per level,
    (qo_indptr, kv_indptr, kv_indices, last_page_len, prefix_lens) into the
    same page pools; the request tables are the usual fields."""
    rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, np.int64)
    B = len(kv_lens)
    lists = []          # (level or -1, index, length)
    for l, groups in enumerate(levels):
        assert sum(g[0] for g in groups) == B
        for gi, (_, plen) in enumerate(groups):
            lists.append((l, gi, int(plen)))
    lists += [(-1, r, int(kv_lens[r])) for r in range(B)]
    data = {(l, i): (rng.standard_normal((L, Hkv, D), dtype=np.float32),
                     rng.standard_normal((L, Hkv, D), dtype=np.float32)) for l, i, L in lists}
    k_scale = v_scale = None
    if kv_dtype == "e4m3":
        amk = np.max([np.abs(k).max(axis=(0, 2)) for k, _ in data.values() if len(k)], axis=0)
        amv = np.max([np.abs(v).max(axis=(0, 2)) for _, v in data.values() if len(v)], axis=0)
        k_scale = (amk / np.float32(448.0)).astype(np.float32)
        v_scale = (amv / np.float32(448.0)).astype(np.float32)
    npages = [(L + ps - 1) // ps for _, _, L in lists]
    P = int(math.ceil(sum(npages) * 1.25)) + 1
    perm = rng.permutation(P).astype(np.int32)
    st = STORAGE[kv_dtype]
    kp = np.full((P, ps, Hkv, D), NAN_BITS[kv_dtype], st)
    vp = kp.copy()
    pages_of = {}
    off = 0
    for (l, i, L), n in zip(lists, npages):
        pages = perm[off:off + n]
        off += n
        pages_of[(l, i)] = pages
        k, v = data[(l, i)]
        if L:
            kb = cast_bits(k, kv_dtype, None if k_scale is None else k_scale[None, :, None])
            vb = cast_bits(v, kv_dtype, None if v_scale is None else v_scale[None, :, None])
            _scatter(kp, pages, L, ps, kb)
            _scatter(vp, pages, L, ps, vb)

    def table(keys):
        lens = [len(data[k][0]) for k in keys]
        n = [(L + ps - 1) // ps for L in lens]
        ip = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        ix = (np.concatenate([pages_of[k] for k in keys]) if keys else
              np.zeros(0, np.int32)).astype(np.int32)
        last = np.array([L - (m - 1) * ps if m else 0 for L, m in zip(lens, n)], np.int32)
        return ip, ix, last, np.asarray(lens, np.int64)

    lv = []
    for l, groups in enumerate(levels):
        qo = np.concatenate([[0], np.cumsum([g[0] for g in groups])]).astype(np.int32)
        ip, ix, last, plens = table([(l, gi) for gi in range(len(groups))])
        lv.append((qo, ip, ix, last, plens))
    ip, ix, last, _ = table([(-1, r) for r in range(B)])
    q = cast_bits(rng.standard_normal((B, Hq, D), dtype=np.float32), q_dtype)
    return Paged(name=name, batch=B, num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                 page_size=ps, q_dtype=q_dtype, kv_dtype=kv_dtype, q=q, k_pages=kp,
                 v_pages=vp, kv_indptr=ip, kv_indices=ix, last_page_len=last,
                 kv_lens=kv_lens.copy(), sm_scale=float(np.float32(1.0 / math.sqrt(D))),
                 k_scale=k_scale, v_scale=v_scale, meta={"levels": lv})


def flatten_cascade(w: Paged) -> Paged:
    """The same keys as one flat page table per request, with no cascade
    level: request r's pages are its group's shared prefix pages followed by
    its own (pages shared, not copied).  Needs whole-page prefixes (config 4's
    8,192 = 512 x 16 tokens) so the concatenated table is contiguous."""
    import copy
    assert w.prefix_kv_indptr is not None
    ps = w.page_size
    assert np.all(w.prefix_lens % ps == 0), "prefix lengths must be whole pages"
    grp = np.repeat(np.arange(len(w.prefix_qo_indptr) - 1), np.diff(w.prefix_qo_indptr))
    tabs, last = [], np.zeros(w.batch, np.int32)
    for r in range(w.batch):
        g = grp[r]
        pre = w.prefix_kv_indices[w.prefix_kv_indptr[g]:w.prefix_kv_indptr[g + 1]]
        own = w.kv_indices[w.kv_indptr[r]:w.kv_indptr[r + 1]]
        tabs.append(np.concatenate([pre, own]))
        last[r] = w.last_page_len[r] if len(own) else (ps if len(pre) else 0)
    f = copy.copy(w)
    f.name = w.name + "_flat"
    f.kv_indptr = np.concatenate([[0], np.cumsum([len(t) for t in tabs])]).astype(np.int32)
    f.kv_indices = np.concatenate(tabs).astype(np.int32)
    f.last_page_len = last
    f.kv_lens = w.kv_lens + w.prefix_lens[grp]
    f.prefix_qo_indptr = f.prefix_kv_indptr = f.prefix_kv_indices = None
    f.prefix_last_page_len = f.prefix_lens = None
    return f
