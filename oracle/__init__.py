"""Test-infrastructure oracle for paged-KV decode attention (CPU, fp64).

ONLY the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and
the oracle shares no code with it.

Two independent implementations live here:

* ``liboracle.so`` built from ``oracle.c`` -- the paged decode / cascade /
  merge oracle in plain C, fp64, two-pass softmax, threads over
  (request, kv head) items.
* ``dense.py`` -- a NumPy brute force over an explicit dense K/V, used to pin
  the C oracle on tiny inputs.

Sources followed: the FlashInfer README ("core features" items 1-3: paged /
vector-sparse attention, GQA head-query fusion, cascade attention,
low-precision KV), the hysenlabs review ("running a first decode": the
q[num_qo_heads, head_dim] / k,v[kv_len, num_kv_heads, head_dim] contract), the
"Pre-compiled cubins for FlashInfer" registry quickstart (kv_indptr,
kv_indices, last_page_len over separate k and v caches) and the
flash-attention summary ("How it works": exact attention).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC_PATH = os.path.join(HERE, "oracle.c")

# dtype codes understood by oracle.c
F16, BF16, E4M3, F32, F64 = 0, 1, 2, 3, 4
DTYPE_CODE = {"f16": F16, "bf16": BF16, "e4m3": E4M3, "f32": F32, "f64": F64}


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain IEEE, no fast-math)."""
    if force or not os.path.exists(LIB_PATH) or (
            os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH)):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-pthread", "-fno-fast-math", SRC_PATH, "-o",
                               tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I, D, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_int64
        L.oracle_f16_to_f64.restype = D
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = D
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3_to_f64.restype = D
        L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_gather_map.restype = I64
        L.oracle_gather_map.argtypes = [I, I, P, P, P, P]
        L.oracle_decode.restype = I
        L.oracle_decode.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P,
                                    D, P, P, P, I, I, D, D, I]
        L.oracle_cascade.restype = I
        L.oracle_cascade.argtypes = [I, I, I, I, I, I, I, P, P, P, I, P, P, P, P,
                                     P, P, P, P, P, D, P, P, P, I, I, D, D, I]
        L.oracle_cascade_levels.restype = I
        L.oracle_cascade_levels.argtypes = [I, I, I, I, I, I, I, P, P, P, I, P, P, P, P, P,
                                            P, P, P, P, P, D, P, P, P, I, I, D, D, I]
        L.oracle_append.restype = I
        L.oracle_append.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P,
                                    D, I, P, P, P, I, I, D, D, I]
        L.oracle_rope_rotate.restype = None
        L.oracle_rope_rotate.argtypes = [P, I, D, D, D, P]
        L.oracle_merge.restype = I
        L.oracle_merge.argtypes = [I, I64, I, I, P, I, P, P, P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt=None):
    if a is None:
        return None
    a = np.asarray(a) if dt is None else np.asarray(a, dtype=dt)
    return np.ascontiguousarray(a)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def decode_scalar(code: int, dtype: str) -> float:
    L = lib()
    if dtype == "f16":
        return L.oracle_f16_to_f64(code)
    if dtype == "bf16":
        return L.oracle_bf16_to_f64(code)
    if dtype == "e4m3":
        return L.oracle_e4m3_to_f64(code)
    raise ValueError(dtype)


def gather_map(page_size, kv_indptr, kv_indices, last_page_len) -> np.ndarray:
    """Physical token slot (page*ps + slot) of every logical token, request-major."""
    indptr = _c(kv_indptr, np.int32)
    indices = _c(kv_indices, np.int32)
    last = _c(last_page_len, np.int32)
    B = len(indptr) - 1
    n = np.diff(indptr).astype(np.int64)
    total = int(np.where(n > 0, (n - 1) * page_size + last, 0).sum())
    out = np.empty(max(total, 1), np.int64)
    k = lib().oracle_gather_map(B, page_size, _ptr(indptr), _ptr(indices),
                                _ptr(last), _ptr(out))
    assert k == total
    return out[:total]


def _rope_args(rope):
    """rope = None or (theta, scale) -> (on, theta, scale) for the C oracle."""
    if rope is None:
        return 0, 1.0, 1.0
    theta, scale = rope
    return 1, float(theta), float(scale)


def _hnd(kv_layout):
    """kv_layout "NHD" (pages [P][ps][Hkv][D]) or "HND" ([P][Hkv][ps][D])."""
    if kv_layout not in ("NHD", "HND"):
        raise ValueError(kv_layout)
    return int(kv_layout == "HND")


def rope_rotate(x, pos, theta=1e4, scale=1.0):
    """The oracle's rotate-half RoPE of one fp64 vector at position pos."""
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib().oracle_rope_rotate(_ptr(x), len(x), float(pos), float(theta), float(scale),
                             _ptr(out))
    return out


def decode(q, k_pages, v_pages, kv_indptr, kv_indices, last_page_len, *,
           num_qo_heads, num_kv_heads, head_dim, page_size, q_dtype, kv_dtype,
           sm_scale, k_scale=None, v_scale=None, unit_mask=None, threads=None,
           rope=None, kv_layout="NHD"):
    """fp64 paged decode.  q/k_pages/v_pages are raw storage arrays (uint16 for
    f16/bf16 bits, uint8 for e4m3 codes, float32/float64 otherwise).
    rope = (theta, scale) applies LLaMA-style rotate-half RoPE (keys at their
    logical index, the query at kv_len - 1).
    Returns (o [B, Hq, D] fp64, lse [B, Hq] fp64)."""
    indptr = _c(kv_indptr, np.int32)
    B = len(indptr) - 1
    o = np.zeros((B, num_qo_heads, head_dim), np.float64)
    lse = np.full((B, num_qo_heads), np.nan, np.float64)
    q, k_pages, v_pages = _c(q), _c(k_pages), _c(v_pages)
    indices, last = _c(kv_indices, np.int32), _c(last_page_len, np.int32)
    ks, vs = _c(k_scale, np.float32), _c(v_scale, np.float32)
    um = _c(unit_mask, np.uint8)
    rc = lib().oracle_decode(B, num_qo_heads, num_kv_heads, head_dim, page_size,
                             DTYPE_CODE[q_dtype], DTYPE_CODE[kv_dtype], _ptr(q),
                             _ptr(k_pages), _ptr(v_pages), _ptr(indptr),
                             _ptr(indices), _ptr(last), _ptr(ks), _ptr(vs),
                             float(sm_scale), _ptr(um), _ptr(o), _ptr(lse),
                             threads or default_threads(), *_rope_args(rope),
                             _hnd(kv_layout))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return o, lse


def cascade_levels(q, k_pages, v_pages, levels, kv_indptr, kv_indices, last_page_len, *,
                   num_qo_heads, num_kv_heads, head_dim, page_size, q_dtype, kv_dtype,
                   sm_scale, k_scale=None, v_scale=None, unit_mask=None, threads=None,
                   rope=None, kv_layout="NHD"):
    """fp64 multi-level cascade: levels = [(qo_indptr, kv_indptr, kv_indices,
    last_page_len), ...] outermost first (qo_indptr partitions the requests
    into contiguous groups); request r attends over its group's prefix at
    every level in order, then its own pages."""
    indptr = _c(kv_indptr, np.int32)
    B = len(indptr) - 1
    o = np.zeros((B, num_qo_heads, head_dim), np.float64)
    lse = np.full((B, num_qo_heads), np.nan, np.float64)
    keep = []
    ptrs = {k: [] for k in ("qo", "ip", "ix", "la")}
    ng = []
    for (qo, ip, ix, la) in levels:
        arrs = [_c(qo, np.int32), _c(ip, np.int32), _c(ix, np.int32), _c(la, np.int32)]
        keep += arrs
        ng.append(len(arrs[0]) - 1)
        for key, a in zip(("qo", "ip", "ix", "la"), arrs):
            ptrs[key].append(_ptr(a))
    nl = len(levels)
    PP = ctypes.c_void_p * max(nl, 1)
    cp = {k: PP(*v) for k, v in ptrs.items()}
    ng_a = np.asarray(ng if ng else [0], np.int32)
    a = [_c(q), _c(k_pages), _c(v_pages), indptr, _c(kv_indices, np.int32),
         _c(last_page_len, np.int32), _c(k_scale, np.float32), _c(v_scale, np.float32),
         _c(unit_mask, np.uint8)]
    rc = lib().oracle_cascade_levels(
        B, num_qo_heads, num_kv_heads, head_dim, page_size, DTYPE_CODE[q_dtype],
        DTYPE_CODE[kv_dtype], _ptr(a[0]), _ptr(a[1]), _ptr(a[2]), nl, _ptr(ng_a),
        ctypes.cast(cp["qo"], ctypes.c_void_p), ctypes.cast(cp["ip"], ctypes.c_void_p),
        ctypes.cast(cp["ix"], ctypes.c_void_p), ctypes.cast(cp["la"], ctypes.c_void_p),
        _ptr(a[3]), _ptr(a[4]), _ptr(a[5]), _ptr(a[6]), _ptr(a[7]), float(sm_scale),
        _ptr(a[8]), _ptr(o), _ptr(lse), threads or default_threads(), *_rope_args(rope),
        _hnd(kv_layout))
    del keep
    if rc != 0:
        raise ValueError("oracle_cascade_levels rejected its arguments")
    return o, lse


def append(q, k_pages, v_pages, qo_indptr, kv_indptr, kv_indices, last_page_len, *,
           num_qo_heads, num_kv_heads, head_dim, page_size, q_dtype, kv_dtype,
           sm_scale, causal=True, k_scale=None, v_scale=None, unit_mask=None,
           threads=None, rope=None, kv_layout="NHD"):
    """fp64 batch append attention.  Request r's query tokens
    qo_indptr[r] .. qo_indptr[r+1]-1 are the last ones of its keys: token i of
    n sits at position L - n + i and (causal) attends keys 0 .. L - n + i.
    q is [total_q, Hq, D] storage; returns (o [total_q, Hq, D], lse
    [total_q, Hq]) fp64.  unit_mask selects (request, kv head) items."""
    indptr = _c(kv_indptr, np.int32)
    qo = _c(qo_indptr, np.int32)
    B = len(indptr) - 1
    nq = int(qo[-1]) if len(qo) else 0
    o = np.zeros((nq, num_qo_heads, head_dim), np.float64)
    lse = np.full((nq, num_qo_heads), np.nan, np.float64)
    q, k_pages, v_pages = _c(q), _c(k_pages), _c(v_pages)
    indices, last = _c(kv_indices, np.int32), _c(last_page_len, np.int32)
    ks, vs = _c(k_scale, np.float32), _c(v_scale, np.float32)
    um = _c(unit_mask, np.uint8)
    rc = lib().oracle_append(B, num_qo_heads, num_kv_heads, head_dim, page_size,
                             DTYPE_CODE[q_dtype], DTYPE_CODE[kv_dtype], _ptr(q),
                             _ptr(k_pages), _ptr(v_pages), _ptr(qo), _ptr(indptr),
                             _ptr(indices), _ptr(last), _ptr(ks), _ptr(vs),
                             float(sm_scale), int(bool(causal)), _ptr(um), _ptr(o),
                             _ptr(lse), threads or default_threads(), *_rope_args(rope),
                             _hnd(kv_layout))
    if rc != 0:
        raise ValueError("oracle_append rejected its arguments")
    return o, lse


def cascade(q, k_pages, v_pages, prefix_qo_indptr, prefix_kv_indptr,
            prefix_kv_indices, prefix_last_page_len, kv_indptr, kv_indices,
            last_page_len, *, num_qo_heads, num_kv_heads, head_dim, page_size,
            q_dtype, kv_dtype, sm_scale, k_scale=None, v_scale=None,
            unit_mask=None, threads=None, rope=None, kv_layout="NHD"):
    """fp64 cascade decode: shared prefix of each request group ++ own pages
    (with rope: prefix tokens at positions 0.., own tokens after them)."""
    indptr = _c(kv_indptr, np.int32)
    B = len(indptr) - 1
    qo_ip = _c(prefix_qo_indptr, np.int32)
    G = len(qo_ip) - 1
    o = np.zeros((B, num_qo_heads, head_dim), np.float64)
    lse = np.full((B, num_qo_heads), np.nan, np.float64)
    arrs = [_c(q), _c(k_pages), _c(v_pages), qo_ip, _c(prefix_kv_indptr, np.int32),
            _c(prefix_kv_indices, np.int32), _c(prefix_last_page_len, np.int32),
            indptr, _c(kv_indices, np.int32), _c(last_page_len, np.int32),
            _c(k_scale, np.float32), _c(v_scale, np.float32), _c(unit_mask, np.uint8)]
    (qa, ka, va, qoa, pia, pxa, pla, ia, xa, la, ksa, vsa, uma) = arrs
    rc = lib().oracle_cascade(B, num_qo_heads, num_kv_heads, head_dim, page_size,
                              DTYPE_CODE[q_dtype], DTYPE_CODE[kv_dtype], _ptr(qa),
                              _ptr(ka), _ptr(va), G, _ptr(qoa), _ptr(pia),
                              _ptr(pxa), _ptr(pla), _ptr(ia), _ptr(xa), _ptr(la),
                              _ptr(ksa), _ptr(vsa), float(sm_scale), _ptr(uma),
                              _ptr(o), _ptr(lse), threads or default_threads(),
                              *_rope_args(rope), _hnd(kv_layout))
    if rc != 0:
        raise ValueError("oracle_cascade rejected its arguments")
    return o, lse


def merge(o_states, lse_states, v_dtype="f64"):
    """Merge attention states over disjoint key sets.
    o_states: [n_states, n_rows, D] raw storage of v_dtype; lse_states:
    [n_states, n_rows] float32/float64 (natural log).  Returns fp64 (o, lse)."""
    o_states = _c(o_states)
    lse_states = _c(lse_states)
    n_states, n_rows, D = o_states.shape
    s_dtype = F64 if lse_states.dtype == np.float64 else F32
    if s_dtype == F32:
        lse_states = _c(lse_states, np.float32)
    o = np.zeros((n_rows, D), np.float64)
    lse = np.zeros(n_rows, np.float64)
    lib().oracle_merge(n_states, n_rows, D, DTYPE_CODE[v_dtype], _ptr(o_states),
                       s_dtype, _ptr(lse_states), _ptr(o), _ptr(lse))
    return o, lse
