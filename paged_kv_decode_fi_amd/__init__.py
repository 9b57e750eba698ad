"""Python binding of libfi_decode.so (argument marshalling only).

Every step of the decode path runs in the HIP kernels behind the C ABI
declared in include/fi_decode.h; torch only provides device memory and the
current stream.  There is no fallback: if the shared library is missing,
importing this package raises.

    plan = Plan(kv_indptr_host, last_page_len_host, num_qo_heads=32,
                num_kv_heads=8, page_size=16, q_dtype="f16", kv_dtype="f16")
    o, lse = plan.run(q, k_pages, v_pages, kv_indptr, kv_indices, last_page_len)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfi_decode.so")

DTYPES = {"f16": 0, "bf16": 1, "e4m3": 2, "f32": 3}
STATUS = {0: "FI_OK", 1: "FI_ERR_INVALID_ARG", 2: "FI_ERR_UNSUPPORTED",
          3: "FI_ERR_WORKSPACE_TOO_SMALL", 4: "FI_ERR_HIP"}
EXPORTS = ("fi_plan", "fi_plan_destroy", "fi_plan_get_stats", "fi_decode_run",
           "fi_cascade_decode", "fi_merge_states", "fi_status_string",
           "fi_last_error", "fi_debug_plan_tiles", "fi_debug_gather",
           "fi_debug_stream_read", "fi_debug_run_stage", "fi_append_run",
           "fi_cascade_decode_levels", "fi_debug_record_walk", "fi_decode_noalloc")


class FiError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class CascadeLevel(ctypes.Structure):
    _fields_ = [("num_groups", ctypes.c_int32), ("qo_indptr", ctypes.c_void_p),
                ("kv_indptr", ctypes.c_void_p), ("last_page_len", ctypes.c_void_p)]


TUNING_FIELDS = ("heads_per_tile", "waves_per_cu", "chunk_min", "prefix_waves",
                 "prefix_tiles_per_cu", "prefix_chunk_min", "cascade_fold", "fold_max_suffix",
                 "append_tiles_pct", "append_chunk_min", "decode_depth", "prefix_split_p",
                 "rope_split_k", "score_path")


class Tuning(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in TUNING_FIELDS]


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_qo_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("q_dtype", ctypes.c_int),
                ("kv_dtype", ctypes.c_int), ("kv_indptr", ctypes.c_void_p),
                ("last_page_len", ctypes.c_void_p),
                ("num_prefix_groups", ctypes.c_int32),
                ("prefix_qo_indptr", ctypes.c_void_p),
                ("prefix_kv_indptr", ctypes.c_void_p),
                ("prefix_last_page_len", ctypes.c_void_p),
                ("chunk_tokens", ctypes.c_int32), ("pos_encoding", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rope_scale", ctypes.c_float),
                ("qo_indptr", ctypes.c_void_p), ("causal", ctypes.c_int32),
                ("kv_layout", ctypes.c_int32), ("num_cascade_levels", ctypes.c_int32),
                ("cascade_levels", ctypes.c_void_p), ("tuning", ctypes.c_void_p)]


class PlanStats(ctypes.Structure):
    _fields_ = [("num_tiles", ctypes.c_int64), ("num_prefix_tiles", ctypes.c_int64),
                ("num_partials", ctypes.c_int64), ("num_merge_units", ctypes.c_int64),
                ("chunk_tokens", ctypes.c_int32), ("prefix_chunk_tokens", ctypes.c_int32),
                ("heads_per_tile", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t), ("num_folded", ctypes.c_int64),
                ("prefix_split_p", ctypes.c_uint32), ("staging_buffers", ctypes.c_int32),
                ("rope_single", ctypes.c_int32), ("valu_heads", ctypes.c_int32),
                ("decode_waves_per_cu", ctypes.c_int32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7).
    # Load it first so this library binds to that one runtime: device
    # pointers and hipStream_t handles from torch are then valid here.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built: run `python -m paged_kv_decode_fi_amd.build` "
            "(there is no non-HIP fallback)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    F = ctypes.c_float
    L.fi_plan.restype = ctypes.c_int
    L.fi_plan.argtypes = [ctypes.POINTER(Problem), I32, P, SZ, ctypes.POINTER(SZ), P,
                          ctypes.POINTER(P)]
    L.fi_plan_destroy.restype = ctypes.c_int
    L.fi_plan_destroy.argtypes = [P]
    L.fi_plan_get_stats.restype = ctypes.c_int
    L.fi_plan_get_stats.argtypes = [P, ctypes.POINTER(PlanStats)]
    L.fi_decode_run.restype = ctypes.c_int
    L.fi_decode_run.argtypes = [P, P, P, P, P, P, P, P, P, F, P, P, P]
    L.fi_cascade_decode.restype = ctypes.c_int
    L.fi_append_run.restype = ctypes.c_int
    L.fi_append_run.argtypes = [P, P, P, P, P, P, P, P, P, F, P, P, P]
    L.fi_cascade_decode_levels.restype = ctypes.c_int
    L.fi_cascade_decode_levels.argtypes = [P, P, P, P, I32, P, P, P, P, P, P, P, P, F, P, P, P]
    L.fi_cascade_decode.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, F, P, P, P]
    L.fi_debug_run_stage.restype = ctypes.c_int
    L.fi_debug_run_stage.argtypes = [P, I32, P, P, P, P, P, P, P, P, P, P, P, F, P, P, P]
    L.fi_decode_noalloc.restype = ctypes.c_int
    L.fi_decode_noalloc.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P, F, P, P, P]
    L.fi_debug_record_walk.restype = ctypes.c_int
    L.fi_debug_record_walk.argtypes = [P, I32, P, P, P, P, P, P, P, P, P, P, P, F, P, P, P, P,
                                       P]
    L.fi_merge_states.restype = ctypes.c_int
    L.fi_merge_states.argtypes = [I32, ctypes.POINTER(P), ctypes.POINTER(P), I64, I32,
                                  ctypes.c_int, P, P, ctypes.c_int, P]
    L.fi_status_string.restype = ctypes.c_char_p
    L.fi_status_string.argtypes = [ctypes.c_int]
    L.fi_last_error.restype = ctypes.c_char_p
    L.fi_last_error.argtypes = []
    L.fi_debug_plan_tiles.restype = ctypes.c_int
    L.fi_debug_plan_tiles.argtypes = [ctypes.POINTER(Problem), I32, P, I64,
                                      ctypes.POINTER(I64)]
    L.fi_debug_gather.restype = ctypes.c_int
    L.fi_debug_gather.argtypes = [I32, I32, P, P, P, P, P, P]
    L.fi_debug_stream_read.restype = ctypes.c_int
    L.fi_debug_stream_read.argtypes = [P, SZ, P, I32, P]
    return L


_LIB = None


def _get_lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use, so that the build module can
    be imported before the library exists)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def __getattr__(name):
    if name == "lib":
        return _get_lib()
    raise AttributeError(name)


def _check(status: int):
    if status != 0:
        raise FiError(status, _get_lib().fi_last_error().decode(errors="replace"))


def _host_i32(a) -> np.ndarray:
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(t, name: str = "tensor", dtype=None) -> Optional[int]:
    """Device pointer of a contiguous GPU torch tensor (of `dtype` when
    given), or None.  A host tensor would reach the kernels as a host
    address, so it is rejected here."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _tables(kv_indptr, kv_indices, last_page_len, prefix=None):
    """Device pointers of the page tables (int32 GPU tensors)."""
    import torch
    names = ("kv_indptr", "kv_indices", "last_page_len")
    out = [_ptr(t, n, torch.int32) for t, n in zip((kv_indptr, kv_indices, last_page_len), names)]
    if prefix is not None:
        out = [_ptr(t, "prefix_" + n, torch.int32) for t, n in zip(prefix, names)] + out
    return out


def _scales(k_scale, v_scale):
    import torch
    return _ptr(k_scale, "k_scale", torch.float32), _ptr(v_scale, "v_scale", torch.float32)


def _np_ptr(a) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


POS_ENCODINGS = {"none": 0, "rope_llama": 1}
KV_LAYOUTS = {"paged": 0, "ragged": 1, "paged_hnd": 2}


def _problem(batch, Hq, Hkv, D, ps, q_dtype, kv_dtype, indptr, last, prefix, chunk,
             pos_encoding="none", rope_theta=0.0, rope_scale=0.0, qo_indptr=None, causal=True,
             kv_layout="paged", levels=None, tuning=None):
    pr = Problem()
    lv_keep = []
    if tuning:
        bad = set(tuning) - set(TUNING_FIELDS)
        if bad:
            raise ValueError(f"unknown tuning fields {sorted(bad)}")
        tu = Tuning(**{k: int(v) for k, v in tuning.items()})
        pr.tuning = ctypes.cast(ctypes.pointer(tu), ctypes.c_void_p)
        lv_keep.append(tu)
    if levels:
        arr = (CascadeLevel * len(levels))()
        for i, (qo, ip, la) in enumerate(levels):
            qo, ip, la = _host_i32(qo), _host_i32(ip), _host_i32(la)
            arr[i].num_groups = len(qo) - 1
            arr[i].qo_indptr, arr[i].kv_indptr = _np_ptr(qo), _np_ptr(ip)
            arr[i].last_page_len = _np_ptr(la) if la is not None else None
            lv_keep += [qo, ip, la]
        pr.num_cascade_levels = len(levels)
        pr.cascade_levels = ctypes.cast(arr, ctypes.c_void_p)
        lv_keep.append(arr)
    pr.kv_layout = KV_LAYOUTS[kv_layout]
    if qo_indptr is not None:
        qo_indptr = _host_i32(qo_indptr)
        pr.qo_indptr, pr.causal = _np_ptr(qo_indptr), int(bool(causal))
    pr.pos_encoding = POS_ENCODINGS[pos_encoding]
    pr.rope_theta, pr.rope_scale = rope_theta, rope_scale
    pr.batch, pr.num_qo_heads, pr.num_kv_heads = batch, Hq, Hkv
    pr.head_dim, pr.page_size = D, ps
    pr.q_dtype, pr.kv_dtype = DTYPES[q_dtype], DTYPES[kv_dtype]
    pr.kv_indptr = _np_ptr(indptr)
    pr.last_page_len = _np_ptr(last) if last is not None else None
    pr.chunk_tokens = chunk
    keep = [indptr, last, qo_indptr] + lv_keep
    if prefix is not None:
        qo, pip, plast = (_host_i32(x) for x in prefix)   # plast None when ragged
        pr.num_prefix_groups = len(qo) - 1
        pr.prefix_qo_indptr, pr.prefix_kv_indptr = _np_ptr(qo), _np_ptr(pip)
        pr.prefix_last_page_len = _np_ptr(plast)
        keep += [qo, pip, plast]
    return pr, keep


def debug_plan_tiles(kv_indptr, last_page_len, *, num_qo_heads, num_kv_heads,
                     page_size, head_dim=128, q_dtype="f16", kv_dtype="f16",
                     prefix=None, num_cus=256, chunk_tokens=0,
                     pos_encoding="none", qo_indptr=None, causal=True,
                     kv_layout="paged", levels=None, tuning=None) -> np.ndarray:
    """Host-only: the plan's work list as an int32 [n, 8] array (request,
    kv_head0, t0, t1, slot, kind, row0, row1)."""
    indptr, last = _host_i32(kv_indptr), _host_i32(last_page_len)
    pr, keep = _problem(len(indptr) - 1, num_qo_heads, num_kv_heads, head_dim,
                        page_size, q_dtype, kv_dtype, indptr, last, prefix, chunk_tokens,
                        pos_encoding, qo_indptr=qo_indptr, causal=causal,
                        kv_layout=kv_layout, levels=levels, tuning=tuning)
    n = ctypes.c_int64(0)
    _check(_get_lib().fi_debug_plan_tiles(ctypes.byref(pr), num_cus, None, 0, ctypes.byref(n)))
    out = np.zeros((max(n.value, 1), 8), np.int32)
    _check(_get_lib().fi_debug_plan_tiles(ctypes.byref(pr), num_cus, out.ctypes.data,
                                   n.value, ctypes.byref(n)))
    del keep
    return out[:n.value]


class Plan:
    """Plan stage: host lengths -> work list in a device workspace.

    kv_indptr / last_page_len are the HOST copies of the page table (numpy or
    torch CPU).  prefix = (prefix_qo_indptr, prefix_kv_indptr,
    prefix_last_page_len) host arrays for cascade decoding.  head_dim: 64,
    128 or 256.  pos_encoding = "rope_llama" applies LLaMA-style RoPE to q
    and the keys on the fly, in decode, cascade and append plans
    (rope_theta / rope_scale <= 0: 1e4 / 1).  qo_indptr (host [B+1]) makes an
    append plan: request r's query tokens qo_indptr[r] .. qo_indptr[r+1]-1
    are the last ones of its keys (causal mask unless causal=False); run it
    with Plan.append_run.  kv_layout="ragged": each request's tokens are
    contiguous rows kv_indptr[r] .. kv_indptr[r+1]-1 of K and V (page_size 1,
    last_page_len and kv_indices may be None); "paged_hnd": head-major pages
    [num_pages][Hkv][page_size][D].  levels = [(qo_indptr, kv_indptr,
    last_page_len), ...] host tables of several shared cascade levels,
    outermost first (in place of prefix); run with Plan.cascade_run_levels.
    tuning: optional dict of fi_tuning fields (how the work is cut, for
    measurement; never what is computed)."""

    def __init__(self, kv_indptr, last_page_len, *, num_qo_heads, num_kv_heads,
                 page_size, head_dim=128, q_dtype="f16", kv_dtype="f16",
                 prefix=None, num_cus=0, chunk_tokens=0, device=None, stream=None,
                 pos_encoding="none", rope_theta=0.0, rope_scale=0.0, qo_indptr=None,
                 causal=True, kv_layout="paged", levels=None, tuning=None):
        import torch
        self.indptr = _host_i32(kv_indptr)
        self.last = _host_i32(last_page_len)
        self.batch = len(self.indptr) - 1
        self.num_qo_heads, self.num_kv_heads = num_qo_heads, num_kv_heads
        self.head_dim, self.page_size = head_dim, page_size
        self.q_dtype, self.kv_dtype = q_dtype, kv_dtype
        self.cascade = prefix is not None or bool(levels)
        self.num_levels = len(levels) if levels else (1 if prefix is not None else 0)
        self.pos_encoding = pos_encoding
        self.append = qo_indptr is not None
        self.qo_indptr = _host_i32(qo_indptr) if self.append else None
        # rows of q / o / lse: query tokens (append) or requests
        self.num_rows = int(self.qo_indptr[-1]) if self.append else self.batch
        pr, keep = _problem(self.batch, num_qo_heads, num_kv_heads, head_dim,
                            page_size, q_dtype, kv_dtype, self.indptr, self.last,
                            prefix, chunk_tokens, pos_encoding, rope_theta, rope_scale,
                            self.qo_indptr, causal, kv_layout, levels, tuning)
        need = ctypes.c_size_t(0)
        _check(_get_lib().fi_plan(ctypes.byref(pr), num_cus, None, 0, ctypes.byref(need), None,
                           None))
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.workspace = torch.empty(max(need.value, 256), dtype=torch.uint8, device=dev)
        self._stream = stream
        h = ctypes.c_void_p(None)
        _check(_get_lib().fi_plan(ctypes.byref(pr), num_cus, self.workspace.data_ptr(),
                           self.workspace.numel(), ctypes.byref(need), _stream(stream),
                           ctypes.byref(h)))
        self.handle = h
        del keep
        st = PlanStats()
        _check(_get_lib().fi_plan_get_stats(self.handle, ctypes.byref(st)))
        self.stats = st.as_dict()

    # ---- run stage ---------------------------------------------------------
    def _outputs(self, q, o, lse):
        import torch
        if o is None:
            o = torch.empty_like(q)
        elif o.dtype != q.dtype or o.shape != q.shape:
            raise ValueError(f"o must be {q.dtype} {tuple(q.shape)}, got {o.dtype} "
                             f"{tuple(o.shape)}")
        if lse is None:
            lse = torch.empty((self.num_rows, self.num_qo_heads), dtype=torch.float32,
                              device=q.device)
        elif lse.dtype != torch.float32 or tuple(lse.shape) != (self.num_rows, self.num_qo_heads):
            raise ValueError(f"lse must be float32 [{self.num_rows}, {self.num_qo_heads}]")
        return o, lse

    def _check_q(self, q):
        import torch
        want = {"f16": torch.float16, "bf16": torch.bfloat16}[self.q_dtype]
        if q.dtype != want or tuple(q.shape) != (self.num_rows, self.num_qo_heads,
                                                 self.head_dim):
            raise ValueError(f"q must be {want} [{self.num_rows}, {self.num_qo_heads}, "
                             f"{self.head_dim}], got {q.dtype} {tuple(q.shape)}")

    def _check_pool(self, k_pages, v_pages):
        es = 1 if self.kv_dtype == "e4m3" else 2
        for t in (k_pages, v_pages):
            row = self.page_size * self.num_kv_heads * self.head_dim * es
            if t.numel() * t.element_size() % row:
                raise ValueError("page pool size is not a whole number of pages")

    def run(self, q, k_pages, v_pages, kv_indptr, kv_indices, last_page_len,
            k_scale=None, v_scale=None, sm_scale: float = 0.0, o=None, lse=None,
            stream=None):
        """Batch paged decode.  Device tensors; returns (o, lse)."""
        if self.cascade or self.append:
            raise ValueError("cascade / append plan: use Plan.cascade_run / Plan.append_run")
        self._check_q(q)
        self._check_pool(k_pages, v_pages)
        o, lse = self._outputs(q, o, lse)
        _check(_get_lib().fi_decode_run(self.handle, _ptr(q, "q"), _ptr(k_pages, "k_pages"),
                                        _ptr(v_pages, "v_pages"),
                                        *_tables(kv_indptr, kv_indices, last_page_len),
                                        *_scales(k_scale, v_scale), float(sm_scale),
                                        _ptr(o, "o"), _ptr(lse, "lse"), _stream(stream)))
        return o, lse

    def append_run(self, q, k_pages, v_pages, kv_indptr, kv_indices, last_page_len,
                   k_scale=None, v_scale=None, sm_scale: float = 0.0, o=None, lse=None,
                   stream=None):
        """Batch append attention: q [total_q, Hq, D] device tensor (query
        tokens of every request, in qo_indptr order).  Returns (o, lse)."""
        if not self.append:
            raise ValueError("plan is not an append plan (make it with qo_indptr)")
        self._check_q(q)
        self._check_pool(k_pages, v_pages)
        o, lse = self._outputs(q, o, lse)
        _check(_get_lib().fi_append_run(self.handle, _ptr(q, "q"), _ptr(k_pages, "k_pages"),
                                        _ptr(v_pages, "v_pages"),
                                        *_tables(kv_indptr, kv_indices, last_page_len),
                                        *_scales(k_scale, v_scale), float(sm_scale),
                                        _ptr(o, "o"), _ptr(lse, "lse"), _stream(stream)))
        return o, lse

    def cascade_run(self, q, k_pages, v_pages, prefix_kv_indptr, prefix_kv_indices,
                    prefix_last_page_len, kv_indptr, kv_indices, last_page_len,
                    k_scale=None, v_scale=None, sm_scale: float = 0.0, o=None, lse=None,
                    stream=None):
        """Cascade (shared prefix + own pages) decode.  Returns (o, lse)."""
        if not self.cascade:
            raise ValueError("plan has no cascade level: use Plan.run")
        self._check_q(q)
        self._check_pool(k_pages, v_pages)
        o, lse = self._outputs(q, o, lse)
        _check(_get_lib().fi_cascade_decode(
            self.handle, _ptr(q, "q"), _ptr(k_pages, "k_pages"), _ptr(v_pages, "v_pages"),
            *_tables(kv_indptr, kv_indices, last_page_len,
                     (prefix_kv_indptr, prefix_kv_indices, prefix_last_page_len)),
            *_scales(k_scale, v_scale), float(sm_scale), _ptr(o, "o"), _ptr(lse, "lse"),
            _stream(stream)))
        return o, lse

    def cascade_run_levels(self, q, k_pages, v_pages, level_tables, kv_indptr, kv_indices,
                           last_page_len, k_scale=None, v_scale=None, sm_scale: float = 0.0,
                           o=None, lse=None, stream=None):
        """Cascade decode over several shared levels: level_tables =
        [(kv_indptr, kv_indices, last_page_len), ...] device tensors,
        outermost first.  Returns (o, lse)."""
        import torch
        if len(level_tables) != self.num_levels:
            raise ValueError(f"the plan has {self.num_levels} levels")
        self._check_q(q)
        self._check_pool(k_pages, v_pages)
        o, lse = self._outputs(q, o, lse)
        n = max(len(level_tables), 1)
        arrs = [(ctypes.c_void_p * n)() for _ in range(3)]
        for i, (ip, ix, la) in enumerate(level_tables):
            arrs[0][i] = _ptr(ip, f"level {i} kv_indptr", torch.int32)
            arrs[1][i] = _ptr(ix, f"level {i} kv_indices", torch.int32)
            arrs[2][i] = _ptr(la, f"level {i} last_page_len", torch.int32)
        _check(_get_lib().fi_cascade_decode_levels(
            self.handle, _ptr(q, "q"), _ptr(k_pages, "k_pages"), _ptr(v_pages, "v_pages"),
            len(level_tables), *(ctypes.cast(a, ctypes.c_void_p) for a in arrs),
            *_tables(kv_indptr, kv_indices, last_page_len), *_scales(k_scale, v_scale),
            float(sm_scale), _ptr(o, "o"), _ptr(lse, "lse"), _stream(stream)))
        return o, lse

    def run_stage(self, stage, q, k_pages, v_pages, kv_indptr, kv_indices, last_page_len,
                  prefix_kv_indptr=None, prefix_kv_indices=None, prefix_last_page_len=None,
                  k_scale=None, v_scale=None, sm_scale: float = 0.0, o=None, lse=None,
                  stream=None):
        """Test / timing hook: ONE kernel of the planned run (stage 0 = decode
        kernel, 1 = cascade prefix kernel, 2 = merge of split states);
        stages 1, 0, 2 in order are the full run."""
        self._check_q(q)
        self._check_pool(k_pages, v_pages)
        o, lse = self._outputs(q, o, lse)
        _check(_get_lib().fi_debug_run_stage(
            self.handle, int(stage), _ptr(q, "q"), _ptr(k_pages, "k_pages"),
            _ptr(v_pages, "v_pages"),
            *_tables(kv_indptr, kv_indices, last_page_len,
                     (prefix_kv_indptr, prefix_kv_indices, prefix_last_page_len)),
            *_scales(k_scale, v_scale), float(sm_scale), _ptr(o, "o"), _ptr(lse, "lse"),
            _stream(stream)))
        return o, lse

    def record_walk(self, stage, rec, rec_base, q, k_pages, v_pages, kv_indptr, kv_indices,
                    last_page_len, prefix_kv_indptr=None, prefix_kv_indices=None,
                    prefix_last_page_len=None, k_scale=None, v_scale=None,
                    sm_scale: float = 0.0, o=None, lse=None, stream=None):
        """Test hook: ONE kernel of the planned run (stage 0 = decode, 1 =
        multi-row) in its record instance, which also writes the K-pool byte
        offset of every K vector it loads into rec (device int64) at
        ((rec_base[list] + token) * Hkv + kv head) * (row bytes / 16) + chunk."""
        import torch
        self._check_q(q)
        self._check_pool(k_pages, v_pages)
        o, lse = self._outputs(q, o, lse)
        _check(_get_lib().fi_debug_record_walk(
            self.handle, int(stage), _ptr(q, "q"), _ptr(k_pages, "k_pages"),
            _ptr(v_pages, "v_pages"),
            *_tables(kv_indptr, kv_indices, last_page_len,
                     (prefix_kv_indptr, prefix_kv_indices, prefix_last_page_len)),
            *_scales(k_scale, v_scale), float(sm_scale), _ptr(o, "o"), _ptr(lse, "lse"),
            _ptr(rec, "rec", torch.int64), _ptr(rec_base, "rec_base", torch.int64),
            _stream(stream)))
        return o, lse

    def destroy(self):
        if getattr(self, "handle", None):
            import torch
            torch.cuda.synchronize(self.workspace.device)
            _get_lib().fi_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def decode_noalloc(q, k_pages, v_pages, kv_indptr, kv_indices, last_page_len, *,
                   kv_indptr_host, last_page_len_host, num_qo_heads, num_kv_heads,
                   page_size, head_dim=128, q_dtype="f16", kv_dtype="f16", k_scale=None,
                   v_scale=None, sm_scale: float = 0.0, chunk_tokens=0, kv_layout="paged",
                   tuning=None, o=None, lse=None, stream=None):
    """Plain decode through fi_decode_noalloc (no workspace: the work list and
    partial states live in the library's static device array).  Host copies
    of kv_indptr / last_page_len decide the split; the device tables are
    read by the kernels.  Returns (o, lse)."""
    import torch
    indptr, last = _host_i32(kv_indptr_host), _host_i32(last_page_len_host)
    batch = len(indptr) - 1
    pr, keep = _problem(batch, num_qo_heads, num_kv_heads, head_dim, page_size, q_dtype,
                        kv_dtype, indptr, last, None, chunk_tokens, kv_layout=kv_layout,
                        tuning=tuning)
    want = {"f16": torch.float16, "bf16": torch.bfloat16}[q_dtype]
    if q.dtype != want or tuple(q.shape) != (batch, num_qo_heads, head_dim):
        raise ValueError(f"q must be {want} [{batch}, {num_qo_heads}, {head_dim}]")
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((batch, num_qo_heads), dtype=torch.float32, device=q.device)
    _check(_get_lib().fi_decode_noalloc(
        ctypes.byref(pr), _ptr(q, "q"), _ptr(k_pages, "k_pages"), _ptr(v_pages, "v_pages"),
        *_tables(kv_indptr, kv_indices, last_page_len), *_scales(k_scale, v_scale),
        float(sm_scale), _ptr(o, "o"), _ptr(lse, "lse", torch.float32), _stream(stream)))
    del keep
    return o, lse


def merge_states(v_states: Sequence, s_states: Sequence, out_dtype=None, v_out=None,
                 s_out=None, stream=None):
    """Merge attention states over disjoint key sets.  Each v [..., D] (f16,
    bf16 or f32 device tensor), each s [...] fp32 natural-log lse with the
    same leading shape.  Returns (v, s)."""
    import torch
    tdt = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}
    v0 = v_states[0]
    rows = v0.numel() // v0.shape[-1]
    D = v0.shape[-1]
    for v, s in zip(v_states, s_states):
        if v.shape != v0.shape or v.dtype != v0.dtype or s.numel() != rows or \
                s.dtype != torch.float32:
            raise ValueError("states must share shape/dtype; lse must be fp32 [rows]")
    odt = v0.dtype if out_dtype is None else out_dtype
    if v_out is None:
        v_out = torch.empty(v0.shape, dtype=odt, device=v0.device)
    if s_out is None:
        s_out = torch.empty(v0.shape[:-1], dtype=torch.float32, device=v0.device)
    n = len(v_states)
    vp = (ctypes.c_void_p * n)(*[_ptr(v) for v in v_states])
    sp = (ctypes.c_void_p * n)(*[_ptr(s) for s in s_states])
    _check(_get_lib().fi_merge_states(n, vp, sp, rows, D, DTYPES[tdt[v0.dtype]], _ptr(v_out),
                               _ptr(s_out), DTYPES[tdt[odt]], _stream(stream)))
    return v_out, s_out


def debug_gather(page_size, kv_indptr, kv_indices, last_page_len, token_indptr,
                 stream=None):
    """Device page walk of every logical token (request-major) -> int64 slots."""
    import torch
    total = int(token_indptr[-1].item())
    out = torch.empty(max(total, 1), dtype=torch.int64, device=kv_indptr.device)
    _check(_get_lib().fi_debug_gather(len(kv_indptr) - 1, page_size, _ptr(kv_indptr),
                               _ptr(kv_indices), _ptr(last_page_len), _ptr(token_indptr),
                               _ptr(out), _stream(stream)))
    return out[:total]


def debug_stream_read(src, sink, num_blocks, stream=None):
    """Plain streaming read of a device tensor (bandwidth ceiling probe)."""
    nbytes = src.numel() * src.element_size()
    _check(_get_lib().fi_debug_stream_read(_ptr(src), nbytes - nbytes % 16, _ptr(sink),
                                    num_blocks, _stream(stream)))

