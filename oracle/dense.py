"""NumPy brute-force attention over a DENSE, already-decoded K/V (test-only).

An implementation independent of ``oracle.c``: no page table, no two-pass
max subtraction (plain exp of the raw scores, valid while scores are small),
numpy's own dtype conversions.  It pins the C oracle on tiny inputs.

Follows the single-request decode contract of the hysenlabs review
("Installing FlashInfer and running a first decode"): q is
[num_qo_heads, head_dim], k and v are [kv_len, num_kv_heads, head_dim]; q
head j reads kv head j // (num_qo_heads // num_kv_heads) (head-query fusion
for grouped-query attention, FlashInfer README "core features" item 3).
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the top half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def ref_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """q [Hq, D], k/v [L, Hkv, D] (float64) -> (o [Hq, D], lse [Hq]).

    o = sum_t exp(x_t) v_t / sum_t exp(x_t), lse = ln sum_t exp(x_t) with
    x_t = sm_scale * q . k_t.  No max subtraction: callers keep |x| small.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Hq, D = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    o = np.zeros((Hq, D))
    lse = np.full(Hq, -np.inf)
    if L == 0:
        return o, lse
    for j in range(Hq):
        h = j // G
        x = sm_scale * (k[:, h, :] @ q[j])          # [L]
        w = np.exp(x)
        o[j] = (w[:, None] * v[:, h, :]).sum(0) / w.sum()
        lse[j] = np.log(w.sum())
    return o, lse


def ref_dense_append(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float,
                     causal: bool = True):
    """Append attention over a dense K/V: q [n, Hq, D] are the last n of the
    L tokens of k/v [L, Hkv, D] (float64).  With the causal mask, query i
    sees keys 0 .. L - n + i (a lower-triangular mask aligned to the bottom
    right of the n x L score matrix).  Returns (o [n, Hq, D], lse [n, Hq]).
    No max subtraction: callers keep |x| small."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, Hq, D = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    allowed = np.ones((n, L), bool)
    if causal:
        allowed = np.tril(allowed, k=L - n)
    o = np.zeros((n, Hq, D))
    lse = np.full((n, Hq), -np.inf)
    for j in range(Hq):
        h = j // G
        x = sm_scale * (q[:, j, :] @ k[:, h, :].T)        # [n, L]
        w = np.where(allowed, np.exp(x), 0.0)
        o[:, j] = (w @ v[:, h, :]) / w.sum(1, keepdims=True)
        lse[:, j] = np.log(w.sum(1))
    return o, lse
