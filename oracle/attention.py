"""fp64 decode attention: one query token per sequence, no mask.

Follows mlxcel issue #2171 ("refactor: one KV storage abstraction with dense
and paged backends"), sections "Proposed Solution" and "Implementation Notes":
attend(q, k, v, scale, mask) takes the paged single-token route only when one
query token arrives with no mask, so the token sees every visible key of its
sequence.  Paging must not change any value (mlxcel #235, "Acceptance
criteria": parity suites stay byte-identical), so this oracle is the plain
definition over the sequence's dense K/V and knows nothing of slabs:

    for each sequence b and query head h, with kv head g = h // (n_q / n_kv):
        s_t = scale * <q[b, h], K_b[t, g]>            t = 0 .. len_b - 1
        w_t = exp(s_t - max_t s_t)
        o[b, h] = sum_t w_t V_b[t, g] / sum_t w_t

An empty sequence (len_b = 0) gives a zero output.  Inputs are fp16 or bf16
bit patterns; they are widened exactly and everything after that is fp64.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """fp16/bf16 bit patterns (uint16) -> float64, exactly."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        # a bf16 value is the top half of the float32 with the same bits
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def attend_one(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of query rows q [G, D] over keys k [n, D], values v [n, Dv]."""
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    s = scale * (k @ q.T)                      # [n, G]
    w = np.exp(s - s.max(axis=0, keepdims=True))
    return (w.T @ v) / w.sum(axis=0)[:, None]  # [G, Dv]


def decode_attention(q: np.ndarray, ks: Sequence[np.ndarray], vs: Sequence[np.ndarray],
                     scale: float) -> np.ndarray:
    """q: float64 [B, n_q, D]; ks[b], vs[b]: float64 [len_b, n_kv, D] -> [B, n_q, D]."""
    B, n_q, D = q.shape
    out = np.zeros((B, n_q, vs[0].shape[-1] if B else D), dtype=np.float64)
    for b in range(B):
        n_kv = ks[b].shape[1]
        G = n_q // n_kv
        for g in range(n_kv):
            heads = slice(g * G, (g + 1) * G)
            out[b, heads] = attend_one(q[b, heads], ks[b][:, g, :], vs[b][:, g, :], scale)
    return out


def decode_attention_bits(q_bits: np.ndarray, k_bits: Sequence[np.ndarray],
                          v_bits: Sequence[np.ndarray], dtype: str, scale: float) -> np.ndarray:
    """decode_attention over fp16/bf16 bit-pattern inputs."""
    return decode_attention(widen(q_bits, dtype), [widen(k, dtype) for k in k_bits],
                            [widen(v, dtype) for v in v_bits], scale)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to fp16/bf16 (nearest even); returned as float64.

    The decode output is stored in the query dtype, rounded once at the end."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "fp16":
        return x.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        m, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
        return np.ldexp(np.rint(m * 256.0), e - 8)  # 8 significant bits
    raise ValueError(dtype)
