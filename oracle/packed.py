"""Packed KV formats: signed Hadamard rotation + token-local affine groups.

Follows mlx-swift-lm PR #142 ("Add packed paged KV formats with bounded
workspace admission"), section "Summary" and the "After" flowchart:

* formats K8/V8, K8/V4, K4/V4 (bits of the K codes / bits of the V codes);
* token-local affine groups with FP32 scale/offset metadata -- here groups of
  32 consecutive values along head_dim of one token-head vector (the packed
  workload), or of 64 (the reading under which K4/V4 costs the five effective
  bits per value and the 3.2x reduction the Summary states);
* a fixed signed Hadamard basis for Q and K: K is rotated before it is
  quantised and the query gets the same rotation, so q'.k' = q.k; V is stored
  unrotated, so the attention output needs no inverse rotation;
* fresh K/V are quantised once, at write time, and attention reads the packed
  pages directly (dequantising values as it reads them).

Readings where the page is silent (each listed with its reason in the design
notes of the repository):

* rotation  x' = H (sigma * x) / sqrt(D), H the Sylvester Hadamard matrix
  (H_1 = [1], H_2n = [[H, H], [H, -H]]), sigma the fixed +-1 vector.  The
  stored K is computed in fp32 by the fast Walsh-Hadamard butterfly network,
  stages h = 1, 2, 4, ..., D/2, each pair (a, b) -> (a + b, a - b), followed
  by one multiply with fp32(1/sqrt(D)) (exact for D = 64, 256);
* affine form: per group, mn = min, mx = max, scale = (mx - mn) / (2^bits - 1),
  offset = mn, code = clamp(rint((x - mn) / scale), 0, 2^bits - 1) with
  round-half-even; all of it fp32; a constant group (scale == 0) gets code 0;
  dequantised value = code * scale + offset;
* record layout of one token-head: the codes (one byte each at 8 bits; two per
  byte at 4 bits, element 2i in the low nibble), then per group the fp32
  scale and the fp32 offset, little endian.
"""

from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .attention import decode_attention, widen

GROUP = 32

FORMATS = {"k8v8": (8, 8), "k8v4": (8, 4), "k4v4": (4, 4)}


def sylvester_hadamard(d: int) -> np.ndarray:
    """The d x d Sylvester Hadamard matrix (entries +-1), float64."""
    assert d >= 1 and d & (d - 1) == 0, "head_dim must be a power of two"
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_exact(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """x' = H (sigma * x) / sqrt(D) in float64 with the explicit matrix."""
    d = x.shape[-1]
    h = sylvester_hadamard(d)
    return (np.asarray(x, np.float64) * signs.astype(np.float64)) @ h.T / np.sqrt(d)


def inv_sqrt_f32(d: int) -> np.float32:
    return np.float32(1.0 / np.sqrt(np.float64(d)))


def rotate_fp32(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """The stored rotation: fp32 fast Walsh-Hadamard transform of sigma * x.

    x: float32 [..., D].  Every operation is one correctly rounded fp32 op."""
    y = np.asarray(x, dtype=np.float32) * signs.astype(np.float32)  # exact sign flips
    d = y.shape[-1]
    h = 1
    while h < d:
        z = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = z[..., 0, :]
        b = z[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(y.shape)
        h *= 2
    return (y * inv_sqrt_f32(d)).astype(np.float32)


def quantise(x: np.ndarray, bits: int, group: int = GROUP) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Affine group quantiser over groups of `group` along the last axis (fp32 ops).

    Returns (codes uint8 [..., D], scale float32 [..., D/group], offset float32 [..., D/group])."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    assert d % group == 0
    g = x.reshape(x.shape[:-1] + (d // group, group))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    levels = np.float32((1 << bits) - 1)
    scale = ((mx - mn) / levels).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1), scale).astype(np.float32)
    t = ((g - mn[..., None]) / safe[..., None]).astype(np.float32)
    codes = np.clip(np.rint(t), 0, levels)
    codes = np.where(scale[..., None] == 0, 0, codes).astype(np.uint8)
    return codes.reshape(x.shape), scale, mn.astype(np.float32)


def dequantise(codes: np.ndarray, scale: np.ndarray, offset: np.ndarray) -> np.ndarray:
    """code * scale + offset, float64, per group (D / number of scales values)."""
    d = codes.shape[-1]
    ng = scale.shape[-1]
    c = codes.astype(np.float64).reshape(codes.shape[:-1] + (ng, d // ng))
    x = c * scale.astype(np.float64)[..., None] + offset.astype(np.float64)[..., None]
    return x.reshape(codes.shape)


def record_bytes(head_dim: int, bits: int, group: int = GROUP) -> int:
    """Bytes of one packed token-head record: codes + fp32 (scale, offset) per group."""
    return head_dim * bits // 8 + (head_dim // group) * 8


def pack(codes: np.ndarray, scale: np.ndarray, offset: np.ndarray, bits: int) -> np.ndarray:
    """Codes + metadata -> uint8 records [..., record_bytes]."""
    codes = np.asarray(codes, dtype=np.uint8)
    if bits == 8:
        payload = codes
    elif bits == 4:
        payload = (codes[..., 0::2] & 0x0F) | ((codes[..., 1::2] & 0x0F) << 4)
    else:
        raise ValueError(bits)
    meta = np.stack([scale.astype("<f4"), offset.astype("<f4")], axis=-1)  # [..., ng, 2]
    # the width is given, not inferred: numpy cannot infer an axis of an empty array
    meta_bytes = np.ascontiguousarray(meta).view(np.uint8).reshape(codes.shape[:-1] + (meta.shape[-2] * 8,))
    return np.concatenate([payload.astype(np.uint8), meta_bytes], axis=-1)


def unpack(records: np.ndarray, head_dim: int, bits: int, group: int = GROUP):
    """uint8 records -> (codes uint8 [..., D], scale f32, offset f32)."""
    records = np.ascontiguousarray(records, dtype=np.uint8)
    nbytes = head_dim * bits // 8
    payload = records[..., :nbytes]
    if bits == 8:
        codes = payload.copy()
    else:
        codes = np.empty(records.shape[:-1] + (head_dim,), np.uint8)
        codes[..., 0::2] = payload & 0x0F
        codes[..., 1::2] = payload >> 4
    meta = np.ascontiguousarray(records[..., nbytes:]).view("<f4")
    meta = meta.reshape(records.shape[:-1] + (head_dim // group, 2))
    return codes, meta[..., 0].astype(np.float32), meta[..., 1].astype(np.float32)


def k_records(k_bits: np.ndarray, signs: np.ndarray, bits: int, group: int = GROUP) -> np.ndarray:
    """bf16 K [..., D] -> packed records of the rotated K (quantised once, at write)."""
    k = widen(k_bits, "bf16").astype(np.float32)  # exact
    codes, scale, offset = quantise(rotate_fp32(k, signs), bits, group)
    return pack(codes, scale, offset, bits)


def v_records(v_bits: np.ndarray, bits: int, group: int = GROUP) -> np.ndarray:
    """bf16 V [..., D] -> packed records of V (unrotated)."""
    v = widen(v_bits, "bf16").astype(np.float32)
    codes, scale, offset = quantise(v, bits, group)
    return pack(codes, scale, offset, bits)


def dequantise_records(records: np.ndarray, head_dim: int, bits: int, group: int = GROUP) -> np.ndarray:
    codes, scale, offset = unpack(records, head_dim, bits, group)
    return dequantise(codes, scale, offset)


def packed_decode_attention(q_bits: np.ndarray, k_recs: Sequence[np.ndarray],
                            v_recs: Sequence[np.ndarray], signs: np.ndarray, fmt: str,
                            head_dim: int, scale: float, group: int = GROUP) -> np.ndarray:
    """Decode attention reading packed pages.

    q_bits: bf16 [B, n_q, D]; k_recs[b], v_recs[b]: uint8 [len_b, n_kv, rec].
    The query is rotated with the same basis (exactly, in fp64); keys and
    values are the dequantised records; the rest is the fp64 definition."""
    kbits, vbits = FORMATS[fmt]
    q_rot = rotate_exact(widen(q_bits, "bf16"), signs)
    ks = [dequantise_records(k, head_dim, kbits, group) for k in k_recs]
    vs = [dequantise_records(v, head_dim, vbits, group) for v in v_recs]
    return decode_attention(q_rot, ks, vs, scale)
