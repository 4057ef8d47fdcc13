"""Helpers shared by the GPU tests: build pools from the seeded inputs, move
bit patterns between numpy and torch, and compare against the oracle."""

from __future__ import annotations

import numpy as np
import torch

from oracle.attention import widen

TOL = 2e-3  # max-abs bound of paged_decode against the fp64 oracle


def torch_dtype(dtype: str):
    return torch.float16 if dtype == "fp16" else torch.bfloat16


def to_device_bits(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """uint16 bit patterns -> device tensor of the 16-bit float dtype."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch_dtype(dtype))


def from_device_bits(t: torch.Tensor) -> np.ndarray:
    """Device 16-bit tensor -> uint16 bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32(x, device="cuda") -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(x, dtype=np.int32), device=device)


def token_targets(rows: np.ndarray, length: int, block_size: int):
    """(row, slot) of every token 0..length-1 of a sequence with block rows `rows`."""
    t = np.arange(length)
    return rows[t // block_size].astype(np.int32), (t % block_size).astype(np.int32)


def half_ulp(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the output dtype at |ref|."""
    mant = 8 if dtype == "bf16" else 11
    e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -14)))
    return 2.0 ** (e - mant)


def decode_error(out_bits: np.ndarray, ref: np.ndarray, dtype: str):
    """(max-abs error, max of error minus half an output ulp)."""
    got = widen(out_bits, dtype)
    err = np.abs(got - ref)
    return float(err.max(initial=0.0)), float((err - half_ulp(ref, dtype)).max(initial=0.0))


def assert_decode_close(out_bits, ref, dtype, tol=TOL, allow_output_rounding=False):
    """paged_decode parity: max-abs <= tol.  With allow_output_rounding the
    final rounding to the 16-bit output dtype (half an ulp at |ref|) is
    allowed on top, for inputs whose outputs are large (short sequences)."""
    plain, beyond = decode_error(out_bits, ref, dtype)
    if allow_output_rounding:
        assert beyond <= tol, (plain, beyond)
    else:
        assert plain <= tol, plain
    return plain


def build_pool(n_layers, lengths, rows, block_size, slab_blocks, n_kv, head_dim, dtype, seed,
               fmt=None, signs=None, max_slabs=None, capacity_rows=None, on_layer=None):
    """A SlabPool holding the seeded K/V of every sequence, written token by
    token through write_block (one call per sequence and layer).

    on_layer(layer, ks, vs) is called with the host bit patterns of each
    layer (lists over sequences, [len_b, n_kv, D]) before they are dropped."""
    import decode_memory_amd as pd
    from synth import kv_bits_for_sequence

    used = [int(r.max()) + 1 for r in rows if len(r)]
    cap = capacity_rows if capacity_rows is not None else (max(used) if used else slab_blocks)
    n_slabs = -(-cap // slab_blocks)
    pool = pd.SlabPool(n_layers, block_size, n_kv, head_dim, slab_blocks,
                       max_slabs if max_slabs is not None else n_slabs + 4,
                       fmt if fmt is not None else dtype, signs)
    pool.reserve_rows(cap)
    for layer in range(n_layers):
        ks, vs = [], []
        for b, n in enumerate(lengths):
            k, v = kv_bits_for_sequence(seed, layer, b, int(n), n_kv, head_dim, dtype)
            ks.append(k)
            vs.append(v)
            if n == 0:
                continue
            r, s = token_targets(rows[b], int(n), block_size)
            pool.write_block(layer, i32(r), i32(s), to_device_bits(k, dtype), to_device_bits(v, dtype))
        if on_layer is not None:
            on_layer(layer, ks, vs)
    return pool


def run_decode(pool, layer, q_bits, table, lengths, dtype, scale, max_len=None, workspace=None):
    """paged_decode through the C ABI; returns output bit patterns [B, n_q, D]."""
    q = to_device_bits(q_bits, dtype)
    out = torch.empty_like(q)
    t = i32(table)
    lens = i32(lengths)
    ml = int(max(lengths)) if max_len is None else max_len
    ws = workspace if workspace is not None else pool.workspace(q.shape[0], q.shape[1], ml)
    pool.paged_decode(layer, q, t, lens, ml, scale, out, ws)
    torch.cuda.synchronize()
    return from_device_bits(out)


def packed_decode_bound(q_bits, k_recs, v_recs, signs, fmt, head_dim, scale, group):
    """Per-output error bound of the packed decode kernel's arithmetic, in fp64
    from the same records (shape [B, n_q, D]).

    The kernel feeds the matrix cores f16 operands.  Value products take
    p * scale as f16 (relative error 2^-11, or 2^-25 absolute below f16's
    normal range, at a power-of-two prescale 2^vk that is at least
    min(1024, 2^(14 - e)) for a largest group scale in [2^e, 2^(e+1))), so
    the value sum is off by at most 2^-11 * sum_t p_t |v_t - offset_t| / l
    plus the subnormal floor; twice that is allowed (fp32 accumulation).
    Scores take q' as two f16 parts (about 22 bits) whose products accumulate
    in fp32 around biased codes: an error below 2^-16 * scale * sum_i
    |q'_i k_i| per score is allowed, and it moves the output by at most that
    times sum_t p_t |v_t - o| / l.  The 2e-3 of the plain tolerance comes on
    top."""
    from oracle.packed import FORMATS, rotate_exact, unpack

    kb, vb = FORMATS[fmt]
    q_rot = rotate_exact(widen(q_bits, "bf16"), signs)  # [B, n_q, D]
    B, n_q, D = q_rot.shape
    out = np.zeros((B, n_q, D))
    for b in range(B):
        if k_recs[b].shape[0] == 0:
            continue
        kc, ks, ko = unpack(k_recs[b], head_dim, kb, group)
        vc, vs, vo = unpack(v_recs[b], head_dim, vb, group)
        ng = head_dim // group
        kh = (kc.astype(np.float64).reshape(kc.shape[:-1] + (ng, group)) * ks[..., None] + ko[..., None]
              ).reshape(kc.shape)                                   # [T, n_kv, D]
        vd = (vc.astype(np.float64).reshape(vc.shape[:-1] + (ng, group)) * vs[..., None])
        vd = vd.reshape(vc.shape)                                   # v - offset
        vh = vd + np.repeat(vo.astype(np.float64), group, axis=-1)  # v
        n_kv = kh.shape[1]
        G = n_q // n_kv
        T = kh.shape[0]
        vmax = float(np.max(vs)) if vs.size else 0.0
        e = np.floor(np.log2(vmax)) if vmax > 0 else -100
        vf = min(1024.0, 2.0 ** (14 - e))
        floor = T * ((1 << vb) - 1) * 2.0 ** -25 / vf
        for h in range(n_q):
            g = h // G
            s = scale * (kh[:, g, :] @ q_rot[b, h])
            s1 = scale * (np.abs(kh[:, g, :]) @ np.abs(q_rot[b, h]))
            w = np.exp(s - s.max())
            l = w.sum()
            o = (w @ vh[:, g, :]) / l
            wterm = (w @ np.abs(vd[:, g, :])) / l
            dv = (w @ np.abs(vh[:, g, :] - o)) / l
            out[b, h] = 2.0 * 2.0 ** -11 * wterm + floor + 2.0 ** -16 * s1.max() * dv
    return out


def assert_packed_close(out_bits, ref, bound, dtype="bf16", tol=TOL):
    """|out - ref| <= tol + half an output ulp at |ref| + bound, element-wise;
    every output finite.  Returns the largest error over its allowance."""
    got = widen(out_bits, dtype)
    assert np.isfinite(got).all(), "non-finite output"
    err = np.abs(got - ref)
    allow = tol + half_ulp(ref, dtype) + bound
    worst = float((err / allow).max(initial=0.0))
    assert worst <= 1.0, (worst, float(err.max()))
    return worst
