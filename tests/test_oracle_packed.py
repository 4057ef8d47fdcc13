"""Pins of the packed-format oracle (CPU only).

Fixed by the mathematics of the Hadamard basis (orthogonality, the textbook
H_4, rotation preserves dot products), by the definition of an affine
quantiser (reconstruction within half a step, min and max hit the end codes,
nearest level by brute force, constant groups exact), by the page's size
statement (mlx-swift-lm PR #142, section "Summary": five effective bits per
K4/V4 value including metadata, 3.2x smaller than BF16), and by the plain
bf16 attention the packed path approximates.
"""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.attention import decode_attention, decode_attention_bits, widen
from oracle.packed import (FORMATS, GROUP, dequantise, dequantise_records, inv_sqrt_f32, k_records,
                           pack, packed_decode_attention, quantise, record_bytes, rotate_exact,
                           rotate_fp32, sylvester_hadamard, unpack, v_records)
from synth import bf16_bits_from_f32, hadamard_signs, kv_bits_for_sequence, q_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_textbook_h4():
    expect = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], float)
    assert np.array_equal(sylvester_hadamard(4), expect)


@pytest.mark.parametrize("d", [2, 8, 64, 128, 256])
def test_hadamard_is_orthogonal(d):
    h = sylvester_hadamard(d)
    assert np.array_equal(h @ h.T, d * np.eye(d))
    assert np.array_equal(h, h.T)


@pytest.mark.parametrize("d", [64, 256])
def test_rotation_preserves_dot_products(d):
    rng = np.random.default_rng(d)
    s = hadamard_signs(3, d)
    q, k = rng.standard_normal((5, d)), rng.standard_normal((7, d))
    qr, kr = rotate_exact(q, s), rotate_exact(k, s)
    np.testing.assert_allclose(qr @ kr.T, q @ k.T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(kr, axis=1), np.linalg.norm(k, axis=1), rtol=1e-13)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp32_butterflies_match_matrix_rotation(d):
    """The stored fp32 FWHT equals the exact rotation to fp32 rounding: each of
    the log2(d) stages adds at most one rounding of relative size 2^-24 to
    partial sums bounded by sqrt(d) * max|x|."""
    rng = np.random.default_rng(d + 1)
    s = hadamard_signs(4, d)
    x = rng.standard_normal((50, d)).astype(np.float32)
    exact = rotate_exact(x.astype(np.float64), s)
    got = rotate_fp32(x, s).astype(np.float64)
    bound = np.log2(d) * 2.0 ** -24 * d * np.abs(x).max(axis=1, keepdims=True) / np.sqrt(d) * 2
    assert (np.abs(got - exact) <= bound).all()


@pytest.mark.parametrize("d", [64, 256])
def test_rotation_of_unit_vectors_gives_signed_columns(d):
    s = hadamard_signs(9, d)
    h = sylvester_hadamard(d)
    for i in (0, 1, d // 2 + 3, d - 1):
        e = np.zeros(d, np.float32)
        e[i] = 1.0
        got = rotate_fp32(e[None], s)[0].astype(np.float64)
        assert np.array_equal(got, s[i] * h[:, i] / np.sqrt(d))  # exact for d = 64, 256


def test_inv_sqrt_exact_for_powers_of_four():
    assert inv_sqrt_f32(64) == np.float32(0.125) and inv_sqrt_f32(256) == np.float32(0.0625)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [32, 64])
def test_quantiser_error_bound_and_end_codes(bits, group):
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((200, 128)).astype(np.float32)
    ng = 128 // group
    codes, scale, offset = quantise(x, bits, group)
    assert scale.shape == (200, ng) and offset.shape == (200, ng)
    assert codes.max() <= (1 << bits) - 1
    xh = dequantise(codes, scale, offset)
    step = np.repeat(scale.astype(np.float64), group, axis=-1)
    assert (np.abs(xh - x) <= step / 2 * (1 + 1e-5) + 1e-6).all()
    g = x.reshape(200, ng, group)
    c = codes.reshape(200, ng, group)
    assert (c[np.arange(200)[:, None], np.arange(ng)[None], g.argmin(-1)] == 0).all()
    assert (c[np.arange(200)[:, None], np.arange(ng)[None], g.argmax(-1)] == (1 << bits) - 1).all()
    assert np.array_equal(offset, g.min(-1))


def test_group_of_64_shares_one_scale_over_a_ramp():
    """x_i = i over one group of 64 at 4 bits: one (scale, offset) = (63/15, 0)
    for the whole group, and code i = rint(i / scale); groups of 32 would give
    two ranges (0..31, 32..63) instead."""
    x = np.arange(64, dtype=np.float32)[None]
    codes, scale, offset = quantise(x, 4, 64)
    assert scale.shape == (1, 1) and scale[0, 0] == np.float32(63) / np.float32(15)
    assert offset[0, 0] == 0
    expect = np.rint(x[0].astype(np.float32) / scale[0, 0]).astype(np.uint8)
    assert np.array_equal(codes[0], expect) and codes[0, -1] == 15 and codes[0, 0] == 0
    c32, s32, o32 = quantise(x, 4, 32)
    assert np.array_equal(o32[0], [0, 32]) and (s32[0] == np.float32(31) / np.float32(15)).all()


@settings(max_examples=200, deadline=None)
@given(st.lists(st.floats(-4, 4, width=32), min_size=64, max_size=64), st.sampled_from([4, 8]),
       st.sampled_from([32, 64]))
def test_quantiser_picks_nearest_level_brute_force(vals, bits, group):
    x = np.array(vals[:group], dtype=np.float32)[None]
    codes, scale, offset = quantise(x, bits, group)
    if scale[0, 0] == 0:
        assert not codes.any()
        return
    levels = np.arange(1 << bits) * np.float64(scale[0, 0]) + np.float64(offset[0, 0])
    dist = np.abs(x[0][:, None].astype(np.float64) - levels[None, :])
    best = dist.min(axis=1)
    chosen = dist[np.arange(group), codes[0]]
    # the chosen level is the nearest one, up to fp32 rounding of (x - mn)/scale
    assert (chosen <= best + 1e-6 * (1 + np.abs(x[0]))).all()


def test_constant_group_is_exact():
    x = np.full((3, 64), 1.7, np.float32)
    x[1, :32] = -0.25
    codes, scale, offset = quantise(x, 4)
    assert not codes.any()
    assert np.array_equal(dequantise(codes, scale, offset), x.astype(np.float64))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [32, 64])
def test_pack_unpack_round_trip_and_nibble_order(bits, group):
    rng = np.random.default_rng(10)
    ng = 64 // group
    codes = rng.integers(0, 1 << bits, size=(4, 3, 64)).astype(np.uint8)
    scale = rng.standard_normal((4, 3, ng)).astype(np.float32)
    offset = rng.standard_normal((4, 3, ng)).astype(np.float32)
    rec = pack(codes, scale, offset, bits)
    assert rec.shape[-1] == record_bytes(64, bits, group) == 64 * bits // 8 + 8 * ng
    c2, s2, o2 = unpack(rec, 64, bits, group)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scale) and np.array_equal(o2, offset)
    one = pack((np.arange(64)[None] % (1 << bits)).astype(np.uint8), np.ones((1, 2), np.float32),
               np.zeros((1, 2), np.float32), bits)
    if bits == 4:
        assert one[0, 0] == 0x10 and one[0, 1] == 0x32       # element 2i low nibble
    else:
        assert one[0, 0] == 0 and one[0, 5] == 5
    assert one[0, 64 * bits // 8: 64 * bits // 8 + 4].view("<f4")[0] == 1.0


def test_golden_effective_bits():
    g = json.load(open(os.path.join(GOLDEN, "packed_sizes.json")))
    d = 256
    bits64 = record_bytes(d, 4, group=g["group_for_five_bits"]) * 8 / d
    assert bits64 == g["k4v4_effective_bits_per_value"]
    assert abs(16 / bits64 - g["k4v4_reduction_vs_bf16"]) < 1e-12
    assert record_bytes(d, 4) * 8 / d == g["group32_effective_bits_k4"]
    assert record_bytes(d, 8) * 8 / d == g["group32_effective_bits_k8"]


@pytest.mark.parametrize("fmt,tol", [("k8v8", 0.01), ("k8v4", 0.06), ("k4v4", 0.08)])
@pytest.mark.parametrize("d,group", [(64, 32), (256, 32), (128, 64), (256, 64)])
def test_packed_decode_approximates_bf16_attention(fmt, tol, d, group):
    """The packed route reproduces bf16 attention up to quantisation error.

    A wrong rotation of q (missing, other signs), a wrong nibble order or a
    wrong metadata order makes the error O(0.1 .. 1); quantisation alone keeps
    it below the per-format bound (the bound is looser at 4 bits: 15 levels
    over the range of a group of 32 or 64 N(0,1) values is a step of about
    0.3)."""
    B, n_kv, G, n = 2, 2, 4, 300
    signs = hadamard_signs(5, d)
    kb, vb = FORMATS[fmt]
    q = q_bits(5, 0, B, n_kv * G, d, "bf16")
    ks, vs, krs, vrs = [], [], [], []
    for b in range(B):
        k, v = kv_bits_for_sequence(5, 0, b, n, n_kv, d, "bf16")
        ks.append(k)
        vs.append(v)
        krs.append(k_records(k, signs, kb, group))
        vrs.append(v_records(v, vb, group))
    ref = decode_attention_bits(q, ks, vs, "bf16", 1 / np.sqrt(d))
    got = packed_decode_attention(q, krs, vrs, signs, fmt, d, 1 / np.sqrt(d), group)
    err = np.abs(got - ref).max()
    assert err < tol, err


@pytest.mark.parametrize("d,group", [(64, 32), (128, 64)])
def test_packed_decode_is_exact_when_quantisation_is_exact(d, group):
    """Keys and values whose rotated / plain groups sit on an exact 8-bit grid
    reconstruct exactly, so packed attention equals the plain definition."""
    n = 40
    signs = hadamard_signs(6, d)
    rng = np.random.default_rng(11)
    # V: integers 0..255 with both ends present in every group -> scale 1, offset 0
    v_int = rng.integers(0, 256, size=(n, 1, d)).astype(np.float32)
    v_int[:, :, 0::group] = 0
    v_int[:, :, 1::group] = 255
    vbits = bf16_bits_from_f32(v_int)  # integers < 256 are exact in bf16
    v_rec = v_records(vbits, 8, group)
    assert np.array_equal(dequantise_records(v_rec, d, 8, group), v_int.astype(np.float64))
    kbits = bf16_bits_from_f32(rng.standard_normal((n, 1, d)).astype(np.float32))
    qb = bf16_bits_from_f32(rng.standard_normal((1, 1, d)).astype(np.float32))
    k_rec = k_records(kbits, signs, 8, group)
    scale = 1 / np.sqrt(d)
    got = packed_decode_attention(qb, [k_rec], [v_rec], signs, "k8v8", d, scale, group)
    # the same keys, dequantised and rotated back (H is symmetric and
    # H H = d I, so x = sigma * (H x') / sqrt(d)), through the plain definition
    khat = dequantise_records(k_rec, d, 8, group)
    k_back = (khat @ sylvester_hadamard(d)) / np.sqrt(d) * signs
    ref = decode_attention(widen(qb, "bf16"), [k_back], [v_int.astype(np.float64)], scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-9)
