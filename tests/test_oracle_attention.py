"""Pins of the fp64 decode-attention oracle (CPU only).

Each check is fixed by the mathematics of softmax attention or by a worked
example, not by the oracle's own code: closed forms (identical keys give the
mean of V, one token gives v0, two tokens give the logistic weights), a
library softmax on tiny inputs, invariances (token permutation, score shift),
limits of the scale, and the GQA head mapping (consecutive query heads share
a kv head; a reading, since the pages do not state it).
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
from hypothesis import given, settings, strategies as st

from oracle.attention import attend_one, decode_attention, decode_attention_bits, round_to_dtype, widen
from synth import bf16_bits_from_f32, f16_bits_from_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_two_token_example():
    g = json.load(open(os.path.join(GOLDEN, "attention_two_tokens.json")))
    q = np.array([g["q"]])
    o = attend_one(q, np.array(g["k"]), np.array(g["v"]), g["scale"])
    assert abs(g["w0"] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    np.testing.assert_allclose(o[0], g["o"], rtol=0, atol=1e-15)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(1)
    k = np.tile(rng.standard_normal(64), (300, 1))
    v = rng.standard_normal((300, 64))
    q = rng.standard_normal((3, 64))
    o = attend_one(q, k, v, 0.125)
    np.testing.assert_allclose(o, np.tile(np.mean(v, axis=0), (3, 1)), rtol=0, atol=1e-12)


def test_one_token_gives_its_value_exactly():
    rng = np.random.default_rng(2)
    k, v, q = rng.standard_normal((1, 32)), rng.standard_normal((1, 32)), rng.standard_normal((2, 32))
    o = attend_one(q, k, v, 0.3)
    assert np.array_equal(o, np.tile(v[0], (2, 1)))


def test_two_tokens_logistic_closed_form():
    rng = np.random.default_rng(3)
    for _ in range(20):
        k, v, q = rng.standard_normal((2, 16)), rng.standard_normal((2, 16)), rng.standard_normal((1, 16))
        s0, s1 = 0.25 * (k[0] @ q[0]), 0.25 * (k[1] @ q[0])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(attend_one(q, k, v, 0.25)[0], w0 * v[0] + (1 - w0) * v[1],
                                   rtol=0, atol=1e-13)


@settings(max_examples=100, deadline=None)
@given(st.integers(1, 12), st.integers(1, 8), st.integers(0, 2**31 - 1))
def test_brute_force_against_library_softmax(n, d, seed):
    rng = np.random.default_rng(seed)
    k, v, q = rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((2, d))
    scale = float(rng.uniform(0.05, 2.0))
    expect = np.empty((2, d))
    for i in range(2):
        p = scipy.special.softmax([scale * float(np.dot(q[i], k[t])) for t in range(n)])
        expect[i] = sum(p[t] * v[t] for t in range(n))
    np.testing.assert_allclose(attend_one(q, k, v, scale), expect, rtol=0, atol=1e-12)


def test_permutation_and_shift_invariance_and_scale_limits():
    rng = np.random.default_rng(4)
    k, v, q = rng.standard_normal((50, 8)), rng.standard_normal((50, 8)), rng.standard_normal((1, 8))
    o = attend_one(q, k, v, 0.5)
    perm = rng.permutation(50)
    np.testing.assert_allclose(attend_one(q, k[perm], v[perm], 0.5), o, atol=1e-13)
    # adding a multiple of q to every key shifts every score by the same amount
    np.testing.assert_allclose(attend_one(q, k + 3.0 * q, v, 0.5), o, atol=1e-12)
    # scale -> 0: uniform weights; large scale: the best-scoring key's value
    np.testing.assert_allclose(attend_one(q, k, v, 1e-14), v.mean(axis=0)[None], atol=1e-12)
    best = int(np.argmax(k @ q[0]))
    np.testing.assert_allclose(attend_one(q, k, v, 1e4), v[best][None], atol=1e-9)


def test_gqa_consecutive_query_heads_share_a_kv_head():
    """Each kv head holds a constant, distinct value vector: output head h must
    equal the constant of kv head h // G."""
    B, n_kv, G, D, n = 2, 4, 3, 8, 17
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, n_kv * G, D))
    ks = [rng.standard_normal((n, n_kv, D)) for _ in range(B)]
    vs = [np.broadcast_to(np.arange(n_kv, dtype=np.float64)[None, :, None] * 10 + b,
                          (n, n_kv, D)).copy() for b in range(B)]
    o = decode_attention(q, ks, vs, 0.3)
    for b in range(B):
        for h in range(n_kv * G):
            np.testing.assert_allclose(o[b, h], 10.0 * (h // G) + b, atol=1e-12)


def test_empty_sequence_gives_zeros():
    q = np.ones((2, 4, 8))
    ks = [np.zeros((0, 2, 8)), np.ones((3, 2, 8))]
    vs = [np.zeros((0, 2, 8)), np.full((3, 2, 8), 2.0)]
    o = decode_attention(q, ks, vs, 1.0)
    assert not o[0].any() and np.allclose(o[1], 2.0)


def test_widen_is_exact():
    x = np.array([0.0, 1.0, -2.5, 3.140625, 65504.0, 2.0 ** -24], dtype=np.float32)
    assert np.array_equal(widen(f16_bits_from_f32(x), "fp16"), x.astype(np.float64))
    xb = np.array([0.0, 1.0, -2.5, 3.140625, 1e30, -2.0 ** -100], dtype=np.float32)
    xb = (bf16_bits_from_f32(xb).astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(widen(bf16_bits_from_f32(xb), "bf16"), xb.astype(np.float64))


def test_round_to_dtype_against_independent_roundings():
    rng = np.random.default_rng(6)
    x32 = rng.standard_normal(20000).astype(np.float32) * np.float32(3)
    # bf16: the bit-level nearest-even rounding of the input generator agrees
    expect = (bf16_bits_from_f32(x32).astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(round_to_dtype(x32.astype(np.float64), "bf16"), expect.astype(np.float64))
    # ties go to even: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    assert round_to_dtype(np.array([1 + 2 ** -8]), "bf16")[0] == 1.0
    assert round_to_dtype(np.array([1 + 3 * 2 ** -8]), "bf16")[0] == 1 + 2 ** -6
    x64 = rng.standard_normal(20000)
    assert np.array_equal(round_to_dtype(x64, "fp16"), x64.astype(np.float16).astype(np.float64))


def test_decode_attention_bits_widens_then_attends():
    rng = np.random.default_rng(8)
    qf = rng.standard_normal((1, 2, 16)).astype(np.float32)
    kf = rng.standard_normal((5, 1, 16)).astype(np.float32)
    vf = rng.standard_normal((5, 1, 16)).astype(np.float32)
    got = decode_attention_bits(f16_bits_from_f32(qf), [f16_bits_from_f32(kf)],
                                [f16_bits_from_f32(vf)], "fp16", 0.25)
    q16, k16, v16 = (a.astype(np.float16).astype(np.float64) for a in (qf, kf, vf))
    for h in range(2):
        p = scipy.special.softmax(0.25 * (k16[:, 0] @ q16[0, h]))
        np.testing.assert_allclose(got[0, h], p @ v16[:, 0], atol=1e-13)
