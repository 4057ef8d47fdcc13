"""The seeded input generators: determinism, dtypes and row layouts (CPU only)."""

import numpy as np

from synth import (WORKLOADS, bf16_bits_from_f32, f16_bits_from_f32, hadamard_signs,
                   kv_bits_for_sequence, make_block_table, monotone_rows, shuffled_rows,
                   workload_lengths)


def test_bf16_rounding_examples():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.0, 0.0, 3.0e38], np.float32)
    assert list(bf16_bits_from_f32(x)) == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x0000, 0x7F62]


def test_generators_are_deterministic_and_sequences_independent():
    a = kv_bits_for_sequence(2, 3, 4, 50, 8, 128, "bf16")
    b = kv_bits_for_sequence(2, 3, 4, 50, 8, 128, "bf16")
    c = kv_bits_for_sequence(2, 3, 5, 50, 8, 128, "bf16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0]) and not np.array_equal(a[0], a[1])
    # a prefix of a longer draw is the shorter draw (streams are per sequence)
    long = kv_bits_for_sequence(2, 3, 4, 80, 8, 128, "bf16")
    assert np.array_equal(long[0][:50], a[0])
    f = f16_bits_from_f32(np.array([1.0, -0.5], np.float32))
    assert list(f) == [0x3C00, 0xB800]


def test_shuffled_rows_are_distinct_and_interleaved():
    w = WORKLOADS["fragmented_64"]
    lens = workload_lengths(w)
    assert lens.min() >= 512 and lens.max() <= 16384 and len(lens) == 64
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 1 << 23]))
    rows, free, R = shuffled_rows(rng, lens, w.block_size, w.slab_blocks)
    flat = np.concatenate(rows)
    assert len(set(flat.tolist())) == len(flat)
    assert len(flat) + len(free) == R and R % w.slab_blocks == 0
    assert set(free).isdisjoint(flat.tolist())
    assert [len(r) for r in rows] == [-(-int(n) // w.block_size) for n in lens]
    t = make_block_table(rows)
    assert t.shape == (64, max(len(r) for r in rows)) and (t[0, len(rows[0]):] == -1).all()


def test_signs_and_monotone_rows():
    s = hadamard_signs(5, 256)
    assert set(np.unique(s).tolist()) == {-1, 1} and s.dtype == np.int8
    rows = monotone_rows([4096] * 8, 32)
    assert [int(r[0]) for r in rows] == [128 * b for b in range(8)]
