"""Pins of the slab-pool oracle (CPU only).

The expected values come from the statements of mlxcel issue #235 ("perf(core):
chunked slab storage for the paged pool ..."): the old single-tensor layout
(section "Problem"), the row mapping and growth by append (section "Proposed
solution: chunked slabs") and the new unit tests it asks for (section
"Acceptance criteria"): a multi-slab span round-trips byte-identically against
the dense reference, growth appends slabs without copying (counter-pinned), and
gather over an interleaved block table is byte-identical.
"""

import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.slab_pool import SlabPoolModel, records_from_u16, u16_from_records
from synth import (WORKLOADS, kv_bits_for_sequence, make_block_table, monotone_rows,
                   shuffled_rows)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fill(pool, layer, rows, k, v):
    """Write a dense sequence k, v [len, n_kv, D] (uint16) block by block."""
    bs = pool.block_size
    n = k.shape[0]
    tok = np.arange(n)
    pool.write(layer, [rows[t // bs] for t in tok], list(tok % bs),
               records_from_u16(k), records_from_u16(v))


def _dense_reference(k):
    """The dense reference of one sequence, in gather_visible's [n_kv, len, D] order."""
    return np.ascontiguousarray(np.transpose(k, (1, 0, 2)))


def test_row_mapping_partitions_the_single_tensor_layout():
    """Concatenating a layer's slabs gives the old one-tensor pool
    [capacity_blocks, block_size, n_kv, D] in which row r is index r."""
    S, bs, n_kv, D = 4, 8, 2, 4
    pool = SlabPoolModel(1, bs, n_kv, 2 * D, 2 * D, S)
    pool.reserve_rows(3 * S)
    rng = np.random.default_rng(0)
    single = np.zeros((3 * S, bs, n_kv, 2 * D), np.uint8)
    for _ in range(40):
        row, slot = int(rng.integers(0, 3 * S)), int(rng.integers(0, bs))
        rec = rng.integers(0, 256, size=(1, n_kv, 2 * D), dtype=np.uint8)
        pool.write(0, [row], [slot], rec, rec)
        single[row, slot] = rec[0]
    assert np.array_equal(np.concatenate(pool.k_slabs[0], axis=0), single)
    assert np.array_equal(np.concatenate(pool.v_slabs[0], axis=0), single)


def test_slab_for_row_examples():
    pool = SlabPoolModel(2, 32, 8, 256, 256, 4)
    pool.reserve_rows(12)
    for row, (slab, r) in {0: (0, 0), 3: (0, 3), 4: (1, 0), 7: (1, 3), 11: (2, 3)}.items():
        ks, vs, rr = pool.slab_for_row(1, row)
        assert ks is pool.k_slabs[1][slab] and vs is pool.v_slabs[1][slab] and rr == r


def test_multi_slab_span_round_trips_against_dense_reference():
    """The tiny workload: 256 tokens in rows 0..7, slabs of 4 blocks (2 slabs)."""
    w = WORKLOADS["tiny"]
    pool = SlabPoolModel(1, w.block_size, w.n_kv_heads, 2 * w.head_dim, 2 * w.head_dim,
                         w.slab_blocks)
    rows = monotone_rows([w.length], w.block_size)[0]
    assert list(rows) == list(range(8))
    pool.reserve_rows(int(rows.max()) + 1)
    assert pool.n_slabs == 2
    k, v = kv_bits_for_sequence(w.seed, 0, 0, w.length, w.n_kv_heads, w.head_dim, w.dtype)
    _fill(pool, 0, rows, k, v)
    gk, gv = pool.gather(0, rows, w.length)
    assert np.array_equal(u16_from_records(gk), _dense_reference(k))
    assert np.array_equal(u16_from_records(gv), _dense_reference(v))
    assert len(pool.split_runs(rows)) == 2


def test_interleaved_block_table_gathers_byte_identically():
    """Sequences share slabs (rows from a shuffled free list); every gathered
    sequence equals its own dense reference, including a ragged last block."""
    S, bs, n_kv, D = 4, 8, 2, 16
    lengths = [37, 64, 5, 90, 1, 0]
    rng = np.random.default_rng(7)
    rows, free, R = shuffled_rows(rng, lengths, bs, S, spare_rows=3)
    pool = SlabPoolModel(2, bs, n_kv, 2 * D, 2 * D, S)
    pool.reserve_rows(R)
    dense = {}
    for layer in range(2):
        for b, n in enumerate(lengths):
            k, v = kv_bits_for_sequence(11, layer, b, n, n_kv, D, "bf16")
            dense[layer, b] = (k, v)
            _fill(pool, layer, rows[b], k, v)
    # interleaving is real: some slab holds blocks of several sequences
    owners = {}
    for b, r in enumerate(rows):
        for row in r:
            owners.setdefault(int(row) // S, set()).add(b)
    assert max(len(s) for s in owners.values()) > 1
    table = make_block_table(rows)
    t_out = max(lengths)
    for layer in range(2):
        bk, bv = pool.gather_batched(layer, table, lengths, t_out)
        for b, n in enumerate(lengths):
            k, v = dense[layer, b]
            assert np.array_equal(u16_from_records(bk[b, :, :n]), _dense_reference(k))
            assert np.array_equal(u16_from_records(bv[b, :, :n]), _dense_reference(v))
            assert not bk[b, :, n:].any() and not bv[b, :, n:].any()


def test_growth_appends_without_copy_counter_pinned():
    S, bs, n_kv, D, L = 4, 8, 2, 8, 3
    pool = SlabPoolModel(L, bs, n_kv, 2 * D, 2 * D, S)
    assert pool.n_slabs == 0 and pool.slab_append_events == 0
    assert pool.reserve_rows(9) == 3                      # ceil(9 / 4)
    assert pool.slab_append_events == 3
    before = [[id(s) for s in pool.k_slabs[l]] for l in range(L)]
    rec = np.full((1, n_kv, 2 * D), 0xAB, np.uint8)
    pool.write(1, [5], [2], rec, rec)
    snapshot = [s.copy() for s in pool.k_slabs[1]]
    assert pool.reserve_rows(9) == 0                      # already there
    assert pool.append_slab() == 3
    assert pool.slab_append_events == 4
    for l in range(L):
        assert [id(s) for s in pool.k_slabs[l][:3]] == before[l]   # same objects
        assert not pool.k_slabs[l][3].any() and not pool.v_slabs[l][3].any()
    for s, old in zip(pool.k_slabs[1], snapshot):
        assert np.array_equal(s, old)                               # contents kept
    kb, vb = pool.slab_bytes()
    assert kb == S * bs * n_kv * 2 * D
    assert pool.bytes_reserved() == L * pool.n_slabs * (kb + vb)


def test_never_written_rows_read_zero():
    pool = SlabPoolModel(1, 4, 2, 6, 6, 2)
    pool.reserve_rows(4)
    gk, gv = pool.gather(0, [3, 0, 2], 10)
    assert gk.shape == (2, 10, 6) and not gk.any() and not gv.any()


def _runs_by_groupby(rows, S):
    out, pos = [], 0
    for slab, grp in itertools.groupby(rows, key=lambda r: int(r) // S):
        n = len(list(grp))
        out.append((slab, pos, n))
        pos += n
    return out


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(0, 63), min_size=0, max_size=40), st.sampled_from([1, 2, 4, 5, 32]))
def test_split_runs_brute_force(rows, S):
    pool = SlabPoolModel(1, 2, 1, 2, 2, S)
    runs = pool.split_runs(rows)
    assert runs == _runs_by_groupby(rows, S)
    # runs tile the list in order, each is one slab, neighbours differ (maximal)
    assert sum(c for _, _, c in runs) == len(rows)
    for i, (slab, first, count) in enumerate(runs):
        assert all(int(r) // S == slab for r in rows[first:first + count])
        if i:
            assert runs[i - 1][0] != slab


def test_golden_slab_geometry_and_run_count():
    g = json.load(open(os.path.join(GOLDEN, "slab_geometry.json")))
    assert g["slab_blocks"] * g["block_size"] == g["tokens_per_layer_slab"]
    assert g["sequence_tokens"] // g["block_size"] == g["sequence_blocks"]
    w = WORKLOADS["qwen3_0p6b_8x4k"]
    assert (w.slab_blocks, w.block_size, w.length) == (g["slab_blocks"], g["block_size"],
                                                       g["sequence_tokens"])
    pool = SlabPoolModel(1, w.block_size, 1, 2, 2, w.slab_blocks)
    for rows in monotone_rows([w.length] * w.batch, w.block_size):
        assert len(pool.split_runs(rows)) == g["runs_when_rows_are_monotone_and_slab_aligned"]
    # an offset of half a slab makes every sequence straddle one more boundary
    for rows in monotone_rows([w.length] * w.batch, w.block_size, offset=16):
        assert len(pool.split_runs(rows)) == 5


def test_u16_record_views_round_trip():
    x = np.arange(24, dtype=np.uint16).reshape(2, 3, 4) * 997
    r = records_from_u16(x)
    assert r.shape == (2, 3, 8) and r[0, 0, 0] == 0 and r[0, 0, 2] == (997 & 0xFF)
    assert np.array_equal(u16_from_records(r), x)


def test_copy_on_write_block_shares_then_isolates_a_block():
    """Touch point 2 of the chunked-slab proposal: copy_on_write_block takes
    the source slice from the source row's slab.  A sequence that takes a
    copy of another's last (partial) block in a different slab gathers
    byte-identically to the original; a later write into the copy leaves the
    original untouched, and no other row of any layer changes."""
    S, bs, n_kv, D = 4, 8, 2, 16
    pool = SlabPoolModel(2, bs, n_kv, 2 * D, 2 * D, S)
    pool.reserve_rows(16)
    rows_a = np.array([1, 6, 9, 2], np.int32)              # slabs 0, 1, 2, 0
    n = 29
    ks, vs = [], []
    for layer in range(2):
        k, v = kv_bits_for_sequence(13, layer, 0, n, n_kv, D, "bf16")
        _fill(pool, layer, rows_a, k, v)
        ks.append(k)
        vs.append(v)
    before = [[s.copy() for s in pool.k_slabs[l] + pool.v_slabs[l]] for l in range(2)]
    pool.copy_block([2], [13])                             # row 13 is in slab 3
    rows_b = np.array([1, 6, 9, 13], np.int32)
    for layer in range(2):
        after = pool.k_slabs[layer] + pool.v_slabs[layer]
        for i, (x, y) in enumerate(zip(before[layer], after)):
            if i % pool.n_slabs == 3:                      # K and V slab 3: only row 1 changed
                assert np.array_equal(np.delete(x, 1, axis=0), np.delete(y, 1, axis=0))
            else:
                assert np.array_equal(x, y)
        gk, gv = pool.gather(layer, rows_b, n)
        assert np.array_equal(u16_from_records(gk), _dense_reference(ks[layer]))
        assert np.array_equal(u16_from_records(gv), _dense_reference(vs[layer]))
    # sequence B appends token 29 into its own copy of the block
    new = np.full((1, n_kv, 2 * D), 0xAB, np.uint8)
    pool.write(0, [13], [n % bs], new, new)
    gk_a, _ = pool.gather(0, rows_a, n)
    gk_b, _ = pool.gather(0, rows_b, n + 1)
    assert np.array_equal(u16_from_records(gk_a), _dense_reference(ks[0]))
    assert np.array_equal(gk_b[:, :n], gk_a) and (gk_b[:, n] == 0xAB).all()


def test_copy_block_reads_every_source_before_writing():
    """Several pairs in one call: each destination gets its source as it was
    before the call (brute force over a tiny pool).  The second call chains
    pairs (a destination is a later pair's source), where copying pair by
    pair would differ; the C ABI leaves that case unspecified, the oracle
    reads first."""
    def fresh():
        pool = SlabPoolModel(1, 2, 1, 4, 4, 2)
        pool.reserve_rows(6)
        for row in range(6):
            rec = np.full((1, 1, 4), row + 1, np.uint8)
            pool.write(0, [row, row], [0, 1], np.repeat(rec, 2, 0), np.repeat(rec, 2, 0))
        return pool

    def values(pool):
        return [int(pool.slab_for_row(0, r)[0][pool.slab_for_row(0, r)[2]][0, 0, 0]) for r in range(6)]

    pool = fresh()
    pool.copy_block([0, 3, 5], [4, 1, 2])
    assert values(pool) == [1, 4, 6, 4, 1, 6]
    pool = fresh()
    pool.copy_block([0, 3, 4], [3, 4, 1])
    assert values(pool) == [1, 5, 3, 1, 4, 6]  # pair by pair would give [1, 1, 3, 1, 1, 6]


def test_fnv1a64_published_vectors():
    """The storage identity fingerprints the Hadamard signs with FNV-1a 64;
    its published test values pin the oracle's implementation."""
    from oracle.slab_pool import fnv1a64
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_block_export_is_the_dense_tokens_and_round_trips():
    """Serde touch point of the chunked-slab proposal: a block's exported
    bytes are its tokens' records (every layer, K then V), here checked
    against the dense sequence itself; importing them into other rows of a
    pool with another slab size gathers the same sequence byte for byte."""
    bs, n_kv, D = 8, 2, 16
    a = SlabPoolModel(2, bs, n_kv, 2 * D, 2 * D, 4)
    a.reserve_rows(12)
    rows_a = np.array([5, 0, 11], np.int32)
    n = 20
    dense = []
    for layer in range(2):
        k, v = kv_bits_for_sequence(17, layer, 0, n, n_kv, D, "bf16")
        _fill(a, layer, rows_a, k, v)
        dense.append((k, v))
    blob = a.export_blocks(rows_a)
    rec = 2 * D
    assert blob.shape == (3, 2 * 2 * bs * n_kv * rec)
    # block 1 (tokens 8..15), layer 1, V: the dense tokens' bytes in order
    row_bytes = bs * n_kv * rec
    at = (2 + 1) * row_bytes
    expect = records_from_u16(dense[1][1][8:16]).reshape(-1)
    assert np.array_equal(blob[1, at:at + row_bytes], expect)
    b = SlabPoolModel(2, bs, n_kv, 2 * D, 2 * D, 3)
    b.reserve_rows(9)
    rows_b = np.array([8, 1, 4], np.int32)
    b.import_blocks(rows_b, blob)
    for layer in range(2):
        for (ga, gb) in zip(a.gather(layer, rows_a, n), b.gather(layer, rows_b, n)):
            assert np.array_equal(ga, gb)
    assert np.array_equal(b.export_blocks(rows_b), blob)
