"""Pins of the footprint accounting (CPU only): closed forms for the
growth-by-copy ladder and the slab pool of mlxcel issue #235 ("Problem",
"Proposed solution: chunked slabs")."""

from oracle.footprint import (blocks_for, dense_bytes, growth_by_copy_peak,
                              slab_pool_capacity)


def test_slab_pool_equals_dense_when_spans_fill_whole_slabs():
    bs, S, tok = 32, 32, 10
    blk = bs * tok
    lengths = [bs * S] * 5                       # each prefill is exactly one slab
    cap = slab_pool_capacity(lengths, bs, S, blk)
    assert cap == [(i + 1) * S * blk for i in range(5)]
    assert cap[-1] == dense_bytes(lengths, tok)


def test_slab_pool_overhead_is_below_one_slab():
    bs, S, blk = 32, 32, 64
    lengths = [4100, 4200, 4297, 4096, 4150, 4250, 4111, 4222]
    cap = slab_pool_capacity(lengths, bs, S, blk)[-1]
    rows = sum(blocks_for(n, bs) for n in lengths)
    # growth appends whole slabs: with the bound below, the capacity is the
    # smallest whole number of slabs that holds the rows
    assert cap % (S * blk) == 0
    assert rows * blk <= cap < (rows + S) * blk
    assert cap > dense_bytes(lengths, blk // bs)


def test_growth_by_copy_ladder_closed_form():
    """n prefills of one growth chunk each: capacities 1, 2, ..., n chunks;
    the cache keeps 1 + ... + (n-1) of them, so the peak is n(n+1)/2 chunks."""
    bs, chunk, blk = 32, 32, 7
    for n in (1, 2, 3, 8):
        peak = growth_by_copy_peak([bs * chunk] * n, bs, chunk, blk)
        assert peak == n * (n + 1) // 2 * chunk * blk


def test_growth_without_crossing_a_chunk_keeps_no_ladder():
    bs, chunk, blk = 32, 32, 1
    assert growth_by_copy_peak([10, 10, 10], bs, chunk, blk) == chunk * blk
