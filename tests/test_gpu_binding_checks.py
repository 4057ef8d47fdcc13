"""The Python binding checks what the C ABI cannot see (it takes raw
pointers): tensor sizes and dtypes against the pool's geometry.  A wrong
argument raises before anything is launched, so nothing is written out of
bounds and the pool and outputs stay as they were."""

import numpy as np
import pytest
import torch

import decode_memory_amd as pd
from synth import hadamard_signs, make_block_table, monotone_rows
from tests.gpu_util import i32

pytestmark = pytest.mark.gpu


def _slabs(pool):
    return [t.clone() for layer in pool.k_slabs + pool.v_slabs for t in layer]


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.fixture
def pool():
    p = pd.SlabPool(1, 32, 8, 128, 4, 4, "bf16")
    p.reserve_rows(4)
    yield p
    p.close()


def test_write_block_checks_sources(pool):
    rows, slots = i32([0, 0, 1]), i32([0, 1, 2])
    before = _slabs(pool)
    short = torch.ones((2, 8, 128), dtype=torch.bfloat16, device="cuda")   # 3 tokens given
    full = torch.ones((3, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        pool.write_block(0, rows, slots, short, full)
    with pytest.raises(ValueError):
        pool.write_block(0, rows, slots, full, short)
    with pytest.raises(ValueError):
        pool.write_block(0, rows, slots, full.to(torch.float16), full)       # pool is bf16
    narrow = torch.ones((3, 8, 64), dtype=torch.bfloat16, device="cuda")  # head_dim 64, pool 128
    with pytest.raises(ValueError):
        pool.write_block(0, rows, slots, narrow, narrow)
    torch.cuda.synchronize()
    assert _same(before, _slabs(pool))


def test_gather_checks_output_sizes(pool):
    lengths = [40, 7]
    table = i32(make_block_table(monotone_rows(lengths, 32)))
    lens = i32(lengths)
    ok = torch.full((2, 8, 40, 256), 7, dtype=torch.uint8, device="cuda")
    small = torch.full((2, 8, 39, 256), 7, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        pool.gather_visible(0, table, lens, 40, small, ok)
    with pytest.raises(ValueError):
        pool.gather_visible(0, table, lens, 40, ok, small)
    with pytest.raises(ValueError):
        pool.gather_visible(0, table, i32([40]), 40, ok, ok)                # lens of one sequence
    torch.cuda.synchronize()
    assert bool((ok == 7).all()) and bool((small == 7).all())


def test_decode_checks_query_and_output(pool):
    lengths = [40, 7]
    table = i32(make_block_table(monotone_rows(lengths, 32)))
    lens = i32(lengths)
    ws = pool.workspace(2, 16, 40)
    q = torch.zeros((2, 16, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    bad_q = [torch.zeros((2, 16, 64), dtype=torch.bfloat16, device="cuda"),    # head_dim 64
             torch.zeros((2, 16, 128), dtype=torch.float16, device="cuda"),    # fp16 on a bf16 pool
             torch.zeros((2, 12, 128), dtype=torch.bfloat16, device="cuda")]   # 12 heads over 8 kv heads
    for bq in bad_q:
        with pytest.raises(ValueError):
            pool.paged_decode(0, bq, table, lens, 40, 0.1, out, ws)
        with pytest.raises(ValueError):
            pool.paged_decode_noalloc(0, bq, table, lens, 40, 0.1, out)
    with pytest.raises(ValueError):
        pool.paged_decode(0, q, table, lens, 40, 0.1, out[:1], ws)              # output of one sequence
    with pytest.raises(ValueError):
        pool.paged_decode(0, q, table[:1], lens, 40, 0.1, out, ws)              # table of one sequence
    kn = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        pool.paged_decode_append(0, q, kn[:1], kn, table, lens, 40, 0.1, out, ws)
    before = _slabs(pool)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    assert _same(before, _slabs(pool))


def test_packed_pool_checks_query_dtype_and_group():
    """A packed pool takes bf16 queries; its decode kernel covers 1, 2 or 4
    query heads per kv head, so 8 is refused by the library before launch."""
    D = 64
    p = pd.SlabPool(1, 32, 8, D, 4, 4, "k4v4", hadamard_signs=hadamard_signs(3, D))
    p.reserve_rows(4)
    lengths = [40]
    table = i32(make_block_table(monotone_rows(lengths, 32)))
    lens = i32(lengths)
    q16 = torch.zeros((1, 32, D), dtype=torch.float16, device="cuda")
    out = torch.full((1, 32, D), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        p.paged_decode(0, q16, table, lens, 40, 0.1, out, p.workspace(1, 32, 40))
    q8 = torch.zeros((1, 64, D), dtype=torch.bfloat16, device="cuda")
    out8 = torch.full_like(q8, 7.0)
    with pytest.raises(pd.PagedKVError) as e:
        p.paged_decode(0, q8, table, lens, 40, 0.1, out8, torch.zeros(1 << 20, dtype=torch.uint8, device="cuda"))
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((out8 == 7.0).all())
    p.close()
