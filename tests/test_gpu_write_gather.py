"""write_block and gather_visible against the oracle's byte-level pool model:
bit-exact slab contents, bit-exact gathered tensors, run counts (mlxcel #235,
"Acceptance criteria": a multi-slab span round-trips byte-identically; gather
over an interleaved block table is byte-identical)."""

import numpy as np
import pytest
import torch

import decode_memory_amd as pd
from oracle.slab_pool import SlabPoolModel, records_from_u16
from synth import WORKLOADS, make_block_table, monotone_rows, normal_device, shuffled_rows, workload_lengths
from tests.gpu_util import build_pool, from_device_bits, i32, to_device_bits, token_targets

pytestmark = pytest.mark.gpu


def _model_from(lengths, rows, n_layers, bs, S, n_kv, D, dtype, seed, cap):
    """The oracle pool filled with the same tokens; built from the generators."""
    m = SlabPoolModel(n_layers, bs, n_kv, 2 * D, 2 * D, S)
    m.reserve_rows(cap)
    return m


def _fill_both(n_layers, lengths, rows, bs, S, n_kv, D, dtype, seed, cap=None):
    used = [int(r.max()) + 1 for r in rows if len(r)]
    cap = cap if cap is not None else max(used)
    model = SlabPoolModel(n_layers, bs, n_kv, 2 * D, 2 * D, S)
    model.reserve_rows(cap)

    def on_layer(layer, ks, vs):
        for b, n in enumerate(lengths):
            if n:
                r, s = token_targets(rows[b], int(n), bs)
                model.write(layer, r, s, records_from_u16(ks[b]), records_from_u16(vs[b]))

    pool = build_pool(n_layers, lengths, rows, bs, S, n_kv, D, dtype, seed, capacity_rows=cap,
                      on_layer=on_layer)
    return pool, model


def _slab_bytes(pool, layer, kv):
    slabs = pool.k_slabs if kv == "k" else pool.v_slabs
    return torch.cat([s for s in slabs[layer]]).cpu().numpy()


def _assert_slabs_equal(pool, model):
    torch.cuda.synchronize()
    for layer in range(model.n_layers):
        for kv, slabs in (("k", model.k_slabs), ("v", model.v_slabs)):
            expect = np.concatenate([s.reshape(-1) for s in slabs[layer]])
            assert np.array_equal(_slab_bytes(pool, layer, kv), expect), (layer, kv)


def _gather(pool, layer, table, lengths, t_out, rec):
    B = len(lengths)
    n_kv = pool.n_kv_heads
    k = torch.full((B, n_kv, t_out, rec), 0x5A, dtype=torch.uint8, device="cuda")
    v = torch.full((B, n_kv, t_out, rec), 0x5A, dtype=torch.uint8, device="cuda")
    runs = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    pool.gather_visible(layer, i32(table), i32(lengths), t_out, k, v, runs)
    torch.cuda.synchronize()
    return k.cpu().numpy(), v.cpu().numpy(), runs.cpu().numpy()


def test_tiny_multi_slab_span_write_and_gather():
    w = WORKLOADS["tiny"]
    lengths = [w.length]
    rows = monotone_rows(lengths, w.block_size)
    pool, model = _fill_both(1, lengths, rows, w.block_size, w.slab_blocks, w.n_kv_heads,
                             w.head_dim, w.dtype, w.seed)
    assert pool.stats()["n_slabs"] == 2
    _assert_slabs_equal(pool, model)
    table = make_block_table(rows)
    k, v, runs = _gather(pool, 0, table, lengths, w.length, 2 * w.head_dim)
    ek, ev = model.gather_batched(0, table, lengths, w.length)
    assert np.array_equal(k, ek) and np.array_equal(v, ev)
    assert list(runs) == [2]
    assert pool.check_error() == 0
    pool.close()


@pytest.mark.parametrize("dtype,D,bs,S", [("bf16", 128, 32, 4), ("fp16", 64, 16, 3),
                                           ("bf16", 256, 64, 5)])
def test_interleaved_table_ragged_lengths(dtype, D, bs, S):
    lengths = [0, 1, bs - 1, bs, bs + 1, 5 * bs + 7, 9 * bs]
    rng = np.random.default_rng(D + bs)
    rows, free, R = shuffled_rows(rng, lengths, bs, S, spare_rows=5)
    n_layers, n_kv = 2, 4
    pool, model = _fill_both(n_layers, lengths, rows, bs, S, n_kv, D, dtype, 17, cap=R)
    _assert_slabs_equal(pool, model)
    table = make_block_table(rows, max_blocks=max(len(r) for r in rows) + 2)
    t_out = max(lengths) + 3                            # zero tail past every length
    for layer in range(n_layers):
        k, v, runs = _gather(pool, layer, table, lengths, t_out, 2 * D)
        ek, ev = model.gather_batched(layer, table, lengths, t_out)
        assert np.array_equal(k, ek) and np.array_equal(v, ev), layer
        expect_runs = [len(model.split_runs(r)) for r in rows]
        assert list(runs) == expect_runs
    assert pool.check_error() == 0
    pool.close()


def test_fragmented_workload_gather_is_byte_identical():
    """The fragmented pool's layout (64 sequences, shuffled free list) at a
    reduced length so the host model stays small; runs ~ blocks per sequence."""
    w = WORKLOADS["fragmented_64"]
    lengths = (workload_lengths(w) // 16).astype(np.int64)
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 1 << 23]))
    rows, free, R = shuffled_rows(rng, lengths, w.block_size, w.slab_blocks)
    pool, model = _fill_both(1, lengths, rows, w.block_size, w.slab_blocks, 2, w.head_dim,
                             w.dtype, w.seed, cap=R)
    table = make_block_table(rows)
    k, v, runs = _gather(pool, 0, table, lengths, int(lengths.max()), 2 * w.head_dim)
    ek, ev = model.gather_batched(0, table, lengths, int(lengths.max()))
    assert np.array_equal(k, ek) and np.array_equal(v, ev)
    expect_runs = [len(model.split_runs(r)) for r in rows]
    assert list(runs) == expect_runs
    nbs = [len(r) for r in rows]
    assert sum(expect_runs) > 0.8 * sum(nbs)            # worst-case fragmentation
    pool.close()


def test_fragmented_workload_gather_full_size():
    """The fragmented pool at its full size (64 sequences U{512..16384},
    536,438 tokens, 8 kv heads, head_dim 128, shuffled free list): every
    gathered record equals the dense source the pool was written from, the
    padding past each length is zero, and each sequence's run count equals
    the oracle's run split of its row list."""
    w = WORKLOADS["fragmented_64"]
    lengths = workload_lengths(w).astype(np.int64)
    B, bs, S, n_kv, D = len(lengths), w.block_size, w.slab_blocks, w.n_kv_heads, w.head_dim
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 1 << 24]))
    rows, _, R = shuffled_rows(rng, lengths, bs, S)
    pool = pd.SlabPool(1, bs, n_kv, D, S, R // S + 2, w.dtype)
    pool.reserve_rows(R)
    dense_k, dense_v = [], []
    for b, n in enumerate(lengths):
        k = normal_device((w.seed, 1 << 24, b, 0), (int(n), n_kv, D), w.dtype, "cuda")
        v = normal_device((w.seed, 1 << 24, b, 1), (int(n), n_kv, D), w.dtype, "cuda")
        r, sl = token_targets(rows[b], int(n), bs)
        pool.write_block(0, i32(r), i32(sl), k, v)
        dense_k.append(k)
        dense_v.append(v)
    t_out = int(lengths.max())
    gk = torch.full((B, n_kv, t_out, D), 7, dtype=torch.int16, device="cuda")
    gv = torch.full_like(gk, 7)
    runs = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    pool.gather_visible(0, i32(make_block_table(rows)), i32(lengths), t_out, gk, gv, runs)
    for b, n in enumerate(lengths):
        n = int(n)
        assert torch.equal(gk[b, :, :n], dense_k[b].transpose(0, 1).view(torch.int16)), b
        assert torch.equal(gv[b, :, :n], dense_v[b].transpose(0, 1).view(torch.int16)), b
        assert not bool(gk[b, :, n:].any()) and not bool(gv[b, :, n:].any()), b
    model = SlabPoolModel(1, bs, n_kv, 2 * D, 2 * D, S)
    assert runs.cpu().tolist() == [len(model.split_runs(r)) for r in rows]
    assert pool.check_error() == 0
    pool.close()


# (n_kv, D): tokens of 256 B of K (several tokens per workgroup), exactly one
# and two 16-byte units per lane (8 kv heads at head_dim 128 and 256), and
# 1.5 units per lane (the looping one-token kernel)
@pytest.mark.parametrize("n_kv,D", [(2, 64), (8, 128), (8, 256), (12, 128)])
def test_write_block_overwrites_and_rejects_out_of_range_targets(n_kv, D):
    bs, S = 32, 2
    pool = pd.SlabPool(1, bs, n_kv, D, S, 4, "bf16")
    pool.reserve_rows(4)
    src = torch.arange(3 * n_kv * D, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    src = src.view(3, n_kv, D)
    rows = i32([1, 99, 3])
    slots = i32([5, 0, 31])
    pool.write_block(0, rows, slots, src, src)
    assert pool.check_error() == pd.DEVERR_WRITE_ROW
    pool.write_block(0, i32([2]), i32([32]), src[:1].contiguous(), src[:1].contiguous())
    assert pool.check_error() == pd.DEVERR_WRITE_SLOT
    assert pool.check_error() == 0                      # cleared by the read
    s0 = pool.slab_view(0, 0, "k").cpu().numpy()        # rows 0, 1
    s1 = pool.slab_view(0, 1, "k").cpu().numpy()        # rows 2, 3
    expect = from_device_bits(src).view(np.uint8).reshape(3, n_kv, 2 * D)
    assert np.array_equal(s0[1, 5], expect[0]) and np.array_equal(s1[1, 31], expect[2])
    assert not s1[0].any()                              # row 2 untouched (bad slot skipped)
    # overwrite in place: last write wins
    pool.write_block(0, i32([1]), i32([5]), src[2:3].contiguous(), src[2:3].contiguous())
    torch.cuda.synchronize()
    assert np.array_equal(pool.slab_view(0, 0, "k").cpu().numpy()[1, 5], expect[2])
    pool.close()


def test_gather_flags_rows_outside_the_pool():
    bs, S, n_kv, D = 32, 2, 2, 64
    pool = pd.SlabPool(1, bs, n_kv, D, S, 4, "bf16")
    pool.reserve_rows(4)
    table = np.array([[0, 7, 1]], np.int32)             # row 7 does not exist
    k, v, runs = _gather(pool, 0, table, [70], 96, 2 * D)
    assert pool.check_error() == pd.DEVERR_TABLE_ROW
    assert not k[0, :, 32:64].any()                     # the bad block reads as zeros
    pool.close()


def _copy_pairs(rows, R, rng, n_pairs):
    """Source rows among those in use, destinations among the free rows."""
    used = np.unique(np.concatenate([r for r in rows if len(r)]))
    free = np.setdiff1d(np.arange(R), used)
    src = rng.choice(used, size=n_pairs, replace=False).astype(np.int32)
    dst = rng.choice(free, size=n_pairs, replace=False).astype(np.int32)
    return src, dst


def test_copy_on_write_block_matches_the_oracle():
    """copy_on_write_block over 3 layers of a fragmented bf16 pool: every
    slab equals the oracle's after the copies, sources that cross slabs
    included; pairs with a row outside the pool are skipped and flagged."""
    lengths = [300, 77, 1000, 32, 5]
    bs, S, n_kv, D = 32, 4, 8, 128
    rows, _, R = shuffled_rows(np.random.default_rng(3), lengths, bs, S, spare_rows=12)
    pool, model = _fill_both(3, lengths, rows, bs, S, n_kv, D, "bf16", 71, cap=R)
    src, dst = _copy_pairs(rows, R, np.random.default_rng(4), 10)
    assert len({int(s) // S for s in src}) > 1 and any(s // S != d // S for s, d in zip(src, dst))
    pool.copy_on_write_block(i32(src), i32(dst))
    model.copy_block(src, dst)
    _assert_slabs_equal(pool, model)
    assert pool.check_error() == 0
    # a source past the pool and a negative destination: skipped, both flagged
    bad_src = np.array([R + 3, int(src[0])], np.int32)
    bad_dst = np.array([int(dst[1]), -1], np.int32)
    pool.copy_on_write_block(i32(bad_src), i32(bad_dst))
    err = pool.check_error()
    assert err & pd.DEVERR_TABLE_ROW and err & pd.DEVERR_WRITE_ROW
    _assert_slabs_equal(pool, model)                      # nothing was written
    pool.close()


@pytest.mark.parametrize("fmt,D", [("k4v4", 64), ("k8v4", 256)])
def test_copy_on_write_block_moves_packed_records(fmt, D):
    """Packed pools: the copy moves records byte for byte (no requantisation);
    the oracle quantises the same bf16 inputs itself."""
    from oracle.packed import FORMATS, k_records, record_bytes, v_records
    from synth import hadamard_signs, kv_bits_for_sequence
    kb, vb = FORMATS[fmt]
    lengths = [200, 64, 33]
    bs, S, n_kv = 32, 4, 8
    rows, _, R = shuffled_rows(np.random.default_rng(D), lengths, bs, S, spare_rows=8)
    signs = hadamard_signs(90 + D, D)
    pool = pd.SlabPool(2, bs, n_kv, D, S, -(-R // S) + 2, fmt, hadamard_signs=signs)
    pool.reserve_rows(R)
    model = SlabPoolModel(2, bs, n_kv, record_bytes(D, kb), record_bytes(D, vb), S)
    model.reserve_rows(R)
    for layer in range(2):
        for b, n in enumerate(lengths):
            k, v = kv_bits_for_sequence(90 + D, layer, b, n, n_kv, D, "bf16")
            r, s = token_targets(rows[b], n, bs)
            pool.write_block(layer, i32(r), i32(s), to_device_bits(k, "bf16"), to_device_bits(v, "bf16"))
            model.write(layer, r, s, k_records(k, signs, kb), v_records(v, vb))
    src, dst = _copy_pairs(rows, R, np.random.default_rng(D + 1), 5)
    pool.copy_on_write_block(i32(src), i32(dst))
    model.copy_block(src, dst)
    torch.cuda.synchronize()
    for layer in range(2):
        for slab in range(model.n_slabs):
            assert np.array_equal(pool.slab_view(layer, slab, "k").cpu().numpy(), model.k_slabs[layer][slab])
            assert np.array_equal(pool.slab_view(layer, slab, "v").cpu().numpy(), model.v_slabs[layer][slab])
    assert pool.check_error() == 0
    pool.close()


def _expected_runs(model, rows, lengths, bs):
    out = []
    for r, n in zip(rows, lengths):
        nb = -(-int(n) // bs)
        out.append(model.split_runs([int(x) for x in r[:nb]]))
    return out


@pytest.mark.parametrize("case", ["monotone_4k", "offset_5_runs", "shuffled_long", "one_row_slabs"])
def test_split_runs_lists_every_run(case):
    """pd_split_runs against the oracle's run split (maximal same-slab runs in
    logical order, as (slab, first block, blocks)): the monotone 8 x 4096
    layout gives exactly 4 runs per sequence, an offset of 16 rows 5, and
    shuffled rows over sequences longer than one 64-block chunk (runs carried
    across chunks) about one run per block; empty sequences have none."""
    bs, n_kv, D = 32, 8, 128
    if case == "monotone_4k":
        lengths, S = [4096] * 8, 32
        rows = monotone_rows(lengths, bs)
    elif case == "offset_5_runs":
        lengths, S = [4096] * 3, 32
        rows = monotone_rows(lengths, bs, offset=16)
    elif case == "shuffled_long":
        lengths, S = [0, 1, 31, 33, 64 * 32, 64 * 32 + 1, 150 * 32 + 5, 7000], 4
        rows, _, _ = shuffled_rows(np.random.default_rng(5), lengths, bs, S, spare_rows=9)
    else:
        lengths, S = [3000, 200, 0, 4096], 1
        rows, _, _ = shuffled_rows(np.random.default_rng(6), lengths, bs, S, spare_rows=2)
    cap = max(int(r.max()) + 1 for r in rows if len(r))
    pool = pd.SlabPool(1, bs, n_kv, D, S, -(-cap // S) + 1, "bf16")
    pool.reserve_rows(cap)
    table = make_block_table(rows, max_blocks=max(len(r) for r in rows) + 3)
    runs, n = pool.split_runs(i32(table), i32(lengths))
    runs, n = runs.cpu().numpy(), n.cpu().numpy()
    model = SlabPoolModel(1, bs, n_kv, 2 * D, 2 * D, S)
    expect = _expected_runs(model, rows, lengths, bs)
    for b, e in enumerate(expect):
        assert n[b] == len(e), (case, b)
        assert [tuple(int(x) for x in t) for t in runs[b, :n[b]]] == e, (case, b)
        assert (runs[b, n[b]:] == -1).all()                     # left as they were
    if case == "monotone_4k":
        assert list(n) == [4] * 8
    if case == "offset_5_runs":
        assert list(n) == [5] * 3
    assert pool.check_error() == 0
    pool.close()


def test_split_runs_flags_rows_outside_the_pool():
    pool = pd.SlabPool(1, 32, 8, 128, 4, 2, "bf16")
    pool.reserve_rows(8)
    table = i32(np.array([[0, 1, 99, 100, 5, -3]], dtype=np.int32))
    runs, n = pool.split_runs(table, i32([6 * 32]))
    assert int(n[0]) == 4
    assert [tuple(int(x) for x in t) for t in runs[0, :4].cpu().numpy()] == [(0, 0, 2), (-1, 2, 2), (1, 4, 1),
                                                                             (-1, 5, 1)]
    assert pool.check_error() == pd.DEVERR_TABLE_ROW
    pool.close()


@pytest.mark.parametrize("fmt,D", [("bf16", 128), ("k4v4", 64)])
def test_duplicate_write_check(fmt, D):
    """With the debug check on, a write_block whose tokens share a (row,
    slot) sets DEVERR_DUPLICATE (which token is stored is unspecified; the
    page's scatter never generates such calls); distinct targets, a target
    outside the pool (reported as such, not as a duplicate) and the check
    turned off leave the bit clear, and the check's bitmap is clear again
    after every call."""
    from synth import hadamard_signs
    extra = {} if fmt == "bf16" else {"hadamard_signs": hadamard_signs(5, D)}
    pool = pd.SlabPool(1, 32, 8, D, 32, 5, fmt, **extra)
    pool.reserve_rows(128)
    dt = torch.bfloat16
    n = 4096
    gen = torch.Generator(device="cuda").manual_seed(3)
    k = torch.randn((n + 1, 8, D), generator=gen, device="cuda").to(dt)
    v = torch.randn((n + 1, 8, D), generator=gen, device="cuda").to(dt)
    t = np.arange(n)
    rows, slots = (t // 32).astype(np.int32), (t % 32).astype(np.int32)   # rows 0..127
    with pytest.raises(pd.PagedKVError):
        pool.set_debug(0x80)
    pool.write_block(0, i32(rows[:3]), i32([5, 5, 5]), k[:3], v[:3])   # off: not checked
    assert pool.check_error() == 0
    pool.set_debug(pd.DEBUG_DUPLICATE_WRITES)
    pool.write_block(0, i32(rows[:n]), i32(slots[:n]), k[:n], v[:n])   # 4096 distinct targets
    assert pool.check_error() == 0
    dup_rows = np.concatenate([rows, rows[1234:1235]])
    dup_slots = np.concatenate([slots, slots[1234:1235]])
    pool.write_block(0, i32(dup_rows), i32(dup_slots), k, v)             # token n repeats token 1234
    assert pool.check_error() == pd.DEVERR_DUPLICATE
    pool.write_block(0, i32(rows[:n]), i32(slots[:n]), k[:n], v[:n])   # the bitmap was cleared
    assert pool.check_error() == 0
    pool.write_block(0, i32([1000, 1000]), i32([0, 0]), k[:2], v[:2])  # outside the pool
    assert pool.check_error() == pd.DEVERR_WRITE_ROW
    pool.set_debug(0)
    pool.write_block(0, i32(dup_rows), i32(dup_slots), k, v)
    assert pool.check_error() == 0
    pool.close()
