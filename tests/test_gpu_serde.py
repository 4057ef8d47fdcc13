"""Block serialisation on the device (mlxcel #235, "Proposed solution",
touch point 6: serde block-content extraction and the restore path through
the row mapping; mlx-swift-lm PR #142, "Summary" and the "After" flowchart:
checkpoints preserve packed bytes exactly and reject incompatible storage
identities before allocation).  Expected bytes come from the oracle's pool
model filled from the same seeded inputs."""

import numpy as np
import pytest
import torch

import decode_memory_amd as pd
from oracle.packed import FORMATS, k_records, record_bytes, v_records
from oracle.slab_pool import SlabPoolModel, records_from_u16, signs_fingerprint
from synth import hadamard_signs, kv_bits_for_sequence, make_block_table, q_bits, shuffled_rows
from tests.gpu_util import i32, to_device_bits, token_targets

pytestmark = pytest.mark.gpu


def _pools(fmt, D, lengths, S, seed, n_layers=2, n_kv=8, bs=32, spare=6, group=32):
    """A device pool and the oracle's model holding the same blocks."""
    rows, _, R = shuffled_rows(np.random.default_rng(seed), lengths, bs, S, spare_rows=spare)
    packed = fmt in FORMATS
    signs = hadamard_signs(seed, D) if packed else None
    kb, vb = FORMATS[fmt] if packed else (16, 16)
    krec = record_bytes(D, kb, group) if packed else 2 * D
    vrec = record_bytes(D, vb, group) if packed else 2 * D
    pool = pd.SlabPool(n_layers, bs, n_kv, D, S, -(-R // S) + 4, fmt, hadamard_signs=signs,
                       group_size=group if packed else 0)
    pool.reserve_rows(R)
    model = SlabPoolModel(n_layers, bs, n_kv, krec, vrec, S)
    model.reserve_rows(R)
    for layer in range(n_layers):
        for b, n in enumerate(lengths):
            k, v = kv_bits_for_sequence(seed, layer, b, n, n_kv, D, "bf16")
            r, s = token_targets(rows[b], n, bs)
            pool.write_block(layer, i32(r), i32(s), to_device_bits(k, "bf16"), to_device_bits(v, "bf16"))
            if packed:
                model.write(layer, r, s, k_records(k, signs, kb, group), v_records(v, vb, group))
            else:
                model.write(layer, r, s, records_from_u16(k), records_from_u16(v))
    return pool, model, rows, R, signs


@pytest.mark.parametrize("fmt,D,group", [("bf16", 128, 0), ("k4v4", 64, 32), ("k8v4", 256, 32),
                                         ("k8v8", 64, 32), ("k4v4", 256, 64)])
def test_export_is_bit_exact_and_round_trips_into_another_pool(fmt, D, group):
    lengths = [100, 33, 64]
    pool, model, rows, R, signs = _pools(fmt, D, lengths, 4, 300 + D, group=group)
    blocks = np.concatenate(rows).astype(np.int32)
    got = pool.export_blocks(i32(blocks)).cpu().numpy()
    assert got.shape[1] == pd.block_bytes(pool.handle)
    assert np.array_equal(got, model.export_blocks(blocks))
    ident = pool.storage_identity()
    assert ident.format == pd.FORMAT_NAMES[fmt] and ident.n_layers == 2
    if fmt in FORMATS:
        assert ident.signs_hash == signs_fingerprint(signs) and ident.group_size == group
    # another pool of the same identity, other slab size, other rows
    other = pd.SlabPool(2, 32, 8, D, 3, 16, fmt, hadamard_signs=signs, group_size=group)
    new_rows = np.arange(len(blocks), dtype=np.int32)[::-1] * 2 + 1
    other.reserve_rows(int(new_rows.max()) + 1)
    other.import_blocks(ident, i32(new_rows), pool.export_blocks(i32(blocks)))
    assert np.array_equal(other.export_blocks(i32(new_rows)).cpu().numpy(), got)
    # the same sequences gather identically through the remapped tables
    remap = dict(zip(blocks.tolist(), new_rows.tolist()))
    table_a = make_block_table(rows)
    table_b = np.where(table_a >= 0, np.vectorize(lambda r: remap.get(int(r), -1))(table_a), -1).astype(np.int32)
    t_out = max(lengths)
    for layer in range(2):
        outs = []
        for p, t in ((pool, table_a), (other, table_b)):
            k = torch.zeros((len(lengths), 8, t_out, pool.k_record_bytes), dtype=torch.uint8, device="cuda")
            v = torch.zeros((len(lengths), 8, t_out, pool.v_record_bytes), dtype=torch.uint8, device="cuda")
            p.gather_visible(layer, i32(t), i32(lengths), t_out, k, v)
            outs.append((k.cpu().numpy(), v.cpu().numpy()))
        assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert pool.check_error() == 0 and other.check_error() == 0
    pool.close()
    other.close()


def test_decode_after_restore_is_bit_identical():
    """A checkpoint written from one pool and restored into a fresh pool with
    another slab size: paged_decode over the restored rows gives the same
    bits (determinism independent of physical rows and slabs)."""
    lengths = [700, 65, 1]
    pool, model, rows, R, _ = _pools("bf16", 128, lengths, 8, 41)
    blocks = np.concatenate(rows).astype(np.int32)
    import tempfile, os
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "blocks.pdkv")
        pool.save_checkpoint(path, i32(blocks))
        fresh = pd.SlabPool(2, 32, 8, 128, 5, 32, "bf16")
        new_rows = np.arange(3, 3 + len(blocks), dtype=np.int32)
        fresh.restore_checkpoint(path, i32(new_rows))
    remap = dict(zip(blocks.tolist(), new_rows.tolist()))
    table_a = make_block_table(rows)
    table_b = np.where(table_a >= 0, np.vectorize(lambda r: remap.get(int(r), -1))(table_a), -1).astype(np.int32)
    q = to_device_bits(q_bits(41, 1, 3, 16, 128, "bf16"), "bf16")
    outs = []
    for p, t in ((pool, table_a), (fresh, table_b)):
        out = torch.empty_like(q)
        ws = p.workspace(3, 16, max(lengths))
        p.paged_decode(1, q, i32(t), i32(lengths), max(lengths), 1 / np.sqrt(128), out, ws)
        outs.append(out.view(torch.int16).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    pool.close()
    fresh.close()


@pytest.mark.parametrize("change", ["format", "head_dim", "signs", "n_layers", "n_kv_heads", "group_size"])
def test_incompatible_identity_is_rejected_before_anything_happens(change):
    lengths = [64, 40]
    D = 128 if change == "group_size" else 64  # groups of 64 need head_dim >= 128
    pool, model, rows, R, signs = _pools("k4v4", D, lengths, 4, 77)
    blocks = np.concatenate(rows).astype(np.int32)
    payload = pool.export_blocks(i32(blocks))
    ident = pool.storage_identity()
    kw = dict(n_layers=2, block_size=32, n_kv=8, D=D, fmt="k4v4", signs=signs, group=32)
    if change == "group_size":
        kw["group"] = 64
    elif change == "format":
        kw["fmt"] = "k8v4"
    elif change == "head_dim":
        kw["D"] = 128
        kw["signs"] = hadamard_signs(77, 128)
    elif change == "signs":
        s2 = np.array(signs).copy()
        s2[3] = -s2[3]
        kw["signs"] = s2
    elif change == "n_layers":
        kw["n_layers"] = 3
    else:
        # packed pools hold 8 kv heads (the packed decode kernel's shape), so
        # blocks of another head count arrive as a foreign checkpoint header
        ident.n_kv_heads = 4
    target = pd.SlabPool(kw["n_layers"], kw["block_size"], kw["n_kv"], kw["D"], 4, 16, kw["fmt"],
                         hadamard_signs=kw["signs"], group_size=kw["group"])
    target.reserve_rows(8)
    before = [s.clone() for s in target.k_slabs[0]]
    with pytest.raises(pd.PagedKVError) as e:
        target.import_blocks(ident, i32(np.arange(len(blocks), dtype=np.int32)), payload)
    assert e.value.status == -7
    # a restore checks the identity before it reserves rows or copies bytes
    import tempfile, os
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "blocks.pdkv")
        torch.cuda.synchronize()
        pd.write_checkpoint(path, ident, payload)  # the (possibly foreign) identity the blocks carry
        slabs_before = target.stats()["n_slabs"]
        with pytest.raises(pd.PagedKVError) as e:
            target.restore_checkpoint(path, i32(np.arange(40, 40 + len(blocks), dtype=np.int32)))
        assert e.value.status == -7
        assert target.stats()["n_slabs"] == slabs_before
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(before, target.k_slabs[0]))
    pool.close()
    target.close()


def test_rows_outside_the_pool_are_flagged():
    lengths = [64]
    pool, model, rows, R, _ = _pools("bf16", 128, lengths, 4, 9, n_layers=1)
    out = pool.export_blocks(i32(np.array([int(rows[0][0]), R + 7], np.int32))).cpu().numpy()
    assert pool.check_error() & pd.DEVERR_TABLE_ROW
    assert not out[1].any()                              # the bad block's slot is zeros
    assert np.array_equal(out[0], model.export_blocks([int(rows[0][0])])[0])
    ident = pool.storage_identity()
    pool.import_blocks(ident, i32(np.array([-1], np.int32)), torch.zeros((1, out.shape[1]), dtype=torch.uint8, device="cuda"))
    assert pool.check_error() & pd.DEVERR_WRITE_ROW
    pool.close()
