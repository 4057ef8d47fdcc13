"""Append then attend in one launch (pd_paged_decode_append) against the two
calls it fuses: pd_write_block of token lens[b] - 1 of every sequence, then
pd_paged_decode (mlxcel #2171, "refactor: one KV storage abstraction with
dense and paged backends", section "Proposed Solution": attend(q, k, v,
scale, mask) takes the new token's K and V; mlxcel #235, "Proposed
solution", touch point 1: the write lands in the slab of its row).  Pool
bytes and outputs are bit-identical to the unfused pair, the outputs are
within tolerance of the oracle's definition over the full sequences, and the
shapes and rows the fused path rejects append nothing."""

import numpy as np
import pytest
import torch

import decode_memory_amd as pd
from oracle.attention import decode_attention_bits
from synth import kv_bits_for_sequence, make_block_table, monotone_rows, q_bits, shuffled_rows
from tests.gpu_util import assert_decode_close, from_device_bits, i32, to_device_bits

pytestmark = pytest.mark.gpu

BS = 32


def _fill(lengths, rows, R, S, n_kv, D, dtype, seed, n_layers=1, fmt=None, signs=None, group=0):
    """A pool holding tokens 0 .. len-2 of every sequence and, in the slot of
    token len-1, the bytes of another token (the append must replace them).
    Returns the pool and the full K/V bit patterns per layer and sequence."""
    pool = pd.SlabPool(n_layers, BS, n_kv, D, S, -(-R // S) + 2, fmt or dtype, hadamard_signs=signs,
                       group_size=group)
    pool.reserve_rows(R)
    kv = []
    for layer in range(n_layers):
        per = []
        for b, n in enumerate(lengths):
            k, v = kv_bits_for_sequence(seed, layer, b, int(n), n_kv, D, dtype)
            per.append((k, v))
            if n == 0:
                continue
            t = np.arange(n)
            kw, vw = k.copy(), v.copy()
            kw[n - 1], vw[n - 1] = k[0], v[n // 2]  # stale bytes where the new token goes
            pool.write_block(layer, i32(rows[b][t // BS]), i32(t % BS), to_device_bits(kw, dtype),
                             to_device_bits(vw, dtype))
        kv.append(per)
    torch.cuda.synchronize()
    return pool, kv


def _new_tokens(kv, layer, lengths, n_kv, D, dtype):
    """[B, n_kv, D] device tensors of token len-1 of every sequence (zeros for
    empty sequences, which append nothing)."""
    kn = np.zeros((len(lengths), n_kv, D), np.uint16)
    vn = np.zeros_like(kn)
    for b, n in enumerate(lengths):
        if n:
            kn[b], vn[b] = kv[layer][b][0][n - 1], kv[layer][b][1][n - 1]
    return to_device_bits(kn, dtype), to_device_bits(vn, dtype)


def _slabs(pool):
    return [s.clone() for s in pool.k_slabs[0] + pool.v_slabs[0]]


@pytest.mark.parametrize("D,G,n_kv,dtype", [(128, 2, 8, "bf16"), (64, 4, 8, "fp16"), (256, 1, 2, "bf16"),
                                            (128, 8, 4, "bf16"), (64, 1, 16, "bf16")])
def test_append_equals_write_then_decode(D, G, n_kv, dtype):
    lengths = [0, 1, 31, 32, 33, 700, 4097]
    seed = 500 + D + G
    rows, _, R = shuffled_rows(np.random.default_rng(seed), lengths, BS, 4, spare_rows=3)
    table = i32(make_block_table(rows))
    lens = i32(lengths)
    B, n_q, ml = len(lengths), n_kv * G, max(lengths)
    qb = q_bits(seed, 0, B, n_q, D, dtype)
    q = to_device_bits(qb, dtype)
    scale = 1 / np.sqrt(D)
    outs, slabs = [], []
    for fused in (False, True):
        pool, kv = _fill(lengths, rows, R, 4, n_kv, D, dtype, seed)
        kn, vn = _new_tokens(kv, 0, lengths, n_kv, D, dtype)
        out = torch.empty_like(q)
        ws = pool.workspace(B, n_q, ml)
        if fused:
            pool.paged_decode_append(0, q, kn, vn, table, lens, ml, scale, out, ws)
        else:
            live = [b for b, n in enumerate(lengths) if n]
            r = i32([int(rows[b][(lengths[b] - 1) // BS]) for b in live])
            s = i32([(lengths[b] - 1) % BS for b in live])
            pool.write_block(0, r, s, kn[live].contiguous(), vn[live].contiguous())
            pool.paged_decode(0, q, table, lens, ml, scale, out, ws)
        torch.cuda.synchronize()
        assert pool.check_error() == 0
        outs.append(from_device_bits(out))
        slabs.append(_slabs(pool))
        pool.close()
    assert np.array_equal(outs[0], outs[1])
    assert all(torch.equal(a, b) for a, b in zip(slabs[0], slabs[1]))
    ref = decode_attention_bits(qb, [k for k, _ in kv[0]], [v for _, v in kv[0]], dtype, scale)
    assert_decode_close(outs[1], ref, dtype, allow_output_rounding=True)


def test_append_with_a_rejected_row_appends_nothing():
    """The new token's block row is outside the pool for one sequence: the
    kernel flags the table row and that sequence's slabs are untouched, while
    the other sequences append."""
    D, G, n_kv, dtype = 128, 2, 8, "bf16"
    lengths = [100, 65]
    rows = monotone_rows(lengths, BS)
    R = int(max(r.max() for r in rows)) + 1
    pool, kv = _fill(lengths, rows, R, 4, n_kv, D, dtype, 61)
    before = _slabs(pool)
    tab = make_block_table(rows)
    tab[1, (lengths[1] - 1) // BS] = R + 50                # beyond capacity_rows
    kn, vn = _new_tokens(kv, 0, lengths, n_kv, D, dtype)
    q = to_device_bits(q_bits(61, 0, 2, n_kv * G, D, dtype), dtype)
    out = torch.empty_like(q)
    pool.paged_decode_append(0, q, kn, vn, i32(tab), i32(lengths), max(lengths), 0.1, out,
                             pool.workspace(2, n_kv * G, max(lengths)))
    assert pool.check_error() == pd.DEVERR_TABLE_ROW
    after = _slabs(pool)
    tok_bytes = n_kv * D * 2
    changed = [i for i, (a, b) in enumerate(zip(before, after)) if not torch.equal(a, b)]
    # only sequence 0's new token changed: one K and one V slab, one token row each
    assert len(changed) == 2
    for i in changed:
        diff = (before[i] != after[i]).nonzero().flatten()
        row0 = int(rows[0][(lengths[0] - 1) // BS]) % 4
        tok = row0 * BS + (lengths[0] - 1) % BS
        assert diff.min() >= tok * tok_bytes and diff.max() < (tok + 1) * tok_bytes
    pool.close()


@pytest.mark.parametrize("fmt,D,G,group", [("k8v8", 64, 4, 32), ("k4v4", 256, 2, 32), ("k8v4", 128, 1, 64),
                                            ("k4v4", 64, 1, 32)])
def test_packed_append_equals_write_then_decode(fmt, D, G, group):
    """Packed pools: the decode kernel's owner workgroup rotates and
    quantises the new token itself (mlx-swift-lm PR #142, "Add packed paged
    KV formats with bounded workspace admission", section "Summary": fresh
    K/V are quantised once); the records it stores are those the quantising
    write_block stores, byte for byte, and so are the outputs."""
    from oracle.packed import FORMATS, k_records, packed_decode_attention, v_records
    from synth import hadamard_signs
    lengths = [0, 1, 31, 32, 33, 700, 2500]
    n_kv, seed = 8, 800 + D + G
    signs = hadamard_signs(seed, D)
    rows, _, R = shuffled_rows(np.random.default_rng(seed), lengths, BS, 4, spare_rows=3)
    table = i32(make_block_table(rows))
    lens = i32(lengths)
    B, n_q, ml = len(lengths), n_kv * G, max(lengths)
    qb = q_bits(seed, 0, B, n_q, D, "bf16")
    q = to_device_bits(qb, "bf16")
    scale = 1 / np.sqrt(D)
    outs, slabs = [], []
    for fused in (False, True):
        pool, kv = _fill(lengths, rows, R, 4, n_kv, D, "bf16", seed, fmt=fmt, signs=signs, group=group)
        kn, vn = _new_tokens(kv, 0, lengths, n_kv, D, "bf16")
        out = torch.empty_like(q)
        ws = pool.workspace(B, n_q, ml)
        if fused:
            pool.paged_decode_append(0, q, kn, vn, table, lens, ml, scale, out, ws)
        else:
            live = [b for b, n in enumerate(lengths) if n]
            r = i32([int(rows[b][(lengths[b] - 1) // BS]) for b in live])
            s = i32([(lengths[b] - 1) % BS for b in live])
            pool.write_block(0, r, s, kn[live].contiguous(), vn[live].contiguous())
            pool.paged_decode(0, q, table, lens, ml, scale, out, ws)
        torch.cuda.synchronize()
        assert pool.check_error() == 0
        outs.append(from_device_bits(out))
        slabs.append(_slabs(pool))
        pool.close()
    assert np.array_equal(outs[0], outs[1])
    assert all(torch.equal(a, b) for a, b in zip(slabs[0], slabs[1]))
    kb, vb = FORMATS[fmt]
    kr = [k_records(k, signs, kb, group) for k, _ in kv[0]]
    vr = [v_records(v, vb, group) for _, v in kv[0]]
    ref = packed_decode_attention(qb, kr, vr, signs, fmt, D, scale, group)
    assert_decode_close(outs[1], ref, "bf16", allow_output_rounding=True)


@pytest.mark.parametrize("case", ["column_kernel", "misaligned"])
def test_append_rejects_what_it_cannot_fuse(case):
    lengths = [40]
    rows = monotone_rows(lengths, BS)
    if case == "column_kernel":                           # 2 x 64 x 2 = 256-byte token rows
        pool = pd.SlabPool(1, BS, 2, 64, 4, 4, "bf16")
        n_kv, D, status = 2, 64, -4
    else:
        pool = pd.SlabPool(1, BS, 8, 128, 4, 4, "bf16")
        n_kv, D, status = 8, 128, -1
    pool.reserve_rows(4)
    q = torch.zeros((1, n_kv, D), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((1, n_kv, D), dtype=torch.bfloat16, device="cuda")
    vn = torch.zeros_like(kn)
    if case == "misaligned":
        buf = torch.zeros(n_kv * D + 8, dtype=torch.bfloat16, device="cuda")
        kn = buf[1:1 + n_kv * D].view(1, n_kv, D)              # 2-byte offset
    before = _slabs(pool)
    with pytest.raises(pd.PagedKVError) as e:
        pd.paged_decode_append(pool.handle, 0, q, kn, vn, i32(make_block_table(rows)), i32(lengths), 40,
                               0.1, torch.empty_like(q), pool.workspace(1, n_kv, 40))
    assert e.value.status == status
    assert all(torch.equal(a, b) for a, b in zip(before, _slabs(pool)))
    pool.close()


@pytest.mark.parametrize("fmt", ["bf16", "k4v4"])
def test_captured_append_step_replays_bit_equal(fmt):
    """Every layer's append-and-attend captured into a HIP graph: each replay,
    with eager steps and synchronisations between replays, gives the eager
    outputs bit for bit (a packed pool quantises the new tokens in the
    replayed launches too)."""
    from synth import hadamard_signs
    packed = fmt != "bf16"
    L, B, n, n_kv, dtype = 3, 4, 700, 8, "bf16"
    G, D = (4, 64) if packed else (2, 128)
    signs = hadamard_signs(71, D) if packed else None
    lengths = [n] * B
    rows = monotone_rows(lengths, BS)
    R = int(max(r.max() for r in rows)) + 1
    pool, kv = _fill(lengths, rows, R, 8, n_kv, D, dtype, 71, n_layers=L, fmt=fmt if packed else None,
                     signs=signs)
    table, lens = i32(make_block_table(rows)), i32(lengths)
    new = [_new_tokens(kv, layer, lengths, n_kv, D, dtype) for layer in range(L)]
    qs = [to_device_bits(q_bits(71, layer, B, n_kv * G, D, dtype), dtype) for layer in range(L)]
    outs = [torch.empty_like(q) for q in qs]
    ws = pool.workspace(B, n_kv * G, n)

    def step():
        for layer in range(L):
            pool.paged_decode_append(layer, qs[layer], new[layer][0], new[layer][1], table, lens, n,
                                     1 / np.sqrt(D), outs[layer], ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        step()
        torch.cuda.synchronize()
        eager = [o.clone() for o in outs]
        for o in outs:
            o.fill_(7)
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(eager, outs))
    qb = q_bits(71, 0, B, n_kv * G, D, dtype)
    if packed:
        from oracle.packed import k_records, packed_decode_attention, v_records
        ref = packed_decode_attention(qb, [k_records(k, signs, 4) for k, _ in kv[0]],
                                      [v_records(v, 4) for _, v in kv[0]], signs, fmt, D, 1 / np.sqrt(D))
    else:
        ref = decode_attention_bits(qb, [k for k, _ in kv[0]], [v for _, v in kv[0]], dtype, 1 / np.sqrt(D))
    assert_decode_close(from_device_bits(outs[0]), ref, dtype)
    assert pool.check_error() == 0
    pool.close()
