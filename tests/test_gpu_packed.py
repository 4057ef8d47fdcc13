"""Packed KV formats on the device against the oracle (mlx-swift-lm PR #142,
"Add packed paged KV formats with bounded workspace admission", section
"Summary"): the quantising write_block produces the oracle's records byte for
byte, gather_visible moves packed records bit-exactly, and paged_decode over
the packed pages matches the oracle's fp64 attention over the same records
(the oracle quantises the same bf16 inputs itself; nothing it reads comes
from the device)."""

import numpy as np
import pytest
import torch

import decode_memory_amd as pd
from oracle.packed import FORMATS, k_records, packed_decode_attention, record_bytes, v_records
from oracle.slab_pool import SlabPoolModel
from synth import (WORKLOADS, bf16_bits_from_f32, hadamard_signs, kv_bits_for_sequence, make_block_table,
                   monotone_rows, q_bits, ranged_bits, shuffled_rows)
from tests.gpu_util import (assert_decode_close, assert_packed_close, from_device_bits, i32,
                            packed_decode_bound, to_device_bits, token_targets)

pytestmark = pytest.mark.gpu

BS = 32


def _packed_pool(fmt, D, lengths, rows, seed, cap, n_kv=8, keep=None, slab_blocks=32, group=32):
    """Write every sequence through the quantising write_block; return the pool,
    the oracle's records of the sequences in `keep` and the sign vector."""
    kb, vb = FORMATS[fmt]
    signs = hadamard_signs(seed, D)
    pool = pd.SlabPool(1, BS, n_kv, D, slab_blocks, -(-cap // slab_blocks) + 2, fmt,
                       hadamard_signs=signs, group_size=group)
    pool.reserve_rows(cap)
    recs = {}
    for b, n in enumerate(lengths):
        if n == 0:
            continue
        k, v = kv_bits_for_sequence(seed, 0, b, int(n), n_kv, D, "bf16")
        r, s = token_targets(rows[b], int(n), BS)
        pool.write_block(0, i32(r), i32(s), to_device_bits(k, "bf16"), to_device_bits(v, "bf16"))
        if keep is None or b in keep:
            recs[b] = (k_records(k, signs, kb, group), v_records(v, vb, group))
    torch.cuda.synchronize()
    return pool, recs, signs


@pytest.mark.parametrize("fmt", ["k8v8", "k8v4", "k4v4"])
@pytest.mark.parametrize("D,group", [(64, 32), (128, 32), (256, 32), (128, 64), (256, 64)])
def test_quantising_write_and_gather_are_bit_exact(fmt, D, group):
    kb, vb = FORMATS[fmt]
    lengths = [70, 1, 33, 0, 256]
    rows, _, R = shuffled_rows(np.random.default_rng(D), lengths, BS, 32, spare_rows=2)
    pool, recs, _ = _packed_pool(fmt, D, lengths, rows, 50 + D, R, group=group)
    krec, vrec = record_bytes(D, kb, group), record_bytes(D, vb, group)
    assert pool.group_size == group
    assert pool.k_record_bytes == krec and pool.v_record_bytes == vrec
    model = SlabPoolModel(1, BS, 8, krec, vrec, 32)
    model.reserve_rows(R)
    for b, (kr, vr) in recs.items():
        r, s = token_targets(rows[b], lengths[b], BS)
        model.write(0, r, s, kr, vr)
    for slab in range(model.n_slabs):
        got_k = pool.slab_view(0, slab, "k").cpu().numpy()
        got_v = pool.slab_view(0, slab, "v").cpu().numpy()
        assert np.array_equal(got_k, model.k_slabs[0][slab]), (fmt, D, group, "K", slab)
        assert np.array_equal(got_v, model.v_slabs[0][slab]), (fmt, D, group, "V", slab)
    table = make_block_table(rows)
    t_out = max(lengths)
    gk = torch.empty((len(lengths), 8, t_out, pool.k_record_bytes), dtype=torch.uint8, device="cuda")
    gv = torch.empty((len(lengths), 8, t_out, pool.v_record_bytes), dtype=torch.uint8, device="cuda")
    pool.gather_visible(0, i32(table), i32(lengths), t_out, gk, gv)
    ek, ev = model.gather_batched(0, table, lengths, t_out)
    assert np.array_equal(gk.cpu().numpy(), ek) and np.array_equal(gv.cpu().numpy(), ev)
    assert pool.check_error() == 0
    pool.close()


def _extreme_vectors(seed, n_tok, D, group, levels):
    """[n_tok, 8, D] float32 vectors whose groups probe the quantiser's edges:
    uniform groups at amplitudes from subnormal (1e-40) through 1e-37 (scale
    below 2^-125 or subnormal) to 1e35 (the rotation of 256 such values stays
    finite), constant groups (0.75 and +0), groups
    one bf16 ulp wide, and groups of exact half-integer quotients (min 0, max
    2^bits - 1, so scale is 1 and round-half-even decides)."""
    rng = np.random.default_rng(seed)
    amps = [1e-40, 1e-39, 4e-39, 2e-38, 1e-37, 1.0, 1e35]
    x = rng.uniform(-1.0, 1.0, size=(n_tok, 8, D // group, group)).astype(np.float32)
    kind = rng.integers(0, len(amps) + 4, size=(n_tok, 8, D // group))
    for k, a in enumerate(amps):
        x[kind == k] *= np.float32(a)
    x[kind == len(amps)] = np.float32(0.75)
    x[kind == len(amps) + 1] = np.float32(0.0)
    ulp = kind == len(amps) + 2                       # 1.0 and the next bf16 value
    x[ulp] = np.where(rng.random(x[ulp].shape) < 0.5, np.float32(1.0), np.float32(1.0078125))
    ties = kind == len(amps) + 3
    top = min(levels, 127)                            # k + 1/2 exact in bf16 for k < 128
    halves = rng.integers(0, top, size=x[ties].shape).astype(np.float32) + np.float32(0.5)
    halves[:, 0], halves[:, 1] = 0.0, float(levels)
    x[ties] = halves
    return x.reshape(n_tok, 8, D)


@pytest.mark.parametrize("fmt", ["k8v8", "k8v4", "k4v4"])
@pytest.mark.parametrize("D,group", [(64, 32), (256, 32), (128, 64)])
def test_quantising_write_extreme_ranges_bit_exact(fmt, D, group):
    """The quantising write at the edges of fp32: subnormal inputs and scales
    (whose reciprocal overflows, so the codes come from the correctly rounded
    division), wide groups, constant and one-ulp groups and exact ties.  The
    records equal the oracle's byte for byte."""
    kb, vb = FORMATS[fmt]
    n = 300
    k = bf16_bits_from_f32(_extreme_vectors(900 + D, n, D, group, (1 << kb) - 1))
    v = bf16_bits_from_f32(_extreme_vectors(901 + D, n, D, group, (1 << vb) - 1))
    signs = hadamard_signs(77, D)
    rows = monotone_rows([n], BS)[0]
    R = len(rows)
    pool = pd.SlabPool(1, BS, 8, D, 4, -(-R // 4) + 1, fmt, hadamard_signs=signs, group_size=group)
    pool.reserve_rows(R)
    r, sl = token_targets(rows, n, BS)
    pool.write_block(0, i32(r), i32(sl), to_device_bits(k, "bf16"), to_device_bits(v, "bf16"))
    torch.cuda.synchronize()
    krec, vrec = record_bytes(D, kb, group), record_bytes(D, vb, group)
    model = SlabPoolModel(1, BS, 8, krec, vrec, 4)
    model.reserve_rows(R)
    model.write(0, r, sl, k_records(k, signs, kb, group), v_records(v, vb, group))
    for slab in range(model.n_slabs):
        assert np.array_equal(pool.slab_view(0, slab, "k").cpu().numpy(), model.k_slabs[0][slab]), (fmt, D, "K", slab)
        assert np.array_equal(pool.slab_view(0, slab, "v").cpu().numpy(), model.v_slabs[0][slab]), (fmt, D, "V", slab)
    assert pool.check_error() == 0
    pool.close()


@pytest.mark.parametrize("fmt", ["k8v8", "k8v4", "k4v4"])
@pytest.mark.parametrize("D,G,group", [(64, 4, 32), (256, 4, 32), (128, 2, 32), (64, 1, 32),
                                       (128, 4, 64), (256, 2, 64), (256, 1, 64)])
def test_packed_decode_matches_oracle(fmt, D, G, group):
    lengths = [300, 1, 45, 0, 1024, 64]
    rows, _, R = shuffled_rows(np.random.default_rng(D + G), lengths, BS, 32, spare_rows=2)
    pool, recs, signs = _packed_pool(fmt, D, lengths, rows, 60 + D + G, R, group=group)
    B = len(lengths)
    q = q_bits(60 + D + G, 0, B, 8 * G, D, "bf16")
    scale = 1.0 / np.sqrt(D)
    kr = [recs[b][0] if b in recs else np.zeros((0, 8, pool.k_record_bytes), np.uint8) for b in range(B)]
    vr = [recs[b][1] if b in recs else np.zeros((0, 8, pool.v_record_bytes), np.uint8) for b in range(B)]
    ref = packed_decode_attention(q, kr, vr, signs, fmt, D, scale, group)
    qd = to_device_bits(q, "bf16")
    out = torch.empty_like(qd)
    ws = pool.workspace(B, 8 * G, max(lengths))
    pool.paged_decode(0, qd, i32(make_block_table(rows)), i32(lengths), max(lengths), scale, out, ws)
    got = from_device_bits(out)
    assert_decode_close(got, ref, "bf16", allow_output_rounding=True)
    long = [b for b, n in enumerate(lengths) if n >= 300]
    assert_decode_close(got[long], ref[long], "bf16")
    assert not got[3].any()
    assert pool.check_error() == 0
    pool.close()


@pytest.mark.parametrize("fmt,D,G", [("k4v4", 64, 4), ("k8v4", 64, 2), ("k4v4", 256, 1)])
def test_packed_decode_skips_blocks_whose_row_is_outside_the_pool(fmt, D, G):
    """A block whose table row is outside the pool adds nothing (its tokens
    are left out) and the call flags PD_DEVERR_TABLE_ROW; the other blocks of
    its split, before and after it, still count.  At head_dim 64, 16
    sequences of at most 125 blocks plan 32 splits (split s takes blocks s,
    s + 32, s + 64, s + 96), so the bad rows of sequence 0 are the first (5),
    second (38), third (77, 94) and fourth (98, 124) block of their splits,
    94 the last of a split of three; at head_dim 256 the plan has 16 splits of
    up to 8 blocks."""
    lengths = [4000, 700, 100, 33, 17, 0, 64, 5, 300, 1, 2, 90, 45, 31, 32, 200]
    rows, _, R = shuffled_rows(np.random.default_rng(31 + D), lengths, BS, 32, spare_rows=4)
    pool, recs, signs = _packed_pool(fmt, D, lengths, rows, 70 + D, R)
    table = make_block_table(rows)
    bad = {0: [5, 38, 77, 98, 94, 124], 1: [21], 2: [3]}
    for b, blocks in bad.items():
        for j in blocks:
            table[b, j] = -1 if j % 2 else 1_000_000
    B = len(lengths)
    kr, vr = [], []
    for b in range(B):
        if b not in recs:
            kr.append(np.zeros((0, 8, pool.k_record_bytes), np.uint8))
            vr.append(np.zeros((0, 8, pool.v_record_bytes), np.uint8))
            continue
        keep = np.ones(lengths[b], bool)
        for j in bad.get(b, []):
            keep[j * BS:(j + 1) * BS] = False
        kr.append(recs[b][0][keep])
        vr.append(recs[b][1][keep])
    q = q_bits(70 + D, 0, B, 8 * G, D, "bf16")
    scale = 1.0 / np.sqrt(D)
    ref = packed_decode_attention(q, kr, vr, signs, fmt, D, scale)
    qd = to_device_bits(q, "bf16")
    out = torch.empty_like(qd)
    ws = pool.workspace(B, 8 * G, max(lengths))
    pool.paged_decode(0, qd, i32(table), i32(lengths), max(lengths), scale, out, ws)
    got = from_device_bits(out)
    assert pool.check_error() == pd.DEVERR_TABLE_ROW
    assert_decode_close(got, ref, "bf16", allow_output_rounding=True)
    assert_decode_close(got[[0, 1, 8, 15]], ref[[0, 1, 8, 15]], "bf16")
    assert not got[5].any()
    pool.close()


@pytest.mark.parametrize("fmt,D,G", [("k8v4", 64, 4), ("k4v4", 256, 2)])
def test_packed_decode_with_more_slabs_than_its_lds_table(fmt, D, G):
    """The packed kernel stages the first 512 slab base pointers of a layer in
    LDS and reads the rest from the pool's table in global memory: one-row
    slabs and a shuffled free list put blocks in slabs on both sides."""
    lengths = [12000, 5000, 3000, 1]
    rows, _, R = shuffled_rows(np.random.default_rng(7 + D), lengths, BS, 1, spare_rows=8)
    table = make_block_table(rows)
    assert int(table.max()) >= 512 and int(table[table >= 0].min()) < 512
    pool, recs, signs = _packed_pool(fmt, D, lengths, rows, 90 + D, R, slab_blocks=1)
    B = len(lengths)
    q = q_bits(90 + D, 0, B, 8 * G, D, "bf16")
    scale = 1.0 / np.sqrt(D)
    ref = packed_decode_attention(q, [recs[b][0] for b in range(B)], [recs[b][1] for b in range(B)],
                                  signs, fmt, D, scale)
    qd = to_device_bits(q, "bf16")
    out = torch.empty_like(qd)
    ws = pool.workspace(B, 8 * G, max(lengths))
    pool.paged_decode(0, qd, i32(table), i32(lengths), max(lengths), scale, out, ws)
    got = from_device_bits(out)
    err = assert_decode_close(got, ref, "bf16", allow_output_rounding=True)
    assert_decode_close(got[:3], ref[:3], "bf16")
    print(f"packed {fmt} D={D}, {R} one-row slabs: max-abs {err:.2e}")
    assert pool.check_error() == 0
    pool.close()


@pytest.mark.parametrize("fmt,D,group", [(f, d, 32) for f in ("k8v8", "k8v4", "k4v4") for d in (64, 256)]
                         + [("k4v4", 256, 64)])
def test_packed_workload_full_size_sampled(fmt, D, group):
    """The packed workload at full size (16 x 16384 tokens, 8 kv heads, GQA 4):
    every sequence is written and decoded on the device; the oracle checks the
    records and outputs of sequences 0, 5, 10 and 15.  Groups of 64 (K4/V4 at
    five bits per value) run at the same size."""
    w = WORKLOADS["packed_16x16k"]
    lengths = [w.length] * w.batch
    rows = monotone_rows(lengths, BS)
    cap = int(rows[-1].max()) + 1
    sample = (0, 5, 10, w.batch - 1)
    pool, recs, signs = _packed_pool(fmt, D, lengths, rows, w.seed, cap, keep=sample, group=group)
    q = q_bits(w.seed, 0, w.batch, w.n_q_heads, D, "bf16")
    scale = 1.0 / np.sqrt(D)
    qd = to_device_bits(q, "bf16")
    out = torch.empty_like(qd)
    table = make_block_table(rows)
    ws = pool.workspace(w.batch, w.n_q_heads, w.length)
    pool.paged_decode(0, qd, i32(table), i32(lengths), w.length, scale, out, ws)
    got = from_device_bits(out)
    # sampled records, through gather_visible of the sampled sequences
    sub = table[list(sample)]
    gk = torch.empty((len(sample), 8, w.length, pool.k_record_bytes), dtype=torch.uint8, device="cuda")
    gv = torch.empty((len(sample), 8, w.length, pool.v_record_bytes), dtype=torch.uint8, device="cuda")
    pool.gather_visible(0, i32(sub), i32([w.length] * len(sample)), w.length, gk, gv)
    gk, gv = gk.cpu().numpy(), gv.cpu().numpy()
    for i, b in enumerate(sample):
        assert np.array_equal(gk[i], recs[b][0].transpose(1, 0, 2)), (fmt, D, b)
        assert np.array_equal(gv[i], recs[b][1].transpose(1, 0, 2)), (fmt, D, b)
    ref = packed_decode_attention(q[list(sample)], [recs[b][0] for b in sample],
                                  [recs[b][1] for b in sample], signs, fmt, D, scale, group)
    err = assert_decode_close(got[list(sample)], ref, "bf16")
    print(f"packed {fmt} D={D} group {group}: max-abs {err:.2e}")
    assert pool.check_error() == 0
    pool.close()


def _ranged_case(fmt, D, G, group, seed, v_amps=None, q_amp=None):
    """A packed pool over sequences of mixed lengths whose V groups alternate
    between +-v_amps[i] (uniform) and whose query is uniform in +-q_amp (or
    N(0, 1) when not given); returns (device output bits, oracle output,
    per-output bound)."""
    kb, vb = FORMATS[fmt]
    lengths = [300, 1, 45, 0, 1024, 64]
    B = len(lengths)
    rows, _, R = shuffled_rows(np.random.default_rng(seed), lengths, BS, 32, spare_rows=2)
    signs = hadamard_signs(seed, D)
    pool = pd.SlabPool(1, BS, 8, D, 32, -(-R // 32) + 2, fmt, hadamard_signs=signs, group_size=group)
    pool.reserve_rows(R)
    kr, vr = [], []
    for b, n in enumerate(lengths):
        k, v = kv_bits_for_sequence(seed, 0, b, n, 8, D, "bf16")
        if v_amps is not None:
            v = ranged_bits(np.random.SeedSequence([seed, b, 7]), (n, 8, D), group, v_amps)
        kr.append(k_records(k, signs, kb, group))
        vr.append(v_records(v, vb, group))
        if n:
            r, sl = token_targets(rows[b], n, BS)
            pool.write_block(0, i32(r), i32(sl), to_device_bits(k, "bf16"), to_device_bits(v, "bf16"))
    if q_amp is None:
        q = q_bits(seed, 0, B, 8 * G, D, "bf16")
    else:
        q = ranged_bits(np.random.SeedSequence([seed, 1 << 20]), (B, 8 * G, D), D, [q_amp])
    scale = 1.0 / np.sqrt(D)
    qd = to_device_bits(q, "bf16")
    out = torch.empty_like(qd)
    ws = pool.workspace(B, 8 * G, max(lengths))
    pool.paged_decode(0, qd, i32(make_block_table(rows)), i32(lengths), max(lengths), scale, out, ws)
    got = from_device_bits(out)
    assert pool.check_error() == 0
    pool.close()
    ref = packed_decode_attention(q, kr, vr, signs, fmt, D, scale, group)
    return got, ref, packed_decode_bound(q, kr, vr, signs, fmt, D, scale, group)


@pytest.mark.parametrize("fmt", ["k8v8", "k8v4", "k4v4"])
@pytest.mark.parametrize("amp", [600.0, 5000.0, 20000.0])
@pytest.mark.parametrize("D,G,group", [(64, 4, 32), (256, 2, 32), (128, 4, 64)])
def test_packed_decode_wide_value_groups(fmt, amp, D, G, group):
    """V groups spanning +-600, +-5000 and +-20000 next to unit-scale groups
    in the same vectors: the record format takes any finite range (fp32 scale
    and offset per group), so the output must be finite and within the
    arithmetic's bound of the oracle over the same records.  At 4 bits a
    range above about 960 (8 bits: 16,300) took p * scale past f16's range
    before the value prescale was lowered as the groups demand."""
    got, ref, bound = _ranged_case(fmt, D, G, group, 700 + D + G + int(amp) % 97, v_amps=[amp, 1.0])
    worst = assert_packed_close(got, ref, bound)
    print(f"{fmt} D={D} G={G} group {group} V +-{amp:g}: error / allowance {worst:.3f}")


@pytest.mark.parametrize("fmt", ["k8v8", "k8v4", "k4v4"])
@pytest.mark.parametrize("q_amp", [8.0, 1.0e6])
@pytest.mark.parametrize("D,G,group", [(64, 4, 32), (256, 4, 32), (128, 2, 64)])
def test_packed_decode_large_norm_query(fmt, q_amp, D, G, group):
    """Queries uniform in +-8 (a sharp softmax over near-tied scores, where
    the scores' precision shows) and in +-1e6 (|q'| far beyond f16's range:
    the query is prescaled by a power of two, and the softmax is one-hot).
    Every output finite and within the arithmetic's bound of the oracle."""
    got, ref, bound = _ranged_case(fmt, D, G, group, 800 + D + G + int(q_amp) % 89, q_amp=q_amp)
    worst = assert_packed_close(got, ref, bound)
    print(f"{fmt} D={D} G={G} group {group} q +-{q_amp:g}: error / allowance {worst:.3f}")
