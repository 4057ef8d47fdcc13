"""The limits of paged_decode: the longest sequence the split plan holds, and
lengths beyond what a call can read.

At block_size 32 the plan holds 64 blocks per split and 1024 splits,
2,097,152 tokens: the only length at which the row kernel and the packed
kernel read 64 blocks per split (the last lane's row and the top bit of the
block mask) and the combine merges 1024 splits (16 per lane).  Keys are all equal there, so the softmax is uniform and
the output is the plain mean of the values, a closed form over the periodic
value pattern (mlxcel #2171, "Proposed Solution": attend(q, k, v, scale,
mask) with one query token; with equal scores it reduces to the mean)."""

import numpy as np
import pytest
import torch

import decode_memory_amd as pd
from oracle.attention import decode_attention_bits, widen
from synth import kv_bits_for_sequence, make_block_table, monotone_rows, q_bits
from tests.gpu_util import assert_decode_close, from_device_bits, i32, to_device_bits

pytestmark = pytest.mark.gpu

BS = 32
MAX_LEN = 64 * 1024 * BS  # blocks per split x splits x block_size


def _bf16(x):
    b = np.asarray(x, np.float32).view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fused", [False, True])
def test_longest_sequence_the_plan_holds(fused):
    n, n_kv, D, P = MAX_LEN, 8, 64, 7
    rng = np.random.default_rng(12)
    kvec = _bf16(rng.standard_normal((n_kv, D)))           # every token's key
    pattern = _bf16(rng.standard_normal((P, n_kv, D)))     # V[t, h] = pattern[(3t + h) % P, h]
    t = np.arange(n)
    sel = (3 * t[:, None] + np.arange(n_kv)[None, :]) % P  # [n, n_kv]
    v_bits = pattern[sel, np.arange(n_kv)[None, :]]       # [n, n_kv, D]
    k_bits = np.broadcast_to(kvec, (n, n_kv, D))
    rows = monotone_rows([n], BS)
    S = 512
    pool = pd.SlabPool(1, BS, n_kv, D, S, n // BS // S + 1, "bf16")
    pool.reserve_rows(n // BS)
    written = n - 1 if fused else n
    pool.write_block(0, i32(rows[0][t[:written] // BS]), i32(t[:written] % BS),
                     to_device_bits(np.ascontiguousarray(k_bits[:written]), "bf16"),
                     to_device_bits(np.ascontiguousarray(v_bits[:written]), "bf16"))
    q = to_device_bits(q_bits(12, 0, 1, n_kv, D, "bf16"), "bf16")
    out = torch.empty_like(q)
    ws = pool.workspace(1, n_kv, n)
    table, lens = i32(make_block_table(rows)), i32([n])
    if fused:
        pool.paged_decode_append(0, q, to_device_bits(kvec[None], "bf16"),
                                 to_device_bits(np.ascontiguousarray(v_bits[n - 1:]), "bf16"),
                                 table, lens, n, 1 / 8, out, ws)
    else:
        pool.paged_decode(0, q, table, lens, n, 1 / 8, out, ws)
    torch.cuda.synchronize()
    assert pool.check_error() == 0
    # closed form: the mean over tokens of the value pattern, per kv head
    ref = np.empty((1, n_kv, D))
    for h in range(n_kv):
        counts = np.bincount(sel[:, h], minlength=P).astype(np.float64)
        ref[0, h] = counts @ widen(pattern[:, h], "bf16") / n
    assert_decode_close(from_device_bits(out), ref, "bf16", allow_output_rounding=True)
    pool.close()


def test_lengths_beyond_the_call_are_clamped_and_flagged():
    """lens[b] beyond what the call's plan holds is clamped to it (the device
    error word says so), a negative length reads nothing, and the host
    rejects a max_len beyond the longest plan."""
    n_kv, G, D = 8, 2, 128
    lengths = [600, 50]
    rows = monotone_rows(lengths, BS)
    pool = pd.SlabPool(1, BS, n_kv, D, 8, 8, "bf16")
    pool.reserve_rows(int(max(r.max() for r in rows)) + 1)
    ks, vs = [], []
    for b, n in enumerate(lengths):
        k, v = kv_bits_for_sequence(31, 0, b, n, n_kv, D, "bf16")
        ks.append(k)
        vs.append(v)
        tt = np.arange(n)
        pool.write_block(0, i32(rows[b][tt // BS]), i32(tt % BS), to_device_bits(k, "bf16"),
                         to_device_bits(v, "bf16"))
    qb = q_bits(31, 0, 2, n_kv * G, D, "bf16")
    q = to_device_bits(qb, "bf16")
    out = torch.empty_like(q)
    table = make_block_table(rows)
    # max_len 100: 4 blocks, one per split, so the call holds 128 tokens
    pool.paged_decode(0, q, i32(table), i32([600, -5]), 100, 1 / np.sqrt(D), out,
                      pool.workspace(2, n_kv * G, 100))
    torch.cuda.synchronize()
    assert pool.check_error() == pd.DEVERR_LENGTH
    got = from_device_bits(out)
    ref = decode_attention_bits(qb[:1], [ks[0][:128]], [vs[0][:128]], "bf16", 1 / np.sqrt(D))
    assert_decode_close(got[:1], ref, "bf16", allow_output_rounding=True)
    assert not got[1].any()
    with pytest.raises(pd.PagedKVError) as e:
        pool.paged_decode(0, q, i32(np.zeros((2, MAX_LEN // BS + 1), np.int32)), i32([1, 1]),
                          MAX_LEN + 1, 0.1, out, pool.workspace(2, n_kv * G, 100))
    assert e.value.status == -4
    pool.close()


@pytest.mark.parametrize("fmt,fused", [("k4v4", False), ("k8v8", False), ("k4v4", True)])
def test_longest_packed_sequence_the_plan_holds(fmt, fused):
    """The packed kernel at the longest plan (1024 splits of 64 blocks): equal
    keys give equal scores, so the output is the mean of the dequantised
    value records (mlx-swift-lm PR #142, "Add packed paged KV formats with
    bounded workspace admission", section "Summary": attention reads the
    packed pages directly), here a closed form over the periodic pattern.
    Fused, the last token (block 65535: split 1023's 64th block) is quantised
    and stored by the decode launch itself."""
    from oracle.packed import FORMATS, dequantise_records, v_records
    from synth import hadamard_signs
    n, n_kv, G, D, P = MAX_LEN, 8, 4, 64, 5
    vb = FORMATS[fmt][1]
    rng = np.random.default_rng(13)
    kvec = _bf16(rng.standard_normal((n_kv, D)))
    pattern = _bf16(rng.standard_normal((P, n_kv, D)))
    t = np.arange(n)
    sel = (2 * t[:, None] + np.arange(n_kv)[None, :]) % P
    v_bits = pattern[sel, np.arange(n_kv)[None, :]]
    k_bits = np.broadcast_to(kvec, (n, n_kv, D))
    rows = monotone_rows([n], BS)
    signs = hadamard_signs(13, D)
    S = 512
    pool = pd.SlabPool(1, BS, n_kv, D, S, n // BS // S + 1, fmt, hadamard_signs=signs)
    pool.reserve_rows(n // BS)
    written = n - 1 if fused else n
    pool.write_block(0, i32(rows[0][t[:written] // BS]), i32(t[:written] % BS),
                     to_device_bits(np.ascontiguousarray(k_bits[:written]), "bf16"),
                     to_device_bits(np.ascontiguousarray(v_bits[:written]), "bf16"))
    q = to_device_bits(q_bits(13, 0, 1, n_kv * G, D, "bf16"), "bf16")
    out = torch.empty_like(q)
    table, lens, ws = i32(make_block_table(rows)), i32([n]), pool.workspace(1, n_kv * G, n)
    if fused:
        pool.paged_decode_append(0, q, to_device_bits(kvec[None], "bf16"),
                                 to_device_bits(np.ascontiguousarray(v_bits[n - 1:]), "bf16"),
                                 table, lens, n, 1 / 8, out, ws)
    else:
        pool.paged_decode(0, q, table, lens, n, 1 / 8, out, ws)
    torch.cuda.synchronize()
    assert pool.check_error() == 0
    deq = dequantise_records(v_records(pattern, vb), D, vb)  # [P, n_kv, D]
    ref = np.empty((1, n_kv * G, D))
    for h in range(n_kv):
        counts = np.bincount(sel[:, h], minlength=P).astype(np.float64)
        ref[0, h * G:(h + 1) * G] = counts @ deq[:, h] / n
    assert_decode_close(from_device_bits(out), ref, "bf16", allow_output_rounding=True)
    pool.close()
