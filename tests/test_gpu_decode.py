"""paged_decode parity against the fp64 oracle, plus the invariants the
method fixes: one token gives v0, identical keys give mean(V), GQA head
sharing, determinism, independence from physical layout, invisible slots
never read (mlxcel #2171, "Proposed Solution" and "Acceptance Criteria";
mlxcel #235, "Proposed solution: chunked slabs")."""

import numpy as np
import pytest
import torch

import decode_memory_amd as pd
from oracle.attention import decode_attention_bits, widen
from synth import (WORKLOADS, kv_bits_for_sequence, make_block_table, monotone_rows, q_bits,
                   shuffled_rows, workload_lengths)
from tests.gpu_util import (TOL, assert_decode_close, build_pool, from_device_bits, i32,
                            run_decode, to_device_bits, token_targets)

pytestmark = pytest.mark.gpu


def _case(lengths, n_kv, G, D, dtype, bs, S, seed, n_layers=1, layout="monotone", scale=None):
    lengths = [int(x) for x in lengths]
    if layout == "monotone":
        rows = monotone_rows(lengths, bs)
        cap = None
    else:
        rows, _, cap = shuffled_rows(np.random.default_rng(seed), lengths, bs, S, spare_rows=3)
    refs = {}
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    B = len(lengths)

    def on_layer(layer, ks, vs):
        q = q_bits(seed, layer, B, n_kv * G, D, dtype)
        refs[layer] = (q, decode_attention_bits(q, ks, vs, dtype, scale))

    if all(len(r) == 0 for r in rows):
        cap = S
    pool = build_pool(n_layers, lengths, rows, bs, S, n_kv, D, dtype, seed, capacity_rows=cap,
                      on_layer=on_layer)
    table = make_block_table(rows)
    return pool, table, refs, scale


def test_tiny_workload():
    w = WORKLOADS["tiny"]
    pool, table, refs, scale = _case([w.length], w.n_kv_heads, w.group, w.head_dim, w.dtype,
                                     w.block_size, w.slab_blocks, w.seed)
    q, ref = refs[0]
    out = run_decode(pool, 0, q, table, [w.length], w.dtype, scale)
    err = assert_decode_close(out, ref, w.dtype)
    print(f"tiny max-abs {err:.3e}")
    pool.close()


SHAPES = [
    # (D, G, bs, dtype, n_kv).  Block size 32 with a token row of whole 1 KiB
    # wave loads (n_kv * D * 2) takes the row-streaming kernel; the rest take
    # the one-head-per-workgroup kernel.
    (128, 2, 32, "bf16", 8), (128, 2, 32, "fp16", 8), (64, 4, 32, "bf16", 8),
    (256, 4, 32, "bf16", 8), (128, 1, 32, "bf16", 4), (128, 8, 32, "fp16", 4),
    (64, 2, 32, "bf16", 16), (256, 2, 32, "fp16", 2),
    (128, 2, 32, "bf16", 2), (128, 1, 16, "fp16", 2), (128, 8, 64, "bf16", 2),
    (64, 1, 64, "fp16", 2), (256, 2, 16, "bf16", 2), (64, 4, 32, "bf16", 4),
]


@pytest.mark.parametrize("D,G,bs,dtype,n_kv", SHAPES)
def test_shapes_ragged_lengths(D, G, bs, dtype, n_kv):
    lengths = [1, 2, bs - 1, bs + 3, 7 * bs, 300, 1000, 0]
    pool, table, refs, scale = _case(lengths, n_kv, G, D, dtype, bs, 5, 100 + D + G + bs + n_kv,
                                     layout="shuffled")
    q, ref = refs[0]
    out = run_decode(pool, 0, q, table, lengths, dtype, scale)
    assert_decode_close(out, ref, dtype, allow_output_rounding=True)
    # sequences of at least 300 tokens meet the plain bound
    long = [b for b, n in enumerate(lengths) if n >= 300]
    assert_decode_close(out[long], ref[long], dtype)
    assert not widen(out[-1], dtype).any()               # empty sequence -> zeros
    assert pool.check_error() == 0
    pool.close()


def test_one_token_gives_its_value_exactly():
    pool, table, refs, scale = _case([1, 1, 1], 2, 2, 128, "bf16", 32, 4, 7)
    q, ref = refs[0]
    out = run_decode(pool, 0, q, table, [1, 1, 1], "bf16", scale)
    for b in range(3):
        k, v = kv_bits_for_sequence(7, 0, b, 1, 2, 128, "bf16")
        for h in range(4):
            assert np.array_equal(out[b, h], v[0, h // 2])
    pool.close()


def test_identical_keys_give_mean_of_values():
    bs, S, n_kv, D, n = 32, 4, 2, 128, 700
    pool = pd.SlabPool(1, bs, n_kv, D, S, 16, "bf16")
    rows = monotone_rows([n], bs)
    pool.reserve_rows(int(rows[0].max()) + 1)
    k1, v = kv_bits_for_sequence(8, 0, 0, n, n_kv, D, "bf16")
    k = np.broadcast_to(k1[:1], k1.shape).copy()
    r, s = token_targets(rows[0], n, bs)
    pool.write_block(0, i32(r), i32(s), to_device_bits(k, "bf16"), to_device_bits(v, "bf16"))
    q = q_bits(8, 0, 1, 4, D, "bf16")
    out = run_decode(pool, 0, q, make_block_table(rows), [n], "bf16", 1 / np.sqrt(D))
    mean = widen(v, "bf16").mean(axis=0)                 # [n_kv, D]
    for h in range(4):
        assert np.abs(widen(out[0, h], "bf16") - mean[h // 2]).max() <= TOL
    pool.close()


def test_gqa_heads_sharing_a_kv_head_with_equal_queries_agree():
    pool, table, refs, scale = _case([500, 77], 2, 4, 64, "bf16", 32, 4, 9)
    q, _ = refs[0]
    q = q.copy()
    q[:, 1] = q[:, 0]                                    # heads 0 and 1 share kv head 0
    q[:, 6] = q[:, 5]                                    # heads 5 and 6 share kv head 1
    out = run_decode(pool, 0, q, table, [500, 77], "bf16", scale)
    assert np.array_equal(out[:, 1], out[:, 0]) and np.array_equal(out[:, 6], out[:, 5])
    assert not np.array_equal(out[:, 4], out[:, 3])
    pool.close()


def test_row_kernel_with_more_slabs_than_its_lds_table():
    """The row kernel stages the first 1024 slab base pointers of a layer in
    LDS and reads the rest from the pool's table in global memory: one-row
    slabs and a shuffled free list put blocks in slabs on both sides."""
    lengths = [20000, 9000, 5000, 1]
    pool, table, refs, scale = _case(lengths, 8, 2, 128, "bf16", 32, 1, 31, layout="shuffled")
    assert int(table.max()) >= 1024 and int(table[table >= 0].min()) < 1024
    q, ref = refs[0]
    out = run_decode(pool, 0, q, table, lengths, "bf16", scale)
    err = assert_decode_close(out, ref, "bf16", allow_output_rounding=True)
    assert_decode_close(out[:3], ref[:3], "bf16")
    print(f"1068 one-row slabs: max-abs {err:.3e}")
    assert pool.check_error() == 0
    pool.close()


def test_deterministic_and_independent_of_physical_layout():
    lengths = [1500, 333, 2048, 64]
    a = _case(lengths, 4, 2, 128, "bf16", 32, 32, 21, layout="monotone")
    b = _case(lengths, 4, 2, 128, "bf16", 32, 4, 21, layout="shuffled")
    q, ref = a[2][0]
    out_a1 = run_decode(a[0], 0, q, a[1], lengths, "bf16", a[3])
    out_a2 = run_decode(a[0], 0, q, a[1], lengths, "bf16", a[3])
    out_b = run_decode(b[0], 0, q, b[1], lengths, "bf16", b[3])
    assert np.array_equal(out_a1, out_a2)                # run to run
    assert np.array_equal(out_a1, out_b)                 # slabs of 32 rows vs 4, shuffled rows
    assert_decode_close(out_a1, ref, "bf16")
    a[0].close()
    b[0].close()


def test_invisible_slots_are_never_read():
    """Fill the unused tail of every last block with NaN: outputs unchanged."""
    lengths = [45, 100, 33]
    pool, table, refs, scale = _case(lengths, 2, 2, 128, "bf16", 32, 4, 31)
    q, ref = refs[0]
    clean = run_decode(pool, 0, q, table, lengths, "bf16", scale)
    nan = np.full((1, 2, 128), 0x7FC0, np.uint16)
    for b, n in enumerate(lengths):
        row = int(table[b, (n - 1) // 32])
        for slot in range(n % 32 or 32, 32):
            t = to_device_bits(nan, "bf16")
            pool.write_block(0, i32([row]), i32([slot]), t, t)
    poisoned = run_decode(pool, 0, q, table, lengths, "bf16", scale)
    assert np.array_equal(clean, poisoned)
    assert_decode_close(clean, ref, "bf16", allow_output_rounding=True)
    pool.close()


def test_one_workspace_serves_every_layer_and_call():
    """The workspace needs no initialisation: start from garbage (NaN bytes),
    reuse it across layers and calls, and take a larger-than-needed one."""
    lengths = [4096, 1000, 3000]
    pool, table, refs, scale = _case(lengths, 2, 2, 128, "bf16", 32, 32, 41, n_layers=3)
    ws = pool.workspace(3, 4, 4096)
    ws.fill_(0xFF)
    big = torch.full((ws.numel() * 2,), 0xFF, dtype=torch.uint8, device="cuda")
    for rep, w_ in enumerate((ws, big, ws)):
        for layer in range(3):
            q, ref = refs[layer]
            out = run_decode(pool, layer, q, table, lengths, "bf16", scale, workspace=w_)
            assert_decode_close(out, ref, "bf16")
    small = ws[: ws.numel() - 256]
    q, _ = refs[0]
    with pytest.raises(pd.PagedKVError) as e:
        run_decode(pool, 0, q, table, lengths, "bf16", scale, workspace=small)
    assert e.value.status == -3
    pool.close()


def test_qwen3_0p6b_shaped_batch_all_layers():
    """The 8 x 4096 qwen3-0.6b-shaped batch (28 layers) at full size, in the
    benchmark's launch configuration, every output checked."""
    w = WORKLOADS["qwen3_0p6b_8x4k"]
    lengths = [w.length] * w.batch
    pool, table, refs, scale = _case(lengths, w.n_kv_heads, w.group, w.head_dim, w.dtype,
                                     w.block_size, w.slab_blocks, w.seed, n_layers=w.n_layers)
    assert pool.stats()["n_slabs"] == 32
    ws = pool.workspace(w.batch, w.n_q_heads, w.length)
    worst = 0.0
    for layer in range(w.n_layers):
        q, ref = refs[layer]
        out = run_decode(pool, layer, q, table, lengths, w.dtype, scale, workspace=ws)
        worst = max(worst, assert_decode_close(out, ref, w.dtype))
    print(f"qwen3-0.6b-shaped 28 layers: max-abs {worst:.3e}")
    pool.close()
