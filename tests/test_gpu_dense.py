"""Dense decode beside paged (mlxcel #2171, "refactor: one KV storage
abstraction with dense and paged backends", sections "Proposed Solution"
and "Acceptance Criteria": one attend over dense or paged storage, and the
two give identical results in a deterministic mode).  The dense call reads
per-sequence contiguous K/V; it is checked bit for bit against paged decode
over the same tokens held in shuffled pool rows, and against the oracle."""

import numpy as np
import pytest
import torch

import decode_memory_amd as pd
from oracle.attention import decode_attention_bits, widen
from synth import kv_bits_for_sequence, make_block_table, q_bits, shuffled_rows
from tests.gpu_util import (assert_decode_close, build_pool, from_device_bits, i32,
                            run_decode, to_device_bits)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,G,n_kv,dtype,lengths", [
    (128, 2, 8, "bf16", [4096] * 8),                       # the qwen3-shaped batch, one layer
    (128, 2, 8, "bf16", [1, 31, 33, 1000, 0, 2500]),
    (64, 4, 8, "fp16", [300, 77, 4096]),
    (256, 8, 2, "bf16", [5000, 1]),
    (128, 1, 4, "fp16", [64, 65, 2047]),
])
def test_dense_is_bit_identical_to_paged(D, G, n_kv, dtype, lengths):
    seed = 500 + D + G
    B, n_q = len(lengths), n_kv * G
    rows, _, R = shuffled_rows(np.random.default_rng(seed), lengths, 32, 4, spare_rows=5)
    seqs = {}

    def keep(layer, ks, vs):
        seqs["k"], seqs["v"] = ks, vs

    pool = build_pool(1, lengths, rows, 32, 4, n_kv, D, dtype, seed, capacity_rows=R, on_layer=keep)
    q = q_bits(seed, 0, B, n_q, D, dtype)
    scale = 1 / np.sqrt(D)
    paged = run_decode(pool, 0, q, make_block_table(rows), lengths, dtype, scale)

    ks = [to_device_bits(k, dtype) if len(k) else torch.zeros((1, n_kv, D), dtype=torch.bfloat16 if dtype == "bf16" else torch.float16, device="cuda") for k in seqs["k"]]
    vs = [to_device_bits(v, dtype) if len(v) else torch.zeros_like(ks[0]) for v in seqs["v"]]
    qd = to_device_bits(q, dtype)
    out = torch.empty_like(qd)
    ml = max(lengths)
    ws = torch.zeros(pd.dense_workspace_bytes(dtype, n_kv, D, B, n_q, ml), dtype=torch.uint8, device="cuda")
    ptrs = pd.dense_pointers(ks, vs)  # built once; the calls allocate nothing
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    pd.dense_decode(qd, ptrs, n_kv, lens, ml, scale, out, ws)
    torch.cuda.synchronize()
    dense = from_device_bits(out)
    assert np.array_equal(dense, paged)
    # on another stream, with the same pointer table
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out_side, ws_side = torch.full_like(out, 7), torch.zeros_like(ws)
    pd.dense_decode(qd, ptrs, n_kv, lens, ml, scale, out_side, ws_side, stream=side)
    side.synchronize()
    assert torch.equal(out_side, out)
    ref = decode_attention_bits(q, seqs["k"], seqs["v"], dtype, scale)
    assert_decode_close(dense, ref, dtype, allow_output_rounding=True)
    for b, n in enumerate(lengths):
        if n == 0:
            assert not widen(dense[b], dtype).any()
    assert pool.check_error() == 0
    pool.close()


def test_dense_rejects_shapes_without_the_row_kernel():
    with pytest.raises(pd.PagedKVError) as e:
        pd.dense_workspace_bytes("bf16", 2, 128, 1, 4, 100)   # 2 x 128 x 2 bytes: half a 1 KiB row
    assert e.value.status == -4
    with pytest.raises(pd.PagedKVError) as e:
        pd.dense_workspace_bytes("k4v4", 8, 64, 1, 32, 100)
    assert e.value.status == -4


def test_dense_decode_checks_its_pointer_table():
    q = torch.zeros((2, 16, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    lens = torch.tensor([5, 5], dtype=torch.int32, device="cuda")
    ws = torch.zeros(pd.dense_workspace_bytes("bf16", 8, 128, 2, 16, 5), dtype=torch.uint8, device="cuda")
    bad = torch.zeros(3, dtype=torch.int64, device="cuda")  # [2, B] needs 4 pointers
    with pytest.raises(ValueError):
        pd.dense_decode(q, bad, 8, lens, 5, 0.1, out, ws)
