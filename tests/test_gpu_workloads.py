"""The fragmented pool (decode steps with growth) and the long-context
workload at their full sizes (mlxcel #235, "Proposed solution: chunked
slabs" and "Acceptance criteria": gather over an interleaved block table is
byte-identical; growth appends slabs during decode without copying)."""

import numpy as np
import pytest
import torch

import decode_memory_amd as pd
from oracle.attention import decode_attention_bits
from synth import (WORKLOADS, kv_bits_for_sequence, make_block_table, monotone_rows,
                   normal_device, q_bits, shuffled_rows, workload_lengths)
from tests.gpu_util import (assert_decode_close, from_device_bits, i32, to_device_bits,
                            token_targets)

pytestmark = pytest.mark.gpu


def _run_fragmented(lengths, spare_rows, steps, seed_tag, allow_output_rounding=False):
    """Write the history of every sequence into rows popped from a shuffled
    free list, then run decode steps: each step appends one token per sequence
    (a new row at each block boundary, a new slab when the free list is empty),
    writes the tokens with one write_block call and decodes the batch."""
    w = WORKLOADS["fragmented_64"]
    bs, S, n_kv, D, G = w.block_size, w.slab_blocks, w.n_kv_heads, w.head_dim, w.group
    B = len(lengths)
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, seed_tag]))
    rows, free, R = shuffled_rows(rng, lengths, bs, S, spare_rows=spare_rows)
    rows = [list(r) for r in rows]
    pool = pd.SlabPool(1, bs, n_kv, D, S, R // S + 8, w.dtype)
    pool.reserve_rows(R)
    kv = [kv_bits_for_sequence(w.seed, 0, b, int(n) + steps, n_kv, D, w.dtype)
          for b, n in enumerate(lengths)]
    for b, n in enumerate(lengths):
        r, s = token_targets(np.asarray(rows[b]), int(n), bs)
        pool.write_block(0, i32(r), i32(s), to_device_bits(kv[b][0][:n], w.dtype),
                         to_device_bits(kv[b][1][:n], w.dtype))
    appended = 0
    lens = [int(n) for n in lengths]
    max_blocks = max(-(-(n + steps) // bs) for n in lens)
    ws = pool.workspace(B, n_kv * G, max(lens) + steps)
    worst = 0.0
    for step in range(steps):
        new_rows, new_slots = [], []
        for b in range(B):
            pos = lens[b]
            if pos % bs == 0:                      # crossing into a new block
                if not free:                       # free list empty: grow the pool
                    first = pool.append_slab() * S
                    free.extend(range(first, first + S))
                    appended += 1
                rows[b].append(free.pop(0))
            new_rows.append(rows[b][pos // bs])
            new_slots.append(pos % bs)
        k_new = np.stack([kv[b][0][lens[b]] for b in range(B)])
        v_new = np.stack([kv[b][1][lens[b]] for b in range(B)])
        pool.write_block(0, i32(new_rows), i32(new_slots), to_device_bits(k_new, w.dtype),
                         to_device_bits(v_new, w.dtype))
        lens = [n + 1 for n in lens]
        q = q_bits(w.seed, 100 + step, B, n_kv * G, D, w.dtype)
        qd = to_device_bits(q, w.dtype)
        out = torch.empty_like(qd)
        table = make_block_table([np.asarray(r, np.int32) for r in rows], max_blocks)
        pool.paged_decode(0, qd, i32(table), i32(lens), max(lens), w.scale, out, ws)
        got = from_device_bits(out)
        ref = decode_attention_bits(q, [kv[b][0][:lens[b]] for b in range(B)],
                                    [kv[b][1][:lens[b]] for b in range(B)], w.dtype, w.scale)
        worst = max(worst, assert_decode_close(got, ref, w.dtype,
                                               allow_output_rounding=allow_output_rounding))
    assert pool.check_error() == 0
    st = pool.stats()
    assert st["slab_append_events"] == R // S + appended and st["bytes_copied_on_growth"] == 0
    pool.close()
    return worst, appended


def test_fragmented_pool_decode_steps_full_size():
    """64 sequences, lengths uniform in [512, 16384], rows from a shuffled free
    list with 64 spare rows (rounded up to whole slabs), 2 decode steps."""
    w = WORKLOADS["fragmented_64"]
    worst, _ = _run_fragmented(workload_lengths(w), 64, 2, 1 << 23)
    print(f"fragmented pool: max-abs {worst:.2e}")


def test_fragmented_pool_grows_during_decode():
    """No spare rows: block-boundary crossings drain the free list and the
    pool appends slabs between decode steps; results stay exact.  Sequences
    are short here (63..991 tokens), so outputs are large and the final bf16
    rounding (half an ulp) is allowed on top of the bound."""
    w = WORKLOADS["fragmented_64"]
    lengths = (workload_lengths(w) // 16 // 32) * 32 + 31  # every sequence crosses at step 1
    worst, appended = _run_fragmented(lengths, 0, 3, 1 << 24, allow_output_rounding=True)
    assert appended >= 1


def _dense_from_device(layer, b, n, n_kv, D, seed):
    k = normal_device((seed, layer, b, 0), (n, n_kv, D), "bf16", "cuda")
    v = normal_device((seed, layer, b, 1), (n, n_kv, D), "bf16", "cuda")
    return k, v


@pytest.mark.parametrize("layout", ["monotone", "shuffled"])
def test_long_context_workload(layout):
    """32 x 16384 tokens in a 28-layer pool (the qwen3-1.7b-shaped long
    context); layers 0 and 27 are filled.  gather_visible of all 32 sequences
    to [32, 8, 16384, 128] is byte-identical to the dense source; paged_decode
    of every sequence matches the oracle and is bit-identical to dense_decode
    over the dense source."""
    w = WORKLOADS["qwen3_1p7b_32x16k"]
    B, n, bs, S, n_kv, D = w.batch, w.length, w.block_size, w.slab_blocks, w.n_kv_heads, w.head_dim
    n_layers = w.n_layers if layout == "monotone" else 1
    layers = (0, w.n_layers - 1) if layout == "monotone" else (0,)
    if layout == "monotone":
        rows = monotone_rows([n] * B, bs)
        R = int(rows[-1].max()) + 1
    else:
        rows, _, R = shuffled_rows(np.random.default_rng(w.seed), [n] * B, bs, S, spare_rows=0)
    pool = pd.SlabPool(n_layers, bs, n_kv, D, S, R // S + 2, w.dtype)
    pool.reserve_rows(R)
    table = i32(make_block_table(rows))
    lens = i32([n] * B)
    ws = pool.workspace(B, w.n_q_heads, n)
    for layer in layers:
        dense_k, dense_v = [], []
        for b in range(B):
            k, v = _dense_from_device(layer, b, n, n_kv, D, w.seed)
            r, s = token_targets(rows[b], n, bs)
            pool.write_block(layer, i32(r), i32(s), k, v)
            dense_k.append(k)
            dense_v.append(v)
        gk = torch.empty((B, n_kv, n, D), dtype=torch.bfloat16, device="cuda")
        gv = torch.empty_like(gk)
        runs = torch.empty(B, dtype=torch.int32, device="cuda")
        pool.gather_visible(layer, table, lens, n, gk, gv, runs)
        for b in range(B):
            assert torch.equal(gk[b].view(torch.int16), dense_k[b].transpose(0, 1).view(torch.int16)), b
            assert torch.equal(gv[b].view(torch.int16), dense_v[b].transpose(0, 1).view(torch.int16)), b
        if layout == "monotone":
            assert runs.cpu().tolist() == [n // bs // S] * B       # 16 same-slab runs each
        del gk, gv
        q = q_bits(w.seed, layer, B, w.n_q_heads, D, w.dtype)
        qd = to_device_bits(q, w.dtype)
        out = torch.empty_like(qd)
        pool.paged_decode(layer, qd, table, lens, n, w.scale, out, ws)
        got = from_device_bits(out)
        # every sequence: the dense backend over the dense source gives the same bits
        dws = torch.zeros(pd.dense_workspace_bytes(w.dtype, n_kv, D, B, w.n_q_heads, n), dtype=torch.uint8,
                          device="cuda")
        dout = torch.empty_like(qd)
        pd.dense_decode(qd, pd.dense_pointers(dense_k, dense_v), n_kv, lens, n, w.scale, dout, dws)
        assert torch.equal(dout.view(torch.int16), out.view(torch.int16))
        del dws, dout
        err = 0.0
        for b0 in range(0, B, 8):  # the oracle over every sequence, 8 at a time
            part = list(range(b0, min(B, b0 + 8)))
            ks = [from_device_bits(dense_k[b]) for b in part]
            vs = [from_device_bits(dense_v[b]) for b in part]
            ref = decode_attention_bits(q[part], ks, vs, w.dtype, w.scale)
            err = max(err, assert_decode_close(got[part], ref, w.dtype))
            del ks, vs, ref
        print(f"long context {layout} layer {layer}: max-abs {err:.2e} over all {B} sequences")
        del dense_k, dense_v
    assert pool.check_error() == 0
    pool.close()
