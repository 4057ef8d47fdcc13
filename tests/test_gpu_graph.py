"""A decode step captured into a HIP graph: write_block of the newest token,
then paged_decode (split and combine) for every layer.  The library launches
on the capturing stream and records no memset; each replay, with eager work
and synchronisations between replays, gives the eager step's outputs bit for
bit."""

import numpy as np
import pytest
import torch

from synth import kv_bits_for_sequence, make_block_table, monotone_rows, q_bits
from tests.gpu_util import build_pool, i32, to_device_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["bf16", "k4v4"])
def test_captured_decode_step_replays_bit_equal(fmt):
    from synth import hadamard_signs
    import decode_memory_amd as pd
    L, B, n, n_kv, G, D = 3, 4, 700, 8, 4 if fmt == "k4v4" else 2, 64 if fmt == "k4v4" else 128
    lengths = [n] * B
    rows = monotone_rows(lengths, 32)
    signs = hadamard_signs(9, D) if fmt == "k4v4" else None
    pool = pd.SlabPool(L, 32, n_kv, D, 8, 16, fmt, hadamard_signs=signs)
    pool.reserve_rows(int(max(r.max() for r in rows)) + 1)
    t = np.arange(n)
    for layer in range(L):
        for b in range(B):
            k, v = kv_bits_for_sequence(9, layer, b, n, n_kv, D, "bf16")
            pool.write_block(layer, i32(rows[b][t // 32]), i32(t % 32), to_device_bits(k, "bf16"),
                             to_device_bits(v, "bf16"))
    table = i32(make_block_table(rows))
    lens = i32(lengths)
    new_rows = i32([int(r[(n - 1) // 32]) for r in rows])
    new_slots = i32([(n - 1) % 32] * B)
    k_new = [to_device_bits(kv_bits_for_sequence(10, layer, 0, B, n_kv, D, "bf16")[0], "bf16") for layer in range(L)]
    v_new = [to_device_bits(kv_bits_for_sequence(10, layer, 0, B, n_kv, D, "bf16")[1], "bf16") for layer in range(L)]
    qs = [to_device_bits(q_bits(9, layer, B, n_kv * G, D, "bf16"), "bf16") for layer in range(L)]
    outs = [torch.empty_like(q) for q in qs]
    ws = pool.workspace(B, n_kv * G, n)

    def step():
        for layer in range(L):
            pool.write_block(layer, new_rows, new_slots, k_new[layer], v_new[layer])
            pool.paged_decode(layer, qs[layer], table, lens, n, 1 / np.sqrt(D), outs[layer], ws)

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
    assert pool.check_error() == 0
    pool.close()
