"""Footprint of sequential distinct prefills on the device (mlxcel #235,
"Problem" and "Acceptance criteria": 8 distinct ~4k-token prompts that each
extend the pool should peak within about 1.15x of the dense backend; growth
appends slabs and copies nothing).  The expected byte counts come from the
oracle's accounting of the same lengths."""

import gc

import numpy as np
import pytest
import torch

import decode_memory_amd as pd
from oracle.footprint import dense_bytes, growth_by_copy_peak, slab_pool_capacity
from synth import WORKLOADS, kv_bits_for_sequence, workload_lengths
from tests.gpu_util import i32, to_device_bits

pytestmark = pytest.mark.gpu


def test_sequential_distinct_prefills_stay_within_the_gate():
    w = WORKLOADS["footprint_8x4k"]
    L, bs, S, n_kv, D = 4, w.block_size, w.slab_blocks, w.n_kv_heads, w.head_dim
    lengths = [int(x) for x in workload_lengths(w)]
    token_bytes = L * n_kv * D * 2 * 2
    block_bytes = bs * token_bytes
    expect = slab_pool_capacity(lengths, bs, S, block_bytes)

    # tensors of earlier tests that only the cycle collector frees would
    # otherwise be freed during this test and come off the measured footprint
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    pool = pd.SlabPool(L, bs, n_kv, D, S, 64, "bf16")
    rows, last = 0, None
    for i, n in enumerate(lengths):
        nb = -(-n // bs)
        pool.reserve_rows(rows + nb)
        st = pool.stats()
        assert st["bytes_reserved"] == expect[i] and st["bytes_copied_on_growth"] == 0
        t = np.arange(n)
        r, sl = i32(rows + t // bs), i32(t % bs)
        for layer in range(L):
            k, v = kv_bits_for_sequence(w.seed, layer, i, n, n_kv, D, "bf16")
            pool.write_block(layer, r, sl, to_device_bits(k, "bf16"), to_device_bits(v, "bf16"))
            last = (rows, n, k) if layer == L - 1 else last
        rows += nb
        del r, sl
    torch.cuda.synchronize()
    # the slab tensors are the whole pool footprint: exactly the reserved bytes
    assert torch.cuda.memory_allocated() - base == pool.stats()["bytes_reserved"]
    assert pool.stats()["slab_append_events"] == pool.stats()["n_slabs"]
    ratio = pool.stats()["bytes_reserved"] / dense_bytes(lengths, token_bytes)
    ladder = growth_by_copy_peak(lengths, bs, 32, block_bytes) / dense_bytes(lengths, token_bytes)
    print(f"slab pool / dense = {ratio:.4f}; growth-by-copy ladder / dense = {ladder:.2f}")
    assert ratio <= 1.15
    # the last prompt's keys of the last layer read back byte for byte
    r0, n, k = last
    gk = torch.zeros((1, n_kv, n, 2 * D), dtype=torch.uint8, device="cuda")
    gv = torch.zeros_like(gk)
    table = i32(np.arange(r0, r0 + -(-n // bs), dtype=np.int32)[None, :])
    pool.gather_visible(L - 1, table, i32([n]), n, gk, gv)
    got = gk.view(torch.int16).cpu().numpy().view(np.uint16)[0]
    assert np.array_equal(got, np.transpose(k, (1, 0, 2)))
    assert pool.check_error() == 0
    pool.close()
