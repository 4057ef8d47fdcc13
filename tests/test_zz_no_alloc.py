"""pd_paged_decode_noalloc: paged_decode with its partials in the library's
static per-device scratch instead of a caller workspace, for callers that
cannot allocate.  Its output must be bit for bit that of pd_paged_decode on
the same inputs (same kernels and split plan), on consecutive calls where
the second is smaller than the first (the scratch keeps the first call's
partials), and a call whose partials exceed the scratch is refused on the
host."""

import sys

import numpy as np
import pytest
import torch

import decode_memory_amd as pd
from oracle.attention import decode_attention_bits
from synth import make_block_table, q_bits, shuffled_rows
from tests.gpu_util import assert_decode_close, build_pool, from_device_bits, i32, to_device_bits

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _pool(lengths, n_kv, G, D, dtype, seed):
    lengths = [int(x) for x in lengths]
    rows, _, cap = shuffled_rows(np.random.default_rng(seed), lengths, 32, 8, spare_rows=3)
    scale = 1.0 / np.sqrt(D)
    refs = {}

    def on_layer(layer, ks, vs):
        q = q_bits(seed, layer, len(lengths), n_kv * G, D, dtype)
        refs[layer] = (q, decode_attention_bits(q, ks, vs, dtype, scale))

    pool = build_pool(1, lengths, rows, 32, 8, n_kv, D, dtype, seed, capacity_rows=cap,
                      on_layer=on_layer)
    return pool, make_block_table(rows), refs[0], scale


def _both(pool, q_np, table, lengths, dtype, scale):
    """(noalloc output, workspace output) as bit patterns."""
    q = to_device_bits(q_np, dtype)
    t, lens = i32(table), i32(lengths)
    ml = int(max(lengths))
    out_na = torch.full_like(q, float("nan"))
    pd.paged_decode_noalloc(pool.handle, 0, q, t, lens, ml, scale, out_na)
    out_ws = torch.full_like(q, float("nan"))
    ws = pool.workspace(q.shape[0], q.shape[1], ml)
    pool.paged_decode(0, q, t, lens, ml, scale, out_ws, ws)
    torch.cuda.synchronize()
    return from_device_bits(out_na), from_device_bits(out_ws)


@pytest.mark.parametrize("fmt_case", [("bf16", 8, 2, 128), ("fp16", 4, 4, 64)])
def test_noalloc_matches_workspace_call_twice_shrinking(fmt_case):
    dtype, n_kv, G, D = fmt_case
    first = [4096, 1500, 33, 0, 2900, 700, 4095, 1]
    second = [300, 45, 1200]  # fewer sequences, shorter: fewer splits than the first call
    _say(f"noalloc {dtype} n_kv={n_kv} G={G} D={D}: first call B={len(first)}")
    pool, table, (q, ref), scale = _pool(first, n_kv, G, D, dtype, 4242 + D)
    na, ws = _both(pool, q, table, first, dtype, scale)
    assert np.array_equal(na, ws)
    assert_decode_close(na, ref, dtype, allow_output_rounding=True)
    assert pool.check_error() == 0
    pool.close()

    _say(f"noalloc {dtype}: second call B={len(second)}")
    pool2, table2, (q2, ref2), scale2 = _pool(second, n_kv, G, D, dtype, 4343 + D)
    na2, ws2 = _both(pool2, q2, table2, second, dtype, scale2)
    assert np.array_equal(na2, ws2)
    assert_decode_close(na2, ref2, dtype, allow_output_rounding=True)
    assert pool2.check_error() == 0
    pool2.close()


@pytest.mark.parametrize("fmt,D,G", [("k4v4", 64, 4), ("k8v8", 256, 2)])
def test_noalloc_packed_matches_workspace_call_twice_shrinking(fmt, D, G):
    """The same for packed pools (the matrix-core kernel's partials in the
    scratch): bit for bit the workspace call's output, on a larger call and
    then a smaller one."""
    from synth import hadamard_signs, monotone_rows
    for step, lengths in enumerate(([3000, 1, 777, 0, 2048, 64], [500, 33])):
        _say(f"noalloc {fmt} D={D} G={G}: call {step + 1}, B={len(lengths)}")
        rows = monotone_rows(lengths, 32)
        cap = max(int(r.max()) + 1 for r in rows if len(r))
        pool = pd.SlabPool(1, 32, 8, D, 8, -(-cap // 8) + 1, fmt, hadamard_signs=hadamard_signs(61 + step, D))
        pool.reserve_rows(cap)
        gen = torch.Generator(device="cuda").manual_seed(100 + step)
        for b, n in enumerate(lengths):
            if n == 0:
                continue
            t = np.arange(n)
            k = torch.randn((n, 8, D), generator=gen, device="cuda").to(torch.bfloat16)
            v = torch.randn((n, 8, D), generator=gen, device="cuda").to(torch.bfloat16)
            pool.write_block(0, i32(rows[b][t // 32]), i32(t % 32), k, v)
        q = torch.randn((len(lengths), 8 * G, D), generator=gen, device="cuda").to(torch.bfloat16)
        t_, lens, ml = i32(make_block_table(rows)), i32(lengths), max(lengths)
        out_na = torch.full_like(q, float("nan"))
        pd.paged_decode_noalloc(pool.handle, 0, q, t_, lens, ml, 1 / np.sqrt(D), out_na)
        out_ws = torch.full_like(q, float("nan"))
        pool.paged_decode(0, q, t_, lens, ml, 1 / np.sqrt(D), out_ws, pool.workspace(len(lengths), 8 * G, ml))
        torch.cuda.synchronize()
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16))
        assert bool(torch.isfinite(out_na).all())
        assert pool.check_error() == 0
        pool.close()


def test_noalloc_refuses_calls_beyond_the_scratch():
    """256 sequences x 32 query heads x 16384 tokens (16 splits) need 68 MB
    of partials, more than the 16 MiB scratch: refused with PD_ERR_CAPACITY
    before any launch, while the workspace call's size query still answers."""
    _say("noalloc: capacity refusal")
    pool = pd.SlabPool(1, 32, 8, 128, 8, 4, "bf16")
    pool.reserve_rows(8)
    B, n_q, ml = 256, 32, 16384
    need = pd.decode_workspace_bytes(pool.handle, B, n_q, ml)
    assert need > SCRATCH_BYTES
    q = torch.zeros((B, n_q, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    table = torch.zeros((B, ml // 32), dtype=torch.int32, device="cuda")
    lens = torch.full((B,), ml, dtype=torch.int32, device="cuda")
    with pytest.raises(pd.PagedKVError) as e:
        pd.paged_decode_noalloc(pool.handle, 0, q, table, lens, ml, 0.1, out)
    assert e.value.status == -3 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing was launched
    pool.close()
