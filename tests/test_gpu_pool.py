"""Slab growth on the device: append never copies, new slabs are zero,
earlier slab addresses stay put, capacity and argument errors leave the pool
unchanged (mlxcel #235, "Proposed solution: chunked slabs" and "Acceptance
criteria": growth appends slabs without copying, counter-pinned)."""

import pytest
import torch

import decode_memory_amd as pd

pytestmark = pytest.mark.gpu


def _pool(**kw):
    args = dict(n_layers=3, block_size=32, n_kv_heads=8, head_dim=128, slab_blocks=4,
                max_slabs=5, fmt="bf16")
    args.update(kw)
    return pd.SlabPool(**args)


def test_growth_is_counter_pinned_and_never_copies():
    p = _pool()
    assert p.stats()["n_slabs"] == 0
    assert p.reserve_rows(9) == 3                          # ceil(9 / 4) slabs, one step
    st = p.stats()
    assert st["slab_append_events"] == 3 and st["capacity_rows"] == 12
    assert st["bytes_copied_on_growth"] == 0
    kb, vb = p.k_slab_bytes, p.v_slab_bytes
    assert kb == 4 * 32 * 8 * 256 and st["bytes_reserved"] == 3 * 3 * (kb + vb)
    before = {(l, r): p.slab_for_row(l, r) for l in range(3) for r in range(12)}
    # write a marker into slab 1 of layer 2, then grow
    p.k_slabs[2][1].fill_(7)
    assert p.reserve_rows(9) == 0
    assert p.append_slab() == 3
    torch.cuda.synchronize()
    for key, val in before.items():
        assert p.slab_for_row(*key) == val                 # addresses unchanged
    assert bool((p.k_slabs[2][1] == 7).all())              # contents unchanged
    for l in range(3):                                     # the new slab is zero
        assert int(p.k_slabs[l][3].count_nonzero()) == 0 and int(p.v_slabs[l][3].count_nonzero()) == 0
    kbase, vbase, r = p.slab_for_row(1, 13)
    assert r == 1 and kbase == p.k_slabs[1][3].data_ptr() and vbase == p.v_slabs[1][3].data_ptr()
    assert p.stats()["slab_append_events"] == 4
    p.close()


def test_append_zero_fills_garbage_memory():
    p = _pool(n_layers=2)
    ks = [torch.full((p.k_slab_bytes,), 0xAB, dtype=torch.uint8, device="cuda") for _ in range(2)]
    vs = [torch.full((p.v_slab_bytes,), 0xCD, dtype=torch.uint8, device="cuda") for _ in range(2)]
    assert pd.append_slab(p.handle, ks, vs) == 0
    torch.cuda.synchronize()
    assert all(int(t.count_nonzero()) == 0 for t in ks + vs)
    p.k_slabs[0].append(ks[0]); p.k_slabs[1].append(ks[1])
    p.v_slabs[0].append(vs[0]); p.v_slabs[1].append(vs[1])
    p.close()


def test_capacity_and_argument_errors_leave_pool_unchanged():
    p = _pool(max_slabs=2)
    p.reserve_rows(8)
    st = p.stats()
    with pytest.raises(pd.PagedKVError) as e:
        p.append_slab()
    assert e.value.status == -3
    with pytest.raises(pd.PagedKVError) as e:
        ks, vs = p._alloc(1)
        pd.reserve_rows(p.handle, 12, ks, vs, 2)            # wrong slab count
    assert e.value.status in (-1, -3)
    assert p.stats() == st
    with pytest.raises(pd.PagedKVError) as e:
        p.slab_for_row(0, 8)
    assert e.value.status == -2
    with pytest.raises(pd.PagedKVError) as e:
        p.slab_for_row(3, 0)
    assert e.value.status == -2
    p.close()


def test_misaligned_slab_memory_is_rejected():
    p = _pool(n_layers=1)
    big = torch.empty(p.k_slab_bytes + 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(pd.PagedKVError) as e:
        pd.append_slab(p.handle, [big[16:]], [big[16:]])
    assert e.value.status == -1
    assert p.stats()["n_slabs"] == 0
    p.close()


def test_append_over_many_layers_records_every_table_entry():
    """An append records each new slab's base pointer in the device tables and
    zero-fills it in one launch per 96 (slab, layer) pairs: 40 layers x 3
    slabs take two launches.  Garbage memory comes back zero, and a token
    written to the last slab of the last layer gathers back through the
    device table entry the second launch wrote."""
    L, n = 40, 3
    p = _pool(n_layers=L, max_slabs=4)
    ks = [torch.full((p.k_slab_bytes,), 0xAB, dtype=torch.uint8, device="cuda") for _ in range(n * L)]
    vs = [torch.full((p.v_slab_bytes,), 0xCD, dtype=torch.uint8, device="cuda") for _ in range(n * L)]
    assert pd.reserve_rows(p.handle, 12, ks, vs, n) == n
    p._adopt(ks, vs, n)
    torch.cuda.synchronize()
    assert all(int(t.count_nonzero()) == 0 for t in ks + vs)
    for layer in (0, L - 1):
        for row in (0, 11):
            kb, vb, r = p.slab_for_row(layer, row)
            assert kb == p.k_slabs[layer][row // 4].data_ptr() and r == row % 4
    k = torch.arange(8 * 128, dtype=torch.float32, device="cuda").view(1, 8, 128).to(torch.bfloat16)
    p.write_block(L - 1, torch.tensor([11], dtype=torch.int32, device="cuda"),
                  torch.tensor([5], dtype=torch.int32, device="cuda"), k, -k)
    table = torch.full((1, 12), -1, dtype=torch.int32, device="cuda")
    table[0, 0] = 11
    out_k = torch.zeros((1, 8, 6, 256), dtype=torch.uint8, device="cuda")
    out_v = torch.zeros_like(out_k)
    p.gather_visible(L - 1, table, torch.tensor([6], dtype=torch.int32, device="cuda"), 6, out_k, out_v)
    torch.cuda.synchronize()
    assert torch.equal(out_k[0, :, 5].view(torch.bfloat16), k[0])
    assert torch.equal(out_v[0, :, 5].view(torch.bfloat16), -k[0])
    assert int(out_k[0, :, :5].count_nonzero()) == 0            # zeroed slots before it
    assert p.check_error() == 0
    p.close()


def test_allocation_failure_mid_append_leaves_pool_unchanged(monkeypatch):
    """The slab memory of an append is allocated by the caller before the
    library is called; an allocation that fails part-way (the fourth of six
    slab tensors here) raises before anything is appended, and the pool's
    counters, addresses and contents are as before.  A later append works."""
    p = _pool(n_layers=3, max_slabs=5)
    p.reserve_rows(4)
    p.k_slabs[1][0].fill_(9)
    st = p.stats()
    addr = [p.slab_for_row(l, 3) for l in range(3)]
    real_empty = torch.empty
    calls = {"n": 0}

    def failing_empty(*a, **kw):
        calls["n"] += 1
        if calls["n"] == 4:
            raise RuntimeError("HIP out of memory (injected)")
        return real_empty(*a, **kw)

    monkeypatch.setattr(torch, "empty", failing_empty)
    with pytest.raises(RuntimeError, match="injected"):
        p.reserve_rows(8)
    monkeypatch.setattr(torch, "empty", real_empty)
    assert p.stats() == st
    assert [p.slab_for_row(l, 3) for l in range(3)] == addr
    with pytest.raises(pd.PagedKVError):
        p.slab_for_row(0, 4)                                   # no slab was added
    torch.cuda.synchronize()
    assert bool((p.k_slabs[1][0] == 9).all())
    assert p.reserve_rows(8) == 1                              # growth still works
    assert p.stats()["n_slabs"] == 2
    p.close()
