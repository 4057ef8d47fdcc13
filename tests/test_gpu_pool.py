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
