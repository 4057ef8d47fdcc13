"""Pool footprint accounting for sequential prefills (test infrastructure).

Follows mlxcel issue #235 ("perf(core): chunked slab storage for the paged
pool to eliminate growth reallocation entirely"):

* section "Problem": before the change a layer's pool was one tensor per K
  and V; growth allocated a larger zeroed tensor, copied the old contents
  and freed the old one, and the freed sizes formed a ladder of strictly
  increasing sizes that no later (bigger) allocation could reuse, so the
  buffer cache kept roughly the sum of the ladder.  Growth went in steps of
  POOL_GROW_CHUNK_BLOCKS (32) blocks, one presize per prefill span;
* section "Proposed solution: chunked slabs": growth appends fixed-size
  slabs, so the allocator high-water mark is exactly the live capacity;
* section "Acceptance criteria": 8 concurrent distinct ~4k-token prompts
  should peak within about 1.15x of the dense backend.

Bytes here are KV-cache bytes only (every layer, K and V); the dense backend
holds each sequence's tokens in tensors of exactly its length.
"""

from __future__ import annotations

from typing import List, Sequence


def blocks_for(length: int, block_size: int) -> int:
    return -(-int(length) // block_size)


def dense_bytes(lengths: Sequence[int], token_bytes: int) -> int:
    """Dense backend: each sequence's own K and V of exactly its length."""
    return sum(int(n) for n in lengths) * token_bytes


def slab_pool_capacity(lengths: Sequence[int], block_size: int, slab_blocks: int,
                       block_bytes: int) -> List[int]:
    """Slab pool after each sequential prefill (rows taken in order, growth
    by whole slabs): bytes reserved after prefill 1, 2, ..."""
    out, rows = [], 0
    for n in lengths:
        rows += blocks_for(n, block_size)
        slabs = -(-rows // slab_blocks)
        out.append(slabs * slab_blocks * block_bytes)
    return out


def growth_by_copy_peak(lengths: Sequence[int], block_size: int, chunk_blocks: int,
                        block_bytes: int) -> int:
    """Single-tensor pool grown by copy, one presize per prefill span: the
    new capacity is the rows in use rounded up to the growth chunk; every
    freed old capacity stays cached.  Peak = live capacity + the ladder of
    earlier capacities."""
    rows, cap, ladder, peak = 0, 0, 0, 0
    for n in lengths:
        rows += blocks_for(n, block_size)
        need = -(-rows // chunk_blocks) * chunk_blocks
        if need > cap:
            if cap:
                ladder += cap           # the old tensor, freed but not reusable
            cap = need
        peak = max(peak, (cap + ladder) * block_bytes)
    return peak
