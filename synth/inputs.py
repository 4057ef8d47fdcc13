"""Seeded generators for the five paged-decode workloads.

Everything here is input preparation: normal samples from numpy's PCG64,
rounded to fp16 (numpy's own round-to-nearest-even cast) or bf16 (round to
nearest even on the float32 bit pattern), sequence lengths, physical row
layouts for block tables, and the +-1 sign vector of the Hadamard basis.

Seeding: workload ``w`` has a base seed.  Sequence ``b`` of layer ``l`` draws
its K from ``SeedSequence([seed, l, b, 0])`` and its V from
``SeedSequence([seed, l, b, 1])``; the query of layer ``l`` from
``SeedSequence([seed, l, 1 << 20])``.  Per-sequence streams let a consumer
generate one sequence at a time, so the 16k-token workloads never need the
whole KV history in host memory at once.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

FP16 = "fp16"
BF16 = "bf16"


# ---------------------------------------------------------------------------
# dtype rounding of generated float32 samples
# ---------------------------------------------------------------------------

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def f16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE half (numpy's nearest-even cast); uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen fp16/bf16 bit patterns to float32 (exact).  Used to build tensors
    and for reporting; the oracle performs its own widening."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == FP16:
        return bits.view(np.float16).astype(np.float32)
    if dtype == BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(dtype)


def normal_bits(seed_seq, shape, dtype: str) -> np.ndarray:
    """N(0,1) float32 samples from PCG64 rounded to ``dtype``; uint16 bits."""
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == FP16:
        return f16_bits_from_f32(x)
    if dtype == BF16:
        return bf16_bits_from_f32(x)
    raise ValueError(dtype)


def ranged_bits(seed_seq, shape, group: int, amplitudes: Sequence[float], dtype: str = BF16) -> np.ndarray:
    """Uniform samples from PCG64 whose value groups (``group`` consecutive
    values along the last axis) lie in [-A, A], A = amplitudes[g % len], for
    group g of a vector; rounded to ``dtype``; uint16 bits.  Stands in for
    keys, values or queries far from unit scale."""
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    x = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    d = shape[-1]
    amp = np.asarray([amplitudes[(i // group) % len(amplitudes)] for i in range(d)], dtype=np.float32)
    x = (x * amp).astype(np.float32)
    return f16_bits_from_f32(x) if dtype == FP16 else bf16_bits_from_f32(x)


def kv_bits_for_sequence(seed: int, layer: int, b: int, length: int, n_kv: int,
                         head_dim: int, dtype: str):
    """K and V of one sequence in one layer: two uint16 arrays [length, n_kv, D]."""
    shape = (length, n_kv, head_dim)
    k = normal_bits(np.random.SeedSequence([seed, layer, b, 0]), shape, dtype)
    v = normal_bits(np.random.SeedSequence([seed, layer, b, 1]), shape, dtype)
    return k, v


def q_bits(seed: int, layer: int, batch: int, n_q: int, head_dim: int, dtype: str):
    """Decode queries of one layer: uint16 [B, n_q, D]."""
    return normal_bits(np.random.SeedSequence([seed, layer, 1 << 20]),
                       (batch, n_q, head_dim), dtype)


def device_seed(key) -> int:
    """Fold an integer tuple into one 63-bit seed for a device generator."""
    state = np.random.SeedSequence(list(key)).generate_state(2, np.uint32)
    return int((int(state[0]) << 31) ^ int(state[1])) & ((1 << 63) - 1)


def normal_device(key, shape, dtype: str, device):
    """N(0,1) samples drawn on the device with torch's seeded generator and
    rounded to fp16/bf16 (torch's nearest-even cast).  Used for the 56 GiB
    long-context workload, which is too large to generate on the host; a test
    copies the sequences it checks back to the host for the oracle."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(device_seed(key))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.float16 if dtype == FP16 else torch.bfloat16)


def hadamard_signs(seed: int, head_dim: int) -> np.ndarray:
    """The fixed +-1 sign vector of the signed Hadamard basis, int8 [D]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1 << 21])))
    return np.where(rng.integers(0, 2, size=head_dim) == 1, 1, -1).astype(np.int8)


# ---------------------------------------------------------------------------
# physical row layouts
# ---------------------------------------------------------------------------

def _n_blocks(length: int, block_size: int) -> int:
    return -(-int(length) // int(block_size))


def monotone_rows(lengths: Sequence[int], block_size: int, offset: int = 0) -> List[np.ndarray]:
    """Rows handed out in order: sequence b owns a contiguous ascending range.

    ``offset`` shifts every row (an offset that is not a multiple of the slab
    size makes each sequence straddle one more slab boundary)."""
    out, nxt = [], int(offset)
    for n in lengths:
        nb = _n_blocks(n, block_size)
        out.append(np.arange(nxt, nxt + nb, dtype=np.int32))
        nxt += nb
    return out


def shuffled_rows(rng: np.random.Generator, lengths: Sequence[int], block_size: int,
                  slab_blocks: int, spare_rows: int = 64):
    """Rows popped from a seeded shuffled free list.

    The free list holds R rows (all blocks plus ``spare_rows``, rounded up to
    whole slabs) in the order of ``rng.permutation(R)``.  Sequences take their
    blocks round-robin, one block at a time, as concurrent sequences would,
    so every slab holds blocks of many sequences.  Returns (rows per sequence,
    remaining free list, R)."""
    nbs = [_n_blocks(n, block_size) for n in lengths]
    total = sum(nbs) + int(spare_rows)
    R = -(-total // slab_blocks) * slab_blocks
    free = [int(r) for r in rng.permutation(R)]
    rows = [[] for _ in nbs]
    pos = 0
    for i in range(max(nbs) if nbs else 0):
        for b, nb in enumerate(nbs):
            if i < nb:
                rows[b].append(free[pos])
                pos += 1
    return [np.asarray(r, dtype=np.int32) for r in rows], free[pos:], R


def make_block_table(rows: Sequence[np.ndarray], max_blocks: Optional[int] = None) -> np.ndarray:
    """Pack per-sequence row lists into an int32 [B, max_blocks] table padded with -1."""
    width = max([len(r) for r in rows] + [0]) if max_blocks is None else int(max_blocks)
    t = np.full((len(rows), max(width, 1)), -1, dtype=np.int32)
    for b, r in enumerate(rows):
        t[b, :len(r)] = r
    return t


# ---------------------------------------------------------------------------
# the workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    n_layers: int
    batch: int
    block_size: int
    slab_blocks: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    layout: str                      # "monotone" | "shuffled"
    length: Optional[int] = None     # equal lengths
    length_range: Optional[tuple] = None  # inclusive uniform range
    head_dims: tuple = ()            # packed workload: head_dim variants
    formats: tuple = ()              # packed workload: formats
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


def workload_lengths(w: Workload) -> np.ndarray:
    """Per-sequence visible lengths (int64 [B])."""
    if w.length is not None:
        return np.full(w.batch, w.length, dtype=np.int64)
    lo, hi = w.length_range
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 1 << 22])))
    return rng.integers(lo, hi, size=w.batch, endpoint=True).astype(np.int64)


WORKLOADS = {
    "tiny": Workload(
        name="tiny", seed=1, n_layers=1, batch=1, length=256, block_size=32,
        slab_blocks=4, n_q_heads=16, n_kv_heads=8, head_dim=128, dtype=FP16,
        layout="monotone",
        notes="1 sequence of 256 tokens = 8 blocks in rows 0..7, 2 slabs of 4 blocks"),
    "qwen3_0p6b_8x4k": Workload(
        name="qwen3_0p6b_8x4k", seed=2, n_layers=28, batch=8, length=4096,
        block_size=32, slab_blocks=32, n_q_heads=16, n_kv_heads=8, head_dim=128,
        dtype=BF16, layout="monotone",
        notes="sequence b owns rows [128b, 128b+128): 4 same-slab runs each"),
    "fragmented_64": Workload(
        name="fragmented_64", seed=3, n_layers=1, batch=64, length_range=(512, 16384),
        block_size=32, slab_blocks=32, n_q_heads=16, n_kv_heads=8, head_dim=128,
        dtype=BF16, layout="shuffled",
        notes="rows from a seeded shuffled free list; one new token per sequence per step"),
    "qwen3_1p7b_32x16k": Workload(
        name="qwen3_1p7b_32x16k", seed=4, n_layers=28, batch=32, length=16384,
        block_size=32, slab_blocks=32, n_q_heads=16, n_kv_heads=8, head_dim=128,
        dtype=BF16, layout="monotone",
        notes="long context; gather_visible to [B, 8, 16384, 128]"),
    "footprint_8x4k": Workload(
        name="footprint_8x4k", seed=6, n_layers=28, batch=8, length_range=(4096, 4300),
        block_size=32, slab_blocks=32, n_q_heads=16, n_kv_heads=8, head_dim=128,
        dtype=BF16, layout="monotone",
        notes="8 distinct ~4.2k-token prompts prefilled one after another; the pool grows each time"),
    "packed_16x16k": Workload(
        name="packed_16x16k", seed=5, n_layers=1, batch=16, length=16384,
        block_size=32, slab_blocks=32, n_q_heads=32, n_kv_heads=8, head_dim=64,
        dtype=BF16, layout="monotone", head_dims=(64, 256),
        formats=("k8v8", "k8v4", "k4v4"),
        notes="packed KV, groups of 32 along head_dim, GQA 4"),
}
