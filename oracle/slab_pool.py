"""Byte-level model of the chunked-slab KV pool.

Follows mlxcel issue #235 ("perf(core): chunked slab storage for the paged pool
to eliminate growth reallocation entirely"), section "Proposed solution:
chunked slabs":

* each layer keeps a list of K slabs and a list of V slabs, every slab shaped
  [slab_blocks, block_size, n_kv_heads, record]; a record is one token-head
  vector (head_dim 16-bit values, or a packed record of codes + metadata);
* physical row r lives in slab r // slab_blocks at position r % slab_blocks;
* growth appends a fresh zero slab (to every layer, since row ids are shared
  by all layers) and never copies; a counter counts append events;
* write_block assigns into the row's slab;
* copy_on_write_block (touch point 2) copies a whole block row, every layer,
  K and V: the source bytes come from the source row's slab and land in the
  destination row's slab;
* serde (touch point 6) extracts a block's bytes from the row's slab, every
  layer, and the restore path writes them back into a row's slab; blocks are
  laid out [n][n_layers][K row, V row];
* gather_visible splits a sequence's block-table rows into maximal same-slab
  runs in logical order, takes each run from its slab, concatenates the runs
  and then reshapes, slices to the visible length and transposes.

Values are held as raw bytes (uint8), so every comparison is bit-exact.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


class SlabPoolModel:
    def __init__(self, n_layers: int, block_size: int, n_kv_heads: int,
                 k_record_bytes: int, v_record_bytes: int, slab_blocks: int):
        assert n_layers > 0 and block_size > 0 and n_kv_heads > 0 and slab_blocks > 0
        self.n_layers = n_layers
        self.block_size = block_size
        self.n_kv_heads = n_kv_heads
        self.k_rec = k_record_bytes
        self.v_rec = v_record_bytes
        self.slab_blocks = slab_blocks
        self.k_slabs: List[List[np.ndarray]] = [[] for _ in range(n_layers)]
        self.v_slabs: List[List[np.ndarray]] = [[] for _ in range(n_layers)]
        self.slab_append_events = 0

    # -- geometry ---------------------------------------------------------
    @property
    def n_slabs(self) -> int:
        return len(self.k_slabs[0])

    @property
    def capacity_rows(self) -> int:
        return self.n_slabs * self.slab_blocks

    def slab_bytes(self) -> Tuple[int, int]:
        """Bytes of one K slab and one V slab of one layer."""
        per = self.slab_blocks * self.block_size * self.n_kv_heads
        return per * self.k_rec, per * self.v_rec

    def bytes_reserved(self) -> int:
        """Sum over every slab of every layer (K and V)."""
        total = 0
        for layer in range(self.n_layers):
            total += sum(s.nbytes for s in self.k_slabs[layer])
            total += sum(s.nbytes for s in self.v_slabs[layer])
        return total

    # -- growth -----------------------------------------------------------
    def append_slab(self) -> int:
        """Append one zero K slab and one zero V slab to every layer.

        Existing slabs are left untouched (no copy).  Returns the new slab index."""
        shape = (self.slab_blocks, self.block_size, self.n_kv_heads)
        for layer in range(self.n_layers):
            self.k_slabs[layer].append(np.zeros(shape + (self.k_rec,), dtype=np.uint8))
            self.v_slabs[layer].append(np.zeros(shape + (self.v_rec,), dtype=np.uint8))
        self.slab_append_events += 1
        return self.n_slabs - 1

    def reserve_rows(self, rows_needed: int) -> int:
        """Append as many slabs as needed so that ``rows_needed`` rows exist.

        Returns the number of slabs appended (presize_for_span)."""
        n = 0
        while self.capacity_rows < rows_needed:
            self.append_slab()
            n += 1
        return n

    # -- mapping ----------------------------------------------------------
    def slab_for_row(self, layer: int, row: int):
        """(K slab, V slab, row_in_slab) of a physical row."""
        slab = row // self.slab_blocks
        return self.k_slabs[layer][slab], self.v_slabs[layer][slab], row % self.slab_blocks

    # -- writes -----------------------------------------------------------
    def write(self, layer: int, rows: Sequence[int], slots: Sequence[int],
              k_records: np.ndarray, v_records: np.ndarray) -> None:
        """Token-granular scatter: token i goes to (rows[i], slots[i]).

        k_records: uint8 [n, n_kv, k_rec]; v_records: uint8 [n, n_kv, v_rec]."""
        k_records = np.asarray(k_records, dtype=np.uint8)
        v_records = np.asarray(v_records, dtype=np.uint8)
        for i, (row, slot) in enumerate(zip(rows, slots)):
            ks, vs, r = self.slab_for_row(layer, int(row))
            ks[r, int(slot)] = k_records[i]
            vs[r, int(slot)] = v_records[i]

    def copy_block(self, src_rows: Sequence[int], dst_rows: Sequence[int]) -> None:
        """Copy block row src_rows[i] onto dst_rows[i] in every layer, K and V.

        All source rows are read before any destination is written."""
        pairs = [(int(s), int(d)) for s, d in zip(src_rows, dst_rows)]
        for layer in range(self.n_layers):
            saved = []
            for src, _ in pairs:
                ks, vs, r = self.slab_for_row(layer, src)
                saved.append((ks[r].copy(), vs[r].copy()))
            for (_, dst), (kb, vb) in zip(pairs, saved):
                kd, vd, r = self.slab_for_row(layer, dst)
                kd[r] = kb
                vd[r] = vb

    def export_blocks(self, rows: Sequence[int]) -> np.ndarray:
        """uint8 [n, n_layers * (K row + V row)]: each block's rows, layer by
        layer, K then V, exactly as stored."""
        out = []
        for row in rows:
            parts = []
            for layer in range(self.n_layers):
                ks, vs, r = self.slab_for_row(layer, int(row))
                parts += [ks[r].reshape(-1), vs[r].reshape(-1)]
            out.append(np.concatenate(parts))
        return np.stack(out) if out else np.zeros((0, 0), np.uint8)

    def import_blocks(self, rows: Sequence[int], data: np.ndarray) -> None:
        """Inverse of export_blocks: block i of data into row rows[i]."""
        kb = self.block_size * self.n_kv_heads * self.k_rec
        vb = self.block_size * self.n_kv_heads * self.v_rec
        for i, row in enumerate(rows):
            at = 0
            for layer in range(self.n_layers):
                ks, vs, r = self.slab_for_row(layer, int(row))
                ks[r] = data[i, at:at + kb].reshape(ks[r].shape)
                vs[r] = data[i, at + kb:at + kb + vb].reshape(vs[r].shape)
                at += kb + vb

    # -- reads ------------------------------------------------------------
    def split_runs(self, rows: Sequence[int]) -> List[Tuple[int, int, int]]:
        """Maximal same-slab runs of a row list, in logical order.

        Returns (slab, first logical block, number of blocks) per run."""
        runs: List[Tuple[int, int, int]] = []
        for i, row in enumerate(rows):
            slab = int(row) // self.slab_blocks
            if runs and runs[-1][0] == slab:
                s, first, count = runs[-1]
                runs[-1] = (s, first, count + 1)
            else:
                runs.append((slab, i, 1))
        return runs

    def gather(self, layer: int, rows: Sequence[int], length: int):
        """One sequence's visible K and V: uint8 [n_kv, length, rec] each."""
        rows = [int(r) for r in rows]
        if length == 0 or not rows:
            return (np.zeros((self.n_kv_heads, 0, self.k_rec), np.uint8),
                    np.zeros((self.n_kv_heads, 0, self.v_rec), np.uint8))
        k_parts, v_parts = [], []
        for slab, first, count in self.split_runs(rows):
            in_slab = [r % self.slab_blocks for r in rows[first:first + count]]
            k_parts.append(np.take(self.k_slabs[layer][slab], in_slab, axis=0))
            v_parts.append(np.take(self.v_slabs[layer][slab], in_slab, axis=0))
        out = []
        for parts, rec in ((k_parts, self.k_rec), (v_parts, self.v_rec)):
            cat = np.concatenate(parts, axis=0)
            flat = cat.reshape(len(rows) * self.block_size, self.n_kv_heads, rec)
            out.append(np.ascontiguousarray(flat[:length].transpose(1, 0, 2)))
        return out[0], out[1]

    def gather_batched(self, layer: int, block_table: np.ndarray, lengths: Sequence[int],
                       t_out: int):
        """Batched gather into [B, n_kv, t_out, rec], zero past each sequence's length."""
        B = len(lengths)
        k = np.zeros((B, self.n_kv_heads, t_out, self.k_rec), np.uint8)
        v = np.zeros((B, self.n_kv_heads, t_out, self.v_rec), np.uint8)
        for b in range(B):
            n = int(lengths[b])
            nb = -(-n // self.block_size)
            kb, vb = self.gather(layer, block_table[b, :nb], n)
            k[b, :, :n] = kb
            v[b, :, :n] = vb
        return k, v


def records_from_u16(bits: np.ndarray) -> np.ndarray:
    """View [..., D] uint16 values as [..., 2D] bytes (little endian)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return bits.view(np.uint8).reshape(bits.shape[:-1] + (bits.shape[-1] * 2,))


def u16_from_records(rec: np.ndarray) -> np.ndarray:
    """Inverse of records_from_u16."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    return rec.view(np.uint16).reshape(rec.shape[:-1] + (rec.shape[-1] // 2,))


def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64 bit: start from the offset basis 14695981039346656037; for
    each byte, xor it in, then multiply by the prime 1099511628211 mod 2^64.
    Serves as the storage identity's fingerprint of the Hadamard signs."""
    h = 14695981039346656037
    for byte in data:
        h ^= byte
        h = (h * 1099511628211) % (1 << 64)
    return h


def signs_fingerprint(signs) -> int:
    """fnv1a64 of the sign vector as stored: +1 -> 0x01, -1 -> 0xFF."""
    return fnv1a64(bytes((int(x) & 0xFF) for x in signs))
