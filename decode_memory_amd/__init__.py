"""Python binding of libpagedkv: paged decode over a chunked-slab KV pool (MI355X).

This is argument marshalling only.  Every step of the path (zero-filling new
slabs, the write scatter, the gather, the decode attention and its combine)
runs in the HIP kernels of ``libpagedkv.so``; torch supplies device memory and
the current stream.  There is no CPU fallback: if the library is missing the
import of :func:`lib` raises.

Functions keep the C names without the ``pd_`` prefix (``pool_create``,
``append_slab``, ``reserve_rows``, ``slab_for_row``, ``write_block``,
``copy_on_write_block``,
``gather_visible``, ``decode_workspace_bytes``, ``paged_decode``,
``pool_stats``, ``pool_check_error``).  :class:`SlabPool` bundles a pool with
the torch tensors that back its slabs.
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch  # loads the HIP runtime that libpagedkv then shares

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

FMT_FP16, FMT_BF16, FMT_K8V8, FMT_K8V4, FMT_K4V4 = 0, 1, 2, 3, 4
FORMAT_NAMES = {"fp16": FMT_FP16, "bf16": FMT_BF16, "k8v8": FMT_K8V8, "k8v4": FMT_K8V4,
                "k4v4": FMT_K4V4}

DEVERR_WRITE_ROW, DEVERR_WRITE_SLOT, DEVERR_TABLE_ROW, DEVERR_LENGTH = 0x1, 0x2, 0x4, 0x8
DEVERR_DUPLICATE = 0x10
DEBUG_DUPLICATE_WRITES = 0x1

STATUS = {0: "PD_OK", -1: "PD_ERR_ARG", -2: "PD_ERR_RANGE", -3: "PD_ERR_CAPACITY",
          -4: "PD_ERR_UNSUPPORTED", -5: "PD_ERR_HIP", -6: "PD_ERR_DEVICE", -7: "PD_ERR_IDENTITY"}


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("slab_blocks", ctypes.c_int32), ("max_slabs", ctypes.c_int32),
                ("format", ctypes.c_int32), ("hadamard_signs", ctypes.POINTER(ctypes.c_int8)),
                ("group_size", ctypes.c_int32)]


class PoolStats(ctypes.Structure):
    _fields_ = [("n_slabs", ctypes.c_int64), ("slab_append_events", ctypes.c_int64),
                ("capacity_rows", ctypes.c_int64), ("bytes_reserved", ctypes.c_int64),
                ("bytes_copied_on_growth", ctypes.c_int64), ("k_slab_bytes", ctypes.c_int64),
                ("v_slab_bytes", ctypes.c_int64), ("k_record_bytes", ctypes.c_int32),
                ("v_record_bytes", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class StorageIdentity(ctypes.Structure):
    """pd_storage_identity: 48 bytes, little endian."""
    _fields_ = [("magic", ctypes.c_uint32), ("layout", ctypes.c_uint32), ("format", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("k_record_bytes", ctypes.c_int32), ("v_record_bytes", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("signs_hash", ctypes.c_uint64)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}

    def to_bytes(self) -> bytes:
        return bytes(self)

    @classmethod
    def from_bytes(cls, b: bytes) -> "StorageIdentity":
        if len(b) != ctypes.sizeof(cls):
            raise ValueError(f"a storage identity is {ctypes.sizeof(cls)} bytes, got {len(b)}")
        return cls.from_buffer_copy(b)


class DenseDesc(ctypes.Structure):
    """pd_dense_desc."""
    _fields_ = [("format", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


EXPORTS = [
    "pd_version", "pd_last_error", "pd_record_bytes", "pd_pool_create", "pd_pool_destroy",
    "pd_slab_bytes", "pd_append_slab", "pd_slabs_needed", "pd_reserve_rows", "pd_slab_for_row",
    "pd_write_block", "pd_copy_on_write_block", "pd_gather_visible", "pd_split_runs",
    "pd_decode_workspace_bytes",
    "pd_paged_decode", "pd_paged_decode_noalloc", "pd_paged_decode_append",
    "pd_paged_decode_split", "pd_paged_decode_combine", "pd_pool_stats", "pd_pool_check_error",
    "pd_pool_set_debug",
    "pd_signs_hash", "pd_storage_identity_of", "pd_identity_check", "pd_block_bytes",
    "pd_export_blocks", "pd_import_blocks", "pd_dense_workspace_bytes", "pd_dense_decode",
]

_lib_handle = None
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_p_i32 = ctypes.POINTER(ctypes.c_int32)
_pp = ctypes.POINTER(ctypes.c_void_p)


def _declare(lib):
    sig = {
        "pd_version": (_i32, []),
        "pd_last_error": (ctypes.c_char_p, []),
        "pd_record_bytes": (_i32, [_i32, _i32, _i32, _p_i32, _p_i32]),
        "pd_pool_create": (_i32, [ctypes.POINTER(PoolDesc), ctypes.POINTER(_vp)]),
        "pd_pool_destroy": (_i32, [_vp]),
        "pd_slab_bytes": (_i32, [_vp, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
        "pd_append_slab": (_i32, [_vp, _pp, _pp, _vp, _p_i32]),
        "pd_slabs_needed": (_i32, [_vp, _i64, _p_i32]),
        "pd_reserve_rows": (_i32, [_vp, _i64, _pp, _pp, _i32, _vp, _p_i32]),
        "pd_slab_for_row": (_i32, [_vp, _i32, _i64, _pp, _pp, _p_i32]),
        "pd_write_block": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
        "pd_copy_on_write_block": (_i32, [_vp, _i32, _vp, _vp, _vp]),
        "pd_gather_visible": (_i32, [_vp, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp]),
        "pd_split_runs": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp]),
        "pd_decode_workspace_bytes": (_i32, [_vp, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
        "pd_paged_decode": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _i32,
                                   ctypes.c_float, _vp, _vp, _sz, _vp]),
        "pd_paged_decode_noalloc": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _i32,
                                           ctypes.c_float, _vp, _vp]),
        "pd_paged_decode_append": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                   ctypes.c_float, _vp, _vp, _sz, _vp]),
        "pd_paged_decode_split": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _i32,
                                         ctypes.c_float, _vp, _vp, _sz, _vp]),
        "pd_paged_decode_combine": (_i32, [_vp, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _i32,
                                           ctypes.c_float, _vp, _vp, _sz, _vp]),
        "pd_pool_stats": (_i32, [_vp, ctypes.POINTER(PoolStats)]),
        "pd_pool_check_error": (_i32, [_vp, _vp, _p_i32]),
        "pd_pool_set_debug": (_i32, [_vp, ctypes.c_uint32]),
        "pd_signs_hash": (_i32, [ctypes.POINTER(ctypes.c_int8), _i32, ctypes.POINTER(ctypes.c_uint64)]),
        "pd_storage_identity_of": (_i32, [_vp, ctypes.POINTER(StorageIdentity)]),
        "pd_identity_check": (_i32, [_vp, ctypes.POINTER(StorageIdentity)]),
        "pd_block_bytes": (_i32, [_vp, ctypes.POINTER(_sz)]),
        "pd_export_blocks": (_i32, [_vp, _i32, _vp, _vp, _sz, _vp]),
        "pd_import_blocks": (_i32, [_vp, ctypes.POINTER(StorageIdentity), _i32, _vp, _vp, _sz, _vp]),
        "pd_dense_workspace_bytes": (_i32, [ctypes.POINTER(DenseDesc), _i32, _i32, _i32, ctypes.POINTER(_sz)]),
        "pd_dense_decode": (_i32, [ctypes.POINTER(DenseDesc), _i32, _i32, _vp, _vp, _vp, _vp, _i32,
                                   ctypes.c_float, _vp, _vp, _sz, _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded libpagedkv (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m decode_memory_amd.build` (or __graft_entry__.build())")
        handle = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
        _declare(handle)
        _lib_handle = handle
    return _lib_handle


def _check(status: int) -> None:
    if status != 0:
        raise PagedKVError(status, lib().pd_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr_array(tensors: Sequence[torch.Tensor]):
    arr = (ctypes.c_void_p * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        arr[i] = t.data_ptr()
    return arr


def _require(t: torch.Tensor, name: str, dtype=None, numel=None):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


# ---------------------------------------------------------------------------
# thin wrappers, one per C entry point
# ---------------------------------------------------------------------------

def version() -> int:
    return lib().pd_version()


def record_bytes(fmt: int, head_dim: int, group_size: int = 0):
    """Bytes of one K and one V token-head record (group_size 0: 32)."""
    k, v = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().pd_record_bytes(fmt, head_dim, group_size, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def pool_create(n_layers, block_size, n_kv_heads, head_dim, slab_blocks, max_slabs, fmt,
                hadamard_signs=None, group_size=0) -> int:
    signs_buf = None
    if hadamard_signs is not None:
        vals = [int(x) for x in hadamard_signs]
        signs_buf = (ctypes.c_int8 * len(vals))(*vals)
    desc = PoolDesc(n_layers, block_size, n_kv_heads, head_dim, slab_blocks, max_slabs, fmt,
                    ctypes.cast(signs_buf, ctypes.POINTER(ctypes.c_int8)) if signs_buf else None,
                    group_size)
    out = ctypes.c_void_p()
    _check(lib().pd_pool_create(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def pool_destroy(pool: int) -> None:
    _check(lib().pd_pool_destroy(pool))


def slab_bytes(pool: int):
    k, v = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().pd_slab_bytes(pool, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def append_slab(pool: int, k_mem: Sequence[torch.Tensor], v_mem: Sequence[torch.Tensor],
                stream=None) -> int:
    idx = ctypes.c_int32(-1)
    _check(lib().pd_append_slab(pool, _ptr_array(k_mem), _ptr_array(v_mem), _stream(stream),
                                ctypes.byref(idx)))
    return idx.value


def slabs_needed(pool: int, rows_needed: int) -> int:
    n = ctypes.c_int32()
    _check(lib().pd_slabs_needed(pool, rows_needed, ctypes.byref(n)))
    return n.value


def reserve_rows(pool: int, rows_needed: int, k_mem, v_mem, n_slabs: int, stream=None) -> int:
    n = ctypes.c_int32()
    _check(lib().pd_reserve_rows(pool, rows_needed, _ptr_array(k_mem), _ptr_array(v_mem), n_slabs,
                                 _stream(stream), ctypes.byref(n)))
    return n.value


def slab_for_row(pool: int, layer: int, row: int):
    kb, vb, r = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_int32()
    _check(lib().pd_slab_for_row(pool, layer, row, ctypes.byref(kb), ctypes.byref(vb),
                                 ctypes.byref(r)))
    return kb.value, vb.value, r.value


def write_block(pool: int, layer: int, rows: torch.Tensor, slots: torch.Tensor,
                k_src: torch.Tensor, v_src: torch.Tensor, stream=None) -> None:
    n = rows.numel()
    _require(rows, "rows", torch.int32)
    _require(slots, "slots", torch.int32, n)
    _require(k_src, "k_src")
    _require(v_src, "v_src")
    _check(lib().pd_write_block(pool, layer, n, _ptr(rows), _ptr(slots), _ptr(k_src), _ptr(v_src),
                                _stream(stream)))


def copy_on_write_block(pool: int, src_rows: torch.Tensor, dst_rows: torch.Tensor,
                        stream=None) -> None:
    """Copy block row src_rows[i] onto dst_rows[i] in every layer, K and V."""
    n = src_rows.numel()
    _require(src_rows, "src_rows", torch.int32)
    _require(dst_rows, "dst_rows", torch.int32, n)
    _check(lib().pd_copy_on_write_block(pool, n, _ptr(src_rows), _ptr(dst_rows), _stream(stream)))


def signs_hash(signs: Sequence[int]) -> int:
    """FNV-1a 64 of the Hadamard sign bytes (host only)."""
    arr = (ctypes.c_int8 * max(1, len(signs)))(*[int(x) for x in signs])
    h = ctypes.c_uint64(0)
    _check(lib().pd_signs_hash(arr, len(signs), ctypes.byref(h)))
    return h.value


def storage_identity(pool: int) -> StorageIdentity:
    out = StorageIdentity()
    _check(lib().pd_storage_identity_of(pool, ctypes.byref(out)))
    return out


def identity_check(pool: int, identity: StorageIdentity) -> None:
    """Raises PagedKVError (status -7) when blocks of `identity` cannot be
    imported into the pool."""
    _check(lib().pd_identity_check(pool, ctypes.byref(identity)))


def block_bytes(pool: int) -> int:
    n = _sz(0)
    _check(lib().pd_block_bytes(pool, ctypes.byref(n)))
    return n.value


def export_blocks(pool: int, rows: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    _require(rows, "rows", torch.int32)
    _require(dst, "dst")
    _check(lib().pd_export_blocks(pool, rows.numel(), _ptr(rows), _ptr(dst),
                                  dst.numel() * dst.element_size(), _stream(stream)))


def import_blocks(pool: int, identity: StorageIdentity, rows: torch.Tensor, src: torch.Tensor,
                  stream=None) -> None:
    _require(rows, "rows", torch.int32)
    _require(src, "src")
    _check(lib().pd_import_blocks(pool, ctypes.byref(identity), rows.numel(), _ptr(rows), _ptr(src),
                                  src.numel() * src.element_size(), _stream(stream)))


def dense_workspace_bytes(fmt, n_kv_heads: int, head_dim: int, B: int, n_q_heads: int,
                          max_len: int) -> int:
    desc = DenseDesc(FORMAT_NAMES[fmt] if isinstance(fmt, str) else int(fmt), n_kv_heads, head_dim)
    n = _sz(0)
    _check(lib().pd_dense_workspace_bytes(ctypes.byref(desc), B, n_q_heads, max_len, ctypes.byref(n)))
    return n.value


def dense_pointers(k_seqs: Sequence[torch.Tensor], v_seqs: Sequence[torch.Tensor],
                   device=None) -> torch.Tensor:
    """The device pointer table dense_decode reads: int64 [2, B], row 0 the
    K and row 1 the V base address of each sequence.  Build it once, when the
    sequences are placed, and keep it (and the sequences) alive while calls
    use it: dense_decode itself allocates nothing."""
    for t in list(k_seqs) + list(v_seqs):
        _require(t, "k/v sequence")
    if len(k_seqs) != len(v_seqs):
        raise ValueError("k_seqs and v_seqs differ in length")
    dev = device if device is not None else (k_seqs[0].device if len(k_seqs) else "cuda")
    return torch.tensor([[t.data_ptr() for t in k_seqs], [t.data_ptr() for t in v_seqs]],
                        dtype=torch.int64, device=dev).reshape(2, len(k_seqs))


def dense_decode(q: torch.Tensor, ptrs: torch.Tensor, n_kv_heads: int, lens: torch.Tensor,
                 max_len: int, scale: float, out: torch.Tensor, workspace: torch.Tensor,
                 stream=None) -> None:
    """Decode over per-sequence contiguous K/V [len_b, n_kv, D] (the dense
    backend), reached through `ptrs` (dense_pointers): bit-identical to
    paged_decode over the same tokens.  Nothing is allocated per call."""
    B, n_q, D = q.shape
    fmt = FMT_FP16 if q.dtype == torch.float16 else FMT_BF16
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError(f"q must be fp16 or bf16, got {q.dtype}")
    desc = DenseDesc(fmt, n_kv_heads, D)
    _require(q, "q")
    _require(out, "out", q.dtype, q.numel())
    _require(lens, "lens", torch.int32, B)
    _require(ptrs, "ptrs", torch.int64, 2 * B)
    _require(workspace, "workspace")
    _check(lib().pd_dense_decode(ctypes.byref(desc), B, n_q, _ptr(q), ptrs.data_ptr(),
                                 ptrs.data_ptr() + 8 * B, _ptr(lens), max_len, float(scale), _ptr(out),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)))


CHECKPOINT_MAGIC = b"PDKVBLK1"


def write_checkpoint(path: str, identity: StorageIdentity, payload: torch.Tensor) -> None:
    """A block checkpoint file: 8-byte magic, the 48-byte storage identity,
    the block count (int64 little endian), then the exported bytes."""
    data = payload.contiguous().view(torch.uint8).cpu().numpy().tobytes()
    n = len(data) // max(1, block_bytes_of(identity))
    with open(path, "wb") as f:
        f.write(CHECKPOINT_MAGIC + identity.to_bytes() + int(n).to_bytes(8, "little") + data)


def read_checkpoint_header(path: str):
    """(identity, n_blocks) of a block checkpoint, reading only its header."""
    size = len(CHECKPOINT_MAGIC) + ctypes.sizeof(StorageIdentity) + 8
    with open(path, "rb") as f:
        head = f.read(size)
    if len(head) != size or not head.startswith(CHECKPOINT_MAGIC):
        raise ValueError(f"{path} is not a block checkpoint")
    ident = StorageIdentity.from_bytes(head[len(CHECKPOINT_MAGIC):-8])
    return ident, int.from_bytes(head[-8:], "little")


def block_bytes_of(identity: StorageIdentity) -> int:
    return (identity.n_layers * identity.block_size * identity.n_kv_heads *
            (identity.k_record_bytes + identity.v_record_bytes))


def gather_visible(pool: int, layer: int, block_table: torch.Tensor, lens: torch.Tensor,
                   t_out: int, k_out: torch.Tensor, v_out: torch.Tensor,
                   n_runs_out: Optional[torch.Tensor] = None, stream=None) -> None:
    B, max_blocks = block_table.shape
    _require(block_table, "block_table", torch.int32)
    _require(lens, "lens", torch.int32, B)
    _require(k_out, "k_out")
    _require(v_out, "v_out")
    if n_runs_out is not None:
        _require(n_runs_out, "n_runs_out", torch.int32, B)
    _check(lib().pd_gather_visible(pool, layer, B, _ptr(block_table), max_blocks, _ptr(lens), t_out,
                                   _ptr(k_out), _ptr(v_out), _ptr(n_runs_out), _stream(stream)))


def split_runs(pool: int, block_table: torch.Tensor, lens: torch.Tensor, runs_out: torch.Tensor,
               n_runs_out: torch.Tensor, stream=None) -> None:
    """pd_split_runs: (slab, first block, blocks) of each same-slab run, per
    sequence, into runs_out [B, max_blocks, 3] and the counts into n_runs_out [B]."""
    B, max_blocks = block_table.shape
    _require(block_table, "block_table", torch.int32)
    _require(lens, "lens", torch.int32, B)
    _require(runs_out, "runs_out", torch.int32, B * max_blocks * 3)
    _require(n_runs_out, "n_runs_out", torch.int32, B)
    _check(lib().pd_split_runs(pool, B, _ptr(block_table), max_blocks, _ptr(lens), _ptr(runs_out),
                               _ptr(n_runs_out), _stream(stream)))


def decode_workspace_bytes(pool: int, B: int, n_q_heads: int, max_len: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().pd_decode_workspace_bytes(pool, B, n_q_heads, max_len, ctypes.byref(n)))
    return n.value


def paged_decode(pool: int, layer: int, q: torch.Tensor, block_table: torch.Tensor,
                 lens: torch.Tensor, max_len: int, scale: float, out: torch.Tensor,
                 workspace: torch.Tensor, stream=None, stage: str = "all") -> None:
    """stage: "all" (pd_paged_decode), "split" or "combine" (its two stages)."""
    fn = {"all": "pd_paged_decode", "split": "pd_paged_decode_split",
          "combine": "pd_paged_decode_combine"}[stage]
    B, n_q, _ = q.shape
    _require(q, "q")
    _require(block_table, "block_table", torch.int32)
    _require(lens, "lens", torch.int32, B)
    _require(out, "out", q.dtype, q.numel())
    _require(workspace, "workspace")
    if block_table.shape[0] != B:
        raise ValueError("block_table rows must equal the batch size")
    _check(getattr(lib(), fn)(pool, layer, B, n_q, _ptr(q), _ptr(block_table),
                                 block_table.shape[1], _ptr(lens), max_len, float(scale), _ptr(out),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)))


def paged_decode_noalloc(pool: int, layer: int, q: torch.Tensor, block_table: torch.Tensor,
                         lens: torch.Tensor, max_len: int, scale: float, out: torch.Tensor,
                         stream=None) -> None:
    """pd_paged_decode_noalloc: paged_decode with the partials in the
    library's static per-device scratch (no workspace, nothing allocated)."""
    B, n_q, _ = q.shape
    _require(q, "q")
    _require(block_table, "block_table", torch.int32)
    _require(lens, "lens", torch.int32, B)
    _require(out, "out", q.dtype, q.numel())
    if block_table.shape[0] != B:
        raise ValueError("block_table rows must equal the batch size")
    _check(lib().pd_paged_decode_noalloc(pool, layer, B, n_q, _ptr(q), _ptr(block_table),
                                         block_table.shape[1], _ptr(lens), max_len, float(scale),
                                         _ptr(out), _stream(stream)))


def paged_decode_append(pool: int, layer: int, q: torch.Tensor, k_new: torch.Tensor,
                        v_new: torch.Tensor, block_table: torch.Tensor, lens: torch.Tensor,
                        max_len: int, scale: float, out: torch.Tensor, workspace: torch.Tensor,
                        stream=None) -> None:
    """pd_paged_decode_append: write token lens[b] - 1 of every sequence from
    k_new/v_new [B, n_kv, D], then attend (one launch of the split kernel)."""
    B, n_q, D = q.shape
    _require(q, "q")
    _require(k_new, "k_new", q.dtype)
    _require(v_new, "v_new", q.dtype, k_new.numel())
    _require(block_table, "block_table", torch.int32)
    _require(lens, "lens", torch.int32, B)
    _require(out, "out", q.dtype, q.numel())
    _require(workspace, "workspace")
    if block_table.shape[0] != B or k_new.shape[0] != B:
        raise ValueError("block_table rows and k_new's first dimension must equal the batch size")
    _check(lib().pd_paged_decode_append(pool, layer, B, n_q, _ptr(q), _ptr(k_new), _ptr(v_new),
                                        _ptr(block_table), block_table.shape[1], _ptr(lens), max_len,
                                        float(scale), _ptr(out), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))


def pool_stats(pool: int) -> dict:
    s = PoolStats()
    _check(lib().pd_pool_stats(pool, ctypes.byref(s)))
    return s.as_dict()


def pool_set_debug(pool: int, flags: int) -> None:
    """Turn the library's debug checks on or off (DEBUG_* bits; 0: all off).
    DEBUG_DUPLICATE_WRITES makes write_block flag DEVERR_DUPLICATE when two
    tokens of one call target the same (row, slot).  Turning it on allocates
    and synchronises: call it at set-up."""
    _check(lib().pd_pool_set_debug(_vp(pool), ctypes.c_uint32(int(flags))))


def pool_check_error(pool: int, stream=None) -> int:
    """Synchronise and return (and clear) the device error bits; never raises for them."""
    bits = ctypes.c_int32(0)
    st = lib().pd_pool_check_error(pool, _stream(stream), ctypes.byref(bits))
    if st not in (0, -6):
        _check(st)
    return bits.value


# ---------------------------------------------------------------------------
# convenience: a pool whose slabs are torch tensors
# ---------------------------------------------------------------------------

class SlabPool:
    """A chunked-slab pool plus the torch tensors that hold its slabs.

    Slab memory is allocated here with torch (uninitialised; the library
    zero-fills it on the current stream) and kept alive until close()."""

    def __init__(self, n_layers: int, block_size: int, n_kv_heads: int, head_dim: int,
                 slab_blocks: int, max_slabs: int, fmt="bf16", hadamard_signs=None,
                 device="cuda", group_size=0):
        self.fmt = FORMAT_NAMES[fmt] if isinstance(fmt, str) else int(fmt)
        self.n_layers, self.block_size, self.n_kv_heads = n_layers, block_size, n_kv_heads
        self.head_dim, self.slab_blocks, self.max_slabs = head_dim, slab_blocks, max_slabs
        self.device = torch.device(device)
        with torch.cuda.device(self.device):
            self.handle = pool_create(n_layers, block_size, n_kv_heads, head_dim, slab_blocks,
                                      max_slabs, self.fmt, hadamard_signs, group_size)
        self.k_slab_bytes, self.v_slab_bytes = slab_bytes(self.handle)
        self.group_size = self.storage_identity().group_size
        self.k_record_bytes, self.v_record_bytes = record_bytes(self.fmt, head_dim, self.group_size)
        self.k_slabs: List[List[torch.Tensor]] = [[] for _ in range(n_layers)]
        self.v_slabs: List[List[torch.Tensor]] = [[] for _ in range(n_layers)]

    # dtype of q / outputs / 16-bit sources
    @property
    def dtype(self):
        return torch.float16 if self.fmt == FMT_FP16 else torch.bfloat16

    def _alloc(self, n: int):
        ks = [torch.empty(self.k_slab_bytes, dtype=torch.uint8, device=self.device)
              for _ in range(n * self.n_layers)]
        vs = [torch.empty(self.v_slab_bytes, dtype=torch.uint8, device=self.device)
              for _ in range(n * self.n_layers)]
        return ks, vs

    def _adopt(self, ks, vs, n):
        for s in range(n):
            for layer in range(self.n_layers):
                self.k_slabs[layer].append(ks[s * self.n_layers + layer])
                self.v_slabs[layer].append(vs[s * self.n_layers + layer])

    def append_slab(self, stream=None) -> int:
        ks, vs = self._alloc(1)
        idx = append_slab(self.handle, ks, vs, stream)
        self._adopt(ks, vs, 1)
        return idx

    def reserve_rows(self, rows_needed: int, stream=None) -> int:
        n = slabs_needed(self.handle, rows_needed)
        if n == 0:
            return 0
        ks, vs = self._alloc(n)
        got = reserve_rows(self.handle, rows_needed, ks, vs, n, stream)
        self._adopt(ks, vs, n)
        return got

    def slab_view(self, layer: int, slab: int, kv: str = "k") -> torch.Tensor:
        """A slab as [slab_blocks, block_size, n_kv_heads, record_bytes] uint8."""
        t = (self.k_slabs if kv == "k" else self.v_slabs)[layer][slab]
        rec = self.k_record_bytes if kv == "k" else self.v_record_bytes
        return t.view(self.slab_blocks, self.block_size, self.n_kv_heads, rec)

    def slab_for_row(self, layer: int, row: int):
        return slab_for_row(self.handle, layer, row)

    # -- argument checks the C ABI cannot make (it sees raw pointers only) --

    def _check_tokens(self, name, t, n):
        """t holds n token rows [n, n_kv_heads, head_dim] in the pool's dtype."""
        _require(t, name, self.dtype)
        if t.numel() != n * self.n_kv_heads * self.head_dim:
            raise ValueError(f"{name} must be [{n}, {self.n_kv_heads}, {self.head_dim}] "
                             f"({n * self.n_kv_heads * self.head_dim} values), got {tuple(t.shape)}")

    def _check_query(self, q, out=None):
        _require(q, "q", self.dtype)
        if q.dim() != 3 or q.shape[2] != self.head_dim or q.shape[1] % self.n_kv_heads:
            raise ValueError(f"q must be [B, n_q_heads, {self.head_dim}] with n_q_heads a multiple of "
                             f"{self.n_kv_heads}, got {tuple(q.shape)}")
        if out is not None:
            _require(out, "out", self.dtype, q.numel())

    def _check_table(self, block_table, lens, B):
        _require(block_table, "block_table", torch.int32)
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError(f"block_table must be [{B}, max_blocks], got {tuple(block_table.shape)}")
        _require(lens, "lens", torch.int32, B)

    def write_block(self, layer, rows, slots, k_src, v_src, stream=None):
        n = rows.numel()
        self._check_tokens("k_src", k_src, n)
        self._check_tokens("v_src", v_src, n)
        write_block(self.handle, layer, rows, slots, k_src, v_src, stream)

    def copy_on_write_block(self, src_rows, dst_rows, stream=None):
        copy_on_write_block(self.handle, src_rows, dst_rows, stream)

    def storage_identity(self) -> StorageIdentity:
        return storage_identity(self.handle)

    def export_blocks(self, rows: torch.Tensor, stream=None) -> torch.Tensor:
        """The bytes of block rows `rows`, every layer: uint8 [n, block_bytes]."""
        dst = torch.empty((rows.numel(), block_bytes(self.handle)), dtype=torch.uint8, device=self.device)
        export_blocks(self.handle, rows, dst, stream)
        return dst

    def import_blocks(self, identity: StorageIdentity, rows: torch.Tensor, payload: torch.Tensor,
                      stream=None) -> None:
        import_blocks(self.handle, identity, rows, payload, stream)

    def save_checkpoint(self, path: str, rows: torch.Tensor) -> None:
        payload = self.export_blocks(rows)
        torch.cuda.synchronize(self.device)
        write_checkpoint(path, self.storage_identity(), payload)

    def restore_checkpoint(self, path: str, rows: torch.Tensor) -> None:
        """Restore a block checkpoint into rows `rows`.  The storage identity
        is checked before anything is allocated: a mismatch raises
        PagedKVError (status -7) with the pool and the device untouched.
        Then the rows are reserved (growth by slab append) and written."""
        ident, n = read_checkpoint_header(path)
        identity_check(self.handle, ident)
        if rows.numel() != n:
            raise ValueError(f"the checkpoint holds {n} blocks, {rows.numel()} rows given")
        size = len(CHECKPOINT_MAGIC) + ctypes.sizeof(StorageIdentity) + 8
        with open(path, "rb") as f:
            f.seek(size)
            data = f.read()
        import numpy as np
        payload = torch.from_numpy(np.frombuffer(data, dtype=np.uint8).copy()).to(self.device)
        if n:
            self.reserve_rows(int(rows.max().item()) + 1)
        import_blocks(self.handle, ident, rows, payload)

    def gather_visible(self, layer, block_table, lens, t_out, k_out, v_out, n_runs_out=None,
                       stream=None):
        B = block_table.shape[0] if block_table.dim() == 2 else -1
        self._check_table(block_table, lens, B)
        for name, t, rec in (("k_out", k_out, self.k_record_bytes), ("v_out", v_out, self.v_record_bytes)):
            _require(t, name)
            need = B * self.n_kv_heads * int(t_out) * rec
            if t.numel() * t.element_size() < need:
                raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes; "
                                 f"[{B}, {self.n_kv_heads}, {t_out}] records need {need}")
        gather_visible(self.handle, layer, block_table, lens, t_out, k_out, v_out, n_runs_out,
                       stream)

    def split_runs(self, block_table, lens, stream=None):
        """The same-slab runs of each sequence: (runs [B, max_blocks, 3] with
        -1 past each sequence's count, n_runs [B]), on the device."""
        B = block_table.shape[0] if block_table.dim() == 2 else -1
        self._check_table(block_table, lens, B)
        runs = torch.full((B, block_table.shape[1], 3), -1, dtype=torch.int32, device=self.device)
        n = torch.empty((B,), dtype=torch.int32, device=self.device)
        split_runs(self.handle, block_table, lens, runs, n, stream)
        return runs, n

    def workspace(self, B: int, n_q_heads: int, max_len: int) -> torch.Tensor:
        """A decode workspace for up to B sequences of at most max_len tokens."""
        n = decode_workspace_bytes(self.handle, B, n_q_heads, max_len)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)

    def paged_decode(self, layer, q, block_table, lens, max_len, scale, out, workspace,
                     stream=None, stage="all"):
        self._check_query(q, out)
        self._check_table(block_table, lens, q.shape[0])
        paged_decode(self.handle, layer, q, block_table, lens, max_len, scale, out, workspace,
                     stream, stage)

    def paged_decode_noalloc(self, layer, q, block_table, lens, max_len, scale, out, stream=None):
        self._check_query(q, out)
        self._check_table(block_table, lens, q.shape[0])
        paged_decode_noalloc(self.handle, layer, q, block_table, lens, max_len, scale, out, stream)

    def paged_decode_append(self, layer, q, k_new, v_new, block_table, lens, max_len, scale, out,
                            workspace, stream=None):
        self._check_query(q, out)
        self._check_table(block_table, lens, q.shape[0])
        self._check_tokens("k_new", k_new, q.shape[0])
        self._check_tokens("v_new", v_new, q.shape[0])
        paged_decode_append(self.handle, layer, q, k_new, v_new, block_table, lens, max_len, scale,
                            out, workspace, stream)

    def stats(self) -> dict:
        return pool_stats(self.handle)

    def check_error(self, stream=None) -> int:
        return pool_check_error(self.handle, stream)

    def set_debug(self, flags: int) -> None:
        pool_set_debug(self.handle, flags)

    def close(self) -> None:
        if getattr(self, "handle", None):
            pool_destroy(self.handle)
            self.handle = None
        self.k_slabs = [[] for _ in range(self.n_layers)]
        self.v_slabs = [[] for _ in range(self.n_layers)]

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
