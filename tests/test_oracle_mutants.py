"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant below is one slip someone could make while writing the oracle
from the pages -- a dropped term, a wrong sign, index or axis, a transposed
operand, swapped fields -- planted into the oracle for the duration of one
case: the function (or method) is replaced wherever it is bound, in the
oracle's modules and in this test's own copies of the pin modules.  The pins
then run, and at least one of them must fail.  Nothing here changes the
oracle on disk; every mutant is undone after its case.
"""

import importlib
import itertools
import sys

import numpy as np
import pytest

import oracle.attention as att
import oracle.footprint as fp
import oracle.packed as pk
import oracle.slab_pool as sp

PIN_MODULES = ["tests.test_oracle_attention", "tests.test_oracle_packed", "tests.test_oracle_pool",
               "tests.test_oracle_footprint"]
# imported before any mutant is bound, so that every rebinding (and its undo)
# reaches the names these modules imported from the oracle
_PIN_MODS = [importlib.import_module(name) for name in PIN_MODULES]


def _pins():
    """Zero-argument calls of every pin, parametrized cases expanded; the
    property-based pins (hypothesis) last, as they shrink a failure slowly."""
    plain, hyp = [], []
    for name, mod in zip(PIN_MODULES, _PIN_MODS):
        for attr, fn in vars(mod).items():
            if not attr.startswith("test_") or not callable(fn):
                continue
            grids = []
            for mark in getattr(fn, "pytestmark", []):
                if mark.name == "parametrize":
                    names = [n.strip() for n in mark.args[0].split(",")]
                    rows = [v if len(names) > 1 else (v,) for v in mark.args[1]]
                    grids.append([dict(zip(names, r)) for r in rows])
            cases = [{}] if not grids else [
                {k: v for part in combo for k, v in part.items()} for combo in itertools.product(*grids)]
            target = hyp if hasattr(fn, "hypothesis") else plain
            target += [(f"{name}::{attr}{c or ''}", fn, c) for c in cases]
    return plain + hyp


def _first_failing_pin():
    for label, fn, kwargs in _pins():
        try:
            fn(**kwargs)
        except Exception:  # an assertion, or the mutant breaking a shape
            return label
    return None


def _rebind(owner, name, new):
    """Replace owner.name (a module function or a class attribute) with new,
    in the owner and in every loaded oracle or pin module that imported it.
    Returns an undo list."""
    old = getattr(owner, name)
    undo = [(owner, name, old)]
    setattr(owner, name, new)
    if isinstance(owner, type):
        return undo
    for modname, mod in list(sys.modules.items()):
        if mod is None or not (modname.startswith("oracle") or modname.startswith("tests.test_oracle")):
            continue
        for k, v in list(vars(mod).items()):
            if v is old and mod is not owner:
                undo.append((mod, k, v))
                setattr(mod, k, new)
    return undo


# ---- mutants: (owner, attribute, replacement) --------------------------------

def m_scale_dropped(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    s = k @ q.T
    w = np.exp(s - s.max(axis=0, keepdims=True))
    return (w.T @ v) / w.sum(axis=0)[:, None]


def m_not_normalised(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    s = scale * (k @ q.T)
    w = np.exp(s - s.max(axis=0, keepdims=True))
    return w.T @ v


def m_score_sign(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    s = -scale * (k @ q.T)
    w = np.exp(s - s.max(axis=0, keepdims=True))
    return (w.T @ v) / w.sum(axis=0)[:, None]


def m_max_over_wrong_axis(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1]))
    s = scale * (k @ q.T)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return (w.T @ v) / w.sum(axis=0)[:, None]


def m_last_token_dropped(q, k, v, scale):
    return _ORIG["attend_one"](q, k[:-1], v[:-1], scale) if k.shape[0] > 1 else _ORIG["attend_one"](q, k, v, scale)


def m_gqa_interleaved(q, ks, vs, scale):
    B, n_q, D = q.shape
    out = np.zeros((B, n_q, vs[0].shape[-1] if B else D))
    for b in range(B):
        n_kv = ks[b].shape[1]
        for h in range(n_q):
            out[b, h:h + 1] = att.attend_one(q[b, h:h + 1], ks[b][:, h % n_kv, :], vs[b][:, h % n_kv, :], scale)
    return out


def m_k_v_swapped(q, ks, vs, scale):
    return _ORIG["decode_attention"](q, vs, ks, scale)


def m_widen_bf16_shift(bits, dtype):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return _ORIG["widen"](bits, dtype)


def m_bf16_round_7_bits(x, dtype):
    if dtype == "bf16":
        m, e = np.frexp(np.asarray(x, np.float64))
        return np.ldexp(np.rint(m * 128.0), e - 7)
    return _ORIG["round_to_dtype"](x, dtype)


def m_rotation_unnormalised(x, signs):
    return _ORIG["rotate_fp32"](x, signs) / pk.inv_sqrt_f32(x.shape[-1])


def m_rotation_unsigned(x, signs):
    return _ORIG["rotate_fp32"](x, np.ones_like(signs))


def m_exact_rotation_by_d(x, signs):
    return _ORIG["rotate_exact"](x, signs) / np.sqrt(x.shape[-1])


def _quantise_with(x, bits, group, levels_of, offset_of, round_fn):
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (d // group, group))
    mn, mx = g.min(axis=-1), g.max(axis=-1)
    levels = np.float32(levels_of(bits))
    scale = ((mx - mn) / levels).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1), scale).astype(np.float32)
    off = offset_of(mn, mx)
    t = ((g - off[..., None]) / safe[..., None]).astype(np.float32)
    codes = np.clip(round_fn(t), 0, (1 << bits) - 1)
    codes = np.where(scale[..., None] == 0, 0, codes).astype(np.uint8)
    return codes.reshape(x.shape), scale, off.astype(np.float32)


def m_offset_is_max(x, bits, group=pk.GROUP):
    return _quantise_with(x, bits, group, lambda b: (1 << b) - 1, lambda mn, mx: mx, np.rint)


def m_levels_off_by_one(x, bits, group=pk.GROUP):
    return _quantise_with(x, bits, group, lambda b: 1 << b, lambda mn, mx: mn, np.rint)


def m_floor_not_round(x, bits, group=pk.GROUP):
    return _quantise_with(x, bits, group, lambda b: (1 << b) - 1, lambda mn, mx: mn, np.floor)


def m_nibbles_swapped(codes, scale, offset, bits):
    if bits == 4:
        c = np.asarray(codes, np.uint8).copy()
        c[..., 0::2], c[..., 1::2] = codes[..., 1::2], codes[..., 0::2]
        return _ORIG["pack"](c, scale, offset, bits)
    return _ORIG["pack"](codes, scale, offset, bits)


def m_meta_swapped(records, head_dim, bits, group=pk.GROUP):
    codes, scale, offset = _ORIG["unpack"](records, head_dim, bits, group)
    return codes, offset, scale


def m_offset_dropped(codes, scale, offset):
    return _ORIG["dequantise"](codes, scale, np.zeros_like(offset))


def m_query_not_rotated(q_bits, k_recs, v_recs, signs, fmt, head_dim, scale, group=pk.GROUP):
    kb, vb = pk.FORMATS[fmt]
    ks = [pk.dequantise_records(k, head_dim, kb, group) for k in k_recs]
    vs = [pk.dequantise_records(v, head_dim, vb, group) for v in v_recs]
    return att.decode_attention(att.widen(q_bits, "bf16"), ks, vs, scale)


def m_keys_not_rotated(k_bits, signs, bits, group=pk.GROUP):
    return _ORIG["v_records"](k_bits, bits, group)


def m_metadata_4_bytes(head_dim, bits, group=pk.GROUP):
    return head_dim * bits // 8 + (head_dim // group) * 4


def m_slab_index_swapped(self, layer, row):
    slab = row % self.slab_blocks
    return self.k_slabs[layer][slab], self.v_slabs[layer][slab], row // self.slab_blocks


def m_runs_never_merge(self, rows):
    return [(int(r) // self.slab_blocks, i, 1) for i, r in enumerate(rows)]


def m_gather_not_transposed(self, layer, rows, length):
    k, v = _ORIG["gather"](self, layer, rows, length)
    return np.ascontiguousarray(k.transpose(1, 0, 2)), np.ascontiguousarray(v.transpose(1, 0, 2))


def m_append_first_layer_only(self):
    shape = (self.slab_blocks, self.block_size, self.n_kv_heads)
    self.k_slabs[0].append(np.zeros(shape + (self.k_rec,), dtype=np.uint8))
    self.v_slabs[0].append(np.zeros(shape + (self.v_rec,), dtype=np.uint8))
    self.slab_append_events += 1
    return self.n_slabs - 1


def m_copy_in_place(self, src_rows, dst_rows):
    for layer in range(self.n_layers):
        for src, dst in zip(src_rows, dst_rows):
            ks, vs, r = self.slab_for_row(layer, int(src))
            kd, vd, rd = self.slab_for_row(layer, int(dst))
            kd[rd] = ks[r]
            vd[rd] = vs[r]


def m_fnv1_order(data):
    h = 0xcbf29ce484222325  # FNV-1: multiply, then xor
    for byte in data:
        h = ((h * 0x100000001b2) & 0xFFFFFFFFFFFFFFFF) ^ byte
    return h


def m_ladder_forgotten(lengths, block_size, chunk_blocks, block_bytes):
    rows, cap = 0, 0
    for n in lengths:
        rows += fp.blocks_for(n, block_size)
        cap = max(cap, -(-rows // chunk_blocks) * chunk_blocks)
    return cap * block_bytes


def m_capacity_in_blocks(lengths, block_size, slab_blocks, block_bytes):
    out, rows = [], 0
    for n in lengths:
        rows += fp.blocks_for(n, block_size)
        out.append(rows * block_bytes)
    return out


_ORIG = {"attend_one": att.attend_one, "decode_attention": att.decode_attention, "widen": att.widen,
         "round_to_dtype": att.round_to_dtype, "rotate_fp32": pk.rotate_fp32, "rotate_exact": pk.rotate_exact,
         "pack": pk.pack, "unpack": pk.unpack, "dequantise": pk.dequantise, "v_records": pk.v_records,
         "gather": sp.SlabPoolModel.gather}

MUTANTS = {
    "attention: scale dropped": (att, "attend_one", m_scale_dropped),
    "attention: no normalisation by the weight sum": (att, "attend_one", m_not_normalised),
    "attention: score sign flipped": (att, "attend_one", m_score_sign),
    "attention: max taken over the query axis": (att, "attend_one", m_max_over_wrong_axis),
    "attention: last visible token dropped": (att, "attend_one", m_last_token_dropped),
    "attention: query head h reads kv head h % n_kv": (att, "decode_attention", m_gqa_interleaved),
    "attention: K and V swapped": (att, "decode_attention", m_k_v_swapped),
    "attention: bf16 widened with a 15-bit shift": (att, "widen", m_widen_bf16_shift),
    "attention: bf16 output rounded to 7 bits": (att, "round_to_dtype", m_bf16_round_7_bits),
    "packed: butterflies without 1/sqrt(D)": (pk, "rotate_fp32", m_rotation_unnormalised),
    "packed: butterflies without the signs": (pk, "rotate_fp32", m_rotation_unsigned),
    "packed: exact rotation divided by D": (pk, "rotate_exact", m_exact_rotation_by_d),
    "packed: offset is the group max": (pk, "quantise", m_offset_is_max),
    "packed: 2^bits levels instead of 2^bits - 1": (pk, "quantise", m_levels_off_by_one),
    "packed: codes floored instead of rounded": (pk, "quantise", m_floor_not_round),
    "packed: nibbles of a byte swapped": (pk, "pack", m_nibbles_swapped),
    "packed: scale and offset swapped on unpack": (pk, "unpack", m_meta_swapped),
    "packed: offset dropped on dequantise": (pk, "dequantise", m_offset_dropped),
    "packed: query not rotated": (pk, "packed_decode_attention", m_query_not_rotated),
    "packed: keys not rotated": (pk, "k_records", m_keys_not_rotated),
    "packed: 4 metadata bytes per group": (pk, "record_bytes", m_metadata_4_bytes),
    "pool: row % S taken as the slab": (sp.SlabPoolModel, "slab_for_row", m_slab_index_swapped),
    "pool: runs never merged": (sp.SlabPoolModel, "split_runs", m_runs_never_merge),
    "pool: gather not transposed": (sp.SlabPoolModel, "gather", m_gather_not_transposed),
    "pool: growth appends to layer 0 only": (sp.SlabPoolModel, "append_slab", m_append_first_layer_only),
    "pool: copy_block writes while it reads": (sp.SlabPoolModel, "copy_block", m_copy_in_place),
    "pool: FNV-1 (multiply before xor) for FNV-1a": (sp, "fnv1a64", m_fnv1_order),
    "footprint: growth by copy forgets the freed ladder": (fp, "growth_by_copy_peak", m_ladder_forgotten),
    "footprint: slab capacity counted in blocks": (fp, "slab_pool_capacity", m_capacity_in_blocks),
}


def test_the_unmutated_oracle_passes_every_pin():
    assert _first_failing_pin() is None


@pytest.mark.parametrize("label", list(MUTANTS))
def test_each_planted_mistake_fails_a_pin(label):
    owner, name, new = MUTANTS[label]
    undo = _rebind(owner, name, new)
    try:
        killed_by = _first_failing_pin()
    finally:
        for obj, attr, old in reversed(undo):
            setattr(obj, attr, old)
    assert killed_by is not None, f"no pin fails with the mutant '{label}'"
