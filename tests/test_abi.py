"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments on the host before touching a device (CPU only)."""

import ctypes
import os
import re

import pytest

import decode_memory_amd as pd
from oracle.packed import record_bytes as oracle_record_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pagedkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pd_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 16
    lib = pd.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(pd.EXPORTS) == names


def test_version_and_record_bytes():
    assert pd.version() == 1
    assert pd.record_bytes(pd.FMT_BF16, 128) == (256, 256)
    assert pd.record_bytes(pd.FMT_FP16, 64) == (128, 128)
    for fmt, (kb, vb) in {pd.FMT_K8V8: (8, 8), pd.FMT_K8V4: (8, 4), pd.FMT_K4V4: (4, 4)}.items():
        for d in (64, 128, 256):
            assert pd.record_bytes(fmt, d) == (oracle_record_bytes(d, kb), oracle_record_bytes(d, vb))
            assert pd.record_bytes(fmt, d, 64) == (oracle_record_bytes(d, kb, 64),
                                                   oracle_record_bytes(d, vb, 64))
    # K4 records with groups of 64 cost five bits per value (the PR #142 Summary figure)
    k4, _ = pd.record_bytes(pd.FMT_K4V4, 256, 64)
    assert k4 * 8 / 256 == 5 and 16 / (k4 * 8 / 256) == 3.2
    with pytest.raises(pd.PagedKVError) as e:
        pd.record_bytes(9, 64)
    assert e.value.status == -1
    with pytest.raises(pd.PagedKVError) as e:
        pd.record_bytes(pd.FMT_K8V8, 64, 48)           # a group must divide head_dim
    assert e.value.status == -1


@pytest.mark.parametrize("kwargs,status", [
    (dict(head_dim=96), -4),                      # no kernel for this head_dim
    (dict(block_size=24), -4),
    (dict(fmt=7), -1),                            # unknown format
    (dict(n_layers=0), -1),
    (dict(slab_blocks=0), -1),
    (dict(fmt=pd.FMT_K4V4, hadamard_signs=None), -1),   # packed needs signs
    (dict(fmt=pd.FMT_K4V4, head_dim=64, hadamard_signs=[1, 0] * 32), -1),  # not +-1
    (dict(fmt=pd.FMT_K4V4, head_dim=64, hadamard_signs=[1] * 64, group_size=64), -4),  # 40-byte records
    (dict(fmt=pd.FMT_K8V8, head_dim=128, hadamard_signs=[1] * 128, group_size=16), -4),
    (dict(fmt=pd.FMT_BF16, group_size=32), -1),  # 16-bit formats have no groups
    # the packed decode kernel takes 8 kv heads: other head counts are refused
    # at create, before anything could be written into a pool it cannot read
    (dict(fmt=pd.FMT_K8V8, n_kv_heads=4, hadamard_signs=[1] * 128), -4),
    (dict(fmt=pd.FMT_K4V4, n_kv_heads=16, hadamard_signs=[1] * 128), -4),
    (dict(fmt=pd.FMT_K8V4, n_kv_heads=1, hadamard_signs=[1] * 128), -4),
])
def test_pool_create_validates_on_host(kwargs, status):
    args = dict(n_layers=2, block_size=32, n_kv_heads=8, head_dim=128, slab_blocks=4,
                max_slabs=8, fmt=pd.FMT_BF16, hadamard_signs=None)
    args.update(kwargs)
    with pytest.raises(pd.PagedKVError) as e:
        pd.pool_create(**args)
    assert e.value.status == status


def test_dense_workspace_query_bounds_the_launch_on_host():
    """Dense decode sizes are checked on the host: the kernels form row
    b * ceil(max_len / 32) + j and the (sequence, query head, split) rows of
    the workspace in 32 bits, so batches past those ranges are argument
    errors, while a qwen3-shaped batch gets its workspace size."""
    per_split = 8 * 16 * (128 + 2) * 4  # B x n_q x (weighted V + max, sum), fp32
    ok = pd.dense_workspace_bytes("bf16", 8, 128, 8, 16, 4096)
    assert ok >= per_split and ok % 4 == 0
    with pytest.raises(pd.PagedKVError) as e:  # 131073 x 16384 rows
        pd.dense_workspace_bytes("bf16", 8, 128, 131073, 8, 524288)
    assert e.value.status == -1
    with pytest.raises(pd.PagedKVError) as e:  # 131073 x 8192 query heads, one split
        pd.dense_workspace_bytes("bf16", 1024, 64, 131073, 8192, 32)
    assert e.value.status == -1
    assert pd.dense_workspace_bytes("bf16", 1024, 64, 131072, 8192, 32) > 0  # 2^30 rows fit


C_PROGRAM = r"""
#include <stdio.h>
#include "pagedkv.h"
int main(void) {
  int32_t k = 0, v = 0;
  uint64_t h = 0;
  const int8_t signs[4] = {1, -1, 1, 1};
  if (pd_record_bytes(PD_FMT_K4V4, 64, 48, &k, &v) != PD_ERR_ARG) return 2;  /* 48 does not divide 64 */
  if (pd_record_bytes(PD_FMT_K8V4, 256, 64, &k, &v) != PD_OK) return 3;
  if (pd_signs_hash(signs, 4, &h) != PD_OK) return 4;
  printf("%d %d %d %llu\n", pd_version(), k, v, (unsigned long long)h);
  return 0;
}
"""


def test_header_compiles_as_c_and_the_library_links(tmp_path):
    """The boundary is a C ABI: a plain C99 program includes pagedkv.h,
    links libpagedkv.so and calls its host-only entry points."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    lib_dir = os.path.dirname(pd.LIB_PATH)
    pd.lib()  # raises if the library has not been built
    src, exe = tmp_path / "abi.c", tmp_path / "abi"
    src.write_text(C_PROGRAM)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
                        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                        str(src), "-L", lib_dir, "-lpagedkv", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, (r.returncode, r.stderr)
    version, k, v, h = (int(x) for x in r.stdout.split())
    assert version == pd.version()
    assert (k, v) == (oracle_record_bytes(256, 8, 64), oracle_record_bytes(256, 4, 64))
    assert h == pd.signs_hash([1, -1, 1, 1])


def test_status_names_cover_the_header():
    """Every pd_status value the header declares has its name in the binding."""
    text = open(os.path.join(ROOT, "include", "pagedkv.h")).read()
    declared = {int(v): n for n, v in re.findall(r"\b(PD_(?:OK|ERR_[A-Z]+))\s*=\s*(-?\d+)", text)}
    assert declared and declared == pd.STATUS


def test_null_pool_is_an_argument_error():
    lib = pd.lib()
    assert lib.pd_pool_stats(None, None) == -1
    assert lib.pd_pool_destroy(None) == 0
    assert lib.pd_write_block(None, 0, 0, None, None, None, None, None) == -1
    assert b"NULL" in lib.pd_last_error()


def test_signs_hash_is_fnv1a_of_the_sign_bytes():
    """pd_signs_hash (host only) against the oracle's FNV-1a over the stored
    sign bytes; a flipped sign changes it."""
    from oracle.slab_pool import signs_fingerprint
    from synth import hadamard_signs
    for D in (64, 128, 256):
        s = [int(x) for x in hadamard_signs(5, D)]
        assert pd.signs_hash(s) == signs_fingerprint(s)
        t = list(s)
        t[D // 2] = -t[D // 2]
        assert pd.signs_hash(t) != pd.signs_hash(s)
    assert pd.signs_hash([]) == 0xCBF29CE484222325


def test_storage_identity_is_48_packed_bytes():
    assert ctypes.sizeof(pd.StorageIdentity) == 48
    ident = pd.StorageIdentity(magic=0x564B4450, layout=1, format=4, n_layers=2, block_size=32,
                               n_kv_heads=8, head_dim=64, k_record_bytes=48, v_record_bytes=48,
                               group_size=32, signs_hash=123)
    b = ident.to_bytes()
    assert b[:4] == b"PDKV" and len(b) == 48
    assert pd.StorageIdentity.from_bytes(b).as_dict() == ident.as_dict()
