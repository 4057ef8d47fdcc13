"""Host checks of the packed write's arithmetic shortcuts (no GPU): the scale
RN(range / levels) from a product and one fma correction equals the IEEE
quotient for every finite non-negative fp32 range at 4 and 8 bits
(mlx-swift-lm PR #142, "Add packed paged KV formats with bounded workspace
admission", section "Summary": fp32 scale per group)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_scale_division_without_divide_is_exact(tmp_path):
    exe = tmp_path / "div_levels"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "host_numerics", "div_levels.c"), "-lm"], check=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("mismatches 0 ") == 2
