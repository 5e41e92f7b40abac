"""The bf16 payload quantization divides by the block scale with a reciprocal
and one fused correction instead of a correctly rounded division per value.
tests/fastdiv_check.c runs that formula on every pair of bf16 values (block
maximum, value) against the correctly rounded quotient; here it is built
with the host compiler and must report no differing code and no differing
quotient above 2^-10. (The GPU kernel's codes are checked bit for bit
against the oracle in tests/test_gpu_4_w8a8.py.)"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fast_quotient_matches_division_on_all_bf16_pairs(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    exe = str(tmp_path / "fastdiv_check")
    src = os.path.join(HERE, "fastdiv_check.c")
    base = [cc, "-O2", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe, "-lm"]
    r = subprocess.run(base[:1] + ["-fopenmp"] + base[1:], capture_output=True, text=True)
    if r.returncode != 0:  # no OpenMP: single-threaded (about a minute)
        r = subprocess.run(base, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=dict(os.environ, OMP_NUM_THREADS="8"))
    assert out.returncode == 0, out.stderr
    m = re.search(r"tested (\d+) code_mismatches (\d+) quotient_mismatches (\d+)", out.stdout)
    assert m, out.stdout
    tested, bad_code, bad_q = map(int, m.groups())
    assert tested > 10 ** 9
    assert bad_code == 0 and bad_q == 0, out.stdout
