"""The float64 exp behind the expansion's row sums, checked on the CPU.

csrc/exp64.h is shared by the device kernels and this host build, so the device
arithmetic itself is what is checked: the 2^(i/64) table against values computed to 60
digits (each must be the nearest float64), the stated error bound (4 + |d|) * 2^-53
against long-double exp over about 1.7 million float32 logit pairs, and the special values the
row sums rely on (exp(0) = 1 exactly, NaN for a NaN or -inf argument, 0 far below)."""

import os
import shutil
import subprocess
import tempfile
from decimal import Decimal, getcontext

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CXX = shutil.which("g++") or shutil.which("c++")


@pytest.fixture(scope="module")
def report():
    if CXX is None:
        pytest.skip("no host C++ compiler")
    d = tempfile.mkdtemp(prefix="exp64_")
    exe = os.path.join(d, "exp64_check")
    r = subprocess.run([CXX, "-O2", "-std=c++17", "-DTV_HD=",
                        "-I", os.path.join(ROOT, "tree_attention_verify_ancestor_amd", "csrc"),
                        os.path.join(ROOT, "tests", "exp64_check.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    lines = {}
    tab = {}
    for ln in out.stdout.splitlines():
        f = ln.split()
        if f[0] == "tab":
            tab[int(f[1])] = float.fromhex(f[2])
        else:
            lines[f[0]] = f[1:]
    shutil.rmtree(d, ignore_errors=True)
    return lines, tab


def test_table_is_correctly_rounded(report):
    _, tab = report
    getcontext().prec = 60
    assert len(tab) == 64
    for i, v in tab.items():
        assert v == float(Decimal(2) ** (Decimal(i) / 64)), i


def test_error_within_stated_bound(report):
    lines, _ = report
    assert int(lines["checked"][0]) > 1_500_000
    assert float(lines["worst"][0]) <= 1.5


def test_special_values(report):
    lines, _ = report
    assert float.fromhex(lines["zero"][0]) == 1.0
    got, ref = (float.fromhex(x) for x in lines["minus_one"])
    assert abs(got - ref) <= 2 * 2.0 ** -53 * ref
    assert lines["nan"][0] == "1" and lines["neg_inf"][0] == "1"
    assert float.fromhex(lines["huge"][0]) == 0.0
    assert float.fromhex(lines["deep"][0]) == 0.0
