"""The dispatch maps an expert id to its PE with a multiply-high division
(epdc::div_magic in csrc/epdc_internal.h).  A host program built from that
header checks it against the divide instruction (tests/host/div_magic_check.cpp)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_div_magic_matches_division(tmp_path):
    import sys
    sys.path.insert(0, ROOT)
    from combine_count_amd import _build as B
    exe = str(tmp_path / "div_magic_check")
    src = os.path.join(ROOT, "tests", "host", "div_magic_check.cpp")
    r = subprocess.run([B.HIPCC, *B.COMMON, src, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 wrong" in r.stdout
