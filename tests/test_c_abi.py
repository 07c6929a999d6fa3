"""The C ABI from plain C (tests/c_abi/epdc_c_consumer.c): it compiles and
links against libepdc.so with gcc alone; on a GPU it runs dispatch, the
gather combine, push and reduce and matches the oracle bit for bit."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "epdc_c_consumer.c")
PKG = os.path.join(ROOT, "combine_count_amd")
ORACLE = os.path.join(ROOT, "oracle")


def build(out):
    import oracle
    oracle.load()  # builds liboracle.so if it is missing or stale
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", SRC,
           "-o", out, f"-L{PKG}", "-lepdc", f"-L{ORACLE}", "-loracle", "-L/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,{PKG}:{ORACLE}:/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def test_c_consumer_builds(tmp_path):
    build(str(tmp_path / "epdc_c_consumer"))


@pytest.mark.gpu
def test_c_consumer_matches_oracle(tmp_path):
    exe = build(str(tmp_path / "epdc_c_consumer"))
    print("[c abi] running the C consumer", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi ok" in r.stdout
