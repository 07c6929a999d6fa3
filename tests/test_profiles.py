"""The committed rocprofv3 counter summaries (profiles/*_pmc.txt) are
self-consistent: the plain-copy calibration read its known size (FETCH_SIZE
counts about half the bytes fetched, WRITE_SIZE all the bytes written), and
the headline kernels' HBM traffic is within 10% above their algorithmic
bytes (more would mean re-reads; less, a broken calibration)."""
import glob
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _read(path):
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


def test_copy_calibration_of_every_counter_summary():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_pmc.txt")))
    assert paths
    for p in paths:
        kv = _read(p)
        assert 1.5 < float(kv["fetch_scale"]) < 2.5, p
        assert 0.8 < float(kv["write_scale"]) < 1.2, p
        assert abs(float(kv["copy_WRITE_SIZE_KiB"]) - 256 * 1024) < 1024, p


def test_headline_traffic_matches_the_algorithmic_bytes():
    import bench
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import workloads
    d, c = bench.algorithmic_bytes(workloads.CONFIGS["gen_zipf_h7168"], 13020)
    for kernel, alg in (("dispatch", d), ("combine", c)):
        kv = _read(os.path.join(ROOT, "profiles", f"{kernel}_gen_zipf_h7168_pmc.txt"))
        ratio = float(kv["hbm_bytes_per_launch"]) / alg
        assert 1.0 <= ratio < 1.1, (kernel, ratio)
