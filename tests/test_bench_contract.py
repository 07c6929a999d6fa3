"""bench.py's command-line contract that holds without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_default_workload():
    """Per-kernel byte counts of the 4096-token h7168 workload at U = 13,020
    unique (token, PE) pairs (the seed-1 value), written out term by term."""
    sys.path.insert(0, ROOT)
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import bench
    import workloads
    w = workloads.CONFIGS["gen_zipf_h7168"]
    U, T, K, W, row = 13020, 4096, 8, 8, 7168 * 2
    d, c = bench.algorithmic_bytes(w, U)
    assert d == T * row + 3 * T * K * 4 + U * row + U * 4 + 2 * U * K * 4 + W * 4 == 246653584
    assert c == 3 * T * K * 4 + U * row + T * row == 245768192
    p, r = bench.push_bytes(w, U)
    assert p == 2 * U * row + U * K * 8 + U * 4 + W * 4
    assert r == T * K * 4 + W * 4 + U * row + U * 4 + T * row


def test_kernel_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    """The counters' validity key: a comment or layout edit keeps it, a code
    edit changes it."""
    sys.path.insert(0, ROOT)
    import bench
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    src.write_text("int f(int a) { return a + 1; }  // add one\n")
    h0 = bench.kernel_source_hash()
    src.write_text("/* a block\n comment */\nint f(int a) {\n    return a + 1;  // plus one\n}\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f(int a) { return a + 2; }  // add one\n")
    assert bench.kernel_source_hash() != h0


def test_cpu_baseline_names_its_host():
    """The CPU figure carries the host it ran on: CPU model and core counts."""
    sys.path.insert(0, ROOT)
    import bench
    h = bench.host_cpu()
    assert set(h) == {"cpu_model", "nproc", "usable_cores"}
    assert h["nproc"] >= 1 and 1 <= h["usable_cores"] <= h["nproc"]
    assert h["cpu_model"] is None or isinstance(h["cpu_model"], str)


def test_timed_path_does_not_import_the_oracle():
    """bench.py's timed path (the package, the input generator and the device
    harness) leaves the oracle unloaded; only its cpu_baseline leg imports it."""
    code = ("import sys; sys.path[:0] = [{root!r}, {tests!r}]\n"
            "import bench, combine_count_amd, workloads, gpu_harness\n"
            "assert 'oracle' not in sys.modules, sorted(m for m in sys.modules if 'oracle' in m)\n"
            "print('ok')\n").format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr[-2000:]


def test_rotation_leaves_no_set_in_the_cache():
    """Every configuration whose inputs are not a few KB rotates enough
    buffer sets that the bytes read or written with cache-allocating
    accesses exceed twice the 256 MB memory-side cache, within the 24 GB
    buffer cap; the 4096-token h7168 workload takes 9 sets."""
    sys.path.insert(0, ROOT)
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import bench
    import workloads

    class _Cuda:
        @staticmethod
        def mem_get_info():
            return 250 << 30, 288 << 30

    class _Torch:
        cuda = _Cuda()

    assert bench.rotation(_Torch, workloads.CONFIGS["gen_zipf_h7168"], False, 0) == 9
    assert bench.rotation(_Torch, workloads.CONFIGS["gen_zipf_h7168"], False, 2) == 2
    for name in ("gen_zipf_h7168", "gen_zipf_h2048", "pr_scale", "epcfg_defaults", "large_weighted",
                 "large_unweighted"):
        w = workloads.CONFIGS[name]
        for push in (False, True):
            n = bench.rotation(_Torch, w, push, 0)
            assert n * bench.cacheable_bytes(w) > bench.COLD_BYTES, (name, push, n)
            assert n * bench.set_bytes(w, push) <= 24 << 30, (name, push, n)
    # x, ids, weights, sendMap and the metadata of at most min(W, K) rows per token
    w = workloads.CONFIGS["gen_zipf_h7168"]
    T, K, row = 4096, 8, 7168 * 2
    assert bench.cacheable_bytes(w) == T * (row + K * 8) + T * K * 4 + T * 8 * (4 + K * 8)
