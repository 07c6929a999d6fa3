"""The launch geometry of the three kernels (epdc::plan_dispatch,
plan_combine and plan_push: host code the launchers run) for the shapes
their rules were measured on.  Every plan gives the same results (the GPU
parity tests cover them all); this pins which one each shape gets, so that a
rule cannot change by accident."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FIELDS = ("cpw", "ntw", "nSlabs", "nSubs", "nBlocks", "full", "local", "selfScan", "xEarly")
ROW_FIELDS = ("cpw", "nSlabs", "waves", "nBlocks", "full")
EXPECT = {
    # (numTokens, rowBytes): (cpw, ntw, nSlabs, nSubs, nBlocks, full, local, selfScan, xEarly)
    # 4096 tokens x h7168 bf16: two 7-chunk slabs, 2048 blocks, tile leaders publish, x after the SCAN
    (4096, 14336): (7, 1, 2, 16, 2048, 1, 0, 0, 0),
    # fp8 rows: one 7-chunk slab, 1024 blocks: every block sums the counts, x after the SCAN
    (4096, 7168): (7, 1, 1, 16, 1024, 1, 0, 1, 0),
    # fp4x2 rows (3.5 KiB): one bound-checked 4-chunk slab, self-summing, x before COUNT
    (4096, 3584): (4, 1, 1, 16, 1024, 0, 0, 1, 1),
    # h2048 bf16: one 4-chunk slab, self-summing, x before COUNT
    (4096, 4096): (4, 1, 1, 16, 1024, 1, 0, 1, 1),
    # fp32 rows: four 7-chunk slabs, 4096 blocks: x before COUNT
    (4096, 28672): (7, 1, 4, 16, 4096, 1, 0, 0, 1),
    # 16384 tokens: 8192 blocks, x before COUNT
    (16384, 14336): (7, 1, 2, 16, 8192, 1, 0, 0, 1),
    # one tile: 2-chunk slabs (at most 4 tiles), local scan
    (1, 14336): (2, 1, 7, 16, 112, 1, 1, 0, 0),
    (8, 14336): (2, 1, 7, 16, 112, 1, 1, 0, 0),
    # two tiles of odd-chunk fp8 rows: 1-chunk slabs, local scan
    (128, 7168): (1, 1, 7, 16, 224, 1, 1, 0, 0),
    # 8 tiles: 7-chunk slabs, still the local scan; 9 tiles: self-summing
    (512, 14336): (7, 1, 2, 16, 256, 1, 1, 0, 0),
    (576, 14336): (7, 1, 2, 16, 288, 1, 0, 1, 0),
    # around the self-summing limit (1024 blocks)
    (2047, 14336): (7, 1, 2, 16, 1024, 1, 0, 1, 0),
    (2049, 14336): (7, 1, 2, 16, 1056, 1, 0, 0, 0),
    # around the x-early limit (2560 blocks): 80 and 81 tiles
    (5120, 14336): (7, 1, 2, 16, 2560, 1, 0, 0, 0),
    (5121, 14336): (7, 1, 2, 16, 2592, 1, 0, 0, 1),
    # 528-byte rows: more than 16384 / 32768 one-token waves take 2 / 4 tokens per wave
    (66000, 528): (1, 2, 1, 8, 8256, 0, 0, 0, 1),
    (132000, 528): (1, 4, 1, 4, 8252, 0, 0, 0, 1),
    # 8-chunk slabs; rows past 8 chunks that are not whole: 8-chunk slabs with bound checks
    (1000, 8192): (8, 1, 1, 16, 256, 1, 0, 1, 0),
    (1000, 9728): (8, 1, 2, 16, 512, 0, 0, 1, 0),
    # no tokens: nothing but recvCount
    (0, 14336): (0, 0, 0, 0, 0, 0, 0, 0, 0),
}


COMBINE = {
    # (numTokens, rowBytes): (cpw, nSlabs, waves, nBlocks, full)
    # 2-chunk slabs when the row splits evenly and that leaves >= 8192 waves
    (4096, 14336): (2, 7, 28672, 7168, 1),      # bf16 out, h7168
    (4096, 28672): (2, 14, 57344, 14336, 1),    # fp32 out
    (4096, 4096): (2, 2, 8192, 2048, 1),        # h2048: exactly 8192 waves
    (1024, 14336): (1, 14, 14336, 3584, 1),     # 7168 two-chunk waves: too few
    (4000, 5632): (2, 3, 12000, 3000, 0),       # 5.5 KiB rows: 6 chunks, the last one checked
    (8, 256): (1, 1, 8, 2, 0),                  # h128: a quarter chunk
    (1, 14336): (1, 14, 14, 4, 1),
}
PUSH = {
    # (landing rows, rowBytes): (cpw, nSlabs, waves, nBlocks, full); slab width as in the dispatch
    (32768, 14336): (7, 2, 65536, 16384, 1),    # 4096 tokens x min(8, 8) landing rows, bf16
    (32768, 28672): (7, 4, 131072, 32768, 1),   # fp32
    (3072, 4096): (4, 1, 3072, 768, 1),
    (1000, 5632): (7, 1, 1000, 250, 0),         # ragged 5.5 KiB rows
    (8, 16384): (8, 2, 16, 4, 1),
}


def _run(exe, kind, table):
    args = [str(v) for shape in table for v in shape]
    r = subprocess.run([exe, kind, *args], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    got = {}
    for line in r.stdout.split("\n"):
        if line.strip():
            v = [int(x) for x in line.split()]
            got[(v[0], v[1])] = tuple(v[2:])
    return got


def test_launch_plans(tmp_path):
    import sys
    sys.path.insert(0, ROOT)
    from combine_count_amd import _build as B
    exe = str(tmp_path / "launch_plan_check")
    src = os.path.join(ROOT, "tests", "host", "launch_plan_check.cpp")
    r = subprocess.run([B.HIPCC, *B.COMMON, src, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    for kind, table, fields in (("dispatch", EXPECT, FIELDS), ("combine", COMBINE, ROW_FIELDS),
                                ("push", PUSH, ROW_FIELDS)):
        got = _run(exe, kind, table)
        for shape, exp in table.items():
            assert got.get(shape) == exp, (f"{kind} {shape}: {dict(zip(fields, got.get(shape, ())))} "
                                           f"!= {dict(zip(fields, exp))}")


def _gpu_parity_shapes():
    """(numTokens, dispatch row bytes) of the dispatches the GPU parity tests run."""
    import workloads
    import test_gpu_parity as P
    import test_gpu_random_shapes as R
    wb = workloads.WIRE_BYTES
    shapes = set()
    for name, _ in P.CONFIG_SEEDS:
        w = workloads.CONFIGS[name]
        shapes.add((w.numTokens, w.dispatchHidden * wb[w.wire]))
    for _name, _W, _Epr, _M, T, _K, H, _routing, _useW in P.EDGE:
        shapes.add((T, H * 2))
    for name, base, wire, comb in P.DTYPES:
        if base is None:
            w = workloads.Workload(name, 5, 3, 700, 650, 7, 1056, "uniform", 1, wire=wire, combineDtype=comb)
        else:
            w = workloads.CONFIGS[base].with_(wire=wire, combineDtype=comb)
        rb = w.dispatchHidden * wb[wire] + (56 * 4 if name == "fp8_rows_with_block_scales" else 0)
        shapes.add((w.numTokens, rb))
    for _id, name, over in P.GRAPH_CASES:
        w = workloads.CONFIGS[name].with_(**(over or {}))
        shapes.add((w.numTokens, w.dispatchHidden * wb[w.wire]))
    for _i, _W, _Epr, _M, T, _K, H, dt, _useW, _routing in R.CASES:
        shapes.add((T, H * wb[dt]))
    return sorted(shapes)


def test_gpu_parity_reaches_the_dispatch_variants(tmp_path):
    """The GPU parity cases reach 36 of the 40 dispatch geometries (slab width x
    tokens per wave x bound checks, and the local scan's) -- all but 7- and
    8-chunk slabs at four tokens per wave (rows of 5.5 KiB and more at over
    132,000 tokens, the same code as the reached ones) -- and every combination
    of SCAN form (tile leader / every block) and x order (each non-local
    geometry is compiled once per x order)."""
    import sys
    sys.path.insert(0, ROOT)
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from combine_count_amd import _build as B
    exe = str(tmp_path / "launch_plan_check")
    r = subprocess.run([B.HIPCC, *B.COMMON, os.path.join(ROOT, "tests", "host", "launch_plan_check.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    shapes = [s for s in _gpu_parity_shapes() if s[0] > 0]
    got = _run(exe, "dispatch", shapes)
    variants, modes = set(), set()
    for cpw, ntw, _nSlabs, _nSubs, _nBlocks, full, local, self_scan, x_early in got.values():
        variants.add((cpw, ntw, full, local))
        if not local:
            modes.add((self_scan, x_early))
    compiled = {(c, n, f, 0) for c in (1, 2, 4, 7, 8) for n in (1, 2, 4) for f in (0, 1)}
    compiled |= {(c, 1, f, 1) for c in (1, 2, 4, 7, 8) for f in (0, 1)}
    missing = compiled - variants
    assert missing <= {(7, 4, 0, 0), (7, 4, 1, 0), (8, 4, 0, 0), (8, 4, 1, 0)}, sorted(missing)
    assert modes == {(0, 0), (0, 1), (1, 0), (1, 1)}, sorted(modes)
