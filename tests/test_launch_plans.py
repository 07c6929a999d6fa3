"""The launch geometry of the three kernels (epdc::plan_dispatch,
plan_combine and plan_push: host code the launchers run) for the shapes
their rules were measured on.  Every plan gives the same results (the GPU
parity tests cover them all); this pins which one each shape gets, so that a
rule cannot change by accident."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FIELDS = ("cpw", "ntw", "nSlabs", "nSubs", "nBlocks", "full", "scan")
ROW_FIELDS = ("cpw", "nSlabs", "waves", "nBlocks", "full")
EXPECT = {
    # (numTokens, rowBytes, worldSize): (cpw, ntw, nSlabs, nSubs, nBlocks, full, scan)
    # scan: 0 local (every block counts the earlier tiles' ids), 1 every block sums the leaders'
    # published counts, 2 the tile leader publishes the tile's base rows
    # 4096 tokens x h7168 bf16: two 7-chunk slabs would fill the GPU (2048 blocks): seven
    # 2-chunk slabs, 7168 blocks, every block sums
    (4096, 14336, 8): (2, 1, 7, 16, 7168, 1, 1),
    # the fill point of 7-chunk slabs (1792 blocks, 7 per CU): 3072 tokens keep them (1536 blocks,
    # leaders publish), 3584 take 2-chunk slabs
    (3072, 14336, 8): (7, 1, 2, 16, 1536, 1, 2),
    (3584, 14336, 8): (2, 1, 7, 16, 6272, 1, 1),
    # ... up to 16384 one-token 2-chunk blocks (146 tiles x 112); 147 tiles keep 7-chunk slabs
    (9344, 14336, 8): (2, 1, 7, 16, 16352, 1, 1),
    (9408, 14336, 8): (7, 1, 2, 16, 4704, 1, 2),
    # h4096 (8 chunks) at 8192 tokens: 2048 8-chunk blocks fill the GPU: 2-chunk slabs
    (8192, 8192, 8): (2, 1, 4, 16, 8192, 1, 1),
    # ... while a block would sum at most 8192 published words (tiles x worldSize rounded up):
    # 129 tiles at 64 PEs keep one 8-chunk slab, tile leaders publish
    (8256, 8192, 64): (8, 1, 1, 16, 2064, 1, 2),
    # fp8 rows (7 chunks): one 7-chunk slab, 1024 blocks, every block sums
    (4096, 7168, 8): (7, 1, 1, 16, 1024, 1, 1),
    # ... at 8192 tokens 7-chunk slabs would pass 1024 blocks: two 4-chunk slabs (4 + 3), every block sums
    (8192, 7168, 8): (4, 1, 2, 16, 4096, 0, 1),
    # fp4x2 rows (3.5 KiB): one bound-checked 4-chunk slab, every block sums
    (4096, 3584, 8): (4, 1, 1, 16, 1024, 0, 1),
    # h2048 bf16: one 4-chunk slab, every block sums
    (4096, 4096, 8): (4, 1, 1, 16, 1024, 1, 1),
    # fp32 rows (28 chunks): fourteen 2-chunk slabs, 14336 blocks, every block sums; at 1536
    # tokens 7-chunk slabs (1536 blocks) stay
    (4096, 28672, 8): (2, 1, 14, 16, 14336, 1, 1),
    (1536, 28672, 8): (7, 1, 4, 16, 1536, 1, 2),
    # 16384 tokens: 8192 blocks, leaders publish
    (16384, 14336, 8): (7, 1, 2, 16, 8192, 1, 2),
    # one tile: 2-chunk slabs (at most 4 tiles), local scan
    (1, 14336, 8): (2, 1, 7, 16, 112, 1, 0),
    (8, 14336, 8): (2, 1, 7, 16, 112, 1, 0),
    # two tiles of odd-chunk fp8 rows: 1-chunk slabs, local scan
    (128, 7168, 8): (1, 1, 7, 16, 224, 1, 0),
    # 8 tiles: 7-chunk slabs, still the local scan; 9 tiles: every block sums
    (512, 14336, 8): (7, 1, 2, 16, 256, 1, 0),
    (576, 14336, 8): (7, 1, 2, 16, 288, 1, 1),
    # around the every-block limit of 7-chunk slabs (1024 blocks)
    (2047, 14336, 8): (7, 1, 2, 16, 1024, 1, 1),
    (2049, 14336, 8): (7, 1, 2, 16, 1056, 1, 2),
    (5121, 14336, 8): (2, 1, 7, 16, 9072, 1, 1),
    # slabs of at most 4 chunks sum in every block at any size while a block sums at most
    # 8192 published words (tiles x worldSize rounded up to a power of two)
    (16384, 3584, 8): (4, 1, 1, 16, 4096, 0, 1),
    (65536, 2048, 8): (2, 1, 1, 16, 16384, 1, 1),
    (8192, 4096, 64): (4, 1, 1, 16, 2048, 1, 1),
    (8256, 4096, 64): (4, 1, 1, 16, 2064, 1, 2),
    (12000, 4096, 40): (4, 1, 1, 16, 3008, 1, 2),
    # 528-byte rows: more than 16384 / 32768 one-token waves take 2 / 4 tokens per wave
    (66000, 528, 8): (1, 2, 1, 8, 8256, 0, 2),
    (132000, 528, 8): (1, 4, 1, 4, 8252, 0, 2),
    # 8-chunk slabs; rows past 8 chunks that are not whole: 8-chunk slabs with bound checks
    (1000, 8192, 8): (8, 1, 1, 16, 256, 1, 1),
    (1000, 9728, 8): (8, 1, 2, 16, 512, 0, 1),
    # no tokens: nothing but recvCount
    (0, 14336, 8): (0, 0, 0, 0, 0, 0, 0),
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
    """Plans of the given shapes: (T, rowBytes, W) for the dispatch, (rows, rowBytes) else."""
    args = [str(v) for shape in table for v in shape]
    r = subprocess.run([exe, kind, *args], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    n = 3 if kind == "dispatch" else 2
    got = {}
    for line in r.stdout.split("\n"):
        if line.strip():
            v = [int(x) for x in line.split()]
            got[tuple(v[:n])] = tuple(v[n:])
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
    """(numTokens, dispatch row bytes, worldSize) of the dispatches the GPU parity tests run."""
    import workloads
    import test_gpu_parity as P
    import test_gpu_random_shapes as R
    wb = workloads.WIRE_BYTES
    shapes = set()
    for name, _ in P.CONFIG_SEEDS:
        w = workloads.CONFIGS[name]
        shapes.add((w.numTokens, w.dispatchHidden * wb[w.wire], w.worldSize))
    for _name, W, _Epr, _M, T, _K, H, _routing, _useW in P.EDGE:
        shapes.add((T, H * 2, W))
    for name, base, wire, comb in P.DTYPES:
        if base is None:
            w = workloads.Workload(name, 5, 3, 700, 650, 7, 1056, "uniform", 1, wire=wire, combineDtype=comb)
        else:
            w = workloads.CONFIGS[base].with_(wire=wire, combineDtype=comb)
        rb = w.dispatchHidden * wb[wire] + (56 * 4 if name == "fp8_rows_with_block_scales" else 0)
        shapes.add((w.numTokens, rb, w.worldSize))
    for _id, name, over in P.GRAPH_CASES:
        w = workloads.CONFIGS[name].with_(**(over or {}))
        shapes.add((w.numTokens, w.dispatchHidden * wb[w.wire], w.worldSize))
    for _i, W, _Epr, _M, T, _K, H, dt, _useW, _routing in R.CASES:
        shapes.add((T, H * wb[dt], W))
    return sorted(shapes)


def _launchable_variants():
    """(cpw, ntw, full, scan) of every dispatch kernel the launcher can run
    (dispatch.hip, launch_fused): one token per wave with any SCAN form; two
    or four tokens per wave only with the tile leaders publishing
    (plan_dispatch gives them only to launches of over 8192 blocks, which
    never scan locally or in every block)."""
    out = set()
    for c in (1, 2, 4, 7, 8):
        for f in (0, 1):
            out |= {(c, 1, f, 0), (c, 1, f, 1), (c, 1, f, 2), (c, 2, f, 2), (c, 4, f, 2)}
    return out


def test_gpu_parity_reaches_every_dispatch_variant(tmp_path):
    """The GPU parity cases reach all 50 compiled dispatch kernels (slab width x
    tokens per wave x bound checks x SCAN form); no plan asks for a kernel
    that is not compiled."""
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
    variants = {(cpw, ntw, full, scan) for cpw, ntw, _nSlabs, _nSubs, _nBlocks, full, scan in got.values()}
    compiled = _launchable_variants()
    assert len(compiled) == 50
    assert variants <= compiled, sorted(variants - compiled)
    assert compiled == variants, sorted(compiled - variants)


def test_random_plans_only_ask_for_compiled_kernels(tmp_path):
    """Over a sweep of token counts (1..300000), row sizes (16 B..64 KiB) and
    world sizes (1..64), every plan names a compiled kernel."""
    import sys
    sys.path.insert(0, ROOT)
    from combine_count_amd import _build as B
    exe = str(tmp_path / "launch_plan_check")
    r = subprocess.run([B.HIPCC, *B.COMMON, os.path.join(ROOT, "tests", "host", "launch_plan_check.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(3))
    shapes = {(int(t), 16 * int(c), int(w)) for t, c, w in zip(rng.integers(1, 300001, 3000),
                                                              rng.integers(1, 4097, 3000), rng.integers(1, 65, 3000))}
    shapes |= {(t, rb, w) for t in (1, 64, 512, 513, 4096, 16384, 65536, 131072, 131073)
               for rb in (16, 1024, 3584, 7168, 14336, 28672, 65536) for w in (1, 8, 64)}
    got = _run(exe, "dispatch", sorted(shapes))
    compiled = _launchable_variants()
    for (T, rb, W), (cpw, ntw, _s, _u, nB, full, scan) in got.items():
        assert (cpw, ntw, full, scan) in compiled, (T, rb, W)
