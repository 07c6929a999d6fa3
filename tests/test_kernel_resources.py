"""Build guard on the gfx950 code itself (CPU: hipcc cross-compiles with the
library's own flags): no kernel spills to scratch, the variants the default
workloads run keep the occupancy they were tuned at, payload rows move as
16-byte non-temporal accesses (the dispatch's stores also device-scope), and
no packed-fp32 instruction is emitted."""
import os
import re
import subprocess

import pytest

from combine_count_amd import _build as B

SOURCES = ["dispatch.hip", "combine.hip", "combine_push.hip"]


def _compile(src, tmpdir):
    asm = os.path.join(tmpdir, src + ".s")
    cmd = [B.HIPCC, *B.DEVICE, *B.COMMON, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", asm,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    res, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = res.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return res, open(asm).read()


@pytest.fixture(scope="module")
def compiled(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("isa"))
    return {src: _compile(src, d) for src in SOURCES}


def _kernel(res, pattern):
    hits = [k for k in res if re.search(pattern, k)]
    assert len(hits) == 1, (pattern, hits)
    return res[hits[0]]


def test_no_scratch_and_no_spills(compiled):
    for src, (res, _) in compiled.items():
        assert res, f"{src}: no resource remarks parsed"
        for name, r in res.items():
            assert r.get("ScratchSize", 0) == 0, (src, name, r)
            # (SGPR spills go to VGPR lanes, not memory: allowed)
            assert r.get("VGPRs Spill", 0) == 0, (src, name, r)


def test_default_variants_keep_their_occupancy(compiled):
    d, c, p = compiled["dispatch.hip"][0], compiled["combine.hip"][0], compiled["combine_push.hip"][0]
    # 4096 tokens x h7168 bf16: dispatch 7-chunk slabs, 1 token per wave, no bound checks,
    # tile leaders publishing (last argument 2); the same slabs where every block sums (1: fp8
    # rows at 4096 tokens) and for launches of at most 8 tiles (0: local scan)
    assert _kernel(d, r"dispatch_kernelILi7ELi1ELb1ELi2EE")["Occupancy"] >= 7
    assert _kernel(d, r"dispatch_kernelILi7ELi1ELb1ELi1EE")["Occupancy"] >= 7
    assert _kernel(d, r"dispatch_kernelILi7ELi1ELb1ELi0EE")["Occupancy"] >= 7
    # 4-chunk slabs where every block sums (h2048; fp4x2 rows bound-checked)
    assert _kernel(d, r"dispatch_kernelILi4ELi1ELb1ELi1EE")["Occupancy"] >= 7
    assert _kernel(d, r"dispatch_kernelILi4ELi1ELb0ELi1EE")["Occupancy"] >= 7
    # launches of at most 4 tiles: 2- (or 1-) chunk slabs under the local scan
    assert _kernel(d, r"dispatch_kernelILi2ELi1ELb1ELi0EE")["Occupancy"] == 8
    assert _kernel(d, r"dispatch_kernelILi1ELi1ELb1ELi0EE")["Occupancy"] == 8
    # gather combine, 2-chunk slabs, bf16 rows and output (up to 8 rows in flight), its
    # landing-row twin, and bf16 rows into an fp32 output
    assert _kernel(c, r"combine_kernelILi2ELb1ELb0ELb0ELb0EE")["Occupancy"] >= 4
    assert _kernel(c, r"combine_kernelILi2ELb1ELb0ELb0ELb1EE")["Occupancy"] >= 4
    assert _kernel(c, r"combine_kernelILi2ELb1ELb0ELb1ELb0EE")["Occupancy"] >= 4
    # 1-chunk slabs (fewer than 8192 two-chunk waves): 7, with the first group's rows in flight
    # while the weights' scales are summed (faster than 8 without that overlap: PR-scale, EpCfg defaults)
    assert _kernel(c, r"combine_kernelILi1ELb1ELb0ELb0ELb0EE")["Occupancy"] >= 7
    assert _kernel(p, r"push_kernelILi7ELb1EE")["Occupancy"] == 8
    for src, (res, _) in compiled.items():
        for name, r in res.items():
            if "Occupancy" in r and "kernel" in name:
                assert r["Occupancy"] >= 3, (src, name, r)


def test_rows_move_as_16_byte_non_temporal_accesses(compiled):
    d, c, p = (compiled[s][1] for s in SOURCES)
    assert re.search(r"buffer_store_dwordx4 .* nt sc1", d), "dispatch row stores (non-temporal, device scope)"
    assert re.search(r"global_load_dwordx4 .* nt", c) and re.search(r"global_store_dwordx4 .* nt", c), "combine"
    assert re.search(r"global_load_dwordx4 .* nt", p) and re.search(r"global_store_dwordx4 .* nt", p), "push"


def test_no_packed_fp32_instructions(compiled):
    for src, (_, asm) in compiled.items():
        assert not re.search(r"\bv_pk_(fma|mul|add)_f32\b", asm), src
