"""HIP library vs the CPU oracle, through the C ABI, on an MI355X.

Dispatch must match bit for bit on every output buffer (windows pre-filled
with sentinels, so untouched rows are checked too); combine must match bit
for bit (both sides accumulate in the same order with one fused multiply-add
per PE).  Inputs are the seeded synthetic workloads of workloads.py at their
full sizes, plus edge shapes: empty and ragged inputs, widths that are not a
multiple of 512, non-power-of-two worldSize / numExpertPerRank, tokens with
more than 8 destinations, the 64-PE / 64-slot maxima and invalid expert ids.
"""
import dataclasses

import numpy as np
import pytest
import torch

import combine_count_amd as epdc
import workloads
from gpu_harness import DeviceRun, assert_bits_equal, assert_dispatch_equal, oracle_combine, oracle_dispatch, out_as

pytestmark = pytest.mark.gpu

CONFIG_SEEDS = [
    ("tiny", 1), ("tiny", 2), ("tiny", 3),
    ("pr_scale", 1), ("pr_scale", 2), ("pr_scale", 3),
    ("epcfg_defaults", 1), ("epcfg_defaults", 2), ("epcfg_defaults", 3),
    ("gen_zipf_h2048", 1), ("gen_zipf_h2048", 2),
    ("gen_zipf_h7168", 1),
    ("gen_edge_t1", 1), ("gen_edge_t1", 2), ("gen_edge_t1", 3),
    ("gen_edge_t8", 1), ("gen_edge_t8", 2), ("gen_edge_t8", 3),
    ("large_unweighted", 1),
    ("large_weighted", 1),
]


def _check_case(w: workloads.Workload, inp: workloads.Inputs, tag: str):
    print(f"[parity] {tag}: {w}", flush=True)
    g = DeviceRun(w, inp)
    g.dispatch()
    torch.cuda.synchronize()
    o = oracle_dispatch(w, inp)
    assert_dispatch_equal(g, o, tag)
    assert g.scratch_clean(), f"{tag}: dispatch left its scratch non-zero (or a wait timed out)"
    if w.numTokens == 0:
        return
    # combine over independent returned rows y
    g.combine()
    torch.cuda.synchronize()
    exp = oracle_combine(w, inp.y, inp, o.sendMap)
    assert_bits_equal(out_as(g), exp, f"{tag} combine")
    # identity expert: the returned rows are the dispatched rows
    if w.wire == w.combineDtype:
        g.combine(y=g.recvX)
        torch.cuda.synchronize()
        exp = oracle_combine(w, o.recvX, inp, o.sendMap)
        assert_bits_equal(out_as(g), exp, f"{tag} identity combine")


@pytest.mark.parametrize("name,seed", CONFIG_SEEDS, ids=[f"{n}-s{s}" for n, s in CONFIG_SEEDS])
def test_config_parity(name, seed):
    w = workloads.CONFIGS[name]
    _check_case(w, workloads.cached_inputs(name, seed), f"{name} seed {seed}")


EDGE = [
    # name, worldSize, numExpertPerRank, maxTokPerRank, numTokens, topk, hiddenDim, routing, useWeights
    ("empty", 4, 4, 64, 0, 2, 128, "uniform", 1),
    ("ragged_w3_epr5_h136", 3, 5, 128, 100, 4, 136, "uniform", 1),
    ("ragged_w5_epr3_h1032", 5, 3, 1024, 1000, 7, 1032, "uniform", 1),
    ("more_than_8_dest", 16, 2, 320, 300, 12, 512, "uniform", 1),
    ("more_than_8_dest_unweighted", 16, 2, 320, 257, 12, 1024, "zipf", 0),
    ("max_w64_k64", 64, 1, 80, 70, 64, 64, "uniform", 1),
    ("single_pe", 1, 8, 96, 65, 3, 8, "uniform", 1),
    ("topk1", 8, 4, 200, 129, 1, 2048, "uniform", 1),
    ("m_gt_t", 8, 32, 4096, 777, 8, 7168, "zipf", 1),
    ("one_token_full_row", 8, 32, 64, 1, 8, 7168, "uniform", 0),
    # geometry paths: 8-chunk slabs (1 and 2 per row); 625 tiles; 2 and 4 tokens per
    # wave (11 KiB rows: eleven 1-chunk slabs, so 94 / 188 tiles pass 16384 / 32768 blocks)
    ("slab8_h4096", 8, 32, 1000, 1000, 8, 4096, "zipf", 1),
    ("slab8_h8192_two_slabs", 4, 16, 300, 300, 6, 8192, "uniform", 1),
    ("t9000_ragged", 8, 32, 9000, 9000, 8, 7168, "uniform", 1),
    ("t40000_h512", 8, 32, 40000, 40000, 8, 512, "uniform", 0),
    ("two_tokens_per_wave_t6000", 2, 4, 6000, 6000, 4, 5632, "uniform", 1),
    ("four_tokens_per_wave_t12000", 2, 4, 12000, 11990, 3, 5632, "zipf", 0),
    # 8 tiles (local-scan range) but 131 one-chunk slabs per row: two tokens per wave, so the
    # scan goes through the scratch
    ("two_tokens_per_wave_8_tiles_h67072", 2, 4, 512, 512, 4, 67072, "uniform", 1),
    ("slab2_h1024", 8, 32, 700, 700, 8, 1024, "zipf", 0),
    # combine in 2-chunk slabs with bound checks (5.5 KiB rows, 4000 tokens x 3 slabs)
    ("combine_slab2_ragged_t4000", 4, 8, 4000, 4000, 6, 2816, "zipf", 1),
    # at the edge of the local scan (8 tiles) and just past it (9 tiles)
    ("local_scan_8_tiles", 8, 8, 512, 512, 8, 2048, "uniform", 1),
    ("scratch_scan_9_tiles", 8, 8, 600, 520, 8, 2048, "zipf", 1),
    # the two SCAN forms around their switch at 1024 blocks (h7168: 32 blocks per tile):
    # 32 tiles, every block sums the counts itself; 33 tiles, the tile leader publishes
    # base rows (both with a ragged last tile); and 63 self-summing tiles of 256-byte rows
    ("self_scan_1024_blocks_t2047", 8, 32, 2048, 2047, 8, 7168, "zipf", 1),
    ("leader_scan_1056_blocks_t2049", 8, 32, 2049, 2049, 8, 7168, "zipf", 1),
    ("self_scan_63_tiles_h128", 4, 8, 4100, 4000, 4, 128, "uniform", 1),
    # around the point where wide slabs fill the GPU (1792 blocks of 7 or 8 chunks): 48 tiles
    # of h7168 keep two 7-chunk slabs (1536 blocks, the tile leaders publish); 57 tiles (a
    # last tile of one token) take seven 2-chunk slabs (6384 blocks, every block sums); 94
    # tiles of h4096 keep one 8-chunk slab (1504 blocks, leaders publish)
    ("wide7_leader_1536_blocks_t3072", 8, 32, 3072, 3072, 8, 7168, "zipf", 1),
    ("slab2_self_6384_blocks_t3585", 8, 32, 3585, 3585, 8, 7168, "zipf", 1),
    ("wide8_leader_1504_blocks_t6000_h4096", 2, 4, 6000, 6000, 3, 4096, "uniform", 1),
    # self-summing with x requested between COUNT and the SCAN's wait (slabs of at most 4
    # chunks), ragged 3.5 KiB rows
    ("self_scan_ragged_h1792", 4, 8, 1000, 1000, 5, 1792, "uniform", 1),
    # the token-count x topk grid of mori PR #599's checks, at 8 PEs / 256 experts / h7168
    # (uniform routing; the Zipf workloads cover the skewed case)
    ("pr_grid_ct512_topk6", 8, 32, 512, 512, 6, 7168, "uniform", 1),
    ("pr_grid_ct512_topk8", 8, 32, 512, 512, 8, 7168, "uniform", 1),
    ("pr_grid_ct1024_topk6", 8, 32, 1024, 1024, 6, 7168, "uniform", 1),
    ("pr_grid_ct1024_topk8", 8, 32, 1024, 1024, 8, 7168, "uniform", 1),
    ("pr_grid_ct2048_topk6", 8, 32, 2048, 2048, 6, 7168, "uniform", 1),
    ("pr_grid_ct2048_topk8", 8, 32, 2048, 2048, 8, 7168, "uniform", 1),
    ("pr_grid_ct4096_topk6", 8, 32, 4096, 4096, 6, 7168, "uniform", 1),
    ("pr_grid_ct4096_topk8", 8, 32, 4096, 4096, 8, 7168, "uniform", 1),
    # 32 KiB rows (four 8-chunk slabs per row)
    ("h16384_rows", 8, 16, 600, 600, 8, 16384, "zipf", 1),
    # rows that are not a whole number of 1 KiB chunks, one per tail-checked slab width
    ("ragged_rows_1p5k", 4, 8, 300, 257, 5, 768, "uniform", 1),
    ("ragged_rows_5p5k", 8, 16, 300, 300, 8, 2816, "zipf", 1),
    ("ragged_rows_9p5k", 8, 16, 200, 130, 8, 4864, "uniform", 0),
    ("ragged_rows_9p5k_5_tiles", 8, 16, 320, 300, 8, 4864, "uniform", 1),  # 8-chunk slabs, local scan
    # ragged rows (5.5 KiB, 7-chunk slabs) in a launch of 3264 blocks, tile leaders publish
    ("ragged_rows_leader_t13000", 8, 16, 13000, 13000, 8, 2816, "uniform", 1),
    # further compiled dispatch variants (slab chunks, tokens per wave, bound checks, scan):
    ("ragged_ntw2_t66000_h264", 2, 4, 66000, 66000, 2, 264, "uniform", 1),       # 1, 2, checked
    ("ragged_ntw4_t132000_h264", 2, 4, 132000, 132000, 2, 264, "zipf", 0),       # 1, 4, checked
    ("ntw2_cpw2_t13200_h5120", 2, 4, 13200, 13200, 3, 5120, "uniform", 1),       # 2, 2
    ("ntw2_cpw4_t22000_h6144", 2, 4, 22000, 22000, 3, 6144, "uniform", 1),       # 4, 2
    ("ntw2_cpw7_t11000_h21504", 2, 4, 11000, 11000, 2, 21504, "uniform", 1),     # 7, 2
    ("ntw2_cpw8_t8300_h32768", 2, 4, 8300, 8300, 2, 32768, "zipf", 1),           # 8, 2
    ("local_ragged_cpw4_t300_h1792", 4, 8, 300, 300, 5, 1792, "uniform", 1),     # 4, 1, checked, local
    ("ragged_scan_t1000_h264", 4, 8, 1000, 1000, 5, 264, "uniform", 1),          # 1, 1, checked, scratch
    ("ragged_ntw2_cpw2_t66000_h768", 2, 4, 66000, 66000, 2, 768, "uniform", 1),  # 2, 2, checked
    ("ragged_ntw4_cpw2_t132000_h768", 2, 4, 132000, 132000, 2, 768, "zipf", 1),  # 2, 4, checked
    ("ragged_ntw2_cpw4_t66000_h1792", 2, 4, 66000, 66000, 2, 1792, "uniform", 0),  # 4, 2, checked
    ("ragged_ntw4_cpw4_t132000_h1792", 2, 4, 132000, 132000, 2, 1792, "uniform", 1),  # 4, 4, checked
    ("ragged_ntw2_cpw7_t66000_h2816", 2, 4, 66000, 66000, 2, 2816, "zipf", 1),   # 7, 2, checked
    ("ragged_ntw2_cpw8_t33000_h4864", 2, 4, 33000, 33000, 2, 4864, "uniform", 1),  # 8, 2, checked
    ("ntw4_cpw2_t26300_h5120", 2, 4, 26300, 26300, 2, 5120, "uniform", 1),       # 2, 4
    # one token per wave, slabs of at most 4 chunks, over 2560 blocks: every block sums
    ("self_cpw4_t10300_h2048", 2, 4, 10300, 10300, 3, 2048, "uniform", 1),        # 4, full
    ("self_cpw4_ragged_t10300_h1792", 2, 4, 10300, 10300, 3, 1792, "zipf", 1),    # 4, checked
    ("self_cpw2_t3400_h3072", 2, 4, 3400, 3400, 3, 3072, "uniform", 1),           # 2, full, 3 slabs
    ("self_cpw2_ragged_t10300_h768", 2, 4, 10300, 10300, 3, 768, "uniform", 0),   # 2, checked
    ("self_cpw1_ragged_t10300_h264", 2, 4, 10300, 10300, 2, 264, "uniform", 1),   # 1, checked
    # x between COUNT and the SCAN's wait with 1-chunk slabs (3 KiB rows: three slabs per row)
    ("self_cpw1_t1000_h1536", 4, 8, 1000, 1000, 5, 1536, "zipf", 1),
    # slabs of at most 4 chunks where a block would sum over 8192 published words (64 PEs,
    # over 128 tiles): the tile leaders publish (2064 and 2576 blocks)
    ("w64_leader_cpw1_ragged_t8256_h264", 64, 2, 8256, 8256, 2, 264, "uniform", 1),
    ("w64_leader_cpw1_t8256_h512", 64, 2, 8256, 8256, 2, 512, "uniform", 0),
    ("w64_leader_cpw2_ragged_t8256_h768", 64, 2, 8256, 8256, 2, 768, "uniform", 1),
    ("w64_leader_cpw2_t8256_h1024", 64, 2, 8256, 8256, 2, 1024, "zipf", 1),
    ("w64_leader_cpw4_ragged_t8256_h1792", 64, 2, 8256, 8256, 2, 1792, "uniform", 0),
    ("w64_leader_cpw4_t8256_h2048", 64, 2, 8256, 8256, 2, 2048, "uniform", 1),
    ("w64_leader_cpw1_ragged_t10300_h264", 64, 2, 10300, 10300, 2, 264, "zipf", 1),
    ("w64_leader_cpw1_t10300_h512", 64, 2, 10300, 10300, 2, 512, "uniform", 1),
    ("w64_leader_cpw2_ragged_t10300_h768", 64, 2, 10300, 10300, 2, 768, "uniform", 0),
    ("w64_leader_cpw2_t10300_h1024", 64, 2, 10300, 10300, 2, 1024, "uniform", 1),
    ("w64_leader_cpw4_ragged_t10300_h1792", 64, 2, 10300, 10300, 2, 1792, "zipf", 1),
    ("w64_leader_cpw4_t10300_h2048", 64, 2, 10300, 10300, 2, 2048, "uniform", 1),
    ("ntw4_cpw4_t43700_h6144", 2, 4, 43700, 43700, 2, 6144, "uniform", 1),       # 4, 4
    # one token per wave, 1504 blocks of slabs of 1, 2 and 4 chunks (every block sums)
    ("self_1504_blocks_cpw1_t6000_h512", 2, 4, 6000, 6000, 3, 512, "uniform", 1),          # 1, 1
    ("self_1504_blocks_cpw1_ragged_t6000_h264", 2, 4, 6000, 6000, 3, 264, "zipf", 1),      # 1, 1, checked
    ("self_1504_blocks_cpw2_t6000_h1024", 2, 4, 6000, 6000, 3, 1024, "uniform", 0),        # 2, 1
    ("self_1504_blocks_cpw2_ragged_t6000_h768", 2, 4, 6000, 6000, 3, 768, "uniform", 1),   # 2, 1, checked
    ("self_1504_blocks_cpw4_t6000_h2048", 2, 4, 6000, 6000, 3, 2048, "zipf", 1),           # 4, 1
    ("self_1504_blocks_cpw4_ragged_t6000_h1792", 2, 4, 6000, 6000, 3, 1792, "uniform", 1),  # 4, 1, checked
    # rows of 8 chunks at 12000 tokens (3008 8-chunk blocks would fill the GPU: 2-chunk slabs,
    # every block sums), and 8-chunk bound-checked slabs with the tile leaders publishing
    ("slab2_self_t12000_h4096", 2, 4, 12000, 12000, 3, 4096, "uniform", 1),    # 8, 1
    ("leader_cpw8_ragged_t6000_h4864", 2, 4, 6000, 6000, 3, 4864, "zipf", 1),   # 8, 1, checked
    # four tokens per wave with 7- and 8-chunk slabs (over 32768 one-token waves)
    ("ntw4_4plus3_t132000_h3584", 2, 4, 132000, 132000, 2, 3584, "uniform", 1),  # 4, 4, checked (7 = 4 + 3)
    ("ntw4_cpw7_w1_t65601_h7168", 1, 4, 65601, 65601, 2, 7168, "uniform", 1),    # 7, 4
    ("ntw4_cpw7_ragged_t132000_h3328", 2, 4, 132000, 132000, 2, 3328, "zipf", 0),  # 7, 4, checked
    ("ntw4_cpw8_t132000_h4096", 2, 4, 132000, 132000, 2, 4096, "uniform", 1),    # 8, 4
    ("ntw4_cpw8_ragged_t66000_h4864", 2, 4, 66000, 66000, 2, 4864, "uniform", 1),  # 8, 4, checked
]


@pytest.mark.parametrize("case", EDGE, ids=[e[0] for e in EDGE])
def test_edge_parity(case):
    name, W, Epr, M, T, K, H, routing, useW = case
    w = workloads.Workload(name, W, Epr, M, T, K, H, routing, useW)
    _check_case(w, workloads.make_inputs(w, 5), name)


DTYPES = [
    # name, base workload, wire (dispatch row type), combine row type
    ("fp8_wire_bf16_combine_h7168", "gen_zipf_h7168", "fp8", "bf16"),
    ("fp4x2_wire_bf16_combine_h7168", "gen_zipf_h7168", "fp4x2", "bf16"),
    ("fp32_both_pr_scale", "pr_scale", "fp32", "fp32"),
    ("fp32_both_h7168", "gen_zipf_h7168", "fp32", "fp32"),  # 14336 2-chunk dispatch blocks, every block sums
    ("bf16_wire_fp32_combine_defaults", "epcfg_defaults", "bf16", "fp32"),
    ("fp8_wire_fp32_combine_tiny", "tiny", "fp8", "fp32"),
    ("fp4x2_wire_ragged", None, "fp4x2", "bf16"),
    ("fp32_both_ragged", None, "fp32", "fp32"),
    ("fp8_wire_large", "large_weighted", "fp8", "bf16"),
    # fp8 rows carrying their scales: 7168 e4m3 values + 56 fp32 block scales = 7392 bytes
    ("fp8_rows_with_block_scales", "gen_zipf_h7168", "fp8", "bf16"),
]


@pytest.mark.parametrize("case", DTYPES, ids=[d[0] for d in DTYPES])
def test_dtype_parity(case):
    """Dispatch of every wire type is a bitwise row copy; combine reduces bf16
    or fp32 rows (a narrow-wire pair is two calls with two cfgs)."""
    name, base, wire, comb = case
    if base is None:  # ragged: rows that are not a whole number of 1 KiB chunks, non-pow2 W/Epr
        w = workloads.Workload(name, 5, 3, 700, 650, 7, 1056, "uniform", 1, wire=wire, combineDtype=comb)
    else:
        w = workloads.CONFIGS[base].with_(name=name, wire=wire, combineDtype=comb)
    inp = workloads.make_inputs(w, 4)
    if name == "fp8_rows_with_block_scales":
        # the dispatch side only: rows are the fp8 payload with its scales appended
        rng = np.random.Generator(np.random.PCG64(17))
        scales = rng.uniform(0.01, 2.0, size=(w.numTokens, 56)).astype(np.float32)
        x = np.concatenate([inp.x, scales.view(np.uint8)], axis=1)
        w = w.with_(hiddenDim=x.shape[1])
        inp = dataclasses.replace(inp, w=w, x=x)
        g = DeviceRun(w, inp)
        g.dispatch()
        torch.cuda.synchronize()
        o = oracle_dispatch(w, inp)
        assert_dispatch_equal(g, o, name)
        got = g.recvX.cpu().numpy()[..., 7168:].copy().view(np.float32)
        for p_ in range(w.worldSize):
            c = int(o.recvCount[p_])
            tok = o.recvTokIdx[p_, :c]
            assert np.array_equal(got[p_, :c], scales[tok]), "forwarded scales differ"
        return
    _check_case(w, inp, name)


SCALES = [
    # name, base workload (None: ragged rows, 5 PEs, 3 experts each, topk 7), wire, scaleDim.
    # The scale rows travel as the fourth metadata field of every received row (MORI JIT v2
    # §4/§5: the dispatch's scales and the out_scales region; mori PR #599's merge notes).
    ("fp8_scales56_h7168", "gen_zipf_h7168", "fp8", 56),  # one scale per 128 values; 4 + 3-chunk slabs, x mid
    ("fp4x2_scales1_h7168", "gen_zipf_h7168", "fp4x2", 1),  # one per token; self-summing, x mid
    ("bf16_scales56_leader_scan", "wide7_leader_1536_blocks_t3072", "bf16", 56),  # tile leaders publish
    ("fp32_scales8_slab2_self", "gen_zipf_h7168", "fp32", 8),  # 14336 2-chunk blocks, every block sums
    ("bf16_scales64_defaults", "epcfg_defaults", "bf16", 64),  # local scan, exactly one wave of scales
    ("fp8_scales65_pr_scale", "pr_scale", "fp8", 65),  # one past a wave: the scale-tail loop
    ("fp8_scales1024_tiny", "tiny", "fp8", 1024),  # the maximum scaleDim
    ("fp8_scales130_ragged", None, "fp8", 130),  # three waves of scales, bound-checked rows
    ("fp8_scales56_edge_t1", "gen_edge_t1", "fp8", 56),
    ("fp8_scales56_large", "large_weighted", "fp8", 56),
    ("bf16_scales3_more_than_8_dest", "more_than_8_dest", "bf16", 3),
    ("bf16_scales5_empty", "empty", "bf16", 5),
]


def _edge_workload(name):
    for e in EDGE:
        if e[0] == name:
            return workloads.Workload(*e)
    raise KeyError(name)


@pytest.mark.parametrize("case", SCALES, ids=[c[0] for c in SCALES])
def test_scale_forwarding(case):
    """Per-token scales are copied bitwise beside every row of their token:
    recvScales whole-buffer equal to the oracle's (sentinels past the counts
    untouched), through every SCAN form."""
    name, base, wire, S = case
    if base is None:
        w = workloads.Workload(name, 5, 3, 700, 650, 7, 1056, "uniform", 1)
    elif base in workloads.CONFIGS:
        w = workloads.CONFIGS[base]
    else:
        w = _edge_workload(base)
    w = w.with_(name=name, wire=wire, combineDtype="bf16", scaleDim=S)
    _check_case(w, workloads.make_inputs(w, 4), name)


OUT_TYPES = [
    # name, base workload (None: ragged), row (combine input) type, output type.  MORI JIT v2
    # §5: the combine outputs bf16 or fp32, chosen apart from the type of the rows it sums.
    ("bf16_rows_fp32_out_tiny", "tiny", "bf16", "fp32"),
    ("bf16_rows_fp32_out_pr_scale", "pr_scale", "bf16", "fp32"),
    ("bf16_rows_fp32_out_defaults", "epcfg_defaults", "bf16", "fp32"),
    ("bf16_rows_fp32_out_h2048", "gen_zipf_h2048", "bf16", "fp32"),
    ("bf16_rows_fp32_out_h7168", "gen_zipf_h7168", "bf16", "fp32"),
    ("bf16_rows_fp32_out_edge_t8", "gen_edge_t8", "bf16", "fp32"),
    ("bf16_rows_fp32_out_large_unweighted", "large_unweighted", "bf16", "fp32"),
    ("bf16_rows_fp32_out_ragged", None, "bf16", "fp32"),
    # H 1408: 2816-byte rows, the last chunk filling its lower half and a quarter of the upper one
    # (a lane's two 8-byte pieces sit in different halves of the chunk, each checked apart)
    ("bf16_rows_fp32_out_ragged_upper_half", "ragged:1408", "bf16", "fp32"),
    ("fp32_rows_bf16_out_defaults", "epcfg_defaults", "fp32", "bf16"),
    ("fp32_rows_bf16_out_h7168", "gen_zipf_h7168", "fp32", "bf16"),
    ("fp32_rows_bf16_out_ragged", None, "fp32", "bf16"),
]


@pytest.mark.parametrize("case", OUT_TYPES, ids=[c[0] for c in OUT_TYPES])
def test_combine_output_types(case):
    """Either row type into either output type, bit for bit (a bf16 output
    is the fp32 accumulator rounded to nearest even, an fp32 output the
    accumulator itself)."""
    name, base, rows, out = case
    if base is None or base.startswith("ragged:"):
        H = 1056 if base is None else int(base.split(":")[1])
        w = workloads.Workload(name, 5, 3, 700, 650, 7, H, "uniform", 1)
    else:
        w = workloads.CONFIGS[base]
    w = w.with_(name=name, wire=rows, combineDtype=rows, outDtype=out)
    _check_case(w, workloads.make_inputs(w, 2), name)


INVALID = [
    # name, W, Epr, K: power-of-two and other experts per rank; topk above 8 (the ids past
    # slot 8 are read one by one)
    ("pow2_epr", 8, 4, 6),
    ("epr5_w6", 6, 5, 6),
    ("epr3_k10", 5, 3, 10),
]


@pytest.mark.parametrize("case", INVALID, ids=[c[0] for c in INVALID])
def test_invalid_expert_ids(case):
    """Ids outside [0, E) are dropped slots: null entry, no row, no weight."""
    name, W, Epr, K = case
    w = workloads.Workload(f"invalid_ids_{name}", W, Epr, 256, 250, K, 1024, "uniform", 1)
    inp = workloads.make_inputs(w, 9)
    rng = np.random.Generator(np.random.PCG64(99))
    ids = inp.expertIds.copy()
    E = w.numExperts
    mask = rng.random(ids.shape) < 0.25
    bad = rng.choice(np.array([-1, -2, E, E + 5, 2**31 - 1, -(2**31)], dtype=np.int64), size=ids.shape)
    ids[mask] = bad[mask].astype(np.int32)
    ids[3, :] = -1  # a token with no valid slot combines to +0
    inp = dataclasses.replace(inp, expertIds=ids)
    _check_case(w, inp, w.name)


DEGENERATE = ["all_to_one_pe", "all_slots_invalid", "all_to_every_pe", "half_tokens_invalid"]


@pytest.mark.parametrize("kind", DEGENERATE)
def test_degenerate_routings(kind):
    """Routings at the edges: every token to PE 3 only (one window full, the
    others empty); every slot invalid (no rows, all nulls, +0 combine);
    every token to all 8 PEs (U = 8T, the window maximum per PE); every
    other token with no valid slot."""
    W, Epr, K, T = 8, 4, 6, 700
    w = workloads.Workload(f"degenerate_{kind}", W, Epr, T, T, K, 1536, "uniform", 1)
    inp = workloads.make_inputs(w, 13)
    rng = np.random.Generator(np.random.PCG64(77))
    if kind == "all_to_one_pe":
        ids = (3 * Epr + rng.integers(0, Epr, size=(T, K))).astype(np.int32)
    elif kind == "all_slots_invalid":
        ids = np.full((T, K), -1, np.int32)
    elif kind == "all_to_every_pe":
        w = w.with_(numExpertPerToken=8)
        inp = workloads.make_inputs(w, 13)
        ids = np.stack([rng.permutation(W) * Epr + rng.integers(0, Epr, W) for _ in range(T)]).astype(np.int32)
    else:
        ids = inp.expertIds.copy()
        ids[::2] = W * Epr + 1
    inp = dataclasses.replace(inp, expertIds=ids)
    _check_case(w, inp, kind)


def test_dirty_scratch_is_flagged_and_stays_in_bounds():
    """A scratch the caller did not zero (its published words hold garbage,
    the header is zero) makes the base rows wrong -- summed garbage can wrap
    to negative rows.  The dispatch must then skip every row outside
    [0, maxTokPerRank), set the scratch error word, and write nothing outside
    its windows: guard rows on both sides of recvX and recvTokIdx stay as
    they were.  (Outputs are invalid in this case; only safety is checked.)"""
    W, Epr, M, T, K, H = 4, 8, 1024, 1024, 6, 1024  # 16 tiles: scanned through the scratch
    w = workloads.Workload("dirty_scratch", W, Epr, M, T, K, H, "uniform", 1)
    inp = workloads.make_inputs(w, 21)
    g = DeviceRun(w, inp)
    guard, rowB = 16, H * 2
    big_x = torch.full((W * M + 2 * guard, rowB), 0x5A, dtype=torch.uint8, device="cuda")
    big_t = torch.full((W * M + 2 * guard,), -424242, dtype=torch.int32, device="cuda")
    g.recvX = big_x[guard:guard + W * M].view(W, M, rowB)
    g.recvTokIdx = big_t[guard:guard + W * M].view(W, M)
    header_words = 4224 // 4
    g.scratch.zero_()
    g.scratch[header_words:] = 0x7FFFFFF0
    torch.cuda.synchronize()
    g.dispatch()
    torch.cuda.synchronize()
    bx, bt = big_x.cpu().numpy(), big_t.cpu().numpy()
    assert (bx[:guard] == 0x5A).all() and (bx[guard + W * M:] == 0x5A).all(), "recvX guard rows written"
    assert (bt[:guard] == -424242).all() and (bt[guard + W * M:] == -424242).all(), "recvTokIdx guard written"
    # Whether a block reads garbage before the real value is published is a
    # race; every garbage base here puts some row outside [0, M) (0x7FFFFFEF
    # per count, so any sum is huge or negative), so wrong outputs are flagged.
    o = oracle_dispatch(w, inp)
    same = (np.array_equal(g.sendMap.cpu().numpy(), o.sendMap)
            and np.array_equal(g.recvCount.cpu().numpy(), o.recvCount))
    assert same or int(g.scratch[2].item()) != 0, "wrong outputs from a dirty scratch were not flagged"


GRAPH_CASES = [
    # id, workload, overrides
    ("epcfg_defaults", "epcfg_defaults", None),  # 2 tiles: 2-chunk slabs, local scan
    ("pr_scale", "pr_scale", None),  # 8 tiles: local scan, scratch untouched
    # 16 tiles, 256 blocks: every block sums the published counts, x mid (4-chunk slabs)
    ("h2048_t1024_self_scan", "gen_zipf_h2048", dict(numTokens=1024, maxTokPerRank=1024)),
    # 1536 blocks of 7-chunk slabs: the tile leaders publish base rows
    ("h7168_t3072_leader_scan", "gen_zipf_h7168", dict(numTokens=3072)),
    # 7168 and 14336 blocks of 2-chunk slabs (bf16 and fp32 rows): every block sums
    ("h7168_t4096_slab2_self", "gen_zipf_h7168", None),
    ("h7168_fp32_slab2_self", "gen_zipf_h7168", dict(wire="fp32", combineDtype="fp32")),
]


@pytest.mark.parametrize("case_id,name,over", GRAPH_CASES, ids=[c[0] for c in GRAPH_CASES])
def test_deterministic_and_graph_replay(case_id, name, over):
    """Two eager runs are bitwise equal; a captured dispatch+combine graph
    replayed several times (eager work and syncs in between) equals eager,
    and the scratch is zero after every replay."""
    w = workloads.CONFIGS[name]
    if over:
        w = w.with_(**over)
        inp = workloads.make_inputs(w, 1)
    else:
        inp = workloads.cached_inputs(name, 1)
    g = DeviceRun(w, inp)
    g.dispatch()
    g.combine()
    torch.cuda.synchronize()
    ref = {k: getattr(g, k).clone() for k in ("recvX", "recvTokIdx", "recvExpertIds", "recvWeights",
                                              "recvCount", "sendMap", "out")}
    g.dispatch()
    g.combine()
    torch.cuda.synchronize()
    for k, v in ref.items():
        assert torch.equal(getattr(g, k).view(torch.int16) if v.dtype == torch.bfloat16 else getattr(g, k),
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v), f"rerun differs: {k}"
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.dispatch(stream=s)  # warm-up on the capture stream
        g.combine(stream=s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        g.dispatch(stream=s)
        g.combine(stream=s)
    for rep in range(4):
        g.recvCount.fill_(-1)
        g.sendMap.fill_(-5)
        g.out.view(torch.int16).fill_(0x1234)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert g.scratch_clean(), f"graph replay {rep} left the dispatch scratch non-zero"
        for k, v in ref.items():
            a = getattr(g, k)
            if v.dtype == torch.bfloat16:
                a, v = a.view(torch.int16), v.view(torch.int16)
            assert torch.equal(a, v), f"graph replay {rep} differs from eager: {k}"


def test_library_is_in_tree():
    lib = epdc.load_library()
    assert lib._name.endswith("combine_count_amd/libepdc.so")
    assert torch.cuda.is_available()


def test_one_scratch_across_varying_token_counts():
    """A serving loop: one scratch buffer, dispatches of different token
    counts (local and scratch-scanned launches mixed, the large ones first)
    enqueued back to back with no sync in between; every call matches the
    oracle and the scratch ends all zero."""
    base = workloads.Workload("varying_T", 8, 32, 4096, 4096, 8, 1024, "zipf", 1)
    counts = [4096, 777, 65, 4096, 1, 2000, 512, 3000]
    runs = []
    shared = None
    for i, T in enumerate(counts):
        w = base.with_(name=f"varying_T{T}", numTokens=T)
        inp = workloads.make_inputs(w, 40 + i)
        g = DeviceRun(w, inp)
        if shared is None:
            shared = g.scratch
        g.scratch = shared
        runs.append((w, inp, g))
    torch.cuda.synchronize()
    for w, inp, g in runs:
        g.dispatch()
        g.combine()
    torch.cuda.synchronize()
    for w, inp, g in runs:
        tag = f"T={w.numTokens}"
        o = oracle_dispatch(w, inp)
        assert_dispatch_equal(g, o, tag)
        assert_bits_equal(out_as(g), oracle_combine(w, inp.y, inp, o.sendMap), f"{tag} combine")
    assert bool((shared == 0).all().item()), "the shared scratch is not all zero after the calls"
