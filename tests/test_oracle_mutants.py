"""Plant plausible mistakes into copies of the oracle, on the CPU, and check
that the pins catch every one of them.

Each mutant is a text substitution applied to oracle/epdc_oracle.c; the
mutated source is compiled into a temporary library and run through the pin
checks of oracle_pins.py (cheapest first) until one fails.  No mutant may
index outside its buffers, so none of them touches the id-range guard.
"""
import os

import pytest

import oracle
import oracle_pins as pins

MUTANTS = [
    # (name, text in the oracle, replacement)
    ("dedup keeps the last slot",
     "for (int32_t j = 0; keep && j < k; ++j)",
     "for (int32_t j = k + 1; keep && j < K; ++j)"),
    ("no dedup",
     "== p) keep = 0;",
     "== p) keep = 1;"),
    ("PE by modulo instead of division",
     "return e / Epr;",
     "return e % W;"),
    ("row index from the token instead of the counter",
     "int32_t r = recvCount[p]++;",
     "int32_t r = (recvCount[p]++, t % M);"),
    ("flat index stride worldSize",
     "sendMap[(int64_t)t * K + k] = (int32_t)row;",
     "sendMap[(int64_t)t * K + k] = (int32_t)(r * W + p);"),
    ("null entry 0 instead of -1",
     "sendMap[(int64_t)t * K + k] = -1; /* the null entry */",
     "sendMap[(int64_t)t * K + k] = 0;"),
    ("metadata: slot stored as token index",
     "recvTokIdx[row] = t;",
     "recvTokIdx[row] = k;"),
    ("expert ids copied from the mirrored token",
     "memcpy(recvExpertIds + row * K, expertIds + (int64_t)t * K,",
     "memcpy(recvExpertIds + row * K, expertIds + (int64_t)(T - 1 - t) * K,"),
    ("weights copied from the mirrored token",
     "memcpy(recvWeights + row * K, weights + (int64_t)t * K,",
     "memcpy(recvWeights + row * K, weights + (int64_t)(T - 1 - t) * K,"),
    ("combine: scale from the kept slot only",
     "for (int32_t k = k0; k < K; ++k)",
     "for (int32_t k = k0; k < k0 + 1; ++k)"),
    ("combine: scale misses the kept slot",
     "for (int32_t k = k0; k < K; ++k)",
     "for (int32_t k = k0 + 1; k < K; ++k)"),
    ("combine: weight subtracted",
     "s = s + weights[(int64_t)t * K + k];",
     "s = s - weights[(int64_t)t * K + k];"),
    ("combine: weights read with the slot index reversed",
     "s = s + weights[(int64_t)t * K + k];",
     "s = s + weights[(int64_t)t * K + (K - 1 - k)];"),
    ("combine: returned row read with swapped stride",
     "const int64_t row = (int64_t)p * M + r;",
     "const int64_t row = (int64_t)r * W + p;"),
    ("dispatch: row copied as bf16 whatever the element size",
     "const int64_t rowBytes = (int64_t)H * elemBytes;",
     "const int64_t rowBytes = (int64_t)H * 2 + 0 * elemBytes;"),
    ("combine fp32: separate multiply and add",
     "for (int32_t h = 0; h < H; ++h) acc[h] = fmaf(s, src[h], acc[h]);",
     "for (int32_t h = 0; h < H; ++h) acc[h] = s * src[h] + acc[h];"),
    ("combine fp32: output rounded to bf16 precision",
     "memcpy(outRow, acc, (size_t)H * sizeof(float));",
     "for (int32_t h = 0; h < H; ++h) ((float *)outRow)[h] = bf16_to_f32(f32_to_bf16_rne(acc[h]));"),
    ("combine: separate multiply and add",
     "acc[h] = fmaf(s, bf16_to_f32(src[h]), acc[h]);",
     "acc[h] = s * bf16_to_f32(src[h]) + acc[h];"),
    ("combine: PEs in reverse slot order",
     "    for (int32_t k0 = 0; k0 < K; ++k0) {\n        int32_t flat",
     "    for (int32_t k0 = K - 1; k0 >= 0; --k0) {\n        int32_t flat"),
    ("combine: accumulator not cleared per token",
     "for (int32_t h = 0; h < H; ++h) acc[h] = 0.0f;",
     ";"),
    ("push: rows of a window land in reverse order",
     "const int64_t L = landOff + r;",
     "const int64_t L = landOff + (n - 1 - r);"),
    ("push: landing offset not advanced past a window",
     "landOff += n;",
     "landOff += 0 * n;"),
    ("push: scale over every valid slot, not only the PE's",
     "if (dest_pe(recvExpertIds[src * K + k], W, Epr) == p)",
     "if (dest_pe(recvExpertIds[src * K + k], W, Epr) >= 0)"),
    ("push: scale from the first slot on the PE only",
     "s = s + recvWeights[src * K + k];",
     "{ s = s + recvWeights[src * K + k]; break; }"),
    ("reduce: forwarded scale ignored",
     "float s = useWeights ? landScale[L] : 1.0f;",
     "float s = useWeights ? 1.0f : 1.0f;"),
    ("reduce: slots in reverse order",
     "        for (int32_t k0 = 0; k0 < K; ++k0) {\n            int32_t flat",
     "        for (int32_t k0 = K - 1; k0 >= 0; --k0) {\n            int32_t flat"),
    ("reduce: landing row from the window row only",
     "int64_t L = landOff[p] + r;",
     "int64_t L = r;"),
    ("reduce: accumulator not cleared per token",
     "memset(acc, 0, (size_t)H * sizeof(float)); /* +0.0f */",
     ";"),
    ("scales copied from the mirrored token",
     "memcpy(recvScales + row * S, scales + (int64_t)t * S,",
     "memcpy(recvScales + row * S, scales + (int64_t)(T - 1 - t) * S,"),
    ("scales not forwarded",
     "if (S > 0)\n                memcpy(recvScales",
     "if (S > (1 << 30))\n                memcpy(recvScales"),
    ("scale row stored at the token's index instead of its row",
     "memcpy(recvScales + row * S,",
     "memcpy(recvScales + ((int64_t)p * M + t % M) * S,"),
    ("combine: output type taken from the rows when they are bf16",
     "    store_row(outRow, acc, H, outFp32);",
     "    store_row(outRow, acc, H, outFp32 & inFp32);"),
    ("reduce: output type taken from the landing rows when they are bf16",
     "store_row((unsigned char *)out + (int64_t)i * outRowBytes, acc, H, outFp32);",
     "store_row((unsigned char *)out + (int64_t)i * outRowBytes, acc, H, outFp32 & inFp32);"),
    ("bf16 rounding by truncation",
     "u += 0x7fffu + lsb;",
     "u += 0u * lsb;"),
    ("bf16 rounding ties away from zero",
     "u += 0x7fffu + lsb;",
     "u += 0x8000u + 0u * lsb;"),
]

# cheapest checks first
ORDER = [
    pins.check_worked_example,
    pins.check_reading_fma_fp32,
    pins.check_combine_fp32,
    pins.check_brute_force_random,
    pins.check_push_landing_brute,
    pins.check_push_capacity,
    pins.check_reading_fma_and_order,
    pins.check_combine_identity_cases,
    pins.check_push_reduce_matches_gather,
    pins.check_combine_fp64_bound,
    pins.check_brute_force_exhaustive,
    pins.check_invariants,
    pins.check_closed_form_unique_pairs,
    pins.check_page_null_entries,
    pins.check_page_staging_bytes,
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for '{name}' not unique in the oracle"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(str(mpath), str(tmp_path / "libmutant.so")))
    for check in ORDER:
        try:
            fails = check(lib)
        except Exception as e:  # a mutant that breaks a check's own preconditions is caught too
            fails = [f"{check.__name__} raised {e!r}"]
        if fails:
            return
    pytest.fail(f"no pin catches the mutant '{name}'")
