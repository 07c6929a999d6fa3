// Checks epdc::div_magic (the dispatch's expert -> PE division) against the
// divide instruction on the host: every divisor 1..20000 and powers of two
// and their neighbours up to 2^31 - 1, at numerators around multiples of the
// divisor, at the ends of the 32-bit range and at pseudo-random points.
#include <cstdio>
#include <cstdint>

#include "../../combine_count_amd/csrc/epdc_internal.h"

static uint32_t quotient(uint32_t n, const epdc::DivMagic &m) {
    const uint32_t t = (uint32_t)(((uint64_t)n * m.magic) >> 32);
    return (t + ((n - t) >> m.sh1)) >> m.sh2;
}

static uint64_t bad = 0, checked = 0;

static void check(uint32_t d, uint32_t n, const epdc::DivMagic &m) {
    ++checked;
    if (quotient(n, m) != n / d) {
        if (bad < 10) std::printf("d=%u n=%u got %u want %u\n", d, n, quotient(n, m), n / d);
        ++bad;
    }
}

static void check_divisor(uint32_t d, uint64_t &rng) {
    const epdc::DivMagic m = epdc::div_magic(d);
    for (uint32_t n = 0; n < 256; ++n) check(d, n, m);
    for (uint64_t k = 1; k * d <= 0xffffffffull; k = k < 64 ? k + 1 : k * 3 + 1) {
        const uint64_t q = k * d;
        check(d, (uint32_t)(q - 1), m);
        check(d, (uint32_t)q, m);
        if (q + 1 <= 0xffffffffull) check(d, (uint32_t)(q + 1), m);
    }
    check(d, 0x7fffffffu, m);
    check(d, 0x80000000u, m);
    check(d, 0xffffffffu, m);
    for (int i = 0; i < 64; ++i) {
        rng = rng * 6364136223846793005ull + 1442695040888963407ull;
        check(d, (uint32_t)(rng >> 32), m);
    }
}

int main() {
    uint64_t rng = 1;
    for (uint32_t d = 1; d <= 20000; ++d) check_divisor(d, rng);
    for (int l = 14; l <= 31; ++l)
        for (int64_t off = -3; off <= 3; ++off) {
            const int64_t d = ((int64_t)1 << l) + off;
            if (d >= 1 && d <= 0x7fffffff) check_divisor((uint32_t)d, rng);
        }
    for (uint32_t d : {46341u, 65535u, 65537u, 1000003u, 123456789u, 2147483647u}) check_divisor(d, rng);
    std::printf("%llu checked, %llu wrong\n", (unsigned long long)checked, (unsigned long long)bad);
    return bad ? 1 : 0;
}
