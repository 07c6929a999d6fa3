// Prints epdc::plan_dispatch (the dispatch's launch geometry, host code in
// csrc/epdc_internal.h) for each "numTokens rowBytes" pair on the command
// line, one line each:
//   T rowBytes cpw ntw nSlabs nSubs nBlocks full local selfScan xEarly
#include <cstdio>
#include <cstdlib>

#include "../../combine_count_amd/csrc/epdc_internal.h"

int main(int argc, char **argv) {
    for (int i = 1; i + 1 < argc; i += 2) {
        const int T = std::atoi(argv[i]), rowBytes = std::atoi(argv[i + 1]);
        const epdc::DispatchPlan p = epdc::plan_dispatch(T, rowBytes);
        std::printf("%d %d %d %d %d %d %lld %d %d %d %d\n", T, rowBytes, p.cpw, p.ntw, p.nSlabs, p.nSubs,
                    (long long)p.nBlocks, (int)p.full, (int)p.local, (int)p.selfScan, (int)p.xEarly);
    }
    return 0;
}
