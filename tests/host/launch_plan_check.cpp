// Prints the launch plans of csrc/epdc_internal.h (host code the launchers
// run) for shapes given on the command line:
//   dispatch T rowBytes W ...  -> T rowBytes W cpw ntw nSlabs nSubs nBlocks full scan
//                                 (scan: 0 local, 1 every block sums, 2 the tile leaders publish)
//   combine  T rowBytes ...    -> T rowBytes cpw nSlabs waves nBlocks full
//   push     L rowBytes ...    -> L rowBytes cpw nSlabs waves nBlocks full   (L = landing rows)
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../combine_count_amd/csrc/epdc_internal.h"

int main(int argc, char **argv) {
    if (argc < 2) return 2;
    const char *kind = argv[1];
    const bool dispatch = !std::strcmp(kind, "dispatch");
    const int step = dispatch ? 3 : 2;
    for (int i = 2; i + step - 1 < argc; i += step) {
        const int n = std::atoi(argv[i]), rowBytes = std::atoi(argv[i + 1]);
        if (dispatch) {
            const int W = std::atoi(argv[i + 2]);
            const epdc::DispatchPlan p = epdc::plan_dispatch(n, rowBytes, W);
            std::printf("%d %d %d %d %d %d %d %lld %d %d\n", n, rowBytes, W, p.cpw, p.ntw, p.nSlabs, p.nSubs,
                        (long long)p.nBlocks, (int)p.full, (int)p.scan);
        } else {
            const epdc::RowPlan p =
                !std::strcmp(kind, "combine") ? epdc::plan_combine(n, rowBytes) : epdc::plan_push(n, rowBytes);
            std::printf("%d %d %d %d %lld %lld %d\n", n, rowBytes, p.cpw, p.nSlabs, (long long)p.waves,
                        (long long)p.nBlocks, (int)p.full);
        }
    }
    return 0;
}
