// Checks xcd_run_block (xcd.h) on the host: for every run length the kernels
// may use and every grid size up to 4100 blocks (plus some large ones), each
// logical block is taken exactly once, and inside every full span of 8 runs
// hardware block b (on XCD b % 8) lands in run b % 8 of that span, so the
// blocks one XCD takes from a span are kRun consecutive logical blocks.
#include <cstdio>
#include <vector>

#include "xcd.h"

template <int L>
static bool check(int nb) {
    constexpr int run = 1 << L, span = moedx::kXcds * run;
    std::vector<int> seen(nb, 0);
    for (int b = 0; b < nb; ++b) {
        const int l = moedx::xcd_run_block<L>(b, nb);
        if (l < 0 || l >= nb || seen[l]++) {
            std::printf("FAIL run=%d nb=%d b=%d -> %d\n", run, nb, b, l);
            return false;
        }
        const int base = b / span * span;
        if (base + span <= nb) {  // a full span: the run of XCD b % 8
            const int want_lo = base + (b % moedx::kXcds) * run;
            if (l < want_lo || l >= want_lo + run) {
                std::printf("FAIL run=%d nb=%d b=%d -> %d outside [%d, %d)\n", run, nb, b, l,
                            want_lo, want_lo + run);
                return false;
            }
        } else if (l != b) {  // the last, partial span keeps the identity
            std::printf("FAIL run=%d nb=%d b=%d -> %d in the partial span\n", run, nb, b, l);
            return false;
        }
    }
    return true;
}

int main() {
    std::vector<int> sizes;
    for (int nb = 1; nb <= 4100; ++nb) sizes.push_back(nb);
    for (int nb : {14336, 14337, 32768, 32769, 65535, 1 << 20}) sizes.push_back(nb);
    long long n = 0;
    for (int nb : sizes) {
        if (!check<0>(nb) || !check<1>(nb) || !check<2>(nb) || !check<3>(nb) || !check<4>(nb) ||
            !check<5>(nb))
            return 1;
        n += 6;
    }
    std::printf("ok %lld\n", n);
    return 0;
}
