// Workgroup order across the eight XCDs of an MI355X.
//
// The dispatcher hands the workgroups of a launch to the XCDs in turn:
// workgroup b runs on XCD b % 8, and each XCD has an L2 of its own.  A kernel
// whose work items read metadata shared by neighbouring items (the rows of a
// token in the combine: its slot buckets, gate weights and group masks) can
// take its logical block from xcd_run_block, so that one XCD runs kRun
// consecutive logical blocks and those lines are fetched into one L2 instead
// of several.
//
// Blocks come in spans of 8 * kRun: hardware block base + 8 j + x (x = XCD,
// 0 <= j < kRun) becomes logical block base + kRun x + j.  Within a span this
// is a bijection, so every logical block of [0, nb) is taken exactly once; a
// last span that does not fill 8 * kRun blocks keeps the identity.
#pragma once

#if defined(__HIPCC__)
#define MOEDX_XCD_HD __host__ __device__
#else
#define MOEDX_XCD_HD
#endif

namespace moedx {

constexpr int kXcds = 8;

// kRunLog2: log2 of the run length; b in [0, nb).
template <int kRunLog2>
MOEDX_XCD_HD inline int xcd_run_block(int b, int nb) {
    constexpr int span = kXcds << kRunLog2;
    const int base = b & ~(span - 1);
    if (base + span > nb) return b;
    const int o = b - base;
    return base + ((o & (kXcds - 1)) << kRunLog2) + (o >> 3);
}

}  // namespace moedx
