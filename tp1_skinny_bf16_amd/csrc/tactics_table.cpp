// tactics_table.cpp -- tactics measured on MI355X, per (N, K, batch bin).
//
// Each row was chosen by timing every candidate tactic on rotated weight
// copies (so no weight bytes come from the caches) and keeping the median
// fastest; ties within 1% go to fewer launches, then the smaller split.
// Rows: {N, K, bin, {kernel, bcap, split, rows, waves, wpc, kc, depth}}.
#include "tactics_table.hpp"

namespace tp1 {

namespace {
struct Entry {
    int N, K, bin;
    proj_tactic_t t;
};

// Measured on one MI355X (256 CUs), rotated weight copies, median of 40
// calls per candidate; each comment gives the chosen tactic's time and
// achieved bandwidth (weight + x + y bytes).
const Entry kTable[] = {
    {7168, 12288, 1, {PROJ_KERNEL_STREAM_DOT2, 1, 1, 4, 4, 8, 0, 0}},  // 32.24 us, 5465.3 GB/s
    {7168, 12288, 2, {PROJ_KERNEL_STREAM_DOT2, 2, 1, 4, 4, 8, 0, 0}},  // 33.64 us, 5239.0 GB/s
    {7168, 12288, 4, {PROJ_KERNEL_MFMA_XS, 16, 4, 4, 1, 2, 128, 2}},  // 34.62 us, 5092.9 GB/s
    {7168, 12288, 8, {PROJ_KERNEL_MFMA_XS, 16, 4, 4, 1, 2, 128, 2}},  // 34.44 us, 5124.0 GB/s
    {7168, 12288, 16, {PROJ_KERNEL_MFMA_XS, 16, 4, 4, 1, 2, 128, 2}},  // 34.86 us, 5071.2 GB/s
    {7168, 12288, 32, {PROJ_KERNEL_MFMA_XS, 32, 4, 4, 2, 2, 128, 1}},  // 37.16 us, 4774.1 GB/s
    {7168, 12288, 64, {PROJ_KERNEL_MFMA_XS, 64, 4, 4, 2, 2, 128, 1}},  // 42.97 us, 4157.6 GB/s
    {7168, 12288, 128, {PROJ_KERNEL_MFMA_XS, 128, 4, 4, 2, 2, 128, 1}},  // 58.85 us, 3078.0 GB/s
    {7168, 12288, 256, {PROJ_KERNEL_MFMA_XS, 256, 2, 4, 4, 1, 128, 1}},  // 120.33 us, 1546.8 GB/s
    {14560, 7168, 1, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 1, 4, 0, 0}},  // 36.04 us, 5792.9 GB/s
    {14560, 7168, 2, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 1, 4, 0, 0}},  // 36.18 us, 5771.7 GB/s
    {14560, 7168, 4, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 1, 4, 0, 0}},  // 36.44 us, 5732.9 GB/s
    {14560, 7168, 8, {PROJ_KERNEL_MFMA_XS, 16, 4, 8, 1, 2, 128, 1}},  // 37.61 us, 5559.2 GB/s
    {14560, 7168, 16, {PROJ_KERNEL_MFMA_XS, 16, 4, 8, 1, 2, 128, 1}},  // 37.96 us, 5517.1 GB/s
    {14560, 7168, 32, {PROJ_KERNEL_MFMA_XS, 32, 4, 8, 2, 2, 128, 1}},  // 40.29 us, 5215.3 GB/s
    {14560, 7168, 64, {PROJ_KERNEL_MFMA_XS, 64, 4, 8, 2, 2, 128, 1}},  // 46.08 us, 4590.1 GB/s
    {14560, 7168, 128, {PROJ_KERNEL_MFMA_XS, 128, 2, 4, 4, 2, 128, 1}},  // 65.71 us, 3261.2 GB/s
    {14560, 7168, 256, {PROJ_KERNEL_MFMA_XS, 256, 1, 4, 4, 1, 128, 1}},  // 139.78 us, 1572.9 GB/s
    {49376, 7168, 1, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1}},  // 103.23 us, 6858.2 GB/s
    {49376, 7168, 2, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1}},  // 103.57 us, 6836.7 GB/s
    {49376, 7168, 4, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1}},  // 103.63 us, 6835.0 GB/s
    {49376, 7168, 8, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1}},  // 103.75 us, 6831.4 GB/s
    {49376, 7168, 16, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1}},  // 104.23 us, 6808.6 GB/s
    {49376, 7168, 32, {PROJ_KERNEL_MFMA_XS, 32, 1, 8, 2, 2, 128, 1}},  // 107.73 us, 6604.2 GB/s
    {49376, 7168, 64, {PROJ_KERNEL_MFMA_XS, 64, 1, 8, 2, 2, 128, 1}},  // 124.7 us, 5734.5 GB/s
    {49376, 7168, 128, {PROJ_KERNEL_MFMA_XS, 128, 1, 4, 4, 2, 128, 1}},  // 228.31 us, 3163.8 GB/s
    {49376, 7168, 256, {PROJ_KERNEL_MFMA_XS, 256, 2, 4, 4, 1, 128, 1}},  // 476.92 us, 1544.9 GB/s
};
}  // namespace

bool lookup_measured_tactic(int N, int K, int bin, proj_tactic_t *out) {
    for (const Entry &e : kTable) {
        if (e.N == N && e.K == K && e.bin == bin && e.t.kernel != 0) {
            *out = e.t;
            return true;
        }
    }
    return false;
}

}  // namespace tp1
