// tactics_table.cpp -- tactics measured on MI355X, per (N, K, batch bin).
//
// Each row was chosen by timing every candidate tactic on rotated weight
// copies (so no weight bytes come from the caches) and keeping the median
// fastest; ties within 1% go to fewer launches, then the smaller split.
// Rows: {N, K, bin, {kernel, bcap, split, rows, waves, wpc, kc, depth, kw}}.
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
    {7168, 12288, 1, {PROJ_KERNEL_STREAM_DOT2, 1, 1, 4, 4, 8, 0, 0, 0}},  // 32.16 us, 5478.8 GB/s
    {7168, 12288, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 2, 128, 3, 1}},  // 32.8 us, 5373.1 GB/s
    {7168, 12288, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 2, 128, 3, 1}},  // 33.06 us, 5333.2 GB/s
    {7168, 12288, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 2, 128, 3, 1}},  // 33.22 us, 5312.2 GB/s
    {7168, 12288, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 2, 128, 3, 1}},  // 33.7 us, 5245.8 GB/s
    {7168, 12288, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 4, 8, 2, 1, 128, 3, 1}},  // 36.52 us, 4857.8 GB/s
    {7168, 12288, 64, {PROJ_KERNEL_MFMA_XS, 64, 4, 4, 4, 2, 128, 1, 0}},  // 43.07 us, 4147.9 GB/s
    {7168, 12288, 128, {PROJ_KERNEL_MFMA_XS, 128, 4, 4, 2, 2, 128, 1, 0}},  // 59.65 us, 3036.7 GB/s
    {7168, 12288, 256, {PROJ_KERNEL_MFMA_XS, 256, 2, 4, 4, 1, 128, 1, 0}},  // 120.14 us, 1549.2 GB/s
    {14560, 7168, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 3, 1}},  // 35.58 us, 5867.8 GB/s
    {14560, 7168, 2, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 1, 4, 0, 0, 0}},  // 36.14 us, 5778.1 GB/s
    {14560, 7168, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 3, 1}},  // 35.88 us, 5822.4 GB/s
    {14560, 7168, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 1}},  // 35.36 us, 5912.9 GB/s
    {14560, 7168, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 1}},  // 35.3 us, 5932.8 GB/s
    {14560, 7168, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 2, 8, 2, 1, 128, 3, 1}},  // 39.7 us, 5292.8 GB/s
    {14560, 7168, 64, {PROJ_KERNEL_MFMA_XS, 64, 4, 8, 2, 2, 128, 1, 0}},  // 46.11 us, 4587.1 GB/s
    {14560, 7168, 128, {PROJ_KERNEL_MFMA_XS, 128, 2, 4, 4, 2, 128, 1, 0}},  // 66.51 us, 3222.0 GB/s
    {14560, 7168, 256, {PROJ_KERNEL_MFMA_XS, 256, 1, 4, 4, 1, 128, 1, 0}},  // 140.3 us, 1567.0 GB/s
    {49376, 7168, 1, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0}},  // 103.83 us, 6818.5 GB/s
    {49376, 7168, 2, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0}},  // 103.25 us, 6857.9 GB/s
    {49376, 7168, 4, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0}},  // 103.77 us, 6825.7 GB/s
    {49376, 7168, 8, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0}},  // 104.07 us, 6810.4 GB/s
    {49376, 7168, 16, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0}},  // 104.11 us, 6816.5 GB/s
    {49376, 7168, 32, {PROJ_KERNEL_MFMA_XS, 32, 1, 8, 2, 2, 128, 1, 0}},  // 107.51 us, 6617.7 GB/s
    {49376, 7168, 64, {PROJ_KERNEL_MFMA_XS, 64, 1, 8, 2, 2, 128, 1, 0}},  // 126.35 us, 5659.6 GB/s
    {49376, 7168, 128, {PROJ_KERNEL_MFMA_XS, 128, 3, 4, 4, 2, 128, 1, 0}},  // 226.55 us, 3188.4 GB/s
    {49376, 7168, 256, {PROJ_KERNEL_MFMA_XS, 256, 2, 4, 4, 1, 128, 1, 0}},  // 477.6 us, 1542.7 GB/s
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
