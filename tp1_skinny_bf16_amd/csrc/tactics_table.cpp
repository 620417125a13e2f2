// tactics_table.cpp -- tactics measured on MI355X, per (N, K, batch bin).
//
// Each row was chosen by timing every candidate tactic on rotated weight
// copies (so no weight bytes come from the caches) and keeping the median
// fastest; ties within 1% go to fewer launches, then the smaller split.
// Rows: {N, K, bin, {kernel, bcap, split, rows, waves, wpc}}.
#include "tactics_table.hpp"

namespace tp1 {

namespace {
struct Entry {
    int N, K, bin;
    proj_tactic_t t;
};

// Measured on one MI355X (256 CUs), rotated weight copies, median of 20-30
// calls per candidate; each comment gives the chosen tactic's time and
// achieved bandwidth (weight + x + y bytes).
const Entry kTable[] = {
    {7168, 12288, 1, {PROJ_KERNEL_STREAM_DOT2, 1, 1, 4, 4, 8}},  // 32.38 us, 5441.6 GB/s
    {7168, 12288, 2, {PROJ_KERNEL_STREAM_DOT2, 2, 1, 4, 4, 8}},  // 33.71 us, 5228.1 GB/s
    {7168, 12288, 4, {PROJ_KERNEL_STREAM_DOT2, 4, 1, 2, 8, 8}},  // 35.26 us, 5000.5 GB/s
    {7168, 12288, 8, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 1, 0}},  // 36.56 us, 4826.9 GB/s
    {7168, 12288, 16, {PROJ_KERNEL_MFMA_LDS, 16, 1, 2, 4, 4}},  // 39.32 us, 4496.0 GB/s
    {7168, 12288, 32, {PROJ_KERNEL_MFMA_LDS, 32, 2, 2, 2, 0}},  // 52.37 us, 3387.5 GB/s
    {7168, 12288, 64, {PROJ_KERNEL_MFMA, 64, 4, 4, 2, 2}},  // 63.93 us, 2794.5 GB/s
    {14560, 7168, 1, {PROJ_KERNEL_STREAM_DOT2, 1, 1, 4, 2, 8}},  // 36.48 us, 5723.0 GB/s
    {14560, 7168, 2, {PROJ_KERNEL_STREAM_DOT2, 2, 1, 4, 4, 8}},  // 37.92 us, 5506.8 GB/s
    {14560, 7168, 4, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 1, 4}},  // 36.62 us, 5704.7 GB/s
    {14560, 7168, 8, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 1, 4}},  // 38.12 us, 5484.8 GB/s
    {14560, 7168, 16, {PROJ_KERNEL_MFMA_LDS, 16, 1, 2, 1, 0}},  // 41.02 us, 5105.5 GB/s
    {14560, 7168, 32, {PROJ_KERNEL_MFMA_LDS, 32, 1, 2, 1, 0}},  // 53.87 us, 3900.6 GB/s
    {14560, 7168, 64, {PROJ_KERNEL_MFMA, 64, 2, 4, 2, 2}},  // 72.29 us, 2925.9 GB/s
    {14560, 7168, 128, {PROJ_KERNEL_MFMA, 128, 2, 4, 1, 2}},  // 126.62 us, 1692.4 GB/s
    {14560, 7168, 256, {PROJ_KERNEL_MFMA, 256, 1, 1, 4, 4}},  // 451.22 us, 487.2 GB/s
    {49376, 7168, 1, {PROJ_KERNEL_STREAM_DOT2, 1, 1, 2, 4, 16}},  // 108.33 us, 6535.3 GB/s
    {49376, 7168, 2, {PROJ_KERNEL_STREAM_DOT2, 2, 1, 2, 8, 16}},  // 109.71 us, 6454.1 GB/s
    {49376, 7168, 4, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 4, 4}},  // 113.23 us, 6255.5 GB/s
    {49376, 7168, 8, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 4, 4}},  // 119.21 us, 5945.5 GB/s
    {49376, 7168, 16, {PROJ_KERNEL_MFMA_LDS, 16, 1, 2, 2, 2}},  // 125.83 us, 5639.9 GB/s
    {49376, 7168, 32, {PROJ_KERNEL_MFMA, 32, 1, 4, 1, 4}},  // 171.28 us, 4153.9 GB/s
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
