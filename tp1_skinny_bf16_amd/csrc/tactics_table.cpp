// tactics_table.cpp -- tactics measured on MI355X, per (N, K, batch bin).
//
// Each row was chosen by timing every candidate tactic on rotated weight
// copies (so no weight bytes come from the caches) and keeping the median
// fastest; ties within 1% go to fewer launches, then the smaller split.
// Rows: {N, K, bin, {kernel, bcap, split, rows, waves, wpc, kc}}.
#include "tactics_table.hpp"

namespace tp1 {

namespace {
struct Entry {
    int N, K, bin;
    proj_tactic_t t;
};

// Measured on one MI355X (256 CUs), rotated weight copies, median of 20
// calls per candidate; each comment gives the chosen tactic's time and
// achieved bandwidth (weight + x + y bytes).
const Entry kTable[] = {
    {7168, 12288, 1, {PROJ_KERNEL_STREAM_DOT2, 1, 1, 4, 4, 8, 0}},  // 32.4 us, 5438.3 GB/s
    {7168, 12288, 2, {PROJ_KERNEL_STREAM_DOT2, 2, 1, 4, 4, 8, 0}},  // 33.86 us, 5204.9 GB/s
    {7168, 12288, 4, {PROJ_KERNEL_STREAM_DOT2, 4, 1, 2, 8, 8, 0}},  // 35.54 us, 4961.1 GB/s
    {7168, 12288, 8, {PROJ_KERNEL_MFMA_XS, 16, 4, 4, 1, 2, 128}},  // 35.34 us, 4993.6 GB/s
    {7168, 12288, 16, {PROJ_KERNEL_MFMA_XS, 16, 4, 4, 1, 2, 128}},  // 35.8 us, 4938.1 GB/s
    {7168, 12288, 32, {PROJ_KERNEL_MFMA_XS, 32, 4, 4, 2, 2, 128}},  // 37.02 us, 4792.2 GB/s
    {7168, 12288, 64, {PROJ_KERNEL_MFMA_XS, 64, 4, 4, 4, 2, 128}},  // 43.05 us, 4149.9 GB/s
    {7168, 12288, 128, {PROJ_KERNEL_MFMA_XS, 128, 4, 4, 4, 2, 128}},  // 59.77 us, 3030.6 GB/s
    {7168, 12288, 256, {PROJ_KERNEL_MFMA_XS, 256, 2, 4, 4, 1, 128}},  // 122.82 us, 1515.4 GB/s
    {14560, 7168, 1, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 1, 4, 0}},  // 36.16 us, 5773.7 GB/s
    {14560, 7168, 2, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 1, 4, 0}},  // 36.24 us, 5762.1 GB/s
    {14560, 7168, 4, {PROJ_KERNEL_MFMA_LDS, 16, 1, 1, 1, 4, 0}},  // 36.64 us, 5701.6 GB/s
    {14560, 7168, 8, {PROJ_KERNEL_MFMA_XS, 16, 4, 8, 1, 2, 128}},  // 37.64 us, 5554.7 GB/s
    {14560, 7168, 16, {PROJ_KERNEL_MFMA_XS, 16, 4, 8, 1, 2, 128}},  // 38.0 us, 5511.2 GB/s
    {14560, 7168, 32, {PROJ_KERNEL_MFMA_XS, 32, 4, 8, 2, 2, 128}},  // 40.26 us, 5219.1 GB/s
    {14560, 7168, 64, {PROJ_KERNEL_MFMA_XS, 64, 4, 8, 2, 2, 128}},  // 46.31 us, 4567.3 GB/s
    {14560, 7168, 128, {PROJ_KERNEL_MFMA_XS, 128, 2, 4, 4, 2, 128}},  // 67.31 us, 3183.7 GB/s
    {14560, 7168, 256, {PROJ_KERNEL_MFMA_XS, 256, 1, 4, 4, 1, 128}},  // 143.62 us, 1530.8 GB/s
    {49376, 7168, 1, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128}},  // 104.25 us, 6791.1 GB/s
    {49376, 7168, 2, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128}},  // 103.27 us, 6856.6 GB/s
    {49376, 7168, 4, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128}},  // 103.67 us, 6832.3 GB/s
    {49376, 7168, 8, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128}},  // 103.63 us, 6839.3 GB/s
    {49376, 7168, 16, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128}},  // 103.61 us, 6849.4 GB/s
    {49376, 7168, 32, {PROJ_KERNEL_MFMA_XS, 32, 1, 8, 2, 2, 128}},  // 106.85 us, 6658.6 GB/s
    {49376, 7168, 64, {PROJ_KERNEL_MFMA_XS, 64, 1, 8, 2, 2, 128}},  // 117.87 us, 6066.8 GB/s
    {49376, 7168, 128, {PROJ_KERNEL_MFMA_XS, 128, 3, 4, 2, 2, 128}},  // 221.85 us, 3255.9 GB/s
    {49376, 7168, 256, {PROJ_KERNEL_MFMA_XS, 256, 2, 4, 4, 1, 128}},  // 490.0 us, 1503.7 GB/s
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
