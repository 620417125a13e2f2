// tactics_table.cpp -- tactics measured on MI355X, per (N, K, batch bin).
//
// Each row was chosen by timing every candidate tactic on rotated weight
// copies (so no weight bytes come from the caches), calls enqueued back to
// back, and keeping the fastest mean per call; ties within 1% go to fewer
// launches, then the smaller split.
// Rows: {N, K, bin, {kernel, bcap, split, rows, waves, wpc, kc, depth, kw, nw, stagger}}.
#include "tactics_table.hpp"

namespace tp1 {

namespace {
struct Entry {
    int N, K, bin;
    proj_tactic_t t;
};

// Measured on MI355X (256 CUs), rotated weight copies, mean of 40 calls
// back to back per candidate; per bin the fastest over three tuning runs on
// the current kernels (one of them without the staggered candidates).  Each
// comment gives the chosen tactic's time and achieved bandwidth (weight + x +
// y bytes).
const Entry kTable[] = {
    {7168, 12288, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 29.0 us, 6075.9 GB/s
    {7168, 12288, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 29.36 us, 6002.7 GB/s
    {7168, 12288, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 29.03 us, 6073.6 GB/s
    {7168, 12288, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 28.39 us, 6216.0 GB/s
    {7168, 12288, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 29.01 us, 6093.9 GB/s
    {7168, 12288, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 4, 8, 2, 1, 128, 3, 1, 8, 1}},  // 32.22 us, 5506.1 GB/s
    {7168, 12288, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 4, 8, 2, 1, 128, 3, 1, 8, 1}},  // 36.2 us, 4935.1 GB/s
    {7168, 12288, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 4, 8, 2, 1, 64, 4, 1, 8, 0}},  // 46.81 us, 3869.7 GB/s
    {7168, 12288, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 4, 8, 4, 1, 64, 3, 1, 8, 0}},  // 68.96 us, 2699.0 GB/s
    {14560, 7168, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4, 0}},  // 32.08 us, 6508.0 GB/s
    {14560, 7168, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4, 0}},  // 32.19 us, 6487.1 GB/s
    {14560, 7168, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4, 0}},  // 32.25 us, 6477.7 GB/s
    {14560, 7168, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4, 0}},  // 32.38 us, 6457.1 GB/s
    {14560, 7168, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4, 0}},  // 32.32 us, 6479.8 GB/s
    {14560, 7168, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 2, 8, 2, 1, 128, 3, 1, 8, 0}},  // 36.29 us, 5790.1 GB/s
    {14560, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 2, 8, 2, 1, 128, 3, 1, 8, 0}},  // 40.83 us, 5180.3 GB/s
    {14560, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 4, 16, 2, 1, 64, 3, 1, 8, 0}},  // 51.14 us, 4190.4 GB/s
    {14560, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 2, 8, 4, 1, 64, 3, 1, 8, 0}},  // 80.54 us, 2729.8 GB/s
    {49376, 7168, 1, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0, 0}},  // 101.91 us, 6947.0 GB/s
    {49376, 7168, 2, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0, 0}},  // 101.97 us, 6944.0 GB/s
    {49376, 7168, 4, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0, 0}},  // 101.97 us, 6946.2 GB/s
    {49376, 7168, 8, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0, 0}},  // 101.87 us, 6957.5 GB/s
    {49376, 7168, 16, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0, 0}},  // 102.64 us, 6914.1 GB/s
    {49376, 7168, 32, {PROJ_KERNEL_MFMA_XS, 32, 1, 8, 2, 2, 128, 1, 0, 0, 0}},  // 107.34 us, 6628.2 GB/s
    {49376, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 1, 16, 2, 1, 64, 3, 1, 8, 1}},  // 112.0 us, 6384.7 GB/s
    {49376, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 1, 16, 2, 1, 64, 3, 1, 8, 1}},  // 153.75 us, 4698.1 GB/s
    {49376, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 1, 16, 4, 1, 32, 4, 1, 8, 0}},  // 250.83 us, 2937.5 GB/s
};
}  // namespace

bool lookup_measured_tactic(int N, int K, int bin, proj_tactic_t *out) {
    // The smallest measured bin at or above `bin` for the shape: its tactic
    // serves any batch up to its capacity, so a plan's own bins (say the
    // verify batches 3, 6, 12 of speculative decoding) take the measured
    // choice of the next power of two above them.
    const Entry *best = nullptr;
    for (const Entry &e : kTable) {
        if (e.N == N && e.K == K && e.bin >= bin && e.t.kernel != 0 &&
            (!best || e.bin < best->bin))
            best = &e;
    }
    if (!best) return false;
    *out = best->t;
    return true;
}

}  // namespace tp1
