// tactics_table.cpp -- tactics measured on MI355X, per (N, K, batch bin).
//
// Each row was chosen by timing every candidate tactic on rotated weight
// copies (so no weight bytes come from the caches), calls enqueued back to
// back, and keeping the fastest mean per call; ties within 1% go to fewer
// launches, then the smaller split.
// Rows: {N, K, bin, {kernel, bcap, split, rows, waves, wpc, kc, depth, kw, nw}}.
#include "tactics_table.hpp"

namespace tp1 {

namespace {
struct Entry {
    int N, K, bin;
    proj_tactic_t t;
};

// Measured on one MI355X (256 CUs), rotated weight copies, mean of 40 calls
// back to back per candidate; each comment gives the chosen tactic's time
// and achieved bandwidth (weight + x + y bytes).
const Entry kTable[] = {
    {7168, 12288, 1, {PROJ_KERNEL_STREAM_DOT2, 1, 1, 4, 4, 8, 0, 0, 0, 0}},  // 30.68 us, 5743.1 GB/s
    {7168, 12288, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 1, 256, 3, 2, 8}},  // 30.8 us, 5722.0 GB/s
    {7168, 12288, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 1, 256, 3, 2, 8}},  // 30.78 us, 5728.3 GB/s
    {7168, 12288, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 1, 256, 3, 2, 8}},  // 31.02 us, 5689.0 GB/s
    {7168, 12288, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 1, 256, 3, 2, 8}},  // 31.64 us, 5587.3 GB/s
    {7168, 12288, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 4, 8, 2, 1, 128, 3, 1, 8}},  // 33.15 us, 5351.6 GB/s
    {7168, 12288, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 4, 8, 2, 1, 128, 3, 1, 8}},  // 37.24 us, 4797.3 GB/s
    {7168, 12288, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 8, 16, 2, 1, 64, 3, 1, 8}},  // 46.91 us, 3861.5 GB/s
    {7168, 12288, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 4, 8, 4, 1, 64, 3, 1, 8}},  // 70.94 us, 2623.7 GB/s
    {14560, 7168, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4}},  // 32.9 us, 6345.8 GB/s
    {14560, 7168, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8}},  // 33.38 us, 6255.8 GB/s
    {14560, 7168, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8}},  // 33.2 us, 6292.3 GB/s
    {14560, 7168, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8}},  // 33.09 us, 6318.5 GB/s
    {14560, 7168, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8}},  // 33.03 us, 6340.5 GB/s
    {14560, 7168, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 2, 8, 2, 1, 128, 3, 1, 8}},  // 36.6 us, 5741.1 GB/s
    {14560, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 2, 8, 2, 1, 128, 3, 1, 8}},  // 41.51 us, 5095.5 GB/s
    {14560, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 4, 16, 2, 1, 64, 3, 1, 8}},  // 52.46 us, 4084.9 GB/s
    {14560, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 2, 8, 4, 1, 64, 3, 1, 8}},  // 82.35 us, 2669.8 GB/s
    {49376, 7168, 1, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0}},  // 101.96 us, 6943.6 GB/s
    {49376, 7168, 2, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0}},  // 101.98 us, 6943.3 GB/s
    {49376, 7168, 4, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0}},  // 102.02 us, 6942.8 GB/s
    {49376, 7168, 8, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0}},  // 102.22 us, 6933.7 GB/s
    {49376, 7168, 16, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0}},  // 102.99 us, 6890.6 GB/s
    {49376, 7168, 32, {PROJ_KERNEL_MFMA_XS, 32, 1, 8, 2, 2, 128, 1, 0, 0}},  // 107.06 us, 6645.6 GB/s
    {49376, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 1, 16, 1, 1, 64, 3, 1, 8}},  // 117.72 us, 6074.5 GB/s
    {49376, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 1, 16, 2, 1, 64, 3, 1, 8}},  // 156.97 us, 4601.7 GB/s
    {49376, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 1, 16, 4, 1, 32, 4, 1, 8}},  // 260.66 us, 2826.7 GB/s
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
