// tactics_table.cpp -- tactics measured on MI355X, per (N, K, batch bin).
//
// Each row was chosen by timing every candidate tactic on rotated weight
// copies (so no weight bytes come from the caches) and keeping the median
// fastest; ties within 1% go to fewer launches, then the smaller split.
// Where several tuning runs measured a bin, the fastest run's choice is kept.
// Rows: {N, K, bin, {kernel, bcap, split, rows, waves, wpc, kc, depth, kw, nw}}.
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
    {7168, 12288, 1, {PROJ_KERNEL_STREAM_DOT2, 1, 1, 4, 4, 8, 0, 0, 0, 0}},  // 32.18 us, 5475.4 GB/s
    {7168, 12288, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 1, 256, 3, 2, 8}},  // 32.58 us, 5409.4 GB/s
    {7168, 12288, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 1, 256, 3, 2, 8}},  // 32.68 us, 5395.2 GB/s
    {7168, 12288, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 1, 256, 3, 2, 8}},  // 32.76 us, 5386.8 GB/s
    {7168, 12288, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 4, 4, 1, 1, 256, 3, 2, 8}},  // 33.2 us, 5324.8 GB/s
    {7168, 12288, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 4, 8, 2, 1, 128, 3, 1, 8}},  // 34.44 us, 5151.2 GB/s
    {7168, 12288, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 4, 8, 2, 1, 128, 3, 1, 8}},  // 38.64 us, 4623.5 GB/s
    {7168, 12288, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 8, 16, 2, 1, 64, 3, 1, 8}},  // 48.03 us, 3771.4 GB/s
    {7168, 12288, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 4, 8, 4, 1, 64, 3, 1, 8}},  // 72.45 us, 2569.0 GB/s
    {14560, 7168, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8}},  // 34.52 us, 6048.0 GB/s
    {14560, 7168, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8}},  // 34.95 us, 5974.8 GB/s
    {14560, 7168, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8}},  // 34.8 us, 6003.0 GB/s
    {14560, 7168, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8}},  // 34.79 us, 6009.8 GB/s
    {14560, 7168, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8}},  // 34.38 us, 6091.5 GB/s
    {14560, 7168, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 2, 8, 2, 1, 128, 3, 1, 8}},  // 38.09 us, 5516.5 GB/s
    {14560, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 2, 8, 2, 1, 128, 3, 1, 8}},  // 42.77 us, 4945.4 GB/s
    {14560, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 4, 16, 2, 1, 64, 3, 1, 8}},  // 53.79 us, 3983.9 GB/s
    {14560, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 2, 8, 4, 1, 64, 3, 1, 8}},  // 84.99 us, 2586.9 GB/s
    {49376, 7168, 1, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0}},  // 103.55 us, 6837.0 GB/s
    {49376, 7168, 2, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0}},  // 103.77 us, 6823.6 GB/s
    {49376, 7168, 4, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0}},  // 103.95 us, 6813.9 GB/s
    {49376, 7168, 8, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0}},  // 103.47 us, 6849.9 GB/s
    {49376, 7168, 16, {PROJ_KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 0}},  // 104.17 us, 6812.6 GB/s
    {49376, 7168, 32, {PROJ_KERNEL_MFMA_XS, 32, 1, 8, 2, 2, 128, 1, 0, 0}},  // 107.65 us, 6609.1 GB/s
    {49376, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 1, 16, 2, 1, 64, 3, 1, 8}},  // 113.3 us, 6311.5 GB/s
    {49376, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 1, 16, 2, 1, 64, 3, 1, 8}},  // 157.48 us, 4586.8 GB/s
    {49376, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 1, 8, 4, 1, 64, 3, 1, 8}},  // 272.53 us, 2703.6 GB/s
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
