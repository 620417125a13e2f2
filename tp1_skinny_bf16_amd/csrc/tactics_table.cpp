// tactics_table.cpp -- tactics measured on MI355X, per (N, K, batch bin).
//
// Each row was chosen by timing every candidate tactic on rotated weight
// copies (so no weight bytes come from the caches), calls enqueued back to
// back, and keeping the fastest mean per call; ties within 1% go to fewer
// launches, then the smaller split.
// Rows: {N, K, bin, {kernel, bcap, split, rows, waves, wpc, kc, depth, kw, nw, stagger}}.
#include "tactics_table.hpp"

#include <algorithm>
#include <cmath>

namespace tp1 {

namespace {
struct Entry {
    int N, K, bin;
    proj_tactic_t t;
};

// Measured on MI355X (256 CUs), rotated weight copies, mean of 40 calls
// back to back per candidate; per bin the fastest over the tuning runs on
// the current kernels (three full runs, one of them without the staggered
// candidates, one more run of the 7168 x 12288 bins up to 16 after the
// 512-wide chunk instances were added, and one of the bins 32..128 of the
// three shapes after the single-pass eight-wave instances with 32- and
// 64-row groups were added).  Each
// comment gives the chosen tactic's time and achieved bandwidth (weight + x +
// y bytes).
const Entry kTable[] = {
    {7168, 12288, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 512, 3, 4, 8, 1}},  // 28.81 us, 6115.9 GB/s
    {7168, 12288, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 512, 3, 4, 8, 1}},  // 28.68 us, 6145.0 GB/s
    {7168, 12288, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 28.88 us, 6105.1 GB/s
    {7168, 12288, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 28.23 us, 6251.2 GB/s
    {7168, 12288, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 29.01 us, 6093.9 GB/s
    {7168, 12288, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 2, 4, 2, 1, 128, 4, 1, 8, 1}},  // 32.06 us, 5533.6 GB/s
    {7168, 12288, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 4, 8, 2, 1, 128, 3, 1, 8, 1}},  // 34.98 us, 5107.2 GB/s
    {7168, 12288, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 4, 8, 2, 1, 64, 4, 1, 8, 0}},  // 45.94 us, 3943.0 GB/s
    {7168, 12288, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 4, 8, 4, 1, 64, 3, 1, 8, 0}},  // 68.96 us, 2699.0 GB/s
    {14560, 7168, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4, 0}},  // 32.08 us, 6508.0 GB/s
    {14560, 7168, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4, 0}},  // 32.19 us, 6487.1 GB/s
    {14560, 7168, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4, 0}},  // 32.25 us, 6477.7 GB/s
    {14560, 7168, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4, 0}},  // 32.38 us, 6457.1 GB/s
    {14560, 7168, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4, 0}},  // 32.32 us, 6479.8 GB/s
    {14560, 7168, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 1, 4, 2, 1, 128, 4, 1, 8, 0}},  // 34.04 us, 6172.8 GB/s
    {14560, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 2, 8, 4, 1, 128, 3, 1, 8, 0}},  // 39.62 us, 5338.5 GB/s
    {14560, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 4, 16, 2, 1, 64, 3, 1, 8, 1}},  // 50.89 us, 4210.9 GB/s
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
    // Per-GPU shards of a G-way tensor-parallel step, G = 2, 4, 8: the input
    // projections column-sharded (N/G x 7168), o_proj row-sharded (7168 x
    // 12288/G); up to 64 rotated copies per shard.  Per bin the faster of a
    // full tuning run and a run of bins 32..128 after the single-pass
    // eight-wave instances were added.  After the split-K pass learned to
    // load every slice before adding, a third full run was checked bin by
    // bin against the table's tactic in alternating pairs on one box: two
    // bins changed (1820 x 7168 and 7168 x 3072 at B = 64).
    {1820, 7168, 1, {PROJ_KERNEL_STREAM_DOT2, 1, 1, 2, 4, 4, 0, 0, 0, 0, 0}},  // 8.89 us, 2937.0 GB/s
    {1820, 7168, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 1, 1, 1, 512, 3, 8, 8, 1}},  // 10.06 us, 2597.2 GB/s
    {1820, 7168, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 2, 1, 1, 1, 512, 3, 8, 8, 0}},  // 10.0 us, 2616.3 GB/s
    {1820, 7168, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 2, 1, 1, 1, 256, 4, 8, 8, 1}},  // 10.01 us, 2620.9 GB/s
    {1820, 7168, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 3, 2, 1, 1, 256, 4, 4, 8, 0}},  // 10.48 us, 2517.1 GB/s
    {1820, 7168, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 4, 2, 1, 1, 256, 4, 4, 8, 0}},  // 11.09 us, 2404.6 GB/s
    {1820, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 8, 4, 2, 1, 128, 4, 1, 8, 0}},  // 12.8 us, 2128.3 GB/s (paired re-check: 13.37 us before)
    {1820, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 8, 4, 4, 1, 64, 4, 1, 8, 0}},  // 18.01 us, 1576.5 GB/s
    {1820, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 8, 8, 8, 1, 64, 3, 1, 8, 0}},  // 26.62 us, 1153.0 GB/s
    {3640, 7168, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 1, 1, 1, 512, 4, 8, 8, 0}},  // 10.75 us, 4856.2 GB/s
    {3640, 7168, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 1, 1, 1, 512, 4, 8, 8, 0}},  // 11.04 us, 4730.6 GB/s
    {3640, 7168, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 1, 1, 1, 512, 4, 8, 8, 0}},  // 11.0 us, 4751.8 GB/s
    {3640, 7168, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 1, 1, 1, 512, 4, 8, 8, 0}},  // 11.54 us, 4536.9 GB/s
    {3640, 7168, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 1, 1, 1, 256, 4, 8, 8, 0}},  // 12.31 us, 4267.2 GB/s
    {3640, 7168, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 4, 4, 2, 1, 128, 4, 1, 8, 0}},  // 14.23 us, 3715.7 GB/s
    {3640, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 4, 4, 4, 1, 128, 4, 1, 8, 0}},  // 17.51 us, 3059.2 GB/s
    {3640, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 4, 4, 4, 1, 64, 4, 1, 8, 1}},  // 23.2 us, 2368.5 GB/s
    {3640, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 8, 8, 4, 1, 64, 3, 1, 8, 0}},  // 31.96 us, 1805.9 GB/s
    {6172, 7168, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 15.59 us, 5677.3 GB/s
    {6172, 7168, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 15.67 us, 5650.0 GB/s
    {6172, 7168, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 15.61 us, 5675.1 GB/s
    {6172, 7168, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 15.87 us, 5588.9 GB/s
    {6172, 7168, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 16.85 us, 5276.5 GB/s
    {6172, 7168, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 2, 4, 2, 1, 128, 4, 1, 8, 0}},  // 19.37 us, 4612.1 GB/s
    {6172, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 4, 8, 2, 1, 128, 3, 1, 8, 0}},  // 23.35 us, 3862.5 GB/s
    {6172, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 4, 8, 2, 1, 64, 4, 1, 8, 1}},  // 31.23 us, 2942.6 GB/s
    {6172, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 4, 8, 4, 1, 64, 3, 1, 8, 0}},  // 44.3 us, 2151.5 GB/s
    {7168, 1536, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 6.24 us, 3531.7 GB/s
    {7168, 1536, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 6.75 us, 3267.4 GB/s
    {7168, 1536, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 6.56 us, 3367.3 GB/s
    {7168, 1536, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 6.52 us, 3398.7 GB/s
    {7168, 1536, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 6.66 us, 3348.1 GB/s
    {7168, 1536, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 7.89 us, 2861.5 GB/s
    {7168, 1536, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 1, 2, 4, 1, 128, 4, 1, 8, 0}},  // 9.37 us, 2469.0 GB/s
    {7168, 1536, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 2, 4, 4, 1, 64, 4, 1, 8, 0}},  // 15.36 us, 1578.7 GB/s
    {7168, 1536, 256, {PROJ_KERNEL_MFMA_XS, 256, 1, 2, 4, 1, 128, 1, 0, 0, 1}},  // 23.79 us, 1112.9 GB/s
    {7168, 3072, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 9.23 us, 4773.6 GB/s
    {7168, 3072, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 9.28 us, 4750.1 GB/s
    {7168, 3072, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 9.37 us, 4708.9 GB/s
    {7168, 3072, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 9.32 us, 4742.9 GB/s
    {7168, 3072, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 9.83 us, 4513.5 GB/s
    {7168, 3072, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 11.69 us, 3823.4 GB/s
    {7168, 3072, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 2, 4, 4, 1, 128, 4, 1, 8, 1}},  // 15.13 us, 2997.4 GB/s (paired re-check: 16.14 us before)
    {7168, 3072, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 2, 4, 4, 1, 64, 4, 1, 8, 1}},  // 20.94 us, 2228.3 GB/s
    {7168, 3072, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 4, 8, 8, 1, 64, 3, 1, 8, 0}},  // 30.39 us, 1621.7 GB/s
    {7168, 6144, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 512, 3, 4, 8, 1}},  // 16.06 us, 5486.1 GB/s
    {7168, 6144, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 15.86 us, 5557.0 GB/s
    {7168, 6144, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 15.86 us, 5560.3 GB/s
    {7168, 6144, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 15.79 us, 5591.7 GB/s
    {7168, 6144, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 16.56 us, 5344.6 GB/s
    {7168, 6144, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 2, 4, 2, 1, 128, 4, 1, 8, 1}},  // 19.06 us, 4665.9 GB/s
    {7168, 6144, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 4, 8, 2, 1, 128, 3, 1, 8, 0}},  // 22.76 us, 3944.8 GB/s
    {7168, 6144, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 4, 8, 2, 1, 64, 4, 1, 8, 0}},  // 30.22 us, 3027.4 GB/s
    {7168, 6144, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 4, 8, 8, 1, 64, 3, 1, 8, 0}},  // 41.26 us, 2300.0 GB/s
    {7280, 7168, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 18.1 us, 5767.7 GB/s
    {7280, 7168, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 17.75 us, 5883.0 GB/s
    {7280, 7168, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 1}},  // 17.8 us, 5869.8 GB/s
    {7280, 7168, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 17.82 us, 5869.7 GB/s
    {7280, 7168, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256, 4, 4, 8, 0}},  // 18.4 us, 5697.2 GB/s
    {7280, 7168, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 2, 4, 2, 1, 128, 4, 1, 8, 0}},  // 21.39 us, 4922.4 GB/s
    {7280, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 4, 8, 2, 1, 128, 3, 1, 8, 0}},  // 25.21 us, 4213.2 GB/s
    {7280, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 4, 8, 2, 1, 64, 4, 1, 8, 1}},  // 31.73 us, 3405.8 GB/s
    {7280, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 4, 8, 4, 1, 64, 3, 1, 8, 0}},  // 45.88 us, 2436.0 GB/s
    {12344, 7168, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8, 0}},  // 28.24 us, 6267.8 GB/s
    {12344, 7168, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8, 0}},  // 28.12 us, 6295.9 GB/s
    {12344, 7168, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8, 0}},  // 28.06 us, 6312.2 GB/s
    {12344, 7168, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8, 0}},  // 28.39 us, 6244.3 GB/s
    {12344, 7168, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8, 0}},  // 28.53 us, 6224.6 GB/s
    {12344, 7168, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 1, 4, 2, 1, 128, 4, 1, 8, 0}},  // 30.52 us, 5839.2 GB/s
    {12344, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 2, 8, 2, 1, 128, 3, 1, 8, 1}},  // 35.76 us, 5018.5 GB/s
    {12344, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 4, 16, 2, 1, 64, 3, 1, 8, 1}},  // 48.05 us, 3786.9 GB/s
    {12344, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 2, 8, 4, 1, 64, 3, 1, 8, 0}},  // 75.26 us, 2484.1 GB/s
    {24688, 7168, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 2, 128, 3, 1, 4, 0}},  // 53.25 us, 6647.7 GB/s
    {24688, 7168, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 2, 128, 3, 1, 4, 0}},  // 53.35 us, 6636.4 GB/s
    {24688, 7168, 4, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 2, 128, 3, 1, 4, 0}},  // 53.15 us, 6663.8 GB/s
    {24688, 7168, 8, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 4, 1, 2, 128, 3, 1, 4, 0}},  // 52.99 us, 6688.8 GB/s
    {24688, 7168, 16, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 8, 1, 1, 128, 3, 1, 4, 0}},  // 52.73 us, 6731.4 GB/s
    {24688, 7168, 32, {PROJ_KERNEL_MFMA_PIPE, 32, 1, 8, 2, 1, 128, 3, 1, 8, 0}},  // 54.15 us, 6573.7 GB/s
    {24688, 7168, 64, {PROJ_KERNEL_MFMA_PIPE, 64, 1, 8, 2, 1, 128, 3, 1, 8, 1}},  // 60.49 us, 5918.4 GB/s
    {24688, 7168, 128, {PROJ_KERNEL_MFMA_PIPE, 128, 2, 16, 2, 1, 64, 3, 1, 8, 1}},  // 82.91 us, 4367.2 GB/s
    {24688, 7168, 256, {PROJ_KERNEL_MFMA_PIPE, 256, 1, 8, 4, 1, 64, 3, 1, 8, 1}},  // 135.88 us, 2724.7 GB/s
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

int nearby_measured_tactics(int N, int K, int bin, proj_tactic_t *out, int max_out) {
    // Shapes measured with a bin at or above `bin`, by distance
    // |ln(N/N')| + |ln(K/K')|, keeping those within ln 2; each gives the
    // tactic of its smallest such bin.
    struct Cand {
        double d;
        const Entry *e;
    };
    Cand c[sizeof kTable / sizeof kTable[0]];
    int n = 0;
    for (const Entry &e : kTable) {
        if (e.bin < bin || e.t.kernel == 0 || (e.N == N && e.K == K)) continue;
        const double d = std::fabs(std::log((double)N / e.N)) + std::fabs(std::log((double)K / e.K));
        if (d > std::log(2.0)) continue;
        int j = 0;
        while (j < n && !(c[j].e->N == e.N && c[j].e->K == e.K)) ++j;
        if (j < n) {
            if (e.bin < c[j].e->bin) c[j].e = &e;  // the smallest bin >= `bin`
            continue;
        }
        c[n++] = Cand{d, &e};
    }
    std::sort(c, c + n, [](const Cand &a, const Cand &b) {
        return a.d < b.d || (a.d == b.d && (a.e->N < b.e->N || (a.e->N == b.e->N && a.e->K < b.e->K)));
    });
    const int m = std::min(n, max_out);
    for (int i = 0; i < m; ++i) out[i] = c[i].e->t;
    return m;
}

}  // namespace tp1
