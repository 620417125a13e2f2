// kernels.hpp -- launch interface of the gfx950 kernels (host side).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/tp1_proj.h"

namespace tp1 {

struct LaunchShape {
    int N, K, B;
    const uint16_t *x;
    long ldx;
    const uint16_t *W;
    uint16_t *y;
    float *ws;          // split-K workspace (S * B * N floats) or nullptr
    int *cnt;           // kSplitCounters zeroed ints for the fused split-K
                        // reduction, or nullptr for the two-pass reduction
    int num_cus;
};

// Arrival counters a plan holds for the fused split-K reduction (one per
// workgroup of a K slice); larger grids fall back to the two-pass reduction.
constexpr long kSplitCounters = 65536;

// Enqueue one projection with tactic t.  Returns a hipError_t.
hipError_t launch_projection(const LaunchShape &s, const proj_tactic_t &t,
                             hipStream_t stream);

// Allow every compiled kernel instance up to `bytes` of dynamic LDS on the
// current device.  Called once per device when a plan is built, so that
// launches never change function attributes (they may be recorded into a
// graph under stream capture, where such calls do not belong).
hipError_t allow_dynamic_lds(size_t bytes);

// Name of the kernel instance(s) a tactic launches (for profiles).
int kernel_name(const LaunchShape &sh, const proj_tactic_t &t, char *buf, size_t len);

// Weight prefetch: read the leading `bytes` (rounded down to 16) of buf with
// cached loads, on 4 workgroups of 256 lanes per compute unit, 128 bytes in
// flight per lane.
hipError_t launch_prefetch(const void *buf, size_t bytes, int num_cus, hipStream_t stream);

// Fixed-duration kernel that touches no memory (`ticks` of the constant-rate
// wall clock), standing in for the attention core between two projections.
hipError_t launch_core_standin(unsigned long long ticks, int num_cus, hipStream_t stream);

// The stand-in core (`ticks`, one sleeping wave per compute unit) and the
// prefetch of the leading `bytes` of buf (as launch_prefetch) in one launch.
hipError_t launch_core_prefetch(unsigned long long ticks, const void *buf, size_t bytes,
                                int num_cus, hipStream_t stream);

// Streaming-read probe (measurement aid).
hipError_t launch_read_probe(const void *buf, size_t bytes, float *sink,
                             int waves_per_cu, int num_cus, hipStream_t stream);

// The LDS-ring load probe (probes.hip): the compiled (rows, piece, depth,
// barrier) combinations, and its launch over `grid` workgroups of 512 lanes.
bool ring_probe_instance_exists(int rows, int piece, int depth, bool barrier);
hipError_t launch_ring_probe(const void *x, const void *w, long pitch, int C, int rows, int piece,
                             int depth, bool barrier, int what, int shared_w, int grid,
                             float *sink, hipStream_t stream);

}  // namespace tp1
