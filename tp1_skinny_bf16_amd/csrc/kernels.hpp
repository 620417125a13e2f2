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
    int num_cus;
};

// Enqueue one projection with tactic t.  Returns a hipError_t.
hipError_t launch_projection(const LaunchShape &s, const proj_tactic_t &t,
                             hipStream_t stream);

// Name of the kernel instance(s) a tactic launches (for profiles).
int kernel_name(int K, const proj_tactic_t &t, char *buf, size_t len);

// Streaming-read probe (measurement aid).
hipError_t launch_read_probe(const void *buf, size_t bytes, float *sink,
                             int waves_per_cu, int num_cus, hipStream_t stream);

}  // namespace tp1
