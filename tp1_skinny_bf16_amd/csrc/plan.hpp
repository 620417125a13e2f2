// plan.hpp -- host-side plan logic of the TP1 projection: argument checks,
// the per-batch tactic table, the bin rule and workspace sizing.  Pure C++:
// no HIP header is included here, so this logic builds and runs on a host
// without a GPU.
#pragma once

#include <cstddef>

#include "../../include/tp1_proj.h"

namespace tp1 {

// Hardware limits of gfx950 the tactics must respect.
constexpr int kWave = 64;
constexpr int kMaxWaves = 16;                 // 1024 threads per workgroup
constexpr size_t kLdsBytes = 160 * 1024;      // LDS per workgroup on gfx950
constexpr int kStreamChunk = 512;             // K elements one wave load covers

struct PlanCore {
    int N = 0, K = 0;
    int nb = 0;
    int batches[PROJ_MAX_BATCHES] = {};
    proj_tactic_t tactics[PROJ_MAX_BATCHES] = {};
    unsigned flags = 0;
    int num_cus = 256;                        // compute units of the device
};

// The compiled shared-tile MFMA instances: X(bcap, rows, waves, kc, depth).
#define TP1_XS_INSTANCES(X)                                                          \
    X(16, 4, 1, 128, 1) X(16, 4, 1, 128, 2) X(16, 4, 1, 256, 2) X(16, 4, 1, 512, 1)  \
    X(16, 8, 1, 128, 1) X(16, 8, 1, 128, 2) X(16, 8, 1, 256, 1) X(16, 16, 1, 128, 1) \
    X(32, 4, 1, 128, 1) X(32, 4, 1, 128, 2) X(32, 4, 2, 128, 1) X(32, 8, 2, 128, 1)  \
    X(32, 8, 2, 256, 1) X(64, 4, 1, 128, 1) X(64, 4, 2, 128, 1) X(64, 4, 2, 128, 2)  \
    X(64, 4, 4, 128, 1) X(64, 8, 2, 128, 1) X(64, 8, 2, 256, 1) X(128, 4, 2, 128, 1) \
    X(128, 4, 4, 128, 1) X(256, 4, 4, 128, 1) X(256, 2, 4, 128, 1)

// The compiled pipelined MFMA instances:
// X(bcap, rows, waves, kw, kc, depth, nw).
#define TP1_PIPE_INSTANCES(X)                                                               \
    X(16, 4, 1, 1, 128, 3, 4) X(16, 4, 1, 1, 128, 4, 4) X(16, 4, 1, 1, 128, 6, 4)           \
    X(16, 4, 1, 1, 256, 3, 4) X(16, 8, 1, 1, 128, 3, 4) X(16, 8, 1, 1, 128, 4, 4)           \
    X(16, 2, 1, 2, 256, 6, 4) X(16, 2, 1, 2, 256, 4, 4) X(16, 2, 1, 2, 128, 8, 4)           \
    X(16, 1, 1, 4, 256, 4, 4) X(16, 1, 1, 4, 256, 6, 4) X(32, 4, 1, 1, 128, 4, 4)           \
    X(32, 4, 1, 1, 128, 6, 4) X(32, 4, 2, 1, 64, 8, 4) X(32, 8, 2, 1, 128, 3, 4)            \
    X(32, 2, 1, 2, 256, 4, 4) X(32, 2, 2, 1, 256, 4, 4) X(64, 4, 2, 1, 64, 8, 4)            \
    X(64, 4, 2, 1, 128, 4, 4) X(64, 4, 4, 1, 64, 8, 4) X(64, 8, 2, 1, 64, 4, 4)             \
    X(64, 8, 2, 1, 64, 6, 4) X(128, 4, 4, 1, 64, 6, 4) X(128, 4, 4, 1, 32, 12, 4)           \
    X(128, 8, 4, 1, 64, 4, 4) X(128, 8, 4, 1, 32, 8, 4) X(256, 4, 4, 1, 32, 7, 4)           \
    X(256, 4, 4, 1, 64, 3, 4) X(256, 8, 4, 1, 32, 6, 4) X(256, 8, 4, 1, 64, 3, 4)           \
    X(64, 16, 2, 1, 64, 3, 8) X(64, 8, 2, 1, 128, 3, 8) X(64, 16, 1, 1, 64, 3, 8)           \
    X(128, 16, 2, 1, 64, 3, 8) X(128, 8, 2, 1, 64, 4, 8) X(128, 16, 4, 1, 32, 4, 8)         \
    X(256, 16, 4, 1, 32, 4, 8) X(256, 8, 4, 1, 64, 3, 8)          \
    X(16, 8, 1, 1, 256, 2, 8) X(16, 4, 1, 2, 256, 3, 8) X(32, 8, 2, 1, 128, 3, 8)           \
    X(64, 8, 4, 1, 128, 3, 8) X(256, 8, 8, 1, 64, 3, 8) X(16, 2, 1, 4, 256, 6, 8)          \
    X(16, 2, 1, 4, 256, 4, 8) X(16, 1, 1, 8, 256, 4, 8) X(32, 2, 1, 4, 256, 4, 8)           \
    X(256, 8, 4, 1, 32, 6, 8) X(128, 8, 2, 1, 32, 8, 8) X(128, 16, 2, 1, 32, 6, 8)          \
    X(64, 8, 2, 1, 64, 6, 8) X(16, 2, 1, 4, 512, 3, 8) X(16, 2, 1, 4, 512, 2, 8)             \
    X(16, 1, 1, 8, 512, 4, 8) X(16, 2, 1, 4, 512, 3, 4) X(16, 1, 1, 8, 512, 3, 8)             \
    X(32, 4, 2, 1, 128, 4, 8) X(32, 4, 1, 2, 128, 4, 8) X(32, 4, 1, 2, 256, 3, 8)             \
    X(32, 2, 2, 2, 256, 4, 8) X(64, 4, 2, 1, 128, 4, 8) X(64, 4, 2, 2, 128, 4, 8)             \
    X(64, 4, 4, 1, 128, 4, 8) X(64, 4, 2, 1, 256, 2, 8) X(64, 2, 4, 1, 128, 4, 8)             \
    X(64, 2, 2, 2, 128, 4, 8) X(128, 4, 2, 1, 64, 4, 8) X(128, 4, 4, 1, 64, 4, 8)

// LDS bytes of an MFMA_XS tactic (x and W chunk tiles, 16 bytes of row pad).
size_t mfma_xs_lds_bytes(const proj_tactic_t &t);

// LDS bytes of an MFMA_PIPE tactic: depth stages of x and W chunk tiles,
// plus the partial tiles of the waves along K.
size_t mfma_pipe_lds_bytes(const proj_tactic_t &t);

// Argument checks of proj_plan (no device access).
int check_plan_args(int N, int K, const int *batches, int n_batches,
                    unsigned flags);

// Index of the bin serving B: the smallest planned batch >= B.  -1 when B is
// out of 1..max(batches).
int bin_index(const PlanCore &p, int B);

// True when a compiled kernel instance exists for the tactic's template
// parameters (kernel, bcap, rows).
bool tactic_instance_exists(const proj_tactic_t &t);

// Validate a tactic for a shape and bin.  Returns PROJ_OK or PROJ_EINVAL.
int check_tactic(int N, int K, int bin, const proj_tactic_t &t);

// FP32 split-K workspace bytes a tactic needs (0 when split == 1).
size_t tactic_workspace(int N, int K, const proj_tactic_t &t);

// K elements per split-K slice for a tactic (rounded to the kernel's step).
int slice_len(int K, const proj_tactic_t &t);

// Number of K slices actually launched (ceil(K / slice_len)).
int slice_count(int K, const proj_tactic_t &t);


// LDS bytes a STREAM tactic stages x into.
size_t stream_lds_bytes(int K, const proj_tactic_t &t);

// Static LDS of a tactic's kernel instance (its __shared__ arrays), which
// the workgroup's LDS must hold beside the dynamic part.
size_t static_lds_bytes(const proj_tactic_t &t);

// Dynamic LDS bytes a tactic's kernel instance is launched with.
size_t dynamic_lds_bytes(int K, const proj_tactic_t &t);

// The tactic for (N, K, bin): the measured table entry when the shape was
// measured, else the default rule.
proj_tactic_t choose_tactic(int N, int K, int bin, int num_cus);

// The default rule alone (exposed for tests).
proj_tactic_t default_tactic(int N, int K, int bin, int num_cus);

// Fill p.tactics for every planned bin.
void fill_tactics(PlanCore &p);

// Workspace bytes the whole plan needs.
size_t plan_workspace(const PlanCore &p);

}  // namespace tp1
