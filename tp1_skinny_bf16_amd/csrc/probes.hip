// probes.hip -- measurement aids beside the projection (not part of it).
//
// ring_probe_kernel issues the loads of the pipelined projection kernel's LDS
// ring and nothing else: eight waves, a ring of D stages of ROWS rows x PIECE
// bytes filled by direct-to-LDS 128-bit loads (one 1 KB block of 64 lanes per
// instruction), one wait and, with BAR, one workgroup barrier per stage, no
// arithmetic and no LDS reads.  It separates what the kernel's loads cost from
// what its multiply costs.  The load and wait helpers are restated here so
// that this file shares no code with the projection's kernels.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace tp1 {
namespace {

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void probe_wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ uint32_t probe_lds_address(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from src into LDS at m0 + 16 * lane (m0 wave-uniform);
// one wait state between the scalar write of M0 and the load that reads it.
__device__ __forceinline__ void probe_load_cached(const void *src, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(m0)
                 : "memory", "m0");
}
__device__ __forceinline__ void probe_load_stream(const void *src, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(src), "s"(m0)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Stage rows 0..63 hold x rows when what has bit 0 (x is [64, K], the same
// block for every workgroup, so L2 serves it; cached loads, as the kernel
// loads x), every other stage row a weight row (a private [64, K] block per
// workgroup, read from HBM, or with shared_w one block for all; non-temporal
// loads, as the kernel loads the weight).  Chunk c of a row is bytes
// [c * PIECE, (c + 1) * PIECE); the workgroup walks C chunks.
template <int ROWS, int PIECE, int D, bool BAR>
__global__ __launch_bounds__(512) void ring_probe_kernel(const char *x, const char *w, long pitch,
                                                         int C, int what, int shared_w,
                                                         float *sink) {
    constexpr int LPR = PIECE / 16;          // lanes per row piece
    constexpr int STAGE = ROWS * PIECE;
    constexpr int NB = STAGE / 1024;         // 1 KB blocks per stage
    constexpr int NI = NB / 8;               // blocks per wave per stage
    static_assert(ROWS == 64 || ROWS == 128, "stage rows");
    static_assert(NI >= 1 && NI * 8 == NB, "blocks split over the eight waves");
    static_assert(D >= 2 && NI * (D - 2) <= 63, "loads in flight");
    extern __shared__ __align__(16) char probe_lds[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint32_t l0 = __builtin_amdgcn_readfirstlane((int)probe_lds_address(probe_lds));
    const char *wb = w + (shared_w ? 0L : (long)blockIdx.x * 64 * pitch);
    int it = 0;
    auto issue = [&]() {
        const int c = it % C;
        const uint32_t st = l0 + (uint32_t)((it % D) * STAGE);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int bi = i * 8 + wave;
            const int slot = bi * 64 + lane;
            const int r = slot / LPR, p = slot % LPR;
            const long off = (long)(r & 63) * pitch + (long)c * PIECE + p * 16;
            const uint32_t m0 = st + (uint32_t)bi * 1024u;
            if ((what & 1) && r < 64)
                probe_load_cached(x + off, m0);
            else
                probe_load_stream(wb + off, m0);
        }
        ++it;
    };
#pragma unroll
    for (int p = 0; p < D - 1; ++p) issue();
    for (int t = 0; t < C; ++t) {
        probe_wait_vmcnt<NI * (D - 2)>();  // this wave's pieces of stage t landed
        if (BAR) __syncthreads();
        issue();
    }
    probe_wait_vmcnt<0>();
    if (lane == 0) sink[blockIdx.x * 8 + wave] = (float)it;
}

}  // namespace

// X(rows, piece, depth, barrier)
#define TP1_RING_PROBE_INSTANCES(X)                                                        \
    X(64, 256, 5, true) X(64, 256, 5, false) X(128, 256, 3, true) X(64, 512, 3, true)      \
    X(64, 512, 3, false) X(64, 1024, 2, true) X(64, 1024, 2, false) X(64, 256, 9, true)    \
    X(128, 256, 5, true) X(64, 128, 9, true) X(128, 128, 9, true)

bool ring_probe_instance_exists(int rows, int piece, int depth, bool barrier) {
#define TP1_RING_MATCH(R, P, DD, BB) \
    if (rows == R && piece == P && depth == DD && barrier == BB) return true;
    TP1_RING_PROBE_INSTANCES(TP1_RING_MATCH)
#undef TP1_RING_MATCH
    return false;
}

hipError_t launch_ring_probe(const void *x, const void *w, long pitch, int C, int rows, int piece,
                             int depth, bool barrier, int what, int shared_w, int grid,
                             float *sink, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
#define TP1_RING_LAUNCH(R, P, DD, BB)                                                        \
    if (rows == R && piece == P && depth == DD && barrier == BB) {                          \
        static bool allowed[64] = {};                                                       \
        if (!allowed[dev]) {                                                                \
            const hipError_t e = hipFuncSetAttribute(                                       \
                reinterpret_cast<const void *>(&ring_probe_kernel<R, P, DD, BB>),           \
                hipFuncAttributeMaxDynamicSharedMemorySize, DD * R * P);                    \
            if (e != hipSuccess) return e;                                                  \
            allowed[dev] = true;                                                            \
        }                                                                                   \
        hipLaunchKernelGGL((ring_probe_kernel<R, P, DD, BB>), dim3((unsigned)grid), dim3(512), \
                           (size_t)DD * R * P, stream, static_cast<const char *>(x),         \
                           static_cast<const char *>(w), pitch, C, what, shared_w, sink);    \
        return hipGetLastError();                                                           \
    }
    TP1_RING_PROBE_INSTANCES(TP1_RING_LAUNCH)
#undef TP1_RING_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace tp1
