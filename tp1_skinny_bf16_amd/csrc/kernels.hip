// kernels.hip -- gfx950 kernels of the TP1 decode projection y = x . W^T.
//
// The operation is the TP1 linear of the vLLM API page "vllm.models.kimi_k3.
// nvidia.specialized_decode.runtime.dep" (section "DepProjection"; the
// page's opening text fixes BF16 inputs/outputs, FP32 accumulation and a
// free split-K summation order).  W is N x K row-major (nn.Linear), x is
// B x K with row stride ldx, y is B x N contiguous.
//
// Kernels:
//   stream_kernel  small batches.  The weight is streamed once from HBM with
//                  128-bit loads, lanes laid along K (a wave reads 1 KB of a
//                  row per load), the K slice of x staged once per workgroup
//                  in LDS, exact BF16 -> FP32 unpacking and IEEE FP32 fused
//                  multiply-adds, then a fixed-order DPP reduction across the
//                  64 lanes.  Each wave owns a contiguous range of rows and
//                  keeps a ring of weight loads in flight across rows.
//   mfma_xs_kernel / mfma_pipe_kernel  a workgroup shares one x tile and
//                  one weight tile per K chunk in LDS; the pipe variant
//                  fills a ring of LDS stages with direct-to-LDS loads several
//                  chunks ahead.
//   splitk_reduce  when K is split across workgroups: sums the FP32 slices
//                  in the fixed order s = 0..S-1 and rounds to BF16 (no
//                  atomics, so results are bitwise reproducible);
//                  splitk_reduce4 does the same four outputs per thread.
//   prefetch_kernel / core_standin_kernel / core_prefetch_kernel
//                  the weight prefetch with cached loads, a memory-free
//                  stand-in for the attention core between two projections,
//                  and both in one launch.
//   read_probe     measurement aid: a plain streaming read of a buffer.
// Every output is rounded once from FP32 to BF16, nearest-even.
#include "kernels.hpp"

#include <cstdio>

#include "plan.hpp"

namespace tp1 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 128-bit loads.  The weight is read exactly once per call, so its loads are
// marked non-temporal; x and staging data use ordinary loads.
__device__ __forceinline__ u32x4 load_stream(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 load_cached(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// BF16 pair dot product into FP32 (v_dot2c_f32_bf16).  Measured on gfx950:
// the products are exact but the three-term addition is not always IEEE
// round-to-nearest (it can differ from it by a few FP32 ulps, and not
// symmetrically in sign), so this arithmetic is a separate tactic.
__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// FP32 -> BF16, round to nearest, ties to even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint16_t to_bf16(float f) {
    unsigned u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Wave-uniform value: the compiler then keeps what derives from it in SGPRs
// and every branch on it scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Exact BF16 -> FP32 of the two halves of a packed pair.
__device__ __forceinline__ float bf_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(unsigned u) { return __uint_as_float(u & 0xFFFF0000u); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 64 lanes of a wave in a fixed tree (so results are bitwise
// reproducible): DPP butterflies inside each 16-lane row (xor 1, xor 2,
// half-row mirror, row mirror), then the four row sums read from lanes
// 0, 16, 32, 48 and added in that order.  Returns the wave-uniform total.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return ((a + b) + c) + d;
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// A split-K partial.  With the in-kernel reduction (through = true) it is an
// agent-scope store, which writes through the XCD's L2 to the device-coherent
// level, so the workgroup that sums it (possibly on another XCD) reads it
// without any L2 write-back; with the two-pass reduction a plain store does,
// since the kernel boundary orders it before splitk_reduce.
__device__ __forceinline__ void store_partial(float *p, float v, bool through) {
    if (through)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

// ---------------------------------------------------------------------------
// Fused split-K reduction.  When K is split over S workgroups (gridDim.y),
// each workgroup writes its FP32 partials for rows [row0, row0 + rows) to
// the workspace through store_partial, waits until those stores have
// completed, and counts its arrival on an integer counter of its row range.
// The workgroup that arrives last reads the S partials with agent-scope
// loads (from the device-coherent level, not a stale L2 line) and sums them
// in the fixed order s = 0..S-1 (the order of the two-pass splitk_reduce, so
// the result does not depend on arrival order), rounds once to BF16, and
// resets the counter for the next call.  Called by every thread of the
// workgroup, after its last partial store.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void splitk_fixup(const float *ws, uint16_t *y, int *cnt, int N,
                                             int B, int row0, int rows) {
    __shared__ int last;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keep the partial stores above the wait
    wait_vmcnt<0>();                          // this thread's partials have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(cnt + blockIdx.x, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        last = old == (int)gridDim.y - 1;
    }
    __syncthreads();
    if (!last) return;
    const int S = gridDim.y;
    const size_t slice = (size_t)B * N;
    const int total = rows * B;
    // U outputs per thread per round, all loads of a slice issued before any
    // is added, so a round costs one memory round trip per slice.
    constexpr int U = 8;
    for (int base = threadIdx.x; base < total; base += (int)blockDim.x * U) {
        size_t o[U];
        float acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = min(base + u * (int)blockDim.x, total - 1);
            const int b = i / rows, r = i - (i / rows) * rows;
            o[u] = (size_t)b * N + row0 + r;
            acc[u] = __hip_atomic_load(ws + o[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        for (int k = 1; k < S; ++k) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = __hip_atomic_load(ws + k * slice + o[u], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u] += v[u];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + u * (int)blockDim.x < total) y[o[u]] = to_bf16(acc[u]);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(cnt + blockIdx.x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Weight-stream kernel (small batches).
//
// Workgroup g owns rows [N*g/G, N*(g+1)/G) of W (so workgroups differ by at
// most one row) for one K slice.  Its rows are cut into groups of R rows and
// each group's K slice into 512-wide chunks; the (group, chunk) steps are
// split evenly over the workgroup's waves, each wave taking a contiguous run
// (so every wave loads the same number of 1 KB pieces, to within one).  A
// step reads R rows x 1 KB with lanes laid along K.  A group that a wave
// covers entirely is reduced over the wave's 64 lanes and written out; a
// group cut by a wave boundary leaves per-wave partial sums in LDS that are
// added in wave order after one barrier at the end.  Loads form a ring of P
// steps issued ahead of use and are unconditional: positions past the
// wave's last step or the workgroup's last row are clamped onto data
// already read (a cache hit) and discarded.  Arithmetic is exact BF16 ->
// FP32 unpacking and IEEE FP32 fused multiply-adds.
// ---------------------------------------------------------------------------
constexpr int kStreamMaxWaves = 8;

struct StreamArgs {
    const uint16_t *x;
    long ldx;
    const uint16_t *W;
    uint16_t *y;
    float *ws;
    int *cnt;   // split-K arrival counters (fused reduction) or nullptr
    int N, K, B;
    int ks;   // K elements per slice (multiple of 8)
    int ksp;  // LDS row pitch of the staged x slice (multiple of 512)
    int S;    // number of K slices (gridDim.y)
};

// Wave whose run [q_v, q_v+1) of T steps split over NW waves holds step q.
__device__ __forceinline__ int wave_of_step(int q, int T, int NW) {
    return (int)(((long)(q + 1) * NW + T - 1) / T) - 1;
}

template <int BC, int R, int P, bool D2>
__global__ __launch_bounds__(512) void stream_kernel(StreamArgs a) {
    extern __shared__ __align__(16) uint16_t xs[];
    __shared__ float part[kStreamMaxWaves][2][R * BC];  // [wave][head/tail][r*BC+b]

    const int s = blockIdx.y;
    const int k0 = s * a.ks;
    const int klen = min(a.K - k0, a.ks);
    const int NW = uniform(blockDim.x >> 6);
    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int row0 = (int)((long)a.N * blockIdx.x / gridDim.x);
    const int rows = (int)((long)a.N * (blockIdx.x + 1) / gridDim.x) - row0;
    const int C = (klen + 511) >> 9;           // 512-wide chunks per row
    const int Gb = (rows + R - 1) / R;         // row groups of this workgroup
    const int Tb = Gb * C;                     // steps of this workgroup
    const int q0 = (int)((long)Tb * wave / NW);
    const int q1 = (int)((long)Tb * (wave + 1) / NW);
    const int T = q1 - q0;                     // steps of this wave
    const bool ragged = (klen & 511) != 0;
    const int lk = lane * 8;
    const uint16_t *wblk = a.W + (size_t)row0 * a.K + k0;

    u32x4 buf[P][R];
    // Load cursor: (group, chunk) of the next step to load; it stops at the
    // wave's last step, so the ring's tail re-reads it instead of running on.
    int lt = 0, lg = q0 / C, lc = q0 - (q0 / C) * C;
    auto load_step = [&](u32x4 (&dst)[R]) {
        const int kk = min(lc * 512 + lk, klen - 8);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(lg * R + r, rows - 1);
            dst[r] = load_stream(wblk + (size_t)row * a.K + kk);
        }
        if (lt < T - 1) {
            ++lt;
            if (++lc == C) { lc = 0; ++lg; }
        }
    };
    // Weight loads go out first; x staging overlaps their latency.
    if (T > 0) {
#pragma unroll
        for (int j = 0; j < P; ++j) load_step(buf[j]);
    }

    // Stage x[0:BC][k0 : k0 + ksp] into LDS, zero past B and past the slice.
    const int vpr = a.ksp >> 3;  // 16-byte vectors per staged row
    for (int i = threadIdx.x; i < BC * vpr; i += blockDim.x) {
        const int b = i / vpr;
        const int kk = (i - b * vpr) << 3;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (b < a.B && kk < klen) v = load_cached(a.x + (size_t)b * a.ldx + k0 + kk);
        *reinterpret_cast<u32x4 *>(xs + b * a.ksp + kk) = v;
    }
    __syncthreads();

    auto store_out = [&](int row, int b, float v) {
        if (a.S == 1)
            a.y[(size_t)b * a.N + row] = to_bf16(v);
        else
            store_partial(a.ws + ((size_t)s * a.B + b) * a.N + row, v, a.cnt != nullptr);
    };

    if (T > 0) {
        float acc[R][BC];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < BC; ++b) acc[r][b] = 0.f;
        int cg = q0 / C, cc = q0 - (q0 / C) * C;  // (group, chunk) being computed
        for (int t0 = 0; t0 < T; t0 += P) {
#pragma unroll
            for (int j = 0; j < P; ++j) {
                if (t0 + j < T) {
                    u32x4 w[R];
#pragma unroll
                    for (int r = 0; r < R; ++r) w[r] = buf[j][r];
                    if (ragged && cc == C - 1) {
                        const bool dead = cc * 512 + lk >= klen;  // past the slice
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            w[r] = dead ? u32x4{0u, 0u, 0u, 0u} : w[r];
                    }
                    const int kk = cc * 512 + lk;
#pragma unroll
                    for (int b = 0; b < BC; ++b) {
                        const u32x4 xv = *reinterpret_cast<const u32x4 *>(xs + b * a.ksp + kk);
                        if constexpr (D2) {
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                float t = acc[r][b];
                                t = dot2(w[r].x, xv.x, t);
                                t = dot2(w[r].y, xv.y, t);
                                t = dot2(w[r].z, xv.z, t);
                                t = dot2(w[r].w, xv.w, t);
                                acc[r][b] = t;
                            }
                            continue;
                        }
                        const float x0 = bf_lo(xv.x), x1 = bf_hi(xv.x), x2 = bf_lo(xv.y),
                                    x3 = bf_hi(xv.y), x4 = bf_lo(xv.z), x5 = bf_hi(xv.z),
                                    x6 = bf_lo(xv.w), x7 = bf_hi(xv.w);
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float t = acc[r][b];
                            t = __builtin_fmaf(bf_lo(w[r].x), x0, t);
                            t = __builtin_fmaf(bf_hi(w[r].x), x1, t);
                            t = __builtin_fmaf(bf_lo(w[r].y), x2, t);
                            t = __builtin_fmaf(bf_hi(w[r].y), x3, t);
                            t = __builtin_fmaf(bf_lo(w[r].z), x4, t);
                            t = __builtin_fmaf(bf_hi(w[r].z), x5, t);
                            t = __builtin_fmaf(bf_lo(w[r].w), x6, t);
                            t = __builtin_fmaf(bf_hi(w[r].w), x7, t);
                            acc[r][b] = t;
                        }
                    }
                }
                load_step(buf[j]);  // refill this slot P steps ahead
                if (t0 + j < T) {
                    if (cc == C - 1 || t0 + j == T - 1) {
                        // The group ends here or the wave's run does: reduce each
                        // (row, batch) over the wave; lane r*BC + b keeps (r, b).
                        float mine = 0.f;
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int b = 0; b < BC; ++b) {
                                const float v = wave_sum(acc[r][b]);
                                if (lane == r * BC + b) mine = v;
                                acc[r][b] = 0.f;
                            }
                        const bool started_here = cg * C >= q0;
                        const int r = lane / BC, b = lane - (lane / BC) * BC;
                        if (lane < R * BC) {
                            if (cc == C - 1 && started_here) {
                                const int row = cg * R + r;
                                if (row < rows && b < a.B) store_out(row0 + row, b, mine);
                            } else {
                                part[wave][started_here ? 1 : 0][lane] = mine;
                            }
                        }
                    }
                    if (++cc == C) { cc = 0; ++cg; }
                }
            }
        }
    }

    // Groups cut by a wave boundary: add the waves' partial sums in wave order.
    __syncthreads();
    const int per = R * BC;
    const int tid = threadIdx.x;
    if (tid < (NW - 1) * per) {
        const int i = tid / per + 1;  // boundary between waves i-1 and i
        const int e = tid - (i - 1) * per;
        const int qi = (int)((long)Tb * i / NW);
        const int qp = (int)((long)Tb * (i - 1) / NW);
        const int g = qi / C;
        const bool split = qi < Tb && (qi - g * C) != 0;
        const bool seen = i > 1 && qp / C == g && (qp - (qp / C) * C) != 0;
        if (split && !seen) {
            const int wlo = wave_of_step(g * C, Tb, NW);
            const int whi = wave_of_step(g * C + C - 1, Tb, NW);
            float sum = 0.f;
            for (int v = wlo; v <= whi; ++v) {
                const int qv = (int)((long)Tb * v / NW);
                const int qv1 = (int)((long)Tb * (v + 1) / NW);
                if (qv == qv1) continue;
                sum += part[v][g * C < qv ? 0 : 1][e];
            }
            const int r = e / BC, b = e - (e / BC) * BC;
            const int row = g * R + r;
            if (row < rows && b < a.B) store_out(row0 + row, b, sum);
        }
    }
    if (a.S > 1 && a.cnt) splitk_fixup(a.ws, a.y, a.cnt, a.N, a.B, row0, rows);
}

// ---------------------------------------------------------------------------
// MFMA operand layout (v_mfma_f32_16x16x32_bf16): lane l supplies row
// (l % 16) of the A operand and column (l % 16) of the B operand, each with 8
// K values of K group (l / 16); the accumulator lane l holds rows
// 4*(l/16) + 0..3 of column l % 16.  The K order inside a group only permutes
// the sum, so a lane takes 8 consecutive K of its row.  x is the A operand
// (tiles of 16 batch rows), W the B operand (tiles of 16 output columns).
// ---------------------------------------------------------------------------
struct MfmaArgs {
    const uint16_t *x;
    long ldx;
    const uint16_t *W;
    uint16_t *y;
    float *ws;
    int *cnt;   // split-K arrival counters (fused reduction) or nullptr
    int N, K, B;
    int ks;    // K elements per slice (multiple of 32)
    int S;
    int stagger;  // 1: workgroup b starts at chunk b mod C of its slice (XS, PIPE)
};

// ---------------------------------------------------------------------------
// Shared-tile MFMA kernel (large batches).
// A workgroup of 4 waves owns rows [N*g/G, N*(g+1)/G) for one K slice and
// walks them in groups of 16*NTB rows.  For each K chunk (128 or 256 wide)
// the workgroup stages the x tile (all 16*MT batch rows) and the W tile (the
// group's rows) in LDS once, both with 256- or 512-byte row pieces,
// and every wave reads its A and B fragments from there: the waves split
// the tile WM x (4/WM), so each holds (MT/WM) x (NTB*WM/4) accumulator tiles
// and reuses each fragment across them.  The next one or two chunks are
// loaded into registers while this one is multiplied; two barriers per chunk.  LDS rows
// are padded by 16 bytes so the 16 rows of a fragment read fall in distinct
// banks.  The stagger option rotates the chunk order per workgroup as in
// mfma_pipe_kernel below.
// ---------------------------------------------------------------------------
template <int MT, int NTB, int WM, int kXsChunk, int PD>
__global__ __launch_bounds__(256) void mfma_xs_kernel(MfmaArgs a) {
    constexpr int kXsPitch = kXsChunk + 8;   // bf16 per LDS row (16 bytes of pad)
    constexpr int WN = 4 / WM;
    constexpr int MTW = MT / WM;             // A tiles per wave
    constexpr int NTW = NTB / WN;            // B tiles per wave
    constexpr int GR = 16 * NTB;             // rows per group
    constexpr int XV = MT * 16 * kXsChunk / 8 / 256;  // x vectors per thread per chunk
    constexpr int WV = GR * kXsChunk / 8 / 256;       // W vectors per thread per chunk
    static_assert((MT * 16 * kXsChunk / 8) % 256 == 0 && (GR * kXsChunk / 8) % 256 == 0,
                  "tiles must split evenly over the workgroup");
    static_assert(MT % WM == 0 && NTB % WN == 0, "tile split");
    static_assert(XV >= 1 && WV >= 1, "chunk too small for the workgroup");
    extern __shared__ __align__(16) uint16_t xs_lds[];
    uint16_t *xt = xs_lds;                               // [16*MT][kXsPitch]
    uint16_t *wt = xs_lds + MT * 16 * kXsPitch;          // [GR][kXsPitch]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int wm = wave / WN, wn = wave - (wave / WN) * WN;
    const int s = blockIdx.y;
    const int k0 = s * a.ks;
    const int klen = min(a.K - k0, a.ks);
    const int row0 = (int)((long)a.N * blockIdx.x / gridDim.x);
    const int rows = (int)((long)a.N * (blockIdx.x + 1) / gridDim.x) - row0;
    const int C = (klen + kXsChunk - 1) / kXsChunk;
    const int Gb = (rows + GR - 1) / GR;
    const int lrow = lane & 15, lgrp = lane >> 4;
    // cooperative load mapping: kXsChunk/8 lanes cover one row piece
    constexpr int LPR = kXsChunk / 8;           // lanes per row piece
    constexpr int RPS = 256 / LPR;              // rows per pass of the workgroup
    const int prow = tid / LPR;                 // row within a pass
    const int pk = (tid % LPR) * 8;             // K offset within the chunk

    auto store_out = [&](int row, int col, float v) {
        if (a.S == 1)
            a.y[(size_t)row * a.N + col] = to_bf16(v);
        else
            store_partial(a.ws + ((size_t)s * a.B + row) * a.N + col, v, a.cnt != nullptr);
    };

    // PD register sets: chunks t+1 .. t+PD are in flight while chunk t is
    // multiplied.
    u32x4 xr[PD][XV], wr[PD][WV];
    const int T = Gb * C;
    if (T == 0) return;  // uniform over the workgroup: no barrier is skipped by part of it

    // Load cursor over (group, chunk); a load past the last step reads the
    // first 16 bytes of x and of W instead (one cache line each for the whole
    // grid, never stored), so every round issues the same loads.  The offset,
    // not the base pointer, is selected: a pointer select becomes a branch.
    int lt = 0, lg = 0, lc = 0;
    const int c0 = a.stagger ? (int)(blockIdx.x % (unsigned)C) : 0;
    auto rotated = [&](int c) { return c + c0 < C ? c + c0 : c + c0 - C; };
    auto load_chunk = [&](u32x4 (&xx)[XV], u32x4 (&ww)[WV]) {
        const size_t live = lt < T ? 1 : 0;
        const int kk = min(rotated(lc) * kXsChunk + pk, klen - 8);
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int b = min(i * RPS + prow, a.B - 1);
            xx[i] = load_cached(a.x + live * ((size_t)b * a.ldx + k0 + kk));
        }
#pragma unroll
        for (int i = 0; i < WV; ++i) {
            const int r = min(lg * GR + i * RPS + prow, rows - 1);
            ww[i] = load_stream(a.W + live * ((size_t)(row0 + r) * a.K + k0 + kk));
        }
        ++lt;
        if (++lc == C) { lc = 0; ++lg; }
    };
    auto store_chunk = [&](const u32x4 (&xx)[XV], const u32x4 (&ww)[WV], int c) {
        const bool dead = c * kXsChunk + pk >= klen;   // past the slice
#pragma unroll
        for (int i = 0; i < XV; ++i)
            *reinterpret_cast<u32x4 *>(xt + (i * RPS + prow) * kXsPitch + pk) = xx[i];
#pragma unroll
        for (int i = 0; i < WV; ++i)
            *reinterpret_cast<u32x4 *>(wt + (i * RPS + prow) * kXsPitch + pk) =
                dead ? u32x4{0u, 0u, 0u, 0u} : ww[i];
    };

    f32x4 acc[MTW][NTW];
#pragma unroll
    for (int m = 0; m < MTW; ++m)
#pragma unroll
        for (int n = 0; n < NTW; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int p = 0; p < PD; ++p) load_chunk(xr[p], wr[p]);
    int g = 0, c = 0;
    for (int t0 = 0; t0 < T; t0 += PD) {
#pragma unroll
        for (int p = 0; p < PD; ++p) {
            if (t0 + p < T) {                // uniform
                __syncthreads();             // every wave is done with the previous tiles
                store_chunk(xr[p], wr[p], rotated(c));
                __syncthreads();             // tiles of this step visible
                load_chunk(xr[p], wr[p]);    // the step PD ahead into this set
                __builtin_amdgcn_sched_barrier(0);   // all loads issue before the MFMAs
#pragma unroll
                for (int j = 0; j < kXsChunk / 32; ++j) {
                    u32x4 bf[NTW];
#pragma unroll
                    for (int n = 0; n < NTW; ++n)
                        bf[n] = *reinterpret_cast<const u32x4 *>(
                            wt + ((wn * NTW + n) * 16 + lrow) * kXsPitch + j * 32 + lgrp * 8);
#pragma unroll
                    for (int m = 0; m < MTW; ++m) {
                        const u32x4 af = *reinterpret_cast<const u32x4 *>(
                            xt + ((wm * MTW + m) * 16 + lrow) * kXsPitch + j * 32 + lgrp * 8);
#pragma unroll
                        for (int n = 0; n < NTW; ++n)
                            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, af),
                                __builtin_bit_cast(bf16x8_t, bf[n]), acc[m][n], 0, 0, 0);
                    }
                }
                if (c == C - 1) {
#pragma unroll
                    for (int m = 0; m < MTW; ++m)
#pragma unroll
                        for (int n = 0; n < NTW; ++n) {
                            const int r = g * GR + (wn * NTW + n) * 16 + lrow;
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                const int b = (wm * MTW + m) * 16 + lgrp * 4 + v;
                                if (b < a.B && r < rows) store_out(b, row0 + r, acc[m][n][v]);
                            }
                            acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
                        }
                }
                if (++c == C) { c = 0; ++g; }
            }
        }
    }
    if (a.S > 1 && a.cnt) splitk_fixup(a.ws, a.y, a.cnt, a.N, a.B, row0, rows);
}

// ---------------------------------------------------------------------------
// Pipelined shared-tile MFMA kernel.
//
// Same work split as mfma_xs_kernel (a workgroup owns a row range of one K
// slice; its four or eight waves step together through (group, chunk) pairs, sharing
// the chunk's x tile [16*MT][KC] and weight tile [16*NTB][KC] in LDS), but
// the tiles are loaded straight into LDS with global_load_lds_dwordx4 into a
// ring of D stages, D-1 chunks ahead of the one being multiplied, so the
// loads in flight do not hold registers and no wave copies data into LDS.
// One barrier per chunk.
//
// Chunk order: with the stagger option workgroup b walks the chunks of its
// slice from chunk b mod C and wraps.  Without it every workgroup reads the
// same K columns at the same time, and when the row pitch is a multiple of a
// few KB those addresses share their low bits across the whole grid; spread
// over K they load the memory channels more evenly (measured on the
// 7168 x 12288 shape: the slowest workgroups finish ~2 us sooner).
//
// LDS layout of a stage: rows of KC/8 16-byte pieces, x rows first, then
// weight rows; piece p of row r sits at position p ^ q(r) of its row, with
// q(r) = r mod (KC/8) for rows of 8 or more pieces and (r >> 1) mod 4 for
// rows of 4.  Measured bank-conflict counts of 128-bit LDS reads on gfx950
// fit 64 four-byte banks served eight lanes (two groups of four) at a time;
// with this swizzle the fragment reads count zero conflicts at every chunk
// width, where a rotation p + r leaves a 2-way conflict, and no row is
// padded.  One load instruction fills 1 KB of consecutive positions (64
// lanes x 16 bytes), so each lane loads the global piece that lands in its
// position.  Pieces past the slice end load 16 zero bytes instead (they meet
// live rows, so they must add nothing); batch rows past B and weight rows
// past the workgroup's rows repeat a live row (their outputs are never
// stored).
//
// The direct-to-LDS loads are issued from inline assembly, so the compiler
// does not track them: the wait for a stage is an explicit vmcnt wait for
// all but the (D-2) younger stages' loads of this wave (vector loads return
// in order), then a barrier for the other waves' pieces.
// ---------------------------------------------------------------------------
__device__ __align__(16) uint16_t kZeroPiece[8];

// LDS byte address of a shared-memory pointer (what M0 and ds_* take).
__device__ __forceinline__ uint32_t lds_address(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from src into LDS at m0 + 16 * lane (m0 uniform).  A
// load that reads M0 right after a scalar write of it needs one wait state.
__device__ __forceinline__ void lds_load16_stream(const void *src, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(src), "s"(m0)
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_load16_cached(const void *src, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(m0)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <int MT, int NTB, int WM, int WK, int KC, int D, int NWV>
__global__ __launch_bounds__(NWV * 64) void mfma_pipe_kernel(MfmaArgs a) {
    static_assert(NWV == 4 || NWV == 8, "four or eight waves");
    static_assert(WM * WK <= NWV && NWV % (WM * WK) == 0, "wave split");
    constexpr int WN = NWV / (WM * WK);
    constexpr int MTW = MT / WM;                 // x tiles per wave
    constexpr int NTW = NTB / WN;                // weight tiles per wave
    constexpr int JW = KC / 32 / WK;             // 32-wide K steps per wave per chunk
    constexpr int XR = 16 * MT;                  // x rows per stage
    constexpr int GR = 16 * NTB;                 // weight rows per group
    constexpr int PP = KC / 8;                   // 16-byte pieces per row
    constexpr int STAGE = (XR + GR) * PP * 16;   // bytes per stage
    constexpr int NB = (XR + GR) * PP / 64;      // 1 KB load blocks per stage
    constexpr int XB = XR * PP / 64;             // of which x blocks
    constexpr int NI = NB / NWV;                 // blocks per wave per stage
    static_assert(PP == 4 || PP == 8 || PP % 16 == 0, "chunk width");
    static_assert(PP <= 64, "a row piece fits one load instruction");
    static_assert(NB % NWV == 0 && (XR * PP) % 64 == 0, "blocks split over the waves");
    static_assert(MT % WM == 0 && NTB % WN == 0, "tile split");
    static_assert(D >= 2 && NI * (D - 2) <= 63, "loads in flight");
    static_assert(JW * WK * 32 == KC, "K steps split over the waves along K");
    extern __shared__ __align__(16) uint16_t pipe_lds[];
    const char *lds = reinterpret_cast<const char *>(pipe_lds);
    const uint32_t lds0 = uniform((int)lds_address(pipe_lds));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int wk = wave / (WM * WN);             // which K steps of a chunk
    const int wmn = wave - wk * (WM * WN);
    const int wm = wmn / WN, wn = wmn - (wmn / WN) * WN;
    const int s = blockIdx.y;
    const int k0 = s * a.ks;
    const int klen = min(a.K - k0, a.ks);
    const int row0 = (int)((long)a.N * blockIdx.x / gridDim.x);
    const int rows = (int)((long)a.N * (blockIdx.x + 1) / gridDim.x) - row0;
    const int C = (klen + KC - 1) / KC;
    const int Gb = (rows + GR - 1) / GR;
    const int T = Gb * C;
    if (T == 0) return;  // uniform over the workgroup
    const int lrow = lane & 15, lgrp = lane >> 4;

    // This lane's piece of each of the wave's load blocks: stage row r and
    // piece p (its K offset within the chunk is 8 * p).
    // The swizzle is its own inverse: position v of row r holds piece v ^ q(r).
    auto swz = [](int r) { return PP == 4 ? (r >> 1) & 3 : r & (PP - 1); };
    int lr[NI], lpk[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int slot = (i * NWV + wave) * 64 + lane;
        const int r = slot / PP;
        lr[i] = r;
        lpk[i] = ((slot % PP) ^ swz(r)) * 8;
    }

    int it = 0, ig = 0, ic = 0;  // the next step to load
    const int c0 = a.stagger ? (int)(blockIdx.x % (unsigned)C) : 0;
    auto issue = [&]() {
        const uint32_t st = lds0 + (uint32_t)((it % D) * STAGE);
        const int cc = ic + c0 < C ? ic + c0 : ic + c0 - C;  // chunk loaded
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int bi = i * NWV + wave;
            const int k = cc * KC + lpk[i];
            const uint32_t m0 = st + (uint32_t)bi * 1024u;
            // Batch rows past B repeat row B-1, and weight rows past the
            // range (all of them in the ring's steps past the last one)
            // repeat the last row: they only feed outputs that are never
            // stored, and real addresses spread these loads over the memory
            // channels like the live ones (a single shared address would
            // queue them all on one).  Only pieces past the slice end must
            // be zero, since they meet live rows.
            if (bi < XB) {
                const int b = min(lr[i], a.B - 1);
                const uint16_t *src =
                    k < klen ? a.x + (size_t)b * a.ldx + k0 + k : kZeroPiece;
                lds_load16_cached(src, m0);
            } else {
                const int r = min(ig * GR + lr[i] - XR, rows - 1);
                const uint16_t *src =
                    k < klen ? a.W + (size_t)(row0 + r) * a.K + k0 + k : kZeroPiece;
                lds_load16_stream(src, m0);
            }
        }
        ++it;
        if (++ic == C) { ic = 0; ++ig; }
    };

    auto store_out = [&](int row, int col, float v) {
        if (a.S == 1)
            a.y[(size_t)row * a.N + col] = to_bf16(v);
        else
            store_partial(a.ws + ((size_t)s * a.B + row) * a.N + col, v, a.cnt != nullptr);
    };

    f32x4 acc[MTW][NTW];
#pragma unroll
    for (int m = 0; m < MTW; ++m)
#pragma unroll
        for (int n = 0; n < NTW; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int p = 0; p < D - 1; ++p) issue();
    int g = 0, c = 0;
    for (int t = 0; t < T; ++t) {
        wait_vmcnt<NI * (D - 2)>();  // this wave's pieces of step t are in LDS
        __syncthreads();             // everyone's are; stage t-1 is free
        issue();                     // step t + D - 1 into the freed stage
        const char *stg = lds + (t % D) * STAGE;
#pragma unroll
        for (int jj = 0; jj < JW; ++jj) {
            const int p = (jj * WK + wk) * 4 + lgrp;
            u32x4 bf[NTW];
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                const int r = XR + (wn * NTW + n) * 16 + lrow;
                bf[n] = *reinterpret_cast<const u32x4 *>(
                    stg + (r * PP + (p ^ swz(r))) * 16);
            }
#pragma unroll
            for (int m = 0; m < MTW; ++m) {
                const int r = (wm * MTW + m) * 16 + lrow;
                const u32x4 af = *reinterpret_cast<const u32x4 *>(
                    stg + (r * PP + (p ^ swz(r))) * 16);
#pragma unroll
                for (int n = 0; n < NTW; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, af), __builtin_bit_cast(bf16x8_t, bf[n]),
                        acc[m][n], 0, 0, 0);
            }
        }
        if (c == C - 1) {
            if constexpr (WK > 1) {
                // Waves along K leave their partial tiles after the ring;
                // the first one adds them in the fixed order wk = 1..WK-1.
                f32x4 *part = reinterpret_cast<f32x4 *>(pipe_lds + D * STAGE / 2);
                if (wk > 0) {
#pragma unroll
                    for (int m = 0; m < MTW; ++m)
#pragma unroll
                        for (int n = 0; n < NTW; ++n)
                            part[(((wk - 1) * WM * WN + wmn) * MTW * NTW + m * NTW + n) * 64 +
                                 lane] = acc[m][n];
                }
                __syncthreads();
                if (wk == 0) {
#pragma unroll
                    for (int q = 1; q < WK; ++q)
#pragma unroll
                        for (int m = 0; m < MTW; ++m)
#pragma unroll
                            for (int n = 0; n < NTW; ++n)
                                acc[m][n] += part[(((q - 1) * WM * WN + wmn) * MTW * NTW +
                                                   m * NTW + n) * 64 + lane];
                }
            }
#pragma unroll
            for (int m = 0; m < MTW; ++m)
#pragma unroll
                for (int n = 0; n < NTW; ++n) {
                    const int r = g * GR + (wn * NTW + n) * 16 + lrow;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int b = (wm * MTW + m) * 16 + lgrp * 4 + v;
                        if (wk == 0 && b < a.B && r < rows) store_out(b, row0 + r, acc[m][n][v]);
                    }
                    acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
        if (++c == C) { c = 0; ++g; }
    }
    // The ring's last loads (zeros past the end) land before the workgroup
    // ends; no wave leaves LDS writes in flight.
    wait_vmcnt<0>();
    if (a.S > 1 && a.cnt) splitk_fixup(a.ws, a.y, a.cnt, a.N, a.B, row0, rows);
}

// ---------------------------------------------------------------------------
// Fixed-order split-K reduction: y[i] = bf16( sum_{s=0}^{S-1} ws[s][i] ),
// added s = 0..S-1 starting from slice 0's value.  SC > 0: S == SC, all
// slices loaded before any is added, so the pass costs one memory round
// trip (a load-add loop waits for each slice in turn); SC == 0: any S, in
// that loop.
// ---------------------------------------------------------------------------
template <int SC>
__global__ __launch_bounds__(256) void splitk_reduce(const float *ws, uint16_t *y,
                                                     long count, int S) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    float acc;
    if constexpr (SC > 0) {
        float v[SC];
#pragma unroll
        for (int j = 0; j < SC; ++j) v[j] = __builtin_nontemporal_load(ws + (size_t)j * count + i);
        acc = v[0];
#pragma unroll
        for (int j = 1; j < SC; ++j) acc += v[j];
    } else {
        acc = ws[i];
        for (int s = 1; s < S; ++s) acc += ws[(size_t)s * count + i];
    }
    y[i] = to_bf16(acc);
}

// The same sum four outputs per thread (count % 4 == 0): one 16-byte load
// per slice and one 8-byte store, each output still added s = 0..S-1.
__device__ __forceinline__ void add4(f32x4 &acc, const f32x4 &v) {
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
}

template <int SC>
__global__ __launch_bounds__(256) void splitk_reduce4(const f32x4 *ws, uint2 *y, long count4,
                                                      int S) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count4) return;
    f32x4 acc;
    if constexpr (SC > 0) {
        f32x4 v[SC];
#pragma unroll
        for (int j = 0; j < SC; ++j)
            v[j] = __builtin_nontemporal_load(ws + (size_t)j * count4 + i);
        acc = v[0];
#pragma unroll
        for (int j = 1; j < SC; ++j) add4(acc, v[j]);
    } else {
        acc = __builtin_nontemporal_load(ws + i);
        for (int s = 1; s < S; ++s) add4(acc, __builtin_nontemporal_load(ws + (size_t)s * count4 + i));
    }
    y[i] = make_uint2((unsigned)to_bf16(acc.x) | ((unsigned)to_bf16(acc.y) << 16),
                      (unsigned)to_bf16(acc.z) | ((unsigned)to_bf16(acc.w) << 16));
}

// ---------------------------------------------------------------------------
// Streaming-read probe.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void read_probe(const u32x4 *buf, size_t n16,
                                                  float *sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    unsigned acc = 0;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(buf + i + j * stride);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0)
        sink[(blockIdx.x * blockDim.x + threadIdx.x) >> 6] = __uint_as_float(acc);
}

// ---------------------------------------------------------------------------
// Weight prefetch: read the leading bytes of a weight with ordinary (cached)
// 128-bit loads, so that they sit in the memory-side cache (MALL) and L2 when
// the projection streams them next.  Nothing is written: an empty asm that
// takes the loaded values keeps the loads alive.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefetch_kernel(const u32x4 *buf, size_t n16) {
    constexpr int U = 8;  // 128 bytes in flight per lane
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const size_t k = i + j * stride;
            v[j] = load_cached(reinterpret_cast<const uint16_t *>(buf + (k < n16 ? k : i)));
        }
#pragma unroll
        for (int j = 0; j < U; ++j) asm volatile("" ::"v"(v[j].x));
    }
}

// ---------------------------------------------------------------------------
// Stand-in for the attention core between the two projections of a layer: a
// kernel of fixed duration that touches no memory (one 64-lane wave per
// compute unit sleeping on the constant-rate clock), so HBM is idle while it
// runs.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void core_standin_kernel(unsigned long long ticks) {
    const unsigned long long t0 = wall_clock64();
    while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(32);
}

// ---------------------------------------------------------------------------
// The stand-in core and a weight prefetch in one launch: workgroups
// 0..core_blocks-1 are the stand-in (their first wave sleeps `ticks` of the
// wall clock, the others leave at once), the rest read the leading bytes of
// a weight with cached 128-bit loads as prefetch_kernel does.  The launch
// lasts as long as the longer of the two.  It models a core kernel that
// issues the next weight's prefetch itself, so no second stream, fork or
// join is needed.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void core_prefetch_kernel(unsigned long long ticks,
                                                            const u32x4 *buf, size_t n16,
                                                            unsigned core_blocks) {
    if (blockIdx.x < core_blocks) {
        if (threadIdx.x >= 64) return;
        const unsigned long long t0 = wall_clock64();
        while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(32);
        return;
    }
    constexpr int U = 8;
    const size_t nb = gridDim.x - core_blocks;
    const size_t stride = nb * blockDim.x;
    for (size_t i = (size_t)(blockIdx.x - core_blocks) * blockDim.x + threadIdx.x; i < n16;
         i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const size_t k = i + j * stride;
            v[j] = load_cached(reinterpret_cast<const uint16_t *>(buf + (k < n16 ? k : i)));
        }
#pragma unroll
        for (int j = 0; j < U; ++j) asm volatile("" ::"v"(v[j].x));
    }
}

// ---------------------------------------------------------------------------
// Host-side dispatch.
// ---------------------------------------------------------------------------
namespace {

int ceil_div_i(long a, long b) { return (int)((a + b - 1) / b); }

// Counters for the fused split-K reduction of a launch with gx workgroups
// per slice, or nullptr when the launch is not split or the plan reduces in
// a second pass (the caller then launches splitk_reduce).
int *fused_counters(const LaunchShape &sh, long gx, int S) {
    return (S > 1 && sh.cnt && gx <= kSplitCounters) ? sh.cnt : nullptr;
}

// Workgroups per K slice of a launch (gridDim.x): wpc waves (STREAM) or
// workgroups (MFMA_XS, MFMA_PIPE) per compute unit over the S slices.  At
// most one workgroup per row.
long grid_x(const LaunchShape &sh, const proj_tactic_t &t) {
    const int S = slice_count(sh.K, t);
    long g;
    if (t.kernel == PROJ_KERNEL_STREAM || t.kernel == PROJ_KERNEL_STREAM_DOT2) {
        const int nw = std::min(t.waves, kStreamMaxWaves);
        g = (long)sh.num_cus * t.wpc / (nw * (long)S);
    } else {
        g = (long)sh.num_cus * std::max(1, t.wpc) / S;
    }
    return std::max(1L, std::min(g, (long)sh.N));
}

// Weight loads in flight per lane: 16 for narrow batches, fewer when the
// accumulators of a wide batch need the registers.
constexpr int stream_ring(int BC, int R) {
    return (BC >= 8 ? 8 : (BC >= 4 ? 12 : 16)) / R > 1
               ? (BC >= 8 ? 8 : (BC >= 4 ? 12 : 16)) / R
               : 2;
}

template <int BC, int R, bool D2>
hipError_t launch_stream_inst(const LaunchShape &sh, const proj_tactic_t &t,
                              hipStream_t stream) {
    constexpr int P = stream_ring(BC, R);
    const int ks = slice_len(sh.K, t);
    const int S = slice_count(sh.K, t);
    const int ksp = ceil_div_i(ks, kStreamChunk) * kStreamChunk;
    const int nw = std::min(t.waves, kStreamMaxWaves);
    const long g = grid_x(sh, t);
    const size_t lds = (size_t)BC * ksp * 2;

    StreamArgs a{sh.x, sh.ldx, sh.W, sh.y, sh.ws, fused_counters(sh, g, S), sh.N, sh.K, sh.B,
                 ks, ksp, S};
    hipLaunchKernelGGL((stream_kernel<BC, R, P, D2>), dim3((unsigned)g, S), dim3(nw * 64), lds,
                       stream, a);
    return hipGetLastError();
}

template <int MT, int NTB, int WM, int KC, int PD>
hipError_t launch_mfma_xs_inst(const LaunchShape &sh, const proj_tactic_t &t,
                               hipStream_t stream) {
    const int ks = slice_len(sh.K, t);
    const int S = slice_count(sh.K, t);
    const long g = grid_x(sh, t);
    const size_t lds = mfma_xs_lds_bytes(t);
    MfmaArgs a{sh.x, sh.ldx, sh.W, sh.y, sh.ws, fused_counters(sh, g, S), sh.N, sh.K, sh.B,
               ks, S, t.stagger};
    hipLaunchKernelGGL((mfma_xs_kernel<MT, NTB, WM, KC, PD>), dim3((unsigned)g, S), dim3(256), lds,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_mfma_xs(const LaunchShape &sh, const proj_tactic_t &t, hipStream_t st) {
    // rows = N tiles per group (NTB); waves = waves along M (WM); kc = K
    // chunk; depth = chunks in flight
#define TP1_XS_CASE(BC, NTB, WM, KC, PD) \
    if (t.bcap == BC && t.rows == NTB && t.waves == WM && t.kc == KC && t.depth == PD) \
        return launch_mfma_xs_inst<BC / 16, NTB, WM, KC, PD>(sh, t, st);
    TP1_XS_INSTANCES(TP1_XS_CASE)
#undef TP1_XS_CASE
    return hipErrorInvalidValue;
}

template <int MT, int NTB, int WM, int WK, int KC, int D, int NWV>
hipError_t launch_mfma_pipe_inst(const LaunchShape &sh, const proj_tactic_t &t,
                                 hipStream_t stream) {
    const int ks = slice_len(sh.K, t);
    const int S = slice_count(sh.K, t);
    const long g = grid_x(sh, t);
    const size_t lds = mfma_pipe_lds_bytes(t);
    MfmaArgs a{sh.x, sh.ldx, sh.W, sh.y, sh.ws, fused_counters(sh, g, S), sh.N, sh.K, sh.B,
               ks, S, t.stagger};
    hipLaunchKernelGGL((mfma_pipe_kernel<MT, NTB, WM, WK, KC, D, NWV>), dim3((unsigned)g, S),
                       dim3(NWV * 64), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_mfma_pipe(const LaunchShape &sh, const proj_tactic_t &t, hipStream_t st) {
    // rows = N tiles per group; waves = waves along M; kw = waves along K;
    // kc = K chunk; depth = LDS stages; nw = waves per workgroup
#define TP1_PIPE_CASE(BC, NTB, WM, WK, KC, D, NWV)                                    \
    if (t.bcap == BC && t.rows == NTB && t.waves == WM && t.kw == WK && t.kc == KC && \
        t.depth == D && t.nw == NWV)                                                  \
        return launch_mfma_pipe_inst<BC / 16, NTB, WM, WK, KC, D, NWV>(sh, t, st);
    TP1_PIPE_INSTANCES(TP1_PIPE_CASE)
#undef TP1_PIPE_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_stream(const LaunchShape &sh, const proj_tactic_t &t,
                         hipStream_t st) {
    const bool d2 = t.kernel == PROJ_KERNEL_STREAM_DOT2;
#define TP1_STREAM_CASE(BC, R)                                                    \
    if (t.bcap == BC && t.rows == R)                                              \
        return d2 ? launch_stream_inst<BC, R, true>(sh, t, st)                    \
                  : launch_stream_inst<BC, R, false>(sh, t, st);
    TP1_STREAM_CASE(1, 1) TP1_STREAM_CASE(1, 2) TP1_STREAM_CASE(1, 4)
    TP1_STREAM_CASE(2, 1) TP1_STREAM_CASE(2, 2) TP1_STREAM_CASE(2, 4)
    TP1_STREAM_CASE(4, 1) TP1_STREAM_CASE(4, 2) TP1_STREAM_CASE(4, 4)
    TP1_STREAM_CASE(8, 1) TP1_STREAM_CASE(8, 2) TP1_STREAM_CASE(8, 4)
#undef TP1_STREAM_CASE
    return hipErrorInvalidValue;
}

// The split-K reduction pass of a call with S = SC slices (SC == 0: any S),
// four outputs per thread when B * N allows it (y is 16-byte aligned:
// proj_run checks it).
template <int SC>
void enqueue_reduce(const LaunchShape &sh, long count, int S, hipStream_t stream) {
    if (count % 4 == 0) {
        const long n = count / 4;
        hipLaunchKernelGGL(splitk_reduce4<SC>, dim3(ceil_div_i(n, 256)), dim3(256), 0, stream,
                           reinterpret_cast<const f32x4 *>(sh.ws),
                           reinterpret_cast<uint2 *>(sh.y), n, S);
    } else {
        hipLaunchKernelGGL(splitk_reduce<SC>, dim3(ceil_div_i(count, 256)), dim3(256), 0,
                           stream, sh.ws, sh.y, count, S);
    }
}

}  // namespace

hipError_t launch_projection(const LaunchShape &sh, const proj_tactic_t &t,
                             hipStream_t stream) {
    hipError_t e;
    if (t.kernel == PROJ_KERNEL_STREAM || t.kernel == PROJ_KERNEL_STREAM_DOT2)
        e = launch_stream(sh, t, stream);
    else if (t.kernel == PROJ_KERNEL_MFMA_XS)
        e = launch_mfma_xs(sh, t, stream);
    else if (t.kernel == PROJ_KERNEL_MFMA_PIPE)
        e = launch_mfma_pipe(sh, t, stream);
    else
        return hipErrorInvalidValue;
    if (e != hipSuccess) return e;
    const int S = slice_count(sh.K, t);
    if (S > 1 && !fused_counters(sh, grid_x(sh, t), S)) {
        const long count = (long)sh.B * sh.N;
        switch (S) {
            case 2: enqueue_reduce<2>(sh, count, S, stream); break;
            case 3: enqueue_reduce<3>(sh, count, S, stream); break;
            case 4: enqueue_reduce<4>(sh, count, S, stream); break;
            case 5: enqueue_reduce<5>(sh, count, S, stream); break;
            case 6: enqueue_reduce<6>(sh, count, S, stream); break;
            case 7: enqueue_reduce<7>(sh, count, S, stream); break;
            case 8: enqueue_reduce<8>(sh, count, S, stream); break;
            default: enqueue_reduce<0>(sh, count, S, stream); break;
        }
        e = hipGetLastError();
    }
    return e;
}

int kernel_name(const LaunchShape &sh, const proj_tactic_t &t, char *buf, size_t len) {
    if (!buf || len == 0) return -1;
    const int S = slice_count(sh.K, t);
    const bool split = S > 1 && !fused_counters(sh, grid_x(sh, t), S);
    // the reduction pass launch_projection picks
    char red[40];
    snprintf(red, sizeof red, "+splitk_reduce%s<%d>", ((long)sh.B * sh.N) % 4 == 0 ? "4" : "",
             S >= 2 && S <= 8 ? S : 0);
    int n;
    if (t.kernel == PROJ_KERNEL_STREAM || t.kernel == PROJ_KERNEL_STREAM_DOT2)
        n = snprintf(buf, len, "stream_kernel<%d, %d, %d, %s>%s", t.bcap, t.rows,
                     stream_ring(t.bcap, t.rows),
                     t.kernel == PROJ_KERNEL_STREAM_DOT2 ? "true" : "false",
                     split ? red : "");
    else if (t.kernel == PROJ_KERNEL_MFMA_XS)
        n = snprintf(buf, len, "mfma_xs_kernel<%d, %d, %d, %d, %d>%s", t.bcap / 16, t.rows,
                     t.waves, t.kc, t.depth, split ? red : "");
    else if (t.kernel == PROJ_KERNEL_MFMA_PIPE)
        n = snprintf(buf, len, "mfma_pipe_kernel<%d, %d, %d, %d, %d, %d, %d>%s", t.bcap / 16,
                     t.rows, t.waves, t.kw, t.kc, t.depth, t.nw, split ? red : "");
    else
        return -1;
    return (n < 0 || (size_t)n >= len) ? -1 : 0;
}

namespace {
// The dynamic LDS a kernel may use is what the workgroup has left beside
// its static __shared__ variables.
template <typename F>
hipError_t allow(F *fn, int bytes) {
    hipFuncAttributes fa;
    hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(fn));
    if (e != hipSuccess) return e;
    const int dyn = bytes - (int)fa.sharedSizeBytes;
    if (dyn <= 0) return hipErrorInvalidValue;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                               hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
}
}  // namespace

hipError_t allow_dynamic_lds(size_t bytes) {
    const int b = (int)bytes;
    hipError_t e = hipSuccess;
    auto keep = [&](hipError_t r) {
        if (e == hipSuccess) e = r;
    };
#define TP1_ALLOW_STREAM(BC, R)                                           \
    keep(allow(&stream_kernel<BC, R, stream_ring(BC, R), false>, b));   \
    keep(allow(&stream_kernel<BC, R, stream_ring(BC, R), true>, b));
    TP1_ALLOW_STREAM(1, 1) TP1_ALLOW_STREAM(1, 2) TP1_ALLOW_STREAM(1, 4)
    TP1_ALLOW_STREAM(2, 1) TP1_ALLOW_STREAM(2, 2) TP1_ALLOW_STREAM(2, 4)
    TP1_ALLOW_STREAM(4, 1) TP1_ALLOW_STREAM(4, 2) TP1_ALLOW_STREAM(4, 4)
    TP1_ALLOW_STREAM(8, 1) TP1_ALLOW_STREAM(8, 2) TP1_ALLOW_STREAM(8, 4)
#undef TP1_ALLOW_STREAM
#define TP1_ALLOW_XS(BC, NTB, WM, KC, PD) \
    keep(allow(&mfma_xs_kernel<BC / 16, NTB, WM, KC, PD>, b));
    TP1_XS_INSTANCES(TP1_ALLOW_XS)
#undef TP1_ALLOW_XS
#define TP1_ALLOW_PIPE(BC, NTB, WM, WK, KC, D, NWV) \
    keep(allow(&mfma_pipe_kernel<BC / 16, NTB, WM, WK, KC, D, NWV>, b));
    TP1_PIPE_INSTANCES(TP1_ALLOW_PIPE)
#undef TP1_ALLOW_PIPE
    return e;
}

hipError_t launch_prefetch(const void *buf, size_t bytes, int num_cus, hipStream_t stream) {
    if (bytes < 16) return hipSuccess;
    const int blocks = std::max(1, num_cus * 4);
    hipLaunchKernelGGL(prefetch_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4 *>(buf), bytes / 16);
    return hipGetLastError();
}

hipError_t launch_core_standin(unsigned long long ticks, int num_cus, hipStream_t stream) {
    hipLaunchKernelGGL(core_standin_kernel, dim3(std::max(1, num_cus)), dim3(64), 0, stream,
                       ticks);
    return hipGetLastError();
}

hipError_t launch_core_prefetch(unsigned long long ticks, const void *buf, size_t bytes,
                                int num_cus, hipStream_t stream) {
    const unsigned core = (unsigned)std::max(1, num_cus);
    const unsigned pf = bytes >= 16 ? core * 4u : 0u;
    hipLaunchKernelGGL(core_prefetch_kernel, dim3(core + pf), dim3(256), 0, stream, ticks,
                       reinterpret_cast<const u32x4 *>(buf), bytes / 16, core);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void *buf, size_t bytes, float *sink,
                             int waves_per_cu, int num_cus, hipStream_t stream) {
    if (waves_per_cu <= 0) waves_per_cu = 8;
    const int blocks = std::max(1, num_cus * waves_per_cu / 4);
    hipLaunchKernelGGL(read_probe, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace tp1
