// proj_abi.hip -- the C ABI declared in include/tp1_proj.h.
//
// proj_plan / proj_run / proj_free follow the vLLM API page
// "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.dep", section
// "DepProjection": construction binds a per-batch tactic table, and run(x,
// out) writes the projection into a caller-owned output.  Here the weight is
// passed per call (one plan serves every layer of a shape) and the batch is
// explicit because raw pointers do not carry it.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <new>

#include "../../include/tp1_proj.h"
#include "kernels.hpp"
#include "plan.hpp"

struct proj_plan_s {
    tp1::PlanCore core;
    int device = -1;
    size_t lds_limit = tp1::kLdsBytes;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    int *cnt = nullptr;  // fused split-K arrival counters (zeroed)
};

namespace {

bool aligned16(const void *p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

int alloc_workspace(proj_plan_s *p, size_t bytes) {
    if (bytes <= p->ws_bytes) return PROJ_OK;
    if (p->core.flags & PROJ_PLAN_HOST_ONLY) {
        p->ws_bytes = bytes;  // bookkeeping only
        return PROJ_OK;
    }
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return PROJ_EHIP;
    if (cur != p->device && hipSetDevice(p->device) != hipSuccess) return PROJ_EHIP;
    int rc = PROJ_OK;
    if (p->ws) {
        if (hipFree(p->ws) != hipSuccess) rc = PROJ_EHIP;  // synchronises
        p->ws = nullptr;
        p->ws_bytes = 0;
    }
    if (rc == PROJ_OK) {
        void *mem = nullptr;
        if (hipMalloc(&mem, bytes) != hipSuccess) {
            (void)hipGetLastError();
            rc = PROJ_ENOMEM;
        } else {
            p->ws = mem;
            p->ws_bytes = bytes;
        }
    }
    if (cur != p->device) (void)hipSetDevice(cur);
    return rc;
}

// Every kernel instance may use up to the device's LDS per workgroup; set
// once per device, before any launch (so no launch sets an attribute).
int prepare_device(int dev, size_t lds) {
    static std::mutex mu;
    static bool done[64] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < 64 && done[dev]) return PROJ_OK;
    if (tp1::allow_dynamic_lds(lds) != hipSuccess) {
        (void)hipGetLastError();
        return PROJ_EHIP;
    }
    if (dev >= 0 && dev < 64) done[dev] = true;
    return PROJ_OK;
}

// Split-K scratch of proj_run_noalloc: a fixed device array, one copy per
// GPU the library runs on, held until the process ends.  In host code its
// name is only a stand-in; the device address comes from
// hipGetSymbolAddress, once per device, and is the only handle used.
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

struct NoallocDevice {
    bool ready = false;
    float *scratch = nullptr;  // device address of `scratch` on this device
    int num_cus = 0;
    size_t lds_limit = tp1::kLdsBytes;
};
constexpr int kMaxDevices = 64;
NoallocDevice g_noalloc[kMaxDevices];
std::mutex g_noalloc_mu;

// First call on a device: its attributes, the kernels' LDS allowance and the
// scratch address.  Allocates nothing.
int noalloc_device(int dev, NoallocDevice **out) {
    if (dev < 0 || dev >= kMaxDevices) return PROJ_EHIP;
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    NoallocDevice &d = g_noalloc[dev];
    if (!d.ready) {
        int cus = 0, lds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess ||
            hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess) {
            (void)hipGetLastError();
            return PROJ_EHIP;
        }
        size_t limit = tp1::kLdsBytes;
        if (lds > 0 && (size_t)lds < limit) limit = (size_t)lds;
        if (prepare_device(dev, limit) != PROJ_OK) return PROJ_EHIP;
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return PROJ_EHIP;
        }
        d.scratch = static_cast<float *>(ptr);
        d.num_cus = cus > 0 ? cus : 256;
        d.lds_limit = limit;
        d.ready = true;
    }
    *out = &d;
    return PROJ_OK;
}

// The layer chain's alignment, checked before its first launch: o_proj reads
// each layer's input projection in place through row stride N_in, so N_in
// must keep rows 16-byte aligned (then every layer's slice of y_in and y_o,
// B*N_in and B*K_in elements apart, starts aligned too); and the first
// layer's operands must be aligned as proj_run requires.
int chain_alignment(const tp1::PlanCore &in, const void *x0, long ldx0, const void *y_in,
                    const void *y_o) {
    if ((in.N % 8) != 0) return PROJ_EALIGN;
    if (!aligned16(x0) || !aligned16(y_in) || !aligned16(y_o)) return PROJ_EALIGN;
    if ((ldx0 % 8) != 0) return PROJ_EALIGN;
    return PROJ_OK;
}

}  // namespace

extern "C" {

const char *proj_strerror(int code) {
    switch (code) {
        case PROJ_OK: return "success";
        case PROJ_EINVAL: return "invalid argument";
        case PROJ_EBATCH: return "batch outside the planned range";
        case PROJ_EALIGN: return "pointer or row stride misaligned (16 bytes / 8 elements)";
        case PROJ_EHIP: return "HIP runtime error";
        case PROJ_ENOMEM: return "out of memory";
        case PROJ_ENODEV: return "plan was built host-only and cannot run";
        case PROJ_ESCRATCH:
            return "the call needs more split-K scratch than the static buffer of "
                   "proj_run_noalloc holds (32 MiB)";
        default: return "unknown status";
    }
}

int proj_plan(int N, int K, const int *batches, int n_batches, unsigned flags,
              proj_plan_t **out) {
    if (!out) return PROJ_EINVAL;
    *out = nullptr;
    int rc = tp1::check_plan_args(N, K, batches, n_batches, flags);
    if (rc != PROJ_OK) return rc;
    proj_plan_s *p = new (std::nothrow) proj_plan_s;
    if (!p) return PROJ_ENOMEM;
    p->core.N = N;
    p->core.K = K;
    p->core.nb = n_batches;
    p->core.flags = flags;
    for (int i = 0; i < n_batches; ++i) p->core.batches[i] = batches[i];
    if (!(flags & PROJ_PLAN_HOST_ONLY)) {
        int dev = -1, cus = 0, lds = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) {
            (void)hipGetLastError();
            delete p;
            return PROJ_EHIP;
        }
        p->device = dev;
        p->core.num_cus = cus > 0 ? cus : 256;
        if (lds > 0 && (size_t)lds < p->lds_limit) p->lds_limit = (size_t)lds;
        if (prepare_device(dev, p->lds_limit) != PROJ_OK) {
            delete p;
            return PROJ_EHIP;
        }
    }
    if ((flags & PROJ_PLAN_SPLIT_FUSED) && !(flags & PROJ_PLAN_HOST_ONLY)) {
        // Counters of the fused split-K reduction: zero once here; every
        // reduction leaves its counter at zero again.
        void *mem = nullptr;
        const size_t bytes = (size_t)tp1::kSplitCounters * sizeof(int);
        if (hipMalloc(&mem, bytes) != hipSuccess) {
            (void)hipGetLastError();
            delete p;
            return PROJ_ENOMEM;
        }
        if (hipMemset(mem, 0, bytes) != hipSuccess) {
            (void)hipFree(mem);
            delete p;
            return PROJ_EHIP;
        }
        p->cnt = static_cast<int *>(mem);
    }
    tp1::fill_tactics(p->core);
    // A device with less LDS per workgroup than the table assumes: split K
    // further until the staged x slice fits.
    for (int i = 0; i < p->core.nb; ++i) {
        proj_tactic_t &t = p->core.tactics[i];
        while ((t.kernel == PROJ_KERNEL_STREAM || t.kernel == PROJ_KERNEL_STREAM_DOT2) &&
               t.split < 64 &&
               tp1::stream_lds_bytes(K, t) + tp1::static_lds_bytes(t) > p->lds_limit)
            ++t.split;
    }
    rc = alloc_workspace(p, tp1::plan_workspace(p->core));
    if (rc != PROJ_OK) {
        if (p->cnt) (void)hipFree(p->cnt);
        delete p;
        return rc;
    }
    *out = p;
    return PROJ_OK;
}

void proj_free(proj_plan_t *plan) {
    if (!plan) return;
    if (plan->ws && !(plan->core.flags & PROJ_PLAN_HOST_ONLY)) {
        int cur = -1;
        if (hipGetDevice(&cur) == hipSuccess && cur != plan->device)
            (void)hipSetDevice(plan->device);
        (void)hipFree(plan->ws);
        if (cur >= 0 && cur != plan->device) (void)hipSetDevice(cur);
    }
    if (plan->cnt) {
        int cur = -1;
        if (hipGetDevice(&cur) == hipSuccess && cur != plan->device)
            (void)hipSetDevice(plan->device);
        (void)hipFree(plan->cnt);
        if (cur >= 0 && cur != plan->device) (void)hipSetDevice(cur);
    }
    delete plan;
}

int proj_plan_tactic(const proj_plan_t *plan, int B, proj_tactic_t *tactic,
                     int *bin) {
    if (!plan || !tactic) return PROJ_EINVAL;
    const int i = tp1::bin_index(plan->core, B);
    if (i < 0) return PROJ_EBATCH;
    *tactic = plan->core.tactics[i];
    if (bin) *bin = plan->core.batches[i];
    return PROJ_OK;
}

int proj_plan_set_tactic(proj_plan_t *plan, int bin, const proj_tactic_t *tactic) {
    if (!plan || !tactic) return PROJ_EINVAL;
    int i = -1;
    for (int j = 0; j < plan->core.nb; ++j)
        if (plan->core.batches[j] == bin) i = j;
    if (i < 0) return PROJ_EINVAL;
    if (tp1::check_tactic(plan->core.N, plan->core.K, bin, *tactic) != PROJ_OK)
        return PROJ_EINVAL;
    if (tp1::dynamic_lds_bytes(plan->core.K, *tactic) + tp1::static_lds_bytes(*tactic) >
        plan->lds_limit)
        return PROJ_EINVAL;
    const int rc = alloc_workspace(plan, tp1::tactic_workspace(plan->core.N, plan->core.K, *tactic));
    if (rc != PROJ_OK) return rc;
    plan->core.tactics[i] = *tactic;
    return PROJ_OK;
}

int proj_plan_kernel_name(const proj_plan_t *plan, int B, char *buf, size_t len) {
    if (!plan || !buf || len == 0) return PROJ_EINVAL;
    const int i = tp1::bin_index(plan->core, B);
    if (i < 0) return PROJ_EBATCH;
    tp1::LaunchShape sh{plan->core.N, plan->core.K, B, nullptr, plan->core.K, nullptr, nullptr,
                        nullptr, plan->cnt, plan->core.num_cus};
    if (plan->core.flags & PROJ_PLAN_HOST_ONLY) {
        // no device counters; name what a device plan would launch
        static int fake;
        if (plan->core.flags & PROJ_PLAN_SPLIT_FUSED) sh.cnt = &fake;
    }
    return tp1::kernel_name(sh, plan->core.tactics[i], buf, len) == 0 ? PROJ_OK : PROJ_EINVAL;
}

size_t proj_plan_workspace_bytes(const proj_plan_t *plan) {
    return plan ? plan->ws_bytes : 0;
}

int proj_run(const proj_plan_t *plan, int B, const void *x, long ldx, const void *W,
             void *y, void *stream) {
    if (!plan) return PROJ_EINVAL;
    const tp1::PlanCore &c = plan->core;
    if (B < 0 || B > c.batches[c.nb - 1]) return PROJ_EBATCH;
    if (ldx == 0) ldx = c.K;
    if (ldx < c.K) return PROJ_EINVAL;
    if (B == 0) return PROJ_OK;
    if (!x || !W || !y) return PROJ_EINVAL;
    if (!aligned16(x) || !aligned16(W) || !aligned16(y) || (ldx % 8) != 0)
        return PROJ_EALIGN;
    // y must not overlap x or W (byte ranges).
    const uintptr_t yb = reinterpret_cast<uintptr_t>(y);
    const uintptr_t ye = yb + (uintptr_t)B * c.N * 2u;
    const uintptr_t xb = reinterpret_cast<uintptr_t>(x);
    const uintptr_t xe = xb + ((uintptr_t)(B - 1) * ldx + c.K) * 2u;
    const uintptr_t wb = reinterpret_cast<uintptr_t>(W);
    const uintptr_t we = wb + (uintptr_t)c.N * c.K * 2u;
    if ((yb < xe && xb < ye) || (yb < we && wb < ye)) return PROJ_EINVAL;
    if (c.flags & PROJ_PLAN_HOST_ONLY) return PROJ_ENODEV;
    // the workspace (and any counters) live on the plan's device: launching
    // on another would hand its kernels another GPU's memory
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != plan->device) return PROJ_EINVAL;
    const int i = tp1::bin_index(c, B);
    if (i < 0) return PROJ_EBATCH;
    const proj_tactic_t &t = c.tactics[i];
    if (tp1::tactic_workspace(c.N, c.K, t) > plan->ws_bytes) return PROJ_EINVAL;
    tp1::LaunchShape sh{c.N,
                        c.K,
                        B,
                        static_cast<const uint16_t *>(x),
                        ldx,
                        static_cast<const uint16_t *>(W),
                        static_cast<uint16_t *>(y),
                        static_cast<float *>(plan->ws),
                        plan->cnt,
                        c.num_cus};
    const hipError_t e = tp1::launch_projection(sh, t, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return PROJ_EHIP;
    return PROJ_OK;
}

int proj_run_layers(const proj_plan_t *in, const proj_plan_t *out, int L, int B,
                    const void *x0, long ldx0, const void *const *W_in,
                    const void *const *W_o, void *y_in, void *y_o, void *stream) {
    if (!in || !out || L < 0 || !W_in || !W_o) return PROJ_EINVAL;
    const tp1::PlanCore &a = in->core;
    const tp1::PlanCore &b = out->core;
    if (b.N != a.K || b.K > a.N) return PROJ_EINVAL;
    if (B < 0 || B > a.batches[a.nb - 1] || B > b.batches[b.nb - 1]) return PROJ_EBATCH;
    if (L == 0 || B == 0) return PROJ_OK;
    if (!x0 || !y_in || !y_o) return PROJ_EINVAL;
    for (int l = 0; l < L; ++l)
        if (!W_in[l] || !W_o[l]) return PROJ_EINVAL;
    const int al = chain_alignment(a, x0, ldx0, y_in, y_o);
    if (al != PROJ_OK) return al;
    const size_t in_stride = (size_t)B * a.N * 2u;   // bytes per layer
    const size_t o_stride = (size_t)B * b.N * 2u;
    const void *x = x0;
    long ldx = ldx0;
    for (int l = 0; l < L; ++l) {
        char *yi = static_cast<char *>(y_in) + l * in_stride;
        char *yo = static_cast<char *>(y_o) + l * o_stride;
        int rc = proj_run(in, B, x, ldx, W_in[l], yi, stream);
        if (rc != PROJ_OK) return rc;
        rc = proj_run(out, B, yi, a.N, W_o[l], yo, stream);
        if (rc != PROJ_OK) return rc;
        x = yo;
        ldx = b.N;
    }
    return PROJ_OK;
}

int proj_prefetch(const void *W, size_t bytes, void *stream) {
    if (bytes == 0) return PROJ_OK;
    if (!W) return PROJ_EINVAL;
    if (!aligned16(W)) return PROJ_EALIGN;
    int dev = -1, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return PROJ_EHIP;
    }
    return tp1::launch_prefetch(W, bytes, cus, static_cast<hipStream_t>(stream)) == hipSuccess
               ? PROJ_OK
               : PROJ_EHIP;
}

int proj_run_layers_overlap(const proj_plan_t *in, const proj_plan_t *out, int L, int B,
                            const void *x0, long ldx0, const void *const *W_in,
                            const void *const *W_o, void *y_in, void *y_o, double core_us,
                            size_t prefetch_bytes, void *stream, void *side_stream) {
    if (!in || !out || L < 0 || !W_in || !W_o) return PROJ_EINVAL;
    if (!(core_us >= 0.0) || core_us > 1.0e6) return PROJ_EINVAL;
    const tp1::PlanCore &a = in->core;
    const tp1::PlanCore &b = out->core;
    if (b.N != a.K || b.K > a.N) return PROJ_EINVAL;
    if (B < 0 || B > a.batches[a.nb - 1] || B > b.batches[b.nb - 1]) return PROJ_EBATCH;
    const size_t wo_bytes = (size_t)b.N * b.K * 2u;
    if (prefetch_bytes > wo_bytes) prefetch_bytes = wo_bytes;
    // side_stream == stream: the prefetch runs inside the stand-in's launch
    const bool in_launch = prefetch_bytes > 0 && side_stream == stream;
    if (prefetch_bytes > 0 && !in_launch && !side_stream) return PROJ_EINVAL;
    if (L == 0 || B == 0) return PROJ_OK;
    if (!x0 || !y_in || !y_o) return PROJ_EINVAL;
    for (int l = 0; l < L; ++l)
        if (!W_in[l] || !W_o[l]) return PROJ_EINVAL;
    const int al = chain_alignment(a, x0, ldx0, y_in, y_o);
    if (al != PROJ_OK) return al;
    if (a.flags & PROJ_PLAN_HOST_ONLY || b.flags & PROJ_PLAN_HOST_ONLY) return PROJ_ENODEV;
    int rate_khz = 0, cus = 0;
    if (hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, in->device) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, in->device) !=
            hipSuccess || rate_khz <= 0) {
        (void)hipGetLastError();
        return PROJ_EHIP;
    }
    const unsigned long long ticks = (unsigned long long)(core_us * rate_khz / 1000.0 + 0.5);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipStream_t side = static_cast<hipStream_t>(side_stream);
    const size_t in_stride = (size_t)B * a.N * 2u;
    const size_t o_stride = (size_t)B * b.N * 2u;
    const void *x = x0;
    long ldx = ldx0;
    int rc = PROJ_OK;
    hipEvent_t fork = nullptr, join = nullptr;
    const bool forked = prefetch_bytes > 0 && !in_launch;
    if (forked &&
        (hipEventCreateWithFlags(&fork, hipEventDisableTiming) != hipSuccess ||
         hipEventCreateWithFlags(&join, hipEventDisableTiming) != hipSuccess)) {
        (void)hipGetLastError();
        if (fork) (void)hipEventDestroy(fork);
        return PROJ_EHIP;
    }
    for (int l = 0; l < L && rc == PROJ_OK; ++l) {
        char *yi = static_cast<char *>(y_in) + l * in_stride;
        char *yo = static_cast<char *>(y_o) + l * o_stride;
        rc = proj_run(in, B, x, ldx, W_in[l], yi, stream);
        if (rc != PROJ_OK) break;
        if (in_launch) {
            // the stand-in core issues the prefetch itself: one launch on
            // `stream`, no second stream
            if (tp1::launch_core_prefetch(ticks, W_o[l], prefetch_bytes, cus, st) != hipSuccess) {
                rc = PROJ_EHIP;
                break;
            }
        } else if (forked) {
            // fork: the side stream starts once the input projection is done
            // (its weight stream no longer competes for HBM) and prefetches
            // the head of this layer's o_proj weight while the core runs
            if (hipEventRecord(fork, st) != hipSuccess ||
                hipStreamWaitEvent(side, fork, 0) != hipSuccess ||
                tp1::launch_prefetch(W_o[l], prefetch_bytes, cus, side) != hipSuccess ||
                hipEventRecord(join, side) != hipSuccess) {
                rc = PROJ_EHIP;
                break;
            }
        }
        if (!in_launch && ticks > 0 && tp1::launch_core_standin(ticks, cus, st) != hipSuccess) {
            rc = PROJ_EHIP;
            break;
        }
        // join: o_proj waits for the prefetch
        if (forked && hipStreamWaitEvent(st, join, 0) != hipSuccess) {
            rc = PROJ_EHIP;
            break;
        }
        rc = proj_run(out, B, yi, a.N, W_o[l], yo, stream);
        x = yo;
        ldx = b.N;
    }
    if (rc == PROJ_EHIP) (void)hipGetLastError();
    // destroying a recorded event is allowed: it is released once complete
    if (fork) (void)hipEventDestroy(fork);
    if (join) (void)hipEventDestroy(join);
    return rc;
}

int proj_run_noalloc(int N, int K, int B, const void *x, long ldx, const void *W, void *y,
                     void *stream) {
    // the batch list of the page's "_bins" rule here: powers of two to 256
    static const int kBins[] = {1, 2, 4, 8, 16, 32, 64, 128, 256};
    constexpr int kNb = (int)(sizeof(kBins) / sizeof(kBins[0]));
    if (tp1::check_plan_args(N, K, kBins, kNb, 0) != PROJ_OK) return PROJ_EINVAL;
    if (B < 0 || B > kBins[kNb - 1]) return PROJ_EBATCH;
    if (ldx == 0) ldx = K;
    if (ldx < K) return PROJ_EINVAL;
    if (B == 0) return PROJ_OK;
    if (!x || !W || !y) return PROJ_EINVAL;
    if (!aligned16(x) || !aligned16(W) || !aligned16(y) || (ldx % 8) != 0)
        return PROJ_EALIGN;
    const uintptr_t yb = reinterpret_cast<uintptr_t>(y);
    const uintptr_t ye = yb + (uintptr_t)B * N * 2u;
    const uintptr_t xb = reinterpret_cast<uintptr_t>(x);
    const uintptr_t xe = xb + ((uintptr_t)(B - 1) * ldx + K) * 2u;
    const uintptr_t wb = reinterpret_cast<uintptr_t>(W);
    const uintptr_t we = wb + (uintptr_t)N * K * 2u;
    if ((yb < xe && xb < ye) || (yb < we && wb < ye)) return PROJ_EINVAL;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return PROJ_EHIP;
    }
    NoallocDevice *d = nullptr;
    const int rc = noalloc_device(dev, &d);
    if (rc != PROJ_OK) return rc;
    int bin = 1;
    while (bin < B) bin <<= 1;
    proj_tactic_t t = tp1::choose_tactic(N, K, bin, d->num_cus);
    while ((t.kernel == PROJ_KERNEL_STREAM || t.kernel == PROJ_KERNEL_STREAM_DOT2) &&
           t.split < 64 && tp1::stream_lds_bytes(K, t) + tp1::static_lds_bytes(t) > d->lds_limit)
        ++t.split;
    if (tp1::tactic_workspace(N, K, t) > kNoallocScratchBytes) return PROJ_ESCRATCH;
    tp1::LaunchShape sh{N,
                        K,
                        B,
                        static_cast<const uint16_t *>(x),
                        ldx,
                        static_cast<const uint16_t *>(W),
                        static_cast<uint16_t *>(y),
                        d->scratch,
                        nullptr,
                        d->num_cus};
    const hipError_t e = tp1::launch_projection(sh, t, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PROJ_OK : PROJ_EHIP;
}

int proj_pack_rows(void *dst, const void *const *src, const int *rows, int n, int K,
                   void *stream) {
    if (!dst || !src || !rows || n < 1 || n > PROJ_MAX_PACK || K <= 0 || (K % 8) != 0)
        return PROJ_EINVAL;
    if (!aligned16(dst)) return PROJ_EALIGN;
    const size_t row_bytes = (size_t)K * 2u;
    size_t total = 0;
    for (int i = 0; i < n; ++i) {
        if (!src[i] || rows[i] < 1) return PROJ_EINVAL;
        if (!aligned16(src[i])) return PROJ_EALIGN;
        total += (size_t)rows[i] * row_bytes;
    }
    // no source may overlap the destination (the copies would read what
    // they have already written)
    const uintptr_t d0 = (uintptr_t)dst, d1 = d0 + total;
    for (int i = 0; i < n; ++i) {
        const uintptr_t s0 = (uintptr_t)src[i], s1 = s0 + (size_t)rows[i] * row_bytes;
        if (s0 < d1 && d0 < s1) return PROJ_EINVAL;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    char *out = static_cast<char *>(dst);
    for (int i = 0; i < n; ++i) {
        const size_t bytes = (size_t)rows[i] * row_bytes;
        if (hipMemcpyAsync(out, src[i], bytes, hipMemcpyDeviceToDevice, st) != hipSuccess) {
            (void)hipGetLastError();
            return PROJ_EHIP;
        }
        out += bytes;
    }
    return PROJ_OK;
}

int proj_read_probe(const void *buf, size_t bytes, float *sink, int waves_per_cu,
                    void *stream) {
    if (!buf || !sink || bytes == 0 || (bytes % 16) != 0) return PROJ_EINVAL;
    if (!aligned16(buf)) return PROJ_EALIGN;
    if (waves_per_cu < 0 || waves_per_cu > 32) return PROJ_EINVAL;
    int dev = -1, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return PROJ_EHIP;
    const hipError_t e = tp1::launch_read_probe(buf, bytes, sink, waves_per_cu, cus,
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PROJ_OK : PROJ_EHIP;
}

int proj_ring_probe(const void *x, const void *w, int K, int rows, int piece, int depth,
                    int barrier, int what, int shared_w, int grid, float *sink, void *stream) {
    if (!x || !w || !sink || K <= 0 || grid < 1 || grid > 65536) return PROJ_EINVAL;
    if (what < 1 || what > 3 || (what == 3) != (rows == 128)) return PROJ_EINVAL;
    if (piece <= 0 || ((long)K * 2) % piece != 0) return PROJ_EINVAL;
    if (!tp1::ring_probe_instance_exists(rows, piece, depth, barrier != 0)) return PROJ_EINVAL;
    if (!aligned16(x) || !aligned16(w) || ((long)K * 2) % 16 != 0) return PROJ_EALIGN;
    const int C = (int)((long)K * 2 / piece);
    const hipError_t e =
        tp1::launch_ring_probe(x, w, (long)K * 2, C, rows, piece, depth, barrier != 0, what,
                               shared_w ? 1 : 0, grid, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return PROJ_EHIP;
    }
    return PROJ_OK;
}

}  // extern "C"
