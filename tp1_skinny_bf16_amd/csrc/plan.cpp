// plan.cpp -- host-side plan logic (no HIP): checks, bins, tactics.
//
// The bin rule is the one of the vLLM API page "vllm.models.kimi_k3.nvidia.
// specialized_decode.runtime.dep", section "_bins": a batch takes the tactic
// of the smallest table key at or above it.  The page falls back to the
// largest key (and to cuBLAS for batches without a split-K tactic); this
// library has no second backend, so a batch above the largest planned one is
// an error instead (PROJ_EBATCH), and every planned batch gets a tactic of
// its own kernels (section "dep_policies" keeps only the split-K ones).
#include "plan.hpp"

#include <algorithm>

#include "tactics_table.hpp"

namespace tp1 {

static int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

static int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

int check_plan_args(int N, int K, const int *batches, int n_batches,
                    unsigned flags) {
    if (N <= 0 || K <= 0 || (K % 8) != 0) return PROJ_EINVAL;
    if (!batches || n_batches < 1 || n_batches > PROJ_MAX_BATCHES)
        return PROJ_EINVAL;
    if (flags & ~(PROJ_PLAN_HOST_ONLY | PROJ_PLAN_SPLIT_FUSED)) return PROJ_EINVAL;
    for (int i = 0; i < n_batches; ++i) {
        if (batches[i] < 1 || batches[i] > PROJ_MAX_BATCH) return PROJ_EINVAL;
        if (i > 0 && batches[i] <= batches[i - 1]) return PROJ_EINVAL;
    }
    // Keep byte offsets far inside 64 bits (a 2^40-element weight is 2 TB).
    if ((long)N * (long)K >= (1L << 40)) return PROJ_EINVAL;
    return PROJ_OK;
}

int bin_index(const PlanCore &p, int B) {
    if (B < 1) return -1;
    for (int i = 0; i < p.nb; ++i)
        if (B <= p.batches[i]) return i;
    return -1;
}

bool tactic_instance_exists(const proj_tactic_t &t) {
    if (t.kernel == PROJ_KERNEL_STREAM || t.kernel == PROJ_KERNEL_STREAM_DOT2)
        return (t.bcap == 1 || t.bcap == 2 || t.bcap == 4 || t.bcap == 8) &&
               (t.rows == 1 || t.rows == 2 || t.rows == 4);
    if (t.kernel == PROJ_KERNEL_MFMA_XS) {
#define TP1_XS_MATCH(BC, NTB, WM, KC, PD) \
        if (t.bcap == BC && t.rows == NTB && t.waves == WM && t.kc == KC && t.depth == PD) \
            return true;
        TP1_XS_INSTANCES(TP1_XS_MATCH)
#undef TP1_XS_MATCH
        return false;
    }
    if (t.kernel == PROJ_KERNEL_MFMA_PIPE) {
#define TP1_PIPE_MATCH(BC, NTB, WM, WK, KC, D, NWV)                                      \
        if (t.bcap == BC && t.rows == NTB && t.waves == WM && t.kw == WK && t.kc == KC && \
            t.depth == D && t.nw == NWV)                                                  \
            return true;
        TP1_PIPE_INSTANCES(TP1_PIPE_MATCH)
#undef TP1_PIPE_MATCH
        return false;
    }
    return false;
}

int slice_len(int K, const proj_tactic_t &t) {
    const int S = std::max(1, t.split);
    // K granularity of a slice: one MFMA step, one shared chunk, or 8
    const int step = t.kernel == PROJ_KERNEL_MFMA_XS || t.kernel == PROJ_KERNEL_MFMA_PIPE
                         ? std::max(t.kc, 32)
                         : 8;
    int ks = ceil_div(K, S);
    ks = ceil_div(ks, step) * step;
    return std::max(ks, step);
}

int slice_count(int K, const proj_tactic_t &t) {
    return ceil_div(K, slice_len(K, t));
}

size_t stream_lds_bytes(int K, const proj_tactic_t &t) {
    const int ks = slice_len(K, t);
    const int ksp = ceil_div(ks, kStreamChunk) * kStreamChunk;
    return (size_t)t.bcap * (size_t)ksp * 2u;
}

size_t static_lds_bytes(const proj_tactic_t &t) {
    // every kernel may run the fused split-K reduction, whose flag is one
    // shared int (16 bytes with alignment); the stream kernel also keeps the
    // wave-boundary partial sums [8 waves][2][rows * bcap] floats
    size_t b = 16;
    if (t.kernel == PROJ_KERNEL_STREAM || t.kernel == PROJ_KERNEL_STREAM_DOT2)
        b += 8u * 2u * (size_t)t.rows * (size_t)t.bcap * sizeof(float);
    return b;
}

size_t dynamic_lds_bytes(int K, const proj_tactic_t &t) {
    if (t.kernel == PROJ_KERNEL_STREAM || t.kernel == PROJ_KERNEL_STREAM_DOT2)
        return stream_lds_bytes(K, t);
    if (t.kernel == PROJ_KERNEL_MFMA_XS) return mfma_xs_lds_bytes(t);
    if (t.kernel == PROJ_KERNEL_MFMA_PIPE) return mfma_pipe_lds_bytes(t);
    return 0;
}

size_t mfma_xs_lds_bytes(const proj_tactic_t &t) {
    return (size_t)(t.bcap + 16 * t.rows) * (size_t)(t.kc + 8) * 2u;
}

size_t mfma_pipe_lds_bytes(const proj_tactic_t &t) {
    const size_t ring = (size_t)t.depth * (size_t)(t.bcap + 16 * t.rows) * (size_t)t.kc * 2u;
    const size_t parts = t.kw > 1 ? (size_t)(t.kw - 1) * (size_t)(t.bcap / 16) *
                                        (size_t)t.rows * 1024u
                                  : 0;
    return ring + parts;
}


size_t tactic_workspace(int N, int K, const proj_tactic_t &t) {
    const int S = slice_count(K, t);
    if (S <= 1) return 0;
    return (size_t)S * (size_t)t.bcap * (size_t)N * sizeof(float);
}

int check_tactic(int N, int K, int bin, const proj_tactic_t &t) {
    if (N <= 0 || K <= 0 || bin < 1) return PROJ_EINVAL;
    if (!tactic_instance_exists(t)) return PROJ_EINVAL;
    if (t.bcap < bin) return PROJ_EINVAL;
    if (t.split < 1 || t.split > 64) return PROJ_EINVAL;
    if (t.waves < 1 || t.waves > kMaxWaves) return PROJ_EINVAL;
    if (t.wpc < 0 || t.wpc > 32) return PROJ_EINVAL;
    if (t.kernel == PROJ_KERNEL_STREAM || t.kernel == PROJ_KERNEL_STREAM_DOT2) {
        if (t.wpc < 1 || t.waves > 8) return PROJ_EINVAL;
    }
    if (t.kernel == PROJ_KERNEL_MFMA_XS || t.kernel == PROJ_KERNEL_MFMA_PIPE) {
        if (t.wpc < 1 || t.wpc > 2) return PROJ_EINVAL;
    } else if (t.kc != 0 || t.depth != 0) {
        return PROJ_EINVAL;
    }
    // the instance's dynamic and static LDS together fit a workgroup
    if (dynamic_lds_bytes(K, t) + static_lds_bytes(t) > kLdsBytes) return PROJ_EINVAL;
    if (t.kernel != PROJ_KERNEL_MFMA_PIPE && (t.kw != 0 || t.nw != 0)) return PROJ_EINVAL;
    if (t.stagger != 0 && t.stagger != 1) return PROJ_EINVAL;
    if (t.stagger && t.kernel != PROJ_KERNEL_MFMA_XS && t.kernel != PROJ_KERNEL_MFMA_PIPE)
        return PROJ_EINVAL;
    return PROJ_OK;
}

proj_tactic_t default_tactic(int N, int K, int bin, int num_cus) {
    // The rule the measured table follows on MI355X: the IEEE weight stream
    // for 1-2 rows, and above that the pipelined shared-tile MFMA kernel
    // with eight waves and one workgroup per compute unit, its tile growing
    // with the batch (16x64 with two waves along K up to 16 rows, then
    // 32x128, 64x128, 128x256 and 256x128) and K split so that a
    // workgroup's row range is about one weight group.
    proj_tactic_t t{};
    if (num_cus < 1) num_cus = 256;
    if (bin <= 2) {
        t.kernel = PROJ_KERNEL_STREAM;
        t.bcap = bin;
        t.rows = 4;
        t.waves = 4;
        t.wpc = 8;
        t.split = 1;
        while (stream_lds_bytes(K, t) > 80 * 1024 && t.split < 16) ++t.split;
        return t;
    }
    t.kernel = PROJ_KERNEL_MFMA_PIPE;
    t.bcap = std::max(16, next_pow2(bin));
    t.nw = 8;
    t.kw = 1;
    t.wpc = 1;
    t.depth = 3;
    switch (t.bcap) {
    case 16: t.rows = 4; t.waves = 1; t.kw = 2; t.kc = 256; break;
    case 32: t.rows = 8; t.waves = 2; t.kc = 128; break;
    case 64: t.rows = 8; t.waves = 2; t.kc = 128; break;
    case 128: t.rows = 16; t.waves = 2; t.kc = 64; break;
    default: t.rows = 8; t.waves = 4; t.kc = 64; break;
    }
    const long group = 16L * t.rows;
    const long rows_per_cu = std::max(1L, (long)N / num_cus);
    const long cap = t.bcap >= 64 ? 8 : 4;
    int S = (int)std::min(cap, std::max(1L, (group + rows_per_cu / 2) / rows_per_cu));
    while (S > 1 && (K + S - 1) / S < t.kc) --S;  // keep at least one chunk per slice
    t.split = S;
    return t;
}

proj_tactic_t choose_tactic(int N, int K, int bin, int num_cus) {
    proj_tactic_t t;
    if (lookup_measured_tactic(N, K, bin, &t) && check_tactic(N, K, bin, t) == PROJ_OK)
        return t;
    // A shape the table has not measured takes the tactic measured for the
    // nearest shape within a factor of two, if it is valid here: a tactic
    // fixes how a row range and a K slice are walked, which carries over
    // between similar shapes better than the default rule does.
    proj_tactic_t near[8];
    const int n = nearby_measured_tactics(N, K, bin, near, 8);
    for (int i = 0; i < n; ++i)
        if (check_tactic(N, K, bin, near[i]) == PROJ_OK) return near[i];
    return default_tactic(N, K, bin, num_cus);
}

void fill_tactics(PlanCore &p) {
    for (int i = 0; i < p.nb; ++i)
        p.tactics[i] = choose_tactic(p.N, p.K, p.batches[i], p.num_cus);
}

size_t plan_workspace(const PlanCore &p) {
    size_t ws = 0;
    for (int i = 0; i < p.nb; ++i)
        ws = std::max(ws, tactic_workspace(p.N, p.K, p.tactics[i]));
    return ws;
}

}  // namespace tp1
