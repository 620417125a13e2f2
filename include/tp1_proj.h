/*
 * tp1_proj.h -- C ABI of the TP1 decode projection on MI355X (gfx950).
 *
 * The operation is the TP1 linear of the vLLM API page
 * "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.dep", section
 * "DepProjection":
 *
 *     y[B, N] = x[B, K] . W^T          (W is N x K, row-major: nn.Linear)
 *
 * with BF16 x, W and y and FP32 accumulation (the page's opening text: the
 * stock layer's precision, FP32 accumulation and BF16 outputs, the split-K
 * summation order free).  Outputs are rounded once from the FP32 sum to the
 * nearest BF16, ties to even.
 *
 * A plan is built once per weight shape for a list of batch sizes (the
 * page's DepProjection binds a weight to a per-batch tactic table; section
 * "_bins" gives the lookup rule, section "dep_policies" the table per batch).
 * Unlike the page, the weight is passed to every run, so one plan serves
 * every layer of the same shape, and there is no second backend: every
 * planned batch runs a hand-written kernel of this library.
 *
 * All pointers to x, W and y are device pointers on the device that was
 * current when the plan was built.  All calls are host calls; proj_run only
 * enqueues work on the given stream and never synchronises.
 */
#ifndef TP1_PROJ_H
#define TP1_PROJ_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Every entry point returns one of these (0 = success). */
enum proj_status {
    PROJ_OK = 0,
    PROJ_EINVAL = -1,  /* bad argument: NULL pointer, N/K <= 0, K % 8 != 0,
                          empty / unsorted / out-of-range batch list, ...   */
    PROJ_EBATCH = -2,  /* run with B < 0 or B > the largest planned batch  */
    PROJ_EALIGN = -3,  /* x, W or y not 16-byte aligned, or ldx % 8 != 0   */
    PROJ_EHIP = -4,    /* a HIP runtime call failed (no device, launch...) */
    PROJ_ENOMEM = -5,  /* host or device allocation failed                 */
    PROJ_ENODEV = -6,  /* the plan was built host-only and cannot run      */
    PROJ_ESCRATCH = -7 /* proj_run_noalloc: the call needs more split-K
                          scratch than its static buffer holds (32 MiB)    */
};

/* Kernel families a tactic can name (values 2 and 4 named two earlier MFMA
 * kernels that no measured tactic chose; they are no longer built and a
 * tactic naming them is refused). */
enum proj_kernel {
    PROJ_KERNEL_STREAM = 1, /* split-K weight stream: VALU dot products,
                               lanes along K, wavefront reductions         */
    PROJ_KERNEL_STREAM_DOT2 = 3, /* the weight stream with v_dot2 BF16 pair
                               products: FP32 accumulation whose additions
                               are not always IEEE round-to-nearest      */
    PROJ_KERNEL_MFMA_XS = 5, /* x and W chunk tiles staged once per
                               workgroup in LDS and shared by its 4 waves
                               (bcap 16..256; rows = 16-row N tiles per
                               group; waves = waves along the batch, 1/2/4;
                               wpc = workgroups per CU, 1 or 2)          */
    PROJ_KERNEL_MFMA_PIPE = 6 /* as MFMA_XS, but the tiles are loaded
                               directly into a ring of `depth` LDS stages,
                               depth-1 chunks ahead of the multiply      */
};

/* Plan flags. */
#define PROJ_PLAN_HOST_ONLY 0x1u /* build and validate the tactic table
                                    without touching a device: the plan can
                                    be queried but proj_run returns
                                    PROJ_ENODEV                             */
#define PROJ_PLAN_SPLIT_FUSED 0x2u /* reduce split-K partials inside the
                                    producing kernel (the last workgroup of a
                                    row range to arrive sums the slices)
                                    instead of with a second kernel; both add
                                    the slices in the fixed order s = 0..S-1,
                                    so results are equal bit for bit.  Slower
                                    on MI355X as measured: every workgroup
                                    waits for its partials to reach the
                                    device-coherent level before it counts
                                    in, and the last one reads them all */

/* Limits checked by proj_plan (and proj_pack_rows). */
#define PROJ_MAX_BATCH 256       /* largest batch a plan may list          */
#define PROJ_MAX_BATCHES 64      /* longest batch list                     */
#define PROJ_MAX_PACK 64         /* most weights proj_pack_rows stacks     */

/*
 * A tactic: how one batch bin runs.  Filled in from the library's measured
 * table; for a shape it has not measured, from the nearest measured shape
 * within a factor of two (|ln(N/N')| + |ln(K/K')| <= ln 2) whose tactic is
 * valid for it, else from a default rule; or set with proj_plan_set_tactic.
 *   kernel : enum proj_kernel
 *   bcap   : batch capacity of the kernel instance (>= the bin)
 *   split  : number of K slices S; S > 1 adds a fixed-order reduction pass
 *   rows   : STREAM: W rows a wave carries per pass (1, 2 or 4)
 *            MFMA_XS, MFMA_PIPE: 16-row weight tiles per group
 *   waves  : STREAM: waves per workgroup (1..8)
 *            MFMA_XS, MFMA_PIPE: waves along the batch
 *   wpc    : STREAM: waves per compute unit the grid is sized for
 *            MFMA_XS, MFMA_PIPE: workgroups per compute unit (1 or 2)
 *   kc     : MFMA_XS, MFMA_PIPE: K chunk staged per step (32..512);
 *            0 elsewhere
 *   depth  : MFMA_XS: chunks loaded into registers ahead of the one being
 *            multiplied (1 or 2); MFMA_PIPE: LDS stages of the ring (3..12);
 *            0 elsewhere
 *   kw     : MFMA_PIPE: waves along K (1, 2 or 4): the waves of a
 *            workgroup split each chunk's K steps kw ways and add their
 *            partial tiles in LDS in a fixed order; 0 elsewhere
 *   nw     : MFMA_PIPE: waves per workgroup (4 or 8); 0 elsewhere
 *   stagger: MFMA_XS, MFMA_PIPE: 1 = workgroup b walks its slice's K chunks
 *            starting at chunk b mod C (C chunks) and wrapping, so the
 *            workgroups' reads in flight are spread over K instead of all
 *            sitting at the same column of their rows; 0 = every workgroup
 *            starts at the first chunk.  The summation order then depends
 *            on the workgroup index only, so results stay reproducible.
 *            0 elsewhere
 */
typedef struct proj_tactic {
    int kernel;
    int bcap;
    int split;
    int rows;
    int waves;
    int wpc;
    int kc;
    int depth;
    int kw;
    int nw;
    int stagger;
} proj_tactic_t;

typedef struct proj_plan_s proj_plan_t;

/*
 * proj_plan -- build a plan for an N x K weight and a list of batch sizes.
 *   N, K      : weight rows / columns; N > 0, K > 0, K % 8 == 0
 *   batches   : strictly increasing, 1 <= b <= PROJ_MAX_BATCH, length
 *               1..PROJ_MAX_BATCHES (host array, not retained)
 *   flags     : 0 or a combination of PROJ_PLAN_HOST_ONLY and
 *               PROJ_PLAN_SPLIT_FUSED
 *   out       : receives the plan (set to NULL on failure)
 * The plan owns an FP32 split-K workspace and (with PROJ_PLAN_SPLIT_FUSED)
 * 256 KiB of zeroed arrival counters, allocated with hipMalloc on the
 * current device (none for host-only plans); proj_free releases them.  The
 * first device plan built on a device also allows every kernel of the
 * library the device's LDS per workgroup (a function attribute, set once),
 * so no later launch sets one.
 * Returns PROJ_OK, PROJ_EINVAL, PROJ_ENOMEM or PROJ_EHIP.
 */
int proj_plan(int N, int K, const int *batches, int n_batches, unsigned flags,
              proj_plan_t **out);

/*
 * proj_run -- enqueue y[0:B] = x[0:B] . W^T on `stream`.
 *   B      : 0 <= B <= max(batches); B == 0 is a no-op.  1 <= B runs the
 *            tactic of the smallest planned batch >= B (the "_bins" rule).
 *   x      : BF16 [B, K] device pointer, row stride ldx elements
 *            (ldx == 0 means K; ldx >= K, ldx % 8 == 0), 16-byte aligned
 *   W      : BF16 [N, K] device pointer, contiguous rows, 16-byte aligned
 *   y      : BF16 [B, N] device pointer, contiguous (row stride N),
 *            16-byte aligned; must not overlap x or W
 *   stream : a hipStream_t of the plan's device (NULL = the default stream)
 * The current device must be the one the plan was built on (its workspace
 * lives there): otherwise PROJ_EINVAL, before any launch.
 * One plan supports one stream at a time: runs on different streams that
 * overlap in time share the plan's workspace and race.
 * proj_run only launches kernels (one, or two with a split-K pass): no
 * allocation, memset, attribute change or synchronisation, so it may be
 * recorded by stream capture into a graph, from its first call on; a
 * replay reads x and W and writes y at the captured addresses.
 * Returns PROJ_OK, PROJ_EINVAL, PROJ_EBATCH, PROJ_EALIGN, PROJ_ENODEV or
 * PROJ_EHIP (launch failure; faults inside a kernel surface at the
 * caller's next synchronisation).
 */
int proj_run(const proj_plan_t *plan, int B, const void *x, long ldx,
             const void *W, void *y, void *stream);

/*
 * proj_run_layers -- multi-layer decode streaming: enqueue, for l = 0..L-1,
 *     y_in[l] = x_l . W_in[l]^T                    (plan `in`,  N_in x K_in)
 *     y_o[l]  = y_in[l][:, 0:K_o] . W_o[l]^T       (plan `out`, N_o x K_o)
 *     x_{l+1} = y_o[l]
 * back to back on one stream, each layer with its own weights, as
 * DepAttention chains its input projection into o_proj on the vLLM API page
 * "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.dep" (section
 * "DepAttention"; here the attention core between them is replaced by a
 * fixed gather of the first K_o columns, read in place through the row
 * stride N_in, without a copy).
 *   in, out : plans with out.N == in.K and out.K <= in.N; B must be within
 *             both plans' batch ranges; in.N % 8 == 0, since o_proj reads
 *             each layer's input projection in place with row stride in.N
 *             (else PROJ_EALIGN, before any launch)
 *   x0      : BF16 [B, K_in], row stride ldx0 (0 = K_in)
 *   W_in    : host array of L device pointers to BF16 [N_in, K_in]
 *   W_o     : host array of L device pointers to BF16 [N_o, K_o]
 *   y_in    : BF16 [L, B, N_in] device buffer (every layer's input projection)
 *   y_o     : BF16 [L, B, N_o] device buffer (every layer's output)
 * Returns as proj_run; on an error no later layer is enqueued.
 */
int proj_run_layers(const proj_plan_t *in, const proj_plan_t *out, int L, int B,
                    const void *x0, long ldx0, const void *const *W_in,
                    const void *const *W_o, void *y_in, void *y_o, void *stream);

/*
 * proj_run_noalloc -- for callers that cannot allocate device memory (code
 * being captured into a graph, tight serving loops, harnesses that forbid
 * allocation): proj_run without a plan, allocating nothing.
 *   N, K, x, ldx, W, y, stream : as for proj_plan / proj_run
 *   B      : 0 <= B <= 256; the tactic is the one a plan for the batches
 *            1, 2, 4, ..., 256 would use for B (the smallest power of two
 *            >= B), chosen by the same measured table and rules
 * Split-K partial sums go to a fixed 32 MiB device array of the library
 * (one per GPU, held until the process ends) instead of a plan's workspace;
 * nothing in it needs to start at zero, since every partial is written
 * before it is read.  Every call on a GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (on different streams, or from different
 * threads) race.  The first call on a device reads its attributes and the
 * array's address and sets the kernels' LDS allowance; none of this
 * allocates.  A tactic needing more than 32 MiB of partial sums returns
 * PROJ_ESCRATCH before any launch (the measured tables stay within 30 MB).
 * Returns PROJ_OK, PROJ_EINVAL, PROJ_EBATCH, PROJ_EALIGN, PROJ_ESCRATCH or
 * PROJ_EHIP.
 */
int proj_run_noalloc(int N, int K, int B, const void *x, long ldx, const void *W, void *y,
                     void *stream);

/*
 * proj_pack_rows -- stack the rows of n weights into one weight, as the MoE
 * layer's split-K front packs the shared expert's gate_up rows and the
 * latent down-projection rows into one [shared gate_up | latent down] weight
 * (vLLM API page "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.dep":
 * its opening text and section "DepMoe", whose front weight is the packed
 * one), so that a single projection launch computes every part:
 *     dst[r0_i + r, :] = src_i[r, :],  r0_i = rows[0] + ... + rows[i-1].
 * With a plan for the packed [sum(rows), K] weight, proj_run's output
 * columns [r0_i, r0_i + rows[i]) are x . src_i^T.
 *   dst    : BF16 [sum(rows), K] device buffer, contiguous, 16-byte aligned
 *   src    : host array of n device pointers to BF16 [rows[i], K],
 *            contiguous, 16-byte aligned; none may overlap dst
 *   rows   : host array of n row counts, each >= 1
 *   n      : 1..PROJ_MAX_PACK
 *   K      : row length in elements, K > 0, K % 8 == 0
 *   stream : a hipStream_t (NULL = the default stream)
 * Enqueues n device-to-device copies on `stream` (weight preparation, done
 * once; not part of a projection call) and returns without waiting.
 * Returns PROJ_OK, PROJ_EINVAL, PROJ_EALIGN or PROJ_EHIP; on an argument
 * error nothing is enqueued.
 */
int proj_pack_rows(void *dst, const void *const *src, const int *rows, int n, int K,
                   void *stream);

/*
 * proj_prefetch -- weight prefetch, the library's counterpart of the "L2
 * weight prefetch for the specialized decode" the vLLM API page
 * "vllm.models.kimi_k3.nvidia.specialized_decode.runtime" lists among its
 * modules.  Enqueue on `stream` a kernel that reads the leading `bytes`
 * (rounded down to 16) of W with ordinary cached loads, so they sit in the
 * memory-side cache (MALL) and L2 when a projection streams W next.  It
 * writes nothing.  Meant for a second stream forked while the GPU's HBM is
 * otherwise idle (see proj_run_layers_overlap).
 *   W : device pointer, 16-byte aligned
 * Returns PROJ_OK, PROJ_EINVAL, PROJ_EALIGN or PROJ_EHIP.
 */
int proj_prefetch(const void *W, size_t bytes, void *stream);

/*
 * proj_run_layers_overlap -- proj_run_layers with the gap between a layer's
 * two projections filled as a decode step fills it: a stand-in for the
 * attention core (a kernel of `core_us` microseconds on `stream` that
 * touches no memory), and, beside it on `side_stream`, the prefetch of the
 * first `prefetch_bytes` of that layer's o_proj weight.  The fork and join
 * follow the vLLM API page "vllm.models.kimi_k3.nvidia.specialized_decode.
 * runtime.hybrid" (section "NoPrefetch": a prefetcher forked before the core
 * and joined after it): the side stream waits for the input projection,
 * prefetches, and o_proj waits for the prefetch.  Outputs are those of
 * proj_run_layers, bit for bit.
 *   core_us        : 0 .. 1e6 (0 = no stand-in)
 *   prefetch_bytes : 0 = no prefetch (side_stream unused); capped at the
 *                    o_proj weight's size
 *   side_stream    : a second stream of the same priority; or `stream`
 *                    itself, and then the prefetch runs inside the
 *                    stand-in's own launch (one kernel whose other
 *                    workgroups prefetch while the stand-in sleeps; it lasts
 *                    as long as the longer of the two), with no fork or join
 * Returns as proj_run_layers (PROJ_EINVAL for a bad core_us, or a prefetch
 * with a NULL side stream beside a non-NULL `stream`).
 */
int proj_run_layers_overlap(const proj_plan_t *in, const proj_plan_t *out, int L, int B,
                            const void *x0, long ldx0, const void *const *W_in,
                            const void *const *W_o, void *y_in, void *y_o, double core_us,
                            size_t prefetch_bytes, void *stream, void *side_stream);

/* proj_free -- release a plan and its workspace.  NULL is a no-op. */
void proj_free(proj_plan_t *plan);

/* proj_strerror -- static text for a status code. */
const char *proj_strerror(int code);

/*
 * proj_plan_tactic -- the tactic proj_run would use for batch B, and the
 * planned bin it falls in (bin may be NULL).  Returns PROJ_EBATCH when B is
 * outside 1..max(batches).
 */
int proj_plan_tactic(const proj_plan_t *plan, int B, proj_tactic_t *tactic,
                     int *bin);

/*
 * proj_plan_set_tactic -- replace the tactic of planned bin `bin` (used to
 * measure candidates).  The tactic is validated against the plan's shape
 * (PROJ_EINVAL when no kernel instance or LDS budget fits it).  When it
 * needs more split-K workspace than the plan holds, the workspace is
 * reallocated (hipFree + hipMalloc, which synchronise the device), so do not
 * call it while runs of this plan are in flight.
 */
int proj_plan_set_tactic(proj_plan_t *plan, int bin,
                         const proj_tactic_t *tactic);

/*
 * proj_plan_kernel_name -- the kernel instance(s) proj_run launches for
 * batch B, as they appear in a profiler's kernel trace, e.g.
 * "stream_kernel<1, 4, 16, false>" or
 * "mfma_pipe_kernel<4, 8, 4, 1, 128, 3, 8>+splitk_reduce4".
 * Writes a NUL-terminated string of at most len bytes into buf.
 */
int proj_plan_kernel_name(const proj_plan_t *plan, int B, char *buf, size_t len);

/* proj_plan_workspace_bytes -- bytes of device workspace the plan holds. */
size_t proj_plan_workspace_bytes(const proj_plan_t *plan);

/*
 * proj_read_probe -- measurement aid, not part of the projection: enqueue a
 * kernel that reads `bytes` (a multiple of 16) from device buffer `buf` with
 * 128-bit loads and writes one float per workgroup into `sink` (device,
 * at least 65536 floats), so the box's plain streaming-read ceiling can be
 * timed with the same loads the projection uses.  `waves_per_cu` sizes the
 * grid (0 = 8).
 */
int proj_read_probe(const void *buf, size_t bytes, float *sink,
                    int waves_per_cu, void *stream);

/*
 * proj_ring_probe -- measurement aid, not part of the projection: enqueue
 * the loads of the pipelined MFMA kernel's LDS ring alone (eight waves per
 * workgroup, a ring of `depth` stages of `rows` rows x `piece` bytes filled
 * by direct-to-LDS 128-bit loads, one wait and, with `barrier`, one
 * workgroup barrier per stage; no arithmetic), over `grid` workgroups, each
 * walking the K * 2 / piece chunks of its rows once.
 *   x       : BF16 [64, K] device buffer; with what & 1, stage rows 0..63
 *             read it with cached loads (every workgroup the same rows)
 *   w       : BF16 [grid * 64, K] device buffer (workgroup g reads rows
 *             64g..64g+63 with non-temporal loads), or [64, K] with shared_w
 *   what    : 1 = x rows only (rows 64), 2 = weight rows only (rows 64),
 *             3 = x rows then weight rows (rows 128)
 *   rows, piece, depth, barrier : one of the compiled combinations (64, 256,
 *             5, 0/1), (128, 256, 3, 1), (64, 512, 3, 0/1), (64, 1024, 2,
 *             0/1), (64, 256, 9, 1), (128, 256, 5, 1), (64, 128, 9, 1),
 *             (128, 128, 9, 1); K * 2 % piece == 0
 *   sink    : device floats, grid * 8 of them (each wave writes one)
 * Returns PROJ_OK, PROJ_EINVAL, PROJ_EALIGN or PROJ_EHIP.
 */
int proj_ring_probe(const void *x, const void *w, int K, int rows, int piece, int depth,
                    int barrier, int what, int shared_w, int grid, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TP1_PROJ_H */
