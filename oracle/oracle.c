/*
 * oracle.c -- plain, slow CPU oracle for the TP1 decode projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header or table
 * with the GPU path.
 *
 * What it computes (vLLM API page "vllm.models.kimi_k3.nvidia.specialized_
 * decode.runtime.dep", section "DepProjection"): the TP1 linear's result is
 * the stock linear's FP32-accumulated BF16 GEMM of the rows x against the
 * weight's transpose, y[B,N] = x[B,K] . W^T with W stored N x K row-major.
 * The opening text of the same page fixes the precision: BF16 inputs, FP32
 * accumulation, BF16 outputs, with the split-K summation order left free.
 * A kernel's only freedom is therefore the order and rounding of its FP32
 * partial sums; the oracle removes both by
 *   1. decoding every BF16 of x and W exactly to double,
 *   2. summing x[b,k]*W[n,k] for k = 0..K-1 in ascending k into one double
 *      (each BF16*BF16 product has at most 16 significant bits, so it is
 *      exact in double; only the running sum rounds, at 2^-53 relative),
 *   3. rounding that double sum once, directly, to the nearest BF16 with
 *      ties to even (no detour through float, which would round twice).
 * Threads split the output elements; every sum stays sequential, so the
 * result does not depend on the thread count.
 *
 * Pins (tests that tie this code to something other than itself):
 *   exact-rational brute force on tiny shapes (bitwise), identity and
 *   one-hot weights at full shapes (bitwise), closed-form constant inputs,
 *   hand-derived round-to-nearest-even ties (tests/golden), scaling /
 *   negation / permutation / linearity invariants, and numpy float64
 *   products rounded by an independent bit-level rounder.  The unrounded
 *   sums S are pinned on their own against exact rational sums (within the
 *   double-accumulation error bound) and against numpy float64 products.
 *
 * Build: gcc -O2 -fno-fast-math -shared -fPIC -pthread (oracle/build.py).
 * Defining ORACLE_MUTANT=<n> plants one deliberate mistake (used only by the
 * test that shows the pins catch plausible mistakes); the default build has
 * none.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* BF16 bit pattern -> double, exactly: a BF16 is the top half of an IEEE
 * binary32, so widening the bits and reinterpreting is exact. */
static double bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> BF16 bit pattern, round to nearest, ties to even, in one step.
 * BF16 keeps 8 significant bits (7 stored) with the binary32 exponent range:
 * normal quantum 2^(e-7) for 2^e <= |s| < 2^(e+1), e >= -126, and the fixed
 * subnormal quantum 2^-133 below 2^-126.  rint() in the default rounding mode
 * rounds half to even, and |s|/q is an exact division by a power of two. */
static uint16_t double_to_bf16(double s)
{
    if (isnan(s))
        return 0x7FC0;
#if ORACLE_MUTANT == 7
    s = (double)(float)s;         /* planted: rounds twice, via float */
#endif
    uint16_t sign = signbit(s) ? 0x8000 : 0x0000;
    double a = fabs(s);
    if (a == 0.0)
        return sign;
    int e2;
    (void)frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) */
    int e = e2 - 1;               /* floor(log2 a) */
    if (e < -126)
        e = -126;
    double q = ldexp(1.0, e - 7);
#if ORACLE_MUTANT == 3
    double n = trunc(a / q);      /* planted: truncation instead of RNE */
#elif ORACLE_MUTANT == 4
    double n = floor(a / q + 0.5);/* planted: ties away from zero */
#else
    double n = rint(a / q);
#endif
    double v = n * q;
    if (v >= 0x1p128)             /* beyond the largest finite BF16 */
        return sign | 0x7F80;
    float f = (float)v;           /* exact: v has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

typedef struct {
    int B, N, K;
    const uint16_t *x;  long ldx;
    const uint16_t *W;  long ldw;
    uint16_t *y;        long ldy;
    double *S;          long lds;
    const double *xd;   /* x decoded to double, [B][K] */
    long begin, end;    /* flat output range [begin, end) over n*B + b */
} job_t;

static void *worker(void *arg)
{
    const job_t *j = (const job_t *)arg;
    for (long t = j->begin; t < j->end; ++t) {
        int n = (int)(t / j->B);
        int b = (int)(t % j->B);
        const double *xr = j->xd + (long)b * j->K;
        const uint16_t *wr = j->W + (long)n * j->ldw;
        double s = 0.0;
#if ORACLE_MUTANT == 1
        for (int k = 0; k < j->K - 1; ++k)   /* planted: drops the last term */
            s += xr[k] * bf16_to_double(wr[k]);
#elif ORACLE_MUTANT == 2
        for (int k = 0; k < j->K; ++k)       /* planted: wrong weight index */
            s += xr[k] * bf16_to_double(wr[(k + 1) % j->K]);
#elif ORACLE_MUTANT == 5
        for (int k = 0; k < j->K; ++k) {     /* planted: float accumulator */
            float sf = (float)s;
            sf += (float)(xr[k] * bf16_to_double(wr[k]));
            s = sf;
        }
#elif ORACLE_MUTANT == 6
        for (int k = 0; k < j->K; ++k)       /* planted: x row index off */
            s += j->xd[(long)((b + 1) % j->B) * j->K + k] * bf16_to_double(wr[k]);
#else
        for (int k = 0; k < j->K; ++k)
            s += xr[k] * bf16_to_double(wr[k]);
#endif
        j->y[(long)b * j->ldy + n] = double_to_bf16(s);
#if ORACLE_MUTANT == 8
        if (j->S)                            /* planted: S stored transposed */
            j->S[(long)n * j->B + b] = s;
#else
        if (j->S)
            j->S[(long)b * j->lds + n] = s;
#endif
    }
    return NULL;
}

/*
 * oracle_proj -- y[b,n] = RNE_bf16( sum_k x[b,k] * W[n,k] ), sum in double.
 *   x: BF16 bits, B rows of K, row stride ldx elements
 *   W: BF16 bits, N rows of K, row stride ldw elements (nn.Linear layout)
 *   y: BF16 bits out, B rows of N, row stride ldy elements
 *   S: optional (NULL) double out, the unrounded sums, row stride lds
 *   threads: worker threads (<= 0 means 1)
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int oracle_proj(int B, int N, int K,
                const uint16_t *x, long ldx,
                const uint16_t *W, long ldw,
                uint16_t *y, long ldy,
                double *S, long lds,
                int threads)
{
    if (B < 0 || N < 0 || K < 0 || (B > 0 && N > 0 && (!x || !W || !y)))
        return -1;
    if (ldx < K || ldw < K || ldy < N || (S && lds < N))
        return -1;
    if (B == 0 || N == 0)
        return 0;
    double *xd = (double *)malloc(sizeof(double) * (size_t)B * (size_t)(K > 0 ? K : 1));
    if (!xd)
        return -1;
    for (int b = 0; b < B; ++b)
        for (int k = 0; k < K; ++k)
            xd[(long)b * K + k] = bf16_to_double(x[(long)b * ldx + k]);

    if (threads <= 0)
        threads = 1;
    long total = (long)B * N;
    if (threads > total)
        threads = (int)total;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)threads);
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)threads);
    if (!tid || !jobs) {
        free(xd); free(tid); free(jobs);
        return -1;
    }
    int started = 0;
    for (int i = 0; i < threads; ++i) {
        job_t *j = &jobs[i];
        j->B = B; j->N = N; j->K = K;
        j->x = x; j->ldx = ldx; j->W = W; j->ldw = ldw;
        j->y = y; j->ldy = ldy; j->S = S; j->lds = lds;
        j->xd = xd;
        j->begin = total * i / threads;
        j->end = total * (i + 1) / threads;
        if (threads == 1) {
            worker(j);
        } else if (pthread_create(&tid[i], NULL, worker, j) == 0) {
            ++started;
        } else {
            worker(j);          /* could not start a thread: do it inline */
            tid[i] = (pthread_t)0;
        }
    }
    if (threads > 1)
        for (int i = 0; i < threads; ++i)
            if (tid[i] != (pthread_t)0)
                pthread_join(tid[i], NULL);
    (void)started;
    free(tid); free(jobs); free(xd);
    return 0;
}

/* Element-wise BF16 rounding of doubles, exposed so the tests can pin the
 * rounding step on its own (hand-made ties, overflow, subnormals). */
void oracle_round_bf16(const double *s, uint16_t *out, long count)
{
    for (long i = 0; i < count; ++i)
        out[i] = double_to_bf16(s[i]);
}

int oracle_mutant(void) { return ORACLE_MUTANT; }
