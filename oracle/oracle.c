/*
 * F64 reference for split-K GEMM with F32 partial slabs and a slab sum.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests/, the smoke check and the CPU
 * baseline leg of bench.py have an independent answer to compare against.
 * It shares no code, header or constant with the HIP library.
 *
 * What it computes (restated from the pages, not copied):
 *   "Aligned shared rows for pipelined NAX on CUDA", section "Contract and
 *   correctness", and "Wider consecutive-weight NAX GEMM", section "Launch
 *   contract and correctness":
 *     A is [M,K] row-major, B is [N,K] row-major, elements are F32, F16 or
 *     BF16.  Split s covers k in [s*kps, min((s+1)*kps, K)) -- every split
 *     starts below K, the splits together cover K and the last one is cut at
 *     K.  The split-K kernel writes partials[s,i,j] = sum over that k range
 *     of A[i,k]*B[j,k]; a separate accumulation pass adds the slabs into the
 *     final [M,N] output.
 *   Both pages check each result against binary64 products formed from the
 *   inputs as they are stored, i.e. after rounding to the element type (same
 *   sections).  That is what this file is: the inputs are decoded exactly
 *   from their stored bits, every product
 *   of two such values is exact in binary64 (at most 24+24 significant
 *   bits), and the products are added in ascending k with one binary64
 *   accumulator.  Beside each value it returns the sum of |products|, the
 *   scale by which an error is normalised.
 *
 * Nothing here is blocked, fused or reordered beyond that definition.  The
 * only concurrency is a split of independent output rows over threads; each
 * output element is still one ascending-k loop.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_F32 0
#define ORACLE_F16 1
#define ORACLE_BF16 2

/* ---------------------------------------------------------------- decoding */

/* IEEE binary32: reinterpret the 32 bits as a C float, widen exactly. */
double oracle_decode_f32(uint32_t bits) {
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* bfloat16 is the upper half of a binary32: shift into place, then widen. */
double oracle_decode_bf16(uint16_t bits) {
    return oracle_decode_f32((uint32_t)bits << 16);
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Decoded from the bit fields by hand so that it does not lean on any
 * half-precision support of the host compiler. */
double oracle_decode_f16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int exp = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (exp == 0) {
        mag = ldexp((double)frac, -24);            /* zero or subnormal */
    } else if (exp == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(1024 + frac), exp - 25); /* (1 + f/1024)*2^(e-15) */
    }
    return sign ? -mag : mag;
}

/* Decode n stored elements of `dtype` into binary64.  Returns 0, or -1 for an
 * unknown dtype. */
int oracle_decode(const void* src, int dtype, int64_t n, double* dst) {
    int64_t t;
    if (dtype == ORACLE_F32) {
        const uint32_t* p = (const uint32_t*)src;
        for (t = 0; t < n; ++t) dst[t] = oracle_decode_f32(p[t]);
    } else if (dtype == ORACLE_F16) {
        const uint16_t* p = (const uint16_t*)src;
        for (t = 0; t < n; ++t) dst[t] = oracle_decode_f16(p[t]);
    } else if (dtype == ORACLE_BF16) {
        const uint16_t* p = (const uint16_t*)src;
        for (t = 0; t < n; ++t) dst[t] = oracle_decode_bf16(p[t]);
    } else {
        return -1;
    }
    return 0;
}

/* ---------------------------------------------------------------- encoding */

/* Round a binary64 value to nearest, ties to even, in a binary format with
 * p significand bits (hidden bit included), minimum normal exponent emin and
 * maximum exponent emax, and return its bits (sign, exponent field, fraction
 * field; bias = emax).  Written from the IEEE-754 definition: the result is
 * the representable value nearest x, the one with an even last significand
 * bit on a tie, infinity if that nearest value would exceed the largest
 * finite one.  Subnormals are kept. */
static uint32_t encode_rne(double x, int p, int emin, int emax) {
    const uint32_t sign = signbit(x) ? 1u : 0u;
    const int ebits = (emax == 127) ? 8 : 5;
    const uint32_t sign_shift = (uint32_t)(ebits + p - 1);
    if (isnan(x)) return (sign << sign_shift) | (((1u << ebits) - 1) << (p - 1)) | (1u << (p - 2));
    double a = fabs(x);
    if (a == 0.0) return sign << sign_shift;
    if (isinf(a)) return (sign << sign_shift) | (((1u << ebits) - 1) << (p - 1));
    int e;
    frexp(a, &e);            /* a = f * 2^e, f in [0.5, 1): leading bit at 2^(e-1) */
    int lead = e - 1;
    if (lead < emin) lead = emin;           /* subnormal range: fixed quantum */
    const double q = ldexp(1.0, lead - (p - 1));
    double n = nearbyint(a / q);            /* a/q is exact: q is a power of two */
    /* A carry can lift n to 2^p: that is the next binade's smallest value. */
    if (n >= ldexp(1.0, p)) { n /= 2; lead += 1; }
    if (lead > emax) return (sign << sign_shift) | (((1u << ebits) - 1) << (p - 1));  /* inf */
    uint32_t exp_field, frac;
    if (n < ldexp(1.0, p - 1)) {            /* subnormal (lead == emin) or zero */
        exp_field = 0;
        frac = (uint32_t)n;
    } else {
        exp_field = (uint32_t)(lead + emax);
        frac = (uint32_t)(n - ldexp(1.0, p - 1));
    }
    return (sign << sign_shift) | (exp_field << (p - 1)) | frac;
}

/* Rounds n binary64 values to `dtype` (ties to even) and stores their bits:
 * uint32 for F32, uint16 for F16 and BF16.  Returns 0, or -1 for an unknown
 * dtype. */
int oracle_encode(const double* src, int dtype, int64_t n, void* dst) {
    int64_t t;
    if (dtype == ORACLE_F32) {
        uint32_t* d = (uint32_t*)dst;
        for (t = 0; t < n; ++t) d[t] = encode_rne(src[t], 24, -126, 127);
    } else if (dtype == ORACLE_F16) {
        uint16_t* d = (uint16_t*)dst;
        for (t = 0; t < n; ++t) d[t] = (uint16_t)encode_rne(src[t], 11, -14, 15);
    } else if (dtype == ORACLE_BF16) {
        uint16_t* d = (uint16_t*)dst;
        for (t = 0; t < n; ++t) d[t] = (uint16_t)encode_rne(src[t], 8, -126, 127);
    } else {
        return -1;
    }
    return 0;
}

/* ------------------------------------------------------------ split bounds */

/* Bounds of split s: [k0, k1) with k1 clamped to K (same sections as above). */
static void split_bounds(int64_t s, int64_t kps, int64_t K, int64_t* k0, int64_t* k1) {
    int64_t lo = s * kps;
    int64_t hi = lo + kps;
    if (hi > K) hi = K;
    *k0 = lo;
    *k1 = hi;
}

/* One dot product over k in [k0,k1), ascending, plus the sum of |terms|. */
static void dot_range(const double* arow, const double* brow, int64_t k0, int64_t k1,
                      double* sum, double* abs_sum) {
    double acc = 0.0, mag = 0.0;
    for (int64_t k = k0; k < k1; ++k) {
        double p = arow[k] * brow[k];
        acc += p;
        mag += fabs(p);
    }
    *sum = acc;
    *abs_sum = mag;
}

/* ------------------------------------------------------------- threading */

typedef struct {
    const double* a;
    const double* b;
    const float* slabs;
    int64_t M, N, K, kps, splits;
    double* out;
    double* out_abs;
    int64_t row_begin, row_end; /* rows of the (split, i) or (i) space */
    int kind;
} job_t;

enum { JOB_PARTIALS = 0, JOB_FULL = 1, JOB_SLAB_SUM = 2 };

static void* run_job(void* arg) {
    job_t* j = (job_t*)arg;
    for (int64_t r = j->row_begin; r < j->row_end; ++r) {
        if (j->kind == JOB_PARTIALS) {
            /* r enumerates (s, i) with s major, matching partials[s, i, :]. */
            int64_t s = r / j->M, i = r % j->M, k0, k1;
            split_bounds(s, j->kps, j->K, &k0, &k1);
            for (int64_t n = 0; n < j->N; ++n) {
                double v, m;
                dot_range(j->a + i * j->K, j->b + n * j->K, k0, k1, &v, &m);
                j->out[r * j->N + n] = v;
                j->out_abs[r * j->N + n] = m;
            }
        } else if (j->kind == JOB_FULL) {
            for (int64_t n = 0; n < j->N; ++n) {
                double v, m;
                dot_range(j->a + r * j->K, j->b + n * j->K, 0, j->K, &v, &m);
                j->out[r * j->N + n] = v;
                j->out_abs[r * j->N + n] = m;
            }
        } else {
            /* Sum of F32 slabs in binary64, ascending s. */
            int64_t MN = j->M * j->N;
            for (int64_t n = 0; n < j->N; ++n) {
                double acc = 0.0, mag = 0.0;
                for (int64_t s = 0; s < j->splits; ++s) {
                    double v = (double)j->slabs[s * MN + r * j->N + n];
                    acc += v;
                    mag += fabs(v);
                }
                j->out[r * j->N + n] = acc;
                j->out_abs[r * j->N + n] = mag;
            }
        }
    }
    return NULL;
}

/* Number of worker threads actually used for `rows` rows. */
static int pick_threads(int requested, int64_t rows) {
    long hw = sysconf(_SC_NPROCESSORS_ONLN);
    int n = requested > 0 ? requested : (hw > 0 ? (int)hw : 1);
    if (n > 256) n = 256;
    if ((int64_t)n > rows) n = rows > 0 ? (int)rows : 1;
    return n;
}

static int run_rows(job_t proto, int64_t rows, int nthreads) {
    int n = pick_threads(nthreads, rows);
    pthread_t tid[256];
    int spawned[256];
    job_t jobs[256];
    for (int t = 0; t < n; ++t) {
        jobs[t] = proto;
        jobs[t].row_begin = rows * t / n;
        jobs[t].row_end = rows * (t + 1) / n;
        spawned[t] = 0;
        if (n > 1 && pthread_create(&tid[t], NULL, run_job, &jobs[t]) == 0)
            spawned[t] = 1;
        else
            run_job(&jobs[t]); /* single thread, or could not spawn: run here */
    }
    for (int t = 0; t < n; ++t)
        if (spawned[t]) pthread_join(tid[t], NULL);
    return n;
}

/* ------------------------------------------------------------ public calls */

/* Threads used by a call with `nthreads` (0 = all online cores) over `rows`. */
int oracle_threads(int nthreads, int64_t rows) { return pick_threads(nthreads, rows); }

/*
 * Partial slabs.  a: [M,K], b: [N,K] (binary64, already decoded).
 * P, DP: [splits, M, N].  Returns the number of threads used, or -1 if the
 * split geometry is not the one the pages allow (some split starting at or
 * past K, or the splits not covering K).
 */
int oracle_splitk_partials(const double* a, const double* b, int64_t M, int64_t N, int64_t K,
                           int64_t kps, int64_t splits, double* P, double* DP, int nthreads) {
    if (M <= 0 || N <= 0 || K <= 0 || kps <= 0 || splits <= 0) return -1;
    if ((splits - 1) * kps >= K || splits * kps < K) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.a = a; j.b = b; j.M = M; j.N = N; j.K = K; j.kps = kps; j.splits = splits;
    j.out = P; j.out_abs = DP; j.kind = JOB_PARTIALS;
    return run_rows(j, splits * M, nthreads);
}

/* Unsplit product C[i,j] = sum over all k of a[i,k]*b[j,k], computed on its
 * own (not from the partials), with DC the sum of |terms|. */
int oracle_gemm_bt(const double* a, const double* b, int64_t M, int64_t N, int64_t K,
                   double* C, double* DC, int nthreads) {
    if (M <= 0 || N <= 0 || K <= 0) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.a = a; j.b = b; j.M = M; j.N = N; j.K = K; j.kps = K; j.splits = 1;
    j.out = C; j.out_abs = DC; j.kind = JOB_FULL;
    return run_rows(j, M, nthreads);
}

/* The accumulation pass: out[i,j] = sum over s of slabs[s,i,j] (F32 slabs,
 * binary64 sum, ascending s), with D the sum of |slab values|. */
int oracle_slab_sum(const float* slabs, int64_t splits, int64_t M, int64_t N,
                    double* out, double* D, int nthreads) {
    if (M <= 0 || N <= 0 || splits <= 0) return -1;
    job_t j;
    memset(&j, 0, sizeof j);
    j.slabs = slabs; j.M = M; j.N = N; j.splits = splits;
    j.out = out; j.out_abs = D; j.kind = JOB_SLAB_SUM;
    return run_rows(j, M, nthreads);
}

/*
 * Sampled outputs, for sizes where the full reference is too slow.  For each
 * of the n (row, col) pairs it returns the split partials P[t, s], their
 * scales DP[t, s] (t-major, `splits` per sample), and the unsplit value and
 * scale C[t], DC[t].  Same arithmetic as the full calls above.
 */
int oracle_sampled(const double* a, const double* b, int64_t M, int64_t N, int64_t K,
                   int64_t kps, int64_t splits, const int64_t* rows, const int64_t* cols,
                   int64_t n, double* P, double* DP, double* C, double* DC) {
    if (M <= 0 || N <= 0 || K <= 0 || kps <= 0 || splits <= 0) return -1;
    if ((splits - 1) * kps >= K || splits * kps < K) return -1;
    for (int64_t t = 0; t < n; ++t) {
        int64_t i = rows[t], c = cols[t];
        if (i < 0 || i >= M || c < 0 || c >= N) return -2;
        for (int64_t s = 0; s < splits; ++s) {
            int64_t k0, k1;
            split_bounds(s, kps, K, &k0, &k1);
            dot_range(a + i * K, b + c * K, k0, k1, &P[t * splits + s], &DP[t * splits + s]);
        }
        dot_range(a + i * K, b + c * K, 0, K, &C[t], &DC[t]);
    }
    return 0;
}
