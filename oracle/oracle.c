/*
 * CPU oracle of the data-parallel update step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg load it; the product
 * never does.  It shares no code, header or table with the GPU library.
 *
 * Sources (pages this follows):
 *  [DT]  "Distributed Training: Split along the Four Axes of Data, Tensor,
 *        Pipeline, and State" (ai-knowledge-map.com).  Paragraphs cited by
 *        topic: mixed-precision state; data-parallel all-reduce; averaging
 *        formula; reduction order; worked example b=4, a=8, n=8; ZeRO
 *        equivalence; checkpoint contents (loss scaling is state).
 *  [DvT] "Data vs Tensor vs Pipeline Parallelism: When to Use Each"
 *        (abhik.ai), section "What each one splits / Data parallelism: split
 *        the batch" (16 bytes per parameter; ZeRO 16*Psi/N).
 *  Adam with bias correction (Kingma & Ba 2015) and decoupled weight decay
 *  (Loshchilov & Hutter 2019): the pages name Adam's two moments only, so the
 *  update takes these published definitions.
 *
 * Arithmetic: every computation is binary64.  A value is rounded to binary32
 * exactly where the method stores it (gradient accumulators, partial sums of
 * the replica reduction, the averaged gradient, master weights, first and
 * second moments) and to bfloat16 / binary16 where it emits the
 * low-precision parameter copy.  Build with -ffp-contract=off, no fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_SCALER_NONE = 0, OR_SCALER_STATIC = 1, OR_SCALER_DYNAMIC = 2 };

/* ------------------------------------------------------------------------ */
/* formats: binary16 and bfloat16, from their definitions                    */
/* ------------------------------------------------------------------------ */

/* 2^k for k = -25 .. 6 (hexadecimal literals: exact). */
static const double pow2_table[32] = {
    0x1p-25, 0x1p-24, 0x1p-23, 0x1p-22, 0x1p-21, 0x1p-20, 0x1p-19, 0x1p-18, 0x1p-17, 0x1p-16, 0x1p-15, 0x1p-14, 0x1p-13, 0x1p-12, 0x1p-11, 0x1p-10, 0x1p-9, 0x1p-8, 0x1p-7, 0x1p-6, 0x1p-5, 0x1p-4, 0x1p-3, 0x1p-2, 0x1p-1, 0x1p0, 0x1p1, 0x1p2, 0x1p3, 0x1p4, 0x1p5, 0x1p6};

static double pow2(int k) { return pow2_table[k + 25]; }

/* Value of a binary16 bit pattern: 1 sign, 5 exponent (bias 15), 10 fraction. */
static double f16_value(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double mag;
    if (e == 0x1F) mag = f ? NAN : INFINITY;
    else if (e == 0) mag = (double)f * pow2(-24);            /* subnormal: f * 2^-24 */
    else mag = (double)(1024 + f) * pow2(e - 25);            /* (1 + f/1024) * 2^(e-15) */
    return (1.0 - 2.0 * sign) * mag;                          /* times +1 or -1: exact */
}

/* Value of a bfloat16 bit pattern: the upper half of a binary32. */
static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return (double)x;
}

/* Round a binary64 value to a binary format with p significand bits
 * (including the implicit bit), minimum normal exponent emin and maximum
 * exponent emax, to nearest with ties to even, keeping subnormals and
 * overflowing to infinity. */
static double round_to_format(double x, int p, int emin, int emax) {
    if (isnan(x) || isinf(x) || x == 0.0) return x;
    int e;
    frexp(fabs(x), &e);                 /* |x| = f * 2^e, f in [0.5, 1): leading bit 2^(e-1) */
    int lead = e - 1;
    int q = (lead < emin ? emin : lead) - (p - 1);   /* exponent of one unit in the last place */
    double r = nearbyint(ldexp(x, -q));              /* default rounding: to nearest, ties to even */
    double y = ldexp(r, q);
    double max_finite = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(y) > max_finite) return copysign(INFINITY, x);
    return y;
}

static uint16_t f16_bits(double y) {      /* y exactly representable in binary16, or inf/nan */
    uint16_t sign = signbit(y) ? 0x8000 : 0;
    double a = fabs(y);
    if (isnan(y)) return (uint16_t)(sign | 0x7E00);
    if (isinf(y)) return (uint16_t)(sign | 0x7C00);
    if (a < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)ldexp(a, 24));
    int e;
    double f = frexp(a, &e);              /* a = f * 2^e, f in [0.5,1) -> biased exponent e - 1 + 15 */
    int frac = (int)ldexp(f * 2.0 - 1.0, 10);
    return (uint16_t)(sign | ((e - 1 + 15) << 10) | frac);
}

static uint16_t bf16_bits(double y) {     /* y exactly representable in bfloat16, or inf/nan */
    if (isnan(y)) return (uint16_t)(signbit(y) ? 0xFFC0 : 0x7FC0);
    float x = (float)y;                   /* exact */
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

static double lp_value(const void* src, int dtype, int64_t i) {
    if (dtype == OR_F32) return (double)((const float*)src)[i];
    uint16_t b = ((const uint16_t*)src)[i];
    return dtype == OR_F16 ? f16_value(b) : bf16_value(b);
}

/* Exported format helpers (pinned against library conversions in tests). */
void oracle_widen(const void* src, int dtype, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (float)lp_value(src, dtype, i);
}

void oracle_narrow(const float* src, int dtype, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) {
        double x = (double)src[i];
        if (dtype == OR_F16) out[i] = f16_bits(round_to_format(x, 11, -14, 15));
        else out[i] = bf16_bits(round_to_format(x, 8, -126, 127));
    }
}

/* ------------------------------------------------------------------------ */
/* step 1: micro-step accumulation  [DT, averaging formula: replica r sums  */
/* its own gradients over the a micro-steps into g_r; worked example: the    */
/* replicas exchange nothing until the last micro-step]                      */
/* ------------------------------------------------------------------------ */
/* acc <- g (first micro-step) or acc + g, stored in binary32. */
void oracle_accumulate(float* acc, const void* g, int gdtype, int64_t n, int first) {
    for (int64_t i = 0; i < n; ++i) {
        double gi = lp_value(g, gdtype, i);
        acc[i] = first ? (float)gi : (float)((double)acc[i] + gi);
    }
}

/* ------------------------------------------------------------------------ */
/* step 2: replica sum and average  [DT, averaging formula:                  */
/* g_bar = (sum_r g_r) / n; reduction-order paragraph: the order changes the */
/* bits, so one order is fixed here: pairwise by levels, (0+1), (2+3), ...,  */
/* an odd last term carried up unchanged; every partial sum stored in        */
/* binary32, the precision of the buffers being reduced]                     */
/* ------------------------------------------------------------------------ */
#define OR_MAX_REPLICAS 64

void oracle_reduce(float* gbar, const void* const* srcs, int src_dtype, int nrep, int64_t n) {
    double vals[OR_MAX_REPLICAS];
    if (nrep < 1 || nrep > OR_MAX_REPLICAS) return;
    for (int64_t i = 0; i < n; ++i) {
        for (int r = 0; r < nrep; ++r) vals[r] = (double)(float)lp_value(srcs[r], src_dtype, i);
        int cnt = nrep;
        while (cnt > 1) {
            int half = cnt / 2;
            for (int j = 0; j < half; ++j) vals[j] = (double)(float)(vals[2 * j] + vals[2 * j + 1]);
            if (cnt & 1) vals[half] = vals[cnt - 1];
            cnt = half + (cnt & 1);
        }
        gbar[i] = (float)(vals[0] / (double)nrep);
    }
}

/* ------------------------------------------------------------------------ */
/* step 3: global statistics of the averaged gradient: sum of squares in     */
/* binary64 and the number of non-finite entries (loss scaling is training   */
/* state [DT, checkpoint contents]; a non-finite gradient skips the update). */
/* ------------------------------------------------------------------------ */
void oracle_stats(const float* gbar, int64_t n, double* sumsq, int64_t* nonfinite) {
    double s = 0.0;
    int64_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        double x = (double)gbar[i];
        if (!isfinite(x)) ++bad;
        s += x * x;
    }
    *sumsq = s;
    *nonfinite = bad;
}

/* ------------------------------------------------------------------------ */
/* step 4: per-step scalars                                                  */
/* ------------------------------------------------------------------------ */
typedef struct {
    int64_t t;               /* applied updates */
    int64_t iter;            /* steps taken, applied or skipped */
    int64_t growth_tracker;  /* consecutive applied steps since the last scale change */
    double beta1_pow;        /* beta1^t */
    double beta2_pow;        /* beta2^t */
    double scale;            /* loss scale S the current gradients carry */
    int32_t found_inf;
    int32_t pad;
    double sumsq;            /* of the scaled averaged gradient */
    double norm;             /* L2 norm of the unscaled averaged gradient */
    double clip;             /* global-norm clip factor, 1 when off or not needed */
    double gscale;           /* clip / S: multiplies the stored averaged gradient */
} oracle_scalars;

typedef struct {
    double beta1, beta2;
    int32_t scaler_mode;
    int32_t growth_interval;
    double init_scale, backoff, growth;
} oracle_cfg;

void oracle_init(oracle_scalars* s, const oracle_cfg* c) {
    memset(s, 0, sizeof(*s));
    s->beta1_pow = 1.0;
    s->beta2_pow = 1.0;
    s->scale = c->scaler_mode == OR_SCALER_NONE ? 1.0 : c->init_scale;
    s->clip = 1.0;
}

/* norm = sqrt(sumsq) / S.  With a non-finite entry the step is skipped: only
 * the step counter moves and a dynamic scale backs off.  Otherwise clip =
 * max_norm / norm when clipping is on and norm exceeds it, t advances and the
 * bias-correction powers are multiplied once more; a dynamic scale grows after
 * growth_interval consecutive applied steps.  The scale update takes effect
 * for the next step's gradients; gscale uses the scale these gradients carry. */
void oracle_finalize(oracle_scalars* s, const oracle_cfg* c, double sumsq, int64_t nonfinite, double max_norm) {
    s->sumsq = sumsq;
    s->found_inf = nonfinite > 0;
    s->norm = sqrt(sumsq) / s->scale;
    if (s->found_inf) {
        s->clip = 1.0;
        s->gscale = 0.0;
        if (c->scaler_mode == OR_SCALER_DYNAMIC) {
            s->scale *= c->backoff;
            s->growth_tracker = 0;
        }
    } else {
        s->clip = (max_norm > 0.0 && s->norm > max_norm) ? max_norm / s->norm : 1.0;
        s->gscale = s->clip / s->scale;
        s->t += 1;
        s->beta1_pow *= c->beta1;
        s->beta2_pow *= c->beta2;
        if (c->scaler_mode == OR_SCALER_DYNAMIC) {
            s->growth_tracker += 1;
            if (s->growth_tracker == c->growth_interval) {
                s->scale *= c->growth;
                s->growth_tracker = 0;
            }
        }
    }
    s->iter += 1;
}

/* ------------------------------------------------------------------------ */
/* step 5: the update on a range of the flat space.  Mixed-precision state   */
/* [DT, mixed-precision paragraph; DvT, 16 bytes per parameter]: binary32    */
/* master w, moments m and v, a low-precision parameter p.  Every replica    */
/* applies this same update with the same g_bar [DT, data-parallel all-reduce*/
/* paragraph]; a shard applies it to its own range only, with the same       */
/* result [DT, ZeRO paragraph: sharding changes layout, not the update].     */
/*   g = g_bar * clip / S                                                    */
/*   m = beta1 m + (1 - beta1) g ; v = beta2 v + (1 - beta2) g^2             */
/*   w = w (1 - lr wd) - (lr / (1 - beta1^t)) m / (sqrt(v) / sqrt(1 - beta2^t) + eps) */
/*   p = RNE_lowp(w)                                                         */
/* A skipped step (non-finite gradient) changes nothing.                     */
/* ------------------------------------------------------------------------ */
void oracle_adamw(float* w, float* m, float* v, uint16_t* p, int pdtype, const float* gbar, int64_t n,
                  const oracle_scalars* s, double lr, double eps, double wd, double beta1, double beta2) {
    if (s->found_inf) return;
    double bc1 = 1.0 - s->beta1_pow;
    double bc2 = 1.0 - s->beta2_pow;
    for (int64_t i = 0; i < n; ++i) {
        double g = (double)gbar[i] * s->gscale;
        double mi = beta1 * (double)m[i] + (1.0 - beta1) * g;
        double vi = beta2 * (double)v[i] + (1.0 - beta2) * (g * g);
        double denom = sqrt(vi) / sqrt(bc2) + eps;
        double wi = (double)w[i] * (1.0 - lr * wd) - (lr / bc1) * (mi / denom);
        m[i] = (float)mi;
        v[i] = (float)vi;
        w[i] = (float)wi;
    }
    if (p) oracle_narrow(w, pdtype, n, p);
}
