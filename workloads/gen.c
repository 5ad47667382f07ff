/*
 * Seeded, counter-based synthetic input generator for the sigmoid-routed MoE layer.
 *
 * This module holds no arithmetic of the layer itself: it only turns (seed, tensor id, element index)
 * into input values. Both the HIP path's harness (bench, GPU tests) and the CPU oracle's harness read
 * their inputs from here, so the two sides see identical bytes.
 *
 * Generator definition (every value is a pure function of its coordinates, so any slice can be made
 * alone and in any order, by any number of threads):
 *   key(seed, tensor)  = mix64(seed * GOLDEN + tensor)
 *   word(ctr)          = mix64(key + (ctr + 1) * GOLDEN)
 *   mix64              = the splitmix64 output function (Steele, Lea and Flood, OOPSLA 2014).
 *
 * Normal samples use inverse-transform sampling on a 16-bit uniform: element i takes 16-bit lane (i & 3)
 * of word(i >> 2) as u in [0, 65536) and returns sigma * PhiInv((u + 0.5) / 65536), where PhiInv is the
 * standard normal quantile, found here by bisection on Phi(x) = erfc(-x / sqrt 2) / 2 from libm. The
 * table reaches +-4.32 sigma. bf16 results are rounded once, to nearest-even, from the double value.
 *
 * Uniform samples use the top 53 bits of word(i): u = (w >> 11) * 2^-53, value = lo + (hi - lo) * u,
 * rounded once to fp32.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t key_of(uint64_t seed, uint64_t tensor) { return mix64(seed * GOLDEN + tensor); }
static inline uint64_t word_of(uint64_t key, uint64_t ctr) { return mix64(key + (ctr + 1) * GOLDEN); }

/* Round a double to bf16, nearest-even, in one step (no double rounding through fp32).
 * Handles zero, normal and subnormal bf16 results; inputs here are finite. */
uint16_t gen_bf16_from_double(double v) {
    uint64_t b;
    memcpy(&b, &v, 8);
    uint16_t sign = (uint16_t)((b >> 63) << 15);
    double a = fabs(v);
    if (a == 0.0) return sign;
    int ex;
    double m = frexp(a, &ex); /* a = m * 2^ex, m in [0.5, 1) */
    /* bf16 normal: value = 1.f * 2^(E-127), E in [1, 254]; here a = (2m) * 2^(ex-1). */
    int e = ex - 1 + 127;
    double q; /* significand scaled to an integer grid of the result's precision */
    int sub = 0;
    if (e >= 1) {
        q = ldexp(m, 8); /* 8 significant bits: [128, 256) */
    } else {
        /* subnormal: grid of 2^-133 */
        q = ldexp(a, 133);
        sub = 1;
    }
    double fl = floor(q);
    double rem = q - fl;
    uint32_t n = (uint32_t)fl;
    if (rem > 0.5 || (rem == 0.5 && (n & 1u))) n++;
    if (sub) {
        /* n counts units of 2^-133; n == 128 rolls into the smallest normal, which is the same bits */
        return (uint16_t)(sign | n);
    }
    if (n == 256u) { n = 128u; e++; }
    if (e >= 255) return (uint16_t)(sign | 0x7F80u); /* overflow to inf (not reached by the workloads) */
    return (uint16_t)(sign | ((uint32_t)e << 7) | (n & 0x7Fu));
}

static double phi_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

static double phi_inv(double p) {
    double lo = -12.0, hi = 12.0;
    for (int it = 0; it < 200 && hi - lo > 0.0; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid == lo || mid == hi) break;
        if (phi_cdf(mid) < p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

static double g_quantile[65536];
static pthread_once_t g_quantile_once = PTHREAD_ONCE_INIT;
static void quantile_init(void) {
    for (int i = 0; i < 65536; ++i) g_quantile[i] = phi_inv(((double)i + 0.5) / 65536.0);
}

/* Standard-normal quantile table entry i (exposed so tests can check the table). */
double gen_normal_quantile(int i) {
    pthread_once(&g_quantile_once, quantile_init);
    if (i < 0 || i > 65535) return 0.0;
    return g_quantile[i];
}

/* The standard normal sample behind element `idx` of tensor `tensor` (double, before any rounding). */
static inline double normal_at(uint64_t key, uint64_t idx) {
    uint64_t w = word_of(key, idx >> 2);
    uint32_t u = (uint32_t)((w >> (16 * (idx & 3))) & 0xFFFFu);
    return g_quantile[u];
}

typedef struct {
    int kind;
    uint64_t key;
    double a, b; /* kind 0: sigma; kind 1: lo, hi */
    uint64_t start, count;
    void* out;
} job_t;

static void* run_job(void* p) {
    job_t* j = (job_t*)p;
    if (j->kind == 0) {
        /* bf16(sigma * q[u]) for all 65536 u, then one lookup per element */
        uint16_t* lut = (uint16_t*)malloc(65536 * sizeof(uint16_t));
        uint16_t* o = (uint16_t*)j->out;
        if (lut) {
            for (int u = 0; u < 65536; ++u) lut[u] = gen_bf16_from_double(j->a * g_quantile[u]);
            uint64_t i = 0;
            for (; i < j->count && ((j->start + i) & 3); ++i) o[i] = gen_bf16_from_double(j->a * normal_at(j->key, j->start + i));
            for (; i + 4 <= j->count; i += 4) {
                uint64_t w = word_of(j->key, (j->start + i) >> 2);
                o[i] = lut[w & 0xFFFF];
                o[i + 1] = lut[(w >> 16) & 0xFFFF];
                o[i + 2] = lut[(w >> 32) & 0xFFFF];
                o[i + 3] = lut[w >> 48];
            }
            for (; i < j->count; ++i) o[i] = gen_bf16_from_double(j->a * normal_at(j->key, j->start + i));
            free(lut);
        } else {
            for (uint64_t i = 0; i < j->count; ++i)
                o[i] = gen_bf16_from_double(j->a * normal_at(j->key, j->start + i));
        }
    } else {
        float* o = (float*)j->out;
        for (uint64_t i = 0; i < j->count; ++i) {
            uint64_t w = word_of(j->key, j->start + i);
            double u = (double)(w >> 11) * (1.0 / 9007199254740992.0);
            o[i] = (float)(j->a + (j->b - j->a) * u);
        }
    }
    return NULL;
}

static void run_parallel(int kind, uint64_t key, double a, double b, uint64_t start, uint64_t count,
                         void* out, size_t elem, int nthreads) {
    pthread_once(&g_quantile_once, quantile_init);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((uint64_t)nthreads > count / 65536 + 1) nthreads = (int)(count / 65536 + 1);
    job_t jobs[256];
    pthread_t th[256];
    uint64_t per = (count + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
    int n = 0;
    for (int t = 0; t < nthreads; ++t) {
        uint64_t s = (uint64_t)t * per;
        if (s >= count) break;
        uint64_t c = count - s < per ? count - s : per;
        jobs[n] = (job_t){kind, key, a, b, start + s, c, (char*)out + s * elem};
        ++n;
    }
    for (int t = 1; t < n; ++t) pthread_create(&th[t], NULL, run_job, &jobs[t]);
    if (n > 0) run_job(&jobs[0]);
    for (int t = 1; t < n; ++t) pthread_join(th[t], NULL);
}

/* out[i] = bf16(sigma * N_i) for elements [start, start + count) of tensor `tensor`. */
void gen_normal_bf16(uint64_t seed, uint32_t tensor, double sigma, uint64_t start, uint64_t count,
                     uint16_t* out, int nthreads) {
    run_parallel(0, key_of(seed, tensor), sigma, 0.0, start, count, out, sizeof(uint16_t), nthreads);
}

/* out[i] = fp32(lo + (hi - lo) * U_i) for elements [start, start + count) of tensor `tensor`. */
void gen_uniform_f32(uint64_t seed, uint32_t tensor, double lo, double hi, uint64_t start, uint64_t count,
                     float* out, int nthreads) {
    run_parallel(1, key_of(seed, tensor), lo, hi, start, count, out, sizeof(float), nthreads);
}

/* Skewed router weight: W[e, h] = bf16(sigma * N_{e*H+h} + alpha * (e + 1)^(-power)), row-major [E, H]:
 * a per-expert offset, ordered by expert index, added to every column entry of that expert. */
void gen_skew_router_bf16(uint64_t seed, uint32_t tensor, int E, int H, double sigma, double alpha,
                          double power, uint16_t* out) {
    pthread_once(&g_quantile_once, quantile_init);
    uint64_t key = key_of(seed, tensor);
    for (int e = 0; e < E; ++e) {
        double off = alpha * pow((double)(e + 1), -power);
        for (int h = 0; h < H; ++h) {
            uint64_t idx = (uint64_t)e * (uint64_t)H + (uint64_t)h;
            out[idx] = gen_bf16_from_double(sigma * normal_at(key, idx) + off);
        }
    }
}

/* Skewed selection bias: b[i] = fp32(coef * ln(1 / (i + 1))). */
void gen_log_bias_f32(int E, double coef, float* out) {
    for (int i = 0; i < E; ++i) out[i] = (float)(coef * log(1.0 / (double)(i + 1)));
}
