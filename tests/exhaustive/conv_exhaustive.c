/*
 * Exhaustive check of the oracle's binary32 conversions (test infrastructure).
 *
 * Every one of the 2^32 binary32 bit patterns is converted by the oracle
 * library (loaded with dlopen; argv[1] is its path) to e4m3fn, e5m2, bf16 and
 * fp16, and each result is compared with an independent rule written here
 * from the formats' definitions: the value of the nearest point of the
 * format's grid (p significand bits, minimum normal exponent emin), found in
 * binary64 arithmetic by scaling to an integer multiple of the ulp and
 * rounding half to even; then, for fp8, magnitudes at or above the largest
 * finite value (and +-inf) saturate to it, and for bf16/fp16 a rounded value
 * above the largest finite one becomes inf.  The oracle's outputs are
 * decoded here from their bit fields (not with the oracle's decoder).  The
 * sign of zero is compared; NaN inputs must give a NaN of the format.
 *
 * Usage: conv_exhaustive <liboracle.so> [threads]   -> exit 0 iff no mismatch
 */
#include <dlfcn.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

typedef void (*fp8_arr_fn)(const float*, int64_t, int, uint8_t*);
typedef void (*u16_arr_fn)(const float*, int64_t, uint16_t*);

static fp8_arr_fn enc_fp8;
static u16_arr_fn enc_bf16, enc_f16;

typedef struct {
    int p;          /* significand bits, implicit bit included */
    int emin;       /* exponent of the smallest normal value */
    double maxfin;  /* largest finite value */
    int saturate;   /* 1: saturate to maxfin; 0: overflow to inf */
} grid_t;

static const grid_t G_E4M3 = {4, -6, 448.0, 1};
static const grid_t G_E5M2 = {3, -14, 57344.0, 1};
static const grid_t G_BF16 = {8, -126, 0x1.FEp127, 0};
static const grid_t G_F16 = {11, -14, 65504.0, 0};

/* 2^i for i in [-200, 200] */
static double POW2[401];

/* the grid value nearest to a >= 0 (finite), ties to the even multiple of the ulp */
static double round_grid(double a, const grid_t* g) {
    if (a == 0.0) return 0.0;
    if (g->saturate && a >= g->maxfin) return g->maxfin;
    /* below half the smallest subnormal everything rounds to 0 (a tie goes to the even 0) */
    const double min_sub = POW2[200 + g->emin - (g->p - 1)];
    if (a <= 0.5 * min_sub) return 0.0;
    int el = ilogb(a);         /* floor(log2 a) */
    if (el < g->emin) el = g->emin;
    const double ulp = POW2[200 + el - (g->p - 1)];
    const double k = a / ulp;  /* exact: ulp is a power of two */
    const double fl = floor(k), fr = k - fl;
    double r;
    if (fr > 0.5) r = fl + 1.0;
    else if (fr < 0.5) r = fl;
    else r = (((int64_t)fl) & 1) == 0 ? fl : fl + 1.0;
    const double v = r * ulp;
    if (v > g->maxfin) return g->saturate ? g->maxfin : INFINITY;
    return v;
}

/* decode from bit fields: value (NaN as NAN) and sign */
static double dec_fp8(uint8_t c, int e5m2, int* sign) {
    const int mb = e5m2 ? 2 : 3, eb = e5m2 ? 5 : 4, bias = e5m2 ? 15 : 7;
    *sign = c >> 7;
    const int E = (c >> mb) & ((1 << eb) - 1), m = c & ((1 << mb) - 1);
    if (!e5m2 && (c & 0x7F) == 0x7F) return NAN;
    if (e5m2 && E == 31) return m ? NAN : INFINITY;
    return E == 0 ? (double)m * POW2[200 + 1 - bias - mb] : (double)((1 << mb) + m) * POW2[200 + E - bias - mb];
}
static double dec_bf16(uint16_t b, int* sign) {
    *sign = b >> 15;
    uint32_t u = (uint32_t)(b & 0x7FFF) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}
static double dec_f16(uint16_t h, int* sign) {
    *sign = h >> 15;
    const int E = (h >> 10) & 31, m = h & 1023;
    if (E == 31) return m ? NAN : INFINITY;
    return E == 0 ? (double)m * POW2[200 - 24] : (double)(1024 + m) * POW2[200 + E - 25];
}

enum { NCONV = 4, CHUNK = 1 << 16 };
static const char* NAMES[NCONV] = {"e4m3fn", "e5m2", "bf16", "f16"};

typedef struct {
    int tid, nthreads;
    uint64_t bad[NCONV];
    uint32_t first_bad[NCONV];
} work_t;

static void* run(void* arg) {
    work_t* w = (work_t*)arg;
    float* v = malloc(sizeof(float) * CHUNK);
    uint8_t* q8[2] = {malloc(CHUNK), malloc(CHUNK)};
    uint16_t* q16[2] = {malloc(2 * CHUNK), malloc(2 * CHUNK)};
    const grid_t* grids[NCONV] = {&G_E4M3, &G_E5M2, &G_BF16, &G_F16};
    for (uint64_t c = (uint64_t)w->tid; c < (1ull << 32) / CHUNK; c += (uint64_t)w->nthreads) {
        const uint32_t base = (uint32_t)(c * CHUNK);
        for (uint32_t i = 0; i < CHUNK; ++i) {
            const uint32_t u = base + i;
            memcpy(&v[i], &u, 4);
        }
        enc_fp8(v, CHUNK, 0, q8[0]);
        enc_fp8(v, CHUNK, 1, q8[1]);
        enc_bf16(v, CHUNK, q16[0]);
        enc_f16(v, CHUNK, q16[1]);
        for (uint32_t i = 0; i < CHUNK; ++i) {
            const double x = (double)v[i];
            const int xs = (base + i) >> 31;
            for (int k = 0; k < NCONV; ++k) {
                int gs;
                const double got = k < 2 ? dec_fp8(q8[k][i], k, &gs) : (k == 2 ? dec_bf16(q16[0][i], &gs)
                                                                               : dec_f16(q16[1][i], &gs));
                int ok;
                if (isnan(x)) {
                    ok = isnan(got);
                } else {
                    const double a = fabs(x);
                    const double want = isinf(a) ? (grids[k]->saturate ? grids[k]->maxfin : INFINITY)
                                                 : round_grid(a, grids[k]);
                    ok = (got == want) && (gs == xs);
                }
                if (!ok) {
                    if (w->bad[k] == 0) w->first_bad[k] = base + i;
                    w->bad[k]++;
                }
            }
        }
    }
    free(v); free(q8[0]); free(q8[1]); free(q16[0]); free(q16[1]);
    return NULL;
}

int main(int argc, char** argv) {
    if (argc < 2) {
        fprintf(stderr, "usage: %s <liboracle.so> [threads]\n", argv[0]);
        return 2;
    }
    void* h = dlopen(argv[1], RTLD_NOW);
    if (!h) { fprintf(stderr, "dlopen: %s\n", dlerror()); return 2; }
    enc_fp8 = (fp8_arr_fn)dlsym(h, "oracle_fp8_encode_array");
    enc_bf16 = (u16_arr_fn)dlsym(h, "oracle_bf16_from_f32_array");
    enc_f16 = (u16_arr_fn)dlsym(h, "oracle_f16_from_f32_array");
    if (!enc_fp8 || !enc_bf16 || !enc_f16) { fprintf(stderr, "missing symbols\n"); return 2; }
    for (int i = -200; i <= 200; ++i) POW2[200 + i] = ldexp(1.0, i);
    int nt = argc > 2 ? atoi(argv[2]) : 8;
    if (nt < 1) nt = 1;
    if (nt > 64) nt = 64;
    pthread_t th[64];
    work_t w[64];
    struct timespec t0, t1;
    clock_gettime(CLOCK_MONOTONIC, &t0);
    for (int t = 0; t < nt; ++t) {
        memset(&w[t], 0, sizeof(w[t]));
        w[t].tid = t;
        w[t].nthreads = nt;
        pthread_create(&th[t], NULL, run, &w[t]);
    }
    uint64_t bad[NCONV] = {0};
    uint32_t first[NCONV] = {0};
    for (int t = 0; t < nt; ++t) {
        pthread_join(th[t], NULL);
        for (int k = 0; k < NCONV; ++k) {
            if (w[t].bad[k] && !bad[k]) first[k] = w[t].first_bad[k];
            bad[k] += w[t].bad[k];
        }
    }
    clock_gettime(CLOCK_MONOTONIC, &t1);
    int rc = 0;
    for (int k = 0; k < NCONV; ++k) {
        printf("%-7s 4294967296 inputs, %llu mismatches", NAMES[k], (unsigned long long)bad[k]);
        if (bad[k]) { printf(" (first at bits 0x%08X)", first[k]); rc = 1; }
        printf("\n");
    }
    printf("%.1f s on %d threads\n", (t1.tv_sec - t0.tv_sec) + 1e-9 * (t1.tv_nsec - t0.tv_nsec), nt);
    return rc;
}
