/*
 * fp8_oracle.c -- plain CPU oracle for the FP8 scaled-cast path.
 *
 * TEST INFRASTRUCTURE ONLY (see fp8_oracle.h).  Written for obviousness, not
 * speed: one element at a time, no blocking, no fusion, no threads.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (x86-64: binary32 arithmetic on SSE, so no excess precision).
 */
#include "fp8_oracle.h"

#include <math.h>
#include <string.h>
#include <xmmintrin.h>

/* ------------------------------------------------------------------------ */
/* bit helpers                                                               */
/* ------------------------------------------------------------------------ */

static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

int oracle_fpu_check(void) {
    /* MXCSR bit 15 = flush-to-zero, bit 6 = denormals-are-zero */
    return (_mm_getcsr() & ((1u << 15) | (1u << 6))) != 0;
}

/* ------------------------------------------------------------------------ */
/* Format descriptions, from the OCP 8-bit floating point specification      */
/* (OFP8).  The ColossalAI fp8.py page picks torch.float8_e4m3fn for "e4m3"   */
/* and torch.float8_e5m2 for "e5m2" (cast_to_fp8) and takes fp8_max from the */
/* format's finfo; the DeepEP "5 Utils" page hard-codes 448 for e4m3fn.      */
/*   E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; only */
/*         S.1111.111 is NaN, so the largest finite is S.1111.110 = 1.75*2^8 */
/*   E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits; IEEE-like:         */
/*         S.11111.00 = inf, S.11111.{01,10,11} = NaN; largest finite is     */
/*         S.11110.11 = 1.75*2^15                                            */
/* ------------------------------------------------------------------------ */

typedef struct {
    int mbits;     /* stored mantissa bits */
    int ebits;     /* exponent field bits */
    int bias;
    int max_code;  /* magnitude code of the largest finite value */
} minifloat_t;

static minifloat_t fp8_format(int fmt) {
    minifloat_t d;
    if (fmt == ORC_E4M3FN) { d.mbits = 3; d.ebits = 4; d.bias = 7;  d.max_code = 0x7E; }
    else                   { d.mbits = 2; d.ebits = 5; d.bias = 15; d.max_code = 0x7B; }
    return d;
}

float oracle_fp8_max(int fmt) { return oracle_fp8_decode((uint8_t)fp8_format(fmt).max_code, fmt); }

/* Closed-form decode: zero exponent field = subnormal m * 2^(1-bias-mbits);
 * otherwise (2^mbits + m) * 2^(E-bias-mbits).  Every code is exact in fp32. */
float oracle_fp8_decode(uint8_t code, int fmt) {
    minifloat_t d = fp8_format(fmt);
    int s = code >> 7;
    int E = (code >> d.mbits) & ((1 << d.ebits) - 1);
    int m = code & ((1 << d.mbits) - 1);
    int all_ones = (1 << d.ebits) - 1;
    if (fmt == ORC_E4M3FN && E == all_ones && m == (1 << d.mbits) - 1)
        return float_of(s ? 0xFFC00000u : 0x7FC00000u);
    if (fmt == ORC_E5M2 && E == all_ones) {
        if (m == 0) return s ? -INFINITY : INFINITY;
        return float_of(s ? 0xFFC00000u : 0x7FC00000u);
    }
    double mag = (E == 0) ? ldexp((double)m, 1 - d.bias - d.mbits)
                          : ldexp((double)((1 << d.mbits) + m), E - d.bias - d.mbits);
    return (float)(s ? -mag : mag);
}

/*
 * Round the magnitude of a finite, nonzero binary32 value onto a minifloat
 * grid with `mbits` stored mantissa bits and smallest normal exponent `emin`,
 * round-to-nearest, ties-to-even.  Returns the unsaturated magnitude code
 * (exponent field << mbits | mantissa), which may exceed the format's range;
 * the caller applies its overflow rule.
 */
static int64_t round_magnitude(uint32_t u, int mbits, int emin, int bias) {
    uint32_t ef = (u >> 23) & 0xFFu;
    uint32_t mf = u & 0x7FFFFFu;
    uint64_t sig;
    int e0;                          /* |v| = sig * 2^e0 exactly */
    if (ef == 0) { sig = mf; e0 = -149; }
    else         { sig = mf | 0x800000u; e0 = (int)ef - 150; }

    int lead = 63 - __builtin_clzll(sig);
    int E = e0 + lead;               /* 2^E <= |v| < 2^(E+1) */
    int qexp = (E > emin ? E : emin) - mbits;   /* grid spacing 2^qexp */
    int shift = qexp - e0;           /* always > 0: binary32 is finer */

    uint64_t k;
    if (shift > 60) {
        k = 0;                       /* sig < 2^24 < half a grid step */
    } else {
        k = sig >> shift;
        uint64_t rem = sig & ((1ull << shift) - 1);
        uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (k & 1))) k += 1;   /* RNE */
    }
    if (k == 0) return 0;
    if (k == (2ull << mbits)) { k >>= 1; qexp += 1; }   /* carry into exponent */

    int64_t efield, mfield;
    if (k >= (1ull << mbits)) {      /* normal */
        efield = (int64_t)qexp + mbits + bias;
        mfield = (int64_t)k - (1ll << mbits);
    } else {                         /* subnormal: only when qexp == emin - mbits */
        efield = 0;
        mfield = (int64_t)k;
    }
    return (efield << mbits) | mfield;
}

/* fp32 -> fp8, RNE, saturating to +-fp8_max (values that round above the
 * largest finite value, and +-inf, become +-max); NaN -> S.1111111;
 * the sign of zero and of underflowing values is kept. */
uint8_t oracle_fp8_encode(float v, int fmt) {
    minifloat_t d = fp8_format(fmt);
    uint32_t u = bits_of(v);
    uint8_t sbit = (uint8_t)((u >> 31) << 7);
    uint32_t ef = (u >> 23) & 0xFFu, mf = u & 0x7FFFFFu;
    if (ef == 0xFF) return mf ? (uint8_t)(sbit | 0x7F) : (uint8_t)(sbit | d.max_code);
    if (ef == 0 && mf == 0) return sbit;
    int64_t code = round_magnitude(u, d.mbits, 1 - d.bias, d.bias);
    if (code > d.max_code) code = d.max_code;
    return (uint8_t)(sbit | (uint8_t)code);
}

/* fp32 -> bf16, RNE; NaN stays NaN (quiet bit set). */
uint16_t oracle_bf16_from_f32(float v) {
    uint32_t u = bits_of(v);
    uint32_t upper = u >> 16, lower = u & 0xFFFFu;
    if (((u >> 23) & 0xFF) == 0xFF && (u & 0x7FFFFF)) return (uint16_t)(upper | 0x0040u);
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;
    return (uint16_t)upper;
}

float oracle_f32_from_bf16(uint16_t b) { return float_of((uint32_t)b << 16); }

/* fp32 -> IEEE binary16, RNE; overflow to +-inf; NaN stays NaN. */
uint16_t oracle_f16_from_f32(float v) {
    uint32_t u = bits_of(v);
    uint16_t sbit = (uint16_t)((u >> 31) << 15);
    uint32_t ef = (u >> 23) & 0xFFu, mf = u & 0x7FFFFFu;
    if (ef == 0xFF) return mf ? (uint16_t)(sbit | 0x7E00u) : (uint16_t)(sbit | 0x7C00u);
    if (ef == 0 && mf == 0) return sbit;
    int64_t code = round_magnitude(u, 10, -14, 15);
    if (code >= 0x7C00) code = 0x7C00;
    return (uint16_t)(sbit | (uint16_t)code);
}

float oracle_f32_from_f16(uint16_t h) {
    int s = h >> 15, E = (h >> 10) & 0x1F, m = h & 0x3FF;
    if (E == 31) {
        if (m == 0) return s ? -INFINITY : INFINITY;
        return float_of(s ? 0xFFC00000u : 0x7FC00000u);
    }
    double mag = (E == 0) ? ldexp((double)m, -24) : ldexp((double)(1024 + m), E - 25);
    return (float)(s ? -mag : mag);
}

void oracle_fp8_encode_array(const float* v, int64_t n, int fmt, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_encode(v[i], fmt);
}
void oracle_fp8_decode_array(const uint8_t* c, int64_t n, int fmt, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_decode(c[i], fmt);
}
void oracle_bf16_from_f32_array(const float* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_f32(v[i]);
}
void oracle_f16_from_f32_array(const float* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_from_f32(v[i]);
}

/* ------------------------------------------------------------------------ */
/* element access                                                            */
/* ------------------------------------------------------------------------ */

/* exact widening of one input element to binary32 (the pages' .float()) */
static float load_elem(const void* x, int dtype, int64_t i) {
    if (dtype == ORC_F32) return ((const float*)x)[i];
    if (dtype == ORC_BF16) return oracle_f32_from_bf16(((const uint16_t*)x)[i]);
    return oracle_f32_from_f16(((const uint16_t*)x)[i]);
}

static void store_elem(void* y, int ydtype, int64_t i, float p) {
    if (ydtype == ORC_F32) ((float*)y)[i] = p;
    else if (ydtype == ORC_BF16) ((uint16_t*)y)[i] = oracle_bf16_from_f32(p);
    else ((uint16_t*)y)[i] = oracle_f16_from_f32(p);
}

static int bad_dtype(int dt) { return dt != ORC_F32 && dt != ORC_BF16 && dt != ORC_F16; }
static int bad_fmt(int f) { return f != ORC_E4M3FN && f != ORC_E5M2; }

/* ------------------------------------------------------------------------ */
/* steps                                                                     */
/* ------------------------------------------------------------------------ */

/* amax = max |x_i| (cast_to_fp8: inp.abs().max().float(); per_token_cast_to_fp8:
 * x.abs().float().amax()).  Max is exact; torch's max propagates NaN. */
float oracle_amax(const void* x, int dtype, int64_t n) {
    float amax = 0.0f;
    int saw_nan = 0;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(load_elem(x, dtype, i));
        if (isnan(a)) saw_nan = 1;
        else if (a > amax) amax = a;
    }
    return saw_nan ? NAN : amax;
}

/* cast_to_fp8, per-tensor branch: torch.where(amax > 0, amax, 1.0) (NaN fails
 * the comparison and so also becomes 1), scale = fp8_max / amax,
 * scale_inv = 1.0 / scale, both binary32 divisions. */
void oracle_per_tensor_scale(float amax, int fmt, float* scale, float* scale_inv) {
    float a = (amax > 0.0f) ? amax : 1.0f;
    float s = oracle_fp8_max(fmt) / a;
    *scale = s;
    *scale_inv = 1.0f / s;
}

/* (scale * inp.float()).to(fp8): one binary32 product, then the fp8 encode */
void oracle_scale_and_cast(const void* x, int dtype, int64_t n, float scale, int fmt, uint8_t* q) {
    for (int64_t i = 0; i < n; ++i) q[i] = oracle_fp8_encode(load_elem(x, dtype, i) * scale, fmt);
}

/* ------------------------------------------------------------------------ */
/* whole operations                                                          */
/* ------------------------------------------------------------------------ */

/* cast_to_fp8(inp, fmt, per_channel_scale=False); an empty input returns
 * scale_inv = 1.0 and touches nothing else. */
int oracle_cast_per_tensor(const void* x, int dtype, int64_t n, int fmt,
                           uint8_t* q, float* scale_inv) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(dtype) || bad_fmt(fmt)) return -2;
    if (n < 0) return -1;
    if (n == 0) { scale_inv[0] = 1.0f; return 0; }
    float scale, sinv;
    oracle_per_tensor_scale(oracle_amax(x, dtype, n), fmt, &scale, &sinv);
    oracle_scale_and_cast(x, dtype, n, scale, fmt, q);
    scale_inv[0] = sinv;
    return 0;
}

/* cast_to_fp8(inp, fmt, per_channel_scale=True) on a 2-D [rows, cols] input:
 * per row, amax_r = max_c |x_rc|, zero (or NaN) -> 1, scale_r = fp8_max/amax_r,
 * scale_inv_r = amax_r / fp8_max (a division by fp8_max, not 1/scale).
 * An empty input (cols == 0) takes the empty branch: every scale_inv_r = 1.0. */
int oracle_cast_per_channel(const void* x, int dtype, int64_t rows, int64_t cols, int fmt,
                            uint8_t* q, float* scale_inv) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(dtype) || bad_fmt(fmt)) return -2;
    if (rows < 0 || cols < 0) return -1;
    int esz = (dtype == ORC_F32) ? 4 : 2;
    float fmax = oracle_fp8_max(fmt);
    for (int64_t r = 0; r < rows; ++r) {
        if (cols == 0) { scale_inv[r] = 1.0f; continue; }
        const void* xr = (const char*)x + r * cols * esz;
        float amax = oracle_amax(xr, dtype, cols);
        float a = (amax > 0.0f) ? amax : 1.0f;
        float scale = fmax / a;
        scale_inv[r] = a / fmax;
        oracle_scale_and_cast(xr, dtype, cols, scale, fmt, q + r * cols);
    }
    return 0;
}

/* per_token_cast_to_fp8: view [rows, cols/128, 128]; per group
 * amax = max(max |x|, 1e-4) (torch.clamp keeps NaN), scale = 448 / amax,
 * q = e4m3fn(fp32(x) * scale), scale_inv = amax / 448.  For e5m2 the same
 * steps with 57344 in place of 448. */
int oracle_cast_per_group128(const void* x, int dtype, int64_t rows, int64_t cols, int fmt,
                             uint8_t* q, float* scale_inv) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(dtype) || bad_fmt(fmt)) return -2;
    if (rows < 0 || cols < 0) return -1;
    if (cols % 128 != 0) return -3;
    int esz = (dtype == ORC_F32) ? 4 : 2;
    float fmax = oracle_fp8_max(fmt);
    const float clamp_min = 1e-4f;
    int64_t groups = cols / 128;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < groups; ++g) {
            int64_t off = r * cols + g * 128;
            const void* xg = (const char*)x + off * esz;
            float amax = oracle_amax(xg, dtype, 128);
            if (amax < clamp_min) amax = clamp_min;
            float scale = fmax / amax;
            scale_inv[r * groups + g] = amax / fmax;
            oracle_scale_and_cast(xg, dtype, 128, scale, fmt, q + off);
        }
    }
    return 0;
}

/* cast_from_fp8 (per-tensor): (scale_inv * inp.float()).to(ret_type) */
int oracle_dequant_per_tensor(const uint8_t* q, int fmt, int64_t n, const float* scale_inv,
                              void* y, int ydtype) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(ydtype) || bad_fmt(fmt)) return -2;
    if (n < 0) return -1;
    for (int64_t i = 0; i < n; ++i)
        store_elem(y, ydtype, i, oracle_fp8_decode(q[i], fmt) * scale_inv[0]);
    return 0;
}

/* cast_from_fp8 (per-channel): scale_inv indexed by row */
int oracle_dequant_per_channel(const uint8_t* q, int fmt, int64_t rows, int64_t cols,
                               const float* scale_inv, void* y, int ydtype) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(ydtype) || bad_fmt(fmt)) return -2;
    if (rows < 0 || cols < 0) return -1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            store_elem(y, ydtype, r * cols + c, oracle_fp8_decode(q[r * cols + c], fmt) * scale_inv[r]);
    return 0;
}

/* inverse of per_token_cast_to_fp8: y[r, c] = dec(q[r, c]) * s[r, c / 128] */
int oracle_dequant_per_group128(const uint8_t* q, int fmt, int64_t rows, int64_t cols,
                                const float* scale_inv, void* y, int ydtype) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(ydtype) || bad_fmt(fmt)) return -2;
    if (rows < 0 || cols < 0) return -1;
    if (cols % 128 != 0) return -3;
    int64_t groups = cols / 128;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            store_elem(y, ydtype, r * cols + c,
                       oracle_fp8_decode(q[r * cols + c], fmt) * scale_inv[r * groups + c / 128]);
    return 0;
}

/* weight_dequant / weight_dequant_kernel: s has shape [ceil(M/128), ceil(N/128)]
 * and the tile (i/128, j/128) uses s[(i/128) * ceil(N/128) + j/128]; the
 * binary32 product is stored into the output type. */
int oracle_weight_dequant_block128(const uint8_t* q, int fmt, int64_t M, int64_t N,
                                   const float* scale_inv, void* y, int ydtype) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(ydtype) || bad_fmt(fmt)) return -2;
    if (M < 0 || N < 0) return -1;
    int64_t nb = (N + 127) / 128;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            store_elem(y, ydtype, i * N + j,
                       oracle_fp8_decode(q[i * N + j], fmt) * scale_inv[(i / 128) * nb + j / 128]);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* reduce step of the compressed collectives                                 */
/* ------------------------------------------------------------------------ */

/* value of v after rounding to the element type (binary32 holds every bf16
 * and fp16 value exactly) */
static float round_to(float v, int dtype) {
    if (dtype == ORC_BF16) return oracle_f32_from_bf16(oracle_bf16_from_f32(v));
    if (dtype == ORC_F16) return oracle_f32_from_f16(oracle_f16_from_f32(v));
    return v;
}

/* ColossalAI fp8.py, _all_reduce_fp8 / _reduce_scatter_fp8 and the DDP hook's
 * sum_and_allgather: summed_out = zeros(input_type); for each received chunk
 * in order, summed_out += cast_from_fp8(chunk, its scale_inv, input_type);
 * then summed_out.div_(world_size) for ReduceOp.AVG.  Each += is an
 * input_type addition (binary32 sum rounded to the type), and the division
 * is a binary32 division rounded to the type. */
int oracle_dequant_sum(const uint8_t* q, int fmt, int64_t W, int64_t n, const float* scale_inv, int average,
                       void* y, int ydtype) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(ydtype) || bad_fmt(fmt)) return -2;
    if (W < 1 || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (int64_t w = 0; w < W; ++w) {
            float term = round_to(oracle_fp8_decode(q[w * n + i], fmt) * scale_inv[w], ydtype);
            acc = round_to(acc + term, ydtype);
        }
        if (average) acc = round_to(acc / (float)W, ydtype);
        store_elem(y, ydtype, i, acc);
    }
    return 0;
}

/* _all_reduce_fp8: the summed chunk is cast again with cast_to_fp8 (per tensor) */
int oracle_dequant_sum_requant(const uint8_t* q, int fmt, int64_t W, int64_t n, const float* scale_inv,
                               int average, void* y, int ydtype, uint8_t* q_out, float* scale_inv_out) {
    int rc = oracle_dequant_sum(q, fmt, W, n, scale_inv, average, y, ydtype);
    if (rc != 0) return rc;
    return oracle_cast_per_tensor(y, ydtype, n, fmt, q_out, scale_inv_out);
}

/* ------------------------------------------------------------------------ */
/* FSDP parameter hook: a global scale from a cross-rank amax                */
/* ------------------------------------------------------------------------ */

/* ColossalAI fp8.py, fp8_compress_fsdp_params_comm_hook: per_tensor_max =
 * inp.abs().max().float(), then torch.where(per_tensor_max > 0, ., 1.0) on
 * each rank before dist.all_reduce(per_tensor_max, op=MAX). */
float oracle_amax_guarded(const void* x, int dtype, int64_t n) {
    float amax = oracle_amax(x, dtype, n);
    return (amax > 0.0f) ? amax : 1.0f;
}

/* the same hook after the all-reduce: scale = fp8_max / per_tensor_max;
 * fp8 = (scale * inp.float()).to(fp8_type) */
int oracle_cast_with_amax(const void* x, int dtype, int64_t n, int fmt, float amax, uint8_t* q, float* scale_out) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(dtype) || bad_fmt(fmt)) return -2;
    if (n < 0) return -1;
    float scale = oracle_fp8_max(fmt) / amax;
    oracle_scale_and_cast(x, dtype, n, scale, fmt, q);
    scale_out[0] = scale;
    return 0;
}

/* the hook's dequant after the all-gather: (fp8_out.float() / scale).to(out.dtype),
 * a binary32 division (not a product with 1/scale) */
int oracle_dequant_div_scale(const uint8_t* q, int fmt, int64_t n, float scale, void* y, int ydtype) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(ydtype) || bad_fmt(fmt)) return -2;
    if (n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) store_elem(y, ydtype, i, oracle_fp8_decode(q[i], fmt) / scale);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* pipeline p2p cast with the format chosen from the data                    */
/* ------------------------------------------------------------------------ */

/* ColossalAI fp8.py, cast_to_fp8_pipeline: (min, max) = aminmax(x);
 * amax = maximum(|min|, |max|) (NaN if any element is NaN); e5m2 when
 * amax > 448 (the e4m3fn maximum), else e4m3fn; scale = 1 when amax == 0,
 * else that format's maximum / amax (binary32 division; a NaN amax fails both
 * comparisons, so e4m3fn with a NaN scale); q = enc(fp32(x) * scale);
 * fp8_scale = 1 / scale.  An empty tensor is taken to have amax 0. */
int oracle_cast_to_fp8_pipeline(const void* x, int dtype, int64_t n, uint8_t* q, float* scale_inv, int* fmt_out) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(dtype)) return -2;
    if (n < 0) return -1;
    float lo = 0.0f, hi = 0.0f;
    int seen = 0, saw_nan = 0;
    for (int64_t i = 0; i < n; ++i) {
        float v = load_elem(x, dtype, i);
        if (isnan(v)) { saw_nan = 1; continue; }
        if (!seen || v < lo) lo = v;
        if (!seen || v > hi) hi = v;
        seen = 1;
    }
    float amax = saw_nan ? NAN : (fabsf(lo) > fabsf(hi) ? fabsf(lo) : fabsf(hi));
    int fmt = (amax > oracle_fp8_max(ORC_E4M3FN)) ? ORC_E5M2 : ORC_E4M3FN;
    float scale = (amax == 0.0f) ? 1.0f : oracle_fp8_max(fmt) / amax;
    oracle_scale_and_cast(x, dtype, n, scale, fmt, q);
    *scale_inv = 1.0f / scale;
    *fmt_out = fmt;
    return 0;
}

/* cast_from_fp8_pipeline: hidden_states.view(fp8).to(dtype) * fp8_scale -- the
 * code converted to the output type (exact for every fp8 value), times the
 * binary32 scale in binary32, rounded to the output type */
int oracle_cast_from_fp8_pipeline(const uint8_t* q, int fmt, int64_t n, float scale_inv, void* y, int ydtype) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(ydtype) || bad_fmt(fmt)) return -2;
    if (n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) store_elem(y, ydtype, i, round_to(oracle_fp8_decode(q[i], fmt), ydtype) * scale_inv);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* packed [scale_inv | payload] slots of the fp8 all-gather                  */
/* ------------------------------------------------------------------------ */

/* ColossalAI fp8.py, all_gather_fp8_lagacy / all_gather_fp8_ring: a rank's
 * slot of the combined buffer is SCALE_BYTES = 4 bytes followed by n fp8
 * codes; cast_to_fp8(x.view(-1), out=slot[4:]) writes the codes and the
 * returned scale_inv is stored into slot[0:4] as a binary32 (host byte
 * order, little-endian here). */
int oracle_cast_to_packed(const void* x, int dtype, int64_t n, int fmt, uint8_t* slot) {
    float scale_inv;
    int rc = oracle_cast_per_tensor(x, dtype, n, fmt, slot + 4, &scale_inv);
    if (rc != 0) return rc;
    memcpy(slot, &scale_inv, 4);
    return 0;
}

/* the receive side: slot w of the combined buffer starts at w * (4 + n);
 * scale = slot[0:4] viewed as binary32, then cast_from_fp8(slot[4:], scale,
 * input_type, out=output_list[w]) -- output w is y + w * n elements */
int oracle_dequant_packed(const uint8_t* slots, int fmt, int64_t W, int64_t n, void* y, int ydtype) {
    if (oracle_fpu_check()) return -9;
    if (bad_dtype(ydtype) || bad_fmt(fmt)) return -2;
    if (W < 0 || n < 0) return -1;
    for (int64_t w = 0; w < W; ++w) {
        const uint8_t* slot = slots + w * (4 + n);
        float scale_inv;
        memcpy(&scale_inv, slot, 4);
        for (int64_t i = 0; i < n; ++i)
            store_elem(y, ydtype, w * n + i, oracle_fp8_decode(slot[4 + i], fmt) * scale_inv);
    }
    return 0;
}
