/*
 * fp8_oracle.h -- plain, slow, single-threaded CPU oracle for the FP8
 * scaled-cast path (quantize: amax -> scale -> cast; dequantize).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or constant with the HIP library in
 * dequantize_amax_reduce_amd/csrc and must never be used as a fallback for it.
 *
 * Sources (the pages this follows):
 *  - ColossalAI `colossalai/quantization/fp8.py` (v0.4.4 mirror page),
 *    functions cast_to_fp8 and cast_from_fp8: per-tensor and per-channel
 *    scaled casts and their inverse.
 *  - "5 Utils" (DeepEP utils notes), section on per_token_cast_to_fp8:
 *    the per-128-element-group quantize.
 *  - "FP8 (8 bits) & FP16 (16 bits)" (CSDN notes on fp8_cast_bf16), sections
 *    weight_dequant and weight_dequant_kernel: the 128x128 block dequant.
 *
 * All floating-point arithmetic is IEEE binary32 (the pages call .float()
 * before every reduction and product), evaluated on x86-64 SSE with no FMA
 * contraction and no flush-to-zero.  Every function checks MXCSR first.
 *
 * Parity pins: every function here is pinned by the CPU tests in tests/
 * (closed forms, exhaustive codes, structured brute force against an
 * exact-rational nearest-value search, invariants, metamorphic scaling).
 * The only "parity unpinned" item is the exact NaN code emitted for NaN
 * input (NaN outputs are compared by class).
 */
#ifndef FP8_ORACLE_H
#define FP8_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types (oracle-local numbering) */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F16 = 2 };
/* fp8 formats (oracle-local numbering) */
enum { ORC_E4M3FN = 0, ORC_E5M2 = 1 };

/* Returns 0 when the FPU state is IEEE (no FTZ/DAZ), nonzero otherwise. */
int oracle_fpu_check(void);

/* --- element codecs ---------------------------------------------------- */
float    oracle_fp8_decode(uint8_t code, int fmt);
uint8_t  oracle_fp8_encode(float v, int fmt);
float    oracle_fp8_max(int fmt);
uint16_t oracle_bf16_from_f32(float v);
float    oracle_f32_from_bf16(uint16_t b);
uint16_t oracle_f16_from_f32(float v);
float    oracle_f32_from_f16(uint16_t h);

/* array forms, for tests */
void oracle_fp8_encode_array(const float* v, int64_t n, int fmt, uint8_t* out);
void oracle_fp8_decode_array(const uint8_t* c, int64_t n, int fmt, float* out);
void oracle_bf16_from_f32_array(const float* v, int64_t n, uint16_t* out);
void oracle_f16_from_f32_array(const float* v, int64_t n, uint16_t* out);

/* --- steps ------------------------------------------------------------- */
/* max |x_i| over n elements, as binary32; NaN anywhere gives NaN; n=0 gives 0 */
float oracle_amax(const void* x, int dtype, int64_t n);
/* per-tensor guard + scale: a = amax>0 ? amax : 1; scale = fp8_max/a; scale_inv = 1/scale */
void  oracle_per_tensor_scale(float amax, int fmt, float* scale, float* scale_inv);
/* q_i = enc(fl32(fp32(x_i) * scale)) for i in [0, n) */
void  oracle_scale_and_cast(const void* x, int dtype, int64_t n, float scale, int fmt, uint8_t* q);

/* --- whole operations -------------------------------------------------- */
int oracle_cast_per_tensor(const void* x, int dtype, int64_t n, int fmt,
                           uint8_t* q, float* scale_inv /*[1]*/);
int oracle_cast_per_channel(const void* x, int dtype, int64_t rows, int64_t cols, int fmt,
                            uint8_t* q, float* scale_inv /*[rows]*/);
int oracle_cast_per_group128(const void* x, int dtype, int64_t rows, int64_t cols, int fmt,
                             uint8_t* q, float* scale_inv /*[rows][cols/128]*/);
int oracle_dequant_per_tensor(const uint8_t* q, int fmt, int64_t n, const float* scale_inv,
                              void* y, int ydtype);
int oracle_dequant_per_channel(const uint8_t* q, int fmt, int64_t rows, int64_t cols,
                               const float* scale_inv, void* y, int ydtype);
int oracle_dequant_per_group128(const uint8_t* q, int fmt, int64_t rows, int64_t cols,
                                const float* scale_inv, void* y, int ydtype);
int oracle_weight_dequant_block128(const uint8_t* q, int fmt, int64_t M, int64_t N,
                                   const float* scale_inv, void* y, int ydtype);

/* --- reduce step of the fp8-compressed all-reduce / reduce-scatter ------ */
/* y[i] = the chunk-ordered sum over w of ydtype(fp32(q[w][i]) * scale_inv[w]),
 * accumulated in ydtype from +0, then divided by W when `average`. */
int oracle_dequant_sum(const uint8_t* q /*[W][n]*/, int fmt, int64_t W, int64_t n,
                       const float* scale_inv /*[W]*/, int average, void* y, int ydtype);
/* the sum above (written to y), then cast_to_fp8(y) per tensor into q_out / scale_inv_out[0] */
int oracle_dequant_sum_requant(const uint8_t* q, int fmt, int64_t W, int64_t n, const float* scale_inv,
                               int average, void* y, int ydtype, uint8_t* q_out, float* scale_inv_out);

/* --- cross-rank global amax (FSDP parameter hook) ----------------------- */
/* where(max|x| > 0, max|x|, 1): the local value each rank contributes to the MAX all-reduce */
float oracle_amax_guarded(const void* x, int dtype, int64_t n);
/* scale = fp8_max / amax (amax: the reduced, guarded value); q = enc(fp32(x) * scale); *scale_out = scale */
int oracle_cast_with_amax(const void* x, int dtype, int64_t n, int fmt, float amax, uint8_t* q, float* scale_out);
/* y = ydtype(fp32(q) / scale): the dequant by division */
int oracle_dequant_div_scale(const uint8_t* q, int fmt, int64_t n, float scale, void* y, int ydtype);

/* --- pipeline p2p cast: the format chosen from the data ----------------- */
/* amax = max(|min|, |max|); *fmt_out = e5m2 if amax > 448 else e4m3fn;
 * scale = 1 if amax == 0 else fp8_max(fmt) / amax; q = enc(fp32(x) * scale);
 * *scale_inv = 1 / scale */
int oracle_cast_to_fp8_pipeline(const void* x, int dtype, int64_t n, uint8_t* q, float* scale_inv, int* fmt_out);
/* y = ydtype(ydtype(fp32(q)) * scale_inv) */
int oracle_cast_from_fp8_pipeline(const uint8_t* q, int fmt, int64_t n, float scale_inv, void* y, int ydtype);

/* --- packed [scale_inv | payload] slots of the fp8 all-gather ---------- */
/* slot[0:4] = binary32 scale_inv of cast_to_fp8(x) per tensor, slot[4:4+n] = its codes */
int oracle_cast_to_packed(const void* x, int dtype, int64_t n, int fmt, uint8_t* slot);
/* W slots at slots + w * (4 + n): y[w * n + i] = ydtype(fp32(code) * slot_w's scale_inv) */
int oracle_dequant_packed(const uint8_t* slots, int fmt, int64_t W, int64_t n, void* y, int ydtype);

#ifdef __cplusplus
}
#endif
#endif
