/*
 * fp8q.h -- C ABI of the FP8 scaled-cast library (quantize: amax -> scale ->
 * cast to fp8; dequantize: fp8 x scale_inv) for AMD Instinct MI355X (gfx950).
 *
 * Conventions for every entry point
 *  - Pointers named x, q, y, scale_inv, amax and workspace are DEVICE pointers
 *    owned by the caller.  Tensors are dense, contiguous and row-major.
 *  - The library allocates nothing, keeps no pointer after returning, holds no
 *    mutable global state and is re-entrant.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL means the default stream).  Inputs must stay valid and unchanged,
 *    and outputs untouched by others, until the stream reaches the work.
 *    Kernel faults surface at the caller's next synchronisation.
 *  - Arguments are validated on the host before any HIP call; a call that
 *    returns an error other than FP8Q_EHIP has enqueued nothing.
 *  - fp8 tensors are uint8 codes of the OCP 8-bit formats: E4M3 ("e4m3fn":
 *    bias 7, no infinities, max 448) or E5M2 (bias 15, IEEE-like, max 57344).
 *  - Sizes are int64 element counts; rows * cols must not overflow int64.
 *
 * Numerics (identical on every path and launch shape)
 *  - amax = max |x| exactly (a max is order-independent); NaN propagates.
 *  - scale and scale_inv are binary32 results of correctly rounded divisions;
 *    products are single binary32 multiplies (no FMA, no reciprocal-multiply).
 *  - fp32 -> fp8 rounds to nearest, ties to even; magnitudes that round above
 *    the format maximum (and +-inf) saturate to +-max; the sign of zero is
 *    kept; NaN encodes as S.1111111.
 *  - fp32 -> bf16 / fp16 outputs round to nearest even (fp16 overflows to inf).
 *
 * Sources: ColossalAI `colossalai/quantization/fp8.py` (cast_to_fp8,
 * cast_from_fp8); DeepEP utils notes "5 Utils" (per_token_cast_to_fp8); CSDN
 * notes "FP8 (8 bits) & FP16 (16 bits)" (weight_dequant,
 * weight_dequant_kernel).
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8Q_ABI_VERSION 1

/* fp8 format: cast_to_fp8's fp8_format ("e4m3" -> float8_e4m3fn, "e5m2" -> float8_e5m2) */
typedef enum { FP8Q_E4M3FN = 0, FP8Q_E5M2 = 1 } fp8q_fmt_t;

/* element type of the high-precision side: cast_to_fp8 accepts float32,
 * float16 and bfloat16; cast_from_fp8's ret_type picks the output type */
typedef enum { FP8Q_F32 = 0, FP8Q_BF16 = 1, FP8Q_F16 = 2 } fp8q_dtype_t;

typedef enum {
    FP8Q_OK = 0,
    FP8Q_EINVAL = 1, /* negative size, int64 overflow, NULL pointer with a non-empty
                        size, NULL workspace, or overlapping input/output ranges */
    FP8Q_EDTYPE = 2, /* unknown fp8 format or element type (cast_to_fp8 / cast_from_fp8
                        raise TypeError for these) */
    FP8Q_ESHAPE = 3, /* per-128-group with cols % 128 != 0 (per_token_cast_to_fp8's assert) */
    FP8Q_EALIGN = 4, /* a pointer not aligned to its element size */
    FP8Q_EHIP = 5    /* a kernel launch failed (hipGetLastError after the launch; an
                        earlier unchecked error on the calling thread is reported too) */
} fp8q_status_t;

/* FP8Q_ABI_VERSION of the built library */
int fp8q_abi_version(void);

/* static, human-readable name of a status code (never NULL) */
const char* fp8q_status_str(fp8q_status_t status);

/* bytes of device workspace (8192) that fp8q_cast_per_tensor,
 * fp8q_cast_to_fp8_pipeline, fp8q_cast_to_packed and fp8q_dequant_sum_requant
 * need.  Its contents are the library's scratch between the passes of one
 * call (amax partials or amax slots); it needs no initialisation and holds
 * nothing the caller reads. */
size_t fp8q_per_tensor_workspace_bytes(void);

/*
 * Global amax (ColossalAI fp8.py, cast_to_fp8, per-tensor branch:
 * inp.abs().max().float()).  Writes max_i |x_i| over n elements to amax[0]
 * (one binary32, device memory, 4-byte aligned); NaN anywhere gives a NaN;
 * n == 0 gives +0.  Two stages: a per-workgroup reduction, then an atomic max
 * on the binary32 bits into amax[0], which the call first clears on `stream`.
 */
fp8q_status_t fp8q_amax(const void* x, fp8q_dtype_t xdtype, int64_t n, float* amax, void* stream);

/*
 * Per-tensor cast (ColossalAI fp8.py, cast_to_fp8 with per_channel_scale=False).
 *   amax = max |x|; a = amax > 0 ? amax : 1 (NaN also gives 1);
 *   scale = fp8_max / a; scale_inv[0] = 1 / scale; q[i] = fp8(fp32(x[i]) * scale).
 * x: n elements of xdtype; q: n bytes; scale_inv: 1 float; workspace: at least
 * fp8q_per_tensor_workspace_bytes() bytes, 4-byte aligned, caller-owned, not
 * shared with a concurrent call.  n == 0 writes scale_inv[0] = 1.0 and nothing
 * else (cast_to_fp8's empty-tensor branch).  Reads x twice (amax pass, then
 * the scale-and-cast pass).
 */
fp8q_status_t fp8q_cast_per_tensor(const void* x, fp8q_dtype_t xdtype, int64_t n, fp8q_fmt_t fmt,
                                   uint8_t* q, float* scale_inv, void* workspace, void* stream);

/*
 * fp8q_cast_per_tensor without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same numerics, passes and outputs as
 * fp8q_cast_per_tensor; it allocates nothing.  The amax partials go to a
 * scratch array the library holds in device memory: 4096 bytes (1024 words)
 * per GPU, created with the code object on each GPU the library runs on and
 * kept until the process ends.  The amax pass never needs more than that,
 * whatever n is, so every n accepted by fp8q_cast_per_tensor is accepted
 * here (FP8Q_EINVAL would report a grid that needed more, before anything is
 * enqueued).  The scratch used is the one on `stream`'s device (the current
 * device for a NULL stream); its address is looked up on the first call per
 * device (FP8Q_EHIP if that lookup fails).  Every call on one GPU shares that
 * GPU's scratch: calls that overlap in time on one GPU (other streams, other
 * threads) race and give wrong results; calls ordered on one stream are safe.
 */
fp8q_status_t fp8q_cast_per_tensor_noalloc(const void* x, fp8q_dtype_t xdtype, int64_t n, fp8q_fmt_t fmt,
                                           uint8_t* q, float* scale_inv, void* stream);

/*
 * Per-channel cast (ColossalAI fp8.py, cast_to_fp8 with per_channel_scale=True;
 * the channel is the last dimension, so one row of x [rows, cols]).
 *   amax_r = max_c |x[r, c]|; a_r = amax_r > 0 ? amax_r : 1;
 *   scale_r = fp8_max / a_r; scale_inv[r] = a_r / fp8_max (not 1 / scale_r);
 *   q[r, c] = fp8(fp32(x[r, c]) * scale_r).
 * scale_inv has `rows` floats (row-indexed).  rows == 0 is a no-op; cols == 0
 * writes scale_inv[r] = 1.0 for every row (the empty-tensor branch).
 */
fp8q_status_t fp8q_cast_per_channel(const void* x, fp8q_dtype_t xdtype, int64_t rows, int64_t cols, fp8q_fmt_t fmt,
                                    uint8_t* q, float* scale_inv, void* stream);

/*
 * Per-128-group cast (DeepEP "5 Utils", per_token_cast_to_fp8: x viewed as
 * [rows, cols/128, 128]).  For every row r and group g (columns 128g..128g+127):
 *   amax = max(max |x|, 1e-4) (binary32 0x38D1B717; NaN propagates);
 *   scale = fp8_max / amax; scale_inv[r, g] = amax / fp8_max;
 *   q = fp8(fp32(x) * scale).
 * fp8_max is 448 for E4M3 (the page's constant) and 57344 for E5M2.
 * cols % 128 != 0 -> FP8Q_ESHAPE.  scale_inv is [rows, cols/128] row-major.
 * rows == 0 or cols == 0 is a no-op.
 */
fp8q_status_t fp8q_cast_per_group128(const void* x, fp8q_dtype_t xdtype, int64_t rows, int64_t cols, fp8q_fmt_t fmt,
                                     uint8_t* q, float* scale_inv, void* stream);

/*
 * The same per-128-group cast computed in another kernel shape, one 64-lane
 * wavefront per group with two elements per lane (4-byte loads, 2-byte code
 * stores), kept so that the shape can be measured beside the kernel that
 * fp8q_cast_per_group128 uses; the results are identical.  On MI355X it is
 * about half as fast as fp8q_cast_per_group128.  Arguments, layout and errors
 * as fp8q_cast_per_group128, and also: x not aligned to two elements or q not
 * to 2 bytes -> FP8Q_EALIGN.
 */
fp8q_status_t fp8q_cast_per_group128_wave64(const void* x, fp8q_dtype_t xdtype, int64_t rows, int64_t cols,
                                            fp8q_fmt_t fmt, uint8_t* q, float* scale_inv, void* stream);

/*
 * Per-tensor dequant (ColossalAI fp8.py, cast_from_fp8, per-tensor):
 *   y[i] = ydtype(fp32(q[i]) * scale_inv[0]) -- the binary32 product rounded
 * once more to bf16/fp16 when ydtype is not F32.  n == 0 is a no-op.
 */
fp8q_status_t fp8q_dequant_per_tensor(const uint8_t* q, fp8q_fmt_t fmt, int64_t n, const float* scale_inv,
                                      void* y, fp8q_dtype_t ydtype, void* stream);

/*
 * Per-channel dequant (ColossalAI fp8.py, cast_from_fp8, per_channel_scale=True):
 *   y[r, c] = ydtype(fp32(q[r, c]) * scale_inv[r]); scale_inv has `rows` floats.
 */
fp8q_status_t fp8q_dequant_per_channel(const uint8_t* q, fp8q_fmt_t fmt, int64_t rows, int64_t cols,
                                       const float* scale_inv, void* y, fp8q_dtype_t ydtype, void* stream);

/*
 * Per-128-group dequant, the inverse of per_token_cast_to_fp8 (DeepEP
 * "5 Utils" names it per_token_cast_back without showing it; this is the
 * plain reading, the same product as cast_from_fp8):
 *   y[r, c] = ydtype(fp32(q[r, c]) * scale_inv[r, c / 128]).
 * cols % 128 != 0 -> FP8Q_ESHAPE.
 */
fp8q_status_t fp8q_dequant_per_group128(const uint8_t* q, fp8q_fmt_t fmt, int64_t rows, int64_t cols,
                                        const float* scale_inv, void* y, fp8q_dtype_t ydtype, void* stream);

/*
 * 128x128 block weight dequant (CSDN "FP8 (8 bits) & FP16 (16 bits)",
 * weight_dequant and weight_dequant_kernel): q is [M, N]; scale_inv is
 * [ceil(M/128), ceil(N/128)] row-major; partial edge tiles are masked;
 *   y[i, j] = ydtype(fp32(q[i, j]) * scale_inv[(i/128) * ceil(N/128) + j/128]).
 * The page stores the product into a bf16 buffer (the default dtype), which
 * is ydtype = FP8Q_BF16; F32 and F16 outputs are also offered.
 */
fp8q_status_t fp8q_weight_dequant_block128(const uint8_t* q, fp8q_fmt_t fmt, int64_t M, int64_t N,
                                           const float* scale_inv, void* y, fp8q_dtype_t ydtype, void* stream);

/*
 * Cross-rank global scale, one rank's parts (ColossalAI fp8.py,
 * fp8_compress_fsdp_params_comm_hook).  The hook computes each rank's
 * per_tensor_max = where(max |x| > 0, max |x|, 1), all-reduces it with MAX,
 * casts with scale = fp8_max / per_tensor_max, all-gathers the fp8 payload
 * and dequantizes it with fp8.float() / scale.  The all-reduce and the
 * all-gather are the caller's (e.g. torch.distributed over RCCL).
 *
 * fp8q_amax_guarded: amax[0] = where(max |x| > 0, max |x|, 1) (a NaN amax or
 *   n == 0 also gives 1); same arguments and stages as fp8q_amax.
 * fp8q_cast_with_amax: scale = fp8_max / amax[0] (a correctly rounded
 *   binary32 division; amax is a device float, typically the all-reduced
 *   value), q[i] = fp8(fp32(x[i]) * scale) with the saturating rule (the given
 *   amax need not bound x), scale_out[0] = scale.  n == 0 writes only the scale.
 * fp8q_dequant_div_scale: y[i] = ydtype(fp32(q[i]) / scale[0]) -- a division by
 *   the scale, which rounds differently from a product with 1 / scale.
 */
fp8q_status_t fp8q_amax_guarded(const void* x, fp8q_dtype_t xdtype, int64_t n, float* amax, void* stream);
fp8q_status_t fp8q_cast_with_amax(const void* x, fp8q_dtype_t xdtype, int64_t n, fp8q_fmt_t fmt, const float* amax, uint8_t* q,
                                  float* scale_out, void* stream);
fp8q_status_t fp8q_dequant_div_scale(const uint8_t* q, fp8q_fmt_t fmt, int64_t n, const float* scale, void* y, fp8q_dtype_t ydtype,
                                     void* stream);

/*
 * Reduce step of an fp8-compressed reduce-scatter / all-reduce, on one rank
 * (ColossalAI fp8.py: _reduce_scatter_fp8's cast_op, _all_reduce_fp8 and the
 * DDP hook's sum_and_allgather).  The rank has received W fp8 chunks of n
 * elements, each cast per tensor by a different rank with its own scale_inv:
 *   q: [W][n] codes (chunk w at q + w * n); scale_inv: [W] floats;
 *   y[i] = sum over w in chunk order of ydtype(fp32(q[w][i]) * scale_inv[w]),
 *          accumulated in ydtype starting from +0 (summed_out = zeros, then
 *          summed_out += cast_from_fp8(...) per chunk: every term and every
 *          partial sum is rounded to ydtype);
 *   average != 0 (ReduceOp.AVG, and the DDP hook): y = ydtype(y / W), a
 *          correctly rounded binary32 division.
 * ydtype is the original tensor's type (input_type on the page).  W >= 1.
 * n == 0 is a no-op.
 */
fp8q_status_t fp8q_dequant_sum(const uint8_t* q, fp8q_fmt_t fmt, int64_t W, int64_t n, const float* scale_inv,
                               int average, void* y, fp8q_dtype_t ydtype, void* stream);

/*
 * fp8q_dequant_sum followed by cast_to_fp8 of the sum, per tensor
 * (_all_reduce_fp8: summed_out_fp8, scale = cast_to_fp8(summed_out)): y
 * receives the sum (it is also the intermediate), q_out[n] its fp8 codes in the
 * same format and scale_inv_out[0] = 1 / scale.  The amax of the sum is folded
 * into `workspace` (at least fp8q_per_tensor_workspace_bytes(), 4-byte
 * aligned, caller-owned) during the sum pass, so y is read once more, by the
 * cast pass.  n == 0 writes scale_inv_out[0] = 1.0 (the empty-tensor branch).
 */
fp8q_status_t fp8q_dequant_sum_requant(const uint8_t* q, fp8q_fmt_t fmt, int64_t W, int64_t n, const float* scale_inv,
                                       int average, void* y, fp8q_dtype_t ydtype, uint8_t* q_out, float* scale_inv_out,
                                       void* workspace, void* stream);

/*
 * Pipeline point-to-point cast with the fp8 format chosen from the data
 * (ColossalAI fp8.py, cast_to_fp8_pipeline and cast_from_fp8_pipeline).  The
 * page picks the format on the host after reading amax back; here the choice
 * is made on the device and handed on in a device word, so neither side
 * waits for the GPU.
 *
 * fp8q_cast_to_fp8_pipeline: amax = max(|min x|, |max x|) (NaN propagates);
 *   fmt_out[0] = FP8Q_E5M2 if amax > 448 (the e4m3fn maximum), else
 *   FP8Q_E4M3FN (also for a NaN amax); scale = 1 if amax == 0, else the chosen
 *   format's maximum / amax (correctly rounded binary32 division);
 *   q[i] = fp8(fp32(x[i]) * scale); scale_inv[0] = 1 / scale.  A NaN amax
 *   gives a NaN scale and NaN codes; an infinite amax gives scale 0.
 *   workspace: as for fp8q_cast_per_tensor.  n == 0 is read as amax 0
 *   (the page's aminmax raises on an empty tensor): scale_inv[0] = 1,
 *   fmt_out[0] = FP8Q_E4M3FN.  fmt_out is a device int32.
 * fp8q_cast_from_fp8_pipeline: fmt is the device int32 the cast wrote;
 *   y[i] = ydtype(ydtype(fp32(q[i])) * scale_inv[0]), the product taken in
 *   binary32 (the fp8 value converts exactly to every ydtype, so this equals
 *   fp8q_dequant_per_tensor in that format).  A format word other than 0 or 1
 *   (the page raises TypeError) writes NaN to every y.  n == 0 is a no-op.
 */
fp8q_status_t fp8q_cast_to_fp8_pipeline(const void* x, fp8q_dtype_t xdtype, int64_t n, uint8_t* q, float* scale_inv,
                                        int32_t* fmt_out, void* workspace, void* stream);
fp8q_status_t fp8q_cast_from_fp8_pipeline(const uint8_t* q, const int32_t* fmt, int64_t n, const float* scale_inv,
                                          void* y, fp8q_dtype_t ydtype, void* stream);

/*
 * Packed [scale_inv | payload] slots of the fp8 all-gather (ColossalAI
 * fp8.py, all_gather_fp8_lagacy and all_gather_fp8_ring).  The combined
 * buffer holds one slot per rank; slot w starts at byte w * (4 + n) and is
 * SCALE_BYTES = 4 bytes of binary32 scale_inv (little-endian) followed by the
 * rank's n fp8 codes.  The exchange itself is the caller's (e.g. RCCL
 * all-gather, or the ring's batched send/recv).
 *
 * fp8q_cast_to_packed: cast_to_fp8(x, per tensor) into one slot: codes at
 *   slot + 4, scale_inv at slot[0..3]; same numerics, stages and workspace
 *   as fp8q_cast_per_tensor.  slot holds 4 + n bytes and must be 4-byte
 *   aligned (the page views slot[0:4] as a float).  n == 0 writes 1.0.
 * fp8q_dequant_packed: the receive side for W slots in one launch: output w
 *   is y + w * n elements, y[w][i] = ydtype(fp32(code_w[i]) * scale_inv_w).
 *   slots must be 4-byte aligned and, when W > 1, n % 4 == 0 (otherwise
 *   FP8Q_EALIGN: the page's float view of a later slot's header needs it).
 *   W == 1 dequantizes one slot, the ring's per-step cast.  W == 0 or
 *   n == 0 is a no-op.
 */
fp8q_status_t fp8q_cast_to_packed(const void* x, fp8q_dtype_t xdtype, int64_t n, fp8q_fmt_t fmt, uint8_t* slot, void* workspace,
                                  void* stream);
fp8q_status_t fp8q_dequant_packed(const uint8_t* slots, fp8q_fmt_t fmt, int64_t W, int64_t n, void* y, fp8q_dtype_t ydtype,
                                  void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FP8Q_H */
