// fp8q_launch.h -- internal interface between the C ABI layer (argument
// validation) and the HIP kernel launchers.  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// element types and fp8 formats (same numbering as the public enums)
enum { kF32 = 0, kBF16 = 1, kF16 = 2 };
enum { kE4M3 = 0, kE5M2 = 1 };

// All launchers enqueue on `st` and never synchronise.  Preconditions
// (checked by the ABI layer): sizes > 0 unless stated, pointers valid and
// aligned to their element size, buffers non-overlapping.
void launch_fill_f32(float* p, int64_t n, float v, hipStream_t st);
// Amax slots (the reduce step's re-cast): kAmaxSlots words, kAmaxSlotStride
// words (128 bytes) apart; the finished amax is their max, folded into slot 0.
constexpr int kAmaxSlots = 64;
constexpr int kAmaxSlotStride = 32;
// Amax partials (the two-pass casts): at most kAmaxPartials words, one per
// workgroup of the amax pass; the cast pass folds them.
constexpr int kAmaxPartials = 1024;
// the stand-alone amax: clears *word, then folds max |x| (binary32 bits) into
// it with one atomic max per workgroup; n may be 0
void launch_amax(const void* x, int dt, int64_t n, uint32_t* word, hipStream_t st);
// the amax pass of a two-pass cast: stores one partial max |x| per workgroup
// to partial[0 .. np) and returns np (1 <= np <= kAmaxPartials); n may be 0
int launch_amax_partials(const void* x, int dt, int64_t n, uint32_t* partial, hipStream_t st);
// the np that launch_amax_partials(x, dt, n, ...) would use, without launching
int amax_partials_count(const void* x, int dt, int64_t n);
// Library-held scratch of the allocation-free per-tensor cast: kScratchWords
// words (the amax pass's partials) in a __device__ array, one copy per GPU.
// scratch_words stores the device address of the copy on `st`'s device
// (taken with hipGetSymbolAddress on the first call per device, with that
// device current) and returns the HIP error of that lookup.
constexpr int kScratchWords = kAmaxPartials;
hipError_t scratch_words(hipStream_t st, uint32_t** out);
// where(amax > 0, amax, 1) applied to ws[0]
void launch_guard_amax(uint32_t* ws, hipStream_t st);
// cast with scale = fp8_max / amax[0] (caller-supplied amax); scale_out[0] = scale
void launch_cast_given_amax(const void* x, int dt, int64_t n, int fmt, const float* amax, uint8_t* q,
                            float* scale_out, hipStream_t st);
// dequant of W packed [scale_inv | n codes] slots into y [W][n]
void launch_dequant_packed(const uint8_t* slots, int fmt, int64_t W, int64_t n, void* y, int ydt, hipStream_t st);
// pipeline cast with amax = max of partial[0 .. np): the format chosen on the
// device, written to fmt_out[0]
void launch_pipeline_cast(const void* x, int dt, int64_t n, const uint32_t* partial, int np, uint8_t* q,
                          float* sinv, int32_t* fmt_out, hipStream_t st);
// per-tensor dequant with the format read from fmt[0] on the device
void launch_dequant_pipeline(const uint8_t* q, int64_t n, const float* sinv, const int32_t* fmt, void* y, int ydt,
                             hipStream_t st);
// the scale-and-cast pass, with amax = max of partial[0], partial[pstride],
// ... (np words: the amax pass's partials with pstride 1, or the amax slots
// with pstride kAmaxSlotStride).  cached: ordinary instead of non-temporal
// memory accesses, for an input the previous kernel just wrote.
void launch_tensor_cast(const void* x, int dt, int64_t n, int fmt, const uint32_t* partial, int np, int pstride,
                        uint8_t* q, float* sinv, hipStream_t st, bool cached = false);
void launch_channel_cast(const void* x, int dt, int64_t rows, int64_t cols, int fmt, uint8_t* q, float* sinv,
                         hipStream_t st);
void launch_group128_cast(const void* x, int dt, int64_t groups, int fmt, uint8_t* q, float* sinv, hipStream_t st);
// the one-wavefront-per-group variant; x aligned to two elements, q to 2 bytes
void launch_group128_cast_wave64(const void* x, int dt, int64_t groups, int fmt, uint8_t* q, float* sinv,
                                 hipStream_t st);
// mode 0: per-tensor scale; mode 2: per-128-group scale over a flat [rows * cols] with cols % 128 == 0;
// mode 3: per-tensor division by sinv[0] (a scale, not its inverse)
void launch_dequant_flat(int mode, const uint8_t* q, int fmt, int64_t n, const float* sinv, void* y, int ydt,
                         hipStream_t st);
void launch_dequant_rows(const uint8_t* q, int fmt, int64_t rows, int64_t cols, const float* sinv, void* y, int ydt,
                         hipStream_t st);
void launch_block128(const uint8_t* q, int fmt, int64_t M, int64_t N, const float* sinv, void* y, int ydt,
                     hipStream_t st);
// y = chunk-ordered in-type sum of the W dequantized chunks of q (W x n), / W if average;
// with ws != nullptr, the kAmaxSlots slots of ws are cleared first and max |y| ends in those slots
// (their max: the cast pass folds them)
void launch_dequant_sum(const uint8_t* q, int fmt, int64_t W, int64_t n, const float* sinv, int average, void* y,
                        int ydt, uint32_t* ws, hipStream_t st);

}  // namespace fp8q
