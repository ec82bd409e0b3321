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
// clears *ws, then folds max |x| (as binary32 bits) into it; n may be 0
void launch_amax(const void* x, int dt, int64_t n, uint32_t* ws, hipStream_t st);
void launch_tensor_cast(const void* x, int dt, int64_t n, int fmt, const uint32_t* ws, uint8_t* q, float* sinv,
                        hipStream_t st);
void launch_channel_cast(const void* x, int dt, int64_t rows, int64_t cols, int fmt, uint8_t* q, float* sinv,
                         hipStream_t st);
void launch_group128_cast(const void* x, int dt, int64_t groups, int fmt, uint8_t* q, float* sinv, hipStream_t st);
// mode 0: per-tensor scale; mode 2: per-128-group scale over a flat [rows * cols] with cols % 128 == 0
void launch_dequant_flat(int mode, const uint8_t* q, int fmt, int64_t n, const float* sinv, void* y, int ydt,
                         hipStream_t st);
void launch_dequant_rows(const uint8_t* q, int fmt, int64_t rows, int64_t cols, const float* sinv, void* y, int ydt,
                         hipStream_t st);
void launch_block128(const uint8_t* q, int fmt, int64_t M, int64_t N, const float* sinv, void* y, int ydt,
                     hipStream_t st);

}  // namespace fp8q
