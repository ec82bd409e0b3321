// fp8q_abi.cpp -- the C ABI declared in include/fp8q.h.
//
// Every entry point validates its arguments on the host first (pure C++, no
// HIP call, no side effect), so that each error code can be produced without
// a GPU; only then does it enqueue kernels on the caller's stream.  The
// library allocates nothing and keeps no state.
#include "fp8q.h"

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "fp8q_launch.h"

namespace {

bool valid_dtype(int dt) { return dt == FP8Q_F32 || dt == FP8Q_BF16 || dt == FP8Q_F16; }
bool valid_fmt(int f) { return f == FP8Q_E4M3FN || f == FP8Q_E5M2; }
int64_t esize(int dt) { return dt == FP8Q_F32 ? 4 : 2; }
bool aligned(const void* p, int64_t a) { return ((uintptr_t)p % (uintptr_t)a) == 0; }

// rows * cols * bytes_per_element without int64 overflow
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// byte ranges [a, a+an) and [b, b+bn) intersect (empty ranges never do)
bool overlap(const void* a, int64_t an, const void* b, int64_t bn) {
    if (an <= 0 || bn <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bn && b0 < a0 + (uintptr_t)an;
}

struct Buf {
    const void* p;
    int64_t bytes;
};

// pairwise overlap check over input/output buffers
bool any_overlap(const Buf* bufs, int n) {
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j)
            if (overlap(bufs[i].p, bufs[i].bytes, bufs[j].p, bufs[j].bytes)) return true;
    return false;
}

fp8q_status_t launched() { return hipGetLastError() == hipSuccess ? FP8Q_OK : FP8Q_EHIP; }

hipStream_t S(void* s) { return (hipStream_t)s; }

// common checks of a 2-D [rows, cols] high-precision <-> fp8 pair
fp8q_status_t check_2d(const void* hp, int hpdt, int64_t rows, int64_t cols, fp8q_fmt_t fmt, const void* q,
                       const float* sinv, int64_t sinv_count, int64_t* n_out) {
    if (!valid_dtype(hpdt) || !valid_fmt(fmt)) return FP8Q_EDTYPE;
    int64_t n, hpbytes, sbytes;
    if (!mul_ok(rows, cols, &n) || !mul_ok(n, esize(hpdt), &hpbytes) || !mul_ok(sinv_count, 4, &sbytes))
        return FP8Q_EINVAL;
    if (n > 0 && (!hp || !q)) return FP8Q_EINVAL;
    if (sinv_count > 0 && !sinv) return FP8Q_EINVAL;
    if ((hp && !aligned(hp, esize(hpdt))) || (sinv && !aligned(sinv, 4))) return FP8Q_EALIGN;
    const Buf b[3] = {{hp, hpbytes}, {q, n}, {sinv, sbytes}};
    if (any_overlap(b, 3)) return FP8Q_EINVAL;
    *n_out = n;
    return FP8Q_OK;
}

}  // namespace

extern "C" {

int fp8q_abi_version(void) { return FP8Q_ABI_VERSION; }

const char* fp8q_status_str(fp8q_status_t status) {
    switch (status) {
        case FP8Q_OK: return "FP8Q_OK";
        case FP8Q_EINVAL: return "FP8Q_EINVAL: invalid size, NULL pointer or overlapping buffers";
        case FP8Q_EDTYPE: return "FP8Q_EDTYPE: unsupported element type or fp8 format";
        case FP8Q_ESHAPE: return "FP8Q_ESHAPE: cols must be a multiple of 128";
        case FP8Q_EALIGN: return "FP8Q_EALIGN: pointer not aligned to its element size";
        case FP8Q_EHIP: return "FP8Q_EHIP: kernel launch failed";
        default: return "FP8Q: unknown status";
    }
}

size_t fp8q_per_tensor_workspace_bytes(void) {
    static_assert(fp8q::kAmaxPartials <= fp8q::kAmaxSlots * fp8q::kAmaxSlotStride, "partials must fit the workspace");
    return sizeof(uint32_t) * fp8q::kAmaxSlots * fp8q::kAmaxSlotStride;
}

fp8q_status_t fp8q_amax(const void* x, fp8q_dtype_t xdtype, int64_t n, float* amax, void* stream) {
    if (!valid_dtype(xdtype)) return FP8Q_EDTYPE;
    int64_t xbytes;
    if (n < 0 || !mul_ok(n, esize(xdtype), &xbytes)) return FP8Q_EINVAL;
    if (!amax || (n > 0 && !x)) return FP8Q_EINVAL;
    if (!aligned(amax, 4) || (x && !aligned(x, esize(xdtype)))) return FP8Q_EALIGN;
    if (overlap(x, xbytes, amax, 4)) return FP8Q_EINVAL;
    fp8q::launch_amax(x, xdtype, n, (uint32_t*)amax, S(stream));
    return launched();
}

fp8q_status_t fp8q_amax_guarded(const void* x, fp8q_dtype_t xdtype, int64_t n, float* amax, void* stream) {
    fp8q_status_t st = fp8q_amax(x, xdtype, n, amax, stream);
    if (st != FP8Q_OK) return st;
    fp8q::launch_guard_amax((uint32_t*)amax, S(stream));
    return launched();
}

fp8q_status_t fp8q_cast_with_amax(const void* x, fp8q_dtype_t xdtype, int64_t n, fp8q_fmt_t fmt, const float* amax, uint8_t* q,
                                  float* scale_out, void* stream) {
    if (n < 0) return FP8Q_EINVAL;
    int64_t nn;
    fp8q_status_t st = check_2d(x, xdtype, 1, n, fmt, q, scale_out, 1, &nn);
    if (st != FP8Q_OK) return st;
    if (!amax) return FP8Q_EINVAL;
    if (!aligned(amax, 4)) return FP8Q_EALIGN;
    const Buf b[4] = {{x, n * esize(xdtype)}, {q, n}, {scale_out, 4}, {amax, 4}};
    if (any_overlap(b, 4)) return FP8Q_EINVAL;
    // n == 0 still launches one workgroup: the scale is written, no element is
    fp8q::launch_cast_given_amax(x, xdtype, n, fmt, amax, q, scale_out, S(stream));
    return launched();
}

fp8q_status_t fp8q_dequant_div_scale(const uint8_t* q, fp8q_fmt_t fmt, int64_t n, const float* scale, void* y, fp8q_dtype_t ydtype,
                                     void* stream) {
    if (n < 0) return FP8Q_EINVAL;
    int64_t nn;
    fp8q_status_t st = check_2d(y, ydtype, 1, n, fmt, q, scale, n > 0 ? 1 : 0, &nn);
    if (st != FP8Q_OK) return st;
    if (n == 0) return FP8Q_OK;
    fp8q::launch_dequant_flat(3, q, fmt, n, scale, y, ydtype, S(stream));
    return launched();
}

fp8q_status_t fp8q_cast_to_fp8_pipeline(const void* x, fp8q_dtype_t xdtype, int64_t n, uint8_t* q, float* scale_inv,
                                        int32_t* fmt_out, void* workspace, void* stream) {
    if (n < 0) return FP8Q_EINVAL;
    int64_t nn;
    fp8q_status_t st = check_2d(x, xdtype, 1, n, FP8Q_E4M3FN, q, scale_inv, 1, &nn);
    if (st != FP8Q_OK) return st;
    if (!workspace || !fmt_out) return FP8Q_EINVAL;
    if (!aligned(workspace, 4) || !aligned(fmt_out, 4)) return FP8Q_EALIGN;
    const int64_t wsb = (int64_t)fp8q_per_tensor_workspace_bytes();
    const Buf b[5] = {{x, n * esize(xdtype)}, {q, n}, {scale_inv, 4}, {workspace, wsb}, {fmt_out, 4}};
    if (any_overlap(b, 5)) return FP8Q_EINVAL;
    // n == 0: the amax pass only clears the slots (amax 0); the cast launches
    // one workgroup that writes scale_inv and the format word
    const int np = fp8q::launch_amax_partials(x, xdtype, n, (uint32_t*)workspace, S(stream));
    fp8q::launch_pipeline_cast(x, xdtype, n, (const uint32_t*)workspace, np, q, scale_inv, fmt_out, S(stream));
    return launched();
}

fp8q_status_t fp8q_cast_from_fp8_pipeline(const uint8_t* q, const int32_t* fmt, int64_t n, const float* scale_inv,
                                          void* y, fp8q_dtype_t ydtype, void* stream) {
    if (n < 0) return FP8Q_EINVAL;
    int64_t nn;
    fp8q_status_t st = check_2d(y, ydtype, 1, n, FP8Q_E4M3FN, q, scale_inv, n > 0 ? 1 : 0, &nn);
    if (st != FP8Q_OK) return st;
    if (n == 0) return FP8Q_OK;
    if (!fmt) return FP8Q_EINVAL;
    if (!aligned(fmt, 4)) return FP8Q_EALIGN;
    const Buf b[3] = {{y, n * esize(ydtype)}, {q, n}, {fmt, 4}};
    if (any_overlap(b, 3)) return FP8Q_EINVAL;
    fp8q::launch_dequant_pipeline(q, n, scale_inv, fmt, y, ydtype, S(stream));
    return launched();
}

fp8q_status_t fp8q_cast_to_packed(const void* x, fp8q_dtype_t xdtype, int64_t n, fp8q_fmt_t fmt, uint8_t* slot, void* workspace,
                                  void* stream) {
    if (!valid_dtype(xdtype) || !valid_fmt(fmt)) return FP8Q_EDTYPE;
    int64_t xbytes;
    if (n < 0 || n > INT64_MAX - 4 || !mul_ok(n, esize(xdtype), &xbytes)) return FP8Q_EINVAL;
    if ((n > 0 && !x) || !slot || !workspace) return FP8Q_EINVAL;
    if ((x && !aligned(x, esize(xdtype))) || !aligned(slot, 4) || !aligned(workspace, 4)) return FP8Q_EALIGN;
    const int64_t wsb = (int64_t)fp8q_per_tensor_workspace_bytes();
    const Buf b[3] = {{x, xbytes}, {slot, 4 + n}, {workspace, wsb}};
    if (any_overlap(b, 3)) return FP8Q_EINVAL;
    if (n == 0) {  // cast_to_fp8's empty-tensor branch: scale_inv = 1.0 in the header
        fp8q::launch_fill_f32((float*)slot, 1, 1.0f, S(stream));
        return launched();
    }
    const int np = fp8q::launch_amax_partials(x, xdtype, n, (uint32_t*)workspace, S(stream));
    fp8q::launch_tensor_cast(x, xdtype, n, fmt, (const uint32_t*)workspace, np, 1, slot + 4, (float*)slot,
                             S(stream));
    return launched();
}

fp8q_status_t fp8q_dequant_packed(const uint8_t* slots, fp8q_fmt_t fmt, int64_t W, int64_t n, void* y, fp8q_dtype_t ydtype,
                                  void* stream) {
    if (!valid_dtype(ydtype) || !valid_fmt(fmt)) return FP8Q_EDTYPE;
    int64_t sbytes, ybytes;
    if (W < 0 || n < 0 || n > INT64_MAX - 4 || !mul_ok(W, 4 + n, &sbytes) || !mul_ok(W, n, &ybytes) ||
        !mul_ok(ybytes, esize(ydtype), &ybytes))
        return FP8Q_EINVAL;
    if (W == 0 || n == 0) return FP8Q_OK;
    if (!slots || !y) return FP8Q_EINVAL;
    if (!aligned(slots, 4) || !aligned(y, esize(ydtype)) || (W > 1 && n % 4 != 0)) return FP8Q_EALIGN;
    const Buf b[2] = {{slots, sbytes}, {y, ybytes}};
    if (any_overlap(b, 2)) return FP8Q_EINVAL;
    fp8q::launch_dequant_packed(slots, fmt, W, n, y, ydtype, S(stream));
    return launched();
}

fp8q_status_t fp8q_cast_per_tensor(const void* x, fp8q_dtype_t xdtype, int64_t n, fp8q_fmt_t fmt, uint8_t* q, float* scale_inv,
                                   void* workspace, void* stream) {
    if (n < 0) return FP8Q_EINVAL;
    int64_t nn;
    fp8q_status_t st = check_2d(x, xdtype, 1, n, fmt, q, scale_inv, 1, &nn);
    if (st != FP8Q_OK) return st;
    if (!workspace) return FP8Q_EINVAL;
    if (!aligned(workspace, 4)) return FP8Q_EALIGN;
    const int64_t wsb = (int64_t)fp8q_per_tensor_workspace_bytes();
    const Buf b[4] = {{x, n * esize(xdtype)}, {q, n}, {scale_inv, 4}, {workspace, wsb}};
    if (any_overlap(b, 4)) return FP8Q_EINVAL;
    if (n == 0) {  // cast_to_fp8's empty-tensor branch: scale_inv = [1.0]
        fp8q::launch_fill_f32(scale_inv, 1, 1.0f, S(stream));
        return launched();
    }
    const int np = fp8q::launch_amax_partials(x, xdtype, n, (uint32_t*)workspace, S(stream));
    fp8q::launch_tensor_cast(x, xdtype, n, fmt, (const uint32_t*)workspace, np, 1, q, scale_inv, S(stream));
    return launched();
}

fp8q_status_t fp8q_cast_per_tensor_noalloc(const void* x, fp8q_dtype_t xdtype, int64_t n, fp8q_fmt_t fmt, uint8_t* q,
                                           float* scale_inv, void* stream) {
    static_assert(fp8q::kAmaxPartials <= fp8q::kScratchWords, "the amax pass must fit the library scratch");
    if (n < 0) return FP8Q_EINVAL;
    int64_t nn;
    fp8q_status_t st = check_2d(x, xdtype, 1, n, fmt, q, scale_inv, 1, &nn);
    if (st != FP8Q_OK) return st;
    if (n == 0) {  // cast_to_fp8's empty-tensor branch: scale_inv = [1.0]
        fp8q::launch_fill_f32(scale_inv, 1, 1.0f, S(stream));
        return launched();
    }
    // the amax pass's grid is capped, so this holds for every n; checked
    // before anything is enqueued all the same
    if (fp8q::amax_partials_count(x, xdtype, n) > fp8q::kScratchWords) return FP8Q_EINVAL;
    uint32_t* partial = nullptr;
    if (fp8q::scratch_words(S(stream), &partial) != hipSuccess) return FP8Q_EHIP;
    const int np = fp8q::launch_amax_partials(x, xdtype, n, partial, S(stream));
    fp8q::launch_tensor_cast(x, xdtype, n, fmt, partial, np, 1, q, scale_inv, S(stream));
    return launched();
}

fp8q_status_t fp8q_cast_per_channel(const void* x, fp8q_dtype_t xdtype, int64_t rows, int64_t cols, fp8q_fmt_t fmt, uint8_t* q,
                                    float* scale_inv, void* stream) {
    int64_t n;
    fp8q_status_t st = check_2d(x, xdtype, rows, cols, fmt, q, scale_inv, rows, &n);
    if (st != FP8Q_OK) return st;
    if (rows == 0) return FP8Q_OK;
    if (cols == 0) {  // empty tensor: every row takes the empty branch's 1.0
        fp8q::launch_fill_f32(scale_inv, rows, 1.0f, S(stream));
        return launched();
    }
    fp8q::launch_channel_cast(x, xdtype, rows, cols, fmt, q, scale_inv, S(stream));
    return launched();
}

fp8q_status_t fp8q_cast_per_group128(const void* x, fp8q_dtype_t xdtype, int64_t rows, int64_t cols, fp8q_fmt_t fmt, uint8_t* q,
                                     float* scale_inv, void* stream) {
    if (!valid_dtype(xdtype) || !valid_fmt(fmt)) return FP8Q_EDTYPE;
    if (rows < 0 || cols < 0) return FP8Q_EINVAL;
    if (cols % 128 != 0) return FP8Q_ESHAPE;
    int64_t groups;
    if (!mul_ok(rows, cols / 128, &groups)) return FP8Q_EINVAL;
    int64_t n;
    fp8q_status_t st = check_2d(x, xdtype, rows, cols, fmt, q, scale_inv, groups, &n);
    if (st != FP8Q_OK) return st;
    if (n == 0) return FP8Q_OK;
    fp8q::launch_group128_cast(x, xdtype, groups, fmt, q, scale_inv, S(stream));
    return launched();
}

fp8q_status_t fp8q_cast_per_group128_wave64(const void* x, fp8q_dtype_t xdtype, int64_t rows, int64_t cols,
                                            fp8q_fmt_t fmt, uint8_t* q, float* scale_inv, void* stream) {
    if (!valid_dtype(xdtype) || !valid_fmt(fmt)) return FP8Q_EDTYPE;
    if (rows < 0 || cols < 0) return FP8Q_EINVAL;
    if (cols % 128 != 0) return FP8Q_ESHAPE;
    int64_t groups;
    if (!mul_ok(rows, cols / 128, &groups)) return FP8Q_EINVAL;
    int64_t n;
    fp8q_status_t st = check_2d(x, xdtype, rows, cols, fmt, q, scale_inv, groups, &n);
    if (st != FP8Q_OK) return st;
    if (n == 0) return FP8Q_OK;
    if (!aligned(x, 2 * esize(xdtype)) || !aligned(q, 2)) return FP8Q_EALIGN;
    fp8q::launch_group128_cast_wave64(x, xdtype, groups, fmt, q, scale_inv, S(stream));
    return launched();
}

fp8q_status_t fp8q_dequant_per_tensor(const uint8_t* q, fp8q_fmt_t fmt, int64_t n, const float* scale_inv, void* y,
                                      fp8q_dtype_t ydtype, void* stream) {
    if (n < 0) return FP8Q_EINVAL;
    int64_t nn;
    fp8q_status_t st = check_2d(y, ydtype, 1, n, fmt, q, scale_inv, n > 0 ? 1 : 0, &nn);
    if (st != FP8Q_OK) return st;
    if (n == 0) return FP8Q_OK;
    fp8q::launch_dequant_flat(0, q, fmt, n, scale_inv, y, ydtype, S(stream));
    return launched();
}

fp8q_status_t fp8q_dequant_per_channel(const uint8_t* q, fp8q_fmt_t fmt, int64_t rows, int64_t cols,
                                       const float* scale_inv, void* y, fp8q_dtype_t ydtype, void* stream) {
    int64_t n;
    fp8q_status_t st = check_2d(y, ydtype, rows, cols, fmt, q, scale_inv, cols > 0 ? rows : 0, &n);
    if (st != FP8Q_OK) return st;
    if (n == 0) return FP8Q_OK;
    fp8q::launch_dequant_rows(q, fmt, rows, cols, scale_inv, y, ydtype, S(stream));
    return launched();
}

fp8q_status_t fp8q_dequant_per_group128(const uint8_t* q, fp8q_fmt_t fmt, int64_t rows, int64_t cols,
                                        const float* scale_inv, void* y, fp8q_dtype_t ydtype, void* stream) {
    if (!valid_dtype(ydtype) || !valid_fmt(fmt)) return FP8Q_EDTYPE;
    if (rows < 0 || cols < 0) return FP8Q_EINVAL;
    if (cols % 128 != 0) return FP8Q_ESHAPE;
    int64_t groups;
    if (!mul_ok(rows, cols / 128, &groups)) return FP8Q_EINVAL;
    int64_t n;
    fp8q_status_t st = check_2d(y, ydtype, rows, cols, fmt, q, scale_inv, groups, &n);
    if (st != FP8Q_OK) return st;
    if (n == 0) return FP8Q_OK;
    fp8q::launch_dequant_flat(2, q, fmt, n, scale_inv, y, ydtype, S(stream));
    return launched();
}

fp8q_status_t fp8q_weight_dequant_block128(const uint8_t* q, fp8q_fmt_t fmt, int64_t M, int64_t N,
                                           const float* scale_inv, void* y, fp8q_dtype_t ydtype, void* stream) {
    if (M < 0 || N < 0) return FP8Q_EINVAL;
    int64_t nscale;  // ceil(M/128) * ceil(N/128), without overflowing M + 127
    if (!mul_ok(M / 128 + (M % 128 != 0), N / 128 + (N % 128 != 0), &nscale)) return FP8Q_EINVAL;
    int64_t n;
    fp8q_status_t st = check_2d(y, ydtype, M, N, fmt, q, scale_inv, nscale, &n);
    if (st != FP8Q_OK) return st;
    if (n == 0) return FP8Q_OK;
    fp8q::launch_block128(q, fmt, M, N, scale_inv, y, ydtype, S(stream));
    return launched();
}

// shared validation of the reduce-step entry points
static fp8q_status_t check_sum(const uint8_t* q, fp8q_fmt_t fmt, int64_t W, int64_t n, const float* scale_inv, const void* y,
                               fp8q_dtype_t ydtype, int64_t* qbytes, int64_t* ybytes, int64_t* sbytes) {
    if (!valid_dtype(ydtype) || !valid_fmt(fmt)) return FP8Q_EDTYPE;
    if (W < 1 || n < 0 || !mul_ok(W, n, qbytes) || !mul_ok(n, esize(ydtype), ybytes) || !mul_ok(W, 4, sbytes))
        return FP8Q_EINVAL;
    if (!scale_inv || (n > 0 && (!q || !y))) return FP8Q_EINVAL;
    if (!aligned(scale_inv, 4) || (y && !aligned(y, esize(ydtype)))) return FP8Q_EALIGN;
    return FP8Q_OK;
}

fp8q_status_t fp8q_dequant_sum(const uint8_t* q, fp8q_fmt_t fmt, int64_t W, int64_t n, const float* scale_inv, int average,
                               void* y, fp8q_dtype_t ydtype, void* stream) {
    int64_t qbytes, ybytes, sbytes;
    fp8q_status_t st = check_sum(q, fmt, W, n, scale_inv, y, ydtype, &qbytes, &ybytes, &sbytes);
    if (st != FP8Q_OK) return st;
    const Buf b[3] = {{q, qbytes}, {scale_inv, sbytes}, {y, ybytes}};
    if (any_overlap(b, 3)) return FP8Q_EINVAL;
    if (n == 0) return FP8Q_OK;
    fp8q::launch_dequant_sum(q, fmt, W, n, scale_inv, average, y, ydtype, nullptr, S(stream));
    return launched();
}

fp8q_status_t fp8q_dequant_sum_requant(const uint8_t* q, fp8q_fmt_t fmt, int64_t W, int64_t n, const float* scale_inv,
                                       int average, void* y, fp8q_dtype_t ydtype, uint8_t* q_out, float* scale_inv_out,
                                       void* workspace, void* stream) {
    int64_t qbytes, ybytes, sbytes;
    fp8q_status_t st = check_sum(q, fmt, W, n, scale_inv, y, ydtype, &qbytes, &ybytes, &sbytes);
    if (st != FP8Q_OK) return st;
    if (!scale_inv_out || !workspace || (n > 0 && !q_out)) return FP8Q_EINVAL;
    if (!aligned(scale_inv_out, 4) || !aligned(workspace, 4)) return FP8Q_EALIGN;
    const int64_t wsb = (int64_t)fp8q_per_tensor_workspace_bytes();
    const Buf b[6] = {{q, qbytes}, {scale_inv, sbytes}, {y, ybytes}, {q_out, n}, {scale_inv_out, 4}, {workspace, wsb}};
    if (any_overlap(b, 6)) return FP8Q_EINVAL;
    if (n == 0) {
        fp8q::launch_fill_f32(scale_inv_out, 1, 1.0f, S(stream));
        return launched();
    }
    fp8q::launch_dequant_sum(q, fmt, W, n, scale_inv, average, y, ydtype, (uint32_t*)workspace, S(stream));
    // the cast pass folds the amax slots the sum pass left in the workspace
    fp8q::launch_tensor_cast(y, ydtype, n, fmt, (const uint32_t*)workspace, fp8q::kAmaxSlots, fp8q::kAmaxSlotStride,
                             q_out, scale_inv_out, S(stream), true);
    return launched();
}

}  // extern "C"
