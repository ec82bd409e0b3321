// fp8q_shift.hip -- launchers of the shifted-stream kernels (fp8q_device.h,
// "shifted streaming"), for views aligned to their element size only: a
// tensor that starts a few elements into its buffer keeps 16-byte (or 8- /
// 4-byte fp8) lane vectors and aligned accesses instead of falling back to
// element-wise kernels.  The flat launchers take chunks of kShiftK = 4
// sub-steps and a grid that covers the tensor (the group cast keeps the
// aligned kernel's kGroupK, the per-channel cast one chunk per row).  Every
// launcher dispatches on the input's dword offset within its aligned vector
// (XDW), a compile-time constant of the kernel.  A translation unit of its
// own, so that the build compiles it beside fp8q_kernels.hip.
#include "fp8q_host.h"

namespace fp8q {
namespace {

// launch(KC<kShiftK>{}, grid) over nvec lane vectors: one size of chunk for
// the shifted flat kernels.  Each wave's set-up (span geometry, edge tests,
// the lane shuffles' boundary values) costs three to four times the scalar
// work of an aligned kernel's, and a longer span spreads it over more bytes.
// On the activation [16384, 7168], views two elements in, K = 4 against
// K = 2: fp32 dequant 101.6 against 116.2 us (K = 8: 109.4), group dequant
// 62.7 against 69.5, per-channel dequant 63.0 against 67.3, both passes of
// the per-tensor cast 103.3 against 108.0, bf16 dequant 63.4 against 65.3.
// A size-dependent K like the vector kernels' would multiply the
// instantiations, already one per input dword offset.
template <typename L> void launch_shift(int64_t nvec, L&& launch) {
    launch(KC<kShiftK>{}, grid((nvec + kShiftK * 256 - 1) / (kShiftK * 256)));
}

template <int DT, int FMT> struct RunGroup128Shift {
    static void run(const void* x, int64_t groups, uint8_t* q, float* sinv, hipStream_t st) {
        constexpr int VE = LaneVE<DT>::value;
        constexpr int64_t CH = kGroupK * (256 / (128 / VE));
        const unsigned nb = grid((groups + CH - 1) / CH);
        with_xdw<16>(x, [&](auto X) {
            k_group128_shift<DT, FMT, kGroupK, decltype(X)::value><<<nb, kThreads, 0, st>>>(x, q, sinv, groups);
        });
    }
};

template <int DT, int FMT> struct RunTensorCastShift {
    static void run(const void* x, int64_t n, const uint32_t* partial, int np, int pstride, uint8_t* q, float* sinv,
                    hipStream_t st) {
        constexpr int VE = LaneVE<DT>::value;
        with_xdw<16>(x, [&](auto X) {
            launch_shift((n + VE - 1) / VE, [&](auto K, unsigned nb) {
                k_tensor_cast_shift<DT, FMT, decltype(K)::value, kNT, decltype(X)::value>
                    <<<nb, kThreads, 0, st>>>(x, n, partial, np, pstride, q, sinv);
            });
        });
    }
};

template <int DT, int FMT> struct RunCastGivenAmaxShift {
    static void run(const void* x, int64_t n, const float* amax, uint8_t* q, float* scale_out, hipStream_t st) {
        constexpr int VE = LaneVE<DT>::value;
        with_xdw<16>(x, [&](auto X) {
            launch_shift((n + VE - 1) / VE, [&](auto K, unsigned nb) {
                k_cast_given_amax_shift<DT, FMT, decltype(K)::value, kNT, decltype(X)::value>
                    <<<nb, kThreads, 0, st>>>(x, n, amax, q, scale_out);
            });
        });
    }
};

template <int DT> void run_pipeline_cast_shift(const void* x, int64_t n, const uint32_t* partial, int np, uint8_t* q,
                                               float* sinv, int32_t* fmt_out, hipStream_t st) {
    constexpr int VE = LaneVE<DT>::value;
    with_xdw<16>(x, [&](auto X) {
        launch_shift((n + VE - 1) / VE, [&](auto K, unsigned nb) {
            k_pipeline_cast_shift<DT, decltype(K)::value, kNT, decltype(X)::value>
                <<<nb, kThreads, 0, st>>>(x, n, partial, np, q, sinv, fmt_out);
        });
    });
}

template <int FMT, int YDT> struct RunDequantFlatShift {
    template <int MODE> static void go(const uint8_t* q, int64_t n, const float* sinv, void* y, hipStream_t st) {
        constexpr int VE = LaneVE<YDT>::value;
        with_xdw<VE>(q, [&](auto X) {
            launch_shift((n + VE - 1) / VE, [&](auto K, unsigned nb) {
                k_dequant_flat_shift<FMT, YDT, MODE, decltype(K)::value, kNT, decltype(X)::value>
                    <<<nb, kThreads, 0, st>>>(q, n, sinv, y);
            });
        });
    }
    static void run(int mode, const uint8_t* q, int64_t n, const float* sinv, void* y, hipStream_t st) {
        if (mode == 0) go<0>(q, n, sinv, y, st);
        else if (mode == 3) go<3>(q, n, sinv, y, st);
        else go<2>(q, n, sinv, y, st);
    }
};

template <int YDT> void run_dequant_pipeline_shift(const uint8_t* q, int64_t n, const float* sinv, const int32_t* fmt,
                                                   void* y, hipStream_t st) {
    constexpr int VE = LaneVE<YDT>::value;
    with_xdw<VE>(q, [&](auto X) {
        launch_shift((n + VE - 1) / VE, [&](auto K, unsigned nb) {
            k_dequant_pipeline_shift<YDT, decltype(K)::value, kNT, decltype(X)::value>
                <<<nb, kThreads, 0, st>>>(q, n, sinv, fmt, y);
        });
    });
}

template <int FMT, int YDT> struct RunDequantRowsShift {
    static void run(const uint8_t* q, int64_t rows, int64_t cols, const float* sinv, void* y, hipStream_t st) {
        constexpr int VE = LaneVE<YDT>::value;
        const int64_t nvec = rows * (cols / VE);
        const DivU32 dv = make_div((uint32_t)(cols / VE));
        with_xdw<VE>(q, [&](auto X) {
            launch_shift(nvec, [&](auto K, unsigned nb) {
                k_dequant_rows_shift<FMT, YDT, decltype(K)::value, kNT, decltype(X)::value>
                    <<<nb, kThreads, 0, st>>>(q, nvec, sinv, y, dv);
            });
        });
    }
};

template <int DT, int FMT> struct RunChannelShift {
    static void run(const void* x, int64_t rows, int64_t cols, uint8_t* q, float* sinv, hipStream_t st, bool* done) {
        constexpr int VE = LaneVE<DT>::value;
        const int64_t nvec = cols / VE;
        *done = cols % VE == 0 && nvec <= 2048;
        if (!*done) return;
        with_xdw<16>(x, [&](auto X) {
            constexpr int XD = decltype(X)::value;
            if (nvec <= 512) k_channel_shift<DT, FMT, 2, XD><<<grid(rows), kThreads, 0, st>>>(x, rows, cols, q, sinv);
            else if (nvec <= 1024) k_channel_shift<DT, FMT, 4, XD><<<grid(rows), kThreads, 0, st>>>(x, rows, cols, q, sinv);
            else k_channel_shift<DT, FMT, 8, XD><<<grid(rows), kThreads, 0, st>>>(x, rows, cols, q, sinv);
        });
    }
};

}  // namespace

bool launch_channel_shift(const void* x, int dt, int64_t rows, int64_t cols, int fmt, uint8_t* q, float* sinv,
                          hipStream_t st) {
    bool done = false;
    dispatch_dt_fmt<RunChannelShift>(dt, fmt, x, rows, cols, q, sinv, st, &done);
    return done;
}

void launch_group128_shift(const void* x, int dt, int64_t groups, int fmt, uint8_t* q, float* sinv, hipStream_t st) {
    dispatch_dt_fmt<RunGroup128Shift>(dt, fmt, x, groups, q, sinv, st);
}

void launch_tensor_cast_shift(const void* x, int dt, int64_t n, int fmt, const uint32_t* partial, int np,
                              int pstride, uint8_t* q, float* sinv, hipStream_t st) {
    dispatch_dt_fmt<RunTensorCastShift>(dt, fmt, x, n, partial, np, pstride, q, sinv, st);
}

void launch_cast_given_amax_shift(const void* x, int dt, int64_t n, int fmt, const float* amax, uint8_t* q,
                                  float* scale_out, hipStream_t st) {
    dispatch_dt_fmt<RunCastGivenAmaxShift>(dt, fmt, x, n, amax, q, scale_out, st);
}

void launch_pipeline_cast_shift(const void* x, int dt, int64_t n, const uint32_t* partial, int np, uint8_t* q,
                                float* sinv, int32_t* fmt_out, hipStream_t st) {
    if (dt == kF32) run_pipeline_cast_shift<kF32>(x, n, partial, np, q, sinv, fmt_out, st);
    else if (dt == kBF16) run_pipeline_cast_shift<kBF16>(x, n, partial, np, q, sinv, fmt_out, st);
    else run_pipeline_cast_shift<kF16>(x, n, partial, np, q, sinv, fmt_out, st);
}

void launch_dequant_flat_shift(int mode, const uint8_t* q, int fmt, int64_t n, const float* sinv, void* y, int ydt,
                               hipStream_t st) {
    dispatch_fmt_ydt<RunDequantFlatShift>(fmt, ydt, mode, q, n, sinv, y, st);
}

void launch_dequant_pipeline_shift(const uint8_t* q, int64_t n, const float* sinv, const int32_t* fmt, void* y,
                                   int ydt, hipStream_t st) {
    if (ydt == kF32) run_dequant_pipeline_shift<kF32>(q, n, sinv, fmt, y, st);
    else if (ydt == kBF16) run_dequant_pipeline_shift<kBF16>(q, n, sinv, fmt, y, st);
    else run_dequant_pipeline_shift<kF16>(q, n, sinv, fmt, y, st);
}

void launch_dequant_rows_shift(const uint8_t* q, int fmt, int64_t rows, int64_t cols, const float* sinv, void* y,
                               int ydt, hipStream_t st) {
    dispatch_fmt_ydt<RunDequantRowsShift>(fmt, ydt, q, rows, cols, sinv, y, st);
}

}  // namespace fp8q
