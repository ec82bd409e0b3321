// fp8q_host.h -- host-side launch helpers shared by the launcher sources
// (fp8q_kernels.hip, fp8q_shift.hip), and the shifted-stream launchers that
// fp8q_kernels.hip calls for views aligned to their element size only.
// Internal; not part of the ABI.
#pragma once
#include <algorithm>
#include <type_traits>

#include "fp8q_device.h"

namespace fp8q {

constexpr int kThreads = 256;
constexpr int64_t kGridCap = 1 << 20;   // grid-stride beyond this many workgroups
constexpr int64_t kAmaxGrid = kAmaxPartials;  // amax-pass workgroups (and partials)
constexpr int64_t kSumAmaxGrid = 8192;  // the reduce step's sum pass when it also folds the amax

constexpr int kGroupK = 2;        // sub-steps per group-cast chunk
constexpr int kShiftK = 4;        // sub-steps per chunk of the shifted flat kernels
constexpr int kFlatK = 2;         // sub-steps per flat chunk outside pick_flat_k's window
constexpr int kAmaxK = 2;         // sub-steps per amax chunk
constexpr int kBlockK = 2;        // sub-steps per block-dequant chunk
constexpr int kBlockRows = 1;     // rows per workgroup in the row-strip fallback
constexpr int kBlockU = 2;        // lane vectors per row per thread in flight there
constexpr int kSumKV = 2;         // lane vectors per thread in the reduce-step sum
constexpr bool kNT = true;        // non-temporal loads/stores for streaming data

inline bool al(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

inline unsigned grid(int64_t units) {
    int64_t b = units < 1 ? 1 : units;
    if (b > kGridCap) b = kGridCap;
    return (unsigned)b;
}

// invariant-divisor constants for dividing a 32-bit lane-vector index by d >= 1
inline DivU32 make_div(uint32_t d) {
    int l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    return DivU32{(uint32_t)((((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d) + 1), l};
}

template <int K> using KC = std::integral_constant<int, K>;

// Sub-steps per chunk (K) of a flat kernel over u1 = ceil(nvec / 256) chunks
// of one sub-step, with a grid covering the tensor.  K = 2 in general; a
// tensor whose K = 2 grid would take two to four dispatch rounds of
// workgroups (256 CUs x 8 resident workgroups = 2048 per round) instead gets
// the K that brings the grid to about one round.  Measured on the flat
// dequants, e4m3fn -> bf16 / fp32 from 2^20 to 2^27 elements: bf16 2^24
// 10.0 us with K = 4 against 11.4 us with K = 2; fp32 2^23 8.3-8.5 against
// 9.9 us; at 2^25 elements and above K = 2 is fastest again (bf16 2^27: 66.6
// us against 71.1 with K = 4), and below 2^23 the choice makes no difference.
inline int pick_flat_k(int64_t u1) {
    if (u1 > 4096 && u1 <= 8192) return 4;
    if (u1 > 8192 && u1 <= 16384) return 8;
    return 2;
}

// launch(KC<K>{}, grid) for the K pick_flat_k chooses over nvec lane vectors
template <typename L> void launch_k(int64_t nvec, L&& launch) {
    const int64_t u1 = (nvec + 255) / 256;
    const int K = pick_flat_k(u1);
    if (K == 8) launch(KC<8>{}, grid((u1 + 7) / 8));
    else if (K == 4) launch(KC<4>{}, grid((u1 + 3) / 4));
    else launch(KC<2>{}, grid((u1 + 1) / 2));
}

template <template <int, int> class F, typename... A>
void dispatch_dt_fmt(int dt, int fmt, A... a) {
    if (dt == kF32) { if (fmt == kE4M3) F<kF32, kE4M3>::run(a...); else F<kF32, kE5M2>::run(a...); }
    else if (dt == kBF16) { if (fmt == kE4M3) F<kBF16, kE4M3>::run(a...); else F<kBF16, kE5M2>::run(a...); }
    else { if (fmt == kE4M3) F<kF16, kE4M3>::run(a...); else F<kF16, kE5M2>::run(a...); }
}

template <template <int, int> class F, typename... A>
void dispatch_fmt_ydt(int fmt, int ydt, A... a) {
    if (fmt == kE4M3) {
        if (ydt == kF32) F<kE4M3, kF32>::run(a...); else if (ydt == kBF16) F<kE4M3, kBF16>::run(a...);
        else F<kE4M3, kF16>::run(a...);
    } else {
        if (ydt == kF32) F<kE5M2, kF32>::run(a...); else if (ydt == kBF16) F<kE5M2, kBF16>::run(a...);
        else F<kE5M2, kF16>::run(a...);
    }
}

// dword offset of p within its IB-byte vector, as a compile-time constant:
// f(KC<d>{}) for d = (p mod IB) / 4
template <int IB, typename F> void with_xdw(const void* p, F&& f) {
    const int d = (int)(((uintptr_t)p & (IB - 1)) >> 2);
    if constexpr (IB == 16) {
        if (d == 0) f(KC<0>{});
        else if (d == 1) f(KC<1>{});
        else if (d == 2) f(KC<2>{});
        else f(KC<3>{});
    } else if constexpr (IB == 8) {
        if (d == 0) f(KC<0>{});
        else f(KC<1>{});
    } else {
        f(KC<0>{});
    }
}

// Shifted-stream launchers (fp8q_shift.hip): the same operations as their
// vector counterparts, for x, q or y aligned to their element size only.
void launch_group128_shift(const void* x, int dt, int64_t groups, int fmt, uint8_t* q, float* sinv, hipStream_t st);
void launch_tensor_cast_shift(const void* x, int dt, int64_t n, int fmt, const uint32_t* partial, int np,
                              int pstride, uint8_t* q, float* sinv, hipStream_t st);
void launch_cast_given_amax_shift(const void* x, int dt, int64_t n, int fmt, const float* amax, uint8_t* q,
                                  float* scale_out, hipStream_t st);
void launch_pipeline_cast_shift(const void* x, int dt, int64_t n, const uint32_t* partial, int np, uint8_t* q,
                                float* sinv, int32_t* fmt_out, hipStream_t st);
// mode 0: per-tensor scale; 2: per-128-group scale; 3: division by sinv[0]
void launch_dequant_flat_shift(int mode, const uint8_t* q, int fmt, int64_t n, const float* sinv, void* y, int ydt,
                               hipStream_t st);
void launch_dequant_pipeline_shift(const uint8_t* q, int64_t n, const float* sinv, const int32_t* fmt, void* y,
                                   int ydt, hipStream_t st);
// the per-channel cast of rows of cols % VE == 0 and at most 2048 lane
// vectors; returns false (launching nothing) for other rows
bool launch_channel_shift(const void* x, int dt, int64_t rows, int64_t cols, int fmt, uint8_t* q, float* sinv,
                          hipStream_t st);
// per-channel: cols % VE == 0 and rows * cols / VE < 2^32
void launch_dequant_rows_shift(const uint8_t* q, int fmt, int64_t rows, int64_t cols, const float* sinv, void* y,
                               int ydt, hipStream_t st);

}  // namespace fp8q
