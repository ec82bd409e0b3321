// fp8q_kernels.hip -- host-side launchers of the FP8 scaled-cast kernels
// (fp8q_device.h) for gfx950.  Each launcher picks the vector kernel when the
// pointers and shape allow 16-byte lane vectors and an element-wise kernel
// otherwise; both produce identical bits.
//
// Launch configuration (MI355X: 256 CUs in 8 XCDs, 64-wide wavefronts),
// chosen by sweeping K, grid size and the non-temporal hint on the
// activation, block-weight and gradient workloads: 256-thread workgroups,
// one chunk of K = 2 sub-steps per workgroup with a grid covering the whole
// tensor (measured faster than fewer, looping workgroups); non-temporal
// loads and stores for the streaming data (1.5-1.8x faster than cached).
// Flat dequants and casts (one-pass, and both passes of the two-pass ones)
// over 1-4 M lane vectors (8-32 M 16-bit elements, 4-16 M fp32 elements)
// take K = 4 or 8 instead (pick_flat_k), which brings their grid to about one
// dispatch round.  The reduce step and the packed dequant (a grid over W
// slots) keep K = 2.
// The amax passes are the exception: their grid is capped at kAmaxGrid
// workgroups that loop over chunks.  In the stand-alone amax every workgroup
// ends in one atomic max on a single word, and those serialise across the 8
// XCDs; in the two-pass casts each workgroup stores one partial, and every
// workgroup of the cast pass folds all of them.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "fp8q_device.h"

namespace fp8q {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kGridCap = 1 << 20;   // grid-stride beyond this many workgroups
constexpr int64_t kAmaxGrid = kAmaxPartials;  // amax-pass workgroups (and partials)
constexpr int64_t kSumAmaxGrid = 8192;  // the reduce step's sum pass when it also folds the amax

constexpr int kGroupK = 2;        // sub-steps per group-cast chunk
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


template <int DT, int FMT> struct RunGroup128 {
    static void run(const void* x, int64_t groups, uint8_t* q, float* sinv, hipStream_t st) {
        constexpr int VE = LaneVE<DT>::value;
        constexpr int64_t CH = kGroupK * (256 / (128 / VE));
        const unsigned nb = grid((groups + CH - 1) / CH);
        if (al(x, 16) && al(q, 4)) {
            k_group128<DT, FMT, kGroupK, kNT><<<nb, kThreads, 0, st>>>(x, q, sinv, groups);
        } else {
            // x is aligned to its element size (checked at the boundary), so
            // x mod 16 is a whole number of elements
            switch (((uintptr_t)x & 15) >> 2) {
                case 0: k_group128_shift<DT, FMT, kGroupK, 0><<<nb, kThreads, 0, st>>>(x, q, sinv, groups); break;
                case 1: k_group128_shift<DT, FMT, kGroupK, 1><<<nb, kThreads, 0, st>>>(x, q, sinv, groups); break;
                case 2: k_group128_shift<DT, FMT, kGroupK, 2><<<nb, kThreads, 0, st>>>(x, q, sinv, groups); break;
                default: k_group128_shift<DT, FMT, kGroupK, 3><<<nb, kThreads, 0, st>>>(x, q, sinv, groups); break;
            }
        }
    }
};

// the one-wavefront-per-group variant (x aligned to two elements, q to 2 bytes)
constexpr int kPairG = 8;          // groups per wave trip
template <int DT, int FMT> struct RunGroup128Wave64 {
    static void run(const void* x, int64_t groups, uint8_t* q, float* sinv, hipStream_t st) {
        const int64_t trips = (groups + kPairG - 1) / kPairG;
        k_group128_pair<DT, FMT, kPairG><<<grid((trips + 3) / 4), kThreads, 0, st>>>(x, q, sinv, groups);
    }
};

// The cast pass of a two-pass cast.  It takes the same sub-steps per chunk
// as the amax pass before it (pick_flat_k over the tensor's lane vectors, in
// both), so that chunk c is cast by workgroup c on the XCD whose L2 the amax
// pass loaded it into (amax workgroup c mod 1024).  A fatter cast chunk over
// K = 2 amax chunks broke that pairing (bf16 [4096, 4096]: 16.5 us against
// 15.1 us); fatter chunks in both passes keep it and gain (14.7 against
// 15.3 us; fp32 26.3 against 27.2).
// cached: ordinary loads and stores instead of non-temporal ones, for the
// reduce step's re-cast, whose input the sum pass has just written (90.4 us
// against 93.1 us for 8 x 2^25 e5m2 chunks); it folds amax slots, not
// partials, and keeps K = 2.
template <int DT, int FMT> struct RunTensorCast {
    static void run(const void* x, int64_t n, const uint32_t* partial, int np, int pstride, uint8_t* q, float* sinv,
                    bool cached, hipStream_t st) {
        constexpr int VE = LaneVE<DT>::value;
        const bool vec = al(x, 16) && al(q, 4);
        if (vec && cached) {
            const unsigned nb = grid((n / VE + kFlatK * 256 - 1) / (kFlatK * 256));
            k_tensor_cast<DT, FMT, true, kFlatK, false><<<nb, kThreads, 0, st>>>(x, n, partial, np, pstride, q, sinv);
        } else if (vec) {
            launch_k(n / VE, [&](auto K, unsigned nb) {
                k_tensor_cast<DT, FMT, true, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(x, n, partial, np,
                                                                                               pstride, q, sinv);
            });
        } else {
            k_tensor_cast<DT, FMT, false, kFlatK, kNT><<<grid((n + 255) / 256), kThreads, 0, st>>>(x, n, partial, np,
                                                                                                  pstride, q, sinv);
        }
    }
};

template <int DT, int FMT> struct RunCastGivenAmax {
    static void run(const void* x, int64_t n, const float* amax, uint8_t* q, float* scale_out, hipStream_t st) {
        constexpr int VE = LaneVE<DT>::value;
        if (al(x, 16) && al(q, 4)) {   // bf16 [4096, 4096]: 11.4 us with K = 4 against 12.1 with K = 2
            launch_k(n / VE, [&](auto K, unsigned nb) {
                k_cast_given_amax<DT, FMT, true, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(x, n, amax, q,
                                                                                                   scale_out);
            });
        } else {
            k_cast_given_amax<DT, FMT, false, kFlatK, kNT><<<grid((n + 255) / 256), kThreads, 0, st>>>(x, n, amax, q,
                                                                                                       scale_out);
        }
    }
};

// Per-channel cast.  16-bit rows of up to 512 lane vectors (4096 elements)
// take two rows per workgroup trip (their loads in flight together); wider
// rows and fp32 take one row per workgroup (fp32 [4096, 4096]: 17.0 us with
// one row, 17.2-17.9 us with two).
template <int DT, int FMT> struct RunChannel {
    static void run(const void* x, int64_t rows, int64_t cols, uint8_t* q, float* sinv, hipStream_t st) {
        constexpr int VE = LaneVE<DT>::value;
        const bool vec = (cols % VE == 0) && al(x, 16) && al(q, 4);
        const int64_t nvec = cols / VE;
        const unsigned nb = grid(rows);
        if constexpr (DT != kF32) {
            const unsigned nb2 = grid((rows + 1) / 2);
            if (vec && nvec <= 256) {
                k_channel_rows<DT, FMT, 1, 2, kNT><<<nb2, kThreads, 0, st>>>(x, rows, cols, q, sinv);
                return;
            }
            if (vec && nvec <= 512) {
                k_channel_rows<DT, FMT, 2, 2, kNT><<<nb2, kThreads, 0, st>>>(x, rows, cols, q, sinv);
                return;
            }
        }
        if (vec && nvec <= 256) k_channel_reg<DT, FMT, 1, kNT><<<nb, kThreads, 0, st>>>(x, rows, cols, q, sinv);
        else if (vec && nvec <= 512) k_channel_reg<DT, FMT, 2, kNT><<<nb, kThreads, 0, st>>>(x, rows, cols, q, sinv);
        else if (vec && nvec <= 1024) k_channel_reg<DT, FMT, 4, kNT><<<nb, kThreads, 0, st>>>(x, rows, cols, q, sinv);
        else if (vec && nvec <= 2048) k_channel_reg<DT, FMT, 8, kNT><<<nb, kThreads, 0, st>>>(x, rows, cols, q, sinv);
        // longer rows: two vector passes over the row (fp32 [256, 131072]: 46 us
        // against 347 us element-wise; bf16 [4000, 16400]: 44 against 120 us)
        else if (vec) k_channel_2pass_vec<DT, FMT, 8, kNT><<<nb, kThreads, 0, st>>>(x, rows, cols, q, sinv);
        else k_channel_2pass<DT, FMT><<<nb, kThreads, 0, st>>>(x, rows, cols, q, sinv);
    }
};

// The stand-alone amax (fp8q_amax, into one caller word): its grid is capped
// at kAmaxGrid workgroups looping over chunks, each ending in one atomic max
// on the word (measured on the gradient workload: 87 us with one word against
// 758 us with one chunk per workgroup, where the atomics serialise; 64 slots
// on separate lines would give 83 us but need a workspace).  Non-temporal
// loads: nothing re-reads x.
template <int DT> void run_amax(const void* x, int64_t n, uint32_t* word, hipStream_t st) {
    k_fill_slots<<<1, 64, 0, st>>>(word, 1, 0u);
    if (n == 0) return;
    constexpr int VE = LaneVE<DT>::value;
    const int64_t cap = kAmaxGrid;
    if (al(x, 16)) {
        const int64_t chunks = (n / VE + kAmaxK * 256 - 1) / (kAmaxK * 256);
        k_amax<DT, true, kAmaxK, kNT><<<(unsigned)std::min(std::max<int64_t>(chunks, 1), cap), kThreads, 0, st>>>(
            x, n, word, 1);
    } else {
        k_amax<DT, false, kAmaxK, false><<<(unsigned)std::min((n + 255) / 256, cap), kThreads, 0, st>>>(x, n, word,
                                                                                                       1);
    }
}

// The amax pass of a two-pass cast: at most kAmaxGrid workgroups, each
// storing one partial (no clearing, no atomics, no fold launch: the cast
// pass folds the partials itself).  Returns the number of partials.
// Ordinary (cached) loads: the cast pass re-reads x, and what this pass
// leaves in L2 and the Infinity Cache it gets for free (per-tensor cast,
// bf16 [4096, 4096]: 20.5 us against 26.9 us with non-temporal loads).
// Two launches instead of four (slot clear, atomics, slot fold): the bf16
// [4096, 4096] cast takes 16.4 us against 20.8 us, fp32 28.5 against 31.9.
// The vector amax pass takes the sub-steps per chunk its cast pass will take
// (pick_flat_k, see RunTensorCast); the element-wise one takes kAmaxK.
template <int DT> int amax_partials_grid(const void* x, int64_t n) {
    constexpr int VE = LaneVE<DT>::value;
    int64_t units = (n + 255) / 256;
    if (al(x, 16)) {
        const int64_t u1 = (n / VE + 255) / 256;
        const int K = pick_flat_k(u1);
        units = (u1 + K - 1) / K;
    }
    return (int)std::min(std::max<int64_t>(units, 1), kAmaxGrid);
}

template <int DT> int run_amax_partials(const void* x, int64_t n, uint32_t* partial, hipStream_t st) {
    constexpr int VE = LaneVE<DT>::value;
    const int g = amax_partials_grid<DT>(x, n);
    if (al(x, 16)) {
        const int K = pick_flat_k((n / VE + 255) / 256);
        if (K == 8) k_amax<DT, true, 8, false, true><<<g, kThreads, 0, st>>>(x, n, partial, 0);
        else if (K == 4) k_amax<DT, true, 4, false, true><<<g, kThreads, 0, st>>>(x, n, partial, 0);
        else k_amax<DT, true, 2, false, true><<<g, kThreads, 0, st>>>(x, n, partial, 0);
    } else {
        k_amax<DT, false, kAmaxK, false, true><<<g, kThreads, 0, st>>>(x, n, partial, 0);
    }
    return g;
}

template <int FMT, int YDT> struct RunDequantFlat {
    template <int MODE> static void go(const uint8_t* q, int64_t n, const float* sinv, void* y, hipStream_t st) {
        constexpr int VE = LaneVE<YDT>::value;
        if (al(q, 4) && al(y, 16)) {
            launch_k(n / VE, [&](auto K, unsigned nb) {
                k_dequant_flat<FMT, YDT, MODE, true, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(q, n, sinv, y);
            });
        } else {
            k_dequant_flat<FMT, YDT, MODE, false, kFlatK, kNT><<<grid((n + 255) / 256), kThreads, 0, st>>>(q, n, sinv,
                                                                                                           y);
        }
    }
    static void run(int mode, const uint8_t* q, int64_t n, const float* sinv, void* y, hipStream_t st) {
        if (mode == 0) go<0>(q, n, sinv, y, st);
        else if (mode == 3) go<3>(q, n, sinv, y, st);
        else go<2>(q, n, sinv, y, st);
    }
};

template <int DT> void run_pipeline_cast(const void* x, int64_t n, const uint32_t* partial, int np, uint8_t* q,
                                         float* sinv, int32_t* fmt_out, hipStream_t st) {
    constexpr int VE = LaneVE<DT>::value;
    if (al(x, 16) && al(q, 4)) {   // the amax pass's sub-steps per chunk (RunTensorCast)
        launch_k(n / VE, [&](auto K, unsigned nb) {
            k_pipeline_cast<DT, true, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(x, n, partial, np, q, sinv,
                                                                                        fmt_out);
        });
    } else {
        k_pipeline_cast<DT, false, kFlatK, kNT><<<grid((n + 255) / 256), kThreads, 0, st>>>(x, n, partial, np, q,
                                                                                             sinv, fmt_out);
    }
}

template <int YDT> void run_dequant_pipeline(const uint8_t* q, int64_t n, const float* sinv, const int32_t* fmt,
                                             void* y, hipStream_t st) {
    constexpr int VE = LaneVE<YDT>::value;
    if (al(q, 4) && al(y, 16)) {   // as the per-tensor dequant: [4096, 4096] -> bf16 10.3 us against 11.6
        launch_k(n / VE, [&](auto K, unsigned nb) {
            k_dequant_pipeline<YDT, true, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(q, n, sinv, fmt, y);
        });
    } else {
        k_dequant_pipeline<YDT, false, kFlatK, kNT><<<grid((n + 255) / 256), kThreads, 0, st>>>(q, n, sinv, fmt, y);
    }
}

template <int FMT, int YDT> struct RunDequantPacked {
    static void run(const uint8_t* slots, int64_t W, int64_t n, void* y, hipStream_t st) {
        constexpr int VE = LaneVE<YDT>::value;
        constexpr int64_t ESZ = ESize<YDT>::value;
        // payloads 4-byte aligned (slots aligned, and n % 4 == 0 when W > 1,
        // both checked by the caller) and every output row 16-B aligned
        const bool vec = al(slots, 4) && al(y, 16) && (W == 1 || (n * ESZ) % 16 == 0);
        const int64_t per_slot = vec ? (n / VE + kFlatK * 256 - 1) / (kFlatK * 256) : (n + 255) / 256;
        const dim3 g(grid(per_slot), (unsigned)std::min<int64_t>(W, 65535));
        if (vec) k_dequant_packed<FMT, YDT, true, kFlatK, kNT><<<g, kThreads, 0, st>>>(slots, W, n, y);
        else k_dequant_packed<FMT, YDT, false, kFlatK, kNT><<<g, kThreads, 0, st>>>(slots, W, n, y);
    }
};

template <int FMT, int YDT> struct RunDequantRows {
    static void run(const uint8_t* q, int64_t rows, int64_t cols, const float* sinv, void* y, hipStream_t st) {
        constexpr int VE = LaneVE<YDT>::value;
        const bool vec = (cols % VE == 0) && al(q, 4) && al(y, 16);
        const int64_t nvec = rows * (cols / VE);
        if (vec && nvec < (int64_t(1) << 32)) {
            const DivU32 dv = make_div((uint32_t)(cols / VE));
            launch_k(nvec, [&](auto K, unsigned nb) {
                k_dequant_rows_flat<FMT, YDT, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(q, nvec, sinv, y, dv);
            });
        } else if (vec) {
            k_dequant_rows<FMT, YDT, true, kNT><<<grid(rows), kThreads, 0, st>>>(q, rows, cols, sinv, y);
        } else {
            k_dequant_rows<FMT, YDT, false, kNT><<<grid(rows), kThreads, 0, st>>>(q, rows, cols, sinv, y);
        }
    }
};

template <int FMT, int YDT> struct RunBlock128 {
    static void run(const uint8_t* q, int64_t M, int64_t N, const float* sinv, void* y, hipStream_t st) {
        constexpr int VE = LaneVE<YDT>::value;
        const int64_t nbn = (N + 127) / 128;
        const int64_t nvec = M * (N / VE);
        if (N % VE == 0 && al(q, 4) && al(y, 16) && nvec < (int64_t(1) << 32)) {
            const uint32_t vpr = (uint32_t)(N / VE);
            const DivU32 dv = make_div(vpr);
            const int64_t chunks = (nvec + kBlockK * 256 - 1) / (kBlockK * 256);
            k_block128_flat<FMT, YDT, kBlockK, kNT><<<grid(chunks), kThreads, 0, st>>>(q, nvec, sinv, y, nbn, vpr, dv);
        } else if (N % VE == 0 && al(q, 4) && al(y, 16)) {
            k_block128_rows<FMT, YDT, kBlockRows, kBlockU, kNT>
                <<<grid((M + kBlockRows - 1) / kBlockRows), kThreads, 0, st>>>(q, M, N, sinv, y, nbn);
        } else {
            k_block128_s<FMT, YDT><<<grid(M), kThreads, 0, st>>>(q, M, N, sinv, y, nbn);
        }
    }
};

template <int FMT, int YDT> struct RunDequantSum {
    static void run(const uint8_t* q, int64_t W, int64_t n, const float* sinv, int average, void* y, uint32_t* ws,
                    hipStream_t st) {
        constexpr int VE = LaneVE<YDT>::value;
        constexpr int KV = kSumKV;
        const bool vec = (n % VE == 0) && al(q, 4) && al(y, 16);
        const int64_t units = vec ? (n / VE + 256 * KV - 1) / (256 * KV) : (n + 255) / 256;
        if (ws) {
            k_fill_slots<<<1, 64, 0, st>>>(ws, kAmaxSlots, 0u);
            const unsigned nb = (unsigned)std::min(std::max<int64_t>(units, 1), kSumAmaxGrid);
            // y is stored through the caches: the re-cast pass reads it next
            if (vec) k_dequant_sum<FMT, YDT, true, true, kNT, KV, false><<<nb, kThreads, 0, st>>>(q, W, n, sinv, average, y, ws, kAmaxSlots);
            else k_dequant_sum<FMT, YDT, false, true, kNT, KV><<<nb, kThreads, 0, st>>>(q, W, n, sinv, average, y, ws, kAmaxSlots);
        } else {
            if (vec) k_dequant_sum<FMT, YDT, true, false, kNT, KV><<<grid(units), kThreads, 0, st>>>(q, W, n, sinv, average, y, ws, 1);
            else k_dequant_sum<FMT, YDT, false, false, kNT, KV><<<grid(units), kThreads, 0, st>>>(q, W, n, sinv, average, y, ws, 1);
        }
    }
};

}  // namespace

void launch_dequant_sum(const uint8_t* q, int fmt, int64_t W, int64_t n, const float* sinv, int average, void* y,
                        int ydt, uint32_t* ws, hipStream_t st) {
    dispatch_fmt_ydt<RunDequantSum>(fmt, ydt, q, W, n, sinv, average, y, ws, st);
}

int amax_partials_count(const void* x, int dt, int64_t n) {
    if (dt == kF32) return amax_partials_grid<kF32>(x, n);
    if (dt == kBF16) return amax_partials_grid<kBF16>(x, n);
    return amax_partials_grid<kF16>(x, n);
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free per-tensor cast (the amax partials), in
// device memory the library holds: every GPU the library runs on gets its own
// copy of this array when the code object loads, kept until the process
// ends.  On the host, `scratch` is only a stand-in symbol: its device address
// on each GPU comes from hipGetSymbolAddress, looked up once per device with
// that device current, and only that address is handed to kernels.  Calls
// that overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint32_t scratch[kScratchWords];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<uint32_t*> g_scratch_addr[kMaxDevices];
}  // namespace

hipError_t scratch_words(hipStream_t st, uint32_t** out) {
    int dev = -1;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    uint32_t* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int cur = -1;
            if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
            void* a = nullptr;
            e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
            if (cur != dev) {
                const hipError_t e2 = hipSetDevice(cur);
                if (e == hipSuccess) e = e2;
            }
            if (e != hipSuccess) return e;
            if (a == nullptr) return hipErrorInvalidSymbol;
            p = (uint32_t*)a;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

void launch_fill_f32(float* p, int64_t n, float v, hipStream_t st) {
    k_fill_f32<<<grid((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(p, n, v);
}

void launch_amax(const void* x, int dt, int64_t n, uint32_t* word, hipStream_t st) {
    if (dt == kF32) run_amax<kF32>(x, n, word, st);
    else if (dt == kBF16) run_amax<kBF16>(x, n, word, st);
    else run_amax<kF16>(x, n, word, st);
}

int launch_amax_partials(const void* x, int dt, int64_t n, uint32_t* partial, hipStream_t st) {
    if (dt == kF32) return run_amax_partials<kF32>(x, n, partial, st);
    if (dt == kBF16) return run_amax_partials<kBF16>(x, n, partial, st);
    return run_amax_partials<kF16>(x, n, partial, st);
}

void launch_tensor_cast(const void* x, int dt, int64_t n, int fmt, const uint32_t* partial, int np, int pstride,
                        uint8_t* q, float* sinv, hipStream_t st, bool cached) {
    dispatch_dt_fmt<RunTensorCast>(dt, fmt, x, n, partial, np, pstride, q, sinv, cached, st);
}

void launch_guard_amax(uint32_t* ws, hipStream_t st) { k_guard_amax<<<1, 64, 0, st>>>(ws); }

void launch_cast_given_amax(const void* x, int dt, int64_t n, int fmt, const float* amax, uint8_t* q,
                            float* scale_out, hipStream_t st) {
    dispatch_dt_fmt<RunCastGivenAmax>(dt, fmt, x, n, amax, q, scale_out, st);
}

void launch_pipeline_cast(const void* x, int dt, int64_t n, const uint32_t* partial, int np, uint8_t* q,
                          float* sinv, int32_t* fmt_out, hipStream_t st) {
    if (dt == kF32) run_pipeline_cast<kF32>(x, n, partial, np, q, sinv, fmt_out, st);
    else if (dt == kBF16) run_pipeline_cast<kBF16>(x, n, partial, np, q, sinv, fmt_out, st);
    else run_pipeline_cast<kF16>(x, n, partial, np, q, sinv, fmt_out, st);
}

void launch_dequant_pipeline(const uint8_t* q, int64_t n, const float* sinv, const int32_t* fmt, void* y, int ydt,
                             hipStream_t st) {
    if (ydt == kF32) run_dequant_pipeline<kF32>(q, n, sinv, fmt, y, st);
    else if (ydt == kBF16) run_dequant_pipeline<kBF16>(q, n, sinv, fmt, y, st);
    else run_dequant_pipeline<kF16>(q, n, sinv, fmt, y, st);
}

void launch_dequant_packed(const uint8_t* slots, int fmt, int64_t W, int64_t n, void* y, int ydt, hipStream_t st) {
    dispatch_fmt_ydt<RunDequantPacked>(fmt, ydt, slots, W, n, y, st);
}

void launch_channel_cast(const void* x, int dt, int64_t rows, int64_t cols, int fmt, uint8_t* q, float* sinv,
                         hipStream_t st) {
    dispatch_dt_fmt<RunChannel>(dt, fmt, x, rows, cols, q, sinv, st);
}

void launch_group128_cast(const void* x, int dt, int64_t groups, int fmt, uint8_t* q, float* sinv,
                          hipStream_t st) {
    dispatch_dt_fmt<RunGroup128>(dt, fmt, x, groups, q, sinv, st);
}

void launch_group128_cast_wave64(const void* x, int dt, int64_t groups, int fmt, uint8_t* q, float* sinv,
                                 hipStream_t st) {
    dispatch_dt_fmt<RunGroup128Wave64>(dt, fmt, x, groups, q, sinv, st);
}

void launch_dequant_flat(int mode, const uint8_t* q, int fmt, int64_t n, const float* sinv, void* y, int ydt,
                         hipStream_t st) {
    dispatch_fmt_ydt<RunDequantFlat>(fmt, ydt, mode, q, n, sinv, y, st);
}

void launch_dequant_rows(const uint8_t* q, int fmt, int64_t rows, int64_t cols, const float* sinv, void* y,
                         int ydt, hipStream_t st) {
    dispatch_fmt_ydt<RunDequantRows>(fmt, ydt, q, rows, cols, sinv, y, st);
}

void launch_block128(const uint8_t* q, int fmt, int64_t M, int64_t N, const float* sinv, void* y, int ydt,
                     hipStream_t st) {
    dispatch_fmt_ydt<RunBlock128>(fmt, ydt, q, M, N, sinv, y, st);
}

}  // namespace fp8q
