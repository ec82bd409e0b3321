// fp8q_kernels.hip -- host-side launchers of the FP8 scaled-cast kernels
// (fp8q_device.h) for gfx950.  Each launcher picks the vector kernel when the
// pointers and shape allow 16-byte lane vectors, the shifted-stream kernel
// (fp8q_shift.hip) for the flat operations when a pointer is aligned only to
// its element size, and an element-wise kernel otherwise; all produce
// identical bits.
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
#include "fp8q_host.h"

namespace fp8q {
namespace {

// clear the amax slots (a kernel rather than hipMemsetAsync, so the call
// can be captured into a HIP graph)
__global__ void k_fill_slots(uint32_t* p, int nslots, uint32_t v) {
    if ((int)threadIdx.x < nslots) p[threadIdx.x * kAmaxSlotStride] = v;
}

// where(amax > 0, amax, 1) in place (a NaN amax also becomes 1), on one word
__global__ void k_guard_amax(uint32_t* p) {
    if (threadIdx.x == 0) {
        const float v = __uint_as_float(p[0]);
        p[0] = __float_as_uint(v > 0.0f ? v : 1.0f);
    }
}

__global__ void k_fill_f32(float* p, int64_t n, float v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}


template <int DT, int FMT> struct RunGroup128 {
    static void run(const void* x, int64_t groups, uint8_t* q, float* sinv, hipStream_t st) {
        constexpr int VE = LaneVE<DT>::value;
        constexpr int64_t CH = kGroupK * (256 / (128 / VE));
        const unsigned nb = grid((groups + CH - 1) / CH);
        if (al(x, 16) && al(q, 4)) {
            k_group128<DT, FMT, kGroupK, kNT><<<nb, kThreads, 0, st>>>(x, q, sinv, groups);
        } else {
            launch_group128_shift(x, DT, groups, FMT, q, sinv, st);
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
            k_tensor_cast<DT, FMT, kFlatK, false><<<nb, kThreads, 0, st>>>(x, n, partial, np, pstride, q, sinv);
        } else if (vec) {
            launch_k(n / VE, [&](auto K, unsigned nb) {
                k_tensor_cast<DT, FMT, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(x, n, partial, np,
                                                                                               pstride, q, sinv);
            });
        } else {   // the shifted stream, with the amax pass's sub-steps per chunk (amax_plan)
            launch_tensor_cast_shift(x, DT, n, FMT, partial, np, pstride, q, sinv, st);
        }
    }
};

template <int DT, int FMT> struct RunCastGivenAmax {
    static void run(const void* x, int64_t n, const float* amax, uint8_t* q, float* scale_out, hipStream_t st) {
        constexpr int VE = LaneVE<DT>::value;
        if (al(x, 16) && al(q, 4)) {   // bf16 [4096, 4096]: 11.4 us with K = 4 against 12.1 with K = 2
            launch_k(n / VE, [&](auto K, unsigned nb) {
                k_cast_given_amax<DT, FMT, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(x, n, amax, q,
                                                                                                   scale_out);
            });
        } else {
            launch_cast_given_amax_shift(x, DT, n, FMT, amax, q, scale_out, st);
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
        // views aligned only to their element size: the shifted stream per row
        else if (!launch_channel_shift(x, DT, rows, cols, FMT, q, sinv, st))
            k_channel_2pass<DT, FMT><<<nb, kThreads, 0, st>>>(x, rows, cols, q, sinv);
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
        k_amax<DT, kAmaxK, kNT><<<(unsigned)std::min(std::max<int64_t>(chunks, 1), cap), kThreads, 0, st>>>(
            x, n, word, 1);
    } else {
        const int64_t mx = (int64_t)((uintptr_t)x & 15);
        const int64_t chunks = ((mx + n * ESize<DT>::value + 15) / 16 + kAmaxK * 256 - 1) / (kAmaxK * 256);
        k_amax_shift<DT, kAmaxK, kNT><<<(unsigned)std::min(std::max<int64_t>(chunks, 1), cap), kThreads, 0, st>>>(
            x, n, word, 1);
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
// The amax pass's sub-steps per chunk K (the cast pass's, so that chunk c is
// read by amax workgroup c mod kAmaxGrid and cast by workgroup c, both on XCD
// c mod 8) and its grid.  Aligned x: chunks of the lane vectors; otherwise
// chunks of the aligned 16-byte vectors that cover x (the shifted stream).
struct AmaxPlan {
    int K;
    int grid;
};
template <int DT> AmaxPlan amax_plan(const void* x, int64_t n) {
    constexpr int VE = LaneVE<DT>::value;
    int64_t u1, units;
    if (al(x, 16)) {
        u1 = (n / VE + 255) / 256;
        units = u1;
    } else {   // the shifted cast pass takes kShiftK sub-steps per chunk
        const int64_t mx = (int64_t)((uintptr_t)x & 15);
        units = ((mx + n * ESize<DT>::value + 15) / 16 + 255) / 256;
        return {kShiftK, (int)std::min(std::max<int64_t>((units + kShiftK - 1) / kShiftK, 1), kAmaxGrid)};
    }
    const int K = pick_flat_k(u1);
    return {K, (int)std::min(std::max<int64_t>((units + K - 1) / K, 1), kAmaxGrid)};
}

template <int DT> int amax_partials_grid(const void* x, int64_t n) { return amax_plan<DT>(x, n).grid; }

template <int DT> int run_amax_partials(const void* x, int64_t n, uint32_t* partial, hipStream_t st) {
    const AmaxPlan p = amax_plan<DT>(x, n);
    const int g = p.grid;
    if (al(x, 16)) {
        if (p.K == 8) k_amax<DT, 8, false, true><<<g, kThreads, 0, st>>>(x, n, partial, 0);
        else if (p.K == 4) k_amax<DT, 4, false, true><<<g, kThreads, 0, st>>>(x, n, partial, 0);
        else k_amax<DT, 2, false, true><<<g, kThreads, 0, st>>>(x, n, partial, 0);
    } else {
        k_amax_shift<DT, kShiftK, false, true><<<g, kThreads, 0, st>>>(x, n, partial, 0);
    }
    return g;
}

template <int FMT, int YDT> struct RunDequantFlat {
    template <int MODE> static void go(const uint8_t* q, int64_t n, const float* sinv, void* y, hipStream_t st) {
        constexpr int VE = LaneVE<YDT>::value;
        if (al(q, 4) && al(y, 16)) {
            launch_k(n / VE, [&](auto K, unsigned nb) {
                k_dequant_flat<FMT, YDT, MODE, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(q, n, sinv, y);
            });
        } else {
            launch_dequant_flat_shift(MODE, q, FMT, n, sinv, y, YDT, st);
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
            k_pipeline_cast<DT, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(x, n, partial, np, q, sinv,
                                                                                        fmt_out);
        });
    } else {
        launch_pipeline_cast_shift(x, DT, n, partial, np, q, sinv, fmt_out, st);
    }
}

template <int YDT> void run_dequant_pipeline(const uint8_t* q, int64_t n, const float* sinv, const int32_t* fmt,
                                             void* y, hipStream_t st) {
    constexpr int VE = LaneVE<YDT>::value;
    if (al(q, 4) && al(y, 16)) {   // as the per-tensor dequant: [4096, 4096] -> bf16 10.3 us against 11.6
        launch_k(n / VE, [&](auto K, unsigned nb) {
            k_dequant_pipeline<YDT, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(q, n, sinv, fmt, y);
        });
    } else {
        launch_dequant_pipeline_shift(q, n, sinv, fmt, y, YDT, st);
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
        const bool whole = cols % VE == 0;   // no lane vector straddles two rows
        const bool vec = whole && al(q, 4) && al(y, 16);
        const int64_t nvec = rows * (cols / VE);
        if (vec && nvec < (int64_t(1) << 32)) {
            const DivU32 dv = make_div((uint32_t)(cols / VE));
            launch_k(nvec, [&](auto K, unsigned nb) {
                k_dequant_rows_flat<FMT, YDT, decltype(K)::value, kNT><<<nb, kThreads, 0, st>>>(q, nvec, sinv, y, dv);
            });
        } else if (whole && nvec < (int64_t(1) << 32)) {
            launch_dequant_rows_shift(q, FMT, rows, cols, sinv, y, YDT, st);
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
