// fp8q_device.h -- device helpers and HIP kernels of the FP8 scaled cast for
// gfx950 (CDNA4).  Included by fp8q_kernels.hip, which holds the launchers.
//
// Quantize: amax reduction (per tensor / per row / per 128-element group) ->
// scale = fp8_max / amax -> binary32 multiply -> hardware fp8 convert.
// Dequantize: hardware fp8 -> fp32 convert -> binary32 multiply by scale_inv
// -> fp32 / bf16 / fp16 store.
//
// Every path is HBM-bound (about 3 bytes per element against a handful of
// VALU ops).  The memory layout rule shared by all vector kernels: each lane
// owns one "lane vector" of VE consecutive elements whose wider side is 16
// bytes (VE = 8 for bf16/fp16, 4 for fp32), and lane t of a workgroup
// sub-step owns lane vector base + t, so every wave-level load or store
// instruction covers one contiguous span (1 KB on the 16-byte side, 256 or
// 512 B on the fp8 side) made of whole 128-byte lines.  Each thread issues K
// such loads before the first use, to keep enough bytes in flight per CU.
//
// amax is computed on the integer bit patterns of |x| (sign bit cleared):
// for non-negative IEEE values the unsigned order of the bits is the numeric
// order, +inf sorts above every finite value and every NaN above +inf, so an
// unsigned max is exact, order-independent and propagates NaN the way torch's
// max does (ColossalAI fp8.py cast_to_fp8; DeepEP "5 Utils"
// per_token_cast_to_fp8).  Cross-lane steps use DPP (no LDS) except the last
// cross-wave step of a row or workgroup reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q_launch.h"

namespace fp8q {

// ---------------------------------------------------------------------------
// formats, vector types, element helpers
// ---------------------------------------------------------------------------

template <int FMT> struct Fp8Fmt;
template <> struct Fp8Fmt<kE4M3> { static constexpr float max = 448.0f; };     // 1.75 * 2^8
template <> struct Fp8Fmt<kE5M2> { static constexpr float max = 57344.0f; };   // 1.75 * 2^15

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));   // 16 bytes
typedef unsigned int v2u __attribute__((ext_vector_type(2)));   // 8 bytes
// 8 bytes of fp8 codes at a 4-byte-aligned address (still one
// global_load/store_dwordx2: gfx950 takes dword-aligned multi-dword global
// accesses).  A packed slot's payload sits 4 bytes after its binary32 header.
typedef unsigned int v2u_a4 __attribute__((ext_vector_type(2), aligned(4)));

// elements per lane vector: the high-precision side is 16 bytes
template <int DT> struct LaneVE { static constexpr int value = (DT == kF32) ? 4 : 8; };
template <int DT> struct ESize { static constexpr int value = (DT == kF32) ? 4 : 2; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// packed max of |a| over the two 16-bit halves of a dword (bf16 or fp16 bits)
__device__ __forceinline__ u16x2 absmax16(u16x2 m, uint32_t w) {
    return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu));
}

// binary32 bits of |amax| from a 16-bit element's |bits|
template <int DT> __device__ __forceinline__ uint32_t abs16_to_f32bits(uint32_t b);
template <> __device__ __forceinline__ uint32_t abs16_to_f32bits<kBF16>(uint32_t b) { return b << 16; }
template <> __device__ __forceinline__ uint32_t abs16_to_f32bits<kF16>(uint32_t b) {
    return __float_as_uint((float)__builtin_bit_cast(_Float16, (uint16_t)b));
}

// Saturating clamp that keeps NaN (the comparison is false for NaN).  The
// hardware convert rounds to nearest even but does not saturate (e4m3fn
// gives NaN from 464 up, e5m2 gives inf from 61440 up).  When a = amax the
// scale fp8_max / a bounds every |x * scale| by fp8_max * (1 + 2^-23), which
// rounds to fp8_max, so the clamp is only needed when a != amax (amax NaN or
// zero, so a = 1) or when scale overflows to +inf (amax < fp8_max / FLT_MAX).
template <int FMT> __device__ __forceinline__ float sat(float v) {
    return fabsf(v) > Fp8Fmt<FMT>::max ? copysignf(Fp8Fmt<FMT>::max, v) : v;
}

// true when products can leave the fp8 range (see sat): amax not > 0 (NaN or
// zero, so a = 1) or an infinite scale
__device__ __forceinline__ bool needs_saturation(uint32_t amax_bits, float scale) {
    return !(__uint_as_float(amax_bits) > 0.0f) || __builtin_isinf(scale);
}

// four binary32 -> four fp8 codes in one dword (byte k = element k)
template <int FMT> __device__ __forceinline__ uint32_t enc4(float a, float b, float c, float d) {
    int r;
    if constexpr (FMT == kE4M3) {
        r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    } else {
        r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
        r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);
    }
    return (uint32_t)r;
}

template <int FMT> __device__ __forceinline__ uint8_t enc1(float a) {
    return (uint8_t)(enc4<FMT>(a, 0.0f, 0.0f, 0.0f) & 0xFFu);
}

// four fp8 codes (one dword) -> four binary32 (exact)
template <int FMT> __device__ __forceinline__ void dec4(uint32_t w, float* o) {
    if constexpr (FMT == kE4M3) {
        auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
        auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
        o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
    } else {
        auto lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
        auto hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
        o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
    }
}

template <int FMT> __device__ __forceinline__ float dec1(uint8_t c) {
    float o[4];
    dec4<FMT>((uint32_t)c, o);
    return o[0];
}

// binary32 -> bf16 pair (RNE, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The product must be rounded to binary32 before the fp16 conversion (two
// roundings, as in (scale_inv * q.float()).to(float16)).  Left alone, the
// compiler folds fmul + fptrunc into v_fma_mixlo_f16, which rounds the exact
// product once; the empty asm pins the binary32 value in a VGPR (no code).
__device__ __forceinline__ float pin_f32(float v) {
    asm("" : "+v"(v));
    return v;
}
__device__ __forceinline__ uint16_t to_f16(float a) { return __builtin_bit_cast(uint16_t, (_Float16)pin_f32(a)); }
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return (uint32_t)to_f16(a) | ((uint32_t)to_f16(b) << 16);
}

// ---------------------------------------------------------------------------
// vector memory access; NT = non-temporal (streaming) hint
// ---------------------------------------------------------------------------

template <bool NT> __device__ __forceinline__ v4u ld16(const void* p) {
    if constexpr (NT) return __builtin_nontemporal_load((const v4u*)p);
    else return *(const v4u*)p;
}
template <bool NT> __device__ __forceinline__ v2u ld8(const void* p) {  // p 4-byte aligned
    v2u_a4 t;
    if constexpr (NT) t = __builtin_nontemporal_load((const v2u_a4*)p);
    else t = *(const v2u_a4*)p;
    return v2u{t.x, t.y};
}
template <bool NT> __device__ __forceinline__ uint32_t ld4(const void* p) {
    if constexpr (NT) return __builtin_nontemporal_load((const uint32_t*)p);
    else return *(const uint32_t*)p;
}
template <bool NT> __device__ __forceinline__ void st16(void* p, v4u v) {
    if constexpr (NT) __builtin_nontemporal_store(v, (v4u*)p);
    else *(v4u*)p = v;
}
template <bool NT> __device__ __forceinline__ void st8(void* p, v2u v) {  // p 4-byte aligned
    const v2u_a4 t = {v.x, v.y};
    if constexpr (NT) __builtin_nontemporal_store(t, (v2u_a4*)p);
    else *(v2u_a4*)p = t;
}
template <bool NT> __device__ __forceinline__ void st4(void* p, uint32_t v) {
    if constexpr (NT) __builtin_nontemporal_store(v, (uint32_t*)p);
    else *(uint32_t*)p = v;
}

// ---------------------------------------------------------------------------
// lane reductions (unsigned max)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// max over each aligned group of L lanes (L = 8, 16, 32 or 64), result in
// every lane: quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror (lane i <-
// lane 7-i within 8), row_mirror (lane i <- lane 15-i within 16), then
// cross-row exchanges
template <int L> __device__ __forceinline__ uint32_t max_lanes(uint32_t v) {
    static_assert(L == 8 || L == 16 || L == 32 || L == 64, "lane group");
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));
    if constexpr (L >= 16) v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));
    if constexpr (L >= 32) v = umax(v, (uint32_t)__shfl_xor((int)v, 16, 64));
    if constexpr (L >= 64) v = umax(v, (uint32_t)__shfl_xor((int)v, 32, 64));
    return v;
}

// max over a 256-thread workgroup; result valid in every thread; every
// thread of the workgroup must call it (it contains barriers)
__device__ __forceinline__ uint32_t block_max256(uint32_t v, uint32_t* lds4) {
    v = max_lanes<64>(v);
    if ((threadIdx.x & 63) == 0) lds4[threadIdx.x >> 6] = v;
    __syncthreads();
    const uint32_t m = umax(umax(lds4[0], lds4[1]), umax(lds4[2], lds4[3]));
    __syncthreads();  // lds4 may be reused by the caller
    return m;
}

// ---------------------------------------------------------------------------
// lane vectors
// ---------------------------------------------------------------------------

// one lane's 16 bytes of high-precision input
template <int DT> struct HpVec {
    static constexpr int VE = LaneVE<DT>::value;
    v4u r;
    template <bool NT> __device__ __forceinline__ void load(const void* p) { r = ld16<NT>(p); }
    __device__ __forceinline__ uint32_t absmax_bits() const {
        if constexpr (DT == kF32) {
            return umax(umax(r.x & 0x7FFFFFFFu, r.y & 0x7FFFFFFFu), umax(r.z & 0x7FFFFFFFu, r.w & 0x7FFFFFFFu));
        } else {
            u16x2 m = {0, 0};
            m = absmax16(m, r.x); m = absmax16(m, r.y); m = absmax16(m, r.z); m = absmax16(m, r.w);
            return abs16_to_f32bits<DT>(umax(m[0], m[1]));
        }
    }
    __device__ __forceinline__ void widen(float* v) const {
        if constexpr (DT == kF32) {
            v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y);
            v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
        } else if constexpr (DT == kBF16) {
            v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x); v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
            v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z); v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
        } else {
            v[0] = f16_lo(r.x); v[1] = f16_hi(r.x); v[2] = f16_lo(r.y); v[3] = f16_hi(r.y);
            v[4] = f16_lo(r.z); v[5] = f16_hi(r.z); v[6] = f16_lo(r.w); v[7] = f16_hi(r.w);
        }
    }
};

// scale VE values and store their fp8 codes (VE bytes) at q
template <int FMT, bool SAT, int VE, bool NT>
__device__ __forceinline__ void scale_encode_store(const float* v, float scale, uint8_t* q) {
    float p[VE];
#pragma unroll
    for (int k = 0; k < VE; ++k) {
        p[k] = v[k] * scale;
        if constexpr (SAT) p[k] = sat<FMT>(p[k]);
    }
    if constexpr (VE == 8) {
        st8<NT>(q, v2u{enc4<FMT>(p[0], p[1], p[2], p[3]), enc4<FMT>(p[4], p[5], p[6], p[7])});
    } else {
        st4<NT>(q, enc4<FMT>(p[0], p[1], p[2], p[3]));
    }
}

// load VE fp8 codes and decode them to binary32 multiplied by s
template <int FMT, int VE, bool NT> struct Fp8Vec {
    uint32_t w[VE / 4];
    __device__ __forceinline__ void load(const uint8_t* p) {
        if constexpr (VE == 8) { const v2u t = ld8<NT>(p); w[0] = t.x; w[1] = t.y; }
        else w[0] = ld4<NT>(p);
    }
    __device__ __forceinline__ void decode_scaled(float s, float* o) const {
#pragma unroll
        for (int k = 0; k < VE / 4; ++k) dec4<FMT>(w[k], o + 4 * k);
#pragma unroll
        for (int k = 0; k < VE; ++k) o[k] = o[k] * s;
    }
};

// store 16 bytes of output (4 fp32 or 8 bf16/fp16) at y + e elements
template <int YDT, bool NT> __device__ __forceinline__ void store_out16(void* y, int64_t e, const float* p) {
    if constexpr (YDT == kF32) {
        st16<NT>((float*)y + e, v4u{__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]),
                                    __float_as_uint(p[3])});
    } else if constexpr (YDT == kBF16) {
        st16<NT>((uint16_t*)y + e, v4u{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                       pack_bf16x2(p[6], p[7])});
    } else {
        st16<NT>((uint16_t*)y + e, v4u{pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]), pack_f16x2(p[4], p[5]),
                                       pack_f16x2(p[6], p[7])});
    }
}

template <int DT> __device__ __forceinline__ float load1(const void* x, int64_t i) {
    if constexpr (DT == kF32) return ((const float*)x)[i];
    else if constexpr (DT == kBF16) return __uint_as_float((uint32_t)((const uint16_t*)x)[i] << 16);
    else return (float)((const _Float16*)x)[i];
}

template <int DT> __device__ __forceinline__ uint32_t absbits1(const void* x, int64_t i) {
    if constexpr (DT == kF32) return ((const uint32_t*)x)[i] & 0x7FFFFFFFu;
    else return abs16_to_f32bits<DT>(((const uint16_t*)x)[i] & 0x7FFFu);
}

template <int YDT> __device__ __forceinline__ void store1(void* y, int64_t e, float p) {
    if constexpr (YDT == kF32) ((float*)y)[e] = p;
    else if constexpr (YDT == kBF16) ((uint16_t*)y)[e] = (uint16_t)(pack_bf16x2(p, 0.0f) & 0xFFFFu);
    else ((uint16_t*)y)[e] = to_f16(p);
}

// ===========================================================================
// per-128-group cast (DeepEP "5 Utils", per_token_cast_to_fp8)
// ===========================================================================

// Group scale from the group's amax (clamped at binary32 1e-4 = 0x38D1B717;
// the comparison form keeps a NaN amax as NaN, like torch.clamp).  For every
// element |x| <= amax, so |x * scale| <= fp8_max (1 + 2^-23): no clamp needed.
template <int FMT> __device__ __forceinline__ void group_scale(uint32_t amax_bits, float& scale, float& sinv) {
    float amax = __uint_as_float(amax_bits);
    const float lo = 1e-4f;
    if (amax < lo) amax = lo;
    scale = Fp8Fmt<FMT>::max / amax;
    sinv = amax / Fp8Fmt<FMT>::max;
}

// Vector path (x 16-B aligned, q 4-byte aligned).  A group of 128
// elements is LPG = 128 / VE consecutive lanes (16 for bf16/fp16, 32 for
// fp32); a workgroup sub-step covers 256 lane vectors = GPS whole groups, and
// one workgroup trip covers a chunk of K sub-steps (K * GPS consecutive
// groups, whose scale_inv entries fill whole cache lines).  NTHR is the
// workgroup size.  Groups are
// consecutive 128-element chunks of the flat array because cols % 128 == 0,
// and group g's scale_inv lives at flat index g.
template <int DT, int FMT, int K, bool NT, int NTHR = 256>
__global__ void __launch_bounds__(NTHR)
k_group128(const void* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ sinv_out, int64_t groups) {
    constexpr int VE = LaneVE<DT>::value;
    constexpr int ESZ = ESize<DT>::value;
    constexpr int LPG = 128 / VE;
    constexpr int GPS = NTHR / LPG;
    constexpr int CH = K * GPS;
    const int lig = threadIdx.x % LPG;  // lane in group
    const int gis = threadIdx.x / LPG;  // group in sub-step
    const int64_t nchunks = (groups + CH - 1) / CH;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        HpVec<DT> v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t g = c * CH + k * GPS + gis;
            if (g < groups) v[k].template load<NT>((const char*)x + (g * 128 + lig * VE) * ESZ);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t g = c * CH + k * GPS + gis;
            if (g < groups) {  // uniform within the LPG lanes of a group
                const uint32_t amax = max_lanes<LPG>(v[k].absmax_bits());
                float scale, sinv;
                group_scale<FMT>(amax, scale, sinv);
                float f[VE];
                v[k].widen(f);
                scale_encode_store<FMT, false, VE, NT>(f, scale, q + g * 128 + lig * VE);
                // a cached store: the chunk's scale_inv entries merge into whole
                // lines in L2 before write-back
                if (lig == 0) sinv_out[g] = sinv;
            }
        }
    }
}

// Unaligned path: one wavefront per group, two elements per lane,
// element-wise loads and byte stores; correct for any alignment of x (to its
// element size) and q.
template <int DT, int FMT>
__global__ void __launch_bounds__(256)
k_group128_wave(const void* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ sinv_out, int64_t groups) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
    for (int64_t g = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64; g < groups; g += waves) {
        const int64_t e0 = g * 128 + 2 * lane;
        const uint32_t m = max_lanes<64>(umax(absbits1<DT>(x, e0), absbits1<DT>(x, e0 + 1)));
        float scale, sinv;
        group_scale<FMT>(m, scale, sinv);
        const uint32_t w = enc4<FMT>(load1<DT>(x, e0) * scale, load1<DT>(x, e0 + 1) * scale, 0.0f, 0.0f);
        q[e0] = (uint8_t)(w & 0xFF);
        q[e0 + 1] = (uint8_t)((w >> 8) & 0xFF);
        if (lane == 0) sinv_out[g] = sinv;
    }
}

// ===========================================================================
// per-tensor (ColossalAI fp8.py, cast_to_fp8, per-tensor branch): global
// amax (stage 1 per workgroup, stage 2 an atomic max on the binary32 bits)
// then the scale-and-cast pass
// ===========================================================================

// Amax slots: stage 2 of the global amax is an atomic max of each
// workgroup's result into slot (workgroup % nslots); slot i is the word at
// i * kAmaxSlotStride, one slot per 128-byte line.  Device-scope atomics
// serialise per cache line, so slots sharing a line gain nothing.

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

// VEC (x 16-B aligned): chunks of K sub-steps x 256 lane vectors per
// workgroup trip; the n % VE tail element-wise by workgroup 0.
// Stage 2: with PART, workgroup b stores its result to amax_bits[b] (one
// partial per workgroup, every workgroup writes, so nothing needs clearing
// and the consumer folds the partials); otherwise an atomic max of each
// workgroup's result into one of `nslots` amax slots (workgroup b uses slot
// b % nslots).
template <int DT, bool VEC, int K, bool NT, bool PART = false>
__global__ void __launch_bounds__(256)
k_amax(const void* __restrict__ x, int64_t n, uint32_t* __restrict__ amax_bits, int nslots) {
    __shared__ uint32_t lds[4];
    constexpr int VE = LaneVE<DT>::value;
    constexpr int ESZ = ESize<DT>::value;
    uint32_t m = 0;
    int64_t done = 0;
    if constexpr (VEC) {
        const int64_t nvec = n / VE;
        const int64_t nchunks = (nvec + K * 256 - 1) / (K * 256);
        for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
            HpVec<DT> v[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int64_t vi = (c * K + k) * 256 + threadIdx.x;
                if (vi < nvec) v[k].template load<NT>((const char*)x + vi * VE * ESZ);
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int64_t vi = (c * K + k) * 256 + threadIdx.x;
                if (vi < nvec) m = umax(m, v[k].absmax_bits());
            }
        }
        done = nvec * VE;
        if (blockIdx.x == 0 && done + threadIdx.x < n) m = umax(m, absbits1<DT>(x, done + threadIdx.x));
    } else {
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
            m = umax(m, absbits1<DT>(x, i));
    }
    m = block_max256(m, lds);
    if constexpr (PART) {
        if (threadIdx.x == 0) amax_bits[blockIdx.x] = m;
    } else {
        if (threadIdx.x == 0 && m != 0) atomicMax(amax_bits + (blockIdx.x % nslots) * kAmaxSlotStride, m);
    }
}

// max over the np partials partial[0], partial[stride], ... (binary32 bits
// of |x|: the amax pass's per-workgroup partials, stride 1, or the amax
// slots, stride kAmaxSlotStride); every thread of the workgroup must call it
// (it contains barriers)
__device__ __forceinline__ uint32_t fold_partials(const uint32_t* __restrict__ partial, int np, int stride,
                                                  uint32_t* lds4) {
    uint32_t a = 0;
    for (int j = threadIdx.x; j < np; j += 256) a = umax(a, partial[j * stride]);
    return block_max256(a, lds4);
}

// scale from the finished amax: a = amax > 0 ? amax : 1 (NaN -> 1),
// scale = fp8_max / a, scale_inv = 1 / scale
template <int FMT> __device__ __forceinline__ void tensor_scale(uint32_t amax_bits, float& scale, float& sinv) {
    const float amax = __uint_as_float(amax_bits);
    const float a = (amax > 0.0f) ? amax : 1.0f;
    scale = Fp8Fmt<FMT>::max / a;
    sinv = 1.0f / scale;
}

template <int DT, int FMT, bool VEC, int K, bool NT, bool SAT>
__device__ __forceinline__ void tensor_cast_body(const void* __restrict__ x, int64_t n, float scale,
                                                 uint8_t* __restrict__ q) {
    constexpr int VE = LaneVE<DT>::value;
    constexpr int ESZ = ESize<DT>::value;
    if constexpr (VEC) {
        const int64_t nvec = n / VE;
        const int64_t nchunks = (nvec + K * 256 - 1) / (K * 256);
        for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
            HpVec<DT> v[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int64_t vi = (c * K + k) * 256 + threadIdx.x;
                if (vi < nvec) v[k].template load<NT>((const char*)x + vi * VE * ESZ);
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int64_t vi = (c * K + k) * 256 + threadIdx.x;
                if (vi < nvec) {
                    float f[VE];
                    v[k].widen(f);
                    scale_encode_store<FMT, SAT, VE, NT>(f, scale, q + vi * VE);
                }
            }
        }
        const int64_t i = nvec * VE + threadIdx.x;
        if (blockIdx.x == 0 && i < n) {
            float p = load1<DT>(x, i) * scale;
            if constexpr (SAT) p = sat<FMT>(p);
            q[i] = enc1<FMT>(p);
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
            float p = load1<DT>(x, i) * scale;
            if constexpr (SAT) p = sat<FMT>(p);
            q[i] = enc1<FMT>(p);
        }
    }
}

// The two-pass casts' second pass.  A workgroup first issues the loads of
// its first chunk, then folds the amax partials (their latency hides behind
// those loads), then scales and converts; with more chunks than workgroups
// it loops over the rest.
template <int DT, int K, bool NT>
__device__ __forceinline__ void chunk_load(HpVec<DT>* v, const void* __restrict__ x, int64_t nvec, int64_t c) {
    constexpr int VE = LaneVE<DT>::value;
    constexpr int ESZ = ESize<DT>::value;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t vi = (c * K + k) * 256 + threadIdx.x;
        if (vi < nvec) v[k].template load<NT>((const char*)x + vi * VE * ESZ);
    }
}

// cast the chunks of this workgroup (the first one already in v) and, in
// workgroup 0, the n % VE tail
template <int DT, int FMT, int K, bool NT, bool SAT>
__device__ __forceinline__ void cast_chunks(HpVec<DT>* v, const void* __restrict__ x, int64_t n, float scale,
                                            uint8_t* __restrict__ q) {
    constexpr int VE = LaneVE<DT>::value;
    const int64_t nvec = n / VE;
    const int64_t nchunks = (nvec + K * 256 - 1) / (K * 256);
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        if (c != (int64_t)blockIdx.x) chunk_load<DT, K, NT>(v, x, nvec, c);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t vi = (c * K + k) * 256 + threadIdx.x;
            if (vi < nvec) {
                float f[VE];
                v[k].widen(f);
                scale_encode_store<FMT, SAT, VE, NT>(f, scale, q + vi * VE);
            }
        }
    }
    const int64_t i = nvec * VE + threadIdx.x;
    if (blockIdx.x == 0 && i < n) {
        float p = load1<DT>(x, i) * scale;
        if constexpr (SAT) p = sat<FMT>(p);
        q[i] = enc1<FMT>(p);
    }
}

// VEC: x 16-B aligned and q 4-byte aligned.  The amax is the max of the np
// partials partial[0], partial[pstride], ...
template <int DT, int FMT, bool VEC, int K, bool NT>
__global__ void __launch_bounds__(256)
k_tensor_cast(const void* __restrict__ x, int64_t n, const uint32_t* __restrict__ partial, int np, int pstride,
              uint8_t* __restrict__ q, float* __restrict__ sinv_out) {
    __shared__ uint32_t lds[4];
    HpVec<DT> v[K];
    if constexpr (VEC) chunk_load<DT, K, NT>(v, x, n / LaneVE<DT>::value, blockIdx.x);
    const uint32_t ab = fold_partials(partial, np, pstride, lds);
    float scale, sinv;
    tensor_scale<FMT>(ab, scale, sinv);
    if (blockIdx.x == 0 && threadIdx.x == 0) sinv_out[0] = sinv;
    const bool saturate = needs_saturation(ab, scale);  // uniform
    if constexpr (VEC) {
        if (saturate) cast_chunks<DT, FMT, K, NT, true>(v, x, n, scale, q);
        else cast_chunks<DT, FMT, K, NT, false>(v, x, n, scale, q);
    } else {
        if (saturate) tensor_cast_body<DT, FMT, false, K, NT, true>(x, n, scale, q);
        else tensor_cast_body<DT, FMT, false, K, NT, false>(x, n, scale, q);
    }
}

// Cast with a caller-supplied amax (ColossalAI fp8.py,
// fp8_compress_fsdp_params_comm_hook: the guarded local amax reduced with MAX
// across ranks): scale = fp8_max / amax, scale_out[0] = scale.  The given
// amax need not bound this tensor's values, so the saturating path is always
// taken.
template <int DT, int FMT, bool VEC, int K, bool NT>
__global__ void __launch_bounds__(256)
k_cast_given_amax(const void* __restrict__ x, int64_t n, const float* __restrict__ amax, uint8_t* __restrict__ q,
                  float* __restrict__ scale_out) {
    const float scale = Fp8Fmt<FMT>::max / amax[0];
    if (blockIdx.x == 0 && threadIdx.x == 0) scale_out[0] = scale;
    tensor_cast_body<DT, FMT, VEC, K, NT, true>(x, n, scale, q);
}

// Pipeline p2p cast with the format chosen on the device (ColossalAI fp8.py,
// cast_to_fp8_pipeline): from the finished amax, e5m2 when amax > 448 (the
// e4m3fn maximum; a NaN amax fails the test) else e4m3fn; scale = 1 when
// amax == 0, else that format's maximum / amax; scale_inv = 1 / scale.
// Workgroup 0 publishes scale_inv and the format word (0 = e4m3fn,
// 1 = e5m2).  Every workgroup takes the same decision from the same
// partials, so the branches are uniform.
template <int DT, int FMT, bool VEC, int K, bool NT>
__device__ __forceinline__ void pipeline_cast_rest(HpVec<DT>* v, const void* __restrict__ x, int64_t n,
                                                   uint32_t ab, uint8_t* __restrict__ q,
                                                   float* __restrict__ sinv_out, int32_t* __restrict__ fmt_out) {
    const float amax = __uint_as_float(ab);
    const float scale = (amax == 0.0f) ? 1.0f : Fp8Fmt<FMT>::max / amax;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        sinv_out[0] = 1.0f / scale;
        fmt_out[0] = FMT;
    }
    const bool saturate = needs_saturation(ab, scale);
    if constexpr (VEC) {
        if (saturate) cast_chunks<DT, FMT, K, NT, true>(v, x, n, scale, q);
        else cast_chunks<DT, FMT, K, NT, false>(v, x, n, scale, q);
    } else {
        if (saturate) tensor_cast_body<DT, FMT, false, K, NT, true>(x, n, scale, q);
        else tensor_cast_body<DT, FMT, false, K, NT, false>(x, n, scale, q);
    }
}

template <int DT, bool VEC, int K, bool NT>
__global__ void __launch_bounds__(256)
k_pipeline_cast(const void* __restrict__ x, int64_t n, const uint32_t* __restrict__ partial, int np,
                uint8_t* __restrict__ q, float* __restrict__ sinv_out, int32_t* __restrict__ fmt_out) {
    __shared__ uint32_t lds[4];
    HpVec<DT> v[K];
    if constexpr (VEC) chunk_load<DT, K, NT>(v, x, n / LaneVE<DT>::value, blockIdx.x);
    const uint32_t ab = fold_partials(partial, np, 1, lds);
    if (__uint_as_float(ab) > Fp8Fmt<kE4M3>::max)
        pipeline_cast_rest<DT, kE5M2, VEC, K, NT>(v, x, n, ab, q, sinv_out, fmt_out);
    else
        pipeline_cast_rest<DT, kE4M3, VEC, K, NT>(v, x, n, ab, q, sinv_out, fmt_out);
}

// ===========================================================================
// per-channel cast (ColossalAI fp8.py, cast_to_fp8 with per_channel_scale):
// one 256-thread workgroup per row
// ===========================================================================

template <int FMT> __device__ __forceinline__ void channel_scale(uint32_t amax_bits, float& scale, float& sinv) {
    const float amax = __uint_as_float(amax_bits);
    const float a = (amax > 0.0f) ? amax : 1.0f;
    scale = Fp8Fmt<FMT>::max / a;
    sinv = a / Fp8Fmt<FMT>::max;
}

// Register-resident rows: cols % VE == 0, x 16-B aligned, q 4-byte aligned and
// cols <= CPT * 256 * VE, so each thread keeps CPT lane vectors of the row in
// VGPRs between the reduction and the cast (one HBM read per element).
template <int DT, int FMT, int CPT, bool NT>
__global__ void __launch_bounds__(256)
k_channel_reg(const void* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ q,
              float* __restrict__ sinv_out) {
    __shared__ uint32_t lds[4];
    constexpr int VE = LaneVE<DT>::value;
    constexpr int ESZ = ESize<DT>::value;
    const int64_t nvec = cols / VE;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const char* xr = (const char*)x + r * cols * ESZ;
        HpVec<DT> v[CPT];
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int64_t vi = k * 256 + threadIdx.x;
            if (vi < nvec) v[k].template load<NT>(xr + vi * VE * ESZ);
        }
#pragma unroll
        for (int k = 0; k < CPT; ++k)
            if (k * 256 + threadIdx.x < nvec) m = umax(m, v[k].absmax_bits());
        m = block_max256(m, lds);
        float scale, sinv;
        channel_scale<FMT>(m, scale, sinv);
        if (threadIdx.x == 0) sinv_out[r] = sinv;
        const bool saturate = needs_saturation(m, scale);
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int64_t vi = k * 256 + threadIdx.x;
            if (vi < nvec) {
                float f[VE];
                v[k].widen(f);
                if (saturate) scale_encode_store<FMT, true, VE, NT>(f, scale, q + r * cols + vi * VE);
                else scale_encode_store<FMT, false, VE, NT>(f, scale, q + r * cols + vi * VE);
            }
        }
    }
}

// Any row length / alignment: pass 1 reduces the row, pass 2 re-reads it (from
// cache for rows up to a few MB) and casts element-wise.
template <int DT, int FMT>
__global__ void __launch_bounds__(256)
k_channel_2pass(const void* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ q,
                float* __restrict__ sinv_out) {
    __shared__ uint32_t lds[4];
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const int64_t base = r * cols;
        uint32_t m = 0;
        for (int64_t c = threadIdx.x; c < cols; c += 256) m = umax(m, absbits1<DT>(x, base + c));
        m = block_max256(m, lds);
        float scale, sinv;
        channel_scale<FMT>(m, scale, sinv);
        if (threadIdx.x == 0) sinv_out[r] = sinv;
        const bool saturate = needs_saturation(m, scale);
        for (int64_t c = threadIdx.x; c < cols; c += 256) {
            float p = load1<DT>(x, base + c) * scale;
            if (saturate) p = sat<FMT>(p);
            q[base + c] = enc1<FMT>(p);
        }
    }
}

// Long rows with the vector layout (cols % VE == 0, x 16-B aligned, q 4-byte
// aligned, cols > 2048 * VE): pass 1 reduces the row with ordinary (cached)
// 16-byte loads, U lane vectors per thread in flight; pass 2 re-reads it,
// mostly from L2 and the Infinity Cache, and casts.
template <int DT, int FMT, int U, bool NT>
__global__ void __launch_bounds__(256)
k_channel_2pass_vec(const void* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ q,
                    float* __restrict__ sinv_out) {
    __shared__ uint32_t lds[4];
    constexpr int VE = LaneVE<DT>::value;
    constexpr int ESZ = ESize<DT>::value;
    const int64_t nvec = cols / VE;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const char* xr = (const char*)x + r * cols * ESZ;
        uint32_t m = 0;
        for (int64_t v0 = threadIdx.x; v0 < nvec; v0 += U * 256) {
            HpVec<DT> v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (v0 + u * 256 < nvec) v[u].template load<false>(xr + (v0 + u * 256) * VE * ESZ);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (v0 + u * 256 < nvec) m = umax(m, v[u].absmax_bits());
        }
        m = block_max256(m, lds);
        float scale, sinv;
        channel_scale<FMT>(m, scale, sinv);
        if (threadIdx.x == 0) sinv_out[r] = sinv;
        const bool saturate = needs_saturation(m, scale);
        for (int64_t v0 = threadIdx.x; v0 < nvec; v0 += U * 256) {
            HpVec<DT> v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (v0 + u * 256 < nvec) v[u].template load<NT>(xr + (v0 + u * 256) * VE * ESZ);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t vi = v0 + u * 256;
                if (vi < nvec) {
                    float f[VE];
                    v[u].widen(f);
                    if (saturate) scale_encode_store<FMT, true, VE, NT>(f, scale, q + r * cols + vi * VE);
                    else scale_encode_store<FMT, false, VE, NT>(f, scale, q + r * cols + vi * VE);
                }
            }
        }
    }
}

// ===========================================================================
// dequant (ColossalAI fp8.py cast_from_fp8; inverse of per_token_cast_to_fp8)
// ===========================================================================

// MODE 0: per-tensor (s = scale_inv[0]); MODE 2: per-128-group over a
// contiguous [rows, cols % 128 == 0] tensor (s = scale_inv[e / 128]);
// MODE 3: per-tensor division by a scale (y = fp32(q) / scale[0], the FSDP
// parameter hook's dequant; a correctly rounded division, not a product with
// 1 / scale).
// VEC: q 4-byte aligned and y 16-B aligned; chunks of K sub-steps x 256
// lane vectors; the n % VE tail element-wise by workgroup 0.
// one element of the flat dequant (the element-wise path and the tail)
template <int FMT, int MODE> __device__ __forceinline__ float flat_elem(uint8_t c, const float* sinv, int64_t i) {
    if constexpr (MODE == 3) return dec1<FMT>(c) / sinv[0];
    else if constexpr (MODE == 2) return dec1<FMT>(c) * sinv[i >> 7];
    else return dec1<FMT>(c) * sinv[0];
}

// Chunks c0, c0 + cstride, ... of one flat tensor; `tail` names the one
// workgroup that also converts the n % VE tail elements.
template <int FMT, int YDT, int MODE, bool VEC, int K, bool NT>
__device__ __forceinline__ void dequant_flat_body(const uint8_t* __restrict__ q, int64_t n,
                                                  const float* __restrict__ sinv, void* __restrict__ y,
                                                  int64_t c0, int64_t cstride, bool tail) {
    constexpr int VE = LaneVE<YDT>::value;
    if constexpr (VEC) {
        const int64_t nvec = n / VE;
        const int64_t nchunks = (nvec + K * 256 - 1) / (K * 256);
        const float s0 = (MODE != 2) ? sinv[0] : 0.0f;
        for (int64_t c = c0; c < nchunks; c += cstride) {
            Fp8Vec<FMT, VE, NT> w[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int64_t vi = (c * K + k) * 256 + threadIdx.x;
                if (vi < nvec) w[k].load(q + vi * VE);
            }
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int64_t vi = (c * K + k) * 256 + threadIdx.x;
                if (vi < nvec) {
                    float p[VE];
                    if constexpr (MODE == 3) {
                        w[k].decode_scaled(1.0f, p);
#pragma unroll
                        for (int e = 0; e < VE; ++e) p[e] = p[e] / s0;
                    } else {
                        w[k].decode_scaled((MODE == 0) ? s0 : sinv[(vi * VE) >> 7], p);
                    }
                    store_out16<YDT, NT>(y, vi * VE, p);
                }
            }
        }
        const int64_t i = nvec * VE + threadIdx.x;
        if (tail && i < n) store1<YDT>(y, i, flat_elem<FMT, MODE>(q[i], sinv, i));
    } else {
        for (int64_t i = c0 * 256 + threadIdx.x; i < n; i += cstride * 256)
            store1<YDT>(y, i, flat_elem<FMT, MODE>(q[i], sinv, i));
    }
}

template <int FMT, int YDT, int MODE, bool VEC, int K, bool NT>
__global__ void __launch_bounds__(256)
k_dequant_flat(const uint8_t* __restrict__ q, int64_t n, const float* __restrict__ sinv, void* __restrict__ y) {
    dequant_flat_body<FMT, YDT, MODE, VEC, K, NT>(q, n, sinv, y, blockIdx.x, gridDim.x, blockIdx.x == 0);
}

// Dequant of W packed slots (ColossalAI fp8.py, all_gather_fp8_lagacy and
// all_gather_fp8_ring, receive side): slot w starts at slots + w * (4 + n)
// with its binary32 scale_inv in bytes 0..3 and n codes after it; output w
// is y + w * n elements, y[w][i] = ydtype(fp32(code) * scale_inv_w).  Grid:
// x = chunks within a slot, y = slots (looping when W exceeds gridDim.y).
// VEC: the slots and every payload 4-byte aligned, every output row 16-B aligned.
template <int FMT, int YDT, bool VEC, int K, bool NT>
__global__ void __launch_bounds__(256)
k_dequant_packed(const uint8_t* __restrict__ slots, int64_t W, int64_t n, void* __restrict__ y) {
    constexpr int ESZ = ESize<YDT>::value;
    for (int64_t w = blockIdx.y; w < W; w += gridDim.y) {
        const uint8_t* slot = slots + w * (4 + n);
        dequant_flat_body<FMT, YDT, 0, VEC, K, NT>(slot + 4, n, (const float*)slot, (char*)y + w * n * ESZ,
                                                   blockIdx.x, gridDim.x, blockIdx.x == 0);
    }
}

// Pipeline dequant (ColossalAI fp8.py, cast_from_fp8_pipeline): the code's
// value converted to the output type (exact for every fp8 value) times the
// binary32 scale_inv in binary32, rounded to the output type -- the per-tensor
// dequant, with the format read from the device word the pipeline cast wrote,
// so the host never waits for it.  Every workgroup reads the same word, so the
// branch is uniform.  A word other than e4m3fn (0) or e5m2 (1) gives NaN
// everywhere.
template <int YDT, bool VEC, int K, bool NT>
__global__ void __launch_bounds__(256)
k_dequant_pipeline(const uint8_t* __restrict__ q, int64_t n, const float* __restrict__ sinv,
                   const int32_t* __restrict__ fmt, void* __restrict__ y) {
    const int32_t f = fmt[0];
    if (f == kE4M3) dequant_flat_body<kE4M3, YDT, 0, VEC, K, NT>(q, n, sinv, y, blockIdx.x, gridDim.x, blockIdx.x == 0);
    else if (f == kE5M2)
        dequant_flat_body<kE5M2, YDT, 0, VEC, K, NT>(q, n, sinv, y, blockIdx.x, gridDim.x, blockIdx.x == 0);
    else
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
            store1<YDT>(y, i, __builtin_nanf(""));
}

// per-channel: one workgroup per row, scale_inv[r] read once per row.
// VEC: cols % VE == 0, q 4-byte aligned, y 16-B aligned.
template <int FMT, int YDT, bool VEC, bool NT>
__global__ void __launch_bounds__(256)
k_dequant_rows(const uint8_t* __restrict__ q, int64_t rows, int64_t cols, const float* __restrict__ sinv,
               void* __restrict__ y) {
    constexpr int VE = LaneVE<YDT>::value;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float s = sinv[r];
        const int64_t base = r * cols;
        if constexpr (VEC) {
            constexpr int K = 2;
            const int64_t nvec = cols / VE;
            for (int64_t v0 = threadIdx.x; v0 < nvec; v0 += K * 256) {
                Fp8Vec<FMT, VE, NT> w[K];
#pragma unroll
                for (int k = 0; k < K; ++k)
                    if (v0 + k * 256 < nvec) w[k].load(q + base + (v0 + k * 256) * VE);
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    if (v0 + k * 256 < nvec) {
                        float p[VE];
                        w[k].decode_scaled(s, p);
                        store_out16<YDT, NT>(y, base + (v0 + k * 256) * VE, p);
                    }
                }
            }
        } else {
            for (int64_t c = threadIdx.x; c < cols; c += 256) store1<YDT>(y, base + c, dec1<FMT>(q[base + c]) * s);
        }
    }
}

// ===========================================================================
// 128x128 block weight dequant (CSDN notes, weight_dequant_kernel)
// ===========================================================================

// Mapping: the pages launch one program per 128x128 tile.  On MI355X a
// workgroup per tile (scale_inv in an SGPR) reached only ~62 % of HBM peak:
// every wave instruction touched 4 rows 7 KB apart and the grid hopped
// between DRAM pages.  Both kernels below instead stream the matrix front to
// back and fetch each lane's tile scale from the 128-column block it falls in
// (a cached load; the whole scale grid is a few KB).
//
// Row-strip mapping (used beyond 2^32 lane vectors): a workgroup
// dequantizes RB whole consecutive rows, so the grid streams the matrix front
// to back instead of jumping between the rows of a 128x128 tile.  Lane t of a sub-step owns lane
// vector t (+ 256 u) of a row; its scale_inv is the cached scalar
// s[(row / 128) * nbn + col / 128] (at most 4 distinct values per wave
// instruction).  U lane vectors per row and all RB rows are loaded before
// the first convert.  Requires N % VE == 0, q 4-byte aligned, y 16-B aligned.
template <int FMT, int YDT, int RB, int U, bool NT>
__global__ void __launch_bounds__(256)
k_block128_rows(const uint8_t* __restrict__ q, int64_t M, int64_t N, const float* __restrict__ sinv,
                void* __restrict__ y, int64_t nbn) {
    constexpr int VE = LaneVE<YDT>::value;
    const int64_t vpr = N / VE;
    for (int64_t r0 = (int64_t)blockIdx.x * RB; r0 < M; r0 += (int64_t)gridDim.x * RB) {
        for (int64_t v0 = threadIdx.x; v0 < vpr; v0 += U * 256) {
            Fp8Vec<FMT, VE, NT> w[RB][U];
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (r0 + r < M && v0 + u * 256 < vpr) w[r][u].load(q + (r0 + r) * N + (v0 + u * 256) * VE);
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const float* srow = sinv + ((r0 + r) >> 7) * nbn;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t v = v0 + u * 256;
                    if (r0 + r < M && v < vpr) {
                        float p[VE];
                        w[r][u].decode_scaled(srow[(v * VE) >> 7], p);
                        store_out16<YDT, NT>(y, (r0 + r) * N + v * VE, p);
                    }
                }
            }
        }
    }
}

// Division of a 32-bit n by an invariant d >= 1 (Granlund-Montgomery):
// with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1 (computed on
// the host), n / d = (umulhi(n, m) + n) >> l, exact for every 32-bit n.
struct DivU32 {
    uint32_t m;
    int l;
};
__device__ __forceinline__ uint32_t div_u32(uint32_t n, DivU32 d) {
    const uint32_t t = __umulhi(n, d.m);
    return (uint32_t)(((uint64_t)t + n) >> d.l);
}

// Flat mapping: the matrix is streamed front to back in chunks of K
// sub-steps x 256 lane vectors, exactly like the flat dequant; each lane finds
// its row by an invariant-divisor division of its lane-vector index by the
// lane vectors per row (vpr), and reads its tile's scale_inv from the cached
// scale row.  Requires N % VE == 0, q 4-byte aligned, y 16-B aligned and
// M * N / VE < 2^32.
template <int FMT, int YDT, int K, bool NT>
__global__ void __launch_bounds__(256)
k_block128_flat(const uint8_t* __restrict__ q, int64_t nvec, const float* __restrict__ sinv,
                void* __restrict__ y, int64_t nbn, uint32_t vpr, DivU32 dvpr) {
    constexpr int VE = LaneVE<YDT>::value;
    const int64_t nchunks = (nvec + K * 256 - 1) / (K * 256);
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        Fp8Vec<FMT, VE, NT> w[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t vi = (c * K + k) * 256 + threadIdx.x;
            if (vi < nvec) w[k].load(q + vi * VE);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t vi = (c * K + k) * 256 + threadIdx.x;
            if (vi < nvec) {
                const uint32_t row = div_u32((uint32_t)vi, dvpr);
                const uint32_t col = (uint32_t)vi - row * vpr;          // lane vector within the row
                const float s = sinv[(int64_t)(row >> 7) * nbn + ((col * VE) >> 7)];
                float p[VE];
                w[k].decode_scaled(s, p);
                store_out16<YDT, NT>(y, vi * VE, p);
            }
        }
    }
}

// any N / alignment: element-wise over rows, one row per workgroup trip
template <int FMT, int YDT>
__global__ void __launch_bounds__(256)
k_block128_s(const uint8_t* __restrict__ q, int64_t M, int64_t N, const float* __restrict__ sinv,
             void* __restrict__ y, int64_t nbn) {
    for (int64_t i = blockIdx.x; i < M; i += gridDim.x) {
        const float* srow = sinv + (i / 128) * nbn;
        for (int64_t j = threadIdx.x; j < N; j += 256)
            store1<YDT>(y, i * N + j, dec1<FMT>(q[i * N + j]) * srow[j / 128]);
    }
}

// ===========================================================================
// reduce step of the fp8-compressed all-reduce / reduce-scatter (ColossalAI
// fp8.py: _all_reduce_fp8, _reduce_scatter_fp8, the DDP hook's
// sum_and_allgather)
// ===========================================================================

// v rounded to the element type, as binary32 (exact widening back)
template <int YDT> __device__ __forceinline__ float round_to(float v) {
    if constexpr (YDT == kBF16) return bf16_lo(pack_bf16x2(v, 0.0f));
    else if constexpr (YDT == kF16) return (float)__builtin_bit_cast(_Float16, to_f16(v));
    else return v;
}

// Round VE binary32 values to the element type in place (exact widening
// back).  bf16 rounds two values per v_cvt_pk_bf16_f32; fp16 has no RNE
// packed convert, so it goes value by value.
template <int YDT, int VE> __device__ __forceinline__ void round_vec(float* v) {
    if constexpr (YDT == kBF16) {
#pragma unroll
        for (int k = 0; k < VE; k += 2) {
            const uint32_t w = pack_bf16x2(v[k], v[k + 1]);
            v[k] = bf16_lo(w);
            v[k + 1] = bf16_hi(w);
        }
    } else if constexpr (YDT == kF16) {
#pragma unroll
        for (int k = 0; k < VE; ++k) v[k] = round_to<YDT>(v[k]);
    }
}

// One term of the sum: ydtype(fp32(q) * scale_inv), added to the running sum
// with the type's rounding (summed_out += cast_from_fp8(...) on an ydtype
// tensor).  The running sum starts at +0 (torch.zeros).
template <int FMT, int YDT, int VE>
__device__ __forceinline__ void sum_term(float* acc, const uint32_t* w, float s) {
    float p[VE];
#pragma unroll
    for (int k = 0; k < VE / 4; ++k) dec4<FMT>(w[k], p + 4 * k);
#pragma unroll
    for (int k = 0; k < VE; ++k) p[k] = p[k] * s;
    round_vec<YDT, VE>(p);
#pragma unroll
    for (int k = 0; k < VE; ++k) acc[k] = acc[k] + p[k];
    round_vec<YDT, VE>(acc);
}

// ydtype(acc / W).  For W a power of two, a * (1/W) is the same exact value
// as a / W (1/W is exact in binary32), so it rounds identically; any other W
// takes the correctly rounded division.
template <int YDT, int VE> __device__ __forceinline__ void average_vec(float* acc, float fW, bool pow2) {
    if (pow2) {
        const float r = 1.0f / fW;
#pragma unroll
        for (int k = 0; k < VE; ++k) acc[k] = acc[k] * r;
    } else {
#pragma unroll
        for (int k = 0; k < VE; ++k) acc[k] = acc[k] / fW;
    }
    round_vec<YDT, VE>(acc);
}

// y[i] = sum over the W chunks of q (chunk w at q + w * n) in chunk order,
// divided by W when `average`; with AMAX, max |y| is folded into the amax
// slots (one atomic max per workgroup, slot blockIdx.x % nslots).
// VEC: n % VE == 0, q 4-byte aligned, y 16-B aligned.  A thread owns KV lane
// vectors 256 apart; chunk loads are issued four chunks at a time for all
// of them before their terms are added.
template <int FMT, int YDT, bool VEC, bool AMAX, bool NT, int KV, bool NTY = NT>
__global__ void __launch_bounds__(256)
k_dequant_sum(const uint8_t* __restrict__ q, int64_t W, int64_t n, const float* __restrict__ sinv, int average,
              void* __restrict__ y, uint32_t* __restrict__ amax_bits, int nslots) {
    __shared__ uint32_t lds[4];
    constexpr int VE = LaneVE<YDT>::value;
    const float fW = (float)W;
    const bool pow2 = (W & (W - 1)) == 0;
    uint32_t m = 0;
    const int64_t nvec = VEC ? n / VE : 0;
    for (int64_t v0 = (int64_t)blockIdx.x * 256 * KV + threadIdx.x; v0 < nvec; v0 += (int64_t)gridDim.x * 256 * KV) {
        float acc[KV][VE];
#pragma unroll
        for (int u = 0; u < KV; ++u)
#pragma unroll
            for (int k = 0; k < VE; ++k) acc[u][k] = 0.0f;
        for (int64_t w0 = 0; w0 < W; w0 += 4) {
            Fp8Vec<FMT, VE, NT> c[KV][4];
#pragma unroll
            for (int u = 0; u < KV; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (w0 + j < W && v0 + u * 256 < nvec) c[u][j].load(q + (w0 + j) * n + (v0 + u * 256) * VE);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (w0 + j < W) {
                    const float s = sinv[w0 + j];
#pragma unroll
                    for (int u = 0; u < KV; ++u) sum_term<FMT, YDT, VE>(acc[u], c[u][j].w, s);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < KV; ++u) {
            const int64_t vi = v0 + u * 256;
            if (vi < nvec) {
                if (average) average_vec<YDT, VE>(acc[u], fW, pow2);
                if constexpr (AMAX) {
#pragma unroll
                    for (int k = 0; k < VE; ++k) m = umax(m, __float_as_uint(acc[u][k]) & 0x7FFFFFFFu);
                }
                store_out16<YDT, NTY>(y, vi * VE, acc[u]);
            }
        }
    }
    // element-wise: the n % VE tail of the vector path, or everything
    const int64_t nthr = (int64_t)gridDim.x * 256;
    for (int64_t i = nvec * VE + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += nthr) {
        float acc = 0.0f;
        for (int64_t w = 0; w < W; ++w) acc = round_to<YDT>(acc + round_to<YDT>(dec1<FMT>(q[w * n + i]) * sinv[w]));
        if (average) acc = round_to<YDT>(pow2 ? acc * (1.0f / fW) : acc / fW);
        if constexpr (AMAX) m = umax(m, __float_as_uint(acc) & 0x7FFFFFFFu);
        store1<YDT>(y, i, acc);
    }
    if constexpr (AMAX) {
        m = block_max256(m, lds);
        if (threadIdx.x == 0 && m != 0) atomicMax(amax_bits + (blockIdx.x % nslots) * kAmaxSlotStride, m);
    }
}

}  // namespace fp8q
