// fp8q_kernels.hip -- HIP kernels of the FP8 scaled cast for gfx950 (CDNA4).
//
// Quantize: amax reduction (per tensor / per row / per 128-element group) ->
// scale = fp8_max / amax -> binary32 multiply -> hardware fp8 convert.
// Dequantize: hardware fp8 -> fp32 convert -> binary32 multiply by scale_inv
// -> fp32 / bf16 / fp16 store.
//
// Every path is memory-bound (about 3 bytes of HBM traffic per element and a
// handful of VALU ops), so the kernels are organised around 16-byte vector
// loads and stores, enough bytes in flight per CU, and reductions that stay in
// registers (DPP lane exchanges; LDS only for the cross-wave step of a row).
//
// amax is computed on the integer bit patterns of |x| (sign bit cleared):
// for non-negative IEEE values the unsigned order of the bits is the numeric
// order, +inf sorts above every finite value and every NaN above +inf, so an
// unsigned max is exact, order-independent and propagates NaN the way torch's
// max does (ColossalAI fp8.py cast_to_fp8; DeepEP "5 Utils"
// per_token_cast_to_fp8).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q_launch.h"

namespace fp8q {

// ---------------------------------------------------------------------------
// formats and element helpers
// ---------------------------------------------------------------------------

template <int FMT> struct Fp8Fmt;
template <> struct Fp8Fmt<kE4M3> { static constexpr float max = 448.0f; };     // 1.75 * 2^8
template <> struct Fp8Fmt<kE5M2> { static constexpr float max = 57344.0f; };   // 1.75 * 2^15

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));   // one 16-byte vector

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
    u16x2 a = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
    return __builtin_elementwise_max(m, a);
}

// binary32 bits of |amax| from a 16-bit element's |bits|
template <int DT> __device__ __forceinline__ uint32_t abs16_to_f32bits(uint32_t b);
template <> __device__ __forceinline__ uint32_t abs16_to_f32bits<kBF16>(uint32_t b) { return b << 16; }
template <> __device__ __forceinline__ uint32_t abs16_to_f32bits<kF16>(uint32_t b) {
    return __float_as_uint((float)__builtin_bit_cast(_Float16, (uint16_t)b));
}

// Saturating clamp that keeps NaN (the comparison is false for NaN).  Only
// needed when scale is +inf (amax below fp8_max / FLT_MAX); for a finite
// scale = fp8_max / a every |x * scale| <= fp8_max * (1 + 2^-23), which the
// round-to-nearest-even convert already maps to fp8_max.
template <int FMT> __device__ __forceinline__ float sat(float v) {
    return fabsf(v) > Fp8Fmt<FMT>::max ? copysignf(Fp8Fmt<FMT>::max, v) : v;
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

// binary32 -> output element bits (RNE)
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

// 16-byte vector memory access; streaming data is touched once, so loads and
// stores are non-temporal
__device__ __forceinline__ v4u ld16(const void* p) {
    return __builtin_nontemporal_load((const v4u*)p);
}
__device__ __forceinline__ void st16(void* p, v4u v) { __builtin_nontemporal_store(v, (v4u*)p); }

// ---------------------------------------------------------------------------
// lane reductions (unsigned max)
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// max over each aligned group of 8 lanes: quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], then row_half_mirror (lane i <- lane 7-i within 8 lanes)
__device__ __forceinline__ uint32_t max8(uint32_t v) {
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));
    return v;
}

// max over the whole 64-lane wavefront, result in every lane
__device__ __forceinline__ uint32_t max64(uint32_t v) {
    v = max8(v);
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));  // row_mirror (16)
    v = umax(v, (uint32_t)__shfl_xor((int)v, 16, 64));
    v = umax(v, (uint32_t)__shfl_xor((int)v, 32, 64));
    return v;
}

// max over a workgroup of `kThreads` threads; result valid in every thread
template <int kThreads> __device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* lds) {
    constexpr int kWaves = kThreads / 64;
    v = max64(v);
    const int wave = threadIdx.x / 64;
    if ((threadIdx.x & 63) == 0) lds[wave] = v;
    __syncthreads();
    uint32_t m = lds[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = umax(m, lds[w]);
    __syncthreads();  // lds may be reused by the caller
    return m;
}

// ---------------------------------------------------------------------------
// loading 16 elements of one lane: values as binary32 and the max of |bits|
// ---------------------------------------------------------------------------

template <int DT> struct Chunk16;

template <> struct Chunk16<kF32> {
    v4u r[4];
    __device__ __forceinline__ void load(const void* p) {
        const char* c = (const char*)p;
        r[0] = ld16(c); r[1] = ld16(c + 16); r[2] = ld16(c + 32); r[3] = ld16(c + 48);
    }
    __device__ __forceinline__ uint32_t absmax_bits() const {
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            m = umax(m, r[k].x & 0x7FFFFFFFu); m = umax(m, r[k].y & 0x7FFFFFFFu);
            m = umax(m, r[k].z & 0x7FFFFFFFu); m = umax(m, r[k].w & 0x7FFFFFFFu);
        }
        return m;
    }
    __device__ __forceinline__ void widen(float* v) const {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[4 * k] = __uint_as_float(r[k].x); v[4 * k + 1] = __uint_as_float(r[k].y);
            v[4 * k + 2] = __uint_as_float(r[k].z); v[4 * k + 3] = __uint_as_float(r[k].w);
        }
    }
};

template <int DT> struct Chunk16Half {
    v4u r[2];
    __device__ __forceinline__ void load(const void* p) {
        const char* c = (const char*)p;
        r[0] = ld16(c); r[1] = ld16(c + 16);
    }
    __device__ __forceinline__ uint32_t absmax_bits() const {
        u16x2 m = {0, 0};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            m = absmax16(m, r[k].x); m = absmax16(m, r[k].y);
            m = absmax16(m, r[k].z); m = absmax16(m, r[k].w);
        }
        return abs16_to_f32bits<DT>(umax(m[0], m[1]));
    }
    __device__ __forceinline__ void widen(float* v) const {
        const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if constexpr (DT == kBF16) { v[2 * k] = bf16_lo(w[k]); v[2 * k + 1] = bf16_hi(w[k]); }
            else { v[2 * k] = f16_lo(w[k]); v[2 * k + 1] = f16_hi(w[k]); }
        }
    }
};
template <> struct Chunk16<kBF16> : Chunk16Half<kBF16> {};
template <> struct Chunk16<kF16> : Chunk16Half<kF16> {};

template <int DT> __device__ __forceinline__ float load1(const void* x, int64_t i) {
    if constexpr (DT == kF32) return ((const float*)x)[i];
    else if constexpr (DT == kBF16) return __uint_as_float((uint32_t)((const uint16_t*)x)[i] << 16);
    else return (float)((const _Float16*)x)[i];
}

template <int DT> __device__ __forceinline__ uint32_t absbits1(const void* x, int64_t i) {
    if constexpr (DT == kF32) return ((const uint32_t*)x)[i] & 0x7FFFFFFFu;
    else return abs16_to_f32bits<DT>(((const uint16_t*)x)[i] & 0x7FFFu);
}

// scale and encode 16 values -> one 16-byte store
template <int FMT, bool SAT> __device__ __forceinline__ v4u scale_enc16(const float* v, float scale) {
    float p[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        p[k] = v[k] * scale;
        if constexpr (SAT) p[k] = sat<FMT>(p[k]);
    }
    v4u o;
    o.x = enc4<FMT>(p[0], p[1], p[2], p[3]);
    o.y = enc4<FMT>(p[4], p[5], p[6], p[7]);
    o.z = enc4<FMT>(p[8], p[9], p[10], p[11]);
    o.w = enc4<FMT>(p[12], p[13], p[14], p[15]);
    return o;
}

// store 16 binary32 results as the output type at element offset e
template <int YDT> __device__ __forceinline__ void store16(void* y, int64_t e, const float* p) {
    if constexpr (YDT == kF32) {
        char* c = (char*)y + e * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v4u o = {__float_as_uint(p[4 * k]), __float_as_uint(p[4 * k + 1]),
                       __float_as_uint(p[4 * k + 2]), __float_as_uint(p[4 * k + 3])};
            st16(c + 16 * k, o);
        }
    } else {
        char* c = (char*)y + e * 2;
        uint32_t w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            w[k] = (YDT == kBF16) ? pack_bf16x2(p[2 * k], p[2 * k + 1]) : pack_f16x2(p[2 * k], p[2 * k + 1]);
        st16(c, v4u{w[0], w[1], w[2], w[3]});
        st16(c + 16, v4u{w[4], w[5], w[6], w[7]});
    }
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
// the comparison form keeps a NaN amax as NaN, like torch.clamp).
template <int FMT> __device__ __forceinline__ void group_scale(uint32_t amax_bits, float& scale, float& sinv) {
    float amax = __uint_as_float(amax_bits);
    const float lo = 1e-4f;
    if (amax < lo) amax = lo;
    scale = Fp8Fmt<FMT>::max / amax;
    sinv = amax / Fp8Fmt<FMT>::max;
}

// Vector path: 8 consecutive lanes own one 128-element group (16 elements,
// i.e. 32 B of bf16 or 64 B of fp32 per lane, one 16-B fp8 store per lane);
// a wavefront covers 8 consecutive groups.  Each thread takes K groups per
// loop trip, issuing all loads before the first reduction.  Groups are
// consecutive 128-element chunks of the flat array because cols % 128 == 0,
// and group g's scale_inv lives at flat index g.
template <int DT, int FMT, int K>
__global__ void __launch_bounds__(256)
k_group128_v(const void* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ sinv_out, int64_t groups) {
    constexpr int ESZ = (DT == kF32) ? 4 : 2;
    const int lane8 = threadIdx.x & 7;
    const int64_t slots = (int64_t)gridDim.x * (blockDim.x / 8);
    const int64_t slot = (int64_t)blockIdx.x * (blockDim.x / 8) + (threadIdx.x >> 3);
    for (int64_t g0 = slot; g0 < groups; g0 += K * slots) {
        Chunk16<DT> c[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t g = g0 + k * slots;
            if (g < groups) c[k].load((const char*)x + (g * 128 + lane8 * 16) * ESZ);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t g = g0 + k * slots;
            if (g < groups) {  // uniform within the 8 lanes of a group
                const uint32_t amax = max8(c[k].absmax_bits());
                float scale, sinv;
                group_scale<FMT>(amax, scale, sinv);
                float v[16];
                c[k].widen(v);
                st16(q + g * 128 + lane8 * 16, scale_enc16<FMT, false>(v, scale));
                if (lane8 == 0) sinv_out[g] = sinv;
            }
        }
    }
}

// Unaligned path: one wavefront per group, two elements per lane, element-wise
// loads and byte stores.  Correct for any alignment of x (to its element size)
// and q.
template <int DT, int FMT>
__global__ void __launch_bounds__(256)
k_group128_s(const void* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ sinv_out, int64_t groups) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
    for (int64_t g = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64; g < groups; g += waves) {
        const int64_t e0 = g * 128 + 2 * lane;
        uint32_t m = umax(absbits1<DT>(x, e0), absbits1<DT>(x, e0 + 1));
        m = max64(m);
        float scale, sinv;
        group_scale<FMT>(m, scale, sinv);
        const uint32_t w = enc4<FMT>(load1<DT>(x, e0) * scale, load1<DT>(x, e0 + 1) * scale, 0.0f, 0.0f);
        q[e0] = (uint8_t)(w & 0xFF);
        q[e0 + 1] = (uint8_t)((w >> 8) & 0xFF);
        if (lane == 0) sinv_out[g] = sinv;
    }
}

// ===========================================================================
// per-tensor: global amax (stage 1 per workgroup, stage 2 atomic max) and the
// scale-and-cast pass (ColossalAI fp8.py, cast_to_fp8, per-tensor branch)
// ===========================================================================

__global__ void k_fill_u32(uint32_t* p, uint32_t v) {
    if (threadIdx.x == 0) p[0] = v;
}

__global__ void k_fill_f32(float* p, int64_t n, float v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// VEC: x is 16-B aligned; then 16-element chunks are read with 16-B loads and
// the n % 16 tail element-wise.
template <int DT, bool VEC, int U>
__global__ void __launch_bounds__(256)
k_amax(const void* __restrict__ x, int64_t n, uint32_t* __restrict__ amax_bits) {
    __shared__ uint32_t lds[4];
    constexpr int ESZ = (DT == kF32) ? 4 : 2;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
    uint32_t m = 0;
    int64_t done = 0;
    if constexpr (VEC) {
        const int64_t chunks = n / 16;
        for (int64_t c0 = tid; c0 < chunks; c0 += U * nthr) {
            Chunk16<DT> c[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c0 + u * nthr < chunks) c[u].load((const char*)x + (c0 + u * nthr) * 16 * ESZ);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c0 + u * nthr < chunks) m = umax(m, c[u].absmax_bits());
        }
        done = chunks * 16;
    }
    for (int64_t i = done + tid; i < n; i += nthr) m = umax(m, absbits1<DT>(x, i));
    m = block_max<256>(m, lds);
    if (threadIdx.x == 0 && m != 0) atomicMax(amax_bits, m);
}

// scale from the finished amax: a = amax > 0 ? amax : 1 (NaN -> 1),
// scale = fp8_max / a, scale_inv = 1 / scale
template <int FMT> __device__ __forceinline__ void tensor_scale(uint32_t amax_bits, float& scale, float& sinv) {
    const float amax = __uint_as_float(amax_bits);
    const float a = (amax > 0.0f) ? amax : 1.0f;
    scale = Fp8Fmt<FMT>::max / a;
    sinv = 1.0f / scale;
}

template <int DT, int FMT, bool VEC, bool SAT>
__device__ __forceinline__ void scale_cast_body(const void* __restrict__ x, int64_t n, float scale,
                                                uint8_t* __restrict__ q) {
    constexpr int ESZ = (DT == kF32) ? 4 : 2;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
    int64_t done = 0;
    if constexpr (VEC) {
        const int64_t chunks = n / 16;
        for (int64_t c = tid; c < chunks; c += nthr) {
            Chunk16<DT> ch;
            ch.load((const char*)x + c * 16 * ESZ);
            float v[16];
            ch.widen(v);
            st16(q + c * 16, scale_enc16<FMT, SAT>(v, scale));
        }
        done = chunks * 16;
    }
    for (int64_t i = done + tid; i < n; i += nthr) {
        float p = load1<DT>(x, i) * scale;
        if constexpr (SAT) p = sat<FMT>(p);
        q[i] = enc1<FMT>(p);
    }
}

template <int DT, int FMT, bool VEC>
__global__ void __launch_bounds__(256)
k_tensor_cast(const void* __restrict__ x, int64_t n, const uint32_t* __restrict__ amax_bits,
              uint8_t* __restrict__ q, float* __restrict__ sinv_out) {
    float scale, sinv;
    tensor_scale<FMT>(amax_bits[0], scale, sinv);
    if (blockIdx.x == 0 && threadIdx.x == 0) sinv_out[0] = sinv;
    if (__builtin_isinf(scale)) scale_cast_body<DT, FMT, VEC, true>(x, n, scale, q);   // uniform branch
    else scale_cast_body<DT, FMT, VEC, false>(x, n, scale, q);
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

// Register-resident rows: cols % 16 == 0, 16-B aligned rows, and
// cols <= CPT * 16 * 256, so each thread keeps CPT 16-element chunks of the row
// in VGPRs between the reduction and the cast (one HBM read per element).
template <int DT, int FMT, int CPT>
__global__ void __launch_bounds__(256)
k_channel_reg(const void* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ q,
              float* __restrict__ sinv_out) {
    __shared__ uint32_t lds[4];
    constexpr int ESZ = (DT == kF32) ? 4 : 2;
    const int64_t chunks = cols / 16;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const char* xr = (const char*)x + r * cols * ESZ;
        Chunk16<DT> c[CPT];
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int64_t ci = threadIdx.x + k * 256;
            if (ci < chunks) c[k].load(xr + ci * 16 * ESZ);
        }
#pragma unroll
        for (int k = 0; k < CPT; ++k)
            if (threadIdx.x + k * 256 < chunks) m = umax(m, c[k].absmax_bits());
        m = block_max<256>(m, lds);
        float scale, sinv;
        channel_scale<FMT>(m, scale, sinv);
        if (threadIdx.x == 0) sinv_out[r] = sinv;
        const bool saturate = __builtin_isinf(scale);
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int64_t ci = threadIdx.x + k * 256;
            if (ci < chunks) {
                float v[16];
                c[k].widen(v);
                const v4u o = saturate ? scale_enc16<FMT, true>(v, scale) : scale_enc16<FMT, false>(v, scale);
                st16(q + r * cols + ci * 16, o);
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
        m = block_max<256>(m, lds);
        float scale, sinv;
        channel_scale<FMT>(m, scale, sinv);
        if (threadIdx.x == 0) sinv_out[r] = sinv;
        const bool saturate = __builtin_isinf(scale);
        for (int64_t c = threadIdx.x; c < cols; c += 256) {
            float p = load1<DT>(x, base + c) * scale;
            if (saturate) p = sat<FMT>(p);
            q[base + c] = enc1<FMT>(p);
        }
    }
}

// ===========================================================================
// dequant (ColossalAI fp8.py cast_from_fp8; inverse of per_token_cast_to_fp8)
// ===========================================================================

// decode 16 codes of one 16-B load and multiply by s
template <int FMT> __device__ __forceinline__ void dec16_scaled(v4u w, float s, float* p) {
    dec4<FMT>(w.x, p); dec4<FMT>(w.y, p + 4); dec4<FMT>(w.z, p + 8); dec4<FMT>(w.w, p + 12);
#pragma unroll
    for (int k = 0; k < 16; ++k) p[k] = p[k] * s;
}

// MODE 0: per-tensor (s = scale_inv[0]); MODE 2: per-128-group over a
// contiguous [rows, cols % 128 == 0] tensor (s = scale_inv[e / 128]).
// VEC: q and y 16-B aligned -> 16-element chunks, tail element-wise.
template <int FMT, int YDT, int MODE, bool VEC>
__global__ void __launch_bounds__(256)
k_dequant_flat(const uint8_t* __restrict__ q, int64_t n, const float* __restrict__ sinv, void* __restrict__ y) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
    int64_t done = 0;
    if constexpr (VEC) {
        const int64_t chunks = n / 16;
        for (int64_t c = tid; c < chunks; c += nthr) {
            const float s = (MODE == 0) ? sinv[0] : sinv[(c * 16) >> 7];
            float p[16];
            dec16_scaled<FMT>(ld16(q + c * 16), s, p);
            store16<YDT>(y, c * 16, p);
        }
        done = chunks * 16;
    }
    for (int64_t i = done + tid; i < n; i += nthr) {
        const float s = (MODE == 0) ? sinv[0] : sinv[i >> 7];
        store1<YDT>(y, i, dec1<FMT>(q[i]) * s);
    }
}

// per-channel: one workgroup per row, scale_inv[r] read once per row
template <int FMT, int YDT, bool VEC>
__global__ void __launch_bounds__(256)
k_dequant_rows(const uint8_t* __restrict__ q, int64_t rows, int64_t cols, const float* __restrict__ sinv,
               void* __restrict__ y) {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float s = sinv[r];
        const int64_t base = r * cols;
        if constexpr (VEC) {
            for (int64_t c = threadIdx.x; c < cols / 16; c += 256) {
                float p[16];
                dec16_scaled<FMT>(ld16(q + base + c * 16), s, p);
                store16<YDT>(y, base + c * 16, p);
            }
        } else {
            for (int64_t c = threadIdx.x; c < cols; c += 256) store1<YDT>(y, base + c, dec1<FMT>(q[base + c]) * s);
        }
    }
}

// ===========================================================================
// 128x128 block weight dequant (CSDN notes, weight_dequant_kernel)
// ===========================================================================

// One workgroup per 128x128 tile; the tile's scale_inv is read once (a
// wave-uniform scalar load).  Each thread owns 16 consecutive columns of
// 128/16 = 8 threads' row segment, so 256 threads cover 32 rows per pass and
// 4 passes cover the tile; all 4 loads are issued before the first convert.
// Requires N % 16 == 0 and 16-B aligned q and y.
template <int FMT, int YDT>
__global__ void __launch_bounds__(256)
k_block128_v(const uint8_t* __restrict__ q, int64_t M, int64_t N, const float* __restrict__ sinv,
             void* __restrict__ y, int64_t nbn, int64_t ntiles) {
    const int cseg = threadIdx.x & 7;    // 16-column segment within the tile
    const int rsub = threadIdx.x >> 3;   // 0..31
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int64_t bm = t / nbn, bn = t - bm * nbn;
        const float s = sinv[t];
        const int64_t col = bn * 128 + cseg * 16;
        const bool col_ok = col < N;
        v4u w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t row = bm * 128 + rsub + 32 * k;
            if (col_ok && row < M) w[k] = ld16(q + row * N + col);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t row = bm * 128 + rsub + 32 * k;
            if (col_ok && row < M) {
                float p[16];
                dec16_scaled<FMT>(w[k], s, p);
                store16<YDT>(y, row * N + col, p);
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
// launchers (host side)
// ===========================================================================

namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxBlocks = 256 * 64;   // grid-stride kernels: 64 workgroups per CU on 256 CUs

inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline unsigned blocks_for(int64_t work_items, int64_t per_block) {
    int64_t b = (work_items + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > kMaxBlocks) b = kMaxBlocks;
    return (unsigned)b;
}

template <template <int, int> class F, typename... A>
void dispatch_dt_fmt(int dt, int fmt, A... a) {
    if (dt == kF32) { if (fmt == kE4M3) F<kF32, kE4M3>::run(a...); else F<kF32, kE5M2>::run(a...); }
    else if (dt == kBF16) { if (fmt == kE4M3) F<kBF16, kE4M3>::run(a...); else F<kBF16, kE5M2>::run(a...); }
    else { if (fmt == kE4M3) F<kF16, kE4M3>::run(a...); else F<kF16, kE5M2>::run(a...); }
}

template <int DT, int FMT> struct RunGroup128 {
    static void run(const void* x, int64_t groups, uint8_t* q, float* sinv, hipStream_t st) {
        if (al16(x) && al16(q)) {
            constexpr int K = 2;
            const unsigned nb = blocks_for((groups + K - 1) / K, kThreads / 8);
            k_group128_v<DT, FMT, K><<<nb, kThreads, 0, st>>>(x, q, sinv, groups);
        } else {
            k_group128_s<DT, FMT><<<blocks_for(groups, kThreads / 64), kThreads, 0, st>>>(x, q, sinv, groups);
        }
    }
};

template <int DT, int FMT> struct RunTensorCast {
    static void run(const void* x, int64_t n, const uint32_t* ws, uint8_t* q, float* sinv, hipStream_t st) {
        const bool vec = al16(x) && al16(q);
        const unsigned nb = blocks_for(vec ? n / 16 + 1 : n, kThreads);
        if (vec) k_tensor_cast<DT, FMT, true><<<nb, kThreads, 0, st>>>(x, n, ws, q, sinv);
        else k_tensor_cast<DT, FMT, false><<<nb, kThreads, 0, st>>>(x, n, ws, q, sinv);
    }
};

template <int DT, int FMT> struct RunChannel {
    static void run(const void* x, int64_t rows, int64_t cols, uint8_t* q, float* sinv, hipStream_t st) {
        const unsigned nb = blocks_for(rows, 1);
        const bool vec = (cols % 16 == 0) && al16(x) && al16(q);
        const int64_t chunks = cols / 16;
        if (vec && chunks <= 256) k_channel_reg<DT, FMT, 1><<<nb, kThreads, 0, st>>>(x, rows, cols, q, sinv);
        else if (vec && chunks <= 512) k_channel_reg<DT, FMT, 2><<<nb, kThreads, 0, st>>>(x, rows, cols, q, sinv);
        else if (vec && chunks <= 1024) k_channel_reg<DT, FMT, 4><<<nb, kThreads, 0, st>>>(x, rows, cols, q, sinv);
        else k_channel_2pass<DT, FMT><<<nb, kThreads, 0, st>>>(x, rows, cols, q, sinv);
    }
};

template <int DT> void run_amax(const void* x, int64_t n, uint32_t* ws, hipStream_t st) {
    k_fill_u32<<<1, 64, 0, st>>>(ws, 0u);
    if (n == 0) return;
    constexpr int U = 4;
    if (al16(x)) {
        const unsigned nb = blocks_for((n / 16 + U - 1) / U + 1, kThreads);
        k_amax<DT, true, U><<<nb, kThreads, 0, st>>>(x, n, ws);
    } else {
        k_amax<DT, false, U><<<blocks_for(n, kThreads), kThreads, 0, st>>>(x, n, ws);
    }
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

template <int FMT, int YDT> struct RunDequantFlat {
    static void run(int mode, const uint8_t* q, int64_t n, const float* sinv, void* y, hipStream_t st) {
        const bool vec = al16(q) && al16(y);
        const unsigned nb = blocks_for(vec ? n / 16 + 1 : n, kThreads);
        if (mode == 0) {
            if (vec) k_dequant_flat<FMT, YDT, 0, true><<<nb, kThreads, 0, st>>>(q, n, sinv, y);
            else k_dequant_flat<FMT, YDT, 0, false><<<nb, kThreads, 0, st>>>(q, n, sinv, y);
        } else {
            if (vec) k_dequant_flat<FMT, YDT, 2, true><<<nb, kThreads, 0, st>>>(q, n, sinv, y);
            else k_dequant_flat<FMT, YDT, 2, false><<<nb, kThreads, 0, st>>>(q, n, sinv, y);
        }
    }
};

template <int FMT, int YDT> struct RunDequantRows {
    static void run(const uint8_t* q, int64_t rows, int64_t cols, const float* sinv, void* y, hipStream_t st) {
        const bool vec = (cols % 16 == 0) && al16(q) && al16(y);
        const unsigned nb = blocks_for(rows, 1);
        if (vec) k_dequant_rows<FMT, YDT, true><<<nb, kThreads, 0, st>>>(q, rows, cols, sinv, y);
        else k_dequant_rows<FMT, YDT, false><<<nb, kThreads, 0, st>>>(q, rows, cols, sinv, y);
    }
};

template <int FMT, int YDT> struct RunBlock128 {
    static void run(const uint8_t* q, int64_t M, int64_t N, const float* sinv, void* y, hipStream_t st) {
        const int64_t nbm = (M + 127) / 128, nbn = (N + 127) / 128;
        if (N % 16 == 0 && al16(q) && al16(y)) {
            const int64_t ntiles = nbm * nbn;
            k_block128_v<FMT, YDT><<<blocks_for(ntiles, 1), kThreads, 0, st>>>(q, M, N, sinv, y, nbn, ntiles);
        } else {
            k_block128_s<FMT, YDT><<<blocks_for(M, 1), kThreads, 0, st>>>(q, M, N, sinv, y, nbn);
        }
    }
};

}  // namespace

void launch_fill_f32(float* p, int64_t n, float v, hipStream_t st) {
    k_fill_f32<<<blocks_for(n, kThreads), kThreads, 0, st>>>(p, n, v);
}

void launch_amax(const void* x, int dt, int64_t n, uint32_t* ws, hipStream_t st) {
    if (dt == kF32) run_amax<kF32>(x, n, ws, st);
    else if (dt == kBF16) run_amax<kBF16>(x, n, ws, st);
    else run_amax<kF16>(x, n, ws, st);
}

void launch_tensor_cast(const void* x, int dt, int64_t n, int fmt, const uint32_t* ws, uint8_t* q, float* sinv,
                        hipStream_t st) {
    dispatch_dt_fmt<RunTensorCast>(dt, fmt, x, n, ws, q, sinv, st);
}

void launch_channel_cast(const void* x, int dt, int64_t rows, int64_t cols, int fmt, uint8_t* q, float* sinv,
                         hipStream_t st) {
    dispatch_dt_fmt<RunChannel>(dt, fmt, x, rows, cols, q, sinv, st);
}

void launch_group128_cast(const void* x, int dt, int64_t groups, int fmt, uint8_t* q, float* sinv,
                          hipStream_t st) {
    dispatch_dt_fmt<RunGroup128>(dt, fmt, x, groups, q, sinv, st);
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
