/*
 * A plain C caller of the fp8q C ABI (no torch, no C++): it allocates device
 * memory with the HIP runtime API, runs a per-128-group cast and its dequant
 * (DeepEP "5 Utils", per_token_cast_to_fp8) and a per-tensor cast (ColossalAI
 * fp8.py, cast_to_fp8) on a stream, and checks properties that follow from
 * the definitions:
 *   - the element holding a group's or the tensor's amax encodes to the
 *     format's largest code, with its sign;
 *   - an all-zero group gets scale_inv = fl32(fl32(1e-4) / 448) (0x346FACAD) and zero codes;
 *   - every dequantized value is within 2^-4 relative of the input (e4m3fn,
 *     for inputs in the normal range), plus the bf16 output rounding;
 *   - argument errors come back as status codes before any work is queued.
 * Prints "c_abi_example: OK" and exits 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8q.h"

#define HIPCHECK(x)                                                              \
    do {                                                                         \
        hipError_t e_ = (x);                                                     \
        if (e_ != hipSuccess) {                                                  \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                            \
        }                                                                        \
    } while (0)
#define FQCHECK(x)                                                               \
    do {                                                                         \
        int s_ = (x);                                                            \
        if (s_ != FP8Q_OK) {                                                     \
            fprintf(stderr, "fp8q error %s at line %d\n", fp8q_status_str(s_), __LINE__); \
            return 1;                                                            \
        }                                                                        \
    } while (0)

static uint16_t to_bf16(float f) { /* inputs below are exact in bf16 */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int main(void) {
    enum { ROWS = 64, COLS = 1024, G = COLS / 128, N = ROWS * COLS };
    uint16_t* hx = malloc(sizeof(uint16_t) * N);
    uint8_t* hq = malloc(N);
    float* hs = malloc(sizeof(float) * ROWS * G);
    uint16_t* hy = malloc(sizeof(uint16_t) * N);
    /* values k/64 for small integers k (exact in bf16), one planted extreme per group, row 5 all zero */
    for (int r = 0; r < ROWS; ++r)
        for (int c = 0; c < COLS; ++c) {
            int k = ((r * 131 + c * 29) % 255) - 127;
            float v = (float)k / 64.0f;
            if (c % 128 == (r * 7) % 128) v = (r % 2 ? -1.0f : 1.0f) * (float)(3 + r % 50);
            if (r == 5) v = 0.0f;
            hx[r * COLS + c] = to_bf16(v);
        }
    void *dx, *dq, *ds, *dy, *dws, *dq2, *ds2;
    HIPCHECK(hipMalloc(&dx, sizeof(uint16_t) * N));
    HIPCHECK(hipMalloc(&dq, N));
    HIPCHECK(hipMalloc(&ds, sizeof(float) * ROWS * G));
    HIPCHECK(hipMalloc(&dy, sizeof(uint16_t) * N));
    HIPCHECK(hipMalloc(&dq2, N));
    HIPCHECK(hipMalloc(&ds2, sizeof(float)));
    HIPCHECK(hipMalloc(&dws, fp8q_per_tensor_workspace_bytes()));
    hipStream_t st;
    HIPCHECK(hipStreamCreate(&st));
    HIPCHECK(hipMemcpy(dx, hx, sizeof(uint16_t) * N, hipMemcpyHostToDevice));

    /* errors are reported before any work is queued */
    if (fp8q_cast_per_group128(dx, FP8Q_BF16, ROWS, 100, FP8Q_E4M3FN, dq, ds, st) != FP8Q_ESHAPE) return 2;
    if (fp8q_cast_per_group128(dx, 7, ROWS, COLS, FP8Q_E4M3FN, dq, ds, st) != FP8Q_EDTYPE) return 2;
    if (fp8q_cast_per_tensor(dx, FP8Q_BF16, N, FP8Q_E5M2, dq2, ds2, NULL, st) != FP8Q_EINVAL) return 2;

    FQCHECK(fp8q_cast_per_group128(dx, FP8Q_BF16, ROWS, COLS, FP8Q_E4M3FN, dq, ds, st));
    FQCHECK(fp8q_dequant_per_group128(dq, FP8Q_E4M3FN, ROWS, COLS, ds, dy, FP8Q_BF16, st));
    FQCHECK(fp8q_cast_per_tensor(dx, FP8Q_BF16, N, FP8Q_E5M2, dq2, ds2, dws, st));
    HIPCHECK(hipStreamSynchronize(st));
    HIPCHECK(hipMemcpy(hq, dq, N, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(hs, ds, sizeof(float) * ROWS * G, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(hy, dy, sizeof(uint16_t) * N, hipMemcpyDeviceToHost));

    int fails = 0;
    for (int r = 0; r < ROWS; ++r)
        for (int g = 0; g < G; ++g) {
            const int base = r * COLS + g * 128;
            float amax = 0.0f;
            int at = -1;
            for (int i = 0; i < 128; ++i)
                if (fabsf(from_bf16(hx[base + i])) > amax) amax = fabsf(from_bf16(hx[base + i])), at = base + i;
            if (r == 5) {
                uint32_t bits;
                memcpy(&bits, &hs[r * G + g], 4);
                if (bits != 0x346FACADu) fails++;
                for (int i = 0; i < 128; ++i) fails += hq[base + i] != 0;
                continue;
            }
            const uint8_t want = (from_bf16(hx[at]) < 0 ? 0x80 : 0x00) | 0x7E;
            if (hq[at] != want) fails++;
            for (int i = 0; i < 128; ++i) {
                const float x = from_bf16(hx[base + i]), y = from_bf16(hy[base + i]);
                if (fabsf(x) / hs[r * G + g] >= 0x1p-6f && fabsf(y - x) > fabsf(x) * (0.0625f * 1.004f + 0x1p-8f)) fails++;
            }
        }
    /* per tensor: the planted 52-magnitude element is the amax; it maps to the e5m2 maximum */
    uint8_t q2[N];
    HIPCHECK(hipMemcpy(q2, dq2, N, hipMemcpyDeviceToHost));
    float tmax = 0.0f;
    int tat = 0;
    for (int i = 0; i < N; ++i)
        if (fabsf(from_bf16(hx[i])) > tmax) tmax = fabsf(from_bf16(hx[i])), tat = i;
    if ((q2[tat] & 0x7F) != 0x7B) fails++;

    HIPCHECK(hipStreamDestroy(st));
    hipFree(dx); hipFree(dq); hipFree(ds); hipFree(dy); hipFree(dq2); hipFree(ds2); hipFree(dws);
    free(hx); free(hq); free(hs); free(hy);
    if (fails) {
        printf("c_abi_example: %d failures\n", fails);
        return 1;
    }
    printf("c_abi_example: OK (ABI version %d)\n", fp8q_abi_version());
    return 0;
}
