// Host-only stand-ins for the HIP launchers (fp8q_launch.h) and for
// hipGetLastError, so that the C ABI layer (fp8q_abi.cpp) can be built with
// g++ -fsanitize=address,undefined and driven from the CPU tests with no GPU
// and no HIP runtime.  Each stub checks the preconditions the ABI layer
// promises its launchers (positive sizes, non-null pointers) and counts its
// calls; fp8q_stub_count / fp8q_stub_reset expose the counts to the tests.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "fp8q_launch.h"

namespace {

struct Count {
    const char* name;
    long n;
};
Count g_counts[] = {{"fill_f32", 0},         {"amax", 0},          {"amax_partials", 0}, {"guard_amax", 0},
                    {"cast_given_amax", 0},  {"dequant_packed", 0}, {"pipeline_cast", 0}, {"dequant_pipeline", 0},
                    {"tensor_cast", 0},      {"channel_cast", 0},  {"group128_cast", 0}, {"dequant_flat", 0},
                    {"dequant_rows", 0},     {"block128", 0},      {"dequant_sum", 0},
                    {"scratch_words", 0},    {"group128_cast_wave64", 0}};

void hit(const char* name) {
    for (Count& c : g_counts)
        if (strcmp(c.name, name) == 0) { ++c.n; return; }
    abort();
}

// a violated launcher precondition is a bug in the ABI layer: stop loudly
void need(bool ok) {
    if (!ok) abort();
}

bool dt_ok(int d) { return d == fp8q::kF32 || d == fp8q::kBF16 || d == fp8q::kF16; }
bool fmt_ok(int f) { return f == fp8q::kE4M3 || f == fp8q::kE5M2; }

}  // namespace

extern "C" long fp8q_stub_count(const char* name) {
    for (const Count& c : g_counts)
        if (strcmp(c.name, name) == 0) return c.n;
    return -1;
}

extern "C" void fp8q_stub_reset(void) {
    for (Count& c : g_counts) c.n = 0;
}

hipError_t hipGetLastError(void) { return hipSuccess; }

namespace fp8q {

void launch_fill_f32(float* p, int64_t n, float, hipStream_t) { need(p && n > 0); hit("fill_f32"); }

void launch_amax(const void* x, int dt, int64_t n, uint32_t* word, hipStream_t) {
    need(word && dt_ok(dt) && n >= 0 && (n == 0 || x));
    hit("amax");
}

int launch_amax_partials(const void* x, int dt, int64_t n, uint32_t* partial, hipStream_t) {
    need(partial && dt_ok(dt) && n >= 0 && (n == 0 || x));
    hit("amax_partials");
    return 1;
}

int amax_partials_count(const void* x, int dt, int64_t n) {
    need(dt_ok(dt) && n >= 0 && (n == 0 || x));
    return 1;
}

// a host array stands in for the device scratch: the stubs never dereference it
uint32_t g_scratch_stub[kScratchWords];

hipError_t scratch_words(hipStream_t, uint32_t** out) {
    need(out != nullptr);
    hit("scratch_words");
    *out = g_scratch_stub;
    return hipSuccess;
}

void launch_guard_amax(uint32_t* ws, hipStream_t) { need(ws != nullptr); hit("guard_amax"); }

void launch_cast_given_amax(const void* x, int dt, int64_t n, int fmt, const float* amax, uint8_t* q,
                            float* scale_out, hipStream_t) {
    need(dt_ok(dt) && fmt_ok(fmt) && amax && scale_out && n >= 0 && (n == 0 || (x && q)));
    hit("cast_given_amax");
}

void launch_dequant_packed(const uint8_t* slots, int fmt, int64_t W, int64_t n, void* y, int ydt, hipStream_t) {
    need(slots && y && fmt_ok(fmt) && dt_ok(ydt) && W > 0 && n > 0);
    hit("dequant_packed");
}

void launch_pipeline_cast(const void* x, int dt, int64_t n, const uint32_t* partial, int np, uint8_t* q,
                          float* sinv, int32_t* fmt_out, hipStream_t) {
    need(dt_ok(dt) && partial && np >= 1 && np <= kAmaxPartials && sinv && fmt_out && (n == 0 || (x && q)));
    hit("pipeline_cast");
}

void launch_dequant_pipeline(const uint8_t* q, int64_t n, const float* sinv, const int32_t* fmt, void* y, int ydt,
                             hipStream_t) {
    need(q && n > 0 && sinv && fmt && y && dt_ok(ydt));
    hit("dequant_pipeline");
}

void launch_tensor_cast(const void* x, int dt, int64_t n, int fmt, const uint32_t* partial, int np, int pstride,
                        uint8_t* q, float* sinv, hipStream_t, bool) {
    need(x && dt_ok(dt) && n > 0 && fmt_ok(fmt) && partial && np >= 1 && pstride >= 1 && q && sinv);
    hit("tensor_cast");
}

void launch_channel_cast(const void* x, int dt, int64_t rows, int64_t cols, int fmt, uint8_t* q, float* sinv,
                         hipStream_t) {
    need(x && dt_ok(dt) && rows > 0 && cols > 0 && fmt_ok(fmt) && q && sinv);
    hit("channel_cast");
}

void launch_group128_cast(const void* x, int dt, int64_t groups, int fmt, uint8_t* q, float* sinv, hipStream_t) {
    need(x && dt_ok(dt) && groups > 0 && fmt_ok(fmt) && q && sinv);
    hit("group128_cast");
}

void launch_group128_cast_wave64(const void* x, int dt, int64_t groups, int fmt, uint8_t* q, float* sinv,
                                 hipStream_t) {
    need(x && dt_ok(dt) && groups > 0 && fmt_ok(fmt) && q && sinv);
    need((uintptr_t)x % (dt == fp8q::kF32 ? 8 : 4) == 0 && (uintptr_t)q % 2 == 0);
    hit("group128_cast_wave64");
}

void launch_dequant_flat(int mode, const uint8_t* q, int fmt, int64_t n, const float* sinv, void* y, int ydt,
                         hipStream_t) {
    need((mode == 0 || mode == 2 || mode == 3) && q && fmt_ok(fmt) && n > 0 && sinv && y && dt_ok(ydt));
    need(mode != 2 || n % 128 == 0);
    hit("dequant_flat");
}

void launch_dequant_rows(const uint8_t* q, int fmt, int64_t rows, int64_t cols, const float* sinv, void* y, int ydt,
                         hipStream_t) {
    need(q && fmt_ok(fmt) && rows > 0 && cols > 0 && sinv && y && dt_ok(ydt));
    hit("dequant_rows");
}

void launch_block128(const uint8_t* q, int fmt, int64_t M, int64_t N, const float* sinv, void* y, int ydt,
                     hipStream_t) {
    need(q && fmt_ok(fmt) && M > 0 && N > 0 && sinv && y && dt_ok(ydt));
    hit("block128");
}

void launch_dequant_sum(const uint8_t* q, int fmt, int64_t W, int64_t n, const float* sinv, int, void* y, int ydt,
                        uint32_t*, hipStream_t) {
    need(q && fmt_ok(fmt) && W >= 1 && n > 0 && sinv && y && dt_ok(ydt));
    hit("dequant_sum");
}

}  // namespace fp8q
