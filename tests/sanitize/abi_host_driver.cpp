// Host-only check of the C ABI's argument validation, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_abi_sanitize.py compiles and runs it on the CPU).
//
// kda_api.hip is compiled unchanged for the host only; the kernel launchers it calls are
// replaced by the stubs below, which record that a launch was requested and touch no
// memory. Every pointer handed to the library is a host address: validation must never
// dereference one, which the sanitizers would report. The driver checks the status of
// every call and that no launcher runs for a rejected call.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/kda.h"

static int g_launches = 0;

namespace kda {
hipError_t launch_decode(bool, bool, bool, int, int, const void*, const void*, const void*,
                         const float*, const void*, const void*, const void*, float, float*,
                         void*, int, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_chunk_map(const int32_t*, int, int, int, void*, int32_t*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_prefill(bool, bool, bool, int, int, const void*, const void*, const void*,
                          const float*, const void*, const void*, const void*, float,
                          const float*, float*, void*, const int32_t*, int, const void*,
                          const int32_t*, uint8_t*, int, int, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_prefill_raw(bool, const void*, const void*, const void*, const void*,
                              const void*, float, const float*, float*, void*, const int32_t*,
                              int, const void*, const int32_t*, uint8_t*, int, int, int,
                              hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
// block size of the bf16 and fp32 layouts at d = 128 (any positive size exercises the
// workspace checks the same way)
size_t prefill_block_bytes(int Dk, int Dv, bool bf16_in) {
    return (size_t)(bf16_in ? 98816 : 147968) * (size_t)Dk * (size_t)Dv / (128 * 128);
}
hipError_t launch_decode_multi(bool, bool, int, int, const void*, const void*, const void*,
                               const float*, const void*, float, float*, const int32_t*, int,
                               float*, void*, int, int, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_prepare_inputs(bool, int, const void*, const void*, const void*, const void*,
                                 float, void*, void*, float*, void*, long long, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_state_copy(float*, const int32_t*, int, const float*, const int32_t*, int,
                             int, long long, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
}  // namespace kda

static int g_failures = 0;
static int g_checks = 0;

// status must equal want; launches must grow by `launched` (0 or the number of launches)
static void expect(const char* what, kda_status got, kda_status want, int before, int launched) {
    ++g_checks;
    const int grew = g_launches - before;
    if (got != want || grew != launched) {
        ++g_failures;
        fprintf(stderr, "FAIL %s: status %s (want %s), launches %d (want %d)\n", what,
                kda_status_string(got), kda_status_string(want), grew, launched);
    }
}

#define CHECK(what, call, want, launched)              \
    do {                                                \
        const int b_ = g_launches;                      \
        const kda_status s_ = (call);                   \
        expect(what, s_, want, b_, launched);           \
    } while (0)

int main() {
    // 16-byte aligned host buffers stand in for device memory (never read or written)
    alignas(256) static uint8_t arena[1 << 16];
    uint8_t* base = arena;
    const void* q = base;
    const void* k = base + 256;
    const void* v = base + 512;
    const float* g = reinterpret_cast<const float*>(base + 768);
    const void* beta = base + 1024;
    void* o = base + 1280;
    float* st = reinterpret_cast<float*>(base + 1536);
    const int32_t* cu = reinterpret_cast<const int32_t*>(base + 1792);
    const void* mis = base + 2;                       // misaligned
    const kda_dtype BF = KDA_DTYPE_BF16, F = KDA_DTYPE_F32, BAD = (kda_dtype)7;

    // status strings
    for (int sv = 0; sv <= 5; ++sv)
        if (!kda_status_string((kda_status)sv)) ++g_failures;

    // workspace size
    size_t bytes = 0;
    CHECK("ws null", kda_fwd_chunked_workspace_size(1, 64, 1, 16, 16, 1, 0, F, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("ws B0", kda_fwd_chunked_workspace_size(0, 64, 1, 16, 16, 1, 0, F, &bytes),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("ws Dk48", kda_fwd_chunked_workspace_size(1, 64, 1, 48, 16, 1, 0, F, &bytes),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("ws dtype", kda_fwd_chunked_workspace_size(1, 64, 1, 16, 16, 1, 0, BAD, &bytes),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("ws varlen B2", kda_fwd_chunked_workspace_size(2, 64, 1, 16, 16, 2, 1, F, &bytes),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("ws varlen N0", kda_fwd_chunked_workspace_size(1, 64, 1, 16, 16, 0, 1, F, &bytes),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("ws huge T", kda_fwd_chunked_workspace_size(1 << 20, 1 << 20, 64, 128, 128, 1, 0, BF,
                                                      &bytes),
          KDA_ERROR_NOT_SUPPORTED, 0);
    CHECK("ws INT_MAX", kda_fwd_chunked_workspace_size(2147483647, 2147483647, 2147483647, 128,
                                                       128, 2147483647, 1, BF, &bytes),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("ws huge H", kda_fwd_chunked_workspace_size(1, 1 << 20, 2147483647, 128, 128, 1, 0,
                                                      BF, &bytes),
          KDA_ERROR_NOT_SUPPORTED, 0);
    CHECK("ws ok", kda_fwd_chunked_workspace_size(1, 8192, 64, 128, 128, 1, 0, BF, &bytes),
          KDA_SUCCESS, 0);
    const size_t need = bytes;
    if (need == 0) ++g_failures;
    size_t need_var = 0;
    CHECK("ws varlen ok", kda_fwd_chunked_workspace_size(1, 8192, 64, 128, 128, 8, 1, BF, &need_var),
          KDA_SUCCESS, 0);
    if (need_var <= need) ++g_failures;   // the packed bound reserves more slots

    // prefill: the workspace pointer is checked for null, size and alignment before any use
    void* ws = base + 4096;
    CHECK("fwd ok", kda_fwd_chunked(q, k, v, g, beta, 1.f, nullptr, nullptr, o, nullptr, 1, 1,
                                    8192, 64, 128, 128, BF, F, ws, need, nullptr),
          KDA_SUCCESS, 1);
    CHECK("fwd varlen ok", kda_fwd_chunked(q, k, v, g, beta, 1.f, st, st, o, cu, 8, 1, 8192, 64,
                                           128, 128, BF, BF, ws, need_var, nullptr),
          KDA_SUCCESS, 2);
    CHECK("fwd small ws", kda_fwd_chunked(q, k, v, g, beta, 1.f, nullptr, nullptr, o, nullptr,
                                          1, 1, 8192, 64, 128, 128, BF, F, ws, need - 1, nullptr),
          KDA_ERROR_WORKSPACE, 0);
    CHECK("fwd null ws", kda_fwd_chunked(q, k, v, g, beta, 1.f, nullptr, nullptr, o, nullptr, 1,
                                         1, 64, 1, 16, 16, F, F, nullptr, 1 << 20, nullptr),
          KDA_ERROR_WORKSPACE, 0);
    CHECK("fwd ws misaligned", kda_fwd_chunked(q, k, v, g, beta, 1.f, nullptr, nullptr, o,
                                               nullptr, 1, 1, 64, 1, 16, 16, F, F, base + 4112,
                                               1 << 20, nullptr),
          KDA_ERROR_WORKSPACE, 0);
    CHECK("fwd null q", kda_fwd_chunked(nullptr, k, v, g, beta, 1.f, nullptr, nullptr, o, nullptr,
                                        1, 1, 64, 1, 16, 16, F, F, ws, need, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("fwd null beta", kda_fwd_chunked(q, k, v, g, nullptr, 1.f, nullptr, nullptr, o, nullptr,
                                           1, 1, 64, 1, 16, 16, F, F, ws, need, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("fwd misaligned k", kda_fwd_chunked(q, mis, v, g, beta, 1.f, nullptr, nullptr, o,
                                              nullptr, 1, 1, 64, 1, 16, 16, F, F, ws, need, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("fwd misaligned cu", kda_fwd_chunked(q, k, v, g, beta, 1.f, nullptr, nullptr, o,
                                               reinterpret_cast<const int32_t*>(base + 1793), 1,
                                               1, 64, 1, 16, 16, F, F, ws, need, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("fwd odtype", kda_fwd_chunked(q, k, v, g, beta, 1.f, nullptr, nullptr, o, nullptr, 1, 1,
                                        64, 1, 16, 16, F, BAD, ws, need, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("fwd varlen B2", kda_fwd_chunked(q, k, v, g, beta, 1.f, nullptr, nullptr, o, cu, 2, 2,
                                           64, 1, 16, 16, F, F, ws, need, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("fwd neg T", kda_fwd_chunked(q, k, v, g, beta, 1.f, nullptr, nullptr, o, nullptr, 1, 1,
                                       -64, 1, 16, 16, F, F, ws, need, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("gdn ok", kda_gdn_fwd_chunked(q, k, v, g, beta, 1.f, nullptr, nullptr, o, nullptr, 1, 1,
                                        8192, 64, 128, 128, BF, F, ws, need, nullptr),
          KDA_SUCCESS, 1);
    CHECK("gdn2 ok", kda_gdn2_fwd_chunked(q, k, v, g, k, v, 1.f, nullptr, nullptr, o, nullptr, 1,
                                          1, 8192, 64, 128, 128, BF, F, ws, need, nullptr),
          KDA_SUCCESS, 1);
    CHECK("gdn2 null w", kda_gdn2_fwd_chunked(q, k, v, g, k, nullptr, 1.f, nullptr, nullptr, o,
                                              nullptr, 1, 1, 64, 1, 16, 16, F, F, ws, need,
                                              nullptr),
          KDA_ERROR_INVALID_VALUE, 0);

    // decode
    CHECK("dec ok", kda_decode_step(q, k, v, g, beta, 1.f, st, o, 256, 64, 128, 128, BF, F,
                                    nullptr),
          KDA_SUCCESS, 1);
    CHECK("dec null state", kda_decode_step(q, k, v, g, beta, 1.f, nullptr, o, 1, 1, 16, 16, F, F,
                                            nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("dec Dv 8", kda_decode_step(q, k, v, g, beta, 1.f, st, o, 1, 1, 16, 8, F, F, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("dec N*H overflow", kda_decode_step(q, k, v, g, beta, 1.f, st, o, 1 << 20, 1 << 12, 16,
                                              16, F, F, nullptr),
          KDA_ERROR_NOT_SUPPORTED, 0);
    CHECK("gdn dec ok", kda_gdn_decode_step(q, k, v, g, beta, 1.f, st, o, 2, 2, 32, 64, F, BF,
                                            nullptr),
          KDA_SUCCESS, 1);
    CHECK("gdn2 dec null b", kda_gdn2_decode_step(q, k, v, g, nullptr, v, 1.f, st, o, 2, 2, 32,
                                                  64, F, BF, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);

    // multi-token decode and state copies
    const int32_t* slots = reinterpret_cast<const int32_t*>(base + 2048);
    CHECK("multi ok", kda_decode_multi(q, k, v, g, beta, 1.f, st, 512, slots, nullptr, o, 256, 4,
                                       64, 128, 128, BF, F, nullptr),
          KDA_SUCCESS, 1);
    CHECK("multi no slots", kda_decode_multi(q, k, v, g, beta, 1.f, st, 8, nullptr, nullptr, o,
                                             16, 4, 1, 16, 16, F, F, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("multi NT overflow", kda_decode_multi(q, k, v, g, beta, 1.f, st, 8, slots, nullptr, o,
                                                1 << 20, 1 << 12, 1, 16, 16, F, F, nullptr),
          KDA_ERROR_NOT_SUPPORTED, 0);
    CHECK("copy none", kda_state_copy(nullptr, 0, nullptr, nullptr, 0, nullptr, 0, 1, 16, 16,
                                      nullptr),
          KDA_SUCCESS, 0);
    CHECK("copy ok", kda_state_copy(st, 8, slots, st, 8, slots, 4, 64, 128, 128, nullptr),
          KDA_SUCCESS, 1);
    CHECK("copy many", kda_state_copy(st, 8, slots, st, 8, slots, 70000, 1, 16, 16, nullptr),
          KDA_ERROR_NOT_SUPPORTED, 0);
    CHECK("copy neg", kda_state_copy(st, 8, slots, st, 8, slots, -1, 1, 16, 16, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);

    // input preparation
    CHECK("prep ok", kda_prepare_inputs(q, k, v, beta, 1.f, o, o, st, o, 8192, 64, 128, BF,
                                        nullptr),
          KDA_SUCCESS, 1);
    CHECK("prep beta misaligned", kda_prepare_inputs(q, k, v, base + 1025, 1.f, o, o, st, o, 8,
                                                     1, 16, BF, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("prep huge", kda_prepare_inputs(q, k, v, beta, 1.f, o, o, st, o, 1LL << 40, 64, 16, F,
                                          nullptr),
          KDA_ERROR_NOT_SUPPORTED, 0);

    // the raw-projection prefill: bf16 at d = 128 only
    CHECK("raw ok", kda_fwd_chunked_raw(q, k, v, g, beta, 1.f, nullptr, nullptr, o, nullptr, 1, 1,
                                        8192, 64, 128, 128, BF, F, ws, need, nullptr),
          KDA_SUCCESS, 1);
    CHECK("raw varlen ok", kda_fwd_chunked_raw(q, k, v, g, beta, 1.f, st, st, o, cu, 8, 1, 8192, 64,
                                               128, 128, BF, BF, ws, need_var, nullptr),
          KDA_SUCCESS, 2);
    CHECK("raw f32", kda_fwd_chunked_raw(q, k, v, g, beta, 1.f, nullptr, nullptr, o, nullptr, 1, 1,
                                         64, 1, 128, 128, F, F, ws, need, nullptr),
          KDA_ERROR_NOT_SUPPORTED, 0);
    CHECK("raw d64", kda_fwd_chunked_raw(q, k, v, g, beta, 1.f, nullptr, nullptr, o, nullptr, 1, 1,
                                         64, 1, 64, 64, BF, F, ws, need, nullptr),
          KDA_ERROR_NOT_SUPPORTED, 0);
    CHECK("raw null a", kda_fwd_chunked_raw(q, k, v, nullptr, beta, 1.f, nullptr, nullptr, o,
                                            nullptr, 1, 1, 64, 1, 128, 128, BF, F, ws, need, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("raw b odd", kda_fwd_chunked_raw(q, k, v, g, base + 1025, 1.f, nullptr, nullptr, o,
                                           nullptr, 1, 1, 64, 1, 128, 128, BF, F, ws, need, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("raw small ws", kda_fwd_chunked_raw(q, k, v, g, beta, 1.f, nullptr, nullptr, o, nullptr,
                                              1, 1, 8192, 64, 128, 128, BF, F, ws, need - 1, nullptr),
          KDA_ERROR_WORKSPACE, 0);

    // the allocation-free prefill: a call beyond the built-in scratch is refused before any
    // device call; argument errors are those of kda_fwd_chunked
    CHECK("noalloc too big", kda_fwd_chunked_noalloc(q, k, v, g, beta, 1.f, nullptr, nullptr, o,
                                                     nullptr, 1, 1, 8192, 64, 128, 128, BF, F,
                                                     nullptr),
          KDA_ERROR_WORKSPACE, 0);
    CHECK("noalloc null beta", kda_fwd_chunked_noalloc(q, k, v, g, nullptr, 1.f, nullptr, nullptr,
                                                       o, nullptr, 1, 1, 64, 1, 16, 16, F, F,
                                                       nullptr),
          KDA_ERROR_INVALID_VALUE, 0);
    CHECK("noalloc bad dims", kda_fwd_chunked_noalloc(q, k, v, g, beta, 1.f, nullptr, nullptr, o,
                                                      nullptr, 1, 1, 64, 1, 24, 16, F, F, nullptr),
          KDA_ERROR_INVALID_VALUE, 0);

    printf("%d checks, %d failures\n", g_checks, g_failures);
    return g_failures == 0 ? 0 : 1;
}
