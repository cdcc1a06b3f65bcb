// Host side of the C ABI declared in include/kda.h: argument validation,
// workspace carving and kernel launches. Every check happens before the first
// launch, so an invalid call enqueues nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/kda.h"

namespace kda {
hipError_t launch_decode(bool sg, bool bf16_in, bool bf16_out, int Dk, int Dv, const void* q,
                         const void* k, const void* v, const float* g, const void* beta,
                         const void* eb, const void* ew, float scale, float* state, void* o,
                         int N, int H, hipStream_t s);
hipError_t launch_chunk_map(const int32_t* cu, int N, int T, int max_slots, void* tab,
                            int32_t* seq_off, hipStream_t s);
hipError_t launch_prefill(bool sg, bool bf16_in, bool bf16_out, int Dk, int Dv, const void* q,
                          const void* k, const void* v, const float* g, const void* beta,
                          const void* eb, const void* ew, float scale, const float* h0,
                          float* ht, void* o, const int32_t* cu, int T, const void* tab,
                          const int32_t* seq_off, uint8_t* blocks, int N, int H, int max_slots,
                          hipStream_t s);
hipError_t launch_prefill_raw(bool bf16_out, const void* q, const void* k, const void* v,
                              const void* a, const void* b, float scale, const float* h0,
                              float* ht, void* o, const int32_t* cu, int T, const void* tab,
                              const int32_t* seq_off, uint8_t* blocks, int N, int H,
                              int max_slots, hipStream_t s);
size_t prefill_block_bytes(int Dk, int Dv, bool bf16_in);
hipError_t launch_decode_multi(bool bf16_in, bool bf16_out, int Dk, int Dv, const void* q,
                               const void* k, const void* v, const float* g, const void* beta,
                               float scale, float* pool, const int32_t* slots, int num_slots,
                               float* snapshots, void* o, int N, int T, int H, hipStream_t s);
hipError_t launch_prepare_inputs(bool bf16_io, int Dk, const void* q, const void* k,
                                 const void* a, const void* b, float scale, void* qo, void* ko,
                                 float* go, void* bo, long long rows, hipStream_t s);
hipError_t launch_state_copy(float* dst, const int32_t* dst_slots, int dst_count,
                             const float* src, const int32_t* src_slots, int src_count,
                             int pairs, long long state_floats, hipStream_t s);
}  // namespace kda

namespace {

bool head_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool dtype_ok(kda_dtype t) { return t == KDA_DTYPE_F32 || t == KDA_DTYPE_BF16; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t ru(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct PrefillPlan {
    long long max_slots = 0;
    int nseq = 0;
    size_t tab_off = 0, seq_off = 0, blocks_off = 0, total = 0;
};

kda_status plan_prefill(int B, int T, int H, int Dk, int Dv, int num_seqs, bool varlen,
                        kda_dtype dtype, PrefillPlan* p) {
    if (B <= 0 || T <= 0 || H <= 0) return KDA_ERROR_INVALID_VALUE;
    if (!head_ok(Dk) || !head_ok(Dv)) return KDA_ERROR_INVALID_VALUE;
    if (!dtype_ok(dtype)) return KDA_ERROR_INVALID_VALUE;
    if (varlen && (B != 1 || num_seqs < 1)) return KDA_ERROR_INVALID_VALUE;
    const long long tokens = (long long)B * T;
    if (tokens > (1LL << 30)) return KDA_ERROR_NOT_SUPPORTED;
    p->nseq = varlen ? num_seqs : B;
    p->max_slots = varlen ? (long long)T / 64 + num_seqs : (long long)B * ((T + 63) / 64);
    if (p->max_slots > (1LL << 30) / H) return KDA_ERROR_NOT_SUPPORTED;
    p->tab_off = 0;
    p->seq_off = ru((size_t)p->max_slots * 16, 256);
    p->blocks_off = p->seq_off + ru((size_t)(p->nseq + 1) * 4, 256);
    p->total = p->blocks_off +
               (size_t)p->max_slots * H * kda::prefill_block_bytes(Dk, Dv, dtype == KDA_DTYPE_BF16);
    return KDA_SUCCESS;
}

// sg: scalar gate (Gated DeltaNet), g holds one value per token and head; eb, ew: the erase
// and write gates of Gated DeltaNet-2, given together in place of beta
kda_status fwd_chunked(bool sg, const void* q, const void* k, const void* v, const float* g,
                       const void* beta, const void* eb, const void* ew, float scale,
                       const float* h0, float* ht, void* o, const int32_t* cu_seqlens,
                       int num_seqs, int B, int T, int H, int Dk, int Dv, kda_dtype dtype,
                       kda_dtype o_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !g || !o) return KDA_ERROR_INVALID_VALUE;
    if (eb || ew ? !(eb && ew) : !beta) return KDA_ERROR_INVALID_VALUE;
    if (!dtype_ok(o_dtype)) return KDA_ERROR_INVALID_VALUE;
    PrefillPlan p;
    const kda_status st = plan_prefill(B, T, H, Dk, Dv, num_seqs, cu_seqlens != nullptr, dtype, &p);
    if (st != KDA_SUCCESS) return st;
    const void* ptrs[] = {q, k, v, g, beta, eb, ew, o, h0, ht};
    for (const void* ptr : ptrs)
        if (ptr && !aligned(ptr, 16)) return KDA_ERROR_INVALID_VALUE;
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return KDA_ERROR_INVALID_VALUE;
    if (!workspace || workspace_bytes < p.total || !aligned(workspace, 256))
        return KDA_ERROR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    void* tab = nullptr;
    int32_t* seq_off = nullptr;
    if (cu_seqlens) {                          // packed sequences: chunk table on the device
        tab = ws + p.tab_off;
        seq_off = reinterpret_cast<int32_t*>(ws + p.seq_off);
        if (kda::launch_chunk_map(cu_seqlens, p.nseq, T, (int)p.max_slots, tab, seq_off, s) !=
            hipSuccess)
            return KDA_ERROR_LAUNCH;
    }
    if (kda::launch_prefill(sg, dtype == KDA_DTYPE_BF16, o_dtype == KDA_DTYPE_BF16, Dk, Dv, q, k,
                            v, g, beta, eb, ew, scale, h0, ht, o, cu_seqlens, T, tab, seq_off,
                            ws + p.blocks_off, p.nseq, H, (int)p.max_slots, s) != hipSuccess)
        return KDA_ERROR_LAUNCH;
    return KDA_SUCCESS;
}

// the raw-projection prefill: same checks and workspace as fwd_chunked
kda_status fwd_chunked_raw(const void* q, const void* k, const void* v, const void* a,
                           const void* b, float scale, const float* h0, float* ht, void* o,
                           const int32_t* cu_seqlens, int num_seqs, int B, int T, int H, int Dk,
                           int Dv, kda_dtype dtype, kda_dtype o_dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !a || !b || !o) return KDA_ERROR_INVALID_VALUE;
    if (!dtype_ok(o_dtype)) return KDA_ERROR_INVALID_VALUE;
    PrefillPlan p;
    const kda_status st = plan_prefill(B, T, H, Dk, Dv, num_seqs, cu_seqlens != nullptr, dtype, &p);
    if (st != KDA_SUCCESS) return st;
    if (dtype != KDA_DTYPE_BF16 || Dk != 128 || Dv != 128) return KDA_ERROR_NOT_SUPPORTED;
    const void* ptrs[] = {q, k, v, a, o, h0, ht};
    for (const void* ptr : ptrs)
        if (ptr && !aligned(ptr, 16)) return KDA_ERROR_INVALID_VALUE;
    if (!aligned(b, 2)) return KDA_ERROR_INVALID_VALUE;
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return KDA_ERROR_INVALID_VALUE;
    if (!workspace || workspace_bytes < p.total || !aligned(workspace, 256))
        return KDA_ERROR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    void* tab = nullptr;
    int32_t* seq_off = nullptr;
    if (cu_seqlens) {
        tab = ws + p.tab_off;
        seq_off = reinterpret_cast<int32_t*>(ws + p.seq_off);
        if (kda::launch_chunk_map(cu_seqlens, p.nseq, T, (int)p.max_slots, tab, seq_off, s) !=
            hipSuccess)
            return KDA_ERROR_LAUNCH;
    }
    if (kda::launch_prefill_raw(o_dtype == KDA_DTYPE_BF16, q, k, v, a, b, scale, h0, ht, o,
                                cu_seqlens, T, tab, seq_off, ws + p.blocks_off, p.nseq, H,
                                (int)p.max_slots, s) != hipSuccess)
        return KDA_ERROR_LAUNCH;
    return KDA_SUCCESS;
}

kda_status decode_step(bool sg, const void* q, const void* k, const void* v, const float* g,
                       const void* beta, const void* eb, const void* ew, float scale,
                       float* state, void* o, int N, int H, int Dk, int Dv, kda_dtype dtype,
                       kda_dtype o_dtype, void* stream) {
    if (!q || !k || !v || !g || !state || !o) return KDA_ERROR_INVALID_VALUE;
    if (eb || ew ? !(eb && ew) : !beta) return KDA_ERROR_INVALID_VALUE;
    if (N <= 0 || H <= 0 || !head_ok(Dk) || !head_ok(Dv)) return KDA_ERROR_INVALID_VALUE;
    if (!dtype_ok(dtype) || !dtype_ok(o_dtype)) return KDA_ERROR_INVALID_VALUE;
    if ((long long)N * H > (1LL << 31) - 1) return KDA_ERROR_NOT_SUPPORTED;
    const void* ptrs[] = {q, k, v, g, beta, eb, ew, state, o};
    for (const void* ptr : ptrs)
        if (ptr && !aligned(ptr, 16)) return KDA_ERROR_INVALID_VALUE;
    if (kda::launch_decode(sg, dtype == KDA_DTYPE_BF16, o_dtype == KDA_DTYPE_BF16, Dk, Dv, q, k, v,
                           g, beta, eb, ew, scale, state, o, N, H,
                           reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return KDA_ERROR_LAUNCH;
    return KDA_SUCCESS;
}

// ------------------------------------------------------------------------------------------
// built-in scratch of kda_fwd_chunked_noalloc: one array per device, held until the process
// ends. Host code never uses the array's name as an address (on the host it is a stand-in,
// not device memory): the device address comes from hipGetSymbolAddress, once per device,
// with that device current.
// ------------------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// device address of the current device's scratch array, or nullptr on failure
void* scratch_of_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
        g_scratch_ptr[dev].store(addr, std::memory_order_release);
        p = addr;
    }
    return p;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_SUCCESS: return "KDA_SUCCESS";
        case KDA_ERROR_INVALID_VALUE: return "KDA_ERROR_INVALID_VALUE";
        case KDA_ERROR_NOT_SUPPORTED: return "KDA_ERROR_NOT_SUPPORTED";
        case KDA_ERROR_WORKSPACE: return "KDA_ERROR_WORKSPACE";
        case KDA_ERROR_LAUNCH: return "KDA_ERROR_LAUNCH";
        default: break;
    }
    return "KDA_ERROR_UNKNOWN";
}

kda_status kda_fwd_chunked_workspace_size(int B, int T, int H, int Dk, int Dv, int num_seqs,
                                          int cu_seqlens_given, kda_dtype dtype, size_t* bytes) {
    if (!bytes) return KDA_ERROR_INVALID_VALUE;
    PrefillPlan p;
    const kda_status st = plan_prefill(B, T, H, Dk, Dv, num_seqs, cu_seqlens_given != 0, dtype, &p);
    if (st != KDA_SUCCESS) return st;
    *bytes = p.total;
    return KDA_SUCCESS;
}

kda_status kda_fwd_chunked(const void* q, const void* k, const void* v, const float* g,
                           const void* beta, float scale, const float* h0, float* ht, void* o,
                           const int32_t* cu_seqlens, int num_seqs, int B, int T, int H, int Dk,
                           int Dv, kda_dtype dtype, kda_dtype o_dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (!beta) return KDA_ERROR_INVALID_VALUE;
    return fwd_chunked(false, q, k, v, g, beta, nullptr, nullptr, scale, h0, ht, o, cu_seqlens,
                       num_seqs, B, T, H, Dk, Dv, dtype, o_dtype, workspace, workspace_bytes,
                       stream);
}

kda_status kda_fwd_chunked_noalloc(const void* q, const void* k, const void* v, const float* g,
                                   const void* beta, float scale, const float* h0, float* ht,
                                   void* o, const int32_t* cu_seqlens, int num_seqs, int B, int T,
                                   int H, int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                                   void* stream) {
    if (!beta) return KDA_ERROR_INVALID_VALUE;
    // the size check first: a call the scratch cannot hold is rejected before any device call
    PrefillPlan p;
    const kda_status st = plan_prefill(B, T, H, Dk, Dv, num_seqs, cu_seqlens != nullptr, dtype, &p);
    if (st != KDA_SUCCESS) return st;
    if (p.total > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERROR_WORKSPACE;
    void* ws = scratch_of_current_device();
    if (!ws) return KDA_ERROR_LAUNCH;
    return fwd_chunked(false, q, k, v, g, beta, nullptr, nullptr, scale, h0, ht, o, cu_seqlens,
                       num_seqs, B, T, H, Dk, Dv, dtype, o_dtype, ws, KDA_NOALLOC_SCRATCH_BYTES,
                       stream);
}

kda_status kda_fwd_chunked_raw(const void* q, const void* k, const void* v, const void* a,
                               const void* b, float scale, const float* h0, float* ht, void* o,
                               const int32_t* cu_seqlens, int num_seqs, int B, int T, int H,
                               int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_chunked_raw(q, k, v, a, b, scale, h0, ht, o, cu_seqlens, num_seqs, B, T, H, Dk,
                           Dv, dtype, o_dtype, workspace, workspace_bytes, stream);
}

kda_status kda_gdn_fwd_chunked(const void* q, const void* k, const void* v, const float* g,
                               const void* beta, float scale, const float* h0, float* ht,
                               void* o, const int32_t* cu_seqlens, int num_seqs, int B, int T,
                               int H, int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
    if (!beta) return KDA_ERROR_INVALID_VALUE;
    return fwd_chunked(true, q, k, v, g, beta, nullptr, nullptr, scale, h0, ht, o, cu_seqlens,
                       num_seqs, B, T, H, Dk, Dv, dtype, o_dtype, workspace, workspace_bytes,
                       stream);
}

kda_status kda_gdn2_fwd_chunked(const void* q, const void* k, const void* v, const float* g,
                                const void* b, const void* w, float scale, const float* h0,
                                float* ht, void* o, const int32_t* cu_seqlens, int num_seqs,
                                int B, int T, int H, int Dk, int Dv, kda_dtype dtype,
                                kda_dtype o_dtype, void* workspace, size_t workspace_bytes,
                                void* stream) {
    if (!b || !w) return KDA_ERROR_INVALID_VALUE;
    return fwd_chunked(false, q, k, v, g, nullptr, b, w, scale, h0, ht, o, cu_seqlens, num_seqs,
                       B, T, H, Dk, Dv, dtype, o_dtype, workspace, workspace_bytes, stream);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const float* g,
                           const void* beta, float scale, float* state, void* o, int N, int H,
                           int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype, void* stream) {
    if (!beta) return KDA_ERROR_INVALID_VALUE;
    return decode_step(false, q, k, v, g, beta, nullptr, nullptr, scale, state, o, N, H, Dk, Dv,
                       dtype, o_dtype, stream);
}

kda_status kda_gdn_decode_step(const void* q, const void* k, const void* v, const float* g,
                               const void* beta, float scale, float* state, void* o, int N,
                               int H, int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                               void* stream) {
    if (!beta) return KDA_ERROR_INVALID_VALUE;
    return decode_step(true, q, k, v, g, beta, nullptr, nullptr, scale, state, o, N, H, Dk, Dv,
                       dtype, o_dtype, stream);
}

kda_status kda_gdn2_decode_step(const void* q, const void* k, const void* v, const float* g,
                                const void* b, const void* w, float scale, float* state, void* o,
                                int N, int H, int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                                void* stream) {
    if (!b || !w) return KDA_ERROR_INVALID_VALUE;
    return decode_step(false, q, k, v, g, nullptr, b, w, scale, state, o, N, H, Dk, Dv, dtype,
                       o_dtype, stream);
}

kda_status kda_decode_multi(const void* q, const void* k, const void* v, const float* g,
                            const void* beta, float scale, float* pool, int num_slots,
                            const int32_t* slots, float* snapshots, void* o, int N, int T,
                            int H, int Dk, int Dv, kda_dtype dtype, kda_dtype o_dtype,
                            void* stream) {
    if (!q || !k || !v || !g || !beta || !pool || !o) return KDA_ERROR_INVALID_VALUE;
    if (N <= 0 || T <= 0 || H <= 0 || num_slots <= 0) return KDA_ERROR_INVALID_VALUE;
    if (!slots && num_slots < N) return KDA_ERROR_INVALID_VALUE;
    if (!head_ok(Dk) || !head_ok(Dv)) return KDA_ERROR_INVALID_VALUE;
    if (!dtype_ok(dtype) || !dtype_ok(o_dtype)) return KDA_ERROR_INVALID_VALUE;
    if ((long long)N * H > (1LL << 31) - 1 || (long long)N * T > (1LL << 31) - 1)
        return KDA_ERROR_NOT_SUPPORTED;
    const void* ptrs[] = {q, k, v, g, beta, pool, snapshots, o};
    for (const void* ptr : ptrs)
        if (ptr && !aligned(ptr, 16)) return KDA_ERROR_INVALID_VALUE;
    if (slots && !aligned(slots, 4)) return KDA_ERROR_INVALID_VALUE;
    if (kda::launch_decode_multi(dtype == KDA_DTYPE_BF16, o_dtype == KDA_DTYPE_BF16, Dk, Dv, q, k,
                                 v, g, beta, scale, pool, slots, num_slots, snapshots, o, N, T,
                                 H, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return KDA_ERROR_LAUNCH;
    return KDA_SUCCESS;
}

kda_status kda_state_copy(float* dst, int dst_count, const int32_t* dst_slots, const float* src,
                          int src_count, const int32_t* src_slots, int pairs, int H, int Dk,
                          int Dv, void* stream) {
    if (pairs == 0) return KDA_SUCCESS;
    if (!dst || !dst_slots || !src || !src_slots) return KDA_ERROR_INVALID_VALUE;
    if (pairs < 0 || dst_count <= 0 || src_count <= 0 || H <= 0) return KDA_ERROR_INVALID_VALUE;
    if (!head_ok(Dk) || !head_ok(Dv)) return KDA_ERROR_INVALID_VALUE;
    if (pairs > 65535) return KDA_ERROR_NOT_SUPPORTED;
    if (!aligned(dst, 16) || !aligned(src, 16) || !aligned(dst_slots, 4) ||
        !aligned(src_slots, 4))
        return KDA_ERROR_INVALID_VALUE;
    if (kda::launch_state_copy(dst, dst_slots, dst_count, src, src_slots, src_count, pairs,
                               (long long)H * Dk * Dv,
                               reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return KDA_ERROR_LAUNCH;
    return KDA_SUCCESS;
}

kda_status kda_prepare_inputs(const void* q, const void* k, const void* a, const void* b,
                              float scale, void* q_out, void* k_out, float* g_out,
                              void* beta_out, long long tokens, int H, int Dk, kda_dtype dtype,
                              void* stream) {
    if (!q || !k || !a || !b || !q_out || !k_out || !g_out || !beta_out)
        return KDA_ERROR_INVALID_VALUE;
    if (tokens <= 0 || H <= 0 || !head_ok(Dk) || !dtype_ok(dtype)) return KDA_ERROR_INVALID_VALUE;
    if (tokens > (1LL << 34) / H) return KDA_ERROR_NOT_SUPPORTED;   // grid size
    const void* ptrs[] = {q, k, a, q_out, k_out, g_out};
    for (const void* ptr : ptrs)
        if (!aligned(ptr, 16)) return KDA_ERROR_INVALID_VALUE;
    const size_t el = dtype == KDA_DTYPE_BF16 ? 2 : 4;
    if (!aligned(b, el) || !aligned(beta_out, el)) return KDA_ERROR_INVALID_VALUE;
    if (kda::launch_prepare_inputs(dtype == KDA_DTYPE_BF16, Dk, q, k, a, b, scale, q_out, k_out,
                                   g_out, beta_out, tokens * H,
                                   reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return KDA_ERROR_LAUNCH;
    return KDA_SUCCESS;
}

}  // extern "C"
