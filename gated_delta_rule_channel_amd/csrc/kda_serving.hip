// Serving-state operations for decode: the recurrent state of a request is
// request-scoped serving state, kept in a pool like a KV-cache slot, and it
// must be carried, copied on a fork and restored on a speculative rollback
// ("Module 03 - KDA I: The Delta-Rule Recurrence", jared-hpc.com, section 5).
//
// decode_multi_kernel: T consecutive tokens per request against the state in
// slot slots[n] of a pool (one workgroup per (request, head)). The state is
// read once, kept in registers across the T steps (each the recurrent step of
// "Kimi Delta Attention (KDA)", "Two schedules for the same recurrence"), and
// written once; optionally the state after every token is written to a
// snapshot array, so that a caller verifying T drafted tokens can restore the
// state after any accepted prefix. The work split is that of the single-step
// decode kernel with at most 512 threads: a thread owns four value columns of
// RPT rows; column sums go
// through lane shuffles and LDS, double-buffered by token parity so that one
// barrier per token suffices. The next token's inputs are loaded, unconverted,
// while the current token is processed.
//
// state_copy_kernel: dst[dst_slots[i]] = src[src_slots[i]] for whole states,
// 16-byte vector copies, one workgroup per (pair, 1024 float4 chunk).
#include "kda_common.h"

namespace kda {

int next_decode_order();                         // alternating state order (kda_decode.hip)

template <int DK, int DV>
struct MultiShape {
    static constexpr int CG = DV / 4;
    static constexpr int NT0 = DK * DV / 16;
    // at most 512 threads (8 rows each at d = 128), two workgroups per CU: the state and two
    // tokens' inputs stay in registers across the token loop (at 128 x 128 the compiler
    // spills 16-128 bytes a lane at this occupancy; one workgroup per CU without spills
    // measured slower)
    static constexpr int NT = NT0 < 64 ? 64 : (NT0 > 512 ? 512 : NT0);
    static constexpr int RS = NT / CG;
    static constexpr int RPT = DK / RS;
    static constexpr int NW = NT / 64;
    static_assert(NT % CG == 0 && DK % RS == 0 && RPT >= 1, "decode tiling");
};

// four consecutive input elements, loaded raw and converted at use
template <typename TI> struct Raw4;
template <> struct Raw4<float> {
    float4 x;
    __device__ __forceinline__ void load(const float* p) { x = *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ float4 get() const { return x; }
};
template <> struct Raw4<bf16> {
    uint2 x;                                                 // two bfloat16 per word
    __device__ __forceinline__ void load(const bf16* p) { x = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ float4 get() const {
        return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                           __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
    }
};

template <typename TI, typename TO, int DK, int DV>
__global__ __launch_bounds__(512, 4) void decode_multi_kernel(
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v,
    const float* __restrict__ g, const TI* __restrict__ beta, float scale,
    float* __restrict__ pool, const int32_t* __restrict__ slots, int num_slots,
    float* __restrict__ snapshots, TO* __restrict__ o, int T, int H, int reverse) {
    using Sh = MultiShape<DK, DV>;
    constexpr int CG = Sh::CG, RS = Sh::RS, RPT = Sh::RPT, NW = Sh::NW;
    __shared__ float4 red_vh[2][NW][CG];
    __shared__ float4 red_rq[2][NW][CG];
    __shared__ float red_kq[2][NW];

    // n * H + h, in the order of this call (alternating between calls, as the one-step decode)
    const int nh = reverse ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
    const int n = nh / H, h = nh % H;
    const int slot = slots ? slots[n] : n;
    if (slot < 0 || slot >= num_slots) return;   // uniform over the workgroup
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rs = tid / CG;
    const int wave = tid >> 6;
    const int lane = tid & 63;

    // inputs of the current token (c*) and of the next one (n*), raw
    float cg_[RPT], ng_[RPT];
    TI ck[RPT], cq[RPT], nk[RPT], nq[RPT], cb, nb;
    Raw4<TI> cv, nv;
    {
        const size_t tok = (size_t)n * T * H + h;
        const float* gb = g + tok * DK;                    // wave-uniform bases
        const TI *kb = k + tok * DK, *qb = q + tok * DK;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rs + RS * i;
            cg_[i] = gb[r];
            ck[i] = kb[r];
            cq[i] = qb[r];
        }
        cv.load(v + tok * DV + 4 * cg);
        cb = beta[tok];
    }
    float* S = pool + ((size_t)slot * H + h) * DK * DV;
    float4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const floatx4 x = reinterpret_cast<const floatx4*>(S + (size_t)(rs + RS * i) * DV)[cg];
        s[i] = make_float4(x[0], x[1], x[2], x[3]);
    }
#pragma unroll 1
    for (int t = 0; t < T; ++t) {
        const size_t tok = ((size_t)n * T + t) * H + h;     // token (n, t) of head h
        if (t + 1 < T) {
            const size_t tn = tok + H;                      // token (n, t + 1)
            const float* gb = g + tn * DK;
            const TI *kb = k + tn * DK, *qb = q + tn * DK;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int r = rs + RS * i;
                ng_[i] = gb[r];
                nk[i] = kb[r];
                nq[i] = qb[r];
            }
            nv.load(v + tn * DV + 4 * cg);
            nb = beta[tn];
        }
        asm volatile("" ::: "memory");                      // keep those loads issued here
        const int b = t & 1;
        float kr[RPT];
        float4 vh = make_float4(0.f, 0.f, 0.f, 0.f), rq = vh;
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float a = fast_exp2(cg_[i] * kLog2e);
            const float kk = to_f(ck[i]);
            const float qq = scale * to_f(cq[i]);
            kr[i] = kk;
            s[i].x *= a; s[i].y *= a; s[i].z *= a; s[i].w *= a;     // forget
            vh.x += kk * s[i].x; vh.y += kk * s[i].y;                // predict
            vh.z += kk * s[i].z; vh.w += kk * s[i].w;
            rq.x += qq * s[i].x; rq.y += qq * s[i].y;                // read of the decayed state
            rq.z += qq * s[i].z; rq.w += qq * s[i].w;
            kq += kk * qq;
        }
#pragma unroll
        for (int m = CG; m < 64; m <<= 1) {
            vh.x += __shfl_xor(vh.x, m); vh.y += __shfl_xor(vh.y, m);
            vh.z += __shfl_xor(vh.z, m); vh.w += __shfl_xor(vh.w, m);
            rq.x += __shfl_xor(rq.x, m); rq.y += __shfl_xor(rq.y, m);
            rq.z += __shfl_xor(rq.z, m); rq.w += __shfl_xor(rq.w, m);
            kq += __shfl_xor(kq, m);
        }
        if (lane < CG) {
            red_vh[b][wave][lane] = vh;
            red_rq[b][wave][lane] = rq;
            if (lane == 0) red_kq[b][wave] = kq;
        }
        // the buffer of this token's parity was last read two tokens ago, before the
        // previous token's barrier
        __syncthreads();
        vh = red_vh[b][0][cg];
        rq = red_rq[b][0][cg];
        kq = red_kq[b][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            const float4 x = red_vh[b][w][cg], y = red_rq[b][w][cg];
            vh.x += x.x; vh.y += x.y; vh.z += x.z; vh.w += x.w;
            rq.x += y.x; rq.y += y.y; rq.z += y.z; rq.w += y.w;
            kq += red_kq[b][w];
        }
        const float bt = to_f(cb);
        const float4 vv = cv.get();
        float4 e;                                                    // correct
        e.x = bt * (vv.x - vh.x); e.y = bt * (vv.y - vh.y);
        e.z = bt * (vv.z - vh.z); e.w = bt * (vv.w - vh.w);
        floatx4* snap = snapshots ? reinterpret_cast<floatx4*>(
                                        snapshots + (((size_t)n * T + t) * H + h) * DK * DV)
                                  : nullptr;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {                              // write
            const int r = rs + RS * i;
            s[i].x += kr[i] * e.x; s[i].y += kr[i] * e.y;
            s[i].z += kr[i] * e.z; s[i].w += kr[i] * e.w;
            if (snap)
                __builtin_nontemporal_store(floatx4{s[i].x, s[i].y, s[i].z, s[i].w},
                                            snap + (r * (DV / 4) + cg));
        }
        if (rs == 0)                                                 // read after the write
            store4(o + tok * DV + 4 * cg, rq.x + kq * e.x, rq.y + kq * e.y, rq.z + kq * e.z,
                   rq.w + kq * e.w);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            cg_[i] = ng_[i];
            ck[i] = nk[i];
            cq[i] = nq[i];
        }
        cv = nv;
        cb = nb;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        __builtin_nontemporal_store(floatx4{s[i].x, s[i].y, s[i].z, s[i].w},
                                    reinterpret_cast<floatx4*>(S + (size_t)(rs + RS * i) * DV) + cg);
}

// dst state dst_slots[i] <- src state src_slots[i]; a state is `words` float4 long
__global__ __launch_bounds__(256) void state_copy_kernel(
    float* __restrict__ dst, const int32_t* __restrict__ dst_slots, int dst_count,
    const float* __restrict__ src, const int32_t* __restrict__ src_slots, int src_count,
    long long words) {
    const int pair = blockIdx.y;
    const int ds = dst_slots[pair], ss = src_slots[pair];
    if (ds < 0 || ds >= dst_count || ss < 0 || ss >= src_count) return;
    const floatx4* s = reinterpret_cast<const floatx4*>(src) + (size_t)ss * words;
    floatx4* d = reinterpret_cast<floatx4*>(dst) + (size_t)ds * words;
    for (long long w = (long long)blockIdx.x * 256 + threadIdx.x; w < words;
         w += (long long)gridDim.x * 256)
        d[w] = s[w];
}

template <typename TI, typename TO, int DK, int DV>
static hipError_t launch_multi_t(const void* q, const void* k, const void* v, const float* g,
                                 const void* beta, float scale, float* pool,
                                 const int32_t* slots, int num_slots, float* snapshots, void* o,
                                 int N, int T, int H, hipStream_t s) {
    hipLaunchKernelGGL((decode_multi_kernel<TI, TO, DK, DV>),
                       dim3((unsigned)((long long)N * H)), dim3(MultiShape<DK, DV>::NT), 0, s,
                       (const TI*)q, (const TI*)k, (const TI*)v, g, (const TI*)beta, scale,
                       pool, slots, num_slots, snapshots, (TO*)o, T, H, next_decode_order());
    return hipGetLastError();
}

template <typename TI, typename TO>
static hipError_t dispatch_multi(int Dk, int Dv, const void* q, const void* k, const void* v,
                                 const float* g, const void* beta, float scale, float* pool,
                                 const int32_t* slots, int num_slots, float* snapshots, void* o,
                                 int N, int T, int H, hipStream_t s) {
#define KDA_MD(DKV, DVV)                                                                    \
    if (Dk == DKV && Dv == DVV)                                                             \
        return launch_multi_t<TI, TO, DKV, DVV>(q, k, v, g, beta, scale, pool, slots,       \
                                                num_slots, snapshots, o, N, T, H, s);
    KDA_MD(16, 16) KDA_MD(16, 32) KDA_MD(16, 64) KDA_MD(16, 128)
    KDA_MD(32, 16) KDA_MD(32, 32) KDA_MD(32, 64) KDA_MD(32, 128)
    KDA_MD(64, 16) KDA_MD(64, 32) KDA_MD(64, 64) KDA_MD(64, 128)
    KDA_MD(128, 16) KDA_MD(128, 32) KDA_MD(128, 64) KDA_MD(128, 128)
#undef KDA_MD
    return hipErrorInvalidValue;
}

hipError_t launch_decode_multi(bool bf16_in, bool bf16_out, int Dk, int Dv, const void* q,
                               const void* k, const void* v, const float* g, const void* beta,
                               float scale, float* pool, const int32_t* slots, int num_slots,
                               float* snapshots, void* o, int N, int T, int H, hipStream_t s) {
#define KDA_MD_ARGS Dk, Dv, q, k, v, g, beta, scale, pool, slots, num_slots, snapshots, o, N, T, H, s
    if (bf16_in) {
        if (bf16_out) return dispatch_multi<bf16, bf16>(KDA_MD_ARGS);
        return dispatch_multi<bf16, float>(KDA_MD_ARGS);
    }
    if (bf16_out) return dispatch_multi<float, bf16>(KDA_MD_ARGS);
    return dispatch_multi<float, float>(KDA_MD_ARGS);
#undef KDA_MD_ARGS
}

hipError_t launch_state_copy(float* dst, const int32_t* dst_slots, int dst_count,
                             const float* src, const int32_t* src_slots, int src_count,
                             int pairs, long long state_floats, hipStream_t s) {
    const long long words = state_floats / 4;
    long long bx = (words + 255) / 256;
    if (bx > 64) bx = 64;                        // each workgroup then loops over its chunks
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)bx, (unsigned)pairs), dim3(256), 0, s,
                       dst, dst_slots, dst_count, src, src_slots, src_count, words);
    return hipGetLastError();
}

}  // namespace kda
