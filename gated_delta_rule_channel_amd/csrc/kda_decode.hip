// Fused KDA decode step: one pass over each (request, head) fp32 state.
//
// One token per request against its persistent state S (Dk x Dv, row = key
// channel), the recurrent schedule of "Kimi Delta Attention (KDA)"
// (brain.bigb.es, "Two schedules for the same recurrence") applied once:
//   S~ = Diag(exp g) S,  v^ = S~^T k,  r = S~^T (s q),  e = beta (v - v^),
//   S  = S~ + k e^T (stored in place),  o = r + (k . s q) e.
// The last identity is the read o = S^T (s q) of the updated state expanded
// through the rank-one write, so the state is read once and written once.
// The cost is the state bytes ("Notes on Linear Attention", zhilingong.com,
// section 3.1: decoding is bound by reading and writing the state).
//
// Work split: one workgroup per (request, head). Thread t owns four
// consecutive value columns (one 16-byte vector per state row) of rows
// rs, rs + RS, ...; a wavefront therefore streams whole contiguous rows. The
// column sums of v^ and r are reduced across rows with lane shuffles inside a
// wavefront and through LDS across wavefronts. State stores are nontemporal
// (each state is written once per step); plain loads measured faster than
// nontemporal ones.
//
// SG selects the scalar gate of Gated DeltaNet ("Notes on Linear Attention",
// section 6): g holds one log-decay per (request, head) and every row of S
// decays by the same factor. EW selects the erase and write gates of Gated
// DeltaNet-2 ("From Fast Weight Programmers to KDA", section "Gated
// DeltaNet-2"): the prediction reads through b * k (b per key channel) and
// the error is w * v - v^ (w per value channel); the write stays at k.
#include <atomic>

#include "kda_common.h"

namespace kda {

// Successive decode steps on a device walk the (request, head) states in alternating order:
// a step's last ~256 MB of state writes are still in the Infinity Cache when the next step
// starts, and the next step then starts on exactly those states (its first reads hit in the
// cache and the dirty lines are rewritten before they reach HBM). Each state is updated on
// its own, so the order never changes a result. Shared by the single- and multi-token steps.
int next_decode_order() {
    static std::atomic<unsigned> calls[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    return (int)(calls[dev].fetch_add(1, std::memory_order_relaxed) & 1u);
}

template <int DK, int DV>
struct DecodeShape {
    static constexpr int CG = DV / 4;                       // 16-byte column groups per row
    // one float4 per thread x 4 rows: more threads per state with fewer rows each measured
    // faster (256 threads x 16 rows: 6 % slower at 128 x 128)
    static constexpr int NT0 = DK * DV / 16;
    static constexpr int NT = NT0 < 64 ? 64 : (NT0 > 1024 ? 1024 : NT0);
    static constexpr int RS = NT / CG;                      // row subgroups
    static constexpr int RPT = DK / RS;                     // rows per thread
    static constexpr int NW = NT / 64;                      // wavefronts
    static_assert(NT % CG == 0 && DK % RS == 0 && RPT >= 1, "decode tiling");
};

template <typename TI, typename TO, int DK, int DV, bool SG, bool EW>
__global__ __launch_bounds__(1024) void decode_kernel(
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v,
    const float* __restrict__ g, const TI* __restrict__ beta, const TI* __restrict__ eb,
    const TI* __restrict__ ew, float scale, float* __restrict__ state, TO* __restrict__ o,
    int reverse) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int CG = Sh::CG, RS = Sh::RS, RPT = Sh::RPT, NW = Sh::NW;
    __shared__ float4 red_vh[NW][CG];
    __shared__ float4 red_rq[NW][CG];
    __shared__ float red_kq[NW];

    // n * H + h, in the order of this step (see next_decode_order)
    const int head = reverse ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rs = tid / CG;
    const int wave = tid >> 6;
    const int lane = tid & 63;

    float* S = state + (size_t)head * DK * DV;
    const TI* qh = q + (size_t)head * DK;
    const TI* kh = k + (size_t)head * DK;
    const float* gh = g + (size_t)head * (SG ? 1 : DK);

    float4 s[RPT];
    float kr[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rs + RS * i;
        const floatx4 t = reinterpret_cast<const floatx4*>(S + (size_t)r * DV)[cg];
        s[i] = make_float4(t[0], t[1], t[2], t[3]);
    }
    float4 vh = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 rq = make_float4(0.f, 0.f, 0.f, 0.f);
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rs + RS * i;
        const float a = fast_exp2(gh[SG ? 0 : r] * kLog2e);
        const float kk = to_f(kh[r]);
        const float qq = scale * to_f(qh[r]);
        kr[i] = kk;
        // the prediction's key: k, or b * k with an erase gate
        const float kp = EW ? kk * to_f(eb[(size_t)head * DK + r]) : kk;
        s[i].x *= a; s[i].y *= a; s[i].z *= a; s[i].w *= a;       // (1) forget
        vh.x += kp * s[i].x; vh.y += kp * s[i].y;                  // (2) predict
        vh.z += kp * s[i].z; vh.w += kp * s[i].w;
        rq.x += qq * s[i].x; rq.y += qq * s[i].y;                  // read of S~
        rq.z += qq * s[i].z; rq.w += qq * s[i].w;
        kq += kk * qq;
    }
    // reduce over the row subgroups held by this wavefront (lane offsets CG, 2CG, ...)
#pragma unroll
    for (int m = CG; m < 64; m <<= 1) {
        vh.x += __shfl_xor(vh.x, m); vh.y += __shfl_xor(vh.y, m);
        vh.z += __shfl_xor(vh.z, m); vh.w += __shfl_xor(vh.w, m);
        rq.x += __shfl_xor(rq.x, m); rq.y += __shfl_xor(rq.y, m);
        rq.z += __shfl_xor(rq.z, m); rq.w += __shfl_xor(rq.w, m);
        kq += __shfl_xor(kq, m);
    }
    if (lane < CG) {
        red_vh[wave][lane] = vh;
        red_rq[wave][lane] = rq;
        if (lane == 0) red_kq[wave] = kq;
    }
    __syncthreads();
    vh = red_vh[0][cg];
    rq = red_rq[0][cg];
    kq = red_kq[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        const float4 a = red_vh[w][cg], b = red_rq[w][cg];
        vh.x += a.x; vh.y += a.y; vh.z += a.z; vh.w += a.w;
        rq.x += b.x; rq.y += b.y; rq.z += b.z; rq.w += b.w;
        kq += red_kq[w];
    }
    const float4 vv = load4f(v + (size_t)head * DV + 4 * cg);
    float4 e;                                                      // (3) correct
    if constexpr (EW) {
        const float4 ww = load4f(ew + (size_t)head * DV + 4 * cg);
        e.x = ww.x * vv.x - vh.x; e.y = ww.y * vv.y - vh.y;
        e.z = ww.z * vv.z - vh.z; e.w = ww.w * vv.w - vh.w;
    } else {
        const float bt = to_f(beta[head]);
        e.x = bt * (vv.x - vh.x); e.y = bt * (vv.y - vh.y);
        e.z = bt * (vv.z - vh.z); e.w = bt * (vv.w - vh.w);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {                                // (4) write, in place
        const int r = rs + RS * i;
        float4 x = s[i];
        x.x += kr[i] * e.x; x.y += kr[i] * e.y; x.z += kr[i] * e.z; x.w += kr[i] * e.w;
        __builtin_nontemporal_store(floatx4{x.x, x.y, x.z, x.w},
                                    reinterpret_cast<floatx4*>(S + (size_t)r * DV) + cg);
    }
    if (rs == 0) {                                                 // (5) read
        store4(o + (size_t)head * DV + 4 * cg, rq.x + kq * e.x, rq.y + kq * e.y,
               rq.z + kq * e.z, rq.w + kq * e.w);
    }
}

template <typename TI, typename TO, int DK, int DV>
static hipError_t launch_decode_t(bool sg, const void* q, const void* k, const void* v,
                                  const float* g, const void* beta, const void* eb,
                                  const void* ew, float scale, float* state, void* o, int N,
                                  int H, hipStream_t stream) {
    const dim3 grid((unsigned)((long long)N * H));
    const dim3 block(DecodeShape<DK, DV>::NT);
    const TI *tq = (const TI*)q, *tk = (const TI*)k, *tv = (const TI*)v, *tb = (const TI*)beta;
    const int rev = next_decode_order();
    if (eb)
        hipLaunchKernelGGL((decode_kernel<TI, TO, DK, DV, false, true>), grid, block, 0, stream,
                           tq, tk, tv, g, tb, (const TI*)eb, (const TI*)ew, scale, state, (TO*)o,
                           rev);
    else if (sg)
        hipLaunchKernelGGL((decode_kernel<TI, TO, DK, DV, true, false>), grid, block, 0, stream,
                           tq, tk, tv, g, tb, nullptr, nullptr, scale, state, (TO*)o, rev);
    else
        hipLaunchKernelGGL((decode_kernel<TI, TO, DK, DV, false, false>), grid, block, 0, stream,
                           tq, tk, tv, g, tb, nullptr, nullptr, scale, state, (TO*)o, rev);
    return hipGetLastError();
}

template <typename TI, typename TO>
static hipError_t dispatch_decode(bool sg, int Dk, int Dv, const void* q, const void* k,
                                  const void* v, const float* g, const void* beta,
                                  const void* eb, const void* ew, float scale, float* state,
                                  void* o, int N, int H, hipStream_t s) {
#define KDA_DEC(DKV, DVV)                                                                   \
    if (Dk == DKV && Dv == DVV)                                                             \
        return launch_decode_t<TI, TO, DKV, DVV>(sg, q, k, v, g, beta, eb, ew, scale, state, \
                                                 o, N, H, s);
    KDA_DEC(16, 16) KDA_DEC(16, 32) KDA_DEC(16, 64) KDA_DEC(16, 128)
    KDA_DEC(32, 16) KDA_DEC(32, 32) KDA_DEC(32, 64) KDA_DEC(32, 128)
    KDA_DEC(64, 16) KDA_DEC(64, 32) KDA_DEC(64, 64) KDA_DEC(64, 128)
    KDA_DEC(128, 16) KDA_DEC(128, 32) KDA_DEC(128, 64) KDA_DEC(128, 128)
#undef KDA_DEC
    return hipErrorInvalidValue;
}

// sg: scalar gate; eb, ew: erase and write gates (non-null together) replacing beta
hipError_t launch_decode(bool sg, bool bf16_in, bool bf16_out, int Dk, int Dv,
                         const void* q, const void* k, const void* v, const float* g,
                         const void* beta, const void* eb, const void* ew, float scale,
                         float* state, void* o, int N, int H, hipStream_t s) {
#define KDA_DEC_ARGS sg, Dk, Dv, q, k, v, g, beta, eb, ew, scale, state, o, N, H, s
    if (bf16_in) {
        if (bf16_out) return dispatch_decode<bf16, bf16>(KDA_DEC_ARGS);
        return dispatch_decode<bf16, float>(KDA_DEC_ARGS);
    }
    if (bf16_out) return dispatch_decode<float, bf16>(KDA_DEC_ARGS);
    return dispatch_decode<float, float>(KDA_DEC_ARGS);
#undef KDA_DEC_ARGS
}

}  // namespace kda
