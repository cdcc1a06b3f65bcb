// Serving-state operations for decode: the recurrent state of a request is
// request-scoped serving state, kept in a pool like a KV-cache slot, and it
// must be carried, copied on a fork and restored on a speculative rollback
// ("Module 03 - KDA I: The Delta-Rule Recurrence", jared-hpc.com, section 5).
//
// decode_multi_kernel: T consecutive tokens per request against the state in
// slot slots[n] of a pool. The state is read once, kept in registers across
// the T steps (each the recurrent step of "Kimi Delta Attention (KDA)", "Two
// schedules for the same recurrence"), and written once; optionally the state
// after every token is written to a snapshot array, so that a caller verifying
// T drafted tokens can restore the state after any accepted prefix.
//
// Column-sliced work split: in one step, value column c of S is forgotten,
// predicted (v^_c = sum_r k_r S~_rc), corrected and written using only column
// c and the per-row alpha, k and q, so the columns are independent for the
// whole token loop. Each wavefront owns CW value columns over all DK rows
// (lane (cq, rg): four columns, DK / RG consecutive rows) and runs every token
// on them without a barrier: the column sums reduce across the row groups of
// the wavefront with a DPP rotate and the permlane16/permlane32 swaps, which
// give every lane of a column the same bits. The token inputs, shared by the
// wavefronts of a state, are staged in LDS in groups of TG tokens, already as
// alpha = exp(g), k, scale q, v and beta in fp32.
//
// state_copy_kernel: dst[dst_slots[i]] = src[src_slots[i]] for whole states,
// 16-byte vector copies, one workgroup per (pair, 1024 float4 chunk).
#include "kda_common.h"

namespace kda {

int next_decode_order();                         // alternating state order (kda_decode.hip)

template <typename TI, int DK, int DV>
struct MultiShape {
    static constexpr int CW = DV < 32 ? DV : 32;            // value columns per wavefront
    static constexpr int CQ = CW / 4;                       // lanes per row (a float4 each)
    static constexpr int RG = 64 / CQ;                      // row groups per wavefront
    static constexpr int RPL = DK / RG;                     // consecutive rows per lane
    static constexpr int RB = RPL < 4 ? RPL : 4;            // rows per LDS vector read
    static constexpr int NW = DV / CW;                      // wavefronts per state
    static constexpr int NT = 64 * NW;
    static constexpr int TG = 8;                            // tokens per staged group
    // staged token (bytes): g fp32 [DK], k, q [DK], v [DV] in the input type, as 16-byte pieces
    static constexpr int SZ = (int)sizeof(TI);
    static constexpr int OK = 4 * DK, OQ = OK + DK * SZ, OV = OQ + DK * SZ;
    static constexpr int TOKB = OV + DV * SZ;
    static constexpr int PIECES = TOKB / 16;
    static_assert(RPL >= 1 && RPL * RG == DK && RPL % RB == 0 && TOKB % 16 == 0, "decode tiling");
};

// sum over the row groups of a wavefront (lane bits log2(CQ) .. 5); every lane of a column
// gets the same bits (each stage adds a pair in an order both partners share)
template <int CQ>
__device__ __forceinline__ float rowgroup_sum(float x) {
    if constexpr (CQ == 4) x += __shfl_xor(x, 4);
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// N consecutive staged values (fp32 or bf16) from LDS, as floats
template <typename T, int N>
__device__ __forceinline__ void lds_vals(float (&x)[N], const uint8_t* p) {
    if constexpr (sizeof(T) == 4) {
        if constexpr (N == 4) {
            const float4 t = *reinterpret_cast<const float4*>(p);
            x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
        } else if constexpr (N == 2) {
            const float2 t = *reinterpret_cast<const float2*>(p);
            x[0] = t.x; x[1] = t.y;
        } else {
            x[0] = *reinterpret_cast<const float*>(p);
        }
    } else {
        if constexpr (N == 4) {
            const u32x2 t = *reinterpret_cast<const u32x2*>(p);
            x[0] = __uint_as_float(t[0] << 16); x[1] = __uint_as_float(t[0] & 0xffff0000u);
            x[2] = __uint_as_float(t[1] << 16); x[3] = __uint_as_float(t[1] & 0xffff0000u);
        } else if constexpr (N == 2) {
            const unsigned t = *reinterpret_cast<const unsigned*>(p);
            x[0] = __uint_as_float(t << 16); x[1] = __uint_as_float(t & 0xffff0000u);
        } else {
            x[0] = __uint_as_float((unsigned)*reinterpret_cast<const unsigned short*>(p) << 16);
        }
    }
}

template <typename TI, typename TO, int DK, int DV>
__global__ __launch_bounds__(256, 4) void decode_multi_kernel(
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v,
    const float* __restrict__ g, const TI* __restrict__ beta, float scale,
    float* __restrict__ pool, const int32_t* __restrict__ slots, int num_slots,
    float* __restrict__ snapshots, TO* __restrict__ o, int T, int H, int reverse) {
    using Sh = MultiShape<TI, DK, DV>;
    constexpr int CW = Sh::CW, CQ = Sh::CQ, RPL = Sh::RPL, RB = Sh::RB, NT = Sh::NT;
    constexpr int NW = Sh::NW, TG = Sh::TG, SZ = Sh::SZ, TOKB = Sh::TOKB, PIECES = Sh::PIECES;
    constexpr int OK = Sh::OK, OQ = Sh::OQ, OV = Sh::OV;
    // the staged pieces of a group, rounded up to whole 1 KB wavefront loads
    constexpr int LOADS = (TG * PIECES + 64 * NW - 1) / (64 * NW);
    __shared__ __attribute__((aligned(16))) uint8_t sIn[LOADS * NW * 1024];
    __shared__ float sBeta[TG];

    // n * H + h, in the order of this call (alternating between calls, as the one-step decode)
    const int nh = reverse ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
    const int n = nh / H, h = nh % H;
    const int slot = slots ? slots[n] : n;
    if (slot < 0 || slot >= num_slots) return;   // uniform over the workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cq = lane % CQ, rg = lane / CQ;
    const int r0 = rg * RPL;                              // first row of this lane
    const int c0 = CW * wave + 4 * cq;                    // first column of this lane

    // the inputs of tokens t0 .. t0 + tg - 1 to LDS, piece by piece straight from global
    // memory (no registers); beta through a register
    auto fill = [&](int t0, int tg) {
        // the lane index through an opaque move, so that the per-lane piece addresses are
        // formed here, on use, rather than hoisted out of the token loop into registers
        int ln;
        asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
#pragma unroll
        for (int f = 0; f < LOADS; ++f) {
            const int blk = f * NW + wave;                // this wavefront's 1 KB of LDS
            const int c = blk * 64 + ln;                  // piece
            if (c < tg * PIECES) {
                const int tk = c / PIECES, b = (c % PIECES) * 16;
                const size_t tok = ((size_t)n * T + t0 + tk) * H + h;
                const void* src =
                    b < OK   ? (const void*)(g + tok * DK + b / 4)
                    : b < OQ ? (const void*)(k + tok * DK + (b - OK) / SZ)
                    : b < OV ? (const void*)(q + tok * DK + (b - OQ) / SZ)
                             : (const void*)(v + tok * DV + (b - OV) / SZ);
                lds_load16(src, sIn + blk * 1024);
            }
        }
        if (tid < tg) sBeta[tid] = to_f(beta[((size_t)n * T + t0 + tid) * H + h]);
    };

    float* S = pool + ((size_t)slot * H + h) * DK * DV;
    fill(0, T < TG ? T : TG);
    floatx4 s[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
        s[i] = *reinterpret_cast<const floatx4*>(S + (size_t)(r0 + i) * DV + c0);
    wait_all_memory();
    __syncthreads();

#pragma unroll 1
    for (int t0 = 0; t0 < T; t0 += TG) {
        const int tg = T - t0 < TG ? T - t0 : TG;
        if (t0 > 0) {
            __syncthreads();                              // every wavefront done with the group
            fill(t0, tg);
            wait_all_memory();
            __syncthreads();
        }
#pragma unroll 1
        for (int u = 0; u < tg; ++u) {
            const uint8_t* in = sIn + u * TOKB;
            const int t = t0 + u;
            floatx4 vh = {0.f, 0.f, 0.f, 0.f}, rq = vh;
            float kq = 0.f;
#pragma unroll
            for (int jb = 0; jb < RPL; jb += RB) {
                float a[RB], kk[RB], qq[RB];
                lds_vals<float>(a, in + 4 * (r0 + jb));
                lds_vals<TI>(kk, in + OK + SZ * (r0 + jb));
                lds_vals<TI>(qq, in + OQ + SZ * (r0 + jb));
#pragma unroll
                for (int e = 0; e < RB; ++e) {
                    floatx4& x = s[jb + e];
                    const float qs = scale * qq[e];
                    x *= fast_exp2(a[e] * kLog2e);                    // forget
                    vh += kk[e] * x;                                  // predict
                    rq += qs * x;                                     // read of S~
                    kq += kk[e] * qs;
                }
                __builtin_amdgcn_sched_barrier(0);            // keep the row blocks in turn
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                vh[c] = rowgroup_sum<CQ>(vh[c]);
                rq[c] = rowgroup_sum<CQ>(rq[c]);
            }
            kq = rowgroup_sum<CQ>(kq);
            float vv[4];
            lds_vals<TI>(vv, in + OV + SZ * c0);
            const float bt = sBeta[u];
            const floatx4 e = bt * (floatx4{vv[0], vv[1], vv[2], vv[3]} - vh);   // correct
            const size_t tok = ((size_t)n * T + t) * H + h;
            float* snap = snapshots ? snapshots + tok * DK * DV : nullptr;
#pragma unroll
            for (int jb = 0; jb < RPL; jb += RB) {                    // write
                float kk[RB];
                lds_vals<TI>(kk, in + OK + SZ * (r0 + jb));
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    s[jb + i] += kk[i] * e;
                    if (snap)
                        __builtin_nontemporal_store(
                            s[jb + i],
                            reinterpret_cast<floatx4*>(snap + (size_t)(r0 + jb + i) * DV + c0));
                }
            }
            if (rg == 0)                                              // read after the write
                store4(o + tok * DV + c0, rq[0] + kq * e[0], rq[1] + kq * e[1],
                       rq[2] + kq * e[2], rq[3] + kq * e[3]);
        }
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i)
        __builtin_nontemporal_store(s[i], reinterpret_cast<floatx4*>(S + (size_t)(r0 + i) * DV + c0));
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
                       dim3((unsigned)((long long)N * H)), dim3(MultiShape<TI, DK, DV>::NT), 0, s,
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
