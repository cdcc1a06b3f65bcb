// Input preparation for the recurrence, one pass over the raw projections:
//   q^ = scale q / |q|,  k^ = k / |k|   (L2 norm over the Dk channels of a token-head row;
//                                         "Notes on Linear Attention", zhilingong.com,
//                                         sections 4 and 5.3: normalised queries and keys)
//   beta = sigmoid(b)                    (the write strength as a sigmoid of a projection,
//                                         "From Fast Weight Programmers to KDA")
//   g = log sigmoid(a)                   (a log-decay in (-inf, 0), one per key channel;
//                                         the pages fix only g = log(alpha) with alpha in
//                                         (0, 1), and a sigmoid of a logit is the plainest
//                                         map onto that range)
// in the layouts the prefill and decode kernels read. The pass is memory-bound: Dk / 8
// lanes own one token-head row, each with 8 consecutive channels (one 16-byte bf16 load or
// two fp32 loads per tensor), and the squared norms are summed with lane shuffles inside
// the row's lane group. A lane reads its elements before it writes them, so q, k and b may
// be overwritten in place (and a by g when both are float32). A row of zeros stays zero.
#include "kda_common.h"

namespace kda {

template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
    static __device__ __forceinline__ void load(const bf16* p, float* o) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[2 * e] = __uint_as_float(w[e] << 16);
            o[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(bf16* p, const float* x) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];            // round to nearest even
        *reinterpret_cast<bf16x8*>(p) = v;
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float* p, float* o) {
        const floatx4 a = reinterpret_cast<const floatx4*>(p)[0];
        const floatx4 b = reinterpret_cast<const floatx4*>(p)[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) { o[e] = a[e]; o[4 + e] = b[e]; }
    }
    static __device__ __forceinline__ void store(float* p, const float* x) {
        reinterpret_cast<floatx4*>(p)[0] = floatx4{x[0], x[1], x[2], x[3]};
        reinterpret_cast<floatx4*>(p)[1] = floatx4{x[4], x[5], x[6], x[7]};
    }
};

template <typename TI, int DK>
__global__ __launch_bounds__(256) void prepare_inputs_kernel(
    const TI* q, const TI* k, const TI* a, const TI* b, float scale, TI* qo, TI* ko,
    float* go, TI* bo, long long rows) {
    constexpr int LPR = DK / 8;                          // lanes per token-head row
    const long long gtid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long row = gtid / LPR;
    const int part = (int)(gtid % LPR);
    const bool valid = row < rows;
    const long long off = valid ? row * DK + 8 * part : 0;
    float xq[8], xk[8], xa[8];
    float sq = 0.f, sk = 0.f;
    if (valid) {
        Vec8<TI>::load(q + off, xq);
        Vec8<TI>::load(k + off, xk);
        Vec8<TI>::load(a + off, xa);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sq += xq[e] * xq[e];
            sk += xk[e] * xk[e];
        }
    }
    // sum over the row's lane group (consecutive lanes; every lane of the wave takes part)
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
        sq += __shfl_xor(sq, m);
        sk += __shfl_xor(sk, m);
    }
    float bl = 0.f;
    if (valid && part == 0) bl = to_f(b[row]);
    if (!valid) return;
    // a zero row stays zero
    const float rq = sq > 0.f ? scale / sqrtf(sq) : 0.f, rk = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;
    float g8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        xq[e] *= rq;
        xk[e] *= rk;
        g8[e] = log_sigmoid(xa[e]);
    }
    Vec8<TI>::store(qo + off, xq);
    Vec8<TI>::store(ko + off, xk);
    Vec8<float>::store(go + off, g8);
    if (part == 0) bo[row] = (TI)sigmoid(bl);
}

template <typename TI>
static hipError_t launch_prepare_t(int Dk, const void* q, const void* k, const void* a,
                                   const void* b, float scale, void* qo, void* ko, float* go,
                                   void* bo, long long rows, hipStream_t s) {
    const long long threads = rows * (Dk / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
#define KDA_PI(DKV)                                                                         \
    if (Dk == DKV) {                                                                        \
        hipLaunchKernelGGL((prepare_inputs_kernel<TI, DKV>), grid, dim3(256), 0, s,         \
                           (const TI*)q, (const TI*)k, (const TI*)a, (const TI*)b, scale,   \
                           (TI*)qo, (TI*)ko, go, (TI*)bo, rows);                            \
        return hipGetLastError();                                                           \
    }
    KDA_PI(16) KDA_PI(32) KDA_PI(64) KDA_PI(128)
#undef KDA_PI
    return hipErrorInvalidValue;
}

hipError_t launch_prepare_inputs(bool bf16_io, int Dk, const void* q, const void* k,
                                 const void* a, const void* b, float scale, void* qo, void* ko,
                                 float* go, void* bo, long long rows, hipStream_t s) {
    if (bf16_io) return launch_prepare_t<bf16>(Dk, q, k, a, b, scale, qo, ko, go, bo, rows, s);
    return launch_prepare_t<float>(Dk, q, k, a, b, scale, qo, ko, go, bo, rows, s);
}

}  // namespace kda
