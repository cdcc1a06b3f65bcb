// Workspace layout of the chunked prefill and the device helpers shared by its kernels
// (the two-pass prep and state kernels, and the fused kernel).
#pragma once

#include "kda_common.h"

namespace kda {

// ------------------------------------------------------------------------------------------
// workspace layout
// ------------------------------------------------------------------------------------------
// One block per (chunk slot, head). Every operand of the state pass is stored in the
// register layout of the MFMA fragment that consumes it, so that one load instruction of a
// wave reads 1 KB of consecutive bytes (16 B per lane). Fragments (8 elements per lane) are
// stored in pairs (a, b). PolSplit: A_qk pairs (3 KB) hold the hi values of a, of b, then the
// extension bytes of both (x rounded to 24 bits = bfloat16 hi + 1 byte, 16 significant
// bits); W, Qd and Kd^T pairs (2.5 KB) hold x rounded to 20 bits (bfloat16 hi + a 4-bit
// nibble). PolF32: 4 KB, two fp32 tiles. U tiles hold 4 values per lane (U is an addend of
// E, not an MFMA operand): PolSplit 768 B in the 24-bit form, PolF32 1 KB of fp32. With
// lane l = m + 16 grp:
//  W, Qd  20-bit pairs [token tile tw][channel steps (2p, 2p+1)]: row 16 tw + m, channels
//         32 kap + 8 grp + e (zero past Dk);
//  Kd^T   20-bit pairs [channel tile ct][token halves (0, 1)]: channel 16 ct + m, tokens
//         32 ks + 8 grp + e;
//  U      tiles [value tile vt][token tile tw]: tokens 16 tw + 4 grp + r, value 16 vt + m;
//  A_qk   pairs [token tile tw][column halves (0, 1)]: row 16 tw + m, columns 32 s + 8 grp + e
//         (token tiles 0 and 1: the second half, all zero, is neither written nor read);
//  exp(G_end) float [Dk].
__host__ __device__ constexpr size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ __device__ constexpr size_t ws_block_bytes(int DK, int DV, size_t PT, size_t UT,
                                                    size_t PN) {
    return round_up((size_t)2 * 4 * (((DK >= 32 ? DK / 32 : 1) + 1) / 2) * PN +
                        (size_t)(DK / 16) * PN + (size_t)(DV / 16) * 4 * UT + 4 * PT +
                        (size_t)DK * 4,
                    256);
}

template <int PTB, int UTB, int PNB, int DK, int DV>
struct WsLayout {
    static constexpr int KS = DK >= 32 ? DK / 32 : 1;   // 32-channel steps (padded)
    static constexpr int NP = (KS + 1) / 2;              // pairs of channel steps
    static constexpr int NCT = DK / 16;                  // 16-channel tiles
    static constexpr int NVT = DV / 16;                  // 16-value tiles
    static constexpr size_t PT = PTB;                    // pair tile
    static constexpr size_t QT = UTB;                    // U tile
    static constexpr size_t PN = PNB;                    // narrower pair tile (W, Qd, Kd^T)
    static constexpr size_t W = 0;
    static constexpr size_t QD = W + 4 * NP * PN;
    static constexpr size_t KDT = QD + 4 * NP * PN;
    static constexpr size_t U = KDT + NCT * PN;
    static constexpr size_t AQ = U + NVT * 4 * QT;
    static constexpr size_t GEND = AQ + 4 * PT;
    static constexpr size_t BYTES = round_up(GEND + DK * sizeof(float), 256);
    static_assert(BYTES == ws_block_bytes(DK, DV, PT, QT, PN), "workspace block size");
};
template <typename Pol, int DK, int DV>
using WsLayoutOf = WsLayout<Pol::kPairBytes, Pol::kUTileBytes, Pol::kPairNBytes, DK, DV>;


__host__ __device__ constexpr int tri_tile(int I, int J) { return I * (I + 1) / 2 + J; }

// input variants of the bf16, d = 128 prep kernel: prepared inputs (KDA), raw projections
// (normalised and gated in the kernel), and Gated DeltaNet-2's erase and write gates
enum PrepMode : int { kPrepPlain = 0, kPrepRaw = 1, kPrepGates = 2 };

// Keeps the compiler from sinking prefetch loads to their first use: loads issued before
// this point stay before it, so they are in flight while the following code runs.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// 32 input elements of a lane (4 token blocks x 8 channels), readable with a wave-uniform
// block index.
template <typename T> struct In32;
template <> struct In32<bf16> {
    u32x16 w;                                            // two bfloat16 per word
    __device__ __forceinline__ void load(int I, const bf16* p) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(p);
        w[4 * I] = x[0]; w[4 * I + 1] = x[1]; w[4 * I + 2] = x[2]; w[4 * I + 3] = x[3];
    }
    __device__ __forceinline__ void zero(int I) {
        w[4 * I] = 0u; w[4 * I + 1] = 0u; w[4 * I + 2] = 0u; w[4 * I + 3] = 0u;
    }
    __device__ __forceinline__ void set(int I, const u32x4& x) {
        w[4 * I] = x[0]; w[4 * I + 1] = x[1]; w[4 * I + 2] = x[2]; w[4 * I + 3] = x[3];
    }
    __device__ __forceinline__ void get8(int I, float* o) const {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const unsigned x = w[4 * I + p];
            o[2 * p] = __uint_as_float(x << 16);
            o[2 * p + 1] = __uint_as_float(x & 0xffff0000u);
        }
    }
    // get8 through an empty asm on each word: the result counts as computed where it is read
    __device__ __forceinline__ void get8p(int I, float* o) const {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            unsigned x = w[4 * I + p];
            asm volatile("" : "+v"(x));
            o[2 * p] = __uint_as_float(x << 16);
            o[2 * p + 1] = __uint_as_float(x & 0xffff0000u);
        }
    }
    // the 8 elements of block I as an exact operand fragment
    __device__ __forceinline__ void frag(int I, PolSplit::Frag& f) const {
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        u32x4 x;
        x[0] = w[4 * I]; x[1] = w[4 * I + 1]; x[2] = w[4 * I + 2]; x[3] = w[4 * I + 3];
        f.hi = __builtin_bit_cast(bf16x8, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) f.lo[e] = (bf16)0.f;
    }
};
template <> struct In32<float> {
    floatx32 v;
    __device__ __forceinline__ void load(int I, const float* p) {
        const float4 a = reinterpret_cast<const float4*>(p)[0];
        const float4 b = reinterpret_cast<const float4*>(p)[1];
        v[8 * I] = a.x; v[8 * I + 1] = a.y; v[8 * I + 2] = a.z; v[8 * I + 3] = a.w;
        v[8 * I + 4] = b.x; v[8 * I + 5] = b.y; v[8 * I + 6] = b.z; v[8 * I + 7] = b.w;
    }
    __device__ __forceinline__ void zero(int I) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * I + e] = 0.f;
    }
    __device__ __forceinline__ void get8(int I, float* o) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = v[8 * I + e];
    }
    __device__ __forceinline__ void get8p(int I, float* o) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = v[8 * I + e];
            asm volatile("" : "+v"(x));
            o[e] = x;
        }
    }
    __device__ __forceinline__ void frag(int I, PolF32::Frag& f) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[e] = v[8 * I + e];
    }
};

// Input staging: bf16 input stages g, k, q (64 KB per task) in LDS; fp32 input (96 KB)
// loads them from global memory at the start of each task.
template <typename TI> struct PrepStage { static constexpr int kBytes = 0; };
template <> struct PrepStage<bf16> {
    static constexpr int kBytes = 65536;
    // byte offsets of wave w's 1 KB parts: q (block I) over T and the start of A_kk, g
    // (block I, rows 8 half .. 8 half + 7) and k (block I) over the rest of A_kk and A_qk;
    // all of it is free once T' is formed
    __device__ static constexpr int q_off(int w, int I) { return (w * 4 + I) * 1024; }
    __device__ static constexpr int g_off(int w, int I, int half) { return 16384 + ((w * 4 + I) * 2 + half) * 1024; }
    __device__ static constexpr int k_off(int w, int I) { return 49152 + (w * 4 + I) * 1024; }
};

// inclusive prefix sums over the 16 lanes of each DPP row, for 8 independent values
__device__ __forceinline__ void row_scan8(float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v[i]), 0x111, 0xf, 0xf, true));
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v[i]), 0x112, 0xf, 0xf, true));
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v[i]), 0x114, 0xf, 0xf, true));
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v[i]), 0x118, 0xf, 0xf, true));
}

template <typename Pol>
__device__ __forceinline__ typename Pol::Frag4 frag4_of(const floatx4& d) {
    typename Pol::Frag4 f;
#pragma unroll
    for (int r = 0; r < 4; ++r) f.set(r, d[r]);
    return f;
}

// ------------------------------------------------------------------------------------------
// state-pass shape (value tile width BV per workgroup)
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int BV>
struct StateShape {
    static constexpr int KS = DK >= 32 ? DK / 32 : 1;
    static constexpr int NP = (KS + 1) / 2;
    static constexpr int DKP = KS * 32;
    static constexpr int NVT = BV / 16;                 // value tiles of the workgroup
    static constexpr int NCT = DK / 16;                 // channel tiles of the state
    static constexpr int CTW = NCT >= 4 ? NCT / 4 : 1;  // channel tiles per S-role wave
    static constexpr int SST = DKP + 8;                 // row stride of the S copy
    static constexpr int EST = 64 + 8;                  // row stride of E
    static constexpr int VT = DV / BV;                  // value tiles per head
};

template <typename Pol, int KS, int NP>
__device__ __forceinline__ void decode_pairs(typename Pol::Frag (&d)[KS],
                                             const typename Pol::PairN (&r)[NP]) {
#pragma unroll
    for (int kap = 0; kap < KS; ++kap) {
        if (kap & 1) Pol::template pairn_decode<1>(d[kap], r[kap >> 1]);
        else Pol::template pairn_decode<0>(d[kap], r[kap >> 1]);
    }
}

}  // namespace kda
