// Shared device helpers for the KDA kernels (gfx950 / CDNA4, wave64).
//
// MFMA conventions used throughout (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32), for a lane l of a wave, with m = l % 16 and
// grp = l / 16:
//   A fragment: row m of the 16 x K tile, K elements 8*grp .. 8*grp+7 of the
//               current 32-wide K slice;
//   B fragment: column m of the K x 16 tile, the same 8 K elements;
//   C/D:        four fp32 values, rows 4*grp + r (r = 0..3), column m.
// Only the pairing of K elements between A and B matters, so any layout that
// gives both operands the same 8 K indices per lane is valid.
//
// Operand precision policies (the MFMA operand type of a kernel):
//   PolF32   -- fp32 operands, eight v_mfma_f32_16x16x4_f32 per 32-wide slice
//               (element e of each lane's fragment is the e-th 4-wide K step).
//   PolSplit -- each fp32 operand x is held as two bfloat16 values,
//               hi = bf16(x) and lo = bf16(x - hi) (about 16 significant bits),
//               and a product is hi*hi + hi*lo + lo*hi: three
//               v_mfma_f32_16x16x32_bf16 with fp32 accumulation. Matrices in
//               LDS keep the hi and lo parts in two planes. Fragment tiles in
//               the workspace hold x rounded to 24 bits (16 significant bits)
//               as its upper 16 bits (a bfloat16, hi) and the next 8 bits
//               (one extension byte); lo = x24 - hi is exact in bfloat16, so
//               the pair is rebuilt without loss from 3 bytes per element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx32 __attribute__((ext_vector_type(32)));
typedef unsigned u32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 64;       // tokens per chunk
constexpr int kBlock = 16;       // tokens per sub-block (MFMA tile edge)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// log(1 + y) for y in [0, 1]: a four-term series below 2^-6 (truncation below y^5 / 5, under
// 2^-24 relative there), else the hardware log2 of 1 + y (its rounding of 1 + y costs at most
// 2^-24 / y <= 2^-18 relative)
__device__ __forceinline__ float log1p_unit(float y) {
    if (y < 0.015625f) return y * (1.f - y * (0.5f - y * (1.f / 3.f - 0.25f * y)));
    return __builtin_amdgcn_logf(1.f + y) * 0.69314718055994531f;
}
// log sigmoid(x) = -(max(-x, 0) + log(1 + e^-|x|)), without overflow
__device__ __forceinline__ float log_sigmoid(float x) {
    return -(fmaxf(-x, 0.f) + log1p_unit(fast_exp2(-fabsf(x) * kLog2e)));
}
__device__ __forceinline__ float sigmoid(float x) {
    return 1.f / (1.f + fast_exp2(-x * kLog2e));
}

// ---- direct loads from global memory to LDS ----
typedef __attribute__((address_space(3))) void* lds_ptr;
// LDS address of a pointer into a __shared__ array: the low 32 bits of its generic address
// (an integer conversion, so no null test is emitted for the address-space cast)
__device__ __forceinline__ lds_ptr lds_addr(void* p) {
    return (lds_ptr)(uintptr_t)(uint32_t)(uintptr_t)p;
}
// 16 (or 4) bytes per lane from global memory to LDS at dst + 16 lane (4 lane); dst is
// wave-uniform. Completion is counted by vmcnt.
__device__ __forceinline__ void lds_load16(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, lds_addr(dst), 16, 0, 0);
}
__device__ __forceinline__ void lds_load4(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, lds_addr(dst), 4, 0, 0);
}
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// ---- input / output element access (q, k, v, beta, o) -----------------------------------
// Load 8 consecutive input elements as floats.
__device__ __forceinline__ void load8f(float* d, const bf16* p) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = (float)x[e];
}
__device__ __forceinline__ void load8f(float* d, const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
    d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
}
// Store 4 consecutive values converted to T.
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
    bf16x4 x;
    x[0] = (bf16)a; x[1] = (bf16)b; x[2] = (bf16)c; x[3] = (bf16)d;
    *reinterpret_cast<bf16x4*>(p) = x;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ float4 load4f(const bf16* p) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
}
__device__ __forceinline__ float4 load4f(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}

// Eight consecutive input elements kept in their input type (packed for bf16).
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (bf16)0.f;
    }
    __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = reinterpret_cast<const float4*>(p)[0];
        b = reinterpret_cast<const float4*>(p)[1];
    }
    __device__ __forceinline__ void zero() { a = make_float4(0.f, 0.f, 0.f, 0.f); b = a; }
    __device__ __forceinline__ float get(int e) const {
        const float4& x = e < 4 ? a : b;
        const int i = e & 3;
        return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
    }
};

// ---- operand policies ----------------------------------------------------------------------
struct PolF32 {
    using Store = float;                    // element type of stored operand matrices
    static constexpr int kPlanes = 1;
    struct Frag {
        float v[8];
        __device__ __forceinline__ void zero() {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.f;
        }
        __device__ __forceinline__ void set(int e, float x) { v[e] = x; }
        __device__ __forceinline__ float get(int e) const { return v[e]; }
        __device__ __forceinline__ void pin_regs() {
#pragma unroll
            for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(v[e]));
        }
    };
    __device__ static __forceinline__ void mma(floatx4& acc, const Frag& a, const Frag& b) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
    }
    // product with an operand b that is exact in the policy's leading part
    __device__ static __forceinline__ void mma_exact(floatx4& acc, const Frag& a, const Frag& b) {
        mma(acc, a, b);
    }
    // 16-wide K fragments (16x16x16 shapes): lane (m, grp) holds K = 4 grp + r, r = 0..3
    struct Frag4 {
        float v[4];
        __device__ __forceinline__ void set(int r, float x) { v[r] = x; }
    };
    __device__ static __forceinline__ void mma16(floatx4& acc, const Frag4& a, const Frag4& b) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[r], b.v[r], acc, 0, 0, 0);
    }
    // element x at index i of a stored matrix whose planes are ps elements apart
    __device__ static __forceinline__ void put(Store* base, size_t i, size_t /*ps*/, float x) {
        base[i] = x;
    }
    // 8 consecutive stored elements (32-byte aligned) into a fragment
    __device__ static __forceinline__ void load(Frag& f, const Store* base, size_t i,
                                                size_t /*ps*/) {
        load8f(f.v, base + i);
    }
    // 4 consecutive elements (16-byte aligned)
    __device__ static __forceinline__ void store4(Store* base, size_t i, size_t /*ps*/, float a,
                                                  float b, float c, float d) {
        *reinterpret_cast<float4*>(base + i) = make_float4(a, b, c, d);
    }
    // ---- fragment tiles in the workspace (two 1 KB parts, lane-contiguous 16 B each) ----
    // part 0 holds elements 0..3 of every lane, part 1 elements 4..7
    using Tile = Frag;                      // fp32 tiles are used as loaded
    __device__ static __forceinline__ void tile_store_vals(void* t, int lane, const float* x) {
        float4* p = reinterpret_cast<float4*>(t);
        p[lane] = make_float4(x[0], x[1], x[2], x[3]);
        p[64 + lane] = make_float4(x[4], x[5], x[6], x[7]);
    }
    __device__ static __forceinline__ void tile_load_raw(Tile& f, const void* t, int lane) {
        const float4* p = reinterpret_cast<const float4*>(t);
        const float4 a = p[lane], b = p[64 + lane];
        f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
        f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    }
    __device__ static __forceinline__ void tile_decode(Frag& f, const Tile& r) { f = r; }
    // pair tiles: two fragment tiles a, b back to back
    static constexpr int kPairBytes = 4096;
    struct Pair { Frag f[2]; };
    __device__ static __forceinline__ void pair_store_vals(void* t, int lane, int which,
                                                           const float* x) {
        tile_store_vals(reinterpret_cast<uint8_t*>(t) + 2048 * which, lane, x);
    }
    __device__ static __forceinline__ void pair_store_quad(void* t, int lane, int which, int half,
                                                           float a, float b, float c, float d) {
        reinterpret_cast<float4*>(reinterpret_cast<uint8_t*>(t) + 2048 * which)[64 * half + lane] =
            make_float4(a, b, c, d);
    }
    __device__ static __forceinline__ void pair_load(Pair& r, const void* t, int lane) {
        tile_load_raw(r.f[0], t, lane);
        tile_load_raw(r.f[1], reinterpret_cast<const uint8_t*>(t) + 2048, lane);
    }
    // fragment a alone (b is not read afterwards)
    __device__ static __forceinline__ void pair_load_a(Pair& r, const void* t, int lane) {
        tile_load_raw(r.f[0], t, lane);
    }
    template <int W>
    __device__ static __forceinline__ void pair_decode(Frag& f, const Pair& r) { f = r.f[W]; }
    // narrower pairs of the bf16 path: full fp32 here
    static constexpr int kPairNBytes = kPairBytes;
    using PairN = Pair;
    __device__ static __forceinline__ void pairn_store_vals(void* t, int lane, int which,
                                                            const float* x) {
        pair_store_vals(t, lane, which, x);
    }
    __device__ static __forceinline__ void pairn_store_quad(void* t, int lane, int which, int half,
                                                            float a, float b, float c, float d) {
        pair_store_quad(t, lane, which, half, a, b, c, d);
    }
    __device__ static __forceinline__ void pairn_load(PairN& r, const void* t, int lane) {
        pair_load(r, t, lane);
    }
    template <int W>
    __device__ static __forceinline__ void pairn_decode(Frag& f, const PairN& r) { f = r.f[W]; }
    // ---- U tiles (1 KB): four fp32 values per lane ----
    static constexpr int kUTileBytes = 1024;
    using URaw = float4;
    __device__ static __forceinline__ void utile_store(void* t, int lane, float a, float b,
                                                       float c, float d) {
        reinterpret_cast<float4*>(t)[lane] = make_float4(a, b, c, d);
    }
    __device__ static __forceinline__ void utile_load(URaw& r, const void* t, int lane) {
        r = reinterpret_cast<const float4*>(t)[lane];
    }
    __device__ static __forceinline__ float4 utile_decode(const URaw& r) { return r; }
    // product with b exact in the leading part (same as mma16 in fp32)
    __device__ static __forceinline__ void mma16_exact(floatx4& acc, const Frag4& a, const Frag4& b) {
        mma16(acc, a, b);
    }
    // x times an exact 0/1 matrix e (an exact copy in fp32)
    __device__ static __forceinline__ void mma_copy(floatx4& acc, const Frag& x, const Frag& e) {
        mma(acc, x, e);
    }
    // x times a 0/1 selection matrix e (a transpose, exact) as a 16-wide K fragment
    __device__ static __forceinline__ Frag4 transpose4(const Frag& x, const Frag& e) {
        floatx4 t = {0.f, 0.f, 0.f, 0.f};
        mma(t, x, e);
        Frag4 f;
#pragma unroll
        for (int r = 0; r < 4; ++r) f.v[r] = t[r];
        return f;
    }
};

struct PolSplit {
    using Store = bf16;
    static constexpr int kPlanes = 2;
    struct Frag {
        bf16x8 hi, lo;
        __device__ __forceinline__ void zero() {
#pragma unroll
            for (int e = 0; e < 8; ++e) { hi[e] = (bf16)0.f; lo[e] = (bf16)0.f; }
        }
        __device__ __forceinline__ void set(int e, float x) {
            const bf16 h = (bf16)x;
            hi[e] = h;
            lo[e] = (bf16)(x - (float)h);
        }
        __device__ __forceinline__ float get(int e) const { return (float)hi[e] + (float)lo[e]; }
        __device__ __forceinline__ void pin_regs() {
            asm volatile("" : "+v"(hi));
            asm volatile("" : "+v"(lo));
        }
    };
    __device__ static __forceinline__ void mma(floatx4& acc, const Frag& a, const Frag& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    }
    // product with an operand b that is exact in bfloat16 (b.lo == 0): two MFMAs
    __device__ static __forceinline__ void mma_exact(floatx4& acc, const Frag& a, const Frag& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    }
    // 16-wide K fragments (16x16x16 shapes): lane (m, grp) holds K = 4 grp + r, r = 0..3
    struct Frag4 {
        bf16x4 hi, lo;
        __device__ __forceinline__ void set(int r, float x) {
            const bf16 h = (bf16)x;
            hi[r] = h;
            lo[r] = (bf16)(x - (float)h);
        }
    };
    __device__ static __forceinline__ void mma16(floatx4& acc, const Frag4& a, const Frag4& b) {
        typedef short short4v __attribute__((ext_vector_type(4)));
        const short4v ah = __builtin_bit_cast(short4v, a.hi), al = __builtin_bit_cast(short4v, a.lo);
        const short4v bh = __builtin_bit_cast(short4v, b.hi), bl = __builtin_bit_cast(short4v, b.lo);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    }
    __device__ static __forceinline__ void put(Store* base, size_t i, size_t ps, float x) {
        const bf16 h = (bf16)x;
        base[i] = h;
        base[ps + i] = (bf16)(x - (float)h);
    }
    __device__ static __forceinline__ void load(Frag& f, const Store* base, size_t i, size_t ps) {
        f.hi = *reinterpret_cast<const bf16x8*>(base + i);
        f.lo = *reinterpret_cast<const bf16x8*>(base + ps + i);
    }
    // 4 consecutive elements (8-byte aligned in each plane)
    __device__ static __forceinline__ void store4(Store* base, size_t i, size_t ps, float a,
                                                  float b, float c, float d) {
        bf16x4 h, l;
        h[0] = (bf16)a; h[1] = (bf16)b; h[2] = (bf16)c; h[3] = (bf16)d;
        l[0] = (bf16)(a - (float)h[0]); l[1] = (bf16)(b - (float)h[1]);
        l[2] = (bf16)(c - (float)h[2]); l[3] = (bf16)(d - (float)h[3]);
        *reinterpret_cast<bf16x4*>(base + i) = h;
        *reinterpret_cast<bf16x4*>(base + ps + i) = l;
    }
    // ---- 24-bit fragments: the eight hi values of a lane (16 B) and their extension bytes
    // (8 B), as held in registers after a pair tile load ----
    struct Tile { bf16x8 hi; u32x2 ext; };
    // x rounded to 24 bits of float32 (16 significant bits), half-way cases away from zero;
    // the low byte is left as is (callers take bytes 1..3 only)
    __device__ static __forceinline__ unsigned round24(float x) {
        return __float_as_uint(x) + 0x80u;
    }
    __device__ static __forceinline__ unsigned ext4(unsigned a, unsigned b, unsigned c,
                                                    unsigned d) {
        return ((a >> 8) & 0xffu) | (b & 0xff00u) | ((c << 8) & 0xff0000u) |
               ((d << 16) & 0xff000000u);
    }
    // hi as stored; lo = (hi with its extension byte) - hi, exact in bfloat16. The two
    // 24-bit values of a word pair are assembled with one byte permute each (v_perm_b32:
    // bytes 4..7 select from the hi word, 0..3 from the extension word, 0x0c gives zero).
    __device__ static __forceinline__ void tile_decode(Frag& f, const Tile& r) {
        f.hi = r.hi;
        const u32x4 w = __builtin_bit_cast(u32x4, r.hi);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const unsigned e = r.ext[p >> 1];
            const unsigned b = 2u * (p & 1);               // byte of element 2p in e
            const unsigned x0 = __builtin_amdgcn_perm(w[p], e, 0x0504000cu | (b << 8));
            const unsigned x1 = __builtin_amdgcn_perm(w[p], e, 0x0706000cu | ((b + 1) << 8));
            const unsigned h0 = w[p] << 16, h1 = w[p] & 0xffff0000u;
            f.lo[2 * p] = (bf16)(__uint_as_float(x0) - __uint_as_float(h0));
            f.lo[2 * p + 1] = (bf16)(__uint_as_float(x1) - __uint_as_float(h1));
        }
    }
    // pair tiles (3 KB): the hi values of fragment a (1 KB), of fragment b (1 KB), then the
    // extension bytes of both (1 KB: 8 B of a, 8 B of b per lane), so two fragments take
    // three 16-byte loads per lane
    static constexpr int kPairBytes = 3072;
    struct Pair { bf16x8 hi[2]; u32x4 ext; };
    __device__ static __forceinline__ void pair_store_vals(void* t, int lane, int which,
                                                           const float* x) {
        unsigned r[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = round24(x[e]);
        u32x4 hw;
#pragma unroll
        for (int p = 0; p < 4; ++p) hw[p] = (r[2 * p] >> 16) | (r[2 * p + 1] & 0xffff0000u);
        u32x2 ew;
        ew[0] = ext4(r[0], r[1], r[2], r[3]);
        ew[1] = ext4(r[4], r[5], r[6], r[7]);
        reinterpret_cast<u32x4*>(t)[64 * which + lane] = hw;
        // half of every 16 B: the other wave of the pair writes the rest, merged in L2
        reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(t) + 2048)[2 * lane + which] = ew;
    }
    __device__ static __forceinline__ void pair_load(Pair& r, const void* t, int lane) {
        const bf16x8* p = reinterpret_cast<const bf16x8*>(t);
        r.hi[0] = p[lane];
        r.hi[1] = p[64 + lane];
        r.ext = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(t) + 2048)[lane];
    }
    // fragment a alone (b is not read afterwards): its hi values and its 8 extension bytes
    __device__ static __forceinline__ void pair_load_a(Pair& r, const void* t, int lane) {
        const bf16x8* p = reinterpret_cast<const bf16x8*>(t);
        r.hi[0] = p[lane];
        const u32x2 e = reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(t) + 2048)[2 * lane];
        r.ext[0] = e[0];
        r.ext[1] = e[1];
    }
    template <int W>
    __device__ static __forceinline__ void pair_decode(Frag& f, const Pair& r) {
        Tile t;
        t.hi = r.hi[W];
        t.ext[0] = r.ext[2 * W];
        t.ext[1] = r.ext[2 * W + 1];
        tile_decode(f, t);
    }
    // ---- 20-bit pair tiles (2.5 KB): x rounded to 20 bits of float32 (12 significant bits,
    // half-way cases away from zero), kept as its bfloat16 hi plus a 4-bit nibble: the hi
    // values of a, of b, then per lane the 8 nibbles of a (4 B) and of b (4 B). The state
    // pass rebuilds lo = (hi with its nibble) - hi, exact in bfloat16 ----
    static constexpr int kPairNBytes = 2560;
    struct PairN { bf16x8 hi[2]; u32x2 nib; };
    __device__ static __forceinline__ unsigned round20(float x) { return __float_as_uint(x) + 0x800u; }
    __device__ static __forceinline__ void pairn_store_vals(void* t, int lane, int which,
                                                            const float* x) {
        unsigned r[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = round20(x[e]);
        u32x4 hw;
        unsigned nb = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) hw[p] = (r[2 * p] >> 16) | (r[2 * p + 1] & 0xffff0000u);
#pragma unroll
        for (int e = 0; e < 8; ++e) nb |= ((r[e] >> 12) & 0xfu) << (4 * e);
        reinterpret_cast<u32x4*>(t)[64 * which + lane] = hw;
        reinterpret_cast<unsigned*>(reinterpret_cast<uint8_t*>(t) + 2048)[2 * lane + which] = nb;
    }
    __device__ static __forceinline__ void pairn_store_quad(void* t, int lane, int which, int half,
                                                            float a, float b, float c, float d) {
        const unsigned r0 = round20(a), r1 = round20(b), r2 = round20(c), r3 = round20(d);
        u32x2 hw;
        hw[0] = (r0 >> 16) | (r1 & 0xffff0000u);
        hw[1] = (r2 >> 16) | (r3 & 0xffff0000u);
        const unsigned nb = ((r0 >> 12) & 0xfu) | (((r1 >> 12) & 0xfu) << 4) |
                            (((r2 >> 12) & 0xfu) << 8) | (((r3 >> 12) & 0xfu) << 12);
        reinterpret_cast<u32x2*>(t)[128 * which + 2 * lane + half] = hw;
        reinterpret_cast<unsigned short*>(reinterpret_cast<uint8_t*>(t) + 2048)[4 * lane + 2 * which + half] =
            (unsigned short)nb;
    }
    __device__ static __forceinline__ void pairn_load(PairN& r, const void* t, int lane) {
        const bf16x8* p = reinterpret_cast<const bf16x8*>(t);
        r.hi[0] = p[lane];
        r.hi[1] = p[64 + lane];
        r.nib = reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(t) + 2048)[lane];
    }
    template <int W>
    __device__ static __forceinline__ void pairn_decode(Frag& f, const PairN& r) {
        f.hi = r.hi[W];
        const u32x4 w = __builtin_bit_cast(u32x4, r.hi[W]);
        const unsigned n = r.nib[W];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const unsigned h0 = w[p] << 16, h1 = w[p] & 0xffff0000u;
            const unsigned x0 = h0 | (__builtin_amdgcn_ubfe(n, 8 * p, 4) << 12);
            const unsigned x1 = h1 | (__builtin_amdgcn_ubfe(n, 8 * p + 4, 4) << 12);
            f.lo[2 * p] = (bf16)(__uint_as_float(x0) - __uint_as_float(h0));
            f.lo[2 * p + 1] = (bf16)(__uint_as_float(x1) - __uint_as_float(h1));
        }
    }
    // ---- U tiles (768 B): four values per lane in the 24-bit form, the hi halves (8 B per
    // lane) then the extension bytes (4 B per lane); U is an addend, so a value is rebuilt
    // as one float32 (one byte permute) ----
    static constexpr int kUTileBytes = 768;
    struct URaw { u32x2 h; unsigned e; };
    __device__ static __forceinline__ void utile_store(void* t, int lane, float a, float b,
                                                       float c, float d) {
        const unsigned r0 = round24(a), r1 = round24(b), r2 = round24(c), r3 = round24(d);
        u32x2 hw;
        hw[0] = (r0 >> 16) | (r1 & 0xffff0000u);
        hw[1] = (r2 >> 16) | (r3 & 0xffff0000u);
        reinterpret_cast<u32x2*>(t)[lane] = hw;
        reinterpret_cast<unsigned*>(reinterpret_cast<uint8_t*>(t) + 512)[lane] = ext4(r0, r1, r2, r3);
    }
    __device__ static __forceinline__ void utile_load(URaw& r, const void* t, int lane) {
        r.h = reinterpret_cast<const u32x2*>(t)[lane];
        r.e = reinterpret_cast<const unsigned*>(reinterpret_cast<const uint8_t*>(t) + 512)[lane];
    }
    __device__ static __forceinline__ float4 utile_decode(const URaw& r) {
        return make_float4(__uint_as_float(__builtin_amdgcn_perm(r.h[0], r.e, 0x0504000cu)),
                           __uint_as_float(__builtin_amdgcn_perm(r.h[0], r.e, 0x0706010cu)),
                           __uint_as_float(__builtin_amdgcn_perm(r.h[1], r.e, 0x0504020cu)),
                           __uint_as_float(__builtin_amdgcn_perm(r.h[1], r.e, 0x0706030cu)));
    }
    // product with b exact in bfloat16 (b.lo == 0): two MFMAs
    __device__ static __forceinline__ void mma16_exact(floatx4& acc, const Frag4& a, const Frag4& b) {
        typedef short short4v __attribute__((ext_vector_type(4)));
        const short4v ah = __builtin_bit_cast(short4v, a.hi), al = __builtin_bit_cast(short4v, a.lo);
        const short4v bh = __builtin_bit_cast(short4v, b.hi);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    }
    // x (exact in bfloat16, x.lo == 0) times an exact 0/1 matrix e: one MFMA
    __device__ static __forceinline__ void mma_copy(floatx4& acc, const Frag& x, const Frag& e) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.hi, e.hi, acc, 0, 0, 0);
    }
    // x times a 0/1 selection matrix e (a transpose) as a 16-wide K fragment: the hi and lo
    // parts are moved by one MFMA each, so both come out exact and need no new split
    __device__ static __forceinline__ Frag4 transpose4(const Frag& x, const Frag& e) {
        floatx4 th = {0.f, 0.f, 0.f, 0.f}, tl = {0.f, 0.f, 0.f, 0.f};
        th = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.hi, e.hi, th, 0, 0, 0);
        tl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.lo, e.hi, tl, 0, 0, 0);
        Frag4 f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f.hi[r] = (bf16)th[r];
            f.lo[r] = (bf16)tl[r];
        }
        return f;
    }
};

// fp32 16 x 16 x 16 product: lane (m, grp) holds a[r] = A[m][4 grp + r] and
// b[r] = B[4 grp + r][m]; acc gets the C layout (rows 4 grp + r, column m).
__device__ __forceinline__ void mma16_f32(floatx4& acc, const float4& a, const float4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
}

// Forces a register value to be computed here: the compiler may not sink its producers
// (decodes, and the waits on the loads they read) past this point.
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float4& x) {
    asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
}

// ---- cross-lane helpers (a DPP row = 16 consecutive lanes = one value of grp) ------------
// one step (row_shr by 1, 2, 4 or 8 lanes: CTRL 0x111, 0x112, 0x114, 0x118) of the
// inclusive row prefix sum, applied to 32 independent values
template <int CTRL>
__device__ __forceinline__ void row_scan16_step(float (&v)[32]) {
#pragma unroll
    for (int i = 0; i < 32; ++i)
        v[i] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v[i]), CTRL, 0xf, 0xf, true));
}
// value of lane n (compile-time) of each row, broadcast to the row
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xf, 0xf, false));
}

// The operand policy of an input type: fp32 inputs keep fp32 MFMA, bf16 inputs use
// split-bf16 operands.
template <typename TI> struct PolOf;
template <> struct PolOf<float> { using type = PolF32; };
template <> struct PolOf<bf16> { using type = PolSplit; };

}  // namespace kda
