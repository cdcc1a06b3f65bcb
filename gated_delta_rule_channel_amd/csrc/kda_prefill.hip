// Chunked KDA prefill for gfx950: chunk map, chunk-parallel prep, serial state pass.
//
// The chunkwise schedule of "Kimi Delta Attention (KDA)" (brain.bigb.es,
// section "Two schedules for the same recurrence"), in the state orientation
// S[d_k][d_v] (row = key channel). For a chunk of C = 64 tokens with incoming
// state S and in-chunk inclusive log-decay prefix sums G_i (per key channel):
//
//   A_kk[i][j] = beta_i sum_c k_i[c] k_j[c] exp(G_i[c] - G_j[c])   j <  i
//   A_qk[i][j] = scale  sum_c q_i[c] k_j[c] exp(G_i[c] - G_j[c])   j <= i
//   T = (I + A_kk)^-1                          (unit lower triangular; the UT
//                                               transform of "From Fast Weight
//                                               Programmers to KDA",
//                                               jonahsamost.bearblog.dev)
//   W = T (beta k exp(G)),  U = T (beta v)     (WY factors; W carries the decay
//                                               from the chunk start)
//   E = U - W S                                (true errors of the chunk)
//   O = (scale q exp(G)) S + A_qk E           (reads S, then in-chunk writes)
//   S' = Diag(exp(G_end)) S + (k exp(G_end - G))^T E
//
// Kernels
//  * chunk_map_kernel (packed sequences only):  cu_seqlens -> table of (token
//    start, length, seq) per chunk slot and the first slot of every sequence, on
//    the device (the host never reads cu_seqlens). A fixed-length batch maps
//    slots arithmetically.
//  * prep_kernel: one workgroup per (chunk, head), fully parallel. Computes
//    everything that does not depend on S and writes it to the workspace:
//    W [64][Dk], Qd = scale q exp(G) [64][Dk], KdT = (k exp(G_end-G))^T
//    [Dk][64], U^T [Dv][64], A_qk [64][64] (operand precision) and exp(G_end)
//    [Dk] (fp32).
//  * state_kernel: one workgroup per (sequence, head, 32-column value tile),
//    the only serial pass; S stays in fp32 MFMA accumulators for the whole
//    sequence, with an operand-precision copy in LDS.
//
// Decay factors. Every exp(G_i - G_j) is formed as a product of two factors
// each bounded by 2^120 (in log2 units x = G log2 e), so nothing overflows or
// loses the range of float32/bfloat16:
//  * off-diagonal 16x16 blocks (row block I > column block J): exp(G_i - G_r)
//    with r the last token before block I (<= 1) times exp(G_r - G_j) (<= 1);
//  * diagonal 16x16 blocks: the same reference r when no channel decays by
//    more than 2^120 inside the block (the column factor exp(G_r - G_j) is then
//    at most 2^120); else the block's 8th row m, exp(G_i - G_m) exp(G_m - G_j),
//    when every |G_i - G_m| is within 120; else pairwise (exp2 of each
//    difference).
// The in-chunk prefix sums are computed per 16-token block (log-space prefix
// sums, as the page's "real Triton implementation" paragraph describes), and
// cross-block factors come from block totals.
#include <atomic>
#include <type_traits>

#include "kda_prefill_shared.h"

namespace kda {

size_t prefill_block_bytes(int Dk, int Dv, bool bf16_in) {
    return bf16_in ? ws_block_bytes(Dk, Dv, PolSplit::kPairBytes, PolSplit::kUTileBytes,
                                    PolSplit::kPairNBytes)
                   : ws_block_bytes(Dk, Dv, PolF32::kPairBytes, PolF32::kUTileBytes,
                                    PolF32::kPairNBytes);
}

// ------------------------------------------------------------------------------------------
// chunk map
// ------------------------------------------------------------------------------------------
// tab[slot] = {token start, length (0 = unused slot), sequence, 0}; seq_off[n] = first slot
// of sequence n, seq_off[N] = number of used slots.
__global__ __launch_bounds__(256) void chunk_map_kernel(const int32_t* __restrict__ cu, int N,
                                                         int T, int max_slots,
                                                         int4* __restrict__ tab,
                                                         int32_t* __restrict__ seq_off) {
    __shared__ int s_scan[256];
    __shared__ int s_carry;
    const int tid = threadIdx.x;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int n = base + tid;
        int st = 0, en = 0, cnt = 0;
        if (n < N) {
            // packed bounds are clamped to [0, T] with en >= st, so a malformed cu_seqlens
            // can only mis-assign tokens, never address outside the inputs
            st = cu ? min(max(cu[n], 0), T) : n * T;
            en = cu ? min(max(cu[n + 1], st), T) : (n + 1) * T;
            const int len = en > st ? en - st : 0;
            cnt = (len + kChunk - 1) / kChunk;
        }
        s_scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int add = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += add;
            __syncthreads();
        }
        const int excl = s_carry + s_scan[tid] - cnt;
        if (n < N) {
            seq_off[n] = excl < max_slots ? excl : max_slots;
            for (int c = 0; c < cnt; ++c) {
                const int slot = excl + c;
                if (slot < max_slots) {
                    const int s0 = st + c * kChunk;
                    const int l = en - s0 < kChunk ? en - s0 : kChunk;
                    tab[slot] = make_int4(s0, l, n, 0);
                }
            }
        }
        __syncthreads();
        if (tid == 255) s_carry += s_scan[255];
        __syncthreads();
    }
    const int total = s_carry < max_slots ? s_carry : max_slots;
    if (tid == 0) seq_off[N] = total;
    for (int s = total + tid; s < max_slots; s += 256) tab[s] = make_int4(0, 0, -1, 0);
}

// ------------------------------------------------------------------------------------------
// prep kernel
// ------------------------------------------------------------------------------------------
// Persistent workgroups (4 waves, two per CU) walk the (chunk, head) tasks with a stride of
// the grid size; consecutive workgroups take the heads of one chunk, so the tasks in flight
// read neighbouring token rows. For bf16 input the next task's g, k, q and beta are copied
// global -> LDS (direct-to-LDS loads, 16 B per lane) while the current task forms W and U,
// into the LDS region that holds the A and T blocks earlier in the task, so a task starts
// from LDS instead of waiting on HBM. Within a task, wave w owns the 32-channel slice
// [32 w, 32 w + 32) of the keys for all 64 tokens, held in MFMA fragment layout: lane
// (m, grp) holds token 16 I + m of every 16-token block I and the 8 channels
// 32 w + 8 grp + e. In-chunk prefix sums are DPP scans across the 16 lanes of a row.
// Each wave forms its slice's partial A_kk / A_qk blocks with MFMAs; the four partials of
// a block are summed in LDS in a fixed order (the waves visit the row blocks in rotated
// order, one writer per block per step), so results are bitwise reproducible. The row
// block of a step is wave-uniform, so per-block registers are read with register-indexed
// moves. T = (I + A_kk)^-1 is formed in fp32: diagonal blocks by forward substitution, the
// rest column block by column block with fp32 MFMAs. W and U use T' = T diag(beta):
// W = T' (k exp G), U = T' v. Register-level transposes (token-major fragments to
// channel-major ones) are products with an identity slice.

// SG: one log-decay per token and head (Gated DeltaNet). EW: Gated DeltaNet-2, where a
// per-key-channel erase gate eb scales the key on the side that reads the old value (row
// operands of A_kk and the operand of W) and a per-value-channel write gate ew scales v
// (U = T (ew v)); beta is not used and T' = T. That variant runs one workgroup per CU.
template <typename TI, int DK, int DV, bool SG, bool EW>
__global__ __launch_bounds__(256, EW ? 1 : 2) void prep_kernel(
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v,
    const float* __restrict__ g, const TI* __restrict__ beta, const TI* __restrict__ eb,
    const TI* __restrict__ ew, float scale, const int4* __restrict__ tab, int T, int nslots,
    uint8_t* __restrict__ ws, int H, long long beta_elems) {
    using Pol = typename PolOf<TI>::type;
    using Frag = typename Pol::Frag;
    using Frag4 = typename Pol::Frag4;
    using Ly = WsLayoutOf<Pol, DK, DV>;
    using Stg = PrepStage<TI>;
    constexpr int NSL = DK >= 32 ? DK / 32 : 1;          // channel slices (32 wide, padded)
    constexpr int NVS = DV >= 32 ? DV / 32 : 1;          // value slices
    // lower 16x16 blocks, rows padded to 20 floats so that 16 lanes reading 4 floats of
    // 16 different rows hit distinct LDS banks: T = (I + A_kk)^-1, A_kk and A_qk. The same
    // region receives the next task's staged inputs as its parts fall free.
    constexpr int kABytes = 3 * 10 * 16 * 20 * 4;
    constexpr int kRBytes = kABytes > Stg::kBytes ? kABytes : Stg::kBytes;
    __shared__ __attribute__((aligned(16))) float sR[kRBytes / 4];
    float (*const sT)[16][20] = reinterpret_cast<float (*)[16][20]>(sR);
    float (*const sKK)[16][20] = reinterpret_cast<float (*)[16][20]>(sR + 10 * 16 * 20);
    float (*const sQK)[16][20] = reinterpret_cast<float (*)[16][20]>(sR + 2 * 10 * 16 * 20);
    uint8_t* const sRb = reinterpret_cast<uint8_t*>(sR);
    __shared__ float sBeta[64];
    __shared__ unsigned sBetaRaw[64];                     // staged word holding beta of token t
    __shared__ float4 sCE[4][NSL * 8];                    // cumulative log-decay at block ends
    __shared__ Frag4 sTp[10][64];                         // T' = T diag(beta) as fragments

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15, grp = lane >> 4;
    const size_t rowq = (size_t)H * DK, rowv = (size_t)H * DV;
    const bool cs = wave < NSL;                  // this wave owns a channel slice
    const int c0 = 32 * wave + 8 * grp;          // first of this lane's 8 channels
    const bool cvalid = cs && c0 < DK;
    const int ntasks = nslots * H;

    // token range of a chunk slot
    auto chunk_of = [&](int slot, int& t0, int& L) {
        if (tab) {                                        // packed sequences: chunk table
            const int4 ci = tab[slot];
            t0 = ci.x;
            L = ci.y;
        } else {                                          // B rows of T tokens
            const int nck = (T + kChunk - 1) / kChunk, row = slot / nck, c = slot % nck;
            t0 = row * T + kChunk * c;
            L = T - kChunk * c < kChunk ? T - kChunk * c : kChunk;
        }
    };
    // issues the staged loads of row block I of a task (bf16 input only): g, k and q of the
    // block, and beta with block 0
    auto stage = [&](int t0, int L, int h, int I) {
        if constexpr (Stg::kBytes > 0) {
            const int row = 16 * I + m;
            if (cvalid && row < L) {
                const size_t off = (size_t)(t0 + row) * rowq + (size_t)h * DK + c0;
                lds_load16(k + off, sRb + Stg::k_off(wave, I));
                lds_load16(q + off, sRb + Stg::q_off(wave, I));
            }
            if constexpr (SG) {
                // scalar gate: the block's 16 values, one per lane, to the start of the part
                if (cs && lane < 16 && 16 * I + lane < L)
                    lds_load4(g + (size_t)(t0 + 16 * I + lane) * H + h, sRb + Stg::g_off(wave, I, 0));
            } else {
                // g (float32): eight lanes per row, so each load covers whole 128-byte rows of
                // the slice (rows 8 hg .. 8 hg + 7 of the block)
#pragma unroll
                for (int hg = 0; hg < 2; ++hg) {
                    const int grow = 16 * I + 8 * hg + (lane >> 3), gc = 32 * wave + 4 * (lane & 7);
                    if (cs && gc < DK && grow < L)
                        lds_load16(g + (size_t)(t0 + grow) * rowq + (size_t)h * DK + gc,
                                   sRb + Stg::g_off(wave, I, hg));
                }
            }
            if (!EW && I == 0 && wave == 0 && lane < L) {
                const size_t e = (size_t)(t0 + lane) * H + h;       // beta element index
                if ((e & 1) == 0 && (long long)e + 1 >= beta_elems) {
                    // the word holding the last element would extend past the array: read
                    // that element alone (once per call, so its wait costs nothing)
                    sBetaRaw[lane] = reinterpret_cast<const unsigned short*>(beta)[e];
                } else {
                    lds_load4(reinterpret_cast<const unsigned*>(beta) + (e >> 1), sBetaRaw);
                }
            }
        }
    };
    // identity slices: Eid[hh] as a B operand maps K index 16 hh + n to column n
    Frag Eid[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) Eid[hh].set(e, (8 * grp + e == 16 * hh + m) ? 1.f : 0.f);

    bool staged = false;                                  // the task's inputs are in LDS
#pragma unroll 1
    for (int task = blockIdx.x; task < ntasks; task += gridDim.x) {
        const int slot = task / H, h = task % H;
        int t0, L;
        chunk_of(slot, t0, L);
        if (L <= 0) {                                         // unused slot (uniform)
            staged = false;
            continue;
        }
        uint8_t* blk = ws + ((size_t)slot * H + h) * Ly::BYTES;
        float* gGend = reinterpret_cast<float*>(blk + Ly::GEND);

        // ---- inputs: g, k, q of the slice for all 64 tokens; beta of the chunk to LDS ----
        floatx32 G;
        In32<TI> K, Q;
        if constexpr (Stg::kBytes > 0) {
            if (!staged) {
#pragma unroll
                for (int I = 0; I < 4; ++I) stage(t0, L, h, I);
                wait_all_memory();
            }
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int row = 16 * I + m;
                if (cvalid && row < L) {
                    if constexpr (SG) {
                        const float gs = reinterpret_cast<const float*>(sRb + Stg::g_off(wave, I, 0))[m];
#pragma unroll
                        for (int e = 0; e < 8; ++e) G[8 * I + e] = gs;
                    } else {
                        // row m of the block sits in part m / 8, its 8 channels at 16-byte
                        // slots 8 (m % 8) + 2 grp and the next
                        const floatx4* gp =
                            reinterpret_cast<const floatx4*>(sRb + Stg::g_off(wave, I, m >> 3)) +
                            8 * (m & 7) + 2 * grp;
                        const floatx4 g0 = gp[0], g1 = gp[1];
                        G[8 * I] = g0[0]; G[8 * I + 1] = g0[1]; G[8 * I + 2] = g0[2]; G[8 * I + 3] = g0[3];
                        G[8 * I + 4] = g1[0]; G[8 * I + 5] = g1[1]; G[8 * I + 6] = g1[2]; G[8 * I + 7] = g1[3];
                    }
                    K.set(I, reinterpret_cast<const u32x4*>(sRb + Stg::k_off(wave, I))[lane]);
                    Q.set(I, reinterpret_cast<const u32x4*>(sRb + Stg::q_off(wave, I))[lane]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) G[8 * I + e] = 0.f;
                    K.zero(I);
                    Q.zero(I);
                }
            }
            if (tid < 64) {
                const size_t e = (size_t)(t0 + tid) * H + h;
                const unsigned w = sBetaRaw[tid];
                sBeta[tid] = tid < L ? (EW ? 1.f : __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16)))
                                     : 0.f;
            }
        } else {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int row = 16 * I + m;
                if (cvalid && row < L) {
                    const size_t off = (size_t)(t0 + row) * rowq + (size_t)h * DK + c0;
                    if constexpr (SG) {
                        const float gs = g[(size_t)(t0 + row) * H + h];
#pragma unroll
                        for (int e = 0; e < 8; ++e) G[8 * I + e] = gs;
                    } else {
                        const floatx4 g0 = reinterpret_cast<const floatx4*>(g + off)[0];
                        const floatx4 g1 = reinterpret_cast<const floatx4*>(g + off)[1];
                        G[8 * I] = g0[0]; G[8 * I + 1] = g0[1]; G[8 * I + 2] = g0[2]; G[8 * I + 3] = g0[3];
                        G[8 * I + 4] = g1[0]; G[8 * I + 5] = g1[1]; G[8 * I + 6] = g1[2]; G[8 * I + 7] = g1[3];
                    }
                    K.load(I, k + off);
                    Q.load(I, q + off);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) G[8 * I + e] = 0.f;
                    K.zero(I);
                    Q.zero(I);
                }
            }
            if (tid < 64) sBeta[tid] = tid < L ? (EW ? 1.f : to_f(beta[(size_t)(t0 + tid) * H + h])) : 0.f;
        }
        // erase gates of the lane's rows and channels (Gated DeltaNet-2), read from global memory
        In32<TI> Eb;
        if constexpr (EW) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int row = 16 * I + m;
                if (cvalid && row < L)
                    Eb.load(I, eb + (size_t)(t0 + row) * rowq + (size_t)h * DK + c0);
                else
                    Eb.zero(I);
            }
        }
        // every wave has its inputs (and is past the previous task's reads of sCE): the staging
        // region becomes the A accumulators (the first partial of each block is stored, the
        // others added, so they need no clearing)
        __syncthreads();

        // ---- block-local prefix sums (log2 units); the cumulative value at each block end goes
        //      to LDS (all 16 lanes of a row hold it), the chunk total stays in registers ----
        float gtot[8];
        {
            float ce[4][8];
            // the lane's 32 scans advance one shift at a time, so consecutive DPP adds are
            // independent and need no hazard wait states (on a plain array: the same steps
            // applied to the elements of the vector type through a reference compiled to
            // wrong code with this toolchain)
            float gs[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) gs[i] = G[i] * kLog2e;
            row_scan16_step<0x111>(gs);
            row_scan16_step<0x112>(gs);
            row_scan16_step<0x114>(gs);
            row_scan16_step<0x118>(gs);
#pragma unroll
            for (int i = 0; i < 32; ++i) G[i] = gs[i];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    acc += row_bcast<15>(G[8 * I + e]);
                    ce[I][e] = acc;
                }
                gtot[e] = acc;
            }
            if (cs && m == 0) {
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    sCE[I][2 * (c0 / 8)] = make_float4(ce[I][0], ce[I][1], ce[I][2], ce[I][3]);
                    sCE[I][2 * (c0 / 8) + 1] = make_float4(ce[I][4], ce[I][5], ce[I][6], ce[I][7]);
                }
            }
        }
        // with a scalar gate the 8 channels of a row hold the same values: reading one of them
        // for all 8 lets the compiler form each decay factor once
        if constexpr (SG) {
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int e = 1; e < 8; ++e) G[8 * I + e] = G[8 * I];
#pragma unroll
            for (int e = 1; e < 8; ++e) gtot[e] = gtot[0];
        }
        // the 8 cumulative values of this lane's channels at the end of block I
        auto ce8 = [&](int I, float* o) {
            const float4 a = sCE[I][2 * (c0 / 8)], b = sCE[I][2 * (c0 / 8) + 1];
            o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
            o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
            if constexpr (SG) {
#pragma unroll
                for (int e = 1; e < 8; ++e) o[e] = o[0];
            }
        };
        if (cvalid && m == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) gGend[c0 + e] = fast_exp2(gtot[e]);
        }
        __syncthreads();                                    // A accumulators zeroed, beta in LDS

        // ---- rotated pass over the row blocks: Qd, Kd^T, partial A blocks. The row block of
        //      a step depends on the wave; each row block is its own instance of the step, so
        //      the register arrays are indexed with constants ----
        auto row_step = [&](auto Ic, int st) {
            constexpr int I = decltype(Ic)::value;
            constexpr int Ip = I > 0 ? I - 1 : 0;
            // the blocks of row I (and the pair (3, 0) with row 0) get their first partial from
            // the channel-slice wave that reaches row I first: wave min(I, NSL - 1), at this step
            const bool first = st == I - (I < NSL - 1 ? I : NSL - 1);
            // the step reads its inputs through empty asm statements, so that no part of it is
            // computed ahead of the loop (that would keep every row block's operands live)
            auto opq = [](float x) { asm volatile("" : "+v"(x)); return x; };
            const int row = 16 * I + m;
            const float bi = sBeta[row];
            float Gl[8], kk[8], qq[8], pf[8], kl[8];
            K.get8p(I, kk);
            Q.get8p(I, qq);
            // key of the reading side (row operands of A_kk): k, or eb * k
            if constexpr (EW) {
                Eb.get8p(I, kl);
#pragma unroll
                for (int e = 0; e < 8; ++e) kl[e] *= kk[e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) kl[e] = kk[e];
            }
            ce8(Ip, pf);                                  // cumulative value before block I
            const float gI0 = SG ? opq(G[8 * I]) : 0.f;   // the row's gate (scalar gate)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                Gl[e] = SG ? gI0 : opq(G[8 * I + e]);
                if (I == 0) pf[e] = 0.f;
            }
            // (a) chunk-start / chunk-end references: Qd and Kd^T to the workspace
            {
                Frag Kd;
                float qdv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float Gc = pf[e] + Gl[e];
                    const float ec = fast_exp2(Gc), ed = fast_exp2(gtot[e] - Gc);
                    qdv[e] = scale * qq[e] * ec;
                    Kd.set(e, kk[e] * ed);
                }
                Pol::pairn_store_vals(blk + Ly::QD + (I * Ly::NP + (wave >> 1)) * Ly::PN, lane,
                                     wave & 1, qdv);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    if (32 * wave + 16 * hh < DK) {
                        floatx4 dk = {0.f, 0.f, 0.f, 0.f};
                        Pol::mma_exact(dk, Kd, Eid[hh]);  // lane (channel n, grp): tokens 4 grp + r
                        const int ct = 2 * wave + hh, ks = I >> 1;
                        Pol::pairn_store_quad(blk + Ly::KDT + ct * Ly::PN,
                                             m + 16 * (2 * (I & 1) + (grp >> 1)), ks, grp & 1,
                                             dk[0], dk[1], dk[2], dk[3]);
                    }
                }
            }
            // row operands with the block-start reference, exp(G_i - G_r) <= 1 (r = end of
            // block I - 1): shared by the diagonal and the off-diagonal blocks of row I
            Frag KA, QA;
            bool far = false;                             // block decays beyond 2^120
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ea = fast_exp2(Gl[e]);
                KA.set(e, bi * kl[e] * ea);
                QA.set(e, scale * qq[e] * ea);
                far |= Gl[e] < -120.f;
            }
            // (b) diagonal block: block-start reference (column factor exp(G_r - G_j) <= 2^120),
            //     else the midpoint of the block, else pairwise
            {
                floatx4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
                bool bad = false;
                if (!__any(far)) {
                    Frag KC;
#pragma unroll
                    for (int e = 0; e < 8; ++e) KC.set(e, kk[e] * fast_exp2(-Gl[e]));
                    Pol::mma(akk, KC, KA);
                    Pol::mma(aqk, KC, QA);
                } else {
                    Frag KE, QE, KR;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float x = Gl[e] - row_bcast<7>(Gl[e]);
                        bad |= fabsf(x) > 120.f;
                        const float e1 = fast_exp2(x), e2 = fast_exp2(-x);
                        KE.set(e, bi * kl[e] * e1);
                        QE.set(e, scale * qq[e] * e1);
                        KR.set(e, kk[e] * e2);
                    }
                    if (!__any(bad)) {
                        Pol::mma(akk, KR, KE);
                        Pol::mma(aqk, KR, QE);
                    }
                }
                if (__any(bad)) {
                    // exact pairwise sums over this slice: entry (i = m, j = jj)
#pragma unroll 1
                    for (int jj = 0; jj < 16; ++jj) {
                        float skk = 0.f, sqk = 0.f;
                        const int src = (lane & 48) | jj;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float Gj = __shfl(Gl[e], src);
                            const float kj = __shfl(kk[e], src);
                            const float d = jj <= m ? fast_exp2(Gl[e] - Gj) : 0.f;
                            skk += kl[e] * kj * d;
                            sqk += scale * qq[e] * kj * d;
                        }
                        skk += __shfl_xor(skk, 16);
                        skk += __shfl_xor(skk, 32);
                        sqk += __shfl_xor(sqk, 16);
                        sqk += __shfl_xor(sqk, 32);
                        if ((jj >> 2) == grp) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (r == (jj & 3)) { akk[r] = bi * skk; aqk[r] = sqk; }
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 4 * grp + r;
                    if (!(j < m)) akk[r] = 0.f;
                    if (!(j <= m)) aqk[r] = 0.f;
                }
                float4* pk = reinterpret_cast<float4*>(&sKK[tri_tile(I, I)][m][4 * grp]);
                float4* pq = reinterpret_cast<float4*>(&sQK[tri_tile(I, I)][m][4 * grp]);
                float4 a = make_float4(0.f, 0.f, 0.f, 0.f), c = a;
                if (!first) {
                    a = *pk;
                    c = *pq;
                }
                a.x += akk[0]; a.y += akk[1]; a.z += akk[2]; a.w += akk[3];
                c.x += aqk[0]; c.y += aqk[1]; c.z += aqk[2]; c.w += aqk[3];
                *pk = a;
                *pq = c;
            }
            // (c) off-diagonal blocks J < I: reference at the end of block I - 1. The pair
            //     (3, 0) is taken by the wave holding row block 0 in this step (that wave has
            //     no other off-diagonal pair), which balances the steps; every pair still gets
            //     one partial per wave and no two waves write one block in the same step.
            // partial of pair (II, J) with row operands KA, QA of block II (pfI = cumulative
            // value before block II)
            auto offdiag = [&](int II, int J, const Frag& KA2, const Frag& QA2, const float* pfI) {
                // k of block J decayed to the start of block II
                const int Jp = J > 0 ? J - 1 : 0;
                float kJ[8], ceJ[8];
                K.get8p(J, kJ);
                ce8(Jp, ceJ);
                Frag b;
                const float gJ0 = SG ? opq(G[8 * J]) : 0.f;  // the row's gate (scalar gate)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float cj = J > 0 ? ceJ[e] : 0.f;
                    b.set(e, kJ[e] * fast_exp2(pfI[e] - cj - (SG ? gJ0 : opq(G[8 * J + e]))));
                }
                floatx4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
                Pol::mma(akk, b, KA2);
                Pol::mma(aqk, b, QA2);
                float4* pk = reinterpret_cast<float4*>(&sKK[tri_tile(II, J)][m][4 * grp]);
                float4* pq = reinterpret_cast<float4*>(&sQK[tri_tile(II, J)][m][4 * grp]);
                float4 a = make_float4(0.f, 0.f, 0.f, 0.f), c = a;
                if (!first) {
                    a = *pk;
                    c = *pq;
                }
                a.x += akk[0]; a.y += akk[1]; a.z += akk[2]; a.w += akk[3];
                c.x += aqk[0]; c.y += aqk[1]; c.z += aqk[2]; c.w += aqk[3];
                *pk = a;
                *pq = c;
            };
            if constexpr (I > 0) {
#pragma unroll
                for (int J = I == 3 ? 1 : 0; J < I; ++J) offdiag(I, J, KA, QA, pf);
            } else {
                // row block 3 of this slice (static registers)
                float k3[8], q3[8], pf3[8];
                K.get8p(3, k3);
                Q.get8p(3, q3);
                if constexpr (EW) {
                    float e3[8];
                    Eb.get8p(3, e3);
#pragma unroll
                    for (int e = 0; e < 8; ++e) k3[e] *= e3[e];
                }
                ce8(2, pf3);
                const float b3 = sBeta[48 + m];
                Frag KA3, QA3;
                const float g30 = SG ? opq(G[24]) : 0.f;    // the row's gate (scalar gate)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float ea = fast_exp2(SG ? g30 : opq(G[24 + e]));
                    KA3.set(e, b3 * k3[e] * ea);
                    QA3.set(e, scale * q3[e] * ea);
                }
                offdiag(3, 0, KA3, QA3, pf3);
            }
        };
#pragma unroll 1
        for (int st = 0; st < 4; ++st) {
            if (cs) {
                switch ((wave + st) & 3) {                    // wave-uniform
                    case 0: row_step(std::integral_constant<int, 0>{}, st); break;
                    case 1: row_step(std::integral_constant<int, 1>{}, st); break;
                    case 2: row_step(std::integral_constant<int, 2>{}, st); break;
                    default: row_step(std::integral_constant<int, 3>{}, st); break;
                }
            }
            __syncthreads();
        }

        // ---- value slice of this wave (for U), loaded now so it lands during the inverse ----
        const int vc0 = 32 * wave + 8 * grp;
        const bool vvalid = wave < NVS && vc0 < DV;
        In32<TI> V, Wr;
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const int row = 16 * I + m;
            if (vvalid && row < L) {
                V.load(I, v + (size_t)(t0 + row) * rowv + (size_t)h * DV + vc0);
                if constexpr (EW) Wr.load(I, ew + (size_t)(t0 + row) * rowv + (size_t)h * DV + vc0);
            } else {
                V.zero(I);
                if constexpr (EW) Wr.zero(I);
            }
        }
        // A_qk fragment tiles of token tile tw = wave (upper blocks zero; the columns 32..63
        // of token tiles 0 and 1, all zero, are not stored: the state pass does not read them)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (s == 1 && wave < 2) continue;                 // wave-uniform
            const int J = 2 * s + (grp >> 1), jl = 8 * (grp & 1);
            float a[8];
            if (J <= wave) {
                const float4 x0 = *reinterpret_cast<const float4*>(&sQK[tri_tile(wave, J)][m][jl]);
                const float4 x1 = *reinterpret_cast<const float4*>(&sQK[tri_tile(wave, J)][m][jl + 4]);
                a[0] = x0.x; a[1] = x0.y; a[2] = x0.z; a[3] = x0.w;
                a[4] = x1.x; a[5] = x1.y; a[6] = x1.z; a[7] = x1.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = 0.f;
            }
            Pol::pair_store_vals(blk + Ly::AQ + wave * Ly::PT, lane, s, a);
        }

        // ---- T = (I + A_kk)^-1: diagonal blocks by forward substitution (fp32). Wave I solves
        //      block (I, I) with all 64 lanes: lane 4 j + q carries column j, and the dot
        //      product of row i is split over the quad (lane q takes columns 4q .. 4q + 3 of A's
        //      row, whose entries on and above the diagonal are zero) and summed with two quad
        //      permutes, so a row costs four FMAs and two adds on the serial path ----
        {
            const int I = wave, j = lane >> 2, q = lane & 3;
            const float* arow = &sKK[tri_tile(I, I)][0][4 * q];
            float xs[4] = {0.f, 0.f, 0.f, 0.f};               // x[4 q + e], the quad's share
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float4 a = *reinterpret_cast<const float4*>(arow + 20 * i);
                float p = a.x * xs[0];
                p = fmaf(a.y, xs[1], p);
                p = fmaf(a.z, xs[2], p);
                p = fmaf(a.w, xs[3], p);
                p += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, p), 0xb1, 0xf, 0xf, false));
                p += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, p), 0x4e, 0xf, 0xf, false));
                const float xi = (i == j) ? 1.f : (i > j ? -p : 0.f);
                if (q == (i >> 2)) xs[i & 3] = xi;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[tri_tile(I, I)][4 * q + e][j] = xs[e];
        }
        __syncthreads();
        // off-diagonal blocks, column block J = wave: T_IJ = -T_II sum_{M=J}^{I-1} A_IM T_MJ
        {
            const int J = wave;
#pragma unroll 1
            for (int I = J + 1; I < 4; ++I) {
                floatx4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
                for (int M = J; M < I; ++M) {
                    const float4 a = *reinterpret_cast<const float4*>(&sKK[tri_tile(I, M)][m][4 * grp]);
                    const float* tb = &sT[tri_tile(M, J)][4 * grp][m];
                    mma16_f32(Y, a, make_float4(tb[0], tb[20], tb[40], tb[60]));
                }
                // (T_II Y)^T = Y^T T_II^T: A = Y in its C layout, B = T_II read by rows
                const float4 d = *reinterpret_cast<const float4*>(&sT[tri_tile(I, I)][m][4 * grp]);
                floatx4 R = {0.f, 0.f, 0.f, 0.f};
                mma16_f32(R, make_float4(Y[0], Y[1], Y[2], Y[3]), d);
                *reinterpret_cast<float4*>(&sT[tri_tile(I, J)][m][4 * grp]) =
                    make_float4(-R[0], -R[1], -R[2], -R[3]);
            }
        }
        __syncthreads();
        // ---- T' = T diag(beta) as operand fragments in LDS, converted once: lane (m, grp) of
        //      tile (I, J) holds T'[16I + m][16J + 4grp + r] ----
        for (int tile = wave; tile < 10; tile += 4) {
            const int I = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int J = tile - I * (I + 1) / 2;
            const float4 t = *reinterpret_cast<const float4*>(&sT[tile][m][4 * grp]);
            const float4 bb = *reinterpret_cast<const float4*>(&sBeta[16 * J + 4 * grp]);
            Frag4 f;
            f.set(0, t.x * bb.x); f.set(1, t.y * bb.y); f.set(2, t.z * bb.z); f.set(3, t.w * bb.w);
            sTp[tile][lane] = f;
        }
        __syncthreads();
        // A_kk, A_qk and T are consumed (T' is in sTp): the next task's g, k, beta and q are
        // staged into their regions, one row block before each block of W below. Issued after
        // the last barrier of the task (a barrier waits for every load into LDS in flight) and
        // spread out, because the issue of a load stalls while the memory system holds too
        // many of them
        bool stage_next = false;
        int t0n = 0, Ln = 0, hn = 0;
        if constexpr (Stg::kBytes > 0) {
            const int nt = task + (int)gridDim.x;
            if (nt < ntasks) {
                chunk_of(nt / H, t0n, Ln);
                hn = nt % H;
                stage_next = Ln > 0;
            }
        }
        staged = stage_next;

        // ---- W = T' (k exp G): W^T(channel half, I) = sum_{J <= I} (k exp G)_J^T T'_IJ^T; the
        //      result lane (m = token, grp) holds W[16 I + m][4 channels]. The operand of block
        //      J is built once and transposed for both 16-channel halves ----
        if (cs) {
            constexpr int NH = DK >= 32 ? 2 : 1;              // channel halves with data
            floatx4 accW[2][4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int I = 0; I < 4; ++I) accW[hh][I] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                if (stage_next) stage(t0n, Ln, hn, J);
                float kJ[8], ceJ[8];
                K.get8(J, kJ);
                if constexpr (EW) {
                    float eJ[8];
                    Eb.get8(J, eJ);
#pragma unroll
                    for (int e = 0; e < 8; ++e) kJ[e] *= eJ[e];
                }
                ce8(J > 0 ? J - 1 : 0, ceJ);
                Frag kg;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float cj = J > 0 ? ceJ[e] : 0.f;
                    kg.set(e, kJ[e] * fast_exp2(cj + G[8 * J + e]));
                }
#pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                    // lane (channel n, grp): tokens 4 grp + r
                    const Frag4 a = Pol::transpose4(kg, Eid[hh]);
#pragma unroll
                    for (int I = J; I < 4; ++I) Pol::mma16(accW[hh][I], a, sTp[tri_tile(I, J)][lane]);
                }
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int I = 0; I < 4; ++I)
                    Pol::pairn_store_quad(blk + Ly::W + (I * Ly::NP + (wave >> 1)) * Ly::PN,
                                         m + 16 * (2 * hh + (grp >> 1)), wave & 1, grp & 1,
                                         accW[hh][I][0], accW[hh][I][1], accW[hh][I][2], accW[hh][I][3]);
        }
        // ---- U = T' v: lane (m = value, grp) of tile (value tile, I) holds U[16 I + 4 grp + r][value] ----
        if (wave < NVS) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                if (32 * wave + 16 * hh < DV) {
                    floatx4 accU[4];
#pragma unroll
                    for (int I = 0; I < 4; ++I) accU[I] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int J = 0; J < 4; ++J) {
                        Frag vb;
                        floatx4 t = {0.f, 0.f, 0.f, 0.f};
                        if constexpr (EW) {
                            // ew v (a product of two inputs: exact in fp32, not in one bf16)
                            float vv[8], wv[8];
                            V.get8(J, vv);
                            Wr.get8(J, wv);
#pragma unroll
                            for (int e = 0; e < 8; ++e) vb.set(e, vv[e] * wv[e]);
                            Pol::mma_exact(t, vb, Eid[hh]);
                        } else {
                            V.frag(J, vb);
                            Pol::mma_copy(t, vb, Eid[hh]);    // lane (value n, grp): tokens 4 grp + r
                        }
                        const Frag4 b = frag4_of<Pol>(t);
                        // v is exact in the input type, ew v is not: it needs the full product
#pragma unroll
                        for (int I = J; I < 4; ++I) {
                            if constexpr (EW)
                                Pol::mma16(accU[I], sTp[tri_tile(I, J)][lane], b);
                            else
                                Pol::mma16_exact(accU[I], sTp[tri_tile(I, J)][lane], b);
                        }
                    }
#pragma unroll
                    for (int I = 0; I < 4; ++I)
                        Pol::utile_store(blk + Ly::U + ((2 * wave + hh) * 4 + I) * Ly::QT, lane,
                                         accU[I][0], accU[I][1], accU[I][2], accU[I][3]);
                }
            }
        }
        // this wave's staged loads have landed before it reads them in the next task
        if (staged) wait_all_memory();
    }
}

// ------------------------------------------------------------------------------------------
// state kernel
// ------------------------------------------------------------------------------------------
// One workgroup of 12 waves per (sequence, head, 32-column value tile), in three roles of
// four waves. Each chunk runs in two phases separated by workgroup barriers:
//   phase A (S_c published): E role (token tile w)  E = U - W S_c      -> LDS
//                            O role (token tile w)  Qd S_c             (registers)
//   phase B (E published):   S role (channel tiles) S_{c+1} = Diag(exp G_end) S_c + Kd^T E
//                                                   -> LDS operand copy, fp32 in registers
//                            O role                 O = Qd S_c + A_qk E, write o
// so the serial chain of a chunk is one product per phase, and every role decodes the next
// chunk's operands and issues later chunks' loads while it is off the chain. The S role
// keeps S in fp32 MFMA accumulators for the whole sequence. All reads of S_c and E happen
// in the phase before they are overwritten, so one LDS copy of each suffices. Every product
// is oriented so that the MFMA result tile has tokens or channels along its rows (4
// consecutive elements per lane); O is formed transposed so that a lane writes 4
// consecutive values of one token.

template <typename TI, typename TO, int DK, int DV, int BV>
__global__ __launch_bounds__(768) void state_kernel(
    const int32_t* __restrict__ cu, int T, const int32_t* __restrict__ seq_off,
    const uint8_t* __restrict__ ws, const float* h0, float* ht,   // ht may equal h0
    TO* __restrict__ o, int N, int H) {
    using Pol = typename PolOf<TI>::type;
    using Frag = typename Pol::Frag;
    using Pair = typename Pol::Pair;
    using St = typename Pol::Store;
    using Sh = StateShape<DK, DV, BV>;
    using Ly = WsLayoutOf<Pol, DK, DV>;
    constexpr int KS = Sh::KS, NP = Sh::NP, NVT = Sh::NVT, NCT = Sh::NCT, CTW = Sh::CTW;
    constexpr int P = Pol::kPlanes;
    __shared__ St SLs[P][BV][Sh::SST];     // operand copy of S [value][channel]
    __shared__ St ELs[P][BV][Sh::EST];     // E [value][token]
    __shared__ float4 sGd[DK / 4];         // exp(G_end) of the chunk in phase B
    St* const SL = &SLs[0][0][0];
    St* const EL = &ELs[0][0][0];
    constexpr size_t psS = (size_t)BV * Sh::SST, psE = (size_t)BV * Sh::EST;

    // blocks b, b+8, b+16, ... share an XCD: keep all value tiles of a chain on one XCD
    const int b = blockIdx.x;
    const int hc = (b / (8 * Sh::VT)) * 8 + (b % 8);
    const int vt = (b / 8) % Sh::VT;
    if (hc >= N * H) return;
    const int n = hc / H, h = hc % H;
    const int v0 = vt * BV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15, grp = lane >> 4;
    const int role = wave >> 2;                    // 0: E, 1: S, 2: O
    const int tw = wave & 3;                       // token tile (E, O) / S-role index
    const bool owns = role == 1 && (NCT >= 4 || tw < NCT);

    // zero the pad channels of the S copy once (only read when DK < 32)
    for (int idx = tid; idx < BV * (Sh::SST - DK); idx += 768) {
        const int r = idx / (Sh::SST - DK), c = DK + idx % (Sh::SST - DK);
        Pol::put(SL, (size_t)r * Sh::SST + c, psS, 0.f);
    }
    // S-role state tiles: channel tile ct = tw + 4 j, value tile vr; lane (n = value, grp)
    // holds S[16 ct + 4 grp + r][v0 + 16 vr + n]
    floatx4 S[CTW][NVT];
    const size_t sbase = ((size_t)n * H + h) * DK * DV;
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
#pragma unroll
        for (int vr = 0; vr < NVT; ++vr) {
            S[j][vr] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (owns) {
                const int c = 16 * (tw + 4 * j) + 4 * grp, vv = v0 + 16 * vr + m;
                if (h0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[j][vr][r] = h0[sbase + (size_t)(c + r) * DV + vv];
                }
                Pol::store4(SL, (size_t)(16 * vr + m) * Sh::SST + c, psS, S[j][vr][0],
                            S[j][vr][1], S[j][vr][2], S[j][vr][3]);
            }
        }
    }

    // The chunks of sequence n are the consecutive slots [c_beg, c_end); chunk c covers
    // tokens [s_beg + 64 (c - c_beg), min(+64, s_end)). No per-chunk table reads happen in
    // the loop (a scalar load there would share lgkmcnt with the LDS traffic). Prefetches
    // are unconditional (index clamped to the last chunk) so the loop has no branches
    // around loads.
    const int nck = (T + kChunk - 1) / kChunk;
    const int c_beg = seq_off ? seq_off[n] : n * nck, c_end = seq_off ? seq_off[n + 1] : (n + 1) * nck;
    // the same clamped bounds as the chunk map
    const int s_beg = cu ? min(max(cu[n], 0), T) : n * T;
    const int s_end = cu ? min(max(cu[n + 1], s_beg), T) : (n + 1) * T;
    const int last = c_end - 1;
    const size_t rowo = (size_t)H * DV;
    auto block = [&](int c) { return ws + ((size_t)c * H + h) * Ly::BYTES; };
    __syncthreads();                               // S copy initialised
    if (c_beg >= c_end) {
        // empty sequence: the state passes through
    } else if (role == 0) {
        // ---- E role: E = U - W S (phase A); loads and decodes W and U (phase B) ----
        __builtin_amdgcn_s_setprio(2);             // on the serial chain: issue before the O role
        struct Raw {
            typename Pol::PairN w[NP];
            typename Pol::URaw u[NVT];
        };
        Raw R0, R1;                                // raw operands of two later chunks
        Frag wd[KS];                               // decoded W of the current chunk
        float4 ud[NVT];
        auto issue = [&](Raw& r, int c) {
            const uint8_t* blk = block(c);
#pragma unroll
            for (int p = 0; p < NP; ++p)
                Pol::pairn_load(r.w[p], blk + Ly::W + (tw * NP + p) * Ly::PN, lane);
#pragma unroll
            for (int vr = 0; vr < NVT; ++vr)
                Pol::utile_load(r.u[vr], blk + Ly::U + ((v0 / 16 + vr) * 4 + tw) * Ly::QT, lane);
            issue_fence();
        };
        auto decode = [&](const Raw& r) {
            decode_pairs<Pol, KS, NP>(wd, r.w);
#pragma unroll
            for (int vr = 0; vr < NVT; ++vr) ud[vr] = Pol::utile_decode(r.u[vr]);
#pragma unroll
            for (int kap = 0; kap < KS; ++kap) wd[kap].pin_regs();
#pragma unroll
            for (int vr = 0; vr < NVT; ++vr) pin(ud[vr]);
        };
        // one chunk; `next` receives chunk c + 2's loads; `cur1` holds chunk c + 1's
        auto chunk = [&](int c, Raw& next, const Raw& cur1) {
            floatx4 acc[NVT];
#pragma unroll
            for (int vr = 0; vr < NVT; ++vr) acc[vr] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kap = 0; kap < KS; ++kap) {
#pragma unroll
                for (int vr = 0; vr < NVT; ++vr) {
                    Frag bS;
                    Pol::load(bS, SL, (size_t)(16 * vr + m) * Sh::SST + 32 * kap + 8 * grp, psS);
                    Pol::mma(acc[vr], wd[kap], bS);
                }
            }
            // lane (n = value, grp) holds E[tokens 16 tw + 4 grp + r][value]
#pragma unroll
            for (int vr = 0; vr < NVT; ++vr)
                Pol::store4(EL, (size_t)(16 * vr + m) * Sh::EST + 16 * tw + 4 * grp, psE,
                            ud[vr].x - acc[vr][0], ud[vr].y - acc[vr][1],
                            ud[vr].z - acc[vr][2], ud[vr].w - acc[vr][3]);
            __syncthreads();                       // phase B: E published
            issue(next, min(c + 2, last));
            decode(cur1);                          // chunk c + 1
            __syncthreads();                       // phase A: S_{c+1} published
        };
        issue(R0, c_beg);
        issue(R1, min(c_beg + 1, last));
        decode(R0);
        int c = c_beg;
#pragma unroll 1
        for (; c + 1 < c_end; c += 2) {
            chunk(c, R0, R1);
            chunk(c + 1, R1, R0);
        }
        if (c < c_end) chunk(c, R0, R1);
    } else if (role == 1) {
        __builtin_amdgcn_s_setprio(2);             // on the serial chain: issue before the O role
        // ---- S role: S' = Diag(exp G_end) S + Kd^T E. exp(G_end) (Dk floats) is fetched by
        //      the first S-role wave alone and shared through LDS ----
        struct Raw {
            typename Pol::PairN k[CTW];
            float2 g;                              // exp(G_end)[2 lane, 2 lane + 1] (wave 4)
        };
        Raw R0, R1;                                // raw operands of two later chunks
        Frag kd[CTW][2];                           // decoded Kd^T of the current chunk
        const bool gload = tw == 0 && 2 * lane < DK;
        auto issue = [&](Raw& r, int c) {
            if (owns) {
                const uint8_t* blk = block(c);
                const float* gGend = reinterpret_cast<const float*>(blk + Ly::GEND);
                if (tw == 0) r.g = reinterpret_cast<const float2*>(gGend)[gload ? lane : 0];
#pragma unroll
                for (int j = 0; j < CTW; ++j) {
                    const int ct = tw + 4 * j;
                    Pol::pairn_load(r.k[j], blk + Ly::KDT + ct * Ly::PN, lane);
                }
                issue_fence();
            }
        };
        // decodes the next chunk's Kd^T and publishes its exp(G_end) (read after the next
        // phase-B barrier; the current values were read before the last one)
        auto decode = [&](const Raw& r) {
            if (owns) {
#pragma unroll
                for (int j = 0; j < CTW; ++j) {
                    Pol::template pairn_decode<0>(kd[j][0], r.k[j]);
                    Pol::template pairn_decode<1>(kd[j][1], r.k[j]);
                    kd[j][0].pin_regs();
                    kd[j][1].pin_regs();
                }
                if (gload) reinterpret_cast<float2*>(&sGd[0])[lane] = r.g;
            }
        };
        auto chunk = [&](int c, Raw& next, const Raw& cur1) {
            __syncthreads();                       // phase B: E published
            if (owns) {
#pragma unroll
                for (int j = 0; j < CTW; ++j) {
                    const int cc = 16 * (tw + 4 * j) + 4 * grp;
                    const float4 gd = sGd[4 * (tw + 4 * j) + grp];
#pragma unroll
                    for (int vr = 0; vr < NVT; ++vr) {
                        S[j][vr][0] *= gd.x;
                        S[j][vr][1] *= gd.y;
                        S[j][vr][2] *= gd.z;
                        S[j][vr][3] *= gd.w;
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            Frag bE;
                            Pol::load(bE, EL, (size_t)(16 * vr + m) * Sh::EST + 32 * ks + 8 * grp, psE);
                            Pol::mma(S[j][vr], kd[j][ks], bE);
                        }
                        Pol::store4(SL, (size_t)(16 * vr + m) * Sh::SST + cc, psS, S[j][vr][0],
                                    S[j][vr][1], S[j][vr][2], S[j][vr][3]);
                    }
                }
            }
            __syncthreads();                       // phase A: S_{c+1} published
            issue(next, min(c + 2, last));
            decode(cur1);                          // chunk c + 1
        };
        issue(R0, c_beg);
        issue(R1, min(c_beg + 1, last));
        decode(R0);
        int c = c_beg;
#pragma unroll 1
        for (; c + 1 < c_end; c += 2) {
            chunk(c, R0, R1);
            chunk(c + 1, R1, R0);
        }
        if (c < c_end) chunk(c, R0, R1);
    } else {
        // ---- O role: O = Qd S_c (phase A, kept in registers) + A_qk E (phase B), then the
        //      output; lane (n = token, grp) holds values 16 vr + 4 grp + r ----
        struct Raw {
            typename Pol::PairN q[NP];
            Pair a;
        };
        Raw R0, R1;                                // raw Qd and A_qk of two later chunks
        Frag qd[KS];                               // decoded Qd, current chunk
        const int nks = tw < 2 ? 1 : 2;            // nonzero column halves of A_qk rows
        // Qd loads are issued in phase A (after Qd S), A_qk loads in phase B (after A_qk E),
        // which spreads the workgroup's load issue over both phases
        auto issue_q = [&](Raw& r, int c) {
            const uint8_t* blk = block(c);
#pragma unroll
            for (int p = 0; p < NP; ++p)
                Pol::pairn_load(r.q[p], blk + Ly::QD + (tw * NP + p) * Ly::PN, lane);
            issue_fence();
        };
        auto issue_a = [&](Raw& r, int c) {
            // token tiles 0 and 1 have no nonzero columns past 31: their second fragment is
            // neither stored nor read
            if (tw < 2) Pol::pair_load_a(r.a, block(c) + Ly::AQ + tw * Ly::PT, lane);
            else Pol::pair_load(r.a, block(c) + Ly::AQ + tw * Ly::PT, lane);
            issue_fence();
        };
        auto decode = [&](const Raw& r) {
            decode_pairs<Pol, KS, NP>(qd, r.q);
#pragma unroll
            for (int kap = 0; kap < KS; ++kap) qd[kap].pin_regs();
        };
        // one chunk; `next` holds this chunk's raw operands (its A_qk is still read) and
        // receives chunk c + 2's loads; `cur1` holds chunk c + 1's
        auto chunk = [&](int c, Raw& next, const Raw& cur1) {
            floatx4 acc[NVT];
#pragma unroll
            for (int vr = 0; vr < NVT; ++vr) acc[vr] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kap = 0; kap < KS; ++kap) {
#pragma unroll
                for (int vr = 0; vr < NVT; ++vr) {
                    Frag bS;
                    Pol::load(bS, SL, (size_t)(16 * vr + m) * Sh::SST + 32 * kap + 8 * grp, psS);
                    Pol::mma(acc[vr], bS, qd[kap]);
                }
            }
            issue_q(next, min(c + 2, last));       // this chunk's Qd is decoded and used
            __syncthreads();                       // phase B: E published
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if (s2 < nks) {
                    Frag aq;
                    if (s2) Pol::template pair_decode<1>(aq, next.a);
                    else Pol::template pair_decode<0>(aq, next.a);
#pragma unroll
                    for (int vr = 0; vr < NVT; ++vr) {
                        Frag bE;
                        Pol::load(bE, EL, (size_t)(16 * vr + m) * Sh::EST + 32 * s2 + 8 * grp, psE);
                        Pol::mma(acc[vr], bE, aq);
                    }
                }
            }
            const int t0 = s_beg + kChunk * (c - c_beg);
            const int len = s_end - t0 < kChunk ? s_end - t0 : kChunk;
            const int tok = 16 * tw + m;
            if (tok < len) {
                TO* orow = o + (size_t)(t0 + tok) * rowo + (size_t)h * DV + v0 + 4 * grp;
#pragma unroll
                for (int vr = 0; vr < NVT; ++vr)
                    store4(orow + 16 * vr, acc[vr][0], acc[vr][1], acc[vr][2], acc[vr][3]);
            }
            issue_a(next, min(c + 2, last));
            decode(cur1);                          // chunk c + 1
            __syncthreads();                       // phase A: S_{c+1} published
        };
        issue_q(R0, c_beg);
        issue_a(R0, c_beg);
        issue_q(R1, min(c_beg + 1, last));
        issue_a(R1, min(c_beg + 1, last));
        decode(R0);
        int c = c_beg;
#pragma unroll 1
        for (; c + 1 < c_end; c += 2) {
            chunk(c, R0, R1);
            chunk(c + 1, R1, R0);
        }
        if (c < c_end) chunk(c, R0, R1);
    }
    if (ht && owns) {
#pragma unroll
        for (int j = 0; j < CTW; ++j) {
#pragma unroll
            for (int vr = 0; vr < NVT; ++vr) {
                const int c = 16 * (tw + 4 * j) + 4 * grp, vv = v0 + 16 * vr + m;
#pragma unroll
                for (int r = 0; r < 4; ++r) ht[sbase + (size_t)(c + r) * DV + vv] = S[j][vr][r];
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------
hipError_t launch_chunk_map(const int32_t* cu, int N, int T, int max_slots, void* tab,
                            int32_t* seq_off, hipStream_t s) {
    hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, s, cu, N, T, max_slots,
                       (int4*)tab, seq_off);
    return hipGetLastError();
}

hipError_t launch_prep_fast(int mode, const void* q, const void* k, const void* v,
                            const void* gate, const void* beta, const void* eb, const void* ew,
                            float scale, const void* tab, int T, int nslots, uint8_t* blocks,
                            int H, long long beta_elems, int cu_count, hipStream_t s);

// compute units of the current device (the prep kernel keeps two workgroups on each)
static hipError_t current_cu_count(int& n) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64 && (n = cache[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n <= 0) return hipErrorInvalidDevice;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return hipSuccess;
}

template <typename TI, typename TO, int DK, int DV>
static hipError_t launch_prefill_t(bool sg, const void* q, const void* k, const void* v,
                                   const float* g, const void* beta, const void* eb,
                                   const void* ew, float scale, const float* h0, float* ht,
                                   void* o, const int32_t* cu, int T, const void* tab,
                                   const int32_t* seq_off, uint8_t* blocks, int N, int H,
                                   int max_slots, hipStream_t s) {
    int cu_count = 0;
    hipError_t ec = current_cu_count(cu_count);
    if (ec != hipSuccess) return ec;
    const long long ntasks = (long long)max_slots * H;
    // two resident workgroups per CU; one for the erase/write-gate variant, whose extra
    // operands need more than half of the register file
    const long long per_cu = eb ? 1 : 2;
    const long long grid = ntasks < per_cu * cu_count ? ntasks : per_cu * cu_count;
    const TI *tq = (const TI*)q, *tk = (const TI*)k, *tv = (const TI*)v, *tb = (const TI*)beta;
    const long long beta_elems = (cu ? (long long)T : (long long)N * T) * H;   // [tokens, H]
    constexpr bool kFastPrep = std::is_same<TI, bf16>::value && DK == 128 && DV == 128;
    if (kFastPrep && !sg)
        ec = launch_prep_fast(eb ? kPrepGates : kPrepPlain, q, k, v, g, beta, eb, ew, scale, tab,
                              T, max_slots, blocks, H, beta_elems, cu_count, s);
    else if (eb)
        hipLaunchKernelGGL((prep_kernel<TI, DK, DV, false, true>), dim3((unsigned)grid), dim3(256),
                           0, s, tq, tk, tv, g, tb, (const TI*)eb, (const TI*)ew, scale,
                           (const int4*)tab, T, max_slots, blocks, H, beta_elems);
    else if (sg)
        hipLaunchKernelGGL((prep_kernel<TI, DK, DV, true, false>), dim3((unsigned)grid), dim3(256),
                           0, s, tq, tk, tv, g, tb, nullptr, nullptr, scale, (const int4*)tab, T,
                           max_slots, blocks, H, beta_elems);
    else
        hipLaunchKernelGGL((prep_kernel<TI, DK, DV, false, false>), dim3((unsigned)grid),
                           dim3(256), 0, s, tq, tk, tv, g, tb, nullptr, nullptr, scale,
                           (const int4*)tab, T, max_slots, blocks, H, beta_elems);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = ec;
    if (e != hipSuccess) return e;
    constexpr int BV = DV >= 32 ? 32 : DV;
    constexpr int VT = DV / BV;
    const long long chains = (long long)N * H;
    const long long nblk = ((chains + 7) / 8) * 8 * VT;
    hipLaunchKernelGGL((state_kernel<TI, TO, DK, DV, BV>), dim3((unsigned)nblk), dim3(768), 0, s,
                       cu, T, seq_off, (const uint8_t*)blocks, h0, ht, (TO*)o, N, H);
    return hipGetLastError();
}

// Prefill from the raw projections (bf16, d_k = d_v = 128): the prep kernel normalises q and
// k and forms g = log sigmoid(a), beta = sigmoid(b) as it reads them; the state pass is the
// usual one.
hipError_t launch_prefill_raw(bool bf16_out, const void* q, const void* k, const void* v,
                              const void* a, const void* b, float scale, const float* h0,
                              float* ht, void* o, const int32_t* cu, int T, const void* tab,
                              const int32_t* seq_off, uint8_t* blocks, int N, int H,
                              int max_slots, hipStream_t s) {
    int cu_count = 0;
    hipError_t e = current_cu_count(cu_count);
    if (e != hipSuccess) return e;
    const long long beta_elems = (cu ? (long long)T : (long long)N * T) * H;
    e = launch_prep_fast(kPrepRaw, q, k, v, a, b, nullptr, nullptr, scale, tab, T, max_slots,
                         blocks, H, beta_elems, cu_count, s);
    if (e != hipSuccess) return e;
    const long long nblk = ((N * (long long)H + 7) / 8) * 8 * 4;
    if (bf16_out)
        hipLaunchKernelGGL((state_kernel<bf16, bf16, 128, 128, 32>), dim3((unsigned)nblk), dim3(768), 0,
                           s, cu, T, seq_off, (const uint8_t*)blocks, h0, ht, (bf16*)o, N, H);
    else
        hipLaunchKernelGGL((state_kernel<bf16, float, 128, 128, 32>), dim3((unsigned)nblk), dim3(768), 0,
                           s, cu, T, seq_off, (const uint8_t*)blocks, h0, ht, (float*)o, N, H);
    return hipGetLastError();
}

template <typename TI, typename TO>
static hipError_t dispatch_prefill(bool sg, int Dk, int Dv, const void* q, const void* k,
                                   const void* v, const float* g, const void* beta,
                                   const void* eb, const void* ew, float scale, const float* h0,
                                   float* ht, void* o, const int32_t* cu, int T, const void* tab,
                                   const int32_t* seq_off, uint8_t* blocks, int N, int H,
                                   int max_slots, hipStream_t s) {
#define KDA_PF(DKV, DVV)                                                                    \
    if (Dk == DKV && Dv == DVV)                                                             \
        return launch_prefill_t<TI, TO, DKV, DVV>(sg, q, k, v, g, beta, eb, ew, scale, h0, ht, \
                                                  o, cu, T, tab, seq_off, blocks, N, H,     \
                                                  max_slots, s);
    KDA_PF(16, 16) KDA_PF(16, 32) KDA_PF(16, 64) KDA_PF(16, 128)
    KDA_PF(32, 16) KDA_PF(32, 32) KDA_PF(32, 64) KDA_PF(32, 128)
    KDA_PF(64, 16) KDA_PF(64, 32) KDA_PF(64, 64) KDA_PF(64, 128)
    KDA_PF(128, 16) KDA_PF(128, 32) KDA_PF(128, 64) KDA_PF(128, 128)
#undef KDA_PF
    return hipErrorInvalidValue;
}

// sg: scalar gate; eb, ew: erase and write gates (non-null together) replacing beta
hipError_t launch_prefill(bool sg, bool bf16_in, bool bf16_out, int Dk, int Dv, const void* q,
                          const void* k, const void* v, const float* g, const void* beta,
                          const void* eb, const void* ew, float scale, const float* h0,
                          float* ht, void* o, const int32_t* cu, int T, const void* tab,
                          const int32_t* seq_off, uint8_t* blocks, int N, int H, int max_slots,
                          hipStream_t s) {
#define KDA_PF_ARGS sg, Dk, Dv, q, k, v, g, beta, eb, ew, scale, h0, ht, o, cu, T, tab, seq_off, \
                    blocks, N, H, max_slots, s
    if (bf16_in) {
        if (bf16_out) return dispatch_prefill<bf16, bf16>(KDA_PF_ARGS);
        return dispatch_prefill<bf16, float>(KDA_PF_ARGS);
    }
    if (bf16_out) return dispatch_prefill<float, bf16>(KDA_PF_ARGS);
    return dispatch_prefill<float, float>(KDA_PF_ARGS);
#undef KDA_PF_ARGS
}

}  // namespace kda
