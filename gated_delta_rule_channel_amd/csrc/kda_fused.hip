// Chunk-parallel preparation of the KDA prefill with factored decay, for bfloat16 input at
// d_k = d_v = 128.
//
// Computes, per (chunk, head), the same workspace block as the general prep kernel (W, Qd,
// Kd^T, U, A_qk and exp(G_end), in the layouts and number formats that the state pass
// reads; see kda_prefill_shared.h) from the chunkwise form of "Kimi Delta Attention (KDA)"
// (brain.bigb.es), section "Two schedules for the same recurrence":
//
//   A_kk[i][j] = beta_i sum_c k_i[c] k_j[c] exp(G_i[c] - G_j[c])     j <  i
//   A_qk[i][j] = scale  sum_c q_i[c] k_j[c] exp(G_i[c] - G_j[c])     j <= i
//   T = (I + A_kk)^-1, T' = T diag(beta), W = T' (k exp G), U = T' v
//   Qd = scale q exp(G), Kd = k exp(G_end - G)
//
// What differs from the general kernel is how the decay factors are formed. Within a chunk
// the 64 tokens form four 16-token blocks; with g in log2 units, let Gl be the prefix sum
// inside a block (inclusive), bt the block's total and e_I = bt_0 + ... + bt_I the
// cumulative value at the end of block I. Every factor the chunk needs is a product of two
// per-element exponentials, formed once per element,
//
//   fr = exp2(Gl)        (row factor, reference at the block start, <= 1)
//   fc = exp2(bt - Gl)   (column factor, reference at the block end, <= 1)
//
// and per-channel factors shared by the 16 rows of a block, formed once per (block,
// channel) and kept in LDS:
//
//   P_r[I] = exp2(e_(I-1))       chunk start -> start of block I
//   P_e[I] = exp2(e_3 - e_I)     end of block I -> chunk end
//   bd[I] = exp2(bt_I), ibd[I] = exp2(-bt_I)
//
// so that, with Kr = beta k fr, Qr = scale q fr and Kc = k fc:
//   A block (I, J < I) = Kr_I (Kc_J * bd_(J+1) ... bd_(I-1))^T     (every factor <= 1)
//   A block (I, I)     = Kr_I (Kc_I * ibd_I)^T                       (<= 2^120, see below)
//   Qd = Qr * P_r, Kd = Kc * P_e, k exp(G) = k fr * P_r.
// The general kernel forms a separate exponential for each element of each block pair and
// each stored operand. A diagonal block whose decay exceeds 2^120 in some channel (ibd
// beyond 2^120) takes the same fallbacks as the general kernel: the block's 8th row as
// reference, else exact pairwise exponentials.
//
// Gated DeltaNet-2 ("From Fast Weight Programmers to KDA", section "Gated DeltaNet-2") runs
// through the same kernel: an erase gate b per key channel replaces beta on the reading
// side (the row operand of A_kk is b k fr and W's operand b k exp(G)), a write gate w per
// value channel scales v (U = T (w v)), and T' = T.
#include "kda_prefill_shared.h"

namespace kda {

namespace {

constexpr int FD = 128;                                  // d_k = d_v of this kernel
using FPol = PolSplit;
using FFrag = PolSplit::Frag;
using FFrag4 = PolSplit::Frag4;
using FLy = WsLayoutOf<PolSplit, FD, FD>;

__device__ __forceinline__ void ld8(float* o, const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// The next task's decay input of a lane, loaded while the current task finishes: g itself
// (float32, 32 values), or in raw mode the gate logits a (bfloat16, 32 values in 16 words)
template <bool RAW> struct GateBuf {
    float v[32];
    __device__ __forceinline__ void load(const void* p, size_t off, int st) {
        load8f(&v[8 * st], reinterpret_cast<const float*>(p) + off);
    }
    __device__ __forceinline__ void zero(int st) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * st + e] = 0.f;
    }
    __device__ __forceinline__ float log_decay(int i) const { return v[i]; }
};
template <> struct GateBuf<true> {
    u32x4 w[4];
    __device__ __forceinline__ void load(const void* p, size_t off, int st) {
        w[st] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16*>(p) + off);
    }
    // rows past the chunk's end: a = +inf, so that g = log sigmoid(a) = 0 (no decay) and the
    // chunk-end decay exp(G_end) counts only the chunk's tokens
    __device__ __forceinline__ void zero(int st) {
        w[st] = u32x4{0x7f807f80u, 0x7f807f80u, 0x7f807f80u, 0x7f807f80u};
    }
    // g = log sigmoid(a)
    __device__ __forceinline__ float log_decay(int i) const {
        const unsigned x = w[i >> 3][(i & 7) >> 1];
        return log_sigmoid(__uint_as_float((i & 1) ? (x & 0xffff0000u) : (x << 16)));
    }
};

}  // namespace

// Persistent workgroups of 4 waves, two per CU, over the (chunk, head) tasks with a stride of
// the grid (consecutive workgroups take the heads of one chunk).
//
// The A phase is token-sliced: wave I owns the 16 tokens of block I over all 128 channels,
// in MFMA fragment layout (lane (m, grp) holds token 16 I + m and, for each 32-channel step
// s, the channels 32 s + 8 grp + e), so every A block of row I is reduced over all channels
// inside wave I and written to LDS once. Column operands of the earlier blocks pass through
// LDS. W and U are channel-sliced (wave w: channels / values [32 w, 32 w + 32)), with the
// operand k exp(G) of every block handed over through LDS in transposed fragment layout.
// The next task's k and q are staged in LDS during the W phase (direct-to-LDS loads) and its
// g is loaded into registers while W and U run.
//
// MODE kPrepRaw: the inputs are the raw projections of the input-preparation entry point (q
// and k not normalised, gate logits a in place of g, write-strength logits b in place of
// beta), and the normalisation q^ = scale q / |q|, k^ = k / |k| (norm over the 128 channels
// of the row, which the four lanes of a row hold between them), g = log sigmoid(a) and
// beta = sigmoid(b) are applied as the inputs are read. MODE kPrepGates: Gated DeltaNet-2,
// with the erase gates eb [tokens, H, 128] and write gates ew [tokens, H, 128] in place of
// beta.
template <int MODE>
__global__ __launch_bounds__(256, 2) void prep_fast_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const void* __restrict__ gate, const bf16* __restrict__ beta, const bf16* __restrict__ eb,
    const bf16* __restrict__ ew, float scale, const int4* __restrict__ tab, int T, int nslots,
    uint8_t* __restrict__ ws, int H, long long beta_elems) {
    constexpr bool RAW = MODE == kPrepRaw, EW = MODE == kPrepGates;
    using Ly = FLy;
    // ---- LDS: one 64 KB region used in turn by the staged q, k (previous task), the A
    //      phase (A_kk, A_qk, factor table, column operands), T, and the W operand ----
    __shared__ __attribute__((aligned(16))) uint8_t sR[65536];
    constexpr int kStgQ = 0, kStgK = 16384;                     // [wave][step] 1 KB parts
    constexpr int kKK = 0, kQK = 12800;                         // [10][16][20] floats each
    constexpr int kFac = 25600;                                 // [4 kinds][4 blocks][128]
    constexpr int kKcStride = 136;                              // floats per row (544 B)
    constexpr int kKc = 33792;                                  // [3][16][136] floats
    constexpr int kT = 33792;                                   // [10][16][20] (after Kc)
    constexpr int kX = 32768;                                   // Frag4 [4][8][64]
    static_assert(kKc + 3 * 16 * kKcStride * 4 <= 65536, "column operands fit");
    static_assert(kX + 4 * 8 * 64 * 16 <= 65536, "W operand fits");
    float (*const sKK)[16][20] = reinterpret_cast<float (*)[16][20]>(sR + kKK);
    float (*const sQK)[16][20] = reinterpret_cast<float (*)[16][20]>(sR + kQK);
    float (*const sT)[16][20] = reinterpret_cast<float (*)[16][20]>(sR + kT);
    // P_r, P_e, ibd per block; the decay products of the pairs two or three blocks apart
    float (*const sFac)[4][FD] = reinterpret_cast<float (*)[4][FD]>(sR + kFac);
    float (*const sKc)[16][kKcStride] = reinterpret_cast<float (*)[16][kKcStride]>(sR + kKc);
    FFrag4 (*const sX)[8][64] = reinterpret_cast<FFrag4 (*)[8][64]>(sR + kX);
    __shared__ float sBeta[64];
    __shared__ unsigned sBetaRaw[64];
    __shared__ __attribute__((aligned(16))) float sBT[4][FD];  // block totals (log2)
    __shared__ FFrag4 sTp[10][64];                              // T' = T diag(beta)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15, grp = lane >> 4;
    const size_t rowq = (size_t)H * FD;
    const int ntasks = nslots * H;

    auto chunk_of = [&](int slot, int& t0, int& L) {
        if (tab) {
            const int4 ci = tab[slot];
            t0 = ci.x;
            L = ci.y;
        } else {
            const int nck = (T + kChunk - 1) / kChunk, row = slot / nck, c = slot % nck;
            t0 = row * T + kChunk * c;
            L = T - kChunk * c < kChunk ? T - kChunk * c : kChunk;
        }
    };
    // staged k and q of channel step s for this wave's rows (token 16 wave + m) of a task,
    // and beta with step 0
    auto stage = [&](int t0, int L, int h, int st) {
        const int row = 16 * wave + m;
        if (row < L) {
            const size_t off = (size_t)(t0 + row) * rowq + (size_t)h * FD + 32 * st + 8 * grp;
            lds_load16(k + off, sR + kStgK + (wave * 4 + st) * 1024);
            lds_load16(q + off, sR + kStgQ + (wave * 4 + st) * 1024);
        }
        if (!EW && st == 0 && wave == 0 && lane < L) {
            const size_t e = (size_t)(t0 + lane) * H + h;
            if ((e & 1) == 0 && (long long)e + 1 >= beta_elems)
                sBetaRaw[lane] = reinterpret_cast<const unsigned short*>(beta)[e];
            else
                lds_load4(reinterpret_cast<const unsigned*>(beta) + (e >> 1), sBetaRaw);
        }
    };
    // decay input of this wave's rows of a task (32 values a lane: steps s, channels
    // 32 s + 8 grp + e)
    auto load_g = [&](GateBuf<RAW>& G, int t0, int L, int h) {
        const int row = 16 * wave + m;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if (row < L)
                G.load(gate, (size_t)(t0 + row) * rowq + (size_t)h * FD + 32 * st + 8 * grp, st);
            else
                G.zero(st);
        }
    };
    FFrag Eid[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) Eid[hh].set(e, (8 * grp + e == 16 * hh + m) ? 1.f : 0.f);

    bool staged = false;
    GateBuf<RAW> Gn;                                            // decay input, next task
#pragma unroll 1
    for (int task = blockIdx.x; task < ntasks; task += gridDim.x) {
        const int slot = task / H, h = task % H;
        int t0, L;
        chunk_of(slot, t0, L);
        if (L <= 0) {
            staged = false;
            continue;
        }
        uint8_t* blk = ws + ((size_t)slot * H + h) * Ly::BYTES;
        const int I = wave;                                     // row block of this wave
        const int row = 16 * I + m;

        // ---- inputs: k, q (staged in LDS), g (registers), beta ----
        if (!staged) {
#pragma unroll
            for (int st = 0; st < 4; ++st) stage(t0, L, h, st);
            load_g(Gn, t0, L, h);
            wait_all_memory();
        }
        float G[32];
        In32<bf16> K, Q;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if (row < L) {
                K.set(st, reinterpret_cast<const u32x4*>(sR + kStgK + (wave * 4 + st) * 1024)[lane]);
                Q.set(st, reinterpret_cast<const u32x4*>(sR + kStgQ + (wave * 4 + st) * 1024)[lane]);
            } else {
                K.zero(st);
                Q.zero(st);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) G[8 * st + e] = Gn.log_decay(8 * st + e) * kLog2e;
        }
        if (tid < 64) {
            const size_t e = (size_t)(t0 + tid) * H + h;
            const unsigned w = EW ? 0u : sBetaRaw[tid];
            const float bv = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
            sBeta[tid] = tid < L ? (EW ? 1.f : RAW ? sigmoid(bv) : bv) : 0.f;
        }
        // erase gates of this lane's row and channels (Gated DeltaNet-2)
        In32<bf16> Eb;
        if constexpr (EW) {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                if (row < L)
                    Eb.load(st, eb + (size_t)(t0 + row) * rowq + (size_t)h * FD + 32 * st + 8 * grp);
                else
                    Eb.zero(st);
            }
        }
        // row scales: k^ = rk k, scale q^ = rq q (raw mode: the norms over the row's 128
        // channels, held by the four lanes m, m + 16, m + 32, m + 48; a zero row stays zero)
        float rk = 1.f, rq = scale;
        if constexpr (RAW) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                float kf[8], qf[8];
                K.get8(st, kf);
                Q.get8(st, qf);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sk += kf[e] * kf[e];
                    sq += qf[e] * qf[e];
                }
            }
            sk += __shfl_xor(sk, 16);
            sk += __shfl_xor(sk, 32);
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
            rk = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;
            rq = sq > 0.f ? scale / sqrtf(sq) : 0.f;
        }
        __syncthreads();                                        // staging region free

        // ---- prefix sums inside the block (DPP row scans over the 16 tokens) and block
        //      totals (log2 units) ----
        row_scan16_step<0x111>(G);
        row_scan16_step<0x112>(G);
        row_scan16_step<0x114>(G);
        row_scan16_step<0x118>(G);
        // (the broadcast from lane 15 runs on every lane; only lane 0 of each row stores it)
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float bt = row_bcast<15>(G[i]);
            if (m == 0) sBT[I][32 * (i >> 3) + 8 * grp + (i & 7)] = bt;
        }
        __syncthreads();                                        // block totals in LDS
        // per-(block, channel) factors: e_I = bt_0 + ... + bt_I; P_r = exp2(e_(I-1)),
        // P_e = exp2(e_3 - e_I), ibd = exp2(-bt_I); exp(G_end) to the workspace block
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int ent = tid + 256 * r, I2 = ent >> 7, c = ent & (FD - 1);
            float ep = 0.f, e3 = 0.f, bt = 0.f;
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                const float b = sBT[J][c];
                if (J < I2) ep += b;
                if (J == I2) bt = b;
                e3 += b;
            }
            const float eI = ep + bt;
            sFac[0][I2][c] = fast_exp2(ep);
            sFac[1][I2][c] = fast_exp2(e3 - eI);
            sFac[2][I2][c] = fast_exp2(-bt);
            // decay between the column and the row block of the pairs two or three blocks
            // apart: entry 1: bd_1 (pair (2, 0)), 2: bd_2 (pair (3, 1)), 3: bd_1 bd_2 (pair (3, 0))
            const float b1 = sBT[1][c], b2 = sBT[2][c];
            sFac[3][I2][c] = fast_exp2(I2 == 1 ? b1 : I2 == 2 ? b2 : b1 + b2);
            if (I2 == 3) reinterpret_cast<float*>(blk + Ly::GEND)[c] = fast_exp2(e3);
        }
        __syncthreads();                                        // factor table complete

        // ---- loop A over the 32-channel steps: k fc (reference at the block end) of blocks
        //      0..2 to LDS for the later rows, and Kd^T = (k fc P_e)^T to the workspace ----
        const float bi = sBeta[row];
        bool far = false;                                       // ibd beyond 2^120
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int c0 = 32 * st + 8 * grp;
            float kf[8], pe[8], ib[8], kc[8];
            K.get8(st, kf);
#pragma unroll
            for (int e = 0; e < 8; ++e) kf[e] *= rk;
            ld8(pe, &sFac[1][I][c0]);
            ld8(ib, &sFac[2][I][c0]);
            FFrag Kd;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = G[8 * st + e];
                kc[e] = kf[e] * fast_exp2(row_bcast<15>(x) - x);
                Kd.set(e, kc[e] * pe[e]);
                far |= ib[e] > 0x1p120f;
            }
            if (I < 3) {
                float4* dst = reinterpret_cast<float4*>(&sKc[I][m][c0]);
                dst[0] = make_float4(kc[0], kc[1], kc[2], kc[3]);
                dst[1] = make_float4(kc[4], kc[5], kc[6], kc[7]);
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                floatx4 dk = {0.f, 0.f, 0.f, 0.f};
                FPol::mma_exact(dk, Kd, Eid[hh]);              // lane (channel n, grp): tokens 4 grp + r
                FPol::pairn_store_quad(blk + Ly::KDT + (2 * st + hh) * Ly::PN,
                                       m + 16 * (2 * (I & 1) + (grp >> 1)), I >> 1, grp & 1,
                                       dk[0], dk[1], dk[2], dk[3]);
            }
        }
        const bool farw = __any(far);
        __syncthreads();                                        // column operands in LDS

        // ---- loop B: row operands Kr = beta k fr, Qr = scale q fr (reference at the block
        //      start), Qd = Qr P_r to the workspace, and every A block of row I at once: the
        //      diagonal with k fc ibd = k exp2(-Gl) (<= 2^120), block J < I with k fc of block J
        //      times the decay of the blocks between J and I (every factor <= 1) ----
        floatx4 akk[3], aqk[3];                                 // [J]: block (I, J), J < I
        floatx4 dkk = {0.f, 0.f, 0.f, 0.f}, dqk = {0.f, 0.f, 0.f, 0.f};   // block (I, I)
#pragma unroll
        for (int J = 0; J < 3; ++J) {
            akk[J] = floatx4{0.f, 0.f, 0.f, 0.f};
            aqk[J] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int c0 = 32 * st + 8 * grp;
            float kf[8], qf[8], pr[8], ib[8], qd[8], kc[8];
            K.get8(st, kf);
            Q.get8(st, qf);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kf[e] *= rk;
                qf[e] *= rq;
            }
            ld8(pr, &sFac[0][I][c0]);
            ld8(ib, &sFac[2][I][c0]);
            if (I < 3) {
                ld8(kc, &sKc[I][m][c0]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = G[8 * st + e];
                    kc[e] = kf[e] * fast_exp2(row_bcast<15>(x) - x);
                }
            }
            float br[8];                                        // beta, or the erase gates
            if constexpr (EW) {
                Eb.get8(st, br);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) br[e] = bi;
            }
            FFrag KR, QR, KD;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = fast_exp2(G[8 * st + e]);
                const float sq = qf[e] * f;
                KR.set(e, br[e] * kf[e] * f);
                QR.set(e, sq);
                qd[e] = sq * pr[e];
                KD.set(e, kc[e] * ib[e]);
            }
            FPol::pairn_store_vals(blk + Ly::QD + (I * Ly::NP + (st >> 1)) * Ly::PN, lane, st & 1, qd);
            if (!farw) {
                FPol::mma(dkk, KD, KR);
                FPol::mma(dqk, KD, QR);
            }
#pragma unroll
            for (int J = 0; J < 3; ++J) {
                if (J < I) {                                    // wave-uniform
                    float kj[8];
                    ld8(kj, &sKc[J][m][c0]);
                    if (I - J >= 2) {
                        float bv[8];
                        ld8(bv, &sFac[3][I == 2 ? 1 : J == 1 ? 2 : 3][c0]);
#pragma unroll
                        for (int e = 0; e < 8; ++e) kj[e] *= bv[e];
                    }
                    FFrag col;
#pragma unroll
                    for (int e = 0; e < 8; ++e) col.set(e, kj[e]);
                    FPol::mma(akk[J], col, KR);
                    FPol::mma(aqk[J], col, QR);
                }
            }
        }

        // ---- a diagonal block decaying beyond 2^120 in some channel: the block's 8th row as
        //      reference, else exact pairwise exponentials. Rare, so its inputs are reloaded from
        //      global memory one channel step at a time (few registers) ----
        if (farw) {
            dkk = floatx4{0.f, 0.f, 0.f, 0.f};
            dqk = floatx4{0.f, 0.f, 0.f, 0.f};
            const bool rv = row < L;
            const size_t off = (size_t)(t0 + (rv ? row : 0)) * rowq + (size_t)h * FD + 8 * grp;
            auto gl8 = [&](int st, float (&x)[8]) {           // prefix sums inside the block
                if (rv) {
                    GateBuf<RAW> gb;
                    gb.load(gate, off + 32 * st, 0);
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = gb.log_decay(e) * kLog2e;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = 0.f;
                }
                row_scan8(x);
            };
            // k, q, and the reading-side key br k (beta k, or the erase gates times k)
            auto kq8 = [&](int st, float (&kf)[8], float (&qf)[8], float (&kb)[8]) {
                if (rv) {
                    load8f(kf, k + off + 32 * st);
                    load8f(qf, q + off + 32 * st);
                    if constexpr (EW) load8f(kb, eb + off + 32 * st);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        kf[e] *= rk;
                        qf[e] *= rq;
                        kb[e] = (EW ? kb[e] : bi) * kf[e];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) kb[e] = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) { kf[e] = 0.f; qf[e] = 0.f; }
                }
            };
            // the 8th-row reference, formed while testing that no channel decays by more than
            // 2^120 over half a block; if one does, its (possibly overflowed) sums are dropped.
            // The next channel step's inputs are loaded (raw) while a step is formed.
            auto far_load = [&](int st, GateBuf<RAW>& gr, u32x4& kr, u32x4& qr, u32x4& er) {
                if (rv) {
                    gr.load(gate, off + 32 * st, 0);
                    kr = *reinterpret_cast<const u32x4*>(k + off + 32 * st);
                    qr = *reinterpret_cast<const u32x4*>(q + off + 32 * st);
                    if constexpr (EW) er = *reinterpret_cast<const u32x4*>(eb + off + 32 * st);
                } else {
                    gr.zero(0);                             // g = 0 on rows past the end
                    kr = u32x4{0u, 0u, 0u, 0u};
                    qr = kr;
                    er = kr;
                }
            };
            auto widen8 = [](const u32x4& w, float (&f)[8]) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    f[2 * p] = __uint_as_float(w[p] << 16);
                    f[2 * p + 1] = __uint_as_float(w[p] & 0xffff0000u);
                }
            };
            bool bad = false;
            GateBuf<RAW> gn;
            u32x4 kn, qn, en;
            far_load(0, gn, kn, qn, en);
#pragma unroll 1
            for (int st = 0; st < 4; ++st) {
                const GateBuf<RAW> gc = gn;
                const u32x4 kc4 = kn, qc4 = qn, ec4 = en;
                if (st < 3) far_load(st + 1, gn, kn, qn, en);
                float x[8], kf[8], qf[8], kb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = gc.log_decay(e) * kLog2e;
                row_scan8(x);
                widen8(kc4, kf);
                widen8(qc4, qf);
                if constexpr (EW) widen8(ec4, kb);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    kf[e] *= rk;
                    qf[e] *= rq;
                    kb[e] = (EW ? kb[e] : bi) * kf[e];
                }
                FFrag KE, QE, KX;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float d = x[e] - row_bcast<7>(x[e]);
                    bad |= fabsf(d) > 120.f;
                    const float e1 = fast_exp2(d), e2 = fast_exp2(-d);
                    KE.set(e, kb[e] * e1);
                    QE.set(e, qf[e] * e1);
                    KX.set(e, kf[e] * e2);
                }
                FPol::mma(dkk, KX, KE);
                FPol::mma(dqk, KX, QE);
            }
            if (__any(bad)) {
                dkk = floatx4{0.f, 0.f, 0.f, 0.f};
                dqk = floatx4{0.f, 0.f, 0.f, 0.f};
                // entry (i = m, j = jj): sums over the channel steps, then over the quarter-rows
#pragma unroll 1
                for (int jj = 0; jj < 16; ++jj) {
                    float skk = 0.f, sqk = 0.f;
                    const int src = (lane & 48) | jj;
#pragma unroll 1
                    for (int st = 0; st < 4; ++st) {
                        float x[8], kf[8], qf[8], kb[8];
                        gl8(st, x);
                        kq8(st, kf, qf, kb);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float Gj = __shfl(x[e], src);
                            const float kj = __shfl(kf[e], src);
                            const float d = jj <= m ? fast_exp2(x[e] - Gj) : 0.f;
                            skk += kb[e] * kj * d;
                            sqk += qf[e] * kj * d;
                        }
                    }
                    skk += __shfl_xor(skk, 16);
                    skk += __shfl_xor(skk, 32);
                    sqk += __shfl_xor(sqk, 16);
                    sqk += __shfl_xor(sqk, 32);
                    if ((jj >> 2) == grp) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (r == (jj & 3)) { dkk[r] = skk; dqk[r] = sqk; }
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 4 * grp + r;
            if (!(j < m)) dkk[r] = 0.f;
            if (!(j <= m)) dqk[r] = 0.f;
        }
        *reinterpret_cast<float4*>(&sKK[tri_tile(I, I)][m][4 * grp]) = make_float4(dkk[0], dkk[1], dkk[2], dkk[3]);
        *reinterpret_cast<float4*>(&sQK[tri_tile(I, I)][m][4 * grp]) = make_float4(dqk[0], dqk[1], dqk[2], dqk[3]);
#pragma unroll
        for (int J = 0; J < 3; ++J) {
            if (J < I) {
                *reinterpret_cast<float4*>(&sKK[tri_tile(I, J)][m][4 * grp]) =
                    make_float4(akk[J][0], akk[J][1], akk[J][2], akk[J][3]);
                *reinterpret_cast<float4*>(&sQK[tri_tile(I, J)][m][4 * grp]) =
                    make_float4(aqk[J][0], aqk[J][1], aqk[J][2], aqk[J][3]);
            }
        }
        __syncthreads();                                        // A_kk, A_qk complete

        // ---- value slice of this wave (for U), loaded now so it lands during the inverse ----
        const int vc0 = 32 * wave + 8 * grp;
        In32<bf16> V, Wg;                                       // v, and the write gates
#pragma unroll
        for (int I2 = 0; I2 < 4; ++I2) {
            if (16 * I2 + m < L) {
                V.load(I2, v + (size_t)(t0 + 16 * I2 + m) * rowq + (size_t)h * FD + vc0);
                if constexpr (EW) Wg.load(I2, ew + (size_t)(t0 + 16 * I2 + m) * rowq + (size_t)h * FD + vc0);
            } else {
                V.zero(I2);
                if constexpr (EW) Wg.zero(I2);
            }
        }
        // A_qk fragment tiles of token tile tw = wave (upper blocks zero; the columns 32..63
        // of token tiles 0 and 1, all zero, are not stored: the state pass does not read them)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            if (s2 == 1 && wave < 2) continue;                // wave-uniform
            const int J = 2 * s2 + (grp >> 1), jl = 8 * (grp & 1);
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
            FPol::pair_store_vals(blk + Ly::AQ + wave * Ly::PT, lane, s2, a);
        }

        // ---- T = (I + A_kk)^-1: diagonal blocks by forward substitution on all 64 lanes
        //      (lane 4 j + q carries column j; the row's dot product is split over the quad),
        //      off-diagonal blocks T_IJ = -T_II sum_M A_IM T_MJ by fp32 MFMA ----
        {
            const int j = lane >> 2, qd = lane & 3;
            const float* arow = &sKK[tri_tile(I, I)][0][4 * qd];
            float xs[4] = {0.f, 0.f, 0.f, 0.f};
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
                if (qd == (i >> 2)) xs[i & 3] = xi;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[tri_tile(I, I)][4 * qd + e][j] = xs[e];
        }
        __syncthreads();
        {
            const int J = wave;
#pragma unroll 1
            for (int I2 = J + 1; I2 < 4; ++I2) {
                floatx4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
                for (int M = J; M < I2; ++M) {
                    const float4 a = *reinterpret_cast<const float4*>(&sKK[tri_tile(I2, M)][m][4 * grp]);
                    const float* tb = &sT[tri_tile(M, J)][4 * grp][m];
                    mma16_f32(Y, a, make_float4(tb[0], tb[20], tb[40], tb[60]));
                }
                const float4 d = *reinterpret_cast<const float4*>(&sT[tri_tile(I2, I2)][m][4 * grp]);
                floatx4 R = {0.f, 0.f, 0.f, 0.f};
                mma16_f32(R, make_float4(Y[0], Y[1], Y[2], Y[3]), d);
                *reinterpret_cast<float4*>(&sT[tri_tile(I2, J)][m][4 * grp]) =
                    make_float4(-R[0], -R[1], -R[2], -R[3]);
            }
        }
        __syncthreads();
        for (int tile = wave; tile < 10; tile += 4) {
            const int I2 = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int J = tile - I2 * (I2 + 1) / 2;
            const float4 t = *reinterpret_cast<const float4*>(&sT[tile][m][4 * grp]);
            const float4 bb = *reinterpret_cast<const float4*>(&sBeta[16 * J + 4 * grp]);
            FFrag4 f;
            f.set(0, t.x * bb.x); f.set(1, t.y * bb.y); f.set(2, t.z * bb.z); f.set(3, t.w * bb.w);
            sTp[tile][lane] = f;
        }
        __syncthreads();                                        // T read: its region is free
        // ---- W's operand of block I, k exp(G) = k fr P_r, transposed to fragments of 16
        //      channels (lane (n = channel, grp): tokens 4 grp + r), to LDS ----
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            float pr[8], kf[8];
            ld8(pr, &sFac[0][I][32 * st + 8 * grp]);
            K.get8(st, kf);
            FFrag xg;
#pragma unroll
            for (int e = 0; e < 8; ++e) kf[e] *= rk;
            if constexpr (EW) {
                float ebv[8];
                Eb.get8(st, ebv);
#pragma unroll
                for (int e = 0; e < 8; ++e) kf[e] *= ebv[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) xg.set(e, kf[e] * fast_exp2(G[8 * st + e]) * pr[e]);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) sX[I][2 * st + hh][lane] = FPol::transpose4(xg, Eid[hh]);
        }
        __syncthreads();                                        // T' and W's operand in LDS

        // the next task: its k, q are staged into the free start of the region during W, its
        // g loaded into registers
        bool stage_next = false;
        int t0n = 0, Ln = 0, hn = 0;
        {
            const int nt = task + (int)gridDim.x;
            if (nt < ntasks) {
                chunk_of(nt / H, t0n, Ln);
                hn = nt % H;
                stage_next = Ln > 0;
            }
        }
        staged = stage_next;
        // (defined on both paths, so the previous task's values are dead during the A phase)
        if (stage_next) {
            load_g(Gn, t0n, Ln, hn);
        } else {
#pragma unroll
            for (int st = 0; st < 4; ++st) Gn.zero(st);
        }

        // ---- W = T' (k exp G) for this wave's 32 channels: the result lane (m = token, grp)
        //      holds W[16 I + m][4 channels] ----
        {
            floatx4 accW[2][4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int I2 = 0; I2 < 4; ++I2) accW[hh][I2] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                if (stage_next) stage(t0n, Ln, hn, J);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const FFrag4 a = sX[J][2 * wave + hh][lane];
#pragma unroll
                    for (int I2 = J; I2 < 4; ++I2) FPol::mma16(accW[hh][I2], a, sTp[tri_tile(I2, J)][lane]);
                }
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int I2 = 0; I2 < 4; ++I2)
                    FPol::pairn_store_quad(blk + Ly::W + (I2 * Ly::NP + (wave >> 1)) * Ly::PN,
                                           m + 16 * (2 * hh + (grp >> 1)), wave & 1, grp & 1,
                                           accW[hh][I2][0], accW[hh][I2][1], accW[hh][I2][2], accW[hh][I2][3]);
        }
        // ---- U = T' v: lane (m = value, grp) of tile (value tile, I) holds U[16 I + 4 grp + r][value] ----
        if constexpr (EW) {
            // U = T (w v): w v is not exact in one bfloat16, so the transpose and the product
            // take both parts; it is formed once per token block for both value halves
            floatx4 accU[2][4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int I2 = 0; I2 < 4; ++I2) accU[hh][I2] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                float vv[8], wv[8];
                V.get8(J, vv);
                Wg.get8(J, wv);
                FFrag vb;
#pragma unroll
                for (int e = 0; e < 8; ++e) vb.set(e, vv[e] * wv[e]);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    floatx4 t = {0.f, 0.f, 0.f, 0.f};
                    FPol::mma_exact(t, vb, Eid[hh]);
                    const FFrag4 b = frag4_of<FPol>(t);
#pragma unroll
                    for (int I2 = J; I2 < 4; ++I2) FPol::mma16(accU[hh][I2], sTp[tri_tile(I2, J)][lane], b);
                }
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int I2 = 0; I2 < 4; ++I2)
                    FPol::utile_store(blk + Ly::U + ((2 * wave + hh) * 4 + I2) * Ly::QT, lane,
                                      accU[hh][I2][0], accU[hh][I2][1], accU[hh][I2][2], accU[hh][I2][3]);
        } else {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                floatx4 accU[4];
#pragma unroll
                for (int I2 = 0; I2 < 4; ++I2) accU[I2] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int J = 0; J < 4; ++J) {
                    FFrag vb;
                    floatx4 t = {0.f, 0.f, 0.f, 0.f};
                    V.frag(J, vb);
                    FPol::mma_copy(t, vb, Eid[hh]);         // v is exact in one bfloat16
                    const FFrag4 b = frag4_of<FPol>(t);
#pragma unroll
                    for (int I2 = J; I2 < 4; ++I2) FPol::mma16_exact(accU[I2], sTp[tri_tile(I2, J)][lane], b);
                }
#pragma unroll
                for (int I2 = 0; I2 < 4; ++I2)
                    FPol::utile_store(blk + Ly::U + ((2 * wave + hh) * 4 + I2) * Ly::QT, lane,
                                      accU[I2][0], accU[I2][1], accU[I2][2], accU[I2][3]);
            }
        }
        if (staged) wait_all_memory();
    }
}

// Launches the prep kernel above over nslots x H tasks (the workspace blocks start at
// `blocks`); two workgroups per CU. kPrepRaw: gate holds the logits a (bf16) and beta the
// logits b, and q, k are normalised in the kernel; otherwise gate is g (float32).
// kPrepGates: eb and ew hold the erase and write gates, beta is unused.
hipError_t launch_prep_fast(int mode, const void* q, const void* k, const void* v,
                            const void* gate, const void* beta, const void* eb, const void* ew,
                            float scale, const void* tab, int T, int nslots, uint8_t* blocks,
                            int H, long long beta_elems, int cu_count, hipStream_t s) {
    const long long ntasks = (long long)nslots * H;
    const long long grid = ntasks < 2LL * cu_count ? ntasks : 2LL * cu_count;
#define KDA_PREP_FAST(M)                                                                     \
    hipLaunchKernelGGL(prep_fast_kernel<M>, dim3((unsigned)grid), dim3(256), 0, s,            \
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, gate, (const bf16*)beta, \
                       (const bf16*)eb, (const bf16*)ew, scale, (const int4*)tab, T, nslots, \
                       blocks, H, beta_elems)
    if (mode == kPrepRaw)
        KDA_PREP_FAST(kPrepRaw);
    else if (mode == kPrepGates)
        KDA_PREP_FAST(kPrepGates);
    else
        KDA_PREP_FAST(kPrepPlain);
#undef KDA_PREP_FAST
    return hipGetLastError();
}

}  // namespace kda
