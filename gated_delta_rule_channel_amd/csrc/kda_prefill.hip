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
//  * chunk_map_kernel:  cu_seqlens -> table of (token start, length, seq) per
//    chunk slot and the first slot of every sequence, on the device (the host
//    never reads cu_seqlens).
//  * prep_kernel: one workgroup per (chunk, head), fully parallel. Computes
//    everything that does not depend on S and writes it to the workspace:
//    W [64][Dk], Qd = scale q exp(G) [64][Dk], KdT = (k exp(G_end-G))^T
//    [Dk][64], U [64][Dv], A_qk [64][64] (operand precision) and exp(G_end)
//    [Dk] (fp32).
//  * state_kernel: one workgroup per (sequence, head, 32-column value tile),
//    the only serial pass; S stays in fp32 MFMA accumulators for the whole
//    sequence, with an operand-precision copy in LDS.
//
// Decay factors. Every exp(G_i - G_j) is formed as a product of two factors
// each bounded by 2^120 (in log2 units x = G log2 e), so nothing overflows or
// loses the range of float32/bfloat16:
//  * off-diagonal 16x16 blocks (row block I > column block J): exp(G_i - G_r)
//    with r the end of block I-1 (<= 1) times exp(G_r - G_j) (<= 1), the
//    latter split as exp(G_end(J) - G_j) * exp(G_r - G_end(J));
//  * diagonal 16x16 blocks: exp(G_i - G_m) * exp(G_m - G_j) with m the 8th
//    row of the block; if some |G_i - G_m| exceeds 120 (log2 units) in the
//    block, that block is computed pairwise instead (exp2 of each difference).
// The in-chunk prefix sums are computed per 16-token block (log-space prefix
// sums, as the page's "real Triton implementation" paragraph describes), and
// cross-block factors come from block totals.
#include "kda_common.h"

namespace kda {

// ------------------------------------------------------------------------------------------
// workspace layout (one block per (chunk slot, head); 4 bytes per operand element in both
// operand policies: fp32, or bf16 hi and lo planes)
// ------------------------------------------------------------------------------------------
__host__ __device__ constexpr size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

template <int DK, int DV>
struct WsLayout {
    static constexpr size_t W = 0;                        // [64][DK]   W
    static constexpr size_t QD = W + 64 * DK * 4;         // [64][DK]   scale q exp(G)
    static constexpr size_t KDT = QD + 64 * DK * 4;       // [DK][64]   (k exp(G_end - G))^T
    static constexpr size_t U = KDT + DK * 64 * 4;        // [64][DV]   U
    static constexpr size_t AQ = U + 64 * DV * 4;         // [64][64]   A_qk
    static constexpr size_t GEND = AQ + 64 * 64 * 4;      // float [DK] exp(G_end)
    static constexpr size_t BYTES = round_up(GEND + DK * sizeof(float), 256);
};

size_t prefill_block_bytes(int Dk, int Dv) {
    return round_up((size_t)4 * (64 * Dk * 3 + 64 * Dv + 64 * 64) + Dk * 4, 256);
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
            st = cu ? cu[n] : n * T;
            en = cu ? cu[n + 1] : (n + 1) * T;
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
template <int DK, int DV>
struct PrepShape {
    static constexpr int KS = DK >= 32 ? DK / 32 : 1;   // 32-wide channel slices (padded)
    static constexpr int DKP = KS * 32;
    static constexpr int GST = DKP + 4;                 // fp32 row stride of the prefix sums
    static constexpr int AST = 64 + 4;                  // fp32 row stride of A_kk and T
    static constexpr int KBST = DKP + 8;                // row stride of k exp(G_end(J) - G)
    static constexpr int TST = 64 + 8;                  // row stride of transposed operands
};

template <typename Pol, int DK, int DV>
struct PrepSmem {
    using Sh = PrepShape<DK, DV>;
    using St = typename Pol::Store;
    static constexpr int P = Pol::kPlanes;
    union {
        float G[64][Sh::GST];        // block-local prefix sums (log2 units); later T
        float T[64][Sh::AST];
    } g;
    float A[64][Sh::AST];            // A_kk (strictly lower, fp32)
    union {
        St KB[P][64][Sh::KBST];      // k exp(G_end(J) - G), per row block J
        St VbT[P][DV][Sh::TST];      // (beta v)^T
    } kv;
    St WopT[P][Sh::DKP][Sh::TST];    // (beta k exp(G))^T
    float lam[4][Sh::DKP];           // block totals
    float mid[4][Sh::DKP];           // prefix sum at the 8th row of each block
    float Pf[4][Sh::DKP];            // exp(G at the end of block I-1), chunk-start reference
    float Z[4][Sh::DKP];             // exp(G_end - G at the end of block I)
    float X[3][Sh::DKP];             // exp(G_r(I) - G_end(J)) for (I,J) = (2,0), (3,0), (3,1)
    float Y[4][16][17];              // per-wave scratch of the block inverse
    int bad[4];                      // diagonal block needs the pairwise path
};

// 16 x 16 x 16 fp32 product on LDS blocks, one wave: lane (r = l/4, cq = l%4) computes
// out[r][4cq .. 4cq+3] (+)= sign * sum_m X[r][m] Y[m][4cq ..].
__device__ __forceinline__ void blk16_mm(float* out, int ost, const float* X, int xst,
                                         const float* Y, int yst, float sign, bool accumulate) {
    const int lane = threadIdx.x & 63;
    const int r = lane >> 2, c0 = (lane & 3) * 4;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const float x = X[r * xst + m];
        const float* y = Y + m * yst + c0;
        a0 += x * y[0]; a1 += x * y[1]; a2 += x * y[2]; a3 += x * y[3];
    }
    float* o = out + r * ost + c0;
    if (accumulate) {
        o[0] += sign * a0; o[1] += sign * a1; o[2] += sign * a2; o[3] += sign * a3;
    } else {
        o[0] = sign * a0; o[1] = sign * a1; o[2] = sign * a2; o[3] = sign * a3;
    }
}

template <typename TI, int DK, int DV>
__global__ __launch_bounds__(256) void prep_kernel(
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v,
    const float* __restrict__ g, const TI* __restrict__ beta, float scale,
    const int4* __restrict__ tab, uint8_t* __restrict__ ws, int H) {
    using Pol = typename PolOf<TI>::type;
    using Frag = typename Pol::Frag;
    using St = typename Pol::Store;
    using Sh = PrepShape<DK, DV>;
    using Ly = WsLayout<DK, DV>;
    constexpr int KS = Sh::KS, DKP = Sh::DKP;
    __shared__ PrepSmem<Pol, DK, DV> sm;
    St* const sKB = &sm.kv.KB[0][0][0];
    St* const sVbT = &sm.kv.VbT[0][0][0];
    St* const sWopT = &sm.WopT[0][0][0];
    constexpr size_t psKB = (size_t)64 * Sh::KBST;
    constexpr size_t psVbT = (size_t)DV * Sh::TST;
    constexpr size_t psWopT = (size_t)DKP * Sh::TST;

    const int slot = blockIdx.x, h = blockIdx.y;
    const int4 ci = tab[slot];
    const int t0 = ci.x, L = ci.y;
    if (L <= 0) return;                                   // uniform per workgroup

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, grp = lane >> 4;
    const size_t rowq = (size_t)H * DK, rowv = (size_t)H * DV;
    uint8_t* blk = ws + ((size_t)slot * H + h) * Ly::BYTES;
    St* gW = reinterpret_cast<St*>(blk + Ly::W);
    St* gQd = reinterpret_cast<St*>(blk + Ly::QD);
    St* gKdT = reinterpret_cast<St*>(blk + Ly::KDT);
    St* gU = reinterpret_cast<St*>(blk + Ly::U);
    St* gAq = reinterpret_cast<St*>(blk + Ly::AQ);
    float* gGend = reinterpret_cast<float*>(blk + Ly::GEND);
    constexpr size_t psW = (size_t)64 * DK, psU = (size_t)64 * DV, psAq = 64 * 64;

    // ---- phase 1: block-local prefix sums of g (log2 units); wave = row block ----
    {
        const int I = wave;
        for (int c = lane; c < DKP; c += 64) {
            float run = 0.f;
#pragma unroll 4
            for (int r = 0; r < 16; ++r) {
                const int i = 16 * I + r;
                float x = 0.f;
                if (c < DK && i < L) x = g[(size_t)(t0 + i) * rowq + (size_t)h * DK + c] * kLog2e;
                run += x;
                sm.g.G[i][c] = run;
                if (r == 7) sm.mid[I][c] = run;
            }
            sm.lam[I][c] = run;
        }
        if (lane == 0) sm.bad[I] = 0;
    }
    // v rows for U, loaded early into registers: thread -> (token row, 8 columns)
    constexpr int VCG = DV / 8;                                  // 8-column groups per row
    constexpr int VRPP = (256 / VCG) < 64 ? (256 / VCG) : 64;   // rows per pass
    constexpr int VPASS = 64 / VRPP;
    const bool vact = tid / VCG < VRPP;
    float vreg[VPASS][8];
    float vbeta[VPASS];
    {
        const int vc = (tid % VCG) * 8;
#pragma unroll
        for (int p = 0; p < VPASS; ++p) {
            const int i = tid / VCG + p * VRPP;
            if (vact && i < L) {
                load8f(vreg[p], v + (size_t)(t0 + i) * rowv + (size_t)h * DV + vc);
                vbeta[p] = to_f(beta[(size_t)(t0 + i) * H + h]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) vreg[p][e] = 0.f;
                vbeta[p] = 0.f;
            }
        }
    }
    __syncthreads();
    // ---- phase 1b: cross-block factors per channel ----
    for (int c = tid; c < DKP; c += 256) {
        const float l0 = sm.lam[0][c], l1 = sm.lam[1][c], l2 = sm.lam[2][c], l3 = sm.lam[3][c];
        sm.Pf[0][c] = 1.f;
        sm.Pf[1][c] = fast_exp2(l0);
        sm.Pf[2][c] = fast_exp2(l0 + l1);
        sm.Pf[3][c] = fast_exp2(l0 + l1 + l2);
        sm.Z[0][c] = fast_exp2(l1 + l2 + l3);
        sm.Z[1][c] = fast_exp2(l2 + l3);
        sm.Z[2][c] = fast_exp2(l3);
        sm.Z[3][c] = 1.f;
        sm.X[0][c] = fast_exp2(l1);          // (2,0)
        sm.X[1][c] = fast_exp2(l1 + l2);     // (3,0)
        sm.X[2][c] = fast_exp2(l2);          // (3,1)
        if (c < DK) gGend[c] = fast_exp2(l0 + l1 + l2 + l3);
    }
    __syncthreads();

    // ---- phase 2: decay factors and operands, MFMA fragment layout ----
    // wave = row block I, lane -> row i = 16 I + m, channels 32 kappa + 8 grp + e.
    // The diagonal block products are accumulated here, slice by slice.
    const int I = wave;
    const int i = 16 * I + m;
    const bool valid = i < L;
    const float bi = valid ? to_f(beta[(size_t)(t0 + i) * H + h]) : 0.f;
    Frag KA[KS], QA[KS];
    floatx4 dkk = {0.f, 0.f, 0.f, 0.f}, dqk = {0.f, 0.f, 0.f, 0.f};
    bool bad = false;
#pragma unroll
    for (int kap = 0; kap < KS; ++kap) {
        const int c0 = 32 * kap + 8 * grp;
        float kf[8], qf[8];
        if (valid && c0 < DK) {
            load8f(kf, k + (size_t)(t0 + i) * rowq + (size_t)h * DK + c0);
            load8f(qf, q + (size_t)(t0 + i) * rowq + (size_t)h * DK + c0);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) { kf[e] = 0.f; qf[e] = 0.f; }
        }
        Frag KE, QE, KR, qd;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = c0 + e;
            const float G = sm.g.G[i][c];
            const float x = G - sm.mid[I][c];
            bad |= fabsf(x) > 120.f;
            const float e1 = fast_exp2(x), e2 = fast_exp2(-x);
            const float ea = fast_exp2(G), eb = fast_exp2(sm.lam[I][c] - G);
            const float kk = kf[e], qq = scale * qf[e];
            KE.set(e, bi * kk * e1);
            QE.set(e, qq * e1);
            KR.set(e, kk * e2);
            const float ka = bi * kk * ea, qa = qq * ea, kb = kk * eb;
            KA[kap].set(e, ka);
            QA[kap].set(e, qa);
            const float p = sm.Pf[I][c];
            qd.set(e, qa * p);
            Pol::put(sKB, (size_t)i * Sh::KBST + c, psKB, kb);
            Pol::put(sWopT, (size_t)c * Sh::TST + i, psWopT, ka * p);
            if (c < DK) Pol::put(gKdT, (size_t)c * 64 + i, psW, kb * sm.Z[I][c]);
        }
        if (c0 < DK) Pol::store(gQd, (size_t)i * DK + c0, psW, qd);
        // diagonal block: entry (row i, column j = 16 I + 4 grp + r) of the transposed product
        Pol::mma(dkk, KR, KE);
        Pol::mma(dqk, KR, QE);
    }
    if (__any(bad) && lane == 0) sm.bad[I] = 1;
    __syncthreads();

    // ---- phase 3: A_kk and A_qk blocks of row block I (transposed MFMA products) ----
    // acc[r] of the product (A = column-block operand, B = row-block operand) holds
    // the entry (row i = 16 I + m, column j = 16 J + 4 grp + r).
    {
        const bool pairwise = sm.bad[I] != 0;
        for (int J = 0; J <= I; ++J) {
            floatx4 akk = dkk, aqk = dqk;
            if (J < I) {
                akk = floatx4{0.f, 0.f, 0.f, 0.f};
                aqk = floatx4{0.f, 0.f, 0.f, 0.f};
                const int xi = (I == 2 && J == 0) ? 0 : (I == 3 && J == 0) ? 1 : 2;
                const bool scaled = J < I - 1;
                const int j = 16 * J + m;
#pragma unroll
                for (int kap = 0; kap < KS; ++kap) {
                    const int c0 = 32 * kap + 8 * grp;
                    Frag b;
                    if (scaled) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            b.set(e, Pol::get(sKB, (size_t)j * Sh::KBST + c0 + e, psKB) *
                                         sm.X[xi][c0 + e]);
                    } else {
                        Pol::load(b, sKB, (size_t)j * Sh::KBST + c0, psKB);
                    }
                    Pol::mma(akk, b, KA[kap]);
                    Pol::mma(aqk, b, QA[kap]);
                }
            }
            const int j0 = 16 * J + 4 * grp;
            float kv4[4], qv4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = j0 + r;
                kv4[r] = (j < i) ? akk[r] : 0.f;
                qv4[r] = (j <= i) ? aqk[r] : 0.f;
            }
            if (!(J == I && pairwise)) {
                *reinterpret_cast<float4*>(&sm.A[i][j0]) = make_float4(kv4[0], kv4[1], kv4[2], kv4[3]);
                Pol::store4(gAq, (size_t)i * 64 + j0, psAq, qv4[0], qv4[1], qv4[2], qv4[3]);
            }
        }
        // upper blocks are zero
        for (int J = I + 1; J < 4; ++J) {
            const int j0 = 16 * J + 4 * grp;
            Pol::store4(gAq, (size_t)i * 64 + j0, psAq, 0.f, 0.f, 0.f, 0.f);
            *reinterpret_cast<float4*>(&sm.A[i][j0]) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (pairwise) {
            // exact path for a diagonal block whose midpoint factors leave 2^+-120
            for (int idx = lane; idx < 256; idx += 64) {
                const int ii = idx >> 4, jj = idx & 15;
                const int ri = 16 * I + ii, rj = 16 * I + jj;
                float skk = 0.f, sqk = 0.f;
                if (jj <= ii && ri < L) {
                    const TI* ki = k + (size_t)(t0 + ri) * rowq + (size_t)h * DK;
                    const TI* qi = q + (size_t)(t0 + ri) * rowq + (size_t)h * DK;
                    const TI* kj = k + (size_t)(t0 + rj) * rowq + (size_t)h * DK;
                    for (int c = 0; c < DK; ++c) {
                        const float d = fast_exp2(sm.g.G[ri][c] - sm.g.G[rj][c]);
                        const float kjc = to_f(kj[c]) * d;
                        skk += to_f(ki[c]) * kjc;
                        sqk += to_f(qi[c]) * kjc;
                    }
                }
                const float bri = ri < L ? to_f(beta[(size_t)(t0 + ri) * H + h]) : 0.f;
                sm.A[ri][rj] = jj < ii ? bri * skk : 0.f;
                Pol::put(gAq, (size_t)ri * 64 + rj, psAq, jj <= ii ? scale * sqk : 0.f);
            }
        }
    }
    __syncthreads();

    // ---- phase 4: T = (I + A_kk)^-1, blocked; G is dead, its space holds T ----
    float (*Tm)[Sh::AST] = sm.g.T;
    {
        // diagonal 16x16 inverses by forward substitution, one column per lane
        if (lane < 16) {
            const int n = lane;
            float x[16];
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) {
                float s = 0.f;
#pragma unroll
                for (int mm = 0; mm < ii; ++mm) s += sm.A[16 * I + ii][16 * I + mm] * x[mm];
                x[ii] = (ii == n) ? 1.f : (ii > n ? -s : 0.f);
            }
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) Tm[16 * I + ii][16 * I + n] = x[ii];
        }
        // zero the strictly-upper blocks of row block I
        for (int idx = lane; idx < 16 * 64; idx += 64) {
            const int ii = idx >> 6, jj = idx & 63;
            if (jj >= 16 * (I + 1)) Tm[16 * I + ii][jj] = 0.f;
        }
    }
    __syncthreads();
    // level d: T[I][I-d] = -T[I][I] * sum_{M=I-d}^{I-1} A[I][M] T[M][I-d]
    for (int d = 1; d <= 3; ++d) {
        const bool act = I >= d;
        const int J = I - d;
        if (act) {
            for (int M = J; M < I; ++M)
                blk16_mm(&sm.Y[I][0][0], 17, &sm.A[16 * I][16 * M], Sh::AST, &Tm[16 * M][16 * J],
                         Sh::AST, 1.f, M != J);
        }
        __syncthreads();
        if (act)
            blk16_mm(&Tm[16 * I][16 * J], Sh::AST, &Tm[16 * I][16 * I], Sh::AST, &sm.Y[I][0][0], 17,
                     -1.f, false);
        __syncthreads();
    }

    // ---- phase 5: (beta v)^T into LDS (KB is dead), then W = T Wop and U = T (beta v) ----
    if (vact) {
        const int vc = (tid % VCG) * 8;
#pragma unroll
        for (int p = 0; p < VPASS; ++p) {
            const int ii = tid / VCG + p * VRPP;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                Pol::put(sVbT, (size_t)(vc + e) * Sh::TST + ii, psVbT, vbeta[p] * vreg[p][e]);
        }
    }
    __syncthreads();
    {
        // wave -> 16 output rows (tokens 16 wave ..); B operand = rows of T (K = tokens j)
        const int it = wave;
        const int nks = it < 2 ? 1 : 2;               // 32-token slices with nonzero T[i][j]
        const int row = 16 * it + m;
        Frag tb[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (s < nks) {
#pragma unroll
                for (int e = 0; e < 8; ++e) tb[s].set(e, Tm[row][32 * s + 8 * grp + e]);
            }
        }
        for (int ct = 0; ct < DK / 16; ++ct) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < nks; ++s) {
                Frag a;
                Pol::load(a, sWopT, (size_t)(16 * ct + m) * Sh::TST + 32 * s + 8 * grp, psWopT);
                Pol::mma(acc, a, tb[s]);
            }
            Pol::store4(gW, (size_t)row * DK + 16 * ct + 4 * grp, psW, acc[0], acc[1], acc[2],
                        acc[3]);
        }
        for (int ct = 0; ct < DV / 16; ++ct) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < nks; ++s) {
                Frag a;
                Pol::load(a, sVbT, (size_t)(16 * ct + m) * Sh::TST + 32 * s + 8 * grp, psVbT);
                Pol::mma(acc, a, tb[s]);
            }
            Pol::store4(gU, (size_t)row * DV + 16 * ct + 4 * grp, psU, acc[0], acc[1], acc[2],
                        acc[3]);
        }
    }
}

// ------------------------------------------------------------------------------------------
// state kernel
// ------------------------------------------------------------------------------------------
template <int DK, int DV, int BV>
struct StateShape {
    static constexpr int KS = DK >= 32 ? DK / 32 : 1;
    static constexpr int DKP = KS * 32;
    static constexpr int NVT = BV / 16;                 // value tiles of the workgroup
    static constexpr int NCT = DK / 16;                 // channel tiles of the state
    static constexpr int NST = NVT * NCT;               // state tiles
    static constexpr int MAXT = (NST + 3) / 4;          // state tiles per wave
    static constexpr int SST = DKP + 8;                 // row stride of the S^T copy
    static constexpr int EST = 64 + 8;                  // row stride of E^T
    static constexpr int VT = DV / BV;                  // value tiles per head
};

template <typename TI, typename TO, int DK, int DV, int BV>
__global__ __launch_bounds__(256) void state_kernel(
    const int4* __restrict__ tab, const int32_t* __restrict__ seq_off,
    const uint8_t* __restrict__ ws, const float* __restrict__ h0, float* __restrict__ ht,
    TO* __restrict__ o, int N, int H) {
    using Pol = typename PolOf<TI>::type;
    using Frag = typename Pol::Frag;
    using St = typename Pol::Store;
    using Sh = StateShape<DK, DV, BV>;
    using Ly = WsLayout<DK, DV>;
    constexpr int KS = Sh::KS, NVT = Sh::NVT, NCT = Sh::NCT, NST = Sh::NST, MAXT = Sh::MAXT;
    constexpr int P = Pol::kPlanes;
    __shared__ St SLs[P][BV][Sh::SST];     // operand copy of S^T [value][channel]
    __shared__ St ELs[P][BV][Sh::EST];     // E^T [value][token]
    St* const SL = &SLs[0][0][0];
    St* const EL = &ELs[0][0][0];
    constexpr size_t psS = (size_t)BV * Sh::SST, psE = (size_t)BV * Sh::EST;
    constexpr size_t psW = (size_t)64 * DK, psU = (size_t)64 * DV, psAq = 64 * 64;

    // blocks b, b+8, b+16, ... share an XCD: keep all value tiles of a chain on one XCD
    const int b = blockIdx.x;
    const int hc = (b / (8 * Sh::VT)) * 8 + (b % 8);
    const int vt = (b / 8) % Sh::VT;
    if (hc >= N * H) return;
    const int n = hc / H, h = hc % H;
    const int v0 = vt * BV;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m = lane & 15, grp = lane >> 4;

    // zero the pad channels of the S^T copy once (only read when DK < 32)
    for (int idx = tid; idx < BV * (Sh::SST - DK); idx += 256) {
        const int r = idx / (Sh::SST - DK), c = DK + idx % (Sh::SST - DK);
        Pol::put(SL, (size_t)r * Sh::SST + c, psS, 0.f);
    }
    // state tiles owned by this wave: s = wave + 4 t -> (value tile s / NCT, channel tile s % NCT)
    floatx4 S[MAXT];
    const size_t sbase = ((size_t)n * H + h) * DK * DV;
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
        const int s = wave + 4 * t;
        S[t] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (s < NST) {
            const int vr = s / NCT, ct = s % NCT;
            const int c = 16 * ct + m, vv = v0 + 16 * vr + 4 * grp;
            if (h0) {
                const float4 x = *reinterpret_cast<const float4*>(h0 + sbase + (size_t)c * DV + vv);
                S[t] = floatx4{x.x, x.y, x.z, x.w};
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Pol::put(SL, (size_t)(16 * vr + 4 * grp + r) * Sh::SST + c, psS, S[t][r]);
        }
    }
    __syncthreads();

    const int c_beg = seq_off[n], c_end = seq_off[n + 1];
    const size_t rowo = (size_t)H * DV;
    for (int cidx = c_beg; cidx < c_end; ++cidx) {
        const int4 ci = tab[cidx];
        const int t0 = ci.x, L = ci.y;
        const uint8_t* blk = ws + ((size_t)cidx * H + h) * Ly::BYTES;
        const St* gW = reinterpret_cast<const St*>(blk + Ly::W);
        const St* gQd = reinterpret_cast<const St*>(blk + Ly::QD);
        const St* gKdT = reinterpret_cast<const St*>(blk + Ly::KDT);
        const St* gU = reinterpret_cast<const St*>(blk + Ly::U);
        const St* gAq = reinterpret_cast<const St*>(blk + Ly::AQ);
        const float* gGend = reinterpret_cast<const float*>(blk + Ly::GEND);

        // E^T = U^T - S^T W^T and O^T = S^T Qd^T for token tile w = wave
        const int tok = 16 * wave + m;
        floatx4 accE[NVT], accO[NVT];
#pragma unroll
        for (int vr = 0; vr < NVT; ++vr) {
            accE[vr] = floatx4{0.f, 0.f, 0.f, 0.f};
            accO[vr] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kap = 0; kap < KS; ++kap) {
            const int c0 = 32 * kap + 8 * grp;
            Frag bw, bq;
            if (c0 < DK) {
                Pol::load(bw, gW, (size_t)tok * DK + c0, psW);
                Pol::load(bq, gQd, (size_t)tok * DK + c0, psW);
            } else {
                bw.zero();
                bq.zero();
            }
#pragma unroll
            for (int vr = 0; vr < NVT; ++vr) {
                Frag a;
                Pol::load(a, SL, (size_t)(16 * vr + m) * Sh::SST + c0, psS);
                Pol::mma(accE[vr], a, bw);
                Pol::mma(accO[vr], a, bq);
            }
        }
#pragma unroll
        for (int vr = 0; vr < NVT; ++vr) {
            const float4 u = Pol::load4f(gU, (size_t)tok * DV + v0 + 16 * vr + 4 * grp, psU);
            const float ur[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = ur[r] - accE[vr][r];
                Pol::put(EL, (size_t)(16 * vr + 4 * grp + r) * Sh::EST + tok, psE, e);
            }
        }
        __syncthreads();
        // O^T += E^T A_qk^T over the in-chunk tokens j <= tok
        {
            const int nks = wave < 2 ? 1 : 2;
            for (int s = 0; s < nks; ++s) {
                Frag bq;
                Pol::load(bq, gAq, (size_t)tok * 64 + 32 * s + 8 * grp, psAq);
#pragma unroll
                for (int vr = 0; vr < NVT; ++vr) {
                    Frag a;
                    Pol::load(a, EL, (size_t)(16 * vr + m) * Sh::EST + 32 * s + 8 * grp, psE);
                    Pol::mma(accO[vr], a, bq);
                }
            }
            if (tok < L) {
                TO* orow = o + (size_t)(t0 + tok) * rowo + (size_t)h * DV + v0;
#pragma unroll
                for (int vr = 0; vr < NVT; ++vr)
                    store4(orow + 16 * vr + 4 * grp, accO[vr][0], accO[vr][1], accO[vr][2],
                           accO[vr][3]);
            }
        }
        // S^T = S^T Diag(exp G_end) + E^T Kd
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            const int s = wave + 4 * t;
            if (s < NST) {
                const int vr = s / NCT, ct = s % NCT;
                const int c = 16 * ct + m;
                const float gd = gGend[c];
#pragma unroll
                for (int r = 0; r < 4; ++r) S[t][r] *= gd;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    Frag a, bk;
                    Pol::load(a, EL, (size_t)(16 * vr + m) * Sh::EST + 32 * ks + 8 * grp, psE);
                    Pol::load(bk, gKdT, (size_t)c * 64 + 32 * ks + 8 * grp, psW);
                    Pol::mma(S[t], a, bk);
                }
            }
        }
        __syncthreads();   // every wave is done reading SL and EL of this chunk
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            const int s = wave + 4 * t;
            if (s < NST) {
                const int vr = s / NCT, ct = s % NCT;
                const int c = 16 * ct + m;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Pol::put(SL, (size_t)(16 * vr + 4 * grp + r) * Sh::SST + c, psS, S[t][r]);
            }
        }
        __syncthreads();
    }
    if (ht) {
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            const int s = wave + 4 * t;
            if (s < NST) {
                const int vr = s / NCT, ct = s % NCT;
                const int c = 16 * ct + m, vv = v0 + 16 * vr + 4 * grp;
                *reinterpret_cast<float4*>(ht + sbase + (size_t)c * DV + vv) =
                    make_float4(S[t][0], S[t][1], S[t][2], S[t][3]);
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

template <typename TI, typename TO, int DK, int DV>
static hipError_t launch_prefill_t(const void* q, const void* k, const void* v, const float* g,
                                   const void* beta, float scale, const float* h0, float* ht,
                                   void* o, const void* tab, const int32_t* seq_off,
                                   uint8_t* blocks, int N, int H, int max_slots, hipStream_t s) {
    hipLaunchKernelGGL((prep_kernel<TI, DK, DV>), dim3(max_slots, H), dim3(256), 0, s,
                       (const TI*)q, (const TI*)k, (const TI*)v, g, (const TI*)beta, scale,
                       (const int4*)tab, blocks, H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int BV = DV >= 32 ? 32 : DV;
    constexpr int VT = DV / BV;
    const long long chains = (long long)N * H;
    const long long nblk = ((chains + 7) / 8) * 8 * VT;
    hipLaunchKernelGGL((state_kernel<TI, TO, DK, DV, BV>), dim3((unsigned)nblk), dim3(256), 0, s,
                       (const int4*)tab, seq_off, (const uint8_t*)blocks, h0, ht, (TO*)o, N, H);
    return hipGetLastError();
}

template <typename TI, typename TO>
static hipError_t dispatch_prefill(int Dk, int Dv, const void* q, const void* k, const void* v,
                                   const float* g, const void* beta, float scale,
                                   const float* h0, float* ht, void* o, const void* tab,
                                   const int32_t* seq_off, uint8_t* blocks, int N, int H,
                                   int max_slots, hipStream_t s) {
#define KDA_PF(DKV, DVV)                                                                    \
    if (Dk == DKV && Dv == DVV)                                                             \
        return launch_prefill_t<TI, TO, DKV, DVV>(q, k, v, g, beta, scale, h0, ht, o, tab,  \
                                                  seq_off, blocks, N, H, max_slots, s);
    KDA_PF(16, 16) KDA_PF(16, 32) KDA_PF(16, 64) KDA_PF(16, 128)
    KDA_PF(32, 16) KDA_PF(32, 32) KDA_PF(32, 64) KDA_PF(32, 128)
    KDA_PF(64, 16) KDA_PF(64, 32) KDA_PF(64, 64) KDA_PF(64, 128)
    KDA_PF(128, 16) KDA_PF(128, 32) KDA_PF(128, 64) KDA_PF(128, 128)
#undef KDA_PF
    return hipErrorInvalidValue;
}

hipError_t launch_prefill(bool bf16_in, bool bf16_out, int Dk, int Dv, const void* q,
                          const void* k, const void* v, const float* g, const void* beta,
                          float scale, const float* h0, float* ht, void* o, const void* tab,
                          const int32_t* seq_off, uint8_t* blocks, int N, int H, int max_slots,
                          hipStream_t s) {
    if (bf16_in) {
        if (bf16_out)
            return dispatch_prefill<bf16, bf16>(Dk, Dv, q, k, v, g, beta, scale, h0, ht, o, tab,
                                                seq_off, blocks, N, H, max_slots, s);
        return dispatch_prefill<bf16, float>(Dk, Dv, q, k, v, g, beta, scale, h0, ht, o, tab,
                                             seq_off, blocks, N, H, max_slots, s);
    }
    if (bf16_out)
        return dispatch_prefill<float, bf16>(Dk, Dv, q, k, v, g, beta, scale, h0, ht, o, tab,
                                             seq_off, blocks, N, H, max_slots, s);
    return dispatch_prefill<float, float>(Dk, Dv, q, k, v, g, beta, scale, h0, ht, o, tab,
                                          seq_off, blocks, N, H, max_slots, s);
}

}  // namespace kda
