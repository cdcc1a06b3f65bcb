/*
 * Float64 CPU oracle of the KDA forward recurrence (plain C + OpenMP).
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library; the KDA
 * library never does, and the two share no source.
 *
 * It computes the recurrence token by token in double precision, one
 * (sequence, head) pair per OpenMP task, with the five steps of
 * "Module 03 - KDA I: The Delta-Rule Recurrence" (jared-hpc.com), section 2,
 * and the beta-scaled error of "Kimi Delta Attention (KDA)" (brain.bigb.es):
 *
 *   (1) S~ = Diag(exp(g_t)) S      decay each key channel (row of S)
 *   (2) v^ = S~^T k_t              prediction
 *   (3) e  = beta_t (v_t - v^)     scaled error
 *   (4) S  = S~ + k_t e^T          rank-one write
 *   (5) o_t = S^T (scale q_t)      read of the updated state
 *
 * Inputs are float arrays holding exactly the values the GPU receives (a
 * bfloat16 value is exact in float); every operation is done in double.
 * Layouts: q, k, g [Ttot, H, Dk]; v [Ttot, H, Dv]; beta [Ttot, H];
 * states [N, H, Dk, Dv] with row = key channel.
 *
 * With a scalar gate (Gated DeltaNet: "Notes on Linear Attention",
 * zhilingong.com, section 6) g is [Ttot, H] and step (1) scales every row of
 * S by the same exp(g_t); the other steps are unchanged.
 *
 * With erase and write gates (Gated DeltaNet-2: "From Fast Weight Programmers
 * to KDA", section "Gated DeltaNet-2") beta is replaced by b [Ttot, H, Dk] and
 * w [Ttot, H, Dv]: (2) predicts through the gated key, v^ = S~^T (b_t * k_t),
 * and (3) becomes e = w_t * v_t - v^.
 *
 * Parity pins: the Python test-suite checks this file against the numpy
 * oracle (same definition, written independently) on the small workloads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int kda_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* threads of the following calls (timing only; results do not depend on it) */
void kda_oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* One (sequence, head) chain over tokens [t0, t1). S is Dk*Dv doubles,
 * updated in place; o gets the outputs of the chain's tokens. */
static void chain(const float* q, const float* k, const float* v, const float* g,
                  int scalar_gate, const float* beta, const float* eb, const float* ew,
                  double scale, int H, int Dk, int Dv, int h,
                  int64_t t0, int64_t t1, double* S, double* o,
                  double* vhat, double* err, double* dec) {
    for (int64_t t = t0; t < t1; ++t) {
        const float* qt = q + (t * H + h) * (int64_t)Dk;
        const float* kt = k + (t * H + h) * (int64_t)Dk;
        const float* vt = v + (t * H + h) * (int64_t)Dv;
        const float* gt = g + (t * H + h) * (int64_t)(scalar_gate ? 1 : Dk);
        const double b = eb ? 0.0 : (double)beta[t * H + h];
        const float* bt = eb ? eb + (t * H + h) * (int64_t)Dk : NULL;
        const float* wt = ew ? ew + (t * H + h) * (int64_t)Dv : NULL;
        for (int c = 0; c < Dk; ++c) dec[c] = exp((double)gt[scalar_gate ? 0 : c]);
        /* (1) forget */
        for (int c = 0; c < Dk; ++c)
            for (int j = 0; j < Dv; ++j) S[c * Dv + j] *= dec[c];
        /* (2) predict: v^ = S~^T k */
        for (int j = 0; j < Dv; ++j) vhat[j] = 0.0;
        for (int c = 0; c < Dk; ++c) {
            const double kc = (double)kt[c] * (bt ? (double)bt[c] : 1.0);
            for (int j = 0; j < Dv; ++j) vhat[j] += S[c * Dv + j] * kc;
        }
        /* (3) correct */
        if (bt)
            for (int j = 0; j < Dv; ++j) err[j] = (double)wt[j] * (double)vt[j] - vhat[j];
        else
            for (int j = 0; j < Dv; ++j) err[j] = b * ((double)vt[j] - vhat[j]);
        /* (4) write */
        for (int c = 0; c < Dk; ++c) {
            const double kc = (double)kt[c];
            for (int j = 0; j < Dv; ++j) S[c * Dv + j] += kc * err[j];
        }
        /* (5) read: o = S^T (scale q) */
        double* ot = o + (t * H + h) * (int64_t)Dv;
        for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
        for (int c = 0; c < Dk; ++c) {
            const double qc = scale * (double)qt[c];
            for (int j = 0; j < Dv; ++j) ot[j] += S[c * Dv + j] * qc;
        }
    }
}

/* Prefill over packed sequences. cu_seqlens is int32[num_seqs + 1] with
 * cu[0] = 0 (fixed-length batches pass n*T). h0 may be NULL (zero state).
 * g is [Ttot, H, Dk], or [Ttot, H] when scalar_gate is non-zero.
 * o: double [Ttot, H, Dv]; ht: double [num_seqs, H, Dk, Dv] (may be NULL).
 * Returns 0, or -1 on allocation failure. */
static int prefill_impl(const float* q, const float* k, const float* v, const float* g,
                        int scalar_gate, const float* beta, const float* eb, const float* ew,
                        double scale, const float* h0, const int32_t* cu_seqlens, int num_seqs,
                        int H, int Dk, int Dv, double* o, double* ht) {
    int failed = 0;
    const int64_t pairs = (int64_t)num_seqs * H;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t p = 0; p < pairs; ++p) {
        const int n = (int)(p / H), h = (int)(p % H);
        double* S = (double*)malloc(sizeof(double) * ((size_t)Dk * Dv + 2 * (size_t)Dv + Dk));
        if (!S) { failed = 1; continue; }
        double* vhat = S + (size_t)Dk * Dv;
        double* err = vhat + Dv;
        double* dec = err + Dv;
        const float* h0p = h0 ? h0 + ((int64_t)n * H + h) * (int64_t)Dk * Dv : NULL;
        for (int64_t i = 0; i < (int64_t)Dk * Dv; ++i) S[i] = h0p ? (double)h0p[i] : 0.0;
        chain(q, k, v, g, scalar_gate, beta, eb, ew, scale, H, Dk, Dv, h, cu_seqlens[n],
              cu_seqlens[n + 1], S, o,
              vhat, err, dec);
        if (ht) memcpy(ht + ((int64_t)n * H + h) * (int64_t)Dk * Dv, S,
                       sizeof(double) * (size_t)Dk * Dv);
        free(S);
    }
    return failed ? -1 : 0;
}

int kda_oracle_prefill(const float* q, const float* k, const float* v, const float* g,
                       int scalar_gate, const float* beta, double scale, const float* h0,
                       const int32_t* cu_seqlens, int num_seqs, int H, int Dk, int Dv,
                       double* o, double* ht) {
    return prefill_impl(q, k, v, g, scalar_gate, beta, NULL, NULL, scale, h0, cu_seqlens,
                        num_seqs, H, Dk, Dv, o, ht);
}

/* Gated DeltaNet-2 prefill: g, b [Ttot, H, Dk]; w [Ttot, H, Dv]; the rest as
 * kda_oracle_prefill. */
int kda_oracle_gdn2_prefill(const float* q, const float* k, const float* v, const float* g,
                            const float* b, const float* w, double scale, const float* h0,
                            const int32_t* cu_seqlens, int num_seqs, int H, int Dk, int Dv,
                            double* o, double* ht) {
    return prefill_impl(q, k, v, g, 0, NULL, b, w, scale, h0, cu_seqlens, num_seqs, H, Dk, Dv,
                        o, ht);
}

static int decode_impl(const float* q, const float* k, const float* v, const float* g,
                       int scalar_gate, const float* beta, const float* eb, const float* ew,
                       double scale, double* state, double* o, int N, int H, int Dk, int Dv) {
    int failed = 0;
    const int64_t pairs = (int64_t)N * H;
#pragma omp parallel for schedule(static) reduction(| : failed)
    for (int64_t p = 0; p < pairs; ++p) {
        double* tmp = (double*)malloc(sizeof(double) * (2 * (size_t)Dv + Dk));
        if (!tmp) { failed = 1; continue; }
        /* a decode step is one token of a chain whose "time" index is the pair */
        const int n = (int)(p / H), h = (int)(p % H);
        chain(q + (int64_t)n * H * Dk, k + (int64_t)n * H * Dk, v + (int64_t)n * H * Dv,
              g + (int64_t)n * H * (scalar_gate ? 1 : Dk), scalar_gate,
              beta ? beta + (int64_t)n * H : NULL, eb ? eb + (int64_t)n * H * Dk : NULL,
              ew ? ew + (int64_t)n * H * Dv : NULL, scale, H, Dk, Dv, h, 0, 1,
              state + p * (int64_t)Dk * Dv, o + (int64_t)n * H * Dv, tmp, tmp + Dv,
              tmp + 2 * Dv);
        free(tmp);
    }
    return failed ? -1 : 0;
}

/* One decode step: q, k [N, H, Dk]; g [N, H, Dk] ([N, H] with scalar_gate);
 * v [N, H, Dv]; beta [N, H]; state double [N, H, Dk, Dv] updated in place;
 * o double [N, H, Dv]. */
int kda_oracle_decode(const float* q, const float* k, const float* v, const float* g,
                      int scalar_gate, const float* beta, double scale, double* state, double* o,
                      int N, int H, int Dk, int Dv) {
    return decode_impl(q, k, v, g, scalar_gate, beta, NULL, NULL, scale, state, o, N, H, Dk, Dv);
}

/* One Gated DeltaNet-2 decode step: g, b [N, H, Dk]; w [N, H, Dv]; the rest as
 * kda_oracle_decode. */
int kda_oracle_gdn2_decode(const float* q, const float* k, const float* v, const float* g,
                           const float* b, const float* w, double scale, double* state,
                           double* o, int N, int H, int Dk, int Dv) {
    return decode_impl(q, k, v, g, 0, NULL, b, w, scale, state, o, N, H, Dk, Dv);
}
