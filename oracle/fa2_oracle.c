/*
 * fa2_oracle.c -- the CPU reference ("oracle") for the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the test suite, the smoke check and the bench's
 * cpu_baseline leg do.  It shares no code, header, constant or helper with
 * the HIP library.
 *
 * What it computes is the plain definition of scaled-dot-product attention,
 * evaluated one query row at a time in IEEE double precision:
 *
 *   for every (b, h) and query row i, with K/V head hk = h / (H / Hk):
 *     J     = {0..N-1}, or {0..min(i, N-1)} when causal          (1)
 *     s_j   = scale * sum_d q[i,d] * k[j,d]          for j in J    (2)
 *     m     = max_{j in J} s_j                                     (3)
 *     e_j   = exp(s_j - m),  l = sum_{j in J} e_j                  (4)
 *     O[i]  = sum_{j in J} e_j * v[j,:] / l                        (5)
 *     L[i]  = m + log(l)                                           (6)
 *
 * Sources for each step:
 *  (2),(5)  "From FlashAttention to FlashAttention 2", section "Background:
 *           FlashAttention 1": O = softmax(QK^T / sqrt(d)) V with the full
 *           score row; the scale is an argument here (the pages always pass
 *           1/sqrt(d)).
 *  (1)      causal visibility is top-left: a query row i sees keys j <= i.
 *           "Writing FlashAttention 2 in Triton", Step 4 (mask keeps
 *           offs_m >= offs_n) and its bug catalogue item on the comparison
 *           direction; "FlashAttention-2 from PyTorch to Triton", the test
 *           harness's tril-masked reference.
 *  (6)      L is the natural-log logsumexp of the *scaled* scores, i.e.
 *           m + log(l): "FlashAttention-2 from PyTorch to Triton", opening
 *           description of the second output L; "From FlashAttention to
 *           FlashAttention 2", section "Backward Pass: Recomputation".
 *  (hk)     grouped-query attention: H / Hk consecutive query heads share one
 *           K/V head ("From FlashAttention to FlashAttention 2", section
 *           "Layer 8": the K/V head index is the query head index divided by
 *           the ratio h / h_k).  Hk == H is ordinary multi-head attention.
 *  (3),(4)  subtracting the row maximum before exponentiating does not
 *           change (5) or (6) mathematically; it keeps exp() finite for the
 *           large-magnitude workloads.  The pages' harness uses
 *           torch.logsumexp / SDPA, which do the same.
 *
 * Masked keys are simply excluded from the sums (no sentinel value).
 * No blocking, fusion or reordering beyond the definition: one fp64 score
 * row per query, materialised, then exponentiated, then used.
 *
 * Inputs are float arrays: fp32 inputs are used as is, and bf16 / fp16
 * inputs are passed as their exact float32 widening, so every input value reaches the
 * fp64 arithmetic exactly.  Build without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define FA2_ORACLE_OK 0
#define FA2_ORACLE_EINVAL 1
#define FA2_ORACLE_ENOMEM 2

int fa2_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One query row of one (b,h) slice: steps (1)-(6) above.  `s` is scratch of
 * length >= N. */
static void oracle_row(const float* qi, const float* kbh, const float* vbh,
                       double* orow, double* lse_out, int64_t i, int64_t N,
                       int64_t D, double scale, int causal, double* s) {
    /* (1) visible keys */
    int64_t n_vis = N;
    if (causal) n_vis = (i + 1 < N) ? (i + 1) : N;

    /* (2) scores and (3) row maximum */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; ++j) {
        const float* kj = kbh + j * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }

    /* (4) weights and their sum */
    double l = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }

    /* (5) weighted sum of value rows, divided by l */
    for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        const float* vj = vbh + j * D;
        const double e = s[j];
        for (int64_t d = 0; d < D; ++d) orow[d] += e * (double)vj[d];
    }
    for (int64_t d = 0; d < D; ++d) orow[d] /= l;

    /* (6) logsumexp */
    *lse_out = m + log(l);
}

/*
 * q: [B,H,M,D], k and v: [B,Hk,N,D], all contiguous row-major floats;
 * H % Hk == 0 (Hk >= 1).
 * rows == NULL: every query row; o is [B,H,M,D] and lse is [B,H,M].
 * rows != NULL: only the n_rows listed rows (each in [0, M)), the same rows
 *   for every (b,h); o is [B,H,n_rows,D] and lse is [B,H,n_rows].
 * n_threads <= 0 uses the OpenMP default.
 * Returns 0 on success, nonzero on invalid arguments or allocation failure.
 */
int fa2_oracle_fwd_gqa(const float* q, const float* k, const float* v, double* o,
                       double* lse, int64_t B, int64_t H, int64_t Hk, int64_t M,
                       int64_t N, int64_t D, double scale, int causal,
                       const int64_t* rows, int64_t n_rows, int n_threads) {
    if (!q || !k || !v || !o || !lse) return FA2_ORACLE_EINVAL;
    if (B < 0 || H < 0 || M < 0 || N <= 0 || D <= 0) return FA2_ORACLE_EINVAL;
    if (Hk < 1 || H % Hk != 0) return FA2_ORACLE_EINVAL;
    const int64_t group = H / Hk;  /* query heads per K/V head */
    const int64_t R = rows ? n_rows : M;
    if (R < 0) return FA2_ORACLE_EINVAL;
    if (rows) {
        for (int64_t r = 0; r < R; ++r)
            if (rows[r] < 0 || rows[r] >= M) return FA2_ORACLE_EINVAL;
    }
    const int64_t BH = B * H;
    const int64_t total = BH * R;
    int status = FA2_ORACLE_OK;

#ifdef _OPENMP
    int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
    {
        double* s = (double*)malloc((size_t)N * sizeof(double));
        if (!s) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = FA2_ORACLE_ENOMEM;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 8)
#endif
        for (int64_t t = 0; t < total; ++t) {
            if (!s) continue;
            const int64_t bh = t / R;
            const int64_t r = t % R;
            const int64_t i = rows ? rows[r] : r;
            const int64_t b = bh / H, h = bh % H;
            const int64_t kvh = b * Hk + h / group; /* (hk) */
            oracle_row(q + (bh * M + i) * D, k + kvh * N * D, v + kvh * N * D,
                       o + (bh * R + r) * D, lse + bh * R + r, i, N, D, scale,
                       causal, s);
        }
        free(s);
    }
    return status;
}

/* Multi-head attention: every query head has its own K/V head (Hk == H). */
int fa2_oracle_fwd(const float* q, const float* k, const float* v, double* o,
                   double* lse, int64_t B, int64_t H, int64_t M, int64_t N,
                   int64_t D, double scale, int causal, const int64_t* rows,
                   int64_t n_rows, int n_threads) {
    return fa2_oracle_fwd_gqa(q, k, v, o, lse, B, H, H > 0 ? H : 1, M, N, D,
                              scale, causal, rows, n_rows, n_threads);
}
