/*
 * fa2_oracle.c -- the CPU reference ("oracle") for the attention forward pass
 * and its gradients (the backward pass, at the end of this file).
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
 *     J     = {0..N-1}, or {0..min(i, N-1)} when causal,         (1)
 *             further cut to i - wl <= j <= i + wr by a sliding
 *             window (wl, wr; a negative side is unbounded)
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
 *           harness's tril-masked reference.  The sliding window is the
 *           window_size = (left, right) option of the entry point described
 *           in "From FlashAttention to FlashAttention 2", section "Layer 1",
 *           (-1 meaning unbounded), a change of the causal mask formula as
 *           "Writing FlashAttention 2 in Triton" puts it (its list of next
 *           steps); measured from the same top-left diagonal j = i.  A row
 *           whose window holds no key gets O = 0 and L = -inf (l = 0: the
 *           guard of that page's bug catalogue item 8 returns O = 0).
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

/* (1) the keys query row i sees: j0 <= j < j0 + n (n <= 0: none) */
static void visible_keys(int64_t i, int64_t N, int causal, int64_t wl, int64_t wr,
                         int64_t* j0, int64_t* n) {
    int64_t lo = 0, hi = N - 1;
    if (causal && i < hi) hi = i;
    if (wr >= 0 && i + wr < hi) hi = i + wr;
    if (wl >= 0 && i - wl > lo) lo = i - wl;
    *j0 = lo;
    *n = hi - lo + 1;
}

/* One query row of one (b,h) slice: steps (2)-(6) above over the visible
 * keys j0 .. j0 + n_vis - 1.  `s` is scratch of length >= N. */
static void oracle_row(const float* qi, const float* kbh, const float* vbh,
                       double* orow, double* lse_out, int64_t j0, int64_t n_vis,
                       int64_t D, double scale, double* s) {
    if (n_vis <= 0) {  /* no visible key: l = 0 */
        for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }
    kbh += j0 * D;
    vbh += j0 * D;

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
 * H % Hk == 0 (Hk >= 1).  wl, wr: sliding window (negative: unbounded).
 * rows == NULL: every query row; o is [B,H,M,D] and lse is [B,H,M].
 * rows != NULL: only the n_rows listed rows (each in [0, M)), the same rows
 *   for every (b,h); o is [B,H,n_rows,D] and lse is [B,H,n_rows].
 * n_threads <= 0 uses the OpenMP default.
 * Returns 0 on success, nonzero on invalid arguments or allocation failure.
 */
int fa2_oracle_fwd_local(const float* q, const float* k, const float* v, double* o,
                         double* lse, int64_t B, int64_t H, int64_t Hk, int64_t M,
                         int64_t N, int64_t D, double scale, int causal, int64_t wl,
                         int64_t wr, const int64_t* rows, int64_t n_rows, int n_threads) {
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
            int64_t j0, n_vis;
            visible_keys(i, N, causal, wl, wr, &j0, &n_vis);
            oracle_row(q + (bh * M + i) * D, k + kvh * N * D, v + kvh * N * D,
                       o + (bh * R + r) * D, lse + bh * R + r, j0, n_vis, D, scale, s);
        }
        free(s);
    }
    return status;
}

/* No sliding window. */
int fa2_oracle_fwd_gqa(const float* q, const float* k, const float* v, double* o,
                       double* lse, int64_t B, int64_t H, int64_t Hk, int64_t M,
                       int64_t N, int64_t D, double scale, int causal,
                       const int64_t* rows, int64_t n_rows, int n_threads) {
    return fa2_oracle_fwd_local(q, k, v, o, lse, B, H, Hk, M, N, D, scale, causal, -1, -1,
                                rows, n_rows, n_threads);
}

/* Multi-head attention: every query head has its own K/V head (Hk == H). */
int fa2_oracle_fwd(const float* q, const float* k, const float* v, double* o,
                   double* lse, int64_t B, int64_t H, int64_t M, int64_t N,
                   int64_t D, double scale, int causal, const int64_t* rows,
                   int64_t n_rows, int n_threads) {
    return fa2_oracle_fwd_gqa(q, k, v, o, lse, B, H, H > 0 ? H : 1, M, N, D,
                              scale, causal, rows, n_rows, n_threads);
}

/*
 * Backward pass (gradients of the forward above with respect to q, k, v for a
 * given upstream gradient dO), the plain chain rule through the softmax,
 * evaluated in IEEE double.  For every (b, h) and query row i, with J and
 * P_ij = e_j / l from steps (1)-(4):
 *
 *   dV[j]   += P_ij * dO[i]                               for j in J   (7)
 *   dP_ij    = <dO[i], V[j]>                                           (8)
 *   D_i      = sum_{j in J} P_ij * dP_ij                               (9)
 *   dS_ij    = P_ij * (dP_ij - D_i)                                    (10)
 *   dQ[i]    = scale * sum_{j in J} dS_ij * K[j]                       (11)
 *   dK[j]   += scale * dS_ij * Q[i]                                    (12)
 *
 * J is the forward's visible set (1), sliding window included; a row with an
 * empty J has no gradient (dQ = 0, nothing added to dK, dV).
 * dK and dV of a K/V head sum over every query head that reads it (hk).
 * Sources: "From FlashAttention to FlashAttention 2", section "Layer 7: The
 * Backward Kernel" (steps 3-7 of its inner loop: dP = dO V^T, dS = P o (dP -
 * rowsum(dO o O)), dV += P^T dO, dK += dS^T Q, dQ = dS K) and section
 * "Backward Pass: Recomputation".  (9) is the definition rowsum(P o dP); it
 * equals rowsum(dO o O) when O is the exact forward output, the form the
 * page uses.  The scale enters (11) and (12) because S = scale * Q K^T.
 * No tiling: one query row at a time, P and dP materialised per row.
 */
static void oracle_bwd_row(const float* qi, const float* doi, const float* kbh,
                           const float* vbh, double* dqi, double* dkbh,
                           double* dvbh, int64_t j0, int64_t n_vis, int64_t D,
                           double scale, double* p, double* dp) {
    for (int64_t d = 0; d < D; ++d) dqi[d] = 0.0;
    if (n_vis <= 0) return; /* a row that sees no key has no gradient */
    kbh += j0 * D;
    vbh += j0 * D;
    dkbh += j0 * D;
    dvbh += j0 * D;
    /* P_ij, steps (2)-(4) of the forward over the visible keys */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_vis; ++j) {
        const float* kj = kbh + j * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];
        p[j] = scale * dot;
        if (p[j] > m) m = p[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (int64_t j = 0; j < n_vis; ++j) p[j] /= l;
    /* (8) and (9) */
    double Di = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        const float* vrow = vbh + j * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)doi[d] * (double)vrow[d];
        dp[j] = dot;
        Di += p[j] * dot;
    }
    /* (7), (10), (11), (12) */
    for (int64_t j = 0; j < n_vis; ++j) {
        const double ds = p[j] * (dp[j] - Di);
        const float* kj = kbh + j * D;
        double* dkj = dkbh + j * D;
        double* dvj = dvbh + j * D;
        for (int64_t d = 0; d < D; ++d) {
            dvj[d] += p[j] * (double)doi[d];
            dqi[d] += scale * ds * (double)kj[d];
            dkj[d] += scale * ds * (double)qi[d];
        }
    }
}

/*
 * q, dO: [B,H,M,D]; k, v: [B,Hk,N,D]; outputs dq [B,H,M,D], dk and dv
 * [B,Hk,N,D] in double.  Work is split over the B*Hk K/V heads (each thread
 * owns its K/V head's dk, dv), so no two threads add into the same row.
 * Returns 0 on success.
 */
int fa2_oracle_bwd_local(const float* q, const float* k, const float* v,
                         const float* dout, double* dq, double* dk, double* dv,
                         int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N,
                         int64_t D, double scale, int causal, int64_t wl, int64_t wr,
                         int n_threads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return FA2_ORACLE_EINVAL;
    if (B < 0 || H < 0 || M < 0 || N <= 0 || D <= 0) return FA2_ORACLE_EINVAL;
    if (Hk < 1 || H % Hk != 0) return FA2_ORACLE_EINVAL;
    const int64_t group = H / Hk;
    const int64_t BHk = B * Hk;
    int status = FA2_ORACLE_OK;
    for (int64_t x = 0; x < BHk * N * D; ++x) { dk[x] = 0.0; dv[x] = 0.0; }
#ifdef _OPENMP
    int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
    {
        double* p = (double*)malloc((size_t)N * sizeof(double));
        double* dp = (double*)malloc((size_t)N * sizeof(double));
        if (!p || !dp) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            status = FA2_ORACLE_ENOMEM;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t bk = 0; bk < BHk; ++bk) {
            if (!p || !dp) continue;
            const int64_t b = bk / Hk, hk = bk % Hk;
            const float* kbh = k + bk * N * D;
            const float* vbh = v + bk * N * D;
            for (int64_t g = 0; g < group; ++g) {
                const int64_t bh = b * H + hk * group + g; /* (hk) */
                for (int64_t i = 0; i < M; ++i) {
                    int64_t j0, n_vis;
                    visible_keys(i, N, causal, wl, wr, &j0, &n_vis); /* (1) */
                    oracle_bwd_row(q + (bh * M + i) * D, dout + (bh * M + i) * D,
                                   kbh, vbh, dq + (bh * M + i) * D,
                                   dk + bk * N * D, dv + bk * N * D, j0, n_vis, D,
                                   scale, p, dp);
                }
            }
        }
        free(p);
        free(dp);
    }
    return status;
}

/* No sliding window. */
int fa2_oracle_bwd_gqa(const float* q, const float* k, const float* v,
                       const float* dout, double* dq, double* dk, double* dv,
                       int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N,
                       int64_t D, double scale, int causal, int n_threads) {
    return fa2_oracle_bwd_local(q, k, v, dout, dq, dk, dv, B, H, Hk, M, N, D, scale,
                                causal, -1, -1, n_threads);
}
