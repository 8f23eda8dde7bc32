/*
 * fa2_c_client.c -- a plain C11 program that uses libfa2 through include/fa2.h
 * only: device buffers from the HIP runtime's C API, the library's entry
 * points with raw pointers and sizes, results checked against the CPU oracle
 * (oracle/libfa2_oracle.so, test infrastructure).  It shows that the boundary
 * needs no C++, no PyTorch and no Python.
 *
 * Cases: fp32 and bf16 forward with grouped K/V heads and a causal mask
 * (fa2_fwd_ex), a split-K/V decode forward with its workspace, and an fp32
 * backward (fa2_bwd).  Exit status 0 when every case is within the parity
 * tolerances (fp32: 1e-4 on O and L; bf16: 2e-2 on O, 1e-3 on L; fp32
 * gradients: 1e-4 x max(max|reference|, 1)), 1 otherwise, 2 on a setup error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fa2.h"

/* the oracle's C entry points (oracle/fa2_oracle.c) */
int fa2_oracle_fwd_gqa(const float* q, const float* k, const float* v, double* o, double* lse, int64_t B,
                       int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D, double scale, int causal,
                       const int64_t* rows, int64_t n_rows, int n_threads);
int fa2_oracle_bwd_gqa(const float* q, const float* k, const float* v, const float* dout, double* dq,
                       double* dk, double* dv, int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N,
                       int64_t D, double scale, int causal, int n_threads);

#define HIP_OK(x)                                                                      \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            exit(2);                                                                   \
        }                                                                              \
    } while (0)

/* inputs: a 64-bit linear congruential generator mapped to [-2, 2) */
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static float next_value(void) {
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((double)(rng_state >> 11) * (4.0 / 9007199254740992.0) - 2.0);
}

/* bf16 of x, round to nearest even (finite inputs) */
static uint16_t to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return x;
}

static void* dev_copy(const void* host, size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes > 0 ? bytes : 1));
    if (host) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

static int failures = 0;
static void report(const char* what, double err, double bound) {
    const int ok = err <= bound;
    printf("%-58s max err %.3e (bound %.1e) %s\n", what, err, bound, ok ? "ok" : "FAIL");
    if (!ok) ++failures;
}

/* One forward case: fp32 inputs (rounded to bf16 first when bf16). */
static void forward_case(const char* what, int dtype, int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N,
                         int64_t D, int causal, int n_splits) {
    fprintf(stderr, "case %s\n", what);
    const size_t nq = (size_t)(B * H * M * D), nk = (size_t)(B * Hk * N * D), nl = (size_t)(B * H * M);
    float* q = malloc(nq * 4);
    float* k = malloc(nk * 4);
    float* v = malloc(nk * 4);
    for (size_t i = 0; i < nq; ++i) q[i] = next_value();
    for (size_t i = 0; i < nk; ++i) k[i] = next_value();
    for (size_t i = 0; i < nk; ++i) v[i] = next_value();
    const size_t elt = dtype == FA2_DTYPE_F32 ? 4 : 2;
    void *hq = q, *hk = k, *hv = v;
    uint16_t *bq = NULL, *bk = NULL, *bv = NULL;
    if (dtype == FA2_DTYPE_BF16) {
        bq = malloc(nq * 2);
        bk = malloc(nk * 2);
        bv = malloc(nk * 2);
        for (size_t i = 0; i < nq; ++i) q[i] = from_bf16(bq[i] = to_bf16(q[i]));
        for (size_t i = 0; i < nk; ++i) k[i] = from_bf16(bk[i] = to_bf16(k[i]));
        for (size_t i = 0; i < nk; ++i) v[i] = from_bf16(bv[i] = to_bf16(v[i]));
        hq = bq, hk = bk, hv = bv;
    }
    void* dq = dev_copy(hq, nq * elt);
    void* dk = dev_copy(hk, nk * elt);
    void* dv = dev_copy(hv, nk * elt);
    void* d_o = dev_copy(NULL, nq * elt);
    float* d_l = dev_copy(NULL, nl * 4);
    void* ws = NULL;
    int64_t ws_bytes = 0;
    const int splits = n_splits == 0 ? fa2_fwd_num_splits(B, H, Hk, M, N, D, causal, dtype) : n_splits;
    if (splits > 1) {
        ws_bytes = fa2_fwd_workspace_bytes(B, H, M, D, splits);
        ws = dev_copy(NULL, (size_t)ws_bytes);
    }
    const double scale = 1.0 / sqrt((double)D);
    const int st = fa2_fwd_ex(dq, dk, dv, d_o, d_l, B, H, Hk, M, N, D, (float)scale, causal, dtype, splits, ws,
                              ws_bytes, NULL);
    if (st != FA2_OK) {
        printf("%s: fa2_fwd_ex returned %d (%s)\n", what, st, fa2_status_string(st));
        ++failures;
        return;
    }
    HIP_OK(hipDeviceSynchronize());
    float* o32 = malloc(nq * 4);
    float* l = malloc(nl * 4);
    if (dtype == FA2_DTYPE_BF16) {
        uint16_t* ob = malloc(nq * 2);
        HIP_OK(hipMemcpy(ob, d_o, nq * 2, hipMemcpyDeviceToHost));
        for (size_t i = 0; i < nq; ++i) o32[i] = from_bf16(ob[i]);
        free(ob);
    } else {
        HIP_OK(hipMemcpy(o32, d_o, nq * 4, hipMemcpyDeviceToHost));
    }
    HIP_OK(hipMemcpy(l, d_l, nl * 4, hipMemcpyDeviceToHost));
    double* o_ref = malloc(nq * 8);
    double* l_ref = malloc(nl * 8);
    if (fa2_oracle_fwd_gqa(q, k, v, o_ref, l_ref, B, H, Hk, M, N, D, scale, causal, NULL, 0, 0) != 0) exit(2);
    double eo = 0.0, el = 0.0;
    for (size_t i = 0; i < nq; ++i) eo = fmax(eo, fabs((double)o32[i] - o_ref[i]));
    for (size_t i = 0; i < nl; ++i) el = fmax(el, fabs((double)l[i] - l_ref[i]));
    char buf[160];
    snprintf(buf, sizeof buf, "%s: O (%d splits)", what, splits);
    report(buf, eo, dtype == FA2_DTYPE_F32 ? 1e-4 : 2e-2);
    snprintf(buf, sizeof buf, "%s: L", what);
    report(buf, el, dtype == FA2_DTYPE_F32 ? 1e-4 : 1e-3);
    HIP_OK(hipFree(dq));
    HIP_OK(hipFree(dk));
    HIP_OK(hipFree(dv));
    HIP_OK(hipFree(d_o));
    HIP_OK(hipFree(d_l));
    if (ws) HIP_OK(hipFree(ws));
    free(q), free(k), free(v), free(bq), free(bk), free(bv), free(o32), free(l), free(o_ref), free(l_ref);
}

/* fp32 forward then backward, gradients against the oracle's chain rule. */
static void backward_case(const char* what, int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
                          int causal) {
    fprintf(stderr, "case %s\n", what);
    const size_t nq = (size_t)(B * H * M * D), nk = (size_t)(B * Hk * N * D), nl = (size_t)(B * H * M);
    float* q = malloc(nq * 4);
    float* k = malloc(nk * 4);
    float* v = malloc(nk * 4);
    float* dout = malloc(nq * 4);
    for (size_t i = 0; i < nq; ++i) q[i] = next_value();
    for (size_t i = 0; i < nk; ++i) k[i] = next_value();
    for (size_t i = 0; i < nk; ++i) v[i] = next_value();
    for (size_t i = 0; i < nq; ++i) dout[i] = next_value();
    float* d_q = dev_copy(q, nq * 4);
    float* d_k = dev_copy(k, nk * 4);
    float* d_v = dev_copy(v, nk * 4);
    float* d_do = dev_copy(dout, nq * 4);
    float* d_o = dev_copy(NULL, nq * 4);
    float* d_l = dev_copy(NULL, nl * 4);
    float* d_dq = dev_copy(NULL, nq * 4);
    float* d_dk = dev_copy(NULL, nk * 4);
    float* d_dv = dev_copy(NULL, nk * 4);
    float* d_delta = dev_copy(NULL, nl * 4);
    const double scale = 1.0 / sqrt((double)D);
    int st = fa2_fwd_ex(d_q, d_k, d_v, d_o, d_l, B, H, Hk, M, N, D, (float)scale, causal, FA2_DTYPE_F32, 1, NULL,
                        0, NULL);
    if (st == FA2_OK)
        st = fa2_bwd(d_q, d_k, d_v, d_o, d_l, d_do, d_dq, d_dk, d_dv, d_delta, B, H, Hk, M, N, D, (float)scale,
                     causal, FA2_DTYPE_F32, NULL);
    if (st != FA2_OK) {
        printf("%s: returned %d (%s)\n", what, st, fa2_status_string(st));
        ++failures;
        return;
    }
    HIP_OK(hipDeviceSynchronize());
    float* g[3] = {malloc(nq * 4), malloc(nk * 4), malloc(nk * 4)};
    HIP_OK(hipMemcpy(g[0], d_dq, nq * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g[1], d_dk, nk * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g[2], d_dv, nk * 4, hipMemcpyDeviceToHost));
    double* r[3] = {malloc(nq * 8), malloc(nk * 8), malloc(nk * 8)};
    if (fa2_oracle_bwd_gqa(q, k, v, dout, r[0], r[1], r[2], B, H, Hk, M, N, D, scale, causal, 0) != 0) exit(2);
    const char* names[3] = {"dq", "dk", "dv"};
    const size_t n[3] = {nq, nk, nk};
    for (int t = 0; t < 3; ++t) {
        double err = 0.0, mag = 0.0;
        for (size_t i = 0; i < n[t]; ++i) {
            err = fmax(err, fabs((double)g[t][i] - r[t][i]));
            mag = fmax(mag, fabs(r[t][i]));
        }
        char buf[160];
        snprintf(buf, sizeof buf, "%s: %s", what, names[t]);
        report(buf, err, 1e-4 * fmax(mag, 1.0));
        free(g[t]);
        free(r[t]);
    }
    float* bufs[] = {d_q, d_k, d_v, d_do, d_o, d_l, d_dq, d_dk, d_dv, d_delta};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
    free(q), free(k), free(v), free(dout);
}

int main(void) {
    /* line-buffered: whatever was printed survives an abnormal end */
    setvbuf(stdout, NULL, _IOLBF, 0);
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
        fprintf(stderr, "no HIP device\n");
        return 2;
    }
    forward_case("fp32 forward, B=2 H=4 Hk=2 M=77 N=150 D=64 causal", FA2_DTYPE_F32, 2, 4, 2, 77, 150, 64, 1, 1);
    forward_case("bf16 forward, B=1 H=8 Hk=2 M=300 N=333 D=128 causal", FA2_DTYPE_BF16, 1, 8, 2, 300, 333, 128, 1,
                 1);
    forward_case("bf16 decode, B=2 H=8 Hk=1 M=3 N=2500 D=128 (auto splits)", FA2_DTYPE_BF16, 2, 8, 1, 3, 2500, 128,
                 0, 0);
    backward_case("fp32 backward, B=1 H=4 Hk=2 M=120 N=90 D=64 causal", 1, 4, 2, 120, 90, 64, 1);
    printf("%s\n", failures ? "FAILED" : "all cases within tolerance");
    return failures ? 1 : 0;
}
