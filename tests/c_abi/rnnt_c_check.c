/*
 * rnnt_c_check.c -- calls librnnt from C through include/rnnt.h alone and
 * compares its results with the fp64 C oracle (oracle/rnnt_oracle.c, linked
 * in: this program is test infrastructure).
 *
 * A small packed batch (three samples, one with U = 0) of deterministic
 * synthetic fp32 logits goes through rnnt_loss_fused with reduction none and
 * again with mean; the per-sample losses (relative 1e-5), the gradient
 * (absolute 1e-5, per sample), the reduced loss, the device status word and
 * two host-side argument errors are checked.  Exit status 0 on agreement.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rnnt.h"

/* the oracle's entry point (oracle/rnnt_oracle.c) */
int rnnt_oracle_sample_ex(const void *x, int dtype, int T, int U, int V, const int *y, int blank, int fused,
                          double clamp, double fastemit_lambda, const int64_t *grad_rows, long n_grad_rows,
                          double *grad, double *alpha_out, double *beta_out, double *loss_alpha,
                          double *loss_beta);
#define ORACLE_F32 1

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 2;                                                                 \
        }                                                                             \
    } while (0)

int main(void) {
    enum { B = 3, V = 13, S = 5 };
    const int32_t T[B] = {7, 4, 9}, U[B] = {3, 0, 5};
    const int blank = V - 1;
    int64_t N = 0, off[B + 1];
    for (int i = 0; i < B; ++i) {
        off[i] = N;
        N += (int64_t)T[i] * (U[i] + 1);
    }
    off[B] = N;
    float *x = malloc(sizeof(float) * N * V);
    int32_t tg[B * S];
    for (int64_t k = 0; k < N * V; ++k) x[k] = 2.0f * (float)sin(0.37 * (double)k + 0.1);
    for (int i = 0; i < B; ++i)
        for (int u = 0; u < S; ++u) tg[i * S + u] = (5 * i + 3 * u + 1) % (V - 1);  /* never the blank */

    size_t ws_bytes = 0;
    if (rnnt_loss_fused_workspace_size(B, V, N, RNNT_F32, T, U, &ws_bytes) != RNNT_SUCCESS) return 3;
    void *d_x, *d_tg, *d_ws, *d_g;
    float *d_loss, *d_red;
    CHECK_HIP(hipMalloc(&d_x, sizeof(float) * N * V));
    CHECK_HIP(hipMalloc(&d_g, sizeof(float) * N * V));
    CHECK_HIP(hipMalloc(&d_tg, sizeof(tg)));
    CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
    CHECK_HIP(hipMalloc((void **)&d_loss, sizeof(float) * B));
    CHECK_HIP(hipMalloc((void **)&d_red, sizeof(float)));
    CHECK_HIP(hipMemcpy(d_x, x, sizeof(float) * N * V, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_tg, tg, sizeof(tg), hipMemcpyHostToDevice));

    /* host-side argument errors come back before anything is enqueued */
    if (rnnt_loss_fused(d_x, RNNT_F32, N + 1, V, d_tg, S, T, U, B, -1, -1.0f, 0.0f, 1, RNNT_REDUCTION_NONE,
                        d_loss, NULL, d_g, d_ws, ws_bytes, NULL) != RNNT_INVALID_VALUE) return 4;
    if (rnnt_loss_fused(d_x, RNNT_F32, N, V, d_tg, S, T, U, B, -1, -1.0f, 0.0f, 1, RNNT_REDUCTION_NONE,
                        d_loss, NULL, d_g, d_ws, ws_bytes / 2, NULL) != RNNT_WORKSPACE_TOO_SMALL) return 5;

    if (rnnt_loss_fused(d_x, RNNT_F32, N, V, d_tg, S, T, U, B, -1, -1.0f, 0.0f, 1, RNNT_REDUCTION_NONE,
                        d_loss, NULL, d_g, d_ws, ws_bytes, NULL) != RNNT_SUCCESS) return 6;
    uint32_t flags = 1234;
    if (rnnt_loss_fused_check(d_ws, NULL, &flags) != RNNT_SUCCESS || flags != 0) return 7;
    float loss[B], red = 0.0f;
    float *g = malloc(sizeof(float) * N * V);
    CHECK_HIP(hipMemcpy(loss, d_loss, sizeof(loss), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(g, d_g, sizeof(float) * N * V, hipMemcpyDeviceToHost));

    double worst_l = 0.0, worst_g = 0.0, sum = 0.0;
    for (int i = 0; i < B; ++i) {
        const int64_t rows = off[i + 1] - off[i];
        double *og = malloc(sizeof(double) * rows * V);
        double la = 0.0, lb = 0.0;
        if (rnnt_oracle_sample_ex(x + off[i] * V, ORACLE_F32, T[i], U[i], V, tg + i * S, blank, 1, -1.0, 0.0, NULL,
                                  -1, og, NULL, NULL, &la, &lb) != 0) return 8;
        const double rel = fabs((double)loss[i] - lb) / fmax(1.0, fabs(lb));
        if (rel > worst_l) worst_l = rel;
        for (int64_t k = 0; k < rows * V; ++k) {
            const double e = fabs((double)g[off[i] * V + k] - og[k]);
            if (e > worst_g) worst_g = e;
        }
        sum += lb;
        free(og);
    }
    /* mean reduction: the reduced loss, and the gradient scaled by 1/B */
    if (rnnt_loss_fused(d_x, RNNT_F32, N, V, d_tg, S, T, U, B, -1, -1.0f, 0.0f, 1, RNNT_REDUCTION_MEAN,
                        d_loss, d_red, d_g, d_ws, ws_bytes, NULL) != RNNT_SUCCESS) return 9;
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(&red, d_red, sizeof(float), hipMemcpyDeviceToHost));
    const double red_rel = fabs((double)red - sum / B) / fmax(1.0, fabs(sum / B));
    printf("c-abi: worst loss rel %.3g, worst grad abs %.3g, mean rel %.3g\n", worst_l, worst_g, red_rel);
    hipFree(d_x); hipFree(d_g); hipFree(d_tg); hipFree(d_ws); hipFree(d_loss); hipFree(d_red);
    free(x); free(g);
    return (worst_l <= 1e-5 && worst_g <= 1e-5 && red_rel <= 1e-5) ? 0 : 1;
}
