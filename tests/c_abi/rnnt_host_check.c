/*
 * rnnt_host_check.c -- drives every host-only path of librnnt's C ABI
 * (include/rnnt.h): argument validation, the longest-first schedule, the
 * workspace layouts, rnnt_plan_describe, the refusals of the allocation-free
 * call and the timing switches.  No call here reaches a kernel launch or a
 * device pointer: every call with device pointers is one the library must
 * refuse on the host (the pointers are placeholders never dereferenced).  It
 * is built against a librnnt whose host code is compiled with the address
 * and undefined-behaviour sanitizers, so any out-of-bounds access, leak-free
 * misuse or undefined operation in the host code aborts the run.
 *
 * Checks, beside the sanitizers: each refusal returns its documented status;
 * rnnt_plan_describe's chunk table covers every lattice node of every
 * sample exactly once, in the row order and in the anti-diagonal order, and
 * lists samples longest first.  Exit status 0 when everything holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rnnt.h"

static int failures = 0;

#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            fprintf(stderr, "FAILED at line %d: %s\n", __LINE__, #cond);     \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

/* placeholders for device pointers on paths the library refuses on the host */
#define DEV(k) ((void *)(uintptr_t)((uint64_t)(k) << 36))

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {
    rng_state = rng_state * 1664525u + 1013904223u;
    return rng_state >> 8;
}

/* The chunk table of a batch must cover every node exactly once. */
static void check_plan(int32_t B, int32_t V, rnnt_dtype dt, const int32_t *T, const int32_t *U) {
    int32_t n_chunks = 0;
    EXPECT(rnnt_plan_describe(B, V, dt, T, U, 0, NULL, NULL, NULL, NULL, NULL, NULL, &n_chunks) == RNNT_SUCCESS);
    if (n_chunks <= 0) {
        ++failures;
        return;
    }
    int32_t *order = malloc(sizeof(int32_t) * B);
    int32_t *cs = malloc(sizeof(int32_t) * n_chunks), *rb = malloc(sizeof(int32_t) * n_chunks);
    int32_t *rc = malloc(sizeof(int32_t) * n_chunks), *dg = malloc(sizeof(int32_t) * n_chunks);
    int32_t *cl = malloc(sizeof(int32_t) * n_chunks);
    int32_t got = 0;
    EXPECT(rnnt_plan_describe(B, V, dt, T, U, n_chunks, order, cs, rb, rc, dg, cl, &got) == RNNT_SUCCESS);
    EXPECT(got == n_chunks);
    /* samples longest first: area T(U+1), then T+U, then index */
    for (int32_t k = 1; k < B; ++k) {
        const int32_t a = order[k - 1], b = order[k];
        const int64_t aa = (int64_t)T[a] * (U[a] + 1), ab = (int64_t)T[b] * (U[b] + 1);
        EXPECT(aa > ab || (aa == ab && (T[a] + U[a] > T[b] + U[b] || (T[a] + U[a] == T[b] + U[b] && a < b))));
    }
    for (int32_t i = 0; i < B; ++i) {
        const int64_t rows = (int64_t)T[i] * (U[i] + 1);
        unsigned char *seen_row = calloc((size_t)rows, 1), *seen_diag = calloc((size_t)rows, 1);
        for (int32_t k = 0; k < n_chunks; ++k) {
            if (cs[k] != i) continue;
            for (int32_t r = 0; r < rc[k]; ++r) {
                const int64_t row = (int64_t)rb[k] + r;
                EXPECT(row >= 0 && row < rows);
                if (row >= 0 && row < rows) seen_row[row]++;
            }
            /* the same count of nodes in anti-diagonal order from (diag, col) */
            int32_t n = dg[k], u = cl[k];
            for (int32_t r = 0; r < rc[k]; ++r) {
                const int32_t t = n - u;
                EXPECT(t >= 0 && t < T[i] && u >= 0 && u <= U[i]);
                if (t >= 0 && t < T[i] && u >= 0 && u <= U[i]) seen_diag[(int64_t)t * (U[i] + 1) + u]++;
                ++u;
                const int32_t hi = n < U[i] ? n : U[i];
                if (u > hi) {
                    ++n;
                    u = n - T[i] + 1 > 0 ? n - T[i] + 1 : 0;
                }
            }
        }
        for (int64_t r = 0; r < rows; ++r) EXPECT(seen_row[r] == 1 && seen_diag[r] == 1);
        free(seen_row);
        free(seen_diag);
    }
    /* a table shorter than the schedule is filled up to its capacity only */
    if (n_chunks > 1) {
        int32_t *small = malloc(sizeof(int32_t) * (n_chunks / 2));
        EXPECT(rnnt_plan_describe(B, V, dt, T, U, n_chunks / 2, NULL, small, NULL, NULL, NULL, NULL, &got) ==
               RNNT_SUCCESS);
        for (int32_t k = 0; k < n_chunks / 2; ++k) EXPECT(small[k] == cs[k]);
        free(small);
    }
    free(order); free(cs); free(rb); free(rc); free(dg); free(cl);
}

int main(void) {
    size_t ws = 0;
    /* status strings */
    for (int s = 0; s <= 5; ++s) EXPECT(rnnt_status_string((rnnt_status)s) != NULL);

    /* workspace sizes: valid batches and each refusal */
    {
        const int32_t T[3] = {5, 1, 9}, U[3] = {2, 0, 7};
        const int64_t N = 5 * 3 + 1 * 1 + 9 * 8;
        EXPECT(rnnt_loss_fused_workspace_size(3, 16, N, RNNT_F32, T, U, &ws) == RNNT_SUCCESS && ws > 0);
        EXPECT(rnnt_loss_fused_workspace_size(3, 16, N + 1, RNNT_F32, T, U, &ws) == RNNT_INVALID_VALUE);
        EXPECT(rnnt_loss_fused_workspace_size(0, 16, 0, RNNT_F32, T, U, &ws) == RNNT_INVALID_VALUE);
        EXPECT(rnnt_loss_fused_workspace_size(3, 0, N, RNNT_F32, T, U, &ws) == RNNT_INVALID_VALUE);
        EXPECT(rnnt_loss_fused_workspace_size(3, 16, N, (rnnt_dtype)7, T, U, &ws) == RNNT_INVALID_VALUE);
        EXPECT(rnnt_loss_fused_workspace_size(3, 16, N, RNNT_F32, NULL, U, &ws) == RNNT_INVALID_VALUE);
        EXPECT(rnnt_loss_fused_workspace_size(3, 16, N, RNNT_F32, T, U, NULL) == RNNT_INVALID_VALUE);
        const int32_t Tz[1] = {0}, Uz[1] = {0}, Ub[1] = {2048}, Uw[1] = {2047}, Tb[1] = {2};
        EXPECT(rnnt_loss_fused_workspace_size(1, 16, 0, RNNT_F32, Tz, Uz, &ws) == RNNT_INVALID_VALUE);
        EXPECT(rnnt_loss_fused_workspace_size(1, 16, 2 * 2049, RNNT_F32, Tb, Ub, &ws) == RNNT_INVALID_VALUE);
        EXPECT(rnnt_loss_fused_workspace_size(1, 16, 2 * 2048, RNNT_F32, Tb, Uw, &ws) == RNNT_SUCCESS && ws > 0);
        const int32_t Un[1] = {-1};
        EXPECT(rnnt_loss_fused_workspace_size(1, 16, 0, RNNT_F32, Tb, Un, &ws) == RNNT_INVALID_VALUE);
        size_t wp = 0;
        EXPECT(rnnt_loss_padded_workspace_size(3, 16, 9, 8, RNNT_F16, T, U, &wp) == RNNT_SUCCESS && wp > 0);
        EXPECT(rnnt_loss_padded_workspace_size(3, 16, 8, 8, RNNT_F16, T, U, &wp) == RNNT_INVALID_VALUE);
        EXPECT(rnnt_loss_padded_workspace_size(3, 16, 9, 7, RNNT_F16, T, U, &wp) == RNNT_INVALID_VALUE);
        const int32_t dur[2] = {2, 16}, bad_dur[1] = {17};
        EXPECT(rnnt_multiblank_workspace_size(3, 16, N, RNNT_F32, T, U, 2, dur, &ws) == RNNT_SUCCESS);
        EXPECT(rnnt_multiblank_workspace_size(3, 16, N, RNNT_F32, T, U, 1, bad_dur, &ws) == RNNT_INVALID_VALUE);
        EXPECT(rnnt_multiblank_workspace_size(3, 16, N, RNNT_F32, T, U, 5, dur, &ws) == RNNT_INVALID_VALUE);
        EXPECT(rnnt_multiblank_padded_workspace_size(3, 16, 9, 8, RNNT_F32, T, U, 2, dur, &ws) == RNNT_SUCCESS);
    }

    /* schedules: random batches (insertion-sorted up to 64 samples, sorted above), odd and even widths */
    for (int trial = 0; trial < 40; ++trial) {
        const int32_t B = 1 + (int32_t)(next_u32() % (trial < 30 ? 64 : 300));
        int32_t *T = malloc(sizeof(int32_t) * B), *U = malloc(sizeof(int32_t) * B);
        for (int32_t i = 0; i < B; ++i) {
            T[i] = 1 + (int32_t)(next_u32() % 120);
            U[i] = (int32_t)(next_u32() % 60);
            if (i > 0 && next_u32() % 5 == 0) { /* ties in the order key: repeat an earlier sample's lengths */
                const int32_t j = (int32_t)(next_u32() % (uint32_t)i);
                T[i] = T[j];
                U[i] = U[j];
            }
        }
        const int32_t V = (trial % 3 == 0) ? 29 : ((trial % 3 == 1) ? 1024 : 4096);
        check_plan(B, V, (trial & 1) ? RNNT_F16 : RNNT_F32, T, U);
        free(T);
        free(U);
    }

    /* calls refused on the host: nothing is enqueued, the placeholders are never read */
    {
        const int32_t T[2] = {6, 4}, U[2] = {3, 2};
        const int64_t N = 6 * 4 + 4 * 3;
        float *loss = DEV(3), *red = DEV(4);
        void *logits = DEV(1), *grad = DEV(5), *work = DEV(6);
        const int32_t *tg = DEV(2);
        size_t need = 0;
        EXPECT(rnnt_loss_fused_workspace_size(2, 8, N, RNNT_F32, T, U, &need) == RNNT_SUCCESS);
        EXPECT(rnnt_loss_fused(logits, RNNT_F32, N, 8, tg, 3, T, U, 2, 8, -1.f, 0.f, 1, RNNT_REDUCTION_SUM, loss,
                               red, grad, work, need, NULL) == RNNT_INVALID_VALUE);               /* blank = V */
        EXPECT(rnnt_loss_fused(logits, RNNT_F32, N, 8, tg, 3, T, U, 2, -9, -1.f, 0.f, 1, RNNT_REDUCTION_SUM, loss,
                               red, grad, work, need, NULL) == RNNT_INVALID_VALUE);               /* blank < -V */
        EXPECT(rnnt_loss_fused(logits, RNNT_F32, N, 8, tg, 3, T, U, 2, -1, -1.f, -0.5f, 1, RNNT_REDUCTION_SUM,
                               loss, red, grad, work, need, NULL) == RNNT_INVALID_VALUE);         /* lambda < 0 */
        EXPECT(rnnt_loss_fused(logits, RNNT_F32, N, 8, tg, 2, T, U, 2, -1, -1.f, 0.f, 1, RNNT_REDUCTION_SUM, loss,
                               red, grad, work, need, NULL) == RNNT_INVALID_VALUE);               /* S < max U */
        EXPECT(rnnt_loss_fused(logits, RNNT_F32, N, 8, tg, 3, T, U, 2, -1, -1.f, 0.f, 1, (rnnt_reduction)9, loss,
                               red, grad, work, need, NULL) == RNNT_INVALID_VALUE);               /* reduction */
        EXPECT(rnnt_loss_fused(logits, RNNT_F32, N, 8, tg, 3, T, U, 2, -1, -1.f, 0.f, 1, RNNT_REDUCTION_SUM, NULL,
                               red, grad, work, need, NULL) == RNNT_INVALID_VALUE);               /* loss NULL */
        EXPECT(rnnt_loss_fused(logits, RNNT_F32, N, 8, tg, 3, T, U, 2, -1, -1.f, 0.f, 1, RNNT_REDUCTION_SUM, loss,
                               red, (char *)logits + 4, work, need, NULL) == RNNT_INVALID_VALUE); /* overlap */
        EXPECT(rnnt_loss_fused(logits, RNNT_F32, N, 8, tg, 3, T, U, 2, -1, -1.f, 0.f, 1, RNNT_REDUCTION_SUM, loss,
                               red, grad, work, need - 1, NULL) == RNNT_WORKSPACE_TOO_SMALL);
        EXPECT(rnnt_loss_fused(logits, RNNT_F32, N, 8, tg, 3, T, U, 2, -1, -1.f, 0.f, 1, RNNT_REDUCTION_SUM, loss,
                               red, grad, (char *)work + 64, need, NULL) == RNNT_INVALID_VALUE);  /* alignment */
        EXPECT(rnnt_loss_padded(logits, RNNT_F32, 5, 4, 8, tg, 3, T, U, 2, -1, -1.f, 0.f, 1, RNNT_REDUCTION_SUM,
                                loss, red, grad, work, 1 << 20, NULL) == RNNT_INVALID_VALUE);     /* T > max_T */
        const int32_t ids[2] = {3, 3}, dur[2] = {2, 3}, ids_blank[1] = {7}, ids_ok[1] = {3};
        EXPECT(rnnt_multiblank_loss(logits, RNNT_F32, N, 8, tg, 3, T, U, 2, -1, 2, ids, dur, 0.f, -1.f, 0.f, 1,
                                    RNNT_REDUCTION_SUM, loss, red, grad, work, 1 << 20, NULL) == RNNT_INVALID_VALUE);
        EXPECT(rnnt_multiblank_loss(logits, RNNT_F32, N, 8, tg, 3, T, U, 2, -1, 1, ids_blank, dur, 0.f, -1.f, 0.f,
                                    1, RNNT_REDUCTION_SUM, loss, red, grad, work, 1 << 20, NULL) ==
               RNNT_INVALID_VALUE);
        EXPECT(rnnt_multiblank_loss(logits, RNNT_F32, N, 8, tg, 3, T, U, 2, -1, 1, ids_ok, dur, INFINITY, -1.f,
                                    0.f, 1, RNNT_REDUCTION_SUM, loss, red, grad, work, 1 << 20, NULL) ==
               RNNT_INVALID_VALUE);                                                                /* sigma inf */
        EXPECT(rnnt_grad_scale(grad, RNNT_F32, N + 1, 8, T, U, 2, loss, 0, work, 1 << 20, NULL) ==
               RNNT_INVALID_VALUE);
        /* allocation-free call: more than 64 samples, and a workspace beyond the fixed scratch */
        int32_t Tm[65], Um[65];
        for (int i = 0; i < 65; ++i) { Tm[i] = 2; Um[i] = 1; }
        EXPECT(rnnt_loss_fused_noalloc(logits, RNNT_F32, 65 * 4, 8, tg, 1, Tm, Um, 65, -1, -1.f, 0.f, 1,
                                       RNNT_REDUCTION_SUM, loss, red, grad, NULL, NULL) == RNNT_INVALID_VALUE);
        const int32_t Tl[1] = {20000}, Ul[1] = {1000};
        EXPECT(rnnt_loss_fused_noalloc(DEV(100), RNNT_F32, (int64_t)20000 * 1001, 8, tg, 1000, Tl, Ul, 1, -1, -1.f,
                                       0.f, 1, RNNT_REDUCTION_SUM, loss, red, DEV(200), NULL, NULL) ==
               RNNT_WORKSPACE_TOO_SMALL);
        EXPECT(rnnt_loss_fused_check(NULL, NULL, NULL) == RNNT_INVALID_VALUE);
    }

    /* timing switches with nothing recorded */
    {
        double ms[4] = {1, 1, 1, 1};
        int32_t n[4] = {1, 1, 1, 1};
        EXPECT(rnnt_timing_enable(1) == RNNT_SUCCESS);
        EXPECT(rnnt_timing_read(ms, n) == RNNT_SUCCESS);
        for (int k = 0; k < 4; ++k) EXPECT(ms[k] == 0.0 && n[k] == 0);
        EXPECT(rnnt_timing_enable(0) == RNNT_SUCCESS);
    }

    printf("host-check: %s (%d failure(s))\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
