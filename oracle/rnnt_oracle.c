/*
 * rnnt_oracle.c -- plain fp64 CPU oracle for the RNN-T loss and its gradient.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link or call this file.  Only the tests,
 * the smoke check and the bench's CPU-baseline leg use it.  It shares no code,
 * header, table or helper with the HIP implementation.
 *
 * What it computes, and where the pages define it:
 *
 *  - Alignment lattice (warp-transducer build post, section 1.1: the loss sums
 *    over every legal alignment path on a 2-D T x (U+1) grid; at each node the
 *    model either emits a vocabulary symbol or emits blank).  A path starts at
 *    node (0,0).  Blank at (t,u) moves to (t+1,u); the next label y_{u+1} at
 *    (t,u) moves to (t,u+1).  The path ends by emitting blank at (T-1,U).
 *    P(y|x) is the sum over paths of the product of the emitted symbols'
 *    probabilities and loss = -log P(y|x).
 *
 *  - Row layout (rnnt-loss-ascend README, "Main features" and the parameter
 *    table): the joiner logits of sample i are packed as T*(U+1) rows of V
 *    classes.  Rows are t-major inside a sample: row t*(U+1)+u is node (t,u).
 *
 *  - log_softmax over V at every node when fused_log_softmax is set; the raw
 *    inputs are used as log-probabilities otherwise (README parameter table).
 *
 *  - Log-space forward/backward variables (README "Value", section 3: both
 *    recursions run in the log domain; the alpha-path and beta-path losses are
 *    computed independently and cross-checked).
 *
 *  - Gradient (README "Value", section 2, the fused gradient formula).  Here it
 *    is obtained by the chain rule written out: first the derivative of the
 *    loss with respect to each log-probability the lattice uses (minus the
 *    posterior probability that the alignment takes that edge), then, when
 *    log_softmax is fused, the log_softmax Jacobian
 *        dL/dx_k = dL/dlp_k - softmax_k * sum_j dL/dlp_j.
 *
 *  - Labels (warp-transducer build post, section 5.2: the labels must not
 *    contain blank).  Reading taken: a target that is not a non-blank class
 *    (equal to blank, or outside [0,V)) is a symbol no alignment can emit, so
 *    the sample has no legal alignment: P(y|x) = 0, loss = +inf and every
 *    gradient element 0 (there is nothing to differentiate).  The result is
 *    computed that way and the call reports ORACLE_BAD_TARGET beside it.
 *
 *  - Clamp (README "Operator features": for clamp > 0 every gradient element
 *    is clipped to [-clamp, clamp]; clamp <= 0 disables it).
 *
 *  - FastEmit (the GPURNNT parameter list of the ESPnet multi-blank utilities
 *    page names fastemit_lambda as the scale of the FastEmit regularisation
 *    and defers its definition to the FastEmit paper, Yu et al. 2021).  The
 *    reading taken here is that paper's gradient rule: the derivative of the
 *    loss with respect to every label-emission log-probability is multiplied
 *    by (1 + lambda), the blank emissions keep theirs, and the reported loss
 *    value is the unregularised one.  lambda = 0 is the plain loss.
 *
 * The loops run row-major over (t,u), never along anti-diagonals, so the
 * oracle has no structure in common with the GPU kernels.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1
#define ORACLE_BAD_TARGET 2
#define ORACLE_NO_MEMORY 3

#define ORACLE_F64 0
#define ORACLE_F32 1
#define ORACLE_F16 2

/* IEEE 754 binary16 -> binary64, exact (every half is a double). */
static double half_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int mant = h & 0x3ff;
    double v;
    if (expo == 0) v = ldexp((double)mant, -24);                 /* zero / subnormal */
    else if (expo == 31) v = mant ? NAN : INFINITY;              /* inf / nan */
    else v = ldexp((double)(mant | 0x400), expo - 25);           /* normal */
    return sign ? -v : v;
}

/* Element k of row r of the sample's input, converted exactly to fp64. */
static double elem(const void *x, int dtype, long r, int V, int k)
{
    const long i = r * (long)V + k;
    if (dtype == ORACLE_F32) return (double)((const float *)x)[i];
    if (dtype == ORACLE_F16) return half_to_double(((const uint16_t *)x)[i]);
    return ((const double *)x)[i];
}

double rnnt_oracle_half_to_double(uint16_t h) { return half_to_double(h); }

/* log(exp(a) + exp(b)) with -inf handled: log(0 + 0) = -inf. */
static double log_add(double a, double b)
{
    if (a == -INFINITY) return b;
    if (b == -INFINITY) return a;
    if (a > b) return a + log1p(exp(b - a));
    return b + log1p(exp(a - b));
}

/* log-sum-exp of one row of V values, shifted by the row maximum. */
static double row_logsumexp(const void *x, int dtype, long r, int V)
{
    double m = -INFINITY;
    for (int k = 0; k < V; ++k) {
        double v = elem(x, dtype, r, V, k);
        if (v > m) m = v;
    }
    if (m == -INFINITY) return -INFINITY;
    double s = 0.0;
    for (int k = 0; k < V; ++k) s += exp(elem(x, dtype, r, V, k) - m);
    return m + log(s);
}

/*
 * One sample.
 *   x        T*(U+1) rows of V values, row-major, of type dtype (ORACLE_F64,
 *            _F32 or _F16); logits, or log-probs when fused == 0.  Values are
 *            converted exactly to fp64 as they are read.
 *   y        U target labels; one outside [0,V) or equal to blank makes the
 *            sample impossible (see "Labels" above).
 *   blank    already normalised to [0,V).
 *   grad_rows, n_grad_rows   sample-local rows whose gradient is wanted
 *            (NULL with n_grad_rows < 0 means every row, in order).
 *   fastemit_lambda  >= 0; scales the label-emission derivatives by
 *            (1 + fastemit_lambda) (0: the plain gradient).
 *   grad     optional n x V output (n = rows requested): d loss / d x of
 *            those rows, clamped if clamp > 0.
 *   alpha, beta  optional T*(U+1) outputs of the log forward / backward
 *            variables (beta(t,u) includes the emissions at (t,u) onwards,
 *            so beta(0,0) = log P(y|x)).
 *   loss_alpha, loss_beta  -log P(y|x) from each recursion.
 * Returns ORACLE_OK, ORACLE_BAD_TARGET (outputs computed, the sample has no
 * alignment because of a label) or an error code (outputs untouched).
 */
int rnnt_oracle_sample_ex(const void *x, int dtype, int T, int U, int V, const int *y, int blank, int fused,
                          double clamp, double fastemit_lambda, const int64_t *grad_rows, long n_grad_rows,
                          double *grad, double *alpha_out, double *beta_out, double *loss_alpha,
                          double *loss_beta)
{
    if (T < 1 || U < 0 || V < 1 || blank < 0 || blank >= V) return ORACLE_BAD_ARGS;
    if (!(fastemit_lambda >= 0.0) || isinf(fastemit_lambda)) return ORACLE_BAD_ARGS;
    if (dtype != ORACLE_F64 && dtype != ORACLE_F32 && dtype != ORACLE_F16) return ORACLE_BAD_ARGS;
    int bad_target = 0;
    for (int u = 0; u < U; ++u)
        if (y[u] < 0 || y[u] >= V || y[u] == blank) bad_target = 1;

    const int U1 = U + 1;
    const long cells = (long)T * U1;
    double *lse = malloc(sizeof(double) * cells);   /* per-node log normaliser */
    double *lpb = malloc(sizeof(double) * cells);   /* log P(blank | t,u) */
    double *lpy = malloc(sizeof(double) * cells);   /* log P(y_{u+1} | t,u), u < U */
    double *al = malloc(sizeof(double) * cells);
    double *be = malloc(sizeof(double) * cells);
    if (!lse || !lpb || !lpy || !al || !be) {
        free(lse); free(lpb); free(lpy); free(al); free(be);
        return ORACLE_NO_MEMORY;
    }

    /* Step 1: per-node normaliser and the two log-probs the lattice uses. */
    for (int t = 0; t < T; ++t) {
        for (int u = 0; u <= U; ++u) {
            long c = (long)t * U1 + u;
            lse[c] = fused ? row_logsumexp(x, dtype, c, V) : 0.0;
            lpb[c] = elem(x, dtype, c, V, blank) - lse[c];
            const int label_ok = (u < U) && y[u] >= 0 && y[u] < V && y[u] != blank;
            lpy[c] = label_ok ? elem(x, dtype, c, V, y[u]) - lse[c] : -INFINITY;
        }
    }

    /* Step 2: forward variable, alpha(t,u) = log of the summed probability
     * of all partial paths from (0,0) that arrive at (t,u). */
    for (int t = 0; t < T; ++t) {
        for (int u = 0; u <= U; ++u) {
            long c = (long)t * U1 + u;
            if (t == 0 && u == 0) { al[c] = 0.0; continue; }
            double from_blank = (t > 0) ? al[c - U1] + lpb[c - U1] : -INFINITY;
            double from_label = (u > 0) ? al[c - 1] + lpy[c - 1] : -INFINITY;
            al[c] = log_add(from_blank, from_label);
        }
    }
    const long last = (long)(T - 1) * U1 + U;
    double logz_alpha = al[last] + lpb[last];

    /* Step 3: backward variable, beta(t,u) = log of the summed probability
     * of all path suffixes from (t,u), the final blank included. */
    for (int t = T - 1; t >= 0; --t) {
        for (int u = U; u >= 0; --u) {
            long c = (long)t * U1 + u;
            if (c == last) { be[c] = lpb[c]; continue; }
            double via_blank = (t < T - 1) ? be[c + U1] + lpb[c] : -INFINITY;
            double via_label = (u < U) ? be[c + 1] + lpy[c] : -INFINITY;
            be[c] = log_add(via_blank, via_label);
        }
    }
    double logz_beta = be[0];

    if (loss_alpha) *loss_alpha = -logz_alpha;
    if (loss_beta) *loss_beta = -logz_beta;
    if (alpha_out) memcpy(alpha_out, al, sizeof(double) * cells);
    if (beta_out) memcpy(beta_out, be, sizeof(double) * cells);

    /* Step 4: gradient of the requested rows, by the chain rule. */
    if (grad) {
        const double logz = logz_beta;
        const long n = (grad_rows == NULL || n_grad_rows < 0) ? cells : n_grad_rows;
        for (long i = 0; i < n; ++i) {
            long c = (grad_rows == NULL || n_grad_rows < 0) ? i : (long)grad_rows[i];
            double *g = grad + i * V;
            if (c < 0 || c >= cells) {
                for (int k = 0; k < V; ++k) g[k] = NAN;
                continue;
            }
            int t = (int)(c / U1), u = (int)(c % U1);
            /* d loss / d lp(blank) and d loss / d lp(y_{u+1}) at this node:
             * minus the posterior probability of taking that edge. */
            double d_blank = 0.0, d_label = 0.0;
            if (logz != -INFINITY) {
                if (t < T - 1)
                    d_blank = -exp(al[c] + lpb[c] + be[c + U1] - logz);
                else if (u == U)
                    d_blank = -exp(al[c] + lpb[c] - logz);
                if (u < U)
                    d_label = -exp(al[c] + lpy[c] + be[c + 1] - logz);
            }
            /* FastEmit: the label edge's derivative weighted by (1 + lambda). */
            d_label *= 1.0 + fastemit_lambda;
            for (int k = 0; k < V; ++k) g[k] = 0.0;
            g[blank] += d_blank;
            if (u < U && d_label != 0.0) g[y[u]] += d_label;   /* non-zero only for a valid label */
            if (fused) {
                double sum_d = d_blank + d_label;
                for (int k = 0; k < V; ++k) {
                    double p = (lse[c] == -INFINITY) ? 0.0 : exp(elem(x, dtype, c, V, k) - lse[c]);
                    g[k] -= p * sum_d;
                }
            }
            if (clamp > 0.0) {
                for (int k = 0; k < V; ++k) {
                    if (g[k] > clamp) g[k] = clamp;
                    if (g[k] < -clamp) g[k] = -clamp;
                }
            }
        }
    }

    free(lse); free(lpb); free(lpy); free(al); free(be);
    return bad_target ? ORACLE_BAD_TARGET : ORACLE_OK;
}

/* fp64 input, gradient of every row (the form the pins use). */
int rnnt_oracle_sample(const double *x, int T, int U, int V, const int *y, int blank, int fused, double clamp,
                       double *grad, double *alpha_out, double *beta_out, double *loss_alpha, double *loss_beta)
{
    return rnnt_oracle_sample_ex(x, ORACLE_F64, T, U, V, y, blank, fused, clamp, 0.0, NULL, -1, grad, alpha_out,
                                 beta_out, loss_alpha, loss_beta);
}

/*
 * Multi-blank transducer (the ESPnet compute_multiblank_grad_kernel page:
 * activations over V + 1 + num_big_blanks classes, a list of big-blank
 * durations, and sigma, the hyper-parameter of logit under-normalisation;
 * the page defers the mathematics to the multi-blank transducer paper).
 * Reading taken:
 *   - besides the standard blank (t,u) -> (t+1,u) and the next label
 *     (t,u) -> (t,u+1), big blank i, class bb_id[i], moves (t,u) -> (t+d_i,u)
 *     with d_i = bb_dur[i] >= 1;
 *   - every emission's log-probability is lowered by sigma:
 *     lp(t,u,k) = x_k - logsumexp(x) - sigma (fused) or x_k - sigma;
 *   - an alignment ends when a blank of any kind moves it from (t,U) to
 *     exactly t = T; blanks that would pass T, or reach T with u < U, are not
 *     part of any alignment;
 *   - loss = -log of the summed alignment probability; the gradient is its
 *     derivative (with the FastEmit weight on the label edges, as above);
 *   - a label that is a blank of either kind or outside [0,V) admits no
 *     alignment (as above): loss +inf, gradient 0, ORACLE_BAD_TARGET.
 * nb = 0 and sigma = 0 is the plain transducer loss.
 */
int rnnt_oracle_multiblank_sample(const void *x, int dtype, int T, int U, int V, const int *y, int blank, int nb,
                                  const int *bb_id, const int *bb_dur, double sigma, int fused, double clamp,
                                  double fastemit_lambda, double *grad, double *loss_alpha, double *loss_beta)
{
    if (T < 1 || U < 0 || V < 1 || blank < 0 || blank >= V || nb < 0) return ORACLE_BAD_ARGS;
    if (dtype != ORACLE_F64 && dtype != ORACLE_F32 && dtype != ORACLE_F16) return ORACLE_BAD_ARGS;
    if (!(fastemit_lambda >= 0.0) || isinf(fastemit_lambda) || !isfinite(sigma)) return ORACLE_BAD_ARGS;
    for (int i = 0; i < nb; ++i) {
        if (bb_id[i] < 0 || bb_id[i] >= V || bb_id[i] == blank || bb_dur[i] < 1) return ORACLE_BAD_ARGS;
        for (int j = 0; j < i; ++j)
            if (bb_id[j] == bb_id[i]) return ORACLE_BAD_ARGS;
    }
    int bad_target = 0;
    for (int u = 0; u < U; ++u) {
        if (y[u] < 0 || y[u] >= V || y[u] == blank) bad_target = 1;
        for (int i = 0; i < nb; ++i)
            if (y[u] == bb_id[i]) bad_target = 1;
    }

    const int U1 = U + 1;
    const long cells = (long)T * U1;
    const int nbb = nb > 0 ? nb : 1;
    double *lse = malloc(sizeof(double) * cells);
    double *lpb = malloc(sizeof(double) * cells);
    double *lpy = malloc(sizeof(double) * cells);
    double *lpg = malloc(sizeof(double) * cells * nbb);   /* big blanks: lpg[c * nb + i] */
    double *al = malloc(sizeof(double) * cells);
    double *be = malloc(sizeof(double) * cells);
    if (!lse || !lpb || !lpy || !lpg || !al || !be) {
        free(lse); free(lpb); free(lpy); free(lpg); free(al); free(be);
        return ORACLE_NO_MEMORY;
    }

    /* Per-node log-probabilities of the edges the lattice uses. */
    for (long c = 0; c < cells; ++c) {
        const int u = (int)(c % U1);
        lse[c] = fused ? row_logsumexp(x, dtype, c, V) : 0.0;
        lpb[c] = elem(x, dtype, c, V, blank) - lse[c] - sigma;
        int label_ok = (u < U) && y[u] >= 0 && y[u] < V && y[u] != blank;
        for (int i = 0; i < nb; ++i) label_ok = label_ok && y[u] != bb_id[i];
        lpy[c] = label_ok ? elem(x, dtype, c, V, y[u]) - lse[c] - sigma : -INFINITY;
        for (int i = 0; i < nb; ++i) lpg[c * nb + i] = elem(x, dtype, c, V, bb_id[i]) - lse[c] - sigma;
    }

    /* Forward: alpha(t,u) sums the partial alignments that arrive at (t,u). */
    for (int t = 0; t < T; ++t) {
        for (int u = 0; u <= U; ++u) {
            const long c = (long)t * U1 + u;
            if (t == 0 && u == 0) { al[c] = 0.0; continue; }
            double a = -INFINITY;
            if (t > 0) a = log_add(a, al[c - U1] + lpb[c - U1]);
            if (u > 0) a = log_add(a, al[c - 1] + lpy[c - 1]);
            for (int i = 0; i < nb; ++i) {
                const int d = bb_dur[i];
                if (t >= d) a = log_add(a, al[c - (long)d * U1] + lpg[(c - (long)d * U1) * nb + i]);
            }
            al[c] = a;
        }
    }
    double logz_alpha = al[(long)(T - 1) * U1 + U] + lpb[(long)(T - 1) * U1 + U];
    for (int i = 0; i < nb; ++i) {
        const int d = bb_dur[i];
        if (T - d >= 0) {
            const long c = (long)(T - d) * U1 + U;
            logz_alpha = log_add(logz_alpha, al[c] + lpg[c * nb + i]);
        }
    }

    /* Backward: beta(t,u) sums the alignment suffixes from (t,u), the final
     * blank included; a blank reaching t = T counts only from u = U. */
    for (int t = T - 1; t >= 0; --t) {
        for (int u = U; u >= 0; --u) {
            const long c = (long)t * U1 + u;
            double b = -INFINITY;
            if (t + 1 < T) b = log_add(b, be[c + U1] + lpb[c]);
            else if (u == U) b = log_add(b, lpb[c]);
            if (u < U) b = log_add(b, be[c + 1] + lpy[c]);
            for (int i = 0; i < nb; ++i) {
                const int d = bb_dur[i];
                if (t + d < T) b = log_add(b, be[c + (long)d * U1] + lpg[c * nb + i]);
                else if (t + d == T && u == U) b = log_add(b, lpg[c * nb + i]);
            }
            be[c] = b;
        }
    }
    const double logz = be[0];
    if (loss_alpha) *loss_alpha = -logz_alpha;
    if (loss_beta) *loss_beta = -logz;

    if (grad) {
        for (long c = 0; c < cells; ++c) {
            const int t = (int)(c / U1), u = (int)(c % U1);
            double *g = grad + c * V;
            for (int k = 0; k < V; ++k) g[k] = 0.0;
            double sum_d = 0.0;
            if (logz != -INFINITY) {
                /* d loss / d lp of each edge leaving (t,u): minus its posterior. */
                double nb_blank = -INFINITY;            /* log beta after the standard blank */
                if (t + 1 < T) nb_blank = be[c + U1];
                else if (u == U) nb_blank = 0.0;
                const double d_blank = -exp(al[c] + lpb[c] + nb_blank - logz);
                g[blank] += d_blank;
                sum_d += d_blank;
                if (u < U) {
                    const double d_label = -(1.0 + fastemit_lambda) * exp(al[c] + lpy[c] + be[c + 1] - logz);
                    if (d_label != 0.0) g[y[u]] += d_label;   /* non-zero only for a valid label */
                    sum_d += d_label;
                }
                for (int i = 0; i < nb; ++i) {
                    const int d = bb_dur[i];
                    double nxt = -INFINITY;
                    if (t + d < T) nxt = be[c + (long)d * U1];
                    else if (t + d == T && u == U) nxt = 0.0;
                    const double d_big = -exp(al[c] + lpg[c * nb + i] + nxt - logz);
                    g[bb_id[i]] += d_big;
                    sum_d += d_big;
                }
            }
            if (fused) {
                for (int k = 0; k < V; ++k) {
                    const double p = (lse[c] == -INFINITY) ? 0.0 : exp(elem(x, dtype, c, V, k) - lse[c]);
                    g[k] -= p * sum_d;
                }
            }
            if (clamp > 0.0) {
                for (int k = 0; k < V; ++k) {
                    if (g[k] > clamp) g[k] = clamp;
                    if (g[k] < -clamp) g[k] = -clamp;
                }
            }
        }
    }
    free(lse); free(lpb); free(lpy); free(lpg); free(al); free(be);
    return bad_target ? ORACLE_BAD_TARGET : ORACLE_OK;
}
