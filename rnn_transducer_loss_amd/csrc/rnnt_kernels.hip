// gfx950 kernels of librnnt: the fused RNN-T loss, forward and backward.
//
// Pass structure (rnnt-loss-ascend README, "Architecture", kernel steps 1-5):
//   rowstats   step 1   per packed row: log-sum-exp over V (fused) and the two
//                       log-probs the lattice uses, log P(blank) and
//                       log P(y_{u+1}), written into the skewed per-node arrays.
//   alpha_beta steps 2-4 one workgroup per sample; wave 0 runs the forward
//                       (alpha) recursion and wave 1 the backward (beta)
//                       recursion, each one anti-diagonal per step (README
//                       "Operator features": every node of an anti-diagonal
//                       has its inputs ready), fp64 log-space accumulators;
//                       the two losses are cross-checked.
//   grad       step 5   per packed row: the fused gradient (README "Value"
//                       section 2), clamp, reduction scale, one write of grad.
//   reduce              none / mean / sum of the per-sample losses.
//
// Nothing here is a dense contraction, so no MFMA: the row passes are bound by
// HBM bandwidth (coalesced 16-byte accesses, wave-shuffle reductions) and the
// recursion by the latency of its T+U dependent steps.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "rnnt_internal.h"

namespace rnnt {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr double kLog2eD = 1.4426950408889634074;
constexpr double kNegInfD = -__builtin_inf();
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- element I/O
template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kVec = 4;  // 16 bytes
    __device__ static float load1(const float *p) { return *p; }
    __device__ static void store1(float *p, float v) { *p = v; }
    __device__ static void loadv(const float *p, float *out) {
        const float4 v = *reinterpret_cast<const float4 *>(p);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
    __device__ static void storev(float *p, const float *in) {
        *reinterpret_cast<float4 *>(p) = make_float4(in[0], in[1], in[2], in[3]);
    }
};
template <> struct Elem<_Float16> {
    static constexpr int kVec = 8;  // 16 bytes
    __device__ static float load1(const _Float16 *p) { return (float)*p; }
    __device__ static void store1(_Float16 *p, float v) { *p = (_Float16)v; }
    __device__ static void loadv(const _Float16 *p, float *out) {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        const h8 v = *reinterpret_cast<const h8 *>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
    }
    __device__ static void storev(_Float16 *p, const float *in) {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        h8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (_Float16)in[i];
        *reinterpret_cast<h8 *>(p) = v;
    }
};

template <typename T, int VEC> __device__ __forceinline__ void load_n(const T *p, float *out) {
    if constexpr (VEC == 1) out[0] = Elem<T>::load1(p);
    else Elem<T>::loadv(p, out);
}
template <typename T, int VEC> __device__ __forceinline__ void store_n(T *p, const float *in) {
    if constexpr (VEC == 1) Elem<T>::store1(p, in[0]);
    else Elem<T>::storev(p, in);
}

// Combine two (max, sum of exp(x - max)) partial states.
__device__ __forceinline__ void lse_merge(float &m, float &s, float mo, float so) {
    const float mn = fmaxf(m, mo);
    const float mr = (mn == kNegInf) ? 0.f : mn;
    s = s * exp2_fast((m - mr) * kLog2e) + so * exp2_fast((mo - mr) * kLog2e);
    m = mn;
}

// log(exp(a) + exp(b)) in fp64 with the correction term in fp32: the argument
// of exp is <= 0 and log1p's argument is in [0, 1], so fp32 costs at most a
// few 1e-8 absolute per step while the fp64 accumulator keeps the large part.
__device__ __forceinline__ double log_add(double a, double b) {
    const double mx = fmax(a, b);
    const double mn = fmin(a, b);
    const float e = exp2_fast((float)(mn - mx) * kLog2e);
    const float l = log2_fast(1.0f + e) * kLn2;
    return (mn == kNegInfD) ? mx : mx + (double)l;
}

// -------------------------------------------------------------- row geometry
// Each row is handled by G consecutive lanes; a wave handles 64/G rows at a
// time and a 256-thread workgroup 4*64/G rows.  Element k of a row goes to
// lane (k / VEC) % G, so every access instruction of a group is contiguous.
template <typename T, int VEC, int G, typename F>
__device__ __forceinline__ void for_rows(const ChunkDesc &c, F &&body) {
    constexpr int RPW = 64 / G;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane / G;
    for (int base = wave * RPW; base < c.row_count; base += 4 * RPW) {
        const int r = base + grp;
        body(r < c.row_count, c.row_begin + (r < c.row_count ? r : 0));
    }
}

// ------------------------------------------------------------- K1: rowstats
template <typename T, int VEC, int G>
__global__ __launch_bounds__(256) void k_rowstats(const T *__restrict__ logits, int V, int blank,
                                                  const SampleDesc *__restrict__ desc,
                                                  const ChunkDesc *__restrict__ chunks,
                                                  const int32_t *__restrict__ targets, int S,
                                                  float *__restrict__ den, float *__restrict__ lpb,
                                                  float *__restrict__ lpy, uint32_t *status) {
    const ChunkDesc c = chunks[blockIdx.x];
    const SampleDesc d = desc[c.sample];
    const int U1 = d.U + 1;
    const int sub = (threadIdx.x & 63) & (G - 1);
    const int nvec = V / VEC;
    for_rows<T, VEC, G>(c, [&](bool active, int lr) {
        const int64_t row = d.row_off + lr;
        const T *p = logits + row * (int64_t)V;
        float m = kNegInf, s = 0.f;
        if (active) {
            int i = sub;
            for (; i + 3 * G < nvec; i += 4 * G) {
                float x[4][VEC];
#pragma unroll
                for (int q = 0; q < 4; ++q) load_n<T, VEC>(p + (int64_t)(i + q * G) * VEC, x[q]);
                float vm = x[0][0];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) vm = fmaxf(vm, x[q][e]);
                const float mn = fmaxf(m, vm);
                const float mr = (mn == kNegInf) ? 0.f : mn;
                const float nm = -mr * kLog2e;
                float acc = s * exp2_fast((m - mr) * kLog2e);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc += exp2_fast(fmaf(x[q][e], kLog2e, nm));
                s = acc;
                m = mn;
            }
            for (; i < nvec; i += G) {
                float x[VEC];
                load_n<T, VEC>(p + (int64_t)i * VEC, x);
                float vm = x[0];
#pragma unroll
                for (int e = 1; e < VEC; ++e) vm = fmaxf(vm, x[e]);
                const float mn = fmaxf(m, vm);
                const float mr = (mn == kNegInf) ? 0.f : mn;
                const float nm = -mr * kLog2e;
                float acc = s * exp2_fast((m - mr) * kLog2e);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc += exp2_fast(fmaf(x[e], kLog2e, nm));
                s = acc;
                m = mn;
            }
        }
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) {
            const float mo = __shfl_xor(m, off, 64);
            const float so = __shfl_xor(s, off, 64);
            lse_merge(m, s, mo, so);
        }
        if (active && sub == 0) {
            const int t = lr / U1;
            const int u = lr - t * U1;
            const float dn = (m == kNegInf) ? kNegInf : m + log2_fast(s) * kLn2;
            den[row] = dn;
            const int64_t slot = d.slot_off + (int64_t)(t + u) * U1 + u;
            const bool dead = (dn == kNegInf);
            lpb[slot] = dead ? kNegInf : Elem<T>::load1(p + blank) - dn;
            float ly = kNegInf;
            if (u < d.U) {
                const int y = targets[(int64_t)d.index * S + u];
                const bool in_range = (y >= 0) && (y < V);
                if (!in_range || y == blank) atomicOr(status, (uint32_t)RNNT_DEV_BAD_TARGET);
                if (in_range && !dead) ly = Elem<T>::load1(p + y) - dn;
            }
            lpy[slot] = ly;
        }
    });
}

// Non-fused inputs are already log-probabilities: gather the two values only.
template <typename T>
__global__ __launch_bounds__(256) void k_gather(const T *__restrict__ logits, int V, int blank,
                                                const SampleDesc *__restrict__ desc,
                                                const ChunkDesc *__restrict__ chunks,
                                                const int32_t *__restrict__ targets, int S,
                                                float *__restrict__ lpb, float *__restrict__ lpy,
                                                uint32_t *status) {
    const ChunkDesc c = chunks[blockIdx.x];
    const SampleDesc d = desc[c.sample];
    const int U1 = d.U + 1;
    for (int r = threadIdx.x; r < c.row_count; r += blockDim.x) {
        const int lr = c.row_begin + r;
        const int t = lr / U1;
        const int u = lr - t * U1;
        const T *p = logits + (d.row_off + lr) * (int64_t)V;
        const int64_t slot = d.slot_off + (int64_t)(t + u) * U1 + u;
        lpb[slot] = Elem<T>::load1(p + blank);
        float ly = kNegInf;
        if (u < d.U) {
            const int y = targets[(int64_t)d.index * S + u];
            const bool in_range = (y >= 0) && (y < V);
            if (!in_range || y == blank) atomicOr(status, (uint32_t)RNNT_DEV_BAD_TARGET);
            if (in_range) ly = Elem<T>::load1(p + y);
        }
        lpy[slot] = ly;
    }
}

// ----------------------------------------------------- K2: alpha/beta sweeps
// Lane l of the wave owns lattice columns u = l + 64*j, j < C.  Anti-diagonal
// n = t+u holds the nodes whose predecessors all lie on diagonal n-1, so one
// step per diagonal advances every node of it at once.  The per-slot
// log-probs of the next PF diagonals are kept in flight in a register ring.
template <int C>
__device__ __forceinline__ void load_diag(const float *__restrict__ lpb, const float *__restrict__ lpy, int n,
                                          int nd, int U1, int lane, float *rb, float *ry) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
        const int u = lane + 64 * j;
        const bool ok = (n >= 0) && (n < nd) && (u < U1);
        const int64_t s = ok ? (int64_t)n * U1 + u : 0;
        rb[j] = ok ? lpb[s] : 0.f;
        ry[j] = ok ? lpy[s] : 0.f;
    }
}

template <int C> __device__ __forceinline__ double pick(const double (&v)[C], int j) {
    double r = v[0];
#pragma unroll
    for (int q = 1; q < C; ++q) r = (q == j) ? v[q] : r;
    return r;
}

// Forward variable: alpha(t,u) = log-sum of all partial alignments reaching
// (t,u).  Messages leaving diagonal n-1: mb = alpha + log P(blank) towards
// (t+1,u) (same lane), my = alpha + log P(y_{u+1}) towards (t,u+1) (next lane).
template <int C, int PF>
__device__ void sweep_alpha(int T, int U, const float *__restrict__ lpb, const float *__restrict__ lpy,
                            double *__restrict__ alpha, double *logz) {
    const int lane = threadIdx.x & 63;
    const int U1 = U + 1;
    const int nd = T + U;
    double mb[C], my[C];
#pragma unroll
    for (int j = 0; j < C; ++j) { mb[j] = kNegInfD; my[j] = kNegInfD; }
    float rb[PF][C], ry[PF][C];
#pragma unroll
    for (int p = 0; p < PF; ++p) load_diag<C>(lpb, lpy, p, nd, U1, lane, rb[p], ry[p]);
    for (int n0 = 0; n0 < nd; n0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int n = n0 + p;
            if (n < nd) {
                const int ulo = max(0, n - T + 1);
                const int uhi = min(n, U);
                double inl[C];
#pragma unroll
                for (int j = 0; j < C; ++j) {
                    const double up = __shfl_up(my[j], 1, 64);
                    const double wrap = (j > 0) ? __shfl(my[j > 0 ? j - 1 : 0], 63, 64) : kNegInfD;
                    inl[j] = (lane == 0) ? wrap : up;
                }
#pragma unroll
                for (int j = 0; j < C; ++j) {
                    const int u = lane + 64 * j;
                    const bool valid = (u >= ulo) && (u <= uhi);
                    const double a = (n == 0) ? 0.0 : log_add(mb[j], inl[j]);
                    if (valid) alpha[(int64_t)n * U1 + u] = a;
                    mb[j] = valid ? a + (double)rb[p][j] : kNegInfD;
                    my[j] = (valid && u < U) ? a + (double)ry[p][j] : kNegInfD;
                }
                load_diag<C>(lpb, lpy, n + PF, nd, U1, lane, rb[p], ry[p]);
            }
        }
    }
    // The last diagonal holds only (T-1, U); its blank message is log P(y|x).
    const double v = pick<C>(mb, U >> 6);
    const double z = __shfl(v, U & 63, 64);
    if (lane == 0) *logz = z;
}

// Backward variable: beta(t,u) = log-sum of all alignment suffixes from (t,u),
// including the final blank, so beta(0,0) = log P(y|x).
template <int C, int PF>
__device__ void sweep_beta(int T, int U, const float *__restrict__ lpb, const float *__restrict__ lpy,
                           double *__restrict__ beta, double *logz) {
    const int lane = threadIdx.x & 63;
    const int U1 = U + 1;
    const int nd = T + U;
    double pv[C];
#pragma unroll
    for (int j = 0; j < C; ++j) pv[j] = kNegInfD;
    float rb[PF][C], ry[PF][C];
#pragma unroll
    for (int p = 0; p < PF; ++p) load_diag<C>(lpb, lpy, nd - 1 - p, nd, U1, lane, rb[p], ry[p]);
    for (int n0 = nd - 1; n0 >= 0; n0 -= PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int n = n0 - p;
            if (n >= 0) {
                const int ulo = max(0, n - T + 1);
                const int uhi = min(n, U);
                double nx[C];
#pragma unroll
                for (int j = 0; j < C; ++j) {
                    const double dn = __shfl_down(pv[j], 1, 64);
                    const double wrap = (j + 1 < C) ? __shfl(pv[j + 1 < C ? j + 1 : j], 0, 64) : kNegInfD;
                    nx[j] = (lane == 63) ? wrap : dn;
                }
#pragma unroll
                for (int j = 0; j < C; ++j) {
                    const int u = lane + 64 * j;
                    const bool valid = (u >= ulo) && (u <= uhi);
                    const double b = (n == nd - 1)
                                         ? (double)rb[p][j]
                                         : log_add(pv[j] + (double)rb[p][j], nx[j] + (double)ry[p][j]);
                    if (valid) beta[(int64_t)n * U1 + u] = b;
                    pv[j] = valid ? b : kNegInfD;
                }
                load_diag<C>(lpb, lpy, n - PF, nd, U1, lane, rb[p], ry[p]);
            }
        }
    }
    const double z = __shfl(pv[0], 0, 64);
    if (lane == 0) *logz = z;
}

template <int C, int PF>
__device__ void run_sweeps(const SampleDesc &d, const float *lpb, const float *lpy, double *alpha,
                           double *beta, double *shz) {
    const int wave = threadIdx.x >> 6;
    if (wave == 0)
        sweep_alpha<C, PF>(d.T, d.U, lpb + d.slot_off, lpy + d.slot_off, alpha + d.slot_off, &shz[0]);
    else
        sweep_beta<C, PF>(d.T, d.U, lpb + d.slot_off, lpy + d.slot_off, beta + d.slot_off, &shz[1]);
}

__global__ __launch_bounds__(128) void k_alpha_beta(const SampleDesc *__restrict__ desc,
                                                    const int32_t *__restrict__ order,
                                                    const float *__restrict__ lpb, const float *__restrict__ lpy,
                                                    double *__restrict__ alpha, double *__restrict__ beta,
                                                    float *__restrict__ loss, uint32_t *status) {
    __shared__ double shz[2];
    const SampleDesc d = desc[order[blockIdx.x]];
    const int U1 = d.U + 1;
    if (U1 <= 64) run_sweeps<1, 8>(d, lpb, lpy, alpha, beta, shz);
    else if (U1 <= 128) run_sweeps<2, 8>(d, lpb, lpy, alpha, beta, shz);
    else if (U1 <= 256) run_sweeps<4, 8>(d, lpb, lpy, alpha, beta, shz);
    else if (U1 <= 512) run_sweeps<8, 4>(d, lpb, lpy, alpha, beta, shz);
    else run_sweeps<16, 4>(d, lpb, lpy, alpha, beta, shz);
    __syncthreads();
    if (threadIdx.x == 0) {
        const double la = -shz[0];
        const double lb = -shz[1];
        loss[d.index] = (float)lb;
        const bool agree = (la == lb) || (fabs(la - lb) <= 1e-4 * fmax(1.0, fabs(lb)));
        if (!agree) atomicOr(status, (uint32_t)RNNT_DEV_LOSS_MISMATCH);
    }
}

// ------------------------------------------------------------ K3: gradient
// g_k = P(k|t,u) * occ(t,u) - [k = blank] flow_b - [k = y_{u+1}] flow_y, where
// occ = exp(alpha + beta - logZ) and the flows are the posterior
// probabilities of leaving (t,u) by blank or by the next label.  P * occ is
// evaluated as exp2(x * log2(e) + shift) with one per-row shift.
struct RowTerms {
    float shift2;  // log2 of (occ * scale / sum_k exp(x_k)), or -inf
    float fb;      // scaled blank flow
    float fy;      // scaled label flow
    int y;         // next label, -1 at u = U or when invalid
};

__device__ __forceinline__ RowTerms row_terms(const SampleDesc &d, int lr, int V, float den_row, double logz,
                                              const float *__restrict__ lpb, const float *__restrict__ lpy,
                                              const double *__restrict__ alpha, const double *__restrict__ beta,
                                              const int32_t *__restrict__ targets, int S, float log2_scale,
                                              float scale, bool fused) {
    const int U1 = d.U + 1;
    const int t = lr / U1;
    const int u = lr - t * U1;
    const int64_t s = d.slot_off + (int64_t)(t + u) * U1 + u;
    const double a = alpha[s];
    double lb = kNegInfD, ly = kNegInfD, lo = kNegInfD;
    if (logz != kNegInfD) {
        lo = a + beta[s] - logz;
        if (t < d.T - 1) lb = a + (double)lpb[s] + beta[s + U1] - logz;
        else if (u == d.U) lb = a + (double)lpb[s] - logz;
        if (u < d.U) ly = a + (double)lpy[s] + beta[s + U1 + 1] - logz;
    }
    RowTerms r;
    r.shift2 = fused ? (float)((lo - (double)den_row) * kLog2eD) + log2_scale : kNegInf;
    r.fb = exp2_fast((float)(lb * kLog2eD)) * scale;
    r.fy = exp2_fast((float)(ly * kLog2eD)) * scale;
    int y = -1;
    if (u < d.U) {
        y = targets[(int64_t)d.index * S + u];
        if (y < 0 || y >= V) y = -1;
    }
    r.y = y;
    return r;
}

template <typename T, int VEC, int G, bool FUSED>
__global__ __launch_bounds__(256) void k_grad(const T *logits, T *grad, int V, int blank,
                                              float clamp, float scale, float log2_scale,
                                              const SampleDesc *__restrict__ desc,
                                              const ChunkDesc *__restrict__ chunks, int n_chunks,
                                              const int32_t *__restrict__ targets, int S,
                                              const float *__restrict__ den, const float *__restrict__ lpb,
                                              const float *__restrict__ lpy, const double *__restrict__ alpha,
                                              const double *__restrict__ beta) {
    // Chunks run in the reverse of the rowstats order, so the rows read last
    // by that pass, the likeliest to still be cached, are read again first.
    const ChunkDesc c = chunks[n_chunks - 1 - blockIdx.x];
    const SampleDesc d = desc[c.sample];
    const double logz = beta[d.slot_off];  // beta(0,0)
    const int sub = (threadIdx.x & 63) & (G - 1);
    const int nvec = V / VEC;
    const float cl = clamp * scale;
    const bool do_clamp = clamp > 0.f;
    for_rows<T, VEC, G>(c, [&](bool active, int lr) {
        if (!active) return;
        const int64_t row = d.row_off + lr;
        const RowTerms rt = row_terms(d, lr, V, FUSED ? den[row] : 0.f, logz, lpb, lpy, alpha, beta, targets, S,
                                      log2_scale, scale, FUSED);
        const T *src = logits + row * (int64_t)V;
        T *dst = grad + row * (int64_t)V;
        for (int i = sub; i < nvec; i += G) {
            float x[VEC];
            if constexpr (FUSED) load_n<T, VEC>(src + (int64_t)i * VEC, x);
            float g[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int k = i * VEC + e;
                float v = 0.f;
                if constexpr (FUSED) v = exp2_fast(fmaf(x[e], kLog2e, rt.shift2));
                v -= (k == blank) ? rt.fb : 0.f;
                v -= (k == rt.y) ? rt.fy : 0.f;
                if (do_clamp) v = fminf(fmaxf(v, -cl), cl);
                g[e] = v;
            }
            store_n<T, VEC>(dst + (int64_t)i * VEC, g);
        }
    });
}

// --------------------------------------------------------------- reduction
__global__ __launch_bounds__(64) void k_reduce(const float *__restrict__ loss, int B, int mean,
                                               float *__restrict__ out) {
    double s = 0.0;
    for (int i = threadIdx.x; i < B; i += 64) s += (double)loss[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (threadIdx.x == 0) out[0] = (float)(mean ? s / (double)B : s);
}

// Upstream-gradient scaling of an already written gradient.
template <typename T, int VEC, int G>
__global__ __launch_bounds__(256) void k_grad_scale(T *grad, int V, const SampleDesc *__restrict__ desc,
                                                    const ChunkDesc *__restrict__ chunks,
                                                    const float *__restrict__ scale, int per_sample) {
    const ChunkDesc c = chunks[blockIdx.x];
    const SampleDesc d = desc[c.sample];
    const float f = scale[per_sample ? d.index : 0];
    if (f == 1.0f) return;
    const int sub = (threadIdx.x & 63) & (G - 1);
    const int nvec = V / VEC;
    for_rows<T, VEC, G>(c, [&](bool active, int lr) {
        if (!active) return;
        T *p = grad + (d.row_off + lr) * (int64_t)V;
        for (int i = sub; i < nvec; i += G) {
            float x[VEC];
            load_n<T, VEC>(p + (int64_t)i * VEC, x);
#pragma unroll
            for (int e = 0; e < VEC; ++e) x[e] *= f;
            store_n<T, VEC>(p + (int64_t)i * VEC, x);
        }
    });
}

// ------------------------------------------------------------- dispatchers
template <typename T, int VEC, int G> struct Tag {
    using type = T;
    static constexpr int vec = VEC;
    static constexpr int g = G;
};

template <typename Fn> hipError_t with_geom(int esize, int vec, int G, Fn &&fn) {
#define RNNT_CASE_G(T, VEC)                                   \
    switch (G) {                                              \
    case 4: return fn(Tag<T, VEC, 4>{});                      \
    case 8: return fn(Tag<T, VEC, 8>{});                      \
    case 16: return fn(Tag<T, VEC, 16>{});                    \
    case 32: return fn(Tag<T, VEC, 32>{});                    \
    default: return fn(Tag<T, VEC, 64>{});                    \
    }
    if (esize == 4) {
        if (vec == 4) { RNNT_CASE_G(float, 4) }
        RNNT_CASE_G(float, 1)
    }
    if (vec == 8) { RNNT_CASE_G(_Float16, 8) }
    RNNT_CASE_G(_Float16, 1)
#undef RNNT_CASE_G
}

}  // namespace

RowGeom row_geometry(int V, int esize, bool aligned16) {
    RowGeom g;
    g.vec = aligned16 ? 16 / esize : 1;
    const int nvec = (V + g.vec - 1) / g.vec;
    int G = 4;
    while (G < 64 && G < nvec) G <<= 1;
    g.lanes_per_row = G;
    g.rows_per_block_iter = 4 * (64 / G);
    return g;
}

#define WS(type, field) reinterpret_cast<type>(a.ws + a.lay.field)

hipError_t launch_rowstats(const LaunchArgs &a, hipStream_t stream) {
    const dim3 grid(a.lay.n_chunks), block(256);
    if (!a.fused) {
        if (a.esize == 4)
            hipLaunchKernelGGL(k_gather<float>, grid, block, 0, stream, static_cast<const float *>(a.logits), a.V,
                               a.blank, WS(const SampleDesc *, desc), WS(const ChunkDesc *, chunks), a.targets, a.S,
                               WS(float *, lpb), WS(float *, lpy), WS(uint32_t *, status));
        else
            hipLaunchKernelGGL(k_gather<_Float16>, grid, block, 0, stream, static_cast<const _Float16 *>(a.logits),
                               a.V, a.blank, WS(const SampleDesc *, desc), WS(const ChunkDesc *, chunks), a.targets,
                               a.S, WS(float *, lpb), WS(float *, lpy), WS(uint32_t *, status));
        return hipGetLastError();
    }
    return with_geom(a.esize, a.geom.vec, a.geom.lanes_per_row, [&](auto tag) {
        using Tg = decltype(tag);
        using T = typename Tg::type;
        hipLaunchKernelGGL((k_rowstats<T, Tg::vec, Tg::g>), grid, block, 0, stream, static_cast<const T *>(a.logits),
                           a.V, a.blank, WS(const SampleDesc *, desc), WS(const ChunkDesc *, chunks), a.targets, a.S,
                           WS(float *, den), WS(float *, lpb), WS(float *, lpy), WS(uint32_t *, status));
        return hipGetLastError();
    });
}

hipError_t launch_alpha_beta(const LaunchArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(k_alpha_beta, dim3(a.B), dim3(128), 0, stream, WS(const SampleDesc *, desc),
                       WS(const int32_t *, order), WS(const float *, lpb), WS(const float *, lpy),
                       WS(double *, alpha), WS(double *, beta), a.loss, WS(uint32_t *, status));
    return hipGetLastError();
}

hipError_t launch_grad(const LaunchArgs &a, hipStream_t stream) {
    const dim3 grid(a.lay.n_chunks), block(256);
    const float log2_scale = log2f(a.grad_scale);
    return with_geom(a.esize, a.geom.vec, a.geom.lanes_per_row, [&](auto tag) {
        using Tg = decltype(tag);
        using T = typename Tg::type;
        if (a.fused)
            hipLaunchKernelGGL((k_grad<T, Tg::vec, Tg::g, true>), grid, block, 0, stream,
                               static_cast<const T *>(a.logits), static_cast<T *>(a.grad), a.V, a.blank, a.clamp,
                               a.grad_scale, log2_scale, WS(const SampleDesc *, desc), WS(const ChunkDesc *, chunks),
                               a.lay.n_chunks, a.targets, a.S, WS(const float *, den), WS(const float *, lpb),
                               WS(const float *, lpy), WS(const double *, alpha), WS(const double *, beta));
        else
            hipLaunchKernelGGL((k_grad<T, Tg::vec, Tg::g, false>), grid, block, 0, stream,
                               static_cast<const T *>(a.logits), static_cast<T *>(a.grad), a.V, a.blank, a.clamp,
                               a.grad_scale, log2_scale, WS(const SampleDesc *, desc), WS(const ChunkDesc *, chunks),
                               a.lay.n_chunks, a.targets, a.S, WS(const float *, den), WS(const float *, lpb),
                               WS(const float *, lpy), WS(const double *, alpha), WS(const double *, beta));
        return hipGetLastError();
    });
}

hipError_t launch_reduce(const LaunchArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(k_reduce, dim3(1), dim3(64), 0, stream, a.loss, a.B, a.reduction == RNNT_REDUCTION_MEAN,
                       a.loss_reduced);
    return hipGetLastError();
}

hipError_t launch_grad_scale(void *grad, int esize, int V, const float *scale, int per_sample, const uint8_t *ws,
                             const WorkspaceLayout &lay, const RowGeom &geom, bool aligned16, hipStream_t stream) {
    (void)aligned16;
    const dim3 grid(lay.n_chunks), block(256);
    const SampleDesc *desc = reinterpret_cast<const SampleDesc *>(ws + lay.desc);
    const ChunkDesc *chunks = reinterpret_cast<const ChunkDesc *>(ws + lay.chunks);
    return with_geom(esize, geom.vec, geom.lanes_per_row, [&](auto tag) {
        using Tg = decltype(tag);
        using T = typename Tg::type;
        hipLaunchKernelGGL((k_grad_scale<T, Tg::vec, Tg::g>), grid, block, 0, stream, static_cast<T *>(grad), V,
                           desc, chunks, scale, per_sample);
        return hipGetLastError();
    });
}

#undef WS

}  // namespace rnnt
