// gfx950 kernels of librnnt: the fused RNN-T loss, forward and backward.
//
// Pass structure (rnnt-loss-ascend README, "Architecture", kernel steps 1-5):
//   rowstats    step 1    per packed row: the row maximum m and log2 of the
//                         sum of exp(x - m) over V (fused), and the two
//                         log-probs the lattice uses, log P(blank) and
//                         log P(y_{u+1}), stored per node in a skewed layout
//                         (one contiguous run per anti-diagonal) both as fp32
//                         log-probs and as fp32 probabilities.  The maximum
//                         is kept apart from the log-sum so that every later
//                         fp32 step works on x - m, which does not depend on
//                         a common offset of the row (log_softmax is
//                         shift-invariant; README parameter table,
//                         fused_log_softmax, and "Value" section 3).
//   alpha_beta  steps 2-4 two single-wave workgroups per sample, one running
//                         the forward (alpha) recursion and the other the
//                         backward (beta) recursion, one anti-diagonal per
//                         step (README "Operator features": every node of an
//                         anti-diagonal has its inputs ready); the two
//                         losses are cross-checked.
//   grad        step 5    per packed row: the fused gradient (README "Value"
//                         section 2), clamp, reduction scale, one write.
//   reduce                none / mean / sum of the per-sample losses.
//
// Batches below 64512 lattice rows, where every launch is mostly fixed cost,
// take three launches instead of six: no chunk-table launch (the row pass
// derives its chunks from descriptors passed as kernel arguments), and one
// two-wave workgroup per sample runs both recursions, their check and the
// log-domain rerun (k_ab_small).
//
// The recursions run in a scaled probability domain: node values are fp64
// mantissas with one power-of-two exponent per group of eight anti-diagonals,
// renormalised exactly (by a power of two).  A step is then one multiply and
// one fused multiply-add per node instead of a log-sum-exp.  A sample whose
// log-probs leave [-80, 80] (so that an fp32 probability could underflow)
// is flagged by rowstats and takes a log-domain variant of the same sweep.
//
// Nothing here is a dense contraction, so no MFMA: the row passes are bound
// by HBM bandwidth (coalesced 16-byte accesses, one row per wave with the next
// row's loads in flight, DPP wave reductions) and the recursion by the latency
// of its T+U dependent steps.
//
// The multi-blank transducer (big blanks with durations) has passes of its
// own, at the end of this file.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "rnnt_internal.h"

namespace rnnt {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr double kLog2eD = 1.4426950408889634074;
constexpr double kLn2D = 0.69314718055994530942;
constexpr double kNegInfD = -__builtin_inf();
constexpr float kNegInf = -__builtin_inff();
constexpr float kProbRange = 80.f;  // |log-prob| bound of the probability-domain sweep
// Per-sample mode word (zeroed by k_plan): the row pass sets kModeLog when a
// log-probability leaves that bound, k_check_ab sets kModeRerun when the
// probability-domain sweeps lost alignment mass; either sends the sample's
// recursions, and the gradient's reads of them, to the log domain.  (Small
// batches: k_ab_small writes the word whole, from the row pass's per-chunk
// flags and its own check.)
constexpr int kModeLog = 1;
constexpr int kModeRerun = 2;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// log2 of a non-negative fp64 value: exponent exactly, mantissa in fp32.
__device__ __forceinline__ double log2_d(double x) {
    const int e = __builtin_amdgcn_frexp_exp(x);
    const float m = (float)__builtin_amdgcn_frexp_mant(x);
    return (double)e + (double)log2_fast(m);
}

// exp(lp) in fp32 for |lp| <= kProbRange, with the exponent split off
// (Cody-Waite) so the rounding of lp * log2(e) does not enter the result.
__device__ __forceinline__ float prob_of(float lp) {
    constexpr float kHi = 1.44269502162933349609375f;  // fp32 nearest to log2(e)
    constexpr float kLo = 1.925963033500011079e-8f;     // log2(e) - kHi
    const float k = rintf(lp * kLog2e);
    const float f = fmaf(lp, kHi, -k) + lp * kLo;
    const float p = __builtin_amdgcn_ldexpf(exp2_fast(f), (int)k);
    return (lp == kNegInf) ? 0.f : p;
}

// log2 of sum_k exp(x_k - m) from s = sum_k exp2(fma(x_k, log2(e), nm)),
// nm = -m * log2(e) rounded to fp32.  Each term is exp2((x_k - m) log2(e)
// + eps) with eps = m log2(e) + nm, the rounding error of nm (up to
// ulp(m log2(e)) / 2, ~6e-5 at m ~ 1000), common to the whole row; fma
// computes eps exactly, so it is taken back out here and the result does not
// depend on the size of m (with log2(e) the same fp32 constant throughout).
__device__ __forceinline__ float log2_sum_shifted(float s, float m, float nm) {
    return log2_fast(s) - fmaf(m, kLog2e, nm);
}

// ------------------------------------------------------------ element I/O
template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ static float load1(const float *p) { return *p; }
    __device__ static void store1(float *p, float v) { *p = v; }
    template <bool NT> __device__ static void loadv(const float *p, float *out) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        f4 v;
        if constexpr (NT) v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
        else v = *reinterpret_cast<const f4 *>(p);
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    }
    template <bool NT> __device__ static void storev(float *p, const float *in) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        f4 v = {in[0], in[1], in[2], in[3]};
        if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<f4 *>(p));
        else *reinterpret_cast<f4 *>(p) = v;
    }
};
template <> struct Elem<_Float16> {
    __device__ static float load1(const _Float16 *p) { return (float)*p; }
    __device__ static void store1(_Float16 *p, float v) { *p = (_Float16)v; }
    template <bool NT> __device__ static void loadv(const _Float16 *p, float *out) {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        h8 v;
        if constexpr (NT) v = __builtin_nontemporal_load(reinterpret_cast<const h8 *>(p));
        else v = *reinterpret_cast<const h8 *>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
    }
    template <bool NT> __device__ static void storev(_Float16 *p, const float *in) {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        h8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (_Float16)in[i];
        if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<h8 *>(p));
        else *reinterpret_cast<h8 *>(p) = v;
    }
};

template <typename T, int VEC, bool NT = false> __device__ __forceinline__ void load_n(const T *p, float *out) {
    if constexpr (VEC == 1) out[0] = Elem<T>::load1(p);
    else Elem<T>::template loadv<NT>(p, out);
}
template <typename T, int VEC, bool NT = false> __device__ __forceinline__ void store_n(T *p, const float *in) {
    if constexpr (VEC == 1) Elem<T>::store1(p, in[0]);
    else Elem<T>::template storev<NT>(p, in);
}

// A 16-byte vector kept as loaded (4 fp32 or 8 fp16, in the element type's
// own vector type), converted to fp32 element by element on use.
template <typename T> struct Raw;
template <> struct Raw<float> {
    static constexpr int kVec = 4;
    typedef float vec __attribute__((ext_vector_type(4)));
    __device__ static float get(const vec &r, int e) { return r[e]; }
    __device__ static vec put(const float *v) {
        vec r = {v[0], v[1], v[2], v[3]};
        return r;
    }
};
template <> struct Raw<_Float16> {
    static constexpr int kVec = 8;
    typedef _Float16 vec __attribute__((ext_vector_type(8)));
    __device__ static float get(const vec &r, int e) { return (float)r[e]; }
    __device__ static vec put(const float *v) {
        vec r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = (_Float16)v[e];
        return r;
    }
};
template <typename T, bool NT> __device__ __forceinline__ typename Raw<T>::vec load_raw(const T *p) {
    using V = typename Raw<T>::vec;
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V *>(p));
    else return *reinterpret_cast<const V *>(p);
}
template <typename T, bool NT> __device__ __forceinline__ void store_raw(T *p, typename Raw<T>::vec v) {
    using V = typename Raw<T>::vec;
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<V *>(p));
    else *reinterpret_cast<V *>(p) = v;
}

// ------------------------------------------------------- wave reductions
// DPP within rows of 16 lanes (quad permutes, row rotates), then row
// broadcasts 15 and 31; the wave result lands in lane 63.
template <int CTRL, int ROWMASK> __device__ __forceinline__ int dpp_i(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWMASK, 0xf, false);
}
template <int CTRL, int ROWMASK> __device__ __forceinline__ float dpp_f(float old, float v) {
    return __int_as_float(dpp_i<CTRL, ROWMASK>(__float_as_int(old), __float_as_int(v)));
}
__device__ __forceinline__ float wave_max_f(float v) {
    v = fmaxf(v, dpp_f<0xb1, 0xf>(v, v));
    v = fmaxf(v, dpp_f<0x4e, 0xf>(v, v));
    v = fmaxf(v, dpp_f<0x124, 0xf>(v, v));
    v = fmaxf(v, dpp_f<0x128, 0xf>(v, v));
    v = fmaxf(v, dpp_f<0x142, 0xa>(v, v));
    v = fmaxf(v, dpp_f<0x143, 0xc>(v, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum_f(float v) {
    v += dpp_f<0xb1, 0xf>(0.f, v);
    v += dpp_f<0x4e, 0xf>(0.f, v);
    v += dpp_f<0x124, 0xf>(0.f, v);
    v += dpp_f<0x128, 0xf>(0.f, v);
    v += dpp_f<0x142, 0xa>(0.f, v);
    v += dpp_f<0x143, 0xc>(0.f, v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ double readlane_d(double v, int l) {
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), l);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), l);
    return __hiloint2double(hi, lo);
}
// Maximum of non-negative values (floating-point exponent fields): lanes a
// stage does not reach read 0, the identity, so each move folds into the
// maximum instruction.
__device__ __forceinline__ int wave_max_nonneg(int v) {
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, true));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, true));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xf, 0xf, true));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, true));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, true));
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, true));
    return __builtin_amdgcn_readlane(v, 63);
}

// ---------------------------------------------------- row statistics output
// Writes what the recursions and the gradient need about node (t,u), at its
// skewed slot: node = {log P(blank), log P(y_{u+1}), the row's reference
// value m, log2 of the row's sum of exp(x - m)} (fused; m is the row maximum,
// or 0 for a row of -inf; both 0 for log-prob inputs) and prob = the two
// probabilities in fp32.  The blank edge leaving t = T-1 below u = U
// leaves the lattice and the label edge at u = U does not exist, so both are
// stored as impossible.  The wide kernel calls it from every lane with
// wave-uniform values (the stores are then unconditional and the compiler's
// wait counts stay exact); the others from one lane per row.
__device__ __forceinline__ void emit_node(const SampleDesc &d, int t, int u, float m, float ls2, float lpb,
                                          float lpy, float4 *__restrict__ node, float2 *__restrict__ prob,
                                          int *mode_word) {
    if (t == d.T - 1 && u < d.U) lpb = kNegInf;
    if (u == d.U) lpy = kNegInf;
    const int64_t slot = d.slot_off + (int64_t)(t + u) * (d.U + 1) + u;
    node[slot] = make_float4(lpb, lpy, m, ls2);
    prob[slot] = make_float2(prob_of(lpb), prob_of(lpy));
    const bool wide = (lpb != kNegInf && fabsf(lpb) > kProbRange) || (lpy != kNegInf && fabsf(lpy) > kProbRange);
    if (wide) atomicOr(mode_word, kModeLog);
}

// Slots u0 .. u1-1 of diagonal n hold no lattice node: give them impossible
// weights, so the recursions read whole diagonals without masks.  `lane`
// of `nl` cooperating threads.
__device__ __forceinline__ void fill_slots(const SampleDesc &d, int n, int u0, int u1, int lane, int nl,
                                           float4 *__restrict__ node, float2 *__restrict__ prob) {
    const int64_t base = d.slot_off + (int64_t)n * (d.U + 1);
    for (int u = u0 + lane; u < u1; u += nl) {
        node[base + u] = make_float4(kNegInf, kNegInf, 0.f, 0.f);
        prob[base + u] = make_float2(0.f, 0.f);
    }
}

// Diagonal order: the first node of diagonal n (u = max(0, n-T+1)) fills the
// slots below it (t >= T), the last (u = min(n, U)) those above it (t < 0).
__device__ __forceinline__ void fill_diagonal_ends(const SampleDesc &d, int n, int u, int lane, int nl,
                                                   float4 *__restrict__ node, float2 *__restrict__ prob) {
    const int lo = max(0, n - d.T + 1), hi = min(n, d.U);
    if (u == lo && lo > 0) fill_slots(d, n, 0, lo, lane, nl, node, prob);
    if (u == hi && hi < d.U) fill_slots(d, n, hi + 1, d.U + 1, lane, nl, node, prob);
}

// Row order: row (0,u) fills column u of the diagonals n < u (t < 0), row
// (T-1,u) column u of the diagonals n >= T+u (t >= T).
__device__ __forceinline__ void fill_columns(const SampleDesc &d, int t, int u, int lane, int nl,
                                             float4 *__restrict__ node, float2 *__restrict__ prob) {
    const int U1 = d.U + 1;
    if (t == 0)
        for (int n = lane; n < u; n += nl) {
            const int64_t s = d.slot_off + (int64_t)n * U1 + u;
            node[s] = make_float4(kNegInf, kNegInf, 0.f, 0.f);
            prob[s] = make_float2(0.f, 0.f);
        }
    if (t == d.T - 1)
        for (int n = d.T + u + lane; n < d.T + d.U; n += nl) {
            const int64_t s = d.slot_off + (int64_t)n * U1 + u;
            node[s] = make_float4(kNegInf, kNegInf, 0.f, 0.f);
            prob[s] = make_float2(0.f, 0.f);
        }
}

// Row of lattice node (t,u) (packed or padded layout).
__device__ __forceinline__ int64_t row_of(const SampleDesc &d, int t, int u) {
    return d.row_off + (int64_t)t * d.tstride + u;
}

// The label y_{u+1} of node (t,u), or -1 at u = U.  A label that is not a
// non-blank class (outside [0, V), or equal to blank: the build post's
// section 5.2 rules blank out of the labels) admits no alignment: its edge
// is read as impossible (-1), and the status word is flagged.
__device__ __forceinline__ int label_of(const SampleDesc &d, int u, int V, int blank,
                                        const int32_t *__restrict__ targets, int S) {
    if (u >= d.U) return -1;
    const int y = targets[(int64_t)d.index * S + u];
    return (y >= 0 && y < V && y != blank) ? y : -1;
}
__device__ __forceinline__ int read_label(const SampleDesc &d, int u, int V, int blank,
                                          const int32_t *__restrict__ targets, int S, uint32_t *status) {
    const int y = label_of(d, u, V, blank, targets, S);
    if (u < d.U && y < 0) atomicOr(status, (uint32_t)RNNT_DEV_BAD_TARGET);
    return y;
}

// Lane-local maximum of a row held the way the wide kernels hold it.  fp16
// rows are reduced in fp16 with packed maxima (exact, and no conversions
// until the last value).
template <typename T, int NV, bool FULL>
__device__ __forceinline__ float row_max(const typename Raw<T>::vec (&x)[NV], int nvec) {
    const int lane = threadIdx.x & 63;
    if constexpr (std::is_same_v<T, _Float16>) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        typename Raw<T>::vec hm = (_Float16)kNegInf;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (FULL || i * 64 + lane < nvec) hm = __builtin_elementwise_maximum(hm, x[i]);
        const h4 m4 = __builtin_elementwise_maximum(__builtin_shufflevector(hm, hm, 0, 1, 2, 3),
                                                __builtin_shufflevector(hm, hm, 4, 5, 6, 7));
        const h2 m2 = __builtin_elementwise_maximum(__builtin_shufflevector(m4, m4, 0, 1),
                                                __builtin_shufflevector(m4, m4, 2, 3));
        return fmaxf((float)m2[0], (float)m2[1]);
    } else {
        float m = kNegInf;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (FULL || i * 64 + lane < nvec)
#pragma unroll
                for (int e = 0; e < Raw<T>::kVec; ++e) m = fmaxf(m, Raw<T>::get(x[i], e));
        return m;
    }
}

// Lattice node of the row `step` rows further on in the same sample (row order).
__device__ __forceinline__ void advance_node(int &t, int &u, int step, int U1) {
    u += step;
    while (u >= U1) {
        u -= U1;
        ++t;
    }
}

// Node `step` nodes further on in diagonal order (anti-diagonal n, then
// column u; diagonal n holds columns max(0, n-T+1) .. min(n, U)).  Stops at
// the last diagonal, so a step past the end of the lattice leaves u out of
// range there.
__device__ __forceinline__ void advance_diag(int &n, int &u, int step, int T, int U) {
    u += step;
    while (u > min(n, U) && n < T + U - 1) {
        u -= min(n, U) + 1;
        ++n;
        u += max(0, n - T + 1);
    }
}

// ------------------------------------------------ row-pass work sources
// Where a row-pass workgroup finds its chunk and its sample, and where it
// reports a sample's log-domain flag and a bad label.
//   TableSrc: the chunk table and descriptors in the workspace (written by
//     k_plan, which also cleared the mode words and the status word that the
//     row pass sets bits in).
//   ArgSrc (batches below 64 K rows, whose every launch is mostly fixed
//     cost): no chunk-table launch.  The descriptors come as kernel
//     arguments, in cost order (kernel arguments may live in host memory, so
//     each workgroup reads them in one round trip: lane k the descriptor of
//     the k-th sample), each workgroup derives its chunk itself and writes
//     it to the chunk table for the gradient pass, and ORs its bits
//     (kModeLog, RNNT_DEV_BAD_TARGET) into a word in LDS that it stores as
//     its own flag word, so nothing needs clearing first; workgroup 0 also
//     stores the descriptors and the order.  The recursion kernel ORs a
//     sample's flag words into its mode and its status bits, the reduction
//     the samples' status bits into the status word.
struct TableSrc {
    const SampleDesc *__restrict__ desc;
    const ChunkDesc *__restrict__ chunks;
    int *__restrict__ mode;
    uint32_t *status;
};
struct ArgSrc {
    PlanArgs pa;  // pa.desc[k]: the k-th sample in cost order (pa.order[k] is its index)
    int rpc;
    ChunkDesc *ws_chunks;
    SampleDesc *ws_desc;
    int32_t *ws_order;
    uint32_t *cflags;
};

// A row-pass workgroup's chunk and sample, and the words its flags go to.
struct RowWork {
    ChunkDesc c;
    SampleDesc d;
    int *mode_word;
    uint32_t *status_word;
};

template <bool DIAG> __device__ __forceinline__ RowWork row_work(const TableSrc &s, uint32_t *) {
    RowWork w;
    w.c = s.chunks[blockIdx.x];
    w.d = s.desc[w.c.sample];
    w.mode_word = &s.mode[w.d.index];
    w.status_word = s.status;
    return w;
}
__device__ __forceinline__ void row_work_end(const TableSrc &, uint32_t *) {}

__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ int64_t readlane_l(int64_t v, int l) {
    const int lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const int hi = __builtin_amdgcn_readlane((int)(v >> 32), l);
    return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// DIAG: the pass walks its chunk in diagonal order (the chunk's first node
// is found by bisection); a row-order pass needs only its rows.
template <bool DIAG> __device__ __forceinline__ RowWork row_work(const ArgSrc &s, uint32_t *flags) {
    const int x = (int)blockIdx.x;
    const int lane = threadIdx.x & 63;
    if (threadIdx.x == 0) *flags = 0u;
    // Chunks are numbered in cost order, so x belongs to the last sample in
    // that order whose first chunk is at most x (every sample has a chunk).
    SampleDesc mine{};
    if (lane < s.pa.B) mine = s.pa.desc[lane];
    const uint64_t hit = __ballot(lane < s.pa.B && mine.chunk0 <= x);
    const int k = 63 - __builtin_clzll(hit);
    RowWork w;
    w.d.row_off = readlane_l(mine.row_off, k);
    w.d.slot_off = readlane_l(mine.slot_off, k);
    w.d.diag_off = readlane_l(mine.diag_off, k);
    w.d.ab_off = readlane_l(mine.ab_off, k);
    w.d.T = readlane_i(mine.T, k);
    w.d.U = readlane_i(mine.U, k);
    w.d.index = readlane_i(mine.index, k);
    w.d.U1p = readlane_i(mine.U1p, k);
    w.d.tstride = readlane_i(mine.tstride, k);
    w.d.chunk0 = readlane_i(mine.chunk0, k);
    if (DIAG) {
        w.c = make_chunk(w.d, w.d.index, x - w.d.chunk0, s.rpc);
    } else {
        const int64_t rows = (int64_t)w.d.T * (w.d.U + 1);
        const int64_t r0 = (int64_t)(x - w.d.chunk0) * s.rpc;
        w.c.sample = w.d.index;
        w.c.row_begin = (int32_t)r0;
        w.c.count = (int32_t)(rows - r0 < s.rpc ? rows - r0 : s.rpc);
        w.c.diag = 0;  // unused in row order
        w.c.col = 0;
    }
    if (threadIdx.x == 0) s.ws_chunks[x] = w.c;
    if (x == 0 && threadIdx.x < 64 && lane < s.pa.B) {
        s.ws_desc[mine.index] = mine;
        s.ws_order[lane] = mine.index;
    }
    w.mode_word = reinterpret_cast<int *>(flags);
    w.status_word = flags;
    __syncthreads();
    return w;
}
__device__ __forceinline__ void row_work_end(const ArgSrc &s, uint32_t *flags) {
    __syncthreads();
    if (threadIdx.x == 0) s.cflags[blockIdx.x] = *flags;
}

// ------------------------------------------------------------ chunk table
// Workgroup k*GX + x writes chunks 256x .. 256x+255 of the k-th sample (in
// cost order with ARGS, else in batch order), with the arithmetic the host
// uses to describe the schedule (make_chunk), so only the sample
// descriptors travel from the host each call.  ARGS: the descriptors come
// as kernel arguments in cost order; workgroup 0 also writes them and the
// order to the workspace and clears the status word and the mode flags.
template <bool ARGS>
__global__ __launch_bounds__(256) void k_plan(const SampleDesc *__restrict__ desc, int rpc, int gx,
                                              ChunkDesc *__restrict__ chunks, PlanArgs pa, SampleDesc *ws_desc,
                                              int32_t *ws_order, int *ws_mode, uint32_t *ws_status) {
    const int k = (int)(blockIdx.x / (unsigned)gx);
    const int x = (int)(blockIdx.x % (unsigned)gx);
    const SampleDesc d = ARGS ? pa.desc[k] : desc[k];
    if (ARGS && blockIdx.x == 0) {
        for (int q = threadIdx.x; q < pa.B; q += blockDim.x) {
            const SampleDesc e = pa.desc[q];
            ws_desc[e.index] = e;
            ws_order[q] = e.index;
            ws_mode[q] = 0;
        }
        if (threadIdx.x == 0) *ws_status = 0u;
    }
    const int64_t rows = (int64_t)d.T * (d.U + 1);
    const int n = (int)((rows + rpc - 1) / rpc);
    const int j = x * 256 + threadIdx.x;
    if (j < n) chunks[d.chunk0 + j] = make_chunk(d, d.index, j, rpc);
}

// ------------------------------------ K1 rowstats, rows wider than 1 KiB
// Rows that do not all start on a 16-byte boundary (ODD: a row length that is
// no multiple of 16 bytes, or logits off such a boundary) are read in the
// 16-byte vectors that cover them, from the one holding the row's first
// element (`lead` elements before it): the slots outside the row, in its first
// and last vectors only, read -inf, which the maximum ignores and the sum of
// exponentials counts as zero.  Such a vector never leaves the 16-byte block,
// so the page, of the row's first or last element.  The vectors x[i] are the
// row's vectors (base + i) * 64 + lane; only the first and the last are
// touched (a test per element of every vector had cost the fp16 row pass a
// third of its speed).
template <typename T, int N>
__device__ __forceinline__ void mask_row_edges(typename Raw<T>::vec (&x)[N], int base, int lead, int nv, int V) {
    constexpr int VEC = Raw<T>::kVec;
    const int lane = threadIdx.x & 63;
    if (base == 0 && lead > 0 && lane == 0) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            if (e < lead) x[0][e] = (T)kNegInf;
    }
    const int last = nv - 1, tail = V + lead - last * VEC;  // valid slots of the last vector: 0 .. tail-1
    if (tail < VEC) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            if ((base + i) == (last >> 6) && lane == (last & 63)) {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (e >= tail) x[i][e] = (T)kNegInf;
            }
    }
}
template <typename T> __device__ __forceinline__ int lead_of(const T *p) {
    return (int)((reinterpret_cast<uintptr_t>(p) & 15u) / sizeof(T));
}

// Rows above 5 KiB: one row per wave (sixteen waves per workgroup, measured
// fastest there: 16 against 8 waves 1.3% faster on 8 KiB and 2.4% on 20 KB
// rows; rows of 1 to 5 KiB take k_rowstats_multi below, eight waves of two
// rows at a time, where one row per wave had measured 8 waves 2% faster than
// 4 and 9% faster than 16; a chunk's nodes in diagonal order, so the waves'
// per-node records land in consecutive slots), the row walked in
// segments of 4 KiB (four 16-byte vectors per lane, non-temporal loads) with
// the next segment's loads in flight (segments of five vectors, two instead
// of three for 8208-byte rows, measured 23% slower).  Holding only two segments, a wave
// needs few registers, so many waves (rows) are in flight per compute unit:
// measured faster than holding whole rows in registers (three row buffers
// of up to 16 vectors per lane) on 4 KiB and 8 KiB rows, and the only form
// for rows beyond 16 KiB.
//
// Each lane keeps a running maximum m of its elements, nm = -m log2(e)
// rounded to fp32, and s = the sum of exp2(fma(x, log2(e), nm)) over its
// elements: one fused multiply-add, one exp2 and one add per element.  When
// m grows, s is multiplied by exp2(nm' - nm), which is exact in this form:
// every term carries the same factor 2^(m log2(e) + nm), the rounding of nm,
// and that factor changes by exactly nm' - nm.  At the end of the row the
// lane's sum, rescaled to the row maximum M, is s exp2(-fma(M, log2(e), nm)):
// the rounding of nm cancels, so no step depends on the size of x, only on
// x - M (an fp32 emulation against exact sums: 2.4e-7 in log2 of the sum at
// offsets from 0 to 30000).  Each lane keeps a running maximum of its
// elements and the sum of exp(x - that maximum), rescaled when it grows; at
// the end of the row the lanes' sums are rescaled to the row maximum and
// added.  Every term is formed from x - maximum, as in the other row passes.
template <typename T, int W, bool ODD, bool MERGE, typename Src>
__global__ __launch_bounds__(64 * W) void k_rowstats_stream(const T *__restrict__ logits, int V, int blank, Src src,
                                                         const int32_t *__restrict__ targets, int S,
                                                         float4 *__restrict__ node, float2 *__restrict__ prob) {
    constexpr int VEC = Raw<T>::kVec;
    constexpr int NS = 4;  // vectors per lane per segment
    using Vec = typename Raw<T>::vec;
    __shared__ uint32_t wg_flags;
    const RowWork wk = row_work<true>(src, &wg_flags);
    const ChunkDesc &c = wk.c;
    const SampleDesc &d = wk.d;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nvec = V / VEC;
    const int nseg = (nvec + 64 * NS - 1) / (64 * NS);
    int n = c.diag, u = c.col;
    advance_diag(n, u, wave, d.T, d.U);
    for (int r = wave; r < c.count; r += W) {
        const T *p = logits + row_of(d, n - u, u) * (int64_t)V;
        const int y = __builtin_amdgcn_readfirstlane(read_label(d, u, V, blank, targets, S, wk.status_word));
        const float hb = Elem<T>::load1(p + blank);
        const float hy = (y >= 0) ? Elem<T>::load1(p + y) : 0.f;
        const int lead = ODD ? lead_of(p) : 0;
        const T *pv = p - lead;
        const int nvr = ODD ? (lead + V + VEC - 1) / VEC : nvec;  // vectors covering the row
        int nsegr = ODD ? (nvr + 64 * NS - 1) / (64 * NS) : nseg;
        // MERGE: a last segment of at most one block of 64 vectors is read as
        // a fifth block of the segment before it (an 8194-byte row in two
        // steps instead of three)
        constexpr int NX = NS + (MERGE ? 1 : 0);
        bool merged = false;
        if constexpr (MERGE) {
            merged = nsegr >= 2 && nvr - (nsegr - 1) * 64 * NS <= 64;
            if (merged) nsegr -= 1;
        }
        auto blocks_of = [&](int sg) { return (MERGE && merged && sg == nsegr - 1) ? NX : NS; };
        auto load_seg = [&](int sg, Vec (&x)[NX]) {
            const int nb = blocks_of(sg);
#pragma unroll
            for (int i = 0; i < NX; ++i) {
                const int vi = (sg * NS + i) * 64 + lane;
                if (i < nb && vi < nvr) x[i] = load_raw<T, true>(pv + (int64_t)vi * VEC);
            }
            if constexpr (ODD) mask_row_edges<T, NX>(x, sg * NS, lead, nvr, V);
        };
        float m = kNegInf, nm = 0.f, s = 0.f;
        auto take_seg = [&](int sg, const Vec (&x)[NX]) {
            const int cnt = min(nvr - sg * NS * 64, blocks_of(sg) * 64);  // the segment's vectors
            const float mn = fmaxf(m, row_max<T, NX, false>(x, cnt));
            const float nmn = (mn == kNegInf) ? 0.f : -mn * kLog2e;
            float acc = (m == kNegInf) ? 0.f : s * exp2_fast(nmn - nm);
#pragma unroll
            for (int i = 0; i < NX; ++i)
                if (i * 64 + lane < cnt)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc += exp2_fast(fmaf(Raw<T>::get(x[i], e), kLog2e, nmn));
            s = acc;
            m = mn;
            nm = nmn;
        };
        Vec xa[NX], xb[NX];
        load_seg(0, xa);
        for (int sg = 0; sg < nsegr; sg += 2) {
            if (sg + 1 < nsegr) load_seg(sg + 1, xb);
            take_seg(sg, xa);
            if (sg + 1 < nsegr) {
                if (sg + 2 < nsegr) load_seg(sg + 2, xa);
                take_seg(sg + 1, xb);
            }
        }
        const float M = wave_max_f(m);
        const bool dead = (M == kNegInf);
        const float mr = dead ? 0.f : M;
        const float part = (s == 0.f) ? 0.f : s * exp2_fast(-fmaf(mr, kLog2e, nm));
        const float ls2 = dead ? 0.f : log2_fast(wave_sum_f(part));
        const float lpb = dead ? kNegInf : (hb - mr) - ls2 * kLn2;
        const float lpy = (dead || y < 0) ? kNegInf : (hy - mr) - ls2 * kLn2;
        emit_node(d, n - u, u, mr, ls2, lpb, lpy, node, prob, wk.mode_word);
        fill_diagonal_ends(d, n, u, lane, 64, node, prob);
        advance_diag(n, u, W, d.T, d.U);
    }
    row_work_end(src, &wg_flags);
}

// Rows of 1 to 5 KiB (one segment of NS = 4 vectors per lane up to 4 KiB, 5
// above, so a row a little over 4 KiB takes one step rather than two): each wave takes R
// of its rows at a time, r, r + W, ..., r + (R-1) W, with the loads of all
// of them in flight together and their reductions interleaved.  Per row the
// arithmetic is the streaming kernel's, lane for lane.  Launched with R = 2
// (4 KiB fp32 rows: 0.438 -> 0.431 ms against one row at a time; four rows
// 0.442).
template <typename T, int W, int R, int NS, bool ODD, typename Src>
__global__ __launch_bounds__(64 * W) void k_rowstats_multi(const T *__restrict__ logits, int V, int blank, Src src,
                                                        const int32_t *__restrict__ targets, int S,
                                                        float4 *__restrict__ node, float2 *__restrict__ prob) {
    constexpr int VEC = Raw<T>::kVec;
    using Vec = typename Raw<T>::vec;
    __shared__ uint32_t wg_flags;
    const RowWork wk = row_work<true>(src, &wg_flags);
    const ChunkDesc &c = wk.c;
    const SampleDesc &d = wk.d;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nvec = V / VEC;
    int n = c.diag, u = c.col;
    advance_diag(n, u, wave, d.T, d.U);
    for (int r = wave; r < c.count; r += R * W) {
        int nr[R], ur[R];
        const T *p[R];
        nr[0] = n;
        ur[0] = u;
#pragma unroll
        for (int k = 1; k < R; ++k) {
            nr[k] = nr[k - 1];
            ur[k] = ur[k - 1];
            advance_diag(nr[k], ur[k], W, d.T, d.U);
        }
#pragma unroll
        for (int k = 0; k < R; ++k)  // rows past the chunk reread its first (in bounds, not stored)
            p[k] = logits + row_of(d, (r + k * W < c.count ? nr[k] - ur[k] : n - u),
                                   (r + k * W < c.count ? ur[k] : u)) * (int64_t)V;
        Vec x[R][NS];
        int lead[R], nv[R];  // ODD: the row's elements before its first 16-byte boundary; vectors covering it
#pragma unroll
        for (int k = 0; k < R; ++k) {
            lead[k] = ODD ? lead_of(p[k]) : 0;
            nv[k] = ODD ? (lead[k] + V + VEC - 1) / VEC : nvec;
        }
        if constexpr (!ODD) {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int vi = i * 64 + lane;
                if (vi < nvec)
#pragma unroll
                    for (int k = 0; k < R; ++k) x[k][i] = load_raw<T, true>(p[k] + (int64_t)vi * VEC);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int vi = i * 64 + lane;
#pragma unroll
                for (int k = 0; k < R; ++k)
                    if (vi < nv[k]) x[k][i] = load_raw<T, true>(p[k] - lead[k] + (int64_t)vi * VEC);
            }
#pragma unroll
            for (int k = 0; k < R; ++k) mask_row_edges<T, NS>(x[k], 0, lead[k], nv[k], V);
        }
        int y[R];
        float hb[R], hy[R];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            y[k] = (r + k * W < c.count)
                       ? __builtin_amdgcn_readfirstlane(read_label(d, ur[k], V, blank, targets, S, wk.status_word))
                       : -1;
            hb[k] = Elem<T>::load1(p[k] + blank);
            hy[k] = (y[k] >= 0) ? Elem<T>::load1(p[k] + y[k]) : 0.f;
        }
        // per row and lane: the maximum m, nm = -m log2(e) and the sum of exp2(fma(x, log2(e), nm))
        float m[R], nm[R], sm[R];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            m[k] = row_max<T, NS, false>(x[k], nv[k]);
            nm[k] = (m[k] == kNegInf) ? 0.f : -m[k] * kLog2e;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < NS; ++i)
                if (i * 64 + lane < nv[k])
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc += exp2_fast(fmaf(Raw<T>::get(x[k][i], e), kLog2e, nm[k]));
            sm[k] = acc;
        }
        float M[R], part[R];
#pragma unroll
        for (int k = 0; k < R; ++k) M[k] = wave_max_f(m[k]);
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const float mr = (M[k] == kNegInf) ? 0.f : M[k];
            part[k] = (sm[k] == 0.f) ? 0.f : sm[k] * exp2_fast(-fmaf(mr, kLog2e, nm[k]));
        }
#pragma unroll
        for (int k = 0; k < R; ++k) part[k] = wave_sum_f(part[k]);
#pragma unroll
        for (int k = 0; k < R; ++k) {
            if (r + k * W >= c.count) break;
            const bool dead = (M[k] == kNegInf);
            const float mr = dead ? 0.f : M[k];
            const float ls2 = dead ? 0.f : log2_fast(part[k]);
            const float lpb = dead ? kNegInf : (hb[k] - mr) - ls2 * kLn2;
            const float lpy = (dead || y[k] < 0) ? kNegInf : (hy[k] - mr) - ls2 * kLn2;
            emit_node(d, nr[k] - ur[k], ur[k], mr, ls2, lpb, lpy, node, prob, wk.mode_word);
            fill_diagonal_ends(d, nr[k], ur[k], lane, 64, node, prob);
        }
        advance_diag(n, u, R * W, d.T, d.U);
    }
    row_work_end(src, &wg_flags);
}

// --------------------------------- K1 rowstats, G < 64 lanes per row (small V)
// Rows in row order (several short rows per wave); each row's outputs go to
// its skewed slot.
template <typename T, int VEC, int G, typename Src>
__global__ __launch_bounds__(256) void k_rowstats_narrow(const T *__restrict__ logits, int V, int blank, Src src,
                                                         const int32_t *__restrict__ targets, int S,
                                                         float4 *__restrict__ node, float2 *__restrict__ prob) {
    constexpr int RPW = 64 / G;
    __shared__ uint32_t wg_flags;
    const RowWork wk = row_work<false>(src, &wg_flags);
    const ChunkDesc &c = wk.c;
    const SampleDesc &d = wk.d;
    const int U1 = d.U + 1;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane & (G - 1);
    const int grp = lane / G;
    const int nvec = V / VEC;
    for (int base = wave * RPW; base < c.count; base += 4 * RPW) {
        const int r = base + grp;
        const bool active = r < c.count;
        const int lr = c.row_begin + (active ? r : 0);
        const int t = lr / U1;
        const int u = lr - t * U1;
        const T *p = logits + row_of(d, t, u) * (int64_t)V;
        float m = kNegInf, s = 0.f;
        if (active) {
            for (int i = sub; i < nvec; i += G) {
                float x[VEC];
                load_n<T, VEC>(p + (int64_t)i * VEC, x);
                float vm = x[0];
#pragma unroll
                for (int e = 1; e < VEC; ++e) vm = fmaxf(vm, x[e]);
                const float mn = fmaxf(m, vm);
                const float mr = (mn == kNegInf) ? 0.f : mn;
                float acc = s * exp2_fast((m - mr) * kLog2e);
                // each lane keeps its own running maximum, so the terms are
                // formed from x - max directly (exact for the terms that matter)
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc += exp2_fast((x[e] - mr) * kLog2e);
                s = acc;
                m = mn;
            }
        }
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) {
            const float mo = __shfl_xor(m, off, 64);
            const float so = __shfl_xor(s, off, 64);
            const float mn = fmaxf(m, mo);
            const float mr = (mn == kNegInf) ? 0.f : mn;
            s = s * exp2_fast((m - mr) * kLog2e) + so * exp2_fast((mo - mr) * kLog2e);
            m = mn;
        }
        if (!active) continue;
        if (sub == 0) {
            const bool dead = (m == kNegInf);
            const float mr = dead ? 0.f : m;
            const float ls2 = dead ? 0.f : log2_fast(s);
            const int y = read_label(d, u, V, blank, targets, S, wk.status_word);
            const float hb = Elem<T>::load1(p + blank);
            const float hy = (y >= 0) ? Elem<T>::load1(p + y) : 0.f;
            const float lpb = dead ? kNegInf : (hb - mr) - ls2 * kLn2;
            const float lpy = (dead || y < 0) ? kNegInf : (hy - mr) - ls2 * kLn2;
            emit_node(d, t, u, mr, ls2, lpb, lpy, node, prob, wk.mode_word);
        }
        if (t == 0 || t == d.T - 1) fill_columns(d, t, u, sub, G, node, prob);
    }
    row_work_end(src, &wg_flags);
}

// Non-fused inputs are already log-probabilities: gather the two values only.
// One node per thread, in the chunk's order (DIAG: diagonal order).
template <typename T, bool DIAG, typename Src>
__global__ __launch_bounds__(256) void k_gather(const T *__restrict__ logits, int V, int blank, Src src,
                                                const int32_t *__restrict__ targets, int S,
                                                float4 *__restrict__ node, float2 *__restrict__ prob) {
    __shared__ uint32_t wg_flags;
    const RowWork wk = row_work<DIAG>(src, &wg_flags);
    const ChunkDesc &c = wk.c;
    const SampleDesc &d = wk.d;
    const int U1 = d.U + 1;
    for (int r = threadIdx.x; r < c.count; r += blockDim.x) {
        int t, u;
        if constexpr (DIAG) {
            int n = c.diag;
            u = c.col;
            advance_diag(n, u, r, d.T, d.U);
            t = n - u;
            fill_diagonal_ends(d, n, u, 0, 1, node, prob);
        } else {
            const int lr = c.row_begin + r;
            t = lr / U1;
            u = lr - t * U1;
            if (t == 0 || t == d.T - 1) fill_columns(d, t, u, 0, 1, node, prob);
        }
        const T *p = logits + row_of(d, t, u) * (int64_t)V;
        const int y = read_label(d, u, V, blank, targets, S, wk.status_word);
        const float lpb = Elem<T>::load1(p + blank);
        const float lpy = (y < 0) ? kNegInf : Elem<T>::load1(p + y);
        emit_node(d, t, u, 0.f, 0.f, lpb, lpy, node, prob, wk.mode_word);
    }
    row_work_end(src, &wg_flags);
}

// ----------------------------------------------------- K2: alpha/beta sweeps
// Lane l owns K consecutive lattice columns in each of G column groups,
// u = 64*K*g + K*l + k (k < K, g < G; U1p = 64*K*G padded columns, K = 1 for
// lattices up to 64 columns wide, 2 up to 128, else 4).  A lane's columns
// move in 16-byte accesses: the fp32 probabilities {P(blank), P(label)} of
// two columns per load, two fp64 values per store (8-byte accesses of one
// column when K = 1).  Only a lane's first column
// needs a value from another lane (the last column of lane l-1, or of lane
// 63 of the previous group for lane 0): one wave rotation per group and a
// select on lane 0 (a plain shift when there is one group).  Diagonal n is
// read and written through buffer resources based at the diagonal, whose
// range check returns zero for the columns past U: those columns start at
// zero and only ever receive zero, because the label edge leaving column U
// is stored as impossible (the log domain, where zero is -inf, clamps its
// reads to column U instead).  Every slot of a diagonal up to U holds
// weights (the row pass fills those outside the lattice with
// "impossible"), so no step needs a mask.  The inputs of PF diagonals are
// loaded one block ahead into one of two register rings used in turn.
//
// Probability domain: node value = mantissa * 2^E, one exponent E per group
// of eight diagonals.  Forward step, from diagonal n to n+1:
//   a(n+1,u) = a(n,u) * pb(n,u) + a(n,u-1) * py(n,u-1)
// from a = 1 at (0,0); one step past the last diagonal leaves
// P(y|x) = a(T-1,U) * pb(T-1,U) in column U.  Backward step:
//   b(n,u) = b(n+1,u) * pb(n,u) + b(n+1,u+1) * py(n,u)
// from b = 1 at (T-1+1, U), the empty suffix after the final blank.  Every
// eighth diagonal is rescaled by 2^-e so its largest value is in [1, 2):
// with |log-prob| <= 80 a value moves by at most 2^+-116.4 per step, so
// eight steps stay inside fp64's normal range.  The exponent that applies to
// forward diagonal n is ealpha[(n + 1) / 8], to backward diagonal n
// ebeta[(nd - n) / 8].
//
// Log domain (fallback): the same recursions in log2 units with
// log2(2^a + 2^b) in place of the sum and log2-prob addition in place of the
// product; all exponents are 0.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

// Raw (unstrided) buffer resource over `bytes` bytes from `base`: each
// dword of a load past `bytes` reads zero without touching memory, a store
// there is dropped.
__device__ __forceinline__ Rsrc buffer_at(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// The weights of a lane's K columns of one group on one diagonal:
// q[h] = {pb(2h), py(2h), pb(2h+1), py(2h+1)}.
template <int K> struct Wts {
    float4 q[K / 2];
    __device__ float pb(int k) const { return (k & 1) ? q[k >> 1].z : q[k >> 1].x; }
    __device__ float py(int k) const { return (k & 1) ? q[k >> 1].w : q[k >> 1].y; }
};
// One column per lane (lattices up to 64 columns wide): {pb, py}.
template <> struct Wts<1> {
    float2 q;
    __device__ float pb(int) const { return q.x; }
    __device__ float py(int) const { return q.y; }
};

struct ProbDomain {
    static constexpr bool kLog = false;
    static constexpr uint32_t kSlot = 8;  // prob[] slot: float2 {P(blank), P(label)}
    __device__ static double zero() { return 0.0; }
    __device__ static double one() { return 1.0; }
    __device__ static double combine(double a, double b) { return a + b; }
    __device__ static double edge(double a, float w) { return a * (double)w; }
    // voff[k]: byte offset of column k of the lane's group (even k used).
    template <int K>
    __device__ static void load(Wts<K> &w, Rsrc r, const uint32_t (&voff)[K], uint32_t soff) {
        if constexpr (K == 1) {
            w.q = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, voff[0], soff, 0));
        } else {
#pragma unroll
            for (int h = 0; h < K / 2; ++h)
                w.q[h] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff[2 * h], soff, 0));
        }
    }
};
struct LogDomain {
    static constexpr bool kLog = true;
    static constexpr uint32_t kSlot = 16;  // node[] slot: float4, of which {log P(blank), log P(label)}
    __device__ static double zero() { return kNegInfD; }
    __device__ static double one() { return 0.0; }
    __device__ static double combine(double a, double b) {
        const double mx = fmax(a, b);
        const double mn = fmin(a, b);
        const float l = log2_fast(1.0f + exp2_fast((float)(mn - mx)));
        return (mn == kNegInfD) ? mx : mx + (double)l;
    }
    __device__ static double edge(double a, float lpv) { return a + (double)lpv * kLog2eD; }
    // The first eight bytes of each column's slot (offsets clamped to column
    // U by the caller: a log-prob of 0 would not be impossible).
    template <int K>
    __device__ static void load(Wts<K> &w, Rsrc r, const uint32_t (&voff)[K], uint32_t soff) {
        if constexpr (K == 1) {
            const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, voff[0], soff, 0);
            w.q = make_float2(__uint_as_float(x[0]), __uint_as_float(x[1]));
        } else {
#pragma unroll
            for (int h = 0; h < K / 2; ++h) {
                const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, voff[2 * h], soff, 0);
                const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(r, voff[2 * h + 1], soff, 0);
                w.q[h] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(y[0]),
                                     __uint_as_float(y[1]));
            }
        }
    }
};

// fp64 lane moves across the wave (two 32-bit DPP moves): rotations (lane l
// receives lane l-1, lane 0 lane 63; or lane l+1, lane 63 lane 0) and
// shifts that give the edge lane zero.
template <int CTRL, bool ZERO_EDGE> __device__ __forceinline__ double lane_move(double x) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), CTRL, 0xf, 0xf, ZERO_EDGE);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), CTRL, 0xf, 0xf, ZERO_EDGE);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double rotate_up(double x) { return lane_move<0x13c, false>(x); }
__device__ __forceinline__ double rotate_down(double x) { return lane_move<0x134, false>(x); }
__device__ __forceinline__ double shift_up_zero(double x) { return lane_move<0x138, true>(x); }
__device__ __forceinline__ double shift_down_zero(double x) { return lane_move<0x130, true>(x); }

template <int K, int G> __device__ __forceinline__ int renorm(double (&a)[G][K]) {
    int eb = 0;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < K; ++k) eb = max(eb, (__double2hiint(a[g][k]) >> 20) & 0x7ff);
    eb = wave_max_nonneg(eb);
    const int sh = eb - 1023;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < K; ++k) a[g][k] = __builtin_amdgcn_ldexp(a[g][k], -sh);
    return sh;
}

template <int K, int G, int PF> struct Ring {
    Wts<K> v[PF][G];
};

// Where a sweep reads and writes: the sample's first weight slot and first
// output slot, the byte sizes of one diagonal of each, and the lane's byte
// offsets inside a diagonal.  Diagonal n is addressed by a scalar offset
// from the sample's base, so one diagonal costs two or three scalar
// instructions instead of a 64-bit base per access.  The range check of a
// buffer access covers the scalar offset as well: a weight resource whose
// record count ends with diagonal n (offset n * w_bytes plus one diagonal)
// reads zero for the columns past U, as a resource based at the diagonal
// would.  The output resource spans the sample's nd diagonals.  Offsets are
// 32-bit: the host keeps a sample's tables below 2^31 bytes.
template <typename D, int K, int G> struct SweepIO {
    const char *w;
    Rsrc rout;
    uint32_t w_bytes;    // U1 * kSlot
    uint32_t out_bytes;  // U1p * 8
    uint32_t win[G][K];
    uint32_t wout[G];

    // col0: the first column this wave holds; row_bytes: the output's
    // diagonal stride (U1p * 8), by default the tile's own width.
    __device__ SweepIO(const char *w_, double *out_, int U, int nd, uint32_t col0 = 0, uint32_t row_bytes = 0)
        : w(w_) {
        const uint32_t lane = threadIdx.x & 63;
        const uint32_t U1 = (uint32_t)U + 1;
        w_bytes = U1 * D::kSlot;
        out_bytes = row_bytes ? row_bytes : 64u * K * G * 8u;
        rout = buffer_at(out_, (uint32_t)nd * out_bytes);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint32_t c = col0 + 64u * K * g + K * lane;
#pragma unroll
            for (int k = 0; k < K; ++k)  // the log domain clamps to U, the probability domain to the range end
                win[g][k] = (D::kLog ? min(c + k, (uint32_t)U) : min(c + k, U1)) * D::kSlot;
            wout[g] = c * 8u;
        }
    }
    // 0 <= n < nd at every call (n is uniform; readfirstlane keeps it in a
    // scalar register where the clamp would otherwise be formed with a
    // vector instruction).
    __device__ void load(Wts<K> (&r)[G], int n) const {
        const uint32_t off = (uint32_t)__builtin_amdgcn_readfirstlane(n) * w_bytes;
        const Rsrc rs = buffer_at(w, off + w_bytes);
#pragma unroll
        for (int g = 0; g < G; ++g) D::template load<K>(r[g], rs, win[g], off);
    }
    __device__ void store(int n, const double (&a)[G][K]) const {
        const uint32_t off = (uint32_t)n * out_bytes;
        if constexpr (K == 1) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const u32x2 v = {(uint32_t)__double2loint(a[g][0]), (uint32_t)__double2hiint(a[g][0])};
                __builtin_amdgcn_raw_buffer_store_b64(v, rout, wout[g], off, 0);
            }
            return;
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int h = 0; h < K / 2; ++h) {
                const u32x4 v = {(uint32_t)__double2loint(a[g][2 * h]), (uint32_t)__double2hiint(a[g][2 * h]),
                                 (uint32_t)__double2loint(a[g][2 * h + 1]),
                                 (uint32_t)__double2hiint(a[g][2 * h + 1])};
                __builtin_amdgcn_raw_buffer_store_b128(v, rout, wout[g] + 16u * h, off, 0);
            }
    }
};

// Diagonals n0, n0+step, ... (clamped into [0, nd)) into ring r.
template <typename D, int K, int G, int PF>
__device__ __forceinline__ void load_block(Ring<K, G, PF> &r, const SweepIO<D, K, G> &io, int n0, int step,
                                           int nd) {
#pragma unroll
    for (int p = 0; p < PF; ++p) io.load(r.v[p], min(max(n0 + step * p, 0), nd - 1));
}

// One forward step: the values of diagonal n (already stored) and its
// weights w give those of diagonal n+1.
template <typename D, int K, int G>
__device__ __forceinline__ void forward_step(double (&a)[G][K], const Wts<K> (&w)[G], bool lane0) {
    double my[G][K], r[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < K; ++k) my[g][k] = D::edge(a[g][k], w[g].py(k));
    if constexpr (G > 1 || D::kLog) {
#pragma unroll
        for (int g = 0; g < G; ++g) r[g] = rotate_up(my[g][K - 1]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        double left;
        if constexpr (G == 1 && !D::kLog) left = shift_up_zero(my[0][K - 1]);
        else left = lane0 ? (g > 0 ? r[g > 0 ? g - 1 : 0] : D::zero()) : r[g];
        a[g][0] = D::combine(D::edge(a[g][0], w[g].pb(0)), left);
#pragma unroll
        for (int k = 1; k < K; ++k) a[g][k] = D::combine(D::edge(a[g][k], w[g].pb(k)), my[g][k - 1]);
    }
}

// One backward step: the values of diagonal n+1 and the weights w of
// diagonal n give those of diagonal n.
template <typename D, int K, int G>
__device__ __forceinline__ void backward_step(double (&b)[G][K], const Wts<K> (&w)[G], bool lane63) {
    double l0[G];
    if constexpr (G > 1 || D::kLog) {
#pragma unroll
        for (int g = 0; g < G; ++g) l0[g] = rotate_down(b[g][0]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        double right;
        if constexpr (G == 1 && !D::kLog) right = shift_down_zero(b[0][0]);
        else right = lane63 ? (g + 1 < G ? l0[g + 1 < G ? g + 1 : g] : D::zero()) : l0[g];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const double nxt = (k + 1 < K) ? b[g][k + 1 < K ? k + 1 : k] : right;
            b[g][k] = D::combine(D::edge(b[g][k], w[g].pb(k)), D::edge(nxt, w[g].py(k)));
        }
    }
}

// One block of PF forward diagonals n0 .. n0+PF-1 from ring r: each
// diagonal is rescaled (every eighth), stored, then stepped.  GUARD: the
// block may run past the last diagonal.
template <typename D, int K, int G, int PF, bool GUARD>
__device__ __forceinline__ void forward_block(const Ring<K, G, PF> &r, const SweepIO<D, K, G> &io, int n0, int nd,
                                              bool lane0, double (&a)[G][K], int &E, int *__restrict__ eout) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        const int n = n0 + p;
        if (!GUARD || n < nd) {
            if (!D::kLog && (n & 7) == 7) {
                E += renorm<K, G>(a);
                eout[(n + 1) >> 3] = E;  // uniform value and address
            }
            io.store(n, a);
            forward_step<D, K, G>(a, r.v[p], lane0);
        }
    }
}

// Proceed: called once the first ring's loads are issued; a sweep that
// returns false there stops (a caller that starts the probability-domain
// sweep before the sample's domain is known, so that those loads and the
// ones deciding the domain are in flight together).
struct AlwaysGo {
    __device__ bool operator()() const { return true; }
};

template <typename D, int K, int G, int PF, typename Go = AlwaysGo>
__device__ __forceinline__ bool sweep_forward(const SampleDesc &d, const char *__restrict__ w, double *__restrict__ out,
                              int *__restrict__ eout, double *log2z, Go go = Go()) {
    const int lane = threadIdx.x & 63;
    const bool lane0 = lane == 0;
    const int U = d.U, nd = d.T + U;
    double a[G][K];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < K; ++k) a[g][k] = (g == 0 && k == 0 && lane0) ? D::one() : D::zero();
    int E = 0;
    if (lane == 0) eout[0] = 0;
    const SweepIO<D, K, G> io(w, out, U, nd);
    Ring<K, G, PF> ra, rb;
    load_block<D, K, G, PF>(ra, io, 0, 1, nd);
    if (!go()) return false;
    int n0 = 0;
    for (; n0 + 2 * PF <= nd; n0 += 2 * PF) {
        load_block<D, K, G, PF>(rb, io, n0 + PF, 1, nd);
        forward_block<D, K, G, PF, false>(ra, io, n0, nd, lane0, a, E, eout);
        load_block<D, K, G, PF>(ra, io, n0 + 2 * PF, 1, nd);
        forward_block<D, K, G, PF, false>(rb, io, n0 + PF, nd, lane0, a, E, eout);
    }
    if (n0 < nd) {
        load_block<D, K, G, PF>(rb, io, n0 + PF, 1, nd);
        forward_block<D, K, G, PF, true>(ra, io, n0, nd, lane0, a, E, eout);
        if (n0 + PF < nd) forward_block<D, K, G, PF, true>(rb, io, n0 + PF, nd, lane0, a, E, eout);
    }
    // One step past the last diagonal: column U holds P(y|x).
    const int gU = U / (64 * K), kU = U % K;
    double v = 0.0;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < K; ++k) v = (g == gU && k == kU) ? a[g][k] : v;
    const double z = __shfl(v, (U % (64 * K)) / K, 64);
    if (lane == 0) *log2z = D::kLog ? z : log2_d(z) + (double)E;
    return true;
}

// One block of PF backward diagonals n0, n0-1, ..., n0-PF+1 from ring r
// (nd-1-n0 is a multiple of PF).
template <typename D, int K, int G, int PF, bool GUARD>
__device__ __forceinline__ void backward_block(const Ring<K, G, PF> &r, const SweepIO<D, K, G> &io, int n0, int nd,
                                               bool lane63, double (&b)[G][K], int &E, int *__restrict__ eout) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        const int n = n0 - p;
        if (!GUARD || n >= 0) {
            backward_step<D, K, G>(b, r.v[p], lane63);
            if (!D::kLog && ((nd - 1 - n) & 7) == 7) {
                E += renorm<K, G>(b);
                eout[(nd - n) >> 3] = E;  // uniform value and address
            }
            io.store(n, b);
        }
    }
}

template <typename D, int K, int G, int PF, typename Go = AlwaysGo>
__device__ __forceinline__ bool sweep_backward(const SampleDesc &d, const char *__restrict__ w, double *__restrict__ out,
                               int *__restrict__ eout, double *log2z, Go go = Go()) {
    const int lane = threadIdx.x & 63;
    const bool lane63 = lane == 63;
    const int U = d.U, nd = d.T + U;
    double b[G][K];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int k = 0; k < K; ++k) b[g][k] = (64 * K * g + K * lane + k == U) ? D::one() : D::zero();
    int E = 0;
    if (lane == 0) eout[0] = 0;
    const SweepIO<D, K, G> io(w, out, U, nd);
    Ring<K, G, PF> ra, rb;
    load_block<D, K, G, PF>(ra, io, nd - 1, -1, nd);
    if (!go()) return false;
    int n0 = nd - 1;
    for (; n0 - 2 * PF + 1 >= 0; n0 -= 2 * PF) {
        load_block<D, K, G, PF>(rb, io, n0 - PF, -1, nd);
        backward_block<D, K, G, PF, false>(ra, io, n0, nd, lane63, b, E, eout);
        load_block<D, K, G, PF>(ra, io, n0 - 2 * PF, -1, nd);
        backward_block<D, K, G, PF, false>(rb, io, n0 - PF, nd, lane63, b, E, eout);
    }
    if (n0 >= 0) {
        load_block<D, K, G, PF>(rb, io, n0 - PF, -1, nd);
        backward_block<D, K, G, PF, true>(ra, io, n0, nd, lane63, b, E, eout);
        if (n0 - PF >= 0) backward_block<D, K, G, PF, true>(rb, io, n0 - PF, nd, lane63, b, E, eout);
    }
    if (lane == 0) *log2z = D::kLog ? b[0][0] : log2_d(b[0][0]) + (double)E;
    return true;
}

// The sweep of one direction in the domain the sample takes.  With a Go
// functor the probability-domain sweep starts first and Go, called once
// its first loads are issued, returns whether the sample stays in that
// domain; if not, the log-domain sweep runs instead.
template <int K, int G, int PF, typename Go = AlwaysGo>
__device__ __forceinline__ void run_sweep(const SampleDesc &d, bool backward, bool log_mode, const float4 *node, const float2 *prob,
                          double *alpha, double *beta, int *ea, int *eb, double *z, Go go = Go()) {
    const int64_t so = d.slot_off;
    const int64_t ao = d.ab_off;
    const int64_t dof = d.diag_off;
    if (!log_mode) {
        const char *w = reinterpret_cast<const char *>(prob + so);
        const bool done = !backward ? sweep_forward<ProbDomain, K, G, PF>(d, w, alpha + ao, ea + dof, z, go)
                                    : sweep_backward<ProbDomain, K, G, PF>(d, w, beta + ao, eb + dof, z, go);
        if (done) return;
    }
    {
        const char *w = reinterpret_cast<const char *>(node + so);
        if (!backward) sweep_forward<LogDomain, K, G, PF>(d, w, alpha + ao, ea + dof, z);
        else sweep_backward<LogDomain, K, G, PF>(d, w, beta + ao, eb + dof, z);
    }
}

// The sweep of one direction of sample d, at its lattice width: PF
// diagonals per prefetch block.  A ring holds G*K/2*PF 16-byte loads (the
// log domain: twice as many 8-byte ones); when a ring is first read, its
// loads, the other ring's and about one block of stores are in flight,
// within the 63 vector memory operations the wait counter tracks.
template <typename Go = AlwaysGo>
__device__ __forceinline__ void sweep_sample(const SampleDesc &d, bool bw, bool lm, const float4 *node,
                                             const float2 *prob, double *alpha, double *beta, int *ealpha,
                                             int *ebeta, double *z, Go go = Go()) {
    switch (d.U1p) {
    case 64: run_sweep<1, 1, 16>(d, bw, lm, node, prob, alpha, beta, ealpha, ebeta, z, go); break;
    case 128: run_sweep<2, 1, 16>(d, bw, lm, node, prob, alpha, beta, ealpha, ebeta, z, go); break;
    case 256: run_sweep<4, 1, 8>(d, bw, lm, node, prob, alpha, beta, ealpha, ebeta, z, go); break;
    case 512: run_sweep<4, 2, 4>(d, bw, lm, node, prob, alpha, beta, ealpha, ebeta, z, go); break;
    case 768: run_sweep<4, 3, 3>(d, bw, lm, node, prob, alpha, beta, ealpha, ebeta, z, go); break;
    default: run_sweep<4, 4, 2>(d, bw, lm, node, prob, alpha, beta, ealpha, ebeta, z, go); break;  // 1024
    }
}

// One wave per workgroup: workgroup 2k runs the forward sweep and 2k+1 the
// backward sweep of the k-th sample in cost order, so the two sweeps of a
// sample run on different compute units and do not share one unit's vector
// memory path.  The backward sweep writes the loss and log2 P(y|x) at
// log2z[i], the forward sweep its own log2 P(y|x) at log2z[B + i]; the
// reduction (reduce_losses) compares the two.
__global__ __launch_bounds__(64) void k_alpha_beta(const SampleDesc *__restrict__ desc,
                                                   const int32_t *__restrict__ order, int B,
                                                   const int *__restrict__ mode, const float4 *__restrict__ node,
                                                   const float2 *__restrict__ prob, double *__restrict__ alpha,
                                                   double *__restrict__ beta, int *__restrict__ ealpha,
                                                   int *__restrict__ ebeta, double *__restrict__ log2z,
                                                   float *__restrict__ loss, int rerun) {
    const SampleDesc d = desc[order[blockIdx.x >> 1]];
    if (d.U1p > kMaxTileU1) return;  // k_ab_wide's
    const int md = mode[d.index];
    if (rerun && !(md & kModeRerun)) return;  // the rerun takes only the samples k_check_ab marked
    const bool bw = (blockIdx.x & 1) != 0;
    const bool lm = md != 0;
    double *z = bw ? &log2z[d.index] : &log2z[B + d.index];
    sweep_sample(d, bw, lm, node, prob, alpha, beta, ealpha, ebeta, z);
    if (bw && threadIdx.x == 0) loss[d.index] = (float)(-log2z[d.index] * kLn2D);
}

// ------------------------------------ lattices wider than 1024 columns
// One workgroup of NW = U1p / 256 waves per sample and direction (a launch
// for each NW in 5..8), wave w holding columns 256w .. 256w+255 with the
// four-column tile, so a diagonal's work is spread over NW waves instead of
// held by one (~600 ns a diagonal at 2048 columns in one wave's registers).
// Per diagonal the only value crossing waves is the edge column: each wave
// leaves it in LDS, one workgroup barrier (LDS only: global stores stay in
// flight), and its neighbour reads it; two slots alternate by diagonal, so a
// slot is rewritten only after the barrier that follows its read.  The
// renormalisation every eighth diagonal takes the largest exponent over all
// waves (LDS and a barrier), so the diagonal keeps one exponent, as in the
// single-wave sweep, and the check and gradient read the tables unchanged.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

struct WideShared {
    double edge[2][8];  // per diagonal parity and wave: the value its neighbour needs
    int emax[8];        // per wave: the largest biased exponent of its columns
};

template <int NW> __device__ __forceinline__ int wide_renorm(double (&a)[1][4], int wave, WideShared &sh) {
    int eb = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) eb = max(eb, (__double2hiint(a[0][k]) >> 20) & 0x7ff);
    eb = wave_max_nonneg(eb);
    if ((threadIdx.x & 63) == 0) sh.emax[wave] = eb;
    lds_barrier();
    int m = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) m = max(m, sh.emax[i]);
    const int s = m - 1023;
#pragma unroll
    for (int k = 0; k < 4; ++k) a[0][k] = __builtin_amdgcn_ldexp(a[0][k], -s);
    return s;
}

// One forward step of wave `wave`: its column 256w takes the previous wave's
// last column (its value times its label weight) through LDS.
template <typename D, int NW>
__device__ __forceinline__ void wide_forward_step(double (&a)[1][4], const Wts<4> &w, int wave, int par,
                                                  WideShared &sh) {
    const int lane = threadIdx.x & 63;
    double my[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) my[k] = D::edge(a[0][k], w.py(k));
    if (lane == 63) sh.edge[par][wave] = my[3];
    lds_barrier();
    double left = rotate_up(my[3]);
    if (lane == 0) left = wave > 0 ? sh.edge[par][wave > 0 ? wave - 1 : 0] : D::zero();
    a[0][0] = D::combine(D::edge(a[0][0], w.pb(0)), left);
#pragma unroll
    for (int k = 1; k < 4; ++k) a[0][k] = D::combine(D::edge(a[0][k], w.pb(k)), my[k - 1]);
}

// One backward step: its column 256w+255 takes the next wave's first column
// (of the diagonal before the step) through LDS.
template <typename D, int NW>
__device__ __forceinline__ void wide_backward_step(double (&b)[1][4], const Wts<4> &w, int wave, int par,
                                                   WideShared &sh) {
    const int lane = threadIdx.x & 63;
    if (lane == 0) sh.edge[par][wave] = b[0][0];
    lds_barrier();
    double right = rotate_down(b[0][0]);
    if (lane == 63) right = wave + 1 < NW ? sh.edge[par][wave + 1 < NW ? wave + 1 : wave] : D::zero();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const double nxt = (k + 1 < 4) ? b[0][k + 1 < 4 ? k + 1 : k] : right;
        b[0][k] = D::combine(D::edge(b[0][k], w.pb(k)), D::edge(nxt, w.py(k)));
    }
}

template <typename D, int NW, int PF>
__device__ __forceinline__ void wide_sweep(const SampleDesc &d, bool bw, const char *__restrict__ w,
                                           double *__restrict__ out, int *__restrict__ eout, double *z,
                                           WideShared &sh) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int U = d.U, nd = d.T + U;
    const int col0 = 256 * wave;
    double a[1][4];
    const int start = bw ? U : 0;  // forward from column 0 of diagonal 0, backward from column U past the end
#pragma unroll
    for (int k = 0; k < 4; ++k) a[0][k] = (col0 + 4 * lane + k == start) ? D::one() : D::zero();
    int E = 0;
    if (wave == 0 && lane == 0) eout[0] = 0;
    const SweepIO<D, 4, 1> io(w, out, U, nd, (uint32_t)col0, (uint32_t)d.U1p * 8u);
    Ring<4, 1, PF> ra, rb;
    // every wave walks the same diagonals, so every wave meets every barrier
    auto block = [&](const Ring<4, 1, PF> &r, int n0) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int n = bw ? n0 - p : n0 + p;
            if (n < 0 || n >= nd) continue;  // uniform
            if (!bw) {
                if (!D::kLog && (n & 7) == 7) {
                    E += wide_renorm<NW>(a, wave, sh);
                    if (wave == 0 && lane == 0) eout[(n + 1) >> 3] = E;
                }
                io.store(n, a);
                wide_forward_step<D, NW>(a, r.v[p][0], wave, n & 1, sh);
            } else {
                wide_backward_step<D, NW>(a, r.v[p][0], wave, n & 1, sh);
                if (!D::kLog && ((nd - 1 - n) & 7) == 7) {
                    E += wide_renorm<NW>(a, wave, sh);
                    if (wave == 0 && lane == 0) eout[(nd - n) >> 3] = E;
                }
                io.store(n, a);
            }
        }
    };
    const int step = bw ? -1 : 1;
    int n0 = bw ? nd - 1 : 0;
    load_block<D, 4, 1, PF>(ra, io, n0, step, nd);
    for (int done = 0; done < nd; done += 2 * PF) {
        load_block<D, 4, 1, PF>(rb, io, n0 + step * PF, step, nd);
        block(ra, n0);
        load_block<D, 4, 1, PF>(ra, io, n0 + 2 * step * PF, step, nd);
        block(rb, n0 + step * PF);
        n0 += 2 * step * PF;
    }
    // forward: one step past the last diagonal, column U holds P(y|x); backward: column 0 of diagonal 0
    const int cz = bw ? 0 : U;
    if ((cz >> 8) == wave) {
        double v = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) v = (k == (cz & 3)) ? a[0][k] : v;
        const double zz = __shfl(v, (cz & 255) >> 2, 64);
        if (lane == 0) *z = D::kLog ? zz : log2_d(zz) + (double)E;
    }
}

// Lattices of 256 * NW columns (U1p), one workgroup of NW waves per sample
// and direction: workgroup 2k the forward and 2k+1 the backward sweep of
// the k-th sample in cost order; other samples' workgroups return at once.
template <int NW>
__global__ __launch_bounds__(64 * NW) void k_ab_wide(const SampleDesc *__restrict__ desc,
                                                     const int32_t *__restrict__ order, int B,
                                                     const int *__restrict__ mode, const float4 *__restrict__ node,
                                                     const float2 *__restrict__ prob, double *__restrict__ alpha,
                                                     double *__restrict__ beta, int *__restrict__ ealpha,
                                                     int *__restrict__ ebeta, double *__restrict__ log2z,
                                                     float *__restrict__ loss, int rerun) {
    __shared__ WideShared sh;
    const SampleDesc d = desc[order[blockIdx.x >> 1]];
    if (d.U1p != 256 * NW) return;  // the whole workgroup
    const int md = mode[d.index];
    if (rerun && !(md & kModeRerun)) return;
    const bool bw = (blockIdx.x & 1) != 0;
    double *z = bw ? &log2z[d.index] : &log2z[B + d.index];
    double *out = bw ? beta + d.ab_off : alpha + d.ab_off;
    int *eout = (bw ? ebeta : ealpha) + d.diag_off;
    if (md == 0) wide_sweep<ProbDomain, NW, 8>(d, bw, reinterpret_cast<const char *>(prob + d.slot_off), out, eout, z, sh);
    else wide_sweep<LogDomain, NW, 8>(d, bw, reinterpret_cast<const char *>(node + d.slot_off), out, eout, z, sh);
    if (bw && threadIdx.x == 0) loss[d.index] = (float)(-log2z[d.index] * kLn2D);
}

// Forward-backward check of the probability-domain recursions.  Every
// alignment passes exactly one node of each anti-diagonal, so the sum over an
// anti-diagonal of alpha * beta is P(y|x) on every diagonal.  The scaled
// sweeps keep one exponent per block of diagonals, so a node far below its
// diagonal's largest value can fall out of fp64's range; that is harmless
// where the node carries no alignment mass (the far corners of long
// diagonals), and it is what a sum off P reveals where it does (a lattice
// whose paths favour one kind of edge by many nats per step, for example).
// Mass lost at a node is missing from every later diagonal's sum (alpha) or
// every earlier one's (beta), so a few diagonals spread over the lattice
// reveal it: one wave for each of 16 per sample (bin midpoints, the last
// being the last diagonal, compared with the backward P).  A sum that
// differs from P by more than 4e-6 in log2 (fp64 sums, log2 to ~1e-7), or P
// itself zero, marks the sample for the log-domain rerun of both its
// recursions.
constexpr int kCheckDiagonals = 16;

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Check diagonal j (of kCheckDiagonals) of sample d by one wave: true when
// the sum of alpha * beta over it is off P(y|x) (2^lz).
__device__ __forceinline__ bool check_diagonal(const SampleDesc &d, int j, const double *__restrict__ alpha,
                                               const double *__restrict__ beta, const int *__restrict__ ealpha,
                                               const int *__restrict__ ebeta, double lz) {
    const int lane = threadIdx.x & 63;
    const int T = d.T, U = d.U, nd = T + U;
    const int n = (j + 1 < kCheckDiagonals) ? (int)(((int64_t)(2 * j + 1) * nd) / (2 * kCheckDiagonals)) : nd - 1;
    const int64_t q = d.ab_off + (int64_t)n * d.U1p;
    double s = 0.0;
    for (int u = max(0, n - T + 1) + lane; u <= min(n, U); u += 64) s += alpha[q + u] * beta[q + u];
    s = wave_sum_d(s);
    const double ls = log2_d(s) + (double)(ealpha[d.diag_off + ((n + 1) >> 3)] + ebeta[d.diag_off + ((nd - n) >> 3)]);
    return !(lz > kNegInfD) || !(s > 0.0) || !(fabs(ls - lz) <= 4e-6);
}

__global__ __launch_bounds__(64) void k_check_ab(const SampleDesc *__restrict__ desc, int *__restrict__ mode,
                                                 const double *__restrict__ alpha, const double *__restrict__ beta,
                                                 const int *__restrict__ ealpha, const int *__restrict__ ebeta,
                                                 const double *__restrict__ log2z) {
    const SampleDesc d = desc[blockIdx.x / kCheckDiagonals];
    const int j = blockIdx.x % kCheckDiagonals;
    if (mode[d.index] != 0) return;  // already in the log domain, or marked
    const bool bad = check_diagonal(d, j, alpha, beta, ealpha, ebeta, log2z[d.index]);
    if (bad && threadIdx.x == 0) atomicOr(&mode[d.index], kModeRerun);
}

// Batches below 64 K rows: one two-wave workgroup per sample (wave 0 the
// forward sweep, wave 1 the backward sweep) that also takes the sample's
// mode from the row pass's flag words, checks its probability-domain
// sweeps on the kCheckDiagonals diagonals (eight per wave) and reruns both
// in the log domain when a check fails: one launch instead of three, the
// workgroup barrier standing in for the kernel boundaries.  Writes the
// sample's mode word for the gradient pass and its loss.
__global__ __launch_bounds__(128) void k_ab_small(const SampleDesc *__restrict__ desc,
                                                  const int32_t *__restrict__ order, int B, int rpc,
                                                  const uint32_t *__restrict__ cflags,
                                                  uint32_t *__restrict__ sflags, int *__restrict__ mode,
                                                  const float4 *__restrict__ node, const float2 *__restrict__ prob,
                                                  double *__restrict__ alpha, double *__restrict__ beta,
                                                  int *__restrict__ ealpha, int *__restrict__ ebeta,
                                                  double *__restrict__ log2z, float *__restrict__ loss) {
    __shared__ int bad_any;
    const SampleDesc d = desc[order[blockIdx.x]];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool bw = wave == 1;
    if (threadIdx.x == 0) bad_any = 0;
    // The sample's domain is the OR of its chunks' flags (four loads per
    // lane in flight); the probability-domain sweep's first loads are issued
    // before it is known.
    int md0 = 0;
    auto domain = [&]() {
        const int nch = (int)(((int64_t)d.T * (d.U + 1) + rpc - 1) / rpc);
        const uint32_t *cf = cflags + d.chunk0;
        uint32_t f = 0;
        for (int j = lane; j < nch; j += 256) {
            uint32_t g[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) g[q] = (j + 64 * q < nch) ? cf[j + 64 * q] : 0u;
            f |= g[0] | g[1] | g[2] | g[3];
        }
        md0 = __any((f & (uint32_t)kModeLog) != 0u) ? kModeLog : 0;
        if (threadIdx.x == 0)
            sflags[d.index] = __any((f & (uint32_t)RNNT_DEV_BAD_TARGET) != 0u) ? (uint32_t)RNNT_DEV_BAD_TARGET : 0u;
        return md0 == 0;
    };
    double *z = bw ? &log2z[d.index] : &log2z[B + d.index];
    sweep_sample(d, bw, false, node, prob, alpha, beta, ealpha, ebeta, z, domain);
    __syncthreads();
    int md = md0;
    if (md == 0) {
        // the check of diagonals wave, wave+2, ..., all eight summed together
        // so that their loads are in flight at once
        constexpr int NQ = kCheckDiagonals / 2;
        const int T = d.T, U = d.U, nd = T + U;
        auto diag_of = [&](int q) {
            const int j = wave + 2 * q;
            return (j + 1 < kCheckDiagonals) ? (int)(((int64_t)(2 * j + 1) * nd) / (2 * kCheckDiagonals)) : nd - 1;
        };
        int n[NQ];
        double s[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            n[q] = diag_of(q);
            s[q] = 0.0;
        }
        // After the reduction below, lanes 8q .. 8q+7 hold the sum of
        // diagonal q: each lane loads that diagonal's exponents and P(y|x)
        // with the first columns.
        const int ql = (lane >> 3) & (NQ - 1);
        const int nl = diag_of(ql);
        const int exl = ealpha[d.diag_off + ((nl + 1) >> 3)] + ebeta[d.diag_off + ((nd - nl) >> 3)];
        const double lz = log2z[d.index];
        for (int u = lane; u <= U; u += 64) {
            double a[NQ], b[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const bool in = u >= n[q] - T + 1 && u <= n[q];
                const int64_t at = d.ab_off + (int64_t)n[q] * d.U1p + u;
                a[q] = in ? alpha[at] : 0.0;
                b[q] = in ? beta[at] : 0.0;
            }
#pragma unroll
            for (int q = 0; q < NQ; ++q) s[q] += a[q] * b[q];
        }
        // Eight sums over the wave in ten lane exchanges: at offsets 32, 16
        // and 8 each lane keeps the half of its sums that its lane bit
        // selects and adds its partner's copy of that half (so afterwards
        // lane bits 5..3 name the diagonal), then offsets 4, 2, 1 finish it;
        // one log2 per lane then serves all eight diagonals.
#pragma unroll
        for (int q = 0; q < NQ / 2; ++q) {
            const bool up = (lane & 32) != 0;
            const double keep = up ? s[q + 4] : s[q], give = up ? s[q] : s[q + 4];
            s[q] = keep + __shfl_xor(give, 32, 64);
        }
#pragma unroll
        for (int q = 0; q < NQ / 4; ++q) {
            const bool up = (lane & 16) != 0;
            const double keep = up ? s[q + 2] : s[q], give = up ? s[q] : s[q + 2];
            s[q] = keep + __shfl_xor(give, 16, 64);
        }
        {
            const bool up = (lane & 8) != 0;
            const double keep = up ? s[1] : s[0], give = up ? s[0] : s[1];
            s[0] = keep + __shfl_xor(give, 8, 64);
        }
#pragma unroll
        for (int off = 4; off > 0; off >>= 1) s[0] += __shfl_xor(s[0], off, 64);
        const double ls = log2_d(s[0]) + (double)exl;
        const bool bad = !(lz > kNegInfD) || __any(!(s[0] > 0.0) || !(fabs(ls - lz) <= 4e-6));
        if (bad && lane == 0) atomicOr(&bad_any, 1);
        __syncthreads();
        if (bad_any) {
            md = kModeRerun;
            sweep_sample(d, bw, true, node, prob, alpha, beta, ealpha, ebeta, z);
        }
    }
    if (threadIdx.x == 0) mode[d.index] = md;
    if (bw && lane == 0) loss[d.index] = (float)(-log2z[d.index] * kLn2D);
}

// --------------------------------------------------------------- reduction
// One wave: cross-checks the two sweeps' log2 P(y|x) of every sample
// (README "Value" section 3), then (out non-null) reduces the per-sample
// losses: sum, or mean over B, in a fixed order.  With status_out set, the
// final status word (every earlier kernel's bits and this one's) is copied
// there.  Run by the first workgroup of the gradient launch, or on its own
// (k_reduce) when there is no gradient pass.
// With sflags (a small batch: each sample's status bits, from the row
// pass's per-chunk flag words) the status word is written whole, their OR
// and this one's bits, instead of adding bits to a word k_plan cleared.
__device__ void reduce_losses(const float *__restrict__ loss, const double *__restrict__ log2z, int B, int mean,
                              float *__restrict__ out, uint32_t *status, uint32_t *status_out,
                              const uint32_t *__restrict__ sflags) {
    double s = 0.0;
    bool agree = true;
    for (int i = threadIdx.x; i < B; i += 64) {
        s += (double)loss[i];
        const double lb = -log2z[i] * kLn2D;
        const double la = -log2z[B + i] * kLn2D;
        agree = agree && ((la == lb) || (fabs(la - lb) <= 1e-4 * fmax(1.0, fabs(lb))));
    }
    uint32_t f = 0;
    if (sflags)
        for (int i = threadIdx.x; i < B; i += 64) f |= sflags[i];
    const uint32_t bad_label = __any((f & (uint32_t)RNNT_DEV_BAD_TARGET) != 0u) ? (uint32_t)RNNT_DEV_BAD_TARGET : 0u;
    const uint32_t bit = __any(!agree) ? (uint32_t)RNNT_DEV_LOSS_MISMATCH : 0u;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (threadIdx.x == 0) {
        uint32_t word;
        if (sflags) {
            word = bad_label | bit;
            *status = word;
        } else {
            word = atomicOr(status, bit) | bit;
        }
        if (status_out) *status_out = word;
        if (out) out[0] = (float)(mean ? s / (double)B : s);
    }
}

// ------------------------------------------------------------ K3: gradient
// g_k = P(k|t,u) * occ(t,u) - [k = blank] flow_b - [k = y_{u+1}] flow_y, where
// occ = alpha*beta/P(y|x) and the flows are the posterior probabilities of
// leaving (t,u) by blank or by the next label.  P * occ is evaluated as
// exp2((x - m) * log2(e) + shift) with the row's maximum m and one per-row
// shift log2(occ * scale) - log2(sum of exp(x - m)): every term is of the
// size of x - m and the shift, never of x itself, so a common offset of the
// row's logits changes nothing (the fp32 rounding of x * log2(e) at large |x|
// would).  With a FastEmit weight lambda (the FastEmit paper's rule: the
// label-emission derivatives times 1 + lambda) the label flow is
// (1 + lambda) flow_y and, through the log_softmax chain rule, the softmax
// term carries occ + lambda flow_y.
struct RowTerms {
    float m;       // the row's reference value (its maximum), 0 if not fused
    float shift2;  // log2(occ * scale) - log2(sum of exp(x - m)), or -inf
    float fb;      // scaled blank flow
    float fy;      // scaled label flow
    int y;         // next label, -1 at u = U or when not a non-blank class
};

struct SampleTerms {
    double log2z;
    bool log_mode;
};

// log2 of a forward (ge = ealpha group index (n+1)/8) or backward (ge =
// (nd-n)/8) node value.
__device__ __forceinline__ double node_log2(const double *__restrict__ v, const int *__restrict__ e, int64_t s,
                                            int ge, bool log_mode) {
    return log_mode ? v[s] : log2_d(v[s]) + (double)e[ge];
}

// Terms of node (t, u) from its skewed slots: the row's maximum, log-sum and
// log-probs (node), alpha, beta and beta of the two successors; the label
// from the targets.
__device__ __forceinline__ RowTerms row_terms(const SampleDesc &d, const SampleTerms &st, int t, int u,
                                              const float4 *__restrict__ node, const double *__restrict__ alpha,
                                              const double *__restrict__ beta, const int *__restrict__ ealpha,
                                              const int *__restrict__ ebeta, float log2_scale, float scale,
                                              float fastemit, float scale_y, bool fused, int V, int blank,
                                              const int32_t *__restrict__ targets, int S) {
    const int U1 = d.U + 1;
    const int n = t + u;
    const int64_t s = d.slot_off + (int64_t)n * U1 + u;      // node slot
    const int64_t q = d.ab_off + (int64_t)n * d.U1p + u;     // alpha / beta slot
    const int U1p = d.U1p;
    const int *ea = ealpha + d.diag_off;
    const int *eb = ebeta + d.diag_off;
    const int nd = d.T + d.U;
    const float4 l = node[s];
    double lb = kNegInfD, ly = kNegInfD, lo = kNegInfD;
    if (st.log2z != kNegInfD) {
        const double a2 = node_log2(alpha, ea, q, (n + 1) >> 3, st.log_mode) - st.log2z;
        lo = a2 + node_log2(beta, eb, q, (nd - n) >> 3, st.log_mode);
        const int gnext = (nd - n - 1) >> 3;
        if (t < d.T - 1) lb = a2 + (double)l.x * kLog2eD + node_log2(beta, eb, q + U1p, gnext, st.log_mode);
        else if (u == d.U) lb = a2 + (double)l.x * kLog2eD;
        if (u < d.U) ly = a2 + (double)l.y * kLog2eD + node_log2(beta, eb, q + U1p + 1, gnext, st.log_mode);
    }
    // occ + lambda flow_y = occ (1 + lambda 2^(ly - lo)); flow_y <= occ, so
    // the exponent is at most about zero.  A node whose occupancy underflowed
    // (a far corner of the lattice in the probability domain) keeps it at
    // zero: -inf + inf would be NaN.
    if (fastemit > 0.f && ly != kNegInfD && lo != kNegInfD)
        lo += (double)log2f(1.f + fastemit * exp2_fast((float)(ly - lo)));
    RowTerms r;
    r.m = l.z;
    r.shift2 = fused ? (float)(lo - (double)l.w) + log2_scale : kNegInf;
    r.fb = exp2_fast((float)lb) * scale;
    r.fy = exp2_fast((float)ly) * scale_y;
    r.y = label_of(d, u, V, blank, targets, S);
    return r;
}

// The reduction the gradient launch's first workgroup performs (on = 0: none).
struct ReduceArgs {
    const float *loss;
    float *out;
    uint32_t *status;
    uint32_t *status_out;
    const uint32_t *sflags;  // small batches: each sample's status bits, else null
    int B, mean, on;
};

struct GradArgs {
    ReduceArgs red;
    int V, blank, n_chunks, S;
    float clamp, scale, log2_scale;
    float fastemit, scale_y;  // FastEmit weight; scale * (1 + fastemit)
    const int32_t *targets;
    const SampleDesc *desc;
    const ChunkDesc *chunks;
    const int *mode;
    const double *log2z;
    const float4 *node;
    const double *alpha;
    const double *beta;
    const int *ealpha;
    const int *ebeta;
};

// The workspace arrays reach the gradient kernels as separate restrict
// parameters, so the compiler knows the gradient stores cannot clobber them
// and reads their wave-uniform elements through the scalar cache.
#define RNNT_GRAD_PARAMS                                                                                      \
    int V, int blank, int n_chunks, int S, float clamp, float scale, float log2_scale, float fastemit,          \
        float scale_y, const int32_t *__restrict__ targets, const SampleDesc *__restrict__ desc,                \
        const ChunkDesc *__restrict__ chunks, const int *__restrict__ mode, const double *__restrict__ log2z,   \
        const float4 *__restrict__ node, const double *__restrict__ alpha, const double *__restrict__ beta,     \
        const int *__restrict__ ealpha, const int *__restrict__ ebeta, ReduceArgs red
#define RNNT_GRAD_ARGS(g)                                                                                    \
    g.V, g.blank, g.n_chunks, g.S, g.clamp, g.scale, g.log2_scale, g.fastemit, g.scale_y, g.targets, g.desc,   \
        g.chunks, g.mode, g.log2z, g.node, g.alpha, g.beta, g.ealpha, g.ebeta, g.red

__device__ __forceinline__ float clamp_to(float v, float cl, bool do_clamp) {
    return do_clamp ? fminf(fmaxf(v, -cl), cl) : v;
}

// The gradient of (part of) one row held the way the wide kernels hold it:
// lane l keeps vectors (i0 + i)*64 + l, i < NV, written to dst (the row).
// The blank and label elements get their flow subtracted in the registers
// of the vector that holds them: element k is element k % VEC of vector
// k / VEC, held by lane (k / VEC) mod 64 as its vector number (k / VEC) / 64.
// The registers are overwritten with the stored gradient.
template <typename T, int NV, bool FULL, bool FUSED, bool CLAMP>
__device__ __forceinline__ void grad_row(typename Raw<T>::vec (&xc)[NV], T *dst, const RowTerms &rt, int blank,
                                         int nvec, float cl, int i0 = 0) {
    constexpr int VEC = Raw<T>::kVec;
    const int lane = threadIdx.x & 63;
    const int vb = blank / VEC, vy = rt.y >= 0 ? rt.y / VEC : -1;  // the vectors holding them
    const int eb = blank - vb * VEC, ey = rt.y - vy * VEC;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = i0 + j;
        const int vi = i * 64 + lane;
        if (FULL || vi < nvec) {
            float gv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float v = 0.f;
                if constexpr (FUSED) v = exp2_fast(fmaf(Raw<T>::get(xc[j], e) - rt.m, kLog2e, rt.shift2));
                gv[e] = v;
            }
            if ((vb >> 6) == i) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) gv[e] -= (vi == vb && e == eb) ? rt.fb : 0.f;
            }
            if (vy >= 0 && (vy >> 6) == i) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) gv[e] -= (vi == vy && e == ey) ? rt.fy : 0.f;
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) gv[e] = clamp_to(gv[e], cl, CLAMP);
            xc[j] = Raw<T>::put(gv);
            store_raw<T, true>(dst + (int64_t)vi * VEC, xc[j]);
        }
    }
}

// The gradient, one wave per workgroup and `split` workgroups per row (SPLIT,
// when the launch fixes it at compile time), each taking a part of NV 16-byte
// vectors per lane (4 KiB at NV = 4; the last part may be partial unless
// FULL).  With NV = 5, parts of part_blocks blocks of 64 vectors and a last
// part of last_blocks: one part of five blocks for a row of 4 to 5 KiB, or parts of four
// and a last one of five where a row would end in a part of at most one block
// (an 8194-byte row: two waves instead of three): each
// wave loads its part
// of the row, computes and stores it, and exits.  Many single-wave
// workgroups of 4 KiB keep enough rows in flight without a prefetch ring
// (and run faster than four-wave workgroups over four rows).  Workgroup b
// takes part (b % PB) % split of row (b % PB) / split of chunk n_chunks-1-b/PB
// (PB = rows per chunk * split, row order), so the chunks run in the reverse of
// the row pass's order, which starts where that pass ended (measured 6%
// faster than the forward order for a write-only gradient, 0.5% otherwise).
// Forms, as measured on MI355X: fused rows take the masked form with the
// split at run time (8 KiB fp16 rows: 2.19 ms against 2.30 ms unmasked);
// log-prob inputs (a write-only pass) take the unmasked form, with the split
// fixed when it is one (4 KiB rows: 0.995 ms against 1.016 at run time and
// 1.045 masked).
template <typename T, bool FUSED, bool CLAMP, int SPLIT, bool FULL, int NV>
__global__ __launch_bounds__(64) void k_grad_rows(const T *logits, T *grad, int blocks_per_chunk,
                                                  int64_t block_base, int split_rt, int part_blocks, int last_blocks,
                                                  RNNT_GRAD_PARAMS) {
    constexpr int VEC = Raw<T>::kVec;
    if (red.on && blockIdx.x == 0)
        reduce_losses(red.loss, log2z, red.B, red.mean, red.out, red.status, red.status_out, red.sflags);
    const int bpc = blocks_per_chunk;
    const int64_t b = block_base + blockIdx.x;
    const ChunkDesc c = chunks[n_chunks - 1 - (int)(b / bpc)];
    const int part = (int)(b % bpc);
    const int split = SPLIT > 0 ? SPLIT : split_rt;
    const int r = part / split;
    if (r >= c.count) return;
    // the part's 64-vector blocks: NV, or (NV = 5) pb each and pb_last in the last part
    const int ip = part % split;
    const int i0 = NV == 4 ? ip * NV : ip * part_blocks;
    const SampleDesc d = desc[c.sample];
    const int lane = threadIdx.x & 63;
    const int nvec = NV == 4 ? V / VEC : min(V / VEC, (i0 + (ip == split - 1 ? last_blocks : part_blocks)) * 64);
    const int U1 = d.U + 1;
    const int t = (c.row_begin + r) / U1;
    const int u = (c.row_begin + r) - t * U1;
    const int64_t row = row_of(d, t, u);
    using Vec = typename Raw<T>::vec;
    Vec x[NV];
    if constexpr (FUSED) {
        const T *p = logits + row * (int64_t)V;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int vi = (i0 + j) * 64 + lane;
            if (FULL || vi < nvec) x[j] = load_raw<T, true>(p + (int64_t)vi * VEC);
        }
    }
    const SampleTerms st{log2z[d.index], mode[d.index] != 0};
    const RowTerms rt = row_terms(d, st, t, u, node, alpha, beta, ealpha, ebeta, log2_scale, scale, fastemit,
                                  scale_y, FUSED, V, blank, targets, S);
    grad_row<T, NV, FULL, FUSED, CLAMP>(x, grad + row * (int64_t)V, rt, blank, nvec, clamp * scale, i0);
}

// The gradient of rows whose boundaries can fall inside a 128-byte line (a
// row length that is no multiple of 128 bytes, or a gradient that is not
// 128-byte aligned), one wave per part of at most 4 KiB as in k_grad_rows.
// A line that holds the end of one row and the start of the next, where the
// two rows are adjacent in memory and in the lattice ((t, u) and (t, u+1), or
// (t, U) and (t+1, 0) when the time steps are packed without padding), is
// written whole by the later row's waves, which compute the earlier row's
// last vectors with that row's terms: written in two pieces by two
// workgroups, each such line cost as much as many whole ones (20000-byte fp32
// rows streamed 7-9% slower than 19968- or 20480-byte ones, 4000-byte rows
// 12% slower than 3968-byte ones).  The vectors a row's waves take, from
// position 0: the kp vectors of the previous row in the line holding the
// row's start (if they are adjacent), then the row's own vectors, except those
// in the line holding its end when the next row takes that line.  A row
// whose predecessor is not adjacent starts mid-line, and its walk begins at
// its first line boundary (vector number i is position (i + h) mod nw, the h
// vectors before that boundary last), so that each instruction's 64 vectors
// still fill whole lines.  Every element is computed as k_grad_rows computes
// it, so both give the same bits.
template <typename T, bool FUSED, bool CLAMP, int NV>
__global__ __launch_bounds__(64) void k_grad_rows_line(const T *logits, T *grad, int blocks_per_chunk,
                                                       int64_t block_base, int split, int part_blocks, int last_blocks,
                                                       RNNT_GRAD_PARAMS) {
    constexpr int VEC = Raw<T>::kVec;
    if (red.on && blockIdx.x == 0)
        reduce_losses(red.loss, log2z, red.B, red.mean, red.out, red.status, red.status_out, red.sflags);
    const int bpc = blocks_per_chunk;
    const int64_t b = block_base + blockIdx.x;
    const ChunkDesc c = chunks[n_chunks - 1 - (int)(b / bpc)];
    const int part = (int)(b % bpc);
    const int r = part / split;
    if (r >= c.count) return;
    // the part's 64-vector blocks (as in k_grad_rows)
    const int ip = part % split;
    const int i0 = NV == 4 ? ip * NV : ip * part_blocks;
    const int iend = NV == 4 ? i0 + NV : i0 + (ip == split - 1 ? last_blocks : part_blocks);
    const SampleDesc d = desc[c.sample];
    const int lane = threadIdx.x & 63;
    const int nvec = V / VEC;
    const int U1 = d.U + 1;
    const int t = (c.row_begin + r) / U1;
    const int u = (c.row_begin + r) - t * U1;
    const int64_t row = row_of(d, t, u);
    // the rows before and after this one in memory, if they are its lattice neighbours
    const bool packed = d.tstride == U1;
    const bool adj_prev = u > 0 || (packed && t > 0);
    const bool adj_next = u < d.U || (packed && t < d.T - 1);
    const uint32_t so = (uint32_t)reinterpret_cast<uintptr_t>(grad + row * (int64_t)V) & 127u;  // start in its line
    const uint32_t eo = (so + (uint32_t)V * (uint32_t)sizeof(T)) & 127u;                       // end in its line
    const int kp = adj_prev ? (int)(so >> 4) : 0;               // the previous row's vectors at the front
    const int nw = kp + nvec - (adj_next ? (int)(eo >> 4) : 0);  // vectors this row's waves take
    // (a part past nw exists only where some row of the launch takes nvec + kp
    // vectors across one more part than the row alone needs)
    if (i0 * 64 >= nw) return;
    const int nwp = min(nw, iend * 64);  // this part's end
    const int h = adj_prev ? 0 : (int)(((128u - so) & 127u) >> 4);
    const int64_t e0 = row * (int64_t)V - (int64_t)kp * VEC;  // element offset of position 0
    auto position = [&](int vi) { const int v = vi + h; return v >= nw ? v - nw : v; };
    using Vec = typename Raw<T>::vec;
    Vec x[NV];
    if constexpr (FUSED) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int vi = (i0 + j) * 64 + lane;
            if (vi < nwp) x[j] = load_raw<T, true>(logits + e0 + (int64_t)position(vi) * VEC);
        }
    }
    const SampleTerms st{log2z[d.index], mode[d.index] != 0};
    const RowTerms rt = row_terms(d, st, t, u, node, alpha, beta, ealpha, ebeta, log2_scale, scale, fastemit,
                                  scale_y, FUSED, V, blank, targets, S);
    // the previous row's terms, for the part that holds its vectors (positions
    // below kp; h = 0 whenever kp > 0, so these are vector numbers 0 .. kp-1)
    RowTerms rp = rt;
    if (kp > 0 && i0 == 0)
        rp = row_terms(d, st, u > 0 ? t : t - 1, u > 0 ? u - 1 : d.U, node, alpha, beta, ealpha, ebeta, log2_scale,
                       scale, fastemit, scale_y, FUSED, V, blank, targets, S);
    // vector numbers of the blank and label elements: this row's vector k at
    // position kp + k (if this row's waves take it), the previous row's at
    // k - (nvec - kp) (if among its last kp vectors); -1 where not taken here
    auto number_of = [&](int pos) { return pos < 0 || pos >= nw ? -1 : (pos >= h ? pos - h : pos - h + nw); };
    const int pb = blank / VEC, eb = blank - pb * VEC;
    const int py = rt.y >= 0 ? rt.y / VEC : -1, ey = rt.y - py * VEC;
    const int pyp = rp.y >= 0 ? rp.y / VEC : -1, eyp = rp.y - pyp * VEC;
    const int vb = number_of(kp + pb), vy = py >= 0 ? number_of(kp + py) : -1;
    const int vbp = kp > 0 ? number_of(pb - (nvec - kp)) : -1;
    const int vyp = (kp > 0 && pyp >= 0) ? number_of(pyp - (nvec - kp)) : -1;
    const float cl = clamp * scale;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = i0 + j;
        const int vi = i * 64 + lane;
        if (vi < nwp) {
            const bool prev = vi < kp;
            const float m = prev ? rp.m : rt.m, shift2 = prev ? rp.shift2 : rt.shift2;
            float gv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float v = 0.f;
                if constexpr (FUSED) v = exp2_fast(fmaf(Raw<T>::get(x[j], e) - m, kLog2e, shift2));
                gv[e] = v;
            }
            if ((vb >> 6) == i) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) gv[e] -= (vi == vb && e == eb) ? rt.fb : 0.f;
            }
            if ((vy >> 6) == i) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) gv[e] -= (vi == vy && e == ey) ? rt.fy : 0.f;
            }
            if (i == 0 && kp > 0) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    gv[e] -= (vi == vbp && e == eb) ? rp.fb : 0.f;
                    gv[e] -= (vi == vyp && e == eyp) ? rp.fy : 0.f;
                }
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) gv[e] = clamp_to(gv[e], cl, CLAMP);
            x[j] = Raw<T>::put(gv);
            store_raw<T, true>(grad + e0 + (int64_t)position(vi) * VEC, x[j]);
        }
    }
}

// The gradient of rows that do not all start on a 16-byte boundary (a row
// length that is no multiple of 16 bytes, or gradient and logits off such a
// boundary by the same amount), in the 16-byte vectors that cover them: as in
// k_grad_rows_line, a row's waves own the bytes from the 128-byte line that
// holds its start, when the previous row is its lattice neighbour in memory
// (else from its first element), to the line that holds its end when the next
// row is (else to its last element), and compute the previous row's elements
// in that first line with the previous row's terms, element by element in the
// vector where the two rows meet.  A vector that reaches past owned bytes (at
// a row edge with no such neighbour) is stored element by element; its load
// reads the whole vector, which stays in the 16-byte block, so the page, of
// an element of the row.  Rows that start mid-line after a non-neighbour are
// walked from their first line boundary.  Each element is computed as in
// k_grad_rows.
template <typename T, bool FUSED, bool CLAMP, int NV>
__global__ __launch_bounds__(64) void k_grad_rows_odd(const T *logits, T *grad, int blocks_per_chunk,
                                                      int64_t block_base, int split, int part_blocks, int last_blocks,
                                                      RNNT_GRAD_PARAMS) {
    constexpr int VEC = Raw<T>::kVec;
    constexpr int ES = (int)sizeof(T);
    if (red.on && blockIdx.x == 0)
        reduce_losses(red.loss, log2z, red.B, red.mean, red.out, red.status, red.status_out, red.sflags);
    const int bpc = blocks_per_chunk;
    const int64_t b = block_base + blockIdx.x;
    const ChunkDesc c = chunks[n_chunks - 1 - (int)(b / bpc)];
    const int part = (int)(b % bpc);
    const int r = part / split;
    if (r >= c.count) return;
    // the part's 64-vector blocks (as in k_grad_rows)
    const int ip = part % split;
    const int i0 = NV == 4 ? ip * NV : ip * part_blocks;
    const int iend = NV == 4 ? i0 + NV : i0 + (ip == split - 1 ? last_blocks : part_blocks);
    const SampleDesc d = desc[c.sample];
    const int lane = threadIdx.x & 63;
    const int U1 = d.U + 1;
    const int t = (c.row_begin + r) / U1;
    const int u = (c.row_begin + r) - t * U1;
    const int64_t row = row_of(d, t, u);
    const bool packed = d.tstride == U1;
    const bool adj_prev = u > 0 || (packed && t > 0);
    const bool adj_next = u < d.U || (packed && t < d.T - 1);
    // byte addresses: the row [rs, re), the owned bytes [a0, a1), the first vector v0
    const uintptr_t rs = reinterpret_cast<uintptr_t>(grad + row * (int64_t)V);
    const uintptr_t re = rs + (uintptr_t)V * ES;
    const uintptr_t a0 = adj_prev ? (rs & ~(uintptr_t)127) : rs;
    const uintptr_t a1 = adj_next ? (re & ~(uintptr_t)127) : re;
    const uintptr_t v0 = a0 & ~(uintptr_t)15;
    const int nw = (int)((((a1 + 15) & ~(uintptr_t)15) - v0) >> 4);  // vectors this row's waves take
    // (a part past nw exists only where some row of the launch needs one more)
    if (i0 * 64 >= nw) return;
    const int nwp = min(nw, iend * 64);  // this part's end
    const int h = adj_prev ? 0 : (int)(((128u - (uint32_t)(v0 & 127u)) & 127u) >> 4);
    // slots (elements from v0): owned [o0, o1), the row's first element at os
    const int o0 = (int)((a0 - v0) / ES), o1 = (int)((a1 - v0) / ES), os = (int)((rs - v0) / ES);
    const int64_t e0 = row * (int64_t)V - os;  // tensor element at slot 0
    auto position = [&](int vi) { const int v = vi + h; return v >= nw ? v - nw : v; };
    using Vec = typename Raw<T>::vec;
    Vec x[NV];
    if constexpr (FUSED) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int vi = (i0 + j) * 64 + lane;
            if (vi < nwp) x[j] = load_raw<T, true>(logits + e0 + (int64_t)position(vi) * VEC);
        }
    }
    const SampleTerms st{log2z[d.index], mode[d.index] != 0};
    const RowTerms rt = row_terms(d, st, t, u, node, alpha, beta, ealpha, ebeta, log2_scale, scale, fastemit,
                                  scale_y, FUSED, V, blank, targets, S);
    // the previous row's last elements, slots o0 .. os-1 (h = 0 here, so
    // within this row's first eight vectors: vector numbers below 64)
    const bool has_prev = o0 < os;
    RowTerms rp = rt;
    if (has_prev && i0 == 0)
        rp = row_terms(d, st, u > 0 ? t : t - 1, u > 0 ? u - 1 : d.U, node, alpha, beta, ealpha, ebeta, log2_scale,
                       scale, fastemit, scale_y, FUSED, V, blank, targets, S);
    // vector numbers and lanes' slots of the blank and label elements: this
    // row's element k at slot os + k, the previous row's at os - V + k; -1
    // where not owned here
    auto number_of = [&](int slot) {
        const int q = slot / VEC;
        return q >= h ? q - h : q - h + nw;
    };
    const int sb = os + blank, sy = rt.y >= 0 ? os + rt.y : -1;
    const int sbp = os - V + blank, syp = rp.y >= 0 ? os - V + rp.y : -1;
    const int vb = sb < o1 ? number_of(sb) : -1;
    const int vy = (sy >= 0 && sy < o1) ? number_of(sy) : -1;
    const int vbp = (has_prev && sbp >= o0) ? number_of(sbp) : -1;
    const int vyp = (has_prev && syp >= o0) ? number_of(syp) : -1;
    const int eb = sb % VEC, ey = sy >= 0 ? sy % VEC : 0;
    const int ebp = sbp >= 0 ? sbp % VEC : 0, eyp = syp >= 0 ? syp % VEC : 0;
    const float cl = clamp * scale;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = i0 + j;
        const int vi = i * 64 + lane;
        if (vi < nwp) {
            const int s0 = position(vi) * VEC;  // the vector's first slot
            float gv[VEC];
            if (i == 0 && has_prev) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const bool prev = s0 + e < os;
                    const float m = prev ? rp.m : rt.m, shift2 = prev ? rp.shift2 : rt.shift2;
                    float v = 0.f;
                    if constexpr (FUSED) v = exp2_fast(fmaf(Raw<T>::get(x[j], e) - m, kLog2e, shift2));
                    gv[e] = v - ((vi == vbp && e == ebp) ? rp.fb : 0.f) - ((vi == vyp && e == eyp) ? rp.fy : 0.f);
                }
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float v = 0.f;
                    if constexpr (FUSED) v = exp2_fast(fmaf(Raw<T>::get(x[j], e) - rt.m, kLog2e, rt.shift2));
                    gv[e] = v;
                }
            }
            if ((vb >> 6) == i) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) gv[e] -= (vi == vb && e == eb) ? rt.fb : 0.f;
            }
            if ((vy >> 6) == i) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) gv[e] -= (vi == vy && e == ey) ? rt.fy : 0.f;
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) gv[e] = clamp_to(gv[e], cl, CLAMP);
            T *dst = grad + e0 + s0;
            if (s0 >= o0 && s0 + VEC <= o1) {
                store_raw<T, true>(dst, Raw<T>::put(gv));
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (s0 + e >= o0 && s0 + e < o1) dst[e] = (T)gv[e];
            }
        }
    }
}

template <typename T, int VEC, int G, bool FUSED>
__global__ __launch_bounds__(256) void k_grad_narrow(const T *logits, T *grad, RNNT_GRAD_PARAMS) {
    constexpr int RPW = 64 / G;
    if (red.on && blockIdx.x == 0 && threadIdx.x < 64)
        reduce_losses(red.loss, log2z, red.B, red.mean, red.out, red.status, red.status_out, red.sflags);
    const ChunkDesc c = chunks[n_chunks - 1 - blockIdx.x];
    const SampleDesc d = desc[c.sample];
    const SampleTerms st{log2z[d.index], mode[d.index] != 0};
    const int U1 = d.U + 1;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane & (G - 1);
    const int grp = lane / G;
    const int nvec = V / VEC;
    const float cl = clamp * scale;
    const bool do_clamp = clamp > 0.f;
    for (int base = wave * RPW; base < c.count; base += 4 * RPW) {
        const int r = base + grp;
        if (r >= c.count) continue;
        const int lr = c.row_begin + r;
        const int t = lr / U1;
        const int u = lr - t * U1;
        const int64_t row = row_of(d, t, u);
        const T *src = logits + row * (int64_t)V;
        // the lane's first vector of the row is loaded before the row's terms,
        // whose loads it does not depend on
        float x0[VEC] = {};
        if constexpr (FUSED)
            if (sub < nvec) load_n<T, VEC>(src + (int64_t)sub * VEC, x0);
        const RowTerms rt = row_terms(d, st, t, u, node, alpha, beta, ealpha, ebeta, log2_scale, scale, fastemit,
                                      scale_y, FUSED, V, blank, targets, S);
        T *dst = grad + row * (int64_t)V;
        const int vb = blank / VEC, vy = rt.y >= 0 ? rt.y / VEC : -1;
        const int eb = blank - vb * VEC, ey = rt.y - vy * VEC;
        for (int i = sub; i < nvec; i += G) {
            float x[VEC];
            if constexpr (FUSED) {
                if (i == sub) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) x[e] = x0[e];
                } else {
                    load_n<T, VEC>(src + (int64_t)i * VEC, x);
                }
            }
            float gv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float v = 0.f;
                if constexpr (FUSED) v = exp2_fast(fmaf(x[e] - rt.m, kLog2e, rt.shift2));
                v -= (i == vb && e == eb) ? rt.fb : 0.f;
                v -= (i == vy && e == ey) ? rt.fy : 0.f;
                gv[e] = clamp_to(v, cl, do_clamp);
            }
            store_n<T, VEC>(dst + (int64_t)i * VEC, gv);
        }
    }
}

__global__ __launch_bounds__(64) void k_reduce(const float *__restrict__ loss, const double *__restrict__ log2z,
                                               int B, int mean, float *__restrict__ out, uint32_t *status,
                                               uint32_t *status_out, const uint32_t *__restrict__ sflags) {
    reduce_losses(loss, log2z, B, mean, out, status, status_out, sflags);
}

// Upstream-gradient scaling of an already written gradient: each workgroup
// takes 4 * 64/G consecutive packed rows; with a per-sample factor, a row's
// sample is found by binary search over the samples' first rows.
template <typename T, int VEC, int G>
__global__ __launch_bounds__(256) void k_grad_scale(T *grad, int V, int64_t N, int B,
                                                    const SampleDesc *__restrict__ desc,
                                                    const float *__restrict__ scale, int per_sample) {
    constexpr int RPW = 64 / G;
    const int lane = threadIdx.x & 63;
    const int sub = lane & (G - 1);
    const int64_t row = (int64_t)blockIdx.x * (4 * RPW) + (threadIdx.x >> 6) * RPW + lane / G;
    if (row >= N) return;
    int s = 0;
    if (per_sample) {
        int lo = 0, hi = B - 1;  // last sample whose first row is <= row
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (desc[mid].row_off <= row) lo = mid;
            else hi = mid - 1;
        }
        s = desc[lo].index;
    }
    const float f = scale[s];
    if (f == 1.0f) return;
    T *p = grad + row * (int64_t)V;
    const int nvec = V / VEC;
    for (int i = sub; i < nvec; i += G) {
        float x[VEC];
        load_n<T, VEC>(p + (int64_t)i * VEC, x);
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[e] *= f;
        store_n<T, VEC>(p + (int64_t)i * VEC, x);
    }
}

// Padded layout: write zeros to every gradient row outside its sample's
// lattice (t >= T_i or u > U_i), so the padded gradient is fully defined.
// One row per group of G lanes; rows of a sample are (t, u) for t < max_T,
// u < max_U1.
template <typename T, int VEC, int G>
__global__ __launch_bounds__(256) void k_zero_padding(T *grad, int V, int B, int max_T, int max_U1,
                                                      const SampleDesc *__restrict__ desc) {
    constexpr int RPW = 64 / G;
    const int64_t per_sample = (int64_t)max_T * max_U1;
    const int64_t rows = per_sample * B;
    const int lane = threadIdx.x & 63;
    const int sub = lane & (G - 1);
    const int nvec = V / VEC;
    const int64_t step = (int64_t)gridDim.x * 4 * RPW;
    for (int64_t row = (int64_t)blockIdx.x * (4 * RPW) + (threadIdx.x >> 6) * RPW + lane / G; row < rows;
         row += step) {
        const int i = (int)(row / per_sample);
        const int64_t r = row - (int64_t)i * per_sample;
        const int t = (int)(r / max_U1);
        const int u = (int)(r - (int64_t)t * max_U1);
        const SampleDesc d = desc[i];
        if (t < d.T && u <= d.U) continue;
        T *p = grad + row * (int64_t)V;
        float z[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) z[e] = 0.f;
        for (int k = sub; k < nvec; k += G) store_n<T, VEC>(p + (int64_t)k * VEC, z);
    }
}

// ------------------------------------------------------------- dispatchers
template <typename T, int VEC, int N> struct Tag {
    using type = T;
    static constexpr int vec = VEC;
    static constexpr int n = N;
};

// Narrow geometry: N = lanes per row.  Wide geometry: N = vectors per lane.
template <typename Fn> hipError_t with_narrow(int esize, int vec, int G, Fn &&fn) {
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
    // Rows of more than 1 KiB: one row per wave in the row pass, one wave per
    // part of 4 or 5 KiB in the gradient pass, in 16-byte vectors (rows not
    // all on 16-byte boundaries span one vector more).
    const int64_t row_bytes = (int64_t)V * esize;
    const int64_t vspan = aligned16 ? row_bytes / 16 : (row_bytes + 30) / 16;
    g.stream_parts = row_bytes > 1024 ? (int)((vspan + 255) / 256) : 0;
    return g;
}

#define WS(type, field) reinterpret_cast<type>(a.ws + a.lay.field)

hipError_t launch_plan(const LaunchArgs &a, const PlanArgs *pa, hipStream_t stream) {
    const int gx = (a.lay.max_sample_chunks + 255) / 256;
    const dim3 grid((unsigned)((int64_t)gx * a.B)), block(256);
    if (pa)
        hipLaunchKernelGGL(k_plan<true>, grid, block, 0, stream, WS(const SampleDesc *, desc), a.lay.rows_per_chunk,
                           gx, WS(ChunkDesc *, chunks), *pa, WS(SampleDesc *, desc), WS(int32_t *, order),
                           WS(int *, mode), WS(uint32_t *, status));
    else
        hipLaunchKernelGGL(k_plan<false>, grid, block, 0, stream, WS(const SampleDesc *, desc), a.lay.rows_per_chunk,
                           gx, WS(ChunkDesc *, chunks), PlanArgs{}, nullptr, nullptr, nullptr, nullptr);
    return hipGetLastError();
}

// The row pass with its work source: the chunk table (TableSrc), or for a
// small batch the descriptors in `pa` (ArgSrc).
template <typename Src>
hipError_t launch_rowstats_with(const LaunchArgs &a, const Src &src, hipStream_t stream) {
    const dim3 grid(a.lay.n_chunks), block(256);
    // one row per wave: the chunks are walked in diagonal order
    const bool diag = a.geom.stream_parts > 0;
    if (!a.fused) {
        auto go = [&](auto tag, auto dtag) {
            using T = decltype(tag);
            constexpr bool D = decltype(dtag)::value;
            hipLaunchKernelGGL((k_gather<T, D, Src>), grid, block, 0, stream, static_cast<const T *>(a.logits), a.V,
                               a.blank, src, a.targets, a.S, WS(float4 *, node), WS(float2 *, prob));
            return hipGetLastError();
        };
        if (a.esize == 4)
            return diag ? go(float{}, std::true_type{}) : go(float{}, std::false_type{});
        return diag ? go(_Float16{}, std::true_type{}) : go(_Float16{}, std::false_type{});
    }
    if (a.geom.stream_parts > 0) {
        auto go = [&](auto tag) {
            using T = decltype(tag);
            // rows of up to 4 KiB in one step of four vectors per lane, up to
            // 5 KiB in one step of five (4112-byte fp32 rows: 0.791 -> 0.608 ms
            // against two segments of the streaming kernel), wider rows streamed
            // (rows not all on 16-byte boundaries: the odd forms, over up to
            // one vector more)
            constexpr int VEC = 16 / (int)sizeof(T);
            const bool odd = !a.aligned16;
            const int nvec = odd ? (a.V + 2 * VEC - 2) / VEC : a.V / VEC;
            // fp32: a row's last segment of at most one block merges into the
            // one before (8196-byte rows: 1.218 -> 1.176 ms; on fp16 rows the
            // same measured 20-40% slower)
            const int nlo = (a.V + VEC - 1) / VEC;  // the fewest vectors covering a row
            auto tiny_tail = [](int nv) { return nv > 512 && (nv - 1) % 256 < 64; };
            const bool merge = sizeof(T) == 4 && (tiny_tail(nvec) || (odd && tiny_tail(nlo)));
            auto kern = odd ? (nvec <= 256   ? k_rowstats_multi<T, 8, 2, 4, true, Src>
                               : nvec <= 320 ? k_rowstats_multi<T, 8, 2, 5, true, Src>
                               : merge       ? k_rowstats_stream<T, 16, true, true, Src>
                                             : k_rowstats_stream<T, 16, true, false, Src>)
                            : (nvec <= 256   ? k_rowstats_multi<T, 8, 2, 4, false, Src>
                               : nvec <= 320 ? k_rowstats_multi<T, 8, 2, 5, false, Src>
                               : merge       ? k_rowstats_stream<T, 16, false, true, Src>
                                             : k_rowstats_stream<T, 16, false, false, Src>);
            const dim3 wblock(nvec <= 320 ? 512 : 1024);
            hipLaunchKernelGGL(kern, grid, wblock, 0, stream, static_cast<const T *>(a.logits), a.V, a.blank, src,
                               a.targets, a.S, WS(float4 *, node), WS(float2 *, prob));
            return hipGetLastError();
        };
        return a.esize == 4 ? go(float{}) : go(_Float16{});
    }
    return with_narrow(a.esize, a.geom.vec, a.geom.lanes_per_row, [&](auto tag) {
        using Tg = decltype(tag);
        using T = typename Tg::type;
        hipLaunchKernelGGL((k_rowstats_narrow<T, Tg::vec, Tg::n, Src>), grid, block, 0, stream,
                           static_cast<const T *>(a.logits), a.V, a.blank, src, a.targets, a.S, WS(float4 *, node),
                           WS(float2 *, prob));
        return hipGetLastError();
    });
}

hipError_t launch_rowstats(const LaunchArgs &a, const PlanArgs *pa, hipStream_t stream) {
    if (a.small) {
        ArgSrc src;
        src.pa = *pa;
        src.rpc = a.lay.rows_per_chunk;
        src.ws_chunks = WS(ChunkDesc *, chunks);
        src.ws_desc = WS(SampleDesc *, desc);
        src.ws_order = WS(int32_t *, order);
        src.cflags = WS(uint32_t *, cflags);
        return launch_rowstats_with(a, src, stream);
    }
    const TableSrc src{WS(const SampleDesc *, desc), WS(const ChunkDesc *, chunks), WS(int *, mode),
                       WS(uint32_t *, status)};
    return launch_rowstats_with(a, src, stream);
}

// The recursions, the forward-backward check of the probability-domain
// samples, and the log-domain rerun of the samples the check marked (a
// launch whose workgroups exit at once when none is).
hipError_t launch_alpha_beta(const LaunchArgs &a, hipStream_t stream) {
    if (a.small) {
        hipLaunchKernelGGL(k_ab_small, dim3(a.B), dim3(128), 0, stream, WS(const SampleDesc *, desc),
                           WS(const int32_t *, order), a.B, a.lay.rows_per_chunk, WS(const uint32_t *, cflags),
                           WS(uint32_t *, sflags), WS(int *, mode), WS(const float4 *, node), WS(const float2 *, prob), WS(double *, alpha),
                           WS(double *, beta), WS(int *, ealpha), WS(int *, ebeta), WS(double *, log2z), a.loss);
        return hipGetLastError();
    }
    for (int rerun = 0; rerun < 2; ++rerun) {
        if (rerun) {
            hipLaunchKernelGGL(k_check_ab, dim3(kCheckDiagonals * a.B), dim3(64), 0, stream, WS(const SampleDesc *, desc),
                               WS(int *, mode), WS(const double *, alpha), WS(const double *, beta),
                               WS(const int *, ealpha), WS(const int *, ebeta), WS(const double *, log2z));
        }
        hipLaunchKernelGGL(k_alpha_beta, dim3(2 * a.B), dim3(64), 0, stream, WS(const SampleDesc *, desc),
                           WS(const int32_t *, order), a.B, WS(const int *, mode), WS(const float4 *, node),
                           WS(const float2 *, prob), WS(double *, alpha), WS(double *, beta), WS(int *, ealpha),
                           WS(int *, ebeta), WS(double *, log2z), a.loss, rerun);
        if (a.max_U1 > kMaxTileU1) {  // lattices of 1280 .. 2048 padded columns: 5 .. 8 waves each
            auto wide = [&](auto kern, int nw) {
                hipLaunchKernelGGL(kern, dim3(2 * a.B), dim3(64 * nw), 0, stream, WS(const SampleDesc *, desc),
                                   WS(const int32_t *, order), a.B, WS(const int *, mode), WS(const float4 *, node),
                                   WS(const float2 *, prob), WS(double *, alpha), WS(double *, beta),
                                   WS(int *, ealpha), WS(int *, ebeta), WS(double *, log2z), a.loss, rerun);
            };
            wide(k_ab_wide<5>, 5);
            wide(k_ab_wide<6>, 6);
            wide(k_ab_wide<7>, 7);
            wide(k_ab_wide<8>, 8);
        }
    }
    return hipGetLastError();
}

// The parts of a row's gradient, `span` the most 16-byte vectors a row's
// waves take: parts of four blocks of 64 vectors (4 KiB), except one part of
// five for a row of 4 to 5 KiB (4112-byte fp32 rows: 1.640 -> 1.335 ms against
// a whole part and one of a single vector; fp16 1.886 -> 1.358) and, for fp32
// rows, a last part of five where the row would end in a part of at most one
// block (8196-byte rows: two waves instead of three, 2.590 -> 2.278 ms; fp16
// rows gain nothing from it).  Parts of five throughout measured 9-10% slower
// on 8208- and 8704-byte rows.
struct PartShape {
    int split, pb, pb_last;
    bool five;  // the kernels with room for five blocks
};
static PartShape part_shape(int span, int esize) {
    const int p4 = (span + 255) / 256;
    if (span > 256 && span <= 320) return {1, 5, 5, true};
    if (esize == 4 && p4 >= 3 && span - (p4 - 1) * 256 <= 64) return {p4 - 1, 4, 5, true};
    return {p4, 4, 4, false};
}

// The gradient, and in its first workgroup the loss check and reduction.
hipError_t launch_grad(const LaunchArgs &a, hipStream_t stream) {
    const dim3 grid(a.lay.n_chunks), block(256);
    GradArgs g;
    g.red.loss = a.loss;
    g.red.out = (a.reduction != RNNT_REDUCTION_NONE) ? a.loss_reduced : nullptr;
    g.red.status = WS(uint32_t *, status);
    g.red.status_out = a.status_out;
    g.red.sflags = a.small ? WS(const uint32_t *, sflags) : nullptr;
    g.red.B = a.B;
    g.red.mean = a.reduction == RNNT_REDUCTION_MEAN;
    g.red.on = 1;
    g.V = a.V;
    g.blank = a.blank;
    g.n_chunks = a.lay.n_chunks;
    g.S = a.S;
    g.targets = a.targets;
    g.clamp = a.clamp;
    g.scale = a.grad_scale;
    g.log2_scale = log2f(a.grad_scale);
    g.fastemit = a.fastemit;
    g.scale_y = a.grad_scale * (1.0f + a.fastemit);
    g.desc = WS(const SampleDesc *, desc);
    g.chunks = WS(const ChunkDesc *, chunks);
    g.mode = WS(const int *, mode);
    g.log2z = WS(const double *, log2z);
    g.node = WS(const float4 *, node);
    g.alpha = WS(const double *, alpha);
    g.beta = WS(const double *, beta);
    g.ealpha = WS(const int *, ealpha);
    g.ebeta = WS(const int *, ebeta);
    // Rows of more than 1 KiB: one single-wave workgroup per part of 4 or 5 KiB
    // of a row.  Rows not all on 16-byte boundaries take k_grad_rows_odd, if
    // the logits (when read) sit at the same offset from such a boundary as
    // the gradient; else the narrow kernels.
    const bool same16 = ((reinterpret_cast<uintptr_t>(a.logits) ^ reinterpret_cast<uintptr_t>(a.grad)) & 15u) == 0;
    if (a.geom.stream_parts > 0 && !a.aligned16 && (!a.fused || same16)) {
        auto rows = [&](auto ttag) -> hipError_t {
            using T = decltype(ttag);
            const T *in = static_cast<const T *>(a.logits);
            T *out = static_cast<T *>(a.grad);
            const bool cl = a.clamp > 0.f;
            void (*kern)(const T *, T *, int, int64_t, int, int, int, int, int, int, int, float, float, float,
                         float, float, const int32_t *, const SampleDesc *, const ChunkDesc *, const int *,
                         const double *, const float4 *, const double *, const double *, const int *, const int *,
                         ReduceArgs);
            // most vectors a row's waves take: the line before the row's
            // start, the row, and the vector holding its end
            const int64_t row_bytes = (int64_t)a.V * a.esize;
            const PartShape ps = part_shape((int)((row_bytes + 127 + 15) / 16 + 1), a.esize);
            const int split = ps.split;
            if (ps.five)
                kern = a.fused ? (cl ? k_grad_rows_odd<T, true, true, 5> : k_grad_rows_odd<T, true, false, 5>)
                               : (cl ? k_grad_rows_odd<T, false, true, 5> : k_grad_rows_odd<T, false, false, 5>);
            else
                kern = a.fused ? (cl ? k_grad_rows_odd<T, true, true, 4> : k_grad_rows_odd<T, true, false, 4>)
                               : (cl ? k_grad_rows_odd<T, false, true, 4> : k_grad_rows_odd<T, false, false, 4>);
            const int bpc = a.lay.rows_per_chunk * split;
            const int64_t total = (int64_t)a.lay.n_chunks * bpc;
            constexpr int64_t kMaxBlocks = (int64_t)1 << 24;
            for (int64_t base = 0; base < total; base += kMaxBlocks) {
                const unsigned nb = (unsigned)std::min<int64_t>(kMaxBlocks, total - base);
                hipLaunchKernelGGL(kern, dim3(nb), dim3(64), 0, stream, in, out, bpc, base, split, ps.pb, ps.pb_last,
                                   RNNT_GRAD_ARGS(g));
                g.red.on = 0;  // the first launch's first workgroup reduces
            }
            return hipGetLastError();
        };
        return a.esize == 4 ? rows(float{}) : rows(_Float16{});
    }
    if (a.geom.stream_parts > 0 && a.aligned16) {
        auto rows = [&](auto ttag) -> hipError_t {
            using T = decltype(ttag);
            const T *in = static_cast<const T *>(a.logits);
            T *out = static_cast<T *>(a.grad);
            const bool cl = a.clamp > 0.f;
            void (*kern)(const T *, T *, int, int64_t, int, int, int, int, int, int, int, float, float, float,
                         float, float, const int32_t *, const SampleDesc *, const ChunkDesc *, const int *,
                         const double *, const float4 *, const double *, const double *, const int *, const int *,
                         ReduceArgs);
            const uint32_t row_bytes = (uint32_t)a.V * (uint32_t)a.esize;
            const int nvec = (int)(row_bytes / 16);
            const bool full = row_bytes % 4096 == 0;  // every part a whole 4 KiB
            // rows that can start inside a 128-byte line: k_grad_rows_line
            const uint32_t g0 = (uint32_t)(reinterpret_cast<uintptr_t>(a.grad) & 127u);
            const bool line = row_bytes % 128 != 0 || g0 != 0;
            // Row starts fall at g0 + k * row_bytes (mod 128), i.e. on the
            // multiples of q = gcd(row_bytes, 128) offset by g0 mod q; a row
            // of k_grad_rows_line takes up to (its start's offset) / 16
            // vectors of the previous row
            uint32_t q = 128;
            while (row_bytes % q != 0) q >>= 1;
            const int span = nvec + (line ? (int)((g0 % q + 128 - q) >> 4) : 0);  // most vectors of a row's waves
            const PartShape ps = part_shape(span, a.esize);
            const bool five = ps.five;
            const int split = ps.split;
            if (line && five)
                kern = a.fused ? (cl ? k_grad_rows_line<T, true, true, 5> : k_grad_rows_line<T, true, false, 5>)
                               : (cl ? k_grad_rows_line<T, false, true, 5> : k_grad_rows_line<T, false, false, 5>);
            else if (line)
                kern = a.fused ? (cl ? k_grad_rows_line<T, true, true, 4> : k_grad_rows_line<T, true, false, 4>)
                               : (cl ? k_grad_rows_line<T, false, true, 4> : k_grad_rows_line<T, false, false, 4>);
            else if (a.fused && five)
                kern = cl ? k_grad_rows<T, true, true, 0, false, 5> : k_grad_rows<T, true, false, 0, false, 5>;
            else if (a.fused)
                kern = cl ? k_grad_rows<T, true, true, 0, false, 4> : k_grad_rows<T, true, false, 0, false, 4>;
            else if (full && a.geom.stream_parts == 1)
                kern = cl ? k_grad_rows<T, false, true, 1, true, 4> : k_grad_rows<T, false, false, 1, true, 4>;
            else if (full)
                kern = cl ? k_grad_rows<T, false, true, 0, true, 4> : k_grad_rows<T, false, false, 0, true, 4>;
            else if (five)
                kern = cl ? k_grad_rows<T, false, true, 0, false, 5> : k_grad_rows<T, false, false, 0, false, 5>;
            else
                kern = cl ? k_grad_rows<T, false, true, 0, false, 4> : k_grad_rows<T, false, false, 0, false, 4>;
            // one launch per 2^24 workgroups, so no launch exceeds 32-bit work-item counts
            const int bpc = a.lay.rows_per_chunk * split;
            const int64_t total = (int64_t)a.lay.n_chunks * bpc;
            constexpr int64_t kMaxBlocks = (int64_t)1 << 24;
            for (int64_t base = 0; base < total; base += kMaxBlocks) {
                const unsigned nb = (unsigned)std::min<int64_t>(kMaxBlocks, total - base);
                hipLaunchKernelGGL(kern, dim3(nb), dim3(64), 0, stream, in, out, bpc, base, split, ps.pb, ps.pb_last,
                                   RNNT_GRAD_ARGS(g));
                g.red.on = 0;  // the first launch's first workgroup reduces
            }
            return hipGetLastError();
        };
        return a.esize == 4 ? rows(float{}) : rows(_Float16{});
    }
    return with_narrow(a.esize, a.geom.vec, a.geom.lanes_per_row, [&](auto tag) {
        using Tg = decltype(tag);
        using T = typename Tg::type;
        if (a.fused)
            hipLaunchKernelGGL((k_grad_narrow<T, Tg::vec, Tg::n, true>), grid, block, 0, stream,
                               static_cast<const T *>(a.logits), static_cast<T *>(a.grad), RNNT_GRAD_ARGS(g));
        else
            hipLaunchKernelGGL((k_grad_narrow<T, Tg::vec, Tg::n, false>), grid, block, 0, stream,
                               static_cast<const T *>(a.logits), static_cast<T *>(a.grad), RNNT_GRAD_ARGS(g));
        return hipGetLastError();
    });
}

hipError_t launch_reduce(const LaunchArgs &a, hipStream_t stream) {
    float *out = (a.reduction != RNNT_REDUCTION_NONE) ? a.loss_reduced : nullptr;
    hipLaunchKernelGGL(k_reduce, dim3(1), dim3(64), 0, stream, a.loss, WS(const double *, log2z), a.B,
                       a.reduction == RNNT_REDUCTION_MEAN, out, WS(uint32_t *, status), a.status_out,
                       a.small ? WS(const uint32_t *, sflags) : nullptr);
    return hipGetLastError();
}

hipError_t launch_grad_scale(void *grad, int esize, int V, int64_t N, int B, const float *scale, int per_sample,
                             const uint8_t *ws, const WorkspaceLayout &lay, const RowGeom &geom,
                             hipStream_t stream) {
    const int64_t rows_per_block = 4 * (64 / geom.lanes_per_row);
    const dim3 grid((unsigned)((N + rows_per_block - 1) / rows_per_block)), block(256);
    const SampleDesc *desc = reinterpret_cast<const SampleDesc *>(ws + lay.desc);
    return with_narrow(esize, geom.vec, geom.lanes_per_row, [&](auto tag) {
        using Tg = decltype(tag);
        using T = typename Tg::type;
        hipLaunchKernelGGL((k_grad_scale<T, Tg::vec, Tg::n>), grid, block, 0, stream, static_cast<T *>(grad), V, N,
                           B, desc, scale, per_sample);
        return hipGetLastError();
    });
}

hipError_t launch_zero_padding(void *grad, int esize, int V, int B, int max_T, int max_U1, const uint8_t *ws,
                               const WorkspaceLayout &lay, const RowGeom &geom, hipStream_t stream) {
    const SampleDesc *desc = reinterpret_cast<const SampleDesc *>(ws + lay.desc);
    const int64_t rows = (int64_t)B * max_T * max_U1;
    const int64_t per_block = 4 * (64 / geom.lanes_per_row);
    const unsigned grid = (unsigned)std::min<int64_t>((rows + per_block - 1) / per_block, 1 << 16);
    return with_narrow(esize, geom.vec, geom.lanes_per_row, [&](auto tag) {
        using Tg = decltype(tag);
        using T = typename Tg::type;
        hipLaunchKernelGGL((k_zero_padding<T, Tg::vec, Tg::n>), dim3(grid), dim3(256), 0, stream,
                           static_cast<T *>(grad), V, B, max_T, max_U1, desc);
        return hipGetLastError();
    });
}

#undef WS

// ====================================================== multi-blank transducer
// The ESPnet compute_multiblank_grad_kernel page: activations over the labels,
// the standard blank and num_big_blanks big blanks, each big blank with a
// duration, and sigma, the logit under-normalisation hyper-parameter.  From
// node (t,u) the standard blank moves to (t+1,u), big blank i to (t+d_i,u)
// and the next label to (t,u+1); every edge's log-probability is lowered by
// sigma; an alignment ends when a blank of any kind reaches t = T exactly at
// u = U.  The sweeps treat that end as a virtual node (T,U) on anti-diagonal
// T+U, with beta(T,U) = 1, so the ends need no special case.
//
// Three passes of their own: per row, the log-normaliser (the row maximum and
// log2 of the sum of exp(x - max), kept apart as in the plain path) and the
// edges' probabilities (fp64 planes in the skewed slots); one wave per sample
// and direction sweeping anti-diagonals in fp64 probabilities renormalised by
// a power of two on every diagonal, with the recent diagonals in an LDS
// ring (a power of two deep, above the longest duration) for the big
// blanks' jumps; and per row, the gradient.  The loss check and reduction are k_reduce's.
namespace {

struct MbParams {
    int nb;
    int ids[kMaxBigBlanks];
    int dur[kMaxBigBlanks];
    int R;        // ring depth: the power of two above the longest duration
    float sigma;
};

// A label must be a class that is neither the standard blank nor a big
// blank; any other value admits no alignment (its edge is impossible).
__device__ __forceinline__ bool mb_label_ok(int y, int V, int blank, const MbParams &mp) {
    bool ok = y >= 0 && y < V && y != blank;
#pragma unroll
    for (int i = 0; i < kMaxBigBlanks; ++i) ok = ok && !(i < mp.nb && y == mp.ids[i]);
    return ok;
}

__device__ __forceinline__ const SampleDesc &mb_sample_of_row(const SampleDesc *__restrict__ desc, int B,
                                                              int64_t r) {
    int lo = 0, hi = B - 1;  // last sample whose first row is <= r (every sample has a row)
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (desc[mid].row_off <= r) lo = mid;
        else hi = mid - 1;
    }
    return desc[lo];
}

// exp(lp) in fp64 for an fp32 log-prob, the exponent split off exactly, so
// a weight far below fp32's range keeps its value.
__device__ __forceinline__ double prob_d(float lp) {
    constexpr float kHi = 1.44269502162933349609375f;
    constexpr float kLo = 1.925963033500011079e-8f;
    const float k = rintf(lp * kLog2e);
    const float f = fmaf(lp, kHi, -k) + lp * kLo;
    const double p = __builtin_amdgcn_ldexp((double)exp2_fast(f), (int)k);
    return (lp < -1100.f) ? 0.0 : p;
}

// Workgroups are dispatched to the 8 XCDs in turn (workgroup b to XCD b % 8),
// each XCD with its own L2.  Logical block of workgroup b when the grid
// (a multiple of 8 workgroups, `per` for each XCD) gives XCD x the
// contiguous blocks [x * per, (x + 1) * per): the per-node records a row
// pass writes near its rows then fill their lines in one L2, not eight.
__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t per) {
    return (b & 7) * per + (b >> 3);
}


// The 2 + nb weights of node (t,u): lane k < 2 + nb stores plane k's, `v`
// its log-probability (less sigma).  Edges that leave the lattice are stored
// as probability zero — the blank out of the last frame below column U, a
// big blank that passes T or reaches it below column U (the label at
// column U arrives as -inf) — and the slots outside the lattice are zeroed,
// one contiguous run per anti-diagonal: node (0,u) zeroes columns u+1..U of
// diagonal u (t < 0), node (T-1,u) columns 0..u of diagonal T+u (t >= T).
// So the sweep reads no slot it must mask.
__device__ __forceinline__ void mb_store_node(const SampleDesc &d, int t, int u, const MbParams &mp, int lane,
                                              float v, double *__restrict__ wp, int64_t n_slots) {
    const int U1 = d.U + 1;
    const int np = 2 + mp.nb;
    if (lane < np) {
        bool gone = (lane == 0) && (t == d.T - 1) && (u < d.U);
#pragma unroll
        for (int i = 0; i < kMaxBigBlanks; ++i) {
            const int te = t + mp.dur[i];
            if (lane == 2 + i) gone = te > d.T || (te == d.T && u < d.U);
        }
        wp[(int64_t)lane * n_slots + d.slot_off + (int64_t)(t + u) * U1 + u] = gone ? 0.0 : prob_d(v);
    }
    if (t == 0 && u < d.U) {
        const int len = d.U - u;  // columns u+1 .. U of anti-diagonal u
        for (int q = lane; q < len * np; q += 64)
            wp[(int64_t)(q / len) * n_slots + d.slot_off + (int64_t)u * U1 + u + 1 + q % len] = 0.0;
    }
    if (t == d.T - 1 && u < d.U) {
        const int len = u + 1;  // columns 0 .. u of anti-diagonal T+u
        for (int q = lane; q < len * np; q += 64)
            wp[(int64_t)(q / len) * n_slots + d.slot_off + (int64_t)(d.T + u) * U1 + q % len] = 0.0;
    }
}

// One wave per packed row, four per workgroup: the row's log-normaliser
// (fused: {maximum, log2 sum of exp(x - maximum)}; {0, 0} for log-prob inputs
// and rows of -inf) and the probabilities, in fp64, of the edges leaving the node
// (their log-probabilities less sigma, exponentiated), at its skewed slot:
// plane 0 the standard blank, plane 1 the next label (0 at u = U or for a
// label outside [0,V)), plane 2+i big blank i.
template <typename T>
__global__ __launch_bounds__(256) void k_mb_rows(const T *__restrict__ logits, int64_t N, int V, int blank,
                                                 int fused, MbParams mp, const SampleDesc *__restrict__ desc,
                                                 int B, const int32_t *__restrict__ targets, int S,
                                                 float2 *__restrict__ den, double *__restrict__ wp,
                                                 int64_t n_slots, uint32_t *status, int64_t row_base) {
    const int lane = threadIdx.x & 63;
    const int64_t r = row_base + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= N) return;
    const SampleDesc d = mb_sample_of_row(desc, B, r);
    const int64_t lr = r - d.row_off;
    const int t = (int)(lr / d.tstride);
    const int u = (int)(lr - (int64_t)t * d.tstride);
    if (t >= d.T || u > d.U) return;  // a padding row of the padded layout
    const T *x = logits + r * (int64_t)V;
    float mr = 0.f, ls2 = 0.f;
    bool dead = false;
    if (fused) {
        float m = kNegInf;
        for (int k = lane; k < V; k += 64) m = fmaxf(m, Elem<T>::load1(x + k));
        m = wave_max_f(m);
        dead = (m == kNegInf);
        float sum = 0.f;
        if (!dead)
            for (int k = lane; k < V; k += 64) sum += exp2_fast((Elem<T>::load1(x + k) - m) * kLog2e);
        sum = wave_sum_f(sum);
        mr = dead ? 0.f : m;
        ls2 = dead ? 0.f : log2_fast(sum);
    }
    if (lane == 0) den[r] = make_float2(mr, ls2);
    float v = kNegInf;
    if (lane < 2 + mp.nb) {
        int k = blank;
        if (lane == 1) {
            k = -1;
            if (u < d.U) {
                const int y = targets[(int64_t)d.index * S + u];
                const bool bad = !mb_label_ok(y, V, blank, mp);
                if (bad) atomicOr(status, (uint32_t)RNNT_DEV_BAD_TARGET);
                k = bad ? -1 : y;
            }
        }
#pragma unroll
        for (int i = 0; i < kMaxBigBlanks; ++i)
            if (lane == 2 + i) k = mp.ids[i];
        v = (k >= 0 && !dead) ? (Elem<T>::load1(x + k) - mr) - ls2 * kLn2 - mp.sigma : kNegInf;
    }
    mb_store_node(d, t, u, mp, lane, v, wp, n_slots);
}

// One wave per (sample, direction): blockIdx 2i runs alpha of sample i,
// 2i+1 beta.  Lane l holds the two adjacent columns 128g + 2l and
// 128g + 2l + 1 of each group g < G, so every edge's weights for its two
// columns arrive in one 16-byte load and its two values leave in one 16-byte
// store; only one neighbour per group and step crosses lanes (a DPP move).
// `cur` is the diagonal just finished, scaled by 2^-E; the LDS ring keeps the
// last R diagonals for the NB big blanks, whose sources lie d_i diagonals
// away, and the lanes of one register their exponents.  The edges'
// probabilities do not depend on the recursion, so those of the next P
// diagonals are in flight while a diagonal is computed (a register ring, one
// slot per step mod P).  No edge is masked: the row pass stores zero weights
// for edges that leave the lattice and for slots outside it, the range check
// zeroes columns past U, and a big blank whose source diagonal does not
// exist reads a ring slot still holding zeros, so nodes outside the lattice
// stay zero by themselves.  One wave issues one instruction at a time here,
// so the step is written for few instructions: no per-lane masks, scalar
// diagonal offsets, exponents moved by lane index.  Stored: every real diagonal of alpha or beta (scaled) and its
// exponent; log2 P(y|x) and, from beta, the loss.
template <int G, int NB> struct MbSweepShape {
    static constexpr int NW = 2 + NB;  // blank, label, big blanks
    // steps in flight: their loads and stores stay within the wait counter's
    // 63, and the ring within 128 registers (160 measured slower)
    static constexpr int P_ops = 56 / (NW * G + G + 1);
    static constexpr int P_regs = 128 / (4 * NW * G);
    static constexpr int P0 = P_ops < P_regs ? P_ops : P_regs;
    static constexpr int P = P0 < 1 ? 1 : (P0 > 8 ? 8 : P0);
};

struct D2 {
    double a, b;  // columns 2l and 2l+1 of a group
};

__device__ __forceinline__ D2 as_d2(u32x4 v) {
    return {__hiloint2double((int)v[1], (int)v[0]), __hiloint2double((int)v[3], (int)v[2])};
}

template <int G, int NB, bool bw, bool LOG>
__device__ __forceinline__ void mb_sweep_dir(const SampleDesc &d, int B, const MbParams &mp,
                                             const double *__restrict__ wp, int64_t n_slots,
                                             double *__restrict__ alpha, double *__restrict__ beta,
                                             int *__restrict__ ealpha, int *__restrict__ ebeta,
                                             double *__restrict__ log2z, float *__restrict__ loss) {
    extern __shared__ double mb_ring[];  // R diagonals of G groups of 64 lanes x 2 values
    constexpr int U1p = 128 * G;
    constexpr int NW = MbSweepShape<G, NB>::NW;
    constexpr int P = MbSweepShape<G, NB>::P;
    const int lane = threadIdx.x;
    const int T = d.T, U = d.U, U1 = U + 1, nd = T + U, R = mp.R, M = R - 1;
    for (int q = lane; q < R * U1p; q += 64) mb_ring[q] = LOG ? kNegInfD : 0.0;
    // ring entry of (diagonal slot s, group g): this lane's pair at 16-byte stride
    auto ring_at = [&](int sslot, int g) -> D2 * {
        return reinterpret_cast<D2 *>(mb_ring + (size_t)(sslot * G + g) * 128) + lane;
    };
    // Lane s holds the exponent of the diagonal in ring slot s (R <= 32 lanes
    // used): written by a select on the lane index and read with readlane,
    // without LDS or lane masks.
    int eh = 0;
    uint32_t vo[G];  // byte offset of the lane's first column in a diagonal
#pragma unroll
    for (int g = 0; g < G; ++g) vo[g] = (uint32_t)(128 * g + 2 * lane) * 8u;
    double *tab = (bw ? beta : alpha) + d.ab_off;
    int *etab = (bw ? ebeta : ealpha) + d.diag_off + d.index;
    // Stores through resources over diagonals 0 .. T+U-1 of the table (the
    // diagonal offset is scalar): the forward sweep's last diagonal, the
    // virtual end's, falls outside and its store is dropped.  A table spans
    // less than 2^31 bytes (checked on the host).
    const Rsrc rtab = buffer_at(tab, (uint32_t)nd * (uint32_t)U1p * 8u);
    const Rsrc retab = buffer_at(etab, (uint32_t)nd * 4u);

    // One buffer resource per plane over the sample's slots, the diagonal
    // chosen by the scalar offset.  The range check covers the scalar offset
    // too, so a record count of (that offset + U1 slots) checks the lane's
    // columns against U: the columns past U read zero without a test.  All
    // planes at one diagonal share the offset and the count; offsets are
    // 32-bit (a sample's span is below 2^31 bytes) and kept scalar with
    // readfirstlane where the compiler would form them with vector
    // instructions.
    const char *pb[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) pb[k] = reinterpret_cast<const char *>(wp + (int64_t)k * n_slots + d.slot_off);
    const uint32_t dbytes = (uint32_t)U1 * 8u;
    auto ld = [&](int k, int diag, uint32_t voff) -> D2 {
        const uint32_t off = (uint32_t)__builtin_amdgcn_readfirstlane(diag) * dbytes;
        return as_d2(__builtin_amdgcn_raw_buffer_load_b128(buffer_at(pb[k], off + dbytes), voff, off, 0));
    };
    // The probabilities step `step` uses, for the lane's two columns (steps
    // past the end load the last step's again; never used).  Forward,
    // diagonal n pulls from n-1 (blank at column u; the label from u-1, moved
    // over by one column below) and n-d_i; backward, every edge leaves the
    // node itself.  A big blank's source diagonal before 0 reads diagonal 0;
    // its source value is zero (below).
    auto load_w = [&](int step, D2 (&w)[G][NW]) {
        const int n = bw ? nd - min(step, nd) : min(step, nd);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (!bw) {
                w[g][0] = ld(0, n - 1, vo[g]);
                w[g][1] = ld(1, n - 1, vo[g]);
#pragma unroll
                for (int i = 0; i < NB; ++i) w[g][2 + i] = ld(2 + i, max(n - mp.dur[i], 0), vo[g]);
            } else {
#pragma unroll
                for (int k = 0; k < NW; ++k) w[g][k] = ld(k, n, vo[g]);
            }
        }
    };

    // start: alpha(0,0) = 1 on diagonal 0; beta of the virtual end (T,U) = 1 on diagonal T+U
    D2 cur[G];
    int E = 0;
    // Diagonal n lives in ring slot n mod R (R a power of two).  A big
    // blank's source diagonal outside [0, T+U] maps to a slot no diagonal has
    // been written to yet (1 <= d_i < R), which still holds the zeros it
    // started with.
    int slot = (bw ? nd : 0) & M;
    {
        const int ue = bw ? U : 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int c0 = 128 * g + 2 * lane;
            const double one = LOG ? 0.0 : 1.0, zero = LOG ? kNegInfD : 0.0;
            cur[g] = {c0 == ue ? one : zero, c0 + 1 == ue ? one : zero};
            *ring_at(slot, g) = cur[g];
        }
        if (!bw) {
#pragma unroll
            for (int g = 0; g < G; ++g) reinterpret_cast<D2 *>(tab + 128 * g)[lane] = cur[g];
            etab[0] = 0;
        }
    }

    auto step_once = [&](int step, const D2 (&w)[G][NW]) {
        const int n = bw ? nd - step : step;
        slot = n & M;
        // big blanks: the source's ring slot and its exponent relative to E
        int sl[NB > 0 ? NB : 1], shg[NB > 0 ? NB : 1];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            sl[i] = (bw ? n + mp.dur[i] : n - mp.dur[i]) & M;
            shg[i] = LOG ? 0 : __builtin_amdgcn_readlane(eh, sl[i]) - E;
        }
        // Cross-lane neighbours.  Forward: column 2l-1 of the finished
        // diagonal and the label weight of column 2l-1 come from lane l-1's
        // second value (lane 0 of group g: lane 63 of group g-1, or zero).
        // Backward: column 2l+2 of the finished diagonal from lane l+1's
        // first value (lane 63 of group g: lane 0 of group g+1, or zero).
        double side_v[G], side_w[G];
        if constexpr (G == 1 && !LOG) {
            side_v[0] = bw ? shift_down_zero(cur[0].a) : shift_up_zero(cur[0].b);
            side_w[0] = bw ? 0.0 : shift_up_zero(w[0][1].b);
        } else {
            const double zv = LOG ? kNegInfD : 0.0;  // an edge lane's missing neighbour
            double nb_v[G], nb_w[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                nb_v[g] = bw ? rotate_down(cur[g].a) : rotate_up(cur[g].b);
                nb_w[g] = bw ? 0.0 : rotate_up(w[g][1].b);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (bw) {
                    side_v[g] = (lane == 63) ? (g + 1 < G ? nb_v[g + 1] : zv) : nb_v[g];
                    side_w[g] = 0.0;
                } else {
                    side_v[g] = (lane == 0) ? (g > 0 ? nb_v[g - 1] : zv) : nb_v[g];
                    side_w[g] = (lane == 0) ? (g > 0 ? nb_w[g - 1] : 0.0) : nb_w[g];
                }
            }
        }
        D2 nx[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            D2 src[NB > 0 ? NB : 1];
#pragma unroll
            for (int i = 0; i < NB; ++i) src[i] = *ring_at(sl[i], g);
            // No masks: every weight of an edge that does not exist is zero
            // (outside-lattice slots and lattice-leaving edges stored as zero
            // by the row pass, columns past U zeroed by the range check), so
            // nodes outside the lattice come out zero by themselves.
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const double wb = h ? w[g][0].b : w[g][0].a;
                const double cv = h ? cur[g].b : cur[g].a;
                // label: forward, weight of column u-1 and value of column u-1; backward, own weight and u+1
                const double wy = bw ? (h ? w[g][1].b : w[g][1].a) : (h ? w[g][1].a : side_w[g]);
                const double sv = bw ? (h ? side_v[g] : cur[g].b) : (h ? cur[g].a : side_v[g]);
                double acc;
                if constexpr (LOG) {
                    // log2 values: the weights' logs, then a log-sum-exp of the 2 + NB terms
                    double tm[2 + NB];
                    tm[0] = log2_d(wb) + cv;
                    tm[1] = log2_d(wy) + sv;
#pragma unroll
                    for (int i = 0; i < NB; ++i)
                        tm[2 + i] = log2_d(h ? w[g][2 + i].b : w[g][2 + i].a) + (h ? src[i].b : src[i].a);
                    double m = tm[0];
#pragma unroll
                    for (int k = 1; k < 2 + NB; ++k) m = fmax(m, tm[k]);
                    float sum = 0.f;
#pragma unroll
                    for (int k = 0; k < 2 + NB; ++k) sum += exp2_fast((float)(tm[k] - m));
                    acc = (m == kNegInfD) ? kNegInfD : m + (double)log2_fast(sum);
                } else {
                    acc = fma(wy, sv, wb * cv);
#pragma unroll
                    for (int i = 0; i < NB; ++i) {
                        // forward from (t-d_i,u); backward to (t+d_i,u)
                        const double wg = h ? w[g][2 + i].b : w[g][2 + i].a;
                        const double sr = h ? src[i].b : src[i].a;
                        acc = fma(wg, __builtin_amdgcn_ldexp(sr, shg[i]), acc);
                    }
                }
                if (h) nx[g].b = acc;
                else nx[g].a = acc;
            }
        }
        // renormalise by a power of two (a diagonal of zeros keeps its exponent)
        int sh = 0;
        if constexpr (!LOG) {
            int eb = 0;
#pragma unroll
            for (int g = 0; g < G; ++g)
                eb = max(eb, max((__double2hiint(nx[g].a) >> 20) & 0x7ff, (__double2hiint(nx[g].b) >> 20) & 0x7ff));
            eb = wave_max_nonneg(eb);
            sh = eb == 0 ? 0 : eb - 1023;
            E += sh;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            cur[g] = {__builtin_amdgcn_ldexp(nx[g].a, -sh), __builtin_amdgcn_ldexp(nx[g].b, -sh)};
            *ring_at(slot, g) = cur[g];
        }
        eh = (lane == slot) ? E : eh;
        const uint32_t so = (uint32_t)n * (uint32_t)U1p * 8u;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const u32x4 v = {(uint32_t)__double2loint(cur[g].a), (uint32_t)__double2hiint(cur[g].a),
                             (uint32_t)__double2loint(cur[g].b), (uint32_t)__double2hiint(cur[g].b)};
            __builtin_amdgcn_raw_buffer_store_b128(v, rtab, vo[g], so, 0);
        }
        // every lane stores the same value: no lane mask
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)E, retab, 0, (uint32_t)n * 4u, 0);
    };

    D2 w[P][G][NW];
#pragma unroll
    for (int q = 0; q < P; ++q) load_w(1 + q, w[q]);
    for (int s0 = 1; s0 <= nd; s0 += P) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            if (s0 + q <= nd) {
                step_once(s0 + q, w[q]);
                load_w(s0 + q + P, w[q]);
            }
        }
    }

    // log2 P(y|x): alpha of the virtual end (T,U), or beta(0,0), read back
    // from the ring slot the last diagonal went to (a register array indexed
    // by the column's group would be kept in scratch)
    const int ue = bw ? 0 : U;
    const D2 mine = *ring_at(slot, ue >> 7);
    const double v = readlane_d((ue & 1) ? mine.b : mine.a, (ue & 127) >> 1);
    const double l2 = LOG ? v : ((v > 0.0) ? log2_d(v) + (double)E : kNegInfD);
    if (lane == 0) {
        if (bw) {
            log2z[d.index] = l2;
            loss[d.index] = (float)(-l2 * kLn2D);
        } else {
            log2z[B + d.index] = l2;
        }
    }
}

// LOG: the log-domain rerun, of the samples k_mb_check marked only.
template <int G, int NB, bool LOG>
__global__ __launch_bounds__(64) void k_mb_sweep(const SampleDesc *__restrict__ desc, int B, MbParams mp,
                                                 const double *__restrict__ wp, int64_t n_slots,
                                                 double *__restrict__ alpha, double *__restrict__ beta,
                                                 int *__restrict__ ealpha, int *__restrict__ ebeta,
                                                 double *__restrict__ log2z, float *__restrict__ loss,
                                                 const int *__restrict__ mode) {
    const SampleDesc d = desc[blockIdx.x >> 1];
    if (LOG && mode[d.index] == 0) return;
    if (blockIdx.x & 1)
        mb_sweep_dir<G, NB, true, LOG>(d, B, mp, wp, n_slots, alpha, beta, ealpha, ebeta, log2z, loss);
    else
        mb_sweep_dir<G, NB, false, LOG>(d, B, mp, wp, n_slots, alpha, beta, ealpha, ebeta, log2z, loss);
}

// Forward-backward check of the probability-domain sweeps.  Every alignment
// emits label u exactly once, so the sum over t of alpha(t,u) P(label)
// beta(t,u+1) is P(y|x) for every u < U.  Renormalising each diagonal by its
// largest value loses the nodes far below it (fp64's range); harmless where
// they carry no alignment mass, wrong where they do (big blanks make
// advancing in t cheap, so on a long lattice the nodes with more frames done
// can lie hundreds of nats above those with more labels done, which finish
// more cheaply).  One wave for each of 16 columns spread over [0, U) per
// sample (bin midpoints, the last column U-1); the terms, on different
// diagonals, are summed as log2 values.  A sum that differs from the
// backward P by more than 4e-6 in log2, or P itself zero, marks the sample
// for the log-domain rerun.  Lattices without labels have one node per
// diagonal and need no check.
__global__ __launch_bounds__(64) void k_mb_check(const SampleDesc *__restrict__ desc, int *__restrict__ mode,
                                                 const double *__restrict__ wp, int64_t n_slots, int U1p,
                                                 const double *__restrict__ alpha, const double *__restrict__ beta,
                                                 const int *__restrict__ ealpha, const int *__restrict__ ebeta,
                                                 const double *__restrict__ log2z) {
    constexpr int J = 16;
    const SampleDesc d = desc[blockIdx.x / J];
    const int j = blockIdx.x % J;
    const int T = d.T, U = d.U, U1 = U + 1;
    if (U == 0 || mode[d.index] != 0) return;
    const int lane = threadIdx.x;
    const double lz = log2z[d.index];
    const int u = (j + 1 < J) ? (int)(((int64_t)(2 * j + 1) * U) / (2 * J)) : U - 1;
    const int64_t eo = d.diag_off + d.index;
    double m = kNegInfD, s = 0.0;
    for (int t = lane; t < T; t += 64) {
        const int n = t + u;
        const double la = log2_d(alpha[d.ab_off + (int64_t)n * U1p + u]) + (double)ealpha[eo + n];
        const double lw = log2_d(wp[n_slots + d.slot_off + (int64_t)n * U1 + u]);
        const double lb = log2_d(beta[d.ab_off + (int64_t)(n + 1) * U1p + u + 1]) + (double)ebeta[eo + n + 1];
        const double l = la + lw + lb;
        if (l > m) {
            s = s * (double)exp2_fast((float)(m - l)) + 1.0;
            m = l;
        } else if (l > kNegInfD) {
            s += (double)exp2_fast((float)(l - m));
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const double m2 = __shfl_xor(m, off, 64);
        const double s2 = __shfl_xor(s, off, 64);
        const double mm = fmax(m, m2);
        s = (mm == kNegInfD) ? 0.0
                             : s * (double)exp2_fast((float)(m - mm)) + s2 * (double)exp2_fast((float)(m2 - mm));
        m = mm;
    }
    const double ls = m + log2_d(s);
    const bool bad = !(lz > kNegInfD) || !(m > kNegInfD) || !(fabs(ls - lz) <= 4e-6);
    if (bad && lane == 0) atomicOr(&mode[d.index], 1);
}

// The gradient terms of packed row r: the softmax shift (occupancy with the
// FastEmit term, log2 domain, minus the row's normaliser) and the scaled
// flows of the edges leaving the node, with the label class.
struct MbRowTerms {
    float m;       // the row's maximum (0 if not fused)
    float shift2;  // log2(occ * scale) - log2(sum of exp(x - m)), or -inf
    float fb, fy;
    float fg[kMaxBigBlanks];
    int y;
};

__device__ __forceinline__ MbRowTerms mb_row_terms(const SampleDesc &d, int64_t r, int t, int u, int V, int blank,
                                                   int fused,
                                                   const MbParams &mp, int U1p, const int32_t *__restrict__ targets,
                                                   int S, const float2 *__restrict__ den,
                                                   const double *__restrict__ wp, int64_t n_slots,
                                                   const double *__restrict__ alpha,
                                                   const double *__restrict__ beta, const int *__restrict__ ealpha,
                                                   const int *__restrict__ ebeta, const double *__restrict__ log2z,
                                                   float scale, float fastemit, bool lm) {
    const int U1 = d.U + 1;
    const int n = t + u;
    const int64_t s = d.slot_off + (int64_t)n * U1 + u;
    const int64_t eo = d.diag_off + d.index;
    const double lz = log2z[d.index];
    // log2 beta of node (t2,u2): the virtual end (T,U) is 1, anything outside the lattice 0
    auto lbeta = [&](int t2, int u2) -> double {
        if (t2 == d.T && u2 == d.U) return 0.0;
        if (t2 >= d.T || u2 > d.U) return kNegInfD;
        const int n2 = t2 + u2;
        const double v = beta[d.ab_off + (int64_t)n2 * U1p + u2];
        return lm ? v : log2_d(v) + (double)ebeta[eo + n2];
    };
    double lo = kNegInfD, lb = kNegInfD, ly = kNegInfD;
    double lg[kMaxBigBlanks];
#pragma unroll
    for (int i = 0; i < kMaxBigBlanks; ++i) lg[i] = kNegInfD;
    if (lz != kNegInfD) {
        const double av = alpha[d.ab_off + (int64_t)n * U1p + u];
        const double la = (lm ? av : log2_d(av) + (double)ealpha[eo + n]) - lz;
        lo = la + lbeta(t, u);
        lb = la + log2_d(wp[s]) + lbeta(t + 1, u);
        if (u < d.U) ly = la + log2_d(wp[n_slots + s]) + lbeta(t, u + 1);
#pragma unroll
        for (int i = 0; i < kMaxBigBlanks; ++i)
            if (i < mp.nb) lg[i] = la + log2_d(wp[(int64_t)(2 + i) * n_slots + s]) + lbeta(t + mp.dur[i], u);
    }
    if (fastemit > 0.f && ly != kNegInfD && lo != kNegInfD)
        lo += (double)log2f(1.f + fastemit * exp2_fast((float)(ly - lo)));
    MbRowTerms rt;
    rt.y = -1;
    if (u < d.U) {
        const int yy = targets[(int64_t)d.index * S + u];
        rt.y = mb_label_ok(yy, V, blank, mp) ? yy : -1;
    }
    rt.fb = exp2_fast((float)lb) * scale;
    rt.fy = exp2_fast((float)ly) * scale * (1.f + fastemit);
#pragma unroll
    for (int i = 0; i < kMaxBigBlanks; ++i) rt.fg[i] = exp2_fast((float)lg[i]) * scale;
    const float2 dn = den[r];
    rt.m = dn.x;
    rt.shift2 = (fused && lo != kNegInfD) ? (float)(lo - (double)dn.y) + log2_fast(scale) : kNegInf;
    return rt;
}

// The gradient for rows the vector form does not take (unaligned, or wider
// than 16 vectors per lane): one wave per row, four per workgroup, scalar
// elements.
template <typename T>
__global__ __launch_bounds__(256) void k_mb_grad(const T *__restrict__ logits, T *__restrict__ grad, int64_t N,
                                                 int V, int blank, int fused, MbParams mp, int U1p,
                                                 const SampleDesc *__restrict__ desc, int B,
                                                 const int32_t *__restrict__ targets, int S,
                                                 const float2 *__restrict__ den, const double *__restrict__ wp,
                                                 int64_t n_slots, const double *__restrict__ alpha,
                                                 const double *__restrict__ beta, const int *__restrict__ ealpha,
                                                 const int *__restrict__ ebeta, const double *__restrict__ log2z,
                                                 const int *__restrict__ mode, float clamp, float scale,
                                                 float fastemit, int64_t row_base) {
    const int lane = threadIdx.x & 63;
    const int64_t r = row_base + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= N) return;
    const SampleDesc d = mb_sample_of_row(desc, B, r);
    const int64_t lr = r - d.row_off;
    const int t = (int)(lr / d.tstride);
    const int u = (int)(lr - (int64_t)t * d.tstride);
    T *g = grad + r * (int64_t)V;
    if (t >= d.T || u > d.U) {  // a padding row of the padded layout: zero gradient
        for (int k = lane; k < V; k += 64) Elem<T>::store1(g + k, 0.f);
        return;
    }
    const MbRowTerms rt = mb_row_terms(d, r, t, u, V, blank, fused, mp, U1p, targets, S, den, wp, n_slots, alpha, beta,
                                       ealpha, ebeta, log2z, scale, fastemit, mode[d.index] != 0);
    const bool do_clamp = clamp > 0.f;
    const float cl = clamp * scale;
    const T *x = logits + r * (int64_t)V;
    for (int k = lane; k < V; k += 64) {
        float v = 0.f;
        if (fused) v = exp2_fast(fmaf(Elem<T>::load1(x + k) - rt.m, kLog2e, rt.shift2));
        v -= (k == blank) ? rt.fb : 0.f;
        v -= (k == rt.y) ? rt.fy : 0.f;
#pragma unroll
        for (int i = 0; i < kMaxBigBlanks; ++i) v -= (i < mp.nb && k == mp.ids[i]) ? rt.fg[i] : 0.f;
        Elem<T>::store1(g + k, clamp_to(v, cl, do_clamp));
    }
}

// The row passes with the row held in 16-byte vectors, lane l holding
// vectors l + 64i, i < NV (rows of at most NV KiB), one row per single-wave
// workgroup: the shape that streams fastest here.  The row pass reads with
// non-temporal loads (4% faster than ordinary loads, and the sweep after it
// finds more of its weights cached).  ODD: rows that do not all start on a
// 16-byte boundary, read in the vectors that cover them from the one holding
// the row's first element, as the plain row pass reads them (mask_row_edges).
template <typename T, int NV, bool FULL, bool ODD>
__global__ __launch_bounds__(64) void k_mb_rows_v(const T *__restrict__ logits, int64_t N, int V, int blank,
                                                  int fused, MbParams mp, const SampleDesc *__restrict__ desc,
                                                  int B, const int32_t *__restrict__ targets, int S,
                                                  float2 *__restrict__ den, double *__restrict__ wp,
                                                  int64_t n_slots, uint32_t *status, int64_t row_base) {
    using Vec = typename Raw<T>::vec;
    constexpr int VEC = Raw<T>::kVec;
    const int lane = threadIdx.x;
    const int64_t r = row_base + xcd_block(blockIdx.x, gridDim.x >> 3);
    if (r >= N) return;
    const T *x = logits + r * (int64_t)V;
    const int lead = ODD ? lead_of(x) : 0;
    const int nvec = ODD ? (lead + V + VEC - 1) / VEC : V / VEC;
    // the row's loads go out before the search for its sample, whose
    // dependent loads they do not need (a padding row of the padded layout
    // is read and then left)
    Vec xv[NV];
    if (fused) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (FULL || i * 64 + lane < nvec)
                xv[i] = load_raw<T, true>(x - lead + (int64_t)(i * 64 + lane) * VEC);
        if constexpr (ODD) mask_row_edges<T, NV>(xv, 0, lead, nvec, V);
    }
    const SampleDesc d = mb_sample_of_row(desc, B, r);
    const int64_t lr = r - d.row_off;
    const int t = (int)(lr / d.tstride);
    const int u = (int)(lr - (int64_t)t * d.tstride);
    if (t >= d.T || u > d.U) return;  // a padding row of the padded layout
    float mr = 0.f, ls2 = 0.f;
    bool dead = false;
    if (fused) {
        const float m = wave_max_f(row_max<T, NV, FULL>(xv, nvec));
        dead = (m == kNegInf);
        mr = dead ? 0.f : m;
        const float nm = -mr * kLog2e;
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (FULL || i * 64 + lane < nvec)
#pragma unroll
                for (int e = 0; e < VEC; ++e) sum += exp2_fast(fmaf(Raw<T>::get(xv[i], e), kLog2e, nm));
        sum = wave_sum_f(sum);
        ls2 = dead ? 0.f : log2_sum_shifted(sum, mr, nm);
    }
    if (lane == 0) den[r] = make_float2(mr, ls2);
    float v = kNegInf;
    if (lane < 2 + mp.nb) {
        int k = blank;
        if (lane == 1) {
            k = -1;
            if (u < d.U) {
                const int y = targets[(int64_t)d.index * S + u];
                const bool bad = !mb_label_ok(y, V, blank, mp);
                if (bad) atomicOr(status, (uint32_t)RNNT_DEV_BAD_TARGET);
                k = bad ? -1 : y;
            }
        }
#pragma unroll
        for (int i = 0; i < kMaxBigBlanks; ++i)
            if (lane == 2 + i) k = mp.ids[i];
        v = (k >= 0 && !dead) ? (Elem<T>::load1(x + k) - mr) - ls2 * kLn2 - mp.sigma : kNegInf;
    }
    mb_store_node(d, t, u, mp, lane, v, wp, n_slots);
}

// Subtracts f from element c of the row in the vector of lane
// (c / VEC) % 64, number (c / VEC) / 64 == i (c < 0: nothing).
template <int VEC>
__device__ __forceinline__ void mb_sub_at(float (&gv)[VEC], int vi, int i, int c, float f) {
    if (c >= 0 && ((c / VEC) >> 6) == i) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) gv[e] -= (vi * VEC + e == c) ? f : 0.f;
    }
}

// ODD: rows that do not all start on a 16-byte boundary (gradient and logits
// at the same offset from one): in the vectors that cover the row, the class
// k at slot lead + k; the row's first and last vectors are stored element by
// element within the row.
template <typename T, int NV, bool FULL, bool ODD>
__global__ __launch_bounds__(64) void k_mb_grad_v(const T *__restrict__ logits, T *__restrict__ grad, int64_t N,
                                                  int V, int blank, int fused, MbParams mp, int U1p,
                                                  const SampleDesc *__restrict__ desc, int B,
                                                  const int32_t *__restrict__ targets, int S,
                                                  const float2 *__restrict__ den, const double *__restrict__ wp,
                                                  int64_t n_slots, const double *__restrict__ alpha,
                                                  const double *__restrict__ beta, const int *__restrict__ ealpha,
                                                  const int *__restrict__ ebeta, const double *__restrict__ log2z,
                                                  const int *__restrict__ mode, float clamp, float scale,
                                                  float fastemit, int64_t row_base) {
    using Vec = typename Raw<T>::vec;
    constexpr int VEC = Raw<T>::kVec;
    const int lane = threadIdx.x;
    // plain order: the XCD-contiguous order of the row pass made this pass slower (0.88 -> 0.94 ms)
    const int64_t r = row_base + (int64_t)blockIdx.x;
    if (r >= N) return;
    T *g = grad + r * (int64_t)V;
    const int lead = ODD ? lead_of(g) : 0;
    const int nvec = ODD ? (lead + V + VEC - 1) / VEC : V / VEC;
    T *gv0 = g - lead;  // the row's first vector
    // the vector of lane vi: stored whole, or element by element where it
    // reaches outside the row (ODD)
    auto store_vec = [&](int vi, const float (&v)[VEC]) {
        const int s0 = vi * VEC;
        if (!ODD || (s0 >= lead && s0 + VEC <= lead + V)) {
            store_raw<T, true>(gv0 + (int64_t)s0, Raw<T>::put(v));
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (s0 + e >= lead && s0 + e < lead + V) gv0[s0 + e] = (T)v[e];
        }
    };
    // the row's loads go out before the search for its sample (as in the
    // row pass)
    Vec xv[NV];
    if (fused) {
        const T *x = logits + r * (int64_t)V - lead;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (FULL || i * 64 + lane < nvec) xv[i] = load_raw<T, true>(x + (int64_t)(i * 64 + lane) * VEC);
    }
    const SampleDesc d = mb_sample_of_row(desc, B, r);
    const int64_t lr = r - d.row_off;
    const int t = (int)(lr / d.tstride);
    const int u = (int)(lr - (int64_t)t * d.tstride);
    if (t >= d.T || u > d.U) {  // a padding row of the padded layout: zero gradient
        const float z[VEC] = {};
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (FULL || i * 64 + lane < nvec) store_vec(i * 64 + lane, z);
        return;
    }
    MbRowTerms rt = mb_row_terms(d, r, t, u, V, blank, fused, mp, U1p, targets, S, den, wp, n_slots, alpha, beta, ealpha,
                                 ebeta, log2z, scale, fastemit, mode[d.index] != 0);
    const bool do_clamp = clamp > 0.f;
    const float cl = clamp * scale;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int vi = i * 64 + lane;
        if (FULL || vi < nvec) {
            float gv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                gv[e] = fused ? exp2_fast(fmaf(Raw<T>::get(xv[i], e) - rt.m, kLog2e, rt.shift2)) : 0.f;
            mb_sub_at<VEC>(gv, vi, i, blank + lead, rt.fb);
            mb_sub_at<VEC>(gv, vi, i, rt.y >= 0 ? rt.y + lead : -1, rt.fy);
#pragma unroll
            for (int k = 0; k < kMaxBigBlanks; ++k)
                mb_sub_at<VEC>(gv, vi, i, k < mp.nb ? mp.ids[k] + lead : -1, rt.fg[k]);
#pragma unroll
            for (int e = 0; e < VEC; ++e) gv[e] = clamp_to(gv[e], cl, do_clamp);
            store_vec(vi, gv);
        }
    }
}

MbParams mb_params(const MbArgs &a) {
    MbParams p{};
    p.nb = a.nb;
    int dmax = 1;
    for (int i = 0; i < kMaxBigBlanks; ++i) {
        p.ids[i] = i < a.nb ? a.ids[i] : -1;
        p.dur[i] = i < a.nb ? a.dur[i] : 1;
        if (i < a.nb) dmax = std::max(dmax, a.dur[i]);
    }
    p.R = 1;
    while (p.R < dmax + 1) p.R <<= 1;
    p.sigma = a.sigma;
    return p;
}

template <typename Fn> hipError_t with_esize(int esize, Fn &&fn) {
    if (esize == 4) return fn(float{});
    return fn(_Float16{});
}

}  // namespace

#define MBWS(type, field) reinterpret_cast<type>(a.ws + a.lay.field)

size_t mb_ring_bytes(int U1p, int max_duration) {
    size_t r = 1;
    while (r < (size_t)max_duration + 1) r <<= 1;
    return r * (size_t)U1p * sizeof(double);
}

// Vectors per lane of the vector row forms (0: the scalar forms): 16-byte
// aligned rows of at most 16 KiB.
// Vectors per lane of the vector row passes (0: the scalar kernels), and
// whether rows need the odd forms: rows not all on 16-byte boundaries, which
// span up to one vector more and need the gradient at the logits' offset
// from such a boundary when both are read and written; rows of up to 1 KiB
// keep the scalar kernels there (their results then do not depend on where
// the rows sit).
static int mb_row_nv(const MbArgs &a, bool &odd) {
    const int64_t rb = (int64_t)a.V * a.esize;
    odd = rb % 16 != 0 || (uintptr_t)a.logits % 16 != 0 || (a.grad && (uintptr_t)a.grad % 16 != 0);
    if (odd && (rb <= 1024 || (a.grad && a.fused && (((uintptr_t)a.logits ^ (uintptr_t)a.grad) & 15u) != 0)))
        return 0;
    const int64_t nvec = odd ? (rb + 32 - 2 * a.esize) / 16 : rb / 16;
    int nv = 1;
    while (nv * 64 < nvec) nv <<= 1;
    return nv <= 16 ? nv : 0;
}

// full: the row fills all nv vectors of every lane (no tail test); odd: the
// odd forms (never full).
template <typename Fn> static hipError_t with_mb_nv(int esize, int nv, bool full, bool odd, Fn &&fn) {
    auto go = [&](auto tag, auto fc, auto oc) -> hipError_t {
        using T = decltype(tag);
        switch (nv) {
        case 1: return fn(T{}, std::integral_constant<int, 1>{}, fc, oc);
        case 2: return fn(T{}, std::integral_constant<int, 2>{}, fc, oc);
        case 4: return fn(T{}, std::integral_constant<int, 4>{}, fc, oc);
        case 8: return fn(T{}, std::integral_constant<int, 8>{}, fc, oc);
        default: return fn(T{}, std::integral_constant<int, 16>{}, fc, oc);
        }
    };
    if (odd)
        return esize == 4 ? go(float{}, std::false_type{}, std::true_type{})
                          : go(_Float16{}, std::false_type{}, std::true_type{});
    if (esize == 4)
        return full ? go(float{}, std::true_type{}, std::false_type{}) : go(float{}, std::false_type{}, std::false_type{});
    return full ? go(_Float16{}, std::true_type{}, std::false_type{})
                : go(_Float16{}, std::false_type{}, std::false_type{});
}

hipError_t launch_mb_rows(const MbArgs &a, hipStream_t stream) {
    const MbParams mp = mb_params(a);
    constexpr int64_t kMaxBlocks = (int64_t)1 << 24;
    bool odd = false;
    const int nv = mb_row_nv(a, odd);
    if (nv > 0)
        return with_mb_nv(a.esize, nv, a.V * a.esize == nv * 1024, odd, [&](auto tag, auto nvc, auto fc, auto oc) {
            using T = decltype(tag);
            constexpr int NV = decltype(nvc)::value;
            constexpr bool FULL = decltype(fc)::value;
            constexpr bool ODD = decltype(oc)::value;
            for (int64_t b0 = 0; b0 < a.N; b0 += kMaxBlocks) {
                // a multiple of 8 workgroups, so each XCD takes a contiguous range of rows
                const unsigned nb = (unsigned)((std::min<int64_t>(kMaxBlocks, a.N - b0) + 7) & ~(int64_t)7);
                hipLaunchKernelGGL((k_mb_rows_v<T, NV, FULL, ODD>), dim3(nb), dim3(64), 0, stream,
                                   static_cast<const T *>(a.logits), a.N, a.V, a.blank, a.fused, mp,
                                   MBWS(const SampleDesc *, desc), a.B, a.targets, a.S, MBWS(float2 *, den),
                                   MBWS(double *, wp), a.lay.n_slots, MBWS(uint32_t *, status), b0);
            }
            return hipGetLastError();
        });
    return with_esize(a.esize, [&](auto tag) {
        using T = decltype(tag);
        const int64_t blocks = (a.N + 3) / 4;
        for (int64_t b0 = 0; b0 < blocks; b0 += kMaxBlocks) {
            const unsigned nb = (unsigned)std::min<int64_t>(kMaxBlocks, blocks - b0);
            hipLaunchKernelGGL(k_mb_rows<T>, dim3(nb), dim3(256), 0, stream, static_cast<const T *>(a.logits), a.N,
                               a.V, a.blank, a.fused, mp, MBWS(const SampleDesc *, desc), a.B, a.targets, a.S,
                               MBWS(float2 *, den), MBWS(double *, wp), a.lay.n_slots, MBWS(uint32_t *, status),
                               b0 * 4);
        }
        return hipGetLastError();
    });
}

hipError_t launch_mb_sweep(const MbArgs &a, hipStream_t stream) {
    const MbParams mp = mb_params(a);
    const size_t lds = mb_ring_bytes(a.lay.U1p, mp.R - 1);
    // The probability-domain sweeps, the forward-backward check, and the
    // log-domain rerun of the samples it marked (a launch whose workgroups
    // exit at once when none is).
    auto go = [&](auto kern, auto klog) {
        hipLaunchKernelGGL(kern, dim3(2 * a.B), dim3(64), lds, stream, MBWS(const SampleDesc *, desc), a.B, mp,
                           MBWS(const double *, wp), a.lay.n_slots, MBWS(double *, alpha), MBWS(double *, beta),
                           MBWS(int *, ealpha), MBWS(int *, ebeta), MBWS(double *, log2z), a.loss,
                           MBWS(const int *, mode));
        hipLaunchKernelGGL(k_mb_check, dim3(16 * a.B), dim3(64), 0, stream, MBWS(const SampleDesc *, desc),
                           MBWS(int *, mode), MBWS(const double *, wp), a.lay.n_slots, a.lay.U1p,
                           MBWS(const double *, alpha), MBWS(const double *, beta), MBWS(const int *, ealpha),
                           MBWS(const int *, ebeta), MBWS(const double *, log2z));
        hipLaunchKernelGGL(klog, dim3(2 * a.B), dim3(64), lds, stream, MBWS(const SampleDesc *, desc), a.B, mp,
                           MBWS(const double *, wp), a.lay.n_slots, MBWS(double *, alpha), MBWS(double *, beta),
                           MBWS(int *, ealpha), MBWS(int *, ebeta), MBWS(double *, log2z), a.loss,
                           MBWS(const int *, mode));
        return hipGetLastError();
    };
    auto by_nb = [&](auto jc) -> hipError_t {
        constexpr int G = decltype(jc)::value;
        switch (a.nb) {
        case 0: return go(k_mb_sweep<G, 0, false>, k_mb_sweep<G, 0, true>);
        case 1: return go(k_mb_sweep<G, 1, false>, k_mb_sweep<G, 1, true>);
        case 2: return go(k_mb_sweep<G, 2, false>, k_mb_sweep<G, 2, true>);
        case 3: return go(k_mb_sweep<G, 3, false>, k_mb_sweep<G, 3, true>);
        case 4: return go(k_mb_sweep<G, 4, false>, k_mb_sweep<G, 4, true>);
        }
        return hipErrorInvalidValue;
    };
    switch (a.lay.U1p / 128) {
    case 1: return by_nb(std::integral_constant<int, 1>{});
    case 2: return by_nb(std::integral_constant<int, 2>{});
    case 4: return by_nb(std::integral_constant<int, 4>{});
    case 8: return by_nb(std::integral_constant<int, 8>{});
    }
    return hipErrorInvalidValue;
}

hipError_t launch_mb_grad(const MbArgs &a, hipStream_t stream) {
    const MbParams mp = mb_params(a);
    constexpr int64_t kMaxBlocks = (int64_t)1 << 24;
    bool odd = false;
    const int nv = mb_row_nv(a, odd);
    if (nv > 0)
        return with_mb_nv(a.esize, nv, a.V * a.esize == nv * 1024, odd, [&](auto tag, auto nvc, auto fc, auto oc) {
            using T = decltype(tag);
            constexpr int NV = decltype(nvc)::value;
            constexpr bool FULL = decltype(fc)::value;
            constexpr bool ODD = decltype(oc)::value;
            for (int64_t b0 = 0; b0 < a.N; b0 += kMaxBlocks) {
                const unsigned nb = (unsigned)std::min<int64_t>(kMaxBlocks, a.N - b0);
                hipLaunchKernelGGL((k_mb_grad_v<T, NV, FULL, ODD>), dim3(nb), dim3(64), 0, stream,
                                   static_cast<const T *>(a.logits), static_cast<T *>(a.grad), a.N, a.V, a.blank,
                                   a.fused, mp, a.lay.U1p, MBWS(const SampleDesc *, desc), a.B, a.targets, a.S,
                                   MBWS(const float2 *, den), MBWS(const double *, wp), a.lay.n_slots,
                                   MBWS(const double *, alpha), MBWS(const double *, beta),
                                   MBWS(const int *, ealpha), MBWS(const int *, ebeta), MBWS(const double *, log2z),
                                   MBWS(const int *, mode), a.clamp, a.grad_scale, a.fastemit, b0);
            }
            return hipGetLastError();
        });
    return with_esize(a.esize, [&](auto tag) {
        using T = decltype(tag);
        const int64_t blocks = (a.N + 3) / 4;
        for (int64_t b0 = 0; b0 < blocks; b0 += kMaxBlocks) {
            const unsigned nb = (unsigned)std::min<int64_t>(kMaxBlocks, blocks - b0);
            hipLaunchKernelGGL(k_mb_grad<T>, dim3(nb), dim3(256), 0, stream, static_cast<const T *>(a.logits),
                               static_cast<T *>(a.grad), a.N, a.V, a.blank, a.fused, mp, a.lay.U1p,
                               MBWS(const SampleDesc *, desc), a.B, a.targets, a.S, MBWS(const float2 *, den),
                               MBWS(const double *, wp), a.lay.n_slots, MBWS(const double *, alpha),
                               MBWS(const double *, beta), MBWS(const int *, ealpha), MBWS(const int *, ebeta),
                               MBWS(const double *, log2z), MBWS(const int *, mode), a.clamp, a.grad_scale,
                               a.fastemit, b0 * 4);
        }
        return hipGetLastError();
    });
}

hipError_t launch_mb_reduce(const MbArgs &a, hipStream_t stream) {
    float *out = (a.reduction != RNNT_REDUCTION_NONE) ? a.loss_reduced : nullptr;
    hipLaunchKernelGGL(k_reduce, dim3(1), dim3(64), 0, stream, a.loss, MBWS(const double *, log2z), a.B,
                       a.reduction == RNNT_REDUCTION_MEAN, out, MBWS(uint32_t *, status), nullptr, nullptr);
    return hipGetLastError();
}

#undef MBWS

}  // namespace rnnt

// ========================================= scratch of the allocation-free call
// rnnt_loss_fused_noalloc takes its workspace from this fixed array instead of
// a caller allocation, for callers that cannot allocate device memory.  Each
// device that loads the library holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address comes from hipGetSymbolAddress, once per device with that
// device current, and only that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[rnnt::kScratchBytes];

namespace rnnt {

hipError_t scratch_address(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace rnnt
