// Internal declarations shared by the librnnt host code (rnnt_api.cpp) and
// its gfx950 kernels (rnnt_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rnnt.h"

namespace rnnt {

// One sample of the batch.  Rows are t-major: row row_off + t*tstride + u is
// lattice node (t,u); tstride = U+1 in the packed layout (samples follow
// each other without padding) and max_U+1 in the padded (B, max_T, max_U+1,
// V) layout, where row_off = i*max_T*(max_U+1).  The per-node values written
// by the row pass live in a skewed layout, one slot per (anti-diagonal
// n = t+u, u): slot_off + n*(U+1) + u, n in [0, T+U), so every anti-diagonal
// is contiguous; slots with t = n-u outside [0, T) hold "impossible"
// weights.  The recursions' outputs (alpha, beta) use the same skewed order
// with the diagonal padded to a whole number of wavefront column groups:
// ab_off + n*U1p + u, U1p = padded_width(U+1), so every lane of the sweep
// owns whole slots.  Per-diagonal values (the recursions' power-of-two
// exponents) are at diag_off + n / 8.
struct SampleDesc {
    int64_t row_off;
    int64_t slot_off;
    int64_t diag_off;
    int64_t ab_off;
    int32_t T;
    int32_t U;
    int32_t index;  // position of the sample in the batch (targets row)
    int32_t U1p;
    int32_t tstride;  // rows between (t,u) and (t+1,u)
    int32_t chunk0;   // index of the sample's first chunk in the chunk table
};

// Padded width of a lattice of width U1 in the alpha/beta sweeps (a 64-wide
// wavefront with K columns per lane per group): 64 (K = 1) up to 64
// columns, 128 (K = 2) up to 128, else a multiple of 256 (K = 4).
inline int padded_width(int U1) { return U1 <= 64 ? 64 : U1 <= 128 ? 128 : (U1 + 255) / 256 * 256; }

// A run of `count` lattice nodes of one sample handed to one workgroup of a
// row pass, in one of two orders:
//   row order: the sample-local rows row_begin .. row_begin+count-1 (the
//     gradient pass, and the row-statistics pass when a wavefront takes
//     several short rows);
//   diagonal order: by anti-diagonal n, then column u, from node
//     (n, u) = (diag, col); node (n, u) is row (n-u)*(U+1) + u (the
//     row-statistics pass when a wavefront takes one row, so that its
//     per-node outputs land in consecutive slots).
// Both orders cut every sample after the same node counts.
struct ChunkDesc {
    int32_t sample;
    int32_t row_begin;
    int32_t count;
    int32_t diag;
    int32_t col;
};

// Lattice nodes of a T x (U+1) lattice on the anti-diagonals before n
// (diagonal m holds columns max(0, m-T+1) .. min(m, U)).
__host__ __device__ inline int64_t diag_prefix(int64_t n, int64_t T, int64_t U) {
    const int64_t a = (n <= U + 1) ? n * (n + 1) / 2 : (U + 1) * (U + 2) / 2 + (n - U - 1) * (U + 1);
    const int64_t b = (n <= T) ? 0 : (n - T) * (n - T + 1) / 2;
    return a - b;
}

// Node number r0 of the lattice in anti-diagonal order (diagonal n, then
// column u): the largest n with diag_prefix(n) <= r0, found by bisection.
__host__ __device__ inline void diag_start(int32_t T, int32_t U, int64_t r0, int32_t &n, int32_t &u) {
    int64_t lo = 0, hi = (int64_t)T + U - 1;  // diag_prefix(lo) <= r0 < diag_prefix(hi + 1)
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        if (diag_prefix(mid, T, U) <= r0) lo = mid;
        else hi = mid - 1;
    }
    n = (int32_t)lo;
    const int64_t first = lo - T + 1 > 0 ? lo - T + 1 : 0;
    u = (int32_t)(first + (r0 - diag_prefix(lo, T, U)));
}

// Chunk j of sample `sample` (descriptor d): rows j*rpc .. in row order, the
// same count of nodes in anti-diagonal order from (diag, col).
__host__ __device__ inline ChunkDesc make_chunk(const SampleDesc &d, int32_t sample, int32_t j, int32_t rpc) {
    const int64_t rows = (int64_t)d.T * (d.U + 1);
    const int64_t r0 = (int64_t)j * rpc;
    ChunkDesc c;
    c.sample = sample;
    c.row_begin = (int32_t)r0;
    c.count = (int32_t)(rows - r0 < rpc ? rows - r0 : rpc);
    diag_start(d.T, d.U, r0, c.diag, c.col);
    return c;
}

// Byte offsets of the workspace regions (each 256-byte aligned).  Everything
// before `chunks` is written by the per-call upload; the chunk table is built
// on the device from the sample descriptors (launch_plan).  Per skewed slot:
//   node  {log P(blank), log P(next label), the row's maximum m and log2 of
//         its sum of exp(x - m) (fused; 0 and 0 for log-prob inputs)};
//   prob  {P(blank), P(next label)} in fp32.
struct WorkspaceLayout {
    size_t status;      // uint32 status word
    size_t mode;        // int32[B]: 1 = log-domain recursion (set by rowstats)
    size_t desc;        // SampleDesc[B]
    size_t order;       // int32[B], samples by decreasing cost
    size_t chunks;      // ChunkDesc[n_chunks]
    size_t cflags;      // uint32[n_chunks]: small batches, the row pass's flag word of each chunk
    size_t sflags;      // uint32[B]: small batches, each sample's status bits (from its chunks' flags)
    size_t node;        // float4[S]
    size_t prob;        // float2[S]
    size_t alpha;       // double[S_ab], padded diagonals
    size_t beta;        // double[S_ab]
    size_t ealpha;      // int32[D + B]: exponent of alpha per group of 8 diagonals
    size_t ebeta;       // int32[D + B]
    size_t log2z;       // double[2B]: log2 P(y|x), beta path at [i], alpha path at [B + i]
    size_t total;
    int64_t n_slots;
    int64_t n_ab_slots;
    int64_t n_diags;
    int64_t n_rows;              // lattice rows, sum_i T_i (U_i + 1)
    int32_t n_chunks;
    int32_t rows_per_chunk;
    int32_t max_sample_chunks;   // most chunks of any one sample
};

// Row-pass geometry chosen from V and the element size.
struct RowGeom {
    int lanes_per_row;  // G: 1..64 lanes cooperate on one row (power of two)
    int vec;            // elements per vector access (1 when rows are not 16-byte aligned)
    int rows_per_block_iter;
    int stream_parts;   // > 0: rows of more than 1 KiB in 16-byte vectors (odd forms for rows off 16-byte
                        // boundaries): the row pass takes one row per wave in segments of 4 or 5 KiB, the
                        // gradient pass one wave per part of 4 or 5 KiB (the launchers choose the parts);
                        // this is the number of 4 KiB parts covering the widest row
};

RowGeom row_geometry(int V, int esize, bool aligned16);

// Kernel launchers (defined in rnnt_kernels.hip).  All enqueue on `stream`
// and return the launch status.
struct LaunchArgs {
    const void *logits;
    void *grad;
    int esize;           // 4 (fp32) or 2 (fp16)
    int64_t N;
    int V;
    int B;
    int S;               // targets row stride
    int blank;           // normalised
    int fused;
    float clamp;         // <= 0: off
    float fastemit;      // FastEmit weight lambda >= 0 on the label-emission derivatives
    float grad_scale;    // 1 or 1/B
    const int32_t *targets;
    float *loss;
    float *loss_reduced;
    int reduction;
    uint8_t *ws;
    WorkspaceLayout lay;
    RowGeom geom;
    int max_U1;          // max_i (U_i + 1)
    bool aligned16;
    uint32_t *status_out;  // device; if set, the reduction kernel copies the final status word there
    bool small;          // a batch below kSmallRows rows with its descriptors in PlanArgs: three launches
};

// Batches below this many rows (and of at most kArgSamples samples) take
// three launches instead of six: the row pass derives its chunks from the
// descriptors passed as kernel arguments (no chunk-table launch), and one
// two-wave workgroup per sample runs both recursions, their check and the
// log-domain rerun.
constexpr int64_t kSmallRows = 64 * 1024 - 1024;

// Batches of up to kArgSamples samples pass their descriptors, in cost
// order, as kernel arguments to the chunk-table kernel (or, for batches
// below kSmallRows rows, to the row pass), which writes them and the order
// to the workspace, so no host-to-device copy is needed.
constexpr int kArgSamples = 64;
struct PlanArgs {
    int32_t B;
    int32_t pad;
    SampleDesc desc[kArgSamples];  // in cost order: desc[k].index is the k-th sample of the longest-first order
};
static_assert(sizeof(PlanArgs) <= 3900, "kernel arguments are limited to 4 KiB");

// `pa` null: the descriptors were uploaded with the workspace header.
hipError_t launch_plan(const LaunchArgs &a, const PlanArgs *pa, hipStream_t stream);
hipError_t launch_rowstats(const LaunchArgs &a, const PlanArgs *pa, hipStream_t stream);
hipError_t launch_alpha_beta(const LaunchArgs &a, hipStream_t stream);
hipError_t launch_grad(const LaunchArgs &a, hipStream_t stream);
hipError_t launch_reduce(const LaunchArgs &a, hipStream_t stream);
hipError_t launch_grad_scale(void *grad, int esize, int V, int64_t N, int B, const float *scale, int per_sample,
                             const uint8_t *ws, const WorkspaceLayout &lay, const RowGeom &geom,
                             hipStream_t stream);
// Padded layout: zero the gradient rows outside every sample's lattice.
hipError_t launch_zero_padding(void *grad, int esize, int V, int B, int max_T, int max_U1, const uint8_t *ws,
                               const WorkspaceLayout &lay, const RowGeom &geom, hipStream_t stream);

// The fixed device scratch used as the workspace of rnnt_loss_fused_noalloc:
// its size, and its address on the current device (hipGetSymbolAddress,
// taken once per device and kept).
constexpr size_t kScratchBytes = (size_t)128 << 20;
static_assert(kScratchBytes == RNNT_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
hipError_t scratch_address(void **ptr);

// Largest lattice width (U+1) the alpha/beta kernels support: up to
// kMaxTileU1 one wave holds a whole anti-diagonal (k_alpha_beta, k_ab_small),
// beyond it several waves share one (k_ab_wide; such batches take the
// six-launch path).
constexpr int kMaxU1 = 2048;
constexpr int kMaxTileU1 = 1024;
constexpr int kMaxMbU1 = 1024;  // the multi-blank sweep: up to eight groups of 128 columns

// ------------------------------------------------- multi-blank transducer
constexpr int kMaxBigBlanks = 4;
constexpr int kMaxBigBlankDuration = 16;
constexpr size_t kMbRingBytes = 64 * 1024;  // LDS of one sweep: the ring of recent diagonals

// Workspace of the multi-blank path.  Byte offsets; the status word is at 0
// and the sample descriptors at 256, as in the plain layout.
struct MbLayout {
    size_t status, desc, mode, den, wp, alpha, beta, ealpha, ebeta, log2z, total;
    int64_t n_slots;    // skewed node slots, sum_i (T_i+U_i)(U_i+1)
    int64_t rows;       // rows of logits and grad: sum_i T_i(U_i+1) packed, B * max_T * max_U1 padded
    int U1p;            // columns of one stored diagonal: 128 times a power of two, for every sample
};

struct MbArgs {
    const void *logits;
    void *grad;
    int esize;
    int64_t N;
    int V, B, S;
    int blank;          // normalised
    int fused;
    float clamp, fastemit, sigma, grad_scale;
    int nb;             // number of big blanks
    int ids[kMaxBigBlanks];
    int dur[kMaxBigBlanks];
    const int32_t *targets;
    float *loss;
    float *loss_reduced;
    int reduction;
    uint8_t *ws;
    MbLayout lay;
};

// LDS bytes of one multi-blank sweep: a ring of R diagonals of U1p fp64
// values, R the power of two above the longest duration.
size_t mb_ring_bytes(int U1p, int max_duration);
hipError_t launch_mb_rows(const MbArgs &a, hipStream_t stream);
hipError_t launch_mb_sweep(const MbArgs &a, hipStream_t stream);
hipError_t launch_mb_grad(const MbArgs &a, hipStream_t stream);
hipError_t launch_mb_reduce(const MbArgs &a, hipStream_t stream);

}  // namespace rnnt
