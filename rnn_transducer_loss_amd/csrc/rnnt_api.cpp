// Host side of librnnt: argument validation, the longest-first schedule, the
// workspace layout, the schedule upload and the kernel launch sequence behind
// the C ABI declared in include/rnnt.h.
//
// The two-phase interface (query the workspace size, then run with a caller
// allocated workspace) and the host-side placement of samples by decreasing
// lattice area follow the rnnt-loss-ascend README ("Architecture": the aclnn
// layer's workspace query and the host's largest-task-first / least-loaded
// balancing; "Operator features": samples sorted by T x U area).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <numeric>
#include <vector>

#include "rnnt_internal.h"

namespace rnnt {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Padded (B, max_T, max_U1, V) layout, or packed when max_T == 0.
struct Padding {
    int32_t max_T = 0;
    int32_t max_U1 = 0;
    bool on() const { return max_T > 0; }
};

struct Plan {
    std::vector<SampleDesc> desc;
    std::vector<int32_t> order;
    WorkspaceLayout lay{};
    int max_U1 = 1;
};

rnnt_status check_lengths(int32_t B, int32_t V, const int32_t *T, const int32_t *U) {
    if (B < 1 || V < 1 || !T || !U) return RNNT_INVALID_VALUE;
    for (int32_t i = 0; i < B; ++i) {
        if (T[i] < 1 || U[i] < 0) return RNNT_INVALID_VALUE;
        if (U[i] + 1 > kMaxU1) return RNNT_INVALID_VALUE;
    }
    return RNNT_SUCCESS;
}

// Samples by decreasing cost: lattice area T*(U+1) (the README's balancing
// key), then the length T+U of the recursion's critical path, then index,
// into ord[B].  The key is a strict total order, so every sorting method
// gives the same result; batches of up to kArgSamples samples take an
// insertion sort, which allocates nothing.
void lpt_order_into(int32_t B, const int32_t *T, const int32_t *U, int32_t *ord) {
    auto before = [&](int32_t a, int32_t b) {
        const int64_t aa = (int64_t)T[a] * (U[a] + 1), ab = (int64_t)T[b] * (U[b] + 1);
        if (aa != ab) return aa > ab;
        const int64_t la = (int64_t)T[a] + U[a], lb = (int64_t)T[b] + U[b];
        if (la != lb) return la > lb;
        return a < b;
    };
    for (int32_t i = 0; i < B; ++i) ord[i] = i;
    if (B <= kArgSamples) {
        for (int32_t i = 1; i < B; ++i) {
            const int32_t v = ord[i];
            int32_t j = i;
            for (; j > 0 && before(v, ord[j - 1]); --j) ord[j] = ord[j - 1];
            ord[j] = v;
        }
    } else {
        std::sort(ord, ord + B, before);
    }
}

// Rows per chunk: about 256 KiB of logits per workgroup, but at least ~1024
// chunks when the batch is small, rounded to a multiple of 64 rows (the most
// rows any row geometry's workgroup takes per iteration), so the chunk table
// does not depend on the geometry.  Below 64 K rows that rounding would
// leave most CUs idle and each workgroup walking its chunk in several
// dependent iterations, so small batches take chunks of a multiple of 8
// rows, ~2048 of them: one iteration each for rows of more than 16 classes.
int32_t rows_per_chunk(int64_t N, int32_t V, int esize) {
    const int64_t row_bytes = (int64_t)V * esize;
    const int64_t by_bytes = std::max<int64_t>(1, (256 * 1024) / std::max<int64_t>(1, row_bytes));
    const int64_t by_count = std::max<int64_t>(1, (N + 1023) / 1024);
    if (by_count < 64) {
        const int64_t small = std::max<int64_t>(1, (N + 2047) / 2048);
        return (int32_t)std::min<int64_t>((std::min(by_bytes, small) + 7) / 8 * 8, 64);
    }
    int64_t r = std::min(by_bytes, by_count);
    r = (r + 63) / 64 * 64;
    return (int32_t)std::min<int64_t>(r, 1 << 16);
}

// The sample descriptors (desc[B]), the longest-first order (order[B]) and
// the workspace layout of a batch, in caller storage; allocates nothing.
// Every sample's rows are cut into chunks of `rows_per_chunk` rows, numbered
// in longest-first sample order (the chunk table itself is built on the
// device from the descriptors, and by make_chunk on the host when asked for).
rnnt_status plan_into(int32_t B, int32_t V, int64_t N, int esize, const int32_t *T, const int32_t *U,
                      const Padding &pad, SampleDesc *desc, int32_t *order, WorkspaceLayout &L, int32_t &max_U1) {
    rnnt_status st = check_lengths(B, V, T, U);
    if (st != RNNT_SUCCESS) return st;
    if (pad.on()) {
        if (pad.max_U1 < 1) return RNNT_INVALID_VALUE;
        for (int32_t i = 0; i < B; ++i)
            if (T[i] > pad.max_T || U[i] + 1 > pad.max_U1) return RNNT_INVALID_VALUE;
        if ((int64_t)B * pad.max_T * pad.max_U1 >= ((int64_t)1 << 62) / std::max(1, V)) return RNNT_INVALID_VALUE;
    }
    int64_t row = 0, slot = 0, diag = 0, ab = 0;
    max_U1 = 1;
    for (int32_t i = 0; i < B; ++i) {
        SampleDesc &d = desc[i];
        d.row_off = pad.on() ? (int64_t)i * pad.max_T * pad.max_U1 : row;
        d.tstride = pad.on() ? pad.max_U1 : U[i] + 1;
        d.chunk0 = 0;
        d.slot_off = slot;
        d.diag_off = diag;
        d.ab_off = ab;
        d.T = T[i];
        d.U = U[i];
        d.index = i;
        d.U1p = padded_width(U[i] + 1);
        // the sweeps address a sample's alpha/beta table (T+U diagonals of
        // U1p fp64 values) and its log-domain weights (T+U diagonals of U+1
        // 16-byte slots) with 32-bit byte offsets
        if (((int64_t)T[i] + U[i]) * std::max<int64_t>(8 * d.U1p, 16 * (U[i] + 1)) >= ((int64_t)1 << 31))
            return RNNT_INVALID_VALUE;
        row += (int64_t)T[i] * (U[i] + 1);
        slot += ((int64_t)T[i] + U[i]) * (U[i] + 1);
        diag += (int64_t)T[i] + U[i];
        ab += ((int64_t)T[i] + U[i]) * d.U1p;
        max_U1 = std::max(max_U1, U[i] + 1);
    }
    if (N >= 0 && row != N) return RNNT_INVALID_VALUE;
    if (row >= ((int64_t)1 << 62) / std::max(1, V)) return RNNT_INVALID_VALUE;
    lpt_order_into(B, T, U, order);
    const int32_t rpc = rows_per_chunk(row, V, esize);
    int64_t n_chunks = 0, max_sample_chunks = 0;
    for (int32_t k = 0; k < B; ++k) {
        const int32_t i = order[k];
        const int64_t rows = (int64_t)T[i] * (U[i] + 1);
        if (rows > INT32_MAX) return RNNT_INVALID_VALUE;
        desc[i].chunk0 = (int32_t)std::min<int64_t>(n_chunks, INT32_MAX);
        const int64_t n = (rows + rpc - 1) / rpc;
        max_sample_chunks = std::max(max_sample_chunks, n);
        n_chunks += n;
    }
    if (n_chunks > INT32_MAX) return RNNT_INVALID_VALUE;
    size_t off = 0;
    L = WorkspaceLayout{};
    L.status = 0;
    off = 256;
    L.mode = off;   off = align_up(off + sizeof(int32_t) * B);
    L.desc = off;   off = align_up(off + sizeof(SampleDesc) * B);
    L.order = off;  off = align_up(off + sizeof(int32_t) * B);
    L.chunks = off; off = align_up(off + sizeof(ChunkDesc) * (size_t)n_chunks);
    L.cflags = off; off = align_up(off + sizeof(uint32_t) * (size_t)n_chunks);
    L.sflags = off; off = align_up(off + sizeof(uint32_t) * (size_t)B);
    L.node = off;   off = align_up(off + 4 * sizeof(float) * (size_t)slot);
    L.prob = off;   off = align_up(off + 2 * sizeof(float) * (size_t)slot);
    L.alpha = off;  off = align_up(off + sizeof(double) * (size_t)ab);
    L.beta = off;   off = align_up(off + sizeof(double) * (size_t)ab);
    L.ealpha = off; off = align_up(off + sizeof(int32_t) * (size_t)(diag + B));
    L.ebeta = off;  off = align_up(off + sizeof(int32_t) * (size_t)(diag + B));
    L.log2z = off;  off = align_up(off + sizeof(double) * 2 * (size_t)B);
    L.total = off;
    L.n_slots = slot;
    L.n_ab_slots = ab;
    L.n_diags = diag;
    L.n_chunks = (int32_t)n_chunks;
    L.n_rows = row;
    L.rows_per_chunk = rpc;
    L.max_sample_chunks = (int32_t)max_sample_chunks;
    return RNNT_SUCCESS;
}

rnnt_status build_plan(int32_t B, int32_t V, int64_t N, int esize, const int32_t *T, const int32_t *U,
                       Plan &p, const Padding &pad = Padding()) {
    rnnt_status st = check_lengths(B, V, T, U);
    if (st != RNNT_SUCCESS) return st;
    p.desc.resize(B);
    p.order.resize(B);
    return plan_into(B, V, N, esize, T, U, pad, p.desc.data(), p.order.data(), p.lay, p.max_U1);
}

int esize_of(rnnt_dtype dt) { return dt == RNNT_F32 ? 4 : (dt == RNNT_F16 ? 2 : 0); }

// ------------------------------------------------------------ upload staging
// A small ring of pinned host buffers per device.  Each upload copies the
// schedule into the next slot, enqueues an asynchronous copy on the caller's
// stream and records an event; a slot is reused only after its event has
// completed, so the caller's host memory is never referenced after return.
struct StagingSlot {
    void *host = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
};
struct StagingRing {
    StagingSlot slot[8];
    int next = 0;
};
std::mutex g_mu;
std::map<int, StagingRing> g_rings;

rnnt_status upload(void *dst, const std::vector<uint8_t> &src, hipStream_t stream) {
    // A captured copy would replay from a staging slot that later calls reuse.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return RNNT_MEMOPS_FAILED;
    if (cap != hipStreamCaptureStatusNone) return RNNT_INVALID_VALUE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return RNNT_MEMOPS_FAILED;
    std::lock_guard<std::mutex> lk(g_mu);
    StagingRing &ring = g_rings[dev];
    StagingSlot &s = ring.slot[ring.next];
    ring.next = (ring.next + 1) % 8;
    if (s.pending) {
        if (hipEventSynchronize(s.ev) != hipSuccess) return RNNT_MEMOPS_FAILED;
        s.pending = false;
    }
    if (!s.ev && hipEventCreateWithFlags(&s.ev, hipEventDisableTiming) != hipSuccess) return RNNT_MEMOPS_FAILED;
    if (s.cap < src.size()) {
        if (s.host) (void)hipHostFree(s.host);
        s.host = nullptr;
        s.cap = 0;
        const size_t want = std::max<size_t>(src.size() + src.size() / 2, 64 * 1024);
        if (hipHostMalloc(&s.host, want, hipHostMallocDefault) != hipSuccess) return RNNT_MEMOPS_FAILED;
        s.cap = want;
    }
    std::memcpy(s.host, src.data(), src.size());
    if (hipMemcpyAsync(dst, s.host, src.size(), hipMemcpyHostToDevice, stream) != hipSuccess)
        return RNNT_MEMOPS_FAILED;
    if (hipEventRecord(s.ev, stream) != hipSuccess) return RNNT_MEMOPS_FAILED;
    s.pending = true;
    return RNNT_SUCCESS;
}

// The header, mode flags, descriptors and order are contiguous at the start
// of the workspace and go up in one copy (the status word and the flags are
// cleared with it); the chunk table after them is built on the device.
std::vector<uint8_t> pack_plan(const Plan &p) {
    std::vector<uint8_t> buf(p.lay.chunks, 0);
    std::memcpy(buf.data() + p.lay.desc, p.desc.data(), sizeof(SampleDesc) * p.desc.size());
    std::memcpy(buf.data() + p.lay.order, p.order.data(), sizeof(int32_t) * p.order.size());
    return buf;
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// The schedule depends only on (B, V, dtype, lengths); the last one built is
// reused when a call repeats them, as training steps and the upstream
// gradient pass do.
struct PlanEntry {
    std::vector<int32_t> key;
    Plan plan;
    std::vector<uint8_t> packed;
    std::unique_ptr<PlanArgs> args;  // batches of up to kArgSamples samples
};
std::mutex g_plan_mu;
std::shared_ptr<const PlanEntry> g_plan_cache;

std::vector<int32_t> plan_key(int32_t B, int32_t V, int esize, const int32_t *T, const int32_t *U,
                              const Padding &pad) {
    std::vector<int32_t> k;
    k.reserve(5 + 2 * (size_t)B);
    k.push_back(B);
    k.push_back(V);
    k.push_back(esize);
    k.push_back(pad.max_T);
    k.push_back(pad.max_U1);
    k.insert(k.end(), T, T + B);
    k.insert(k.end(), U, U + B);
    return k;
}

rnnt_status get_plan(int32_t B, int32_t V, int64_t N, int esize, const int32_t *T, const int32_t *U,
                     std::shared_ptr<const PlanEntry> &out, const Padding &pad = Padding()) {
    rnnt_status st = check_lengths(B, V, T, U);
    if (st != RNNT_SUCCESS) return st;
    std::vector<int32_t> key = plan_key(B, V, esize, T, U, pad);
    {
        std::lock_guard<std::mutex> lk(g_plan_mu);
        if (g_plan_cache && g_plan_cache->key == key) out = g_plan_cache;
        else out.reset();
    }
    if (!out) {
        auto e = std::make_shared<PlanEntry>();
        st = build_plan(B, V, -1, esize, T, U, e->plan, pad);
        if (st != RNNT_SUCCESS) return st;
        e->key = std::move(key);
        e->packed = pack_plan(e->plan);
        if (B <= kArgSamples) {
            e->args.reset(new PlanArgs{});
            e->args->B = B;
            for (int32_t k = 0; k < B; ++k) e->args->desc[k] = e->plan.desc[e->plan.order[k]];
        }
        std::lock_guard<std::mutex> lk(g_plan_mu);
        g_plan_cache = e;
        out = e;
    }
    int64_t rows = 0;
    for (int32_t i = 0; i < B; ++i) rows += (int64_t)T[i] * (U[i] + 1);
    if (N >= 0 && rows != N) return RNNT_INVALID_VALUE;
    return RNNT_SUCCESS;
}

// ------------------------------------------------------------- kernel timing
constexpr int kTimedKernels = 4;
struct TimingState {
    bool on = false;
    std::vector<hipEvent_t> pool;                       // reusable events
    std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> recs;  // (kernel, (start, stop))
    size_t used = 0;
};
std::mutex g_time_mu;
TimingState g_time;

hipEvent_t timing_event() {
    if (g_time.used == g_time.pool.size()) {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        g_time.pool.push_back(e);
    }
    return g_time.pool[g_time.used++];
}

// Launches `fn` on `stream`, bracketed by timing events when timing is on.
template <typename F> hipError_t timed(int kernel, hipStream_t stream, F &&fn) {
    std::unique_lock<std::mutex> lk(g_time_mu);
    if (!g_time.on) {
        lk.unlock();
        return fn();
    }
    hipEvent_t a = timing_event(), b = timing_event();
    if (a) (void)hipEventRecord(a, stream);
    const hipError_t err = fn();
    if (b) (void)hipEventRecord(b, stream);
    if (a && b) g_time.recs.push_back({kernel, {a, b}});
    return err;
}

}  // namespace
}  // namespace rnnt

using namespace rnnt;

extern "C" {

const char *rnnt_status_string(rnnt_status s) {
    switch (s) {
    case RNNT_SUCCESS: return "success";
    case RNNT_INVALID_VALUE: return "invalid argument value";
    case RNNT_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RNNT_MEMOPS_FAILED: return "HIP memory operation failed";
    case RNNT_EXECUTION_FAILED: return "kernel launch failed";
    default: break;
    }
    return "unknown status";
}

rnnt_status rnnt_loss_fused_workspace_size(int32_t B, int32_t V, int64_t N, rnnt_dtype dtype,
                                           const int32_t *logit_lengths, const int32_t *target_lengths,
                                           size_t *workspace_bytes) {
    const int es = esize_of(dtype);
    if (!es || !workspace_bytes || N < 0) return RNNT_INVALID_VALUE;
    std::shared_ptr<const PlanEntry> e;
    rnnt_status st = get_plan(B, V, N, es, logit_lengths, target_lengths, e);
    if (st != RNNT_SUCCESS) return st;
    *workspace_bytes = e->plan.lay.total;
    return RNNT_SUCCESS;
}

rnnt_status rnnt_plan_describe(int32_t B, int32_t V, rnnt_dtype dtype, const int32_t *logit_lengths,
                               const int32_t *target_lengths, int32_t cap, int32_t *sample_order,
                               int32_t *chunk_sample, int32_t *chunk_row_begin, int32_t *chunk_row_count,
                               int32_t *chunk_diag, int32_t *chunk_col, int32_t *n_chunks) {
    const int es = esize_of(dtype);
    if (!es || cap < 0) return RNNT_INVALID_VALUE;
    Plan p;
    rnnt_status st = build_plan(B, V, -1, es, logit_lengths, target_lengths, p);
    if (st != RNNT_SUCCESS) return st;
    if (sample_order)
        for (int32_t k = 0; k < B && k < cap; ++k) sample_order[k] = p.order[k];
    const int32_t nc = p.lay.n_chunks;
    const int32_t rpc = p.lay.rows_per_chunk;
    for (int32_t o = 0; o < B; ++o) {  // chunks of the samples in longest-first order
        const int32_t i = p.order[o];
        const SampleDesc &d = p.desc[i];
        const int64_t rows = (int64_t)d.T * (d.U + 1);
        const int32_t n = (int32_t)((rows + rpc - 1) / rpc);
        for (int32_t j = 0; j < n; ++j) {
            const int32_t k = d.chunk0 + j;
            if (k >= cap) break;
            const ChunkDesc c = make_chunk(d, i, j, rpc);
            if (chunk_sample) chunk_sample[k] = c.sample;
            if (chunk_row_begin) chunk_row_begin[k] = c.row_begin;
            if (chunk_row_count) chunk_row_count[k] = c.count;
            if (chunk_diag) chunk_diag[k] = c.diag;
            if (chunk_col) chunk_col[k] = c.col;
        }
    }
    if (n_chunks) *n_chunks = nc;
    return RNNT_SUCCESS;
}

}  // extern "C"

namespace rnnt {
namespace {

// Host checks of one call, before anything is enqueued; `aligned16` tells
// whether the rows can be moved in 16-byte vectors.
rnnt_status check_call(const void *logits, int es, int64_t N, int32_t V, const int32_t *targets, int32_t S,
                       const int32_t *logit_lengths, const int32_t *target_lengths, int32_t B, int64_t blank,
                       float fastemit_lambda, rnnt_reduction reduction, const float *loss, const void *grad,
                       const Padding &pad, bool &aligned16) {
    if (!es || V < 1 || B < 1) return RNNT_INVALID_VALUE;
    if (pad.on() ? (pad.max_U1 < 1) : (N < 0)) return RNNT_INVALID_VALUE;
    if (reduction != RNNT_REDUCTION_NONE && reduction != RNNT_REDUCTION_MEAN && reduction != RNNT_REDUCTION_SUM)
        return RNNT_INVALID_VALUE;
    if (blank < -(int64_t)V || blank > (int64_t)V - 1) return RNNT_INVALID_VALUE;
    if (!(fastemit_lambda >= 0.0f) || std::isinf(fastemit_lambda)) return RNNT_INVALID_VALUE;
    if (!logit_lengths || !target_lengths || !loss) return RNNT_INVALID_VALUE;
    rnnt_status st = check_lengths(B, V, logit_lengths, target_lengths);
    if (st != RNNT_SUCCESS) return st;
    const int64_t rows = pad.on() ? (int64_t)B * pad.max_T * pad.max_U1 : N;
    if (rows > 0 && !logits) return RNNT_INVALID_VALUE;
    int32_t maxU = 0;
    for (int32_t i = 0; i < B; ++i) maxU = std::max(maxU, target_lengths[i]);
    if (maxU > 0 && (!targets || S < maxU)) return RNNT_INVALID_VALUE;
    if (S < 0) return RNNT_INVALID_VALUE;
    const size_t bytes = (size_t)rows * (size_t)V * (size_t)es;
    if (grad && grad != logits && bytes > 0 && ranges_overlap(grad, bytes, logits, bytes)) return RNNT_INVALID_VALUE;
    aligned16 = ((int64_t)V * es) % 16 == 0 && ((uintptr_t)logits % 16 == 0) && (!grad || (uintptr_t)grad % 16 == 0);
    return RNNT_SUCCESS;
}

LaunchArgs launch_args(const void *logits, int es, int64_t rows, int32_t V, const int32_t *targets, int32_t S,
                       int32_t B, int64_t blank, float clamp, float fastemit_lambda, int fused_log_softmax,
                       rnnt_reduction reduction, float *loss, float *loss_reduced, void *grad, void *ws,
                       const WorkspaceLayout &lay, int32_t max_U1, bool aligned16) {
    LaunchArgs a{};
    a.logits = logits;
    a.grad = grad;
    a.esize = es;
    a.N = rows;
    a.V = V;
    a.B = B;
    a.S = S;
    a.blank = (int)(blank < 0 ? blank + V : blank);
    a.fused = fused_log_softmax ? 1 : 0;
    a.clamp = clamp;
    a.fastemit = fastemit_lambda;
    a.grad_scale = reduction == RNNT_REDUCTION_MEAN ? 1.0f / (float)B : 1.0f;
    a.targets = targets;
    a.loss = loss;
    a.loss_reduced = loss_reduced;
    a.reduction = reduction;
    a.ws = static_cast<uint8_t *>(ws);
    a.lay = lay;
    a.geom = row_geometry(V, es, aligned16);
    a.max_U1 = max_U1;
    a.aligned16 = aligned16;
    a.status_out = nullptr;
    return a;
}

// The kernels of one call, in order, on `stream`: the chunk table (and, with
// `pa`, the descriptors it carries as kernel arguments), row statistics, the
// recursions and their check, the gradient with the loss reduction in its
// first workgroup (score-only: the reduction alone), the padding rows' zeros.
// `timing`: bracket the passes with the bench's timing events.
rnnt_status enqueue_path(const LaunchArgs &a, const PlanArgs *pa, const Padding &pad, bool timing,
                         hipStream_t stream) {
    auto run = [&](int k, auto &&fn) { return timing ? timed(k, stream, fn) : fn(); };
    if (!a.small && launch_plan(a, pa, stream) != hipSuccess) return RNNT_EXECUTION_FAILED;
    if (a.lay.n_chunks > 0 && run(0, [&] { return launch_rowstats(a, pa, stream); }) != hipSuccess)
        return RNNT_EXECUTION_FAILED;
    if (run(1, [&] { return launch_alpha_beta(a, stream); }) != hipSuccess) return RNNT_EXECUTION_FAILED;
    if (a.grad && a.lay.n_chunks > 0 && run(2, [&] { return launch_grad(a, stream); }) != hipSuccess)
        return RNNT_EXECUTION_FAILED;
    if (a.grad && pad.on() &&
        launch_zero_padding(a.grad, a.esize, a.V, a.B, pad.max_T, pad.max_U1, a.ws, a.lay, a.geom, stream) !=
            hipSuccess)
        return RNNT_EXECUTION_FAILED;
    // with a gradient pass its first workgroup has reduced the losses; without one, a launch of its own
    if (!(a.grad && a.lay.n_chunks > 0) && run(3, [&] { return launch_reduce(a, stream); }) != hipSuccess)
        return RNNT_EXECUTION_FAILED;
    return RNNT_SUCCESS;
}

// The loss and gradient for the packed layout (pad off, N rows) or the
// padded (B, max_T, max_U1, V) layout (pad on, N ignored).
rnnt_status loss_impl(const void *logits, rnnt_dtype dtype, int64_t N, int32_t V, const int32_t *targets, int32_t S,
                      const int32_t *logit_lengths, const int32_t *target_lengths, int32_t B, int64_t blank,
                      float clamp, float fastemit_lambda, int fused_log_softmax, rnnt_reduction reduction,
                      float *loss, float *loss_reduced, void *grad, void *workspace, size_t workspace_bytes,
                      hipStream_t stream, const Padding &pad) {
    const int es = esize_of(dtype);
    bool aligned16 = false;
    rnnt_status st = check_call(logits, es, N, V, targets, S, logit_lengths, target_lengths, B, blank,
                                fastemit_lambda, reduction, loss, grad, pad, aligned16);
    if (st != RNNT_SUCCESS) return st;
    if (!workspace) return RNNT_INVALID_VALUE;
    std::shared_ptr<const PlanEntry> e;
    st = get_plan(B, V, pad.on() ? -1 : N, es, logit_lengths, target_lengths, e, pad);
    if (st != RNNT_SUCCESS) return st;
    const Plan &plan = e->plan;
    if (workspace_bytes < plan.lay.total) return RNNT_WORKSPACE_TOO_SMALL;
    if ((uintptr_t)workspace % kAlign != 0) return RNNT_INVALID_VALUE;
    if (!e->args) {
        st = upload(workspace, e->packed, stream);
        if (st != RNNT_SUCCESS) return st;
    }
    const int64_t rows = pad.on() ? (int64_t)B * pad.max_T * pad.max_U1 : N;
    LaunchArgs a = launch_args(logits, es, rows, V, targets, S, B, blank, clamp, fastemit_lambda,
                               fused_log_softmax, reduction, loss, loss_reduced, grad, workspace, plan.lay,
                               plan.max_U1, aligned16);
    a.small = e->args && plan.lay.n_rows <= kSmallRows && a.max_U1 <= kMaxTileU1;
    return enqueue_path(a, e->args.get(), pad, true, stream);
}

// ------------------------------------------------- multi-blank transducer
// Samples in batch order; every sample's diagonals are stored U1p wide, U1p a
// power-of-two multiple of 64 covering the widest lattice.
struct MbPlan {
    std::vector<SampleDesc> desc;
    MbLayout lay{};
};

rnnt_status build_mb_plan(int32_t B, int32_t V, int64_t N, const int32_t *T, const int32_t *U, int32_t nb,
                          const int32_t *dur, MbPlan &p, const Padding &pad = Padding()) {
    rnnt_status st = check_lengths(B, V, T, U);
    if (st != RNNT_SUCCESS) return st;
    if (pad.on()) {
        if (pad.max_U1 < 1) return RNNT_INVALID_VALUE;
        for (int32_t i = 0; i < B; ++i)
            if (T[i] > pad.max_T || U[i] + 1 > pad.max_U1) return RNNT_INVALID_VALUE;
        if ((int64_t)B * pad.max_T * pad.max_U1 >= ((int64_t)1 << 62) / std::max(1, V)) return RNNT_INVALID_VALUE;
    }
    if (nb < 0 || nb > kMaxBigBlanks || (nb > 0 && !dur)) return RNNT_INVALID_VALUE;
    int dmax = 1;
    for (int32_t i = 0; i < nb; ++i) {
        if (dur[i] < 1 || dur[i] > kMaxBigBlankDuration) return RNNT_INVALID_VALUE;
        dmax = std::max(dmax, (int)dur[i]);
    }
    int max_U1 = 1;
    for (int32_t i = 0; i < B; ++i) max_U1 = std::max(max_U1, U[i] + 1);
    if (max_U1 > kMaxMbU1) return RNNT_INVALID_VALUE;
    int G = 1;  // groups of 128 columns (two per lane) in the sweep
    while (128 * G < max_U1) G <<= 1;
    const int U1p = 128 * G;
    // the sweep addresses a sample's weights and its alpha/beta table (T+U
    // diagonals of U1p slots) with 32-bit byte offsets
    for (int32_t i = 0; i < B; ++i)
        if (((int64_t)T[i] + U[i]) * U1p * 8 >= ((int64_t)1 << 31)) return RNNT_INVALID_VALUE;
    if (mb_ring_bytes(U1p, dmax) > kMbRingBytes) return RNNT_INVALID_VALUE;
    p.desc.resize(B);
    int64_t row = 0, slot = 0, diag = 0, ab = 0;
    for (int32_t i = 0; i < B; ++i) {
        SampleDesc &d = p.desc[i];
        // packed: rows follow each other; padded: sample i's block starts at i * max_T * max_U1 and a frame
        // is max_U1 rows
        d.row_off = pad.on() ? (int64_t)i * pad.max_T * pad.max_U1 : row;
        d.slot_off = slot;
        d.diag_off = diag;
        d.ab_off = ab;
        d.T = T[i];
        d.U = U[i];
        d.index = i;
        d.U1p = U1p;
        d.tstride = pad.on() ? pad.max_U1 : U[i] + 1;
        d.chunk0 = 0;
        row += (int64_t)T[i] * (U[i] + 1);
        slot += ((int64_t)T[i] + U[i]) * (U[i] + 1);
        diag += (int64_t)T[i] + U[i];
        ab += ((int64_t)T[i] + U[i]) * U1p;
    }
    if (N >= 0 && row != N) return RNNT_INVALID_VALUE;
    if (row >= ((int64_t)1 << 62) / std::max(1, V)) return RNNT_INVALID_VALUE;
    const int64_t phys = pad.on() ? (int64_t)B * pad.max_T * pad.max_U1 : row;  // rows of logits and grad
    MbLayout &L = p.lay;
    size_t off = 0;
    L.status = 0;
    off = 256;
    L.desc = off;   off = align_up(off + sizeof(SampleDesc) * B);
    L.mode = off;   off = align_up(off + sizeof(int32_t) * B);  // per sample: 1 = recursions in the log domain
    // per row: the maximum and log2 of the sum of exp(x - maximum), fp32
    L.den = off;    off = align_up(off + 2 * sizeof(float) * (size_t)phys);
    // the sweep's 16-byte loads of a lane's column pair may reach one slot past a plane's last
    L.wp = off;     off = align_up(off + sizeof(double) * ((size_t)(2 + nb) * (size_t)slot + 2));
    L.alpha = off;  off = align_up(off + sizeof(double) * (size_t)ab);
    L.beta = off;   off = align_up(off + sizeof(double) * (size_t)ab);
    L.ealpha = off; off = align_up(off + sizeof(int32_t) * (size_t)(diag + B));
    L.ebeta = off;  off = align_up(off + sizeof(int32_t) * (size_t)(diag + B));
    L.log2z = off;  off = align_up(off + sizeof(double) * 2 * (size_t)B);
    L.total = off;
    L.n_slots = slot;
    L.U1p = U1p;
    L.rows = phys;
    return RNNT_SUCCESS;
}

rnnt_status multiblank_impl(const void *logits, rnnt_dtype dtype, int64_t N, int32_t V, const int32_t *targets,
                            int32_t S, const int32_t *T, const int32_t *U, int32_t B, int64_t blank, int32_t nb,
                            const int32_t *ids, const int32_t *dur, float sigma, float clamp, float fastemit,
                            int fused, rnnt_reduction reduction, float *loss, float *loss_reduced, void *grad,
                            void *workspace, size_t workspace_bytes, hipStream_t stream,
                            const Padding &pad = Padding()) {
    const int es = esize_of(dtype);
    if (!es || V < 1 || B < 1) return RNNT_INVALID_VALUE;
    if (pad.on() ? (pad.max_U1 < 1) : (N < 0)) return RNNT_INVALID_VALUE;
    if (reduction != RNNT_REDUCTION_NONE && reduction != RNNT_REDUCTION_MEAN && reduction != RNNT_REDUCTION_SUM)
        return RNNT_INVALID_VALUE;
    if (blank < -(int64_t)V || blank > (int64_t)V - 1) return RNNT_INVALID_VALUE;
    const int bn = (int)(blank < 0 ? blank + V : blank);
    if (!(fastemit >= 0.0f) || std::isinf(fastemit) || !std::isfinite(sigma)) return RNNT_INVALID_VALUE;
    if (!T || !U || !loss || !workspace) return RNNT_INVALID_VALUE;
    if (nb < 0 || nb > kMaxBigBlanks || (nb > 0 && (!ids || !dur))) return RNNT_INVALID_VALUE;
    for (int32_t i = 0; i < nb; ++i) {
        if (ids[i] < 0 || ids[i] >= V || ids[i] == bn) return RNNT_INVALID_VALUE;
        for (int32_t j = 0; j < i; ++j)
            if (ids[j] == ids[i]) return RNNT_INVALID_VALUE;
    }
    const int64_t rows = pad.on() ? (int64_t)B * pad.max_T * pad.max_U1 : N;
    if (rows > 0 && !logits) return RNNT_INVALID_VALUE;
    int32_t maxU = 0;
    for (int32_t i = 0; i < B; ++i) maxU = std::max(maxU, U[i]);
    if (maxU > 0 && (!targets || S < maxU)) return RNNT_INVALID_VALUE;
    if (S < 0) return RNNT_INVALID_VALUE;
    const size_t bytes = (size_t)rows * (size_t)V * (size_t)es;
    if (grad && grad != logits && bytes > 0 && ranges_overlap(grad, bytes, logits, bytes)) return RNNT_INVALID_VALUE;
    MbPlan plan;
    rnnt_status st = build_mb_plan(B, V, pad.on() ? -1 : N, T, U, nb, dur, plan, pad);
    if (st != RNNT_SUCCESS) return st;
    if (workspace_bytes < plan.lay.total) return RNNT_WORKSPACE_TOO_SMALL;
    if ((uintptr_t)workspace % kAlign != 0) return RNNT_INVALID_VALUE;

    // the status word (cleared), the descriptors and the mode words (cleared) go up in one copy
    std::vector<uint8_t> head(plan.lay.mode + sizeof(int32_t) * B, 0);
    std::memcpy(head.data() + plan.lay.desc, plan.desc.data(), sizeof(SampleDesc) * B);
    st = upload(workspace, head, stream);
    if (st != RNNT_SUCCESS) return st;

    MbArgs a{};
    a.logits = logits;
    a.grad = grad;
    a.esize = es;
    a.N = plan.lay.rows;
    a.V = V;
    a.B = B;
    a.S = S;
    a.blank = bn;
    a.fused = fused ? 1 : 0;
    a.clamp = clamp;
    a.fastemit = fastemit;
    a.sigma = sigma;
    a.grad_scale = reduction == RNNT_REDUCTION_MEAN ? 1.0f / (float)B : 1.0f;
    a.nb = nb;
    for (int32_t i = 0; i < nb; ++i) {
        a.ids[i] = ids[i];
        a.dur[i] = dur[i];
    }
    a.targets = targets;
    a.loss = loss;
    a.loss_reduced = loss_reduced;
    a.reduction = reduction;
    a.ws = static_cast<uint8_t *>(workspace);
    a.lay = plan.lay;
    if (a.N > 0 && timed(0, stream, [&] { return launch_mb_rows(a, stream); }) != hipSuccess)
        return RNNT_EXECUTION_FAILED;
    if (timed(1, stream, [&] { return launch_mb_sweep(a, stream); }) != hipSuccess) return RNNT_EXECUTION_FAILED;
    if (grad && a.N > 0 && timed(2, stream, [&] { return launch_mb_grad(a, stream); }) != hipSuccess)
        return RNNT_EXECUTION_FAILED;
    if (timed(3, stream, [&] { return launch_mb_reduce(a, stream); }) != hipSuccess) return RNNT_EXECUTION_FAILED;
    return RNNT_SUCCESS;
}

// The multi-blank gradient's upstream scaling: the descriptors the loss call
// left at byte 256 of its workspace give each sample's first row (packed, or
// its padded block), which is all k_grad_scale reads.
rnnt_status mb_grad_scale_impl(void *grad, rnnt_dtype dtype, int64_t N, int32_t V, const int32_t *T,
                               const int32_t *U, int32_t B, const float *scale, int per_sample,
                               const void *workspace, size_t workspace_bytes, hipStream_t stream,
                               const Padding &pad) {
    const int es = esize_of(dtype);
    if (!es || !grad || !scale || !workspace || V < 1 || B < 1) return RNNT_INVALID_VALUE;
    rnnt_status st = check_lengths(B, V, T, U);
    if (st != RNNT_SUCCESS) return st;
    int64_t rows = 0;
    if (pad.on()) {
        for (int32_t i = 0; i < B; ++i)
            if (T[i] > pad.max_T || U[i] + 1 > pad.max_U1) return RNNT_INVALID_VALUE;
        rows = (int64_t)B * pad.max_T * pad.max_U1;
    } else {
        for (int32_t i = 0; i < B; ++i) rows += (int64_t)T[i] * (U[i] + 1);
        if (rows != N) return RNNT_INVALID_VALUE;
    }
    WorkspaceLayout L{};
    L.desc = 256;  // where build_mb_plan puts the descriptors
    if (workspace_bytes < L.desc + sizeof(SampleDesc) * (size_t)B) return RNNT_WORKSPACE_TOO_SMALL;
    if (rows == 0) return RNNT_SUCCESS;
    const bool aligned16 = ((int64_t)V * es) % 16 == 0 && (uintptr_t)grad % 16 == 0;
    if (launch_grad_scale(grad, es, V, rows, B, scale, per_sample, static_cast<const uint8_t *>(workspace), L,
                          row_geometry(V, es, aligned16), stream) != hipSuccess)
        return RNNT_EXECUTION_FAILED;
    return RNNT_SUCCESS;
}

rnnt_status grad_scale_impl(void *grad, rnnt_dtype dtype, int64_t N, int32_t V, const int32_t *logit_lengths,
                            const int32_t *target_lengths, int32_t B, const float *scale, int per_sample,
                            const void *workspace, size_t workspace_bytes, hipStream_t stream, const Padding &pad) {
    const int es = esize_of(dtype);
    if (!es || !grad || !scale || !workspace || V < 1 || B < 1) return RNNT_INVALID_VALUE;
    if (pad.on() ? (pad.max_U1 < 1) : (N < 0)) return RNNT_INVALID_VALUE;
    std::shared_ptr<const PlanEntry> e;
    rnnt_status st = get_plan(B, V, pad.on() ? -1 : N, es, logit_lengths, target_lengths, e, pad);
    if (st != RNNT_SUCCESS) return st;
    const Plan &p = e->plan;
    if (workspace_bytes < p.lay.total) return RNNT_WORKSPACE_TOO_SMALL;
    const int64_t rows = pad.on() ? (int64_t)B * pad.max_T * pad.max_U1 : N;
    if (rows == 0) return RNNT_SUCCESS;
    const bool aligned16 = ((int64_t)V * es) % 16 == 0 && (uintptr_t)grad % 16 == 0;
    if (launch_grad_scale(grad, es, V, rows, B, scale, per_sample, static_cast<const uint8_t *>(workspace), p.lay,
                          row_geometry(V, es, aligned16), stream) != hipSuccess)
        return RNNT_EXECUTION_FAILED;
    return RNNT_SUCCESS;
}

}  // namespace
}  // namespace rnnt

extern "C" {

rnnt_status rnnt_loss_fused(const void *logits, rnnt_dtype dtype, int64_t N, int32_t V, const int32_t *targets,
                            int32_t S, const int32_t *logit_lengths, const int32_t *target_lengths, int32_t B,
                            int64_t blank, float clamp, float fastemit_lambda, int fused_log_softmax,
                            rnnt_reduction reduction, float *loss, float *loss_reduced, void *grad, void *workspace,
                            size_t workspace_bytes, rnnt_stream_t stream) {
    return loss_impl(logits, dtype, N, V, targets, S, logit_lengths, target_lengths, B, blank, clamp,
                     fastemit_lambda, fused_log_softmax, reduction, loss, loss_reduced, grad, workspace, workspace_bytes,
                     static_cast<hipStream_t>(stream), Padding());
}

rnnt_status rnnt_loss_fused_noalloc(const void *logits, rnnt_dtype dtype, int64_t N, int32_t V,
                                    const int32_t *targets, int32_t S, const int32_t *logit_lengths,
                                    const int32_t *target_lengths, int32_t B, int64_t blank, float clamp,
                                    float fastemit_lambda, int fused_log_softmax, rnnt_reduction reduction,
                                    float *loss, float *loss_reduced, void *grad, uint32_t *dev_status,
                                    rnnt_stream_t stream_) {
    // Everything below lives on the stack or in the device's fixed scratch:
    // no device, pinned or host heap allocation, no plan cache, no timing
    // events.  The schedule travels as kernel arguments, hence B <= 64.
    const hipStream_t stream = static_cast<hipStream_t>(stream_);
    const int es = esize_of(dtype);
    bool aligned16 = false;
    rnnt_status st = check_call(logits, es, N, V, targets, S, logit_lengths, target_lengths, B, blank,
                                fastemit_lambda, reduction, loss, grad, Padding(), aligned16);
    if (st != RNNT_SUCCESS) return st;
    if (B > kArgSamples) return RNNT_INVALID_VALUE;
    SampleDesc desc[kArgSamples];
    int32_t order[kArgSamples];
    WorkspaceLayout lay{};
    int32_t max_U1 = 1;
    st = plan_into(B, V, N, es, logit_lengths, target_lengths, Padding(), desc, order, lay, max_U1);
    if (st != RNNT_SUCCESS) return st;
    PlanArgs pa{};
    pa.B = B;
    for (int32_t k = 0; k < B; ++k) pa.desc[k] = desc[order[k]];
    if (lay.total > kScratchBytes) return RNNT_WORKSPACE_TOO_SMALL;
    void *ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return RNNT_MEMOPS_FAILED;
    LaunchArgs a = launch_args(logits, es, N, V, targets, S, B, blank, clamp, fastemit_lambda, fused_log_softmax,
                               reduction, loss, loss_reduced, grad, ws, lay, max_U1, aligned16);
    a.status_out = dev_status;
    a.small = lay.n_rows <= kSmallRows && a.max_U1 <= kMaxTileU1;
    return enqueue_path(a, &pa, Padding(), false, stream);
}

rnnt_status rnnt_loss_padded_workspace_size(int32_t B, int32_t V, int32_t max_T, int32_t max_U1, rnnt_dtype dtype,
                                            const int32_t *logit_lengths, const int32_t *target_lengths,
                                            size_t *workspace_bytes) {
    const int es = esize_of(dtype);
    if (!es || !workspace_bytes || max_T < 1 || max_U1 < 1) return RNNT_INVALID_VALUE;
    Padding pad;
    pad.max_T = max_T;
    pad.max_U1 = max_U1;
    std::shared_ptr<const PlanEntry> e;
    rnnt_status st = get_plan(B, V, -1, es, logit_lengths, target_lengths, e, pad);
    if (st != RNNT_SUCCESS) return st;
    *workspace_bytes = e->plan.lay.total;
    return RNNT_SUCCESS;
}

rnnt_status rnnt_loss_padded(const void *logits, rnnt_dtype dtype, int32_t max_T, int32_t max_U1, int32_t V,
                             const int32_t *targets, int32_t S, const int32_t *logit_lengths,
                             const int32_t *target_lengths, int32_t B, int64_t blank, float clamp,
                             float fastemit_lambda, int fused_log_softmax, rnnt_reduction reduction, float *loss,
                             float *loss_reduced, void *grad, void *workspace, size_t workspace_bytes,
                             rnnt_stream_t stream) {
    if (max_T < 1 || max_U1 < 1) return RNNT_INVALID_VALUE;
    Padding pad;
    pad.max_T = max_T;
    pad.max_U1 = max_U1;
    return loss_impl(logits, dtype, -1, V, targets, S, logit_lengths, target_lengths, B, blank, clamp,
                     fastemit_lambda, fused_log_softmax, reduction, loss, loss_reduced, grad, workspace, workspace_bytes,
                     static_cast<hipStream_t>(stream), pad);
}

rnnt_status rnnt_grad_scale(void *grad, rnnt_dtype dtype, int64_t N, int32_t V, const int32_t *logit_lengths,
                            const int32_t *target_lengths, int32_t B, const float *scale, int per_sample,
                            const void *workspace, size_t workspace_bytes, rnnt_stream_t stream) {
    return grad_scale_impl(grad, dtype, N, V, logit_lengths, target_lengths, B, scale, per_sample, workspace,
                           workspace_bytes, static_cast<hipStream_t>(stream), Padding());
}

rnnt_status rnnt_grad_scale_padded(void *grad, rnnt_dtype dtype, int32_t max_T, int32_t max_U1, int32_t V,
                                   const int32_t *logit_lengths, const int32_t *target_lengths, int32_t B,
                                   const float *scale, int per_sample, const void *workspace,
                                   size_t workspace_bytes, rnnt_stream_t stream) {
    if (max_T < 1 || max_U1 < 1) return RNNT_INVALID_VALUE;
    Padding pad;
    pad.max_T = max_T;
    pad.max_U1 = max_U1;
    return grad_scale_impl(grad, dtype, -1, V, logit_lengths, target_lengths, B, scale, per_sample, workspace,
                           workspace_bytes, static_cast<hipStream_t>(stream), pad);
}

rnnt_status rnnt_multiblank_workspace_size(int32_t B, int32_t V, int64_t N, rnnt_dtype dtype,
                                           const int32_t *logit_lengths, const int32_t *target_lengths,
                                           int32_t num_big_blanks, const int32_t *big_blank_durations,
                                           size_t *workspace_bytes) {
    if (!esize_of(dtype) || !workspace_bytes || N < 0) return RNNT_INVALID_VALUE;
    MbPlan p;
    rnnt_status st = build_mb_plan(B, V, N, logit_lengths, target_lengths, num_big_blanks, big_blank_durations, p);
    if (st != RNNT_SUCCESS) return st;
    *workspace_bytes = p.lay.total;
    return RNNT_SUCCESS;
}

rnnt_status rnnt_multiblank_loss(const void *logits, rnnt_dtype dtype, int64_t N, int32_t V, const int32_t *targets,
                                 int32_t S, const int32_t *logit_lengths, const int32_t *target_lengths, int32_t B,
                                 int64_t blank, int32_t num_big_blanks, const int32_t *big_blank_ids,
                                 const int32_t *big_blank_durations, float sigma, float clamp,
                                 float fastemit_lambda, int fused_log_softmax, rnnt_reduction reduction, float *loss,
                                 float *loss_reduced, void *grad, void *workspace, size_t workspace_bytes,
                                 rnnt_stream_t stream) {
    return multiblank_impl(logits, dtype, N, V, targets, S, logit_lengths, target_lengths, B, blank, num_big_blanks,
                           big_blank_ids, big_blank_durations, sigma, clamp, fastemit_lambda, fused_log_softmax,
                           reduction, loss, loss_reduced, grad, workspace, workspace_bytes,
                           static_cast<hipStream_t>(stream));
}

rnnt_status rnnt_multiblank_padded_workspace_size(int32_t B, int32_t V, int32_t max_T, int32_t max_U1,
                                                  rnnt_dtype dtype, const int32_t *logit_lengths,
                                                  const int32_t *target_lengths, int32_t num_big_blanks,
                                                  const int32_t *big_blank_durations, size_t *workspace_bytes) {
    if (!esize_of(dtype) || !workspace_bytes || max_T < 1 || max_U1 < 1) return RNNT_INVALID_VALUE;
    Padding pad;
    pad.max_T = max_T;
    pad.max_U1 = max_U1;
    MbPlan p;
    rnnt_status st = build_mb_plan(B, V, -1, logit_lengths, target_lengths, num_big_blanks, big_blank_durations, p,
                                   pad);
    if (st != RNNT_SUCCESS) return st;
    *workspace_bytes = p.lay.total;
    return RNNT_SUCCESS;
}

rnnt_status rnnt_multiblank_loss_padded(const void *logits, rnnt_dtype dtype, int32_t max_T, int32_t max_U1,
                                        int32_t V, const int32_t *targets, int32_t S, const int32_t *logit_lengths,
                                        const int32_t *target_lengths, int32_t B, int64_t blank,
                                        int32_t num_big_blanks, const int32_t *big_blank_ids,
                                        const int32_t *big_blank_durations, float sigma, float clamp,
                                        float fastemit_lambda, int fused_log_softmax, rnnt_reduction reduction,
                                        float *loss, float *loss_reduced, void *grad, void *workspace,
                                        size_t workspace_bytes, rnnt_stream_t stream) {
    if (max_T < 1 || max_U1 < 1) return RNNT_INVALID_VALUE;
    Padding pad;
    pad.max_T = max_T;
    pad.max_U1 = max_U1;
    return multiblank_impl(logits, dtype, -1, V, targets, S, logit_lengths, target_lengths, B, blank, num_big_blanks,
                           big_blank_ids, big_blank_durations, sigma, clamp, fastemit_lambda, fused_log_softmax,
                           reduction, loss, loss_reduced, grad, workspace, workspace_bytes,
                           static_cast<hipStream_t>(stream), pad);
}

rnnt_status rnnt_multiblank_grad_scale(void *grad, rnnt_dtype dtype, int64_t N, int32_t V,
                                       const int32_t *logit_lengths, const int32_t *target_lengths, int32_t B,
                                       const float *scale, int per_sample, const void *workspace,
                                       size_t workspace_bytes, rnnt_stream_t stream) {
    return mb_grad_scale_impl(grad, dtype, N, V, logit_lengths, target_lengths, B, scale, per_sample, workspace,
                              workspace_bytes, static_cast<hipStream_t>(stream), Padding());
}

rnnt_status rnnt_multiblank_grad_scale_padded(void *grad, rnnt_dtype dtype, int32_t max_T, int32_t max_U1,
                                              int32_t V, const int32_t *logit_lengths,
                                              const int32_t *target_lengths, int32_t B, const float *scale,
                                              int per_sample, const void *workspace, size_t workspace_bytes,
                                              rnnt_stream_t stream) {
    if (max_T < 1 || max_U1 < 1) return RNNT_INVALID_VALUE;
    Padding pad;
    pad.max_T = max_T;
    pad.max_U1 = max_U1;
    return mb_grad_scale_impl(grad, dtype, -1, V, logit_lengths, target_lengths, B, scale, per_sample, workspace,
                              workspace_bytes, static_cast<hipStream_t>(stream), pad);
}

rnnt_status rnnt_timing_enable(int on) {
    std::lock_guard<std::mutex> lk(g_time_mu);
    g_time.on = on != 0;
    g_time.recs.clear();
    g_time.used = 0;
    return RNNT_SUCCESS;
}

rnnt_status rnnt_timing_read(double *ms, int32_t *launches) {
    std::lock_guard<std::mutex> lk(g_time_mu);
    double acc[kTimedKernels] = {0, 0, 0, 0};
    int32_t cnt[kTimedKernels] = {0, 0, 0, 0};
    for (auto &r : g_time.recs) {
        if (hipEventSynchronize(r.second.second) != hipSuccess) return RNNT_MEMOPS_FAILED;
        float t = 0.f;
        if (hipEventElapsedTime(&t, r.second.first, r.second.second) != hipSuccess) return RNNT_MEMOPS_FAILED;
        acc[r.first] += t;
        cnt[r.first] += 1;
    }
    for (int k = 0; k < kTimedKernels; ++k) {
        if (ms) ms[k] = acc[k];
        if (launches) launches[k] = cnt[k];
    }
    return RNNT_SUCCESS;
}

rnnt_status rnnt_loss_fused_check(void *workspace, rnnt_stream_t stream_, uint32_t *dev_flags) {
    if (!workspace || !dev_flags) return RNNT_INVALID_VALUE;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    uint32_t v = 0;
    if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return RNNT_MEMOPS_FAILED;
    if (hipStreamSynchronize(stream) != hipSuccess) return RNNT_MEMOPS_FAILED;
    *dev_flags = v;
    return RNNT_SUCCESS;
}

}  // extern "C"
