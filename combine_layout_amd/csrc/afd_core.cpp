// afd_core.cpp -- host side of the C ABI: configuration checks, workspace
// plan, the per-round state machine and the launch plan.  It makes no HIP
// call itself; every device action goes through the be_* backend hooks.
//
// Round order (afdEP-comm API contract page, "Roles and tensors": one
// unmatched dispatch per Buffer, the receipt kept unchanged through the
// matching reply): every source dispatches once, then each partition
// receives once and replies once with its receipt, then every source
// collects once.

#include <cstring>
#include <mutex>
#include <new>

#include "afd_plan.h"

using namespace afd;

namespace {

enum Phase { kIdle = 0, kDispatching, kExchanging, kCollecting };

struct Part {
    void *rows = nullptr;
    float *scales = nullptr;
    float *roww = nullptr;
    int64_t cap = 0;
    bool bound = false;
};

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

struct afd_ctx {
    afd_config cfg{};
    int E_loc = 0;
    int64_t row_bytes = 0;
    char *ws = nullptr;
    size_t ws_bytes = 0;
    WorkspacePlan wp;
    Part part[kMaxParts];

    // round state
    uint64_t round = 0;
    Phase phase = kIdle;
    int bucket = 0, rhc = 0;
    bool dispatched[kMaxSources] = {};
    int ndispatched = 0;
    bool received[kMaxParts] = {};
    int nreceived = 0;
    bool launched = false;
    bool replied[kMaxParts] = {};
    int nreplied = 0;
    bool collected[kMaxSources] = {};
    int ncollected = 0;
    int T[kMaxSources] = {};
    void *out_user[kMaxSources] = {};
    int64_t recv_rows[kMaxParts] = {};
    int32_t host_ends[kMaxExperts] = {};
    bool route_error = false;
    bool round_cached = false;     // this round reuses the last layout
    RoundPlan plan;

    // how the last round whose dispatch work was enqueued runs
    afd_round_info info{};

    // the last layout whose dispatch work was enqueued (for cached rounds)
    bool layout_valid = false;
    int layout_bucket = 0;
    int layout_T[kMaxSources] = {};

    // afd_create_static: the device whose static context this is, else -1
    int static_dev = -1;

    // polls of a one-launch dispatch's wait before it gives up
    int wait_polls = kDefaultWaitPolls;
};

namespace {
// Host state of the contexts made by afd_create_static, one per device.
afd_ctx g_static_ctx[kMaxDevices];
bool g_static_used[kMaxDevices] = {};
std::mutex g_static_mu;
}  // namespace

namespace {

afd_status check_config(const afd_config *c)
{
    if (!c) return AFD_E_ARG;
    if (c->num_sources < 1 || c->num_sources > kMaxSources) return AFD_E_SHAPE;
    if (c->num_partitions < 1 || c->num_partitions > kMaxParts) return AFD_E_SHAPE;
    if (c->num_experts < 1 || c->num_experts > kMaxExperts) return AFD_E_SHAPE;
    if (c->num_experts % c->num_partitions != 0) return AFD_E_SHAPE;
    if (c->topk < 1 || c->topk > kMaxTopk || c->topk > c->num_experts) return AFD_E_SHAPE;
    if (c->hidden < 256 || c->hidden % 256 != 0) return AFD_E_SHAPE;
    if (c->expert_alignment < 1) return AFD_E_SHAPE;
    if (c->capacity < 1) return AFD_E_SHAPE;
    if (c->dtype != AFD_BF16 && c->dtype != AFD_FP8_E4M3) return AFD_E_SHAPE;
    if (c->combine != AFD_COMBINE_ONCE && c->combine != AFD_COMBINE_PER_STAGE &&
        c->combine != AFD_COMBINE_PER_STAGE_FP8)
        return AFD_E_SHAPE;
    if (c->combine != AFD_COMBINE_ONCE && c->num_partitions < 2) return AFD_E_SHAPE;
    if (c->dispatch != AFD_DISPATCH_AUTO && c->dispatch != AFD_DISPATCH_SPLIT && c->dispatch != AFD_DISPATCH_ONE_LAUNCH)
        return AFD_E_SHAPE;
    // index ranges used by the kernels: tokens * K in int32, rows below 2^24
    const int64_t ntok = int64_t(c->num_sources) * c->capacity;
    if (ntok * c->topk >= (int64_t(1) << 31)) return AFD_E_SHAPE;
    const int64_t E_loc = c->num_experts / c->num_partitions;
    const int64_t rmax = ntok * (c->topk < E_loc ? c->topk : E_loc) + E_loc * (c->expert_alignment - 1);
    if (rmax >= (int64_t(1) << 24)) return AFD_E_SHAPE;
    return AFD_OK;
}

int64_t rows_bound(const afd_config &c, int32_t bucket)
{
    const int64_t E_loc = c.num_experts / c.num_partitions;
    const int64_t kk = c.topk < E_loc ? c.topk : E_loc;
    return int64_t(c.num_sources) * bucket * kk + E_loc * (c.expert_alignment - 1);
}

WorkspacePlan plan_workspace(const afd_config &c)
{
    WorkspacePlan w;
    auto a = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t ntok = size_t(c.num_sources) * c.capacity;
    // every source starts on a tile boundary of the tiled token space
    w.nblk_max = int(c.num_sources * ((c.capacity + kLayoutTileMin - 1) / kLayoutTileMin));
    size_t off = 0;
    w.err = off;
    off += 256;
    w.ends = off;
    off += a(size_t(c.num_experts) * 4);
    w.blkcnt = off;
    off += a(size_t(align_up(w.nblk_max, 4)) * c.num_experts * 4);
    w.packed = off;
    off += a(ntok * c.topk * 4);
    w.slot = off;
    off += a(ntok * c.topk * 8 + 64);   // + slack for the combine's 64-byte slot reads
    w.inbox = off;
    if (c.num_partitions == 1) off += a(ntok * c.hidden * 2);
    w.partials = off;
    if (c.combine != AFD_COMBINE_ONCE)
        off += a(size_t(c.num_partitions) * ntok * size_t(partial_row_bytes(c.combine, c.hidden)));
    w.tcount = off;
    off += a(size_t(kLayoutMaxTiles) * tcount_pitch(c.num_experts) * 4 +
             size_t(kLayoutMaxTiles + 1) * tcount_pitch(c.num_experts) * 8);
    w.ready = off;
    off += a(size_t(kReadyCopies + kDoneGroups) * kReadyStride * 4);
    w.total = off;
    return w;
}

void reset_round(afd_ctx *c)
{
    std::memset(c->dispatched, 0, sizeof(c->dispatched));
    std::memset(c->received, 0, sizeof(c->received));
    std::memset(c->replied, 0, sizeof(c->replied));
    std::memset(c->collected, 0, sizeof(c->collected));
    std::memset(c->T, 0, sizeof(c->T));
    std::memset(c->out_user, 0, sizeof(c->out_user));
    c->ndispatched = c->nreceived = c->nreplied = c->ncollected = 0;
    c->launched = false;
    c->route_error = false;
    c->round_cached = false;
    RoundPlan fresh;
    c->plan = fresh;
}

void *inbox_of(afd_ctx *c, int s)
{
    return c->ws + c->wp.inbox + size_t(s) * c->cfg.capacity * c->cfg.hidden * 2;
}

// Fill the launch plan from the recorded dispatches and bound arenas.
void build_plan(afd_ctx *c, bool cached)
{
    RoundPlan &p = c->plan;
    const afd_config &g = c->cfg;
    p.N = g.num_sources;
    p.F = g.num_partitions;
    p.E = g.num_experts;
    p.E_loc = c->E_loc;
    p.K = g.topk;
    p.H = g.hidden;
    p.alpha = g.expert_alignment;
    p.fp8 = g.dtype == AFD_FP8_E4M3;
    p.capacity = g.capacity;
    p.combine = g.combine;
    p.prow = partial_row_bytes(g.combine, g.hidden);
    p.row_bytes = c->row_bytes;
    p.G = g.hidden / 128;
    p.tok_off[0] = 0;
    for (int s = 0; s < p.N; ++s) p.tok_off[s + 1] = p.tok_off[s] + c->T[s];
    p.ntok = p.tok_off[p.N];
    // a round without tokens has empty expert ranges at any E and H: its
    // dispatch only clears ends[]
    p.empty = p.ntok == 0;
    p.fused = !p.empty && p.ntok <= kFusedMaxTokens && int64_t(p.ntok) * p.K <= kFusedMaxIds &&
              p.E <= kFusedMaxExperts && p.row_bytes / 16 <= kFusedMaxCols;
    p.tile = place_sources(c->T, p.N, p.voff);
    p.nblk = p.fused || p.empty ? 1 : p.voff[p.N] / p.tile;   // the one-kernel dispatch has no tiles
    p.cached = cached;
    // the one-launch dispatch publishes at most kLayoutMaxTiles tile counts,
    // one expert per thread of a workgroup
    p.onepass = g.dispatch == AFD_DISPATCH_ONE_LAUNCH && !cached && !p.empty && !p.fused &&
                p.nblk <= kLayoutMaxTiles && p.E <= kMaxExpertsOneLaunch;
    p.wait_polls = c->wait_polls;
    for (int s = 0; s < p.N; ++s) p.out[s] = p.F == 1 ? inbox_of(c, s) : c->out_user[s];
    for (int f = 0; f < p.F; ++f) {
        p.rows[f] = c->part[f].rows;
        p.scales[f] = c->part[f].scales;
        p.roww[f] = c->part[f].roww;
    }
    p.err = reinterpret_cast<uint64_t *>(c->ws + c->wp.err);
    p.ends = reinterpret_cast<int32_t *>(c->ws + c->wp.ends);
    p.blkcnt = reinterpret_cast<int32_t *>(c->ws + c->wp.blkcnt);
    p.packed = reinterpret_cast<int32_t *>(c->ws + c->wp.packed);
    p.slot = reinterpret_cast<int32_t *>(c->ws + c->wp.slot);
    p.partials = g.combine != AFD_COMBINE_ONCE ? reinterpret_cast<uint8_t *>(c->ws + c->wp.partials) : nullptr;
    p.tcount = reinterpret_cast<uint32_t *>(c->ws + c->wp.tcount);
    p.ready = reinterpret_cast<uint32_t *>(c->ws + c->wp.ready);
    p.sync = reinterpret_cast<uint32_t *>(c->ws + kSyncOffset);
}

// Which kernels the round just enqueued runs (mirrors the executor's choice
// in be_launch_dispatch and the reply/collect launches).
void record_info(afd_ctx *c)
{
    const RoundPlan &p = c->plan;
    afd_round_info &i = c->info;
    i = afd_round_info{};
    i.round = c->round;
    i.tokens = p.ntok;
    if (p.cached) {
        i.dispatch_path = AFD_PATH_CACHED;
        i.dispatch_kernels = p.ntok > 0 ? 1 : 0;
    } else if (p.onepass) {
        i.dispatch_path = AFD_PATH_ONE_LAUNCH;
        i.dispatch_kernels = 1;
        i.layout_tiles = p.nblk;
        i.tile_tokens = p.tile;
    } else if (p.empty) {
        i.dispatch_path = AFD_PATH_EMPTY;
        i.dispatch_kernels = 1;
    } else if (p.fused) {
        i.dispatch_path = AFD_PATH_ONE_KERNEL;
        i.dispatch_kernels = 1;
    } else {
        i.dispatch_path = AFD_PATH_TILED;
        i.dispatch_kernels = 2;
        i.layout_tiles = p.nblk;
        i.tile_tokens = p.tile;
    }
    if (p.ntok > 0) {
        i.combine_kernels = p.combine == AFD_COMBINE_ONCE ? 1 : p.F;
    }
}

}  // namespace

extern "C" {

afd_status afd_set_dispatch_wait(afd_ctx *c, int32_t polls)
{
    if (!c) return AFD_E_ARG;
    c->wait_polls = polls;
    return AFD_OK;
}

afd_status afd_get_round_info(const afd_ctx *c, afd_round_info *info)
{
    if (!c || !info) return AFD_E_ARG;
    *info = c->info;
    return AFD_OK;
}

const char *afd_status_string(afd_status st)
{
    switch (st) {
    case AFD_OK: return "ok";
    case AFD_E_ARG: return "invalid argument";
    case AFD_E_SHAPE: return "invalid configuration or shape";
    case AFD_E_ORDER: return "call out of round order";
    case AFD_E_CAPACITY: return "buffer too small for the round";
    case AFD_E_ROUTE: return "invalid expert ids were routed (skipped)";
    case AFD_E_HIP: return "HIP runtime failure";
    case AFD_E_TIMEOUT: return "a one-launch dispatch gave up waiting between workgroups";
    }
    return "unknown status";
}

afd_status afd_query(const afd_config *cfg, int32_t bucket, size_t *workspace_bytes, int64_t *rows_bound_out)
{
    afd_status st = check_config(cfg);
    if (st != AFD_OK) return st;
    if (bucket < 1 || bucket > cfg->capacity) return AFD_E_ARG;
    if (workspace_bytes) *workspace_bytes = plan_workspace(*cfg).total;
    if (rows_bound_out) *rows_bound_out = rows_bound(*cfg, bucket);
    return AFD_OK;
}

static void init_ctx(afd_ctx *c, const afd_config *cfg, void *workspace, size_t workspace_bytes,
                     const WorkspacePlan &wp)
{
    c->cfg = *cfg;
    c->E_loc = cfg->num_experts / cfg->num_partitions;
    c->row_bytes = int64_t(cfg->hidden) * (cfg->dtype == AFD_FP8_E4M3 ? 1 : 2);
    c->ws = static_cast<char *>(workspace);
    c->ws_bytes = workspace_bytes;
    c->wp = wp;
}

afd_status afd_create(const afd_config *cfg, void *workspace, size_t workspace_bytes, afd_ctx **out)
{
    if (!out) return AFD_E_ARG;
    *out = nullptr;
    afd_status st = check_config(cfg);
    if (st != AFD_OK) return st;
    if (!workspace || !aligned(workspace, 256)) return AFD_E_ARG;
    WorkspacePlan wp = plan_workspace(*cfg);
    if (workspace_bytes < wp.total) return AFD_E_CAPACITY;
    afd_ctx *c = new (std::nothrow) afd_ctx;
    if (!c) return AFD_E_ARG;
    init_ctx(c, cfg, workspace, workspace_bytes, wp);
    if (be_init_workspace(workspace, wp) != 0) {
        delete c;
        return AFD_E_HIP;
    }
    *out = c;
    return AFD_OK;
}

afd_status afd_create_static(const afd_config *cfg, afd_ctx **out)
{
    if (!out) return AFD_E_ARG;
    *out = nullptr;
    afd_status st = check_config(cfg);
    if (st != AFD_OK) return st;
    const WorkspacePlan wp = plan_workspace(*cfg);
    if (wp.total > kStaticScratchBytes) return AFD_E_CAPACITY;
    int dev = -1;
    void *ws = nullptr;
    if (be_static_scratch(&dev, &ws) != 0 || dev < 0 || dev >= kMaxDevices || !ws) return AFD_E_HIP;
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (g_static_used[dev]) return AFD_E_ORDER;
    afd_ctx *c = &g_static_ctx[dev];
    *c = afd_ctx{};
    init_ctx(c, cfg, ws, kStaticScratchBytes, wp);
    c->static_dev = dev;
    if (be_init_static(ws, wp) != 0) return AFD_E_HIP;
    g_static_used[dev] = true;
    *out = c;
    return AFD_OK;
}

afd_status afd_bind_partition(afd_ctx *c, int32_t f, void *rows, float *scales, float *row_weights,
                              int64_t rows_cap)
{
    if (!c) return AFD_E_ARG;
    if (f < 0 || f >= c->cfg.num_partitions) return AFD_E_ARG;
    // allowed until a round's dispatch work is enqueued, so a receive that
    // failed (a smaller arena than the bucket needs) can be retried
    if (c->phase != kIdle && c->launched) return AFD_E_ORDER;
    if (rows_cap < 0) return AFD_E_ARG;
    if (rows_cap > 0) {
        if (!rows || !row_weights || !aligned(rows, 16) || !aligned(row_weights, 4)) return AFD_E_ARG;
        const bool fp8 = c->cfg.dtype == AFD_FP8_E4M3;
        if (fp8 && (!scales || !aligned(scales, 4))) return AFD_E_ARG;
        if (!fp8 && scales) return AFD_E_ARG;
    }
    Part &p = c->part[f];
    p.rows = rows;
    p.scales = scales;
    p.roww = row_weights;
    p.cap = rows_cap;
    p.bound = true;
    return AFD_OK;
}

afd_status afd_destroy(afd_ctx *c)
{
    if (!c) return AFD_OK;
    int rc = be_device_sync();
    if (c->static_dev >= 0) {
        std::lock_guard<std::mutex> lock(g_static_mu);
        g_static_used[c->static_dev] = false;
        c->static_dev = -1;
    } else {
        delete c;
    }
    return rc == 0 ? AFD_OK : AFD_E_HIP;
}

// Checks and records one source's round inputs; ids is NULL for a cached
// round (the layout of the last enqueued dispatch is reused).
static afd_status record_dispatch(afd_ctx *c, int32_t s, int32_t T, const void *x, const int32_t *ids,
                                  const float *weights, const float *x_scale, int64_t sst, int64_t ssg,
                                  void *out_bf16, int32_t bucket, int32_t rhc, bool cached)
{
    if (!c) return AFD_E_ARG;
    const afd_config &g = c->cfg;
    if (s < 0 || s >= g.num_sources) return AFD_E_ARG;
    if (c->phase != kIdle && c->phase != kDispatching) return AFD_E_ORDER;
    if (c->phase == kDispatching && c->dispatched[s]) return AFD_E_ORDER;
    if (c->phase == kDispatching && cached != c->round_cached) return AFD_E_ORDER;
    if (cached && !c->layout_valid) return AFD_E_ORDER;
    if (bucket < 1 || bucket > g.capacity) return AFD_E_ARG;
    if (rhc != 0 && rhc != 1) return AFD_E_ARG;
    if (c->phase == kDispatching && (bucket != c->bucket || rhc != c->rhc)) return AFD_E_ARG;
    if (cached && bucket != c->layout_bucket) return AFD_E_ARG;
    if (T < 0 || T > bucket) return AFD_E_SHAPE;
    if (cached && T != c->layout_T[s]) return AFD_E_SHAPE;
    const bool fp8 = g.dtype == AFD_FP8_E4M3;
    if (T > 0) {
        if (!x || (!ids && !cached) || !weights) return AFD_E_ARG;
        if (!aligned(x, 16) || !aligned(ids, 4) || !aligned(weights, 4)) return AFD_E_ARG;
        if (fp8) {
            if (!x_scale || !aligned(x_scale, 4) || sst < 0 || ssg < 0) return AFD_E_ARG;
        }
        if (g.num_partitions > 1 && !out_bf16) return AFD_E_ARG;
    }
    if (!fp8 && x_scale) return AFD_E_ARG;
    if (out_bf16 && !aligned(out_bf16, 16)) return AFD_E_ARG;

    if (c->phase == kIdle) {
        reset_round(c);
        c->round += 1;
        c->bucket = bucket;
        c->rhc = rhc;
        c->round_cached = cached;
        c->phase = kDispatching;
    }
    RoundPlan &p = c->plan;
    p.x[s] = T > 0 ? x : nullptr;
    p.ids[s] = (T > 0 && !cached) ? ids : nullptr;
    p.w[s] = T > 0 ? weights : nullptr;
    p.scale[s] = (fp8 && T > 0) ? x_scale : nullptr;
    p.sst[s] = sst;
    p.ssg[s] = ssg;
    c->T[s] = T;
    c->out_user[s] = out_bf16;
    c->dispatched[s] = true;
    c->ndispatched += 1;
    if (c->ndispatched == g.num_sources) c->phase = kExchanging;
    return AFD_OK;
}

afd_status afd_source_dispatch(afd_ctx *c, int32_t s, int32_t T, const void *x, const int32_t *ids,
                               const float *weights, const float *x_scale, int64_t sst, int64_t ssg,
                               void *out_bf16, int32_t bucket, int32_t rhc, void *stream)
{
    (void)stream;
    return record_dispatch(c, s, T, x, ids, weights, x_scale, sst, ssg, out_bf16, bucket, rhc, false);
}

afd_status afd_source_dispatch_cached(afd_ctx *c, int32_t s, int32_t T, const void *x, const float *weights,
                                      const float *x_scale, int64_t sst, int64_t ssg, void *out_bf16,
                                      int32_t bucket, void *stream)
{
    (void)stream;
    return record_dispatch(c, s, T, x, nullptr, weights, x_scale, sst, ssg, out_bf16, bucket, 0, true);
}

afd_status afd_worker_receive(afd_ctx *c, int32_t f, int32_t bucket, int32_t rhc, int32_t *host_counts,
                              afd_receive *out, void *stream)
{
    if (!c || !out) return AFD_E_ARG;
    const afd_config &g = c->cfg;
    if (f < 0 || f >= g.num_partitions) return AFD_E_ARG;
    if (c->phase != kExchanging) return AFD_E_ORDER;
    if (c->received[f]) return AFD_E_ORDER;
    if (bucket != c->bucket || rhc != c->rhc) return AFD_E_ARG;
    if (host_counts && !rhc) return AFD_E_ARG;

    if (!c->launched) {
        const int64_t need = rows_bound(g, c->bucket);
        for (int q = 0; q < g.num_partitions; ++q)
            if (!c->part[q].bound || c->part[q].cap < need) return AFD_E_CAPACITY;
        if (rhc) {
            int capturing = 0;
            if (be_is_capturing(stream, &capturing) != 0) return AFD_E_HIP;
            if (capturing) return AFD_E_ARG;
        }
        build_plan(c, c->round_cached);
        if (be_launch_dispatch(c->plan, stream) != 0) return AFD_E_HIP;
        c->launched = true;
        record_info(c);
        c->layout_valid = true;
        c->layout_bucket = c->bucket;
        for (int q = 0; q < g.num_sources; ++q) c->layout_T[q] = c->T[q];
        for (int q = 0; q < g.num_partitions; ++q) c->recv_rows[q] = need;
        if (rhc) {
            uint64_t word = kNoError;
            if (be_read_ends(c->plan, stream, c->host_ends, &word) != 0) return AFD_E_HIP;
            c->route_error = word != kNoError;
            for (int q = 0; q < g.num_partitions; ++q) {
                const int32_t last = c->host_ends[q * c->E_loc + c->E_loc - 1];
                c->recv_rows[q] = align_up(last, g.expert_alignment);
            }
        }
    }

    const int E_loc = c->E_loc;
    if (rhc && host_counts) {
        int64_t prev = 0;
        for (int j = 0; j < E_loc; ++j) {
            const int64_t end = c->host_ends[f * E_loc + j];
            const int64_t start = align_up(prev, g.expert_alignment);
            host_counts[j] = int32_t(align_up(end - start, g.expert_alignment));
            prev = end;
        }
    }
    out->rows = c->part[f].rows;
    out->scales = c->part[f].scales;
    out->weights = c->part[f].roww;
    out->ends = reinterpret_cast<const int32_t *>(c->ws + c->wp.ends) + size_t(f) * E_loc;
    out->receive_rows = c->recv_rows[f];
    out->receipt.round = c->round;
    out->receipt.partition = f;
    out->receipt.reserved = 0;
    c->received[f] = true;
    c->nreceived += 1;
    return (rhc && c->route_error) ? AFD_E_ROUTE : AFD_OK;
}

afd_status afd_worker_reply(afd_ctx *c, int32_t f, const void *reply, int64_t receive_rows,
                            const afd_receipt *receipt, void *stream)
{
    if (!c || !receipt) return AFD_E_ARG;
    if (f < 0 || f >= c->cfg.num_partitions) return AFD_E_ARG;
    if (c->phase != kExchanging) return AFD_E_ORDER;
    if (!c->received[f] || c->replied[f]) return AFD_E_ORDER;
    if (receipt->round != c->round || receipt->partition != f) return AFD_E_ORDER;
    if (receive_rows != c->recv_rows[f]) return AFD_E_SHAPE;
    if (receive_rows > 0 && (!reply || !aligned(reply, 16))) return AFD_E_ARG;
    c->plan.reply[f] = reply;
    const bool staged = c->cfg.combine != AFD_COMBINE_ONCE;
    const bool last = c->nreplied + 1 == c->cfg.num_partitions;
    // per-stage: every reply runs its partition's stage one, the last one
    // together with stage two for every source; once: the last reply runs
    // the whole combine
    if (c->plan.ntok > 0 && (staged || last)) {
        const int rc = !staged ? be_launch_combine(c->plan, stream)
                       : last  ? be_launch_last(c->plan, f, stream)
                               : be_launch_partial(c->plan, f, stream);
        if (rc != 0) {
            c->plan.reply[f] = nullptr;
            return AFD_E_HIP;
        }
    }
    c->replied[f] = true;
    c->nreplied += 1;
    if (last) c->phase = kCollecting;
    return AFD_OK;
}

afd_status afd_source_collect(afd_ctx *c, int32_t s, int32_t view, const void **result, int64_t *row_stride,
                              void *stream)
{
    if (!c || !result) return AFD_E_ARG;
    const afd_config &g = c->cfg;
    if (s < 0 || s >= g.num_sources) return AFD_E_ARG;
    if (view != 0 && view != 1) return AFD_E_ARG;
    if (c->phase != kCollecting) return AFD_E_ORDER;
    if (c->collected[s]) return AFD_E_ORDER;
    const void *res;
    if (g.num_partitions > 1) {
        res = c->out_user[s];
    } else if (view) {
        res = inbox_of(c, s);
    } else {
        if (!c->out_user[s] && c->T[s] > 0) return AFD_E_ARG;
        if (c->T[s] > 0 &&
            be_launch_copy(inbox_of(c, s), c->out_user[s], int64_t(c->T[s]) * g.hidden * 2, stream) != 0)
            return AFD_E_HIP;
        res = c->out_user[s];
    }
    *result = res;
    if (row_stride) *row_stride = g.hidden;
    c->collected[s] = true;
    c->ncollected += 1;
    if (c->ncollected == g.num_sources) c->phase = kIdle;
    return AFD_OK;
}

afd_status afd_get_partials(afd_ctx *c, int32_t s, int32_t f, const void **rows, int64_t *row_bytes)
{
    if (!c || !rows) return AFD_E_ARG;
    const afd_config &g = c->cfg;
    if (g.combine == AFD_COMBINE_ONCE) return AFD_E_ARG;
    if (s < 0 || s >= g.num_sources || f < 0 || f >= g.num_partitions) return AFD_E_ARG;
    const int64_t prow = partial_row_bytes(g.combine, g.hidden);
    *rows = c->ws + c->wp.partials + size_t((int64_t(f) * g.num_sources + s) * g.capacity * prow);
    if (row_bytes) *row_bytes = prow;
    return AFD_OK;
}

afd_status afd_get_error(afd_ctx *c, void *stream, int32_t clear, int32_t *code, int32_t *s, int32_t *t,
                         int32_t *k)
{
    if (!c) return AFD_E_ARG;
    if (clear != 0 && clear != 1) return AFD_E_ARG;
    int capturing = 0;
    if (be_is_capturing(stream, &capturing) != 0) return AFD_E_HIP;
    if (capturing) return AFD_E_ARG;
    uint64_t word = kNoError;
    if (be_read_error(reinterpret_cast<uint64_t *>(c->ws + c->wp.err), stream, clear, &word) != 0)
        return AFD_E_HIP;
    int stalled = 0;
    if (be_read_stall(reinterpret_cast<uint32_t *>(c->ws + kSyncOffset), stream, clear, &stalled) != 0)
        return AFD_E_HIP;
    const bool set = word != kNoError;
    if (code) *code = set ? int32_t(word & 0xFFFF) : AFD_ROUTE_NONE;
    if (s) *s = set ? int32_t(word >> 56) : -1;
    if (t) *t = set ? int32_t((word >> 24) & 0xFFFFFFFFull) : -1;
    if (k) *k = set ? int32_t((word >> 16) & 0xFF) : -1;
    if (stalled) return AFD_E_TIMEOUT;
    return set ? AFD_E_ROUTE : AFD_OK;
}

}  // extern "C"
