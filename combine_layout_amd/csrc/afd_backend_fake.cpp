// afd_backend_fake.cpp -- a recording backend for CPU-only tests of the host
// core.  Linked with afd_core.cpp into a separate host library: every device
// action is appended to a text log instead of running, so the state machine,
// the argument checks and the launch plan can be exercised without a GPU.
// Never linked into the HIP library.

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "afd_plan.h"

namespace {
std::vector<std::string> g_log;
std::vector<int32_t> g_ends;
std::vector<afd::TileRec> g_tiles;   // the last dispatch's layout tile records
uint64_t g_err = afd::kNoError;
int g_stall = 0;
int g_capturing = 0;
int g_fail = 0;

void logf(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
void logf(const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_log.emplace_back(buf);
}
}  // namespace

namespace afd {

int be_init_workspace(void *, const WorkspacePlan &wp)
{
    logf("init total=%zu nblk_max=%d", wp.total, wp.nblk_max);
    return g_fail;
}

int be_is_capturing(void *, int *capturing)
{
    *capturing = g_capturing;
    return 0;
}

int be_launch_dispatch(const RoundPlan &p, void *)
{
    TileRec tr[kLayoutMaxTiles];
    g_tiles.assign(tr, tr + layout_tiles(p, tr));
    std::string srcs;
    for (int s = 0; s < p.N; ++s) {
        char b[64];
        snprintf(b, sizeof(b), "%s%d", s ? "," : "", p.tok_off[s + 1] - p.tok_off[s]);
        srcs += b;
    }
    if (p.cached) {
        logf("dispatch cached ntok=%d T=%s", p.ntok, srcs.c_str());
    } else if (p.empty) {
        logf("dispatch empty E=%d T=%s", p.E, srcs.c_str());
    } else if (p.onepass) {
        logf("dispatch onepass ntok=%d nblk=%d T=%s tile=%d wait=%d", p.ntok, p.nblk, srcs.c_str(), p.tile,
             p.wait_polls);
    } else if (p.fused) {
        logf("dispatch fused=1 ntok=%d nblk=%d T=%s", p.ntok, p.nblk, srcs.c_str());
    } else {
        std::string vo;
        for (int s = 0; s <= p.N; ++s) {
            char b[32];
            snprintf(b, sizeof(b), "%s%d", s ? "," : "", p.voff[s]);
            vo += b;
        }
        logf("dispatch fused=0 ntok=%d nblk=%d T=%s tile=%d voff=%s", p.ntok, p.nblk, srcs.c_str(), p.tile, vo.c_str());
    }
    return g_fail;
}

int be_read_ends(const RoundPlan &p, void *, int32_t *host_ends, uint64_t *err_word)
{
    logf("read_ends E=%d", p.E);
    for (int e = 0; e < p.E; ++e) host_ends[e] = e < int(g_ends.size()) ? g_ends[e] : 0;
    *err_word = g_err;
    return g_fail;
}

int be_launch_combine(const RoundPlan &p, void *)
{
    std::string outs;
    for (int s = 0; s < p.N; ++s) {
        char b[64];
        snprintf(b, sizeof(b), "%s%p", s ? "," : "", p.out[s]);
        outs += b;
    }
    logf("combine ntok=%d out=%s", p.ntok, outs.c_str());
    return g_fail;
}

int be_launch_partial(const RoundPlan &p, int f, void *)
{
    logf("partial f=%d ntok=%d prow=%lld base=%p", f, p.ntok, static_cast<long long>(p.prow),
         static_cast<void *>(p.partials));
    return g_fail;
}

int be_launch_last(const RoundPlan &p, int f, void *)
{
    std::string outs;
    for (int s = 0; s < p.N; ++s) {
        char b[64];
        snprintf(b, sizeof(b), "%s%p", s ? "," : "", p.out[s]);
        outs += b;
    }
    logf("last f=%d ntok=%d prow=%lld base=%p out=%s", f, p.ntok, static_cast<long long>(p.prow),
         static_cast<void *>(p.partials), outs.c_str());
    return g_fail;
}

int be_launch_copy(const void *src, void *dst, int64_t bytes, void *)
{
    logf("copy %p->%p bytes=%lld", src, dst, static_cast<long long>(bytes));
    return g_fail;
}

int be_read_error(uint64_t *, void *, int clear, uint64_t *word)
{
    logf("read_error clear=%d", clear);
    *word = g_err;
    if (clear) g_err = kNoError;
    return g_fail;
}

int be_read_stall(uint32_t *, void *, int clear, int *stalled)
{
    *stalled = g_stall;
    if (clear) g_stall = 0;
    return g_fail;
}

int be_device_sync()
{
    logf("sync");
    return 0;
}

int be_static_scratch(int *device, void **ptr)
{
    *device = 0;
    *ptr = reinterpret_cast<void *>(uintptr_t(1) << 32);   // a fake, aligned "device" address
    return g_fail;
}

int be_init_static(void *ws, const WorkspacePlan &wp)
{
    logf("init_static ws=%p total=%zu", ws, wp.total);
    return g_fail;
}

}  // namespace afd

extern "C" {
int afd_fake_log_size() { return int(g_log.size()); }
int afd_fake_log_get(int i, char *buf, int n)
{
    if (i < 0 || i >= int(g_log.size()) || n <= 0) return -1;
    std::snprintf(buf, size_t(n), "%s", g_log[size_t(i)].c_str());
    return 0;
}
void afd_fake_log_clear() { g_log.clear(); }
void afd_fake_set_ends(const int32_t *ends, int n, uint64_t err)
{
    g_ends.assign(ends, ends + n);
    g_err = err;
}
void afd_fake_set_capturing(int c) { g_capturing = c; }
void afd_fake_set_stall(int s) { g_stall = s; }
void afd_fake_set_fail(int f) { g_fail = f; }
// The last dispatch's layout tile records as (src, t0, n, g0) quadruples;
// returns their number (0: no table).
int afd_fake_tiles(int32_t *out, int max)
{
    const int n = int(g_tiles.size());
    for (int b = 0; b < n && b < max; ++b) {
        out[4 * b] = g_tiles[size_t(b)].src;
        out[4 * b + 1] = g_tiles[size_t(b)].t0;
        out[4 * b + 2] = g_tiles[size_t(b)].n;
        out[4 * b + 3] = g_tiles[size_t(b)].g0;
    }
    return n;
}
}
