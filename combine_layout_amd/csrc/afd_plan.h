// afd_plan.h -- host-side plan of one round, shared by the host core and the
// backends (the HIP executor, or the recording backend used by CPU tests).
// Plain C++17; no HIP types.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/afd.h"

namespace afd {

constexpr int kMaxSources = AFD_MAX_SOURCES;
constexpr int kMaxParts = AFD_MAX_PARTITIONS;
constexpr int kMaxExperts = AFD_MAX_EXPERTS;
constexpr int kMaxTopk = AFD_MAX_TOPK;

// Tokens handled by one workgroup of the layout kernel: 1, 2 or 4
// wavefronts of 64 lanes, one token per lane (a wavefront's 64 tokens form
// one chunk).
constexpr int kLayoutTileMin = 64;
constexpr int kLayoutTile = 256;
// Tile counts of an expert the scatter requests at entry (beyond this many
// tiles it sums them in a loop), and the number of tile records the layout
// kernel's arguments carry (rounds with more tiles find each tile's source
// from the source offsets instead).
constexpr int kLayoutMaxTiles = 32;
// Small rounds rebuild the layout inside every scatter workgroup (one kernel
// for the whole dispatch): at most this many tokens, ids (staged in LDS) and
// experts, and rows of at most this many 16-byte columns.
constexpr int kFusedMaxTokens = 512;
constexpr int kFusedMaxIds = 4096;
constexpr int kFusedMaxExperts = 256;
constexpr int kFusedMaxCols = 2048;

// Sticky route-error word: (s << 56) | (t << 24) | (k << 16) | code, so the
// numeric minimum is the first offender in (source, token, k) order.
constexpr uint64_t kNoError = ~0ull;

// The workspace's first 256 bytes: the route-error word at 0, and the
// one-launch dispatch's words (uint32) at byte 64: launch counter at index
// 0, finished workgroup groups at 16, the sticky gave-up flag at 32.
constexpr size_t kSyncOffset = 64;
constexpr int kSyncDone = 16;
constexpr int kSyncStall = 32;
constexpr int kDefaultWaitPolls = 1000000;
// The one-launch dispatch's ready flag, in this many copies one 128-byte
// line apart, so that the scatter workgroups' polls spread over many lines
// instead of all reading one word.
constexpr int kReadyCopies = 64;
constexpr int kReadyStride = 32;   // uint32 words between copies (and between group counters)
// Finished workgroups of a one-launch dispatch are counted in this many
// group counters (workgroup b in group b % kDoneGroups), each on a line of
// its own after the flag copies; the last of a group counts the group in
// the workspace's finished-group word.
constexpr int kDoneGroups = 16;
// Experts of a round the one-launch dispatch takes (its hand-off reads four
// experts' words per lane of one wavefront).
constexpr int kMaxExpertsOneLaunch = 256;

// Largest combine output (bytes) written with streaming stores.
constexpr int64_t kCombineStreamOutBytes = int64_t(4) << 20;

// Words between consecutive tiles' runs of the one-launch dispatch's tile
// counts (tile-major, each run on whole 128-byte lines).
#ifdef __HIPCC__
__host__ __device__
#endif
inline int tcount_pitch(int E) { return (E + 31) / 32 * 32; }

inline int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Larger rounds place every source on a tile boundary of a "tiled" token
// space: source s occupies slots [voff[s], voff[s] + T[s]), and the slots up
// to the next boundary are empty.  Every layout tile, and every scatter
// workgroup inside it, then holds the tokens of a single source, whose
// record a kernel reads once.  The tile is the smallest of 64, 128 and 256
// tokens that keeps the round within kLayoutMaxTiles tiles, so mid-size
// rounds spread their layout over more workgroups.  Returns the tile.
inline int place_sources(const int *T, int N, int *voff)
{
    for (int tile = kLayoutTileMin;; tile *= 2) {
        voff[0] = 0;
        for (int s = 0; s < N; ++s) voff[s + 1] = voff[s] + int(align_up(T[s], tile));
        if (tile == kLayoutTile || voff[N] / tile <= kLayoutMaxTiles) return tile;
    }
}

// Bytes of one stage-one row of the per-stage combine: BF16 [H], or H E4M3
// codes followed by H/128 scale bytes, padded to a multiple of 32.
inline int64_t partial_row_bytes(int combine, int H)
{
    return combine == AFD_COMBINE_PER_STAGE_FP8 ? H + align_up(H / 128, 32) : int64_t(H) * 2;
}

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WorkspacePlan {
    size_t err = 0;        // uint64 sticky route-error word
    size_t ends = 0;       // int32 [E]
    size_t blkcnt = 0;     // int32 [E][pitch] live choices per layout tile (expert-major;
                           // pitch = tiles rounded up to 4)
    size_t packed = 0;     // int32 [N*capacity*K] (expert << 16 | rank in tile), -1 skipped
    size_t slot = 0;       // int32x2 [N*capacity*K] {part << 24 | row, weight bits}, then 64
                           // bytes of slack (the combine reads slots 64 bytes at a time)
    size_t inbox = 0;      // BF16 [N][capacity][H] (one partition only)
    size_t partials = 0;   // per-stage combine: [F][N][capacity] rows of partial_row_bytes
    size_t tcount = 0;     // one-launch dispatch: uint32 [kLayoutMaxTiles][tcount_pitch(E)] tagged tile counts,
                           // then uint64 [kLayoutMaxTiles + 1][tcount_pitch(E)] tagged first rows per tile and
                           // expert, and the ends
    size_t ready = 0;      // one-launch dispatch: uint32 ready flag, kReadyCopies copies kReadyStride apart,
                           // then kDoneGroups finished-workgroup counters at the same stride
    size_t total = 0;
    int nblk_max = 0;
};

// Everything a backend needs to run one round; pointers are device
// addresses recorded from the caller.
struct RoundPlan {
    // configuration
    int N = 0, F = 0, E = 0, E_loc = 0, K = 0, H = 0, alpha = 1, fp8 = 0, capacity = 0;
    int combine = AFD_COMBINE_ONCE;
    int64_t prow = 0;        // per-stage combine: bytes of one partial row
    int64_t row_bytes = 0;   // H * bytes per activation
    int G = 0;               // H / 128 scale blocks per row
    // tokens, concatenated over sources in order
    int ntok = 0;
    int tok_off[kMaxSources + 1] = {};
    bool fused = false;      // one-kernel dispatch
    bool empty = false;      // no tokens: the dispatch only clears ends[]
    bool onepass = false;    // one-launch dispatch (counting and scatter in one kernel)
    bool cached = false;     // scatter from the slot map of the last layout
    int nblk = 0;            // layout tiles (split path)
    int tile = 0;            // tokens per layout tile
    int voff[kMaxSources + 1] = {};   // first tiled slot of each source (voff[N]: slots)
    // per source
    const void *x[kMaxSources] = {};
    const int32_t *ids[kMaxSources] = {};
    const float *w[kMaxSources] = {};
    const float *scale[kMaxSources] = {};
    int64_t sst[kMaxSources] = {}, ssg[kMaxSources] = {};
    void *out[kMaxSources] = {};       // combine destination (out_bf16 or inbox)
    // per partition
    void *rows[kMaxParts] = {};
    float *scales[kMaxParts] = {};
    float *roww[kMaxParts] = {};
    const void *reply[kMaxParts] = {};
    // workspace
    uint64_t *err = nullptr;
    int32_t *ends = nullptr;
    int32_t *blkcnt = nullptr;
    int32_t *packed = nullptr;
    int32_t *slot = nullptr;
    // per-stage combine: row (f, s, t) at partials + ((f * N + s) * capacity + t) * prow
    uint8_t *partials = nullptr;
    // one-launch dispatch
    uint32_t *tcount = nullptr;   // [kLayoutMaxTiles][tcount_pitch(E)]
    uint32_t *ready = nullptr;    // [(kReadyCopies + kDoneGroups) * kReadyStride]
    uint32_t *sync = nullptr;     // launch counter, finished workgroups, gave-up flag
    int wait_polls = kDefaultWaitPolls;
};

// Layout tile records of a round of at most kLayoutMaxTiles tiles: tile b
// holds tokens t0 .. t0 + n - 1 of source src, the first of them token g0 of
// the round.  The layout kernel reads its tile's record instead of finding
// its source.  Returns the number of records; 0 when no layout kernel runs
// (one-kernel or cached dispatch) or the round has more tiles.
struct TileRec {
    int src, t0, n, g0;
};

inline int layout_tiles(const RoundPlan &p, TileRec *out)
{
    if (p.fused || p.cached || p.empty || p.nblk > kLayoutMaxTiles) return 0;
    for (int b = 0; b < p.nblk; ++b) {
        int s = 0;   // the last source whose span starts at or before the tile (empty spans are skipped)
        while (s + 1 < p.N && b * p.tile >= p.voff[s + 1]) ++s;
        const int t0 = b * p.tile - p.voff[s];
        const int T = p.tok_off[s + 1] - p.tok_off[s];
        out[b] = TileRec{s, t0, T - t0 < p.tile ? T - t0 : p.tile, p.tok_off[s] + t0};
    }
    return p.nblk;
}

// Contexts made by afd_create_static use a static scratch array of this many
// bytes per GPU as their workspace (one such context per device at a time).
constexpr size_t kStaticScratchBytes = size_t(AFD_STATIC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

// ---- backend: implemented by the HIP executor or the recording fake ----
// Each returns 0 on success, nonzero on a runtime failure.
int be_init_workspace(void *workspace, const WorkspacePlan &wp);
int be_is_capturing(void *stream, int *capturing);
int be_launch_dispatch(const RoundPlan &p, void *stream);
int be_read_ends(const RoundPlan &p, void *stream, int32_t *host_ends, uint64_t *err_word);
int be_launch_combine(const RoundPlan &p, void *stream);
int be_launch_partial(const RoundPlan &p, int f, void *stream);   // per-stage combine, stage one
int be_launch_last(const RoundPlan &p, int f, void *stream);      // per-stage: the last reply's stage one + stage two
int be_launch_copy(const void *src, void *dst, int64_t bytes, void *stream);
int be_read_error(uint64_t *dev_err, void *stream, int clear, uint64_t *word);
// The one-launch dispatch's gave-up flag (and clears it when asked).
int be_read_stall(uint32_t *dev_sync, void *stream, int clear, int *stalled);
int be_device_sync();
// The current device and the address of its static scratch array (found
// once per device); no allocation.
int be_static_scratch(int *device, void **ptr);
// Initialise a static scratch workspace (the error word) with a kernel on
// the null stream and wait for it; no allocation, no host-to-device copy.
int be_init_static(void *workspace, const WorkspacePlan &wp);

}  // namespace afd
