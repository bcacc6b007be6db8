// afd_kernels.hip -- gfx950 kernels of the AFD dispatch/combine round and the
// HIP executor behind the be_* hooks of afd_plan.h.
//
// What the round computes (afdEP-comm API contract page, "Roles and
// tensors"):
//   dispatch: every live (source, token, k) choice of expert e copies the
//     token's row into partition e/E_loc's expert-major arena.  Expert j of a
//     partition occupies [align_up(ends[j-1], alpha), ends[j]); inside it rows
//     follow (source, token) order.  Invalid ids are skipped and the first
//     offender is recorded (design page, section 8: routes are checked
//     in-kernel before any derived index or store).
//   combine: out[t] = bf16( sum over live k, ascending, of w_k * reply[slot_k] )
//     accumulated in float32 (contract page: routing weight applied exactly
//     once; BF16 result in original token order).
//
// Kernels
//   k_fused   dispatch for small rounds (<= kFusedMaxTokens tokens): every
//             workgroup rebuilds the whole layout in LDS from the ids, then
//             scatters its own token.  One launch for the dispatch.
//   k_layout  dispatch, larger rounds, step 1: tiles of 64, 128 or 256
//             slots of a tiled token space in which every source starts on
//             a tile boundary; per 64-token chunk an LDS bit mask per expert
//             gives each choice its rank (popcount of the lanes below it);
//             writes each tile's count per expert and every choice's rank
//             inside its tile.
//   k_scatter dispatch, step 2: every workgroup sums the tile counts into
//             its tile's first row per expert (and ends[]), then each
//             wavefront copies its tokens' rows once from HBM into registers
//             and stores them to each live slot.
//   k_combine one wavefront per (token, column segment): reads the token's
//             slots with scalar loads, gathers the live reply rows with
//             16-byte loads, float32 multiply-then-add in ascending k,
//             rounds once to bfloat16.
//   k_copy    inbox -> caller output (single-partition collect without view).
//   k_scatter_cached  dispatch of a round that reuses the last layout: the
//             slot map already holds every live choice's partition and row,
//             so each token's row, scales and new weights go straight to
//             their slots (64, 128 or 256 lanes per token by row length).
//   k_partial per-stage combine, stage one (at partition f's reply): one
//             wavefront per (token, column segment) sums the token's live rows
//             of partition f like k_combine, rounds to a BF16 partial and
//             stores it, or its FP8 form (codes plus one power-of-two scale
//             byte per 128 elements, found with a 16-lane max), into the
//             source's partial rows in the workspace.
//   k_last    per-stage combine at the round's last reply: that partition's
//             stage one as in k_partial, then stage two for every source:
//             adds each token's partials in float32, partitions in ascending
//             order of their last live top-k lane, and rounds once to BF16.
//   k_dispatch1  the dispatch as one launch (AFD_DISPATCH_ONE_LAUNCH): the
//             first 32 workgroups count one tile each and publish tagged
//             counts; every other workgroup ranks its own tokens, waits (a
//             bounded poll) for the counts of this launch, and scatters as
//             k_scatter does (design page, section 16: counts first, then
//             the expansion).
//   k_zero_ends, k_init_ws  a round without tokens; a fresh static workspace.
//
// Nothing here uses MFMA: the round is data movement plus one multiply-add
// per reply element, bound by HBM bandwidth.  Expanded rows are written and
// replies read with non-temporal hints: each byte is touched once, and
// keeping them out of the caches stops a round's row writes from evicting
// (and writing back into) the next kernel's working set.

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "afd_plan.h"

// Workspace of the contexts made by afd_create_static: one array per GPU,
// held from the library's first use of the device until the process ends.
// In host code this name is only a stand-in for the device array: host code
// uses the address hipGetSymbolAddress returns for the current device
// (be_static_scratch), never the name itself.
static __device__ __align__(256) unsigned char scratch[afd::kStaticScratchBytes];

namespace afd {
namespace {

constexpr int kWave = 64;

// 16-byte vector as a native clang vector (keeps register arrays in VGPRs).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

// Pointers into global memory.  Accesses through generic pointers become
// flat instructions, which count on both the vector-memory and the LDS
// counters: the compiler then waits for every outstanding load before any
// later use of a flat load, and every LDS wait also waits for flat stores.
template <typename T>
using gptr = __attribute__((address_space(1))) T *;
template <typename T>
using lptr = __attribute__((address_space(3))) T *;

// ---------------------------------------------------------------- args ----

// One record per source, 64 bytes: a kernel reads the record of a source
// it has just identified with a single scalar load.
struct SourceArgs {
    const uint8_t *x;        // [T, row_bytes]
    const float *w;          // [T, K]
    const int32_t *ids;      // [T, K]
    const float *scale;      // FP8 only: scale of (t, block b) at t * sst + b * ssg
    int64_t sst, ssg;
    int32_t off;             // first token of the source in the round's token order
    int32_t T;               // tokens of the source
    int32_t voff;            // first slot of the source in the tiled token space
    int32_t pad;
};

// The scalars of a dispatch, 128 bytes that a kernel reads with two
// 64-byte scalar loads at entry (read field by field, the compiler fetches
// each field where it is first used, one dependent round trip at a time).
struct DispatchHdr {
    int32_t *blkcnt;         // [E][cpitch] tile counts
    int32_t *packed;         // [ntok][K] (expert << 16 | rank in tile), -1 skipped
    int32_t *slot;           // [ntok][K] {part << 24 | row, weight bits}
    int32_t *ends;           // [E]
    uint64_t *err;           // sticky route-error word
    int64_t row_bytes;
    int N, ntok, K, E, E_loc, alpha, nblk, cpitch, nvec, G, fp8, tile;
    uint32_t *tcount;        // one-launch dispatch: [kLayoutMaxTiles][tcount_pitch(E)] tagged tile counts
    uint32_t *sync;          // one-launch dispatch: launch counter, finished workgroups, gave-up flag
    int wait_polls;          // one-launch dispatch: polls before giving up
    int pad;
    uint32_t *ready;         // one-launch dispatch: ready flag copies
};

// Layout tile record, 16 bytes, for rounds of at most kLayoutMaxTiles tiles:
// a layout workgroup reads its tile's record at an address known at entry
// (from its block index alone), in the same batch of scalar loads as the
// header, instead of finding its source first.  Every tile of the tiled
// token space holds at least one token, so n = 0 marks a round without the
// table (more tiles, or the one-kernel dispatch).
struct TileArgs {
    const int32_t *ids;      // ids of the tile's first token
    int32_t g0;              // the tile's first token in the round's order
    int32_t ns;              // tokens of the tile | source << 16
};

struct DispatchArgs {
    DispatchHdr h;
    int voff[kMaxSources];   // first slot of each source in the tiled token space
    SourceArgs src[kMaxSources];
    uint8_t *rows[kMaxParts];
    float *scales[kMaxParts];
    float *roww[kMaxParts];
    int tok_off[kMaxSources + 1];
    TileArgs tiles[kLayoutMaxTiles];
};

// The header as a kernel holds it: the same fields, global pointers.
struct Hdr {
    gptr<int32_t> blkcnt, packed, slot, ends;
    gptr<unsigned long long> err;
    int64_t row_bytes;
    int N, ntok, K, E, E_loc, alpha, nblk, cpitch, nvec, G, fp8, tile;
    gptr<uint32_t> tcount, sync, ready;
    int wait_polls;
};

__device__ __forceinline__ Hdr load_hdr(const DispatchArgs &a, u32x16 &r0, u32x16 &r1)
{
    static_assert(sizeof(DispatchHdr) == 128, "two 64-byte blocks");
    r0 = reinterpret_cast<const u32x16 *>(&a.h)[0];
    r1 = reinterpret_cast<const u32x16 *>(&a.h)[1];
    auto u64 = [&](int i) { return (uint64_t(r0[i + 1]) << 32) | uint64_t(r0[i]); };
    Hdr h;
    h.blkcnt = (gptr<int32_t>)u64(0);
    h.packed = (gptr<int32_t>)u64(2);
    h.slot = (gptr<int32_t>)u64(4);
    h.ends = (gptr<int32_t>)u64(6);
    h.err = (gptr<unsigned long long>)u64(8);
    h.row_bytes = int64_t(u64(10));
    h.N = int(r0[12]);
    h.ntok = int(r0[13]);
    h.K = int(r0[14]);
    h.E = int(r0[15]);
    h.E_loc = int(r1[0]);
    h.alpha = int(r1[1]);
    h.nblk = int(r1[2]);
    h.cpitch = int(r1[3]);
    h.nvec = int(r1[4]);
    h.G = int(r1[5]);
    h.fp8 = int(r1[6]);
    h.tile = int(r1[7]);
    h.tcount = (gptr<uint32_t>)((uint64_t(r1[9]) << 32) | uint64_t(r1[8]));
    h.sync = (gptr<uint32_t>)((uint64_t(r1[11]) << 32) | uint64_t(r1[10]));
    h.wait_polls = int(r1[12]);
    h.ready = (gptr<uint32_t>)((uint64_t(r1[15]) << 32) | uint64_t(r1[14]));
    return h;
}

__device__ __forceinline__ Hdr load_hdr(const DispatchArgs &a)
{
    u32x16 r0, r1;
    return load_hdr(a, r0, r1);
}

// Per-stage combine: partial row of (partition f, source s, token t) at
// partials + ((f * N + s) * capacity + t) * prow.
struct StageArgs {
    const uint16_t *reply;   // stage one: partition f's replies
    uint8_t *partials;
    const int32_t *slot;
    int64_t prow;
    int tok_off[kMaxSources + 1];
    int N, F, ntok, K, H, nvec, nseg, capacity, f;
    uint16_t *outs[kMaxSources];   // stage two: every source's output
};

// The combine's scalars and the first four partitions' reply bases fill the
// first 64 bytes, and the token offsets start at byte 64, so a wavefront
// reads each with one 64-byte scalar load.
struct CombineArgs {
    const int32_t *slot;     // [ntok][K] {part << 24 | row, weight bits}, 64 bytes of slack at the end
    int N, ntok, K, H, nvec, nseg;
    const uint16_t *reply4[4];   // reply[0..3] again (rounds of at most four partitions select from these)
    int tok_off[kMaxSources + 1];
    const uint16_t *reply[kMaxParts];
    uint16_t *out[kMaxSources];
};

// ------------------------------------------------------------- helpers ----
//
// Kernel arguments live in the constant kernarg segment.  Indexing one of
// its arrays with a value that differs between lanes becomes a dependent
// vector load per lane, so kernels index them only with wave-uniform values
// (scalar loads); lanes that need per-lane lookups read small LDS copies.


__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int wave_id() { return uni(threadIdx.x / kWave); }

// Source of global token g from an LDS copy of the token offsets.
__device__ __forceinline__ int src_of_lds(const int *tok_off, int N, int g)
{
    int s = 0;
    for (int q = 1; q < N; ++q) s += g >= tok_off[q] ? 1 : 0;
    return s;
}

// The first tokens of sources 0..15 as one 64-byte scalar load.
__device__ __forceinline__ u32x16 load_offsets(const int (&tok_off)[kMaxSources + 1])
{
    static_assert(kMaxSources == 16, "offsets of every source in one 64-byte load");
    return *reinterpret_cast<const u32x16 *>(tok_off);
}

// Source of global token g for a wave-uniform g, and the source's first
// token: the last source q whose first token is at or before g (offsets are
// nondecreasing; empty sources share their successor's offset).
__device__ __forceinline__ int source_of(const u32x16 &to, int N, int g, int &first)
{
    int s = 0, t0 = 0;
#pragma unroll
    for (int q = 1; q < kMaxSources; ++q)
        if (q < N && g >= int(to[q])) {
            s = q;
            t0 = int(to[q]);
        }
    first = uni(t0);
    return uni(s);
}

// The record of source s (wave-uniform), read as one 64-byte scalar load:
// field by field, the compiler fetches each field where it is first used,
// one dependent scalar round trip at a time.
struct SourceRec {
    const uint8_t *x;
    const float *w;
    const int32_t *ids;
    const float *scale;
    int64_t sst, ssg;
    int off, T, voff;
};

__device__ __forceinline__ SourceRec load_source(const DispatchArgs &a, int s)
{
    static_assert(sizeof(SourceArgs) == 64, "one record per 64 bytes");
    const u32x16 r = reinterpret_cast<const u32x16 *>(a.src)[s];
    auto u64 = [&](int i) { return (uint64_t(r[i + 1]) << 32) | uint64_t(r[i]); };
    SourceRec o;
    o.x = reinterpret_cast<const uint8_t *>(u64(0));
    o.w = reinterpret_cast<const float *>(u64(2));
    o.ids = reinterpret_cast<const int32_t *>(u64(4));
    o.scale = reinterpret_cast<const float *>(u64(6));
    o.sst = int64_t(u64(8));
    o.ssg = int64_t(u64(10));
    o.off = int(r[12]);
    o.T = int(r[13]);
    o.voff = int(r[14]);
    return o;
}

// Source whose span of the tiled token space holds the wave-uniform slot v
// (sources start on tile boundaries; empty sources have empty spans).
__device__ __forceinline__ int source_of_tiled(const DispatchArgs &a, int N, int v)
{
    const u32x16 vo = *reinterpret_cast<const u32x16 *>(a.voff);
    int s = 0;
#pragma unroll
    for (int q = 1; q < kMaxSources; ++q) s += (q < N && v >= int(vo[q])) ? 1 : 0;
    return uni(s);
}

__device__ __forceinline__ uint64_t make_err(int s, int t, int k, unsigned code)
{
    return (uint64_t(s) << 56) | (uint64_t(uint32_t(t)) << 24) | (uint64_t(k) << 16) | uint64_t(code);
}

// s_waitcnt immediate that waits for the vector memory counter alone to
// reach zero (expcnt and lgkmcnt fields at their maximum).
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ int align_up_i(int v, int a) { return (v + a - 1) / a * a; }

// x / d for x >= 0, d >= 1, with a shift when d is a power of two (the
// common case for the wave-uniform sizes it divides)
__device__ __forceinline__ int div_pow2_or(int x, int d)
{
    return (d & (d - 1)) == 0 ? x >> __builtin_ctz(uint32_t(d)) : x / d;
}

// Partition of expert e (0 <= e < 2^19; experts number at most 512) with
// E_loc experts per partition, without an integer division.  (e + 1/2) /
// E_loc lies at least 1/(2 E_loc) from every integer; the float product with
// the hardware reciprocal (1 ulp) is off by less than (e + 1/2) / E_loc *
// 2^-21, which is smaller, so truncating it gives floor(e / E_loc).
__device__ __forceinline__ int part_of(int e, int E_loc)
{
    return int((float(e) + 0.5f) * __builtin_amdgcn_rcpf(float(E_loc)));
}

// Workgroup barrier that orders LDS only.  __syncthreads() is a full
// workgroup fence: it waits for every outstanding global load and store of
// the wave (the vector-memory counter), which would stall on row loads and
// store acknowledgements that the LDS phase does not need.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 64 lanes of a wavefront: DPP row shifts by
// 1, 2, 4, 8 inside each 16-lane row, then lane 15 of each row added into
// the next row (rows 1, 3) and lane 31 into rows 2, 3.  Lanes without a
// source lane read 0.
__device__ __forceinline__ int wave_inclusive_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Exclusive prefix sum of vals[0..n) (LDS, visible to the block), in place.
// Wavefront 0 does it alone, lane l owning ceil(n / 64) consecutive entries;
// one barrier then publishes the result to the block.
__device__ void block_exclusive_scan(int *vals, int n)
{
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        const int per = (n + kWave - 1) / kWave;
        const int lo = lane * per;
        const int hi = lo + per < n ? lo + per : n;
        int sum = 0;
        for (int i = lo; i < hi; ++i) sum += vals[i];
        int run = wave_inclusive_scan(sum) - sum;
        for (int i = lo; i < hi; ++i) {
            const int v = vals[i];
            vals[i] = run;
            run += v;
        }
    }
    lds_barrier();
}

// Copy of a kernel-argument pointer array into LDS (thread 0, constant
// offsets), so lanes can look entries up by their own index.
template <typename T, int M>
__device__ __forceinline__ void table_to_lds(uint64_t *dst, T *const (&arr)[M])
{
#pragma unroll
    for (int q = 0; q < M; ++q) dst[q] = reinterpret_cast<uint64_t>(arr[q]);
}

// Route rule of the contract page for one token's ids ev[0..KMAX), where
// entries past K hold -1: -1 skips; other negatives, ids >= E and repeats of
// an earlier valid id are errors and are skipped too.  Returns the bit set
// of live choices; a token that breaks the rule also records its first error
// (lowest k) in `err`.  Repeats are found by comparing with the earlier ids
// in registers.  The common case (every id valid or -1) is compares and
// selects only; the error word is built only for a lane that needs it.
template <int KMAX>
__device__ __forceinline__ uint32_t classify_token(const int (&ev)[KMAX], int E, int s, int t, uint64_t &err)
{
    uint32_t live = 0;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int e = ev[k];
        bool dup = false;
#pragma unroll
        for (int j = 0; j < k; ++j) dup |= ev[j] == e;
        const bool ok = uint32_t(e) < uint32_t(E) && !dup;
        live |= ok ? (1u << k) : 0u;
        bad |= !ok && e != -1;
    }
    if (bad) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int e = ev[k];
            bool dup = false;
#pragma unroll
            for (int j = 0; j < k; ++j) dup |= ev[j] == e;
            const unsigned code = e < -1 ? unsigned(AFD_ROUTE_NEG)
                                  : e >= E ? unsigned(AFD_ROUTE_RANGE)
                                  : (e >= 0 && dup) ? unsigned(AFD_ROUTE_DUP) : 0u;
            if (code != 0 && err == kNoError) err = make_err(s, t, k, code);
        }
    }
    return live;
}

// The route check's common case without pairwise compares: at most eight
// ids per token and E <= 248.  The ids go into two 32-bit words, one byte
// each, a skipped choice (-1) as byte 248 + k, which equals neither an id
// nor another skip; two equal ids are then a zero byte in the XOR of a word
// with a byte rotation of itself or of the other word (eight such XORs
// cover all 28 pairs).  Returns true, with the live set, when every id is
// in [-1, E) and no id repeats; otherwise classify_token decides.  As SGPR
// lane masks the 28 compares form a dependent chain of scalar ORs; here it
// is about forty independent vector operations.
template <int KMAX>
__device__ __forceinline__ bool routes_plain(const int (&ev)[KMAX], int E, uint32_t &live)
{
    if (KMAX != 8 || E > 248) return false;
    // e + 1 is 0 for a skip and in [1, E] for a valid id; anything else
    // (below -1 or at least E) makes the largest e + 1 exceed E
    uint32_t w0 = 0, w1 = 0, lv = 0, mx = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const uint32_t e1 = uint32_t(ev[k]) + 1u;
        mx = e1 > mx ? e1 : mx;
        lv |= e1 != 0u ? (1u << k) : 0u;
        const uint32_t b = (e1 != 0u ? e1 - 1u : 248u + uint32_t(k)) << (8 * (k & 3));
        if (k < 4) w0 |= b;
        else w1 |= b;
    }
    const uint32_t odd = mx > uint32_t(E) ? 1u : 0u;
    auto rot = [](uint32_t v, int r) { return (v << r) | (v >> (32 - r)); };
    auto zb = [](uint32_t v) { return (v - 0x01010101u) & ~v & 0x80808080u; };   // nonzero iff a byte is 0
    const uint32_t z = zb(w0 ^ rot(w0, 8)) | zb(w0 ^ rot(w0, 16)) | zb(w1 ^ rot(w1, 8)) | zb(w1 ^ rot(w1, 16)) |
                       zb(w0 ^ w1) | zb(w0 ^ rot(w1, 8)) | zb(w0 ^ rot(w1, 16)) | zb(w0 ^ rot(w1, 24));
    live = lv;
    return (z | odd) == 0;
}

// ------------------------------------------------------------- kernels ----

// Token gg's KMAX ids from the round's id array in LDS (entries past K are
// -1); one 16-byte read per four ids when K is a multiple of four, since a
// token's ids are then 16-byte aligned.
template <int KMAX>
__device__ __forceinline__ void token_ids_lds(const int *sids, int gg, int K, int (&ev)[KMAX])
{
    if ((K & 3) == 0) {
#pragma unroll
        for (int q = 0; q < KMAX / 4; ++q) {
            u32x4 v4 = u32x4{~0u, ~0u, ~0u, ~0u};
            if (4 * q < K) v4 = reinterpret_cast<const u32x4 *>(sids + gg * K)[q];
            ev[4 * q] = int(v4.x);
            ev[4 * q + 1] = int(v4.y);
            ev[4 * q + 2] = int(v4.z);
            ev[4 * q + 3] = int(v4.w);
        }
    } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int val = sids[gg * K + (k < K ? k : K - 1)];
            ev[k] = k < K ? val : -1;
        }
    }
}

// Dispatch in one kernel for small rounds (at most kFusedMaxTokens tokens,
// kFusedMaxIds ids, kFusedMaxExperts experts).  Block g scatters token g,
// each thread holding up to VMAX 16-byte columns of the row.  The row, the
// token's weights and scales and every id of the round are requested at
// entry.  The block then needs two histograms of the round's live choices:
// over all tokens (for the aligned starts of every expert) and over the
// tokens before g (the rank of g's row inside each of its experts, since a
// token holds an expert at most once):
//   row(g, e) = start_e + #{live choices of e in tokens before g}.
// Both are kept in one LDS word per expert (all tokens in the low 16 bits,
// earlier tokens in the high 16), so each choice costs one atomic.  The
// leading scalar arguments (the first two sources' rows, ids and token
// counts, K and nvec) are preloaded into SGPRs by the hardware.  Three forms:
//   kFusedAny  any number of sources: every id of the round is copied
//              straight into LDS (global_load_lds) after the row, and the
//              first barrier waits for every load;
//   kFusedFew  at most two sources: the same, with the row and the ids
//              addressed from the preloaded arguments alone, so they are
//              requested before any load from the argument block returns;
//   kFusedReg  at most two sources, K = 8 and 16-byte aligned ids: every
//              thread loads its two tokens' ids (tid and tid + 256, clamped
//              to the round) into registers and lane k of every wavefront
//              loads token g's id k, so no id passes through LDS.  Every
//              load is unconditional, with in-bounds indices, so the
//              counting waits for the ids alone, not for the row or the
//              weights (whose address comes from the argument block), and
//              the barriers order LDS only.
constexpr int kFusedAny = 0, kFusedFew = 1, kFusedReg = 2;

template <int VMAX, int KMAX, int MODE>
__global__ __launch_bounds__(256) void k_fused(const uint8_t *px0, const uint8_t *px1, const int32_t *pids0,
                                               const int32_t *pids1, int pT0, int pT1, int pK, int pnvec,
                                               DispatchArgs a)
{
    constexpr bool FEW = MODE != kFusedAny, REG = MODE == kFusedReg;
    static_assert(!REG || KMAX == 8, "register ids: eight per token");
    static_assert(kFusedMaxTokens == 512, "register ids: two tokens per thread");
    extern __shared__ __align__(16) unsigned char lds[];
    __shared__ int s_off[kMaxSources + 1];
    __shared__ uint32_t s_live, s_slow;
    __shared__ uint64_t s_prow[kMaxParts], s_pw[kMaxParts], s_ps[kMaxParts];
    // per expert (+ spare): all | before << 16; aligned counts, then their
    // exclusive prefix
    __shared__ int hist[kFusedMaxExperts + 1], pfx[kFusedMaxExperts];
    int *sids = reinterpret_cast<int *>(lds);   // [ntok * K] (not REG; first: 16-byte aligned)
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
    const int g = blockIdx.x;

    // 1. request every load: ids, row, weights, scales
    auto ids_to_lds = [&](const int32_t *qids, int lo, int n, int K) {
        const gptr<const int32_t> src = (gptr<const int32_t>)qids;
        if ((K & 3) == 0 && (reinterpret_cast<uintptr_t>(qids) & 15u) == 0) {
            // 16 bytes per lane: a wavefront moves 256 ids per instruction
            for (int base = wave * 4 * kWave; base < n; base += 16 * kWave)
                if (base + 4 * lane < n)
                    __builtin_amdgcn_global_load_lds((gptr<void>)(src + base + 4 * lane), (lptr<void>)(sids + lo + base),
                                                     16, 0, 0);
        } else {
            for (int base = wave * kWave; base < n; base += 256)
                if (base + lane < n)
                    __builtin_amdgcn_global_load_lds((gptr<void>)(src + base + lane), (lptr<void>)(sids + lo + base), 4,
                                                     0, 0);
        }
    };
    auto row_loads = [&](u32x4 (&v)[VMAX], const uint8_t *xrow, int nvec) {
        const gptr<const u32x4> xs = (gptr<const u32x4>)xrow;
#pragma unroll
        for (int i = 0; i < VMAX; ++i) {
            const int c = tid + i * 256;
            if (c < nvec) v[i] = xs[c];
        }
    };
    u32x4 v[VMAX];
    int s, t0;
    bool mine;
    int ev0[KMAX], ev1[KMAX];                   // REG: tokens tid and tid + 256
    int eg = -1;                                // REG: token g's id `lane` (lanes < 8)
    if constexpr (FEW) {
        mine = g < pT0 + pT1;
        s = g < pT0 ? 0 : 1;
        t0 = s ? pT0 : 0;
        if constexpr (REG) {
            // one block per token of the round (mine), K = 8
            const int nt = pT0 + pT1;
            auto tok = [&](int gg) {
                return (gptr<const u32x4>)((gg < pT0 ? pids0 + int64_t(gg) * 8 : pids1 + int64_t(gg - pT0) * 8));
            };
            const gptr<const u32x4> p0 = tok(tid < nt ? tid : nt - 1);
            const gptr<const u32x4> p1 = tok(tid + 256 < nt ? tid + 256 : nt - 1);
            const u32x4 a0 = p0[0], a1 = p0[1], b0 = p1[0], b1 = p1[1];
            eg = ((gptr<const int32_t>)tok(g))[lane < 8 ? lane : 0];
            ev0[0] = int(a0.x), ev0[1] = int(a0.y), ev0[2] = int(a0.z), ev0[3] = int(a0.w);
            ev0[4] = int(a1.x), ev0[5] = int(a1.y), ev0[6] = int(a1.z), ev0[7] = int(a1.w);
            ev1[0] = int(b0.x), ev1[1] = int(b0.y), ev1[2] = int(b0.z), ev1[3] = int(b0.w);
            ev1[4] = int(b1.x), ev1[5] = int(b1.y), ev1[6] = int(b1.z), ev1[7] = int(b1.w);
            const gptr<const u32x4> xs = (gptr<const u32x4>)((s ? px1 : px0) + int64_t(g - t0) * pnvec * 16);
#pragma unroll
            for (int i = 0; i < VMAX; ++i) {
                const int c = tid + i * 256;
                v[i] = xs[c < pnvec ? c : 0];
            }
        } else {
            if (mine) row_loads(v, (s ? px1 : px0) + int64_t(g - t0) * pnvec * 16, pnvec);
            ids_to_lds(pids0, 0, pT0 * pK, pK);
            if (pT1 > 0) ids_to_lds(pids1, pT0 * pK, pT1 * pK, pK);
        }
    }
    const Hdr h = load_hdr(a);
    const int E = h.E, K = h.K, ntok = h.ntok, G = h.G, N = h.N;
    if constexpr (!FEW) {
        mine = g < ntok;
        s = source_of(load_offsets(a.tok_off), N, mine ? g : 0, t0);
        const SourceRec sx = load_source(a, s);
        if (mine) row_loads(v, sx.x + int64_t(g - t0) * h.row_bytes, h.nvec);
    }
    const SourceRec src = load_source(a, s);
    const int t = g - t0;
    float wk = 0.0f;
    float scv = 0.0f;
    const bool myscale = mine && h.fp8 && tid < G;
    if constexpr (REG) {
        // unconditional, in bounds: BF16 rounds point the scale load at the
        // token's weights, whose value is not used
        wk = ((gptr<const float>)src.w)[int64_t(t) * K + (tid < K ? tid : 0)];
        const bool fp8 = h.fp8 != 0;
        const float *sbase = fp8 ? src.scale : src.w;
        const int64_t sst = fp8 ? src.sst : int64_t(K);
        const int64_t sgl = fp8 ? int64_t(tid < G ? tid : 0) * src.ssg : 0;
        scv = ((gptr<const float>)sbase)[int64_t(t) * sst + sgl];
    } else {
        if (mine && tid < K) wk = ((gptr<const float>)src.w)[int64_t(t) * K + tid];
        if (myscale) scv = ((gptr<const float>)src.scale)[int64_t(t) * src.sst + int64_t(tid) * src.ssg];
    }
    if constexpr (!FEW) {
        for (int q = 0; q < N; ++q) {
            const SourceRec rq = load_source(a, q);
            ids_to_lds(rq.ids, rq.off * K, rq.T * K, K);
        }
    }
    // pointer tables, one per wavefront (lane 0)
    if (lane == 0) {
        if (wave == 0) table_to_lds(s_prow, a.rows);
        if (wave == 1) table_to_lds(s_pw, a.roww);
        if (wave == 2) table_to_lds(s_ps, a.scales);
        if (wave == 3 && blockIdx.x == 0)
            for (int q = 0; q <= N; ++q) s_off[q] = a.tok_off[q];
    }
    for (int i = tid; i < E + 1; i += 256) hist[i] = 0;
    if (tid == 0) s_slow = 0u;
    if constexpr (REG) lds_barrier();
    else __syncthreads();

    // 2. route check and the two histograms (choices that are not live
    // count into the spare slot at index E).  Tokens that pass the
    // compare-free check count at once; the others (repeats, invalid ids,
    // E > 248) are counted in a second pass that only a block holding such
    // a token runs, so the common round carries none of its code.
    auto count = [&](int gg, const int (&e)[KMAX], uint32_t live) {
        const int inc = gg < g ? 0x10001 : 1;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) atomicAdd(&hist[((live >> k) & 1u) ? e[k] : E], inc);
        if (gg == g) s_live = live;
    };
    uint32_t failed = 0;             // bit i: this thread's i-th token needs the second pass
    if constexpr (REG) {
        uint32_t live;
        if (tid < ntok) {
            if (routes_plain<KMAX>(ev0, E, live)) count(tid, ev0, live);
            else failed = 1u;
        }
        if (tid + 256 < ntok) {
            if (routes_plain<KMAX>(ev1, E, live)) count(tid + 256, ev1, live);
            else failed |= 2u;
        }
    } else {
        for (int gg = tid, i = 0; gg < ntok; gg += 256, ++i) {
            int e[KMAX];
            token_ids_lds<KMAX>(sids, gg, K, e);
            uint32_t live;
            if (routes_plain<KMAX>(e, E, live)) count(gg, e, live);
            else failed |= 1u << i;
        }
    }
    if (failed != 0) s_slow = 1u;
    lds_barrier();
    if (s_slow != 0u) {
        uint64_t err = kNoError;
        for (int gg = tid, i = 0; gg < ntok; gg += 256, ++i) {
            if (((failed >> i) & 1u) == 0u) continue;
            int e[KMAX];
            if constexpr (REG) {
#pragma unroll
                for (int k = 0; k < KMAX; ++k) e[k] = i == 0 ? ev0[k] : ev1[k];
            } else {
                token_ids_lds<KMAX>(sids, gg, K, e);
            }
            int ss = 0, tt = 0;
            if (blockIdx.x == 0) {
                ss = src_of_lds(s_off, N, gg);
                tt = gg - s_off[ss];
            }
            count(gg, e, classify_token<KMAX>(e, E, ss, tt, err));
        }
        if (blockIdx.x == 0 && err != kNoError)
            __hip_atomic_fetch_min(h.err, err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lds_barrier();
    }

    // 3. aligned starts: pfx[e] = sum of aligned counts of experts < e (all
    // partitions); expert e starts at pfx[e] - pfx[first expert of its part].
    // Wavefront 0 reads the counts in one batch (in-bounds indices, E <= 256:
    // at most 4 experts per lane), aligns them (a mask for a power-of-two
    // alignment) and scans them, then one barrier.
    if (wave == 0) {
        const int per = (E + kWave - 1) / kWave;
        const int lo = lane * per;
        int c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = hist[lo + i < E ? lo + i : E] & 0xFFFF;
        const int al = h.alpha;
        const bool pow2 = (al & (al - 1)) == 0;
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int up = pow2 ? (c[i] + al - 1) & -al : align_up_i(c[i], al);
            c[i] = i < per && lo + i < E ? up : 0;
            sum += c[i];
        }
        int run = wave_inclusive_scan(sum) - sum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < per && lo + i < E) pfx[lo + i] = run;
            run += c[i];
        }
    }
    lds_barrier();
    if (!mine) return;                          // (never block 0: a round here has a token)

    // 4. slot of choice k: lane k of every wavefront computes it (those of
    // wavefront 0 also write the slot map and the row weight); the stores
    // below take each wavefront's own addresses by lane broadcast
    uint64_t d = 0, ds = 0;
    int packed = -1;
    if (lane < K && ((s_live >> lane) & 1u)) {
        const int e = REG ? eg : sids[g * K + lane];
        const int part = part_of(e, h.E_loc);
        const int row = pfx[e] - pfx[part * h.E_loc] + (hist[e] >> 16);
        packed = (part << 24) | row;
        d = s_prow[part] + uint64_t(row) * uint64_t(h.row_bytes);
        ds = s_ps[part] + uint64_t(row) * uint64_t(G) * 4u;
        if (wave == 0) ((gptr<float>)s_pw[part])[row] = wk;
    }
    if (wave == 0 && lane < K) {
        i32x2 sl;
        sl.x = packed;
        sl.y = __float_as_int(wk);
        ((gptr<i32x2>)h.slot)[int64_t(g) * K + lane] = sl;
    }

    // 5. stores: the row to every live slot, and the FP8 scales
    const int dlo = int(uint32_t(d)), dhi = int(uint32_t(d >> 32));
    const int slo = int(uint32_t(ds)), shi = int(uint32_t(ds >> 32));
    for (int k = 0; k < K; ++k) {
        const uint64_t dk = uint64_t(uint32_t(__builtin_amdgcn_readlane(dlo, k))) |
                            (uint64_t(uint32_t(__builtin_amdgcn_readlane(dhi, k))) << 32);
        if (dk == 0) continue;
        const gptr<u32x4> dst = (gptr<u32x4>)dk;
#pragma unroll
        for (int i = 0; i < VMAX; ++i) {
            const int c = tid + i * 256;
            if (c < h.nvec) __builtin_nontemporal_store(v[i], &dst[c]);
        }
        if (myscale) {
            const uint64_t sk = uint64_t(uint32_t(__builtin_amdgcn_readlane(slo, k))) |
                                (uint64_t(uint32_t(__builtin_amdgcn_readlane(shi, k))) << 32);
            ((gptr<float>)sk)[tid] = scv;
        }
    }
    // ends, once the rows are on their way (nothing in this kernel waits
    // for them)
    if (blockIdx.x == 0)
        for (int e = tid; e < E; e += 256) h.ends[e] = pfx[e] - pfx[part_of(e, h.E_loc) * h.E_loc] + (hist[e] & 0xFFFF);
}

// Tile histogram of larger rounds.  Block = NW wavefronts = one tile of
// 64 * NW slots of the tiled token space (all of one source), lane = token.
// blkcnt[e][tile] = live choices of expert e in the tile; packed[g][k] =
// (expert << 16) | rank of the choice among the tile's choices of that
// expert (token order), or -1.  Tiles follow (source, token) order, so
// adding the counts of earlier tiles ranks a choice within its expert.
template <int KMAX, int NW>
__global__ __launch_bounds__(NW * 64) void k_layout(DispatchArgs a)
{
    static_assert(sizeof(TileArgs) == 16, "one tile record per 16 bytes");
    const u32x4 tr = reinterpret_cast<const u32x4 *>(a.tiles)[blockIdx.x < kLayoutMaxTiles ? blockIdx.x : 0];
    const Hdr h = load_hdr(a);
    // the header's second half with the first batch of scalar loads, not
    // after the ids arrive (where its first uses are)
    asm volatile("" ::"s"(h.cpitch));
    extern __shared__ __align__(16) unsigned char lds[];
    const int E = h.E, K = h.K;
    constexpr int TILE = NW * kWave;
    // per wavefront, a lane mask per expert and one spare word per lane
    // (choices that are not live mark their lane's own spare, so they never
    // contend for one address)
    const int MS = E + kWave;
    unsigned long long *mask = reinterpret_cast<unsigned long long *>(lds);  // [NW][E + 64]
    int *pre = reinterpret_cast<int *>(mask + size_t(NW) * MS);               // [NW][E]
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    // the tile lies in one source's span of the tiled token space: its
    // first token's ids, its token count and its first token in the round
    int s, n_tile, g_first;
    const int32_t *ids_first;
    if ((tr.w & 0xFFFFu) != 0) {
        ids_first = reinterpret_cast<const int32_t *>((uint64_t(tr.y) << 32) | uint64_t(tr.x));
        g_first = int(tr.z);
        n_tile = int(tr.w & 0xFFFFu);
        s = int(tr.w >> 16);
    } else {
        s = source_of_tiled(a, h.N, blockIdx.x * TILE);
        const SourceRec src = load_source(a, s);
        const int t_first = blockIdx.x * TILE - src.voff;
        ids_first = src.ids + int64_t(t_first) * K;
        g_first = src.off + t_first;
        n_tile = src.T - t_first;
    }
    const bool have = tid < n_tile;
    const int g = g_first + tid;                           // the lane's token in the round's order

    int ev[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) ev[k] = -1;
    if (have) {
        // 16-byte loads when the token's ids are 16-byte aligned (fewer
        // memory instructions on the layout's critical path)
        const gptr<const int32_t> idp = (gptr<const int32_t>)ids_first + int64_t(tid) * K;
        if ((K & 3) == 0 && (reinterpret_cast<uintptr_t>(idp) & 15u) == 0) {
#pragma unroll
            for (int q = 0; q < KMAX / 4; ++q) {
                u32x4 v4 = u32x4{~0u, ~0u, ~0u, ~0u};
                if (4 * q < K) v4 = ((gptr<const u32x4>)idp)[q];
                ev[4 * q] = int(v4.x);
                ev[4 * q + 1] = int(v4.y);
                ev[4 * q + 2] = int(v4.z);
                ev[4 * q + 3] = int(v4.w);
            }
        } else {
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                const int val = idp[k < K ? k : K - 1];
                ev[k] = k < K ? val : -1;
            }
        }
    }
    for (int i = tid; i < NW * MS; i += TILE) mask[i] = 0ull;
    lds_barrier();
    uint32_t live = 0;
    {
        uint64_t err = kNoError;
        if (!routes_plain<KMAX>(ev, E, live))
            live = classify_token<KMAX>(ev, E, s, g - a.tok_off[s], err);   // token index used only for an error
        if (err != kNoError) __hip_atomic_fetch_min(h.err, err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // mark the token's lane bit per live expert (others into the lane's spare)
        unsigned long long *mrow = mask + size_t(wave) * MS;
        const unsigned long long bit = 1ull << lane;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) atomicOr(&mrow[((live >> k) & 1u) ? ev[k] : E + lane], bit);
    }
    lds_barrier();
    for (int e = tid; e < E; e += TILE) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            pre[w * E + e] = run;
            run += __popcll(mask[w * MS + e]);
        }
        h.blkcnt[e * h.cpitch + blockIdx.x] = run;
    }
    lds_barrier();
    if (have) {
        const unsigned long long below = (1ull << lane) - 1ull;
        const unsigned long long *mrow = mask + size_t(wave) * MS;
        const gptr<int32_t> pk = h.packed + int64_t(g) * K;
        int vals[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const bool l = (live >> k) & 1u;
            const int e = l ? ev[k] : 0;
            vals[k] = l ? ((e << 16) | (pre[wave * E + e] + __popcll(mrow[e] & below))) : -1;
        }
        if ((K & 3) == 0) {          // packed is 256-byte aligned, so each token's row is 16-byte aligned
#pragma unroll
            for (int q = 0; q < KMAX / 4; ++q)
                if (4 * q < K)
                    ((gptr<u32x4>)pk)[q] = u32x4{uint32_t(vals[4 * q]), uint32_t(vals[4 * q + 1]),
                                                 uint32_t(vals[4 * q + 2]), uint32_t(vals[4 * q + 3])};
        } else {
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (k < K) pk[k] = vals[k];
        }
    }
}

// Scatter of larger rounds.  Block = 4 wavefronts; wavefront w handles the
// W = 4 / VMAX (at least 1) consecutive slots of the tiled token space
// starting at block_first + w * W (a block's slots lie in one layout tile,
// so all its tokens come from one source).  Small blocks put several on
// each CU, which keeps more stores in flight per CU.  Every block turns the
// tile counts into this tile's first row per expert itself:
//   base[e] = start_e + sum of counts of e in earlier tiles,
//   start_e = aligned prefix of the partition's experts before e,
// which needs no communication between blocks.  The tile counts are
// requested first and the rows, ranks and weights right after, so the scan
// (LDS-only barriers) runs while the rows are still in flight.
template <int VMAX>
__global__ __launch_bounds__(256) void k_scatter(DispatchArgs a)
{
    const Hdr h = load_hdr(a);
    constexpr int W = VMAX >= 4 ? 1 : 4 / VMAX;     // tokens per wavefront (1 KB .. 4 KB of row per lane set)
    constexpr int TB = 4 * W;
    constexpr int PRE = 32;                     // tile counts of its expert a thread requests at entry
    extern __shared__ __align__(16) unsigned char lds[];
    __shared__ uint64_t s_prow[kMaxParts], s_pw[kMaxParts], s_ps[kMaxParts];
    const int E = h.E, K = h.K, nvec = h.nvec, nblk = h.nblk;
    int *base = reinterpret_cast<int *>(lds);   // [E]
    int *A = base + E;                          // [E]
    int *Cs = A + E;                            // [E]
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
    const int v_first = blockIdx.x * TB;        // first slot of the tiled token space
    const int tile = v_first / h.tile;
    const SourceRec src = load_source(a, source_of_tiled(a, h.N, v_first));
    const int T_s = src.T;
    const int t_first = v_first - src.voff + wave * W;    // source token of the wavefront's first slot
    const int g_src = src.off;
    const bool pre_all = nblk <= PRE;

    // 1. tile counts first (thread e: expert e's run of counts, 16 bytes
    // per load, every load unconditional with an in-bounds index), then the
    // rows, ranks, weights and scales of this wavefront's tokens.  Nothing
    // loaded is examined before the sums below, which wait for the counts
    // alone; the rows stay in flight through the scan.
    u32x4 cv4[PRE / 4];
    {
        const gptr<const u32x4> cp = (gptr<const u32x4>)(h.blkcnt + int64_t(tid < E ? tid : 0) * h.cpitch);
        const int nq = h.cpitch / 4;
#pragma unroll
        for (int q = 0; q < PRE / 4; ++q) cv4[q] = cp[q < nq ? q : 0];
    }
    // keep the count loads ahead of the row loads: the vector memory
    // counter completes in issue order, so a row load moved before them
    // would delay the sums by a cold row fetch
    __builtin_amdgcn_sched_barrier(0);
    u32x4 v[W][VMAX];
    int pk[W];
    float wk[W];
    float scv[W];                               // FP8: scale of block `lane` of each token
    // Slots past the source's last token load that token again (T_s >= 1:
    // a workgroup lies in a non-empty source's span) and store nothing.
    // BF16 rounds point the scale load at the token's weights, a valid
    // address whose value is not used.
    {
        const int kl = lane < K ? lane : 0;
        const bool fp8 = h.fp8 != 0;
        const float *sbase = fp8 ? src.scale : src.w;
        const int64_t sst = fp8 ? src.sst : int64_t(K);
        const int64_t sgl = fp8 ? int64_t(lane < h.G ? lane : 0) * src.ssg : 0;
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const int t = t_first + j < T_s ? t_first + j : T_s - 1;
            const gptr<const u32x4> xs = (gptr<const u32x4>)(src.x + int64_t(t) * h.row_bytes);
#pragma unroll
            for (int i = 0; i < VMAX; ++i) {
                const int c = i * kWave + lane;
                v[j][i] = xs[c < nvec ? c : 0];
            }
            pk[j] = h.packed[int64_t(g_src + t) * K + kl];
            wk[j] = ((gptr<const float>)src.w)[int64_t(t) * K + kl];
            scv[j] = ((gptr<const float>)sbase)[int64_t(t) * sst + sgl];
        }
    }
    if (lane == 0) {
        if (wave == 0) table_to_lds(s_prow, a.rows);
        if (wave == 1) table_to_lds(s_pw, a.roww);
        if (wave == 2) table_to_lds(s_ps, a.scales);
    }

    // 2. this tile's first row of every expert
    for (int e = tid; e < E; e += 256) {
        int C = 0, before = 0;
        if (e == tid && pre_all) {
#pragma unroll
            for (int q = 0; q < PRE / 4; ++q) {
                const int c4[4] = {int(cv4[q].x), int(cv4[q].y), int(cv4[q].z), int(cv4[q].w)};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int b = 4 * q + i;
                    const int c = b < nblk ? c4[i] : 0;
                    C += c;
                    before += b < tile ? c : 0;
                }
            }
        } else {
            const gptr<const int32_t> cp = (gptr<const int32_t>)h.blkcnt + int64_t(e) * h.cpitch;
            for (int b = 0; b < nblk; ++b) {
                const int c = cp[b];
                C += c;
                before += b < tile ? c : 0;
            }
        }
        A[e] = align_up_i(C, h.alpha);
        Cs[e] = C;
        base[e] = before;
    }
    lds_barrier();
    block_exclusive_scan(A, E);
    for (int e = tid; e < E; e += 256) {
        const int start = A[e] - A[(e / h.E_loc) * h.E_loc];
        base[e] += start;
        if (blockIdx.x == 0) h.ends[e] = start + Cs[e];
    }
    lds_barrier();
    // Every row, rank, weight and scale of the wavefront's tokens was
    // requested at entry: wait for all of them here, once.  The vector
    // memory counter also counts stores on this GPU, so a wait for one of
    // these loads placed after a token's stores (the compiler cannot count
    // stores issued in a loop) would also wait for those stores to be
    // acknowledged, serialising the tokens of a wavefront.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // 3. slots and stores, token by token; lane k owns choice k and the
    // address of its row, which the store loop broadcasts
#pragma unroll
    for (int j = 0; j < W; ++j) {
        const int t = t_first + j;
        if (t >= T_s) break;                    // the rest of the wavefront's slots are empty
        const int g = g_src + t;
        int part = -1, row = -1;
        uint64_t d = 0, ds = 0;
        const int pkj = lane < K ? pk[j] : -1;
        if (pkj >= 0) {
            const int e = pkj >> 16;
            row = base[e] + (pkj & 0xFFFF);
            part = e / h.E_loc;
            d = s_prow[part] + uint64_t(row) * uint64_t(h.row_bytes);
            ds = s_ps[part] + uint64_t(row) * uint64_t(h.G) * 4u;
            ((gptr<float>)s_pw[part])[row] = wk[j];
        }
        if (lane < K) {
            i32x2 sl;
            sl.x = part < 0 ? -1 : ((part << 24) | row);
            sl.y = __float_as_int(wk[j]);
            ((gptr<i32x2>)h.slot)[int64_t(g) * K + lane] = sl;
        }
        const int dlo = int(uint32_t(d)), dhi = int(uint32_t(d >> 32));
        for (int k = 0; k < K; ++k) {
            const uint64_t dk = uint64_t(uint32_t(__builtin_amdgcn_readlane(dlo, k))) |
                                (uint64_t(uint32_t(__builtin_amdgcn_readlane(dhi, k))) << 32);
            if (dk == 0) continue;
            const gptr<u32x4> dst = (gptr<u32x4>)dk;
#pragma unroll
            for (int i = 0; i < VMAX; ++i) {
                const int c = i * kWave + lane;
                if (c < nvec) __builtin_nontemporal_store(v[j][i], &dst[c]);
            }
        }
        // rows longer than 64 * VMAX columns: the remaining columns, chunk by chunk
        if (nvec > kWave * VMAX) {
            const gptr<const u32x4> xs = (gptr<const u32x4>)(src.x + int64_t(t) * h.row_bytes);
            for (int cb = kWave * VMAX; cb < nvec; cb += kWave * VMAX) {
                u32x4 r[VMAX];
#pragma unroll
                for (int i = 0; i < VMAX; ++i) {
                    const int c = cb + i * kWave + lane;
                    if (c < nvec) r[i] = xs[c];
                }
                for (int k = 0; k < K; ++k) {
                    const uint64_t dk = uint64_t(uint32_t(__builtin_amdgcn_readlane(dlo, k))) |
                                        (uint64_t(uint32_t(__builtin_amdgcn_readlane(dhi, k))) << 32);
                    if (dk == 0) continue;
                    const gptr<u32x4> dst = (gptr<u32x4>)dk;
#pragma unroll
                    for (int i = 0; i < VMAX; ++i) {
                        const int c = cb + i * kWave + lane;
                        if (c < nvec) __builtin_nontemporal_store(r[i], &dst[c]);
                    }
                }
            }
        }
        if (h.fp8) {
            const int G = h.G;
            const int slo = int(uint32_t(ds)), shi = int(uint32_t(ds >> 32));
            if (lane < G) {
                for (int k = 0; k < K; ++k) {
                    const uint64_t sk = uint64_t(uint32_t(__builtin_amdgcn_readlane(slo, k))) |
                                        (uint64_t(uint32_t(__builtin_amdgcn_readlane(shi, k))) << 32);
                    if (sk == 0) continue;
                    ((gptr<float>)sk)[lane] = scv[j];
                }
            }
            if (G > kWave) {
                // rows of more than 64 scale blocks (H > 8192): the other
                // blocks are loaded here, and waited for before leaving, so
                // that no load is left pending into the next token's stores
                const gptr<const float> sc = (gptr<const float>)src.scale + int64_t(t) * src.sst;
                for (int b = kWave + lane; b < G; b += kWave) {
                    const float val = sc[int64_t(b) * src.ssg];
                    for (int k = 0; k < K; ++k) {
                        const uint64_t sk = uint64_t(uint32_t(__builtin_amdgcn_readlane(slo, k))) |
                                            (uint64_t(uint32_t(__builtin_amdgcn_readlane(shi, k))) << 32);
                        if (sk == 0) continue;
                        ((gptr<float>)sk)[b] = val;
                    }
                }
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            }
        }
    }
}

// ---------------------------------------------------- one-launch dispatch ----
//
// Counts first, then the expansion, in one launch (design page, section 16)
// for rounds of at most kLayoutMaxTiles layout tiles and
// kMaxExpertsOneLaunch experts.  One workgroup of five wavefronts per TB
// slots of the tiled token space, as k_scatter has (at least
// kLayoutMaxTiles + 1), so the grid fits the GPU as the split path's
// scatter does.  Before its own slots, workgroup b < kLayoutMaxTiles counts
// the live choices of layout tile b per expert and publishes them as
// tagged words (tag << 9 | count; a tile holds at most 256 tokens) with
// device-scope stores, tile-major; a workgroup past the round's last tile
// publishes zeros, so every launch rewrites every word and a stale word
// always carries another launch's tag.  Workgroup kLayoutMaxTiles, the
// finisher, polls those words at device scope until every tile of the
// round carries the launch's tag, computes every tile's first row per
// expert (the aligned start of the expert plus its counts in earlier
// tiles) and the ends, publishes them as tagged 64-bit words, and right
// behind them sets all copies of a ready flag to the launch's tag.
// Every workgroup then scatters its slots as k_scatter does with its first
// four wavefronts, which rank their tokens' choices inside their tile
// themselves (lane masks over the tile's tokens up to their own, as
// k_layout builds them).  Its fifth wavefront holds no row loads, so its
// polls are not queued behind them: it polls one copy of the flag (eight
// or so workgroups per copy) until it reads a tag, then reads its tile's
// first rows (and the first workgroup the ends) through the caches,
// reading a word again at device scope while its tag differs from the
// flag's.
// The counting duties never wait and the finisher waits only for them;
// all of them belong to the lowest block indices, so the hand-off completes
// whatever number of workgroups is resident at once.  Every wait is
// bounded: past h.wait_polls polls a workgroup sets the sticky gave-up
// flag, marks its tokens' choices skipped in the slot map (the combine then
// reads nothing for them), clears ends[] if it is the first, stores no row
// and exits.  Every workgroup counts itself finished once it no longer
// reads the counters or flags (right after its hand-off, while its stores
// proceed), in one of several group counters; the last one advances the
// launch counter and clears the counters and the flags, and stream order
// shows the next launch the new values.  Choices that are not live mark a
// spare word of their own lane, in the counting histogram as in the rank
// masks, so idle lanes past a tile's tokens never contend for one LDS
// address.

constexpr int kTagShift = 9;
constexpr uint32_t kTagMask = 0x7FFFFFu;
constexpr int kD1Waves = 5;                    // four scatter wavefronts and the hand-off wavefront
constexpr int kD1Threads = kD1Waves * kWave;

// Tag of the launch whose counter reads `launch`: never 0 (the value of a
// cleared word and of a flag not yet set), and different for consecutive
// launches, also where the 32-bit counter wraps.
__device__ __forceinline__ uint32_t launch_tag(uint32_t launch) { return launch % kTagMask + 1u; }

// One lane: this workgroup no longer reads the launch's counters or flags.
// It counts itself in its group's counter; the last of a group counts the
// group, and the last group clears everything for the next launch and
// advances the launch counter.  (Counters per group, each on its own line,
// keep the grid's finishing workgroups from queueing on one address.)
__device__ __forceinline__ void onepass_done(const Hdr &h)
{
    const int grp = int(blockIdx.x) % kDoneGroups;
    const uint32_t gsize = (gridDim.x - uint32_t(grp) + kDoneGroups - 1u) / kDoneGroups;
    const gptr<uint32_t> gc = h.ready + (kReadyCopies + grp) * kReadyStride;
    if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u != gsize) return;
    const uint32_t ngroups = gridDim.x < uint32_t(kDoneGroups) ? gridDim.x : uint32_t(kDoneGroups);
    if (__hip_atomic_fetch_add(&h.sync[kSyncDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u != ngroups)
        return;
    for (int c = 0; c < kReadyCopies + kDoneGroups; ++c)
        __hip_atomic_store(&h.ready[c * kReadyStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&h.sync[kSyncDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&h.sync[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Ids of the token in tile slot `slot` (-1 past K or when `have` is false).
template <int KMAX>
__device__ __forceinline__ void load_token_ids(const int32_t *ids_first, int slot, int K, bool have, int (&ev)[KMAX])
{
#pragma unroll
    for (int k = 0; k < KMAX; ++k) ev[k] = -1;
    if (!have) return;
    const gptr<const int32_t> idp = (gptr<const int32_t>)ids_first + int64_t(slot) * K;
    if ((K & 3) == 0 && (reinterpret_cast<uintptr_t>(idp) & 15u) == 0) {
#pragma unroll
        for (int q = 0; q < KMAX / 4; ++q) {
            u32x4 v4 = u32x4{~0u, ~0u, ~0u, ~0u};
            if (4 * q < K) v4 = ((gptr<const u32x4>)idp)[q];
            ev[4 * q] = int(v4.x);
            ev[4 * q + 1] = int(v4.y);
            ev[4 * q + 2] = int(v4.z);
            ev[4 * q + 3] = int(v4.w);
        }
    } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int val = idp[k < K ? k : K - 1];
            ev[k] = k < K ? val : -1;
        }
    }
}

template <int KMAX, int VMAX>
__global__ __launch_bounds__(kD1Threads) void k_dispatch1(DispatchArgs a)
{
    static_assert(kLayoutMaxTiles == 32, "tile counts read into 32 registers");
    const u32x4 tr = reinterpret_cast<const u32x4 *>(a.tiles)[blockIdx.x < kLayoutMaxTiles ? blockIdx.x : 0];
    const Hdr h = load_hdr(a);
    extern __shared__ __align__(16) unsigned char lds[];
    const int E = h.E, K = h.K, nblk = h.nblk;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
    constexpr int W = VMAX >= 4 ? 1 : 4 / VMAX;
    constexpr int TB = 4 * W;
    // LDS: the scatter's arrays first, then the counting or finishing duty's
    const int duty_lds = 4 * (E + kWave) * 8 + 4 * E * 4 + TB * K * 4 + 2 * E * 4;

    if (blockIdx.x < kLayoutMaxTiles) {
        // ---- counting duty of tile b: route check, count, publish
        const uint32_t tag =
            launch_tag(__hip_atomic_load(&h.sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        // a count per expert, then one spare per lane for choices that are
        // not live (so they never contend for one address)
        int *hist = reinterpret_cast<int *>(lds + duty_lds);   // [E + 64]
        const int b = blockIdx.x;
        for (int i = tid; i < E + kWave; i += kD1Threads) hist[i] = 0;
        const int n_tile = b < nblk ? int(tr.w & 0xFFFFu) : 0;
        const int s = int(tr.w >> 16);
        const int32_t *ids_first = reinterpret_cast<const int32_t *>((uint64_t(tr.y) << 32) | uint64_t(tr.x));
        int ev[KMAX];
        load_token_ids<KMAX>(ids_first, tid, K, tid < n_tile, ev);
        lds_barrier();
        if (wave * kWave < n_tile) {     // wavefronts past the tile's tokens count nothing
            uint64_t err = kNoError;
            const int g = int(tr.z) + tid;
            uint32_t live;
            if (!routes_plain<KMAX>(ev, E, live)) live = classify_token<KMAX>(ev, E, s, g - a.tok_off[s], err);
            if (err != kNoError) __hip_atomic_fetch_min(h.err, err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int k = 0; k < KMAX; ++k) atomicAdd(&hist[((live >> k) & 1u) ? ev[k] : E + lane], 1);
        }
        lds_barrier();
        // tile-major, one run of whole 128-byte lines per tile, so every
        // line is written by one workgroup only
        for (int e = tid; e < E; e += kD1Threads)
            __hip_atomic_store(&h.tcount[b * tcount_pitch(E) + e], (tag << kTagShift) | uint32_t(hist[e]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // then on to this workgroup's own slots: the count stores land
        // before the launch ends, and the finisher reads every word until
        // it carries this launch's tag
    }

    if (blockIdx.x == kLayoutMaxTiles) {
        // ---- the finisher: thread e polls expert e's tagged word of every
        // tile at device scope until all of the round's tiles carry this
        // launch's tag (bounded), then the workgroup turns the counts into
        // every tile's first row per expert (the expert's aligned start plus
        // its counts in earlier tiles) and the partition-local ends,
        // published as tagged 64-bit words (tag << 32 | value), and right
        // behind them sets every copy of the ready flag to the tag
        const uint32_t tag =
            launch_tag(__hip_atomic_load(&h.sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        __shared__ int s_bad;
        int *A = reinterpret_cast<int *>(lds + duty_lds);   // [E] aligned counts, then their exclusive prefix
        if (tid == 0) s_bad = 0;
        lds_barrier();
        const int pitch = tcount_pitch(E);
        uint32_t cw[kLayoutMaxTiles];
        int C = 0;
        if (tid < E) {
            for (int it = 0;; ++it) {
                if (it > h.wait_polls) {
                    s_bad = 1;
                    break;
                }
#pragma unroll
                for (int bb = 0; bb < kLayoutMaxTiles; ++bb)
                    cw[bb] = __hip_atomic_load(&h.tcount[bb * pitch + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                bool fresh = true;
#pragma unroll
                for (int bb = 0; bb < kLayoutMaxTiles; ++bb)
                    fresh = fresh && (bb >= nblk || (cw[bb] >> kTagShift) == tag);
                if (fresh) break;
                __builtin_amdgcn_s_sleep(1);
            }
#pragma unroll
            for (int bb = 0; bb < kLayoutMaxTiles; ++bb)
                C += bb < nblk ? int(cw[bb] & ((1u << kTagShift) - 1u)) : 0;
            A[tid] = align_up_i(C, h.alpha);
        }
        lds_barrier();
        block_exclusive_scan(A, E);
        if (tid < E && !s_bad) {
            const gptr<unsigned long long> tb = (gptr<unsigned long long>)(h.tcount + kLayoutMaxTiles * pitch);
            const int start = A[tid] - A[part_of(tid, h.E_loc) * h.E_loc];
            const unsigned long long tg = uint64_t(tag) << 32;
            int run = start;
#pragma unroll
            for (int bb = 0; bb < kLayoutMaxTiles; ++bb) {
                __hip_atomic_store(&tb[bb * pitch + tid], tg | uint32_t(run), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                run += bb < nblk ? int(cw[bb] & ((1u << kTagShift) - 1u)) : 0;
            }
            __hip_atomic_store(&tb[kLayoutMaxTiles * pitch + tid], tg | uint32_t(start + C), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        // the flag right behind the bases, without waiting for them: a
        // scatter workgroup that reads a base before it lands sees another
        // launch's tag and reads it again
        if (s_bad) {
            if (tid == 0) __hip_atomic_store(&h.sync[kSyncStall], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (wave == 0) {
            for (int c = lane; c < kReadyCopies; c += kWave)
                __hip_atomic_store(&h.ready[c * kReadyStride], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // the flag stores acknowledged before this workgroup can be counted
        // finished (the last finished workgroup clears the flags for the
        // next launch, and a flag store in flight must not land after that),
        // then on to its own slots
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        lds_barrier();
    }

    // ---- scatter: wavefronts 0-3 hold W tokens each, TB in all; wavefront
    // 4 makes the hand-off.  A workgroup past the last slot (the grid has at
    // least kLayoutMaxTiles + 1 workgroups) only counts itself finished.
    constexpr int HW = kD1Waves - 1;             // the hand-off wavefront
    if (int(blockIdx.x) * TB >= h.nblk * h.tile) {
        if (wave == 0 && lane == 0) onepass_done(h);
        return;
    }
    __shared__ uint64_t s_prow[kMaxParts], s_pw[kMaxParts], s_ps[kMaxParts];
    __shared__ int s_gaveup;
    const int MS = E + kWave;                    // lane masks per expert, then a spare per lane
    unsigned long long *mask = reinterpret_cast<unsigned long long *>(lds);   // [4][E + 64]
    int *pre = reinterpret_cast<int *>(mask + 4 * MS);                        // [4][E]
    int *pkl = pre + 4 * E;                                                   // [TB][K] (expert << 16 | rank), -1
    int *base = pkl + TB * K;                                                 // [E] this tile's first row per expert
    int *Cs = base + E;                                                       // [E] ends (first workgroup)
    const int nvec = h.nvec;
    const int jb = blockIdx.x;
    const int v_first = jb * TB;                 // first slot of the tiled token space
    const int tile = v_first / h.tile;
    const SourceRec src = load_source(a, source_of_tiled(a, h.N, v_first));
    const int T_s = src.T;
    const int t_first = v_first - src.voff + wave * W;    // source token of the wavefront's first slot
    const int g_src = src.off;

    // 1. the ids of the tile's tokens up to this workgroup's last slot
    // (thread = slot of the tile, so wavefronts 0-3), then the rows,
    // weights and scales of the scatter wavefronts' tokens: loads complete
    // in issue order, so the ids (needed first, for the ranks) go ahead of
    // the rows.  The hand-off wavefront loads nothing here.
    const int o = v_first - tile * h.tile;       // this workgroup's first slot inside its tile
    const int tt0 = tile * h.tile - src.voff;    // source token of the tile's first slot
    int ev[KMAX];
    load_token_ids<KMAX>(src.ids + int64_t(tt0) * K, tid, K, tid < o + TB && tt0 + tid < T_s, ev);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 v[W][VMAX];
    float wk[W];
    float scv[W];
    if (wave < HW) {
        const int kl = lane < K ? lane : 0;
        const bool fp8 = h.fp8 != 0;
        const float *sbase = fp8 ? src.scale : src.w;
        const int64_t sst = fp8 ? src.sst : int64_t(K);
        const int64_t sgl = fp8 ? int64_t(lane < h.G ? lane : 0) * src.ssg : 0;
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const int t = t_first + j < T_s ? t_first + j : T_s - 1;
            const gptr<const u32x4> xs = (gptr<const u32x4>)(src.x + int64_t(t) * h.row_bytes);
#pragma unroll
            for (int i = 0; i < VMAX; ++i) {
                const int c = i * kWave + lane;
                v[j][i] = xs[c < nvec ? c : 0];
            }
            wk[j] = ((gptr<const float>)src.w)[int64_t(t) * K + kl];
            scv[j] = ((gptr<const float>)sbase)[int64_t(t) * sst + sgl];
        }
    }
    if (lane == 0) {
        if (wave == 0) table_to_lds(s_prow, a.rows);
        if (wave == 1) table_to_lds(s_pw, a.roww);
        if (wave == 2) table_to_lds(s_ps, a.scales);
        if (wave == 3) s_gaveup = 0;
    }
    for (int i = tid; i < 4 * MS; i += kD1Threads) mask[i] = 0ull;
    lds_barrier();

    // 2. in-tile ranks of this workgroup's tokens (route errors are recorded
    // by the counting workgroups)
    uint32_t live = 0;
    if (wave < HW && wave * kWave < o + TB) {    // wavefronts past this workgroup's slots mark nothing
        uint64_t err_unused = kNoError;
        if (!routes_plain<KMAX>(ev, E, live)) live = classify_token<KMAX>(ev, E, 0, 0, err_unused);
        unsigned long long *mrow = mask + size_t(wave) * MS;
        const unsigned long long bit = 1ull << lane;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) atomicOr(&mrow[((live >> k) & 1u) ? ev[k] : E + lane], bit);
    }
    lds_barrier();
    for (int e = tid; e < E; e += kD1Threads) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            pre[w * E + e] = run;
            run += __popcll(mask[w * MS + e]);
        }
    }
    lds_barrier();
    if (tid >= o && tid < o + TB) {
        const unsigned long long below = (1ull << lane) - 1ull;
        const unsigned long long *mrow = mask + size_t(wave) * MS;
        int *dst = pkl + (tid - o) * K;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const bool l = (live >> k) & 1u;
            const int e = l ? ev[k] : 0;
            if (k < K) dst[k] = l ? ((e << 16) | (pre[wave * E + e] + __popcll(mrow[e] & below))) : -1;
        }
    }

    // 3. the hand-off: wavefront 4, which has no loads of its own in flight
    // (its polls do not queue behind the rows), polls this workgroup's copy
    // of the ready flag until it holds a launch's tag (bounded; every lane
    // reads the same word, one request per poll), then reads this tile's
    // first row of every expert (and, in the first workgroup, the ends)
    // through the caches, lane l taking experts l, l + 64, ...; a word whose
    // tag differs from the flag's is read again at device scope (bounded).
    // No cache holds a copy from before the words were final: kernels start
    // with invalidated caches and nothing reads a word before the flag.
    if (wave == HW) {
        const gptr<uint32_t> rf = h.ready + (jb % kReadyCopies) * kReadyStride;
        uint32_t tg = 0;
        for (int it = 0; it <= h.wait_polls; ++it) {
            tg = __hip_atomic_load(rf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tg != 0u) break;
            __builtin_amdgcn_s_sleep(1);
        }
        tg = uint32_t(__builtin_amdgcn_readfirstlane(int(tg)));
        bool gave = tg == 0u;
        // nothing below is moved above the poll
        asm volatile("" ::: "memory");
        if (!gave) {
            static_assert(kMaxExpertsOneLaunch <= 4 * kWave, "four experts per lane");
            const int pitch = tcount_pitch(E);
            const gptr<unsigned long long> tb = (gptr<unsigned long long>)(h.tcount + kLayoutMaxTiles * pitch);
            const int nrow = jb == 0 ? 2 : 1;      // this tile's bases; the ends row for the first workgroup
            unsigned long long w[2][4];
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int e = q * kWave + lane < E ? q * kWave + lane : E - 1;
                    const int row = r == 0 ? tile : kLayoutMaxTiles;
                    w[r][q] = (r < nrow && q * kWave < E) ? ((gptr<const unsigned long long>)tb)[row * pitch + e] : 0ull;
                }
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (r >= nrow || q * kWave >= E) continue;
                    const int e = q * kWave + lane < E ? q * kWave + lane : E - 1;
                    const int row = r == 0 ? tile : kLayoutMaxTiles;
                    for (int it = 0; uint32_t(w[r][q] >> 32) != tg; ++it) {
                        if (it > h.wait_polls) {
                            gave = true;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                        w[r][q] = __hip_atomic_load(&tb[row * pitch + e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    if (q * kWave + lane < E) (r == 0 ? base : Cs)[q * kWave + lane] = int(uint32_t(w[r][q]));
                }
            gave = __builtin_amdgcn_ballot_w64(gave) != 0;
        }
        if (lane == 0 && gave) s_gaveup = 1;
    }
    lds_barrier();
    if (s_gaveup) {
        // no bases: this workgroup's choices are skipped, nothing is stored
        if (tid == 0) __hip_atomic_store(&h.sync[kSyncStall], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (wave < HW) {
#pragma unroll
            for (int j = 0; j < W; ++j) {
                const int t = t_first + j;
                if (t < T_s && lane < K) {
                    i32x2 sl;
                    sl.x = -1;
                    sl.y = __float_as_int(wk[j]);
                    ((gptr<i32x2>)h.slot)[int64_t(g_src + t) * K + lane] = sl;
                }
            }
        }
        if (jb == 0)
            for (int e = tid; e < E; e += kD1Threads) h.ends[e] = 0;
        if (wave == HW && lane == 0) onepass_done(h);
        return;
    }
    if (jb == 0)
        for (int e = tid; e < E; e += kD1Threads) h.ends[e] = Cs[e];
    if (wave == HW) {
        // the counters and flags are no longer read by this workgroup
        if (lane == 0) onepass_done(h);
        return;
    }
    // every row, weight and scale load has been waited for here, once,
    // before the first store (see k_scatter)
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // 5. slots and stores, token by token (as k_scatter)
#pragma unroll
    for (int j = 0; j < W; ++j) {
        const int t = t_first + j;
        if (t >= T_s) break;
        const int g = g_src + t;
        int part = -1, row = -1;
        uint64_t d = 0, ds = 0;
        const int pkj = lane < K ? pkl[(wave * W + j) * K + lane] : -1;
        if (pkj >= 0) {
            const int e = pkj >> 16;
            row = base[e] + (pkj & 0xFFFF);
            part = e / h.E_loc;
            d = s_prow[part] + uint64_t(row) * uint64_t(h.row_bytes);
            ds = s_ps[part] + uint64_t(row) * uint64_t(h.G) * 4u;
            ((gptr<float>)s_pw[part])[row] = wk[j];
        }
        if (lane < K) {
            i32x2 sl;
            sl.x = part < 0 ? -1 : ((part << 24) | row);
            sl.y = __float_as_int(wk[j]);
            ((gptr<i32x2>)h.slot)[int64_t(g) * K + lane] = sl;
        }
        const int dlo = int(uint32_t(d)), dhi = int(uint32_t(d >> 32));
        for (int k = 0; k < K; ++k) {
            const uint64_t dk = uint64_t(uint32_t(__builtin_amdgcn_readlane(dlo, k))) |
                                (uint64_t(uint32_t(__builtin_amdgcn_readlane(dhi, k))) << 32);
            if (dk == 0) continue;
            const gptr<u32x4> dst = (gptr<u32x4>)dk;
#pragma unroll
            for (int i = 0; i < VMAX; ++i) {
                const int c = i * kWave + lane;
                if (c < nvec) __builtin_nontemporal_store(v[j][i], &dst[c]);
            }
        }
        if (nvec > kWave * VMAX) {
            const gptr<const u32x4> xs = (gptr<const u32x4>)(src.x + int64_t(t) * h.row_bytes);
            for (int cb = kWave * VMAX; cb < nvec; cb += kWave * VMAX) {
                u32x4 r[VMAX];
#pragma unroll
                for (int i = 0; i < VMAX; ++i) {
                    const int c = cb + i * kWave + lane;
                    if (c < nvec) r[i] = xs[c];
                }
                for (int k = 0; k < K; ++k) {
                    const uint64_t dk = uint64_t(uint32_t(__builtin_amdgcn_readlane(dlo, k))) |
                                        (uint64_t(uint32_t(__builtin_amdgcn_readlane(dhi, k))) << 32);
                    if (dk == 0) continue;
                    const gptr<u32x4> dst = (gptr<u32x4>)dk;
#pragma unroll
                    for (int i = 0; i < VMAX; ++i) {
                        const int c = cb + i * kWave + lane;
                        if (c < nvec) __builtin_nontemporal_store(r[i], &dst[c]);
                    }
                }
            }
        }
        if (h.fp8) {
            const int G = h.G;
            const int slo = int(uint32_t(ds)), shi = int(uint32_t(ds >> 32));
            if (lane < G) {
                for (int k = 0; k < K; ++k) {
                    const uint64_t sk = uint64_t(uint32_t(__builtin_amdgcn_readlane(slo, k))) |
                                        (uint64_t(uint32_t(__builtin_amdgcn_readlane(shi, k))) << 32);
                    if (sk == 0) continue;
                    ((gptr<float>)sk)[lane] = scv[j];
                }
            }
            if (G > kWave) {
                const gptr<const float> sc = (gptr<const float>)src.scale + int64_t(t) * src.sst;
                for (int bb = kWave + lane; bb < G; bb += kWave) {
                    const float val = sc[int64_t(bb) * src.ssg];
                    for (int k = 0; k < K; ++k) {
                        const uint64_t sk = uint64_t(uint32_t(__builtin_amdgcn_readlane(slo, k))) |
                                            (uint64_t(uint32_t(__builtin_amdgcn_readlane(shi, k))) << 32);
                        if (sk == 0) continue;
                        ((gptr<float>)sk)[bb] = val;
                    }
                }
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            }
        }
    }
}

// Dispatch of a cached round.  Block = 256 threads = 256 / LPT tokens, LPT
// (64, 128 or 256) lanes per token, each lane holding VMAX 16-byte columns
// (column i * LPT + lane of its token); longer rows loop over chunks.  Every
// wavefront of a token reads the token's K slots itself (no hand-off between
// wavefronts); the token's first wavefront also writes the new weights into
// the slot map and the row weights.  The leading scalar arguments (lanes
// per token, the slot map's address, the first two sources' rows, their
// token counts as T0 | T1 << 16, and K | nvec << 8) are preloaded into SGPRs
// by the hardware; rounds of at most two sources (FEW) address the row and
// the slots from them alone, ahead of any load from the argument block.
template <int VMAX, bool FEW>
__global__ __launch_bounds__(256) void k_scatter_cached(int lpt, const int32_t *pslot, const uint8_t *px0,
                                                        const uint8_t *px1, int pT01, int pKnv, DispatchArgs a)
{
    __shared__ uint64_t s_prow[kMaxParts], s_pw[kMaxParts], s_ps[kMaxParts];
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
    const int wpt = lpt / kWave;                          // wavefronts per token
    const int g = blockIdx.x * (256 / lpt) + wave / wpt;
    const int tl = (wave % wpt) * kWave + lane;           // lane within the token
    u32x4 v[VMAX];
    i32x2 sl;
    sl.x = -1;
    sl.y = 0;
    auto row_and_slots = [&](const uint8_t *x, int t, int K, int nvec) {
        const gptr<const u32x4> xs = (gptr<const u32x4>)(x + int64_t(t) * nvec * 16);
#pragma unroll
        for (int i = 0; i < VMAX; ++i) {
            const int c = i * lpt + tl;
            v[i] = xs[c < nvec ? c : 0];
        }
        if (lane < K) sl = ((gptr<const i32x2>)pslot)[int64_t(g) * K + lane];
    };
    int s = 0, t0 = 0;
    bool have = false;
    if constexpr (FEW) {
        const int T0 = pT01 & 0xFFFF, T1 = pT01 >> 16;
        have = g < T0 + T1;
        s = g < T0 ? 0 : 1;
        t0 = s ? T0 : 0;
        if (have) row_and_slots(s ? px1 : px0, g - t0, pKnv & 0xFF, pKnv >> 8);
    }
    u32x16 r0, r1;
    const Hdr h = load_hdr(a, r0, r1);
    const int K = h.K, nvec = h.nvec;
    if constexpr (!FEW) {
        const u32x16 to = load_offsets(a.tok_off);
        // both header halves, the offsets and lpt in one batch of scalar loads
        // (left alone, the compiler requests each where it is first used and
        // waits for it there: three dependent round trips before the record)
        asm volatile("" ::"s"(r0), "s"(r1), "s"(to), "s"(lpt));
        have = g < h.ntok;
        s = source_of(to, h.N, have ? g : 0, t0);
        const SourceRec rx = load_source(a, s);
        if (have) row_and_slots(rx.x, g - t0, K, nvec);
    }
    const SourceRec src = load_source(a, s);
    const int t = (have ? g : 0) - t0;
    float wk = 0.0f;
    float scv = 0.0f;                                     // FP8: scale of block `lane` (first wavefront)
    if (have) {
        if (lane < K) wk = ((gptr<const float>)src.w)[int64_t(t) * K + lane];
        if (h.fp8 && tl < kWave && tl < h.G) scv = ((gptr<const float>)src.scale)[int64_t(t) * src.sst + int64_t(tl) * src.ssg];
    }
    if (lane == 0) {
        if (wave == 0) table_to_lds(s_prow, a.rows);
        if (wave == 1) table_to_lds(s_pw, a.roww);
        if (wave == 2) table_to_lds(s_ps, a.scales);
    }
    lds_barrier();
    if (!have) return;
    uint64_t d = 0, ds = 0;
    if (lane < K && sl.x >= 0) {
        const int part = sl.x >> 24;
        const int row = sl.x & 0xFFFFFF;
        d = s_prow[part] + uint64_t(row) * uint64_t(h.row_bytes);
        ds = s_ps[part] + uint64_t(row) * uint64_t(h.G) * 4u;
        if (tl < kWave) {
            ((gptr<float>)s_pw[part])[row] = wk;
            h.slot[(int64_t(g) * K + lane) * 2 + 1] = __float_as_int(wk);
        }
    }
    const int dlo = int(uint32_t(d)), dhi = int(uint32_t(d >> 32));
    for (int k = 0; k < K; ++k) {
        const uint64_t dk = uint64_t(uint32_t(__builtin_amdgcn_readlane(dlo, k))) |
                            (uint64_t(uint32_t(__builtin_amdgcn_readlane(dhi, k))) << 32);
        if (dk == 0) continue;
        const gptr<u32x4> dst = (gptr<u32x4>)dk;
#pragma unroll
        for (int i = 0; i < VMAX; ++i) {
            const int c = i * lpt + tl;
            if (c < nvec) __builtin_nontemporal_store(v[i], &dst[c]);
        }
    }
    // rows longer than lpt * VMAX columns: the remaining columns, chunk by chunk
    if (nvec > lpt * VMAX) {
        const gptr<const u32x4> xs = (gptr<const u32x4>)(src.x + int64_t(t) * h.row_bytes);
        for (int cb = lpt * VMAX; cb < nvec; cb += lpt * VMAX) {
            u32x4 r[VMAX];
#pragma unroll
            for (int i = 0; i < VMAX; ++i) {
                const int c = cb + i * lpt + tl;
                if (c < nvec) r[i] = xs[c];
            }
            for (int k = 0; k < K; ++k) {
                const uint64_t dk = uint64_t(uint32_t(__builtin_amdgcn_readlane(dlo, k))) |
                                    (uint64_t(uint32_t(__builtin_amdgcn_readlane(dhi, k))) << 32);
                if (dk == 0) continue;
                const gptr<u32x4> dst = (gptr<u32x4>)dk;
#pragma unroll
                for (int i = 0; i < VMAX; ++i) {
                    const int c = cb + i * lpt + tl;
                    if (c < nvec) __builtin_nontemporal_store(r[i], &dst[c]);
                }
            }
        }
    }
    if (h.fp8 && tl < kWave) {
        const int slo = int(uint32_t(ds)), shi = int(uint32_t(ds >> 32));
        if (lane < h.G) {
            for (int k = 0; k < K; ++k) {
                const uint64_t sk = uint64_t(uint32_t(__builtin_amdgcn_readlane(slo, k))) |
                                    (uint64_t(uint32_t(__builtin_amdgcn_readlane(shi, k))) << 32);
                if (sk == 0) continue;
                ((gptr<float>)sk)[lane] = scv;
            }
        }
        // rows of more than 64 scale blocks (H > 8192): the other blocks
        const gptr<const float> sc = (gptr<const float>)src.scale + int64_t(t) * src.sst;
        for (int b = kWave + lane; b < h.G; b += kWave) {
            const float val = sc[int64_t(b) * src.ssg];
            for (int k = 0; k < K; ++k) {
                const uint64_t sk = uint64_t(uint32_t(__builtin_amdgcn_readlane(slo, k))) |
                                    (uint64_t(uint32_t(__builtin_amdgcn_readlane(shi, k))) << 32);
                if (sk == 0) continue;
                ((gptr<float>)sk)[b] = val;
            }
        }
    }
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Combine: one wavefront per (token, segment of 64*VPL 16-byte columns).
// The token's slots arrive as wave-uniform values, one 64-byte scalar load
// per eight choices (the slot map does not change during the kernel).  The
// slot map's address, the sizes and the first two reply bases are leading
// scalar arguments, which the hardware preloads into SGPRs, so the slot
// load is the first memory request.  With at most NB = 2 or 4 partitions
// each choice's reply base is selected from those (the third and fourth
// from the argument block, loaded alongside the slots), so the only round
// trip before the row loads is the slots' (the two-way select is the
// cheaper one, which shows at decode).  With more partitions (NB = 0) the
// bases are looked up in the kernel arguments by partition number, all
// eight requested before one wait.  The wavefront then issues every live
// row's loads before it accumulates, in ascending k, with a float32 multiply
// and a separate add.  The output rows of the first two sources and the
// first source's token count are preloaded arguments too (out1 is null
// unless there are exactly two sources; with one, t1 = ntok and no token
// reaches it): a token of source 0 or 1 finds its
// output row with no memory request, so the wavefront's last step is the
// store rather than a chain of argument loads (the number of sources, the
// offsets, the source's output base), which would add their latency once
// per kernel.  Tokens past the first source of a round with more sources
// still search the offsets in the argument block.  NT: streaming stores for
// the output, chosen for small rounds (see be_launch_combine).
template <int VPL, int NB, bool NT>
__global__ __launch_bounds__(256) void k_combine(const int32_t *slot, uint64_t rb0, uint64_t rb1, uint64_t out0,
                                                 uint64_t out1, int ntok, int K, int H, int t1, CombineArgs a)
{
#pragma clang fp contract(off)
    static_assert(offsetof(CombineArgs, reply4) == 32 && offsetof(CombineArgs, tok_off) == 64,
                  "scalars and four bases in the first 64 bytes, offsets at byte 64");
    const u32x16 hv = *reinterpret_cast<const u32x16 *>(&a);
    const int nvec = H >> 3, nseg = (nvec + kWave * VPL - 1) / (kWave * VPL);
    auto base4 = [&](uint32_t q) { return (uint64_t(hv[9 + 2 * q]) << 32) | uint64_t(hv[8 + 2 * q]); };
    const uint64_t rb2 = base4(2), rb3 = base4(3);
    const int lane = threadIdx.x & (kWave - 1);
    const int gw = blockIdx.x * 4 + wave_id();
    const int g = div_pow2_or(gw, nseg);
    const int seg = gw - g * nseg;
    if (g >= ntok) return;
    const int c0 = seg * kWave * VPL + lane;
    const uint64_t rowb = uint64_t(H) * 2u;
    float acc[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += 8) {
        // slots k0 .. k0 + 7 (entries past K belong to the next token, or
        // to the region's slack, and are not used)
        const u32x16 sv = *(__attribute__((address_space(4))) const u32x16 *)(slot + (int64_t(g) * K + k0) * 2);
        u32x4 y[8][VPL];
        uint64_t rk[8], b[8];
        // partition numbers are masked into the tables, so even the unused
        // entries select inside them
        if (NB == 2) {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) b[kk] = (sv[2 * kk] >> 24) & 1u ? rb1 : rb0;
        } else if (NB == 4) {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const uint32_t q = (sv[2 * kk] >> 24) & 3u;
                b[kk] = q & 2u ? (q & 1u ? rb3 : rb2) : (q & 1u ? rb1 : rb0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                b[kk] = reinterpret_cast<uint64_t>(a.reply[(int(sv[2 * kk]) >> 24) & (kMaxParts - 1)]);
            // keeps the eight loads ahead of their first use (otherwise each
            // is sunk into its choice's branch with a wait of its own)
            asm volatile("" ::"s"(b[0]), "s"(b[1]), "s"(b[2]), "s"(b[3]), "s"(b[4]), "s"(b[5]), "s"(b[6]), "s"(b[7]));
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int sl = int(sv[2 * kk]);
            rk[kk] = (k0 + kk < K && sl >= 0) ? b[kk] + uint64_t(sl & 0xFFFFFF) * rowb : 0;
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const gptr<const u32x4> src = (gptr<const u32x4>)rk[kk];
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int c = c0 + i * kWave;
                y[kk][i] = (rk[kk] != 0 && c < nvec) ? __builtin_nontemporal_load(&src[c]) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            if (rk[kk] == 0) continue;
            const float w = __uint_as_float(sv[2 * kk + 1]);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const uint32_t q[4] = {y[kk][i].x, y[kk][i].y, y[kk][i].z, y[kk][i].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float lo = __uint_as_float(q[j] << 16);
                    const float hi = __uint_as_float(q[j] & 0xFFFF0000u);
                    const float plo = w * lo;
                    const float phi = w * hi;
                    acc[i][2 * j] = acc[i][2 * j] + plo;
                    acc[i][2 * j + 1] = acc[i][2 * j + 1] + phi;
                }
            }
        }
    }
    // the token's output row: sources 0 and 1 from the preloaded bases, any
    // later one through the offsets (wave-uniform branch)
    uint64_t ob = out0;
    int t0 = 0;
    if (g >= t1) {
        if (out1 != 0) {
            ob = out1;
            t0 = t1;
        } else {
            const int s = source_of(load_offsets(a.tok_off), a.N, g, t0);
            ob = reinterpret_cast<uint64_t>(a.out[s]);
        }
    }
    const gptr<u32x4> o = (gptr<u32x4>)(ob + uint64_t(g - t0) * rowb);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int c = c0 + i * kWave;
        if (c < nvec) {
            u32x4 r;
            r.x = bf16_rne_bits(acc[i][0]) | (bf16_rne_bits(acc[i][1]) << 16);
            r.y = bf16_rne_bits(acc[i][2]) | (bf16_rne_bits(acc[i][3]) << 16);
            r.z = bf16_rne_bits(acc[i][4]) | (bf16_rne_bits(acc[i][5]) << 16);
            r.w = bf16_rne_bits(acc[i][6]) | (bf16_rne_bits(acc[i][7]) << 16);
            if constexpr (NT)
                __builtin_nontemporal_store(r, &o[c]);
            else
                o[c] = r;
        }
    }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// float8_e4m3fn codes of four scaled values (bytes 0..3 of the result):
// the hardware conversion rounds to the nearest even code.  The inputs are
// within 448 after the exact power-of-two scaling except for infinities,
// which are clamped to 448 first (they decode back to infinity at the top
// scale); NaN elements get the NaN code with their sign.
__device__ __forceinline__ uint32_t e4m3_codes4(float x0, float x1, float x2, float x3)
{
    const float c0 = __builtin_fminf(__builtin_fmaxf(x0, -448.0f), 448.0f);
    const float c1 = __builtin_fminf(__builtin_fmaxf(x1, -448.0f), 448.0f);
    const float c2 = __builtin_fminf(__builtin_fmaxf(x2, -448.0f), 448.0f);
    const float c3 = __builtin_fminf(__builtin_fmaxf(x3, -448.0f), 448.0f);
    uint32_t w = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false)) & 0xFFFFu;
    w = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, int(w), true));
    const float xs[4] = {x0, x1, x2, x3};
    bool nan = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) nan |= xs[j] != xs[j];
    if (__ballot(nan) != 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t code = ((__float_as_uint(xs[j]) >> 24) & 0x80u) | 0x7Fu;
            w = xs[j] != xs[j] ? ((w & ~(0xFFu << (8 * j))) | (code << (8 * j))) : w;
        }
    }
    return w;
}

// Scale exponent of a group from the float32 bits of its amax: the smallest
// e with amax <= 448 * 2^e = 1.75 * 2^(e + 8), at least -117 (an infinite
// amax gives 120).
__device__ __forceinline__ int fp8_group_exponent(uint32_t amax_bits)
{
    if (amax_bits < 0x00800000u) return -117;                                   // zero or subnormal
    const int ex = int(amax_bits >> 23) - 127;
    const int e = (amax_bits & 0x7FFFFFu) <= 0x600000u ? ex - 8 : ex - 7;
    return e < -117 ? -117 : e;
}

// Stage one of the per-stage combine for partition f, one token and one
// segment of 64 * VPL 16-byte columns: the token's live rows of f (lanes
// with `mine`) weighted and summed in ascending k in FP32, rounded once and
// stored as the token's partial row.  ys/sfs return each column group as
// stored, in the form load_partial reads it back (the FP8 codes with the
// group's scale byte), so a caller can add the partial without reloading
// it.  Every lane of the wavefront takes part (the FP8 group maximum is a
// cross-lane reduction).
template <bool FP8, int VPL>
__device__ __forceinline__ void stage_one(const uint16_t *reply, int H, int K, int64_t prow, int lane, int seg, int2 sl,
                                          bool mine, uint8_t *row, u32x4 (&ys)[VPL], uint32_t (&sfs)[VPL])
{
#pragma clang fp contract(off)
    const int nvec = H >> 3;
    const int c0 = seg * kWave * VPL + lane;
    uint64_t raddr = 0;
    if (mine) raddr = reinterpret_cast<uint64_t>(reply) + uint64_t(sl.x & 0xFFFFFF) * uint64_t(H) * 2u;
    const int rlo = int(uint32_t(raddr)), rhi = int(uint32_t(raddr >> 32));
    float acc[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += 8) {
        u32x4 y[8][VPL];
        uint64_t rk[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            rk[kk] = uint64_t(uint32_t(__builtin_amdgcn_readlane(rlo, k0 + kk))) |
                     (uint64_t(uint32_t(__builtin_amdgcn_readlane(rhi, k0 + kk))) << 32);
            const gptr<const u32x4> src = (gptr<const u32x4>)rk[kk];
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int c = c0 + i * kWave;
                y[kk][i] = (rk[kk] != 0 && c < nvec) ? __builtin_nontemporal_load(&src[c]) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            if (rk[kk] == 0) continue;
            const float w = __int_as_float(__builtin_amdgcn_readlane(sl.y, k0 + kk));
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const uint32_t q[4] = {y[kk][i].x, y[kk][i].y, y[kk][i].z, y[kk][i].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float plo = w * __uint_as_float(q[j] << 16);
                    const float phi = w * __uint_as_float(q[j] & 0xFFFF0000u);
                    acc[i][2 * j] = acc[i][2 * j] + plo;
                    acc[i][2 * j + 1] = acc[i][2 * j + 1] + phi;
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int c = c0 + i * kWave;
        uint32_t b[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = bf16_rne_bits(acc[i][j]);
        if (!FP8) {
            u32x4 r;
            r.x = b[0] | (b[1] << 16);
            r.y = b[2] | (b[3] << 16);
            r.z = b[4] | (b[5] << 16);
            r.w = b[6] | (b[7] << 16);
            if (c < nvec) reinterpret_cast<u32x4 *>(row)[c] = r;
            ys[i] = r;
            sfs[i] = 0;
            continue;
        }
        // FP8: a group of 128 elements is 16 lanes; amax over the magnitudes
        // of its non-NaN elements (integer order equals float order for them)
        uint32_t am = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t m = (b[j] << 16) & 0x7FFFFFFFu;
            am = (m <= 0x7F800000u && m > am) ? m : am;
        }
        // max over the 16-lane DPP row: rotations by 1, 2, 4 and 8
        {
            uint32_t o = uint32_t(__builtin_amdgcn_update_dpp(0, int(am), 0x121, 0xF, 0xF, false));  // row_ror:1
            am = o > am ? o : am;
            o = uint32_t(__builtin_amdgcn_update_dpp(0, int(am), 0x122, 0xF, 0xF, false));           // row_ror:2
            am = o > am ? o : am;
            o = uint32_t(__builtin_amdgcn_update_dpp(0, int(am), 0x124, 0xF, 0xF, false));           // row_ror:4
            am = o > am ? o : am;
            o = uint32_t(__builtin_amdgcn_update_dpp(0, int(am), 0x128, 0xF, 0xF, false));           // row_ror:8
            am = o > am ? o : am;
        }
        const int e = fp8_group_exponent(am);
        const float inv = __uint_as_float(uint32_t(127 - e) << 23);              // 2^-e, a normal float
        const uint32_t lo = e4m3_codes4(__uint_as_float(b[0] << 16) * inv, __uint_as_float(b[1] << 16) * inv,
                                        __uint_as_float(b[2] << 16) * inv, __uint_as_float(b[3] << 16) * inv);
        const uint32_t hi = e4m3_codes4(__uint_as_float(b[4] << 16) * inv, __uint_as_float(b[5] << 16) * inv,
                                        __uint_as_float(b[6] << 16) * inv, __uint_as_float(b[7] << 16) * inv);
        if (c < nvec) {
            uint2 v2;
            v2.x = lo;
            v2.y = hi;
            reinterpret_cast<uint2 *>(row)[c] = v2;
            if ((lane & 15) == 0) row[H + c / 16] = uint8_t(127 + e);
        }
        ys[i] = u32x4{lo, hi, 0u, 0u};
        sfs[i] = uint32_t(127 + e);
    }
    if (FP8) {
        const int G = H / 128;
        const int pad = int(prow) - H - G;
        if (seg == 0 && lane < pad) row[H + G + lane] = 0;
    }
}

// Stage one of the per-stage combine for partition f: one wavefront per
// (token, segment of 64 * VPL 16-byte columns).  A token has about K/F live
// rows in one partition, so a wavefront may take VPL columns per lane to
// keep more row loads in flight.  The slot map's and the reply's addresses,
// K, H, the segment count, the token count and f are leading scalar
// arguments, preloaded into SGPRs, so the slot load is the first request.
template <bool FP8, int VPL>
__global__ __launch_bounds__(256) void k_partial(const int32_t *pslot, const uint16_t *preply, int pK, int pH,
                                                 int pnseg, int pntok, int pf, StageArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int gw = blockIdx.x * 4 + wave_id();
    const int g = div_pow2_or(gw, pnseg);
    const int seg = gw - g * pnseg;
    if (g >= pntok) return;
    int2 sl;
    sl.x = -1;
    sl.y = 0;
    if (lane < pK) sl = reinterpret_cast<const int2 *>(pslot)[int64_t(g) * pK + lane];
    const bool mine = sl.x >= 0 && (sl.x >> 24) == pf;
    if (__ballot(mine) == 0) return;                 // no live choice of g in f: no partial
    int t0;
    const int s = source_of(load_offsets(a.tok_off), a.N, g, t0);
    const int t = g - t0;
    uint8_t *row = a.partials + ((int64_t(pf) * a.N + s) * a.capacity + t) * a.prow;
    u32x4 ys[VPL];
    uint32_t sfs[VPL];
    stage_one<FP8, VPL>(preply, pH, pK, a.prow, lane, seg, sl, mine, row, ys, sfs);
}

// One partial row segment added into a stage-two accumulator.
template <bool FP8>
__device__ __forceinline__ void add_partial(float (&acc)[8], const u32x4 &y, uint32_t sf)
{
#pragma clang fp contract(off)
    if (!FP8) {
        const uint32_t q[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[2 * j] = acc[2 * j] + __uint_as_float(q[j] << 16);
            acc[2 * j + 1] = acc[2 * j + 1] + __uint_as_float(q[j] & 0xFFFF0000u);
        }
    } else {
        // the hardware conversion decodes E4M3 exactly; the power-of-two
        // scale keeps every nonzero product a normal float
        const float scale = __uint_as_float(sf << 23);                         // 2^(byte - 127)
        const f32x2 v[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(int(y.x), false), __builtin_amdgcn_cvt_pk_f32_fp8(int(y.x), true),
                            __builtin_amdgcn_cvt_pk_f32_fp8(int(y.y), false), __builtin_amdgcn_cvt_pk_f32_fp8(int(y.y), true)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float p0 = v[j].x * scale;
            const float p1 = v[j].y * scale;
            acc[2 * j] = acc[2 * j] + p0;
            acc[2 * j + 1] = acc[2 * j + 1] + p1;
        }
    }
}

// One segment of a partial row: 16 bytes (BF16) or 8 code bytes plus the
// group's scale byte (FP8).
template <bool FP8>
__device__ __forceinline__ void load_partial(const uint8_t *row, int c, int H, u32x4 &y, uint32_t &sf)
{
    if (!FP8) {
        y = reinterpret_cast<const u32x4 *>(row)[c];
        sf = 0;
    } else {
        const uint2 v = reinterpret_cast<const uint2 *>(row)[c];
        y = u32x4{v.x, v.y, 0u, 0u};
        sf = row[H + c / 16];
    }
}

// The round's last reply: partition f's stage one and stage two for every
// source in one launch, one wavefront per (token, 64-column segment).  The
// wavefront computes and stores the token's partial of f as k_partial
// does, then adds the token's partials: a partition's partial is added when
// no later live top-k lane of the token maps to that partition, so
// partitions are visited in ascending order of their last live lane.  The
// term of f is its partial as stored (for FP8 the decoded codes), taken
// from registers instead of being read back, so the sum is the same as with
// every partial reloaded.  A partial row's address does not depend on the
// slot map: with at most four partitions the other partitions' rows are
// requested before the reply rows, all in flight together (rows of a
// partition without a live choice of the token are loaded but never added).
template <bool FP8>
__global__ __launch_bounds__(256) void k_last(const int32_t *pslot, const uint16_t *preply, int pK, int pH, int pnseg,
                                              int pntok, int pf, StageArgs a)
{
#pragma clang fp contract(off)
    const int lane = threadIdx.x & (kWave - 1);
    const int gw = blockIdx.x * 4 + wave_id();
    const int g = div_pow2_or(gw, pnseg);
    const int seg = gw - g * pnseg;
    if (g >= pntok) return;
    int2 sl;
    sl.x = -1;
    sl.y = 0;
    if (lane < pK) sl = reinterpret_cast<const int2 *>(pslot)[int64_t(g) * pK + lane];
    const int part = sl.x >= 0 ? (sl.x >> 24) : -1;
    int t0;
    const int s = source_of(load_offsets(a.tok_off), a.N, g, t0);
    const int t = g - t0;
    const int c = seg * kWave + lane;
    const bool col = c < (pH >> 3);
    const int64_t fstride = int64_t(a.N) * a.capacity * a.prow;
    uint8_t *base = a.partials + (int64_t(s) * a.capacity + t) * a.prow;
    constexpr int SPEC = 4;
    const bool spec = a.F <= SPEC;
    u32x4 ys[SPEC];
    uint32_t sfs[SPEC];
#pragma unroll
    for (int i = 0; i < SPEC; ++i) {
        ys[i] = u32x4{0u, 0u, 0u, 0u};
        sfs[i] = 127u;
        if (spec && i < a.F && i != pf && col) load_partial<FP8>(base + i * fstride, c, pH, ys[i], sfs[i]);
    }
    const bool mine = part == pf;
    u32x4 yf = u32x4{0u, 0u, 0u, 0u};
    uint32_t sff = 127u;
    if (__ballot(mine) != 0) {
        u32x4 y1[1];
        uint32_t s1[1];
        stage_one<FP8, 1>(preply, pH, pK, a.prow, lane, seg, sl, mine, base + pf * fstride, y1, s1);
        yf = y1[0];
        sff = s1[0];
    }
    bool last = part >= 0;
    for (int j = 0; j < pK; ++j) {
        const int pj = __builtin_amdgcn_readlane(part, j);
        last = last && !(j > lane && pj == part);
    }
    uint64_t lm = __ballot(last);
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    if (spec) {
        while (lm != 0) {
            const int k = __builtin_ctzll(lm);
            lm &= lm - 1;
            const int f = __builtin_amdgcn_readlane(part, k);
            u32x4 y = ys[0];
            uint32_t sf = sfs[0];
#pragma unroll
            for (int i = 1; i < SPEC; ++i) {
                y = f == i ? ys[i] : y;
                sf = f == i ? sfs[i] : sf;
            }
            y = f == pf ? yf : y;
            sf = f == pf ? sff : sf;
            add_partial<FP8>(acc, y, sf);
        }
    } else {
        while (lm != 0) {
            u32x4 y[4];
            uint32_t sf[4];
            int n = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                y[i] = u32x4{0u, 0u, 0u, 0u};
                sf[i] = 127u;
                if (lm != 0) {
                    const int k = __builtin_ctzll(lm);
                    lm &= lm - 1;
                    const int f = __builtin_amdgcn_readlane(part, k);
                    if (f == pf) {
                        y[i] = yf;
                        sf[i] = sff;
                    } else if (col) {
                        load_partial<FP8>(base + int64_t(f) * fstride, c, pH, y[i], sf[i]);
                    }
                    n = i + 1;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < n) add_partial<FP8>(acc, y[i], sf[i]);
        }
    }
    if (col) {
        u32x4 r;
        r.x = bf16_rne_bits(acc[0]) | (bf16_rne_bits(acc[1]) << 16);
        r.y = bf16_rne_bits(acc[2]) | (bf16_rne_bits(acc[3]) << 16);
        r.z = bf16_rne_bits(acc[4]) | (bf16_rne_bits(acc[5]) << 16);
        r.w = bf16_rne_bits(acc[6]) | (bf16_rne_bits(acc[7]) << 16);
        reinterpret_cast<u32x4 *>(a.outs[s] + int64_t(t) * a.H)[c] = r;
    }
}

// A fresh static-scratch workspace: the route-error word starts as "none",
// and the one-launch dispatch's counters and tagged tile counts as zero.
__global__ __launch_bounds__(256) void k_init_ws(unsigned long long *err, uint32_t *sync, uint32_t *tcount,
                                                 int ncount)
{
    if (threadIdx.x == 0) *err = kNoError;
    if (threadIdx.x < 48) sync[threadIdx.x] = 0u;
    for (int i = threadIdx.x; i < ncount; i += 256) tcount[i] = 0u;
}

// Dispatch of a round without tokens: every expert's range is empty.
__global__ __launch_bounds__(256) void k_zero_ends(int32_t *ends, int E)
{
    for (int e = threadIdx.x; e < E; e += 256) ends[e] = 0;
}

__global__ __launch_bounds__(256) void k_copy(const u32x4 *src, u32x4 *dst, int64_t n)
{
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
        dst[i] = src[i];
}

// ------------------------------------------------------------ executor ----

DispatchArgs make_dispatch_args(const RoundPlan &p)
{
    DispatchArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int s = 0; s < p.N; ++s) {
        SourceArgs &r = a.src[s];
        r.ids = p.ids[s];
        r.x = static_cast<const uint8_t *>(p.x[s]);
        r.w = p.w[s];
        r.scale = p.fp8 ? p.scale[s] : nullptr;
        r.sst = p.sst[s];
        r.ssg = p.ssg[s];
        r.off = p.tok_off[s];
        r.T = p.tok_off[s + 1] - p.tok_off[s];
        r.voff = p.voff[s];
    }
    for (int f = 0; f < p.F; ++f) {
        a.rows[f] = static_cast<uint8_t *>(p.rows[f]);
        a.scales[f] = p.scales[f];
        a.roww[f] = p.roww[f];
    }
    for (int s = 0; s <= p.N; ++s) a.tok_off[s] = p.tok_off[s];
    for (int s = 0; s < p.N; ++s) a.voff[s] = p.voff[s];
    a.h.N = p.N;
    a.h.ntok = p.ntok;
    a.h.K = p.K;
    a.h.E = p.E;
    a.h.E_loc = p.E_loc;
    a.h.alpha = p.alpha;
    a.h.nblk = p.nblk;
    a.h.cpitch = (p.nblk + 3) / 4 * 4;
    a.h.tile = p.tile;
    a.h.nvec = int(p.row_bytes / 16);
    a.h.G = p.G;
    a.h.fp8 = p.fp8;
    a.h.row_bytes = p.row_bytes;
    a.h.err = p.err;
    a.h.ends = p.ends;
    a.h.blkcnt = p.blkcnt;
    a.h.packed = p.packed;
    a.h.slot = p.slot;
    a.h.tcount = p.tcount;
    a.h.sync = p.sync;
    a.h.ready = p.ready;
    a.h.wait_polls = p.wait_polls;
    TileRec tr[kLayoutMaxTiles];
    const int ntr = layout_tiles(p, tr);
    for (int b = 0; b < ntr; ++b) {
        a.tiles[b].ids = p.ids[tr[b].src] + int64_t(tr[b].t0) * p.K;
        a.tiles[b].g0 = tr[b].g0;
        a.tiles[b].ns = tr[b].n | (tr[b].src << 16);
    }
    return a;
}

int vmax_for(int nvec)
{
    const int per = (nvec + kWave - 1) / kWave;
    if (per <= 1) return 1;
    if (per <= 2) return 2;
    if (per <= 4) return 4;
    return 8;
}

int launched_ok() { return hipGetLastError() == hipSuccess ? 0 : 1; }

// The first two sources of a round as leading scalar kernel arguments.  The
// library is built with kernel-argument preloading, so the hardware places
// a kernel's leading scalar arguments in SGPRs before its waves start; for
// rounds of at most two sources the one-kernel dispatch addresses its first
// loads (the row and every id) from these alone, with no fetch from the
// argument block in front of them.
struct FirstSources {
    bool two = false;          // the round has at most two sources
    bool reg = false;          // and eight ids per token, 16-byte aligned: ids in registers
    const uint8_t *x0 = nullptr, *x1 = nullptr;
    const int32_t *ids0 = nullptr, *ids1 = nullptr;
    int T0 = 0, T1 = 0;
};

FirstSources first_sources(const DispatchArgs &a)
{
    FirstSources f;
    f.two = a.h.N <= 2;
    f.x0 = a.src[0].x;
    f.ids0 = a.src[0].ids;
    f.T0 = a.src[0].T;
    if (a.h.N >= 2) {
        f.x1 = a.src[1].x;
        f.ids1 = a.src[1].ids;
        f.T1 = a.src[1].T;
    }
    f.reg = f.two && a.h.K == 8 &&
            ((reinterpret_cast<uintptr_t>(f.ids0) | reinterpret_cast<uintptr_t>(f.ids1)) & 15u) == 0;
    return f;
}

template <int VMAX>
int launch_fused_v(const DispatchArgs &a, bool k32, dim3 grid, size_t lds, hipStream_t st)
{
    const FirstSources f = first_sources(a);
#define AFD_FUSED(KM, FW)                                                                                          \
    hipLaunchKernelGGL((k_fused<VMAX, KM, FW>), grid, dim3(256), lds, st, f.x0, f.x1, f.ids0, f.ids1, f.T0, f.T1,     \
                       a.h.K, a.h.nvec, a)
    if (k32) {
        if (f.two) AFD_FUSED(32, kFusedFew);
        else AFD_FUSED(32, kFusedAny);
    } else {
        if (f.reg) AFD_FUSED(8, kFusedReg);
        else if (f.two) AFD_FUSED(8, kFusedFew);
        else AFD_FUSED(8, kFusedAny);
    }
#undef AFD_FUSED
    return launched_ok();
}

// One-launch dispatch: one workgroup per TB slots of the tiled token space
// (at least kLayoutMaxTiles + 1 workgroups: the first kLayoutMaxTiles also
// count a tile each, the next one also finishes the counts).
template <int VMAX>
int launch_onepass_v(const DispatchArgs &a, bool k32, int nslots, int E, int K, hipStream_t st)
{
    constexpr int TB = 4 * (VMAX >= 4 ? 1 : 4 / VMAX);
    const size_t scatter_lds = size_t(4) * (E + kWave) * 8 + size_t(4) * E * 4 + size_t(TB) * K * 4 + size_t(2) * E * 4;
    const size_t duty_lds = size_t(E + kWave) * 4;   // counts and lane spares, or the finisher's aligned scan
    const size_t lds = scatter_lds + duty_lds;
    const int nscatter = nslots / TB;
    const dim3 grid(nscatter > kLayoutMaxTiles + 1 ? nscatter : kLayoutMaxTiles + 1);
    if (k32) hipLaunchKernelGGL((k_dispatch1<32, VMAX>), grid, dim3(kD1Threads), lds, st, a);
    else hipLaunchKernelGGL((k_dispatch1<8, VMAX>), grid, dim3(kD1Threads), lds, st, a);
    return launched_ok();
}

template <int VMAX>
int launch_cached_v(const DispatchArgs &a, int lpt, hipStream_t st)
{
    const int tpb = 256 / lpt;
    const dim3 grid((a.h.ntok + tpb - 1) / tpb);
    const int T1 = a.h.N >= 2 ? a.src[1].T : 0;
    const bool few = a.h.N <= 2 && a.src[0].T <= 0xFFFF && T1 <= 0x7FFF && a.h.nvec <= 0x7FFFFF;
    const int T01 = few ? a.src[0].T | (T1 << 16) : 0;
    const int Knv = a.h.K | ((a.h.nvec & 0x7FFFFF) << 8);
    const uint8_t *x1 = a.h.N >= 2 ? a.src[1].x : nullptr;
    if (few)
        hipLaunchKernelGGL((k_scatter_cached<VMAX, true>), grid, dim3(256), 0, st, lpt, a.h.slot, a.src[0].x, x1, T01,
                           Knv, a);
    else
        hipLaunchKernelGGL((k_scatter_cached<VMAX, false>), grid, dim3(256), 0, st, lpt, a.h.slot, a.src[0].x, x1, T01,
                           Knv, a);
    return launched_ok();
}

// One workgroup per TB slots of the tiled token space (TB divides every
// tile size, and the slots are a whole number of tiles).
template <int VMAX>
int launch_scatter_v(const DispatchArgs &a, int nslots, int E, hipStream_t st)
{
    constexpr int TB = 4 * (VMAX >= 4 ? 1 : 4 / VMAX);
    const size_t lds = size_t(E) * 12;
    hipLaunchKernelGGL(k_scatter<VMAX>, dim3(nslots / TB), dim3(256), lds, st, a);
    return launched_ok();
}

// 16-byte columns per lane of a stage-one wavefront (two measured slower)
constexpr int kPartialVpl = 1;

StageArgs make_stage_args(const RoundPlan &p)
{
    StageArgs a;
    std::memset(&a, 0, sizeof(a));
    a.partials = p.partials;
    a.slot = p.slot;
    a.prow = p.prow;
    for (int s = 0; s <= p.N; ++s) a.tok_off[s] = p.tok_off[s];
    a.N = p.N;
    a.F = p.F;
    a.ntok = p.ntok;
    a.K = p.K;
    a.H = p.H;
    a.nvec = p.H / 8;
    a.nseg = (a.nvec + kWave - 1) / kWave;
    a.capacity = p.capacity;
    return a;
}

}  // namespace

int be_init_workspace(void *workspace, const WorkspacePlan &wp)
{
    // the error word "none", the one-launch dispatch's counters zero, and its
    // tagged tile counts zero (tag 0 is never a launch's tag)
    uint64_t hdr[32];
    std::memset(hdr, 0, sizeof(hdr));
    hdr[wp.err / 8] = kNoError;
    if (hipMemcpy(workspace, hdr, sizeof(hdr), hipMemcpyHostToDevice) != hipSuccess) return 1;
    if (hipMemset(static_cast<char *>(workspace) + wp.tcount, 0, wp.total - wp.tcount) != hipSuccess) return 1;
    return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}

int be_is_capturing(void *stream, int *capturing)
{
    hipStreamCaptureStatus stt = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &stt) != hipSuccess) return 1;
    *capturing = stt != hipStreamCaptureStatusNone;
    return 0;
}

int be_launch_dispatch(const RoundPlan &p, void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    const DispatchArgs a = make_dispatch_args(p);
    const bool k32 = p.K > 8;
    const int vm = vmax_for(a.h.nvec);
    if (p.cached) {
        if (p.ntok == 0) return 0;
        // lanes per token: the row's columns rounded up to 64, 128 or 256
        const int lpt = a.h.nvec <= 64 ? 64 : a.h.nvec <= 128 ? 128 : 256;
        const int per = (a.h.nvec + lpt - 1) / lpt;
        switch (per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : 8) {
        case 1: return launch_cached_v<1>(a, lpt, st);
        case 2: return launch_cached_v<2>(a, lpt, st);
        case 4: return launch_cached_v<4>(a, lpt, st);
        default: return launch_cached_v<8>(a, lpt, st);
        }
    }
    if (p.empty) {
        hipLaunchKernelGGL(k_zero_ends, dim3(1), dim3(256), 0, st, p.ends, p.E);
        return launched_ok();
    }
    if (p.onepass) {
        switch (vm) {
        case 1: return launch_onepass_v<1>(a, k32, p.voff[p.N], p.E, p.K, st);
        case 2: return launch_onepass_v<2>(a, k32, p.voff[p.N], p.E, p.K, st);
        case 4: return launch_onepass_v<4>(a, k32, p.voff[p.N], p.E, p.K, st);
        default: return launch_onepass_v<8>(a, k32, p.voff[p.N], p.E, p.K, st);
        }
    }
    if (p.fused) {
        // one block per token; 256 threads hold the row, VMAX columns each
        const int per = (a.h.nvec + 255) / 256;
        const int vm_f = per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : 8;
        const size_t lds = size_t(p.ntok) * p.K * 4;
        dim3 grid(p.ntok);
        switch (vm_f) {
        case 1: return launch_fused_v<1>(a, k32, grid, lds, st);
        case 2: return launch_fused_v<2>(a, k32, grid, lds, st);
        case 4: return launch_fused_v<4>(a, k32, grid, lds, st);
        default: return launch_fused_v<8>(a, k32, grid, lds, st);
        }
    }
    {
        // one workgroup per tile of 64, 128 or 256 tokens, one lane per token
        const int nw = p.tile / kWave;
        const size_t lds = size_t(nw) * (p.E + kWave) * 8 + size_t(nw) * p.E * 4;
        const dim3 grid(p.nblk), blk(p.tile);
        if (nw == 1) {
            if (k32) hipLaunchKernelGGL((k_layout<32, 1>), grid, blk, lds, st, a);
            else hipLaunchKernelGGL((k_layout<8, 1>), grid, blk, lds, st, a);
        } else if (nw == 2) {
            if (k32) hipLaunchKernelGGL((k_layout<32, 2>), grid, blk, lds, st, a);
            else hipLaunchKernelGGL((k_layout<8, 2>), grid, blk, lds, st, a);
        } else {
            if (k32) hipLaunchKernelGGL((k_layout<32, 4>), grid, blk, lds, st, a);
            else hipLaunchKernelGGL((k_layout<8, 4>), grid, blk, lds, st, a);
        }
    }
    if (launched_ok()) return 1;
    switch (vm) {
    case 1: return launch_scatter_v<1>(a, p.voff[p.N], p.E, st);
    case 2: return launch_scatter_v<2>(a, p.voff[p.N], p.E, st);
    case 4: return launch_scatter_v<4>(a, p.voff[p.N], p.E, st);
    default: return launch_scatter_v<8>(a, p.voff[p.N], p.E, st);
    }
}

int be_read_ends(const RoundPlan &p, void *stream, int32_t *host_ends, uint64_t *err_word)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(host_ends, p.ends, size_t(p.E) * 4, hipMemcpyDeviceToHost, st) != hipSuccess) return 1;
    if (hipMemcpyAsync(err_word, p.err, 8, hipMemcpyDeviceToHost, st) != hipSuccess) return 1;
    return hipStreamSynchronize(st) == hipSuccess ? 0 : 1;
}

int be_launch_combine(const RoundPlan &p, void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    CombineArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int f = 0; f < p.F; ++f) a.reply[f] = static_cast<const uint16_t *>(p.reply[f]);
    for (int f = 0; f < 4 && f < p.F; ++f) a.reply4[f] = a.reply[f];
    for (int s = 0; s < p.N; ++s) a.out[s] = static_cast<uint16_t *>(p.out[s]);
    for (int s = 0; s <= p.N; ++s) a.tok_off[s] = p.tok_off[s];
    a.N = p.N;
    a.ntok = p.ntok;
    a.K = p.K;
    a.H = p.H;
    a.nvec = p.H / 8;
    a.slot = p.slot;
    a.nseg = (a.nvec + kWave - 1) / kWave;
    const int64_t waves = int64_t(p.ntok) * a.nseg;
    dim3 grid(unsigned((waves + 3) / 4));
    const uint64_t rb0 = reinterpret_cast<uint64_t>(a.reply4[0]), rb1 = reinterpret_cast<uint64_t>(a.reply4[1]);
    // output rows of sources 0 and 1; with more sources out1 is null and
    // tokens from t1 on look their source up in the offsets
    const uint64_t out0 = reinterpret_cast<uint64_t>(a.out[0]);
    const uint64_t out1 = p.N == 2 ? reinterpret_cast<uint64_t>(a.out[1]) : 0;
    const int t1 = p.N > 1 ? p.tok_off[1] : p.ntok;
    // Streaming output stores when the output is small (decode-sized):
    // 0.13 us faster per 1 MiB decode round, presumably as fewer dirty lines
    // are left in L2 for the kernel's end to write back.  With 8 and 24 MiB
    // outputs they measured slower (by up to 1 us a round), with 16 MiB
    // within noise, so larger outputs keep the default policy.
    const bool nt = int64_t(p.ntok) * p.H * 2 <= kCombineStreamOutBytes;
#define AFD_COMBINE(NB, NT) \
    hipLaunchKernelGGL((k_combine<1, NB, NT>), grid, dim3(256), 0, st, a.slot, rb0, rb1, out0, out1, a.ntok, a.K, a.H, t1, a)
    if (p.F <= 2) {
        if (nt) AFD_COMBINE(2, true);
        else AFD_COMBINE(2, false);
    } else if (p.F <= 4) {
        if (nt) AFD_COMBINE(4, true);
        else AFD_COMBINE(4, false);
    } else {
        if (nt) AFD_COMBINE(0, true);
        else AFD_COMBINE(0, false);
    }
#undef AFD_COMBINE
    return launched_ok();
}

int be_launch_partial(const RoundPlan &p, int f, void *stream)
{
    constexpr int VPL = kPartialVpl;
    StageArgs a = make_stage_args(p);
    a.f = f;
    a.reply = static_cast<const uint16_t *>(p.reply[f]);
    a.nseg = (a.nvec + kWave * VPL - 1) / (kWave * VPL);
    const int64_t waves = int64_t(p.ntok) * a.nseg;
    dim3 grid(unsigned((waves + 3) / 4));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.combine == AFD_COMBINE_PER_STAGE_FP8)
        hipLaunchKernelGGL((k_partial<true, VPL>), grid, dim3(256), 0, st, a.slot, a.reply, a.K, a.H, a.nseg, a.ntok, a.f, a);
    else
        hipLaunchKernelGGL((k_partial<false, VPL>), grid, dim3(256), 0, st, a.slot, a.reply, a.K, a.H, a.nseg, a.ntok, a.f, a);
    return launched_ok();
}

int be_launch_last(const RoundPlan &p, int f, void *stream)
{
    StageArgs a = make_stage_args(p);
    a.f = f;
    a.reply = static_cast<const uint16_t *>(p.reply[f]);
    for (int s = 0; s < p.N; ++s) a.outs[s] = static_cast<uint16_t *>(p.out[s]);
    const int64_t waves = int64_t(p.ntok) * a.nseg;
    if (waves == 0) return 0;
    dim3 grid(unsigned((waves + 3) / 4));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.combine == AFD_COMBINE_PER_STAGE_FP8)
        hipLaunchKernelGGL(k_last<true>, grid, dim3(256), 0, st, a.slot, a.reply, a.K, a.H, a.nseg, a.ntok, a.f, a);
    else
        hipLaunchKernelGGL(k_last<false>, grid, dim3(256), 0, st, a.slot, a.reply, a.K, a.H, a.nseg, a.ntok, a.f, a);
    return launched_ok();
}

int be_launch_copy(const void *src, void *dst, int64_t bytes, void *stream)
{
    const int64_t n = bytes / 16;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) return 0;
    hipLaunchKernelGGL(k_copy, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n);
    return launched_ok();
}

int be_read_stall(uint32_t *dev_sync, void *stream, int clear, int *stalled)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint32_t v = 0;
    if (hipMemcpyAsync(&v, dev_sync + kSyncStall, 4, hipMemcpyDeviceToHost, st) != hipSuccess) return 1;
    if (hipStreamSynchronize(st) != hipSuccess) return 1;
    *stalled = v != 0;
    if (clear && v != 0) {
        const uint32_t zero = 0;
        if (hipMemcpyAsync(dev_sync + kSyncStall, &zero, 4, hipMemcpyHostToDevice, st) != hipSuccess) return 1;
        if (hipStreamSynchronize(st) != hipSuccess) return 1;
    }
    return 0;
}

int be_read_error(uint64_t *dev_err, void *stream, int clear, uint64_t *word)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(word, dev_err, 8, hipMemcpyDeviceToHost, st) != hipSuccess) return 1;
    if (hipStreamSynchronize(st) != hipSuccess) return 1;
    if (clear) {
        const uint64_t none = kNoError;
        if (hipMemcpyAsync(dev_err, &none, 8, hipMemcpyHostToDevice, st) != hipSuccess) return 1;
        if (hipStreamSynchronize(st) != hipSuccess) return 1;
    }
    return 0;
}

int be_device_sync() { return hipDeviceSynchronize() == hipSuccess ? 0 : 1; }

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int be_static_scratch(int *device, void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // this device's copy of the array, with the device current
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return 1;
        g_scratch_ptr[dev] = p;
    }
    *device = dev;
    *ptr = g_scratch_ptr[dev];
    return 0;
}

int be_init_static(void *workspace, const WorkspacePlan &wp)
{
    char *ws = static_cast<char *>(workspace);
    auto *err = reinterpret_cast<unsigned long long *>(ws + wp.err);
    hipLaunchKernelGGL(k_init_ws, dim3(1), dim3(256), 0, nullptr, err, reinterpret_cast<uint32_t *>(ws + kSyncOffset),
                       reinterpret_cast<uint32_t *>(ws + wp.tcount), int((wp.total - wp.tcount) / 4));
    if (launched_ok()) return 1;
    return hipStreamSynchronize(nullptr) == hipSuccess ? 0 : 1;
}

}  // namespace afd
