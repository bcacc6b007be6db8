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
//             scatters its own four tokens.  One launch for the dispatch.
//   k_layout  dispatch, larger rounds, step 1: 512-token tiles; per 64-token
//             chunk an LDS bit mask per expert gives each choice its rank
//             (popcount of the lanes below it); the last tile to finish scans
//             the tile counts into ends[] and per-tile row bases.
//   k_scatter dispatch, step 2: one wavefront per token copies the row once
//             from HBM into registers and stores it to each live slot.
//   k_combine one wavefront per (token, column segment): gathers the live
//             reply rows with 16-byte loads, float32 multiply-then-add in
//             ascending k, rounds once to bfloat16.
//   k_copy    inbox -> caller output (single-partition collect without view).
//
// Nothing here uses MFMA: the round is data movement plus one multiply-add
// per reply element, bound by HBM bandwidth.

#include <hip/hip_runtime.h>

#include <cstring>

#include "afd_plan.h"

namespace afd {
namespace {

constexpr int kWave = 64;

// 16-byte vector as a native clang vector (keeps register arrays in VGPRs).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- args ----

struct DispatchArgs {
    const int32_t *ids[kMaxSources];
    const uint8_t *x[kMaxSources];
    const float *w[kMaxSources];
    const float *scale[kMaxSources];
    int64_t sst[kMaxSources];
    int64_t ssg[kMaxSources];
    uint8_t *rows[kMaxParts];
    float *scales[kMaxParts];
    float *roww[kMaxParts];
    int tok_off[kMaxSources + 1];
    int N, ntok, K, E, E_loc, alpha, nblk, nvec, G;
    int64_t row_bytes;
    uint64_t *err;
    uint32_t *counter;
    int32_t *ends;
    int32_t *blkcnt;
    int32_t *blkbase;
    int32_t *packed;
    int32_t *slot;
};

struct CombineArgs {
    const uint16_t *reply[kMaxParts];
    uint16_t *out[kMaxSources];
    int tok_off[kMaxSources + 1];
    int N, ntok, K, H, nvec, nseg;
    const int32_t *slot;
};

// ------------------------------------------------------------- helpers ----

__device__ __forceinline__ int src_of(const int *tok_off, int N, int g)
{
    int s = 0;
    while (s + 1 < N && g >= tok_off[s + 1]) ++s;
    return s;
}

__device__ __forceinline__ uint64_t make_err(int s, int t, int k, unsigned code)
{
    return (uint64_t(s) << 56) | (uint64_t(uint32_t(t)) << 24) | (uint64_t(k) << 16) | uint64_t(code);
}

__device__ __forceinline__ int align_up_i(int v, int a) { return (v + a - 1) / a * a; }

__device__ __forceinline__ int load_agent(const int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix sum of vals[0..n) (LDS), in place, by a block of BLOCK
// threads; each thread owns ceil(n / BLOCK) consecutive entries.
template <int BLOCK>
__device__ void block_exclusive_scan(int *vals, int n, int *wave_tot)
{
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int per = (n + BLOCK - 1) / BLOCK;
    const int lo = tid * per;
    const int hi = lo + per < n ? lo + per : n;
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += vals[i];
    int x = sum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    if (lane == kWave - 1) wave_tot[tid / kWave] = x;
    __syncthreads();
    if (tid < kWave) {
        const int v = tid < BLOCK / kWave ? wave_tot[tid] : 0;
        int xi = v;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(xi, d, kWave);
            if (tid >= d) xi += y;
        }
        if (tid < BLOCK / kWave) wave_tot[tid] = xi - v;
    }
    __syncthreads();
    int run = wave_tot[tid / kWave] + x - sum;
    for (int i = lo; i < hi; ++i) {
        const int v = vals[i];
        vals[i] = run;
        run += v;
    }
    __syncthreads();
}

// Classify the K choices of one token (route rule of the contract page) and
// mark the live ones in the chunk's per-expert lane masks.  A duplicate is
// detected by the token's own bit already being set in the expert's mask.
template <int KMAX>
__device__ __forceinline__ uint32_t classify_token(const int (&ev)[KMAX], int K, int E, unsigned long long *mask_row,
                                                   unsigned long long bit, int s, int t, uint64_t &err)
{
    uint32_t live = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k >= K) break;
        const int e = ev[k];
        unsigned code = 0;
        if (e == -1) {
        } else if (e < -1) {
            code = AFD_ROUTE_NEG;
        } else if (e >= E) {
            code = AFD_ROUTE_RANGE;
        } else {
            const unsigned long long old = atomicOr(&mask_row[e], bit);
            if (old & bit) code = AFD_ROUTE_DUP;
            else live |= 1u << k;
        }
        if (code != 0 && err == kNoError) err = make_err(s, t, k, code);
    }
    return live;
}

// Store one token's row to each of its live slots, plus the slot map, the
// per-row weights and (FP8) the block scales.  `part`/`row` of choice k are
// held by lane k.  The first chunk of the row is already in v[].
template <int VMAX>
__device__ __forceinline__ void scatter_token(const DispatchArgs &a, int g, int s, int t, int lane, int part,
                                              int row, const u32x4 *xs, u32x4 (&v)[VMAX])
{
    const int K = a.K;
    if (lane < K) {
        const float wk = a.w[s][int64_t(t) * K + lane];
        int2 sl;
        sl.x = part < 0 ? -1 : ((part << 24) | row);
        sl.y = __float_as_int(wk);
        reinterpret_cast<int2 *>(a.slot)[int64_t(g) * K + lane] = sl;
        if (part >= 0) a.roww[part][row] = wk;
    }
    const int nvec = a.nvec;
    for (int base = 0; base < nvec; base += kWave * VMAX) {
        if (base > 0) {
#pragma unroll
            for (int i = 0; i < VMAX; ++i) {
                const int c = base + i * kWave + lane;
                if (c < nvec) v[i] = xs[c];
            }
        }
        for (int k = 0; k < K; ++k) {
            const int pr = __builtin_amdgcn_readlane(part, k);
            if (pr < 0) continue;
            const int rw = __builtin_amdgcn_readlane(row, k);
            u32x4 *dst = reinterpret_cast<u32x4 *>(a.rows[pr] + int64_t(rw) * a.row_bytes);
#pragma unroll
            for (int i = 0; i < VMAX; ++i) {
                const int c = base + i * kWave + lane;
                if (c < nvec) dst[c] = v[i];
            }
        }
    }
    if (a.scale[s] != nullptr) {
        const float *sc = a.scale[s] + int64_t(t) * a.sst[s];
        const int G = a.G;
        for (int k = 0; k < K; ++k) {
            const int pr = __builtin_amdgcn_readlane(part, k);
            if (pr < 0) continue;
            const int rw = __builtin_amdgcn_readlane(row, k);
            float *dst = a.scales[pr] + int64_t(rw) * G;
            for (int b = lane; b < G; b += kWave) dst[b] = sc[int64_t(b) * a.ssg[s]];
        }
    }
}

// ------------------------------------------------------------- kernels ----

// Dispatch in one kernel (rounds of at most kFusedMaxTokens tokens).
// Block = 4 wavefronts; block b scatters tokens 4b..4b+3 (one per wavefront)
// after building the full layout in LDS.
template <int VMAX, int KMAX>
__global__ __launch_bounds__(256) void k_fused(DispatchArgs a)
{
    extern __shared__ __align__(16) unsigned char lds[];
    __shared__ int s_tot[4];
    const int E = a.E, K = a.K, ntok = a.ntok;
    const int nchunk = (ntok + kWave - 1) / kWave;
    unsigned long long *mask = reinterpret_cast<unsigned long long *>(lds);  // [nchunk][E]
    int *pre = reinterpret_cast<int *>(mask + size_t(nchunk) * E);            // [nchunk][E]
    int *pfx = pre + size_t(nchunk) * E;                                      // [E]
    uint32_t *livebits = reinterpret_cast<uint32_t *>(pfx + E);               // [ntok]

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int g = blockIdx.x * 4 + tid / kWave;
    const bool mine = g < ntok;

    // 1. start this wavefront's row load; its latency overlaps the layout
    int s = 0, t = 0;
    const u32x4 *xs = nullptr;
    u32x4 v[VMAX];
    if (mine) {
        s = src_of(a.tok_off, a.N, g);
        t = g - a.tok_off[s];
        xs = reinterpret_cast<const u32x4 *>(a.x[s] + int64_t(t) * a.row_bytes);
#pragma unroll
        for (int i = 0; i < VMAX; ++i) {
            const int c = i * kWave + lane;
            if (c < a.nvec) v[i] = xs[c];
        }
    }

    // 2. route check and per-chunk lane masks of every token
    for (int i = tid; i < nchunk * E; i += 256) mask[i] = 0ull;
    __syncthreads();
    uint64_t err = kNoError;
    for (int gg = tid; gg < ntok; gg += 256) {
        const int ss = src_of(a.tok_off, a.N, gg);
        const int tt = gg - a.tok_off[ss];
        const int32_t *idp = a.ids[ss] + int64_t(tt) * K;
        int ev[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) ev[k] = k < K ? idp[k] : -1;
        livebits[gg] = classify_token<KMAX>(ev, K, E, mask + size_t(gg / kWave) * E, 1ull << (gg % kWave), ss, tt, err);
    }
    if (blockIdx.x == 0 && err != kNoError) atomicMin(reinterpret_cast<unsigned long long *>(a.err), err);
    __syncthreads();

    // 3. per expert: exclusive prefix over chunks; aligned total
    for (int e = tid; e < E; e += 256) {
        int run = 0;
        for (int c = 0; c < nchunk; ++c) {
            pre[c * E + e] = run;
            run += __popcll(mask[c * E + e]);
        }
        pfx[e] = align_up_i(run, a.alpha);
    }
    __syncthreads();
    // pfx[e] = sum of aligned counts of experts < e (all partitions); the
    // start of expert e inside its partition is pfx[e] - pfx[first of part]
    block_exclusive_scan<256>(pfx, E, s_tot);

    if (blockIdx.x == 0) {
        for (int e = tid; e < E; e += 256) {
            const int C = nchunk ? pre[(nchunk - 1) * E + e] + __popcll(mask[(nchunk - 1) * E + e]) : 0;
            a.ends[e] = pfx[e] - pfx[(e / a.E_loc) * a.E_loc] + C;
        }
    }
    if (!mine) return;

    // 4. rows of this wavefront's token: lane k holds choice k
    int part = -1, row = -1;
    if (lane < K && ((livebits[g] >> lane) & 1u)) {
        const int e = a.ids[s][int64_t(t) * K + lane];
        const int c = g / kWave;
        const unsigned long long below = (1ull << (g % kWave)) - 1ull;
        row = pfx[e] - pfx[(e / a.E_loc) * a.E_loc] + pre[c * E + e] + __popcll(mask[c * E + e] & below);
        part = e / a.E_loc;
    }
    scatter_token<VMAX>(a, g, s, t, lane, part, row, xs, v);
}

// Layout of larger rounds.  Block = 8 wavefronts = one 512-token tile; lane
// = token.  packed[g][k] = (expert << 16) | rank of the choice among the
// tile's choices of that expert, or -1.  The last tile to arrive scans the
// tile counts into ends[] and blkbase[tile][e] (first row of the tile's run).
template <int KMAX>
__global__ __launch_bounds__(512) void k_layout(DispatchArgs a)
{
    extern __shared__ __align__(16) unsigned char lds[];
    __shared__ int s_tot[8];
    __shared__ int s_last;
    const int E = a.E, K = a.K;
    unsigned long long *mask = reinterpret_cast<unsigned long long *>(lds);  // [8][E]
    int *pre = reinterpret_cast<int *>(mask + size_t(8) * E);                 // [8][E]
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    const int g = blockIdx.x * kLayoutTile + tid;

    for (int i = tid; i < 8 * E; i += 512) mask[i] = 0ull;
    __syncthreads();
    int ev[KMAX];
    uint32_t live = 0;
    const bool have = g < a.ntok;
    if (have) {
        const int s = src_of(a.tok_off, a.N, g);
        const int t = g - a.tok_off[s];
        const int32_t *idp = a.ids[s] + int64_t(t) * K;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) ev[k] = k < K ? idp[k] : -1;
        uint64_t err = kNoError;
        live = classify_token<KMAX>(ev, K, E, mask + size_t(wave) * E, 1ull << lane, s, t, err);
        if (err != kNoError) atomicMin(reinterpret_cast<unsigned long long *>(a.err), err);
    }
    __syncthreads();
    for (int e = tid; e < E; e += 512) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            pre[w * E + e] = run;
            run += __popcll(mask[w * E + e]);
        }
        a.blkcnt[blockIdx.x * E + e] = run;
    }
    __syncthreads();
    if (have) {
        const unsigned long long below = (1ull << lane) - 1ull;
        int32_t *pk = a.packed + int64_t(g) * K;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) break;
            int val = -1;
            if ((live >> k) & 1u) {
                const int e = ev[k];
                val = (e << 16) | (pre[wave * E + e] + __popcll(mask[wave * E + e] & below));
            }
            pk[k] = val;
        }
    }

    // last tile to finish: scan the tile counts
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(a.counter, 1u) == unsigned(a.nblk - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    int *A = pre;  // reuse LDS: [E]
    int C = 0;
    if (tid < E) {
        for (int b = 0; b < a.nblk; ++b) C += load_agent(a.blkcnt + b * E + tid);
        A[tid] = align_up_i(C, a.alpha);
    }
    __syncthreads();
    block_exclusive_scan<512>(A, E, s_tot);
    if (tid < E) {
        const int start = A[tid] - A[(tid / a.E_loc) * a.E_loc];
        a.ends[tid] = start + C;
        int run = start;
        for (int b = 0; b < a.nblk; ++b) {
            a.blkbase[b * E + tid] = run;
            run += load_agent(a.blkcnt + b * E + tid);
        }
    }
    if (tid == 0) __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Scatter of larger rounds: one wavefront per token.
template <int VMAX>
__global__ __launch_bounds__(256) void k_scatter(DispatchArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int g = blockIdx.x * 4 + threadIdx.x / kWave;
    if (g >= a.ntok) return;
    const int s = src_of(a.tok_off, a.N, g);
    const int t = g - a.tok_off[s];
    const u32x4 *xs = reinterpret_cast<const u32x4 *>(a.x[s] + int64_t(t) * a.row_bytes);
    u32x4 v[VMAX];
#pragma unroll
    for (int i = 0; i < VMAX; ++i) {
        const int c = i * kWave + lane;
        if (c < a.nvec) v[i] = xs[c];
    }
    int part = -1, row = -1;
    if (lane < a.K) {
        const int pk = a.packed[int64_t(g) * a.K + lane];
        if (pk >= 0) {
            const int e = pk >> 16;
            row = a.blkbase[(g / kLayoutTile) * a.E + e] + (pk & 0xFFFF);
            part = e / a.E_loc;
        }
    }
    scatter_token<VMAX>(a, g, s, t, lane, part, row, xs, v);
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Combine: one wavefront per (token, segment of 64*VPL 16-byte columns).
template <int VPL>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a)
{
#pragma clang fp contract(off)
    const int lane = threadIdx.x & (kWave - 1);
    const int gw = blockIdx.x * 4 + threadIdx.x / kWave;
    const int g = gw / a.nseg;
    const int seg = gw - g * a.nseg;
    if (g >= a.ntok) return;
    const int s = src_of(a.tok_off, a.N, g);
    const int t = g - a.tok_off[s];
    int sl_row = -1, sl_w = 0;
    if (lane < a.K) {
        const int2 sl = reinterpret_cast<const int2 *>(a.slot)[int64_t(g) * a.K + lane];
        sl_row = sl.x;
        sl_w = sl.y;
    }
    const int nvec = a.nvec;
    const int c0 = seg * kWave * VPL + lane;
    float acc[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    for (int k0 = 0; k0 < a.K; k0 += 8) {
        u32x4 y[8][VPL];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int pr = __builtin_amdgcn_readlane(sl_row, k0 + kk);
            if (pr >= 0) {
                const u32x4 *src = reinterpret_cast<const u32x4 *>(a.reply[pr >> 24] + int64_t(pr & 0xFFFFFF) * a.H);
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int c = c0 + i * kWave;
                    y[kk][i] = c < nvec ? src[c] : u32x4{0u, 0u, 0u, 0u};
                }
            } else {
#pragma unroll
                for (int i = 0; i < VPL; ++i) y[kk][i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int pr = __builtin_amdgcn_readlane(sl_row, k0 + kk);
            if (pr < 0) continue;
            const float w = __int_as_float(__builtin_amdgcn_readlane(sl_w, k0 + kk));
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
    u32x4 *o = reinterpret_cast<u32x4 *>(a.out[s] + int64_t(t) * a.H);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int c = c0 + i * kWave;
        if (c < nvec) {
            u32x4 r;
            r.x = bf16_rne_bits(acc[i][0]) | (bf16_rne_bits(acc[i][1]) << 16);
            r.y = bf16_rne_bits(acc[i][2]) | (bf16_rne_bits(acc[i][3]) << 16);
            r.z = bf16_rne_bits(acc[i][4]) | (bf16_rne_bits(acc[i][5]) << 16);
            r.w = bf16_rne_bits(acc[i][6]) | (bf16_rne_bits(acc[i][7]) << 16);
            o[c] = r;
        }
    }
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
        a.ids[s] = p.ids[s];
        a.x[s] = static_cast<const uint8_t *>(p.x[s]);
        a.w[s] = p.w[s];
        a.scale[s] = p.fp8 ? p.scale[s] : nullptr;
        a.sst[s] = p.sst[s];
        a.ssg[s] = p.ssg[s];
    }
    for (int f = 0; f < p.F; ++f) {
        a.rows[f] = static_cast<uint8_t *>(p.rows[f]);
        a.scales[f] = p.scales[f];
        a.roww[f] = p.roww[f];
    }
    for (int s = 0; s <= p.N; ++s) a.tok_off[s] = p.tok_off[s];
    a.N = p.N;
    a.ntok = p.ntok;
    a.K = p.K;
    a.E = p.E;
    a.E_loc = p.E_loc;
    a.alpha = p.alpha;
    a.nblk = p.nblk;
    a.nvec = int(p.row_bytes / 16);
    a.G = p.G;
    a.row_bytes = p.row_bytes;
    a.err = p.err;
    a.counter = p.counter;
    a.ends = p.ends;
    a.blkcnt = p.blkcnt;
    a.blkbase = p.blkbase;
    a.packed = p.packed;
    a.slot = p.slot;
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

template <int VMAX>
int launch_fused_v(const DispatchArgs &a, bool k32, dim3 grid, size_t lds, hipStream_t st)
{
    if (k32) hipLaunchKernelGGL((k_fused<VMAX, 32>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((k_fused<VMAX, 8>), grid, dim3(256), lds, st, a);
    return launched_ok();
}

template <int VMAX>
int launch_scatter_v(const DispatchArgs &a, dim3 grid, hipStream_t st)
{
    hipLaunchKernelGGL(k_scatter<VMAX>, grid, dim3(256), 0, st, a);
    return launched_ok();
}

}  // namespace

int be_init_workspace(void *workspace, const WorkspacePlan &wp)
{
    uint64_t hdr[32];
    std::memset(hdr, 0, sizeof(hdr));
    hdr[wp.err / 8] = kNoError;  // counter (at byte 8) stays 0
    if (hipMemcpy(workspace, hdr, sizeof(hdr), hipMemcpyHostToDevice) != hipSuccess) return 1;
    return 0;
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
    const int vm = vmax_for(a.nvec);
    if (p.fused) {
        const int nchunk = (p.ntok + kWave - 1) / kWave;
        const size_t lds = size_t(nchunk) * p.E * 12 + size_t(p.E) * 4 + size_t(p.ntok) * 4;
        dim3 grid(p.ntok > 0 ? (p.ntok + 3) / 4 : 1);
        switch (vm) {
        case 1: return launch_fused_v<1>(a, k32, grid, lds, st);
        case 2: return launch_fused_v<2>(a, k32, grid, lds, st);
        case 4: return launch_fused_v<4>(a, k32, grid, lds, st);
        default: return launch_fused_v<8>(a, k32, grid, lds, st);
        }
    }
    const size_t lds = size_t(8) * p.E * 12;
    if (k32) hipLaunchKernelGGL(k_layout<32>, dim3(p.nblk), dim3(512), lds, st, a);
    else hipLaunchKernelGGL(k_layout<8>, dim3(p.nblk), dim3(512), lds, st, a);
    if (launched_ok()) return 1;
    dim3 grid((p.ntok + 3) / 4);
    switch (vm) {
    case 1: return launch_scatter_v<1>(a, grid, st);
    case 2: return launch_scatter_v<2>(a, grid, st);
    case 4: return launch_scatter_v<4>(a, grid, st);
    default: return launch_scatter_v<8>(a, grid, st);
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
    for (int s = 0; s < p.N; ++s) a.out[s] = static_cast<uint16_t *>(p.out[s]);
    for (int s = 0; s <= p.N; ++s) a.tok_off[s] = p.tok_off[s];
    a.N = p.N;
    a.ntok = p.ntok;
    a.K = p.K;
    a.H = p.H;
    a.nvec = p.H / 8;
    a.slot = p.slot;
    const int64_t waves1 = int64_t(p.ntok) * ((a.nvec + kWave - 1) / kWave);
    int vpl = 1;
    if (waves1 >= 32768) vpl = 4;
    else if (waves1 >= 8192) vpl = 2;
    a.nseg = (a.nvec + kWave * vpl - 1) / (kWave * vpl);
    const int64_t waves = int64_t(p.ntok) * a.nseg;
    dim3 grid(unsigned((waves + 3) / 4));
    if (vpl == 4) hipLaunchKernelGGL(k_combine<4>, grid, dim3(256), 0, st, a);
    else if (vpl == 2) hipLaunchKernelGGL(k_combine<2>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(k_combine<1>, grid, dim3(256), 0, st, a);
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

}  // namespace afd
