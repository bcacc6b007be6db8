/*
 * afd.h -- C ABI of the MI355X AFD expert-parallel dispatch/combine library.
 *
 * The four role calls mirror the afdEP-comm API contract page ("Roles and
 * tensors": source_dispatch, worker_receive, worker_reply, source_collect).
 * On one GPU a single context plays every role: N Attention sources and F
 * FFN partitions are logical slices of one device's memory.
 *
 *   dispatch: each source's tokens x[T,H] and top-k expert ids become
 *             expert-major receive rows of the partition owning the expert,
 *             with per-expert prefix sums ends[] (contract page: expert e
 *             occupies [align_up(ends[e-1], alpha), ends[e]), ends[-1] = 0).
 *             Inside an expert, rows are ordered by source, then token.
 *   combine:  every token's live reply rows are weighted once by their
 *             routing weight, summed in float32 in ascending k and rounded
 *             once to bfloat16, in the original token order.
 *
 * Conventions for every call:
 *   - Pointers named "device" are device (HBM) addresses; everything else
 *     is host memory.  The caller allocates all device memory: the
 *     workspace (sized by afd_query), the per-partition receive arenas,
 *     inputs, outputs and replies.  The library allocates no device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All GPU work of a call is enqueued on it; there is no internal stream.
 *   - A negative status means nothing was enqueued and the context state is
 *     unchanged -- except AFD_E_ROUTE, which reports invalid routes found by
 *     a call that finished its work and synchronised (see afd_get_error).
 *   - A context is single-threaded: calls on one context must not overlap.
 */
#ifndef AFD_H
#define AFD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AFD_MAX_SOURCES 16
#define AFD_MAX_PARTITIONS 16
#define AFD_MAX_EXPERTS 512
#define AFD_MAX_TOPK 32
/* Bytes of the static scratch array per GPU behind afd_create_static. */
#define AFD_STATIC_SCRATCH_BYTES (64u << 20)

typedef struct afd_ctx afd_ctx;

typedef enum {
    AFD_OK = 0,
    AFD_E_ARG = -1,       /* bad pointer, flag, bucket or option */
    AFD_E_SHAPE = -2,     /* bad configuration or tensor shape */
    AFD_E_ORDER = -3,     /* call out of the round order */
    AFD_E_CAPACITY = -4,  /* a buffer is smaller than the round needs */
    AFD_E_ROUTE = -5,     /* invalid expert ids were seen (work was done) */
    AFD_E_HIP = -6,       /* a HIP runtime call failed */
    AFD_E_TIMEOUT = -7    /* a one-launch dispatch gave up waiting between workgroups */
} afd_status;

typedef enum { AFD_BF16 = 0, AFD_FP8_E4M3 = 1 } afd_dtype;

/*
 * How the combine rounds (afdEP-comm design page; section 6 on rounding per
 * reduction stage, section 19 on FP8 combine replies).
 *   AFD_COMBINE_ONCE           one float32 sum over every live choice of a
 *                              token in ascending k, rounded once to BF16;
 *                              runs at the round's last worker_reply.
 *   AFD_COMBINE_PER_STAGE      the shape of a combine spread over FFN GPUs:
 *                              worker_reply(f) reduces partition f's live
 *                              rows of every token into one BF16 partial
 *                              (float32 sum in ascending k, one rounding);
 *                              stage two sums each token's partials in
 *                              float32, partitions ordered by the last live
 *                              top-k lane that maps to them, and rounds once
 *                              (on one GPU the round's last worker_reply
 *                              runs its own stage one and this stage for
 *                              every source, in one launch).
 *   AFD_COMBINE_PER_STAGE_FP8  as AFD_COMBINE_PER_STAGE, but each partial
 *                              is carried as E4M3 codes with one
 *                              power-of-two scale per 128 elements: e is the
 *                              smallest integer with amax <= 448 * 2^e, at
 *                              least -117 (an infinite amax gives 120);
 *                              code = e4m3(v * 2^-e) to nearest even (an
 *                              infinite value saturates to 448); the row is
 *                              H codes, then H/128 bytes 127 + e, zero padded
 *                              to H + align32(H/128) bytes.  Lossy: at most
 *                              amax/16 of its group per element.
 * The per-stage modes need num_partitions >= 2 (with one partition the
 * single partial is the final result).
 */
typedef enum { AFD_COMBINE_ONCE = 0, AFD_COMBINE_PER_STAGE = 1, AFD_COMBINE_PER_STAGE_FP8 = 2 } afd_combine_mode;

/*
 * How a round's dispatch is launched (design page, section 16: counts
 * first, then the expansion).  Rounds of at most 512 tokens always take the
 * one-kernel dispatch, and cached rounds the cached scatter.
 *   AFD_DISPATCH_AUTO        the library chooses (currently AFD_DISPATCH_SPLIT)
 *   AFD_DISPATCH_SPLIT       a layout kernel over token tiles, then the scatter
 *   AFD_DISPATCH_ONE_LAUNCH  one launch: its first 32 workgroups count one
 *                            tile each and publish the counts; the next one
 *                            waits for them and publishes every tile's
 *                            first row per expert; every other workgroup
 *                            ranks its tokens inside their tile itself,
 *                            waits for its tile's first rows (bounded waits
 *                            throughout) and scatters.  Applies to rounds of
 *                            at most 32 tiles (8192 token slots) and 256
 *                            experts; other rounds take the split path.
 */
typedef enum { AFD_DISPATCH_AUTO = 0, AFD_DISPATCH_SPLIT = 1, AFD_DISPATCH_ONE_LAUNCH = 2 } afd_dispatch_mode;

/* Route error codes (contract page: ids unique per token, in [0, E), or -1). */
typedef enum { AFD_ROUTE_NONE = 0, AFD_ROUTE_RANGE = 1, AFD_ROUTE_NEG = 2, AFD_ROUTE_DUP = 3 } afd_route_code;

/*
 * Configuration (contract page, "Roles and tensors").
 *   num_sources      N Attention sources, 1..AFD_MAX_SOURCES
 *   num_partitions   F FFN partitions, 1..AFD_MAX_PARTITIONS; partition f owns
 *                    experts [f*E/F, (f+1)*E/F)
 *   num_experts      E, divisible by F, at most AFD_MAX_EXPERTS
 *   topk             K, 1 <= K <= min(32, E)
 *   hidden           H, a positive multiple of 256
 *   expert_alignment alpha >= 1: every expert's first row is a multiple of it
 *   capacity         the largest bucket (tokens per source) ever used
 *   dtype            activation format: BF16, or float8_e4m3fn with FP32
 *                    block-128 scales [T, H/128]
 *   combine          afd_combine_mode (fixed for the context's lifetime)
 *   dispatch         afd_dispatch_mode (fixed for the context's lifetime)
 */
typedef struct {
    int32_t num_sources;
    int32_t num_partitions;
    int32_t num_experts;
    int32_t topk;
    int32_t hidden;
    int32_t expert_alignment;
    int32_t capacity;
    int32_t dtype;   /* afd_dtype */
    int32_t combine;  /* afd_combine_mode */
    int32_t dispatch; /* afd_dispatch_mode */
} afd_config;

/* Opaque receipt (contract page: keep it unchanged through the matching
 * reply).  Identifies the round and the partition. */
typedef struct {
    uint64_t round;
    int32_t partition;
    int32_t reserved;
} afd_receipt;

/* What worker_receive hands a partition (contract page: expert-major rows,
 * weights, device expert prefix sums and an opaque receipt).  All pointers
 * are device views into the partition's bound arena or the workspace. */
typedef struct {
    void *rows;             /* device [receive_rows, H] BF16 or E4M3, expert-major */
    float *scales;          /* device [receive_rows, H/128] FP32 (FP8 only, else NULL) */
    float *weights;         /* device [receive_rows] FP32 routing weight of each row
                               (informational: the combine applies the weights) */
    const int32_t *ends;    /* device [E/F] prefix sums of the local experts */
    int64_t receive_rows;   /* exact with read_host_counts, else the conservative bound */
    afd_receipt receipt;
} afd_receive;

/*
 * afd_query: workspace bytes for `cfg`, and the conservative receive-row
 * bound of one partition at `bucket` tokens per source:
 *     R_max(bucket) = N * bucket * min(K, E/F) + (E/F) * (alpha - 1),
 * which bounds sum_j align_up(C_j, alpha) for every routing (contract page:
 * without host counts the receive capacity is conservative and counts only
 * Attention sources).  Pure host computation.  Either output may be NULL.
 * Errors: AFD_E_SHAPE for an invalid config, AFD_E_ARG for a bucket outside
 * [1, capacity].
 */
afd_status afd_query(const afd_config *cfg, int32_t bucket, size_t *workspace_bytes, int64_t *rows_bound);

/*
 * afd_create (contract page: the Buffer, which owns the exchange's state and
 * storage, and whose set-up and close() happen outside graph capture): make a
 * context over a caller-owned device workspace of at least afd_query bytes
 * (256-byte aligned).  Initialises the workspace's error word and counters
 * with a synchronous device write, so it is not for a capturing stream.  The
 * workspace must stay allocated until afd_destroy.
 * Errors: AFD_E_SHAPE (config), AFD_E_ARG (NULL or misaligned pointer),
 * AFD_E_CAPACITY (workspace too small), AFD_E_HIP.
 */
afd_status afd_create(const afd_config *cfg, void *workspace, size_t workspace_bytes, afd_ctx **out);

/*
 * afd_create_static: afd_create for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  It takes no workspace: the context's workspace is the
 * library's static scratch array on the current device,
 * AFD_STATIC_SCRATCH_BYTES (64 MiB) per GPU, held from the library's first
 * use of that device until the process ends, and its host state is static
 * storage too.  The caller still allocates and binds the receive arenas and
 * passes inputs, outputs and replies; every later call works as on a context
 * from afd_create.  It calls no hipMalloc, hipFree or other allocating
 * routine; it launches one tiny kernel on the null stream and waits for it,
 * so (like afd_create) it is called outside capture.  One such context may
 * exist per device at a time: all of them share the device's array, which
 * keeps the last round's contents, so rounds that overlap on one device
 * race.  afd_destroy releases it.
 * Errors: AFD_E_ARG (NULL), AFD_E_SHAPE (config), AFD_E_CAPACITY (the
 * config's workspace, afd_query's bytes, exceeds AFD_STATIC_SCRATCH_BYTES),
 * AFD_E_ORDER (the device's static context exists), AFD_E_HIP.
 */
afd_status afd_create_static(const afd_config *cfg, afd_ctx **out);

/*
 * afd_bind_partition (contract page, "Graphs, streams and lifetime": receive
 * tensors are distinct from the registered transport buffers, and FFN
 * bounds count the Attention sources): bind partition f's receive arena
 * (device, caller-owned), sized for the conservative receive bound:
 *   rows        [rows_cap, H] BF16 or E4M3 (16-byte aligned)
 *   scales      [rows_cap, H/128] FP32, FP8 only (NULL for BF16)
 *   row_weights [rows_cap] FP32
 * Call between rounds, or inside a round until its first afd_worker_receive
 * has enqueued the dispatch work (so a receive that failed with
 * AFD_E_CAPACITY can be retried after binding a larger arena); never while a
 * stream is being captured.  Every round needs rows_cap >= R_max(bucket).
 * Errors: AFD_E_ARG (index, NULL or misaligned pointer), AFD_E_ORDER (the
 * round's dispatch work is already enqueued).
 */
afd_status afd_bind_partition(afd_ctx *ctx, int32_t f, void *rows, float *scales, float *row_weights,
                              int64_t rows_cap);

/* afd_destroy (contract page: close() synchronises outstanding work and
 * frees the Buffer's storage; graphs are destroyed before it): synchronise
 * the device and free the host context.  Frees no device memory (the caller
 * owns it).  Replaying a graph that captured calls on the context after
 * this is undefined.  NULL is accepted. */
afd_status afd_destroy(afd_ctx *ctx);

/*
 * afd_source_dispatch (contract page: source_dispatch(x, ids, weights,
 * x_scale, bucket, read_host_counts)).  Records source s's round inputs;
 * enqueues nothing (the layout and scatter of every source run together at
 * the round's first afd_worker_receive, which reads each x row once).
 *   x        device [T, H] contiguous, BF16 or E4M3 (16-byte aligned)
 *   ids      device [T, K] int32: -1 skips a choice
 *   weights  device [T, K] FP32
 *   x_scale  device FP32, element (t, b) at x_scale[t*stride_t + b*stride_g]
 *            for b < H/128 (FP8 only; NULL for BF16); strides >= 0
 *   out_bf16 device [T, H] BF16 result (16-byte aligned); required when F > 1,
 *            optional when F == 1 (then only source_collect(view=1) is valid)
 * T = 0 is an empty source (x, ids, weights may be NULL).  Needs
 * T <= bucket <= capacity; bucket and read_host_counts must be the same on
 * every call of a round.  x, ids, weights and x_scale must stay unchanged
 * until the round's dispatch work has run (stream order covers this when
 * they are produced on the same stream).
 * Errors: AFD_E_ORDER (s already dispatched this round, or the previous
 * round is not collected), AFD_E_ARG, AFD_E_SHAPE.
 */
afd_status afd_source_dispatch(afd_ctx *ctx, int32_t s, int32_t T, const void *x, const int32_t *ids,
                               const float *weights, const float *x_scale, int64_t scale_stride_t,
                               int64_t scale_stride_g, void *out_bf16, int32_t bucket,
                               int32_t read_host_counts, void *stream);

/*
 * afd_source_dispatch_cached (ElasticBuffer page, "Cached Dispatch": a
 * dispatch given the handle of an earlier one reuses its layout, skipping
 * the layout computation and any host synchronisation).  Records source s's
 * round inputs like afd_source_dispatch, but without ids: the round reuses
 * the receive layout of the last round whose dispatch work was enqueued on
 * this context (every slot, ends[] and the route-error word stay as that
 * round left them), so its dispatch is the scatter of x, scales and the new
 * weights alone.  The caller guarantees that the routes are unchanged; the
 * new weights are applied (row weights and the combine).
 *   T must equal source s's token count in that layout, and bucket its
 *   bucket; read_host_counts is not available (the round never syncs).
 * Every source of a round must dispatch the same way (all cached or none).
 * Errors: AFD_E_ORDER (no layout yet, or mixed with afd_source_dispatch in
 * a round, or out of round order), AFD_E_SHAPE (T differs from the layout),
 * AFD_E_ARG (pointers, alignment, bucket).
 */
afd_status afd_source_dispatch_cached(afd_ctx *ctx, int32_t s, int32_t T, const void *x, const float *weights,
                                      const float *x_scale, int64_t scale_stride_t, int64_t scale_stride_g,
                                      void *out_bf16, int32_t bucket, void *stream);

/*
 * afd_worker_receive (contract page: worker_receive(bucket,
 * read_host_counts)).  Needs every source dispatched.  The round's first
 * receive enqueues the route check, layout and scatter for ALL partitions on
 * `stream`; later receives enqueue nothing.  With read_host_counts = 1 the
 * first receive synchronises `stream` and host_counts (if not NULL) gets the
 * aligned per-expert counts align_up(C_j, alpha) of partition f, and
 * receive_rows is exact; not allowed while `stream` is being captured.
 * Errors: AFD_E_ORDER, AFD_E_ARG, AFD_E_CAPACITY (arena smaller than
 * R_max(bucket)), AFD_E_HIP, AFD_E_ROUTE (read_host_counts = 1 and the
 * sticky error word is set: the call completed, the outputs hold the
 * sanitised layout with invalid choices skipped).
 */
afd_status afd_worker_receive(afd_ctx *ctx, int32_t f, int32_t bucket, int32_t read_host_counts,
                              int32_t *host_counts, afd_receive *out, void *stream);

/*
 * afd_worker_reply (contract page: worker_reply(rows, receipt)).  reply_bf16
 * is device [receive_rows, H] BF16 covering the entire receive shape, with
 * each live row's expert output in place; replies are unweighted (the
 * combine applies each routing weight exactly once).  Padding rows are never
 * read.  AFD_COMBINE_ONCE: the round's last reply enqueues the combine for
 * every source on `stream`; every reply must be complete in `stream` order
 * by then.  Per-stage modes: each reply enqueues partition f's stage one
 * (its partials, from its own reply only) on `stream`; the round's last
 * reply enqueues its stage one and stage two for every source as one
 * launch (every earlier reply's stage one must be complete in `stream`
 * order by then).
 * Errors: AFD_E_ORDER (not received, already replied, or a receipt of
 * another round or partition), AFD_E_ARG.
 */
afd_status afd_worker_reply(afd_ctx *ctx, int32_t f, const void *reply_bf16, int64_t receive_rows,
                            const afd_receipt *receipt, void *stream);

/*
 * afd_source_collect (contract page: source_collect(view)).  Needs every
 * partition replied.  *result is device BF16 [T, H] in token order with row
 * stride *row_stride elements.
 *   F > 1: the source's out_bf16, complete in the order of the stream of
 *          the round's last reply (nothing is enqueued).
 *   F = 1, view = 1: a read-only view of the source's combine inbox in the
 *          workspace, valid until the next afd_source_dispatch (design page
 *          section 13); nothing is enqueued.
 *   F = 1, view = 0: the inbox is copied into out_bf16 on `stream`.
 * Errors: AFD_E_ORDER, AFD_E_ARG (view = 0 without out_bf16), AFD_E_HIP.
 */
afd_status afd_source_collect(afd_ctx *ctx, int32_t s, int32_t view, const void **result,
                              int64_t *row_stride, void *stream);

/*
 * afd_set_dispatch_wait: the number of polls a workgroup of a one-launch
 * dispatch makes for what another workgroup publishes (the tile counts, or
 * its tile's first rows) before it gives up (default
 * 1,000,000, about a second; a negative value gives up at once).  A
 * workgroup that gives up stores no rows and marks its tokens' choices as
 * skipped, so the round's outputs are defined (its tokens' outputs are +0);
 * afd_get_error then reports AFD_E_TIMEOUT.  Host state only.
 * Errors: AFD_E_ARG (NULL).
 */
afd_status afd_set_dispatch_wait(afd_ctx *ctx, int32_t polls);

/*
 * afd_get_error: synchronise `stream` and read the sticky route-error word:
 * the first invalid choice in (source, token, k) order among every round
 * since the last clear, with its code (afd_route_code).  Invalid choices are
 * skipped everywhere (count, rank, scatter, combine), so nothing is written
 * out of bounds.  clear = 1 resets the word.  Outputs may be NULL.
 * Returns AFD_OK (no error), AFD_E_ROUTE (word set), AFD_E_TIMEOUT (a
 * one-launch dispatch gave up waiting since the last clear; sticky the same
 * way, reported before route errors), AFD_E_ARG (stream capturing),
 * AFD_E_HIP.
 */
afd_status afd_get_error(afd_ctx *ctx, void *stream, int32_t clear, int32_t *code, int32_t *s, int32_t *t,
                         int32_t *k);

/*
 * afd_get_partials: where the per-stage combine keeps source s's stage-one
 * rows from partition f (the source's combine inbox region for that FFN on
 * the design page).  *rows is device memory inside the workspace, T rows of
 * *row_bytes bytes: BF16 [H] for AFD_COMBINE_PER_STAGE, the FP8 row format
 * above for AFD_COMBINE_PER_STAGE_FP8.  A token's row is written only when
 * it has a live choice in f; other rows are unspecified.  Read-only; valid
 * from partition f's reply until its reply in the next round.  Enqueues
 * nothing.  Errors: AFD_E_ARG (index, NULL, or AFD_COMBINE_ONCE).
 */
afd_status afd_get_partials(afd_ctx *ctx, int32_t s, int32_t f, const void **rows, int64_t *row_bytes);

/* How a round's dispatch ran (afd_round_info.dispatch_path). */
typedef enum {
    AFD_PATH_NONE = 0,        /* no dispatch enqueued yet */
    AFD_PATH_ONE_KERNEL = 1,  /* small rounds: layout and scatter in one kernel */
    AFD_PATH_TILED = 2,       /* layout kernel over token tiles, then the scatter */
    AFD_PATH_CACHED = 3,      /* afd_source_dispatch_cached: the scatter alone */
    AFD_PATH_EMPTY = 4,       /* no tokens: ends[] cleared */
    AFD_PATH_ONE_LAUNCH = 5   /* AFD_DISPATCH_ONE_LAUNCH: counting and scatter in one launch */
} afd_dispatch_path;

typedef struct {
    uint64_t round;            /* the round described (0: none yet) */
    int32_t dispatch_path;     /* afd_dispatch_path */
    int32_t dispatch_kernels;  /* kernels the round's dispatch launched */
    int32_t combine_kernels;   /* kernels its combine launches: 1 (AFD_COMBINE_ONCE
                                  with tokens), F (per stage, with tokens), 0 */
    int32_t tokens;            /* tokens over every source */
    int32_t layout_tiles;      /* AFD_PATH_TILED: layout workgroups; else 0 */
    int32_t tile_tokens;       /* AFD_PATH_TILED: token slots per layout tile; else 0 */
} afd_round_info;

/*
 * afd_get_round_info (design page, "3:1 Attention:FFN: where the time goes",
 * which accounts a round kernel by kernel): which kernels the last round
 * whose dispatch work was enqueued runs, for per-kernel accounting.  Host
 * state only; enqueues nothing and never synchronises.
 * Errors: AFD_E_ARG (NULL).
 */
afd_status afd_get_round_info(const afd_ctx *ctx, afd_round_info *info);

/* afd_status_string: a static description of a status. */
const char *afd_status_string(afd_status st);

#ifdef __cplusplus
}
#endif
#endif /* AFD_H */
