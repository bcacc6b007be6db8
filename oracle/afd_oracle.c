/*
 * afd_oracle.c -- plain CPU reference of the AFD expert-parallel dispatch and
 * combine (the "hot path" of the afdEP-comm exchange), written from the
 * afdEP-comm design and API-contract pages.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links, includes or calls
 * this file; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no source, header, table or helper
 * with the GPU path.
 *
 * Everything here is plain loops, in the order the method defines it, and
 * single-threaded.  Build: gcc -std=c99 -O2 -ffp-contract=off -fPIC -shared.
 * A second build with -fopenmp exists for timing only: it runs the row copy
 * and the combine's token loop on several threads (every token's rows and
 * output are its own, so the results are the same bits); counting, the
 * aligned prefix and the slots stay serial.
 *
 * Pins (tests/): layout against an independent brute-force sort and
 * invariants; combine against the float64 closed form with identity experts,
 * a scipy.sparse routing-matrix product and exact special cases; number
 * formats against torch's casts.  The per-stage combine (one BF16 partial
 * per FFN partition, optionally carried as E4M3 with power-of-two scales,
 * then a float32 sum of the partials) is pinned by composition with the
 * pinned single-rounding combine, an E4M3 encoder checked against torch's
 * cast, scale exponents against their closed form, and hand-derived values
 * that fix the order in which partials are added.
 *
 * Notation: N sources (s), T[s] tokens each, K choices per token, E experts,
 * F partitions owning E_loc = E/F consecutive experts each, alignment alpha,
 * hidden size H.  Tokens are numbered globally g = sum_{s'<s} T[s'] + t, so
 * increasing g is the (source, token) order.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_BAD_CONFIG (-1)

/* Route classification codes (shared meaning with the library's error word,
 * but defined here independently). */
#define ORC_ROUTE_RANGE 1
#define ORC_ROUTE_NEG 2
#define ORC_ROUTE_DUP 3

static int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

/* ---- number formats ---------------------------------------------------- */

/* bfloat16 is the upper half of an IEEE binary32 pattern. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round binary32 to bfloat16, nearest with ties to even; NaN -> 0x7FC0. */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return 0x7FC0;
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* float8_e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
 * is subnormal (step 2^-9); 0x7F / 0xFF are NaN; no infinities. */
static float e4m3_to_f32(uint8_t q)
{
    int sign = q >> 7;
    int e = (q >> 3) & 0xF;
    int m = q & 7;
    float v;
    if (e == 0xF && m == 7) {
        uint32_t nan = 0x7FC00000u;
        memcpy(&v, &nan, 4);
        return v;
    }
    if (e == 0) {
        v = (float)m / 512.0f;                 /* m * 2^-9, exact */
    } else {
        float p = 1.0f;
        int k;
        if (e >= 7) for (k = 7; k < e; ++k) p *= 2.0f;
        else for (k = e; k < 7; ++k) p *= 0.5f;
        v = (1.0f + (float)m / 8.0f) * p;       /* exact in binary32 */
    }
    return sign ? -v : v;
}

/* ---- configuration and shapes (API contract page, "Roles and tensors") -- */

/* A round is valid when the hidden size is a positive multiple of 256, the
 * top-k satisfies 1 <= K <= min(32, E), the experts split evenly over the F
 * FFN partitions, the alignment is at least 1, and every source's token
 * count fits the bucket, which fits the capacity: 0 <= T[s] <= bucket <=
 * capacity.  There is at least one source and one partition, and a bucket
 * holds at least one token (reading: a bucket is the token count a capture
 * is specialised for, so an empty one specialises nothing).  Returns ORC_OK
 * or ORC_BAD_CONFIG. */
int orc_check_config(int N, const int32_t *T, int bucket, int capacity, int E, int F, int K, int H, int alpha)
{
    int s;
    if (N < 1 || E < 1 || F < 1 || K < 1 || alpha < 1 || H < 256) return ORC_BAD_CONFIG;
    if (H % 256 != 0) return ORC_BAD_CONFIG;
    if (K > 32 || K > E) return ORC_BAD_CONFIG;
    if (E % F != 0) return ORC_BAD_CONFIG;
    if (bucket < 1 || bucket > capacity) return ORC_BAD_CONFIG;
    for (s = 0; s < N; ++s)
        if (T[s] < 0 || T[s] > bucket) return ORC_BAD_CONFIG;
    return ORC_OK;
}

/* ---- layout ------------------------------------------------------------ */

/*
 * orc_layout: the receive layout of one round.
 *
 * Route rule (API contract page, "Roles and tensors"; design page section 8
 * on invalid routes): each id must be -1 (skip) or an expert in [0, E) that
 * is not already live at an earlier k of the same token.  Visiting (s,t,k)
 * in lexicographic order, a choice is
 *   -1             -> skipped
 *   < -1           -> NEG error, skipped
 *   >= E           -> RANGE error, skipped
 *   equal to a live id at an earlier k of the token -> DUP error, skipped
 *   otherwise      -> live.
 * The first error in that order is reported in err[0..3] = {code, s, t, k}
 * (code 0 when every route is valid).
 *
 * Ownership (same section): partition f owns experts [f*E_loc, (f+1)*E_loc).
 *
 * Prefix sums (API contract page, "receive prefix sum ends[e]"): expert j of
 * a partition occupies rows [align_up(ends[j-1], alpha), ends[j]) with
 * ends[-1] = 0, i.e. start_j = align_up(ends_{j-1}, alpha) and
 * ends_j = start_j + C_j with C_j its number of live choices.  Host counts
 * are the aligned counts align_up(C_j, alpha); the partition's exact row
 * count is align_up(ends_last, alpha).
 *
 * Row order inside an expert: ascending source, then ascending token (the
 * deterministic order this implementation fixes where the pages' atomics
 * leave any order valid).  A cursor per expert walks the live choices in
 * (s, t, k) order.
 *
 * Outputs: ends[E] (partition f's entry j at f*E_loc+j), host_counts[E],
 * rows_exact[F], slot_part/slot_row[ntok*K] (-1 where skipped), err[4].
 */
int orc_layout(int N, const int32_t *T, const int32_t *ids, int E, int F, int K, int alpha,
               int32_t *ends, int32_t *host_counts, int64_t *rows_exact,
               int32_t *slot_part, int32_t *slot_row, int32_t *err)
{
    int E_loc, s, t, k, kk, e, f, j;
    int64_t g, ntok = 0;
    int64_t *C, *start, *cursor;
    unsigned char *live;

    if (N < 1 || E < 1 || F < 1 || K < 1 || alpha < 1 || E % F != 0) return ORC_BAD_CONFIG;
    E_loc = E / F;
    for (s = 0; s < N; ++s) {
        if (T[s] < 0) return ORC_BAD_CONFIG;
        ntok += T[s];
    }
    C = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    start = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    cursor = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    live = (unsigned char *)calloc((size_t)(ntok * K + 1), 1);
    err[0] = err[1] = err[2] = err[3] = 0;

    /* 1. classify every choice */
    g = 0;
    for (s = 0; s < N; ++s) {
        for (t = 0; t < T[s]; ++t, ++g) {
            const int32_t *row = ids + g * K;
            for (k = 0; k < K; ++k) {
                int code = 0;
                e = row[k];
                if (e == -1) {
                    code = 0;                       /* skipped, no error */
                } else if (e < -1) {
                    code = ORC_ROUTE_NEG;
                } else if (e >= E) {
                    code = ORC_ROUTE_RANGE;
                } else {
                    int dup = 0;
                    for (kk = 0; kk < k; ++kk)
                        if (live[g * K + kk] && row[kk] == e) dup = 1;
                    if (dup) code = ORC_ROUTE_DUP;
                    else live[g * K + k] = 1;
                }
                if (code != 0 && err[0] == 0) {
                    err[0] = code; err[1] = s; err[2] = t; err[3] = k;
                }
            }
        }
    }

    /* 2. live count per expert */
    for (g = 0; g < ntok; ++g)
        for (k = 0; k < K; ++k)
            if (live[g * K + k]) C[ids[g * K + k]] += 1;

    /* 3. aligned prefix per partition */
    for (f = 0; f < F; ++f) {
        int64_t prev_end = 0;
        for (j = 0; j < E_loc; ++j) {
            e = f * E_loc + j;
            start[e] = align_up(prev_end, alpha);
            ends[e] = (int32_t)(start[e] + C[e]);
            host_counts[e] = (int32_t)align_up(C[e], alpha);
            prev_end = ends[e];
        }
        rows_exact[f] = align_up(prev_end, alpha);
    }

    /* 4. slots: (source, token) order inside each expert */
    for (g = 0; g < ntok; ++g) {
        for (k = 0; k < K; ++k) {
            if (live[g * K + k]) {
                e = ids[g * K + k];
                slot_part[g * K + k] = e / E_loc;
                slot_row[g * K + k] = (int32_t)(start[e] + cursor[e]);
                cursor[e] += 1;
            } else {
                slot_part[g * K + k] = -1;
                slot_row[g * K + k] = -1;
            }
        }
    }
    free(C); free(start); free(cursor); free(live);
    return ORC_OK;
}

/* ---- dispatch ---------------------------------------------------------- */

/*
 * orc_dispatch: expert-major receive rows (API contract page, worker_receive
 * returns expert-major rows and their weights; DeepEP's copy epilogue writes
 * each received token into its expert slots).  For every live choice
 * (g, k) -> (f, row): rows_f[row] = x[g] byte for byte and
 * row_w_f[row] = w[g][k].  Padding rows are left untouched.
 * x is the concatenation of every source's [T, H] rows (row_bytes each).
 */
void orc_dispatch(int64_t ntok, int K, const uint8_t *x, int64_t row_bytes, const float *w,
                  const int32_t *slot_part, const int32_t *slot_row,
                  uint8_t *const *rows, float *const *row_w)
{
    int64_t g;
    int k;
#pragma omp parallel for private(k) schedule(static)
    for (g = 0; g < ntok; ++g) {
        for (k = 0; k < K; ++k) {
            int32_t f = slot_part[g * K + k];
            int32_t r = slot_row[g * K + k];
            if (f < 0) continue;
            memcpy(rows[f] + (int64_t)r * row_bytes, x + g * row_bytes, (size_t)row_bytes);
            row_w[f][r] = w[g * K + k];
        }
    }
}

/*
 * orc_dispatch_scales: FP8 block scales travel with their rows (API contract
 * page: FP32 block-128 scales [T, H/128], strided views allowed).  Source
 * s's scale of token t, block b, is at scale_src[s][t*stride_t[s] +
 * b*stride_g[s]]; the receive side stores them densely, [rows, G].
 */
void orc_dispatch_scales(int N, const int32_t *T, int K, int G, const float *const *scale_src,
                         const int64_t *stride_t, const int64_t *stride_g,
                         const int32_t *slot_part, const int32_t *slot_row, float *const *scales)
{
    int s, t, k, b;
    int64_t g = 0;
    for (s = 0; s < N; ++s) {
        for (t = 0; t < T[s]; ++t, ++g) {
            for (k = 0; k < K; ++k) {
                int32_t f = slot_part[g * K + k];
                int32_t r = slot_row[g * K + k];
                if (f < 0) continue;
                for (b = 0; b < G; ++b)
                    scales[f][(int64_t)r * G + b] =
                        scale_src[s][(int64_t)t * stride_t[s] + (int64_t)b * stride_g[s]];
            }
        }
    }
}

/* ---- identity experts (the synthetic FFN stand-in) ---------------------- */

/*
 * Expert e's reply scales its row by s_e = 1 + e/E and rounds to bfloat16:
 * y = bf16(x * s_e) for BF16 rows, y = bf16((q * scale_b) * s_e) for FP8
 * rows (two float32 products, each rounded).  Rows of partition f's local
 * expert j are [align_up(ends[j-1], alpha), ends[j]); other rows of y are
 * not written.
 */
static float expert_scale(int e, int E) { return 1.0f + (float)e / (float)E; }

void orc_identity_experts(int fp8, int E, int F, int f, int alpha, int H, const int32_t *ends,
                          const uint8_t *rows, const float *scales, uint16_t *y)
{
    int E_loc = E / F, j, h;
    int64_t prev_end = 0, r;
    int G = H / 128;
    for (j = 0; j < E_loc; ++j) {
        int e = f * E_loc + j;
        int64_t st = align_up(prev_end, alpha);
        int64_t en = ends[e];
        float se = expert_scale(e, E);
        for (r = st; r < en; ++r) {
            for (h = 0; h < H; ++h) {
                float v;
                if (fp8) {
                    float xv = e4m3_to_f32(rows[r * H + h]) * scales[r * G + h / 128];
                    v = xv * se;
                } else {
                    uint16_t b;
                    memcpy(&b, rows + (r * H + h) * 2, 2);
                    v = bf16_to_f32(b) * se;
                }
                y[r * H + h] = f32_to_bf16_rne(v);
            }
        }
        prev_end = en;
    }
}

/* ---- combine ----------------------------------------------------------- */

/*
 * orc_combine: the source-side result (API contract page, source_collect:
 * BF16 [T, H] summed over the selected experts in original token order; the
 * routing weight is applied exactly once).  Replies are unweighted expert
 * outputs, so per element
 *     out[g][h] = bf16( sum over live k, ascending, of w[g][k] * y[slot][h] )
 * accumulated in float32 from +0 (each product rounded, then added).  A token
 * with no live choice gives +0 (design page section 13: rows of tokens with
 * no valid route are zero).
 */
void orc_combine(int64_t ntok, int K, int H, const float *w, const int32_t *slot_part,
                 const int32_t *slot_row, const uint16_t *const *y, uint16_t *out)
{
    int64_t g;
    int k, h;
#pragma omp parallel private(k, h)
    {
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);   /* one accumulator row per thread */
#pragma omp for schedule(static)
    for (g = 0; g < ntok; ++g) {
        for (h = 0; h < H; ++h) acc[h] = 0.0f;
        for (k = 0; k < K; ++k) {
            int32_t f = slot_part[g * K + k];
            int32_t r = slot_row[g * K + k];
            float wk = w[g * K + k];
            if (f < 0) continue;
            for (h = 0; h < H; ++h) {
                float p = wk * bf16_to_f32(y[f][(int64_t)r * H + h]);
                acc[h] = acc[h] + p;
            }
        }
        for (h = 0; h < H; ++h) out[g * H + h] = f32_to_bf16_rne(acc[h]);
    }
    free(acc);
    }
}

/* Threads the row copy and the combine use: 1, or the OpenMP team size in
 * the timing build. */
int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Exposed for the number-format pins. */
void orc_bf16_round(const float *in, uint16_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

void orc_e4m3_decode(const uint8_t *in, float *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = e4m3_to_f32(in[i]);
}

/* ---- per-stage combine (design page: two-domain rounding in section 6, ---
 * ---- FP8 combine replies in section 19) --------------------------------- */

/*
 * float8_e4m3fn encoding: the representable value nearest to v, ties to the
 * even code (even mantissa).  Magnitudes at or above 448, the largest finite
 * value, give 448 (only an infinite input reaches that here: the scaling
 * below keeps every finite input within 448).  NaN keeps its sign and gives
 * the NaN code.  Found by a binary search over the 127 non-negative codes,
 * whose values increase with the code.
 */
static uint8_t f32_to_e4m3_rne(float v)
{
    uint32_t u;
    uint8_t sign;
    double a, lo_v, hi_v;
    int lo = 0, hi = 126, c;
    memcpy(&u, &v, 4);
    sign = (u >> 31) ? 0x80 : 0x00;
    if (v != v) return (uint8_t)(sign | 0x7F);
    a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    while (lo < hi) {                       /* largest code with value <= a */
        int mid = (lo + hi + 1) / 2;
        if ((double)e4m3_to_f32((uint8_t)mid) <= a) lo = mid;
        else hi = mid - 1;
    }
    c = lo;
    lo_v = (double)e4m3_to_f32((uint8_t)c);
    if (lo_v != a) {
        hi_v = (double)e4m3_to_f32((uint8_t)(c + 1));
        if (hi_v - a < a - lo_v || (hi_v - a == a - lo_v && ((c + 1) & 1) == 0)) c = c + 1;
    }
    return (uint8_t)(sign | c);
}

/*
 * Exponent e of a 128-element group's power-of-two scale (section 19): the
 * smallest integer with amax <= 448 * 2^e, but at least -117, so that every
 * nonzero dequantised value stays a normal float32; an infinite amax takes
 * the top scale 2^120, the largest exponent any finite BF16 amax needs.
 */
static int fp8_group_exponent(float amax)
{
    int e = -117;
    if (isinf(amax)) return 120;
    while ((double)amax > 448.0 * ldexp(1.0, e)) e += 1;
    return e;
}

/* Bytes of one FP8 partial row (section 19's row format): H codes, then one
 * scale byte 127 + e per group, padded to a multiple of 32. */
int64_t orc_fp8_row_bytes(int H)
{
    return (int64_t)H + (H / 128 + 31) / 32 * 32;
}

/*
 * orc_combine_partials: stage one, on the FFN side.  Partition f reduces
 * each token's live rows that it holds (design page, section 6: the
 * hybrid combine rounds each FFN partial to BF16 before the cross-domain
 * sum):
 *     partial[f][g][h] = bf16( sum over live k of g with slot_part == f,
 *                              ascending, of w[g][k] * y_f[row][h] )
 * in float32 from +0, each product rounded and then added.  has[f*ntok+g]
 * is 1 when token g has a live choice in f (only then is the row written).
 */
void orc_combine_partials(int64_t ntok, int K, int H, int F, const float *w, const int32_t *slot_part,
                          const int32_t *slot_row, const uint16_t *const *y, uint16_t *partial, uint8_t *has)
{
    int64_t g;
    int k, h, f;
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);
    for (f = 0; f < F; ++f) {
        for (g = 0; g < ntok; ++g) {
            int any = 0;
            for (h = 0; h < H; ++h) acc[h] = 0.0f;
            for (k = 0; k < K; ++k) {
                int32_t row = slot_row[g * K + k];
                float wt = w[g * K + k];
                if (slot_part[g * K + k] != f) continue;
                any = 1;
                for (h = 0; h < H; ++h) {
                    float prod = wt * bf16_to_f32(y[f][(int64_t)row * H + h]);
                    acc[h] = acc[h] + prod;
                }
            }
            has[(int64_t)f * ntok + g] = (uint8_t)any;
            if (!any) continue;
            for (h = 0; h < H; ++h) partial[((int64_t)f * ntok + g) * H + h] = f32_to_bf16_rne(acc[h]);
        }
    }
    free(acc);
}

/*
 * orc_quantize_fp8_row: the FP8 form of one BF16 partial row (section 19).
 * Per group of 128 elements: amax over the magnitudes of its non-NaN
 * elements (0 if none), e = fp8_group_exponent(amax), code of element i =
 * e4m3(v_i * 2^-e) (the scaling is exact), scale byte 127 + e stored after
 * the H codes; the row's padding bytes are zero.
 */
void orc_quantize_fp8_row(int H, const uint16_t *partial, uint8_t *dst)
{
    int G = H / 128, b, i;
    int64_t n = orc_fp8_row_bytes(H);
    for (i = H + G; i < n; ++i) dst[i] = 0;
    for (b = 0; b < G; ++b) {
        float amax = 0.0f;
        int e;
        for (i = 0; i < 128; ++i) {
            float v = fabsf(bf16_to_f32(partial[b * 128 + i]));
            if (v == v && v > amax) amax = v;
        }
        e = fp8_group_exponent(amax);
        for (i = 0; i < 128; ++i)
            dst[b * 128 + i] = f32_to_e4m3_rne(ldexpf(bf16_to_f32(partial[b * 128 + i]), -e));
        dst[H + b] = (uint8_t)(127 + e);
    }
}

/*
 * orc_combine_stages: stage two, on the source side (section 19: the
 * source dequantises each FFN row and sums the rows in float32 in slot
 * order, the ascending order of the last top-k lane that maps to each
 * partition, then rounds once to BF16).  For token g the partitions holding
 * a live choice are visited in ascending order of their last live k;
 *     out[g][h] = bf16( +0 + value_f0[h] + value_f1[h] + ... )
 * where value is the BF16 partial (fp8 = 0) or, from the FP8 row,
 * e4m3(code) * 2^(scale byte - 127) (fp8 = 1).  Tokens without a live
 * choice give +0.  partial is [F][ntok][H] BF16; qrows is [F][ntok][row]
 * bytes with row = orc_fp8_row_bytes(H).
 */
void orc_combine_stages(int64_t ntok, int K, int H, int fp8, const int32_t *slot_part,
                        const uint16_t *partial, const uint8_t *qrows, uint16_t *out)
{
    int64_t g, rb = orc_fp8_row_bytes(H);
    int k, kk, h;
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);
    for (g = 0; g < ntok; ++g) {
        for (h = 0; h < H; ++h) acc[h] = 0.0f;
        for (k = 0; k < K; ++k) {
            int32_t f = slot_part[g * K + k];
            int last = 1;
            if (f < 0) continue;
            for (kk = k + 1; kk < K; ++kk)
                if (slot_part[g * K + kk] == f) last = 0;
            if (!last) continue;
            for (h = 0; h < H; ++h) {
                float v;
                if (fp8) {
                    const uint8_t *row = qrows + ((int64_t)f * ntok + g) * rb;
                    v = ldexpf(e4m3_to_f32(row[h]), (int)row[H + h / 128] - 127);
                } else {
                    v = bf16_to_f32(partial[((int64_t)f * ntok + g) * H + h]);
                }
                acc[h] = acc[h] + v;
            }
        }
        for (h = 0; h < H; ++h) out[g * H + h] = f32_to_bf16_rne(acc[h]);
    }
    free(acc);
}

/* Exposed for the encoder pin. */
void orc_e4m3_encode(const float *in, uint8_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = f32_to_e4m3_rne(in[i]);
}
