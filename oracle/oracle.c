/*
 * CPU ORACLE for MoE token dispatch / combine -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded C.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no code
 * with the HIP implementation and never calls it.
 *
 * Source of the definitions: "NJU x Huawei UBEP: Reengineering MoE Expert
 * Parallelism" (kad8.com).
 *   - opening section: every token is sent to the device hosting each expert it
 *     selected, and the results are gathered back to the token in the Combine
 *     phase (dispatch / combine);
 *   - "BSP Serialization": the dispatch pipeline is send tokens, send token
 *     counts, calculate offsets, reorder tokens;
 *   - "Kernel Decomposition": metadata work is token counting, prefix sums and
 *     offset calculation.
 * The pages give no formula for any of these.  The readings taken here:
 *   - expert e lives on rank floor(e / (E/R)); token t belongs to source rank
 *     floor(t / (T/R)) and to chunk floor(t / (T/C));
 *   - one receive row per (token, slot) pair, no de-duplication;
 *   - a rank's receive region holds its rows in (token, slot) order and the
 *     regions are packed back to back in rank order;
 *   - combine is an fp32 fused-multiply-add chain over slots 0..k-1 starting
 *     from +0.0f, rounded once to bf16 (round to nearest, ties to even);
 *   - fp8 payload: per token and per block of 128 channels, scale
 *     s = amax / 448 (IEEE fp32 division; s = 1 when amax = 0) and code
 *     q = E4M3(x / s), rounded to nearest with ties to even and saturated at
 *     +-448 (OCP 8-bit floating point, E4M3 "FN" flavour: bias 7, no infinity).
 * Every function here computes exactly that definition with plain loops.
 *
 * The gate (router) step before the path follows the same pages' opening
 * section, where each token's gate selects the experts it is sent to; the
 * pages give no formula.  Readings taken here (oracle_gate):
 *   - the k experts with the largest logits, larger first, equal logits in
 *     ascending expert id;
 *   - group-limited routing: the E experts form `groups` contiguous groups; a
 *     group's score is its largest plus its second-largest logit (one fp32
 *     addition; the largest alone for one-expert groups); the keep_groups
 *     best groups (ties to the lower group id) are the only candidates;
 *   - every selection decision is an exact fp32 comparison of logits or of
 *     group scores;
 *   - weights over the selected experts: softmax, exp(z_j - z_max) / sum, or
 *     sigmoid-normalised, s(z_j) / sum s(z_i) with s(z) = 1 / (1 + exp(-z)),
 *     evaluated in double and rounded once to fp32.
 *
 * Parity status: every function is pinned by the CPU tests (library special
 * cases, brute force on tiny inputs, exact rational arithmetic, closed forms).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ------------------------------------------------------------------------ */
/* shape rules that the definition itself needs                             */
/* ------------------------------------------------------------------------ */
int oracle_check_shape(int64_t T, int64_t H, int32_t E, int32_t k, int32_t R, int32_t C,
                       int fp8)
{
    if (T <= 0 || H <= 0 || E <= 0 || k <= 0 || R <= 0 || C <= 0) return ORACLE_INVALID_ARG;
    if (k > E) return ORACLE_INVALID_ARG;            /* k distinct experts per token */
    if (E % R != 0) return ORACLE_INVALID_ARG;       /* equal expert blocks per rank  */
    if (T % R != 0) return ORACLE_INVALID_ARG;       /* equal token blocks per source */
    if (T % C != 0) return ORACLE_INVALID_ARG;       /* equal token blocks per chunk  */
    if (fp8 && H % 128 != 0) return ORACLE_INVALID_ARG; /* whole 128-channel blocks */
    if (T * (int64_t)k >= ((int64_t)1 << 30)) return ORACLE_INVALID_ARG;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* layout: counts -> exclusive prefix sums -> stable positions              */
/* ------------------------------------------------------------------------ */
int oracle_layout(int64_t T, int32_t E, int32_t k, int32_t R, int32_t C,
                  const int32_t *topk_idx,
                  int32_t *pos, int32_t *expert_count, int32_t *rank_count,
                  int32_t *recv_offset, int32_t *send_offset, int32_t *chunk_offset,
                  int32_t *recv_src)
{
    int st = oracle_check_shape(T, 8, E, k, R, C, 0);
    if (st != ORACLE_OK) return st;
    for (int64_t i = 0; i < T * k; ++i)
        if (topk_idx[i] < 0 || topk_idx[i] >= E) return ORACLE_BAD_EXPERT_ID;

    const int32_t epr = E / R;          /* experts per rank  */
    const int64_t tps = T / R;          /* tokens per source */
    const int64_t tpc = T / C;          /* tokens per chunk  */

    int32_t *sd_count = calloc((size_t)R * R, sizeof(int32_t));
    int32_t *cd_count = calloc((size_t)C * R, sizeof(int32_t));
    int32_t *cursor = calloc((size_t)R, sizeof(int32_t));
    if (!sd_count || !cd_count || !cursor) {
        free(sd_count); free(cd_count); free(cursor);
        return ORACLE_UNSUPPORTED;
    }

    /* 1. token counts */
    for (int32_t e = 0; e < E; ++e) expert_count[e] = 0;
    for (int32_t d = 0; d < R; ++d) rank_count[d] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = topk_idx[t * k + j];
            int32_t d = e / epr;
            int64_t s = t / tps;
            int64_t c = t / tpc;
            expert_count[e] += 1;
            rank_count[d] += 1;
            sd_count[s * R + d] += 1;
            cd_count[c * R + d] += 1;
        }
    }

    /* 2. exclusive prefix sums */
    recv_offset[0] = 0;
    for (int32_t d = 0; d < R; ++d) recv_offset[d + 1] = recv_offset[d] + rank_count[d];
    for (int32_t d = 0; d < R; ++d) {
        int32_t run = 0;
        for (int32_t s = 0; s < R; ++s) {
            send_offset[s * R + d] = run;
            run += sd_count[s * R + d];
        }
    }
    if (chunk_offset) {
        for (int32_t d = 0; d < R; ++d) {
            int32_t run = 0;
            for (int32_t c = 0; c < C; ++c) {
                chunk_offset[c * R + d] = run;
                run += cd_count[c * R + d];
            }
        }
    }

    /* 3. stable positions: rows in (destination rank, token, slot) order */
    for (int32_t d = 0; d < R; ++d) cursor[d] = recv_offset[d];
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t d = topk_idx[t * k + j] / epr;
            int32_t p = cursor[d]++;
            pos[t * k + j] = p;
            if (recv_src) recv_src[p] = (int32_t)(t * k + j);
        }
    }

    free(sd_count); free(cd_count); free(cursor);
    return ORACLE_OK;
}

/* Expert-grouped layout: the same counts and offsets as oracle_layout, but
 * the rows inside each rank's region are ordered by (expert, token, slot),
 * so each expert's rows are one contiguous run -- the order a grouped expert
 * computation reads.  (The pages fix only that each token goes to the
 * device of each expert it selected and comes back; the order inside a
 * region is this build's choice.)  Experts of rank d are E/R consecutive
 * ids, so the runs of rank d's experts tile region d in expert order:
 *   expert_offset[e] = sum of expert_count[e'] for e' < e  (E+1 entries),
 *   pos[t][j]        = expert_offset[e] + #{(t', j') < (t, j) : idx = e},
 *   recv_offset[d]   = expert_offset[d * E/R].
 * send_offset and chunk_offset keep their meaning as row counts
 * (rows to rank d from earlier source ranks / chunks). */
int oracle_layout_grouped(int64_t T, int32_t E, int32_t k, int32_t R, int32_t C,
                          const int32_t *topk_idx,
                          int32_t *pos, int32_t *expert_count, int32_t *expert_offset,
                          int32_t *rank_count, int32_t *recv_offset, int32_t *send_offset,
                          int32_t *chunk_offset, int32_t *recv_src)
{
    int st = oracle_check_shape(T, 8, E, k, R, C, 0);
    if (st != ORACLE_OK) return st;
    for (int64_t i = 0; i < T * k; ++i)
        if (topk_idx[i] < 0 || topk_idx[i] >= E) return ORACLE_BAD_EXPERT_ID;

    const int32_t epr = E / R;
    const int64_t tps = T / R;
    const int64_t tpc = T / C;

    int32_t *sd_count = calloc((size_t)R * R, sizeof(int32_t));
    int32_t *cd_count = calloc((size_t)C * R, sizeof(int32_t));
    int32_t *cursor = calloc((size_t)E, sizeof(int32_t));
    if (!sd_count || !cd_count || !cursor) {
        free(sd_count); free(cd_count); free(cursor);
        return ORACLE_UNSUPPORTED;
    }

    /* 1. token counts per expert, per rank, per (source, rank), per (chunk, rank) */
    for (int32_t e = 0; e < E; ++e) expert_count[e] = 0;
    for (int32_t d = 0; d < R; ++d) rank_count[d] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t e = topk_idx[t * k + j];
            int32_t d = e / epr;
            expert_count[e] += 1;
            rank_count[d] += 1;
            sd_count[(t / tps) * R + d] += 1;
            cd_count[(t / tpc) * R + d] += 1;
        }
    }

    /* 2. exclusive prefix sums: over experts, then the rank starts from them */
    expert_offset[0] = 0;
    for (int32_t e = 0; e < E; ++e) expert_offset[e + 1] = expert_offset[e] + expert_count[e];
    for (int32_t d = 0; d <= R; ++d) recv_offset[d] = expert_offset[d * epr];
    for (int32_t d = 0; d < R; ++d) {
        int32_t run = 0;
        for (int32_t s = 0; s < R; ++s) {
            send_offset[s * R + d] = run;
            run += sd_count[s * R + d];
        }
    }
    if (chunk_offset) {
        for (int32_t d = 0; d < R; ++d) {
            int32_t run = 0;
            for (int32_t c = 0; c < C; ++c) {
                chunk_offset[c * R + d] = run;
                run += cd_count[c * R + d];
            }
        }
    }

    /* 3. stable positions: rows in (expert, token, slot) order */
    for (int32_t e = 0; e < E; ++e) cursor[e] = expert_offset[e];
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t p = cursor[topk_idx[t * k + j]]++;
            pos[t * k + j] = p;
            if (recv_src) recv_src[p] = (int32_t)(t * k + j);
        }
    }

    free(sd_count); free(cd_count); free(cursor);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* number formats                                                           */
/* ------------------------------------------------------------------------ */
static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

float oracle_bf16_to_f32(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

/* Nearest bf16, ties to the even one.  bf16 keeps the top 16 bits of fp32;
 * `lo` drops the low 16 bits (toward zero), `hi` is the next bf16 away from
 * zero.  Compare the dropped half against one half unit. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u = bits_from_f32(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);   /* quiet NaN */
    uint32_t lo = u >> 16;
    uint32_t hi = lo + 1u;
    uint32_t rest = u & 0xFFFFu;
    if (rest < 0x8000u) return (uint16_t)lo;
    if (rest > 0x8000u) return (uint16_t)hi;
    return (uint16_t)((lo & 1u) ? hi : lo);
}

/* Closed-form E4M3FN value of a code: sign S, exponent field X (4 bits, bias 7),
 * mantissa M (3 bits).  X = 0 is subnormal 2^-6 * M/8; X = 15, M = 7 is NaN. */
float oracle_e4m3_to_f32(uint8_t c)
{
    int S = c >> 7, X = (c >> 3) & 15, M = c & 7;
    double v;
    if (X == 15 && M == 7) return NAN;
    if (X == 0) v = ldexp((double)M / 8.0, -6);
    else v = ldexp(1.0 + (double)M / 8.0, X - 7);
    return (float)(S ? -v : v);
}

/* Values of the 127 non-negative finite codes 0x00..0x7E, in increasing order. */
static double e4m3_value[127];
static int e4m3_value_ready = 0;

static void e4m3_build_values(void)
{
    for (int c = 0; c < 127; ++c) e4m3_value[c] = (double)oracle_e4m3_to_f32((uint8_t)c);
    e4m3_value_ready = 1;
}

/* Nearest E4M3FN code, ties to the even code, magnitudes beyond 448 saturate
 * to 448.  Binary-search the value table for the largest code not above |f|,
 * then compare the distances to it and to the next code; in double these
 * distances are exact for fp32 operands below 448. */
uint8_t oracle_f32_to_e4m3(float f)
{
    if (!e4m3_value_ready) e4m3_build_values();
    if (isnan(f)) return 0x7F;
    uint8_t sign = signbit(f) ? 0x80 : 0x00;
    double a = fabs((double)f);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int lo = 0, hi = 126;                       /* e4m3_value[lo] <= a < e4m3_value[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e4m3_value[mid] <= a) lo = mid; else hi = mid;
    }
    double dlo = a - e4m3_value[lo], dhi = e4m3_value[hi] - a;
    int pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = hi;
    else pick = (lo & 1) ? hi : lo;
    return (uint8_t)(sign | pick);
}

/* ------------------------------------------------------------------------ */
/* dispatch                                                                 */
/* ------------------------------------------------------------------------ */
void oracle_dispatch_bf16(int64_t T, int64_t H, int32_t k, const uint16_t *x,
                          const int32_t *pos, uint16_t *recv)
{
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j)
            memcpy(recv + (int64_t)pos[t * k + j] * H, x + t * H, (size_t)H * sizeof(uint16_t));
}

void oracle_dispatch_fp8(int64_t T, int64_t H, int32_t k, const uint16_t *x,
                         const int32_t *pos, uint8_t *recv8, float *recv_scale)
{
    const int64_t nb = H / 128;
    uint8_t q[128];
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t *xb = x + t * H + b * 128;
            float amax = 0.0f;
            for (int c = 0; c < 128; ++c) {
                float v = fabsf(oracle_bf16_to_f32(xb[c]));
                if (v > amax) amax = v;
            }
            float s = amax > 0.0f ? amax / 448.0f : 1.0f;
            for (int c = 0; c < 128; ++c) q[c] = oracle_f32_to_e4m3(oracle_bf16_to_f32(xb[c]) / s);
            for (int32_t j = 0; j < k; ++j) {
                int64_t p = pos[t * k + j];
                memcpy(recv8 + p * H + b * 128, q, 128);
                recv_scale[p * nb + b] = s;
            }
        }
    }
}

/* identity expert for an fp8 payload: y = bf16(decode(q) * s), one fp32 multiply */
void oracle_identity_fp8(int64_t rows, int64_t H, const uint8_t *q, const float *scale,
                         uint16_t *y)
{
    const int64_t nb = H / 128;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < H; ++c)
            y[r * H + c] = oracle_f32_to_bf16(oracle_e4m3_to_f32(q[r * H + c]) *
                                              scale[r * nb + c / 128]);
}

/* ------------------------------------------------------------------------ */
/* combine                                                                  */
/* ------------------------------------------------------------------------ */
void oracle_combine(int64_t T, int64_t H, int32_t k, const uint16_t *y, const int32_t *pos,
                    const float *topk_w, uint16_t *out)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t c = 0; c < H; ++c) {
            float acc = 0.0f;
            for (int32_t j = 0; j < k; ++j) {
                float v = oracle_bf16_to_f32(y[(int64_t)pos[t * k + j] * H + c]);
                acc = fmaf(topk_w[t * k + j], v, acc);
            }
            out[t * H + c] = oracle_f32_to_bf16(acc);
        }
    }
}

/* element-wise helpers exposed for the pins */
void oracle_f32_to_e4m3_array(int64_t n, const float *in, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_e4m3(in[i]);
}
void oracle_f32_to_bf16_array(int64_t n, const float *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]);
}
void oracle_e4m3_to_f32_array(int64_t n, const uint8_t *in, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_to_f32(in[i]);
}

/* ------------------------------------------------------------------------ */
/* gate: logits -> top-k expert ids and normalised weights                  */
/* ------------------------------------------------------------------------ */

/* a ranks before b: larger value first, equal values in ascending id */
static int gate_before(float va, int32_t a, float vb, int32_t b)
{
    return va > vb || (va == vb && a < b);
}

int oracle_gate(int64_t T, int32_t E, int32_t k, int32_t groups, int32_t keep_groups, int norm,
                const float *logits, int32_t *topk_idx, float *topk_w)
{
    if (T <= 0 || E <= 0 || k <= 0 || groups <= 0 || keep_groups <= 0) return ORACLE_INVALID_ARG;
    if (E % groups != 0 || keep_groups > groups) return ORACLE_INVALID_ARG;
    if (norm != ORACLE_GATE_SOFTMAX && norm != ORACLE_GATE_SIGMOID) return ORACLE_INVALID_ARG;
    const int32_t gsize = E / groups;
    if (k > keep_groups * gsize) return ORACLE_INVALID_ARG;
    unsigned char *allowed = malloc((size_t)E);
    unsigned char *taken = malloc((size_t)E);
    float *gscore = malloc(sizeof(float) * (size_t)groups);
    unsigned char *gtaken = malloc((size_t)groups);
    double *val = malloc(sizeof(double) * (size_t)k);
    if (!allowed || !taken || !gscore || !gtaken || !val) {
        free(allowed); free(taken); free(gscore); free(gtaken); free(val);
        return ORACLE_INVALID_ARG;
    }
    for (int64_t t = 0; t < T; ++t) {
        const float *z = logits + t * E;
        /* group scores: best plus second best logit of each group */
        for (int32_t g = 0; g < groups; ++g) {
            int32_t b1 = -1, b2 = -1;
            for (int32_t e = g * gsize; e < (g + 1) * gsize; ++e) {
                if (b1 < 0 || gate_before(z[e], e, z[b1], b1)) { b2 = b1; b1 = e; }
                else if (b2 < 0 || gate_before(z[e], e, z[b2], b2)) { b2 = e; }
            }
            gscore[g] = b2 < 0 ? z[b1] : z[b1] + z[b2];
            gtaken[g] = 0;
        }
        /* the keep_groups best groups */
        memset(allowed, 0, (size_t)E);
        for (int32_t r = 0; r < keep_groups; ++r) {
            int32_t best = -1;
            for (int32_t g = 0; g < groups; ++g)
                if (!gtaken[g] && (best < 0 || gate_before(gscore[g], g, gscore[best], best))) best = g;
            gtaken[best] = 1;
            for (int32_t e = best * gsize; e < (best + 1) * gsize; ++e) allowed[e] = 1;
        }
        /* the k best allowed experts, in rank order */
        memset(taken, 0, (size_t)E);
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e)
                if (allowed[e] && !taken[e] && (best < 0 || gate_before(z[e], e, z[best], best)))
                    best = e;
            taken[best] = 1;
            topk_idx[t * k + j] = best;
        }
        /* weights, in double, rounded once */
        double sum = 0.0;
        const double zmax = (double)z[topk_idx[t * k]];
        for (int32_t j = 0; j < k; ++j) {
            const double zj = (double)z[topk_idx[t * k + j]];
            val[j] = norm == ORACLE_GATE_SOFTMAX ? exp(zj - zmax) : 1.0 / (1.0 + exp(-zj));
            sum += val[j];
        }
        for (int32_t j = 0; j < k; ++j) topk_w[t * k + j] = (float)(val[j] / sum);
    }
    free(allowed); free(taken); free(gscore); free(gtaken); free(val);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* per-expert linear map (a real expert between dispatch and combine)       */
/* ------------------------------------------------------------------------ */

/* Nearest bf16 (ties to even) of a finite double, rounded once from the
 * double: 8 significant bits.  Results of magnitude below 2^-126 (bf16
 * subnormals) are outside what this oracle is used for and go through fp32. */
uint16_t oracle_f64_to_bf16(double v)
{
    if (v == 0.0) return signbit(v) ? 0x8000u : 0x0000u;
    if (fabs(v) < 0x1p-126) return oracle_f32_to_bf16((float)v);
    int ex;
    double m = frexp(v, &ex);            /* v = m * 2^ex, 0.5 <= |m| < 1 */
    double q = nearbyint(m * 256.0);     /* 8 significant bits, ties to even */
    float f = (float)ldexp(q, ex - 8);   /* exact: 8 bits fit in fp32 */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* y[r][n] = bf16( sum over c of x[r][c] * w[e][n][c] ) for every row r of
 * expert e's run [expert_offset[e], expert_offset[e+1]), the sum taken
 * in double (exact for H <= 2^22 products of bf16 values, up to the final
 * rounding of the sum itself) and rounded once to bf16.  x and y are bf16
 * [rows][H] and [rows][N]; w is bf16 [E][N][H] (row n of expert e's weight,
 * channels contiguous). */
void oracle_expert_linear(int32_t E, int64_t H, int64_t N, const int32_t *expert_offset,
                          const uint16_t *x, const uint16_t *w, uint16_t *y)
{
    for (int32_t e = 0; e < E; ++e) {
        const uint16_t *we = w + (int64_t)e * N * H;
        for (int64_t r = expert_offset[e]; r < expert_offset[e + 1]; ++r) {
            const uint16_t *xr = x + r * H;
            for (int64_t n = 0; n < N; ++n) {
                const uint16_t *wn = we + n * H;
                double acc = 0.0;
                for (int64_t c = 0; c < H; ++c)
                    acc += (double)oracle_bf16_to_f32(xr[c]) * (double)oracle_bf16_to_f32(wn[c]);
                y[r * N + n] = oracle_f64_to_bf16(acc);
            }
        }
    }
}
