/*
 * ep_oracle.c -- plain, slow, single-threaded CPU oracle for the MoE
 * expert-parallel dispatch layout, dispatch pack and combine.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * calls it, and the two share no source, header, table or helper.
 *
 * Every function is written for a reader to check by eye against the pages it
 * follows (web pages on DeepSeek's DeepEP):
 *   [V1]  "DeepEP V1 Legacy guide" (zskr.cn): §5.1 (normal-mode example:
 *         get_dispatch_layout, dispatch, combine), §5.2(1) (the four layout
 *         outputs), §5.2(6) (FP8 input with one float scale per 128 channels,
 *         BF16 weighted reduction in combine), §6.1 (experts split evenly over
 *         ranks), §6.3 (use_fp8 receive shape; -1 in topk_idx is legal).
 *   [ASC] "DeepEP Ascend Deep Dive" (kongchang.com): "Two Transfers: Dispatch
 *         and Combine" (one copy per destination card; weighted sum at the
 *         origin), "Dispatch's Three Phases and FP8 Compression" (phase 1:
 *         the expand layout, one clone per routed expert grouped by expert,
 *         each expert queue zero-padded to a multiple of 128; phase 2: count
 *         per expert and per card; phase 3: receive-source map; amax -> ratio
 *         -> multiply -> convert).
 *   [L14] "Lesson 14: DeepSeek DeepEP" (hpc.payai.win): §3 (low-latency call
 *         sketch: fixed-shape receive buffer [local experts, M * ranks,
 *         hidden] and a per-expert count), and the dispatch/combine simulator
 *         exercise (append per (token, k); weighted sum per token).
 *
 * Conventions the pages leave open are fixed here: receive slots follow
 * (token, k) order, so exactly one slot assignment is correct; experts sit on
 * ranks in contiguous blocks (the only placement the pages show); FP8 is
 * E4M3FN rounded to nearest-even after clamping to +-448; the block amax has a
 * 1e-4 floor so an all-zero block never divides by zero; the combine adds in
 * ascending k with fp32 fused multiply-add and rounds to bf16 once.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fPIC -shared (no fast-math), so
 * every float operation below is one IEEE binary32 operation in the order
 * written.
 */
#define _POSIX_C_SOURCE 200809L /* clock_gettime, for the timed path below */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#define ORACLE_OK 0
#define ORACLE_BAD_EXPERT_ID 1 /* an id >= E or < -1 was seen (treated as -1) */
#define ORACLE_BAD_SLOT 2      /* an expert_slot outside [0, S) was seen      */
#define ORACLE_BAD_ARGS 4      /* shapes that make no sense                   */

/* ---------------------------------------------------------------- formats */

/* bf16 is the upper half of a binary32; widening is exact. */
float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 to bf16, to nearest, ties to even: keep the upper 16 bits
 * and add one unit in their last place when the dropped 16 bits are above
 * half, or exactly half with an odd kept part.  NaN stays a (quiet) NaN. */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

/* OCP FP8 E4M3FN ([V1] §5.2(6) names torch's float8_e4m3fn): 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; no infinity; S.1111.111 is
 * NaN; largest finite magnitude 448 (code 0x7E).  Normal codes hold
 * (1 + m/8) * 2^(E-7) for E = 1..15, subnormal codes m * 2^-9. */
double oracle_e4m3fn_decode(uint8_t c)
{
    int s = c >> 7;
    int E = (c >> 3) & 15;
    int m = c & 7;
    if (E == 15 && m == 7)
        return NAN;
    double v = (E == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), E - 10);
    return s ? -v : v;
}

/* Encode a finite binary32 with |v| <= 448 to E4M3FN, rounding to nearest
 * with ties to an even mantissa.  The sign is kept (so -tiny -> 0x80).
 * All double arithmetic below is exact: v has 24 significant bits. */
uint8_t oracle_e4m3fn_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a < 0x1p-6) {
        /* subnormal range: a = q * 2^-9 with q in [0, 8); q rounds to
         * m in 0..8, and m = 8 is exactly code 0x08 = 2^-6. */
        double m = nearbyint(a * 0x1p9);
        return (uint8_t)(sign | (uint8_t)m);
    }
    int ex;
    frexp(a, &ex);  /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1; /* a in [2^e, 2^(e+1)), e in [-6, 8] */
    double m = nearbyint((ldexp(a, -e) - 1.0) * 8.0);
    if (m == 8.0) { /* mantissa rounded up into the next binade */
        e += 1;
        m = 0.0;
    }
    return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | (int)m));
}

/* ---------------------------------------------------------------- routing */

/* [V1] §6.3: -1 means "no expert at this position" and is legal input.  Any
 * other id outside [0, E) is treated the same way and reported. */
static int32_t routed_expert(int64_t id, int32_t E, int *status)
{
    if (id == -1)
        return -1;
    if (id < 0 || id >= (int64_t)E) {
        *status |= ORACLE_BAD_EXPERT_ID;
        return -1;
    }
    return (int32_t)id;
}

/* [V1] §6.1 (E % R == 0, E / R local experts per rank) and [ASC] "Why MoE
 * Needs a Dedicated Communication Library" (256 experts over 8 cards, 32
 * each): expert e lives on rank e / L in a contiguous block, L = E / R. */
static int32_t rank_of(int32_t e, int32_t E, int32_t R)
{
    return e / (E / R);
}

/* ----------------------------------------------------------------- layout */

/* Dispatch layout ([V1] §5.2(1); [ASC] "Dispatch's Three Phases", phase 2:
 * count per expert and per destination card; [ASC] "Two Transfers": a card
 * receives one copy of a token however many of its experts live there).
 *
 * Walk the entries in (t, k) order:
 *   valid entry, expert e:  expert_slot[t,k] = running count of e, then +1;
 *                           mark rank(e) in the token's rank set;
 *   masked entry:           expert_slot[t,k] = -1.
 * Then for each rank r of the token's set (r ascending):
 *   is_token_in_rank[t,r] = 1, rank_slot[t,r] = running count of r, then +1;
 * and 0 / -1 for ranks outside the set.
 * Outputs: num_tokens_per_expert (counts with multiplicity),
 * num_tokens_per_rank (each token at most once per rank), expert_offset =
 * exclusive prefix of num_tokens_per_expert with expert_offset[E] = number of
 * valid entries (nullable). */
int oracle_layout(int32_t N, int32_t K, int32_t E, int32_t R, const int64_t *topk_idx,
                  int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                  uint8_t *is_token_in_rank, int32_t *expert_slot, int32_t *rank_slot,
                  int32_t *expert_offset)
{
    if (N < 0 || K < 1 || E < 1 || R < 1 || E % R != 0)
        return ORACLE_BAD_ARGS;
    int status = ORACLE_OK;
    uint8_t *in_set = (uint8_t *)calloc((size_t)R, 1);
    if (!in_set)
        return ORACLE_BAD_ARGS;
    for (int32_t e = 0; e < E; ++e)
        num_tokens_per_expert[e] = 0;
    for (int32_t r = 0; r < R; ++r)
        num_tokens_per_rank[r] = 0;

    for (int32_t t = 0; t < N; ++t) {
        memset(in_set, 0, (size_t)R);
        for (int32_t k = 0; k < K; ++k) {
            size_t i = (size_t)t * K + k;
            int32_t e = routed_expert(topk_idx[i], E, &status);
            if (e < 0) {
                expert_slot[i] = -1;
                continue;
            }
            expert_slot[i] = num_tokens_per_expert[e];
            num_tokens_per_expert[e] += 1;
            in_set[rank_of(e, E, R)] = 1;
        }
        for (int32_t r = 0; r < R; ++r) {
            size_t i = (size_t)t * R + r;
            if (in_set[r]) {
                is_token_in_rank[i] = 1;
                rank_slot[i] = num_tokens_per_rank[r];
                num_tokens_per_rank[r] += 1;
            } else {
                is_token_in_rank[i] = 0;
                rank_slot[i] = -1;
            }
        }
    }
    if (expert_offset) {
        int32_t run = 0;
        for (int32_t e = 0; e < E; ++e) {
            expert_offset[e] = run;
            run += num_tokens_per_expert[e];
        }
        expert_offset[E] = run;
    }
    free(in_set);
    return status;
}

/* ------------------------------------------------------------ FP8 payload */

/* One token row to FP8 with one fp32 scale per 128 channels ([V1] §5.2(6):
 * scales of shape [tokens, hidden / 128]; [ASC] "Dispatch's Three Phases and
 * FP8 Compression": find the max magnitude, form the ratio, multiply, convert,
 * and ship the scale so the receiver can undo it).  For block b:
 *   a     = max |x|           over the 128 channels (exact)
 *   a'    = max(a, 1e-4)      floor so an all-zero block divides safely
 *   inv   = 448 / a'          (one rounded fp32 division)
 *   scale = a' / 448          (one rounded fp32 division; what ships)
 *   q     = E4M3FN_RNE(clamp(x * inv, -448, 448))
 * The receiver reconstructs x ~ q * scale. */
/* a' = max(max_c |x[c]|, 1e-4) over one 128-channel block (exact). */
static float block_amax_floored(const uint16_t *xb)
{
    float a = 0.0f;
    for (int c = 0; c < 128; ++c) {
        float m = fabsf(oracle_bf16_to_f32(xb[c]));
        if (m > a)
            a = m;
    }
    return (a > 1e-4f) ? a : 1e-4f;
}

void oracle_quantize_row(int32_t H, const uint16_t *x_row, uint8_t *q_row, float *scales)
{
    for (int32_t b = 0; b < H / 128; ++b) {
        const uint16_t *xb = x_row + (size_t)b * 128;
        float ap = block_amax_floored(xb);
        float inv = 448.0f / ap;
        float scale = ap / 448.0f;
        scales[b] = scale;
        for (int c = 0; c < 128; ++c) {
            float v = oracle_bf16_to_f32(xb[c]) * inv;
            if (v > 448.0f)
                v = 448.0f;
            if (v < -448.0f)
                v = -448.0f;
            q_row[(size_t)b * 128 + c] = oracle_e4m3fn_encode(v);
        }
    }
}

/* Power-of-two scales ([V1] §6.3 names round_scale: scales rounded to powers
 * of two, and use_ue8m0: those scales stored as 8-bit exponents).  For block
 * amax a' (floored as above) the scale is the smallest power of two p = 2^e
 * with 448 * p >= a', so every |x / p| <= 448 and nothing clips; found by
 * exact comparisons in double (448 * 2^e is exact).  Then
 *   q = E4M3FN_RNE(clamp(RN(x * 2^-e), -448, 448)).
 * UE8M0 stores the byte e + 127 (value 2^(byte - 127)). */
int oracle_pow2_scale_exponent(float ap)
{
    int e;
    frexp((double)ap, &e); /* ap in [2^(e-1), 2^e) */
    e -= 9;                /* 448 * 2^(e-1) < 2^(e+8) / 2 <= ap: no smaller e can hold */
    while (ldexp(448.0, e) < (double)ap)
        e += 1;            /* step up to the first e with 448 * 2^e >= ap */
    return e;
}

#define ORACLE_SCALE_FP32 0
#define ORACLE_SCALE_POW2 1
#define ORACLE_SCALE_UE8M0 2

/* One token row to FP8 with power-of-two block scales: e per block into
 * exps[b]; the fp32 scale is 2^e. */
void oracle_quantize_row_pow2(int32_t H, const uint16_t *x_row, uint8_t *q_row, int32_t *exps)
{
    for (int32_t b = 0; b < H / 128; ++b) {
        const uint16_t *xb = x_row + (size_t)b * 128;
        float ap = block_amax_floored(xb);
        int e = oracle_pow2_scale_exponent(ap);
        exps[b] = e;
        float inv = (float)ldexp(1.0, -e);
        for (int c = 0; c < 128; ++c) {
            float v = oracle_bf16_to_f32(xb[c]) * inv;
            if (v > 448.0f)
                v = 448.0f;
            if (v < -448.0f)
                v = -448.0f;
            q_row[(size_t)b * 128 + c] = oracle_e4m3fn_encode(v);
        }
    }
}

/* What an identity expert returns for an FP8 row: bf16_RNE(float(q) * scale),
 * one rounded fp32 product per channel (float(q) is exact). */
void oracle_dequant_row(int32_t H, const uint8_t *q_row, const float *scales, uint16_t *y_row)
{
    for (int32_t c = 0; c < H; ++c) {
        float qv = (float)oracle_e4m3fn_decode(q_row[c]);
        float v = qv * scales[c / 128];
        y_row[c] = oracle_bf16_rne(v);
    }
}

/* ------------------------------------------------------------------- pack */

/* Dispatch pack into fixed-shape per-expert receive buffers ([L14] §3: data
 * [local experts, M * ranks, hidden] plus a count per local expert; [V1] §6.3
 * the same shape for use_fp8; [ASC] phase 3: a map of which slot holds which
 * token).  Global layout here: recv_x[e][j] with e the global expert id
 * (rank r owns e in [r*L, (r+1)*L)) and j < S.
 *
 * For each token t (in order) the payload is formed once: the bf16 row, or
 * the FP8 row and its scales.  Then for each valid (t,k), e = topk_idx[t,k],
 * j = expert_slot[t,k]:
 *   recv_x[e][j] = payload, recv_scales[e][j][:] = scales (FP8 only),
 *   recv_src_idx[e][j] = t.
 * Rows j >= count_e are not written. */
/* Scale storage of one receive row ([V1] §5.2(6) and §6.3):
 *   fp32 formats: G floats (the scale, or 2^e);
 *   UE8M0: ceil(G/4) 32-bit words, byte j of word w = e + 127 of block
 *   4w + j (little-endian), bytes past the last block 0. */
static int32_t scale_words(int32_t G, int32_t fmt)
{
    return fmt == ORACLE_SCALE_UE8M0 ? (G + 3) / 4 : G;
}

/* The payload of one token, formed once and copied to each destination: the
 * FP8 bytes, and the scales as fp32 (G values) or packed UE8M0 (W words). */
typedef struct {
    int32_t H, G, W, use_fp8, fmt;
    uint8_t *q;
    float *sc;
    int32_t *ex;
    uint32_t *packed;
} payload;

static int payload_init(payload *p, int32_t H, int32_t use_fp8, int32_t fmt)
{
    p->H = H;
    p->G = H / 128;
    p->W = scale_words(p->G, fmt);
    p->use_fp8 = use_fp8;
    p->fmt = fmt;
    p->q = (uint8_t *)malloc((size_t)H);
    p->sc = (float *)malloc(sizeof(float) * (size_t)(p->G > 0 ? p->G : 1));
    p->ex = (int32_t *)malloc(sizeof(int32_t) * (size_t)(p->G > 0 ? p->G : 1));
    p->packed = (uint32_t *)calloc((size_t)(p->W > 0 ? p->W : 1), sizeof(uint32_t));
    return p->q && p->sc && p->ex && p->packed;
}

static void payload_free(payload *p)
{
    free(p->q);
    free(p->sc);
    free(p->ex);
    free(p->packed);
}

/* Quantise token row xt (FP8 only; a BF16 payload is the row itself). */
static void payload_form(payload *p, const uint16_t *xt)
{
    if (!p->use_fp8)
        return;
    if (p->fmt == ORACLE_SCALE_FP32) {
        oracle_quantize_row(p->H, xt, p->q, p->sc);
        return;
    }
    oracle_quantize_row_pow2(p->H, xt, p->q, p->ex);
    for (int32_t b = 0; b < p->G; ++b)
        p->sc[b] = (float)ldexp(1.0, p->ex[b]);
    for (int32_t w = 0; w < p->W; ++w)
        p->packed[w] = 0;
    for (int32_t b = 0; b < p->G; ++b)
        p->packed[b / 4] |= (uint32_t)(p->ex[b] + 127) << (8 * (b % 4));
}

/* Copy the payload of token row xt into receive row `row`. */
static void payload_store(const payload *p, const uint16_t *xt, size_t row, void *recv_x,
                          void *recv_scales)
{
    const int32_t H = p->H, G = p->G, W = p->W;
    if (p->use_fp8) {
        memcpy((uint8_t *)recv_x + row * H, p->q, (size_t)H);
        if (p->fmt == ORACLE_SCALE_UE8M0)
            memcpy((uint32_t *)recv_scales + row * W, p->packed, sizeof(uint32_t) * (size_t)W);
        else
            memcpy((float *)recv_scales + row * G, p->sc, sizeof(float) * (size_t)G);
    } else {
        memcpy((uint16_t *)recv_x + row * H, xt, sizeof(uint16_t) * (size_t)H);
    }
}

/* Zero a receive row and its scales (expand-layout padding). */
static void payload_zero(const payload *p, size_t row, void *recv_x, void *recv_scales)
{
    const int32_t H = p->H;
    if (p->use_fp8) {
        memset((uint8_t *)recv_x + row * H, 0, (size_t)H);
        if (p->fmt == ORACLE_SCALE_UE8M0)
            memset((uint32_t *)recv_scales + row * p->W, 0, sizeof(uint32_t) * (size_t)p->W);
        else
            memset((float *)recv_scales + row * p->G, 0, sizeof(float) * (size_t)p->G);
    } else {
        memset((uint16_t *)recv_x + row * H, 0, sizeof(uint16_t) * (size_t)H);
    }
}

static int fmt_ok(int32_t H, int32_t use_fp8, int32_t fmt)
{
    return !(H < 1 || (use_fp8 && H % 128 != 0) || fmt < 0 || fmt > 2 || (!use_fp8 && fmt != 0));
}

int oracle_pack_fmt(int32_t N, int32_t H, int32_t K, int32_t E, int32_t S, int32_t use_fp8,
                    int32_t scale_fmt, const uint16_t *x, const int64_t *topk_idx,
                    const int32_t *expert_slot, void *recv_x, void *recv_scales,
                    int32_t *recv_src_idx)
{
    if (N < 0 || K < 1 || E < 1 || S < 0 || !fmt_ok(H, use_fp8, scale_fmt))
        return ORACLE_BAD_ARGS;
    int status = ORACLE_OK;
    payload p;
    if (!payload_init(&p, H, use_fp8, scale_fmt)) {
        payload_free(&p);
        return ORACLE_BAD_ARGS;
    }
    for (int32_t t = 0; t < N; ++t) {
        const uint16_t *xt = x + (size_t)t * H;
        payload_form(&p, xt);
        for (int32_t k = 0; k < K; ++k) {
            size_t i = (size_t)t * K + k;
            int32_t e = routed_expert(topk_idx[i], E, &status);
            if (e < 0)
                continue;
            int32_t j = expert_slot[i];
            if (j < 0 || j >= S) {
                status |= ORACLE_BAD_SLOT;
                continue;
            }
            size_t row = (size_t)e * S + j;
            payload_store(&p, xt, row, recv_x, recv_scales);
            recv_src_idx[row] = t;
        }
    }
    payload_free(&p);
    return status;
}

int oracle_pack(int32_t N, int32_t H, int32_t K, int32_t E, int32_t S, int32_t use_fp8,
                const uint16_t *x, const int64_t *topk_idx, const int32_t *expert_slot,
                void *recv_x, float *recv_scales, int32_t *recv_src_idx)
{
    return oracle_pack_fmt(N, H, K, E, S, use_fp8, ORACLE_SCALE_FP32, x, topk_idx, expert_slot,
                           recv_x, recv_scales, recv_src_idx);
}

/* ---------------------------------------------------------------- combine */

/* Combine ([ASC] "Two Transfers" and "Combine: More Output, Same Cost":
 * results come back to the origin, are weighted by the router scores and
 * summed; [V1] §5.2(6): the reduction is BF16 in, BF16 out; [L14] exercise:
 * combined[i] += w[i,k] * out(i, e)).  Per token t and channel c:
 *   acc = +0
 *   for k = 0..K-1 with a valid expert e and slot j:
 *       acc = fmaf(w[t,k], float(y[e][j][c]), acc)
 *   acc = acc + float(bias[t][c])        (only when bias is not NULL)
 *   out[t,c] = bf16_RNE(acc)
 * A token with every entry masked gets +0 (or its bias row).  The bias is
 * the shared expert's output folded into the combine's epilogue ([ASC]
 * "Combine: More Output, Same Cost": added as a bias at the end, in the same
 * pass), so it is added after the weighted sum, before the one rounding. */
static void add_bias_row(float *acc, const uint16_t *bias_row, int32_t H)
{
    if (!bias_row)
        return;
    for (int32_t c = 0; c < H; ++c)
        acc[c] = acc[c] + oracle_bf16_to_f32(bias_row[c]);
}

int oracle_combine(int32_t N, int32_t H, int32_t K, int32_t E, int32_t S, const uint16_t *y,
                   const int64_t *topk_idx, const float *topk_weights,
                   const int32_t *expert_slot, const uint16_t *bias, uint16_t *combined_x)
{
    if (N < 0 || H < 1 || K < 1 || E < 1 || S < 0)
        return ORACLE_BAD_ARGS;
    int status = ORACLE_OK;
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);
    if (!acc)
        return ORACLE_BAD_ARGS;
    for (int32_t t = 0; t < N; ++t) {
        for (int32_t c = 0; c < H; ++c)
            acc[c] = 0.0f;
        for (int32_t k = 0; k < K; ++k) {
            size_t i = (size_t)t * K + k;
            int32_t e = routed_expert(topk_idx[i], E, &status);
            if (e < 0)
                continue;
            int32_t j = expert_slot[i];
            if (j < 0 || j >= S) {
                status |= ORACLE_BAD_SLOT;
                continue;
            }
            const uint16_t *yr = y + ((size_t)e * S + j) * H;
            float w = topk_weights[i];
            for (int32_t c = 0; c < H; ++c)
                acc[c] = fmaf(w, oracle_bf16_to_f32(yr[c]), acc[c]);
        }
        add_bias_row(acc, bias ? bias + (size_t)t * H : NULL, H);
        for (int32_t c = 0; c < H; ++c)
            combined_x[(size_t)t * H + c] = oracle_bf16_rne(acc[c]);
    }
    free(acc);
    return status;
}

/* ---------------------------------------------------- expand layout */

/* Expert alignment ([ASC] "Dispatch's Three Phases", phase 1: each expert's
 * queue is padded to a multiple of 128 because the grouped GEMM after it
 * takes only 128-aligned inputs).  With alignment A (A <= 1: none), expert
 * e's queue holds round_up(count_e, A) rows and starts at
 *   offset[e] = sum over e' < e of round_up(count_e', A);
 * offset[E] is the total.  An expert with no tokens gets no rows. */
void oracle_aligned_offsets(int32_t E, const int32_t *counts, int32_t A, int32_t *offsets)
{
    int32_t a = A > 1 ? A : 1;
    int32_t run = 0;
    for (int32_t e = 0; e < E; ++e) {
        offsets[e] = run;
        run += (counts[e] + a - 1) / a * a;
    }
    offsets[E] = run;
}

/* Dispatch pack into the expand layout ([ASC] phase 1: one clone of the
 * token per routed expert, grouped by expert, each queue zero-padded; [ASC]
 * phase 3: the receive-source map).  One buffer of T rows; the clone of
 * valid entry (t,k) with expert e and slot j sits at row offset[e] + j
 * (offsets from oracle_aligned_offsets, slots from oracle_layout).  A slot
 * must fall inside its expert's queue (offset[e] + j < offset[e+1] <= T),
 * else the entry is skipped and reported.  Padding rows
 * [offset[e] + counts[e], offset[e+1]) are zero bytes with zero scales and
 * source -1; rows at or past offset[E] are not written. */
int oracle_pack_expand(int32_t N, int32_t H, int32_t K, int32_t E, int32_t T, int32_t use_fp8,
                       int32_t scale_fmt, const uint16_t *x, const int64_t *topk_idx,
                       const int32_t *expert_slot, const int32_t *expert_offset,
                       const int32_t *counts, void *recv_x, void *recv_scales,
                       int32_t *recv_src_idx)
{
    if (N < 0 || K < 1 || E < 1 || T < 0 || !fmt_ok(H, use_fp8, scale_fmt))
        return ORACLE_BAD_ARGS;
    int status = ORACLE_OK;
    payload p;
    if (!payload_init(&p, H, use_fp8, scale_fmt)) {
        payload_free(&p);
        return ORACLE_BAD_ARGS;
    }
    for (int32_t t = 0; t < N; ++t) {
        const uint16_t *xt = x + (size_t)t * H;
        payload_form(&p, xt);
        for (int32_t k = 0; k < K; ++k) {
            size_t i = (size_t)t * K + k;
            int32_t e = routed_expert(topk_idx[i], E, &status);
            if (e < 0)
                continue;
            int64_t row = (int64_t)expert_offset[e] + expert_slot[i];
            if (expert_slot[i] < 0 || row >= expert_offset[e + 1] || expert_offset[e + 1] > T) {
                status |= ORACLE_BAD_SLOT;
                continue;
            }
            payload_store(&p, xt, (size_t)row, recv_x, recv_scales);
            recv_src_idx[row] = t;
        }
    }
    for (int32_t e = 0; e < E; ++e) {
        for (int64_t row = (int64_t)expert_offset[e] + counts[e]; row < expert_offset[e + 1];
             ++row) {
            if (row < 0 || row >= T)
                continue;
            payload_zero(&p, (size_t)row, recv_x, recv_scales);
            recv_src_idx[row] = -1;
        }
    }
    payload_free(&p);
    return status;
}

/* Combine from expert outputs in the expand layout: as oracle_combine, with
 * the output row of entry (t,k) at offset[e] + j of a T-row buffer (and the
 * same optional bias). */
int oracle_combine_expand(int32_t N, int32_t H, int32_t K, int32_t E, int32_t T, const uint16_t *y,
                          const int64_t *topk_idx, const float *topk_weights,
                          const int32_t *expert_slot, const int32_t *expert_offset,
                          const uint16_t *bias, uint16_t *combined_x)
{
    if (N < 0 || H < 1 || K < 1 || E < 1 || T < 0)
        return ORACLE_BAD_ARGS;
    int status = ORACLE_OK;
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);
    if (!acc)
        return ORACLE_BAD_ARGS;
    for (int32_t t = 0; t < N; ++t) {
        for (int32_t c = 0; c < H; ++c)
            acc[c] = 0.0f;
        for (int32_t k = 0; k < K; ++k) {
            size_t i = (size_t)t * K + k;
            int32_t e = routed_expert(topk_idx[i], E, &status);
            if (e < 0)
                continue;
            int64_t row = (int64_t)expert_offset[e] + expert_slot[i];
            if (expert_slot[i] < 0 || row >= expert_offset[e + 1] || expert_offset[e + 1] > T) {
                status |= ORACLE_BAD_SLOT;
                continue;
            }
            const uint16_t *yr = y + (size_t)row * H;
            float w = topk_weights[i];
            for (int32_t c = 0; c < H; ++c)
                acc[c] = fmaf(w, oracle_bf16_to_f32(yr[c]), acc[c]);
        }
        add_bias_row(acc, bias ? bias + (size_t)t * H : NULL, H);
        for (int32_t c = 0; c < H; ++c)
            combined_x[(size_t)t * H + c] = oracle_bf16_rne(acc[c]);
    }
    free(acc);
    return status;
}

/* ------------------------------------------------------ normal mode */

/* Normal-mode dispatch ([V1] §5.1: dispatch returns recv_x, recv_topk_idx,
 * recv_topk_weights and the per-expert receive counts; [L14] §2(3) and [ASC]
 * "Two Transfers": a token crosses to a card once however many of its
 * experts live there).  Rank r's receive buffer has M rows; token t, if its
 * rank set holds r, sits at row j = rank_slot[t,r] (from oracle_layout) of
 * rank r:
 *   recv_x[r][j]            = the token's payload (formed once per token);
 *   recv_src_idx[r][j]      = t;
 *   recv_topk_idx[r][j][k]  = e - r*L if entry (t,k) routes to expert e on
 *                             rank r (the local expert id), else -1;
 *   recv_topk_weights[r][j][k] = topk_weights[t,k] for those entries, else 0
 *                             (skipped when either weight pointer is NULL).
 * A slot j >= M is skipped and reported; rows j >= num_tokens_per_rank[r]
 * are not written. */
int oracle_dispatch_normal(int32_t N, int32_t H, int32_t K, int32_t E, int32_t R, int32_t M,
                           int32_t use_fp8, int32_t scale_fmt, const uint16_t *x,
                           const int64_t *topk_idx, const float *topk_weights,
                           const int32_t *rank_slot, void *recv_x, void *recv_scales,
                           int64_t *recv_topk_idx, float *recv_topk_weights,
                           int32_t *recv_src_idx)
{
    if (N < 0 || K < 1 || E < 1 || R < 1 || E % R != 0 || M < 0 || !fmt_ok(H, use_fp8, scale_fmt))
        return ORACLE_BAD_ARGS;
    int status = ORACLE_OK;
    const int32_t L = E / R;
    payload p;
    if (!payload_init(&p, H, use_fp8, scale_fmt)) {
        payload_free(&p);
        return ORACLE_BAD_ARGS;
    }
    for (int32_t t = 0; t < N; ++t) {
        const uint16_t *xt = x + (size_t)t * H;
        payload_form(&p, xt);
        for (int32_t r = 0; r < R; ++r) {
            int32_t j = rank_slot[(size_t)t * R + r];
            if (j < 0)
                continue; /* token not sent to rank r */
            if (j >= M) {
                status |= ORACLE_BAD_SLOT;
                continue;
            }
            size_t row = (size_t)r * M + j;
            payload_store(&p, xt, row, recv_x, recv_scales);
            recv_src_idx[row] = t;
            for (int32_t k = 0; k < K; ++k) {
                size_t i = (size_t)t * K + k;
                int32_t e = routed_expert(topk_idx[i], E, &status);
                int local = e >= 0 && rank_of(e, E, R) == r;
                recv_topk_idx[row * K + k] = local ? (int64_t)(e - r * L) : -1;
                if (topk_weights && recv_topk_weights)
                    recv_topk_weights[row * K + k] = local ? topk_weights[i] : 0.0f;
            }
        }
    }
    payload_free(&p);
    return status;
}

/* Normal-mode combine ([V1] §5.1: combine takes one row per received token
 * and the handle, and also reduces a topk_weights tensor of the received
 * layout; dispatch's backward is such a combine, so the reduction is the
 * adjoint of dispatch's copy: a plain sum over the ranks the token was sent
 * to).  Per token t, ranks r ascending with j = rank_slot[t,r] >= 0:
 *   acc[c]  = acc[c] + float(y[r][j][c])            (from +0; fp32)
 *   wacc[k] = wacc[k] + recv_topk_weights[r][j][k]  (from +0; fp32)
 *   acc[c]  = acc[c] + float(bias[t][c])           (only when bias is not NULL)
 *   combined_x[t][c] = bf16_RNE(acc[c]); combined_topk_weights[t][k] = wacc[k]
 * (the weight reduction only when both weight pointers are non-NULL).  A
 * token sent nowhere gets +0 (or its bias row). */
int oracle_combine_normal(int32_t N, int32_t H, int32_t K, int32_t R, int32_t M, const uint16_t *y,
                          const int32_t *rank_slot, const float *recv_topk_weights,
                          const uint16_t *bias, uint16_t *combined_x,
                          float *combined_topk_weights)
{
    if (N < 0 || H < 1 || K < 1 || R < 1 || M < 0)
        return ORACLE_BAD_ARGS;
    int status = ORACLE_OK;
    const int with_w = recv_topk_weights && combined_topk_weights;
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);
    float *wacc = (float *)malloc(sizeof(float) * (size_t)K);
    if (!acc || !wacc) {
        free(acc);
        free(wacc);
        return ORACLE_BAD_ARGS;
    }
    for (int32_t t = 0; t < N; ++t) {
        for (int32_t c = 0; c < H; ++c)
            acc[c] = 0.0f;
        for (int32_t k = 0; k < K; ++k)
            wacc[k] = 0.0f;
        for (int32_t r = 0; r < R; ++r) {
            int32_t j = rank_slot[(size_t)t * R + r];
            if (j < 0)
                continue;
            if (j >= M) {
                status |= ORACLE_BAD_SLOT;
                continue;
            }
            size_t row = (size_t)r * M + j;
            const uint16_t *yr = y + row * H;
            for (int32_t c = 0; c < H; ++c)
                acc[c] = acc[c] + oracle_bf16_to_f32(yr[c]);
            if (with_w)
                for (int32_t k = 0; k < K; ++k)
                    wacc[k] = wacc[k] + recv_topk_weights[row * K + k];
        }
        add_bias_row(acc, bias ? bias + (size_t)t * H : NULL, H);
        for (int32_t c = 0; c < H; ++c)
            combined_x[(size_t)t * H + c] = oracle_bf16_rne(acc[c]);
        if (with_w)
            for (int32_t k = 0; k < K; ++k)
                combined_topk_weights[(size_t)t * K + k] = wacc[k];
    }
    free(acc);
    free(wacc);
    return status;
}

/* ---------------------------------------------------------------- gating */

#define ORACLE_GATE_MAX_SOFTMAX 0
#define ORACLE_GATE_SUM_SIGMOID 1

/* Group-limited top-k gating, the step before the layout ([V1] §1 and §2.1:
 * the normal kernels serve group-limited gating, benchmarked as top-4 groups
 * then top-8 experts; [L14] §3 Q3: each token reaches at most 4 nodes).
 *
 * Experts are split into G groups of L = E / G consecutive experts.  Per
 * token t, with router scores s[t, 0..E-1], under one of two rules:
 *   ORACLE_GATE_MAX_SOFTMAX: a group's score is the largest score of its
 *     experts (exact); the weights are the softmax of the picked scores
 *     ([L14] exercise: normalised softmax gating weights);
 *   ORACLE_GATE_SUM_SIGMOID: a group's score is the binary32 sum of its
 *     experts' scores taken in ascending expert index from +0, each addition
 *     rounded to nearest even (the order is part of the definition, so both
 *     sides rank the groups identically); the weights are the sigmoids of
 *     the picked scores normalised to sum 1 (the prefill benchmark routing:
 *     top-4 groups by summed scores, then top-8 experts).
 * Then, for both rules:
 *   keep the TG groups with the largest group score (ties: the lower group
 *     index);
 *   topk_idx[t, 0..K-1] = the K experts of the kept groups with the largest
 *     s, in that order (ties: the lower expert index);
 *   topk_weights[t, k]: MAX_SOFTMAX exp(s_k - s_0) / sum_j exp(s_j - s_0);
 *     SUM_SIGMOID sig(s_k) / sum_j sig(s_j), sig(v) = 1 / (1 + exp(-v));
 *     both evaluated in double over the K picks, then rounded to float.
 * Needs 1 <= TG <= G, E % G == 0, K <= TG * L and a known rule.  Scores and
 * group sums are finite. */
int oracle_group_limited_topk(int32_t N, int32_t E, int32_t G, int32_t TG, int32_t K,
                              int32_t rule, const float *scores, int64_t *topk_idx,
                              float *topk_weights)
{
    if (N < 0 || E < 1 || G < 1 || E % G != 0 || TG < 1 || TG > G || K < 1 || K > TG * (E / G))
        return ORACLE_BAD_ARGS;
    if (rule != ORACLE_GATE_MAX_SOFTMAX && rule != ORACLE_GATE_SUM_SIGMOID)
        return ORACLE_BAD_ARGS;
    const int32_t L = E / G;
    float *gs = (float *)malloc(sizeof(float) * (size_t)G);
    uint8_t *kept = (uint8_t *)malloc((size_t)G);
    uint8_t *taken = (uint8_t *)malloc((size_t)E);
    double *z = (double *)malloc(sizeof(double) * (size_t)K);
    if (!gs || !kept || !taken || !z) {
        free(gs);
        free(kept);
        free(taken);
        free(z);
        return ORACLE_BAD_ARGS;
    }
    for (int32_t t = 0; t < N; ++t) {
        const float *st = scores + (size_t)t * E;
        for (int32_t g = 0; g < G; ++g) {
            if (rule == ORACLE_GATE_MAX_SOFTMAX) {
                gs[g] = st[g * L];
                for (int32_t i = 1; i < L; ++i)
                    if (st[g * L + i] > gs[g])
                        gs[g] = st[g * L + i];
            } else {
                float acc = 0.0f;
                for (int32_t i = 0; i < L; ++i)
                    acc = acc + st[g * L + i];
                gs[g] = acc;
            }
            kept[g] = 0;
        }
        for (int32_t n = 0; n < TG; ++n) {
            int32_t best = -1;
            for (int32_t g = 0; g < G; ++g)
                if (!kept[g] && (best < 0 || gs[g] > gs[best]))
                    best = g;
            kept[best] = 1;
        }
        for (int32_t e = 0; e < E; ++e)
            taken[e] = 0;
        for (int32_t k = 0; k < K; ++k) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e)
                if (kept[e / L] && !taken[e] && (best < 0 || st[e] > st[best]))
                    best = e;
            taken[best] = 1;
            topk_idx[(size_t)t * K + k] = best;
        }
        double sum = 0.0;
        const double top = st[topk_idx[(size_t)t * K]];
        for (int32_t k = 0; k < K; ++k) {
            const double v = st[topk_idx[(size_t)t * K + k]];
            z[k] = rule == ORACLE_GATE_MAX_SOFTMAX ? exp(v - top) : 1.0 / (1.0 + exp(-v));
            sum += z[k];
        }
        for (int32_t k = 0; k < K; ++k)
            topk_weights[(size_t)t * K + k] = (float)(z[k] / sum);
    }
    free(gs);
    free(kept);
    free(taken);
    free(z);
    return ORACLE_OK;
}

/* ------------------------------------------------ LogFMT combine payload */

/* [V1] §6.2: the low-latency combine message carries, per 128 channels, a
 * min/max header followed by the hidden data; [V1] §7.1: the low-latency
 * test has a LogFMT combine switch.  The pages define nothing further.  The
 * reading used here (an 8-bit logarithmic format) is:
 *   L(a)   = log2(a) rounded to the nearest binary32, for a > 0;
 *   header = per 128-channel block b, lo_b = min and hi_b = max of L(|x|)
 *            over the block's nonzero channels (both 0 when there are none);
 *   code   = one byte per channel: bit 7 the sign, bits 0..6 a magnitude code
 *            m; m = 0 is zero (code 0x00, either sign), otherwise
 *            m = 1 + rint(RN(RN(L(|x|) - lo) * RN(126 / (hi - lo)))) clamped
 *            to [1, 127] (rint ties to even; m = 1 when hi == lo): codes
 *            1..127 spread evenly over [lo, hi] in the log domain;
 *   decode = sign * RN(2^RN(lo + RN((m - 1) * RN((hi - lo) / 126)))), and 0
 *            for m = 0.
 * Every step before the exponential is an IEEE binary32 operation, so the
 * codes are exact; the decoded value is within half a log-domain step
 * (plus rounding) of |x|. */

/* L(a): log2 of a positive float, rounded to nearest binary32 (evaluated in
 * double, then rounded once; an exhaustive pin over every bf16 input checks
 * that this is the correctly rounded value). */
float oracle_log2_rn(float a) { return (float)log2((double)a); }

void oracle_logfmt_encode_row(int32_t H, const uint16_t *x, uint8_t *codes, float *header)
{
    for (int32_t b = 0; b < H / 128; ++b) {
        const uint16_t *xb = x + (size_t)b * 128;
        int any = 0;
        float lo = 0.0f, hi = 0.0f;
        for (int32_t c = 0; c < 128; ++c) {
            const float v = oracle_bf16_to_f32(xb[c]);
            if (v != 0.0f) {
                const float l = oracle_log2_rn(fabsf(v));
                if (!any || l < lo)
                    lo = l;
                if (!any || l > hi)
                    hi = l;
                any = 1;
            }
        }
        header[2 * b] = lo;
        header[2 * b + 1] = hi;
        const float span = hi - lo;
        const float inv = span > 0.0f ? 126.0f / span : 0.0f;
        for (int32_t c = 0; c < 128; ++c) {
            const float v = oracle_bf16_to_f32(xb[c]);
            uint8_t code = 0;
            if (v != 0.0f) {
                const float q = (oracle_log2_rn(fabsf(v)) - lo) * inv;
                int m = 1 + (int)nearbyintf(q);
                m = m < 1 ? 1 : m > 127 ? 127 : m;
                code = (uint8_t)((v < 0.0f ? 0x80 : 0x00) | m);
            }
            codes[(size_t)b * 128 + c] = code;
        }
    }
}

float oracle_logfmt_decode(uint8_t code, float lo, float hi)
{
    const int m = code & 0x7F;
    if (m == 0)
        return 0.0f;
    const float step = (hi - lo) / 126.0f;
    const float d = lo + (float)(m - 1) * step;
    const float mag = (float)exp2((double)d);
    return (code & 0x80) ? -mag : mag;
}

/* rows x [R, H] bf16 -> codes [R, H], headers [R, H/128, 2] (lo, hi). */
void oracle_logfmt_encode_rows(int64_t rows, int32_t H, const uint16_t *x, uint8_t *codes,
                               float *headers)
{
    for (int64_t r = 0; r < rows; ++r)
        oracle_logfmt_encode_row(H, x + (size_t)r * H, codes + (size_t)r * H,
                                 headers + (size_t)r * (H / 128) * 2);
}

/* codes [R, H], headers [R, H/128, 2] -> float values [R, H]. */
void oracle_logfmt_decode_rows(int64_t rows, int32_t H, const uint8_t *codes, const float *headers,
                               float *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t c = 0; c < H; ++c) {
            const float *hd = headers + ((size_t)r * (H / 128) + c / 128) * 2;
            out[(size_t)r * H + c] = oracle_logfmt_decode(codes[(size_t)r * H + c], hd[0], hd[1]);
        }
}

/* Combine of expert outputs carried as LogFMT ([V1] §6.2 and §7.1): as
 * oracle_combine, with each expert value the decoded float of its code:
 *   acc = +0; for k = 0..K-1 with a valid expert e and slot j:
 *       acc = fmaf(w[t,k], decode(codes[e][j][c], header[e][j][c / 128]), acc)
 *   acc = acc + float(bias[t][c]) (when bias is not NULL); out = bf16_RNE(acc). */
int oracle_combine_logfmt(int32_t N, int32_t H, int32_t K, int32_t E, int32_t S,
                          const uint8_t *codes, const float *headers, const int64_t *topk_idx,
                          const float *topk_weights, const int32_t *expert_slot,
                          const uint16_t *bias, uint16_t *combined_x)
{
    if (N < 0 || H < 128 || H % 128 != 0 || K < 1 || E < 1 || S < 0)
        return ORACLE_BAD_ARGS;
    int status = ORACLE_OK;
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);
    float *y = (float *)malloc(sizeof(float) * (size_t)H);
    if (!acc || !y) {
        free(acc);
        free(y);
        return ORACLE_BAD_ARGS;
    }
    for (int32_t t = 0; t < N; ++t) {
        memset(acc, 0, sizeof(float) * (size_t)H); /* +0.0f */
        for (int32_t k = 0; k < K; ++k) {
            const size_t i = (size_t)t * K + k;
            const int32_t e = routed_expert(topk_idx[i], E, &status);
            if (e < 0)
                continue;
            const int32_t j = expert_slot[i];
            if (j < 0 || j >= S) {
                status |= ORACLE_BAD_SLOT;
                continue;
            }
            /* the expert's output row, decoded */
            const size_t row = (size_t)e * S + j;
            oracle_logfmt_decode_rows(1, H, codes + row * H, headers + row * (H / 128) * 2, y);
            const float w = topk_weights[i];
            for (int32_t c = 0; c < H; ++c)
                acc[c] = fmaf(w, y[c], acc[c]);
        }
        add_bias_row(acc, bias ? bias + (size_t)t * H : NULL, H);
        for (int32_t c = 0; c < H; ++c)
            combined_x[(size_t)t * H + c] = oracle_bf16_rne(acc[c]);
    }
    free(acc);
    free(y);
    return status;
}

/* ------------------------------------------------- array forms for pinning */

void oracle_e4m3fn_encode_array(int64_t n, const float *v, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3fn_encode(v[i]);
}

void oracle_e4m3fn_decode_array(int64_t n, const uint8_t *c, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3fn_decode(c[i]);
}

void oracle_bf16_rne_array(int64_t n, const float *v, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(v[i]);
}

void oracle_quantize_rows(int32_t N, int32_t H, const uint16_t *x, uint8_t *q, float *scales)
{
    for (int32_t t = 0; t < N; ++t)
        oracle_quantize_row(H, x + (size_t)t * H, q + (size_t)t * H, scales + (size_t)t * (H / 128));
}

void oracle_dequant_rows(int32_t N, int32_t H, const uint8_t *q, const float *scales, uint16_t *y)
{
    for (int32_t t = 0; t < N; ++t)
        oracle_dequant_row(H, q + (size_t)t * H, scales + (size_t)t * (H / 128), y + (size_t)t * H);
}

void oracle_quantize_rows_pow2(int32_t N, int32_t H, const uint16_t *x, uint8_t *q, int32_t *exps)
{
    for (int32_t t = 0; t < N; ++t)
        oracle_quantize_row_pow2(H, x + (size_t)t * H, q + (size_t)t * H, exps + (size_t)t * (H / 128));
}

/* ------------------------------------------------ timed path (CPU baseline) */

static double now_seconds(void)
{
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

/* The whole path -- layout, pack (FP32 scales), combine -- on buffers the
 * caller allocated beforehand, each phase timed on its own with the
 * monotonic clock (seconds[0..2] = layout, pack, combine), so the figures
 * hold the oracle's arithmetic and memory traffic only, not allocation.
 * expert_out [E, S, H] is the combine's input.  Returns the OR of the three
 * statuses. */
int oracle_timed_path(int32_t N, int32_t H, int32_t K, int32_t E, int32_t R, int32_t S,
                      int32_t use_fp8, const uint16_t *x, const int64_t *topk_idx,
                      const float *topk_weights, const uint16_t *expert_out,
                      int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                      uint8_t *is_token_in_rank, int32_t *expert_slot, int32_t *rank_slot,
                      int32_t *expert_offset, void *recv_x, float *recv_scales,
                      int32_t *recv_src_idx, uint16_t *combined_x, double *seconds)
{
    double t0 = now_seconds();
    int st = oracle_layout(N, K, E, R, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                           is_token_in_rank, expert_slot, rank_slot, expert_offset);
    double t1 = now_seconds();
    st |= oracle_pack(N, H, K, E, S, use_fp8, x, topk_idx, expert_slot, recv_x, recv_scales,
                      recv_src_idx);
    double t2 = now_seconds();
    st |= oracle_combine(N, H, K, E, S, expert_out, topk_idx, topk_weights, expert_slot, NULL,
                         combined_x);
    double t3 = now_seconds();
    seconds[0] = t1 - t0;
    seconds[1] = t2 - t1;
    seconds[2] = t3 - t2;
    return st;
}

void oracle_log2_rn_array(int64_t n, const float *a, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_log2_rn(a[i]);
}
