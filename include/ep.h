/*
 * ep.h -- C ABI of the MI355X (gfx950) MoE expert-parallel dispatch layout,
 * dispatch pack and combine library (libep_mi355x.so).
 *
 * The operations and their arguments follow DeepSeek's DeepEP as described on
 * these pages:
 *   [V1]  "DeepEP V1 Legacy guide" (zskr.cn): §5.1 (get_dispatch_layout,
 *         dispatch and combine of the normal kernels), §5.2(1) (the layout's
 *         outputs), §5.2(6) (FP8 tokens with one float scale per 128 channels;
 *         BF16 weighted reduction), §6.1 and §6.3 (low-latency dispatch:
 *         num_max_dispatch_tokens_per_rank, experts split evenly over ranks,
 *         receive data [local experts, M * ranks, hidden], -1 in topk_idx is
 *         legal), §8.2 (fixed-size buffers at maximum capacity);
 *   [ASC] "DeepEP Ascend Deep Dive" (kongchang.com): "Two Transfers: Dispatch
 *         and Combine" (one copy per destination card; weighted sum at the
 *         origin), "Dispatch's Three Phases and FP8 Compression" (phase 1: the
 *         expand layout with 128-aligned, zero-padded expert queues; phase 2:
 *         counts per expert and per card; phase 3: the receive-source map);
 *   [L14] "Lesson 14: DeepSeek DeepEP" (hpc.payai.win): §3 (low-latency call
 *         sequence: x [tokens, hidden] bf16, topk_idx [tokens, topk] global
 *         expert ids, receive data plus a count per local expert, combine
 *         with topk_weights and the handle).
 *
 * One GPU plays every logical EP rank: rank r owns experts [r*L, (r+1)*L),
 * L = E / R, and its receive buffer is the slice recv_x[r*L : (r+1)*L] of one
 * [E, S, H] buffer in this GPU's HBM; its per-expert counts are the slice
 * num_tokens_per_expert[r*L : (r+1)*L].  Two more receive layouts exist: the
 * expand layout (ep_dispatch_expand, ep_combine_expand) and the normal-mode
 * rank-major layout (ep_dispatch_normal, ep_combine_normal).
 *
 * Conventions of every entry point:
 *  - Pointers are DEVICE pointers unless the comment says "host".  The caller
 *    allocates and frees every buffer; each must stay valid until the stream
 *    work completes.  The library never allocates and never synchronises the
 *    host.  Its only process-wide state: per-device memos of how many waves
 *    of each multi-item combine kernel fit on the GPU and of the device's
 *    compute units (facts about the compiled kernels and the device, from the
 *    runtime's queries, stored atomically on first use), and
 *    ep_layout_noalloc's static scratch array with its per-device address
 *    (looked up at the first call on a device).  None changes any result.  Calls are reentrant -- except
 *    ep_layout_noalloc calls that overlap on one GPU, which share its scratch
 *    -- and may be captured into a HIP graph.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    null stream).  Entry points return EP_OK once the work is enqueued.
 *  - Static errors (bad shape, capacity, null or misaligned pointer, too small
 *    a workspace) are found on the host BEFORE anything is enqueued, and the
 *    call returns their code.  A failed launch returns EP_ERR_HIP.
 *  - Data-dependent problems are reported through the optional device word
 *    `status` (nullable) by atomic OR of EP_STATUS_* bits; the library never
 *    clears it.  An expert id >= E or < -1 is treated like -1 (masked) and
 *    sets EP_STATUS_BAD_EXPERT_ID; an expert_slot outside [0, S) for a routed
 *    entry is skipped and sets EP_STATUS_BAD_SLOT.
 *  - Arrays are dense row-major.  Token rows (x, recv_x, expert_out,
 *    combined_x) must be 16-byte aligned; every other array must be aligned to
 *    its element size.
 *  - Inputs must hold finite values; the FP8 bytes of a non-finite input are
 *    unspecified (but every write stays inside its row).
 */
#ifndef EP_MI355X_H
#define EP_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define EP_OK 0
#define EP_ERR_NULL 1        /* a required pointer is NULL                            */
#define EP_ERR_SHAPE 2       /* N < 0, H, K, E or R out of range, E % R != 0, FP8 with
                                H % 128 != 0, BF16 with H % 8 != 0, a bad
                                scale_format, expert_alignment < 0                   */
#define EP_ERR_CAPACITY 3    /* N > M or S < M: the fixed upper bounds are never grown
                                ([V1] §6.1 and §8.4; [L14] capacity discussion)       */
#define EP_ERR_ALIGN 4       /* a pointer is not aligned as required                  */
#define EP_ERR_UNSUPPORTED 5 /* a size the library does not support (see limits)     */
#define EP_ERR_HIP 6         /* a HIP launch failed                                   */
#define EP_ERR_WORKSPACE 7   /* workspace NULL or smaller than ep_query_sizes says    */
#define EP_ERR_SCRATCH 8     /* ep_layout_noalloc: the shape's layout scratch is larger
                                than EP_NOALLOC_SCRATCH_BYTES                        */

/* Bits OR-ed into the optional device status word. */
#define EP_STATUS_BAD_EXPERT_ID 1u
#define EP_STATUS_BAD_SLOT 2u

/* Limits of the library. */
#define EP_MAX_EXPERTS 1024 /* E */
#define EP_MAX_RANKS 64     /* R: a token's rank set is one 64-bit mask          */
#define EP_MAX_TOPK 32      /* K */
#define EP_MAX_ALIGNMENT 1024 /* expert_alignment */
#define EP_MAX_GROUPS 64      /* num_groups of ep_group_limited_topk */
/* Bytes of the static per-device scratch of ep_layout_noalloc (1 MiB):
 * enough for ep_layout's histograms of up to 253,952 tokens at E = 256,
 * R = 8, or 61,440 tokens at E = 1024, R = 64. */
#define EP_NOALLOC_SCRATCH_BYTES (1u << 20)

/* The problem's shape ([V1] §5.1 and §6.1; [L14] §3).  Passed by host pointer. */
typedef struct {
    int32_t num_tokens;  /* N >= 0: tokens on this (source) rank                      */
    int32_t hidden;      /* H >= 8, H % 8 == 0; H % 128 == 0 when use_fp8           */
    int32_t num_topk;    /* K in [1, EP_MAX_TOPK]: routing entries per token         */
    int32_t num_experts; /* E in [1, EP_MAX_EXPERTS]                                  */
    int32_t num_ranks;   /* R in [1, EP_MAX_RANKS], E % R == 0: logical EP ranks      */
    int32_t num_max_dispatch_tokens_per_rank; /* M >= max(N, 1): fixed token bound   */
    int32_t expert_capacity; /* S >= M: rows per expert receive buffer (the pages'
                                low-latency shape uses S = R * M)                    */
    int32_t use_fp8;     /* 0: BF16 rows; 1: E4M3FN rows + a scale per 128 channels  */
    int32_t scale_format; /* FP8 scale per 128-channel block ([V1] §5.2(6), §6.3):
                             EP_SCALE_FP32  (0) fp32 a'/448;
                             EP_SCALE_POW2  (1) fp32 power of two ("round_scale");
                             EP_SCALE_UE8M0 (2) that power of two as an 8-bit
                             exponent, four per 32-bit word ("use_ue8m0").
                             Must be 0 when use_fp8 == 0. */
    int32_t expert_alignment; /* A in [0, EP_MAX_ALIGNMENT]; 0 and 1 mean none.
                             ep_layout's expert_offset is the exclusive prefix
                             of round_up(count_e, A): the queue starts of the
                             expand layout ([ASC] phase 1: queues padded to a
                             multiple of 128 for the grouped GEMM).  Also the
                             per-expert receive counts of normal mode rounded
                             up the same way are expert_offset[e+1] -
                             expert_offset[e]. */
} ep_shape;

/* Scale formats of ep_shape.scale_format. */
#define EP_SCALE_FP32 0
#define EP_SCALE_POW2 1
#define EP_SCALE_UE8M0 2

/* Bytes of every buffer for a shape (0 for a buffer the shape does not use). */
typedef struct {
    size_t recv_x;                /* E*S*H (FP8) or E*S*H*2 (BF16)                    */
    size_t recv_scales;           /* E*S*(H/128)*4 (FP8 fp32 scales),
                                     E*S*ceil(H/512)*4 (UE8M0), else 0              */
    size_t recv_src_idx;          /* E*S*4                                            */
    size_t expert_out;            /* E*S*H*2: bf16 expert outputs read by combine     */
    size_t combined_x;            /* N*H*2                                            */
    size_t num_tokens_per_rank;   /* R*4                                              */
    size_t num_tokens_per_expert; /* E*4                                              */
    size_t is_token_in_rank;      /* N*R                                              */
    size_t expert_slot;           /* N*K*4                                            */
    size_t rank_slot;             /* N*R*4                                            */
    size_t expert_offset;         /* (E+1)*4                                          */
    size_t layout_workspace;      /* scratch for ep_layout(_dispatch) (0: none)       */
    /* normal mode (ep_dispatch_normal / ep_combine_normal), M rows per rank: */
    size_t recv_x_normal;         /* R*M*H (FP8) or R*M*H*2 (BF16)                    */
    size_t recv_scales_normal;    /* R*M*(H/128)*4, R*M*ceil(H/512)*4 (UE8M0), or 0   */
    size_t recv_topk_idx;         /* R*M*K*8                                          */
    size_t recv_topk_weights;     /* R*M*K*4                                          */
    size_t recv_src_idx_normal;   /* R*M*4                                            */
    size_t expert_out_normal;     /* R*M*H*2: bf16 rows read by ep_combine_normal     */
    size_t combined_topk_weights; /* N*K*4                                            */
    /* expand layout, T = M*K + E*(A-1) rows (A = max(expert_alignment, 1)):    */
    size_t recv_x_expand;         /* T*H (FP8) or T*H*2 (BF16)                        */
    size_t recv_scales_expand;    /* T*(H/128)*4, T*ceil(H/512)*4 (UE8M0), or 0       */
    size_t recv_src_idx_expand;   /* T*4                                              */
    size_t expert_out_expand;     /* T*H*2: bf16 rows read by ep_combine_expand       */
    /* LogFMT combine payload (H % 128 == 0, else 0):                          */
    size_t logfmt_codes;          /* E*S*H: one code byte per channel                 */
    size_t logfmt_headers;        /* E*S*(H/128)*8: (lo, hi) fp32 per 128 channels    */
} ep_sizes;

/* Host only.  Fills `out` (host) with the byte size of every buffer for
 * `shape` (host).  Returns EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_CAPACITY or
 * EP_ERR_UNSUPPORTED. */
int ep_query_sizes(const ep_shape *shape, ep_sizes *out);

/* Dispatch layout ([V1] §5.2(1): tokens per rank, tokens per expert and the
 * is_token_in_rank mask computed from topk_idx before any data moves; [ASC]
 * phase 2: count per expert and per destination card; [ASC] "Two Transfers":
 * a card receives a token once however many of its experts live there).
 *
 * In:  topk_idx [N, K] int64, global expert ids, -1 = no expert ([V1] §6.3).
 * Out (all written in full, no pre-zeroing needed):
 *   num_tokens_per_expert [E] int32  valid entries per expert (with multiplicity);
 *   num_tokens_per_rank   [R] int32  tokens with >= 1 valid entry on rank r;
 *   is_token_in_rank   [N, R] uint8  1 iff token t has a valid entry on rank r;
 *   expert_slot        [N, K] int32  receive row of entry (t, k) in its expert's
 *       buffer: the number of entries (t', k') before (t, k) in (token, k)
 *       order with the same expert; -1 for masked entries;
 *   rank_slot          [N, R] int32  the number of tokens t' < t in rank r's set,
 *       -1 where token t is not in the set (each token appears at most once per
 *       rank; this is the one row per (token, rank) a link would carry);
 *   expert_offset      [E+1]  int32  exclusive prefix of num_tokens_per_expert
 *       rounded up to multiples of A = max(expert_alignment, 1); with A = 1,
 *       expert_offset[E] = number of valid entries.  Nullable (required by
 *       ep_dispatch_expand and ep_combine_expand).
 * expert_slot is the handle that ep_dispatch and ep_combine take ([V1] §5.2(4):
 * the handle holds the routing metadata and can be reused while the routing is
 * unchanged).
 * workspace: device scratch of at least ep_sizes.layout_workspace bytes (the
 *   size ep_layout_dispatch needs; ep_layout uses its first B * round_up(E +
 *   R, 4) * 4 bytes, B = ceil(N / 256), none when B == 1), 16-byte aligned,
 *   owned by the caller, contents irrelevant on entry and meaningless after;
 *   NULL allowed when ep_layout needs none.  Calls sharing one
 *   workspace must be ordered on one stream.
 * status: nullable device word (see conventions). */
int ep_layout(const ep_shape *shape, const int64_t *topk_idx, int32_t *num_tokens_per_rank,
              int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank, int32_t *expert_slot,
              int32_t *rank_slot, int32_t *expert_offset, void *workspace, size_t workspace_bytes,
              uint32_t *status, void *stream);

/* ep_layout without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, outputs, status bits and error codes
 * are those of ep_layout; the per-block histograms go to a static device
 * array of EP_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends (its address is looked up at the first call
 * on each device).  The call allocates nothing.
 * The scratch belongs to the device of `stream` (the current device when
 * `stream` is NULL); every call on one GPU shares it, so calls that may
 * overlap on one GPU (different streams, or host threads without ordering)
 * race and must be serialised by the caller.  Nothing in it needs clearing:
 * each call writes every histogram row before it reads one.
 * Returns EP_ERR_SCRATCH, before anything is enqueued, when the shape needs
 * more than EP_NOALLOC_SCRATCH_BYTES (it needs B * round_up(E + R, 4) * 4
 * bytes, B = ceil(N / 256), none when B == 1),
 * and EP_ERR_HIP when the device address cannot be looked up. */
int ep_layout_noalloc(const ep_shape *shape, const int64_t *topk_idx,
                      int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                      uint8_t *is_token_in_rank, int32_t *expert_slot, int32_t *rank_slot,
                      int32_t *expert_offset, uint32_t *status, void *stream);

/* Dispatch pack into the fixed-shape per-expert receive buffers ([L14] §3 and
 * [V1] §6.3: data [local experts, M * ranks, hidden] with a count per local
 * expert; [V1] §5.2(6): FP8 E4M3FN with one fp32 scale per 128 channels;
 * [ASC] "Dispatch's Three Phases and FP8 Compression": amax, ratio, multiply,
 * convert; the scale travels with the token).
 *
 * In:  x [N, H] bf16 bits; topk_idx [N, K]; expert_slot [N, K] from ep_layout.
 * Out: recv_x [E, S, H]: row expert_slot[t,k] of expert topk_idx[t,k] receives
 *        token t (BF16: a bit copy; FP8: per 128-channel block b, with
 *        a = max|x|, a' = max(a, 1e-4):
 *          EP_SCALE_FP32: inv = RN(448 / a'), scale = RN(a' / 448);
 *          EP_SCALE_POW2 / EP_SCALE_UE8M0: scale = 2^e for the smallest e with
 *            448 * 2^e >= a' (no element clips), inv = 2^-e;
 *        q = E4M3FN_RNE(clamp(RN(x * inv), -448, 448)));
 *      recv_scales (FP8 only; NULL when use_fp8 == 0):
 *        EP_SCALE_FP32 / EP_SCALE_POW2: fp32 [E, S, H/128], the scale per block;
 *        EP_SCALE_UE8M0: uint32 [E, S, ceil(H/512)], byte j of word w = e + 127
 *          of block 4w + j (little-endian), bytes past the last block 0;
 *      recv_src_idx [E, S] int32: the source token t of each written row.
 * Each token is read and quantised once and written once per valid entry.
 * Rows at or beyond num_tokens_per_expert[e] are never written. */
int ep_dispatch(const ep_shape *shape, const uint16_t *x, const int64_t *topk_idx,
                const int32_t *expert_slot, void *recv_x, void *recv_scales,
                int32_t *recv_src_idx, uint32_t *status, void *stream);

/* Layout and dispatch pack in one call ([V1] §5.2(1): the layout is computed
 * from topk_idx before the dispatch moves data; [V1] §6.1 and §2.2: the
 * low-latency decode path, 128 tokens per batch).  Outputs, status bits and
 * error codes are exactly those of ep_layout followed by ep_dispatch on the
 * same stream; the arguments are the union of theirs.
 *
 * Up to 256 tokens it is one launch: each token's block counts the expert
 * ids of the tokens before it and derives the token's slots from those
 * counts, so the pack needs no separate layout pass.  From 257 to 1,024
 * tokens the layout's per-block histogram kernel runs first, and each
 * token's block adds the histograms of the blocks before its own to its
 * count of the earlier tokens of its block.  Above 1,024 tokens it is two
 * launches: each 256-token block ranks its own entries (each entry's rank
 * among the block's entries with its expert, each token's among the block's
 * tokens sent to a rank) and writes its histogram row; then one block per
 * token (per two tokens when hidden <= 4,096) adds the counts of the earlier
 * blocks to its local ranks, writes the token's layout rows and packs it,
 * while one more block sums every row into the totals and the offset scan.  Above 256 tokens it needs a workspace of
 * ep_sizes.layout_workspace bytes (which covers ep_layout's too; above 1,024
 * tokens it also holds the local ranks, 8 * N * K bytes); NULL with
 * workspace_bytes 0 is allowed up to 256 tokens. */
int ep_layout_dispatch(const ep_shape *shape, const int64_t *topk_idx, const uint16_t *x,
                       int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                       uint8_t *is_token_in_rank, int32_t *expert_slot, int32_t *rank_slot,
                       int32_t *expert_offset, void *workspace, size_t workspace_bytes,
                       void *recv_x, void *recv_scales, int32_t *recv_src_idx, uint32_t *status,
                       void *stream);

/* Combine: top-k weighted gather-reduce back into token order ([ASC] "Two
 * Transfers" and "Combine: More Output, Same Cost": outputs return to the
 * origin and are summed with the router weights; [V1] §5.2(6): BF16 in and
 * out; [L14] §3: combine takes expert_out, topk_idx, topk_weights and the
 * handle).
 *
 * In:  expert_out [E, S, H] bf16 bits (rows < count are read); topk_idx
 *      [N, K]; topk_weights [N, K] fp32; expert_slot [N, K] from ep_layout;
 *      bias [N, H] bf16 bits, nullable, 16-byte aligned: the shared expert's
 *      output, added in the epilogue ([ASC] "Combine: More Output, Same
 *      Cost": folded in at the end of the same pass).
 * Out: combined_x [N, H] bf16 bits:
 *        acc = +0; for k = 0..K-1 with a valid expert e:
 *            acc = fmaf(topk_weights[t,k], float(expert_out[e][slot][c]), acc);
 *        acc = acc + float(bias[t][c])   (when bias is not NULL);
 *        combined_x[t,c] = bf16 round-to-nearest-even(acc).
 *      A token whose entries are all masked gets +0 (or its bias row). */
int ep_combine(const ep_shape *shape, const uint16_t *expert_out, const int64_t *topk_idx,
               const float *topk_weights, const int32_t *expert_slot, const uint16_t *bias,
               uint16_t *combined_x, uint32_t *status, void *stream);

/* LogFMT combine payload ([V1] §6.2: the low-latency combine message is a
 * min/max header per 128 channels followed by the hidden data; [V1] §7.1:
 * the low-latency test's LogFMT combine).  The pages define no more; the
 * format used (8 bits per channel, logarithmic):
 *   L(a)   = log2(a) rounded to the nearest binary32 (a > 0);
 *   header = per 128-channel block b: lo = min, hi = max of L(|x|) over the
 *            block's nonzero channels (0, 0 when there are none);
 *   code   = bit 7 the sign, bits 0..6 m: m = 0 for a zero, otherwise
 *            m = 1 + rint(RN(RN(L(|x|) - lo) * RN(126 / (hi - lo)))) clamped to
 *            [1, 127] (rint: ties to even; m = 1 when hi == lo), each RN a
 *            binary32 rounding;
 *   value  = sign * 2^RN(lo + RN((m - 1) * RN((hi - lo) / 126))), 0 for m = 0
 *            (within half a log-domain step, (hi - lo) / 252, of |x|).
 * Requires H % 128 == 0 (EP_ERR_SHAPE otherwise) and finite inputs. */

/* Encode the expert outputs the routing references: for every valid entry
 * (t, k) with expert e and slot j = expert_slot[t,k] < S, row (e, j) of
 * expert_out [E, S, H] bf16 becomes codes [E, S, H] uint8 (16-byte aligned)
 * and headers [E, S, H/128, 2] fp32 (lo, hi; 8-byte aligned).  Other rows are
 * not written.  Status bits as ep_combine. */
int ep_logfmt_encode(const ep_shape *shape, const uint16_t *expert_out, const int64_t *topk_idx,
                     const int32_t *expert_slot, uint8_t *codes, float *headers,
                     uint32_t *status, void *stream);

/* Combine of LogFMT expert outputs: as ep_combine, with each expert value
 * the decoded float of its code (codes [E, S, H], headers [E, S, H/128, 2]
 * from ep_logfmt_encode):
 *   acc = +0; for k = 0..K-1 with a valid expert e and slot j:
 *       acc = fmaf(topk_weights[t,k], value(codes[e][j][c], header[e][j][c/128]), acc);
 *   acc = acc + float(bias[t][c]) (when bias is not NULL);
 *   combined_x[t,c] = bf16 round-to-nearest-even(acc).
 * The exponential is the device's fp32 exp2f (within an ulp of the binary32
 * rounding of the definition). */
int ep_combine_logfmt(const ep_shape *shape, const uint8_t *codes, const float *headers,
                      const int64_t *topk_idx, const float *topk_weights,
                      const int32_t *expert_slot, const uint16_t *bias, uint16_t *combined_x,
                      uint32_t *status, void *stream);

/* Dispatch pack into the expand layout ([ASC] "Dispatch's Three Phases and
 * FP8 Compression", phase 1: each token is cloned once per routed expert, the
 * clones are grouped by expert, and each expert's queue is padded with zero
 * rows to a multiple of the expert alignment, because the grouped GEMM after
 * it takes only aligned row counts; phase 3: the receive-source map).
 *
 * In:  x, topk_idx, expert_slot as for ep_dispatch; expert_offset [E+1] and
 *      num_tokens_per_expert [E] from ep_layout run with the same shape
 *      (expert_offset then holds the aligned queue starts).
 * Out: one buffer of T = M*K + E*(A-1) rows (A = max(expert_alignment, 1)):
 *      recv_x [T, H] (FP8 bytes or bf16), recv_scales [T, H/128] fp32 or
 *      [T, ceil(H/512)] UE8M0 words (FP8 only, NULL otherwise), recv_src_idx
 *      [T] int32.  Entry (t, k) with expert e goes to row expert_offset[e] +
 *      expert_slot[t,k] with the payload ep_dispatch writes; padding rows
 *      [expert_offset[e] + count_e, expert_offset[e+1]) get zero bytes, zero
 *      scales and source -1; rows at or past expert_offset[E] are not
 *      written.  An entry whose row falls outside its expert's queue or past T
 *      is skipped and sets EP_STATUS_BAD_SLOT. */
int ep_dispatch_expand(const ep_shape *shape, const uint16_t *x, const int64_t *topk_idx,
                       const int32_t *expert_slot, const int32_t *expert_offset,
                       const int32_t *num_tokens_per_expert, void *recv_x, void *recv_scales,
                       int32_t *recv_src_idx, uint32_t *status, void *stream);

/* Combine from expert outputs in the expand layout: as ep_combine (bias
 * included), with the output row of entry (t, k) at expert_offset[e] +
 * expert_slot[t,k] of expert_out [T, H] bf16 (same bounds rule as
 * ep_dispatch_expand). */
int ep_combine_expand(const ep_shape *shape, const uint16_t *expert_out, const int64_t *topk_idx,
                      const float *topk_weights, const int32_t *expert_slot,
                      const int32_t *expert_offset, const uint16_t *bias, uint16_t *combined_x,
                      uint32_t *status, void *stream);

/* Normal-mode dispatch ([V1] §5.1: dispatch returns recv_x, recv_topk_idx,
 * recv_topk_weights and the per-expert receive counts, and its handle holds
 * the source index; [L14] §2(3) and [ASC] "Two Transfers": a token reaches a
 * rank once however many of its experts live there).
 *
 * In:  x [N, H] bf16 bits; topk_idx [N, K]; topk_weights [N, K] fp32
 *      (nullable); rank_slot [N, R] from ep_layout.
 * Out: rank r's rows are r*M .. r*M + num_tokens_per_rank[r] - 1 of
 *        recv_x [R, M, H] (the ep_dispatch payload: FP8 bytes or bf16),
 *        recv_scales [R, M, H/128] fp32 or [R, M, ceil(H/512)] UE8M0 words
 *          (FP8 only, NULL otherwise),
 *        recv_topk_idx [R, M, K] int64: e - r*L for an entry routed to expert
 *          e on rank r (the local expert id), -1 otherwise,
 *        recv_topk_weights [R, M, K] fp32: topk_weights[t,k] for those
 *          entries, 0 otherwise (written only when both weight pointers are
 *          non-NULL),
 *        recv_src_idx [R, M] int32: the source token t;
 *      token t with rank_slot[t,r] = j >= 0 fills row j of rank r.  Rows at or
 *      past num_tokens_per_rank[r] are not written.  A slot j >= M is skipped
 *      and sets EP_STATUS_BAD_SLOT; an expert id outside [-1, E) of a token
 *      that is written sets EP_STATUS_BAD_EXPERT_ID. */
int ep_dispatch_normal(const ep_shape *shape, const uint16_t *x, const int64_t *topk_idx,
                       const float *topk_weights, const int32_t *rank_slot, void *recv_x,
                       void *recv_scales, int64_t *recv_topk_idx, float *recv_topk_weights,
                       int32_t *recv_src_idx, uint32_t *status, void *stream);

/* Normal-mode combine ([V1] §5.1: combine takes one row per received token
 * and the handle, and can reduce a tensor of per-row top-k weights; the
 * backward of dispatch is such a combine, so the reduction is a plain sum over
 * the ranks the token was sent to -- the expert layer applied the weights).
 *
 * In:  x [R, M, H] bf16 bits, one row per received token (rows < count are
 *      read); rank_slot [N, R] from ep_layout; recv_topk_weights [R, M, K]
 *      fp32 (nullable); bias [N, H] bf16 bits (nullable, as in ep_combine).
 * Out: combined_x [N, H] bf16 bits:
 *        acc = +0; for r = 0..R-1 with j = rank_slot[t,r] in [0, M):
 *            acc = acc + float(x[r][j][c]);
 *        acc = acc + float(bias[t][c])   (when bias is not NULL);
 *        combined_x[t,c] = bf16 round-to-nearest-even(acc);
 *      combined_topk_weights [N, K] fp32 (nullable; written when
 *        recv_topk_weights is given): the same fp32 sum over the same rows.
 *      A token sent nowhere gets +0 (or its bias row).
 * The backward pair of [V1] §5.1 is this pair of entry points: dispatch's
 * backward is ep_combine_normal of (grad_recv_x, grad_recv_topk_weights);
 * combine's backward is ep_dispatch_normal (BF16) of grad_combined_x.  The
 * sum over ranks is exactly the adjoint of the copy to each rank. */
int ep_combine_normal(const ep_shape *shape, const uint16_t *x, const int32_t *rank_slot,
                      const float *recv_topk_weights, const uint16_t *bias, uint16_t *combined_x,
                      float *combined_topk_weights, uint32_t *status, void *stream);

/* Rules of ep_group_limited_topk: how a group is scored and how the picks
 * are weighted. */
#define EP_GATE_MAX_SOFTMAX 0 /* group score = its best expert's score;
                                 weights = softmax of the picked scores   */
#define EP_GATE_SUM_SIGMOID 1 /* group score = binary32 sum of its experts'
                                 scores, ascending expert index, from +0;
                                 weights = sigmoids of the picked scores
                                 normalised to sum 1                       */

/* Group-limited top-k gating, the step that produces topk_idx for
 * ep_layout ([V1] §1 and §2.1: the normal kernels serve group-limited
 * gating, benchmarked with top-4 groups then top-8 experts; [L14] §3 Q3: a
 * token reaches at most 4 nodes; [L14] exercise: normalised softmax gating
 * weights).
 *
 * In:  shape (num_tokens N, num_experts E, num_topk K are used; the rest is
 *      validated as for the other entry points); scores [N, E] fp32 router
 *      scores, finite (and, for EP_GATE_SUM_SIGMOID, with finite group
 *      sums); num_groups G in [1, EP_MAX_GROUPS] with E % G == 0: group g
 *      holds experts [g*E/G, (g+1)*E/G); topk_groups TG in [1, G];
 *      K <= TG * E/G; rule EP_GATE_MAX_SOFTMAX or EP_GATE_SUM_SIGMOID.
 * Out: topk_idx [N, K] int64: per token, each group gets the rule's score
 *        (EP_GATE_MAX_SOFTMAX: the best expert's score, exact;
 *        EP_GATE_SUM_SIGMOID: acc = +0; for the group's experts in ascending
 *        index acc = RN(acc + s), the binary32 sum in that order); the TG
 *        best groups are kept (ties: lower group index); the K best experts
 *        of the kept groups, best first (ties: lower expert index);
 *      topk_weights [N, K] fp32 (nullable), over the K picks s_0..s_{K-1}:
 *        EP_GATE_MAX_SOFTMAX exp(s_k - s_0) / sum_j exp(s_j - s_0);
 *        EP_GATE_SUM_SIGMOID sig(s_k) / sum_j sig(s_j), sig(v) = 1/(1+exp(-v))
 *        (fp32 expf and division; the picks are exact).
 * Errors: EP_ERR_SHAPE for G, TG, K or rule outside the rules above,
 * EP_ERR_UNSUPPORTED for G > EP_MAX_GROUPS. */
int ep_group_limited_topk(const ep_shape *shape, int32_t num_groups, int32_t topk_groups,
                          int32_t rule, const float *scores, int64_t *topk_idx,
                          float *topk_weights, void *stream);

/* Host only.  A static string naming a return code. */
const char *ep_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_H */
