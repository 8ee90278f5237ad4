// dispatch.hip -- dispatch pack on gfx950, into three receive layouts.
//
// Writes each token into receive buffers, optionally as FP8 E4M3FN with one
// scale per 128 channels (DeepEP V1 Legacy guide §5.2(6); DeepEP Ascend deep
// dive, "Dispatch's Three Phases and FP8 Compression": amax, ratio, multiply,
// convert, ship the scale with the token):
//  - per-expert rows [E, S, H] (Lesson 14 §3 and V1 guide §6.3: data
//    [local experts, M * ranks, hidden] with a count per local expert);
//  - the expand layout (Ascend deep dive, phase 1): one clone per routed
//    expert in one buffer, expert queues zero-padded to the alignment;
//  - normal mode (V1 guide §5.1): one row per (token, rank) in rank-major
//    buffers, with the token's routing entries as local expert ids and the
//    weights that travel with the row.
//
// Work item = one wave on one (token, 1024-channel chunk).  The wave reads its
// chunk of x once (16-byte non-temporal loads: x is read exactly once),
// quantises it once in registers, then stores it to every destination row of
// the token.  HBM traffic is therefore one read of x and one write per
// destination row, the minimum for each layout.
//
// FP8 lane map: 8 lanes per 128-channel block, 16 channels (32 bytes of bf16
// in, 16 bytes of FP8 out) per lane; the block amax is a 3-step DPP
// reduction over the 8 lanes.  The block scale is a'/448 or, for the
// power-of-two formats (V1 guide §6.3, round_scale and use_ue8m0), 2^e with e
// read off the exponent and mantissa bits of a'; the packed UE8M0 word of
// blocks 4w..4w+3 is gathered by shuffles into the first lane of block 4w.
// BF16 lane map: two 16-byte units per lane (unit = 8 channels), so each store
// instruction covers 1 KiB contiguous.
//
// Per-expert and expand destinations are taken KB entries at a time: the
// (expert id, slot) pairs arrive together (one vector load per lane,
// broadcast with readlane), and the stores of the batch follow back to back.
// Normal-mode destinations are the set bits of a ballot over the token's
// rank_slot row.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 1024; // channels per work item

// Power-of-two block scale: the smallest e with 448 * 2^e >= ap.  With
// ap = (1 + m / 2^23) * 2^E (ap >= 1e-4 is a normal float) and 448 = 1.75 * 2^8
// that is e = E - 8, plus 1 when the mantissa fraction exceeds 0.75.
__device__ __forceinline__ int pow2_scale_exponent(float ap)
{
    const uint32_t bits = __float_as_uint(ap);
    const int E = (int)((bits >> 23) & 0xFFu) - 127;
    return E - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
}

__device__ __forceinline__ float exp2_int(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// Where one lane's FP8 output of a (token, chunk) goes in a receive row.
struct Fp8Lane {
    int32_t G, W;   // scale blocks per row; UE8M0 words per row
    int32_t g, ch;  // this lane's block and first channel
    bool active;    // g < G
    bool word_lane; // first lane of blocks 4w..4w+3 with w < W
};

__device__ __forceinline__ Fp8Lane fp8_lane(int32_t H, int32_t chunk, int lane)
{
    Fp8Lane l;
    l.G = H / 128;
    l.W = (l.G + 3) / 4;
    l.g = chunk * (kChunk / 128) + (lane >> 3);
    l.active = l.g < l.G;
    l.ch = l.g * 128 + (lane & 7) * 16;
    l.word_lane = (lane & 31) == 0 && (l.g >> 2) < l.W;
    return l;
}

// The FP8 payload of one lane: 16 E4M3FN bytes, its block's fp32 scale and,
// for UE8M0, the packed exponent word (meaningful on word lanes).
struct Fp8Payload {
    uint4 q;
    float scale;
    uint32_t ue8m0_word;
};

// Quantise one lane's 16 channels of bf16 (in0, in1) on the FP8 lane map.
template <int SF>
__device__ __forceinline__ Fp8Payload quantize_regs(const uint4 &in0, const uint4 &in1,
                                                    const Fp8Lane &l, int lane)
{
    const uint32_t w[8] = {in0.x, in0.y, in0.z, in0.w, in1.x, in1.y, in1.z, in1.w};
    float f[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        amax = fmaxf(amax, fabsf(f[i]));
    amax = fmax8(amax);
    const float ap = fmaxf(amax, 1e-4f);
    Fp8Payload p;
    float inv;
    int e2 = 0;
    if (SF == EP_SCALE_FP32) {
        inv = 448.0f / ap;     // correctly rounded fp32 division
        p.scale = ap / 448.0f; // correctly rounded fp32 division
    } else {
        e2 = pow2_scale_exponent(ap); // in [-22, 120] for finite input
        inv = exp2_int(-e2);
        p.scale = exp2_int(e2);
    }
    p.ue8m0_word = 0;
    if (SF == EP_SCALE_UE8M0) {
        // bytes of blocks past the row end are 0
        const uint32_t byte = l.active ? (uint32_t)(e2 + 127) : 0u;
        p.ue8m0_word = byte | ((uint32_t)__shfl(byte, lane + 8, 64) << 8) |
                       ((uint32_t)__shfl(byte, lane + 16, 64) << 16) |
                       ((uint32_t)__shfl(byte, lane + 24, 64) << 24);
    }
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = clamp448(f[i] * inv);
    p.q.x = e4m3fn_x4_hw(v[0], v[1], v[2], v[3]);
    p.q.y = e4m3fn_x4_hw(v[4], v[5], v[6], v[7]);
    p.q.z = e4m3fn_x4_hw(v[8], v[9], v[10], v[11]);
    p.q.w = e4m3fn_x4_hw(v[12], v[13], v[14], v[15]);
    return p;
}

// Load one lane's bf16 of a (token, chunk) and quantise it.
template <int SF>
__device__ __forceinline__ Fp8Payload quantize_lane(const uint16_t *__restrict__ x_row,
                                                    const Fp8Lane &l, int lane)
{
    uint4 in0 = make_uint4(0, 0, 0, 0), in1 = make_uint4(0, 0, 0, 0);
    if (l.active) {
        const uint4 *src = reinterpret_cast<const uint4 *>(x_row + l.ch);
        in0 = load_stream(src);
        in1 = load_stream(src + 1);
    }
    return quantize_regs<SF>(in0, in1, l, lane);
}

// One lane's share of an FP8 receive row (bytes and scales).
template <int SF>
__device__ __forceinline__ void store_fp8(const Fp8Payload &p, const Fp8Lane &l, int lane,
                                          int64_t row, int32_t H, uint8_t *__restrict__ recv_x,
                                          void *__restrict__ recv_scales)
{
    if (l.active)
        *reinterpret_cast<uint4 *>(recv_x + (size_t)row * H + l.ch) = p.q;
    if (SF == EP_SCALE_UE8M0) {
        if (l.word_lane)
            static_cast<uint32_t *>(recv_scales)[(size_t)row * l.W + (l.g >> 2)] = p.ue8m0_word;
    } else if (l.active && (lane & 7) == 0) {
        static_cast<float *>(recv_scales)[(size_t)row * l.G + l.g] = p.scale;
    }
}

// Where one lane's BF16 units of a (token, chunk) lie.
struct Bf16Lane {
    int32_t u0, u1, units;
};

__device__ __forceinline__ Bf16Lane bf16_lane(int32_t H, int32_t chunk, int lane)
{
    Bf16Lane l;
    l.units = H / 8;
    l.u0 = chunk * (kChunk / 8) + lane;
    l.u1 = l.u0 + 64;
    return l;
}

__device__ __forceinline__ void store_bf16(const uint4 &a0, const uint4 &a1, const Bf16Lane &l,
                                           int64_t row, int32_t H, uint16_t *__restrict__ recv_x)
{
    uint4 *dst = reinterpret_cast<uint4 *>(recv_x + (size_t)row * H);
    if (l.u0 < l.units)
        dst[l.u0] = a0;
    if (l.u1 < l.units)
        dst[l.u1] = a1;
}

// The raw bf16 of one lane's share of a (token, chunk): the 32 bytes the FP8
// lane map quantises, or the two 16-byte units of the BF16 lane map.  Lanes
// past the row end keep their inputs.
template <bool FP8>
__device__ __forceinline__ void load_chunk(const uint16_t *__restrict__ x_row, int32_t H,
                                           int32_t chunk, int lane, uint4 &in0, uint4 &in1)
{
    if (FP8) {
        const Fp8Lane l = fp8_lane(H, chunk, lane);
        if (l.active) {
            const uint4 *src = reinterpret_cast<const uint4 *>(x_row + l.ch);
            in0 = load_stream(src);
            in1 = load_stream(src + 1);
        }
    } else {
        const Bf16Lane l = bf16_lane(H, chunk, lane);
        const uint4 *src = reinterpret_cast<const uint4 *>(x_row);
        if (l.u0 < l.units)
            in0 = load_stream(src + l.u0);
        if (l.u1 < l.units)
            in1 = load_stream(src + l.u1);
    }
}

// Expand-layout padding (Ascend deep dive, phase 1: the empty slots of a
// queue are zeros): rows [offset[e] + count[e], offset[e+1]) below T get zero
// bytes, zero scales and source -1, one (expert, chunk) per wave.
template <bool FP8, int SF>
__device__ void zero_padding(int32_t e, int32_t chunk, int lane, int32_t H,
                             const int32_t *__restrict__ offset, const int32_t *__restrict__ counts,
                             int64_t T, void *__restrict__ recv_x, void *__restrict__ recv_scales,
                             int32_t *__restrict__ recv_src_idx)
{
    const int64_t first = max((int64_t)offset[e] + counts[e], (int64_t)0);
    const int64_t end = min((int64_t)offset[e + 1], T);
    const uint4 z = make_uint4(0, 0, 0, 0);
    if (FP8) {
        const Fp8Lane l = fp8_lane(H, chunk, lane);
        Fp8Payload p;
        p.q = z;
        p.scale = 0.0f;
        p.ue8m0_word = 0;
        for (int64_t row = first; row < end; ++row) {
            store_fp8<SF>(p, l, lane, row, H, static_cast<uint8_t *>(recv_x), recv_scales);
            if (chunk == 0 && lane == 0)
                recv_src_idx[row] = -1;
        }
    } else {
        const Bf16Lane l = bf16_lane(H, chunk, lane);
        for (int64_t row = first; row < end; ++row) {
            store_bf16(z, z, l, row, H, static_cast<uint16_t *>(recv_x));
            if (chunk == 0 && lane == 0)
                recv_src_idx[row] = -1;
        }
    }
}

// Per-expert / expand pack.  Items [0, pad_items) zero the expand padding,
// one per (expert, chunk) (pad_items = 0 for the per-expert layout); the rest
// are (token, chunk) items.  Padding items come first so that their longer
// loops start early.
template <int KB, int SF, bool FP8, class Rows>
__global__ __launch_bounds__(kThreads) void pack_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t nchunks, int32_t pad_items, Rows rows,
    const int32_t *__restrict__ counts, const uint16_t *__restrict__ x,
    const int64_t *__restrict__ topk_idx, const int32_t *__restrict__ expert_slot,
    void *__restrict__ recv_x, void *__restrict__ recv_scales, int32_t *__restrict__ recv_src_idx,
    uint32_t *status)
{
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t item = blockIdx.x * kWaves + wave; // host keeps the item count < 2^31
    if (item < (uint32_t)pad_items) {
        if constexpr (__is_same(Rows, ExpandRows)) {
            const int32_t e = (int32_t)(item / (uint32_t)nchunks);
            const int32_t chunk = (int32_t)(item - (uint32_t)e * (uint32_t)nchunks);
            zero_padding<FP8, SF>(e, chunk, lane, H, rows.offset, counts, rows.T, recv_x,
                                  recv_scales, recv_src_idx);
        }
        return;
    }
    item -= (uint32_t)pad_items;
    if (item >= (uint32_t)N * (uint32_t)nchunks)
        return;
    const uint32_t t = item / (uint32_t)nchunks;
    const int32_t chunk = (int32_t)(item - t * (uint32_t)nchunks);
    const uint16_t *x_row = x + (size_t)t * H;

    Fp8Lane fl;
    Fp8Payload p;
    Bf16Lane bl;
    uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
    if (FP8) {
        fl = fp8_lane(H, chunk, lane);
        p = quantize_lane<SF>(x_row, fl, lane);
    } else {
        bl = bf16_lane(H, chunk, lane);
        const uint4 *src = reinterpret_cast<const uint4 *>(x_row);
        if (bl.u0 < bl.units)
            a0 = load_stream(src + bl.u0);
        if (bl.u1 < bl.units)
            a1 = load_stream(src + bl.u1);
    }

    uint32_t flags = 0;
    const int64_t *idx_t = topk_idx + (size_t)t * K;
    const int32_t *slot_t = expert_slot + (size_t)t * K;
    for (int k0 = 0; k0 < K; k0 += KB) {
        int64_t row[KB];
        float unused[KB];
        fetch_entries<KB>(idx_t, slot_t, nullptr, k0, K, E, rows, lane, row, unused, flags);
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            if (row[b] >= 0) {
                if (FP8)
                    store_fp8<SF>(p, fl, lane, row[b], H, static_cast<uint8_t *>(recv_x),
                                  recv_scales);
                else
                    store_bf16(a0, a1, bl, row[b], H, static_cast<uint16_t *>(recv_x));
                if (chunk == 0 && lane == 0)
                    recv_src_idx[row[b]] = (int32_t)t;
            }
        }
    }
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

// Normal-mode pack: the token's destinations are the ranks r with
// 0 <= rank_slot[t, r] < M, row r * M + rank_slot[t, r].  The chunk-0 wave
// also writes the row's routing entries: lane k < K writes
//   recv_topk_idx[row][k]     = e - r * L if entry k routes to expert e on r,
//                               else -1;
//   recv_topk_weights[row][k] = topk_weights[t][k] for those entries, else 0.
template <int SF, bool FP8>
__global__ __launch_bounds__(kThreads) void pack_normal_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t R, int32_t M, int32_t nchunks,
    const uint16_t *__restrict__ x, const int64_t *__restrict__ topk_idx,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ rank_slot,
    void *__restrict__ recv_x, void *__restrict__ recv_scales,
    int64_t *__restrict__ recv_topk_idx, float *__restrict__ recv_topk_weights,
    int32_t *__restrict__ recv_src_idx, uint32_t *status)
{
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t item = blockIdx.x * kWaves + wave; // host keeps N * nchunks < 2^31
    if (item >= (uint32_t)N * (uint32_t)nchunks)
        return;
    const uint32_t t = item / (uint32_t)nchunks;
    const int32_t chunk = (int32_t)(item - t * (uint32_t)nchunks);
    const uint16_t *x_row = x + (size_t)t * H;
    const int32_t L = E / R;

    // this chunk of x, in flight while the rank-slot row loads
    uint4 in0 = make_uint4(0, 0, 0, 0), in1 = make_uint4(0, 0, 0, 0);
    load_chunk<FP8>(x_row, H, chunk, lane, in0, in1);
    uint32_t flags = 0;
    int32_t j;
    uint64_t dest = rank_destinations(rank_slot + (size_t)t * R, R, M, lane, j, flags);
    // the token's routing entries (chunk-0 waves write them per destination)
    int64_t id = -1;
    float wt = 0.0f;
    if (chunk == 0) {
        const int kk = min(lane, K - 1);
        id = topk_idx[(size_t)t * K + kk];
        if (topk_weights)
            wt = topk_weights[(size_t)t * K + kk];
        if (dest && __ballot(lane < K && id != -1 && (id < 0 || id >= (int64_t)E)))
            flags |= EP_STATUS_BAD_EXPERT_ID;
    }
    const bool routed = id >= 0 && id < (int64_t)E;
    const int32_t id_rank = routed ? (int32_t)id / L : -1;

    Fp8Lane fl;
    Fp8Payload p;
    Bf16Lane bl;
    const uint4 a0 = in0, a1 = in1;
    if (FP8) {
        fl = fp8_lane(H, chunk, lane);
        p = quantize_regs<SF>(in0, in1, fl, lane);
    } else {
        bl = bf16_lane(H, chunk, lane);
    }

    while (dest) {
        const int r = __builtin_ctzll(dest);
        dest &= dest - 1;
        const int64_t row = (int64_t)r * M + __builtin_amdgcn_readlane(j, r);
        if (FP8)
            store_fp8<SF>(p, fl, lane, row, H, static_cast<uint8_t *>(recv_x), recv_scales);
        else
            store_bf16(a0, a1, bl, row, H, static_cast<uint16_t *>(recv_x));
        if (chunk == 0) {
            if (lane == 0)
                recv_src_idx[row] = (int32_t)t;
            if (lane < K) {
                const bool local = id_rank == r;
                recv_topk_idx[(size_t)row * K + lane] = local ? id - (int64_t)r * L : -1;
                if (topk_weights && recv_topk_weights)
                    recv_topk_weights[(size_t)row * K + lane] = local ? wt : 0.0f;
            }
        }
    }
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

// Layout and per-expert pack in one launch.  Block t + 1 owns token t.
// Tokens fall into the layout's count blocks of tpb tokens; when the batch
// spans more than one, `hist` holds each count block's histogram (experts,
// then tokens per rank) and is otherwise null.  Block t + 1 counts, in LDS,
// the expert ids of the tokens of its own count block that precede t (thread
// i takes the i-th) and the ranks those tokens go to, and adds the earlier
// count blocks' histograms at the columns it needs: the experts of its own
// entries and every rank.  The slot of entry (t, k) -- the number of earlier
// entries with the same expert in (token, k) order -- is then that expert's
// sum plus the entries of t before k with the same expert, and the token's
// rank slot at rank r is the number of earlier tokens sent to r.  Wave w
// packs chunks w, w + W, ... (W waves per block) exactly as pack_kernel does,
// and wave 0 writes the token's layout rows.  Block 0 writes the totals and
// the offset scan: the column sums of every histogram, or, with a single
// count block, its own count of every token; it comes first so that it is
// not the launch's last block to start.  Each wave's first two chunks of x
// are loaded together with the ids, so their latencies overlap, and
// quantised once the slots are known.  Counting work per block is at most
// tpb - 1 tokens (or N for block 0 without histograms), which the host keeps
// within one thread per token.
constexpr int kSmallThreads = 512;   // no histograms: counting up to kFusedMaxTokens tokens
constexpr int kCountedThreads = 256; // with histograms: count blocks of up to 256 tokens

template <int KMAX, int SF, bool FP8, int THREADS>
__global__ __launch_bounds__(THREADS) void layout_pack_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t R, int32_t S, int32_t A, int32_t nchunks,
    const int32_t *__restrict__ hist, int32_t tpb, int32_t stride,
    const uint16_t *__restrict__ x, const int64_t *__restrict__ topk_idx,
    int32_t *__restrict__ num_tokens_per_rank, int32_t *__restrict__ num_tokens_per_expert,
    uint8_t *__restrict__ is_token_in_rank, int32_t *__restrict__ expert_slot,
    int32_t *__restrict__ rank_slot, int32_t *__restrict__ expert_offset,
    void *__restrict__ recv_x, void *__restrict__ recv_scales, int32_t *__restrict__ recv_src_idx,
    uint32_t *status)
{
    constexpr int kWavesPerBlock = THREADS / 64;
    constexpr int kHistLoads = 4; // histogram values in flight per thread
    __shared__ int32_t s_hist[EP_MAX_EXPERTS + EP_MAX_RANKS]; // experts, then ranks
    __shared__ int32_t s_base[EP_MAX_TOPK + EP_MAX_RANKS];    // own entries' experts, then ranks
    __shared__ int32_t s_own[EP_MAX_TOPK];                    // this token's experts (-1: none)
    __shared__ int32_t s_bad;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = (int)blockIdx.x - 1; // the token, or -1 for the totals block
    const int W = E + R;
    const uint32_t magic = rank_magic(E / R);
    const bool own = t >= 0;
    // the tokens this block counts, [c0, c1), and the number of earlier
    // count blocks whose histograms it adds
    const int c0 = own && hist ? t / tpb * tpb : 0;
    const int c1 = own ? t : (hist ? 0 : N);
    const int nb = hist ? (own ? t / tpb : (N + tpb - 1) / tpb) : 0;

    // 1. loads: ids of the counted token `c0 + tid`; this token's entry
    //    `lane` (every wave); the raw x of this wave's first two chunks
    int32_t e[KMAX];
    uint32_t bad = 0;
    load_token<KMAX>(topk_idx, (int64_t)c0 + tid, c1, K, E, e, bad);
    const int64_t id = own ? topk_idx[(size_t)t * K + min(lane, K - 1)] : -1;
    const uint16_t *x_row = x + (size_t)(own ? t : 0) * H;
    uint4 xr[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        xr[c][0] = make_uint4(0, 0, 0, 0);
        xr[c][1] = make_uint4(0, 0, 0, 0);
        const int chunk = wave + c * kWavesPerBlock;
        if (own && chunk < nchunks)
            load_chunk<FP8>(x_row, H, chunk, lane, xr[c][0], xr[c][1]);
    }
    for (int i = tid; i < W; i += THREADS)
        s_hist[i] = 0;
    for (int i = tid; i < K + R; i += THREADS)
        s_base[i] = 0;
    if (tid == 0)
        s_bad = 0;
    // this token's entries: lane k < K of every wave holds entry k
    const bool in_k = lane < K;
    const bool routed = in_k && id >= 0 && id < (int64_t)E;
    const int32_t e32 = routed ? (int32_t)id : -1;
    if (wave == 0 && in_k)
        s_own[lane] = e32;
    __syncthreads();

    // 2. counts of the counted tokens' entries and of their ranks
    uint64_t ranks = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (e[k] >= 0) {
            atomicAdd(&s_hist[e[k]], 1);
            ranks |= 1ull << rank_of(e[k], magic);
        }
    }
    for (uint64_t m = ranks; m; m &= m - 1)
        atomicAdd(&s_hist[E + __builtin_ctzll(m)], 1);
    if (bad)
        s_bad = 1;
    // histogram values: a token's block takes pair i = (count block
    // i / (K + R), column i % (K + R)), where column k < K is entry k's
    // expert and the rest are the ranks; the totals block takes every column
    // of every row
    const int cols = own ? K + R : W;
    const int n = nb * cols;
    for (int i0 = tid; i0 < n; i0 += THREADS * kHistLoads) {
        int32_t v[kHistLoads];
        int32_t dst[kHistLoads];
#pragma unroll
        for (int u = 0; u < kHistLoads; ++u) {
            const int i = i0 + u * THREADS;
            const int blk = i / cols;
            const int c = i - blk * cols;
            const int col = !own ? c : c < K ? s_own[min(c, K - 1)] : E + (c - K);
            dst[u] = i < n && col >= 0 ? c : -1;
            v[u] = dst[u] >= 0 ? hist[(size_t)blk * stride + col] : 0;
        }
#pragma unroll
        for (int u = 0; u < kHistLoads; ++u)
            if (dst[u] >= 0)
                atomicAdd(own ? &s_base[dst[u]] : &s_hist[dst[u]], v[u]);
    }
    __syncthreads();

    if (!own) {
        // 3a. totals block: counts, then the offset scan on wave 0 (each
        //     lane a run of consecutive experts)
        for (int i = tid; i < W; i += THREADS) {
            if (i < E)
                num_tokens_per_expert[i] = s_hist[i];
            else
                num_tokens_per_rank[i - E] = s_hist[i];
        }
        if (wave == 0 && expert_offset) {
            const int per = (E + 63) / 64;
            const int first = lane * per;
            int local = 0;
            for (int i = 0; i < per; ++i)
                if (first + i < E)
                    local += (s_hist[first + i] + A - 1) / A * A;
            int incl = local;
            for (int off = 1; off < 64; off <<= 1) {
                const int up = __shfl_up(incl, off, 64);
                if (lane >= off)
                    incl += up;
            }
            int run = incl - local;
            for (int i = 0; i < per; ++i) {
                if (first + i < E) {
                    expert_offset[first + i] = run;
                    run += (s_hist[first + i] + A - 1) / A * A;
                }
            }
            if (lane == 63)
                expert_offset[E] = incl;
        }
        if (tid == 0 && status && s_bad)
            atomicOr(status, EP_STATUS_BAD_EXPERT_ID);
        return;
    }

    // 3b. slots of this token's entries and ranks
    int occ = 0;
    uint64_t tok_ranks = 0;
    for (int k2 = 0; k2 < K; ++k2) {
        const int32_t o = __builtin_amdgcn_readlane(e32, k2);
        occ += (k2 < lane && o >= 0 && o == e32) ? 1 : 0;
        if (o >= 0)
            tok_ranks |= 1ull << rank_of(o, magic);
    }
    const int32_t slot = routed ? s_base[lane] + s_hist[e32] + occ : -1;
    const bool slot_ok = routed && slot < S;
    const int64_t row = slot_ok ? (int64_t)e32 * S + slot : -1;
    uint32_t flags = 0;
    if (__ballot(in_k && id != -1 && !routed))
        flags |= EP_STATUS_BAD_EXPERT_ID;
    if (__ballot(routed && !slot_ok))
        flags |= EP_STATUS_BAD_SLOT;
    if (wave == 0) {
        if (in_k)
            expert_slot[(size_t)t * K + lane] = slot;
        if (lane < R) {
            const bool in = (tok_ranks >> lane) & 1ull;
            rank_slot[(size_t)t * R + lane] = in ? s_base[K + lane] + s_hist[E + lane] : -1;
            is_token_in_rank[(size_t)t * R + lane] = in ? 1 : 0;
        }
        if (flags && status && lane == 0)
            atomicOr(status, flags);
    }

    // 4. pack: the first two chunks are loaded; later ones load here
    const int32_t r_lo = (int32_t)(uint32_t)(uint64_t)row;
    const int32_t r_hi = (int32_t)(uint32_t)((uint64_t)row >> 32);
    for (int chunk = wave, c = 0; chunk < nchunks; chunk += kWavesPerBlock, ++c) {
        uint4 in0 = make_uint4(0, 0, 0, 0), in1 = make_uint4(0, 0, 0, 0);
        if (c == 0) {
            in0 = xr[0][0];
            in1 = xr[0][1];
        } else if (c == 1) {
            in0 = xr[1][0];
            in1 = xr[1][1];
        } else {
            load_chunk<FP8>(x_row, H, chunk, lane, in0, in1);
        }
        Fp8Lane fl;
        Fp8Payload p;
        Bf16Lane bl;
        if (FP8) {
            fl = fp8_lane(H, chunk, lane);
            p = quantize_regs<SF>(in0, in1, fl, lane);
        } else {
            bl = bf16_lane(H, chunk, lane);
        }
        for (int k2 = 0; k2 < K; ++k2) {
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane(r_lo, k2);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane(r_hi, k2);
            const int64_t r = (int64_t)(((uint64_t)hi << 32) | lo);
            if (r < 0)
                continue;
            if (FP8)
                store_fp8<SF>(p, fl, lane, r, H, static_cast<uint8_t *>(recv_x), recv_scales);
            else
                store_bf16(in0, in1, bl, r, H, static_cast<uint16_t *>(recv_x));
            if (chunk == 0 && lane == 0)
                recv_src_idx[r] = (int32_t)t;
        }
    }
}

// Sum over each group of G consecutive lanes (G a power of two up to 64),
// every lane of the group ending with it: DPP moves within 8 lanes and the
// 16-lane row, cross-row steps by lane permutes.
template <int G>
__device__ __forceinline__ int group_sum(int v)
{
    if (G >= 2)
        v += (int)dpp<kDppXor1>((uint32_t)v);
    if (G >= 4)
        v += (int)dpp<kDppXor2>((uint32_t)v);
    if (G >= 8)
        v += (int)dpp<kDppHalfMirror>((uint32_t)v);
    if (G >= 16)
        v += __shfl_xor(v, 8, 64);
    if (G >= 32)
        v += __shfl_xor(v, 16, 64);
    if (G >= 64)
        v += __shfl_xor(v, 32, 64);
    return v;
}

// The pack of ep_layout_dispatch above kFusedCountedMaxTokens tokens: the
// layout left each entry's rank within its 256-token block (local_slot) and
// one histogram row per block; an entry's slot is its local slot plus the
// counts of its expert in every earlier block.  Each block packs T tokens
// (T = 2 when a token has at most kWaves chunks, so every wave still gets two
// chunks; otherwise 1); block 0 sums every histogram row into the totals and
// writes the offset scan.  Item j of a block is chunk j mod nchunks of its
// token j / nchunks:
//  1. every wave loads x of its first two items;
//  2. wave q < T computes the rows of the block's token q once: a group of
//     64 / KB lanes takes entry k of a batch, each lane a share of the earlier
//     blocks' rows, and a reduction within the group gives the prefix; the
//     same for the column of the entry's rank.  It writes the token's
//     expert_slot row, its rank rows and recv_src_idx, and leaves the rows in
//     LDS;
//  3. after one barrier, wave w quantises items w, w + 4, ... once and stores
//     each to every row of its token, as pack_kernel does.
template <int KB, int SF, bool FP8, int T>
__global__ __launch_bounds__(kThreads) void pack_local_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t R, int32_t S, int32_t A, int32_t nchunks,
    int32_t tpb, int32_t B, int32_t stride, const int32_t *__restrict__ hist,
    const int32_t *__restrict__ local_slot, const int32_t *__restrict__ local_rank,
    const uint16_t *__restrict__ x, const int64_t *__restrict__ topk_idx,
    int32_t *__restrict__ num_tokens_per_rank, int32_t *__restrict__ num_tokens_per_expert,
    uint8_t *__restrict__ is_token_in_rank, int32_t *__restrict__ expert_slot,
    int32_t *__restrict__ rank_slot, int32_t *__restrict__ expert_offset, void *__restrict__ recv_x,
    void *__restrict__ recv_scales, int32_t *__restrict__ recv_src_idx, uint32_t *status)
{
    static_assert(KB == 1 || KB == 2 || KB == 4 || KB == 8, "KB divides the wave");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (blockIdx.x == 0) {
        // totals: column sums of all B rows, then the counts and the scan
        __shared__ int32_t s_tot[EP_MAX_EXPERTS + EP_MAX_RANKS];
        const int W = E + R;
        for (int c = threadIdx.x; c < W; c += kThreads) {
            int sum = 0;
            for (int r = 0; r < B; ++r)
                sum += hist[(size_t)r * stride + c];
            s_tot[c] = sum;
            if (c < E)
                num_tokens_per_expert[c] = sum;
            else
                num_tokens_per_rank[c - E] = sum;
        }
        __syncthreads();
        if (wave == 0 && expert_offset) {
            const int per = (E + 63) / 64;
            const int first = lane * per;
            int local = 0;
            for (int i = 0; i < per; ++i)
                if (first + i < E)
                    local += (s_tot[first + i] + A - 1) / A * A;
            int incl = local;
            for (int off = 1; off < 64; off <<= 1) {
                const int up = __shfl_up(incl, off, 64);
                if (lane >= off)
                    incl += up;
            }
            int run = incl - local;
            for (int i = 0; i < per; ++i) {
                if (first + i < E) {
                    expert_offset[first + i] = run;
                    run += (s_tot[first + i] + A - 1) / A * A;
                }
            }
            if (lane == 63)
                expert_offset[E] = incl;
        }
        return;
    }
    static_assert(T >= 1 && T <= kWaves, "a wave per token's rows");
    __shared__ int64_t s_row[T][EP_MAX_TOPK];
    const uint32_t t0 = (blockIdx.x - 1) * (uint32_t)T; // host launches 1 + ceil(N / T) blocks
    const int tokens = min(T, N - (int)t0);
    const int items = tokens * nchunks;

    // 1. x of this wave's first two items
    uint4 xr[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        xr[c][0] = make_uint4(0, 0, 0, 0);
        xr[c][1] = make_uint4(0, 0, 0, 0);
        const int j = wave + c * kWaves;
        if (j < items) {
            const int q = T == 1 ? 0 : j / nchunks;
            load_chunk<FP8>(x + (size_t)(t0 + q) * H, H, j - q * nchunks, lane, xr[c][0], xr[c][1]);
        }
    }

    // 2. each token's rows and layout rows (wave q for token q)
    if (wave < tokens) {
        const uint32_t t = t0 + wave;
        constexpr int G = 64 / KB;
        const int blk = (int)(t / (uint32_t)tpb); // earlier blocks: 0 .. blk-1
        const int kq = lane / G;
        const int m = lane & (G - 1);
        const uint32_t magic = rank_magic(E / R);
        uint32_t flags = 0;
        int32_t my_local = -1, my_before = 0; // lane r < R: rank r
        const int64_t *idx_t = topk_idx + (size_t)t * K;
        const int32_t *ls_t = local_slot + (size_t)t * K;
        const int32_t *lr_t = local_rank + (size_t)t * K;
        for (int k0 = 0; k0 < K; k0 += KB) {
            const int kk = min(k0 + kq, K - 1);
            const bool in_k = k0 + kq < K;
            const int64_t id = idx_t[kk];
            const int32_t ls = ls_t[kk];
            const int32_t lr0 = lr_t[kk];
            const bool routed = in_k && id >= 0 && id < (int64_t)E;
            const int32_t e32 = routed ? (int32_t)id : 0;
            const int32_t rk = routed ? rank_of(e32, magic) : 0;
            int acc = 0, racc = 0;
            if (routed) {
                for (int r = m; r < blk; r += G) {
                    acc += hist[(size_t)r * stride + e32];
                    racc += hist[(size_t)r * stride + E + rk];
                }
            }
            acc = group_sum<G>(acc);
            racc = group_sum<G>(racc);
            const int32_t slot = ls + acc;
            const bool slot_ok = routed && slot < S;
            const int64_t rr = slot_ok ? (int64_t)e32 * S + slot : -1;
            const bool head = m == 0; // one lane per entry
            if (__ballot(head && in_k && id != -1 && !routed))
                flags |= EP_STATUS_BAD_EXPERT_ID;
            if (__ballot(head && routed && !slot_ok))
                flags |= EP_STATUS_BAD_SLOT;
            if (head && in_k) {
                expert_slot[(size_t)t * K + k0 + kq] = routed ? slot : -1;
                s_row[wave][k0 + kq] = rr;
                if (rr >= 0)
                    recv_src_idx[rr] = (int32_t)t;
            }
            const int32_t lr = routed ? lr0 : -1;
#pragma unroll
            for (int bb = 0; bb < KB; ++bb) {
                const int32_t rk_b = __builtin_amdgcn_readlane(routed ? rk : -1, bb * G);
                const int32_t lr_b = __builtin_amdgcn_readlane(lr, bb * G);
                const int32_t before_b = __builtin_amdgcn_readlane(racc, bb * G);
                if (rk_b == lane && lr_b >= 0) {
                    my_local = lr_b;
                    my_before = before_b;
                }
            }
        }
        if (lane < R) {
            rank_slot[(size_t)t * R + lane] = my_local >= 0 ? my_local + my_before : -1;
            is_token_in_rank[(size_t)t * R + lane] = my_local >= 0 ? 1 : 0;
        }
        if (flags && status && lane == 0)
            atomicOr(status, flags);
    }
    __syncthreads();

    // 3. pack: the first two items are loaded; later ones load here
    for (int j = wave, c = 0; j < items; j += kWaves, ++c) {
        const int q = T == 1 ? 0 : j / nchunks;
        const int chunk = j - q * nchunks;
        uint4 in0 = make_uint4(0, 0, 0, 0), in1 = make_uint4(0, 0, 0, 0);
        if (c == 0) {
            in0 = xr[0][0];
            in1 = xr[0][1];
        } else if (c == 1) {
            in0 = xr[1][0];
            in1 = xr[1][1];
        } else {
            load_chunk<FP8>(x + (size_t)(t0 + q) * H, H, chunk, lane, in0, in1);
        }
        Fp8Lane fl;
        Fp8Payload p;
        Bf16Lane bl;
        if (FP8) {
            fl = fp8_lane(H, chunk, lane);
            p = quantize_regs<SF>(in0, in1, fl, lane);
        } else {
            bl = bf16_lane(H, chunk, lane);
        }
        for (int k = 0; k < K; ++k) {
            const int64_t row = s_row[q][k];
            if (row < 0)
                continue;
            if (FP8)
                store_fp8<SF>(p, fl, lane, row, H, static_cast<uint8_t *>(recv_x), recv_scales);
            else
                store_bf16(in0, in1, bl, row, H, static_cast<uint16_t *>(recv_x));
        }
    }
}

int batch_of(int K) { return K == 1 ? 1 : K == 2 ? 2 : K <= 4 ? 4 : 8; }

// Launch of the per-expert / expand pack for every (batch, scale format,
// FP8 / BF16) combination.
template <class Rows>
hipError_t launch_pack(const ep_shape &s, int32_t pad_items, const Rows &rows,
                       const int32_t *counts, const uint16_t *x, const int64_t *topk_idx,
                       const int32_t *expert_slot, void *recv_x, void *recv_scales,
                       int32_t *recv_src_idx, uint32_t *status, hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, E = s.num_experts;
    const int nchunks = (H + kChunk - 1) / kChunk;
    const int64_t items = (int64_t)pad_items + (int64_t)N * nchunks;
    if (items == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((items + kWaves - 1) / kWaves));
    const int kb = batch_of(K);
#define EP_PACK(KB, SF, FP8)                                                                       \
    hipLaunchKernelGGL((pack_kernel<KB, SF, FP8, Rows>), grid, dim3(kThreads), 0, stream, N, H, K, \
                       E, nchunks, pad_items, rows, counts, x, topk_idx, expert_slot, recv_x,      \
                       recv_scales, recv_src_idx, status)
#define EP_PACK_KB(SF, FP8)                                                                        \
    do {                                                                                           \
        if (kb == 1)                                                                               \
            EP_PACK(1, SF, FP8);                                                                   \
        else if (kb == 2)                                                                          \
            EP_PACK(2, SF, FP8);                                                                   \
        else if (kb == 4)                                                                          \
            EP_PACK(4, SF, FP8);                                                                   \
        else                                                                                       \
            EP_PACK(8, SF, FP8);                                                                   \
    } while (0)
    if (!s.use_fp8)
        EP_PACK_KB(EP_SCALE_FP32, false);
    else if (s.scale_format == EP_SCALE_POW2)
        EP_PACK_KB(EP_SCALE_POW2, true);
    else if (s.scale_format == EP_SCALE_UE8M0)
        EP_PACK_KB(EP_SCALE_UE8M0, true);
    else
        EP_PACK_KB(EP_SCALE_FP32, true);
#undef EP_PACK_KB
#undef EP_PACK
    return hipGetLastError();
}

} // namespace

hipError_t launch_dispatch(const ep_shape &s, const uint16_t *x, const int64_t *topk_idx,
                           const int32_t *expert_slot, void *recv_x, void *recv_scales,
                           int32_t *recv_src_idx, uint32_t *status, hipStream_t stream)
{
    return launch_pack(s, 0, DenseRows{s.expert_capacity}, nullptr, x, topk_idx, expert_slot,
                       recv_x, recv_scales, recv_src_idx, status, stream);
}

hipError_t launch_layout_dispatch(const ep_shape &s, const LayoutPlan &plan, const int32_t *hist,
                                  const uint16_t *x, const int64_t *topk_idx,
                                  int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                                  uint8_t *is_token_in_rank, int32_t *expert_slot,
                                  int32_t *rank_slot, int32_t *expert_offset, void *recv_x,
                                  void *recv_scales, int32_t *recv_src_idx, uint32_t *status,
                                  hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, E = s.num_experts;
    const int R = s.num_ranks, S = s.expert_capacity, A = expert_alignment(s);
    const int nchunks = (H + kChunk - 1) / kChunk;
    const int tpb = plan.tokens_per_block, stride = plan.hist_stride;
    // One counting thread per token: without histograms a 512-thread block
    // (8 waves, all chunks of a 7,168-wide row at once) counts up to every
    // token; with them a 256-thread block (twice the blocks per CU) counts
    // the earlier tokens of one count block.
    if (hist ? tpb > kCountedThreads || N > kFusedCountedMaxTokens : N > kFusedMaxTokens)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(N + 1));
#define EP_FUSED(KMAX, SF, FP8, T)                                                                 \
    hipLaunchKernelGGL((layout_pack_kernel<KMAX, SF, FP8, T>), grid, dim3(T), 0, stream, N, H, K, \
                       E, R, S, A, nchunks, hist, tpb, stride, x, topk_idx, num_tokens_per_rank,   \
                       num_tokens_per_expert, is_token_in_rank, expert_slot, rank_slot,            \
                       expert_offset, recv_x, recv_scales, recv_src_idx, status)
#define EP_FUSED_T(KMAX, SF, FP8)                                                                  \
    do {                                                                                           \
        if (hist)                                                                                  \
            EP_FUSED(KMAX, SF, FP8, kCountedThreads);                                              \
        else                                                                                       \
            EP_FUSED(KMAX, SF, FP8, kSmallThreads);                                                \
    } while (0)
#define EP_FUSED_SF(KMAX)                                                                          \
    do {                                                                                           \
        if (!s.use_fp8)                                                                            \
            EP_FUSED_T(KMAX, EP_SCALE_FP32, false);                                                \
        else if (s.scale_format == EP_SCALE_POW2)                                                  \
            EP_FUSED_T(KMAX, EP_SCALE_POW2, true);                                                 \
        else if (s.scale_format == EP_SCALE_UE8M0)                                                 \
            EP_FUSED_T(KMAX, EP_SCALE_UE8M0, true);                                                \
        else                                                                                       \
            EP_FUSED_T(KMAX, EP_SCALE_FP32, true);                                                 \
    } while (0)
    if (K <= 8)
        EP_FUSED_SF(8);
    else if (K <= 16)
        EP_FUSED_SF(16);
    else
        EP_FUSED_SF(EP_MAX_TOPK);
#undef EP_FUSED_SF
#undef EP_FUSED_T
#undef EP_FUSED
    return hipGetLastError();
}

hipError_t launch_dispatch_local(const ep_shape &s, const LayoutPlan &plan, const LocalWorkspace &ws,
                                 const uint16_t *x, const int64_t *topk_idx,
                                 int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                                 uint8_t *is_token_in_rank, int32_t *expert_slot,
                                 int32_t *rank_slot, int32_t *expert_offset, void *recv_x,
                                 void *recv_scales, int32_t *recv_src_idx, uint32_t *status,
                                 hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, E = s.num_experts;
    const int R = s.num_ranks, S = s.expert_capacity, A = expert_alignment(s);
    if (N == 0)
        return hipSuccess;
    const int nchunks = (H + kChunk - 1) / kChunk;
    // two tokens per block when a token has no more chunks than a block has
    // waves (each wave then still packs two chunks), else one
    const int T = nchunks <= kWaves ? 2 : 1;
    const dim3 grid((unsigned)(1 + (N + T - 1) / T)); // block 0: totals
    const int kb = batch_of(K);
#define EP_LOCAL_T(KB, SF, FP8, TT)                                                                \
    hipLaunchKernelGGL((pack_local_kernel<KB, SF, FP8, TT>), grid, dim3(kThreads), 0, stream, N,   \
                       H, K, E, R, S, A, nchunks, plan.tokens_per_block, plan.num_blocks,          \
                       plan.hist_stride, ws.hist, ws.local_slot, ws.local_rank, x, topk_idx,       \
                       num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank, expert_slot,  \
                       rank_slot, expert_offset, recv_x, recv_scales, recv_src_idx, status)
#define EP_LOCAL(KB, SF, FP8)                                                                      \
    do {                                                                                           \
        if (T == 2)                                                                                \
            EP_LOCAL_T(KB, SF, FP8, 2);                                                            \
        else                                                                                       \
            EP_LOCAL_T(KB, SF, FP8, 1);                                                            \
    } while (0)
#define EP_LOCAL_KB(SF, FP8)                                                                       \
    do {                                                                                           \
        if (kb == 1)                                                                               \
            EP_LOCAL(1, SF, FP8);                                                                  \
        else if (kb == 2)                                                                          \
            EP_LOCAL(2, SF, FP8);                                                                  \
        else if (kb == 4)                                                                          \
            EP_LOCAL(4, SF, FP8);                                                                  \
        else                                                                                       \
            EP_LOCAL(8, SF, FP8);                                                                  \
    } while (0)
    if (!s.use_fp8)
        EP_LOCAL_KB(EP_SCALE_FP32, false);
    else if (s.scale_format == EP_SCALE_POW2)
        EP_LOCAL_KB(EP_SCALE_POW2, true);
    else if (s.scale_format == EP_SCALE_UE8M0)
        EP_LOCAL_KB(EP_SCALE_UE8M0, true);
    else
        EP_LOCAL_KB(EP_SCALE_FP32, true);
#undef EP_LOCAL_KB
#undef EP_LOCAL
#undef EP_LOCAL_T
    return hipGetLastError();
}

hipError_t launch_dispatch_expand(const ep_shape &s, const uint16_t *x, const int64_t *topk_idx,
                                  const int32_t *expert_slot, const int32_t *expert_offset,
                                  const int32_t *num_tokens_per_expert, void *recv_x,
                                  void *recv_scales, int32_t *recv_src_idx, uint32_t *status,
                                  hipStream_t stream)
{
    const int nchunks = (s.hidden + kChunk - 1) / kChunk;
    return launch_pack(s, s.num_experts * nchunks, ExpandRows{expert_offset, expand_rows(s)},
                       num_tokens_per_expert, x, topk_idx, expert_slot, recv_x, recv_scales,
                       recv_src_idx, status, stream);
}

hipError_t launch_dispatch_normal(const ep_shape &s, const uint16_t *x, const int64_t *topk_idx,
                                  const float *topk_weights, const int32_t *rank_slot,
                                  void *recv_x, void *recv_scales, int64_t *recv_topk_idx,
                                  float *recv_topk_weights, int32_t *recv_src_idx,
                                  uint32_t *status, hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, E = s.num_experts;
    const int R = s.num_ranks, M = s.num_max_dispatch_tokens_per_rank;
    if (N == 0)
        return hipSuccess;
    const int nchunks = (H + kChunk - 1) / kChunk;
    const int64_t items = (int64_t)N * nchunks;
    const dim3 grid((unsigned)((items + kWaves - 1) / kWaves));
#define EP_PACK_NORMAL(SF, FP8)                                                                    \
    hipLaunchKernelGGL((pack_normal_kernel<SF, FP8>), grid, dim3(kThreads), 0, stream, N, H, K, E, \
                       R, M, nchunks, x, topk_idx, topk_weights, rank_slot, recv_x, recv_scales,   \
                       recv_topk_idx, recv_topk_weights, recv_src_idx, status)
    if (!s.use_fp8)
        EP_PACK_NORMAL(EP_SCALE_FP32, false);
    else if (s.scale_format == EP_SCALE_POW2)
        EP_PACK_NORMAL(EP_SCALE_POW2, true);
    else if (s.scale_format == EP_SCALE_UE8M0)
        EP_PACK_NORMAL(EP_SCALE_UE8M0, true);
    else
        EP_PACK_NORMAL(EP_SCALE_FP32, true);
#undef EP_PACK_NORMAL
    return hipGetLastError();
}

} // namespace ep
