// layout.hip -- dispatch layout on gfx950 (DeepEP V1 Legacy guide §5.2(1):
// tokens per rank, tokens per expert and is_token_in_rank, computed from
// topk_idx before any data moves; DeepEP Ascend deep dive, "Dispatch's Three
// Phases": count per expert and per destination card; "Two Transfers": a card
// gets one copy of a token however many of its experts it hosts).
//
// Receive slots follow (token, k) order: the slot of entry (t, k) is the
// number of entries before it with the same expert, so the result is unique
// and the kernels are deterministic by construction (no global atomics).
//
// Tokens are split into blocks of 256, one token per lane, the token's K
// expert ids held in registers.  Two kernels:
//   count : per-block histogram -> workspace[b][0..E+R) (expert entries, and
//           tokens per rank, each token counted once per rank);
//   assign: each block sums the histograms of the blocks before it (one
//           coalesced pass with all loads in flight), ranks its own entries
//           with LDS bitmaps -- one 64-bit word per (wave, expert) and per
//           (wave, rank), bit = lane.  One pass over the columns turns the
//           words into a base per (wave, column): earlier blocks' count plus
//           the popcounts of the earlier waves' words.  An entry's slot is
//           then its wave's base plus the popcount of the lower bits of its
//           own wave's word.  One extra block sums every histogram row at the
//           same time and writes the totals and the offset scan.
// The count kernel is skipped when one block covers every token; that block
// then counts its own totals.
//
// A token may name one expert more than once.  Each repeat gets its own
// slot in k order: occurrence o of an expert within a token is ranked in
// bitmap "layer" o, and an entry's prefix sums the layers.  Routings without
// repeats take exactly one layer.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = 256; // = tokens per block, one per lane
constexpr int kGroups = kThreads / 64;
constexpr int kHistBatch = 8; // int4 histogram loads in flight per thread
// Up to this many ranks, per-rank work is one ballot per rank; above it, each
// token visits only its own ranks (at most K of them) with LDS atomics.
constexpr int kBallotRanks = 16;

__device__ __forceinline__ uint64_t bits_below(int bit) { return (1ull << bit) - 1ull; }

// Number of entries of `e` among the block's tokens before this lane's token
// (same layer): lower bits of this wave's word plus the earlier waves' words.
__device__ __forceinline__ int prefix_in_block(const uint64_t *words, int stride, int g, int lane)
{
    int cnt = __popcll(words[g * stride] & bits_below(lane));
#pragma unroll
    for (int g2 = 0; g2 < kGroups - 1; ++g2)
        if (g2 < g)
            cnt += __popcll(words[g2 * stride]);
    return cnt;
}

template <int KMAX>
__global__ __launch_bounds__(kThreads) void layout_count_kernel(
    int32_t N, int32_t K, int32_t E, int32_t R, int32_t L, int32_t stride,
    const int64_t *__restrict__ topk_idx, int32_t *__restrict__ hist)
{
    extern __shared__ int32_t s_cnt[]; // [E + R]
    const int tid = threadIdx.x;
    int32_t e[KMAX];
    uint32_t bad = 0;
    load_token<KMAX>(topk_idx, (int64_t)blockIdx.x * kThreads + tid, N, K, E, e, bad);
    for (int i = tid; i < E + R; i += kThreads)
        s_cnt[i] = 0;
    __syncthreads();
    const uint32_t magic = rank_magic(L);
    uint64_t ranks = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (e[k] >= 0) {
            atomicAdd(&s_cnt[e[k]], 1);
            ranks |= 1ull << rank_of(e[k], magic);
        }
    }
    // tokens per rank: one ballot per rank gives the wave's count directly;
    // with many ranks each token adds itself to its own ranks instead
    if (R <= kBallotRanks) {
        for (int r = 0; r < R; ++r) {
            const uint64_t m = __ballot((ranks >> r) & 1ull);
            if ((tid & 63) == 0 && m)
                atomicAdd(&s_cnt[E + r], __popcll(m));
        }
    } else {
        for (uint64_t m = ranks; m; m &= m - 1)
            atomicAdd(&s_cnt[E + __builtin_ctzll(m)], 1);
    }
    __syncthreads();
    int32_t *row = hist + (size_t)blockIdx.x * stride;
    for (int i = tid; i < stride; i += kThreads)
        row[i] = i < E + R ? s_cnt[i] : 0;
}

__host__ __device__ inline size_t assign_lds_bytes(int E, int R)
{
    // bitmaps [kGroups][E + R] (u64), wave bases [kGroups][E + R], totals
    // [E + R], misc [8]
    return sizeof(uint64_t) * (size_t)kGroups * (E + R) + sizeof(int32_t) * (size_t)kGroups * (E + R) +
           sizeof(int32_t) * (size_t)(E + R) + sizeof(int32_t) * 8;
}

// Rows of expert queue with c entries under expert alignment A >= 1 (the
// expand layout of the Ascend deep dive, phase 1: queues padded to a
// multiple of A; A = 1 gives the plain count).
__device__ __forceinline__ int aligned_count(int c, int A) { return (c + A - 1) / A * A; }

// Totals in s_tot[0..E+R) (LDS, complete) -> num_tokens_per_expert,
// num_tokens_per_rank and the exclusive offset scan of the aligned counts
// (expert_offset nullable).  Called by all kThreads threads of one block;
// uses s_misc[4..8).
__device__ void write_totals_and_offsets(int E, int R, int A, const int32_t *s_tot, int32_t *s_misc,
                                         int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                                         int32_t *expert_offset)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int g = tid >> 6;
    for (int i = tid; i < E + R; i += kThreads) {
        if (i < E)
            num_tokens_per_expert[i] = s_tot[i];
        else
            num_tokens_per_rank[i - E] = s_tot[i];
    }
    if (!expert_offset)
        return;
    const int per = (E + kThreads - 1) / kThreads;
    const int start = tid * per;
    int local = 0;
    for (int i = 0; i < per; ++i)
        if (start + i < E)
            local += aligned_count(s_tot[start + i], A);
    int incl = local;
    for (int off = 1; off < 64; off <<= 1) {
        const int up = __shfl_up(incl, off, 64);
        if (lane >= off)
            incl += up;
    }
    if (lane == 63)
        s_misc[4 + g] = incl;
    __syncthreads();
    int woff = 0;
    for (int g2 = 0; g2 < g; ++g2)
        woff += s_misc[4 + g2];
    int run = woff + incl - local;
    for (int i = 0; i < per; ++i) {
        if (start + i < E) {
            expert_offset[start + i] = run;
            run += aligned_count(s_tot[start + i], A);
        }
    }
    if (tid == kThreads - 1)
        expert_offset[E] = woff + incl;
}

// The extra block of a multi-block layout: column sums of all B histogram
// rows (int4 loads, kHistBatch in flight per thread), then totals and scan.
__device__ void layout_totals(int B, int E, int R, int A, int stride, const int32_t *__restrict__ hist,
                              int32_t *s_tot, int32_t *s_misc, int32_t *num_tokens_per_rank,
                              int32_t *num_tokens_per_expert, int32_t *expert_offset)
{
    const int tid = threadIdx.x;
    for (int i = tid; i < E + R; i += kThreads)
        s_tot[i] = 0;
    __syncthreads();
    const int n4 = B * (stride / 4);
    const int4 *h4 = reinterpret_cast<const int4 *>(hist);
    for (int i0 = tid; i0 < n4; i0 += kThreads * kHistBatch) {
        int4 hv[kHistBatch];
#pragma unroll
        for (int u = 0; u < kHistBatch; ++u) {
            const int i = i0 + u * kThreads;
            hv[u] = i < n4 ? h4[i] : make_int4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kHistBatch; ++u) {
            const int i = i0 + u * kThreads;
            if (i < n4) {
                const int c = (i * 4) % stride;
                if (c < E + R)
                    atomicAdd(&s_tot[c], hv[u].x);
                if (c + 1 < E + R)
                    atomicAdd(&s_tot[c + 1], hv[u].y);
                if (c + 2 < E + R)
                    atomicAdd(&s_tot[c + 2], hv[u].z);
                if (c + 3 < E + R)
                    atomicAdd(&s_tot[c + 3], hv[u].w);
            }
        }
    }
    __syncthreads();
    write_totals_and_offsets(E, R, A, s_tot, s_misc, num_tokens_per_rank, num_tokens_per_expert,
                             expert_offset);
}

template <int KMAX>
__global__ __launch_bounds__(kThreads) void layout_assign_kernel(
    int32_t N, int32_t K, int32_t E, int32_t R, int32_t L, int32_t A, int32_t stride,
    const int64_t *__restrict__ topk_idx, const int32_t *__restrict__ hist,
    int32_t *__restrict__ num_tokens_per_rank, int32_t *__restrict__ num_tokens_per_expert,
    uint8_t *__restrict__ is_token_in_rank, int32_t *__restrict__ expert_slot,
    int32_t *__restrict__ rank_slot, int32_t *__restrict__ expert_offset, uint32_t *status)
{
    extern __shared__ __align__(16) char lds_raw[];
    const int W = E + R; // one column per expert, then one per rank
    uint64_t *s_bm = reinterpret_cast<uint64_t *>(lds_raw); // [kGroups][W]: expert, then rank words
    int32_t *s_wb = reinterpret_cast<int32_t *>(s_bm + (size_t)kGroups * W); // [kGroups][W]
    int32_t *s_tot = s_wb + (size_t)kGroups * W;                             // [W]
    int32_t *s_misc = s_tot + W;                                             // [8]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int g = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x;
    const int num_token_blocks = hist ? (int)gridDim.x - 1 : 1;
    if (b == num_token_blocks) {
        // the extra block: totals are the column sums of every block's
        // histogram; it writes them and the offset scan while the other
        // blocks rank their tokens
        layout_totals(num_token_blocks, E, R, A, stride, hist, s_tot, s_misc, num_tokens_per_rank,
                      num_tokens_per_expert, expert_offset);
        return;
    }
    // with a single token block there is no histogram: that block counts
    const bool last_block = hist == nullptr;
    const int64_t t = (int64_t)b * kThreads + tid;
    const bool live = t < N;

    // 1. this token's ids and the first slice of the earlier blocks'
    //    histograms (both in flight while LDS is cleared)
    int32_t e[KMAX];
    uint32_t bad = 0;
    load_token<KMAX>(topk_idx, t, N, K, E, e, bad);
    const int n4 = b * (stride / 4); // the first b histogram rows are one contiguous span
    const int4 *h4 = reinterpret_cast<const int4 *>(hist);
    int4 hv[kHistBatch];
#pragma unroll
    for (int u = 0; u < kHistBatch; ++u) {
        const int i = tid + u * kThreads;
        hv[u] = i < n4 ? h4[i] : make_int4(0, 0, 0, 0);
    }
    for (int i = tid; i < kGroups * W; i += kThreads)
        s_bm[i] = 0ull;
    for (int i = tid; i < W; i += kThreads)
        s_wb[i] = 0; // row 0: the earlier blocks' counts
    if (tid < 8)
        s_misc[tid] = 0;
    const bool vec_rows = (R & 3) == 0 && (reinterpret_cast<uintptr_t>(rank_slot) & 15) == 0 &&
                          (reinterpret_cast<uintptr_t>(is_token_in_rank) & 3) == 0;
    if (R > kBallotRanks) {
        // many ranks: the block's rank rows as "not sent", written by the
        // whole block in address order; each token's own ranks are written
        // over them after the barriers below, which order the two writes
        const int64_t t0 = (int64_t)b * kThreads;
        const int64_t rows = min((int64_t)N - t0, (int64_t)kThreads);
        if (rows > 0) {
            const int64_t n = rows * R; // entries in the block's span
            int32_t *rs_span = rank_slot + t0 * R;
            uint8_t *mask_span = is_token_in_rank + t0 * R;
            if (vec_rows) {
                for (int64_t i = tid; i < n / 4; i += kThreads) {
                    reinterpret_cast<int4 *>(rs_span)[i] = make_int4(-1, -1, -1, -1);
                    reinterpret_cast<uint32_t *>(mask_span)[i] = 0u;
                }
            } else {
                for (int64_t i = tid; i < n; i += kThreads) {
                    rs_span[i] = -1;
                    mask_span[i] = 0;
                }
            }
        }
    }

    // 2. within-token occurrence index of each entry's expert, and rank set
    const uint32_t magic = rank_magic(L);
    int occ[KMAX];
    int maxocc = 0;
    uint64_t ranks = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        occ[k] = 0;
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2)
            occ[k] += (e[k] >= 0 && e[k2] == e[k]) ? 1 : 0;
        maxocc = max(maxocc, occ[k]);
        if (e[k] >= 0)
            ranks |= 1ull << rank_of(e[k], magic);
    }
    __syncthreads(); // LDS cleared

    // 3. counts of all earlier blocks into row 0 of s_wb: the slice loaded
    //    above, then further slices of kHistBatch int4 per thread
    for (int i0 = tid; i0 < n4; i0 += kThreads * kHistBatch) {
        if (i0 != tid) {
#pragma unroll
            for (int u = 0; u < kHistBatch; ++u) {
                const int i = i0 + u * kThreads;
                hv[u] = i < n4 ? h4[i] : make_int4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < kHistBatch; ++u) {
            const int i = i0 + u * kThreads;
            if (i < n4) {
                const int c = (i * 4) % stride;
                if (c < W)
                    atomicAdd(&s_wb[c], hv[u].x);
                if (c + 1 < W)
                    atomicAdd(&s_wb[c + 1], hv[u].y);
                if (c + 2 < W)
                    atomicAdd(&s_wb[c + 2], hv[u].z);
                if (c + 3 < W)
                    atomicAdd(&s_wb[c + 3], hv[u].w);
            }
        }
    }

    // 4. layer-0 bitmaps (first occurrences) and rank words
    uint64_t *my_words = s_bm + (size_t)g * W;
    const uint64_t bit = 1ull << lane;
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        if (e[k] >= 0 && occ[k] == 0)
            atomicOr((unsigned long long *)&my_words[e[k]], (unsigned long long)bit);
    // rank words: one ballot per rank gives this wave's word directly; with
    // many ranks each token sets its bit in its own ranks' words
    if (R <= kBallotRanks) {
        for (int r = 0; r < R; ++r) {
            const uint64_t m = __ballot((ranks >> r) & 1ull);
            if (lane == 0)
                my_words[E + r] = m;
        }
    } else {
        for (uint64_t m = ranks; m; m &= m - 1)
            atomicOr((unsigned long long *)&my_words[E + __builtin_ctzll(m)], (unsigned long long)bit);
    }
    if (maxocc > 0)
        atomicMax(&s_misc[0], maxocc);
    if (bad)
        atomicOr(&s_misc[1], 1);
    __syncthreads();

    // 5. wave bases: s_wb[g][c] = earlier blocks' entries of column c plus
    //    this block's in waves before g; the running sum past the last wave
    //    is the block's total, which a single block keeps as the totals
    for (int c = tid; c < W; c += kThreads) {
        int run = s_wb[c];
#pragma unroll
        for (int g2 = 0; g2 < kGroups; ++g2) {
            if (g2 > 0)
                s_wb[g2 * W + c] = run;
            run += __popcll(s_bm[g2 * W + c]);
        }
        s_tot[c] = run;
    }
    __syncthreads();

    // pre[k]: wave base of the expert + earlier lanes of this wave (layer 0)
    // + earlier entries of this token (occ)
    const int32_t *my_base = s_wb + (size_t)g * W;
    const uint64_t below = bits_below(lane);
    int pre[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        pre[k] = e[k] >= 0 ? my_base[e[k]] + __popcll(my_words[e[k]] & below) + occ[k] : 0;
    // rank slots of the token's ranks (read before a repeat layer reuses the words)
    int32_t rs[kBallotRanks];
    if (R <= kBallotRanks) {
#pragma unroll
        for (int r = 0; r < kBallotRanks; ++r)
            rs[r] = (r < R && ((ranks >> r) & 1ull))
                        ? my_base[E + r] + __popcll(my_words[E + r] & below)
                        : -1;
    }
    if (live && R > kBallotRanks) {
        // many ranks: the token's own ranks, over the block's fill
        uint8_t *mask_out = is_token_in_rank + t * R;
        int32_t *rslot_out = rank_slot + t * R;
        for (uint64_t m = ranks; m; m &= m - 1) {
            const int r = __builtin_ctzll(m);
            rslot_out[r] = my_base[E + r] + __popcll(my_words[E + r] & below);
            mask_out[r] = 1;
        }
    }

    // 6. repeated experts: one more bitmap layer per occurrence index
    const int layers = s_misc[0] + 1;
    for (int layer = 1; layer < layers; ++layer) {
        __syncthreads(); // every read of the previous layer is done
        for (int i = tid; i < kGroups * W; i += kThreads)
            s_bm[i] = 0ull;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (e[k] >= 0 && occ[k] == layer)
                atomicOr((unsigned long long *)&my_words[e[k]], (unsigned long long)bit);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (e[k] >= 0)
                pre[k] += prefix_in_block(&s_bm[e[k]], W, g, lane);
        if (last_block) {
            for (int i = tid; i < E; i += kThreads) {
                int c = 0;
                for (int g2 = 0; g2 < kGroups; ++g2)
                    c += __popcll(s_bm[g2 * W + i]);
                s_tot[i] += c;
            }
        }
    }

    // 7. this token's outputs (16-byte stores where the row allows them)
    if (live) {
        int32_t slot[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            slot[k] = e[k] >= 0 ? pre[k] : -1;
        int32_t *slot_out = expert_slot + t * K;
        if ((K & 3) == 0 && (reinterpret_cast<uintptr_t>(slot_out) & 15) == 0) {
#pragma unroll
            for (int q = 0; q < KMAX / 4; ++q)
                if (4 * q < K)
                    reinterpret_cast<int4 *>(slot_out)[q] =
                        make_int4(slot[4 * q], slot[4 * q + 1], slot[4 * q + 2], slot[4 * q + 3]);
        } else {
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (k < K)
                    slot_out[k] = slot[k];
        }
        if (R <= kBallotRanks) {
            uint8_t *mask_out = is_token_in_rank + t * R;
            int32_t *rslot_out = rank_slot + t * R;
#pragma unroll
            for (int r0 = 0; r0 < kBallotRanks; r0 += 4) {
                if (r0 < R) {
                    uint32_t m = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        m |= (rs[r0 + q] >= 0 ? 1u : 0u) << (8 * q);
                    if (vec_rows) {
                        *reinterpret_cast<int4 *>(rslot_out + r0) =
                            make_int4(rs[r0], rs[r0 + 1], rs[r0 + 2], rs[r0 + 3]);
                        *reinterpret_cast<uint32_t *>(mask_out + r0) = m;
                    } else {
                        for (int q = 0; q < 4 && r0 + q < R; ++q) {
                            rslot_out[r0 + q] = rs[r0 + q];
                            mask_out[r0 + q] = (uint8_t)((m >> (8 * q)) & 1u);
                        }
                    }
                }
            }
        }
    }
    if (tid == 0 && status && s_misc[1])
        atomicOr(status, EP_STATUS_BAD_EXPERT_ID);

    // 8. single token block: it holds every count; write totals and the scan
    if (last_block) {
        __syncthreads();
        write_totals_and_offsets(E, R, A, s_tot, s_misc, num_tokens_per_rank,
                                 num_tokens_per_expert, expert_offset);
    }
}

// Local ranking: the first launch of ep_layout_dispatch above
// kFusedCountedMaxTokens tokens.  Each 256-token block ranks its own entries
// exactly as the assign kernel does, but against its own tokens only:
// local_slot[t, k] is entry (t, k)'s rank among the block's entries with the
// same expert, local_rank[t, k] the token's rank among the block's tokens
// sent to the rank of expert k (-1 for a masked entry), and hist row b
// (stride ints) gets the block's entries per expert, repeats included, then
// its tokens per rank, then zeros.  No block reads another block's output:
// the pack that follows adds each token's prefix over the earlier blocks'
// rows.
template <int KMAX>
__global__ __launch_bounds__(kThreads) void layout_local_kernel(
    int32_t N, int32_t K, int32_t E, int32_t R, int32_t L, int32_t stride,
    const int64_t *__restrict__ topk_idx, int32_t *__restrict__ hist,
    int32_t *__restrict__ local_slot, int32_t *__restrict__ local_rank, uint32_t *status)
{
    extern __shared__ __align__(16) char lds_raw[];
    const int b = blockIdx.x;
    const int W = E + R;
    uint64_t *s_bm = reinterpret_cast<uint64_t *>(lds_raw);                  // [kGroups][W]
    int32_t *s_wb = reinterpret_cast<int32_t *>(s_bm + (size_t)kGroups * W); // [kGroups][W]
    int32_t *s_tot = s_wb + (size_t)kGroups * W;                             // [W]
    int32_t *s_misc = s_tot + W;                                             // [8]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int g = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t = (int64_t)b * kThreads + tid;

    int32_t e[KMAX];
    uint32_t bad = 0;
    load_token<KMAX>(topk_idx, t, N, K, E, e, bad);
    for (int i = tid; i < kGroups * W; i += kThreads)
        s_bm[i] = 0ull;
    if (tid < 8)
        s_misc[tid] = 0;

    const uint32_t magic = rank_magic(L);
    int occ[KMAX];
    int rk[KMAX];
    int maxocc = 0;
    uint64_t ranks = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        occ[k] = 0;
#pragma unroll
        for (int k2 = 0; k2 < k; ++k2)
            occ[k] += (e[k] >= 0 && e[k2] == e[k]) ? 1 : 0;
        maxocc = max(maxocc, occ[k]);
        rk[k] = e[k] >= 0 ? rank_of(e[k], magic) : 0;
        if (e[k] >= 0)
            ranks |= 1ull << rk[k];
    }
    __syncthreads(); // LDS cleared

    // layer-0 bitmaps (first occurrences) and rank words, bit = lane
    uint64_t *my_words = s_bm + (size_t)g * W;
    const uint64_t bit = 1ull << lane;
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        if (e[k] >= 0 && occ[k] == 0)
            atomicOr((unsigned long long *)&my_words[e[k]], (unsigned long long)bit);
    if (R <= kBallotRanks) {
        for (int r = 0; r < R; ++r) {
            const uint64_t m = __ballot((ranks >> r) & 1ull);
            if (lane == 0)
                my_words[E + r] = m;
        }
    } else {
        for (uint64_t m = ranks; m; m &= m - 1)
            atomicOr((unsigned long long *)&my_words[E + __builtin_ctzll(m)], (unsigned long long)bit);
    }
    if (maxocc > 0)
        atomicMax(&s_misc[0], maxocc);
    if (bad)
        atomicOr(&s_misc[1], 1);
    __syncthreads();

    // wave bases within the block; past the last wave, the block's count
    for (int c = tid; c < W; c += kThreads) {
        int run = 0;
#pragma unroll
        for (int g2 = 0; g2 < kGroups; ++g2) {
            s_wb[g2 * W + c] = run;
            run += __popcll(s_bm[g2 * W + c]);
        }
        s_tot[c] = run;
    }
    __syncthreads();

    // layer 0: each entry's slot and rank slot go out at once; a repeat
    // layer (rare) adds to the stored slot, so no per-entry array stays live
    const int32_t *my_base = s_wb + (size_t)g * W;
    const uint64_t below = bits_below(lane);
    const bool own = t < N;
    int32_t *ls = local_slot + (own ? t : 0) * K;
    int32_t *lrk = local_rank + (own ? t : 0) * K;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (own && k < K) {
            ls[k] = e[k] >= 0 ? my_base[e[k]] + __popcll(my_words[e[k]] & below) + occ[k] : -1;
            lrk[k] = e[k] >= 0 ? my_base[E + rk[k]] + __popcll(my_words[E + rk[k]] & below) : -1;
        }
    }

    // repeated experts: one more bitmap layer per occurrence index, each also
    // counted in the block's expert columns
    const int layers = s_misc[0] + 1;
    for (int layer = 1; layer < layers; ++layer) {
        __syncthreads();
        for (int i = tid; i < kGroups * W; i += kThreads)
            s_bm[i] = 0ull;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (e[k] >= 0 && occ[k] == layer)
                atomicOr((unsigned long long *)&my_words[e[k]], (unsigned long long)bit);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (own && k < K && e[k] >= 0)
                ls[k] += prefix_in_block(&s_bm[e[k]], W, g, lane);
        for (int i = tid; i < E; i += kThreads) {
            int c = 0;
            for (int g2 = 0; g2 < kGroups; ++g2)
                c += __popcll(s_bm[g2 * W + i]);
            s_tot[i] += c;
        }
    }
    __syncthreads(); // s_tot complete
    int32_t *row = hist + (size_t)b * stride;
    for (int c = tid; c < stride; c += kThreads)
        row[c] = c < W ? s_tot[c] : 0;
    if (tid == 0 && status && s_misc[1])
        atomicOr(status, EP_STATUS_BAD_EXPERT_ID);
}


} // namespace

bool plan_layout(const ep_shape &s, LayoutPlan *plan)
{
    const int N = s.num_tokens, E = s.num_experts, R = s.num_ranks;
    plan->tokens_per_block = kThreads;
    plan->num_blocks = N > 0 ? (N + kThreads - 1) / kThreads : 1;
    plan->hist_stride = (E + R + 3) / 4 * 4;
    plan->lds_bytes = assign_lds_bytes(E, R);
    plan->workspace_bytes =
        plan->num_blocks > 1 ? sizeof(int32_t) * (size_t)plan->num_blocks * plan->hist_stride : 0;
    return plan->lds_bytes <= 64 * 1024;
}

hipError_t launch_layout(const ep_shape &s, const LayoutPlan &plan, const int64_t *topk_idx,
                         int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                         uint8_t *is_token_in_rank, int32_t *expert_slot, int32_t *rank_slot,
                         int32_t *expert_offset, int32_t *workspace, uint32_t *status,
                         hipStream_t stream)
{
    const int N = s.num_tokens, K = s.num_topk, E = s.num_experts, R = s.num_ranks;
    const int L = E / R;
    const int A = expert_alignment(s);
    const int B = plan.num_blocks, stride = plan.hist_stride;
    const size_t count_lds = sizeof(int32_t) * (size_t)(E + R);
#define EP_LAYOUT_LAUNCH(KMAX)                                                                     \
    do {                                                                                           \
        if (B > 1)                                                                                 \
            hipLaunchKernelGGL(layout_count_kernel<KMAX>, dim3(B), dim3(kThreads), count_lds,      \
                               stream, N, K, E, R, L, stride, topk_idx, workspace);                \
        hipLaunchKernelGGL(layout_assign_kernel<KMAX>, dim3(B > 1 ? B + 1 : 1), dim3(kThreads),   \
                           plan.lds_bytes, stream, N, K, E, R, L, A, stride, topk_idx,             \
                           B > 1 ? workspace : nullptr,                                            \
                           num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,           \
                           expert_slot, rank_slot, expert_offset, status);                         \
    } while (0)
    if (K <= 8)
        EP_LAYOUT_LAUNCH(8);
    else if (K <= 16)
        EP_LAYOUT_LAUNCH(16);
    else
        EP_LAYOUT_LAUNCH(EP_MAX_TOPK);
#undef EP_LAYOUT_LAUNCH
    return hipGetLastError();
}

hipError_t launch_layout_count(const ep_shape &s, const LayoutPlan &plan, const int64_t *topk_idx,
                               int32_t *workspace, hipStream_t stream)
{
    const int N = s.num_tokens, K = s.num_topk, E = s.num_experts, R = s.num_ranks;
    const int B = plan.num_blocks;
    if (B <= 1)
        return hipSuccess;
    const size_t count_lds = sizeof(int32_t) * (size_t)(E + R);
    if (K <= 8)
        hipLaunchKernelGGL(layout_count_kernel<8>, dim3(B), dim3(kThreads), count_lds, stream, N, K,
                           E, R, E / R, plan.hist_stride, topk_idx, workspace);
    else if (K <= 16)
        hipLaunchKernelGGL(layout_count_kernel<16>, dim3(B), dim3(kThreads), count_lds, stream, N,
                           K, E, R, E / R, plan.hist_stride, topk_idx, workspace);
    else
        hipLaunchKernelGGL(layout_count_kernel<EP_MAX_TOPK>, dim3(B), dim3(kThreads), count_lds,
                           stream, N, K, E, R, E / R, plan.hist_stride, topk_idx, workspace);
    return hipGetLastError();
}

hipError_t launch_layout_local(const ep_shape &s, const LayoutPlan &plan, const int64_t *topk_idx,
                               const LocalWorkspace &ws, uint32_t *status, hipStream_t stream)
{
    const int N = s.num_tokens, K = s.num_topk, E = s.num_experts, R = s.num_ranks;
    if (N == 0)
        return hipSuccess;
#define EP_LOCAL_LAUNCH(KMAX)                                                                      \
    hipLaunchKernelGGL(layout_local_kernel<KMAX>, dim3(plan.num_blocks), dim3(kThreads),           \
                       plan.lds_bytes, stream, N, K, E, R, E / R, plan.hist_stride, topk_idx,      \
                       ws.hist, ws.local_slot, ws.local_rank, status)
    if (K <= 8)
        EP_LOCAL_LAUNCH(8);
    else if (K <= 16)
        EP_LOCAL_LAUNCH(16);
    else
        EP_LOCAL_LAUNCH(EP_MAX_TOPK);
#undef EP_LOCAL_LAUNCH
    return hipGetLastError();
}

} // namespace ep
