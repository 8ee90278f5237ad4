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
// Tokens are split into blocks of T (64/128/256).  Two kernels:
//   count : per-block histogram -> workspace[b][0..E+R) (expert entries, and
//           tokens per rank, each token counted once per rank);
//   assign: each block sums the histograms of the blocks before it (one
//           coalesced pass, all loads in flight), ranks its own entries with
//           per-64-token LDS bitmaps (bit = token within its 64-token group;
//           an entry's in-block prefix is popcount of the lower bits of its
//           expert's word plus the popcounts of the earlier groups' words),
//           and the last block writes the totals and the offset scan.
// The count kernel is skipped when one block covers every token.
//
// A token may name one expert more than once.  Each repeat gets its own
// slot in k order: occurrence o of an expert within a token is ranked in
// bitmap "layer" o, and an entry's prefix sums the layers.  Routings without
// repeats take exactly one layer.
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr size_t kLdsBudget = 64 * 1024;

__device__ __forceinline__ int32_t routed_expert(int64_t id, int32_t E, uint32_t &bad)
{
    if (id == -1)
        return -1;
    if (id < 0 || id >= (int64_t)E) {
        bad = 1u;
        return -1;
    }
    return (int32_t)id;
}

__device__ __forceinline__ uint64_t bits_below(int bit) { return (1ull << bit) - 1ull; }

// Per-block histogram: hist[b][e] = valid entries of expert e among block b's
// tokens; hist[b][E + r] = tokens of block b with at least one entry on rank
// r.  Padding columns up to `stride` are written as 0.
__global__ __launch_bounds__(kThreads) void layout_count_kernel(
    int32_t N, int32_t K, int32_t E, int32_t R, int32_t L, int32_t T, int32_t stride,
    const int64_t *__restrict__ topk_idx, int32_t *__restrict__ hist)
{
    extern __shared__ int32_t s_cnt[]; // [E + R]
    const int tid = threadIdx.x;
    for (int i = tid; i < E + R; i += kThreads)
        s_cnt[i] = 0;
    __syncthreads();

    const int64_t t0 = (int64_t)blockIdx.x * T;
    const int nt = (int)min((int64_t)T, (int64_t)N - t0);
    const int64_t *ids = topk_idx + t0 * K;
    uint32_t bad = 0;
    for (int j = tid; j < nt * K; j += kThreads) {
        const int32_t e = routed_expert(ids[j], E, bad);
        if (e >= 0)
            atomicAdd(&s_cnt[e], 1);
    }
    for (int tl = tid; tl < nt; tl += kThreads) {
        uint64_t ranks = 0;
        for (int k = 0; k < K; ++k) {
            const int32_t e = routed_expert(ids[tl * K + k], E, bad);
            if (e >= 0)
                ranks |= 1ull << (e / L);
        }
        while (ranks) {
            const int r = __builtin_ctzll(ranks);
            atomicAdd(&s_cnt[E + r], 1);
            ranks &= ranks - 1ull;
        }
    }
    __syncthreads();
    int32_t *row = hist + (size_t)blockIdx.x * stride;
    for (int i = tid; i < stride; i += kThreads)
        row[i] = i < E + R ? s_cnt[i] : 0;
}

struct AssignLds {
    uint64_t *bm;   // [G][E]  expert bitmaps of one layer
    uint64_t *rbm;  // [G][R]  rank bitmaps
    int32_t *ids;   // [T*K]   validated expert ids (-1 = masked)
    int32_t *acc;   // [T*K]   in-block prefix of each entry
    int32_t *base;  // [E+R]   counts of all earlier blocks
    int32_t *blk;   // [E+R]   this block's counts, then the totals
    int32_t *misc;  // [8]     0: layers, 1: bad id, 4..7: wave sums
    uint8_t *occ;   // [T*K]   occurrence index of the entry's expert in its token
};

__device__ AssignLds carve(char *p, int G, int T, int K, int E, int R)
{
    AssignLds s;
    s.bm = (uint64_t *)p;
    p += sizeof(uint64_t) * (size_t)G * E;
    s.rbm = (uint64_t *)p;
    p += sizeof(uint64_t) * (size_t)G * R;
    s.ids = (int32_t *)p;
    p += sizeof(int32_t) * (size_t)T * K;
    s.acc = (int32_t *)p;
    p += sizeof(int32_t) * (size_t)T * K;
    s.base = (int32_t *)p;
    p += sizeof(int32_t) * (size_t)(E + R);
    s.blk = (int32_t *)p;
    p += sizeof(int32_t) * (size_t)(E + R);
    s.misc = (int32_t *)p;
    p += sizeof(int32_t) * 8;
    s.occ = (uint8_t *)p;
    return s;
}

__host__ __device__ inline size_t assign_lds_bytes(int T, int K, int E, int R)
{
    const int G = T / 64;
    return sizeof(uint64_t) * (size_t)G * (E + R) + sizeof(int32_t) * (size_t)T * K * 2 +
           sizeof(int32_t) * (size_t)(E + R) * 2 + sizeof(int32_t) * 8 + (size_t)T * K;
}

__global__ __launch_bounds__(kThreads) void layout_assign_kernel(
    int32_t N, int32_t K, int32_t E, int32_t R, int32_t L, int32_t T, int32_t stride,
    const int64_t *__restrict__ topk_idx, const int32_t *__restrict__ hist,
    int32_t *__restrict__ num_tokens_per_rank, int32_t *__restrict__ num_tokens_per_expert,
    uint8_t *__restrict__ is_token_in_rank, int32_t *__restrict__ expert_slot,
    int32_t *__restrict__ rank_slot, int32_t *__restrict__ expert_offset, uint32_t *status)
{
    extern __shared__ __align__(16) char lds_raw[];
    const int G = T / 64;
    AssignLds s = carve(lds_raw, G, T, K, E, R);
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int64_t t0 = (int64_t)b * T;
    const int nt = (int)max((int64_t)0, min((int64_t)T, (int64_t)N - t0));
    const int nent = nt * K;
    const int64_t *ids = topk_idx + t0 * K;

    // 1. zero the block's counters, stage validated ids
    for (int i = tid; i < E + R; i += kThreads) {
        s.base[i] = 0;
        s.blk[i] = 0;
    }
    if (tid < 8)
        s.misc[tid] = tid == 0 ? 1 : 0;
    uint32_t bad = 0;
    for (int j = tid; j < nent; j += kThreads)
        s.ids[j] = routed_expert(ids[j], E, bad);
    __syncthreads();
    if (bad)
        atomicOr(&s.misc[1], 1);

    // 2. counts of all earlier blocks: the first b rows of the histogram are
    //    one contiguous span; load it as int4 with eight loads in flight.
    if (b > 0) {
        const int n4 = b * (stride / 4);
        const int4 *h4 = reinterpret_cast<const int4 *>(hist);
        for (int i0 = tid; i0 < n4; i0 += kThreads * 8) {
            int4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kThreads;
                v[u] = i < n4 ? h4[i] : make_int4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kThreads;
                if (i < n4) {
                    const int c = (i * 4) % stride;
                    if (c < E + R)
                        atomicAdd(&s.base[c], v[u].x);
                    if (c + 1 < E + R)
                        atomicAdd(&s.base[c + 1], v[u].y);
                    if (c + 2 < E + R)
                        atomicAdd(&s.base[c + 2], v[u].z);
                    if (c + 3 < E + R)
                        atomicAdd(&s.base[c + 3], v[u].w);
                }
            }
        }
    }

    // 3. occurrence of each entry's expert among the token's earlier entries
    for (int j = tid; j < nent; j += kThreads) {
        const int32_t e = s.ids[j];
        int occ = 0;
        if (e >= 0) {
            const int tl = j / K;
            for (int k2 = tl * K; k2 < j; ++k2)
                occ += s.ids[k2] == e;
        }
        s.occ[j] = (uint8_t)occ;
        s.acc[j] = occ;
        if (occ > 0)
            atomicMax(&s.misc[0], occ + 1);
    }
    __syncthreads();
    const int layers = s.misc[0];

    // 4. rank entries layer by layer (one layer without repeated experts)
    for (int layer = 0; layer < layers; ++layer) {
        for (int i = tid; i < G * E; i += kThreads)
            s.bm[i] = 0ull;
        if (layer == 0)
            for (int i = tid; i < G * R; i += kThreads)
                s.rbm[i] = 0ull;
        __syncthreads();
        for (int j = tid; j < nent; j += kThreads) {
            const int32_t e = s.ids[j];
            if (e >= 0 && s.occ[j] == layer) {
                const int tl = j / K;
                const uint64_t bit = 1ull << (tl & 63);
                atomicOr((unsigned long long *)&s.bm[(tl >> 6) * E + e], (unsigned long long)bit);
                if (layer == 0)
                    atomicOr((unsigned long long *)&s.rbm[(tl >> 6) * R + e / L],
                             (unsigned long long)bit);
            }
        }
        __syncthreads();
        for (int j = tid; j < nent; j += kThreads) {
            const int32_t e = s.ids[j];
            if (e >= 0) {
                const int tl = j / K;
                const int g = tl >> 6;
                int cnt = __popcll(s.bm[g * E + e] & bits_below(tl & 63));
                for (int g2 = 0; g2 < g; ++g2)
                    cnt += __popcll(s.bm[g2 * E + e]);
                s.acc[j] += cnt;
            }
        }
        for (int i = tid; i < E; i += kThreads) {
            int tot = 0;
            for (int g2 = 0; g2 < G; ++g2)
                tot += __popcll(s.bm[g2 * E + i]);
            s.blk[i] += tot;
        }
        __syncthreads();
    }

    // 5. expert slots
    int32_t *slot_out = expert_slot + t0 * K;
    for (int j = tid; j < nent; j += kThreads) {
        const int32_t e = s.ids[j];
        slot_out[j] = e >= 0 ? s.base[e] + s.acc[j] : -1;
    }

    // 6. rank mask and rank slots, one (token, rank) pair per thread
    uint8_t *mask_out = is_token_in_rank + t0 * R;
    int32_t *rslot_out = rank_slot + t0 * R;
    for (int q = tid; q < nt * R; q += kThreads) {
        const int tl = q / R;
        const int r = q - tl * R;
        const int g = tl >> 6;
        const uint64_t word = s.rbm[g * R + r];
        const bool in = (word >> (tl & 63)) & 1ull;
        int cnt = __popcll(word & bits_below(tl & 63));
        for (int g2 = 0; g2 < g; ++g2)
            cnt += __popcll(s.rbm[g2 * R + r]);
        mask_out[q] = in ? 1 : 0;
        rslot_out[q] = in ? s.base[E + r] + cnt : -1;
    }
    for (int i = tid; i < R; i += kThreads) {
        int tot = 0;
        for (int g2 = 0; g2 < G; ++g2)
            tot += __popcll(s.rbm[g2 * R + i]);
        s.blk[E + i] = tot;
    }
    if (tid == 0 && status && s.misc[1])
        atomicOr(status, EP_STATUS_BAD_EXPERT_ID);

    // 7. the last block holds every count: write totals and the offset scan
    if (b == (int)gridDim.x - 1) {
        __syncthreads();
        for (int i = tid; i < E + R; i += kThreads) {
            const int tot = s.base[i] + s.blk[i];
            if (i < E)
                num_tokens_per_expert[i] = tot;
            else
                num_tokens_per_rank[i - E] = tot;
            s.blk[i] = tot;
        }
        __syncthreads();
        if (expert_offset) {
            const int per = (E + kThreads - 1) / kThreads;
            const int start = tid * per;
            int local = 0;
            for (int i = 0; i < per; ++i)
                if (start + i < E)
                    local += s.blk[start + i];
            const int lane = tid & 63;
            const int wave = tid >> 6;
            int incl = local;
            for (int off = 1; off < 64; off <<= 1) {
                const int up = __shfl_up(incl, off, 64);
                if (lane >= off)
                    incl += up;
            }
            if (lane == 63)
                s.misc[4 + wave] = incl;
            __syncthreads();
            int woff = 0;
            for (int w2 = 0; w2 < wave; ++w2)
                woff += s.misc[4 + w2];
            int run = woff + incl - local;
            for (int i = 0; i < per; ++i) {
                if (start + i < E) {
                    expert_offset[start + i] = run;
                    run += s.blk[start + i];
                }
            }
            if (tid == kThreads - 1)
                expert_offset[E] = woff + incl;
        }
    }
}

} // namespace

bool plan_layout(const ep_shape &s, LayoutPlan *plan)
{
    const int N = s.num_tokens, K = s.num_topk, E = s.num_experts, R = s.num_ranks;
    for (int T = 256; T >= 64; T /= 2) {
        const size_t lds = assign_lds_bytes(T, K, E, R);
        if (lds <= kLdsBudget) {
            plan->tokens_per_block = T;
            plan->num_blocks = N > 0 ? (N + T - 1) / T : 1;
            plan->hist_stride = (E + R + 3) / 4 * 4;
            plan->lds_bytes = lds;
            plan->workspace_bytes =
                plan->num_blocks > 1 ? sizeof(int32_t) * (size_t)plan->num_blocks * plan->hist_stride : 0;
            return true;
        }
    }
    return false;
}

hipError_t launch_layout(const ep_shape &s, const LayoutPlan &plan, const int64_t *topk_idx,
                         int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                         uint8_t *is_token_in_rank, int32_t *expert_slot, int32_t *rank_slot,
                         int32_t *expert_offset, int32_t *workspace, uint32_t *status,
                         hipStream_t stream)
{
    const int N = s.num_tokens, K = s.num_topk, E = s.num_experts, R = s.num_ranks;
    const int L = E / R;
    const int T = plan.tokens_per_block, B = plan.num_blocks, stride = plan.hist_stride;
    if (B > 1) {
        hipLaunchKernelGGL(layout_count_kernel, dim3(B), dim3(kThreads),
                           sizeof(int32_t) * (size_t)(E + R), stream, N, K, E, R, L, T, stride,
                           topk_idx, workspace);
    }
    hipLaunchKernelGGL(layout_assign_kernel, dim3(B), dim3(kThreads), plan.lds_bytes, stream, N, K,
                       E, R, L, T, stride, topk_idx, workspace, num_tokens_per_rank,
                       num_tokens_per_expert, is_token_in_rank, expert_slot, rank_slot,
                       expert_offset, status);
    return hipGetLastError();
}

} // namespace ep
