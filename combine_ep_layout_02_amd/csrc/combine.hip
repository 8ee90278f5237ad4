// combine.hip -- combine kernels on gfx950.
//
// Top-k weighted combine (per-expert and expand layouts): each token's expert
// outputs return to the token and are summed with the router weights (DeepEP
// Ascend deep dive, "Two Transfers" and "Combine: More Output, Same Cost";
// DeepEP V1 Legacy guide §5.2(6): BF16 in, BF16 out; Lesson 14, follow-up 1:
// reduce on chip instead of gathering every output back to HBM first).
//
//   acc = +0; for k ascending with a valid expert: acc = fmaf(w[t,k], y, acc);
//   acc = acc + bias[t]   (optional: the shared expert's output, folded into
//                          the epilogue -- Ascend deep dive, "Combine: More
//                          Output, Same Cost")
//   out = bf16 round-to-nearest-even(acc)
//
// Normal-mode combine (V1 guide §5.1): one row per (token, rank) comes back
// and the token's rows are summed in ascending rank order (the expert layer
// applied the weights that travelled with the row); a tensor of per-row
// top-k weights may be reduced the same way.
//
//   acc = +0; for r ascending with a row at rank r: acc = acc + y[r][row];
//   acc = acc + bias[t] (optional); out = bf16 round-to-nearest-even(acc)
//
// Work item = one wave on one (token, 1024-channel chunk); each lane owns two
// 8-channel units (16-byte loads, so every load instruction reads 1 KiB
// contiguous of one row), marked non-temporal since every row is read
// exactly once.  Rows are taken KB at a time: the KB row numbers arrive
// together (one vector load per lane, broadcast with readlane), then every
// row load of the batch is issued before the first add.  The adds run in a
// fixed order, so the fp32 sum is the same chain on every run (deterministic,
// no atomics).
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 1024; // channels per work item

__device__ __forceinline__ void fma_unit(float (&acc)[8], float w, const uint4 &v)
{
    acc[0] = fmaf(w, bf16_lo(v.x), acc[0]);
    acc[1] = fmaf(w, bf16_hi(v.x), acc[1]);
    acc[2] = fmaf(w, bf16_lo(v.y), acc[2]);
    acc[3] = fmaf(w, bf16_hi(v.y), acc[3]);
    acc[4] = fmaf(w, bf16_lo(v.z), acc[4]);
    acc[5] = fmaf(w, bf16_hi(v.z), acc[5]);
    acc[6] = fmaf(w, bf16_lo(v.w), acc[6]);
    acc[7] = fmaf(w, bf16_hi(v.w), acc[7]);
}

__device__ __forceinline__ void add_unit(float (&acc)[8], const uint4 &v)
{
    acc[0] = acc[0] + bf16_lo(v.x);
    acc[1] = acc[1] + bf16_hi(v.x);
    acc[2] = acc[2] + bf16_lo(v.y);
    acc[3] = acc[3] + bf16_hi(v.y);
    acc[4] = acc[4] + bf16_lo(v.z);
    acc[5] = acc[5] + bf16_hi(v.z);
    acc[6] = acc[6] + bf16_lo(v.w);
    acc[7] = acc[7] + bf16_hi(v.w);
}

__device__ __forceinline__ uint4 to_bf16_unit(const float (&acc)[8])
{
    return make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                      pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
}

// The two units of one lane in a (token, chunk) item.  Lanes past the row
// end load the row's last unit (in bounds, unused), so the loads need no
// per-lane branch.
struct Units {
    int32_t u0, u1, l0, l1;
    bool has0, has1;
};

__device__ __forceinline__ Units units_of(int32_t H, uint32_t chunk, int lane)
{
    Units u;
    const int32_t units = H / 8;
    u.u0 = (int32_t)chunk * (kChunk / 8) + lane;
    u.u1 = u.u0 + 64;
    u.has0 = u.u0 < units;
    u.has1 = u.u1 < units;
    u.l0 = min(u.u0, units - 1);
    u.l1 = min(u.u1, units - 1);
    return u;
}

// The bias row's two units of this lane (read once: non-temporal), issued
// before the row loads so its latency overlaps theirs.
__device__ __forceinline__ void load_bias(const uint16_t *__restrict__ bias_row, const Units &u,
                                          uint4 &b0, uint4 &b1)
{
    const uint4 *r = reinterpret_cast<const uint4 *>(bias_row);
    b0 = load_stream(r + u.l0);
    b1 = load_stream(r + u.l1);
}

__device__ __forceinline__ void store_out(uint16_t *__restrict__ out_row, const Units &u,
                                          const float (&acc0)[8], const float (&acc1)[8])
{
    uint4 *dst = reinterpret_cast<uint4 *>(out_row);
    if (u.has0)
        dst[u.u0] = to_bf16_unit(acc0);
    if (u.has1)
        dst[u.u1] = to_bf16_unit(acc1);
}

template <int KB, bool BIAS, class Rows>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t nchunks, Rows rows,
    const uint16_t *__restrict__ y, const int64_t *__restrict__ topk_idx,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ expert_slot,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ out, uint32_t *status)
{
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t item = blockIdx.x * kWaves + wave; // host keeps N * nchunks < 2^31
    if (item >= (uint32_t)N * (uint32_t)nchunks)
        return;
    const uint32_t t = item / (uint32_t)nchunks;
    const uint32_t chunk = item - t * (uint32_t)nchunks;
    const Units u = units_of(H, chunk, lane);
    uint4 b0, b1;
    if (BIAS)
        load_bias(bias + (size_t)t * H, u, b0, b1);

    float acc0[8], acc1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        acc0[i] = 0.0f;
        acc1[i] = 0.0f;
    }
    uint32_t flags = 0;
    const int64_t *idx_t = topk_idx + (size_t)t * K;
    const int32_t *slot_t = expert_slot + (size_t)t * K;
    const float *w_t = topk_weights + (size_t)t * K;
    for (int k0 = 0; k0 < K; k0 += KB) {
        int64_t row[KB];
        float wk[KB];
        fetch_entries<KB>(idx_t, slot_t, w_t, k0, K, E, rows, lane, row, wk, flags);
        // every row load of the batch is issued before the first FMA; an
        // entry without a row reads row 0 (in bounds) and is not accumulated
        uint4 v0[KB], v1[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const uint4 *r = reinterpret_cast<const uint4 *>(y + (size_t)max(row[b], (int64_t)0) * H);
            v0[b] = load_stream(r + u.l0);
            v1[b] = load_stream(r + u.l1);
        }
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            if (row[b] >= 0) {
                fma_unit(acc0, wk[b], v0[b]);
                fma_unit(acc1, wk[b], v1[b]);
            }
        }
    }
    if (BIAS) {
        add_unit(acc0, b0);
        add_unit(acc1, b1);
    }
    store_out(out + (size_t)t * H, u, acc0, acc1);
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

// Normal-mode combine: rows y[r * M + rank_slot[t, r]] for the ranks r the
// token was sent to, KB ranks per batch in ascending order.  The chunk-0 wave
// also reduces recv_topk_weights (lane k < K) over the same rows.
template <int KB, bool BIAS>
__global__ __launch_bounds__(kThreads) void combine_normal_kernel(
    int32_t N, int32_t H, int32_t K, int32_t R, int32_t M, int32_t nchunks,
    const uint16_t *__restrict__ y, const int32_t *__restrict__ rank_slot,
    const float *__restrict__ recv_topk_weights, const uint16_t *__restrict__ bias,
    uint16_t *__restrict__ out, float *__restrict__ combined_topk_weights, uint32_t *status)
{
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t item = blockIdx.x * kWaves + wave; // host keeps N * nchunks < 2^31
    if (item >= (uint32_t)N * (uint32_t)nchunks)
        return;
    const uint32_t t = item / (uint32_t)nchunks;
    const uint32_t chunk = item - t * (uint32_t)nchunks;
    const Units u = units_of(H, chunk, lane);
    const bool with_w = chunk == 0 && recv_topk_weights && combined_topk_weights;
    uint4 b0, b1;
    if (BIAS)
        load_bias(bias + (size_t)t * H, u, b0, b1);

    uint32_t flags = 0;
    int32_t j;
    uint64_t dest = rank_destinations(rank_slot + (size_t)t * R, R, M, lane, j, flags);
    float acc0[8], acc1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        acc0[i] = 0.0f;
        acc1[i] = 0.0f;
    }
    float wacc = 0.0f;
    while (dest) {
        int64_t row[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            row[b] = -1;
            if (dest) {
                const int r = __builtin_ctzll(dest);
                dest &= dest - 1;
                row[b] = (int64_t)r * M + __builtin_amdgcn_readlane(j, r);
            }
        }
        uint4 v0[KB], v1[KB];
        float wv[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const int64_t rb = max(row[b], (int64_t)0);
            const uint4 *r = reinterpret_cast<const uint4 *>(y + (size_t)rb * H);
            v0[b] = load_stream(r + u.l0);
            v1[b] = load_stream(r + u.l1);
            wv[b] = (with_w && row[b] >= 0 && lane < K) ? recv_topk_weights[(size_t)rb * K + lane]
                                                       : 0.0f;
        }
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            if (row[b] >= 0) {
                add_unit(acc0, v0[b]);
                add_unit(acc1, v1[b]);
                wacc = wacc + wv[b];
            }
        }
    }
    if (BIAS) {
        add_unit(acc0, b0);
        add_unit(acc1, b1);
    }
    store_out(out + (size_t)t * H, u, acc0, acc1);
    if (with_w && lane < K)
        combined_topk_weights[(size_t)t * K + lane] = wacc;
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

template <class Rows>
hipError_t launch_topk_combine(const ep_shape &s, const Rows &rows, const uint16_t *expert_out,
                               const int64_t *topk_idx, const float *topk_weights,
                               const int32_t *expert_slot, const uint16_t *bias,
                               uint16_t *combined_x, uint32_t *status, hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, E = s.num_experts;
    if (N == 0)
        return hipSuccess;
    const int nchunks = (H + kChunk - 1) / kChunk;
    const int64_t items = (int64_t)N * nchunks;
    const dim3 grid((unsigned)((items + kWaves - 1) / kWaves));
#define EP_COMBINE(KB, BIAS)                                                                       \
    hipLaunchKernelGGL((combine_kernel<KB, BIAS, Rows>), grid, dim3(kThreads), 0, stream, N, H, K, \
                       E, nchunks, rows, expert_out, topk_idx, topk_weights, expert_slot, bias,    \
                       combined_x, status)
#define EP_COMBINE_KB(BIAS)                                                                        \
    do {                                                                                           \
        if (K == 1)                                                                                \
            EP_COMBINE(1, BIAS);                                                                   \
        else if (K == 2)                                                                           \
            EP_COMBINE(2, BIAS);                                                                   \
        else if (K <= 4)                                                                           \
            EP_COMBINE(4, BIAS);                                                                   \
        else                                                                                       \
            EP_COMBINE(8, BIAS);                                                                   \
    } while (0)
    if (bias)
        EP_COMBINE_KB(true);
    else
        EP_COMBINE_KB(false);
#undef EP_COMBINE_KB
#undef EP_COMBINE
    return hipGetLastError();
}

} // namespace

hipError_t launch_combine(const ep_shape &s, const uint16_t *expert_out, const int64_t *topk_idx,
                          const float *topk_weights, const int32_t *expert_slot,
                          const uint16_t *bias, uint16_t *combined_x, uint32_t *status,
                          hipStream_t stream)
{
    return launch_topk_combine(s, DenseRows{s.expert_capacity}, expert_out, topk_idx, topk_weights,
                               expert_slot, bias, combined_x, status, stream);
}

hipError_t launch_combine_expand(const ep_shape &s, const uint16_t *expert_out,
                                 const int64_t *topk_idx, const float *topk_weights,
                                 const int32_t *expert_slot, const int32_t *expert_offset,
                                 const uint16_t *bias, uint16_t *combined_x, uint32_t *status,
                                 hipStream_t stream)
{
    return launch_topk_combine(s, ExpandRows{expert_offset, expand_rows(s)}, expert_out, topk_idx,
                               topk_weights, expert_slot, bias, combined_x, status, stream);
}

hipError_t launch_combine_normal(const ep_shape &s, const uint16_t *x, const int32_t *rank_slot,
                                 const float *recv_topk_weights, const uint16_t *bias,
                                 uint16_t *combined_x, float *combined_topk_weights,
                                 uint32_t *status, hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, R = s.num_ranks;
    const int M = s.num_max_dispatch_tokens_per_rank;
    if (N == 0)
        return hipSuccess;
    const int nchunks = (H + kChunk - 1) / kChunk;
    const int64_t items = (int64_t)N * nchunks;
    const dim3 grid((unsigned)((items + kWaves - 1) / kWaves));
    if (bias)
        hipLaunchKernelGGL((combine_normal_kernel<8, true>), grid, dim3(kThreads), 0, stream, N, H,
                           K, R, M, nchunks, x, rank_slot, recv_topk_weights, bias, combined_x,
                           combined_topk_weights, status);
    else
        hipLaunchKernelGGL((combine_normal_kernel<8, false>), grid, dim3(kThreads), 0, stream, N,
                           H, K, R, M, nchunks, x, rank_slot, recv_topk_weights, bias, combined_x,
                           combined_topk_weights, status);
    return hipGetLastError();
}

} // namespace ep
