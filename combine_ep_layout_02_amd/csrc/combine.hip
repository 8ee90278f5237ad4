// combine.hip -- top-k weighted gather-reduce on gfx950.
//
// Each token's expert outputs return to the token and are summed with the
// router weights (DeepEP Ascend deep dive, "Two Transfers" and "Combine: More
// Output, Same Cost"; DeepEP V1 Legacy guide §5.2(6): BF16 in, BF16 out;
// Lesson 14, follow-up 1: reduce on chip instead of gathering every output
// back to HBM first).
//
//   acc = +0; for k ascending with a valid expert: acc = fmaf(w[t,k], y, acc);
//   out = bf16 round-to-nearest-even(acc)
//
// Work item = one wave on one (token, 1024-channel chunk); each lane owns two
// 8-channel units (16-byte loads, so every load instruction reads 1 KiB
// contiguous of one expert row), marked non-temporal since every expert row
// is read exactly once.  Entries are taken KB at a time: the KB
// (expert id, slot, weight) triples arrive together (one vector load per lane,
// broadcast with readlane), then every row load of the batch is issued before
// the first FMA.  The FMAs run in ascending k, so the fp32 sum is the same
// chain on every run (deterministic, no atomics).
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

__device__ __forceinline__ uint4 to_bf16_unit(const float (&acc)[8])
{
    return make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                      pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
}

template <int KB>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t S, int32_t nchunks,
    const uint16_t *__restrict__ y, const int64_t *__restrict__ topk_idx,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ expert_slot,
    uint16_t *__restrict__ out, uint32_t *status)
{
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t item = blockIdx.x * kWaves + wave; // host keeps N * nchunks < 2^31
    if (item >= (uint32_t)N * (uint32_t)nchunks)
        return;
    const uint32_t t = item / (uint32_t)nchunks;
    const uint32_t chunk = item - t * (uint32_t)nchunks;
    const int32_t units = H / 8;
    const int32_t u0 = (int32_t)chunk * (kChunk / 8) + lane;
    const int32_t u1 = u0 + 64;
    const bool has0 = u0 < units, has1 = u1 < units;
    // lanes past the row end load the row's last unit (in bounds, unused), so
    // the loads need no per-lane branch
    const int32_t l0 = min(u0, units - 1), l1 = min(u1, units - 1);

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
        fetch_entries<KB>(idx_t, slot_t, w_t, k0, K, E, S, lane, row, wk, flags);
        // every row load of the batch is issued before the first FMA; an
        // entry without a row reads row 0 (in bounds) and is not accumulated
        uint4 v0[KB], v1[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const uint4 *r = reinterpret_cast<const uint4 *>(y + (size_t)max(row[b], (int64_t)0) * H);
            v0[b] = load_stream(r + l0);
            v1[b] = load_stream(r + l1);
        }
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            if (row[b] >= 0) {
                fma_unit(acc0, wk[b], v0[b]);
                fma_unit(acc1, wk[b], v1[b]);
            }
        }
    }
    uint4 *dst = reinterpret_cast<uint4 *>(out + (size_t)t * H);
    if (has0)
        dst[u0] = to_bf16_unit(acc0);
    if (has1)
        dst[u1] = to_bf16_unit(acc1);
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

} // namespace

hipError_t launch_combine(const ep_shape &s, const uint16_t *expert_out, const int64_t *topk_idx,
                          const float *topk_weights, const int32_t *expert_slot,
                          uint16_t *combined_x, uint32_t *status, hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, E = s.num_experts;
    const int S = s.expert_capacity;
    if (N == 0)
        return hipSuccess;
    const int nchunks = (H + kChunk - 1) / kChunk;
    const int64_t items = (int64_t)N * nchunks;
    const dim3 grid((unsigned)((items + kWaves - 1) / kWaves));
#define EP_COMBINE_ARGS N, H, K, E, S, nchunks, expert_out, topk_idx, topk_weights, expert_slot, \
                        combined_x, status
    if (K == 1)
        hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(kThreads), 0, stream, EP_COMBINE_ARGS);
    else if (K == 2)
        hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(kThreads), 0, stream, EP_COMBINE_ARGS);
    else if (K <= 4)
        hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(kThreads), 0, stream, EP_COMBINE_ARGS);
    else
        hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(kThreads), 0, stream, EP_COMBINE_ARGS);
#undef EP_COMBINE_ARGS
    return hipGetLastError();
}

} // namespace ep
