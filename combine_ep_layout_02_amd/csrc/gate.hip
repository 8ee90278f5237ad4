// gate.hip -- group-limited top-k gating on gfx950, the step in front of the
// layout (DeepEP V1 Legacy guide §1 and §2.1: group-limited gating, top-4
// groups then top-8 experts; Lesson 14 §3 Q3: at most 4 nodes per token; its
// exercise: normalised softmax gating weights).
//
// Per token: a group's score is its best expert's score; the TG best groups
// are kept (ties: lower group index); the K best experts of the kept groups
// are picked, best first (ties: lower expert index); the weights are the
// softmax of the picked scores.
//
// Work item = one wave per token.  Lane l holds experts i * 64 + l (so each
// load instruction reads 64 consecutive scores).  Scores become
// order-preserving 32-bit keys (after adding +0, so -0 and +0 compare equal,
// as floats do); the group maxima are LDS atomicMax on those keys.  Every pick
// -- a group, then an expert -- is a wave-wide maximum of the 64-bit key
// (score key << 32 | ~index), so the larger score wins and equal scores go to
// the lower index, without a branch per compare.  All decisions are exact
// comparisons of the inputs, so they match the CPU definition bit for bit;
// only the weights involve rounding (expf and one division per pick).
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Order-preserving key of a finite float: larger float -> larger key; every
// finite float maps above 0, which marks "no candidate".
__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t b = __float_as_uint(f + 0.0f); // -0 -> +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

template <int V>
__global__ __launch_bounds__(kThreads) void gate_kernel(int32_t N, int32_t E, int32_t G,
                                                        int32_t TG, int32_t K,
                                                        const float *__restrict__ scores,
                                                        int64_t *__restrict__ topk_idx,
                                                        float *__restrict__ topk_weights)
{
    __shared__ uint32_t s_gkey[kWaves][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kWaves + wave;
    const bool live = t < N; // waves past the last token still take part in the barriers
    const int32_t L = E / G;

    uint32_t key[V];
    bool valid[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int32_t e = i * 64 + lane;
        valid[i] = live && e < E;
        key[i] = valid[i] ? order_key(scores[t * E + e]) : 0u;
    }
    s_gkey[wave][lane] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < V; ++i)
        if (valid[i])
            atomicMax(&s_gkey[wave][(i * 64 + lane) / L], key[i]);
    __syncthreads();
    const uint32_t gk = lane < G ? s_gkey[wave][lane] : 0u;

    // the TG best groups
    uint64_t kept = 0;
    for (int n = 0; n < TG; ++n) {
        const bool cand = lane < G && !((kept >> lane) & 1u);
        const uint64_t c = cand ? ((uint64_t)gk << 32) | (uint32_t)~(uint32_t)lane : 0u;
        const uint64_t best = wave_max_u64(c);
        kept |= 1ull << (~(uint32_t)best & 63u);
    }

    // the K best experts of the kept groups; lane k keeps pick k
    bool taken[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        taken[i] = !valid[i] || !((kept >> ((i * 64 + lane) / L)) & 1u);
    int64_t my_idx = -1;
    float my_score = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint64_t c = 0;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const uint64_t ci = ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(i * 64 + lane);
            if (!taken[i] && ci > c)
                c = ci;
        }
        const uint64_t best = wave_max_u64(c);
        const uint32_t e = ~(uint32_t)best; // the host ensures K candidates exist
#pragma unroll
        for (int i = 0; i < V; ++i)
            if ((uint32_t)(i * 64 + lane) == e)
                taken[i] = true;
        if (lane == k) {
            my_idx = (int64_t)e;
            my_score = key_value((uint32_t)(best >> 32));
        }
    }

    // softmax of the picks, summed in pick order
    const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_score), 0));
    const float z = lane < K ? expf(my_score - top) : 0.0f;
    float sum = 0.0f;
    for (int k = 0; k < K; ++k)
        sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), k));
    if (live && lane < K) {
        topk_idx[t * K + lane] = my_idx;
        if (topk_weights)
            topk_weights[t * K + lane] = z / sum;
    }
}

} // namespace

hipError_t launch_gate(const ep_shape &s, int32_t num_groups, int32_t topk_groups,
                       const float *scores, int64_t *topk_idx, float *topk_weights,
                       hipStream_t stream)
{
    const int N = s.num_tokens, E = s.num_experts, K = s.num_topk;
    if (N == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((N + kWaves - 1) / kWaves));
#define EP_GATE(V)                                                                                 \
    hipLaunchKernelGGL(gate_kernel<V>, grid, dim3(kThreads), 0, stream, N, E, num_groups,          \
                       topk_groups, K, scores, topk_idx, topk_weights)
    if (E <= 64)
        EP_GATE(1);
    else if (E <= 128)
        EP_GATE(2);
    else if (E <= 256)
        EP_GATE(4);
    else if (E <= 512)
        EP_GATE(8);
    else
        EP_GATE(16);
#undef EP_GATE
    return hipGetLastError();
}

} // namespace ep
