// gate.hip -- group-limited top-k gating on gfx950, the step in front of the
// layout (DeepEP V1 Legacy guide §1 and §2.1: group-limited gating, top-4
// groups then top-8 experts; Lesson 14 §3 Q3: at most 4 nodes per token; its
// exercise: normalised softmax gating weights).
//
// Per token, under one of two rules for the group score and the weights:
//   EP_GATE_MAX_SOFTMAX: a group's score is its best expert's score; the
//     weights are the softmax of the picked scores;
//   EP_GATE_SUM_SIGMOID: a group's score is the binary32 sum of its experts'
//     scores in ascending expert index from +0 (one lane per group adds them
//     one after another, so the rounding is the definition's); the weights
//     are the sigmoids of the picked scores normalised to sum 1.
// Then the TG best groups are kept (ties: lower group index) and the K best
// experts of the kept groups are picked, best first (ties: lower expert
// index).
//
// Work item = one wave per token.  Lane l holds experts i * 64 + l (so each
// load instruction reads 64 consecutive scores, and the index order of the
// experts is the order of (i, lane)).  Scores become order-preserving 32-bit
// keys (after adding +0, so -0 and +0 compare equal, as floats do).  The group
// maxima are LDS atomicMax on the keys; group sums are taken by lane g from
// the wave's scores staged in LDS.  Selection moves no data through memory:
//   groups:  group g's rank is the number of groups whose (key, lower index)
//            beats it (G readlanes); the TG lowest ranks are kept;
//   experts: K rounds, each taking the largest remaining candidate key (a
//            register-only wave maximum: DPP inside rows of 16 lanes, then the
//            four row maxima by readlane) at the lowest expert index holding
//            it (one ballot per key slot), which lane k keeps for pick k.
// All decisions are exact comparisons of the inputs (or of sums rounded in
// the defined order), so they match the CPU definition bit for bit; only the
// weights involve further rounding (expf and one division per pick).
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

// Maximum of v over the wave: DPP moves inside each row of 16 lanes (swap
// neighbours, swap pairs, rotate by 4, rotate by 8 -- after which every lane
// of a row holds the row's maximum), then the four row maxima by readlane.
// Register-only: no LDS traffic.
__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
    constexpr int kQuadSwap1 = 0xB1; // quad_perm [1, 0, 3, 2]
    constexpr int kQuadSwap2 = 0x4E; // quad_perm [2, 3, 0, 1]
    constexpr int kRowRor4 = 0x124;  // row_ror:4
    constexpr int kRowRor8 = 0x128;  // row_ror:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kQuadSwap1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kQuadSwap2, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowRor4, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kRowRor8, 0xF, 0xF, false));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

template <int V, int RULE>
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
    const bool live = t < N; // waves past the last token take part in the barriers only
    const int32_t L = E / G;

    uint32_t key[V];
    int32_t grp[V];
    bool valid[V];
    float sc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int32_t e = i * 64 + lane;
        valid[i] = live && e < E;
        sc[i] = valid[i] ? scores[t * E + e] : 0.0f;
        key[i] = valid[i] ? order_key(sc[i]) : 0u;
        grp[i] = e / L;
    }
    uint32_t gk;
    if constexpr (RULE == EP_GATE_MAX_SOFTMAX) {
        s_gkey[wave][lane] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < V; ++i)
            if (valid[i])
                atomicMax(&s_gkey[wave][grp[i]], key[i]);
        __syncthreads();
        if (!live)
            return;
        gk = lane < G ? s_gkey[wave][lane] : 0u;
    } else {
        // the wave's scores in LDS, then lane g adds group g's scores in
        // ascending expert index from +0 (each sum a finite float, so its
        // key is above 0)
        __shared__ float s_sc[kWaves][V * 64];
#pragma unroll
        for (int i = 0; i < V; ++i)
            s_sc[wave][i * 64 + lane] = sc[i];
        __syncthreads();
        if (!live)
            return;
        float acc = 0.0f;
        if (lane < G)
            for (int32_t i = 0; i < L; ++i)
                acc = acc + s_sc[wave][lane * L + i];
        gk = lane < G ? order_key(acc) : 0u;
    }

    // groups: rank of group `lane` among the G group keys (ties: lower index)
    int grank = 0;
    for (int g = 0; g < G; ++g) {
        const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)gk, g);
        grank += (o > gk || (o == gk && g < lane)) ? 1 : 0;
    }
    const uint64_t kept = __ballot(lane < G && grank < TG);

    // experts: candidate keys, 0 where not a candidate
    uint32_t c[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        c[i] = (valid[i] && ((kept >> grp[i]) & 1u)) ? key[i] : 0u;
    // K rounds: the largest remaining candidate key, the lowest expert index
    // holding it (index order is (i, lane)), taken out; lane k keeps pick k.
    // Equal keys therefore go out in index order, as the definition wants.
    int64_t my_idx = -1;
    float my_score = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint32_t m = c[0];
#pragma unroll
        for (int i = 1; i < V; ++i)
            m = max(m, c[i]);
        const uint32_t top = wave_max(m);
        int pick_i = 0, pick_l = 0;
#pragma unroll
        for (int i = V - 1; i >= 0; --i) {
            const uint64_t b = __ballot(c[i] == top);
            if (b) {
                pick_i = i;
                pick_l = __builtin_ctzll(b);
            }
        }
#pragma unroll
        for (int i = 0; i < V; ++i)
            if (i == pick_i && lane == pick_l)
                c[i] = 0u;
        if (lane == k) {
            my_idx = (int64_t)(pick_i * 64 + pick_l);
            my_score = key_value(top);
        }
    }

    // the weights: softmax of the picks, or their sigmoids, normalised by the
    // sum taken in pick order
    float z = 0.0f;
    if constexpr (RULE == EP_GATE_MAX_SOFTMAX) {
        const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_score), 0));
        z = lane < K ? expf(my_score - top) : 0.0f;
    } else {
        z = lane < K ? 1.0f / (1.0f + expf(-my_score)) : 0.0f;
    }
    float sum = 0.0f;
    for (int k = 0; k < K; ++k)
        sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), k));
    if (lane < K) {
        topk_idx[t * K + lane] = my_idx;
        if (topk_weights)
            topk_weights[t * K + lane] = z / sum;
    }
}

} // namespace

hipError_t launch_gate(const ep_shape &s, int32_t num_groups, int32_t topk_groups, int32_t rule,
                       const float *scores, int64_t *topk_idx, float *topk_weights,
                       hipStream_t stream)
{
    const int N = s.num_tokens, E = s.num_experts, K = s.num_topk;
    if (N == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((N + kWaves - 1) / kWaves));
#define EP_GATE(V)                                                                                 \
    do {                                                                                           \
        if (rule == EP_GATE_SUM_SIGMOID)                                                           \
            hipLaunchKernelGGL((gate_kernel<V, EP_GATE_SUM_SIGMOID>), grid, dim3(kThreads), 0,     \
                               stream, N, E, num_groups, topk_groups, K, scores, topk_idx,         \
                               topk_weights);                                                      \
        else                                                                                       \
            hipLaunchKernelGGL((gate_kernel<V, EP_GATE_MAX_SOFTMAX>), grid, dim3(kThreads), 0,     \
                               stream, N, E, num_groups, topk_groups, K, scores, topk_idx,         \
                               topk_weights);                                                      \
    } while (0)
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
