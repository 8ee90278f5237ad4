// dispatch.hip -- dispatch pack on gfx950.
//
// Writes each token into the fixed-shape per-expert receive buffers (Lesson 14
// §3 and DeepEP V1 Legacy guide §6.3: data [local experts, M * ranks, hidden]
// with a count per local expert), optionally as FP8 E4M3FN with one fp32
// scale per 128 channels (V1 guide §5.2(6); Ascend deep dive, "Dispatch's
// Three Phases and FP8 Compression": amax, ratio, multiply, convert, ship the
// scale with the token).
//
// Work item = one wave on one (token, 1024-channel chunk).  The wave reads its
// chunk of x once (16-byte loads), quantises it once in registers, then stores
// it to every valid destination row of the token (topk_idx / expert_slot are
// wave-uniform scalar loads).  HBM traffic is therefore one read of x and one
// write per (token, expert) entry, the minimum for this receive layout.
//
// FP8 lane map: 8 lanes per 128-channel block, 16 channels (32 bytes of bf16
// in, 16 bytes of FP8 out) per lane; the block amax is a 3-step xor-shuffle
// reduction over the 8 lanes.  BF16 lane map: two 16-byte units per lane
// (unit = 8 channels), so each store instruction covers 1 KiB contiguous.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 1024; // channels per work item

template <bool kHwConvert>
__global__ __launch_bounds__(kThreads) void pack_fp8_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t S, int32_t nchunks,
    const uint16_t *__restrict__ x, const int64_t *__restrict__ topk_idx,
    const int32_t *__restrict__ expert_slot, uint8_t *__restrict__ recv_x,
    float *__restrict__ recv_scales, int32_t *__restrict__ recv_src_idx, uint32_t *status)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
    if (item >= (int64_t)N * nchunks)
        return;
    const int32_t t = (int32_t)(item / nchunks);
    const int32_t chunk = (int32_t)(item - (int64_t)t * nchunks);
    const int32_t G = H / 128;
    const int32_t g = chunk * (kChunk / 128) + (lane >> 3);
    const bool active = g < G;
    const int32_t ch = g * 128 + (lane & 7) * 16;

    uint4 in0 = make_uint4(0, 0, 0, 0), in1 = make_uint4(0, 0, 0, 0);
    if (active) {
        const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t * H + ch);
        in0 = src[0];
        in1 = src[1];
    }
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
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    const float ap = fmaxf(amax, 1e-4f);
    const float inv = 448.0f / ap;   // correctly rounded fp32 division
    const float scale = ap / 448.0f; // correctly rounded fp32 division
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = clamp448(f[i] * inv);
    uint4 q;
    if (kHwConvert) {
        q.x = e4m3fn_x4_hw(v[0], v[1], v[2], v[3]);
        q.y = e4m3fn_x4_hw(v[4], v[5], v[6], v[7]);
        q.z = e4m3fn_x4_hw(v[8], v[9], v[10], v[11]);
        q.w = e4m3fn_x4_hw(v[12], v[13], v[14], v[15]);
    } else {
        q.x = e4m3fn_x4_sw(v[0], v[1], v[2], v[3]);
        q.y = e4m3fn_x4_sw(v[4], v[5], v[6], v[7]);
        q.z = e4m3fn_x4_sw(v[8], v[9], v[10], v[11]);
        q.w = e4m3fn_x4_sw(v[12], v[13], v[14], v[15]);
    }

    uint32_t flags = 0;
    const int64_t *idx_t = topk_idx + (size_t)t * K;
    const int32_t *slot_t = expert_slot + (size_t)t * K;
    for (int k = 0; k < K; ++k) {
        const int64_t id = idx_t[k];
        if (id < 0 || id >= (int64_t)E) {
            if (id != -1)
                flags |= EP_STATUS_BAD_EXPERT_ID;
            continue;
        }
        const int32_t j = slot_t[k];
        if (j < 0 || j >= S) {
            flags |= EP_STATUS_BAD_SLOT;
            continue;
        }
        const size_t row = (size_t)id * S + j;
        if (active) {
            *reinterpret_cast<uint4 *>(recv_x + row * H + ch) = q;
            if ((lane & 7) == 0)
                recv_scales[row * G + g] = scale;
        }
        if (chunk == 0 && lane == 0)
            recv_src_idx[row] = t;
    }
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

__global__ __launch_bounds__(kThreads) void pack_bf16_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t S, int32_t nchunks,
    const uint16_t *__restrict__ x, const int64_t *__restrict__ topk_idx,
    const int32_t *__restrict__ expert_slot, uint16_t *__restrict__ recv_x,
    int32_t *__restrict__ recv_src_idx, uint32_t *status)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t item = (int64_t)blockIdx.x * kWaves + wave;
    if (item >= (int64_t)N * nchunks)
        return;
    const int32_t t = (int32_t)(item / nchunks);
    const int32_t chunk = (int32_t)(item - (int64_t)t * nchunks);
    const int32_t units = H / 8;
    const int32_t u0 = chunk * (kChunk / 8) + lane;
    const int32_t u1 = u0 + 64;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t * H);
    uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
    if (u0 < units)
        a0 = src[u0];
    if (u1 < units)
        a1 = src[u1];

    uint32_t flags = 0;
    const int64_t *idx_t = topk_idx + (size_t)t * K;
    const int32_t *slot_t = expert_slot + (size_t)t * K;
    for (int k = 0; k < K; ++k) {
        const int64_t id = idx_t[k];
        if (id < 0 || id >= (int64_t)E) {
            if (id != -1)
                flags |= EP_STATUS_BAD_EXPERT_ID;
            continue;
        }
        const int32_t j = slot_t[k];
        if (j < 0 || j >= S) {
            flags |= EP_STATUS_BAD_SLOT;
            continue;
        }
        const size_t row = (size_t)id * S + j;
        uint4 *dst = reinterpret_cast<uint4 *>(recv_x + row * H);
        if (u0 < units)
            dst[u0] = a0;
        if (u1 < units)
            dst[u1] = a1;
        if (chunk == 0 && lane == 0)
            recv_src_idx[row] = t;
    }
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

} // namespace

hipError_t launch_dispatch(const ep_shape &s, const uint16_t *x, const int64_t *topk_idx,
                           const int32_t *expert_slot, void *recv_x, float *recv_scales,
                           int32_t *recv_src_idx, uint32_t *status, hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, E = s.num_experts;
    const int S = s.expert_capacity;
    if (N == 0)
        return hipSuccess;
    const int nchunks = (H + kChunk - 1) / kChunk;
    const int64_t items = (int64_t)N * nchunks;
    const dim3 grid((unsigned)((items + kWaves - 1) / kWaves));
    if (s.use_fp8) {
        hipLaunchKernelGGL(pack_fp8_kernel<true>, grid, dim3(kThreads), 0, stream, N, H, K, E, S,
                           nchunks, x, topk_idx, expert_slot, static_cast<uint8_t *>(recv_x),
                           recv_scales, recv_src_idx, status);
    } else {
        hipLaunchKernelGGL(pack_bf16_kernel, grid, dim3(kThreads), 0, stream, N, H, K, E, S,
                           nchunks, x, topk_idx, expert_slot, static_cast<uint16_t *>(recv_x),
                           recv_src_idx, status);
    }
    return hipGetLastError();
}

} // namespace ep
