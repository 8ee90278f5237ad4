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
// chunk of x once (16-byte non-temporal loads: x is read exactly once),
// quantises it once in registers, then stores
// it to every valid destination row of the token (topk_idx / expert_slot are
// wave-uniform scalar loads).  HBM traffic is therefore one read of x and one
// write per (token, expert) entry, the minimum for this receive layout.
//
// FP8 lane map: 8 lanes per 128-channel block, 16 channels (32 bytes of bf16
// in, 16 bytes of FP8 out) per lane; the block amax is a 3-step xor-shuffle
// reduction over the 8 lanes.  The block scale is a'/448 or, for the
// power-of-two formats (DeepEP V1 Legacy guide §6.3, round_scale and
// use_ue8m0), 2^e with e read off the exponent and mantissa bits of a'; the
// packed UE8M0 word of blocks 4w..4w+3 is gathered by shuffles into the first
// lane of block 4w.  BF16 lane map: two 16-byte units per lane (unit = 8
// channels), so each store instruction covers 1 KiB contiguous.
//
// Destinations are taken KB entries at a time: the (expert id, slot) pairs
// arrive together (one vector load per lane, broadcast with readlane), and
// the stores of the batch follow back to back.
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

template <int KB, int SF>
__global__ __launch_bounds__(kThreads) void pack_fp8_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t S, int32_t nchunks,
    const uint16_t *__restrict__ x, const int64_t *__restrict__ topk_idx,
    const int32_t *__restrict__ expert_slot, uint8_t *__restrict__ recv_x,
    void *__restrict__ recv_scales_raw, int32_t *__restrict__ recv_src_idx, uint32_t *status)
{
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t item = blockIdx.x * kWaves + wave; // host keeps N * nchunks < 2^31
    if (item >= (uint32_t)N * (uint32_t)nchunks)
        return;
    const uint32_t t = item / (uint32_t)nchunks;
    const int32_t chunk = (int32_t)(item - t * (uint32_t)nchunks);
    const int32_t G = H / 128;
    const int32_t g = chunk * (kChunk / 128) + (lane >> 3);
    const bool active = g < G;
    const int32_t ch = g * 128 + (lane & 7) * 16;

    uint4 in0 = make_uint4(0, 0, 0, 0), in1 = make_uint4(0, 0, 0, 0);
    if (active) {
        const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t * H + ch);
        in0 = load_stream(src);
        in1 = load_stream(src + 1);
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
    float inv, scale;
    int e2 = 0;
    if (SF == EP_SCALE_FP32) {
        inv = 448.0f / ap;   // correctly rounded fp32 division
        scale = ap / 448.0f; // correctly rounded fp32 division
    } else {
        e2 = pow2_scale_exponent(ap); // in [-22, 120] for finite input
        inv = exp2_int(-e2);
        scale = exp2_int(e2);
    }
    // UE8M0: the first lane of every 4 blocks packs their 4 exponent bytes
    // (bytes of blocks past the row end are 0)
    uint32_t ue8m0_word = 0;
    const int32_t W = (G + 3) / 4;
    const bool word_lane = (lane & 31) == 0 && (g >> 2) < W;
    if (SF == EP_SCALE_UE8M0) {
        const uint32_t byte = active ? (uint32_t)(e2 + 127) : 0u;
        ue8m0_word = byte | ((uint32_t)__shfl(byte, lane + 8, 64) << 8) |
                     ((uint32_t)__shfl(byte, lane + 16, 64) << 16) |
                     ((uint32_t)__shfl(byte, lane + 24, 64) << 24);
    }
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = clamp448(f[i] * inv);
    uint4 q;
    q.x = e4m3fn_x4_hw(v[0], v[1], v[2], v[3]);
    q.y = e4m3fn_x4_hw(v[4], v[5], v[6], v[7]);
    q.z = e4m3fn_x4_hw(v[8], v[9], v[10], v[11]);
    q.w = e4m3fn_x4_hw(v[12], v[13], v[14], v[15]);

    uint32_t flags = 0;
    const int64_t *idx_t = topk_idx + (size_t)t * K;
    const int32_t *slot_t = expert_slot + (size_t)t * K;
    for (int k0 = 0; k0 < K; k0 += KB) {
        int64_t row[KB];
        float unused[KB];
        fetch_entries<KB>(idx_t, slot_t, nullptr, k0, K, E, S, lane, row, unused, flags);
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            if (row[b] >= 0) {
                if (active)
                    *reinterpret_cast<uint4 *>(recv_x + (size_t)row[b] * H + ch) = q;
                if (SF == EP_SCALE_UE8M0) {
                    if (word_lane)
                        static_cast<uint32_t *>(recv_scales_raw)[(size_t)row[b] * W + (g >> 2)] =
                            ue8m0_word;
                } else if (active && (lane & 7) == 0) {
                    static_cast<float *>(recv_scales_raw)[(size_t)row[b] * G + g] = scale;
                }
                if (chunk == 0 && lane == 0)
                    recv_src_idx[row[b]] = (int32_t)t;
            }
        }
    }
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

template <int KB>
__global__ __launch_bounds__(kThreads) void pack_bf16_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t S, int32_t nchunks,
    const uint16_t *__restrict__ x, const int64_t *__restrict__ topk_idx,
    const int32_t *__restrict__ expert_slot, uint16_t *__restrict__ recv_x,
    int32_t *__restrict__ recv_src_idx, uint32_t *status)
{
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t item = blockIdx.x * kWaves + wave; // host keeps N * nchunks < 2^31
    if (item >= (uint32_t)N * (uint32_t)nchunks)
        return;
    const uint32_t t = item / (uint32_t)nchunks;
    const int32_t chunk = (int32_t)(item - t * (uint32_t)nchunks);
    const int32_t units = H / 8;
    const int32_t u0 = chunk * (kChunk / 8) + lane;
    const int32_t u1 = u0 + 64;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t * H);
    uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
    if (u0 < units)
        a0 = load_stream(src + u0);
    if (u1 < units)
        a1 = load_stream(src + u1);

    uint32_t flags = 0;
    const int64_t *idx_t = topk_idx + (size_t)t * K;
    const int32_t *slot_t = expert_slot + (size_t)t * K;
    for (int k0 = 0; k0 < K; k0 += KB) {
        int64_t row[KB];
        float unused[KB];
        fetch_entries<KB>(idx_t, slot_t, nullptr, k0, K, E, S, lane, row, unused, flags);
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            if (row[b] >= 0) {
                uint4 *dst = reinterpret_cast<uint4 *>(recv_x + (size_t)row[b] * H);
                if (u0 < units)
                    dst[u0] = a0;
                if (u1 < units)
                    dst[u1] = a1;
                if (chunk == 0 && lane == 0)
                    recv_src_idx[row[b]] = (int32_t)t;
            }
        }
    }
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

} // namespace

hipError_t launch_dispatch(const ep_shape &s, const uint16_t *x, const int64_t *topk_idx,
                           const int32_t *expert_slot, void *recv_x, void *recv_scales,
                           int32_t *recv_src_idx, uint32_t *status, hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, E = s.num_experts;
    const int S = s.expert_capacity;
    if (N == 0)
        return hipSuccess;
    const int nchunks = (H + kChunk - 1) / kChunk;
    const int64_t items = (int64_t)N * nchunks;
    const dim3 grid((unsigned)((items + kWaves - 1) / kWaves));
    const int kb = K == 1 ? 1 : K == 2 ? 2 : K <= 4 ? 4 : 8;
    if (s.use_fp8) {
        uint8_t *rx = static_cast<uint8_t *>(recv_x);
#define EP_PACK_FP8(KB, SF)                                                                        \
    hipLaunchKernelGGL((pack_fp8_kernel<KB, SF>), grid, dim3(kThreads), 0, stream, N, H, K, E, S,  \
                       nchunks, x, topk_idx, expert_slot, rx, recv_scales, recv_src_idx, status)
#define EP_PACK_FP8_SF(SF)                                                                         \
    do {                                                                                           \
        if (kb == 1)                                                                               \
            EP_PACK_FP8(1, SF);                                                                    \
        else if (kb == 2)                                                                          \
            EP_PACK_FP8(2, SF);                                                                    \
        else if (kb == 4)                                                                          \
            EP_PACK_FP8(4, SF);                                                                    \
        else                                                                                       \
            EP_PACK_FP8(8, SF);                                                                    \
    } while (0)
        if (s.scale_format == EP_SCALE_POW2)
            EP_PACK_FP8_SF(EP_SCALE_POW2);
        else if (s.scale_format == EP_SCALE_UE8M0)
            EP_PACK_FP8_SF(EP_SCALE_UE8M0);
        else
            EP_PACK_FP8_SF(EP_SCALE_FP32);
#undef EP_PACK_FP8_SF
#undef EP_PACK_FP8
    } else {
        uint16_t *rx = static_cast<uint16_t *>(recv_x);
#define EP_PACK_BF16(KB)                                                                           \
    hipLaunchKernelGGL(pack_bf16_kernel<KB>, grid, dim3(kThreads), 0, stream, N, H, K, E, S,       \
                       nchunks, x, topk_idx, expert_slot, rx, recv_src_idx, status)
        if (kb == 1)
            EP_PACK_BF16(1);
        else if (kb == 2)
            EP_PACK_BF16(2);
        else if (kb == 4)
            EP_PACK_BF16(4);
        else
            EP_PACK_BF16(8);
#undef EP_PACK_BF16
    }
    return hipGetLastError();
}

} // namespace ep
