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
//
// Entries come in batches of 1, 2, 4, 6 or 8 (the smallest that holds K, or
// 8): with K = 5 or 6 no lane of a batch of 8 loads a row only to drop it.
//
// When one round of resident waves would not cover every item but 14 rounds
// would (K <= 8; e.g. 4,096 tokens of 7,168 channels), the top-k combine
// instead runs a grid that is resident all at once, 8 or 14 items per wave,
// and each wave stores its outputs after its last read: HBM loses bandwidth
// when reads and writes interleave, and this moves the writes towards the
// end.  Same arithmetic per item.  Larger batches run the one-item kernel.
#include <atomic>

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

// One (token, chunk) item of the top-k combine: the lane's two output units
// as bf16 (o0, o1), and the status bits of the token's entries.
template <int KB, bool BIAS, class Rows>
__device__ __forceinline__ void combine_item(uint32_t t, uint32_t chunk, int lane, int32_t H,
                                             int32_t K, int32_t E, const Rows &rows,
                                             const uint16_t *__restrict__ y,
                                             const int64_t *__restrict__ topk_idx,
                                             const float *__restrict__ topk_weights,
                                             const int32_t *__restrict__ expert_slot,
                                             const uint16_t *__restrict__ bias, const Units &u,
                                             uint4 &o0, uint4 &o1, uint32_t &flags)
{
    uint4 b0, b1;
    if (BIAS)
        load_bias(bias + (size_t)t * H, u, b0, b1);
    float acc0[8], acc1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        acc0[i] = 0.0f;
        acc1[i] = 0.0f;
    }
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
    o0 = to_bf16_unit(acc0);
    o1 = to_bf16_unit(acc1);
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
    uint4 o0, o1;
    uint32_t flags = 0;
    combine_item<KB, BIAS, Rows>(t, chunk, lane, H, K, E, rows, y, topk_idx, topk_weights,
                                 expert_slot, bias, u, o0, o1, flags);
    uint4 *dst = reinterpret_cast<uint4 *>(out + (size_t)t * H);
    if (u.has0)
        dst[u.u0] = o0;
    if (u.has1)
        dst[u.u1] = o1;
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

// The routing entries of one item as loaded (lane k < K holds entry k):
// expert id, slot and weight, not yet checked or broadcast.
struct RawEntries {
    int64_t id;
    int32_t slot;
    float w;
};

__device__ __forceinline__ RawEntries load_raw_entries(const int64_t *__restrict__ topk_idx,
                                                       const int32_t *__restrict__ expert_slot,
                                                       const float *__restrict__ topk_weights,
                                                       uint32_t t, int32_t K, int lane)
{
    const size_t at = (size_t)t * K + min(lane, K - 1);
    return RawEntries{topk_idx[at], expert_slot[at], topk_weights[at]};
}

// A grid of G waves small enough to be resident all at once (K <= KB, KB 6
// or 8: one batch of entries per item).  Wave w takes items w, w + G, ... < total,
// keeps their outputs in registers and stores them after its last item:
// HBM loses bandwidth when reads and writes interleave, and with every wave
// reading first and writing last the writes come as one burst at the end.
// The next item's entries are loaded while the current item's rows are in
// flight.  The arithmetic per item is that of combine_kernel.
template <bool BIAS, class Rows, int ITEMS, int KB>
__global__ __launch_bounds__(kThreads) void combine_multi_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t nchunks, Rows rows,
    const uint16_t *__restrict__ y, const int64_t *__restrict__ topk_idx,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ expert_slot,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ out, uint32_t *status)
{
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t w = blockIdx.x * kWaves + wave;
    const uint32_t G = gridDim.x * kWaves;
    const uint32_t total = (uint32_t)N * (uint32_t)nchunks; // host keeps it < 2^31
    uint4 o0[ITEMS], o1[ITEMS];
    RawEntries next = load_raw_entries(topk_idx, expert_slot, topk_weights,
                                       w < total ? w / (uint32_t)nchunks : 0, K, lane);
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t item = w + (uint32_t)j * G;
        if (item >= total)
            break;
        const uint32_t t = item / (uint32_t)nchunks;
        const uint32_t chunk = item - t * (uint32_t)nchunks;
        const Units u = units_of(H, chunk, lane);
        // this item's rows and weights, broadcast from lanes 0..K-1
        const RawEntries cur = next;
        uint32_t flags = 0;
        const bool in_k = lane < K;
        const bool routed = cur.id >= 0 && cur.id < (int64_t)E;
        bool slot_ok;
        const int64_t rr = rows.row(routed ? cur.id : 0, cur.slot, slot_ok);
        const int64_t r = (in_k && routed && slot_ok) ? rr : -1;
        if (__ballot(in_k && cur.id != -1 && !routed))
            flags |= EP_STATUS_BAD_EXPERT_ID;
        if (__ballot(in_k && routed && !slot_ok))
            flags |= EP_STATUS_BAD_SLOT;
        const int32_t r_lo = (int32_t)(uint32_t)(uint64_t)r;
        const int32_t r_hi = (int32_t)(uint32_t)((uint64_t)r >> 32);
        int64_t row[KB];
        float wk[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane(r_lo, b);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane(r_hi, b);
            row[b] = (int64_t)(((uint64_t)hi << 32) | lo);
            wk[b] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cur.w), b));
        }
        uint4 b0, b1;
        if (BIAS)
            load_bias(bias + (size_t)t * H, u, b0, b1);
        uint4 v0[KB], v1[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const uint4 *rp = reinterpret_cast<const uint4 *>(y + (size_t)max(row[b], (int64_t)0) * H);
            v0[b] = load_stream(rp + u.l0);
            v1[b] = load_stream(rp + u.l1);
        }
        // the next item's entries fly with this item's rows
        const uint32_t item_n = item + G;
        if (j + 1 < ITEMS && item_n < total)
            next = load_raw_entries(topk_idx, expert_slot, topk_weights, item_n / (uint32_t)nchunks,
                                    K, lane);
        float acc0[8], acc1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc0[i] = 0.0f;
            acc1[i] = 0.0f;
        }
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            if (row[b] >= 0) {
                fma_unit(acc0, wk[b], v0[b]);
                fma_unit(acc1, wk[b], v1[b]);
            }
        }
        if (BIAS) {
            add_unit(acc0, b0);
            add_unit(acc1, b1);
        }
        o0[j] = to_bf16_unit(acc0);
        o1[j] = to_bf16_unit(acc1);
        // pin the packed bf16 words here: left alone, the compiler moves the
        // packing to the stores and keeps 16 fp32 values per item alive
        asm volatile("" : "+v"(o0[j].x), "+v"(o0[j].y), "+v"(o0[j].z), "+v"(o0[j].w));
        asm volatile("" : "+v"(o1[j].x), "+v"(o1[j].y), "+v"(o1[j].z), "+v"(o1[j].w));
        // the token's chunk-0 item reports its entries' status bits
        if (chunk == 0 && flags && status && lane == 0)
            atomicOr(status, flags);
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint32_t item = w + (uint32_t)j * G;
        if (item < total) {
            const uint32_t t = item / (uint32_t)nchunks;
            const uint32_t chunk = item - t * (uint32_t)nchunks;
            const Units u = units_of(H, chunk, lane);
            uint4 *dst = reinterpret_cast<uint4 *>(out + (size_t)t * H);
            if (u.has0)
                dst[u.u0] = o0[j];
            if (u.has1)
                dst[u.u1] = o1[j];
        }
    }
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

// Items per wave for the top-k combine: 1 (a wave per item) when one round of
// resident waves covers every item or when more than kMaxItems per wave would
// be needed; otherwise the smallest instantiated count whose grid is resident
// all at once (occupancy of that instantiation times the compute units).
constexpr int kMaxItems = 14;

// Waves of KERNEL that fit on the current device at once (occupancy of its
// 256-thread blocks times the compute units), 0 if unknown.  Memoised per
// device: the answer depends only on the compiled kernel and the device.
template <auto KERNEL>
int64_t resident_waves()
{
    constexpr int kDevices = 64;
    static std::atomic<int64_t> known[kDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 0;
    if (dev < kDevices) {
        const int64_t w = known[dev].load(std::memory_order_relaxed);
        if (w > 0)
            return w;
    }
    int cus = 0, blocks = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void *>(KERNEL),
                                                     kThreads, 0) != hipSuccess)
        return 0;
    const int64_t w = (int64_t)cus * blocks * kWaves;
    if (dev < kDevices)
        known[dev].store(w, std::memory_order_relaxed);
    return w;
}

template <int KB, bool BIAS, class Rows>
hipError_t launch_topk_combine_kb(const ep_shape &s, const Rows &rows, const uint16_t *expert_out,
                                  const int64_t *topk_idx, const float *topk_weights,
                                  const int32_t *expert_slot, const uint16_t *bias,
                                  uint16_t *combined_x, uint32_t *status, hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, E = s.num_experts;
    const int nchunks = (H + kChunk - 1) / kChunk;
    const int64_t items = (int64_t)N * nchunks;
    // several items per wave for 4 < K <= 8 (batches of 6 or 8) when one
    // round of resident waves of the one-item kernel does not cover every item
    int per_wave = 1;
    if constexpr (KB == 8 || KB == 6) {
        if (K <= KB && items > resident_waves<combine_kernel<KB, BIAS, Rows>>()) {
            if (items <= 8 * resident_waves<combine_multi_kernel<BIAS, Rows, 8, KB>>())
                per_wave = 8;
            else if (items <= kMaxItems * resident_waves<combine_multi_kernel<BIAS, Rows, kMaxItems, KB>>())
                per_wave = kMaxItems;
        }
    }
    const int64_t waves = (items + per_wave - 1) / per_wave;
    const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
#define EP_COMBINE_ARGS                                                                            \
    grid, dim3(kThreads), 0, stream, N, H, K, E, nchunks, rows, expert_out, topk_idx,              \
        topk_weights, expert_slot, bias, combined_x, status
    if constexpr (KB == 8 || KB == 6) {
        if (per_wave == 8) {
            hipLaunchKernelGGL((combine_multi_kernel<BIAS, Rows, 8, KB>), EP_COMBINE_ARGS);
            return hipGetLastError();
        }
        if (per_wave == kMaxItems) {
            hipLaunchKernelGGL((combine_multi_kernel<BIAS, Rows, kMaxItems, KB>), EP_COMBINE_ARGS);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((combine_kernel<KB, BIAS, Rows>), EP_COMBINE_ARGS);
#undef EP_COMBINE_ARGS
    return hipGetLastError();
}

template <class Rows>
hipError_t launch_topk_combine(const ep_shape &s, const Rows &rows, const uint16_t *expert_out,
                               const int64_t *topk_idx, const float *topk_weights,
                               const int32_t *expert_slot, const uint16_t *bias,
                               uint16_t *combined_x, uint32_t *status, hipStream_t stream)
{
    if (s.num_tokens == 0)
        return hipSuccess;
    const int K = s.num_topk;
#define EP_COMBINE_KB(KB, BIAS)                                                                    \
    launch_topk_combine_kb<KB, BIAS, Rows>(s, rows, expert_out, topk_idx, topk_weights,            \
                                           expert_slot, bias, combined_x, status, stream)
#define EP_COMBINE_BIAS(BIAS)                                                                      \
    (K == 1 ? EP_COMBINE_KB(1, BIAS)                                                               \
            : K == 2 ? EP_COMBINE_KB(2, BIAS) : K <= 4 ? EP_COMBINE_KB(4, BIAS) : K <= 6 ? EP_COMBINE_KB(6, BIAS) : EP_COMBINE_KB(8, BIAS))
    return bias ? EP_COMBINE_BIAS(true) : EP_COMBINE_BIAS(false);
#undef EP_COMBINE_BIAS
#undef EP_COMBINE_KB
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
