// logfmt.hip -- the LogFMT combine payload on gfx950: expert outputs carried
// as one byte per channel plus a (lo, hi) header per 128 channels, and the
// top-k combine that reads them.
//
// DeepEP V1 Legacy guide §6.2: the low-latency combine message is a min/max
// header per 128 channels followed by the hidden data; §7.1: the low-latency
// test has a LogFMT combine switch.  The format (an 8-bit logarithmic one):
//   L(a)   = log2(a) rounded to the nearest binary32, a > 0;
//   header = per 128-channel block, lo / hi = min / max of L(|x|) over the
//            block's nonzero channels (0, 0 when there are none);
//   code   = bit 7 the sign, bits 0..6 m: 0 for zero, else
//            m = 1 + rint(RN(RN(L(|x|) - lo) * RN(126 / (hi - lo)))) clamped
//            to [1, 127] (ties to even; 1 when hi == lo);
//   decode = sign * 2^RN(lo + RN((m - 1) * RN((hi - lo) / 126))).
// Every step of the encoding is a binary32 operation, so codes and headers
// are exact; only the decode's exponential rounds differently from the
// definition (within a unit in the last place).
//
// L of a bf16 value: with |x| = 2^e * (1 + f/128) (subnormals normalised
// first), L = RN32(e + T[f]), T[f] = log2(1 + f/128) in binary64 from a
// 128-entry table each block builds in LDS.  binary64 leaves 29 bits of
// margin before the rounding to binary32; every bf16 input is checked
// against the correctly rounded value by ep_probe_log2_bf16.
//
// Work item = one wave on one (token, 1024-channel chunk), as in the pack
// and the combine (large batches run the encoder as a resident grid whose
// blocks first build L for all 2^15 magnitudes in LDS and then loop over
// items); a lane owns 16 channels (32 bytes of bf16, 16 code bytes)
// and 8 lanes make one 128-channel block, whose min and max take three DPP
// moves.  The encoder takes the token's routed rows (e, slot) -- each
// expert output row is referenced by exactly one (token, k) -- loads every
// row of a batch of 8 entries before encoding the first, and writes the
// codes and headers in place of the bf16 row.  The combine loads every
// row's codes and header of a batch before decoding the first, then runs
// the combine's k-ordered fp32 FMA chain.  The decode (a multiply, an add
// and an exponential per channel) makes the combine compute-bound on one
// GPU: it reads 42 % fewer bytes than the BF16 combine and takes about as
// long; the bytes it saves are link bytes when expert outputs cross GPUs.
#include <algorithm>
#include <atomic>

#include "ep_device.h"
#include "ep_internal.h"
#include "ep_probe.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = 1024; // channels per work item
constexpr int kKB = 8;       // routing entries per batch

// T[f] = log2(1 + f / 128), f = 0..127, built by the block's first 128
// threads (1 + f/128 is exact in binary64).  Needs a barrier after.
__device__ __forceinline__ void build_log2_table(double *T)
{
    if (threadIdx.x < 128)
        T[threadIdx.x] = log2(1.0 + (double)threadIdx.x * (1.0 / 128.0));
}

// L of a nonzero bf16 magnitude (bits 0..14 of the pattern, not 0).
__device__ __forceinline__ float log2_rn_bf16(uint32_t mag, const double *T)
{
    const uint32_t ex = mag >> 7, mant = mag & 127u;
    int e;
    uint32_t f;
    if (ex != 0) {
        e = (int)ex - 127;
        f = mant;
    } else {
        // subnormal: mant * 2^-133, mant in 1..127; p = position of the top bit
        const int p = 31 - __builtin_clz(mant);
        e = -133 + p;
        f = (mant << (7 - p)) & 127u;
    }
    return (float)((double)e + T[f]);
}

// One lane's place on the (token, chunk) lane map: block g, first channel ch.
struct LfLane {
    int32_t G, g, ch;
    bool active;
};

__device__ __forceinline__ LfLane lf_lane(int32_t H, int32_t chunk, int lane)
{
    LfLane l;
    l.G = H / 128;
    l.g = chunk * (kChunk / 128) + (lane >> 3);
    l.active = l.g < l.G;
    l.ch = l.g * 128 + (lane & 7) * 16;
    return l;
}

// L of a normal bf16 magnitude (exponent field 1..255): no branch.  A zero
// magnitude gives a finite value that the caller discards.
__device__ __forceinline__ float log2_rn_normal(uint32_t mag, const double *T)
{
    return (float)((double)((int)(mag >> 7) - 127) + T[mag & 127u]);
}

// Encode one lane's 16 channels (in0, in1: bf16 pairs) into 16 code bytes,
// with the block's (lo, hi) from its 8 lanes.  Called by every lane.
//
// L is non-decreasing in the magnitude bits, so lo and hi are L of the
// block's smallest nonzero and largest magnitude: integer min / max over
// the bits, then two logarithms per lane.  Lanes holding a subnormal take
// the general logarithm for all 16 channels; the others, almost always all
// of them, the branch-free one.  With lo <= L <= hi, RN(L - lo) <= hi - lo and
// inv <= (126 / (hi - lo)) (1 + 2^-24), so q <= 126 + 2^-17 and rint(q) <= 126:
// the clamp of the code to [1, 127] never acts on a nonzero channel and is
// left out.  rint(q) is read off RN(q + 1.5 * 2^23), exact for 0 <= q < 2^22
// (the sum is rounded to an integer, ties to even, as rint does).
__device__ __forceinline__ void encode_lane(const uint4 &in0, const uint4 &in1, const double *T,
                                            uint4 &codes, float &lo, float &hi)
{
    const uint32_t w[8] = {in0.x, in0.y, in0.z, in0.w, in1.x, in1.y, in1.z, in1.w};
    uint32_t mag[16], sgn[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        mag[2 * i] = w[i] & 0x7FFFu;
        mag[2 * i + 1] = (w[i] >> 16) & 0x7FFFu;
        sgn[2 * i] = (w[i] >> 8) & 0x80u;
        sgn[2 * i + 1] = (w[i] >> 24) & 0x80u;
    }
    // smallest nonzero magnitude minus one (a zero wraps to the largest
    // value and drops out), largest magnitude
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        mn = min(mn, mag[i] - 1u);
        mx = max(mx, mag[i]);
    }
    const bool subnormal = mn < 0x7Fu; // a nonzero magnitude below 2^-126
    mn = min8(mn);
    mx = max8(mx);
    const bool any = mx != 0u;
    lo = any ? log2_rn_bf16(mn + 1u, T) : 0.0f;
    hi = any ? log2_rn_bf16(mx, T) : 0.0f;
    const float span = hi - lo;
    const float inv = span > 0.0f ? 126.0f / span : 0.0f; // correctly rounded division
    float l[16];
    if (subnormal) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            l[i] = log2_rn_bf16(max(mag[i], 1u), T);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            l[i] = log2_rn_normal(mag[i], T);
    }
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float q = (l[i] - lo) * inv;
        const uint32_t m = __float_as_uint(q + 12582912.0f) - 0x4B3FFFFFu; // 1 + rint(q)
        const uint32_t code = mag[i] ? (sgn[i] | m) : 0u;
        out[i >> 2] |= code << (8 * (i & 3));
    }
    codes = make_uint4(out[0], out[1], out[2], out[3]);
}

// encode_lane with every logarithm read from a table of L over all 2^15
// magnitudes (entry 0 unused), the same values log2_rn_bf16 gives, and the
// integer work done on packed halves or four bytes at a time:
//  - magnitudes stay packed two per word; the block's smallest nonzero
//    magnitude (minus one, a zero wrapping to 0xFFFF) and largest come from
//    packed 16-bit min / max;
//  - rint(q) is the low byte of RN(q + 1.5 * 2^23) (q <= 126 + 2^-17 on a
//    nonzero channel); v_perm_b32 gathers the low bytes of four of them
//    into one word, and masking each byte to 7 bits keeps the garbage of
//    zero channels from carrying when 1 is added to every byte;
//  - the sign bytes and the nonzero masks come from bits 15 and 31 of the
//    input words (and of magnitude + 0x7FFF per half) with v_perm_b32's
//    sign-replicating selectors.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 halves(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t word(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
// v_perm_b32 selectors: result byte i takes selector byte i; 0..3 pick a
// byte of the second operand, 4..7 of the first, 8 / 9 / 10 / 11 give 0xFF
// or 0x00 by bit 15 / 31 of the second / first operand, 12 gives 0x00.
constexpr uint32_t kPermLowBytes01 = 0x0C0C0400u; // b0 of second, b0 of first -> bytes 0, 1
constexpr uint32_t kPermLowBytes23 = 0x04000C0Cu; // b0 of second, b0 of first -> bytes 2, 3
constexpr uint32_t kPermHalfSigns = 0x0B0A0908u;  // bits 15, 31 of second, then of first

__device__ __forceinline__ void encode_lane_table(const uint4 &in0, const uint4 &in1, const float *L,
                                                  uint4 &codes, float &lo, float &hi)
{
    const uint32_t w[8] = {in0.x, in0.y, in0.z, in0.w, in1.x, in1.y, in1.z, in1.w};
    uint32_t m2[8];
    u16x2 mnv = {0xFFFF, 0xFFFF}, mxv = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        m2[i] = w[i] & 0x7FFF7FFFu;
        const u16x2 v = halves(m2[i]);
        mnv = __builtin_elementwise_min(mnv, v - (u16x2)(1));
        mxv = __builtin_elementwise_max(mxv, v);
    }
    uint32_t mn = min((uint32_t)mnv.x, (uint32_t)mnv.y);
    uint32_t mx = max((uint32_t)mxv.x, (uint32_t)mxv.y);
    mn = min8(mn);
    mx = max8(mx);
    const bool any = mx != 0u;
    lo = any ? L[(mn + 1u) & 0x7FFFu] : 0.0f;
    hi = any ? L[mx] : 0.0f;
    const float span = hi - lo;
    const float inv = span > 0.0f ? 126.0f / span : 0.0f; // correctly rounded division
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // channels 4j .. 4j+3: the low and high halves of words 2j, 2j+1
        uint32_t t[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t m = m2[2 * j + (e >> 1)];
            const uint32_t mag = (e & 1) ? m >> 16 : m & 0xFFFFu;
            const float q = (L[mag] - lo) * inv;
            t[e] = __float_as_uint(q + 12582912.0f);
        }
        const uint32_t r = (__builtin_amdgcn_perm(t[1], t[0], kPermLowBytes01) |
                            __builtin_amdgcn_perm(t[3], t[2], kPermLowBytes23)) & 0x7F7F7F7Fu;
        const uint32_t sgn = __builtin_amdgcn_perm(w[2 * j + 1], w[2 * j], kPermHalfSigns) & 0x80808080u;
        const uint32_t nz = __builtin_amdgcn_perm(word(halves(m2[2 * j + 1]) + (u16x2)(0x7FFF)),
                                                  word(halves(m2[2 * j]) + (u16x2)(0x7FFF)),
                                                  kPermHalfSigns);
        out[j] = ((r + 0x01010101u) | sgn) & nz;
    }
    codes = make_uint4(out[0], out[1], out[2], out[3]);
}

template <int KB, class Rows>
__global__ __launch_bounds__(kThreads) void logfmt_encode_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t nchunks, Rows rows,
    const uint16_t *__restrict__ y, const int64_t *__restrict__ topk_idx,
    const int32_t *__restrict__ expert_slot, uint8_t *__restrict__ codes,
    float *__restrict__ headers, uint32_t *status)
{
    __shared__ double s_T[128];
    build_log2_table(s_T);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t item = blockIdx.x * kWaves + wave; // host keeps N * nchunks < 2^31
    if (item >= (uint32_t)N * (uint32_t)nchunks)
        return;
    const uint32_t t = item / (uint32_t)nchunks;
    const int32_t chunk = (int32_t)(item - t * (uint32_t)nchunks);
    const LfLane l = lf_lane(H, chunk, lane);
    const int32_t ch = l.active ? l.ch : 0; // lanes past the row end read channel 0 (unused)
    uint32_t flags = 0;
    const int64_t *idx_t = topk_idx + (size_t)t * K;
    const int32_t *slot_t = expert_slot + (size_t)t * K;
    for (int k0 = 0; k0 < K; k0 += KB) {
        int64_t row[KB];
        float unused[KB];
        fetch_entries<KB>(idx_t, slot_t, nullptr, k0, K, E, rows, lane, row, unused, flags);
        uint4 a0[KB], a1[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const uint4 *src = reinterpret_cast<const uint4 *>(y + (size_t)max(row[b], (int64_t)0) * H + ch);
            a0[b] = load_stream(src);
            a1[b] = load_stream(src + 1);
        }
        // every row of the batch is encoded (an entry without a row encodes
        // row 0 and stores nothing), so no row's loads wait inside a branch
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            uint4 c;
            float lo, hi;
            encode_lane(a0[b], a1[b], s_T, c, lo, hi);
            if (row[b] >= 0 && l.active) {
                *reinterpret_cast<uint4 *>(codes + (size_t)row[b] * H + l.ch) = c;
                if ((lane & 7) == 0)
                    *reinterpret_cast<float2 *>(headers + ((size_t)row[b] * l.G + l.g) * 2) =
                        make_float2(lo, hi);
            }
        }
    }
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

// The encoder for large batches: blocks of 1,024 threads, one per compute
// unit, each first building L for every bf16 magnitude in LDS (32,768 floats,
// 128 KiB, from the same T and the same arithmetic as log2_rn_bf16), then
// looping over work items (wave w of the grid takes items w, w + G, ...).  A
// channel's logarithm is then one LDS read: the encoder drops from about 20
// to about 14 instructions per channel.
constexpr int kTabThreads = 1024;
constexpr int kTabWaves = kTabThreads / 64;
constexpr int kMagnitudes = 1 << 15;
// Below this many work items the per-item encoder is faster: each table
// block spends a few microseconds building its table first (at 128 tokens x
// 7,168: 12.5 us per-item against 22.9 us with the table).
constexpr int64_t kTableMinItems = 4096;

template <int KB, class Rows>
__global__ __launch_bounds__(kTabThreads) void logfmt_encode_table_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t nchunks, Rows rows,
    const uint16_t *__restrict__ y, const int64_t *__restrict__ topk_idx,
    const int32_t *__restrict__ expert_slot, uint8_t *__restrict__ codes,
    float *__restrict__ headers, uint32_t *status)
{
    __shared__ float s_L[kMagnitudes];
    __shared__ double s_T[128];
    build_log2_table(s_T);
    __syncthreads();
    for (int m = threadIdx.x; m < kMagnitudes; m += kTabThreads)
        s_L[m] = m ? log2_rn_bf16((uint32_t)m, s_T) : 0.0f;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t total = (uint32_t)N * (uint32_t)nchunks; // host keeps it < 2^31
    const uint32_t G = gridDim.x * kTabWaves;
    uint32_t flags = 0;
    for (uint32_t item = blockIdx.x * kTabWaves + wave; item < total; item += G) {
        const uint32_t t = item / (uint32_t)nchunks;
        const int32_t chunk = (int32_t)(item - t * (uint32_t)nchunks);
        const LfLane l = lf_lane(H, chunk, lane);
        const int32_t ch = l.active ? l.ch : 0;
        const int64_t *idx_t = topk_idx + (size_t)t * K;
        const int32_t *slot_t = expert_slot + (size_t)t * K;
        for (int k0 = 0; k0 < K; k0 += KB) {
            int64_t row[KB];
            float unused[KB];
            fetch_entries<KB>(idx_t, slot_t, nullptr, k0, K, E, rows, lane, row, unused, flags);
            uint4 a0[KB], a1[KB];
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                const uint4 *src =
                    reinterpret_cast<const uint4 *>(y + (size_t)max(row[b], (int64_t)0) * H + ch);
                a0[b] = load_stream(src);
                a1[b] = load_stream(src + 1);
            }
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                uint4 c;
                float lo, hi;
                encode_lane_table(a0[b], a1[b], s_L, c, lo, hi);
                if (row[b] >= 0 && l.active) {
                    *reinterpret_cast<uint4 *>(codes + (size_t)row[b] * H + l.ch) = c;
                    if ((lane & 7) == 0)
                        *reinterpret_cast<float2 *>(headers + ((size_t)row[b] * l.G + l.g) * 2) =
                            make_float2(lo, hi);
                }
            }
        }
    }
    if (flags && status && lane == 0)
        atomicOr(status, flags);
}

// Decode one lane's 16 codes and add w * value to acc, ascending channel.
// When the block's lo >= -126 every decoded value is a normal float and the
// hardware exponential is used directly (the branch is uniform over the
// lane's 16 values); otherwise exp2f, which scales subnormal results.
template <bool NORMAL>
__device__ __forceinline__ void fma_decoded_lane(float (&acc)[16], float w, const uint4 &c,
                                                 float lo, float step)
{
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t code = (cw[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        const uint32_t m = code & 0x7Fu;
        const float d = lo + (float)((int)m - 1) * step;
        const float e = NORMAL ? __builtin_amdgcn_exp2f(d) : exp2f(d);
        const float mag = m ? e : 0.0f;
        acc[i] = fmaf(w, __uint_as_float(__float_as_uint(mag) | ((code & 0x80u) << 24)), acc[i]);
    }
}

__device__ __forceinline__ void fma_decoded(float (&acc)[16], float w, const uint4 &c, float lo,
                                            float hi)
{
    const float step = (hi - lo) / 126.0f; // correctly rounded division
    if (lo >= -126.0f)
        fma_decoded_lane<true>(acc, w, c, lo, step);
    else
        fma_decoded_lane<false>(acc, w, c, lo, step);
}

template <int KB, bool BIAS, class Rows>
__global__ __launch_bounds__(kThreads) void logfmt_combine_kernel(
    int32_t N, int32_t H, int32_t K, int32_t E, int32_t nchunks, Rows rows,
    const uint8_t *__restrict__ codes, const float *__restrict__ headers,
    const int64_t *__restrict__ topk_idx, const float *__restrict__ topk_weights,
    const int32_t *__restrict__ expert_slot, const uint16_t *__restrict__ bias,
    uint16_t *__restrict__ out, uint32_t *status)
{
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t item = blockIdx.x * kWaves + wave; // host keeps N * nchunks < 2^31
    if (item >= (uint32_t)N * (uint32_t)nchunks)
        return;
    const uint32_t t = item / (uint32_t)nchunks;
    const int32_t chunk = (int32_t)(item - t * (uint32_t)nchunks);
    const LfLane l = lf_lane(H, chunk, lane);
    const int32_t ch = l.active ? l.ch : 0; // lanes past the row end read channel 0 (unused)
    const int32_t g = l.active ? l.g : 0;
    uint4 b0 = make_uint4(0, 0, 0, 0), b1 = make_uint4(0, 0, 0, 0);
    if (BIAS) {
        const uint4 *br = reinterpret_cast<const uint4 *>(bias + (size_t)t * H + ch);
        b0 = load_stream(br);
        b1 = load_stream(br + 1);
    }
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        acc[i] = 0.0f;
    uint32_t flags = 0;
    const int64_t *idx_t = topk_idx + (size_t)t * K;
    const int32_t *slot_t = expert_slot + (size_t)t * K;
    const float *w_t = topk_weights + (size_t)t * K;
    const int32_t G = H / 128;
    for (int k0 = 0; k0 < K; k0 += KB) {
        int64_t row[KB];
        float wk[KB];
        fetch_entries<KB>(idx_t, slot_t, w_t, k0, K, E, rows, lane, row, wk, flags);
        // every row's codes and header of the batch in flight before the
        // first decode; an entry without a row reads row 0 and is not added
        uint4 c[KB];
        float2 hd[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const size_t r = (size_t)max(row[b], (int64_t)0);
            c[b] = load_stream(reinterpret_cast<const uint4 *>(codes + r * H + ch));
            hd[b] = *reinterpret_cast<const float2 *>(headers + (r * G + g) * 2);
        }
#pragma unroll
        for (int b = 0; b < KB; ++b)
            if (row[b] >= 0)
                fma_decoded(acc, wk[b], c[b], hd[b].x, hd[b].y);
    }
    if (BIAS) {
        const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc[2 * i] = acc[2 * i] + bf16_lo(bw[i]);
            acc[2 * i + 1] = acc[2 * i + 1] + bf16_hi(bw[i]);
        }
    }
    if (l.active) {
        uint4 *dst = reinterpret_cast<uint4 *>(out + (size_t)t * H + l.ch);
        dst[0] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                            pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
        dst[1] = make_uint4(pack_bf16x2(acc[8], acc[9]), pack_bf16x2(acc[10], acc[11]),
                            pack_bf16x2(acc[12], acc[13]), pack_bf16x2(acc[14], acc[15]));
    }
    if (flags && status && lane == 0 && chunk == 0)
        atomicOr(status, flags);
}

__global__ __launch_bounds__(kThreads) void log2_probe_kernel(const uint16_t *__restrict__ bits,
                                                              float *__restrict__ out, int64_t n)
{
    __shared__ double s_T[128];
    build_log2_table(s_T);
    __syncthreads();
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n)
        return;
    const uint32_t mag = bits[i] & 0x7FFFu;
    out[i] = mag ? log2_rn_bf16(mag, s_T) : -__builtin_inff();
}

} // namespace

namespace {
// Compute units of the current device, memoised per device (0 if unknown).
int compute_units()
{
    constexpr int kDevices = 64;
    static std::atomic<int> known[kDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 0;
    if (dev < kDevices) {
        const int c = known[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (dev < kDevices)
        known[dev].store(cus, std::memory_order_relaxed);
    return cus;
}
} // namespace

hipError_t launch_logfmt_encode(const ep_shape &s, const uint16_t *expert_out,
                                const int64_t *topk_idx, const int32_t *expert_slot,
                                uint8_t *codes, float *headers, uint32_t *status,
                                hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, E = s.num_experts;
    if (N == 0)
        return hipSuccess;
    const int nchunks = (H + kChunk - 1) / kChunk;
    const int64_t items = (int64_t)N * nchunks;
    const int cus = compute_units();
    if (cus > 0 && items >= kTableMinItems) {
        const int64_t blocks = std::min<int64_t>(cus, (items + kTabWaves - 1) / kTabWaves);
        hipLaunchKernelGGL((logfmt_encode_table_kernel<kKB, DenseRows>), dim3((unsigned)blocks),
                           dim3(kTabThreads), 0, stream, N, H, K, E, nchunks,
                           DenseRows{s.expert_capacity}, expert_out, topk_idx, expert_slot, codes,
                           headers, status);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((items + kWaves - 1) / kWaves));
    hipLaunchKernelGGL((logfmt_encode_kernel<kKB, DenseRows>), grid, dim3(kThreads), 0, stream, N, H,
                       K, E, nchunks, DenseRows{s.expert_capacity}, expert_out, topk_idx,
                       expert_slot, codes, headers, status);
    return hipGetLastError();
}

hipError_t launch_combine_logfmt(const ep_shape &s, const uint8_t *codes, const float *headers,
                                 const int64_t *topk_idx, const float *topk_weights,
                                 const int32_t *expert_slot, const uint16_t *bias,
                                 uint16_t *combined_x, uint32_t *status, hipStream_t stream)
{
    const int N = s.num_tokens, H = s.hidden, K = s.num_topk, E = s.num_experts;
    if (N == 0)
        return hipSuccess;
    const int nchunks = (H + kChunk - 1) / kChunk;
    const dim3 grid((unsigned)(((int64_t)N * nchunks + kWaves - 1) / kWaves));
#define EP_LF_COMBINE(KB, BIAS)                                                                    \
    hipLaunchKernelGGL((logfmt_combine_kernel<KB, BIAS, DenseRows>), grid, dim3(kThreads), 0,      \
                       stream, N, H, K, E, nchunks, DenseRows{s.expert_capacity}, codes, headers,  \
                       topk_idx, topk_weights, expert_slot, bias, combined_x, status)
    if (bias) {
        if (K <= 4)
            EP_LF_COMBINE(4, true);
        else
            EP_LF_COMBINE(8, true);
    } else {
        if (K <= 4)
            EP_LF_COMBINE(4, false);
        else
            EP_LF_COMBINE(8, false);
    }
#undef EP_LF_COMBINE
    return hipGetLastError();
}

} // namespace ep

extern "C" int ep_probe_log2_bf16(const uint16_t *bits, float *out, int64_t n, void *stream)
{
    if (n < 0)
        return EP_ERR_SHAPE;
    if (n == 0)
        return EP_OK;
    if (!bits || !out)
        return EP_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(bits) & 1) || (reinterpret_cast<uintptr_t>(out) & 3))
        return EP_ERR_ALIGN;
    const dim3 grid((unsigned)((n + ep::kThreads - 1) / ep::kThreads));
    hipLaunchKernelGGL(ep::log2_probe_kernel, grid, dim3(ep::kThreads), 0,
                       static_cast<hipStream_t>(stream), bits, out, n);
    return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
}
