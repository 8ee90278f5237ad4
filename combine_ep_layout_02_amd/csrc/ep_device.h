// ep_device.h -- small device helpers shared by the layout, pack and combine
// kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

// 16-byte load marked non-temporal (streamed, read once).  On gfx950 this
// keeps read-once rows from displacing cache lines; streamed reads measure
// about 20 % faster than plain loads for data far larger than the caches.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4 *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Reductions over the 8 lanes of one 128-channel block (lanes 8j..8j+7) with
// DPP moves instead of LDS permutes: swap neighbours (quad permutation
// 1,0,3,2), swap pairs (2,3,0,1), then mirror the half-row, which pairs each
// lane of one quad with a lane of the other.  Every lane ends with the
// group's result.
constexpr int kDppXor1 = 0xB1;        // quad_perm:[1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm:[2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t min8(uint32_t v)
{
    v = min(v, dpp<kDppXor1>(v));
    v = min(v, dpp<kDppXor2>(v));
    return min(v, dpp<kDppHalfMirror>(v));
}
__device__ __forceinline__ uint32_t max8(uint32_t v)
{
    v = max(v, dpp<kDppXor1>(v));
    v = max(v, dpp<kDppXor2>(v));
    return max(v, dpp<kDppHalfMirror>(v));
}
__device__ __forceinline__ float fmax8(float v)
{
    v = fmaxf(v, __uint_as_float(dpp<kDppXor1>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp<kDppXor2>(__float_as_uint(v))));
    return fmaxf(v, __uint_as_float(dpp<kDppHalfMirror>(__float_as_uint(v))));
}

// bf16 bit pattern (low 16 bits of h) -> float: exact widening.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x0040u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// E4M3FN (OCP FP8) of a float already clamped to [-448, 448], round to nearest
// even, written from the format's bit layout: the code of a normal magnitude
// is its binary32 exponent/mantissa bits shifted down by 20 and rebased from
// bias 127 to bias 7, plus one when the 20 dropped bits are above half (or
// exactly half with an odd kept bit); the carry of that +1 moves into the
// exponent as the format requires.  Magnitudes below 2^-6 are multiples of
// 2^-9: scale by 512 (exact) and round to an integer 0..8.
__device__ __forceinline__ uint32_t e4m3fn_from_clamped_sw(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a < 0x3C800000u) { // |v| < 2^-6
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    } else {
        const uint32_t dropped = a & 0xFFFFFu;
        code = (a >> 20) - (120u << 3);
        if (dropped > 0x80000u || (dropped == 0x80000u && (code & 1u)))
            code += 1u;
    }
    return sign | code;
}

// Four clamped floats -> four E4M3FN bytes (byte i from argument i), using the
// gfx950 packed conversion (OCP E4M3, round to nearest even).
__device__ __forceinline__ uint32_t e4m3fn_x4_hw(float a, float b, float c, float d)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ uint32_t e4m3fn_x4_sw(float a, float b, float c, float d)
{
    return e4m3fn_from_clamped_sw(a) | (e4m3fn_from_clamped_sw(b) << 8) |
           (e4m3fn_from_clamped_sw(c) << 16) | (e4m3fn_from_clamped_sw(d) << 24);
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// e / L for 0 <= e < 1024 and 1 <= L <= 1024 as a multiply and a shift:
// with m = ceil(2^21 / L) the error of e * m / 2^21 against e / L is below
// e * L / (L * 2^21) < 1 / L, too small to cross the next multiple of 1 / L.
__device__ __forceinline__ uint32_t rank_magic(int32_t L) { return ((1u << 21) + L - 1) / L; }
__device__ __forceinline__ int rank_of(int32_t e, uint32_t magic)
{
    return (int)(((uint32_t)e * magic) >> 21);
}

// Token t's K expert ids into e[0..KMAX): ids outside [0, E) become -1 (and
// set `bad` unless they are -1); k >= K or a token past N gives -1.
template <int KMAX>
__device__ __forceinline__ void load_token(const int64_t *__restrict__ topk_idx, int64_t t,
                                           int32_t N, int32_t K, int32_t E, int32_t (&e)[KMAX],
                                           uint32_t &bad)
{
    int64_t v[KMAX];
    if ((K & 1) == 0 && (reinterpret_cast<uintptr_t>(topk_idx) & 15) == 0) {
        // an even K on a 16-byte aligned base keeps every row aligned: two
        // ids per load
        const longlong2 *row = reinterpret_cast<const longlong2 *>(topk_idx + t * K);
#pragma unroll
        for (int q = 0; q < KMAX / 2; ++q) {
            const longlong2 p = (t < N && 2 * q < K) ? row[q] : make_longlong2(-1, -1);
            v[2 * q] = p.x;
            v[2 * q + 1] = p.y;
        }
    } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            v[k] = (t < N && k < K) ? topk_idx[t * K + k] : -1;
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const bool ok = v[k] >= 0 && v[k] < (int64_t)E;
        if (!ok && v[k] != -1)
            bad = 1u;
        e[k] = ok ? (int32_t)v[k] : -1;
    }
}

// Where the receive row of (expert e, slot j) lies, and whether it exists.
//  DenseRows:  the per-expert layout [E, S, ...]: row e * S + j, 0 <= j < S
//              (Lesson 14 §3 and DeepEP V1 Legacy guide §6.3);
//  ExpandRows: the expand layout (DeepEP Ascend deep dive, "Dispatch's Three
//              Phases", phase 1): one buffer of T rows, expert e's queue is
//              [offset[e], offset[e+1]); row offset[e] + j must fall inside it
//              and below T.
// `e` is already a routed id in [0, E).
struct DenseRows {
    int32_t S;
    __device__ __forceinline__ int64_t row(int64_t e, int32_t j, bool &ok) const
    {
        ok = j >= 0 && j < S;
        return e * S + j;
    }
};

struct ExpandRows {
    const int32_t *offset; // [E + 1]
    int64_t T;
    __device__ __forceinline__ int64_t row(int64_t e, int32_t j, bool &ok) const
    {
        const int64_t begin = offset[e], end = offset[e + 1];
        const int64_t r = begin + j;
        ok = j >= 0 && begin >= 0 && r < end && end <= T;
        return r;
    }
};

// Receive rows of entries k0 .. k0+KB-1 of one token, for a whole wave.
// Lanes 0..KB-1 each load one entry (expert id, slot and, when `w_t` is not
// NULL, weight) with an ordinary vector load -- indices are clamped to the
// token's last entry, so every lane's load is in bounds -- and the results are
// broadcast with readlane, so all KB entries arrive after a single wait (the
// expand layout adds one dependent load of the expert's queue bounds).
// row[b] = the entry's receive row (see DenseRows / ExpandRows) for a routed
// entry whose row exists, else -1; an id outside [-1, E) or a missing row
// also sets its status bit.
template <int KB, class Rows>
__device__ __forceinline__ void fetch_entries(const int64_t *__restrict__ idx_t,
                                              const int32_t *__restrict__ slot_t,
                                              const float *__restrict__ w_t, int k0, int K, int E,
                                              const Rows &rows, int lane, int64_t (&row)[KB],
                                              float (&w)[KB], uint32_t &flags)
{
    static_assert(KB >= 1 && KB <= 64, "one entry per lane");
    const int kk = min(k0 + lane, K - 1);
    const int64_t id = idx_t[kk];
    const int32_t j = slot_t[kk];
    const float wv = w_t ? w_t[kk] : 0.0f;
    const bool in_k = lane < KB && k0 + lane < K;
    const bool routed = id >= 0 && id < (int64_t)E;
    bool slot_ok;
    const int64_t rr = rows.row(routed ? id : 0, j, slot_ok);
    const int64_t r = (in_k && routed && slot_ok) ? rr : -1;
    if (__ballot(in_k && id != -1 && !routed))
        flags |= EP_STATUS_BAD_EXPERT_ID;
    if (__ballot(in_k && routed && !slot_ok))
        flags |= EP_STATUS_BAD_SLOT;
    const int32_t r_lo = (int32_t)(uint32_t)(uint64_t)r;
    const int32_t r_hi = (int32_t)(uint32_t)((uint64_t)r >> 32);
    const int32_t w_bits = __float_as_int(wv);
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane(r_lo, b);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane(r_hi, b);
        row[b] = (int64_t)(((uint64_t)hi << 32) | lo);
        w[b] = __int_as_float(__builtin_amdgcn_readlane(w_bits, b));
    }
}

// The ranks a token was sent to (normal mode, DeepEP V1 Legacy guide §5.1):
// lane r < R loads rank_slot[t, r]; the returned mask has bit r set when the
// token has a row 0 <= j < M at rank r, and `j` holds that lane's slot (read
// it for rank r with readlane).  A slot >= M sets EP_STATUS_BAD_SLOT.
__device__ __forceinline__ uint64_t rank_destinations(const int32_t *__restrict__ rank_slot_t,
                                                      int R, int M, int lane, int32_t &j,
                                                      uint32_t &flags)
{
    j = rank_slot_t[min(lane, R - 1)];
    const bool mine = lane < R;
    if (__ballot(mine && j >= M))
        flags |= EP_STATUS_BAD_SLOT;
    return __ballot(mine && j >= 0 && j < M);
}

} // namespace ep
