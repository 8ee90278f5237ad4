// ep_abi.hip -- the C ABI declared in include/ep.h: host-side validation,
// buffer sizes and launches on the caller's stream.  Every static check runs
// before anything is enqueued; no entry point allocates or synchronises.
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "ep_internal.h"

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(const ep_shape *s)
{
    if (!s)
        return EP_ERR_NULL;
    const int64_t N = s->num_tokens, H = s->hidden, K = s->num_topk, E = s->num_experts,
                  R = s->num_ranks, M = s->num_max_dispatch_tokens_per_rank,
                  S = s->expert_capacity;
    if (N < 0 || H < 8 || H % 8 != 0 || K < 1 || E < 1 || R < 1 || E % R != 0)
        return EP_ERR_SHAPE;
    if (s->use_fp8 != 0 && s->use_fp8 != 1)
        return EP_ERR_SHAPE;
    if (s->use_fp8 && H % 128 != 0)
        return EP_ERR_SHAPE;
    if (s->scale_format < EP_SCALE_FP32 || s->scale_format > EP_SCALE_UE8M0 ||
        (!s->use_fp8 && s->scale_format != EP_SCALE_FP32))
        return EP_ERR_SHAPE;
    if (s->expert_alignment < 0)
        return EP_ERR_SHAPE;
    if (K > EP_MAX_TOPK || E > EP_MAX_EXPERTS || R > EP_MAX_RANKS ||
        s->expert_alignment > EP_MAX_ALIGNMENT)
        return EP_ERR_UNSUPPORTED;
    if (M < 1 || N > M || S < M)
        return EP_ERR_CAPACITY;
    // indices stay within int32 where the kernels keep them in 32 bits, and
    // byte offsets within int64
    if (N * K > INT32_MAX || N * R > INT32_MAX || E * S > INT32_MAX)
        return EP_ERR_UNSUPPORTED;
    if (E * S > INT64_MAX / (H * 2))
        return EP_ERR_UNSUPPORTED;
    // normal-mode rows (R * M) and expand rows (T) are numbered in 32 bits
    if (R * M > INT32_MAX || ep::expand_rows(*s) > INT32_MAX)
        return EP_ERR_UNSUPPORTED;
    // pack and combine number their work items (token or expand-padding
    // expert, 1024-channel chunk) in 32 bits
    if ((N + E) * ((H + 1023) / 1024) > INT32_MAX)
        return EP_ERR_UNSUPPORTED;
    ep::LayoutPlan plan;
    if (!ep::plan_layout(*s, &plan))
        return EP_ERR_UNSUPPORTED;
    return EP_OK;
}

// Scratch of ep_layout_noalloc: the layout's per-block histograms live in
// this file-scope device array instead of a caller workspace.  Every GPU the
// library runs on holds its own copy until the process ends.  On the host the
// name `scratch` is only a stand-in, not a device address, so it is never
// passed to a kernel: its address on each device is looked up once, with that
// device current, and kept in scratch_addr[].  Calls that overlap on one GPU
// share the array and race; the histograms need no clearing (the count
// kernel writes every row before the assign kernel reads it).
static __device__ __align__(256) unsigned char scratch[EP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_addr[kMaxDevices];
std::mutex scratch_mutex;

// Device address of `scratch` on device `dev` (looked up at the first call
// on that device).
hipError_t scratch_on(int dev, void **out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mutex);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            int cur = 0;
            hipError_t err = hipGetDevice(&cur);
            if (err == hipSuccess && cur != dev)
                err = hipSetDevice(dev);
            if (err != hipSuccess)
                return err;
            err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
            if (err != hipSuccess)
                return err;
            if (back != hipSuccess)
                return back;
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

// The host checks of ep_layout that do not concern the workspace: shape,
// null and misaligned pointers.
int layout_args(const ep_shape *s, const int64_t *topk_idx, const int32_t *num_tokens_per_rank,
                const int32_t *num_tokens_per_expert, const uint8_t *is_token_in_rank,
                const int32_t *expert_slot, const int32_t *rank_slot, const int32_t *expert_offset,
                const uint32_t *status)
{
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    const bool has_tokens = s->num_tokens > 0;
    if (!num_tokens_per_rank || !num_tokens_per_expert)
        return EP_ERR_NULL;
    if (has_tokens && (!topk_idx || !is_token_in_rank || !expert_slot || !rank_slot))
        return EP_ERR_NULL;
    if (!aligned(topk_idx, 8) || !aligned(num_tokens_per_rank, 4) ||
        !aligned(num_tokens_per_expert, 4) || !aligned(expert_slot, 4) || !aligned(rank_slot, 4) ||
        !aligned(expert_offset, 4) || !aligned(status, 4))
        return EP_ERR_ALIGN;
    return EP_OK;
}

} // namespace

extern "C" {

const char *ep_strerror(int code)
{
    switch (code) {
    case EP_OK:
        return "EP_OK";
    case EP_ERR_NULL:
        return "EP_ERR_NULL: a required pointer is NULL";
    case EP_ERR_SHAPE:
        return "EP_ERR_SHAPE: invalid shape";
    case EP_ERR_CAPACITY:
        return "EP_ERR_CAPACITY: num_tokens > num_max_dispatch_tokens_per_rank or "
               "expert_capacity < num_max_dispatch_tokens_per_rank";
    case EP_ERR_ALIGN:
        return "EP_ERR_ALIGN: misaligned pointer";
    case EP_ERR_UNSUPPORTED:
        return "EP_ERR_UNSUPPORTED: size outside the library's limits";
    case EP_ERR_HIP:
        return "EP_ERR_HIP: kernel launch failed";
    case EP_ERR_WORKSPACE:
        return "EP_ERR_WORKSPACE: layout workspace missing or too small";
    case EP_ERR_SCRATCH:
        return "EP_ERR_SCRATCH: the layout needs more scratch than ep_layout_noalloc's static "
               "buffer holds (EP_NOALLOC_SCRATCH_BYTES); use ep_layout with a workspace";
    default:
        return "unknown ep status code";
    }
}

int ep_query_sizes(const ep_shape *s, ep_sizes *out)
{
    if (!out)
        return EP_ERR_NULL;
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    const size_t N = s->num_tokens, H = s->hidden, K = s->num_topk, E = s->num_experts,
                 R = s->num_ranks, S = s->expert_capacity;
    const size_t rows = E * S;
    out->recv_x = rows * H * (s->use_fp8 ? 1 : 2);
    const size_t G = H / 128;
    out->recv_scales = !s->use_fp8 ? 0
                       : s->scale_format == EP_SCALE_UE8M0 ? rows * ((G + 3) / 4) * sizeof(uint32_t)
                                                           : rows * G * sizeof(float);
    out->recv_src_idx = rows * sizeof(int32_t);
    out->expert_out = rows * H * 2;
    out->combined_x = N * H * 2;
    out->num_tokens_per_rank = R * sizeof(int32_t);
    out->num_tokens_per_expert = E * sizeof(int32_t);
    out->is_token_in_rank = N * R;
    out->expert_slot = N * K * sizeof(int32_t);
    out->rank_slot = N * R * sizeof(int32_t);
    out->expert_offset = (E + 1) * sizeof(int32_t);
    ep::LayoutPlan plan;
    ep::plan_layout(*s, &plan);
    out->layout_workspace = ep::layout_dispatch_workspace(*s, plan);
    const size_t M = s->num_max_dispatch_tokens_per_rank;
    const size_t scale_row = !s->use_fp8 ? 0
                             : s->scale_format == EP_SCALE_UE8M0 ? ((G + 3) / 4) * sizeof(uint32_t)
                                                                 : G * sizeof(float);
    const size_t nrows = R * M;
    out->recv_x_normal = nrows * H * (s->use_fp8 ? 1 : 2);
    out->recv_scales_normal = nrows * scale_row;
    out->recv_topk_idx = nrows * K * sizeof(int64_t);
    out->recv_topk_weights = nrows * K * sizeof(float);
    out->recv_src_idx_normal = nrows * sizeof(int32_t);
    out->expert_out_normal = nrows * H * 2;
    out->combined_topk_weights = N * K * sizeof(float);
    const size_t T = (size_t)ep::expand_rows(*s);
    out->recv_x_expand = T * H * (s->use_fp8 ? 1 : 2);
    out->recv_scales_expand = T * scale_row;
    out->recv_src_idx_expand = T * sizeof(int32_t);
    out->expert_out_expand = T * H * 2;
    out->logfmt_codes = H % 128 == 0 ? rows * H : 0;
    out->logfmt_headers = H % 128 == 0 ? rows * (H / 128) * 2 * sizeof(float) : 0;
    return EP_OK;
}

int ep_layout(const ep_shape *s, const int64_t *topk_idx, int32_t *num_tokens_per_rank,
              int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank, int32_t *expert_slot,
              int32_t *rank_slot, int32_t *expert_offset, void *workspace, size_t workspace_bytes,
              uint32_t *status, void *stream)
{
    const int rc = layout_args(s, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                               is_token_in_rank, expert_slot, rank_slot, expert_offset, status);
    if (rc != EP_OK)
        return rc;
    if (!aligned(workspace, 16))
        return EP_ERR_ALIGN;
    ep::LayoutPlan plan;
    ep::plan_layout(*s, &plan);
    if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
        return EP_ERR_WORKSPACE;
    const hipError_t err = ep::launch_layout(
        *s, plan, topk_idx, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,
        expert_slot, rank_slot, expert_offset, static_cast<int32_t *>(workspace), status,
        static_cast<hipStream_t>(stream));
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_layout_noalloc(const ep_shape *s, const int64_t *topk_idx, int32_t *num_tokens_per_rank,
                      int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                      int32_t *expert_slot, int32_t *rank_slot, int32_t *expert_offset,
                      uint32_t *status, void *stream)
{
    const int rc = layout_args(s, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                               is_token_in_rank, expert_slot, rank_slot, expert_offset, status);
    if (rc != EP_OK)
        return rc;
    ep::LayoutPlan plan;
    ep::plan_layout(*s, &plan);
    if (plan.workspace_bytes > EP_NOALLOC_SCRATCH_BYTES)
        return EP_ERR_SCRATCH;
    // the scratch of the stream's device (its address is looked up at the
    // first call on that device)
    int dev = 0;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if ((st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev)) != hipSuccess)
        return EP_ERR_HIP;
    void *ws = nullptr;
    if (scratch_on(dev, &ws) != hipSuccess)
        return EP_ERR_HIP;
    const hipError_t err = ep::launch_layout(
        *s, plan, topk_idx, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,
        expert_slot, rank_slot, expert_offset, static_cast<int32_t *>(ws), status, st);
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_dispatch(const ep_shape *s, const uint16_t *x, const int64_t *topk_idx,
                const int32_t *expert_slot, void *recv_x, void *recv_scales,
                int32_t *recv_src_idx, uint32_t *status, void *stream)
{
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    if (s->num_tokens == 0)
        return EP_OK;
    if (!x || !topk_idx || !expert_slot || !recv_x || !recv_src_idx)
        return EP_ERR_NULL;
    if (s->use_fp8 && !recv_scales)
        return EP_ERR_NULL;
    if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 8) ||
        !aligned(expert_slot, 4) || !aligned(recv_scales, 4) || !aligned(recv_src_idx, 4) ||
        !aligned(status, 4))
        return EP_ERR_ALIGN;
    const hipError_t err =
        ep::launch_dispatch(*s, x, topk_idx, expert_slot, recv_x, recv_scales, recv_src_idx,
                            status, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_layout_dispatch(const ep_shape *s, const int64_t *topk_idx, const uint16_t *x,
                       int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                       uint8_t *is_token_in_rank, int32_t *expert_slot, int32_t *rank_slot,
                       int32_t *expert_offset, void *workspace, size_t workspace_bytes,
                       void *recv_x, void *recv_scales, int32_t *recv_src_idx, uint32_t *status,
                       void *stream)
{
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    const bool has_tokens = s->num_tokens > 0;
    // the checks of ep_layout, then those of ep_dispatch
    if (!num_tokens_per_rank || !num_tokens_per_expert)
        return EP_ERR_NULL;
    if (has_tokens && (!topk_idx || !is_token_in_rank || !expert_slot || !rank_slot))
        return EP_ERR_NULL;
    if (!aligned(topk_idx, 8) || !aligned(num_tokens_per_rank, 4) ||
        !aligned(num_tokens_per_expert, 4) || !aligned(expert_slot, 4) || !aligned(rank_slot, 4) ||
        !aligned(expert_offset, 4) || !aligned(status, 4) || !aligned(workspace, 16))
        return EP_ERR_ALIGN;
    ep::LayoutPlan plan;
    ep::plan_layout(*s, &plan);
    const size_t need = ep::layout_dispatch_workspace(*s, plan);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return EP_ERR_WORKSPACE;
    if (has_tokens) {
        if (!x || !recv_x || !recv_src_idx)
            return EP_ERR_NULL;
        if (s->use_fp8 && !recv_scales)
            return EP_ERR_NULL;
        if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(recv_scales, 4) ||
            !aligned(recv_src_idx, 4))
            return EP_ERR_ALIGN;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    // up to 256 tokens one kernel; up to 1,024 the layout's count kernel and
    // then one kernel for the rest; above that the layout's local ranking
    // and the pack that adds each token's prefix over the earlier blocks
    const int N = s->num_tokens;
    int32_t *ws = static_cast<int32_t *>(workspace);
    hipError_t err;
    if (N <= ep::kFusedMaxTokens) {
        err = ep::launch_layout_dispatch(*s, plan, nullptr, x, topk_idx, num_tokens_per_rank,
                                         num_tokens_per_expert, is_token_in_rank, expert_slot,
                                         rank_slot, expert_offset, recv_x, recv_scales,
                                         recv_src_idx, status, st);
    } else if (N <= ep::kFusedCountedMaxTokens) {
        err = ep::launch_layout_count(*s, plan, topk_idx, ws, st);
        if (err == hipSuccess)
            err = ep::launch_layout_dispatch(*s, plan, ws, x, topk_idx, num_tokens_per_rank,
                                             num_tokens_per_expert, is_token_in_rank, expert_slot,
                                             rank_slot, expert_offset, recv_x, recv_scales,
                                             recv_src_idx, status, st);
    } else {
        const ep::LocalWorkspace lw = ep::local_workspace(workspace, plan, *s);
        err = ep::launch_layout_local(*s, plan, topk_idx, lw, status, st);
        if (err == hipSuccess)
            err = ep::launch_dispatch_local(*s, plan, lw, x, topk_idx, num_tokens_per_rank,
                                            num_tokens_per_expert, is_token_in_rank, expert_slot,
                                            rank_slot, expert_offset, recv_x, recv_scales,
                                            recv_src_idx, status, st);
    }
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_combine(const ep_shape *s, const uint16_t *expert_out, const int64_t *topk_idx,
               const float *topk_weights, const int32_t *expert_slot, const uint16_t *bias,
               uint16_t *combined_x, uint32_t *status, void *stream)
{
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    if (s->num_tokens == 0)
        return EP_OK;
    if (!expert_out || !topk_idx || !topk_weights || !expert_slot || !combined_x)
        return EP_ERR_NULL;
    if (!aligned(expert_out, 16) || !aligned(combined_x, 16) || !aligned(bias, 16) ||
        !aligned(topk_idx, 8) || !aligned(topk_weights, 4) || !aligned(expert_slot, 4) ||
        !aligned(status, 4))
        return EP_ERR_ALIGN;
    const hipError_t err =
        ep::launch_combine(*s, expert_out, topk_idx, topk_weights, expert_slot, bias, combined_x,
                           status, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_dispatch_expand(const ep_shape *s, const uint16_t *x, const int64_t *topk_idx,
                       const int32_t *expert_slot, const int32_t *expert_offset,
                       const int32_t *num_tokens_per_expert, void *recv_x, void *recv_scales,
                       int32_t *recv_src_idx, uint32_t *status, void *stream)
{
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    // the padding rows are written even without tokens (every queue is then
    // empty, so nothing is), but the offsets and counts are always read
    if (!expert_offset || !num_tokens_per_expert || !recv_x || !recv_src_idx)
        return EP_ERR_NULL;
    if (s->num_tokens > 0 && (!x || !topk_idx || !expert_slot))
        return EP_ERR_NULL;
    if (s->use_fp8 && !recv_scales)
        return EP_ERR_NULL;
    if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 8) ||
        !aligned(expert_slot, 4) || !aligned(expert_offset, 4) ||
        !aligned(num_tokens_per_expert, 4) || !aligned(recv_scales, 4) ||
        !aligned(recv_src_idx, 4) || !aligned(status, 4))
        return EP_ERR_ALIGN;
    const hipError_t err = ep::launch_dispatch_expand(
        *s, x, topk_idx, expert_slot, expert_offset, num_tokens_per_expert, recv_x, recv_scales,
        recv_src_idx, status, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_combine_expand(const ep_shape *s, const uint16_t *expert_out, const int64_t *topk_idx,
                      const float *topk_weights, const int32_t *expert_slot,
                      const int32_t *expert_offset, const uint16_t *bias, uint16_t *combined_x,
                      uint32_t *status, void *stream)
{
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    if (s->num_tokens == 0)
        return EP_OK;
    if (!expert_out || !topk_idx || !topk_weights || !expert_slot || !expert_offset || !combined_x)
        return EP_ERR_NULL;
    if (!aligned(expert_out, 16) || !aligned(combined_x, 16) || !aligned(bias, 16) ||
        !aligned(topk_idx, 8) || !aligned(topk_weights, 4) || !aligned(expert_slot, 4) ||
        !aligned(expert_offset, 4) || !aligned(status, 4))
        return EP_ERR_ALIGN;
    const hipError_t err =
        ep::launch_combine_expand(*s, expert_out, topk_idx, topk_weights, expert_slot,
                                  expert_offset, bias, combined_x, status,
                                  static_cast<hipStream_t>(stream));
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_dispatch_normal(const ep_shape *s, const uint16_t *x, const int64_t *topk_idx,
                       const float *topk_weights, const int32_t *rank_slot, void *recv_x,
                       void *recv_scales, int64_t *recv_topk_idx, float *recv_topk_weights,
                       int32_t *recv_src_idx, uint32_t *status, void *stream)
{
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    if (s->num_tokens == 0)
        return EP_OK;
    if (!x || !topk_idx || !rank_slot || !recv_x || !recv_topk_idx || !recv_src_idx)
        return EP_ERR_NULL;
    if (s->use_fp8 && !recv_scales)
        return EP_ERR_NULL;
    if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 8) ||
        !aligned(topk_weights, 4) || !aligned(rank_slot, 4) || !aligned(recv_scales, 4) ||
        !aligned(recv_topk_idx, 8) || !aligned(recv_topk_weights, 4) ||
        !aligned(recv_src_idx, 4) || !aligned(status, 4))
        return EP_ERR_ALIGN;
    const hipError_t err = ep::launch_dispatch_normal(
        *s, x, topk_idx, topk_weights, rank_slot, recv_x, recv_scales, recv_topk_idx,
        recv_topk_weights, recv_src_idx, status, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_combine_normal(const ep_shape *s, const uint16_t *x, const int32_t *rank_slot,
                      const float *recv_topk_weights, const uint16_t *bias,
                      uint16_t *combined_x, float *combined_topk_weights, uint32_t *status,
                      void *stream)
{
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    if (s->num_tokens == 0)
        return EP_OK;
    if (!x || !rank_slot || !combined_x)
        return EP_ERR_NULL;
    if (recv_topk_weights && !combined_topk_weights)
        return EP_ERR_NULL;
    if (!aligned(x, 16) || !aligned(combined_x, 16) || !aligned(bias, 16) ||
        !aligned(rank_slot, 4) || !aligned(recv_topk_weights, 4) ||
        !aligned(combined_topk_weights, 4) || !aligned(status, 4))
        return EP_ERR_ALIGN;
    const hipError_t err = ep::launch_combine_normal(*s, x, rank_slot, recv_topk_weights, bias,
                                                     combined_x, combined_topk_weights, status,
                                                     static_cast<hipStream_t>(stream));
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_logfmt_encode(const ep_shape *s, const uint16_t *expert_out, const int64_t *topk_idx,
                     const int32_t *expert_slot, uint8_t *codes, float *headers,
                     uint32_t *status, void *stream)
{
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    if (s->hidden % 128 != 0)
        return EP_ERR_SHAPE;
    if (s->num_tokens == 0)
        return EP_OK;
    if (!expert_out || !topk_idx || !expert_slot || !codes || !headers)
        return EP_ERR_NULL;
    if (!aligned(expert_out, 16) || !aligned(codes, 16) || !aligned(headers, 8) ||
        !aligned(topk_idx, 8) || !aligned(expert_slot, 4) || !aligned(status, 4))
        return EP_ERR_ALIGN;
    const hipError_t err = ep::launch_logfmt_encode(*s, expert_out, topk_idx, expert_slot, codes,
                                                    headers, status, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_combine_logfmt(const ep_shape *s, const uint8_t *codes, const float *headers,
                      const int64_t *topk_idx, const float *topk_weights,
                      const int32_t *expert_slot, const uint16_t *bias, uint16_t *combined_x,
                      uint32_t *status, void *stream)
{
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    if (s->hidden % 128 != 0)
        return EP_ERR_SHAPE;
    if (s->num_tokens == 0)
        return EP_OK;
    if (!codes || !headers || !topk_idx || !topk_weights || !expert_slot || !combined_x)
        return EP_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(headers, 8) || !aligned(combined_x, 16) ||
        !aligned(bias, 16) || !aligned(topk_idx, 8) || !aligned(topk_weights, 4) ||
        !aligned(expert_slot, 4) || !aligned(status, 4))
        return EP_ERR_ALIGN;
    const hipError_t err =
        ep::launch_combine_logfmt(*s, codes, headers, topk_idx, topk_weights, expert_slot, bias,
                                  combined_x, status, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_group_limited_topk(const ep_shape *s, int32_t num_groups, int32_t topk_groups,
                          int32_t rule, const float *scores, int64_t *topk_idx,
                          float *topk_weights, void *stream)
{
    const int rc = check_shape(s);
    if (rc != EP_OK)
        return rc;
    const int32_t E = s->num_experts, K = s->num_topk;
    if (num_groups > EP_MAX_GROUPS)
        return EP_ERR_UNSUPPORTED;
    if (num_groups < 1 || E % num_groups != 0 || topk_groups < 1 || topk_groups > num_groups ||
        (int64_t)K > (int64_t)topk_groups * (E / num_groups))
        return EP_ERR_SHAPE;
    if (rule != EP_GATE_MAX_SOFTMAX && rule != EP_GATE_SUM_SIGMOID)
        return EP_ERR_SHAPE;
    if (s->num_tokens == 0)
        return EP_OK;
    if (!scores || !topk_idx)
        return EP_ERR_NULL;
    if (!aligned(scores, 4) || !aligned(topk_idx, 8) || !aligned(topk_weights, 4))
        return EP_ERR_ALIGN;
    const hipError_t err = ep::launch_gate(*s, num_groups, topk_groups, rule, scores, topk_idx,
                                           topk_weights, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

} // extern "C"
