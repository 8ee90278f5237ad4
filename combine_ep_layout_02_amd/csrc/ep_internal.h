// ep_internal.h -- launchers shared between the C-ABI host code and the
// kernel translation units of libep_mi355x.so.  Host code validates every
// argument before it calls a launcher; launchers only size grids and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

// ---- dispatch layout ---------------------------------------------------
// The layout splits tokens into blocks of `tokens_per_block` (256) and runs
// two kernels: a per-block histogram (skipped when one block covers every
// token) and a pass that adds the histograms of earlier blocks to each
// block's local ranking.
struct LayoutPlan {
    int tokens_per_block;   // T
    int num_blocks;         // B = ceil(N / T), at least 1
    int hist_stride;        // ints per histogram row: round_up(E + R, 4)
    size_t lds_bytes;       // dynamic LDS of the assign kernel
    size_t workspace_bytes; // B * hist_stride * 4 when B > 1, else 0
};

// Returns false when the assign kernel's LDS does not fit in 64 KiB.
bool plan_layout(const ep_shape &s, LayoutPlan *plan);

hipError_t launch_layout(const ep_shape &s, const LayoutPlan &plan, const int64_t *topk_idx,
                         int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                         uint8_t *is_token_in_rank, int32_t *expert_slot, int32_t *rank_slot,
                         int32_t *expert_offset, int32_t *workspace, uint32_t *status,
                         hipStream_t stream);

// Expert alignment of the expand layout (1 when the shape sets none).
inline int32_t expert_alignment(const ep_shape &s)
{
    return s.expert_alignment > 1 ? s.expert_alignment : 1;
}

// Rows of the expand-layout buffer: the valid entries (at most M * K) plus at
// most A - 1 padding rows per expert.
inline int64_t expand_rows(const ep_shape &s)
{
    return (int64_t)s.num_max_dispatch_tokens_per_rank * s.num_topk +
           (int64_t)s.num_experts * (expert_alignment(s) - 1);
}

// ---- dispatch pack -------------------------------------------------------
hipError_t launch_dispatch(const ep_shape &s, const uint16_t *x, const int64_t *topk_idx,
                           const int32_t *expert_slot, void *recv_x, void *recv_scales,
                           int32_t *recv_src_idx, uint32_t *status, hipStream_t stream);

// The layout's first kernel alone: one histogram row per count block into
// `workspace` (nothing when plan.num_blocks == 1).
hipError_t launch_layout_count(const ep_shape &s, const LayoutPlan &plan, const int64_t *topk_idx,
                               int32_t *workspace, hipStream_t stream);

// Layout and per-expert pack in one launch: the same outputs as
// launch_layout followed by launch_dispatch.  Up to kFusedMaxTokens tokens
// (one count block) it is the only launch and `hist` is null; up to
// kFusedCountedMaxTokens it follows launch_layout_count, with `hist` = that
// workspace.  Larger batches take launch_layout and launch_dispatch, which
// measured faster there: the fused blocks' counting then costs more than the
// layout's second kernel.
constexpr int kFusedMaxTokens = 256;
constexpr int kFusedCountedMaxTokens = 1024;

// ep_layout_dispatch above kFusedCountedMaxTokens: the layout ranks each
// 256-token block on its own (launch_layout_local), then the pack adds each
// token's prefix over the earlier blocks (launch_dispatch_local).  Workspace:
// the histogram rows [B][hist_stride], then local slots and local rank slots
// [N][K] each.
struct LocalWorkspace {
    int32_t *hist;       // [B][hist_stride]
    int32_t *local_slot; // [N][K]
    int32_t *local_rank; // [N][K]
};

inline LocalWorkspace local_workspace(void *ws, const LayoutPlan &plan, const ep_shape &s)
{
    LocalWorkspace w;
    w.hist = static_cast<int32_t *>(ws);
    w.local_slot = w.hist + (size_t)plan.num_blocks * plan.hist_stride;
    w.local_rank = w.local_slot + (size_t)s.num_tokens * s.num_topk;
    return w;
}

inline size_t local_workspace_bytes(const LayoutPlan &plan, const ep_shape &s)
{
    return sizeof(int32_t) * ((size_t)plan.num_blocks * plan.hist_stride +
                              2 * (size_t)s.num_tokens * s.num_topk);
}

// Workspace bytes ep_layout_dispatch needs for a shape (at least what
// ep_layout needs).
inline size_t layout_dispatch_workspace(const ep_shape &s, const LayoutPlan &plan)
{
    return s.num_tokens <= kFusedCountedMaxTokens ? plan.workspace_bytes
                                                  : local_workspace_bytes(plan, s);
}

hipError_t launch_layout_local(const ep_shape &s, const LayoutPlan &plan, const int64_t *topk_idx,
                               const LocalWorkspace &ws, uint32_t *status, hipStream_t stream);

hipError_t launch_dispatch_local(const ep_shape &s, const LayoutPlan &plan, const LocalWorkspace &ws,
                                 const uint16_t *x, const int64_t *topk_idx,
                                 int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                                 uint8_t *is_token_in_rank, int32_t *expert_slot,
                                 int32_t *rank_slot, int32_t *expert_offset, void *recv_x,
                                 void *recv_scales, int32_t *recv_src_idx, uint32_t *status,
                                 hipStream_t stream);
hipError_t launch_layout_dispatch(const ep_shape &s, const LayoutPlan &plan, const int32_t *hist,
                                  const uint16_t *x, const int64_t *topk_idx,
                                  int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                                  uint8_t *is_token_in_rank, int32_t *expert_slot,
                                  int32_t *rank_slot, int32_t *expert_offset, void *recv_x,
                                  void *recv_scales, int32_t *recv_src_idx, uint32_t *status,
                                  hipStream_t stream);

hipError_t launch_dispatch_expand(const ep_shape &s, const uint16_t *x, const int64_t *topk_idx,
                                  const int32_t *expert_slot, const int32_t *expert_offset,
                                  const int32_t *num_tokens_per_expert, void *recv_x,
                                  void *recv_scales, int32_t *recv_src_idx, uint32_t *status,
                                  hipStream_t stream);

hipError_t launch_dispatch_normal(const ep_shape &s, const uint16_t *x, const int64_t *topk_idx,
                                  const float *topk_weights, const int32_t *rank_slot,
                                  void *recv_x, void *recv_scales, int64_t *recv_topk_idx,
                                  float *recv_topk_weights, int32_t *recv_src_idx,
                                  uint32_t *status, hipStream_t stream);

// ---- gating ----------------------------------------------------------------
hipError_t launch_gate(const ep_shape &s, int32_t num_groups, int32_t topk_groups, int32_t rule,
                       const float *scores, int64_t *topk_idx, float *topk_weights,
                       hipStream_t stream);

// ---- combine ---------------------------------------------------------------
hipError_t launch_combine(const ep_shape &s, const uint16_t *expert_out, const int64_t *topk_idx,
                          const float *topk_weights, const int32_t *expert_slot,
                          const uint16_t *bias, uint16_t *combined_x, uint32_t *status,
                          hipStream_t stream);

hipError_t launch_combine_expand(const ep_shape &s, const uint16_t *expert_out,
                                 const int64_t *topk_idx, const float *topk_weights,
                                 const int32_t *expert_slot, const int32_t *expert_offset,
                                 const uint16_t *bias, uint16_t *combined_x, uint32_t *status,
                                 hipStream_t stream);

hipError_t launch_logfmt_encode(const ep_shape &s, const uint16_t *expert_out,
                                const int64_t *topk_idx, const int32_t *expert_slot,
                                uint8_t *codes, float *headers, uint32_t *status,
                                hipStream_t stream);

hipError_t launch_combine_logfmt(const ep_shape &s, const uint8_t *codes, const float *headers,
                                 const int64_t *topk_idx, const float *topk_weights,
                                 const int32_t *expert_slot, const uint16_t *bias,
                                 uint16_t *combined_x, uint32_t *status, hipStream_t stream);

hipError_t launch_combine_normal(const ep_shape &s, const uint16_t *x, const int32_t *rank_slot,
                                 const float *recv_topk_weights, const uint16_t *bias,
                                 uint16_t *combined_x, float *combined_topk_weights,
                                 uint32_t *status, hipStream_t stream);

} // namespace ep
