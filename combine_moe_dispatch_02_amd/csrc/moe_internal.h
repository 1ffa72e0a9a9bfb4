// Internal declarations shared by the library's HIP sources (not installed).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "moe_ep.h"

namespace moe {

// Layout kernels: one workgroup owns a contiguous chunk of slots.
constexpr int kLayoutThreads = 512;                 // 8 wavefronts
constexpr int kLayoutWaves = kLayoutThreads / 64;
constexpr int kLayoutSteps = 4;                     // 64-slot steps per wavefront
constexpr int kLayoutChunk = kLayoutThreads * kLayoutSteps;  // 2048 slots per workgroup

inline int layout_blocks(int64_t slots) {
  int64_t b = (slots + kLayoutChunk - 1) / kLayoutChunk;
  return b < 1 ? 1 : (int)b;
}

// Payload kernels: every wavefront is one independent work item, a
// (token, column slice) pair; a workgroup is kItemWaves such items.
constexpr int kItemWaves = 4;
constexpr int kSlotBatch = 8;   // row indices fetched (and rows read) per batch

// Device views of the workspace regions.
struct LayoutArrays {
  int32_t* status;     // [MOE_EP_STATUS_WORDS]
  int32_t* counts_e;   // [E]
  int32_t* offsets_e;  // [E + 1]
  int32_t* counts_r;   // [R]
  int32_t* offsets_r;  // [R + 1]
  int32_t* hist;       // [layout_blocks(T_max * k)][E] per-workgroup histograms
  int32_t* pos;        // [T_max * k]
  int32_t* src_idx;    // [T_max * k]
};

// Workspace regions of the rank-deduplicated layout.
struct RankArrays {
  int32_t* status;    // [MOE_EP_STATUS_WORDS]
  int32_t* counts;    // [R] tokens per rank
  int32_t* offsets;   // [R + 1]
  int32_t* hist;      // [layout_blocks(T_max * k)][R]
  int32_t* slot_row;  // [T_max * k] row of the (token, rank) pair a slot opens, else -1
  int32_t* rank_pos;  // [T_max * R] row of each (token, rank) pair, -1 if none
  int32_t* src;       // [T_max * min(k, R)] token of each row
};

// Host-side launchers; each returns the hipError_t of its launches.
hipError_t launch_layout(const int32_t* d_idx, int num_tokens, int topk, int num_experts,
                         int num_ranks, const LayoutArrays& a, hipStream_t stream);

hipError_t launch_rank_layout(const int32_t* d_idx, int num_tokens, int topk, int num_experts,
                              int num_ranks, const RankArrays& a, hipStream_t stream);

// Dispatch of dtype (moe_dtype_t) through the table d_pos[T, k]. `rows` is
// the row count of the expert-major buffer; rows outside it are never read
// or written, whatever pos holds. `max_blocks` > 0 caps the grid (item_grid).
hipError_t launch_dispatch(int dtype, const void* d_x, const int32_t* d_pos, void* d_out,
                           void* d_scales, int64_t rows, int num_tokens, int topk, int hidden,
                           int max_blocks, hipStream_t stream);

// Fixed-capacity (decode-time) layout and dispatch in one launch: rows
// [e*capacity, (e+1)*capacity) belong to expert e. Records d_pos [T, k],
// d_counts [E] and d_status [4] (invalid, placed, T, dropped).
hipError_t launch_dispatch_fixed(int dtype, const void* d_x, const int32_t* d_idx,
                                 int num_tokens, int topk, int num_experts, int capacity,
                                 int32_t* d_pos, int32_t* d_counts, int32_t* d_status,
                                 void* d_out, void* d_scales, int hidden, int max_blocks,
                                 hipStream_t stream);

// Router: top-k of each token's logits and the weights (score: moe_score_t).
hipError_t launch_route(const float* d_logits, int num_tokens, int num_experts, int topk,
                        int score, int32_t* d_idx, float* d_w, hipStream_t stream);

hipError_t launch_combine(const void* d_y, int64_t rows, const float* d_w, const int32_t* d_pos,
                          void* d_out, int num_tokens, int topk, int hidden, int max_blocks,
                          hipStream_t stream);

// Index of the calling wavefront in its workgroup, as a wavefront-uniform
// (scalar) value, so that addresses derived from it use scalar loads.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// Grid for num_items wavefront work items: one workgroup per kItemWaves
// items, or at most max_blocks workgroups (> 0), whose wavefronts then loop.
inline dim3 item_grid(int64_t num_items, int max_blocks) {
  int64_t blocks = (num_items + kItemWaves - 1) / kItemWaves;
  if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
  return dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks));
}

hipError_t launch_rank_meta(const int32_t* d_idx, const float* d_w, const int32_t* d_slot_row,
                            int num_tokens, int topk, int num_experts, int num_ranks, int64_t rows,
                            int32_t* d_recv_idx, float* d_recv_w, hipStream_t stream);

hipError_t launch_combine_ranks(const void* d_y, int64_t rows, const int32_t* d_rank_pos,
                                void* d_out, int num_tokens, int num_ranks, int hidden,
                                int max_blocks, hipStream_t stream);

}  // namespace moe
