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
constexpr int kLayoutSteps = 2;                     // 64-slot steps per wavefront
constexpr int kLayoutChunk = kLayoutThreads * kLayoutSteps;  // 1024 slots per workgroup
// Up to this many slots one workgroup lays out everything in one launch.
constexpr int kLayoutSingleSteps = 8;
constexpr int kLayoutSingleChunk = kLayoutThreads * kLayoutSingleSteps;  // 4096 slots

// Up to this many workgroups the expert layout is one launch in which each
// workgroup counts every slot itself (no histogram kernel before it). Each
// workgroup's count costs about 0.18 us per 1024-slot chunk (the rate of LDS
// atomics on one compute unit), the second launch about 2-3 us, so one
// launch pays up to here: top-8 of 256, same box, one launch / two, us:
// 8 chunks 6.75 / 9.66, 16 chunks 8.26 / 8.44, 24 chunks (T=4096, top-6 of
// 64) 9.15 / 9.66, 32 chunks 11.2 / 9.07, 64 chunks 17.2 / 10.2.
constexpr int kLayoutFusedBlocks = 24;

inline int layout_blocks(int64_t slots) {
  int64_t b = (slots + kLayoutChunk - 1) / kLayoutChunk;
  return b < 1 ? 1 : (int)b;
}

// Payload kernels: every wavefront is one independent work item, a
// (token, column slice) pair; a workgroup is kItemWaves such items (combine:
// kCombineWaves). (The standard bf16 dispatch instead gives each item a
// workgroup whose wavefronts share the item's slots.) A workgroup cap is
// counted in workgroups of kItemWaves; every kernel keeps that wavefront count.
constexpr int kItemWaves = 4;
constexpr int kSlotBatch = 8;   // row indices fetched (and rows read) per batch
// Combine's workgroups hold two items: same-box A/B at T=4096, H=7168,
// k=8 (two runs each, back to back over rotating buffers), combine 91.8 and
// 92.6 us at four wavefronts per workgroup, 89.1 and 89.1 at two, 88.9 and
// 89.9 at one.
constexpr int kCombineWaves = 2;

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
  // Row lists of the blocked bf16 dispatch (null when a caller has none):
  // [dispatch_order_entries(T_max, k)] (row, token) pairs, block b's at b * bs,
  // (-1, -1) past the block's rows.
  int2* order;
};

// Blocked bf16 dispatch. The slots are cut into dispatch blocks of
// block_chunks layout chunks (bs = block_chunks * kLayoutChunk slots); the
// layout lists each block's rows in ascending row order, and the dispatch
// gives block b to the workgroups of XCD slot b % kXcds, which walk the list:
// every wavefront copies one 1 KiB slice of x[token] to out[row]. The rows a
// block writes at once are then a run of consecutive rows per expert, and the
// x rows of its tokens are read once from HBM (prefetched in token order) and
// re-read from that XCD's L2.
constexpr int kXcds = MOE_EP_XCDS;
// x bytes a dispatch block's tokens may hold: 7/8 of one XCD's 4 MiB L2, so
// that the tail of one block and the head of the next still fit it. Blocks
// of the full 4 MiB were slower wherever a slot walked several of them
// (same box, x from HBM, us, blocks of 4 MiB / 2 MiB: T=16384, H=4096,
// top-8 of 128, Zipf routing 203.4 / 194; T=4096, H=4096, 51.8 / 47.8).
constexpr int64_t kBlockXBytes = int64_t(7) << 19;

// The blocked form re-reads each token's x once per row from the cache
// hierarchy, which holds while the batch's x fits well inside the 256 MB
// last-level cache; its early burst of x only while x takes little more than
// half of it. Same box, x from HBM, us, blocked with the burst / blocked
// without it / per-slot form: T=8192, H=7168 (x 117 MB) 181 / 192 / 199;
// T=16384, H=4096 (134 MB) 196-203 / 206-208 / 215 (with Zipf routing
// 195-197 / 190-191 / 205); T=12288, H=7168 (176 MB) 369 / 287 / 302;
// T=16384, H=7168 (235 MB) 480 / 419 / 393; T=32768, H=4096 (268 MB) 531 /
// 467-472 / 437.
constexpr int64_t kBlockedMaxXBytes = int64_t(192) << 20;
constexpr int64_t kPrefetchMaxXBytes = int64_t(144) << 20;

// Layout chunks per dispatch block for num_tokens x topk slots of `hidden`
// bf16 channels, or 0 when the blocked form is not used: fewer than one block
// per XCD slot, one chunk's tokens already holding more than kBlockXBytes of
// x, or the batch's x more than kBlockedMaxXBytes. A power of two (the dispatch finds a row's block with a shift) with
// at most kBlockXBytes of x and at most chunks / kXcds chunks, chosen so that
// the busiest XCD slot gets as few chunks as possible (blocks b, b + 8, ...
// share a slot: with 24 chunks, blocks of 2 would give four slots 4 chunks
// and four slots 2), the larger block on a tie.
inline int dispatch_block_chunks(int num_tokens, int topk, int hidden) {
  const int64_t slots = int64_t(num_tokens) * topk;
  const int64_t chunks = (slots + kLayoutChunk - 1) / kLayoutChunk;
  if (topk <= 0 || hidden <= 0 || chunks < kXcds) return 0;
  if (int64_t(num_tokens) * 2 * hidden > kBlockedMaxXBytes) return 0;
  const int64_t chunk_x = int64_t(kLayoutChunk) * 2 * hidden / topk;
  if (chunk_x > kBlockXBytes) return 0;
  int64_t best = 1, best_load = (chunks + kXcds - 1) / kXcds;
  for (int64_t m = 2; m * chunk_x <= kBlockXBytes && m <= chunks / kXcds; m *= 2) {
    const int64_t blocks = (chunks + m - 1) / m;
    const int64_t load = (blocks + kXcds - 1) / kXcds * m;
    if (load <= best_load) {
      best = m;
      best_load = load;
    }
  }
  return static_cast<int>(best);
}

// Unsigned division by a divisor fixed at launch (Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, n / d equals
// (mulhi(n, m) + n) >> l for every n < 2^31 (the sum then fits in 32 bits).
// The kernels that use it do one multiply-high, one add and one shift per
// division instead of a division routine.
struct FastDiv {
  uint32_t mul;
  uint32_t shift;
};

inline FastDiv make_fast_div(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  return FastDiv{static_cast<uint32_t>(m), l};
}

__host__ __device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv d) {
  const uint32_t hi = static_cast<uint32_t>((static_cast<uint64_t>(n) * d.mul) >> 32);
  return (hi + n) >> d.shift;
}

// Entries of the order list for up to max_tokens x topk slots: every block
// holds bs entries, and the last block of any batch ends at most
// block_chunks - 1 <= chunks / kXcds chunks past the last slot.
inline int64_t dispatch_order_entries(int max_tokens, int topk) {
  const int64_t chunks = layout_blocks(int64_t(max_tokens) * topk);
  return (chunks + chunks / kXcds + 1) * kLayoutChunk;
}

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

// moe_dispatch_layout_noalloc: capacity of the static histogram array, in
// int32 entries (MOE_EP_NOALLOC_SCRATCH_BYTES).
constexpr size_t kNoallocScratchInts = MOE_EP_NOALLOC_SCRATCH_BYTES / sizeof(int32_t);

// Device address of this GPU's static histogram array (looked up on the first
// call on each device, with that device current).
hipError_t layout_scratch(int32_t** out);

// Histogram entries a layout of num_tokens x topk slots over num_experts
// needs (0 when one workgroup does it all).
size_t layout_scratch_ints(int num_tokens, int topk, int num_experts);

// Host-side launchers; each returns the hipError_t of its launches.
// block_chunks > 0 also writes a.order for the blocked bf16 dispatch
// (dispatch_block_chunks of the batch; needs more than 4096 slots).
hipError_t launch_layout(const int32_t* d_idx, int num_tokens, int topk, int num_experts,
                         int num_ranks, const LayoutArrays& a, hipStream_t stream,
                         int block_chunks = 0);

hipError_t launch_rank_layout(const int32_t* d_idx, int num_tokens, int topk, int num_experts,
                              int num_ranks, const RankArrays& a, hipStream_t stream);

// Dispatch of dtype (moe_dtype_t) through the table d_pos[T, k]. `rows` is
// the row count of the expert-major buffer; rows outside it are never read
// or written, whatever pos holds. `max_blocks` > 0 caps the grid (item_grid).
hipError_t launch_dispatch(int dtype, const void* d_x, const int32_t* d_pos, void* d_out,
                           void* d_scales, int64_t rows, int num_tokens, int topk, int hidden,
                           int max_blocks, hipStream_t stream);

// Blocked bf16 dispatch through the lists a layout with block_chunks wrote.
hipError_t launch_dispatch_blocks(const void* d_x, const int2* d_order, void* d_out, int64_t rows,
                                  int num_tokens, int topk, int hidden, int block_chunks,
                                  hipStream_t stream);

// bf16 dispatch of the rank-deduplicated layout, whose table has many -1
// slots: one wavefront per (token, slice) loops over the slots (where
// launch_dispatch gives every slot a wavefront of its own), and the
// wavefronts of slice 0 also write the receiver metadata d_recv_idx /
// d_recv_w [rows, topk] of the token's rows.
hipError_t launch_dispatch_ranks(const void* d_x, const int32_t* d_slot_row, void* d_out,
                                 int64_t rows, int num_tokens, int topk, int hidden,
                                 int max_blocks, const int32_t* d_idx, const float* d_w,
                                 int num_experts, int num_ranks, int32_t* d_recv_idx,
                                 float* d_recv_w, hipStream_t stream);

// Fixed-capacity (decode-time) layout and dispatch in one launch: rows
// [e*capacity, (e+1)*capacity) belong to expert e. Records d_pos [T, k],
// d_counts [E] and d_status [4] (invalid, placed, T, dropped).
hipError_t launch_dispatch_fixed(int dtype, const void* d_x, const int32_t* d_idx,
                                 int num_tokens, int topk, int num_experts, int capacity,
                                 int32_t* d_pos, int32_t* d_counts, int32_t* d_status,
                                 void* d_out, void* d_scales, int hidden, int max_blocks,
                                 hipStream_t stream);

// Standard (packed) layout and dispatch in one launch, for small batches: the
// same pos, src_idx, counts, offsets and status as launch_layout, and the
// same rows as launch_dispatch.
hipError_t launch_layout_dispatch(int dtype, const void* d_x, const int32_t* d_idx,
                                  int num_tokens, int topk, int num_experts, int num_ranks,
                                  const LayoutArrays& a, void* d_out, void* d_scales, int hidden,
                                  int max_blocks, hipStream_t stream);

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

// Cross-lane reductions with DPP (GFX9 encoding): two quad permutations, then
// the half-row and row mirrors, leave every lane of a 16-lane row holding the
// row's reduction; four readlanes combine the rows into a scalar.
constexpr int kDppQuadSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within each 8
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i within each 16

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t dpp_umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Maximum of v over the wavefront, as a scalar.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_umax(v, dpp_u32<kDppQuadSwap1>(v));
  v = dpp_umax(v, dpp_u32<kDppQuadSwap2>(v));
  v = dpp_umax(v, dpp_u32<kDppRowHalfMirror>(v));
  v = dpp_umax(v, dpp_u32<kDppRowMirror>(v));
  return dpp_umax(dpp_umax(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
                  dpp_umax(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Sum of v over the wavefront (modulo 2^32), as a scalar.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u32<kDppQuadSwap1>(v);
  v += dpp_u32<kDppQuadSwap2>(v);
  v += dpp_u32<kDppRowHalfMirror>(v);
  v += dpp_u32<kDppRowMirror>(v);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 0)) +
         static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 16)) +
         static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 32)) +
         static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 48));
}

// Grid for num_items wavefront work items: one workgroup per kItemWaves
// items, or at most max_blocks workgroups (> 0), whose wavefronts then loop.
inline dim3 item_grid(int64_t num_items, int max_blocks) {
  int64_t blocks = (num_items + kItemWaves - 1) / kItemWaves;
  if (max_blocks > 0 && blocks > max_blocks) blocks = max_blocks;
  return dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks));
}

// Grid for num_items wavefront work items in workgroups of `waves`
// wavefronts. A cap of max_blocks (> 0) workgroups of kItemWaves keeps its
// wavefront count: at most max_blocks * kItemWaves / waves workgroups.
inline dim3 wave_grid(int64_t num_items, int waves, int max_blocks) {
  int64_t blocks = (num_items + waves - 1) / waves;
  if (max_blocks > 0) {
    int64_t cap = int64_t(max_blocks) * kItemWaves / waves;
    if (cap < 1) cap = 1;
    if (blocks > cap) blocks = cap;
  }
  return dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks));
}

hipError_t launch_combine_ranks(const void* d_y, int64_t rows, const int32_t* d_rank_pos,
                                void* d_out, int num_tokens, int num_ranks, int hidden,
                                int max_blocks, hipStream_t stream);

}  // namespace moe
