// Combine: gather each token's k expert-output rows back to token order as a
// router-weighted sum.
//
// Combine is the second half of an MoE layer's exchange: the expert outputs
// go back to the positions their tokens came from ("Inside the Nebius +
// PyTorch DeepSeek V3 recipe", section "Mixture-of-experts and wide expert
// parallelism"). Here that is
//   out[t] = bf16_rne( sum_{j = 0..k-1, pos[t,j] >= 0} w[t,j] * y[pos[t,j]] )
// accumulated in fp32 in the fixed slot order j = 0, 1, ..., k-1 (one fused
// multiply-add per term, starting from +0), so the result does not depend on
// scheduling.
//
// Work decomposition as in dispatch: every wavefront is one (token, 1 KiB
// column slice) work item, two items to a workgroup. It fetches the token's
// row indices and weights with scalar loads, issues the 16-byte loads of up
// to 8 slot rows back to back (8 independent reads in flight per lane), then
// accumulates them in slot order and writes the bf16 slice with one 16-byte
// store per lane.
//
// Combine is the last reader of the expert outputs, so those rows are read
// with non-temporal loads, and the token rows are written with non-temporal
// stores: neither needs to stay in L2 or the last-level cache. Measured on
// MI355X in a dispatch -> FP8 dispatch -> combine sequence, this cut the
// sequence from about 298 us to 274 us at T=4096, H=7168, k=8: the streamed
// reads no longer evict (and so write back) the dirty lines the dispatches
// left in the last-level cache.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? ((u >> 16) | 0x40u) : r;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// acc += w * row (one fused multiply-add per channel) when `use`, else acc is
// left exactly as it is (a select, so that the loads of every slot still
// issue together; adding a zero product instead would turn an acc of -0 into
// +0).
__device__ __forceinline__ void accumulate(float (&acc)[8], bool use, float w, const u32x4& r) {
  const float f[8] = {bf16_lo(r.x), bf16_hi(r.x), bf16_lo(r.y), bf16_hi(r.y),
                      bf16_lo(r.z), bf16_hi(r.z), bf16_lo(r.w), bf16_hi(r.w)};
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = use ? __builtin_fmaf(w, f[i], acc[i]) : acc[i];
}

// kWeighted = false sums the rows unweighted (weight 1, w unused): the final
// reduction of the rank-deduplicated exchange, over the per-rank partial rows
// of each token in ascending rank order. kBatch: rows loaded together (8, or
// the power of two that covers a smaller topk, so that no load is issued for
// slots past topk: at top-2 the 8-row batch repeated the last row six times
// and ran at 46% of 8 TB/s).
template <bool kWeighted, int kBatch>
__global__ __launch_bounds__(64 * kCombineWaves) void combine_kernel(
    const u32x4* __restrict__ y, const float* __restrict__ w, const int32_t* __restrict__ pos,
    u32x4* __restrict__ out, int num_tokens, int topk, int nvec, int slices, int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int nitems = num_tokens * slices;
  for (int item = blockIdx.x * kCombineWaves + wave_index(); item < nitems;
       item += gridDim.x * kCombineWaves) {
    const int t = item / slices;
    const int v = (item - t * slices) * 64 + lane;
    const bool active = v < nvec;
    // Every load below is unconditional so the compiler issues them back to
    // back: lanes past the row end read its last piece, and slots that do not
    // contribute read a valid row (padding slots past k reuse slot k-1's row,
    // so they cost no extra HBM traffic); their data is never used.
    const size_t vc = active ? v : nvec - 1;
    const int32_t* pt = pos + static_cast<size_t>(t) * topk;
    const float* wt = kWeighted ? w + static_cast<size_t>(t) * topk : nullptr;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < topk; j0 += kBatch) {
      int p[kBatch];
      float wj[kBatch];
      bool use[kBatch];
      if (j0 + kBatch <= topk) {   // full batch: contiguous, merges into wide scalar loads
#pragma unroll
        for (int jj = 0; jj < kBatch; ++jj) {
          p[jj] = pt[j0 + jj];
          wj[jj] = kWeighted ? wt[j0 + jj] : 1.0f;
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < kBatch; ++jj) {
          const int j = j0 + jj < topk ? j0 + jj : topk - 1;
          p[jj] = pt[j];
          wj[jj] = kWeighted ? wt[j] : 1.0f;
        }
      }
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) {
        const bool row_ok = p[jj] >= 0 && p[jj] < rows;
        use[jj] = j0 + jj < topk && row_ok;
        p[jj] = row_ok ? p[jj] : 0;
      }
      u32x4 r[kBatch];
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj)
        r[jj] = __builtin_nontemporal_load(&y[static_cast<size_t>(p[jj]) * nvec + vc]);
      // Unused slots leave acc untouched; selecting instead of branching keeps
      // the loads above in one batch.
#pragma unroll
      for (int jj = 0; jj < kBatch; ++jj) accumulate(acc, use[jj], wj[jj], r[jj]);
    }
    if (active) {
      u32x4 o;
      o.x = pack_bf16(acc[0], acc[1]);
      o.y = pack_bf16(acc[2], acc[3]);
      o.z = pack_bf16(acc[4], acc[5]);
      o.w = pack_bf16(acc[6], acc[7]);
      __builtin_nontemporal_store(o, &out[static_cast<size_t>(t) * nvec + v]);
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* d_y, int64_t rows, const float* d_w, const int32_t* d_pos,
                          void* d_out, int num_tokens, int topk, int hidden, int max_blocks,
                          hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int nvec = hidden / 8;
  const int slices = (nvec + 63) / 64;
  const dim3 grid = wave_grid(int64_t(num_tokens) * slices, kCombineWaves, max_blocks);
  const dim3 block(64 * kCombineWaves);
  const u32x4* y = static_cast<const u32x4*>(d_y);
  u32x4* out = static_cast<u32x4*>(d_out);
  if (topk <= 2)
    hipLaunchKernelGGL((combine_kernel<true, 2>), grid, block, 0, stream, y, d_w, d_pos, out,
                       num_tokens, topk, nvec, slices, rows);
  else if (topk <= 4)
    hipLaunchKernelGGL((combine_kernel<true, 4>), grid, block, 0, stream, y, d_w, d_pos, out,
                       num_tokens, topk, nvec, slices, rows);
  else
    hipLaunchKernelGGL((combine_kernel<true, kSlotBatch>), grid, block, 0, stream, y, d_w, d_pos,
                       out, num_tokens, topk, nvec, slices, rows);
  return hipGetLastError();
}

hipError_t launch_combine_ranks(const void* d_y, int64_t rows, const int32_t* d_rank_pos,
                                void* d_out, int num_tokens, int num_ranks, int hidden,
                                int max_blocks, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int nvec = hidden / 8;
  const int slices = (nvec + 63) / 64;
  const dim3 grid = wave_grid(int64_t(num_tokens) * slices, kCombineWaves, max_blocks);
  const dim3 block(64 * kCombineWaves);
  const u32x4* y = static_cast<const u32x4*>(d_y);
  u32x4* out = static_cast<u32x4*>(d_out);
  // The rows of one token are its R per-rank partial sums: the same batch
  // sizes as the weighted combine, by R. Same-box A/B at T=4096, H=7168,
  // top-8 of 256, us, 8-row batch against the matched one: R=2 44.6 -> 30.3,
  // R=4 51.2 -> 44.9, R=8 unchanged (59.5); T=8192, H=4096, top-2 of 8, R=2
  // 49.2 -> 29.5.
  if (num_ranks <= 2)
    hipLaunchKernelGGL((combine_kernel<false, 2>), grid, block, 0, stream, y, nullptr, d_rank_pos,
                       out, num_tokens, num_ranks, nvec, slices, rows);
  else if (num_ranks <= 4)
    hipLaunchKernelGGL((combine_kernel<false, 4>), grid, block, 0, stream, y, nullptr, d_rank_pos,
                       out, num_tokens, num_ranks, nvec, slices, rows);
  else
    hipLaunchKernelGGL((combine_kernel<false, kSlotBatch>), grid, block, 0, stream, y, nullptr,
                       d_rank_pos, out, num_tokens, num_ranks, nvec, slices, rows);
  return hipGetLastError();
}

}  // namespace moe
