// Router: each token's top-k experts and their combine weights.
//
// The pages have each token activate the top-k of the experts ("Inside the
// Nebius + PyTorch DeepSeek V3 recipe", section "Mixture-of-experts and wide
// expert parallelism"; 8 of 256 for DeepSeek V3). Selection here: the k
// largest logits in descending order, equal logits to the lower expert id,
// -0 equal to +0. Weights over the selected experts: softmax, or sigmoid
// scores divided by their sum (the DeepSeek-V3-style gate, no extra scale).
//
// One wavefront per token, no LDS and no barrier. Lane l holds the logits of
// experts l, l+64, l+128, ... as unsigned order keys (the bit pattern mapped
// so that unsigned order is numeric order, -0 folded onto +0). Each of the k
// rounds: every lane takes its best live key (the lower id on ties), the
// wavefront maximum is formed with four DPP steps inside each 16-lane row
// and four readlanes across rows (so it is a scalar), and the expert holding
// it is read from the one lane a ballot finds, or, when several lanes tie,
// the lowest expert id among them by a second such reduction. The winner's
// owner lane retires it, and lane `round` keeps it. Lanes 0..k-1 then
// compute the weights in fp32 and a DPP row sum adds them in a fixed order.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);   // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Sum of lanes 0..31 (the rest hold 0), in a fixed order, as a scalar (DPP
// row sums as in wave_sum_u32, then rows 0 and 1).
__device__ __forceinline__ float sum_lanes_0_31(float v) {
  v += __uint_as_float(dpp_u32<kDppQuadSwap1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppQuadSwap2>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppRowHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppRowMirror>(__float_as_uint(v)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
}

// kPer: logits per lane (experts <= 64 * kPer).
template <int kPer>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    int num_tokens, int num_experts, int topk,
                                                    int sigmoid, int32_t* __restrict__ idx,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  for (int t = blockIdx.x * 4 + wave_index(); t < num_tokens; t += gridDim.x * 4) {
    const float* row = logits + static_cast<size_t>(t) * num_experts;
    uint32_t key[kPer];
    bool live[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = i * 64 + lane;
      live[i] = e < num_experts;
      key[i] = live[i] ? order_bits(row[e]) : 0u;
    }
    float sel_v = 0.0f;
    int sel_e = 0;
    for (int r = 0; r < topk; ++r) {
      bool have = false;
      uint32_t best = 0u;
      int bi = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (live[i] && (!have || key[i] > best)) {
          best = key[i];
          bi = i;
          have = true;
        }
      }
      const uint32_t top = wave_max_u32(have ? best : 0u);
      // Lowest expert id holding the maximum: the maximum of ~id over the
      // lanes that hold it (at least one does).
      // Usually one lane holds the maximum, and a ballot names it; only a tie
      // across lanes needs the second reduction. Same-box A/B against the
      // reduction every round, us: T=16384, top-8 of 128 14.9 -> 12.9; T=4096,
      // top-8 of 256 8.0 -> 7.7, top-6 of 64 4.3 -> 3.9, top-2 of 8 2.8 -> 2.7;
      // T=128 unchanged (4.8).
      const bool tied = have && best == top;
      const uint64_t tmask = __ballot(tied);
      int e;
      if (__popcll(tmask) == 1) {
        const int src = static_cast<int>(__builtin_ctzll(tmask));
        e = __builtin_amdgcn_readlane(bi * 64 + lane, src);
      } else {
        e = static_cast<int>(~wave_max_u32(tied ? ~static_cast<uint32_t>(bi * 64 + lane) : 0u));
      }
      if (lane == (e & 63)) {
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          if (i == (e >> 6)) live[i] = false;
      }
      if (lane == r) {
        sel_v = from_order_bits(top);
        sel_e = e;
      }
    }
    const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_v), 0));
    float z = 0.0f;
    if (lane < topk) z = sigmoid ? 1.0f / (1.0f + expf(-sel_v)) : expf(sel_v - top);
    const float sum = sum_lanes_0_31(z);
    if (lane < topk) {
      idx[static_cast<size_t>(t) * topk + lane] = sel_e;
      w[static_cast<size_t>(t) * topk + lane] = z / sum;
    }
  }
}

}  // namespace

hipError_t launch_route(const float* d_logits, int num_tokens, int num_experts, int topk,
                        int score, int32_t* d_idx, float* d_w, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const dim3 grid((num_tokens + 3) / 4), block(256);
  const int sig = score == MOE_SCORE_SIGMOID ? 1 : 0;
  if (num_experts <= 64)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, stream, d_logits, num_tokens, num_experts,
                       topk, sig, d_idx, d_w);
  else if (num_experts <= 128)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, stream, d_logits, num_tokens, num_experts,
                       topk, sig, d_idx, d_w);
  else if (num_experts <= 256)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, stream, d_logits, num_tokens, num_experts,
                       topk, sig, d_idx, d_w);
  else if (num_experts <= 512)
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, stream, d_logits, num_tokens, num_experts,
                       topk, sig, d_idx, d_w);
  else
    hipLaunchKernelGGL(route_kernel<16>, grid, block, 0, stream, d_logits, num_tokens, num_experts,
                       topk, sig, d_idx, d_w);
  return hipGetLastError();
}

}  // namespace moe
