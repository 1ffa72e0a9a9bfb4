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
// experts l, l+64, l+128, ... as 64-bit keys: the high word is the logit's
// bit pattern mapped to an unsigned order (sign-magnitude -> biased), the low
// word ~expert, so the unsigned maximum is the largest logit and, among equal
// ones, the lowest id. Each of the k rounds takes the wavefront maximum of
// the keys (6 butterfly steps of two 32-bit shuffles), clears the winner's
// key in its owner lane, and leaves the winner with lane `round`. The weights
// are then computed by lanes 0..k-1 in fp32 and summed by a butterfly.
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, 64);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, 64);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
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
    uint64_t key[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = i * 64 + lane;
      key[i] = e < num_experts
                   ? (static_cast<uint64_t>(order_bits(row[e])) << 32) | (~static_cast<uint32_t>(e))
                   : 0ull;   // below every real key
    }
    float sel_v = 0.0f;
    int sel_e = 0;
    for (int r = 0; r < topk; ++r) {
      uint64_t best = key[0];
#pragma unroll
      for (int i = 1; i < kPer; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const int e = static_cast<int>(~static_cast<uint32_t>(best));
      if (lane == (e & 63)) {
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          if (i == (e >> 6)) key[i] = 0ull;
      }
      if (lane == r) {
        sel_v = from_order_bits(static_cast<uint32_t>(best >> 32));
        sel_e = e;
      }
    }
    const float top = __shfl(sel_v, 0, 64);   // the largest selected logit
    float z = 0.0f;
    if (lane < topk) z = sigmoid ? 1.0f / (1.0f + expf(-sel_v)) : expf(sel_v - top);
    const float sum = wave_sum(z);
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
