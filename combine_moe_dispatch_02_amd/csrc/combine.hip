// Combine: gather each token's k expert-output rows back to token order as a
// router-weighted sum.
//
// Per the pages, combine "returns expert outputs to their original positions"
// ("Inside the Nebius + PyTorch DeepSeek V3 recipe", section "Mixture-of-experts
// and wide expert parallelism"). Here that is
//   out[t] = bf16_rne( sum_{j = 0..k-1, pos[t,j] >= 0} w[t,j] * y[pos[t,j]] )
// accumulated in fp32 in the fixed slot order j = 0, 1, ..., k-1 (one fused
// multiply-add per term), so the result does not depend on scheduling.
//
// A workgroup owns whole tokens. Each lane owns 16-byte pieces of the output
// row; for every piece it issues the loads of up to 8 slots' rows before
// accumulating any of them, so each lane keeps 8 independent 16-byte reads in
// flight, and writes the bf16 result with one 16-byte store.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCombineThreads = 128;
constexpr int kSlotBatch = 8;

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

__device__ __forceinline__ void accumulate(float (&acc)[8], float w, const u32x4& r) {
  acc[0] = __builtin_fmaf(w, bf16_lo(r.x), acc[0]);
  acc[1] = __builtin_fmaf(w, bf16_hi(r.x), acc[1]);
  acc[2] = __builtin_fmaf(w, bf16_lo(r.y), acc[2]);
  acc[3] = __builtin_fmaf(w, bf16_hi(r.y), acc[3]);
  acc[4] = __builtin_fmaf(w, bf16_lo(r.z), acc[4]);
  acc[5] = __builtin_fmaf(w, bf16_hi(r.z), acc[5]);
  acc[6] = __builtin_fmaf(w, bf16_lo(r.w), acc[6]);
  acc[7] = __builtin_fmaf(w, bf16_hi(r.w), acc[7]);
}

template <int U>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const u32x4* __restrict__ y, const float* __restrict__ w, const int32_t* __restrict__ pos,
    u32x4* __restrict__ out, int num_tokens, int topk, int nvec, int64_t rows) {
  for (int t = blockIdx.x; t < num_tokens; t += gridDim.x) {
    const int32_t* pt = pos + static_cast<size_t>(t) * topk;
    const float* wt = w + static_cast<size_t>(t) * topk;
    for (int v0 = threadIdx.x; v0 < nvec; v0 += U * kCombineThreads) {
      float acc[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;

      for (int j0 = 0; j0 < topk; j0 += kSlotBatch) {
        u32x4 r[kSlotBatch][U];
        int p[kSlotBatch];
#pragma unroll
        for (int jj = 0; jj < kSlotBatch; ++jj) {
          p[jj] = j0 + jj < topk ? pt[j0 + jj] : -1;
          if (p[jj] >= rows) p[jj] = -1;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kCombineThreads;
            r[jj][u] = u32x4{0u, 0u, 0u, 0u};
            if (p[jj] >= 0 && v < nvec) r[jj][u] = y[static_cast<size_t>(p[jj]) * nvec + v];
          }
        }
#pragma unroll
        for (int jj = 0; jj < kSlotBatch; ++jj) {
          if (p[jj] < 0) continue;
          const float wj = wt[j0 + jj];
#pragma unroll
          for (int u = 0; u < U; ++u) accumulate(acc[u], wj, r[jj][u]);
        }
      }

#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * kCombineThreads;
        if (v < nvec) {
          u32x4 o;
          o.x = pack_bf16(acc[u][0], acc[u][1]);
          o.y = pack_bf16(acc[u][2], acc[u][3]);
          o.z = pack_bf16(acc[u][4], acc[u][5]);
          o.w = pack_bf16(acc[u][6], acc[u][7]);
          out[static_cast<size_t>(t) * nvec + v] = o;
        }
      }
    }
  }
}

template <int U>
hipError_t launch(const void* d_y, int64_t rows, const float* d_w, const int32_t* d_pos,
                  void* d_out, int num_tokens, int topk, int nvec, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel<U>, dim3(num_tokens), dim3(kCombineThreads), 0, stream,
                     static_cast<const u32x4*>(d_y), d_w, d_pos, static_cast<u32x4*>(d_out),
                     num_tokens, topk, nvec, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* d_y, int64_t rows, const float* d_w, const int32_t* d_pos,
                          void* d_out, int num_tokens, int topk, int hidden, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int nvec = hidden / 8;
  // Two 16-byte pieces per lane per pass keeps 2 x 8 row reads in flight
  // without spilling the accumulators.
  if (nvec <= kCombineThreads) return launch<1>(d_y, rows, d_w, d_pos, d_out, num_tokens, topk, nvec, stream);
  return launch<2>(d_y, rows, d_w, d_pos, d_out, num_tokens, topk, nvec, stream);
}

}  // namespace moe
