// Dispatch: scatter each token row to the k rows its layout assigned.
//
// Per the pages, dispatch "sends tokens to their assigned experts" ("Inside
// the Nebius + PyTorch DeepSeek V3 recipe", section "Mixture-of-experts and
// wide expert parallelism") into buffers preallocated for the worst case
// (Hybrid-EP news item, "Availability and Integration"), optionally as FP8
// ("MoE / Hybrid-EP Validation", "Communication path comparison" and "FP8
// dispatch restriction").
//
// Both kernels read each token row from HBM exactly once into registers and
// write it k times, 16 bytes per lane per store, so a wavefront writes 1 KiB
// of one destination row per store instruction. A workgroup owns whole
// tokens; no two workgroups write the same row, so there are no atomics.
//
// FP8 E4M3 (OCP, max 448) quantisation is fused and done once per token:
// each lane holds 16 channels, 8 consecutive lanes form one 128-channel block,
// amax is reduced across those 8 lanes, scale = amax / 448 (IEEE division),
// and each code is the nearest-even E4M3 value of the IEEE quotient x / scale,
// converted by the hardware fp32 -> fp8 instruction. The quotient is clamped
// to +-448 first: it can exceed 448 by at most one fp32 ulp, which rounds to
// 448 anyway, and the clamp keeps the conversion away from its overflow
// handling. A block whose amax is 0 gets scale 0 and its signed-zero inputs
// as codes.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kDispatchThreads = 128;
constexpr int kFp8MaxThreads = 512;

template <int U>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_bf16_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos, u32x4* __restrict__ out,
    int num_tokens, int topk, int nvec, int64_t rows) {
  for (int t = blockIdx.x; t < num_tokens; t += gridDim.x) {
    const u32x4* src = x + static_cast<size_t>(t) * nvec;
    const int32_t* pt = pos + static_cast<size_t>(t) * topk;
    for (int v0 = threadIdx.x; v0 < nvec; v0 += U * kDispatchThreads) {
      u32x4 r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * kDispatchThreads;
        if (v < nvec) r[u] = src[v];
      }
      for (int j = 0; j < topk; ++j) {
        const int p = pt[j];
        if (p < 0 || p >= rows) continue;
        u32x4* dst = out + static_cast<size_t>(p) * nvec;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int v = v0 + u * kDispatchThreads;
          if (v < nvec) dst[v] = r[u];
        }
      }
    }
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four fp32 values -> four E4M3 codes packed little-endian in one dword.
__device__ __forceinline__ uint32_t pack_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

__global__ __launch_bounds__(kFp8MaxThreads) void dispatch_fp8_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos, u32x4* __restrict__ out,
    float* __restrict__ scales, int num_tokens, int topk, int hidden, int64_t rows) {
  const int units = hidden >> 4;    // 16 channels per lane
  const int nscale = hidden >> 7;   // one scale per 128 channels
  for (int t = blockIdx.x; t < num_tokens; t += gridDim.x) {
    const u32x4* src = x + static_cast<size_t>(t) * (hidden >> 3);
    const int32_t* pt = pos + static_cast<size_t>(t) * topk;
    // blockDim.x is a multiple of 64 and units a multiple of 8, so every
    // 8-lane group is either wholly inside the loop or wholly outside it.
    for (int u = threadIdx.x; u < units; u += blockDim.x) {
      const u32x4 a = src[2 * u];
      const u32x4 b = src[2 * u + 1];
      float f[16] = {bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y),
                     bf16_lo(a.z), bf16_hi(a.z), bf16_lo(a.w), bf16_hi(a.w),
                     bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y),
                     bf16_lo(b.z), bf16_hi(b.z), bf16_lo(b.w), bf16_hi(b.w)};
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(f[i]));
      m = fmaxf(m, __shfl_xor(m, 1, 64));
      m = fmaxf(m, __shfl_xor(m, 2, 64));
      m = fmaxf(m, __shfl_xor(m, 4, 64));
      const float scale = m / 448.0f;
      if (m > 0.0f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] = __builtin_amdgcn_fmed3f(f[i] / scale, -448.0f, 448.0f);
      }
      u32x4 q;
      q.x = pack_e4m3(f[0], f[1], f[2], f[3]);
      q.y = pack_e4m3(f[4], f[5], f[6], f[7]);
      q.z = pack_e4m3(f[8], f[9], f[10], f[11]);
      q.w = pack_e4m3(f[12], f[13], f[14], f[15]);
      const bool scale_lane = (threadIdx.x & 7) == 0;
      for (int j = 0; j < topk; ++j) {
        const int p = pt[j];
        if (p < 0 || p >= rows) continue;
        out[static_cast<size_t>(p) * units + u] = q;
        if (scale_lane) scales[static_cast<size_t>(p) * nscale + (u >> 3)] = scale;
      }
    }
  }
}

template <int U>
hipError_t launch_bf16(const void* d_x, const int32_t* d_pos, void* d_out, int num_tokens,
                       int topk, int nvec, int64_t rows, hipStream_t stream) {
  hipLaunchKernelGGL(dispatch_bf16_kernel<U>, dim3(num_tokens), dim3(kDispatchThreads), 0, stream,
                     static_cast<const u32x4*>(d_x), d_pos, static_cast<u32x4*>(d_out),
                     num_tokens, topk, nvec, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch_bf16(const void* d_x, const int32_t* d_pos, void* d_out,
                                int64_t rows, int num_tokens, int topk, int hidden,
                                hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int nvec = hidden / 8;
  const int per_thread = (nvec + kDispatchThreads - 1) / kDispatchThreads;
  switch (per_thread) {
    case 1: return launch_bf16<1>(d_x, d_pos, d_out, num_tokens, topk, nvec, rows, stream);
    case 2: return launch_bf16<2>(d_x, d_pos, d_out, num_tokens, topk, nvec, rows, stream);
    case 3: return launch_bf16<3>(d_x, d_pos, d_out, num_tokens, topk, nvec, rows, stream);
    case 4: return launch_bf16<4>(d_x, d_pos, d_out, num_tokens, topk, nvec, rows, stream);
    case 5: return launch_bf16<5>(d_x, d_pos, d_out, num_tokens, topk, nvec, rows, stream);
    case 6: return launch_bf16<6>(d_x, d_pos, d_out, num_tokens, topk, nvec, rows, stream);
    case 7: return launch_bf16<7>(d_x, d_pos, d_out, num_tokens, topk, nvec, rows, stream);
    default: return launch_bf16<8>(d_x, d_pos, d_out, num_tokens, topk, nvec, rows, stream);
  }
}

hipError_t launch_dispatch_fp8(const void* d_x, const int32_t* d_pos, void* d_out,
                               float* d_scales, int64_t rows, int num_tokens, int topk,
                               int hidden, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int units = hidden / 16;
  int threads = ((units + 63) / 64) * 64;
  if (threads > kFp8MaxThreads) threads = kFp8MaxThreads;
  hipLaunchKernelGGL(dispatch_fp8_kernel, dim3(num_tokens), dim3(threads), 0, stream,
                     static_cast<const u32x4*>(d_x), d_pos, static_cast<u32x4*>(d_out), d_scales,
                     num_tokens, topk, hidden, rows);
  return hipGetLastError();
}

}  // namespace moe
