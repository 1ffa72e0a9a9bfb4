// Exhaustive checks of the FP8 steps the dispatch kernels run (csrc/e4m3.h):
//   e4m3_sweep: a GPU test hands this program a range of fp32 bit patterns,
//     and it writes the code the kernels' saturate-then-convert steps give
//     each one; the test compares them on the host, chunk by chunk, with an
//     independent conversion.
//   e4m3_quotient_sweep: for a range of positive finite bf16 amax values and
//     every bf16 x, the E4M3 code of the kernels' quotient (e4m3_quotient on
//     scales that e4m3_fast_scale admits, else the IEEE division) against the
//     code of the IEEE quotient x / (amax / 448), counting disagreements.
// Built by tests/hip/build.py into libe4m3_sweep.so.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "e4m3.h"

namespace {

// Word i holds the codes of bit patterns first + 4i .. first + 4i + 3
// (modulo 2^32), lowest pattern in the lowest byte.
__global__ __launch_bounds__(256) void e4m3_sweep_kernel(uint32_t first, uint32_t nwords,
                                                         uint32_t* __restrict__ out) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < nwords;
       i += gridDim.x * blockDim.x) {
    const uint32_t b = first + 4u * i;
    out[i] = moe::pack_e4m3(moe::e4m3_saturate(__uint_as_float(b)),
                            moe::e4m3_saturate(__uint_as_float(b + 1u)),
                            moe::e4m3_saturate(__uint_as_float(b + 2u)),
                            moe::e4m3_saturate(__uint_as_float(b + 3u)));
  }
}

__device__ __forceinline__ uint32_t code_of(float v) {
  return moe::pack_e4m3(moe::e4m3_saturate(v), 0.0f, 0.0f, 0.0f) & 0xFFu;
}

// Thread = (amax bf16 pattern first_amax + i, high byte of x); it runs the
// 256 x patterns of that high byte. counts[0]: disagreements with |x| <= amax
// or x NaN (the inputs a real block holds: amax is the block's largest
// magnitude); counts[1]: disagreements elsewhere (|x| > amax, which no block
// holds); counts[2]: pairs that took the fast path. example: the last
// in-domain disagreement as (amax bits << 16) | x bits.
__global__ __launch_bounds__(256) void quotient_sweep_kernel(uint32_t first_amax, uint32_t n_amax,
                                                             uint32_t* __restrict__ counts,
                                                             uint32_t* __restrict__ example) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t ai = gid >> 8, xhi = gid & 255u;
  if (ai >= n_amax) return;
  const uint32_t abits = first_amax + ai;
  const float m = __uint_as_float(abits << 16);
  const float s = m / 448.0f;
  const bool fast = moe::e4m3_fast_scale(s);
  const float y = 1.0f / s;
  uint32_t in_domain = 0, outside = 0, last = 0;
  for (uint32_t xlo = 0; xlo < 256u; ++xlo) {
    const uint32_t xb = (xhi << 8) | xlo;
    const float x = __uint_as_float(xb << 16);
    const uint32_t want = code_of(x / s);
    const uint32_t got = code_of(fast ? moe::e4m3_quotient(x, s, y) : x / s);
    if (want != got) {
      if (__builtin_isnan(x) || fabsf(x) <= m) {
        ++in_domain;
        last = (abits << 16) | xb;
      } else {
        ++outside;
      }
    }
  }
  if (in_domain) {
    atomicAdd(&counts[0], in_domain);
    *example = last;
  }
  if (outside) atomicAdd(&counts[1], outside);
  if (fast) atomicAdd(&counts[2], 256u);
}

}  // namespace

// Quotient check over the bf16 amax patterns first_amax .. first_amax +
// n_amax - 1 (each a positive finite bf16: 0x0001 .. 0x7F7F) against every
// bf16 x, adding into d_counts[0..2] (see quotient_sweep_kernel; the caller
// zeroes them) and d_example[0], enqueued on `stream`. Returns 0, 1 for an
// invalid argument (nothing enqueued), 2 if the launch failed.
extern "C" int e4m3_quotient_sweep(uint32_t first_amax, uint32_t n_amax, void* d_counts,
                                   void* d_example, hipStream_t stream) {
  if (d_counts == nullptr || d_example == nullptr || first_amax == 0u ||
      n_amax > 0x7F7Fu || first_amax + n_amax > 0x7F80u ||
      reinterpret_cast<uintptr_t>(d_counts) % 4u != 0u ||
      reinterpret_cast<uintptr_t>(d_example) % 4u != 0u)
    return 1;
  if (n_amax == 0u) return 0;
  const uint32_t threads = n_amax * 256u;
  hipLaunchKernelGGL(quotient_sweep_kernel, dim3((threads + 255u) / 256u), dim3(256), 0, stream,
                     first_amax, n_amax, static_cast<uint32_t*>(d_counts),
                     static_cast<uint32_t*>(d_example));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Codes of the `count` fp32 bit patterns first, first + 1, ... (modulo 2^32)
// into d_codes[0 .. count), enqueued on `stream`. count must be a multiple of
// 4 and d_codes a 4-byte-aligned device buffer of at least count bytes.
// Returns 0, 1 for an invalid argument (nothing enqueued), 2 if the launch
// failed.
extern "C" int e4m3_sweep(uint32_t first, uint32_t count, void* d_codes, hipStream_t stream) {
  if (d_codes == nullptr || count % 4u != 0u || reinterpret_cast<uintptr_t>(d_codes) % 4u != 0u)
    return 1;
  const uint32_t nwords = count / 4u;
  if (nwords == 0u) return 0;
  uint32_t blocks = (nwords + 255u) / 256u;
  if (blocks > 65536u) blocks = 65536u;
  hipLaunchKernelGGL(e4m3_sweep_kernel, dim3(blocks), dim3(256), 0, stream, first, nwords,
                     static_cast<uint32_t*>(d_codes));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
