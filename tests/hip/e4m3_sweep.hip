// Exhaustive check of the fp32 -> E4M3 conversion the FP8 and MXFP8 dispatch
// kernels use (csrc/e4m3.h): a GPU test hands this program a range of fp32 bit
// patterns, and it writes the code the kernels' saturate-then-convert steps
// give each one. The test compares them on the host, chunk by chunk, with an
// independent conversion. Built by tests/hip/build.py into libe4m3_sweep.so.
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

}  // namespace

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
