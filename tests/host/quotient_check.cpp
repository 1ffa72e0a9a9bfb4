// Host check of e4m3_quotient (csrc/e4m3.h), the FP8 kernels' x / scale: the
// same function compiled for the host against the host's IEEE division, for
// x over every bf16 pattern and amax over every exponent field with five
// significands plus every significand in the binades at the edges of the
// fast path and around 1. Where the quotient can round to a nonzero E4M3 code
// (|x / s| >= 2^-11) it must equal the IEEE quotient bit for bit; below that it
// must keep the sign and stay under 2^-10 (so the code is the same signed
// zero); NaN inputs must give a NaN of the same sign. Only the inputs a block
// can hold: |x| <= amax, or x NaN. Exit status 0 when every check holds.
// (A single correction step already agrees on every pair checked here; the
// second is the one Markstein's theorem needs for the general case, and the
// GPU sweep checks the codes of all pairs.)
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "e4m3.h"

namespace {

float from_bits(uint32_t b) {
  float f;
  std::memcpy(&f, &b, 4);
  return f;
}
uint32_t bits_of(float f) {
  uint32_t b;
  std::memcpy(&b, &f, 4);
  return b;
}

}  // namespace

int main() {
  std::vector<uint32_t> amax_bits;
  for (uint32_t e = 0; e < 255; ++e)
    for (uint32_t m : {0u, 1u, 0x3Fu, 0x40u, 0x7Fu})
      if ((e << 7 | m) != 0) amax_bits.push_back(e << 7 | m);
  for (uint32_t e : {1u, 2u, 3u, 0x29u, 0x2Au, 0x7Eu, 0x7Fu, 0x80u, 0xFDu, 0xFEu})
    for (uint32_t m = 0; m < 128; ++m) amax_bits.push_back(e << 7 | m);
  long long checked = 0, fast_pairs = 0, failures = 0;
  for (uint32_t ab : amax_bits) {
    const float amax = from_bits(ab << 16);
    const float s = amax / 448.0f;
    const bool fast = moe::e4m3_fast_scale(s);
    if (!fast) continue;   // the kernels divide there
    const float y = 1.0f / s;
    for (uint32_t xb = 0; xb < 65536; ++xb) {
      const float x = from_bits(xb << 16);
      if (!(std::isnan(x) || std::fabs(x) <= amax)) continue;
      ++fast_pairs;
      const float want = x / s;
      const float got = moe::e4m3_quotient(x, s, y);
      bool ok;
      if (std::isnan(want))
        ok = std::isnan(got) && std::signbit(got) == std::signbit(want);
      else if (std::fabs(want) >= 0x1p-11f)
        ok = bits_of(got) == bits_of(want);
      else
        ok = std::fabs(got) < 0x1p-10f && std::signbit(got) == std::signbit(want);
      ++checked;
      if (!ok && failures++ < 5)
        std::printf("FAIL amax 0x%04x x 0x%04x: want %a got %a\n", ab, xb, want, got);
    }
  }
  std::printf("%lld pairs on the fast path checked over %zu amax values, %lld failures\n",
              checked, amax_bits.size(), failures);
  return failures == 0 && fast_pairs > 50000000LL ? 0 : 1;
}
