// Host-side checks of the blocked bf16 dispatch's sizing rules and of the
// multiply-high division its kernel uses (csrc/moe_internal.h): built and
// run on the CPU by tests/test_block_rule_host.py; no GPU call.
#include <cstdint>
#include <cstdio>
#include <random>

#include "moe_internal.h"

namespace {

int failures = 0;

void fail(const char* what, long long a, long long b, long long c) {
  if (failures++ < 20) std::printf("FAIL %s (%lld, %lld, %lld)\n", what, a, b, c);
}

// fast_div against integer division: every divisor up to 4096 and the
// divisors the kernel uses, on small, random, boundary and near-multiple n.
void check_fast_div() {
  std::mt19937_64 rng(12345);
  auto check = [&](uint32_t d) {
    const moe::FastDiv f = moe::make_fast_div(d);
    auto one = [&](uint32_t n) {
      if (moe::fast_div(n, f) != n / d) fail("fast_div", n, d, moe::fast_div(n, f));
    };
    for (uint32_t n = 0; n < 4096; ++n) one(n);
    for (int i = 0; i < 2000; ++i) one(static_cast<uint32_t>(rng() & 0x7FFFFFFFu));
    for (uint32_t n = 0x7FFFFFFFu - 64; n <= 0x7FFFFFFEu; ++n) one(n);
    one(0x7FFFFFFFu);
    for (uint64_t q = 1; q * d < 0x7FFFFFFFull; q = q * 3 + 1) {
      const uint64_t m = q * d;
      one(static_cast<uint32_t>(m - 1));
      one(static_cast<uint32_t>(m));
      if (m + 1 <= 0x7FFFFFFFull) one(static_cast<uint32_t>(m + 1));
    }
  };
  for (uint32_t d = 1; d <= 4096; ++d) check(d);
  for (uint32_t d : {65537u, 1000003u, (1u << 20) + 7, 0x40000001u, 0x7FFFFFFFu}) check(d);
}

// dispatch_block_chunks and the list capacity over a sweep of shapes.
void check_block_rule() {
  const int hiddens[] = {8, 128, 512, 2048, 4096, 4992, 7168, 7176, 8192, 16384, 16392};
  long long used = 0;
  for (int k = 1; k <= MOE_EP_MAX_TOPK; ++k)
    for (int hidden : hiddens)
      for (int T = 1; T <= 70000; T += (T < 2048 ? 7 : 211)) {
        const int m = moe::dispatch_block_chunks(T, k, hidden);
        const int64_t slots = int64_t(T) * k;
        const int64_t chunks = (slots + moe::kLayoutChunk - 1) / moe::kLayoutChunk;
        if (m == 0) continue;
        ++used;
        if (m & (m - 1)) fail("block chunks not a power of two", T, k, m);
        if (chunks < moe::kXcds) fail("fewer chunks than XCD slots", T, k, m);
        if (m > chunks / moe::kXcds) fail("block above chunks / 8", T, k, m);
        const int64_t bs = int64_t(m) * moe::kLayoutChunk;
        const int64_t chunk_x = int64_t(moe::kLayoutChunk) * 2 * hidden / k;
        if (m * chunk_x > moe::kBlockXBytes) fail("block x above the limit", T, k, m);
        if (int64_t(T) * 2 * hidden > moe::kBlockedMaxXBytes) fail("batch x above the limit", T, k, m);
        const int64_t nblocks = (chunks + m - 1) / m;
        const int64_t per_slot = (nblocks + moe::kXcds - 1) / moe::kXcds;
        const int64_t tpb = bs / k + 2;
        // the lists of this batch fit the workspace of any T_max >= T
        if (nblocks * bs > moe::dispatch_order_entries(T, k)) fail("lists above capacity", T, k, m);
        // every block's slots span at most tpb tokens
        for (int64_t b = 0; b < nblocks; ++b) {
          const int64_t first = b * bs, end = std::min(first + bs, slots);
          if ((end - 1) / k - first / k + 1 > tpb) fail("token span above tpb", T, k, b);
        }
        // the kernel's indices stay below 2^31
        const int64_t slices = (hidden / 8 + 63) / 64;
        if (per_slot * bs * slices + 4 > 0x7FFFFFFF) fail("item index range", T, k, m);
      }
  if (used < 1000) fail("too few shapes took the blocked form", used, 0, 0);
  // the shapes the benchmark measures
  if (moe::dispatch_block_chunks(4096, 8, 7168) != 2) fail("V3-like rule", 4096, 8, 7168);
  if (moe::dispatch_block_chunks(4096, 6, 2048) != 1) fail("16B-like rule", 4096, 6, 2048);
  if (moe::dispatch_block_chunks(16384, 8, 4096) != 2) fail("Qwen3-like rule", 16384, 8, 4096);
  if (moe::dispatch_block_chunks(12288, 8, 7168) != 2) fail("x of 176 MB", 12288, 8, 7168);
  // the batch's x above 192 MiB: the per-slot form
  if (moe::dispatch_block_chunks(16384, 8, 7168) != 0) fail("x of 235 MB", 16384, 8, 7168);
  if (moe::dispatch_block_chunks(32768, 8, 4096) != 0) fail("x of 268 MB", 32768, 8, 4096);
  if (moe::dispatch_block_chunks(4096, 8, 4096) != 2) fail("H=4096 rule", 4096, 8, 4096);
  if (moe::dispatch_block_chunks(16384, 6, 2048) != 4) fail("16B-like rule, long batch", 16384, 6, 2048);
  // one chunk's tokens above 7/8 of an L2: the per-slot form
  if (moe::dispatch_block_chunks(65536, 2, 7168) != 0) fail("top-2 at H=7168", 65536, 2, 7168);
  if (moe::dispatch_block_chunks(896, 8, 7168) != 0) fail("under 8 chunks", 896, 8, 7168);
  if (moe::dispatch_block_chunks(897, 8, 7168) != 1) fail("8 chunks", 897, 8, 7168);
}

}  // namespace

int main() {
  check_fast_div();
  check_block_rule();
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("block rule ok\n");
  return 0;
}
