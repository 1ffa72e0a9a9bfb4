/* Plain-C use of the library's C ABI (no Python, no torch): layout, bf16
 * dispatch and combine with identity experts, plus one host-side error. The
 * round trip runs uncapped and under two workgroup caps (moe_set_max_workgroups:
 * 7 takes the bf16 dispatch's one-wavefront-per-item form, 600 its
 * slot-spread form; both loop over items).
 *
 * With weights of exactly 1/k, combine(dispatch(x)) rounds back to x bit for
 * bit (the fp32 sum of k copies of x/k is exact), except that -0 comes back
 * as +0 (the sum starts from +0). Also checks that the per-expert counts
 * read through moe_layout_view sum to T*k and that a too-small output buffer
 * is refused on the host with MOE_ERR_INVALID_ARG. Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_ep.h"

#define CHECK_HIP(call)                                                          \
  do {                                                                           \
    hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);           \
      return 2;                                                                  \
    }                                                                            \
  } while (0)

#define CHECK_MOE(call)                                                          \
  do {                                                                           \
    int s_ = (call);                                                             \
    if (s_ != MOE_OK) {                                                          \
      fprintf(stderr, "%s: %s\n", moe_status_string(s_), moe_last_error());      \
      return 3;                                                                  \
    }                                                                            \
  } while (0)

static uint64_t lcg_state = 12345;
static uint32_t lcg(void) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg_state >> 33);
}

int main(void) {
  const int T = 1000, H = 1024, K = 4, E = 32, R = 4;
  const moe_config_t cfg = {T, H, K, E, R};
  const size_t ws_bytes = moe_workspace_bytes(&cfg);
  if (ws_bytes == 0) {
    fprintf(stderr, "moe_workspace_bytes: %s\n", moe_last_error());
    return 3;
  }

  int32_t* ids = malloc(sizeof(int32_t) * T * K);
  float* w = malloc(sizeof(float) * T * K);
  uint16_t* x = malloc(sizeof(uint16_t) * T * H);
  uint16_t* out = malloc(sizeof(uint16_t) * T * H);
  int32_t* counts = malloc(sizeof(int32_t) * E);
  if (!ids || !w || !x || !out || !counts) return 4;
  for (int i = 0; i < T * K; ++i) {
    ids[i] = (int32_t)(lcg() % E);
    w[i] = 1.0f / K;
  }
  for (int i = 0; i < T * H; ++i) {
    /* finite bf16: sign, exponent 100..154, any mantissa; some signed zeros */
    const uint32_t r = lcg();
    x[i] = (r % 97 == 0) ? (uint16_t)((r >> 8) & 0x8000u)
                         : (uint16_t)((r & 0x8000u) | ((100u + (r >> 16) % 55u) << 7) | (r & 0x7Fu));
  }

  void *d_ws, *d_x, *d_rows, *d_out;
  int32_t* d_ids;
  float* d_w;
  CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
  CHECK_HIP(hipMalloc((void**)&d_ids, sizeof(int32_t) * T * K));
  CHECK_HIP(hipMalloc((void**)&d_w, sizeof(float) * T * K));
  CHECK_HIP(hipMalloc(&d_x, sizeof(uint16_t) * T * H));
  CHECK_HIP(hipMalloc(&d_rows, sizeof(uint16_t) * (size_t)T * K * H));
  CHECK_HIP(hipMalloc(&d_out, sizeof(uint16_t) * T * H));
  CHECK_HIP(hipMemcpy(d_ids, ids, sizeof(int32_t) * T * K, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_w, w, sizeof(float) * T * K, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_x, x, sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  moe_handle_t h;
  CHECK_MOE(moe_handle_create(&cfg, d_ws, ws_bytes, &h));
  CHECK_MOE(moe_dispatch_layout(h, d_ids, T, stream));

  /* A buffer one row short of the worst case is refused before any launch. */
  if (moe_dispatch(h, d_x, MOE_DTYPE_BF16, d_rows, NULL, (int64_t)T * K - 1, stream) !=
      MOE_ERR_INVALID_ARG) {
    fprintf(stderr, "short output buffer was not refused\n");
    return 5;
  }
  const int32_t caps[3] = {0, 7, 600};
  for (int c = 0; c < 3; ++c) {
    CHECK_HIP(hipMemsetAsync(d_rows, 0xFF, sizeof(uint16_t) * (size_t)T * K * H, stream));
    CHECK_HIP(hipMemsetAsync(d_out, 0xFF, sizeof(uint16_t) * T * H, stream));
    CHECK_MOE(moe_set_max_workgroups(h, caps[c]));
    CHECK_MOE(moe_dispatch(h, d_x, MOE_DTYPE_BF16, d_rows, NULL, (int64_t)T * K, stream));
    CHECK_MOE(moe_combine(h, d_rows, (int64_t)T * K, d_w, d_out, stream));

    moe_layout_view_t view;
    CHECK_MOE(moe_layout_view(h, &view));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(counts, view.counts_e, sizeof(int32_t) * E, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(out, d_out, sizeof(uint16_t) * T * H, hipMemcpyDeviceToHost));

    long total = 0;
    for (int e = 0; e < E; ++e) total += counts[e];
    if (total != (long)T * K) {
      fprintf(stderr, "counts sum to %ld, expected %d\n", total, T * K);
      return 6;
    }
    long bad = 0;
    for (int i = 0; i < T * H; ++i) {
      const uint16_t want = x[i] == 0x8000u ? 0 : x[i];
      if (out[i] != want) ++bad;
    }
    if (bad) {
      fprintf(stderr, "%ld elements differ after the round trip (workgroup cap %d)\n", bad,
              caps[c]);
      return 7;
    }
  }

  moe_handle_destroy(h);
  CHECK_HIP(hipStreamDestroy(stream));
  hipFree(d_ws); hipFree(d_ids); hipFree(d_w); hipFree(d_x); hipFree(d_rows); hipFree(d_out);
  free(ids); free(w); free(x); free(out); free(counts);
  printf("abi_roundtrip ok: %d tokens, top-%d of %d experts, hidden %d, workgroup caps 0/7/600\n",
         T, K, E, H);
  return 0;
}
