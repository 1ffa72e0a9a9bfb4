// Dispatch: scatter each token row to the k rows its layout assigned.
//
// Dispatch is the first half of an MoE layer's exchange: each token's row goes
// to every expert its router picked ("Inside the Nebius + PyTorch DeepSeek V3
// recipe", section "Mixture-of-experts and wide expert parallelism"), into
// buffers sized for the worst case because routing is only known at run time
// (Hybrid-EP news item, "Availability and Integration"), optionally as FP8
// ("MoE / Hybrid-EP Validation", "Communication path comparison" and "FP8
// dispatch restriction").
//
// Work decomposition: no workgroup waits for another. The Hybrid-EP news
// item ("Technical Structure") describes each CUDA block as an independent
// channel with no cross-block synchronisation; here the independent unit is
// a (token, column slice) item. FP8/MXFP8 (and bf16 through the
// rank-deduplicated table): one wavefront per item, kItemWaves items per
// workgroup; the wavefront fetches the token's k row indices with scalar
// loads, reads its slice of the token row once (16 bytes per lane) and
// writes it to the k destination rows with 16-byte stores. Standard bf16:
// from kXcds layout chunks on (while a chunk's tokens hold at most
// kBlockXBytes of x and the batch at most kBlockedMaxXBytes) the blocked
// form, whose wavefronts each copy one 1 KiB
// slice of one row along the layout's block lists, the blocks of an XCD slot
// one after another (dispatch_bf16_blocks_kernel); otherwise one workgroup
// per item, the token's slots spread over its wavefronts
// (dispatch_bf16_slots_kernel), or under a cap below kSlotsFormMinCap
// workgroups the one-wavefront form. No two wavefronts write the same bytes:
// no atomics, and no barrier in any form.
//
// Row stores are non-temporal: each dispatched row is written once and its
// next reader (the expert computation) is another kernel, so the rows stream
// to HBM instead of filling the last-level cache with dirty lines that a
// later kernel would have to write back. Measured back to back over rotating
// buffers (T=4096, H=7168, k=8): bf16 dispatch 107 -> 95 us, FP8 69 -> 50 us.
// The 4-byte scale stores stay cached: as partial lines, non-temporal they
// were slower.
//
// FP8 E4M3 (OCP, max 448) quantisation is fused and done once per token: a
// lane holds 16 channels, 8 consecutive lanes form one 128-channel block,
// amax is reduced across those 8 lanes, scale = amax / 448 (IEEE division),
// and each code is the nearest-even E4M3 value of the IEEE quotient
// x / scale, converted by the hardware fp32 -> fp8 instruction. The quotient
// itself comes from e4m3_quotient (the same value as an IEEE division, from
// one reciprocal per lane and four fmas per element): per-op with x from HBM
// and the workloads' routing, same box, 57.2-57.5 -> 56.8-57.1 us at T=4096,
// H=7168, k=8; 126.6-126.8 -> 125.3-126.0 at T=16384, H=4096; unchanged at
// T=4096, H=2048, top-6 (13.3-13.4). The quotient
// is clamped to +-448 first, which keeps the conversion away from its
// overflow handling. With a normal fp32 scale the quotient exceeds 448 by at
// most one fp32 ulp (which rounds to 448 anyway); with a subnormal scale
// (amax below about 448 * 2^-126) the scale itself has lost precision and the
// quotient can lie well above 448 (amax = 2^-133 gives about 448.9): there the
// clamp is what makes the amax element's code 448, the nearest E4M3 value of
// the exact ratio. A block whose amax is 0 gets scale 0 and its signed-zero
// inputs as codes.
//
// Decode-time (fixed-capacity) dispatch does layout and payload in one launch.
// DeepEP's second kernel family serves decode ("Inside the Nebius + PyTorch
// DeepSeek V3 recipe", section "DeepEP"); its receive buffers have a shape
// that does not depend on the routing. Here expert e owns rows
// [e*C, (e+1)*C); a slot's row is e*C plus its stable rank among the slots
// routed to e (token order, then slot order), and slots ranked C or more are
// dropped. A workgroup takes one token and four of its column slices, one per
// wavefront. A slot's rank is the number of matching ids among the earlier
// slots: below kFixedSharedFrom tokens each wavefront counts them itself (no
// barrier at all); from there on the four wavefronts split the count and add
// their shares through LDS. The last workgroup of the grid builds the
// per-expert histogram in LDS and publishes counts and status. No workgroup
// waits for another. The counting is O(T*k) per workgroup, which is why this
// path is limited to small batches (MOE_EP_LL_MAX_TOKENS).
#include <type_traits>

#include "e4m3.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Row indices of slots j0 .. j0+kSlotBatch-1 of one token (pt points at its
// k entries). The loads are unconditional (clamped to slot k-1) so they issue
// back to back; slots past k, skipped slots (-1) and rows outside [0, rows)
// come back as -1.
__device__ __forceinline__ void load_rows(const int32_t* __restrict__ pt, int j0, int topk,
                                          int64_t rows, int (&p)[kSlotBatch]) {
  if (j0 + kSlotBatch <= topk) {   // full batch: contiguous, merges into wide scalar loads
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) p[jj] = pt[j0 + jj];
  } else {
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) p[jj] = pt[j0 + jj < topk ? j0 + jj : topk - 1];
  }
#pragma unroll
  for (int jj = 0; jj < kSlotBatch; ++jj)
    if (j0 + jj >= topk || p[jj] < 0 || p[jj] >= rows) p[jj] = -1;
}

// Row stores are non-temporal: the dispatched rows stream to HBM without
// displacing other data from the last-level cache.
__device__ __forceinline__ void store_row(u32x4* dst, const u32x4& v) {
  __builtin_nontemporal_store(v, dst);
}

// Completes the load of v here, on every path. The stores that follow each
// sit in a branch of their own (one per slot, skipped for -1 rows); without
// this point the compiler cannot tell at each branch whether v's load has
// completed, and waits for every earlier memory operation -- the previous
// store's write acknowledgement included -- before each store. Measured at
// T=4096, H=7168, k=8 with x read from HBM: rows in token order 90.2 -> 85.7
// us; the workload's scattered rows unchanged (100.2 vs 100.5 us).
__device__ __forceinline__ void loaded(const u32x4& v) { asm volatile("" ::"v"(v)); }

// Where a payload function finds the destination rows of token t's slots:
// rows_of fills p[] for slots j0 .. j0+kSlotBatch-1 (-1: no row).

// Standard layout: the table pos[T, k] written by the layout kernels. The
// standard kernels take it as a restrict-qualified argument of their own:
// then the compiler may read it through the scalar cache (no store of the
// kernel can change it), and the index loads count against lgkmcnt, apart
// from the vector loads of x that the stores wait for.

// Row of slot j of token t in the table, or -1 if outside [0, rows).
__device__ __forceinline__ int table_row(const int32_t* __restrict__ pos, int topk, int64_t rows,
                                         int t, int j) {
  const int p = pos[static_cast<size_t>(t) * topk + j];
  return p >= 0 && p < rows ? p : -1;
}

// Decode-time layout: the token's rows, computed by its workgroup into LDS.
struct SharedRows {
  const int32_t* s_pos;   // [topk] in LDS
  int topk;
  __device__ __forceinline__ void rows_of(int, int j0, int (&p)[kSlotBatch]) const {
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) p[jj] = j0 + jj < topk ? s_pos[j0 + jj] : -1;
  }
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Lane u's 16 channels of the row at src (zeros for an inactive lane).
__device__ __forceinline__ void load_lane16(const u32x4* __restrict__ src, int u, bool active,
                                            u32x4& a, u32x4& b) {
  a = {0u, 0u, 0u, 0u};
  b = {0u, 0u, 0u, 0u};
  if (active) {
    a = src[2 * u];
    b = src[2 * u + 1];
  }
}

// FP8 E4M3 quantisation of one lane's 16 channels a, b (unit u of a row; 8
// consecutive lanes form a 128-channel block): codes q and the block scale.
__device__ __forceinline__ void quantize_fp8(const u32x4& a, const u32x4& b, u32x4& q,
                                             float& scale) {
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
  scale = m / 448.0f;
  if (m > 0.0f) {
    if (e4m3_fast_scale(scale)) {   // every finite scale of bf16 data above 2^-90
      const float y = 1.0f / scale;
#pragma unroll
      for (int i = 0; i < 16; ++i) f[i] = e4m3_saturate(e4m3_quotient(f[i], scale, y));
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) f[i] = e4m3_saturate(f[i] / scale);
    }
  }
  q.x = pack_e4m3(f[0], f[1], f[2], f[3]);
  q.y = pack_e4m3(f[4], f[5], f[6], f[7]);
  q.z = pack_e4m3(f[8], f[9], f[10], f[11]);
  q.w = pack_e4m3(f[12], f[13], f[14], f[15]);
}

// The same, loading unit u of the row at src first.
__device__ __forceinline__ void quantize_fp8(const u32x4* __restrict__ src, int u, bool active,
                                             u32x4& q, float& scale) {
  u32x4 a, b;
  load_lane16(src, u, active, a, b);
  quantize_fp8(a, b, q, scale);
}

// MXFP8 quantisation of one lane's 16 channels (a lane pair is one 32-channel
// block): codes q and, in lanes 8i, the dword of four E8M0 codes of blocks
// u/2 .. u/2+3.
__device__ __forceinline__ void quantize_mxfp8(const u32x4& a, const u32x4& b, int lane,
                                               u32x4& q, uint32_t& word) {
  float f[16] = {bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y),
                 bf16_lo(a.z), bf16_hi(a.z), bf16_lo(a.w), bf16_hi(a.w),
                 bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y),
                 bf16_lo(b.z), bf16_hi(b.z), bf16_lo(b.w), bf16_hi(b.w)};
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(f[i]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  const uint32_t mb = __float_as_uint(m);
  int shared = -127;
  if (mb != 0u) {
    const int fl = mb >= 0x00800000u ? static_cast<int>(mb >> 23) - 127   // normal
                                     : 31 - __clz(mb) - 149;                // subnormal
    shared = fl - 8 < -127 ? -127 : (fl - 8 > 127 ? 127 : fl - 8);
  }
  const float inv = __uint_as_float(static_cast<uint32_t>(127 - shared) << 23);   // 2^-shared
#pragma unroll
  for (int i = 0; i < 16; ++i) f[i] = e4m3_saturate(f[i] * inv);
  q.x = pack_e4m3(f[0], f[1], f[2], f[3]);
  q.y = pack_e4m3(f[4], f[5], f[6], f[7]);
  q.z = pack_e4m3(f[8], f[9], f[10], f[11]);
  q.w = pack_e4m3(f[12], f[13], f[14], f[15]);
  // Lane 8i gathers the codes of blocks u/2 .. u/2+3 (lanes 8i, 8i+2, 8i+4, 8i+6).
  const uint32_t code = static_cast<uint32_t>(shared + 127);
  const uint32_t c1 = __shfl(code, lane + 2, 64);
  const uint32_t c2 = __shfl(code, lane + 4, 64);
  const uint32_t c3 = __shfl(code, lane + 6, 64);
  word = code | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// The same, loading unit u of the row at src first.
__device__ __forceinline__ void quantize_mxfp8(const u32x4* __restrict__ src, int u, int lane,
                                               bool active, u32x4& q, uint32_t& word) {
  u32x4 a, b;
  load_lane16(src, u, active, a, b);
  quantize_mxfp8(a, b, lane, q, word);
}

// Payload of one (token t, column slice) work item for each dtype; `rows`
// supplies the destination rows. A lane moves 16 bytes per access.

// bf16: a 512-channel slice (8 channels per lane), read once, stored to every row.
template <class Rows>
__device__ __forceinline__ void bf16_item(const u32x4* __restrict__ x, const Rows& rows,
                                          u32x4* __restrict__ out, int t, int slice, int nvec,
                                          int topk) {
  const int lane = threadIdx.x & 63;
  const int v = slice * 64 + lane;
  const bool active = v < nvec;
  u32x4 r = {0u, 0u, 0u, 0u};
  if (active) r = x[static_cast<size_t>(t) * nvec + v];
  loaded(r);
  for (int j0 = 0; j0 < topk; j0 += kSlotBatch) {
    int p[kSlotBatch];
    rows.rows_of(t, j0, p);
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj)
      if (p[jj] >= 0 && active) store_row(&out[static_cast<size_t>(p[jj]) * nvec + v], r);
  }
}

// FP8 E4M3 with one fp32 scale per 128 channels: a 1024-channel slice.
template <class Rows>
__device__ __forceinline__ void fp8_item(const u32x4* __restrict__ x, const Rows& rows,
                                         u32x4* __restrict__ out, float* __restrict__ scales,
                                         int t, int slice, int hidden, int topk) {
  const int lane = threadIdx.x & 63;
  const int units = hidden >> 4;    // 16 channels per lane
  const int nscale = hidden >> 7;   // one scale per 128 channels
  const int u = slice * 64 + lane;
  // units is a multiple of 8, so each 8-lane group is wholly active or not.
  const bool active = u < units;
  u32x4 q;
  float scale;
  quantize_fp8(x + static_cast<size_t>(t) * (hidden >> 3), u, active, q, scale);
  const bool scale_lane = active && (lane & 7) == 0;
  for (int j0 = 0; j0 < topk; j0 += kSlotBatch) {
    int p[kSlotBatch];
    rows.rows_of(t, j0, p);
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) {
      if (p[jj] < 0) continue;
      if (active) store_row(&out[static_cast<size_t>(p[jj]) * units + u], q);
      if (scale_lane) scales[static_cast<size_t>(p[jj]) * nscale + (u >> 3)] = scale;
    }
  }
}

// MXFP8 (OCP Microscaling v1.0, E4M3 elements): 32-channel blocks share an
// E8M0 power-of-two scale. A lane holds 16 channels, so a block is a lane
// pair; shared = floor(log2 amax) - 8 (8: exponent of E4M3's largest normal),
// clamped to E8M0's [-127, 127], read off amax's fp32 bit fields. Elements are
// x * 2^-shared (exact: a power of two, and every product that can round to a
// nonzero code is a normal fp32), clamped to +-448 and converted by the
// hardware fp32 -> fp8 instruction (round-to-nearest-even). An all-zero block
// gets code 0 and signed-zero elements. Four E8M0 bytes go out per dword
// store. The Hybrid-EP news item ("Efficiency Numbers") reports its Qwen3 run
// in MXFP8.
template <class Rows>
__device__ __forceinline__ void mxfp8_item(const u32x4* __restrict__ x, const Rows& rows,
                                           u32x4* __restrict__ out, uint32_t* __restrict__ scales,
                                           int t, int slice, int hidden, int topk) {
  const int lane = threadIdx.x & 63;
  const int units = hidden >> 4;           // 16 channels per lane
  const int scale_words = hidden >> 7;     // 4 one-byte scales per dword, per row
  const int u = slice * 64 + lane;
  // units is a multiple of 8, so each 8-lane group is wholly active or not.
  const bool active = u < units;
  u32x4 q;
  uint32_t word;
  quantize_mxfp8(x + static_cast<size_t>(t) * (hidden >> 3), u, lane, active, q, word);
  const bool scale_lane = active && (lane & 7) == 0;
  for (int j0 = 0; j0 < topk; j0 += kSlotBatch) {
    int p[kSlotBatch];
    rows.rows_of(t, j0, p);
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) {
      if (p[jj] < 0) continue;
      if (active) store_row(&out[static_cast<size_t>(p[jj]) * units + u], q);
      if (scale_lane) scales[static_cast<size_t>(p[jj]) * scale_words + (u >> 3)] = word;
    }
  }
}

// Channels per lane and slices per token of each dtype.
__host__ __device__ constexpr int lane_channels(int dtype) {
  return dtype == MOE_DTYPE_BF16 ? 8 : 16;
}

// The scale pointer of each dtype (fp32 per 128 channels, or four E8M0 bytes
// per dword); the kernels take it typed and restrict-qualified, so that the
// compiler knows scale stores never alias the row indices it loads.
template <int kDtype>
using ScalePtr = typename std::conditional<kDtype == MOE_DTYPE_MXFP8_E4M3, uint32_t, float>::type*;

template <int kDtype, class Rows>
__device__ __forceinline__ void payload_item(const u32x4* __restrict__ x, const Rows& rows,
                                             u32x4* __restrict__ out,
                                             ScalePtr<kDtype> __restrict__ scales, int t,
                                             int slice, int hidden, int topk) {
  if constexpr (kDtype == MOE_DTYPE_BF16)
    bf16_item(x, rows, out, t, slice, hidden >> 3, topk);
  else if constexpr (kDtype == MOE_DTYPE_FP8_E4M3)
    fp8_item(x, rows, out, scales, t, slice, hidden, topk);
  else
    mxfp8_item(x, rows, out, scales, t, slice, hidden, topk);
}

// Standard FP8/MXFP8 dispatch, and bf16 dispatch through a table where many
// slots are -1 (the rank-deduplicated layout): every wavefront is one
// independent (token, slice) item and loops over the token's slots, so a
// skipped slot costs no wavefront; workgroups [0, payload_blocks) loop over
// the items. The bodies are written out per dtype (rather than through the
// payload functions above, which the decode-time kernel uses): with them
// written out, hipcc keeps the contiguous-batch fast path for the row
// indices, worth 1-2.5% here.
// Receiver metadata of the rank-deduplicated exchange. For each (token,
// rank) row p of token t (opened by slot jr: pos[t, jr] = p) and each slot j
// of t, entry (p, j) says whether slot j's expert lives on that row's rank --
// its local id e - r*E/R and its weight -- or not (-1 and 0).
struct RankMeta {
  const int32_t* idx;   // [T, k] expert ids
  const float* w;       // [T, k] weights
  int num_experts, per_rank;
  int32_t* recv_idx;    // [rows, k]
  float* recv_w;        // [rows, k]
};

// Token t's k x k metadata entries, spread over the wavefront's lanes (one
// (row slot jr, slot j) pair per lane and step; consecutive lanes write
// consecutive entries of a row).
__device__ __forceinline__ void write_rank_meta(const RankMeta& m, const int32_t* __restrict__ pos,
                                                int t, int topk, int64_t rows, int lane) {
  const int base = t * topk;
  for (int q = lane; q < topk * topk; q += 64) {
    const int jr = q / topk, j = q - jr * topk;
    const int p = pos[base + jr];
    if (p < 0 || p >= rows) continue;
    const int e = m.idx[base + j];
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(m.num_experts);
    const int rr = m.idx[base + jr] / m.per_rank;   // the opening slot's expert is valid
    const bool local = valid && e / m.per_rank == rr;
    m.recv_idx[static_cast<size_t>(p) * topk + j] = local ? e - rr * m.per_rank : -1;
    m.recv_w[static_cast<size_t>(p) * topk + j] = local ? m.w[base + j] : 0.0f;
  }
}

// kMeta: the rank-deduplicated exchange, whose first-slice wavefront of each
// token also writes the token's receiver metadata (a kernel of its own for
// it took a 4.4 us launch of the 67 us call at T=4096, H=7168, k=8).
template <bool kMeta>
__global__ __launch_bounds__(64 * kItemWaves) void dispatch_bf16_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos, int topk, int64_t rows,
    u32x4* __restrict__ out, int num_tokens, int nvec, int slices, int payload_blocks,
    RankMeta meta) {
  const int lane = threadIdx.x & 63;
  const int nitems = num_tokens * slices;
  for (int item = blockIdx.x * kItemWaves + wave_index(); item < nitems;
       item += payload_blocks * kItemWaves) {
    const int t = item / slices;
    const int slice = item - t * slices;
    const int v = slice * 64 + lane;
    const bool active = v < nvec;
    u32x4 r = {0u, 0u, 0u, 0u};
    if (active) r = x[static_cast<size_t>(t) * nvec + v];
    loaded(r);
    for (int j0 = 0; j0 < topk; j0 += kSlotBatch) {
      int p[kSlotBatch];
      load_rows(pos + static_cast<size_t>(t) * topk, j0, topk, rows, p);
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj)
        if (p[jj] >= 0 && active) store_row(&out[static_cast<size_t>(p[jj]) * nvec + v], r);
    }
    if constexpr (kMeta)
      if (slice == 0) write_rank_meta(meta, pos, t, topk, rows, lane);
  }
}

// bf16 dispatch with the slots spread over a workgroup: a workgroup is one
// (token, 512-channel slice) item, and its W = min(ceil(k/2), kSlotWaves)
// wavefronts take slots w, w + W, ... (two each at k = 8). Every wavefront
// loads the same 1 KiB of x (one HBM read; the other wavefronts of the
// workgroup find it in the cache) and stores it once per slot. A wavefront
// that issues fewer stores lets the scatter reach HBM faster: plain
// sequential writes of the same 470 MB take 73 us at one 1 KiB store per
// wavefront and 90 us at eight. One slot per wavefront is faster still while
// x is cache-resident (T=4096, H=7168: 90-92 vs 93-95 us) but 15-25% slower
// than two when x comes from HBM (T=16384, H=4096: 282 vs 219 us; T=8192,
// H=7168: 256 vs 205 us), where eight wavefronts wait on one cold load; two
// slots per wavefront is the faster of the two designs or within 2% of it
// at every shape measured, and beats one wavefront looping over all k slots
// by 3-10% once x comes from HBM.
constexpr int kSlotWaves = 8;
constexpr int kSlotsPerWave = 2;
// Under a workgroup cap the wavefronts are few, and the form above keeps one
// item in flight per four of them; looping over all k slots in one wavefront
// (dispatch_bf16_kernel) keeps four. Same-box A/B at T=4096, H=7168, k=8
// (GB/s, slots form / loop, two runs): cap 16 247-248 / 602-603, 128
// 1828-1834 / 4158-4181, 256 3423-3430 / 5565-5596, 512 5800-5935 /
// 5570-5582, 1024 5556-5610 / 5466-5617. So the loop below 512 workgroups.
constexpr int kSlotsFormMinCap = 512;

// Slots a wavefront of the slot-spread form stores: kSlotsPerWave up to
// k = 2 * kSlotWaves, at most ceil(MOE_EP_MAX_TOPK / kSlotWaves) beyond.
constexpr int kMaxSlotsPerWave = (MOE_EP_MAX_TOPK + kSlotWaves - 1) / kSlotWaves;

template <int kPer>
__global__ __launch_bounds__(64 * kSlotWaves) void dispatch_bf16_slots_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos, int topk, int64_t rows,
    u32x4* __restrict__ out, int num_tokens, int nvec, int slices, int payload_blocks) {
  const int lane = threadIdx.x & 63;
  const int waves = __builtin_amdgcn_readfirstlane(static_cast<int>(blockDim.x >> 6));
  const int w = wave_index();
  const int nitems = num_tokens * slices;
  for (int item = blockIdx.x; item < nitems; item += payload_blocks) {
    const int t = item / slices;
    const int v = (item - t * slices) * 64 + lane;
    const bool active = v < nvec;
    // The wavefront's row indices first (scalar loads), then x: both are in
    // flight together and the stores wait once. With x read from HBM this
    // measured 102.0 -> 100.8 us at T=4096, H=7168, k=8 back to back (96.6
    // -> 91.4 us as isolated launches); loaded after x, each index load
    // added its own latency to the wavefront's.
    // Unconditional loads (slot indices clamped to k-1) so that they issue
    // back to back; slots past k are then dropped.
    int p[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = w + i * waves;
      p[i] = table_row(pos, topk, rows, t, j < topk ? j : topk - 1);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (w + i * waves >= topk) p[i] = -1;
    u32x4 r = {0u, 0u, 0u, 0u};
    if (active) r = x[static_cast<size_t>(t) * nvec + v];
    loaded(r);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (p[i] >= 0 && active) store_row(&out[static_cast<size_t>(p[i]) * nvec + v], r);
  }
}

// Blocked bf16 dispatch (the standard path from kXcds dispatch blocks on; the
// layout lists each block's rows, see dispatch_block_chunks). Workgroup g
// works for XCD slot g % kXcds -- the hardware hands consecutive workgroups
// to the 8 XCDs in turn, so slot s runs on one XCD -- and the slot's
// wavefront items walk its blocks s, s + 8, ... one after another: block by
// block, row by row in ascending order, the row's 1 KiB slices side by side.
// A wavefront copies one slice of x[token] to out[row]. So one XCD writes a
// run of consecutive rows per expert at a time instead of rows of all
// experts at once, and reads its tokens' x through its own L2.
//
// Each of the slot's first wavefront items also loads one x slice of the
// slot's tokens, in token order, kBlockPrefetchItems items ahead of its own
// position, after its own store (vector loads retire in order, so a load
// ahead of the store would hold the store back until it returned): the
// slot's x then comes from HBM as one sequential burst early in the kernel
// and the copies find it in L2 or the last-level cache, where the copies
// alone would read each x row from HBM at the random moment its first row
// comes up. Measured (probes, x from HBM / x cached, us):
//   T=4096, H=7168, top-8 of 256: per-slot form 98.4-100.7 / 90.1-93.2;
//     blocks of 2 chunks (3.5 MB of x) 94.8-96.9 / 76.9-77.4 without the
//     prefetch, 91.6 / 85.3 with it (issued before the store: 92.2 / 95.0);
//     blocks of 1 chunk 91.1-92.8 / 87.7-92.2 with it; blocks of 4 chunks
//     (7 MB, more x than an L2 holds) 111; without the XCD pinning 116-133.
//   T=4096, H=2048, top-6 of 64: per-slot form 22.7-22.8 / 18.5-19.0; blocks
//     of 1 chunk 21.8 / 17.2 with the prefetch, 23.1-23.2 / 17.7 without;
//     blocks of 2 chunks (12 blocks over 8 slots) 24.2-28.0.
//   T=16384, H=4096, top-8 of 128 (16.8 MB of x per slot, more than an L2
//     holds; the burst then lands in the last-level cache), x from HBM
//     only, one box: per-slot form 218.7, blocks of 2 chunks 197.6 with the
//     prefetch, 207.0 without; with Zipf routing per-slot 203.4, blocks of 2
//     chunks 191-198 with it, 190.2 without, of 4 chunks (4 MB) 203-210.
//     T=8192, H=7168: per-slot 203.6, blocked 185.8 with it, 194.0 without.
//     T=16384, H=2048, top-6 of 64: per-slot 80.6, blocked 77.4 with it,
//     82.7 without. A prefetch spread evenly over the kernel, one block ahead,
//     was slower at every shape (112-301), and so was one where each
//     block's last items fetched the next block (88-95 at T=4096, H=7168,
//     225-246 with Zipf routing).
// A wavefront moves only 1 KiB, so its scalar work bounded the kernel at
// first: the same form with runtime divisions took 139-153 us, with a
// separate list-length load and signed guards 100 us. Hence blocks of a
// power of two chunks (a shift), one multiply-high division by the slice
// count, lists padded with (-1, -1) instead of a length, unsigned guards;
// two slices per wavefront, or one slice of 2-8 rows, measured 94-106 us.
// Past that the scalar unit no longer bounds it (the address arithmetic
// moved to the vector unit, 13 fewer scalar instructions, measured the same
// 90.5 us). Correctness never depends on where a workgroup runs.
// How far ahead (in the slot's items) the first items prefetch: same-box
// A/B, x from HBM, us at 256 / 512 / 1024 / 2048 items: T=4096, H=2048,
// top-6 21.3 / 21.2 / 22.0 / 23.7; T=4096, H=7168, top-8 90.9 / 90.9 / 90.8 /
// 91.8; T=16384, H=4096, Zipf routing 191 / 190.6 / 191.6 / 193.
constexpr int kBlockPrefetchItems = 512;

__global__ __launch_bounds__(64 * kItemWaves) void dispatch_bf16_blocks_kernel(
    const u32x4* __restrict__ x, const int2* __restrict__ order, u32x4* __restrict__ out,
    uint32_t rows, uint32_t num_tokens, int topk, int nvec, int slices, int nblocks, int bs_log2,
    int tpb, uint32_t prefetch_items, FastDiv div_slices, FastDiv div_tpb, FastDiv div_topk) {
  const int lane = threadIdx.x & 63;
  const int slot = static_cast<int>(blockIdx.x) & (kXcds - 1);
  const int li = static_cast<int>(blockIdx.x / kXcds) * kItemWaves + wave_index();
  const int ri_all = fast_div(li, div_slices);           // row of the slot's sequence
  const int sl = li - ri_all * slices;
  const int b = slot + kXcds * (ri_all >> bs_log2);
  if (b >= nblocks) return;
  const int2 rt = order[(static_cast<size_t>(b) << bs_log2) + (ri_all & ((1 << bs_log2) - 1))];
  // The copy: one unconditional load (clamped), one guarded store.
  const bool ok = static_cast<uint32_t>(rt.x) < rows && static_cast<uint32_t>(rt.y) < num_tokens;
  const int v = sl * 64 + lane;
  const int vc = v < nvec ? v : nvec - 1;
  const u32x4 r = x[static_cast<size_t>(ok ? rt.y : 0) * nvec + vc];
  loaded(r);
  if (ok && v < nvec) store_row(&out[static_cast<size_t>(rt.x) * nvec + v], r);
  // Prefetch: position li + ahead of the slot's token-order sequence of x
  // slices, tpb token positions per block (a block's slots [b*bs, (b+1)*bs)
  // span at most bs/k + 2 tokens; positions past its last token re-read it).
  const uint32_t pi = static_cast<uint32_t>(li) + kBlockPrefetchItems;
  if (pi < prefetch_items) {
    const int lt_all = fast_div(pi, div_slices);
    const int psl = static_cast<int>(pi) - lt_all * slices;
    const int pj = fast_div(lt_all, div_tpb);
    const int pb = slot + kXcds * pj;
    if (pb < nblocks) {
      const int first_slot = pb << bs_log2;
      int end_slot = first_slot + (1 << bs_log2);
      const int all_slots = static_cast<int>(num_tokens) * topk;
      end_slot = end_slot < all_slots ? end_slot : all_slots;
      int tok = static_cast<int>(fast_div(first_slot, div_topk)) + (lt_all - pj * tpb);
      const int last = fast_div(end_slot - 1, div_topk);
      tok = tok < last ? tok : last;
      int pv = psl * 64 + lane;
      pv = pv < nvec ? pv : nvec - 1;
      const u32x4 pf = x[static_cast<size_t>(tok) * nvec + pv];
      asm volatile("" ::"v"(pf));
    }
  }
}

// FP8 and MXFP8 dispatch: each wavefront also loads the x slice of the item
// kPrefetchItems items ahead (a clamped, always-valid address) and keeps it
// only until its own item is done, so that the later wavefront finds its x
// in L2. A wavefront here moves 2 KiB in and 8 KiB out and quantises in
// between, so a cold x load is a large part of its life; measured at T=4096,
// H=7168, k=8 with x read from HBM, 59.3 -> 56.5 us (x cache-resident: 47.8
// -> 47.0 us); 2048 / 3072 / 6144 items ahead gave 57.8 / 57.0 / 56.0 us
// with x from HBM and 47.1 / 47.0 / 47.4 cached. The bf16 dispatch, whose
// wavefronts carry less work each, gained nothing from it at any distance.
constexpr int kPrefetchItems = 4096;

// Lane u's 16 channels of the item kPrefetchItems ahead of `item` (or of the
// last item), read to warm L2 for that item's wavefront.
__device__ __forceinline__ void prefetch_lane16(const u32x4* __restrict__ x, int item, int nitems,
                                                int slices, int units, int hidden, int lane,
                                                u32x4& a, u32x4& b) {
  int pi = item + kPrefetchItems;
  pi = pi < nitems ? pi : nitems - 1;
  const int pt = pi / slices;
  int pu = (pi - pt * slices) * 64 + lane;
  pu = pu < units ? pu : units - 1;
  const u32x4* src = x + static_cast<size_t>(pt) * (hidden >> 3);
  a = src[2 * pu];
  b = src[2 * pu + 1];
}

// Keeps the prefetched registers alive to this point without using them, so
// that the compiler neither drops the prefetch loads nor reuses their
// registers (which would make the first wait cover them too).
__device__ __forceinline__ void retire_prefetch(const u32x4& a, const u32x4& b) {
  asm volatile("" ::"v"(a), "v"(b));
}

__global__ __launch_bounds__(64 * kItemWaves) void dispatch_fp8_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos, int topk, int64_t rows,
    u32x4* __restrict__ out,
    float* __restrict__ scales, int num_tokens, int hidden, int slices, int payload_blocks) {
  const int lane = threadIdx.x & 63;
  const int units = hidden >> 4;    // 16 channels per lane
  const int nscale = hidden >> 7;   // one scale per 128 channels
  const int nitems = num_tokens * slices;
  for (int item = blockIdx.x * kItemWaves + wave_index(); item < nitems;
       item += payload_blocks * kItemWaves) {
    const int t = item / slices;
    const int slice = item - t * slices;
    const int u = slice * 64 + lane;
    // units is a multiple of 8, so each 8-lane group is wholly active or not.
    const bool active = u < units;
    // x first (unconditional loads, clamped to the row's last unit), then
    // the prefetch and the first batch of row indices: all in flight before
    // the wait for x.
    const u32x4* xr = x + static_cast<size_t>(t) * (hidden >> 3);
    const int uc = active ? u : units - 1;
    const u32x4 a = xr[2 * uc], b = xr[2 * uc + 1];
    u32x4 pa, pb;
    prefetch_lane16(x, item, nitems, slices, units, hidden, lane, pa, pb);
    int p[kSlotBatch];
    load_rows(pos + static_cast<size_t>(t) * topk, 0, topk, rows, p);
    u32x4 q;
    float scale;
    quantize_fp8(a, b, q, scale);
    const bool scale_lane = active && (lane & 7) == 0;
    for (int j0 = 0; j0 < topk; j0 += kSlotBatch) {
      if (j0 > 0) load_rows(pos + static_cast<size_t>(t) * topk, j0, topk, rows, p);
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj) {
        if (p[jj] < 0) continue;
        if (active) store_row(&out[static_cast<size_t>(p[jj]) * units + u], q);
        if (scale_lane) scales[static_cast<size_t>(p[jj]) * nscale + (u >> 3)] = scale;
      }
    }
    retire_prefetch(pa, pb);
  }
}

__global__ __launch_bounds__(64 * kItemWaves) void dispatch_mxfp8_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pos, int topk, int64_t rows,
    u32x4* __restrict__ out,
    uint32_t* __restrict__ scales, int num_tokens, int hidden, int slices, int payload_blocks) {
  const int lane = threadIdx.x & 63;
  const int units = hidden >> 4;           // 16 channels per lane
  const int scale_words = hidden >> 7;     // 4 one-byte scales per dword, per row
  const int nitems = num_tokens * slices;
  for (int item = blockIdx.x * kItemWaves + wave_index(); item < nitems;
       item += payload_blocks * kItemWaves) {
    const int t = item / slices;
    const int slice = item - t * slices;
    const int u = slice * 64 + lane;
    // units is a multiple of 8, so each 8-lane group is wholly active or not.
    const bool active = u < units;
    // As in the FP8 kernel: x, the prefetch and the first row indices in
    // flight together.
    const u32x4* xr = x + static_cast<size_t>(t) * (hidden >> 3);
    const int uc = active ? u : units - 1;
    const u32x4 a = xr[2 * uc], b = xr[2 * uc + 1];
    u32x4 pa, pb;
    prefetch_lane16(x, item, nitems, slices, units, hidden, lane, pa, pb);
    int p[kSlotBatch];
    load_rows(pos + static_cast<size_t>(t) * topk, 0, topk, rows, p);
    u32x4 q;
    uint32_t word;
    quantize_mxfp8(a, b, lane, q, word);
    const bool scale_lane = active && (lane & 7) == 0;
    for (int j0 = 0; j0 < topk; j0 += kSlotBatch) {
      if (j0 > 0) load_rows(pos + static_cast<size_t>(t) * topk, j0, topk, rows, p);
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj) {
        if (p[jj] < 0) continue;
        if (active) store_row(&out[static_cast<size_t>(p[jj]) * units + u], q);
        if (scale_lane) scales[static_cast<size_t>(p[jj]) * scale_words + (u >> 3)] = word;
      }
    }
    retire_prefetch(pa, pb);
  }
}

// Decode-time (fixed-capacity) layout: expert e owns rows [e*C, (e+1)*C); a
// slot's row is e*C plus its rank among the slots routed to e in (token,
// slot) order, or -1 from rank C on (dropped).
constexpr int kRankLoads = 16;
constexpr int kCountLoads = 8;
constexpr int kFixedWaves = 4;   // wavefronts (column slices) per decode-time workgroup
constexpr int kFixedSharedFrom = 256;   // tokens from which a workgroup shares the rank count

// Layout computed inside the dispatch kernel, in one of two forms:
//   fixed capacity (kPacked = false): expert e owns rows [e*C, (e+1)*C); a
//     slot's row is e*C + r, r = earlier slots with its id, dropped from C on;
//   packed (kPacked = true): the standard layout -- a slot's row is the number
//     of valid slots with a smaller id plus r, so expert e's rows start at
//     offsets_e[e] -- exactly what the layout kernels produce.
template <bool kPacked>
struct FusedLayout {
  const int32_t* idx;   // [T, k] expert ids
  int topk, num_experts, capacity;   // capacity: fixed form only
  int32_t* pos;         // [T, k] rows, recorded for combine
  int32_t* counts;      // [E] rows per expert (at most C in the fixed form)
  int32_t* status;      // fixed: invalid, placed, T, dropped; packed: invalid, rows, T, 0
  // packed form only
  int32_t* offsets;        // [E + 1]
  int32_t* group_counts;   // [R]
  int32_t* group_offsets;  // [R + 1]
  int32_t* src;            // [T * k] token of each row, -1 past the valid total
  int num_groups;          // R
  int per_group;           // E / R

  // Per-lane counts for slots j0 .. j0+kSlotBatch-1 of token t (ids e[]),
  // one packed counter per slot: low 16 bits = earlier slots with the same
  // id, high 16 bits (packed form) = valid slots with a smaller id (both below
  // 2^15 since T*k <= MOE_EP_LL_MAX_TOKENS * MOE_EP_MAX_TOPK). The ids are
  // read in chunks of 64, strided by `waves` wavefronts starting at chunk
  // `wave` (kRankLoads chunks in flight), over the earlier tokens' slots
  // [0, t*k) -- or all slots for the packed form; wavefront 0 adds the
  // token's own earlier slots (`own`: this token's id of slot `lane`).
  __device__ __forceinline__ void count_batch(int t, int j0, int wave, int waves, int own,
                                              int slots, const int (&e)[kSlotBatch],
                                              uint32_t (&cnt)[kSlotBatch]) const {
    const int base = t * topk;
    const int lane = threadIdx.x & 63;
    const int end = kPacked ? slots : base;
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) cnt[jj] = 0u;
    const int stride = waves * 64;
    for (int c = wave * 64; c < end; c += stride * kRankLoads) {
      int id[kRankLoads];
#pragma unroll
      for (int q = 0; q < kRankLoads; ++q) {
        const int s = c + q * stride + lane;
        id[q] = idx[s < end ? s : 0];
        if (s >= end) id[q] = -1;
      }
#pragma unroll
      for (int q = 0; q < kRankLoads; ++q) {
        const bool earlier = c + q * stride + lane < base;
#pragma unroll
        for (int jj = 0; jj < kSlotBatch; ++jj) {
          if (kPacked) {
            cnt[jj] += (earlier && id[q] == e[jj]) ? 1u : 0u;
            cnt[jj] += static_cast<unsigned>(id[q]) < static_cast<unsigned>(e[jj]) ? 0x10000u : 0u;
          } else {
            cnt[jj] += id[q] == e[jj] ? 1u : 0u;
          }
        }
      }
    }
    if (wave == 0) {
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj)
        cnt[jj] += (lane < j0 + jj && own == e[jj]) ? 1u : 0u;
    }
  }

  __device__ __forceinline__ void batch_ids(int t, int j0, int (&e)[kSlotBatch]) const {
    const int base = t * topk;
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj)
      e[jj] = idx[base + (j0 + jj < topk ? j0 + jj : topk - 1)];
  }

  // Row of a slot with id e from its summed counter, or -1.
  __device__ __forceinline__ int row_of(int e, uint32_t sum) const {
    if (static_cast<unsigned>(e) >= static_cast<unsigned>(num_experts)) return -1;
    const int same = static_cast<int>(sum & 0xFFFFu);
    if (kPacked) return static_cast<int>(sum >> 16) + same;
    return same < capacity ? e * capacity + same : -1;
  }

  // Record slot j of token t at row p (the one wavefront or thread that owns it).
  __device__ __forceinline__ void record(int t, int j, int p) const {
    pos[t * topk + j] = p;
    if (kPacked && p >= 0) src[p] = t;
  }

  // This wavefront's share of the counters of token t's slots (one of
  // `waves`), summed over its lanes into part[slot]. Returns this token's id
  // of slot `lane` (lanes < topk).
  __device__ __forceinline__ int rank_share(int t, int wave, int waves, int slots,
                                            int32_t* part) const {
    const int lane = threadIdx.x & 63;
    const int own = idx[t * topk + (lane < topk ? lane : 0)];
    for (int j0 = 0; j0 < topk; j0 += kSlotBatch) {
      int e[kSlotBatch];
      uint32_t cnt[kSlotBatch];
      batch_ids(t, j0, e);
      count_batch(t, j0, wave, waves, own, slots, e, cnt);
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj) {
        const uint32_t sum = wave_sum_u32(cnt[jj]);
        if (lane == 0 && j0 + jj < topk) part[j0 + jj] = static_cast<int32_t>(sum);
      }
    }
    return own;
  }

  // Run by the grid's last workgroup: histogram of all slots in LDS, then the
  // per-expert counts and the status words; in the packed form also the
  // exclusive scan over experts, the per-rank counts and offsets, and -1 for
  // the row sources past the valid total.
  __device__ void counts_block(int num_tokens) const {
    __shared__ int hist[MOE_EP_MAX_EXPERTS];
    __shared__ int tally[2];   // invalid slots, dropped slots
    __shared__ int s_wsum[kFixedWaves];
    const int tid = threadIdx.x, nthreads = blockDim.x;
    for (int e = tid; e < num_experts; e += nthreads) hist[e] = 0;
    if (tid < 2) tally[tid] = 0;
    __syncthreads();
    const int slots = num_tokens * topk;
    int bad = 0;
    // kCountLoads ids per thread are loaded before any is counted, so the
    // loads overlap instead of each waiting on the one before.
    for (int base = 0; base < slots; base += nthreads * kCountLoads) {
      int id[kCountLoads];
#pragma unroll
      for (int q = 0; q < kCountLoads; ++q) {
        const int s = base + q * nthreads + tid;
        id[q] = s < slots ? idx[s] : 0;
      }
#pragma unroll
      for (int q = 0; q < kCountLoads; ++q) {
        if (base + q * nthreads + tid >= slots) continue;
        if (static_cast<unsigned>(id[q]) < static_cast<unsigned>(num_experts))
          atomicAdd(&hist[id[q]], 1);
        else
          ++bad;
      }
    }
    if (bad) atomicAdd(&tally[0], bad);
    __syncthreads();
    if (!kPacked) {
      int drop = 0;
      for (int e = tid; e < num_experts; e += nthreads) {
        const int c = hist[e];
        counts[e] = c < capacity ? c : capacity;
        drop += c > capacity ? c - capacity : 0;
      }
      if (drop) atomicAdd(&tally[1], drop);
      __syncthreads();
      if (tid == 0) {
        status[0] = tally[0];
        status[1] = slots - tally[0] - tally[1];
        status[2] = num_tokens;
        status[3] = tally[1];
      }
      return;
    }
    // Exclusive scan over experts: thread tid sums experts [tid*c, tid*c + c),
    // c = ceil(E / nthreads) <= 4; a wavefront scan and the wavefront totals
    // give each thread its start.
    const int lane = tid & 63, wave = tid >> 6;
    const int c = (num_experts + nthreads - 1) / nthreads;
    const int e0 = tid * c;
    int local = 0;
    for (int e = e0; e < e0 + c && e < num_experts; ++e) local += hist[e];
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(incl, d, 64);
      if (lane >= d) incl += up;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wave; ++w) run += s_wsum[w];
    int total = 0;
    for (int w = 0; w < nthreads / 64; ++w) total += s_wsum[w];
    __syncthreads();   // everyone has read s_wsum and hist[e0 .. e0+c)
    for (int e = e0; e < e0 + c && e < num_experts; ++e) {
      const int n = hist[e];
      counts[e] = n;
      offsets[e] = run;
      hist[e] = run;   // keep the offsets for the per-rank figures
      run += n;
    }
    __syncthreads();
    for (int r = tid; r < num_groups; r += nthreads) {
      const int a = hist[r * per_group];
      const int b = r + 1 < num_groups ? hist[(r + 1) * per_group] : total;
      group_counts[r] = b - a;
      group_offsets[r] = a;
    }
    for (int p = total + tid; p < slots; p += nthreads) src[p] = -1;
    if (tid == 0) {
      offsets[num_experts] = total;
      group_offsets[num_groups] = total;
      status[0] = tally[0];
      status[1] = total;
      status[2] = num_tokens;
      status[3] = 0;
    }
  }
};
// Fused-layout rows computed by one wavefront alone (small batches): the whole
// count, no LDS and no barrier. `record` makes it store the token's rows
// (one wavefront per token does).
template <bool kPacked>
struct WaveRows {
  FusedLayout<kPacked> fl;
  int slots;
  bool record;
  __device__ __forceinline__ void rows_of(int t, int j0, int (&p)[kSlotBatch]) const {
    const int lane = threadIdx.x & 63;
    const int topk = fl.topk;
    const int own = fl.idx[t * topk + (lane < topk ? lane : 0)];
    int e[kSlotBatch];
    uint32_t cnt[kSlotBatch];
    fl.batch_ids(t, j0, e);
    fl.count_batch(t, j0, 0, 1, own, slots, e, cnt);
    int mine = -1;
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) {
      const uint32_t sum = wave_sum_u32(cnt[jj]);
      p[jj] = j0 + jj < topk ? fl.row_of(e[jj], sum) : -1;
      if (lane == jj) mine = p[jj];
    }
    if (record && lane < kSlotBatch && j0 + lane < topk) fl.record(t, j0 + lane, mine);
  }
};

// Dispatch with the layout computed in the same launch: a workgroup of
// kFixedWaves wavefronts takes one (token, group of kFixedWaves column
// slices) item, looping over items when the grid is capped; each wavefront
// moves one slice, and the group holding slice 0 records the token's rows.
// kShared: the wavefronts split the count and add their shares through LDS
// (larger batches); otherwise each counts alone (no barrier). The grid's last
// workgroup publishes the counts. No workgroup waits for another.
template <int kDtype, bool kPacked, bool kShared>
__global__ __launch_bounds__(64 * kFixedWaves) void dispatch_fused_kernel(
    const u32x4* __restrict__ x, FusedLayout<kPacked> fl, u32x4* __restrict__ out,
    ScalePtr<kDtype> __restrict__ scales, int num_tokens, int hidden, int slices, int groups,
    int work_blocks) {
  __shared__ int32_t s_part[kFixedWaves][MOE_EP_MAX_TOPK];
  __shared__ int32_t s_pos[MOE_EP_MAX_TOPK];
  if (static_cast<int>(blockIdx.x) == work_blocks) {
    fl.counts_block(num_tokens);
    return;
  }
  const int wave = wave_index();
  const int topk = fl.topk;
  const int nitems = num_tokens * groups;
  const int slots = num_tokens * topk;
  if constexpr (!kShared) {   // each wavefront ranks its token's slots itself
    for (int item = blockIdx.x; item < nitems; item += work_blocks) {
      const int t = item / groups;
      const int slice = (item - t * groups) * kFixedWaves + wave;
      if (slice >= slices) continue;
      const WaveRows<kPacked> rows{fl, slots, slice == 0};
      payload_item<kDtype>(x, rows, out, scales, t, slice, hidden, topk);
    }
    return;
  }
  const SharedRows rows{s_pos, topk};
  for (int item = blockIdx.x; item < nitems; item += work_blocks) {
    const int t = item / groups;
    const int g = item - t * groups;
    const int own = fl.rank_share(t, wave, kFixedWaves, slots, s_part[wave]);
    __syncthreads();
    const int j = threadIdx.x;   // lanes 0 .. topk-1 of wavefront 0, which hold the ids
    if (j < topk) {
      uint32_t sum = 0u;
#pragma unroll
      for (int w = 0; w < kFixedWaves; ++w) sum += static_cast<uint32_t>(s_part[w][j]);
      const int p = fl.row_of(own, sum);
      s_pos[j] = p;
      if (g == 0) fl.record(t, j, p);
    }
    __syncthreads();
    const int slice = g * kFixedWaves + wave;
    if (slice < slices) payload_item<kDtype>(x, rows, out, scales, t, slice, hidden, topk);
    __syncthreads();   // s_part and s_pos are rewritten for the next item
  }
}

}  // namespace

hipError_t launch_dispatch(int dtype, const void* d_x, const int32_t* d_pos, void* d_out,
                           void* d_scales, int64_t rows, int num_tokens, int topk, int hidden,
                           int max_blocks, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int slices = (hidden / lane_channels(dtype) + 63) / 64;
  const dim3 grid = item_grid(int64_t(num_tokens) * slices, max_blocks), block(64 * kItemWaves);
  const int payload = static_cast<int>(grid.x);
  const u32x4* x = static_cast<const u32x4*>(d_x);
  u32x4* out = static_cast<u32x4*>(d_out);
  if (dtype == MOE_DTYPE_BF16 && max_blocks > 0 && max_blocks < kSlotsFormMinCap &&
      int64_t(max_blocks) * kItemWaves < int64_t(num_tokens) * slices) {
    // Capped below kSlotsFormMinCap workgroups: each wavefront takes one item
    // and all of its k slots.
    hipLaunchKernelGGL(dispatch_bf16_kernel<false>, grid, block, 0, stream, x, d_pos, topk, rows,
                       out, num_tokens, hidden / 8, slices, payload, RankMeta{});
  } else if (dtype == MOE_DTYPE_BF16) {
    // One workgroup of min(ceil(k / kSlotsPerWave), kSlotWaves) wavefronts
    // per item; a cap keeps the wavefront count of max_blocks workgroups of
    // kItemWaves.
    const int want = (topk + kSlotsPerWave - 1) / kSlotsPerWave;
    const int waves = want < kSlotWaves ? want : kSlotWaves;
    // Every slot belongs to one of the waves' entries (topk <= MOE_EP_MAX_TOPK,
    // checked at handle creation): kSlotsPerWave each while waves covers
    // ceil(k / 2), kMaxSlotsPerWave once waves is capped at kSlotWaves.
    const int per = waves * kSlotsPerWave >= topk ? kSlotsPerWave : kMaxSlotsPerWave;
    if (waves * per < topk) return hipErrorInvalidValue;
    int64_t blocks = int64_t(num_tokens) * slices;
    if (max_blocks > 0) {
      int64_t cap = int64_t(max_blocks) * kItemWaves / waves;
      if (cap < 1) cap = 1;
      if (blocks > cap) blocks = cap;
    }
    if (per == kSlotsPerWave)
      hipLaunchKernelGGL(dispatch_bf16_slots_kernel<kSlotsPerWave>,
                         dim3(static_cast<unsigned>(blocks)), dim3(64 * waves), 0, stream, x, d_pos,
                         topk, rows, out, num_tokens, hidden / 8, slices, static_cast<int>(blocks));
    else
      hipLaunchKernelGGL(dispatch_bf16_slots_kernel<kMaxSlotsPerWave>,
                         dim3(static_cast<unsigned>(blocks)), dim3(64 * waves), 0, stream, x, d_pos,
                         topk, rows, out, num_tokens, hidden / 8, slices, static_cast<int>(blocks));
  } else if (dtype == MOE_DTYPE_FP8_E4M3)
    hipLaunchKernelGGL(dispatch_fp8_kernel, grid, block, 0, stream, x, d_pos, topk, rows, out,
                       static_cast<float*>(d_scales), num_tokens, hidden, slices, payload);
  else
    hipLaunchKernelGGL(dispatch_mxfp8_kernel, grid, block, 0, stream, x, d_pos, topk, rows, out,
                       static_cast<uint32_t*>(d_scales), num_tokens, hidden, slices, payload);
  return hipGetLastError();
}

hipError_t launch_dispatch_blocks(const void* d_x, const int2* d_order, void* d_out, int64_t rows,
                                  int num_tokens, int topk, int hidden, int block_chunks,
                                  hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int chunks = layout_blocks(int64_t(num_tokens) * topk);
  // The lists hold (chunks + chunks / kXcds + 1) * kLayoutChunk entries: a
  // block of more than chunks / kXcds chunks could run past them.
  if (d_order == nullptr || block_chunks <= 0 || block_chunks > chunks / kXcds ||
      (block_chunks & (block_chunks - 1)) != 0)
    return hipErrorInvalidValue;
  const int nvec = hidden / 8;
  const int slices = (nvec + 63) / 64;
  const int bs = block_chunks * kLayoutChunk;
  int bs_log2 = 0;
  while ((1 << bs_log2) < bs) ++bs_log2;
  const int nblocks = (chunks + block_chunks - 1) / block_chunks;
  const int per_slot = (nblocks + kXcds - 1) / kXcds;
  const int tpb = bs / topk + 2;
  // Every index the kernel forms stays below 2^31 (fast_div's range).
  const int64_t slot_items = int64_t(per_slot) * bs * slices;
  // The early burst of x only while the batch's x leaves room in the
  // last-level cache (kPrefetchMaxXBytes).
  const int64_t prefetch_items =
      int64_t(num_tokens) * 2 * hidden > kPrefetchMaxXBytes ? 0 : int64_t(per_slot) * tpb * slices;
  if (slot_items + kItemWaves > 0x7FFFFFFF || prefetch_items > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int64_t grid = (slot_items + kItemWaves - 1) / kItemWaves * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const uint32_t rows32 = rows < 0x7FFFFFFF ? static_cast<uint32_t>(rows) : 0x7FFFFFFFu;
  hipLaunchKernelGGL(dispatch_bf16_blocks_kernel, dim3(static_cast<unsigned>(grid)),
                     dim3(64 * kItemWaves), 0, stream, static_cast<const u32x4*>(d_x), d_order,
                     static_cast<u32x4*>(d_out), rows32, static_cast<uint32_t>(num_tokens), topk,
                     nvec, slices, nblocks, bs_log2, tpb, static_cast<uint32_t>(prefetch_items),
                     make_fast_div(slices), make_fast_div(tpb), make_fast_div(topk));
  return hipGetLastError();
}

hipError_t launch_dispatch_ranks(const void* d_x, const int32_t* d_slot_row, void* d_out,
                                 int64_t rows, int num_tokens, int topk, int hidden,
                                 int max_blocks, const int32_t* d_idx, const float* d_w,
                                 int num_experts, int num_ranks, int32_t* d_recv_idx,
                                 float* d_recv_w, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int slices = (hidden / 8 + 63) / 64;
  const dim3 grid = item_grid(int64_t(num_tokens) * slices, max_blocks), block(64 * kItemWaves);
  const RankMeta meta{d_idx, d_w, num_experts, num_experts / num_ranks, d_recv_idx, d_recv_w};
  hipLaunchKernelGGL(dispatch_bf16_kernel<true>, grid, block, 0, stream,
                     static_cast<const u32x4*>(d_x), d_slot_row, topk, rows,
                     static_cast<u32x4*>(d_out), num_tokens, hidden / 8, slices,
                     static_cast<int>(grid.x), meta);
  return hipGetLastError();
}

namespace {

template <bool kPacked>
hipError_t launch_fused(int dtype, const void* d_x, const FusedLayout<kPacked>& fl,
                        int num_tokens, void* d_out, void* d_scales, int hidden, int max_blocks,
                        hipStream_t stream) {
  const int slices = (hidden / lane_channels(dtype) + 63) / 64;
  const int groups = (slices + kFixedWaves - 1) / kFixedWaves;
  int work_blocks = num_tokens * groups;
  if (max_blocks > 0 && work_blocks > max_blocks) work_blocks = max_blocks;
  const dim3 grid(work_blocks + 1), block(64 * kFixedWaves);   // + the counts workgroup
  const u32x4* x = static_cast<const u32x4*>(d_x);
  u32x4* out = static_cast<u32x4*>(d_out);
  // Below kFixedSharedFrom tokens each wavefront ranks its slots alone (no
  // barrier); from there on a workgroup's wavefronts share the count.
  const bool shared = num_tokens >= kFixedSharedFrom;
#define MOE_FUSED_LAUNCH(DT, SHARED, SCALES)                                                     \
  hipLaunchKernelGGL((dispatch_fused_kernel<DT, kPacked, SHARED>), grid, block, 0, stream, x, fl, \
                     out, static_cast<SCALES*>(d_scales), num_tokens, hidden, slices, groups,     \
                     work_blocks)
  if (dtype == MOE_DTYPE_BF16) {
    if (shared) MOE_FUSED_LAUNCH(MOE_DTYPE_BF16, true, float);
    else MOE_FUSED_LAUNCH(MOE_DTYPE_BF16, false, float);
  } else if (dtype == MOE_DTYPE_FP8_E4M3) {
    if (shared) MOE_FUSED_LAUNCH(MOE_DTYPE_FP8_E4M3, true, float);
    else MOE_FUSED_LAUNCH(MOE_DTYPE_FP8_E4M3, false, float);
  } else {
    if (shared) MOE_FUSED_LAUNCH(MOE_DTYPE_MXFP8_E4M3, true, uint32_t);
    else MOE_FUSED_LAUNCH(MOE_DTYPE_MXFP8_E4M3, false, uint32_t);
  }
#undef MOE_FUSED_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch_fixed(int dtype, const void* d_x, const int32_t* d_idx,
                                 int num_tokens, int topk, int num_experts, int capacity,
                                 int32_t* d_pos, int32_t* d_counts, int32_t* d_status,
                                 void* d_out, void* d_scales, int hidden, int max_blocks,
                                 hipStream_t stream) {
  const FusedLayout<false> fl{d_idx, topk, num_experts, capacity, d_pos, d_counts, d_status,
                              nullptr, nullptr, nullptr, nullptr, 0, 1};
  return launch_fused(dtype, d_x, fl, num_tokens, d_out, d_scales, hidden, max_blocks, stream);
}

hipError_t launch_layout_dispatch(int dtype, const void* d_x, const int32_t* d_idx,
                                  int num_tokens, int topk, int num_experts, int num_ranks,
                                  const LayoutArrays& a, void* d_out, void* d_scales, int hidden,
                                  int max_blocks, hipStream_t stream) {
  const FusedLayout<true> fl{d_idx, topk, num_experts, 0, a.pos, a.counts_e, a.status,
                             a.offsets_e, a.counts_r, a.offsets_r, a.src_idx, num_ranks,
                             num_experts / num_ranks};
  return launch_fused(dtype, d_x, fl, num_tokens, d_out, d_scales, hidden, max_blocks, stream);
}

}  // namespace moe
