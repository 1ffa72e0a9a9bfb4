// Dispatch: scatter each token row to the k rows its layout assigned.
//
// Per the pages, dispatch "sends tokens to their assigned experts" ("Inside
// the Nebius + PyTorch DeepSeek V3 recipe", section "Mixture-of-experts and
// wide expert parallelism") into buffers preallocated for the worst case
// (Hybrid-EP news item, "Availability and Integration"), optionally as FP8
// ("MoE / Hybrid-EP Validation", "Communication path comparison" and "FP8
// dispatch restriction").
//
// Work decomposition: every wavefront is an independent work item, one
// (token, column slice) pair, and a workgroup is just kItemWaves such items.
// The Hybrid-EP news item ("Technical Structure") describes each CUDA block
// as an independent channel with no cross-block synchronisation; here the
// independent unit is the 64-lane wavefront, which has no barrier at all.
// A wavefront fetches the token's k row indices with scalar loads up front,
// reads its slice of the token row from HBM once (16 bytes per lane, so 1 KiB
// per wavefront for bf16), and writes it to the k destination rows with
// 16-byte stores. No two wavefronts write the same bytes: no atomics.
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
// is clamped to +-448 first: it can exceed 448 by at most one fp32 ulp, which
// rounds to 448 anyway, and the clamp keeps the conversion away from its
// overflow handling. A block whose amax is 0 gets scale 0 and its
// signed-zero inputs as codes.
//
// Decode-time (fixed-capacity) dispatch does layout and payload in one launch.
// DeepEP's second kernel family serves decode ("Inside the Nebius + PyTorch
// DeepSeek V3 recipe", section "DeepEP"); its receive buffers have a shape
// that does not depend on the routing. Here expert e owns rows
// [e*C, (e+1)*C); a slot's row is e*C plus its stable rank among the slots
// routed to e (token order, then slot order), and slots ranked C or more are
// dropped. Each wavefront computes the ranks of its own token's slots by
// counting matching ids among all earlier slots (one coalesced load and one
// ballot per 64 slots and slot), so no workgroup waits for another; the last
// workgroup of the grid builds the per-expert histogram in LDS and publishes
// counts and status. The counting costs O(T*k) per wavefront, which is why
// this path is limited to small batches (MOE_EP_LL_MAX_TOKENS).
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

// Where a payload kernel finds the destination rows of token t's slots.
// rows_of fills p[] for slots j0 .. j0+kSlotBatch-1 (-1: no row); `record`
// is true for exactly one wavefront per token (its first column slice).

// Standard layout: the table pos[T, k] written by the layout kernels.
struct TableRows {
  static constexpr bool kCountsBlock = false;
  const int32_t* pos;
  int topk;
  int64_t rows;
  __device__ __forceinline__ void rows_of(int t, int j0, bool, int (&p)[kSlotBatch]) const {
    load_rows(pos + static_cast<size_t>(t) * topk, j0, topk, rows, p);
  }
  __device__ void counts_block(int) const {}
};

// Fixed-capacity layout, computed on the fly (decode-time dispatch).
constexpr int kRankLoads = 16;
constexpr int kCountLoads = 8;
struct FixedCapacityRows {
  static constexpr bool kCountsBlock = true;
  const int32_t* idx;   // [T, k] expert ids
  int topk, num_experts, capacity;
  int32_t* pos;         // [T, k] rows, recorded for combine
  int32_t* counts;      // [E] rows received per expert
  int32_t* status;      // [4] invalid, placed, T, dropped

  __device__ __forceinline__ void rows_of(int t, int j0, bool record, int (&p)[kSlotBatch]) const {
    const int base = t * topk;
    int e[kSlotBatch], rank[kSlotBatch];
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) {
      e[jj] = idx[base + (j0 + jj < topk ? j0 + jj : topk - 1)];
      rank[jj] = 0;
    }
    // Rank of slot (t, j) = number of earlier slots with the same id: the
    // slots of earlier tokens, [0, base), plus slots j' < j of this token.
    // Each lane counts matches in its registers (one compare and one add per
    // id and slot; kRankLoads chunks of 64 ids in flight), then one wavefront
    // sum per slot.
    const int lane = threadIdx.x & 63;
    uint32_t cnt[kSlotBatch];
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) cnt[jj] = 0u;
    for (int c = 0; c < base; c += 64 * kRankLoads) {
      int id[kRankLoads];
#pragma unroll
      for (int q = 0; q < kRankLoads; ++q) {
        const int s = c + q * 64 + lane;
        id[q] = idx[s < base ? s : 0];
        if (s >= base) id[q] = -1;
      }
#pragma unroll
      for (int q = 0; q < kRankLoads; ++q)
#pragma unroll
        for (int jj = 0; jj < kSlotBatch; ++jj) cnt[jj] += id[q] == e[jj] ? 1u : 0u;
    }
    const int own = idx[base + (lane < topk ? lane : 0)];   // this token's ids, lanes < topk
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) {
      cnt[jj] += (lane < j0 + jj && own == e[jj]) ? 1u : 0u;
      rank[jj] = static_cast<int>(wave_sum_u32(cnt[jj]));
    }
    int mine = -1;
#pragma unroll
    for (int jj = 0; jj < kSlotBatch; ++jj) {
      const bool ok = j0 + jj < topk && static_cast<unsigned>(e[jj]) <
                      static_cast<unsigned>(num_experts) && rank[jj] < capacity;
      p[jj] = ok ? e[jj] * capacity + rank[jj] : -1;
      if (lane == jj) mine = p[jj];
    }
    if (record && lane < kSlotBatch && j0 + lane < topk) pos[base + j0 + lane] = mine;
  }

  // Run by the grid's last workgroup: histogram of all slots in LDS, then
  // per-expert counts (clamped to the capacity) and the status words.
  __device__ void counts_block(int num_tokens) const {
    __shared__ int hist[MOE_EP_MAX_EXPERTS];
    __shared__ int tally[2];   // invalid slots, dropped slots
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
  }
};

// Payload kernels. Workgroups [0, payload_blocks) run the (token, slice)
// items; with a FixedCapacityRows source one more workgroup follows and
// publishes the counts.
template <class Rows>
__global__ __launch_bounds__(64 * kItemWaves) void dispatch_bf16_kernel(
    const u32x4* __restrict__ x, Rows src_rows, u32x4* __restrict__ out, int num_tokens,
    int nvec, int slices, int payload_blocks) {
  if constexpr (Rows::kCountsBlock) {
    if (static_cast<int>(blockIdx.x) == payload_blocks) {
      src_rows.counts_block(num_tokens);
      return;
    }
  }
  const int lane = threadIdx.x & 63;
  const int nitems = num_tokens * slices;
  const int topk = src_rows.topk;
  for (int item = blockIdx.x * kItemWaves + wave_index(); item < nitems;
       item += payload_blocks * kItemWaves) {
    const int t = item / slices;
    const int slice = item - t * slices;
    const int v = slice * 64 + lane;
    const bool active = v < nvec;
    u32x4 r = {0u, 0u, 0u, 0u};
    if (active) r = x[static_cast<size_t>(t) * nvec + v];
    for (int j0 = 0; j0 < topk; j0 += kSlotBatch) {
      int p[kSlotBatch];
      src_rows.rows_of(t, j0, slice == 0, p);
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj)
        if (p[jj] >= 0 && active) store_row(&out[static_cast<size_t>(p[jj]) * nvec + v], r);
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

template <class Rows>
__global__ __launch_bounds__(64 * kItemWaves) void dispatch_fp8_kernel(
    const u32x4* __restrict__ x, Rows src_rows, u32x4* __restrict__ out,
    float* __restrict__ scales, int num_tokens, int hidden, int slices, int payload_blocks) {
  if constexpr (Rows::kCountsBlock) {
    if (static_cast<int>(blockIdx.x) == payload_blocks) {
      src_rows.counts_block(num_tokens);
      return;
    }
  }
  const int lane = threadIdx.x & 63;
  const int units = hidden >> 4;    // 16 channels per lane
  const int nscale = hidden >> 7;   // one scale per 128 channels
  const int nitems = num_tokens * slices;
  const int topk = src_rows.topk;
  for (int item = blockIdx.x * kItemWaves + wave_index(); item < nitems;
       item += payload_blocks * kItemWaves) {
    const int t = item / slices;
    const int slice = item - t * slices;
    const int u = slice * 64 + lane;
    // units is a multiple of 8, so each 8-lane group is wholly active or not.
    const bool active = u < units;
    const u32x4* src = x + static_cast<size_t>(t) * (hidden >> 3);
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (active) {
      a = src[2 * u];
      b = src[2 * u + 1];
    }
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
    const bool scale_lane = active && (lane & 7) == 0;
    for (int j0 = 0; j0 < topk; j0 += kSlotBatch) {
      int p[kSlotBatch];
      src_rows.rows_of(t, j0, slice == 0, p);
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj) {
        if (p[jj] < 0) continue;
        if (active) store_row(&out[static_cast<size_t>(p[jj]) * units + u], q);
        if (scale_lane) scales[static_cast<size_t>(p[jj]) * nscale + (u >> 3)] = scale;
      }
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
__global__ __launch_bounds__(64 * kItemWaves) void dispatch_mxfp8_kernel(
    const u32x4* __restrict__ x, Rows src_rows, u32x4* __restrict__ out,
    uint32_t* __restrict__ scales, int num_tokens, int hidden, int slices, int payload_blocks) {
  if constexpr (Rows::kCountsBlock) {
    if (static_cast<int>(blockIdx.x) == payload_blocks) {
      src_rows.counts_block(num_tokens);
      return;
    }
  }
  const int lane = threadIdx.x & 63;
  const int units = hidden >> 4;           // 16 channels per lane
  const int scale_words = hidden >> 7;     // 4 one-byte scales per dword, per row
  const int nitems = num_tokens * slices;
  const int topk = src_rows.topk;
  for (int item = blockIdx.x * kItemWaves + wave_index(); item < nitems;
       item += payload_blocks * kItemWaves) {
    const int t = item / slices;
    const int slice = item - t * slices;
    const int u = slice * 64 + lane;
    // units is a multiple of 8, so each 8-lane group is wholly active or not.
    const bool active = u < units;
    const u32x4* src = x + static_cast<size_t>(t) * (hidden >> 3);
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (active) {
      a = src[2 * u];
      b = src[2 * u + 1];
    }
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
    for (int i = 0; i < 16; ++i) f[i] = __builtin_amdgcn_fmed3f(f[i] * inv, -448.0f, 448.0f);
    u32x4 q;
    q.x = pack_e4m3(f[0], f[1], f[2], f[3]);
    q.y = pack_e4m3(f[4], f[5], f[6], f[7]);
    q.z = pack_e4m3(f[8], f[9], f[10], f[11]);
    q.w = pack_e4m3(f[12], f[13], f[14], f[15]);
    // Lane 8i gathers the codes of blocks u/2 .. u/2+3 (lanes 8i, 8i+2, 8i+4, 8i+6).
    const uint32_t code = static_cast<uint32_t>(shared + 127);
    const uint32_t c1 = __shfl(code, lane + 2, 64);
    const uint32_t c2 = __shfl(code, lane + 4, 64);
    const uint32_t c3 = __shfl(code, lane + 6, 64);
    const uint32_t word = code | (c1 << 8) | (c2 << 16) | (c3 << 24);
    const bool scale_lane = active && (lane & 7) == 0;
    for (int j0 = 0; j0 < topk; j0 += kSlotBatch) {
      int p[kSlotBatch];
      src_rows.rows_of(t, j0, slice == 0, p);
#pragma unroll
      for (int jj = 0; jj < kSlotBatch; ++jj) {
        if (p[jj] < 0) continue;
        if (active) store_row(&out[static_cast<size_t>(p[jj]) * units + u], q);
        if (scale_lane) scales[static_cast<size_t>(p[jj]) * scale_words + (u >> 3)] = word;
      }
    }
  }
}

// Receiver metadata of the rank-deduplicated exchange. One thread per slot
// (t, j): for each (token, rank) row p of token t (opened by slot jr), entry
// (p, j) says whether slot j's expert lives on that row's rank -- its local id
// e - r*E/R and its weight -- or not (-1 and 0).
__global__ __launch_bounds__(256) void rank_meta_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w,
    const int32_t* __restrict__ slot_row, int num_tokens, int topk, int num_experts,
    int per_rank, int64_t rows, int32_t* __restrict__ recv_idx, float* __restrict__ recv_w) {
  const int slot = blockIdx.x * blockDim.x + threadIdx.x;
  if (slot >= num_tokens * topk) return;
  const int t = slot / topk, j = slot - t * topk;
  const int e = idx[slot];
  const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(num_experts);
  const int r = valid ? e / per_rank : -1;
  const float wj = w[slot];
  for (int jr = 0; jr < topk; ++jr) {
    const int p = slot_row[t * topk + jr];
    if (p < 0 || p >= rows) continue;
    const int rr = idx[t * topk + jr] / per_rank;   // the opening slot's expert is valid
    const bool local = valid && r == rr;
    recv_idx[static_cast<size_t>(p) * topk + j] = local ? e - rr * per_rank : -1;
    recv_w[static_cast<size_t>(p) * topk + j] = local ? wj : 0.0f;
  }
}

}  // namespace

hipError_t launch_rank_meta(const int32_t* d_idx, const float* d_w, const int32_t* d_slot_row,
                            int num_tokens, int topk, int num_experts, int num_ranks, int64_t rows,
                            int32_t* d_recv_idx, float* d_recv_w, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int slots = num_tokens * topk;
  hipLaunchKernelGGL(rank_meta_kernel, dim3((slots + 255) / 256), dim3(256), 0, stream, d_idx, d_w,
                     d_slot_row, num_tokens, topk, num_experts, num_experts / num_ranks, rows,
                     d_recv_idx, d_recv_w);
  return hipGetLastError();
}

// Grid of a payload kernel: work-item workgroups (capped by max_blocks),
// plus the counts workgroup for the fixed-capacity layout.
template <class Rows>
hipError_t launch_payload(int dtype, const void* d_x, const Rows& src_rows, void* d_out,
                          void* d_scales, int num_tokens, int hidden, int max_blocks,
                          hipStream_t stream) {
  const int per_lane = dtype == MOE_DTYPE_BF16 ? 8 : 16;   // channels per lane
  const int slices = (hidden / per_lane + 63) / 64;
  const int payload = num_tokens == 0 ? 0
                      : static_cast<int>(item_grid(int64_t(num_tokens) * slices, max_blocks).x);
  const int blocks = payload + (Rows::kCountsBlock ? 1 : 0);
  if (blocks == 0) return hipSuccess;
  const dim3 grid(blocks), block(64 * kItemWaves);
  const u32x4* x = static_cast<const u32x4*>(d_x);
  u32x4* out = static_cast<u32x4*>(d_out);
  if (dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL(dispatch_bf16_kernel<Rows>, grid, block, 0, stream, x, src_rows, out,
                       num_tokens, hidden / 8, slices, payload);
  else if (dtype == MOE_DTYPE_FP8_E4M3)
    hipLaunchKernelGGL(dispatch_fp8_kernel<Rows>, grid, block, 0, stream, x, src_rows, out,
                       static_cast<float*>(d_scales), num_tokens, hidden, slices, payload);
  else
    hipLaunchKernelGGL(dispatch_mxfp8_kernel<Rows>, grid, block, 0, stream, x, src_rows, out,
                       static_cast<uint32_t*>(d_scales), num_tokens, hidden, slices, payload);
  return hipGetLastError();
}

hipError_t launch_dispatch(int dtype, const void* d_x, const int32_t* d_pos, void* d_out,
                           void* d_scales, int64_t rows, int num_tokens, int topk, int hidden,
                           int max_blocks, hipStream_t stream) {
  return launch_payload(dtype, d_x, TableRows{d_pos, topk, rows}, d_out, d_scales, num_tokens,
                        hidden, max_blocks, stream);
}

hipError_t launch_dispatch_fixed(int dtype, const void* d_x, const int32_t* d_idx,
                                 int num_tokens, int topk, int num_experts, int capacity,
                                 int32_t* d_pos, int32_t* d_counts, int32_t* d_status,
                                 void* d_out, void* d_scales, int hidden, int max_blocks,
                                 hipStream_t stream) {
  const FixedCapacityRows src{d_idx, topk, num_experts, capacity, d_pos, d_counts, d_status};
  return launch_payload(dtype, d_x, src, d_out, d_scales, num_tokens, hidden, max_blocks, stream);
}

}  // namespace moe
