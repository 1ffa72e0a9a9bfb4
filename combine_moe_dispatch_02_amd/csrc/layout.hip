// Layout: per-expert histogram, exclusive scan and stable placement of the
// routed (token, slot) pairs.
//
// The pages ("Inside the Nebius + PyTorch DeepSeek V3 recipe", section
// "Mixture-of-experts and wide expert parallelism"; "MoE / Hybrid-EP
// Validation", "Design principles") fix only that each token goes to the k
// experts its router picked and that experts are partitioned over EP ranks.
// The placement is the stable counting sort of the T*k slots by expert id in
// (token, slot) order, with experts split contiguously over R virtual ranks.
//
// Two launches, no grid-wide synchronisation:
//   1. layout_hist_kernel   -- each workgroup counts the expert ids of its own
//      chunk of 2048 slots into an LDS histogram and writes it out.
//   2. layout_place_kernel  -- each workgroup sums the histograms column-wise
//      (all workgroups for the expert totals, earlier ones for its own base),
//      scans the totals over experts, then walks its chunk again in slot order
//      and assigns rows. Workgroup 0 also publishes counts and offsets.
//
// Inside a wavefront, lanes that hold the same expert id find each other with
// ceil(log2 E) ballots (one per id bit); the lowest lane of each group does
// the single LDS update for the group, and every lane's rank inside its group
// is the number of group lanes below it (mbcnt).
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Mask of the lanes of this wavefront whose expert id equals this lane's.
// Every lane of the wavefront must call it (it issues ballots).
__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool valid, int nbits) {
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return valid ? peers : 0ull;
}

__global__ __launch_bounds__(kLayoutThreads) void layout_hist_kernel(
    const int32_t* __restrict__ idx, int slots, int num_experts, int nbits,
    int32_t* __restrict__ hist) {
  __shared__ int32_t s_hist[MOE_EP_MAX_EXPERTS];
  const int tid = threadIdx.x;
  for (int e = tid; e < num_experts; e += kLayoutThreads) s_hist[e] = 0;
  __syncthreads();

  const int lane = tid & 63;
  const int base = blockIdx.x * kLayoutChunk + (tid >> 6) * (kLayoutSteps * 64);
  int ids[kLayoutSteps];
#pragma unroll
  for (int s = 0; s < kLayoutSteps; ++s) {
    const int slot = base + s * 64 + lane;
    ids[s] = slot < slots ? idx[slot] : -1;
  }
#pragma unroll
  for (int s = 0; s < kLayoutSteps; ++s) {
    const int e = ids[s];
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(num_experts);
    const uint64_t peers = same_expert_lanes(e, valid, nbits);
    if (valid && lanes_below(peers) == 0) atomicAdd(&s_hist[e], __popcll(peers));
  }
  __syncthreads();
  int32_t* out = hist + static_cast<size_t>(blockIdx.x) * num_experts;
  for (int e = tid; e < num_experts; e += kLayoutThreads) out[e] = s_hist[e];
}

__global__ __launch_bounds__(kLayoutThreads) void layout_place_kernel(
    const int32_t* __restrict__ idx, int slots, int topk, int num_experts, int num_ranks,
    int nbits, const int32_t* __restrict__ hist, LayoutArrays a) {
  // s_cur[w * E + e]: wavefront w's running row cursor for expert e.
  __shared__ int32_t s_cur[kLayoutWaves * MOE_EP_MAX_EXPERTS];
  __shared__ int32_t s_off[MOE_EP_MAX_EXPERTS + 1];
  __shared__ int32_t s_pre[MOE_EP_MAX_EXPERTS];
  __shared__ int32_t s_wsum[kLayoutWaves];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int E = num_experts;
  const int nblocks = gridDim.x;

  for (int i = tid; i < kLayoutWaves * E; i += kLayoutThreads) s_cur[i] = 0;

  // Column sums of the per-workgroup histograms: the expert totals, and the
  // part that earlier workgroups (earlier slots) contribute.
  for (int e = tid; e < E; e += kLayoutThreads) {
    int tot = 0, pre = 0;
#pragma unroll 16
    for (int b = 0; b < nblocks; ++b) {
      const int v = hist[static_cast<size_t>(b) * E + e];
      tot += v;
      pre += b < static_cast<int>(blockIdx.x) ? v : 0;
    }
    s_off[e] = tot;
    s_pre[e] = pre;
  }
  __syncthreads();

  // Pass 1 over this workgroup's chunk: per-wavefront histograms.
  const int base = blockIdx.x * kLayoutChunk + wave * (kLayoutSteps * 64);
  int ids[kLayoutSteps];
  uint64_t peers[kLayoutSteps];
#pragma unroll
  for (int s = 0; s < kLayoutSteps; ++s) {
    const int slot = base + s * 64 + lane;
    ids[s] = slot < slots ? idx[slot] : -1;
  }
  int32_t* my_cur = s_cur + wave * E;
#pragma unroll
  for (int s = 0; s < kLayoutSteps; ++s) {
    const int e = ids[s];
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
    peers[s] = same_expert_lanes(e, valid, nbits);
    // Group leaders hold distinct ids within a step and the row belongs to
    // this wavefront alone, so a plain read-modify-write is race free.
    if (valid && lanes_below(peers[s]) == 0) my_cur[e] += __popcll(peers[s]);
  }

  // Exclusive scan of the totals over experts (two entries per thread, E <= 1024).
  {
    const int i0 = 2 * tid, i1 = 2 * tid + 1;
    const int v0 = i0 < E ? s_off[i0] : 0;
    const int v1 = i1 < E ? s_off[i1] : 0;
    const int local = v0 + v1;
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(incl, d, 64);
      if (lane >= d) incl += up;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) {
      const int ws = s_wsum[w];
      before += w < wave ? ws : 0;
      total += ws;
    }
    const int excl = before + incl - local;
    if (i0 < E) s_off[i0] = excl;
    if (i1 < E) s_off[i1] = excl + v0;
    if (tid == 0) s_off[E] = total;
  }
  __syncthreads();

  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += kLayoutThreads) {
      a.counts_e[e] = s_off[e + 1] - s_off[e];
      a.offsets_e[e] = s_off[e];
    }
    const int per = E / num_ranks;
    for (int r = tid; r < num_ranks; r += kLayoutThreads) {
      a.counts_r[r] = s_off[(r + 1) * per] - s_off[r * per];
      a.offsets_r[r] = s_off[r * per];
    }
    if (tid == 0) {
      a.offsets_e[E] = s_off[E];
      a.offsets_r[num_ranks] = s_off[E];
      a.status[0] = slots - s_off[E];   // skipped (invalid) slots
      a.status[1] = s_off[E];           // rows in use
      a.status[2] = slots / (topk > 0 ? topk : 1);
      a.status[3] = 0;
    }
  }

  // Cursors: expert start + earlier workgroups + earlier wavefronts here.
  for (int e = tid; e < E; e += kLayoutThreads) {
    int run = s_off[e] + s_pre[e];
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) {
      const int c = s_cur[w * E + e];
      s_cur[w * E + e] = run;
      run += c;
    }
  }
  __syncthreads();

  // Pass 2: rows in slot order. All lanes of a group read the cursor before
  // the leader advances it (LDS operations of one wavefront stay in order).
#pragma unroll
  for (int s = 0; s < kLayoutSteps; ++s) {
    const int slot = base + s * 64 + lane;
    const int e = ids[s];
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
    int p = -1;
    if (valid) {
      const int c = my_cur[e];
      p = c + static_cast<int>(lanes_below(peers[s]));
      if (lanes_below(peers[s]) == 0) my_cur[e] = c + __popcll(peers[s]);
    }
    if (slot < slots) {
      a.pos[slot] = p;
      if (valid && p < slots) a.src_idx[p] = slot / topk;
    }
  }

  // Rows past the valid total hold no token.
  const int total = s_off[E];
  for (int r = total + blockIdx.x * kLayoutThreads + tid; r < slots; r += nblocks * kLayoutThreads)
    a.src_idx[r] = -1;
}

}  // namespace

hipError_t launch_layout(const int32_t* d_idx, int num_tokens, int topk, int num_experts,
                         int num_ranks, const LayoutArrays& a, hipStream_t stream) {
  const int slots = num_tokens * topk;
  const int nblocks = layout_blocks(slots);
  int nbits = 0;
  while ((1 << nbits) < num_experts) ++nbits;
  hipLaunchKernelGGL(layout_hist_kernel, dim3(nblocks), dim3(kLayoutThreads), 0, stream, d_idx,
                     slots, num_experts, nbits, a.hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(layout_place_kernel, dim3(nblocks), dim3(kLayoutThreads), 0, stream, d_idx,
                     slots, topk, num_experts, num_ranks, nbits, a.hist, a);
  return hipGetLastError();
}

}  // namespace moe
