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
// The same two kernels also build the rank-deduplicated layout (one row per
// (token, virtual rank) pair, the rows an expert-parallel exchange actually
// sends); the pass is selected at compile time (see Buckets).
//
// Two launches, no grid-wide synchronisation:
//   1. layout_hist_kernel   -- each workgroup counts the expert ids of its own
//      chunk of 1024 slots into an LDS histogram and writes it out.
//   2. layout_place_kernel  -- each workgroup sums the histograms column-wise
//      (all workgroups for the expert totals, earlier ones for its own base),
//      scans the totals over experts, then walks its chunk again in slot order
//      and assigns rows. Workgroup 0 also publishes counts and offsets.
// Up to 4096 slots (512 tokens at top-8) one workgroup of the place kernel
// does both, each wavefront taking 128, 256 or 512 slots (as few as cover
// them): its own per-wavefront counts are the totals. Beyond that,
// workgroups of 1024 slots; for the expert pass up to kLayoutFusedBlocks of
// them, the place kernel alone, each workgroup counting every slot itself.
//
// Inside a wavefront, lanes that hold the same expert id find each other with
// ceil(log2 E) ballots (one per id bit); the lowest lane of each group does
// the single LDS update for the group, and every lane's rank inside its group
// is the number of group lanes below it (mbcnt).
#include <mutex>

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

// What a layout pass sorts: every slot (t, j) falls into one bucket, or none.
//   expert pass: bucket = the slot's expert id;
//   rank pass:   bucket = the rank holding the slot's expert, but only for the
//                first slot of the token that reaches that rank, so that each
//                (token, rank) pair is counted and placed exactly once.
// Slots whose expert id lies outside [0, E) fall into no bucket.
struct Buckets {
  const int32_t* idx;  // [T * k] expert ids
  int slots;           // T * k
  int topk;            // k
  int num_experts;     // E
  uint32_t rank_mul;   // ceil(2^20 / (E / R)): rank = (e * rank_mul) >> 20, exact for E <= 1024
  int nbuckets;        // E (expert pass) or R (rank pass)
  int nbits;           // bits of a bucket id
  int capacity;        // rows: T * k (expert pass) or T * min(k, R) (rank pass)
};

// Where a pass writes (pointers into the workspace).
struct LayoutOut {
  int32_t* hist;           // [workgroups][nbuckets]
  int32_t* counts;         // [nbuckets]
  int32_t* offsets;        // [nbuckets + 1]
  int32_t* group_counts;   // expert pass: per-rank counts [R]
  int32_t* group_offsets;  // expert pass: per-rank offsets [R + 1]
  int32_t* pos;            // [T * k] row of each bucketed slot, -1 otherwise
  int32_t* src;            // [capacity] token of each row, -1 past the total
  int32_t* status;         // [MOE_EP_STATUS_WORDS]
  int32_t* rank_pos;       // rank pass: [T * R] row of each (token, rank), -1 if none
  int num_groups;          // R
  int per_rank;            // E / R
  int2* order;             // expert pass, block_chunks > 0: rows of each dispatch block
  int block_chunks;        // chunks per dispatch block; 0: no lists
};

__device__ __forceinline__ int rank_of(const Buckets& b, int e) {
  return static_cast<int>((static_cast<uint32_t>(e) * b.rank_mul) >> 20);
}

// Buckets of this wavefront's kSteps 64-slot steps starting at `base` (lane
// l of step s holds slot base + 64 s + l). Every lane must call it.
template <bool kRanks, int kSteps>
__device__ __forceinline__ void load_buckets(const Buckets& b, int base, int lane,
                                             int (&ids)[kSteps]) {
  int raw[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int slot = base + s * 64 + lane;
    raw[s] = slot < b.slots ? b.idx[slot] : -1;
  }
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int e = raw[s];
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(b.num_experts);
    if (!kRanks) {
      ids[s] = valid ? e : -1;
      continue;
    }
    // A slot opens its (token, rank) pair unless an earlier slot of the same
    // token reaches the same rank. The d-th earlier slot sits d lanes below in
    // the same step, or, for a token that starts in the previous step, in
    // memory (read only then).
    const int slot = base + s * 64 + lane;
    const int r = valid ? rank_of(b, e) : -1;
    const int j = slot % b.topk;
    bool first = valid;
    for (int d = 1; d < b.topk; ++d) {   // uniform trip count: every lane shuffles
      const int other = __shfl(r, lane >= d ? lane - d : lane, 64);
      if (valid && d <= j) {   // slot - d >= t*k >= 0 and slot < slots
        int ro = other;
        if (lane < d) {
          const int f = b.idx[slot - d];
          ro = static_cast<unsigned>(f) < static_cast<unsigned>(b.num_experts) ? rank_of(b, f) : -1;
        }
        if (ro == r) first = false;
      }
    }
    ids[s] = first ? r : -1;
  }
}

template <bool kRanks>
__global__ __launch_bounds__(kLayoutThreads) void layout_hist_kernel(Buckets b, LayoutOut o) {
  __shared__ int32_t s_hist[MOE_EP_MAX_EXPERTS];
  const int tid = threadIdx.x;
  for (int e = tid; e < b.nbuckets; e += kLayoutThreads) s_hist[e] = 0;
  if (kRanks) {   // every (token, rank) starts as "not routed there"
    const int cells = (b.slots / b.topk) * o.num_groups;
    for (int i = blockIdx.x * kLayoutThreads + tid; i < cells; i += gridDim.x * kLayoutThreads)
      o.rank_pos[i] = -1;
  }
  __syncthreads();

  const int lane = tid & 63;
  const int base = blockIdx.x * kLayoutChunk + (tid >> 6) * (kLayoutSteps * 64);
  int ids[kLayoutSteps];
  load_buckets<kRanks, kLayoutSteps>(b, base, lane, ids);
#pragma unroll
  for (int s = 0; s < kLayoutSteps; ++s) {
    const int e = ids[s];
    const bool valid = e >= 0;
    const uint64_t peers = same_expert_lanes(e, valid, b.nbits);
    if (valid && lanes_below(peers) == 0) atomicAdd(&s_hist[e], __popcll(peers));
  }
  __syncthreads();
  int32_t* out = o.hist + static_cast<size_t>(blockIdx.x) * b.nbuckets;
  for (int e = tid; e < b.nbuckets; e += kLayoutThreads) out[e] = s_hist[e];
}

// Exclusive scans of a[0 .. n) and, with kTwo, b[0 .. n) in LDS, in place
// (n <= 2 * kLayoutThreads: two entries per thread), with a[n] and b[n] the
// totals; both arrays go through the same shuffles and barriers. Every thread
// of the workgroup calls it, after the arrays are complete; they and wsum
// (2 * kLayoutWaves words) are free again on return.
template <bool kTwo>
__device__ __forceinline__ void workgroup_exclusive_scan(int32_t* a, int32_t* b, int n,
                                                         int32_t* wsum) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i0 = 2 * tid, i1 = 2 * tid + 1;
  const int a0 = i0 < n ? a[i0] : 0, a1 = i1 < n ? a[i1] : 0;
  const int b0 = kTwo && i0 < n ? b[i0] : 0, b1 = kTwo && i1 < n ? b[i1] : 0;
  const int la = a0 + a1, lb = b0 + b1;
  int ia = la, ib = lb;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int ua = __shfl_up(ia, d, 64);
    const int ub = kTwo ? __shfl_up(ib, d, 64) : 0;
    if (lane >= d) {
      ia += ua;
      ib += ub;
    }
  }
  if (lane == 63) {
    wsum[wave] = ia;
    if (kTwo) wsum[kLayoutWaves + wave] = ib;
  }
  __syncthreads();
  int before_a = 0, total_a = 0, before_b = 0, total_b = 0;
#pragma unroll
  for (int w = 0; w < kLayoutWaves; ++w) {
    const int wa = wsum[w];
    before_a += w < wave ? wa : 0;
    total_a += wa;
    if (kTwo) {
      const int wb = wsum[kLayoutWaves + w];
      before_b += w < wave ? wb : 0;
      total_b += wb;
    }
  }
  const int ea = before_a + ia - la;
  if (i0 < n) a[i0] = ea;
  if (i1 < n) a[i1] = ea + a0;
  if (tid == 0) a[n] = total_a;
  if (kTwo) {
    const int eb = before_b + ib - lb;
    if (i0 < n) b[i0] = eb;
    if (i1 < n) b[i1] = eb + b0;
    if (tid == 0) b[n] = total_b;
  }
  __syncthreads();
}

// kSteps: 64-slot steps per wavefront. kSingle: one workgroup holds every
// slot (up to kLayoutThreads * kSteps); no histogram kernel ran before it.
// kFused (expert pass, several workgroups, up to kLayoutFusedBlocks): no
// histogram kernel either; every workgroup counts all slots itself.
//
// Expert pass with o.block_chunks > 0 (several workgroups): the chunks are
// grouped into dispatch blocks of block_chunks chunks, and the kernel also
// lists each block's rows in ascending row order. Rows of bucket e that come
// from block B form one run, starting after the rows earlier blocks put in e
// (the column sum over earlier blocks' chunks), so a row's place in B's list
// is the number of B's rows in buckets below e plus its rank in that run.
template <bool kRanks, int kSteps, bool kSingle, bool kLists, bool kFused = false>
__global__ __launch_bounds__(kLayoutThreads) void layout_place_kernel(Buckets b, LayoutOut o) {
  static_assert(!kLists || (!kRanks && !kSingle), "lists: expert pass, several workgroups");
  static_assert(!kFused || (!kRanks && !kSingle), "fused: expert pass, several workgroups");
  // s_cur[w * E + e]: wavefront w's running row cursor for bucket e.
  __shared__ int32_t s_cur[kLayoutWaves * MOE_EP_MAX_EXPERTS];
  __shared__ int32_t s_off[MOE_EP_MAX_EXPERTS + 1];
  __shared__ int32_t s_pre[MOE_EP_MAX_EXPERTS];
  __shared__ int32_t s_wsum[2 * kLayoutWaves];
  // Dispatch lists: rows of each bucket in earlier blocks; then the block's
  // own count per bucket, scanned.
  __shared__ int32_t s_bpre[kLists ? MOE_EP_MAX_EXPERTS : 1];
  __shared__ int32_t s_bscan[kLists ? MOE_EP_MAX_EXPERTS + 1 : 1];
  // Partial column sums when several threads share a bucket.
  __shared__ int32_t s_part[kSingle || kFused ? 1 : 2][kSingle || kFused ? 1 : kLayoutThreads];
  // Fused: counts per bucket of four ranges of chunks (see below).
  __shared__ int32_t s_range[kFused ? 4 * MOE_EP_MAX_EXPERTS : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int E = b.nbuckets;
  const int nblocks = gridDim.x;
  const int block_first = kLists ? static_cast<int>(blockIdx.x) / o.block_chunks * o.block_chunks : 0;
  const int block_end = kLists ? min(block_first + o.block_chunks, nblocks) : 0;

  for (int i = tid; i < kLayoutWaves * E; i += kLayoutThreads) s_cur[i] = 0;
  if constexpr (kFused)
    for (int i = tid; i < 4 * E; i += kLayoutThreads) s_range[i] = 0;
  if (kRanks && kSingle) {   // every (token, rank) starts as "not routed there"
    const int cells = (b.slots / b.topk) * o.num_groups;
    for (int i = tid; i < cells; i += kLayoutThreads) o.rank_pos[i] = -1;
  }

  // This wavefront's slot ids, loaded first so that their latency overlaps
  // the histogram reads below.
  const int base = blockIdx.x * (kLayoutThreads * kSteps) + wave * (kSteps * 64);
  int ids[kSteps];
  load_buckets<kRanks, kSteps>(b, base, lane, ids);

  // Column sums of the per-workgroup histograms: the bucket totals, the part
  // that earlier workgroups (earlier slots) contribute and, for the dispatch
  // lists, the parts of earlier blocks and of this workgroup's own block.
  // With fewer buckets than threads, `parts` threads share a bucket, each
  // summing a contiguous range of the histograms, and LDS adds the ranges up
  // (the sums are latency-bound: each thread's loads come back in batches of
  // 16, so fewer loads per thread is less time; it pays from 64 workgroups:
  // layout 14.3 -> 11.7 us at 131,072 slots over 128 experts, nothing
  // measurable at 32 workgroups).
  if constexpr (kFused) {
    // Every workgroup counts every slot, by plain LDS atomics (a count needs
    // no per-lane rank, so no ballot grouping), into one of four ranges of
    // chunks: before this workgroup's dispatch block, the block's chunks
    // before this one, this one and the block's later chunks, and the chunks
    // after the block (without lists the block is this chunk alone). The
    // ids are read from L2 after the first workgroup of an XCD brings them
    // in, sixteen 64-slot steps per wavefront in flight at a time. The range
    // is uniform over a step (16 steps to a chunk).
    __syncthreads();   // s_range cleared
    const int me = static_cast<int>(blockIdx.x);
    const int lo = kLists ? block_first : me, hi = kLists ? block_end : me;
    constexpr int kStepsPerChunk = kLayoutChunk / 64;
    constexpr int kBatch = 16;
    const int steps = (b.slots + 63) / 64;
    for (int st0 = wave; st0 < steps; st0 += kBatch * kLayoutWaves) {
      int v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int slot = (st0 + u * kLayoutWaves) * 64 + lane;
        v[u] = slot < b.slots ? b.idx[slot] : -1;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int c = (st0 + u * kLayoutWaves) / kStepsPerChunk;
        const int r = c < lo ? 0 : c < me ? 1 : c < hi ? 2 : 3;
        if (static_cast<unsigned>(v[u]) < static_cast<unsigned>(b.num_experts))
          atomicAdd(&s_range[r * E + v[u]], 1);
      }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kLayoutThreads) {
      const int before = s_range[e], mine = s_range[E + e];
      const int rest = s_range[2 * E + e], after = s_range[3 * E + e];
      s_off[e] = before + mine + rest + after;
      s_pre[e] = before + mine;
      if constexpr (kLists) {
        s_bpre[e] = before;
        s_bscan[e] = mine + rest;
      }
    }
  } else if (!kSingle) {
    int parts = 1;
    while (nblocks >= 64 && parts * 2 * E <= kLayoutThreads && parts < kLayoutWaves) parts *= 2;
    const int me = static_cast<int>(blockIdx.x);
    if (parts == 1) {
      for (int e = tid; e < E; e += kLayoutThreads) {
        int tot = 0, pre = 0;
#pragma unroll 16
        for (int g = 0; g < nblocks; ++g) {
          const int v = o.hist[static_cast<size_t>(g) * E + e];
          tot += v;
          pre += g < me ? v : 0;
        }
        s_off[e] = tot;
        s_pre[e] = pre;
      }
    } else {
      for (int i = tid; i < E * parts; i += kLayoutThreads) {
        const int e = i % E, part = i / E;
        const int g0 = part * nblocks / parts, g1 = (part + 1) * nblocks / parts;
        int tot = 0, pre = 0;
#pragma unroll 16
        for (int g = g0; g < g1; ++g) {
          const int v = o.hist[static_cast<size_t>(g) * E + e];
          tot += v;
          pre += g < me ? v : 0;
        }
        s_part[0][i] = tot;
        s_part[1][i] = pre;
      }
      __syncthreads();
      for (int e = tid; e < E; e += kLayoutThreads) {
        int tot = 0, pre = 0;
        for (int q = 0; q < parts; ++q) {
          tot += s_part[0][q * E + e];
          pre += s_part[1][q * E + e];
        }
        s_off[e] = tot;
        s_pre[e] = pre;
      }
    }
    if constexpr (kLists) {
      // The block's own chunks: its count per bucket, and (from this
      // workgroup's prefix) the part of earlier blocks. Same thread-to-bucket
      // mapping as above, so s_pre[e] is this thread's own write.
      for (int e = tid; e < E; e += kLayoutThreads) {
        int own = 0, mine = 0;
        for (int g = block_first; g < block_end; ++g) {
          const int v = o.hist[static_cast<size_t>(g) * E + e];
          own += v;
          mine += g < me ? v : 0;
        }
        s_bpre[e] = s_pre[e] - mine;
        s_bscan[e] = own;
      }
    }
  }
  __syncthreads();

  // Pass 1 over this workgroup's chunk: per-wavefront histograms.
  uint64_t peers[kSteps];
  int32_t* my_cur = s_cur + wave * E;
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int e = ids[s];
    const bool valid = e >= 0;
    peers[s] = same_expert_lanes(e, valid, b.nbits);
    // Group leaders hold distinct ids within a step and the row belongs to
    // this wavefront alone, so a plain read-modify-write is race free.
    if (valid && lanes_below(peers[s]) == 0) my_cur[e] += __popcll(peers[s]);
  }

  if (kSingle) {   // the totals are the sums of the wavefronts' counts
    __syncthreads();
    for (int e = tid; e < E; e += kLayoutThreads) {
      int tot = 0;
#pragma unroll
      for (int w = 0; w < kLayoutWaves; ++w) tot += s_cur[w * E + e];
      s_off[e] = tot;
      s_pre[e] = 0;
    }
    __syncthreads();
  }

  // Exclusive scans over buckets: the totals (bucket offsets), and for the
  // dispatch lists the block's own counts.
  if constexpr (kLists) {
    workgroup_exclusive_scan<true>(s_off, s_bscan, E, s_wsum);
    // A row p of bucket e lands at list place p - (s_off[e] + s_bpre[e]) +
    // s_bscan[e]; keep that offset per bucket (in s_bpre).
    for (int e = tid; e < E; e += kLayoutThreads) s_bpre[e] = s_bscan[e] - s_off[e] - s_bpre[e];
    // The block's first workgroup marks the entries past its rows (invalid
    // slots, the tail of a last block) as (-1, -1).
    if (static_cast<int>(blockIdx.x) == block_first) {
      const int bs = o.block_chunks * kLayoutChunk;
      int2* list = o.order + static_cast<size_t>(block_first / o.block_chunks) * bs;
      for (int i = s_bscan[E] + tid; i < bs; i += kLayoutThreads) list[i] = make_int2(-1, -1);
    }
  } else {
    workgroup_exclusive_scan<false>(s_off, nullptr, E, s_wsum);
  }

  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += kLayoutThreads) {
      o.counts[e] = s_off[e + 1] - s_off[e];
      o.offsets[e] = s_off[e];
    }
    if (!kRanks) {
      const int per = o.per_rank;
      for (int r = tid; r < o.num_groups; r += kLayoutThreads) {
        o.group_counts[r] = s_off[(r + 1) * per] - s_off[r * per];
        o.group_offsets[r] = s_off[r * per];
      }
    }
    if (tid == 0) {
      o.offsets[E] = s_off[E];
      if (!kRanks) o.group_offsets[o.num_groups] = s_off[E];
      const int num_tokens = b.slots / (b.topk > 0 ? b.topk : 1);
      if (kRanks) {
        o.status[0] = s_off[E];           // rows in use: (token, rank) pairs
        o.status[1] = num_tokens;
        o.status[2] = 0;
      } else {
        o.status[0] = b.slots - s_off[E];  // skipped (invalid) slots
        o.status[1] = s_off[E];            // rows in use
        o.status[2] = num_tokens;
      }
      o.status[3] = 0;
    }
  }

  // Cursors: bucket start + earlier workgroups + earlier wavefronts here.
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
  for (int s = 0; s < kSteps; ++s) {
    const int slot = base + s * 64 + lane;
    const int e = ids[s];
    int p = -1;
    if (e >= 0) {
      const int c = my_cur[e];
      p = c + static_cast<int>(lanes_below(peers[s]));
      if (lanes_below(peers[s]) == 0) my_cur[e] = c + __popcll(peers[s]);
    }
    if (slot < b.slots) {
      o.pos[slot] = p;
      if (e >= 0 && p < b.capacity) {
        const int t = slot / b.topk;
        o.src[p] = t;
        if (kRanks) o.rank_pos[static_cast<size_t>(t) * o.num_groups + e] = p;
        if constexpr (kLists) {
          // Place in the block's list: its rows in lower buckets, then the
          // rank of p in bucket e's run of this block.
          const int bs = o.block_chunks * kLayoutChunk;
          const int li = p + s_bpre[e];
          if (li >= 0 && li < bs)
            o.order[static_cast<size_t>(block_first / o.block_chunks) * bs + li] = make_int2(p, t);
        }
      }
    }
  }

  // Rows past the valid total hold no token.
  const int total = s_off[E];
  for (int r = total + blockIdx.x * kLayoutThreads + tid; r < b.capacity;
       r += nblocks * kLayoutThreads)
    o.src[r] = -1;
}

int bits_for(int n) {
  int nbits = 0;
  while ((1 << nbits) < n) ++nbits;
  return nbits;
}

template <bool kRanks>
hipError_t launch_pass(const Buckets& b, const LayoutOut& o, hipStream_t stream) {
  const int nblocks = layout_blocks(b.slots);
  if (b.slots <= kLayoutSingleChunk) {   // one workgroup, as few steps as cover the slots
    if (b.slots <= kLayoutThreads * 2)
      hipLaunchKernelGGL((layout_place_kernel<kRanks, 2, true, false>), dim3(1), dim3(kLayoutThreads),
                         0, stream, b, o);
    else if (b.slots <= kLayoutThreads * 4)
      hipLaunchKernelGGL((layout_place_kernel<kRanks, 4, true, false>), dim3(1), dim3(kLayoutThreads),
                         0, stream, b, o);
    else
      hipLaunchKernelGGL((layout_place_kernel<kRanks, kLayoutSingleSteps, true, false>), dim3(1),
                         dim3(kLayoutThreads), 0, stream, b, o);
    return hipGetLastError();
  }
  if constexpr (!kRanks) {
    if (nblocks <= kLayoutFusedBlocks) {   // one launch: every workgroup counts all slots
      if (o.block_chunks > 0)
        hipLaunchKernelGGL((layout_place_kernel<false, kLayoutSteps, false, true, true>),
                           dim3(nblocks), dim3(kLayoutThreads), 0, stream, b, o);
      else
        hipLaunchKernelGGL((layout_place_kernel<false, kLayoutSteps, false, false, true>),
                           dim3(nblocks), dim3(kLayoutThreads), 0, stream, b, o);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL(layout_hist_kernel<kRanks>, dim3(nblocks), dim3(kLayoutThreads), 0, stream,
                     b, o);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if constexpr (!kRanks) {
    if (o.block_chunks > 0) {
      hipLaunchKernelGGL((layout_place_kernel<false, kLayoutSteps, false, true>), dim3(nblocks),
                         dim3(kLayoutThreads), 0, stream, b, o);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((layout_place_kernel<kRanks, kLayoutSteps, false, false>), dim3(nblocks),
                     dim3(kLayoutThreads), 0, stream, b, o);
  return hipGetLastError();
}

}  // namespace

// Multiplier that divides by `per` (1 <= per <= 1024) exactly for ids below
// 1024: floor(e / per) == (e * ceil(2^20 / per)) >> 20 whenever e * per < 2^20.
uint32_t rank_multiplier(int per) { return ((1u << 20) + per - 1) / per; }

hipError_t launch_layout(const int32_t* d_idx, int num_tokens, int topk, int num_experts,
                         int num_ranks, const LayoutArrays& a, hipStream_t stream,
                         int block_chunks) {
  const int per = num_experts / num_ranks;
  Buckets b{d_idx, num_tokens * topk, topk, num_experts, rank_multiplier(per),
            num_experts, bits_for(num_experts), num_tokens * topk};
  // Lists only where several place workgroups run and the arrays exist.
  const bool lists = block_chunks > 0 && b.slots > kLayoutSingleChunk && a.order != nullptr;
  LayoutOut o{a.hist, a.counts_e, a.offsets_e, a.counts_r, a.offsets_r, a.pos, a.src_idx,
              a.status, nullptr, num_ranks, per, lists ? a.order : nullptr,
              lists ? block_chunks : 0};
  return launch_pass<false>(b, o, stream);
}

// ---- Layout without a workspace ---------------------------------------------
// The per-workgroup histograms of moe_dispatch_layout_noalloc live in this
// file-scope device array, one copy per GPU, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only
// a stand-in for the symbol): layout_scratch() looks up its device address
// once per device, with that device current, and the kernels take that
// pointer. Every call on a GPU shares its copy; the histogram kernel writes
// every entry the place kernel then reads, so nothing needs clearing between
// calls, and calls that overlap on one GPU race.
static __device__ __align__(256) int32_t g_layout_scratch[kNoallocScratchInts];

hipError_t layout_scratch(int32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static int32_t* ptr[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(g_layout_scratch));
    ptr[dev] = err[dev] == hipSuccess ? static_cast<int32_t*>(p) : nullptr;
  });
  if (err[dev] != hipSuccess) return err[dev];
  *out = ptr[dev];
  return hipSuccess;
}

size_t layout_scratch_ints(int num_tokens, int topk, int num_experts) {
  const int64_t slots = int64_t(num_tokens) * topk;
  if (slots <= kLayoutSingleChunk) return 0;   // one workgroup, no histograms
  // one launch, every workgroup counting all slots itself: no histograms
  if (layout_blocks(slots) <= kLayoutFusedBlocks) return 0;
  return static_cast<size_t>(layout_blocks(slots)) * static_cast<size_t>(num_experts);
}

hipError_t launch_rank_layout(const int32_t* d_idx, int num_tokens, int topk, int num_experts,
                              int num_ranks, const RankArrays& a, hipStream_t stream) {
  const int per = num_experts / num_ranks;
  const int rows = num_tokens * (topk < num_ranks ? topk : num_ranks);
  Buckets b{d_idx, num_tokens * topk, topk, num_experts, rank_multiplier(per),
            num_ranks, bits_for(num_ranks), rows};
  LayoutOut o{a.hist, a.counts, a.offsets, nullptr, nullptr, a.slot_row, a.src,
              a.status, a.rank_pos, num_ranks, per, nullptr, 0};
  return launch_pass<true>(b, o, stream);
}

}  // namespace moe
