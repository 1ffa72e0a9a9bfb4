// C ABI of the dispatch/combine library: argument checks, workspace carving,
// handle state and error reporting. Kernels live in layout.hip, dispatch.hip,
// combine.hip and router.hip.
//
// Conventions (declared in moe_ep.h): nothing throws across the ABI, host-side
// argument errors enqueue nothing, device work is asynchronous on the caller's
// stream, and an unsupported configuration is refused at handle creation with
// a message that says what to change -- the fail-fast behaviour the "MoE /
// Hybrid-EP Validation" page describes under "When EP crosses a node in an
// intra-node-only build".
#include <stdarg.h>
#include <stdio.h>

#include <new>
#include <string>

#include "moe_internal.h"

struct moe_handle {
  moe_config_t cfg;
  char* ws;
  size_t ws_bytes;
  moe::LayoutArrays arrays;
  moe::RankArrays rank;
  bool ready;
  int32_t num_tokens;
  bool rank_ready;
  int32_t rank_num_tokens;
  int32_t max_workgroups;  // 0: one workgroup per 4 work items
  int32_t order_chunks;    // blocked bf16 dispatch: chunks per block of the last layout, 0: none
  // Decode-time (fixed-capacity) state.
  int32_t* ll_pos;     // [min(T_max, LL max) * k]
  int32_t* ll_counts;  // [E]
  int32_t* ll_status;  // [MOE_EP_STATUS_WORDS]
  bool ll_ready;
  int32_t ll_num_tokens;
  int32_t ll_capacity;
};

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return MOE_OK;
}

constexpr size_t kAlign = 256;
constexpr int64_t kMaxSlots = int64_t(1) << 30;  // rows and slots stay far from int32 overflow
constexpr int64_t kMaxItems = int64_t(1) << 30;
constexpr int32_t kLayoutDispatchFusedBelow = 640;   // tokens; see moe_layout_dispatch

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Region offsets inside the workspace; returns the total size.
struct Carve {
  size_t status, counts_e, offsets_e, counts_r, offsets_r, hist, pos, src_idx, order;
  size_t r_status, r_counts, r_offsets, r_hist, r_slot_row, r_rank_pos, r_src;
  size_t ll_pos, ll_counts, ll_status;
  size_t total;
};

Carve carve(const moe_config_t& c) {
  const int64_t slots = int64_t(c.max_tokens) * c.topk;
  Carve r;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  r.status = take(sizeof(int32_t) * MOE_EP_STATUS_WORDS);
  r.counts_e = take(sizeof(int32_t) * c.num_experts);
  r.offsets_e = take(sizeof(int32_t) * (c.num_experts + 1));
  r.counts_r = take(sizeof(int32_t) * c.num_ranks);
  r.offsets_r = take(sizeof(int32_t) * (c.num_ranks + 1));
  r.hist = take(sizeof(int32_t) * size_t(moe::layout_blocks(slots)) * c.num_experts);
  r.pos = take(sizeof(int32_t) * size_t(slots));
  r.src_idx = take(sizeof(int32_t) * size_t(slots));
  r.order = take(sizeof(int2) * size_t(moe::dispatch_order_entries(c.max_tokens, c.topk)));
  const int64_t rank_rows = int64_t(c.max_tokens) * (c.topk < c.num_ranks ? c.topk : c.num_ranks);
  r.r_status = take(sizeof(int32_t) * MOE_EP_STATUS_WORDS);
  r.r_counts = take(sizeof(int32_t) * c.num_ranks);
  r.r_offsets = take(sizeof(int32_t) * (c.num_ranks + 1));
  r.r_hist = take(sizeof(int32_t) * size_t(moe::layout_blocks(slots)) * c.num_ranks);
  r.r_slot_row = take(sizeof(int32_t) * size_t(slots));
  r.r_rank_pos = take(sizeof(int32_t) * size_t(c.max_tokens) * c.num_ranks);
  r.r_src = take(sizeof(int32_t) * size_t(rank_rows));
  const int64_t ll_tokens = c.max_tokens < MOE_EP_LL_MAX_TOKENS ? c.max_tokens : MOE_EP_LL_MAX_TOKENS;
  r.ll_pos = take(sizeof(int32_t) * size_t(ll_tokens) * c.topk);
  r.ll_counts = take(sizeof(int32_t) * c.num_experts);
  r.ll_status = take(sizeof(int32_t) * MOE_EP_STATUS_WORDS);
  r.total = off;
  return r;
}

int check_config(const moe_config_t* c) {
  if (c == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_config_t pointer is NULL");
  if (c->max_tokens < 0)
    return fail(MOE_ERR_INVALID_ARG, "max_tokens=%d must be >= 0", c->max_tokens);
  if (c->hidden <= 0) return fail(MOE_ERR_INVALID_ARG, "hidden=%d must be > 0", c->hidden);
  if (c->num_experts <= 0)
    return fail(MOE_ERR_INVALID_ARG, "num_experts=%d must be > 0", c->num_experts);
  if (c->num_ranks <= 0) return fail(MOE_ERR_INVALID_ARG, "num_ranks=%d must be > 0", c->num_ranks);
  if (c->topk <= 0) return fail(MOE_ERR_INVALID_ARG, "topk=%d must be > 0", c->topk);
  if (c->hidden % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED,
                "hidden=%d is not a multiple of 8: rows move in 16-byte pieces; pad hidden to a "
                "multiple of 8",
                c->hidden);
  if (c->num_experts > MOE_EP_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED,
                "num_experts=%d exceeds the supported maximum %d: split the experts over more "
                "EP groups or rebuild with a larger MOE_EP_MAX_EXPERTS",
                c->num_experts, MOE_EP_MAX_EXPERTS);
  if (c->num_experts % c->num_ranks != 0)
    return fail(MOE_ERR_UNSUPPORTED,
                "num_experts=%d is not a multiple of num_ranks=%d: each virtual rank holds a "
                "contiguous, equal share of the experts; choose num_ranks dividing num_experts",
                c->num_experts, c->num_ranks);
  if (c->topk > c->num_experts)
    return fail(MOE_ERR_UNSUPPORTED, "topk=%d exceeds num_experts=%d", c->topk, c->num_experts);
  if (c->topk > MOE_EP_MAX_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "topk=%d exceeds the supported maximum %d", c->topk,
                MOE_EP_MAX_TOPK);
  // Payload kernels index (token, 512-channel slice) work items with int.
  if (int64_t(c->max_tokens) * ((c->hidden / 8 + 63) / 64) > kMaxItems)
    return fail(MOE_ERR_UNSUPPORTED,
                "max_tokens=%d with hidden=%d exceeds %lld work items: use several handles over "
                "token chunks",
                c->max_tokens, c->hidden, (long long)kMaxItems);
  if (int64_t(c->max_tokens) * c->topk > kMaxSlots)
    return fail(MOE_ERR_UNSUPPORTED,
                "max_tokens*topk=%lld exceeds %lld rows: use several handles over token chunks",
                (long long)(int64_t(c->max_tokens) * c->topk), (long long)kMaxSlots);
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_ready(moe_handle_t h, const char* fn) {
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  if (!h->ready)
    return fail(MOE_ERR_STATE, "%s: no layout yet; call moe_dispatch_layout first", fn);
  return MOE_OK;
}

int64_t rank_capacity(const moe_handle* h) {
  return int64_t(h->rank_num_tokens) * (h->cfg.topk < h->cfg.num_ranks ? h->cfg.topk
                                                                         : h->cfg.num_ranks);
}

int check_rank_ready(moe_handle_t h, const char* fn) {
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  if (!h->rank_ready)
    return fail(MOE_ERR_STATE, "%s: no rank layout yet; call moe_rank_layout first", fn);
  return MOE_OK;
}

int hip_status(hipError_t err, const char* fn) {
  if (err == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: HIP error %d (%s)", fn, int(err), hipGetErrorString(err));
}

// Layout into the handle's workspace; with lists for the blocked bf16
// dispatch wherever that form applies to the batch.
hipError_t handle_layout(moe_handle_t h, const int32_t* d_idx, int32_t num_tokens,
                         hipStream_t stream) {
  // (dispatch_block_chunks is 0 below 8 chunks, so the lists never meet the
  // one-workgroup layout, which writes none.)
  const int block_chunks = moe::dispatch_block_chunks(num_tokens, h->cfg.topk, h->cfg.hidden);
  h->order_chunks = 0;
  const hipError_t err = moe::launch_layout(d_idx, num_tokens, h->cfg.topk, h->cfg.num_experts,
                                            h->cfg.num_ranks, h->arrays, stream, block_chunks);
  if (err == hipSuccess) h->order_chunks = block_chunks;
  return err;
}

// Dispatch through the handle's last layout: the blocked form for bf16 when
// the layout listed the blocks and no workgroup cap is set, else the forms
// that read the position table.
hipError_t handle_dispatch(moe_handle_t h, int dtype, const void* d_x, void* d_out, void* d_scales,
                           int64_t out_rows, int32_t num_tokens, hipStream_t stream) {
  if (dtype == MOE_DTYPE_BF16 && h->max_workgroups == 0 && h->order_chunks > 0)
    return moe::launch_dispatch_blocks(d_x, h->arrays.order, d_out, out_rows, num_tokens,
                                       h->cfg.topk, h->cfg.hidden, h->order_chunks, stream);
  return moe::launch_dispatch(dtype, d_x, h->arrays.pos, d_out, d_scales, out_rows, num_tokens,
                              h->cfg.topk, h->cfg.hidden, h->max_workgroups, stream);
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_config_t* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  ok();
  return carve(*cfg).total;
}

int moe_handle_create(const moe_config_t* cfg, void* d_workspace, size_t ws_bytes,
                      moe_handle_t* out) {
  if (out == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_handle_create: out is NULL");
  *out = nullptr;
  const int st = check_config(cfg);
  if (st != MOE_OK) return st;
  const Carve c = carve(*cfg);
  if (d_workspace == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_handle_create: workspace is NULL");
  if (!aligned(d_workspace, kAlign))
    return fail(MOE_ERR_INVALID_ARG, "moe_handle_create: workspace must be %zu-byte aligned", kAlign);
  if (ws_bytes < c.total)
    return fail(MOE_ERR_INVALID_ARG, "moe_handle_create: workspace has %zu bytes, needs %zu",
                ws_bytes, c.total);
  moe_handle* h = new (std::nothrow) moe_handle;
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_handle_create: out of host memory");
  h->cfg = *cfg;
  h->ws = static_cast<char*>(d_workspace);
  h->ws_bytes = ws_bytes;
  auto at = [&](size_t off) { return reinterpret_cast<int32_t*>(h->ws + off); };
  h->arrays.status = at(c.status);
  h->arrays.counts_e = at(c.counts_e);
  h->arrays.offsets_e = at(c.offsets_e);
  h->arrays.counts_r = at(c.counts_r);
  h->arrays.offsets_r = at(c.offsets_r);
  h->arrays.hist = at(c.hist);
  h->arrays.pos = at(c.pos);
  h->arrays.src_idx = at(c.src_idx);
  h->arrays.order = reinterpret_cast<int2*>(h->ws + c.order);
  h->rank.status = at(c.r_status);
  h->rank.counts = at(c.r_counts);
  h->rank.offsets = at(c.r_offsets);
  h->rank.hist = at(c.r_hist);
  h->rank.slot_row = at(c.r_slot_row);
  h->rank.rank_pos = at(c.r_rank_pos);
  h->rank.src = at(c.r_src);
  h->ready = false;
  h->num_tokens = 0;
  h->rank_ready = false;
  h->rank_num_tokens = 0;
  h->max_workgroups = 0;
  h->order_chunks = 0;
  h->ll_pos = at(c.ll_pos);
  h->ll_counts = at(c.ll_counts);
  h->ll_status = at(c.ll_status);
  h->ll_ready = false;
  h->ll_num_tokens = 0;
  h->ll_capacity = 0;
  *out = h;
  return ok();
}

void moe_handle_destroy(moe_handle_t h) { delete h; }

int moe_dispatch_layout(moe_handle_t h, const int32_t* d_topk_idx, int32_t num_tokens,
                        hipStream_t stream) {
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch_layout: handle is NULL");
  if (num_tokens < 0 || num_tokens > h->cfg.max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch_layout: num_tokens=%d outside [0, %d]",
                num_tokens, h->cfg.max_tokens);
  if (num_tokens > 0 && d_topk_idx == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch_layout: topk_idx is NULL");
  if (!aligned(d_topk_idx, 4))
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch_layout: topk_idx must be 4-byte aligned");
  const hipError_t err = handle_layout(h, d_topk_idx, num_tokens, stream);
  if (err != hipSuccess) {
    h->ready = false;
    return hip_status(err, "moe_dispatch_layout");
  }
  h->ready = true;
  h->num_tokens = num_tokens;
  return ok();
}

int moe_dispatch_layout_noalloc(const int32_t* d_topk_idx, int32_t num_tokens, int32_t topk,
                                int32_t num_experts, int32_t num_ranks, int32_t* d_pos,
                                int32_t* d_src_idx, int32_t* d_counts_e, int32_t* d_offsets_e,
                                int32_t* d_counts_r, int32_t* d_offsets_r, int32_t* d_status,
                                hipStream_t stream) {
  const char* fn = "moe_dispatch_layout_noalloc";
  if (num_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "%s: num_tokens=%d must be >= 0", fn, num_tokens);
  const moe_config_t c{num_tokens, 8, topk, num_experts, num_ranks};   // hidden plays no part
  const int st = check_config(&c);
  if (st != MOE_OK) return st;
  if (d_counts_e == nullptr || d_offsets_e == nullptr || d_counts_r == nullptr ||
      d_offsets_r == nullptr || d_status == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "%s: counts, offsets and status must not be NULL", fn);
  if (num_tokens > 0 && (d_topk_idx == nullptr || d_pos == nullptr || d_src_idx == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_idx, pos and src_idx must not be NULL", fn);
  for (const void* p : {static_cast<const void*>(d_topk_idx), static_cast<const void*>(d_pos),
                        static_cast<const void*>(d_src_idx), static_cast<const void*>(d_counts_e),
                        static_cast<const void*>(d_offsets_e), static_cast<const void*>(d_counts_r),
                        static_cast<const void*>(d_offsets_r), static_cast<const void*>(d_status)})
    if (!aligned(p, 4)) return fail(MOE_ERR_INVALID_ARG, "%s: arrays must be 4-byte aligned", fn);
  const size_t need = moe::layout_scratch_ints(num_tokens, topk, num_experts);
  if (need > moe::kNoallocScratchInts)
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: %d tokens x top-%d over %d experts need %zu bytes of histogram scratch; the "
                "static array holds %zu: lay out fewer tokens per call, or use "
                "moe_dispatch_layout with a workspace",
                fn, num_tokens, topk, num_experts, need * sizeof(int32_t),
                size_t(MOE_EP_NOALLOC_SCRATCH_BYTES));
  int32_t* scratch = nullptr;
  hipError_t err = moe::layout_scratch(&scratch);
  if (err != hipSuccess) return hip_status(err, fn);
  // no block lists: moe_dispatch never reads this layout
  const moe::LayoutArrays a{d_status, d_counts_e, d_offsets_e, d_counts_r, d_offsets_r,
                            scratch,  d_pos,      d_src_idx,   nullptr};
  err = moe::launch_layout(d_topk_idx, num_tokens, topk, num_experts, num_ranks, a, stream);
  return hip_status(err, fn);
}

int moe_layout_view(moe_handle_t h, moe_layout_view_t* out) {
  if (out == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_layout_view: out is NULL");
  const int st = check_ready(h, "moe_layout_view");
  if (st != MOE_OK) return st;
  out->pos = h->arrays.pos;
  out->src_idx = h->arrays.src_idx;
  out->counts_e = h->arrays.counts_e;
  out->offsets_e = h->arrays.offsets_e;
  out->counts_r = h->arrays.counts_r;
  out->offsets_r = h->arrays.offsets_r;
  out->status = h->arrays.status;
  out->num_tokens = h->num_tokens;
  out->capacity = int64_t(h->num_tokens) * h->cfg.topk;
  return ok();
}

int moe_dispatch(moe_handle_t h, const void* d_x, int dtype, void* d_out, void* d_scales,
                 int64_t out_rows, hipStream_t stream) {
  const int st = check_ready(h, "moe_dispatch");
  if (st != MOE_OK) return st;
  const int64_t capacity = int64_t(h->num_tokens) * h->cfg.topk;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3 && dtype != MOE_DTYPE_MXFP8_E4M3)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: unknown dtype %d", dtype);
  if (out_rows < capacity)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_dispatch: out_rows=%lld is below the worst-case capacity num_tokens*topk=%lld",
                (long long)out_rows, (long long)capacity);
  if (dtype != MOE_DTYPE_BF16 && h->cfg.hidden % MOE_EP_FP8_BLOCK != 0)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_dispatch: FP8 and MXFP8 need hidden to be a multiple of %d; hidden=%d",
                MOE_EP_FP8_BLOCK, h->cfg.hidden);
  if (h->num_tokens == 0) return ok();
  if (d_x == nullptr || d_out == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: x or out is NULL");
  if (!aligned(d_x, 16) || !aligned(d_out, 16))
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: x and out must be 16-byte aligned");
  if (dtype != MOE_DTYPE_BF16 && d_scales == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: FP8 dispatch needs a scales buffer");
  if (dtype != MOE_DTYPE_BF16 && !aligned(d_scales, 4))
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: scales must be 4-byte aligned");
  const hipError_t err =
      handle_dispatch(h, dtype, d_x, d_out, d_scales, out_rows, h->num_tokens, stream);
  return hip_status(err, "moe_dispatch");
}

int moe_combine(moe_handle_t h, const void* d_y, int64_t y_rows, const float* d_w, void* d_out,
                hipStream_t stream) {
  const int st = check_ready(h, "moe_combine");
  if (st != MOE_OK) return st;
  const int64_t capacity = int64_t(h->num_tokens) * h->cfg.topk;
  if (y_rows < capacity)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_combine: y_rows=%lld is below the capacity num_tokens*topk=%lld",
                (long long)y_rows, (long long)capacity);
  if (h->num_tokens == 0) return ok();
  if (d_y == nullptr || d_w == nullptr || d_out == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: y, w or out is NULL");
  if (!aligned(d_y, 16) || !aligned(d_out, 16) || !aligned(d_w, 4))
    return fail(MOE_ERR_INVALID_ARG,
                "moe_combine: y and out must be 16-byte aligned, w 4-byte aligned");
  const hipError_t err = moe::launch_combine(d_y, y_rows, d_w, h->arrays.pos, d_out,
                                             h->num_tokens, h->cfg.topk, h->cfg.hidden,
                                             h->max_workgroups, stream);
  return hip_status(err, "moe_combine");
}

int moe_rank_layout(moe_handle_t h, const int32_t* d_topk_idx, int32_t num_tokens,
                    hipStream_t stream) {
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_rank_layout: handle is NULL");
  if (num_tokens < 0 || num_tokens > h->cfg.max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "moe_rank_layout: num_tokens=%d outside [0, %d]", num_tokens,
                h->cfg.max_tokens);
  if (num_tokens > 0 && d_topk_idx == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_rank_layout: topk_idx is NULL");
  if (!aligned(d_topk_idx, 4))
    return fail(MOE_ERR_INVALID_ARG, "moe_rank_layout: topk_idx must be 4-byte aligned");
  const hipError_t err = moe::launch_rank_layout(d_topk_idx, num_tokens, h->cfg.topk,
                                                 h->cfg.num_experts, h->cfg.num_ranks, h->rank,
                                                 stream);
  if (err != hipSuccess) {
    h->rank_ready = false;
    return hip_status(err, "moe_rank_layout");
  }
  h->rank_ready = true;
  h->rank_num_tokens = num_tokens;
  return ok();
}

int moe_rank_layout_view(moe_handle_t h, moe_rank_layout_view_t* out) {
  if (out == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_rank_layout_view: out is NULL");
  const int st = check_rank_ready(h, "moe_rank_layout_view");
  if (st != MOE_OK) return st;
  out->rank_pos = h->rank.rank_pos;
  out->slot_row = h->rank.slot_row;
  out->src_idx = h->rank.src;
  out->counts_r = h->rank.counts;
  out->offsets_r = h->rank.offsets;
  out->status = h->rank.status;
  out->num_tokens = h->rank_num_tokens;
  out->capacity = rank_capacity(h);
  return ok();
}

int moe_dispatch_ranks(moe_handle_t h, const void* d_x, const int32_t* d_topk_idx,
                       const float* d_w, void* d_out, int32_t* d_recv_idx, float* d_recv_w,
                       int64_t out_rows, hipStream_t stream) {
  const int st = check_rank_ready(h, "moe_dispatch_ranks");
  if (st != MOE_OK) return st;
  const int64_t capacity = rank_capacity(h);
  if (out_rows < capacity)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_dispatch_ranks: out_rows=%lld is below the capacity num_tokens*min(topk,R)=%lld",
                (long long)out_rows, (long long)capacity);
  if (h->rank_num_tokens == 0) return ok();
  if (d_x == nullptr || d_topk_idx == nullptr || d_w == nullptr || d_out == nullptr ||
      d_recv_idx == nullptr || d_recv_w == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch_ranks: a pointer argument is NULL");
  if (!aligned(d_x, 16) || !aligned(d_out, 16) || !aligned(d_topk_idx, 4) || !aligned(d_w, 4) ||
      !aligned(d_recv_idx, 4) || !aligned(d_recv_w, 4))
    return fail(MOE_ERR_INVALID_ARG,
                "moe_dispatch_ranks: x and out must be 16-byte aligned, the rest 4-byte aligned");
  const hipError_t err = moe::launch_dispatch_ranks(
      d_x, h->rank.slot_row, d_out, out_rows, h->rank_num_tokens, h->cfg.topk, h->cfg.hidden,
      h->max_workgroups, d_topk_idx, d_w, h->cfg.num_experts, h->cfg.num_ranks, d_recv_idx,
      d_recv_w, stream);
  return hip_status(err, "moe_dispatch_ranks");
}

int moe_combine_ranks(moe_handle_t h, const void* d_y, int64_t y_rows, void* d_out,
                      hipStream_t stream) {
  const int st = check_rank_ready(h, "moe_combine_ranks");
  if (st != MOE_OK) return st;
  const int64_t capacity = rank_capacity(h);
  if (y_rows < capacity)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_combine_ranks: y_rows=%lld is below the capacity num_tokens*min(topk,R)=%lld",
                (long long)y_rows, (long long)capacity);
  if (h->rank_num_tokens == 0) return ok();
  if (d_y == nullptr || d_out == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine_ranks: y or out is NULL");
  if (!aligned(d_y, 16) || !aligned(d_out, 16))
    return fail(MOE_ERR_INVALID_ARG, "moe_combine_ranks: y and out must be 16-byte aligned");
  const hipError_t err =
      moe::launch_combine_ranks(d_y, y_rows, h->rank.rank_pos, d_out, h->rank_num_tokens,
                                h->cfg.num_ranks, h->cfg.hidden, h->max_workgroups, stream);
  return hip_status(err, "moe_combine_ranks");
}

int moe_set_max_workgroups(moe_handle_t h, int32_t max_workgroups) {
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_set_max_workgroups: handle is NULL");
  if (max_workgroups < 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_set_max_workgroups: max_workgroups=%d must be >= 0",
                max_workgroups);
  h->max_workgroups = max_workgroups;
  return ok();
}

int moe_cu_mask(int32_t total_cus, int32_t num_cus, uint32_t* mask, int32_t mask_words) {
  if (mask == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_cu_mask: mask is NULL");
  const int32_t per = total_cus / MOE_EP_XCDS;   // compute units per XCD
  if (total_cus <= 0 || total_cus % MOE_EP_XCDS != 0 || per % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_cu_mask: total_cus=%d must be %d XCDs times a multiple of 8 compute units",
                total_cus, MOE_EP_XCDS);
  if (num_cus < MOE_EP_XCDS || num_cus > total_cus || num_cus % MOE_EP_XCDS != 0)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_cu_mask: num_cus=%d must be a multiple of %d in [%d, %d] (an equal share of "
                "every XCD)", num_cus, MOE_EP_XCDS, MOE_EP_XCDS, total_cus);
  if (int64_t(mask_words) * 32 < total_cus)
    return fail(MOE_ERR_INVALID_ARG, "moe_cu_mask: mask_words=%d cannot hold %d bits", mask_words,
                total_cus);
  for (int32_t i = 0; i < mask_words; ++i) mask[i] = 0u;
  // Bit b = per*x + 8*((x + q/8) % (per/8)) + (x + q) % 8 for XCD share x and
  // q = 0 .. num_cus/XCDS - 1. Whether the driver assigns bit b to XCD b % 8
  // (interleaved) or to XCD b / per (contiguous), every XCD gets exactly
  // num_cus / XCDS bits, and so does the complement; with the interleaved
  // assignment each XCD's bits also cycle through its shader engines.
  const int32_t m = num_cus / MOE_EP_XCDS, groups = per / 8;
  for (int32_t x = 0; x < MOE_EP_XCDS; ++x)
    for (int32_t q = 0; q < m; ++q) {
      const int32_t b = per * x + 8 * ((x + q / 8) % groups) + (x + q) % 8;
      mask[b / 32] |= 1u << (b % 32);
    }
  return ok();
}

int moe_stream_create_cu_limited(int32_t num_cus, hipStream_t* out) {
  if (out == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_stream_create_cu_limited: out is NULL");
  int dev = 0, total = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&total, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return hip_status(err, "moe_stream_create_cu_limited");
  uint32_t mask[64];
  if (total > 64 * 32)
    return fail(MOE_ERR_UNSUPPORTED, "moe_stream_create_cu_limited: %d compute units", total);
  const int words = (total + 31) / 32;
  const int st = moe_cu_mask(total, num_cus, mask, words);
  if (st != MOE_OK) return st;
  err = hipExtStreamCreateWithCUMask(out, static_cast<uint32_t>(words), mask);
  if (err != hipSuccess) return hip_status(err, "moe_stream_create_cu_limited");
  return ok();
}

int moe_stream_destroy(hipStream_t stream) {
  if (stream == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_stream_destroy: stream is NULL");
  return hip_status(hipStreamDestroy(stream), "moe_stream_destroy");
}

int moe_route(moe_handle_t h, const float* d_logits, int32_t num_tokens, int score,
              int32_t* d_topk_idx, float* d_topk_w, hipStream_t stream) {
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_route: handle is NULL");
  if (num_tokens < 0 || num_tokens > h->cfg.max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: num_tokens=%d outside [0, %d]", num_tokens,
                h->cfg.max_tokens);
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: unknown score %d", score);
  if (num_tokens == 0) return ok();
  if (d_logits == nullptr || d_topk_idx == nullptr || d_topk_w == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: logits, topk_idx or topk_w is NULL");
  if (!aligned(d_logits, 4) || !aligned(d_topk_idx, 4) || !aligned(d_topk_w, 4))
    return fail(MOE_ERR_INVALID_ARG, "moe_route: pointers must be 4-byte aligned");
  const hipError_t err = moe::launch_route(d_logits, num_tokens, h->cfg.num_experts, h->cfg.topk,
                                           score, d_topk_idx, d_topk_w, stream);
  return hip_status(err, "moe_route");
}

int moe_layout_dispatch(moe_handle_t h, const int32_t* d_topk_idx, int32_t num_tokens,
                        const void* d_x, int dtype, void* d_out, void* d_scales,
                        int64_t out_rows, hipStream_t stream) {
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_layout_dispatch: handle is NULL");
  const int32_t limit =
      h->cfg.max_tokens < MOE_EP_LL_MAX_TOKENS ? h->cfg.max_tokens : MOE_EP_LL_MAX_TOKENS;
  if (num_tokens < 0 || num_tokens > limit)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_layout_dispatch: num_tokens=%d outside [0, %d] (min of max_tokens and "
                "MOE_EP_LL_MAX_TOKENS; use moe_dispatch_layout + moe_dispatch for large batches)",
                num_tokens, limit);
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3 && dtype != MOE_DTYPE_MXFP8_E4M3)
    return fail(MOE_ERR_INVALID_ARG, "moe_layout_dispatch: unknown dtype %d", dtype);
  const int64_t capacity = int64_t(num_tokens) * h->cfg.topk;
  if (out_rows < capacity)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_layout_dispatch: out_rows=%lld is below the worst-case capacity "
                "num_tokens*topk=%lld",
                (long long)out_rows, (long long)capacity);
  if (dtype != MOE_DTYPE_BF16 && h->cfg.hidden % MOE_EP_FP8_BLOCK != 0)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_layout_dispatch: FP8 and MXFP8 need hidden to be a multiple of %d; hidden=%d",
                MOE_EP_FP8_BLOCK, h->cfg.hidden);
  if (num_tokens > 0 && (d_topk_idx == nullptr || d_x == nullptr || d_out == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "moe_layout_dispatch: topk_idx, x or out is NULL");
  if (num_tokens > 0 && dtype != MOE_DTYPE_BF16 && d_scales == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_layout_dispatch: FP8 dispatch needs a scales buffer");
  if (!aligned(d_topk_idx, 4) || !aligned(d_x, 16) || !aligned(d_out, 16) || !aligned(d_scales, 4))
    return fail(MOE_ERR_INVALID_ARG,
                "moe_layout_dispatch: x and out must be 16-byte aligned, topk_idx and scales "
                "4-byte");
  // The one-launch kernel counts over all T*k slots per workgroup; from
  // kLayoutDispatchFusedBelow tokens on the two launches are faster (measured:
  // 18.9 vs 23.8 us at 512 tokens, 46.2 vs 35.5 us at 1024, H=7168, top-8 of
  // 256), and they give the same results.
  hipError_t err;
  if (num_tokens < kLayoutDispatchFusedBelow) {
    h->order_chunks = 0;   // the one-launch form writes no block lists
    err = moe::launch_layout_dispatch(dtype, d_x, d_topk_idx, num_tokens, h->cfg.topk,
                                      h->cfg.num_experts, h->cfg.num_ranks, h->arrays, d_out,
                                      d_scales, h->cfg.hidden, h->max_workgroups, stream);
  } else {
    err = handle_layout(h, d_topk_idx, num_tokens, stream);
    if (err == hipSuccess)
      err = handle_dispatch(h, dtype, d_x, d_out, d_scales, out_rows, num_tokens, stream);
  }
  if (err != hipSuccess) {
    h->ready = false;
    return hip_status(err, "moe_layout_dispatch");
  }
  h->ready = true;
  h->num_tokens = num_tokens;
  return ok();
}

int moe_ll_dispatch(moe_handle_t h, const int32_t* d_topk_idx, int32_t num_tokens,
                    int32_t capacity, const void* d_x, int dtype, void* d_out, void* d_scales,
                    int64_t out_rows, hipStream_t stream) {
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_ll_dispatch: handle is NULL");
  const int32_t limit =
      h->cfg.max_tokens < MOE_EP_LL_MAX_TOKENS ? h->cfg.max_tokens : MOE_EP_LL_MAX_TOKENS;
  if (num_tokens < 0 || num_tokens > limit)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_ll_dispatch: num_tokens=%d outside [0, %d] (min of max_tokens and "
                "MOE_EP_LL_MAX_TOKENS; use moe_dispatch_layout + moe_dispatch for large batches)",
                num_tokens, limit);
  if (capacity < 1)
    return fail(MOE_ERR_INVALID_ARG, "moe_ll_dispatch: capacity=%d must be >= 1", capacity);
  const int64_t rows = int64_t(h->cfg.num_experts) * capacity;
  if (rows > kMaxSlots)
    return fail(MOE_ERR_UNSUPPORTED, "moe_ll_dispatch: num_experts*capacity=%lld exceeds %lld rows",
                (long long)rows, (long long)kMaxSlots);
  if (out_rows < rows)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_ll_dispatch: out_rows=%lld is below num_experts*capacity=%lld",
                (long long)out_rows, (long long)rows);
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_FP8_E4M3 && dtype != MOE_DTYPE_MXFP8_E4M3)
    return fail(MOE_ERR_INVALID_ARG, "moe_ll_dispatch: unknown dtype %d", dtype);
  if (dtype != MOE_DTYPE_BF16 && h->cfg.hidden % MOE_EP_FP8_BLOCK != 0)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_ll_dispatch: FP8 and MXFP8 need hidden to be a multiple of %d; hidden=%d",
                MOE_EP_FP8_BLOCK, h->cfg.hidden);
  if (num_tokens > 0 && (d_topk_idx == nullptr || d_x == nullptr || d_out == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "moe_ll_dispatch: topk_idx, x or out is NULL");
  if (num_tokens > 0 && dtype != MOE_DTYPE_BF16 && d_scales == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_ll_dispatch: FP8 dispatch needs a scales buffer");
  if (!aligned(d_topk_idx, 4) || !aligned(d_x, 16) || !aligned(d_out, 16) || !aligned(d_scales, 4))
    return fail(MOE_ERR_INVALID_ARG,
                "moe_ll_dispatch: x and out must be 16-byte aligned, topk_idx and scales 4-byte");
  const hipError_t err = moe::launch_dispatch_fixed(
      dtype, d_x, d_topk_idx, num_tokens, h->cfg.topk, h->cfg.num_experts, capacity, h->ll_pos,
      h->ll_counts, h->ll_status, d_out, d_scales, h->cfg.hidden, h->max_workgroups, stream);
  if (err != hipSuccess) {
    h->ll_ready = false;
    return hip_status(err, "moe_ll_dispatch");
  }
  h->ll_ready = true;
  h->ll_num_tokens = num_tokens;
  h->ll_capacity = capacity;
  return ok();
}

int moe_ll_view(moe_handle_t h, moe_ll_view_t* out) {
  if (out == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_ll_view: out is NULL");
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_ll_view: handle is NULL");
  if (!h->ll_ready)
    return fail(MOE_ERR_STATE, "moe_ll_view: no decode-time dispatch yet; call moe_ll_dispatch");
  out->pos = h->ll_pos;
  out->counts = h->ll_counts;
  out->status = h->ll_status;
  out->num_tokens = h->ll_num_tokens;
  out->capacity = h->ll_capacity;
  out->rows = int64_t(h->cfg.num_experts) * h->ll_capacity;
  return ok();
}

int moe_ll_combine(moe_handle_t h, const void* d_y, int64_t y_rows, const float* d_w,
                   void* d_out, hipStream_t stream) {
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "moe_ll_combine: handle is NULL");
  if (!h->ll_ready)
    return fail(MOE_ERR_STATE, "moe_ll_combine: no decode-time dispatch yet; call moe_ll_dispatch");
  const int64_t rows = int64_t(h->cfg.num_experts) * h->ll_capacity;
  if (y_rows < rows)
    return fail(MOE_ERR_INVALID_ARG, "moe_ll_combine: y_rows=%lld is below num_experts*capacity=%lld",
                (long long)y_rows, (long long)rows);
  if (h->ll_num_tokens == 0) return ok();
  if (d_y == nullptr || d_w == nullptr || d_out == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "moe_ll_combine: y, w or out is NULL");
  if (!aligned(d_y, 16) || !aligned(d_out, 16) || !aligned(d_w, 4))
    return fail(MOE_ERR_INVALID_ARG,
                "moe_ll_combine: y and out must be 16-byte aligned, w 4-byte aligned");
  const hipError_t err = moe::launch_combine(d_y, y_rows, d_w, h->ll_pos, d_out, h->ll_num_tokens,
                                             h->cfg.topk, h->cfg.hidden, h->max_workgroups, stream);
  return hip_status(err, "moe_ll_combine");
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_STATE: return "MOE_ERR_STATE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
