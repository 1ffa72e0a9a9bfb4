/*
 * moe_ep.h -- MoE expert-parallel token dispatch and combine on one GPU
 * (AMD Instinct MI355X, gfx950).
 *
 * What the operations are, per the source pages:
 *   - "Inside the Nebius + PyTorch DeepSeek V3 recipe", section
 *     "Mixture-of-experts and wide expert parallelism": each MoE layer
 *     exchanges tokens twice -- dispatch moves every token to the experts its
 *     router chose, and combine brings each expert's output back to the place
 *     of the token it belongs to.
 *   - Hybrid-EP news item, "Technical Structure": the library's two core
 *     operators are dispatch and combine; "Availability and Integration":
 *     buffers are preallocated for the worst case because routing is dynamic.
 *   - "MoE / Hybrid-EP Validation", table "Communication path comparison"
 *     and "FP8 dispatch restriction": dispatch may carry an FP8 payload; the
 *     measured shape is hidden 7168, 4096 tokens per rank, top-8, EP = 8
 *     ranks inside one node; "When EP crosses a node in an intra-node-only
 *     build": an unsupported configuration is refused at start-up with a
 *     message that names the fix.
 *
 * This library computes one EP rank's share of that work in local HBM: the
 * expert-major receive buffer is laid out for R virtual ranks (experts split
 * contiguously, E/R per rank), so rank r's rows form one contiguous slab.
 *
 * Layout rules (the pages give no formula; these are the plain readings):
 *   - slots (t, j), t < num_tokens, j < topk, are sorted stably by expert id
 *     in (t, j) order; pos[t*topk + j] is the row of slot (t, j);
 *   - counts_e[e] = number of slots routed to expert e, offsets_e is their
 *     exclusive prefix sum (E + 1 entries), counts_r / offsets_r the same per
 *     virtual rank, src_idx[row] = token of that row;
 *   - ids outside [0, E) are skipped: pos = -1, not counted, no row written,
 *     no contribution to combine; status[0] counts them;
 *   - capacity = num_tokens * topk rows (the worst case); rows at or past
 *     offsets_e[E] are unused and have src_idx = -1.
 *
 * Data formats: token ids int32; activations bf16 (bit patterns, row-major
 * [rows, hidden]); weights fp32 [num_tokens, topk]; FP8 payload OCP E4M3
 * ("e4m3fn", max 448) bytes with one fp32 scale per 128 channels:
 * scale = amax / 448 (fp32, correctly rounded), code = E4M3
 * round-to-nearest-even of the fp32 quotient x / scale; an all-zero block has
 * scale 0 and signed-zero codes. Combine: out[t] = bf16_rne(sum over j in
 * order 0..topk-1 of w[t,j] * y[pos[t,j]]) accumulated in fp32.
 *
 * Conventions:
 *   - every call returns a moe_status_t; nothing throws or aborts;
 *   - argument errors are found on the host and then nothing is enqueued;
 *   - device work is enqueued on the given stream and never synchronised;
 *   - device pointers must be 16-byte aligned, rows contiguous;
 *   - a handle is used by one stream at a time (calls on one handle from
 *     two streams race on its workspace);
 *   - moe_last_error() returns this thread's text for the last failure.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Limits checked at handle creation (MOE_ERR_UNSUPPORTED beyond them). */
#define MOE_EP_MAX_EXPERTS 1024
#define MOE_EP_MAX_TOPK 32
#define MOE_EP_FP8_BLOCK 128
#define MOE_EP_STATUS_WORDS 4
#define MOE_EP_LL_MAX_TOKENS 1024 /* num_tokens limit of the decode-time calls */
#define MOE_EP_XCDS 8             /* accelerator dies (XCDs) of an MI355X; CU masks split evenly */
#define MOE_EP_NOALLOC_SCRATCH_BYTES (2u << 20) /* per-GPU static scratch of the no-alloc layout */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, misaligned pointer, size out of range */
  MOE_ERR_UNSUPPORTED = 2, /* configuration outside the library's limits */
  MOE_ERR_STATE = 3,       /* dispatch/combine before a layout */
  MOE_ERR_HIP = 4          /* the HIP runtime refused a launch */
} moe_status_t;

typedef enum {
  MOE_DTYPE_BF16 = 0,      /* payload rows are bf16, copied bit for bit */
  MOE_DTYPE_FP8_E4M3 = 1,  /* E4M3 bytes + one fp32 scale per 128 channels */
  MOE_DTYPE_MXFP8_E4M3 = 2 /* OCP MX: E4M3 bytes + one E8M0 byte per 32 channels */
} moe_dtype_t;

typedef enum {
  MOE_SCORE_SOFTMAX = 0, /* w_j = exp(l_j) / sum_i exp(l_i) over the selected experts */
  MOE_SCORE_SIGMOID = 1  /* w_j = s_j / sum_i s_i, s = 1 / (1 + exp(-l)) */
} moe_score_t;

/* Fixed at handle creation. max_tokens bounds num_tokens of every layout. */
typedef struct {
  int32_t max_tokens;  /* T_max >= 0 */
  int32_t hidden;      /* H, multiple of 8 (of 128 for FP8 dispatch) */
  int32_t topk;        /* k, 1 <= k <= min(E, MOE_EP_MAX_TOPK) */
  int32_t num_experts; /* E, 1 <= E <= MOE_EP_MAX_EXPERTS */
  int32_t num_ranks;   /* R, virtual EP ranks, E % R == 0 */
} moe_config_t;

typedef struct moe_handle* moe_handle_t;

/* Device pointers into the handle's workspace, valid after a layout call has
 * been enqueued (their contents are valid once that stream work completes). */
typedef struct {
  int32_t* pos;       /* [num_tokens * topk] row of each slot, -1 if skipped */
  int32_t* src_idx;   /* [capacity] token of each row, -1 if unused */
  int32_t* counts_e;  /* [E] */
  int32_t* offsets_e; /* [E + 1] */
  int32_t* counts_r;  /* [R] */
  int32_t* offsets_r; /* [R + 1] */
  int32_t* status;    /* [MOE_EP_STATUS_WORDS]; [0] = skipped (invalid) slots */
  int32_t num_tokens; /* T of the last layout */
  int64_t capacity;   /* num_tokens * topk */
} moe_layout_view_t;

/* Bytes of device workspace a handle with this configuration needs, or 0 if
 * the configuration is invalid (moe_last_error() says why). */
size_t moe_workspace_bytes(const moe_config_t* cfg);

/* Validate cfg and bind a caller-owned device workspace (ws_bytes >=
 * moe_workspace_bytes(cfg), 256-byte aligned). The workspace stays owned by
 * the caller and must outlive the handle; the handle itself (host memory) is
 * owned by the library and released by moe_handle_destroy. Enqueues nothing.
 * MOE_ERR_UNSUPPORTED names the limit and the fix. */
int moe_handle_create(const moe_config_t* cfg, void* d_workspace, size_t ws_bytes,
                      moe_handle_t* out);

/* Release the host-side handle; the workspace is not touched. NULL is a no-op. */
void moe_handle_destroy(moe_handle_t h);

/* Layout: histogram, exclusive scan and stable placement of the routed slots.
 * d_topk_idx: int32 [num_tokens, topk] row-major, 0 <= num_tokens <= max_tokens.
 * Writes pos, src_idx, counts, offsets and status into the workspace on
 * `stream`; no host synchronisation. Marks the handle ready for dispatch and
 * combine with this num_tokens. For batches of at least 8 x 1024 slots whose
 * 1024-slot chunks each cover at most 3.5 MiB of x (1024 / topk tokens of
 * 2 * hidden bytes) and whose x is at most 192 MiB (num_tokens * 2 * hidden
 * bytes), it also writes, per block of consecutive slots, the
 * block's rows in ascending order (row, token), which the bf16 dispatch then
 * copies block by block, one XCD per block: the same rows, written one run per
 * expert at a time. */
int moe_dispatch_layout(moe_handle_t h, const int32_t* d_topk_idx, int32_t num_tokens,
                        hipStream_t stream);

/* Device pointers and sizes of the last layout (MOE_ERR_STATE before one). */
int moe_layout_view(moe_handle_t h, moe_layout_view_t* out);

/* Layout that allocates nothing and needs no handle or workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Computes exactly what
 * moe_dispatch_layout computes for a handle with this topk, num_experts and
 * num_ranks, into caller-owned device arrays: d_pos [num_tokens * topk],
 * d_src_idx [num_tokens * topk], d_counts_e [num_experts], d_offsets_e
 * [num_experts + 1], d_counts_r [num_ranks], d_offsets_r [num_ranks + 1],
 * d_status [MOE_EP_STATUS_WORDS] (all int32, 4-byte aligned; d_topk_idx,
 * d_pos and d_src_idx may be NULL when num_tokens is 0). The layout's
 * per-workgroup histograms go to a static device array of
 * MOE_EP_NOALLOC_SCRATCH_BYTES that each GPU holds until the process ends:
 * ceil(num_tokens * topk / 1024) * num_experts * 4 bytes must fit in it (e.g.
 * 2,097,152 slots at 256 experts; no histograms at all up to 24 * 1024
 * slots, which are laid out in one launch), else MOE_ERR_UNSUPPORTED and
 * nothing is enqueued. The configuration limits
 * are moe_handle_create's. Every call on one GPU shares that GPU's array, so
 * calls that may overlap on one GPU (other streams, other threads) race:
 * order them on one stream. The first call on each device looks the array up
 * (no allocation); no call allocates or frees memory. Enqueued on `stream`,
 * no host synchronisation. The results feed dispatch and combine only through
 * a handle's layout (moe_dispatch_layout); this call is for callers that
 * consume pos / offsets themselves. */
int moe_dispatch_layout_noalloc(const int32_t* d_topk_idx, int32_t num_tokens, int32_t topk,
                                int32_t num_experts, int32_t num_ranks, int32_t* d_pos,
                                int32_t* d_src_idx, int32_t* d_counts_e, int32_t* d_offsets_e,
                                int32_t* d_counts_r, int32_t* d_offsets_r, int32_t* d_status,
                                hipStream_t stream);

/* Dispatch: scatter token rows into the expert-major buffer.
 * d_x: bf16 [num_tokens, hidden]. out_rows >= capacity of the last layout.
 *   MOE_DTYPE_BF16:       d_out bf16 [out_rows, hidden], d_scales ignored;
 *   MOE_DTYPE_FP8_E4M3:   d_out uint8 [out_rows, hidden], d_scales fp32
 *                         [out_rows, hidden / 128] (hidden % 128 == 0);
 *   MOE_DTYPE_MXFP8_E4M3: d_out uint8 [out_rows, hidden], d_scales uint8 E8M0
 *                         [out_rows, hidden / 32] (hidden % 128 == 0; OCP
 *                         Microscaling v1.0: shared exponent floor(log2
 *                         amax) - 8 clamped to [-127, 127], elements E4M3
 *                         nearest-even of x / 2^shared clamped to +-448;
 *                         an all-zero block has code 0).
 * Row pos[t*k+j] receives token t; rows past the valid total are not written.
 * The bf16 rows are bit-identical whichever kernel form the layout selected
 * (the per-XCD block form above, or one workgroup per token slice; a workgroup
 * cap, moe_set_max_workgroups, always selects the latter). */
int moe_dispatch(moe_handle_t h, const void* d_x, int dtype, void* d_out, void* d_scales,
                 int64_t out_rows, hipStream_t stream);

/* Combine: top-k weighted gather back to token order.
 * d_y: bf16 [y_rows, hidden] indexed by the same rows as dispatch,
 * y_rows >= capacity; d_w: fp32 [num_tokens, topk]; d_out: bf16
 * [num_tokens, hidden]. A token whose slots are all skipped gets zeros. */
int moe_combine(moe_handle_t h, const void* d_y, int64_t y_rows, const float* d_w, void* d_out,
                hipStream_t stream);

/* ---- Rank-deduplicated exchange --------------------------------------------
 * What an expert-parallel exchange carries ("Inside the Nebius + PyTorch
 * DeepSeek V3 recipe", section "Mixture-of-experts and wide expert
 * parallelism": each rank holds a subset of the experts): a token routed to
 * several experts on one rank is sent to that rank once. Rows are grouped by
 * virtual rank, tokens in token order within a rank; capacity (the worst
 * case) is num_tokens * min(topk, R) rows. Each row carries the token's k
 * slots as the receiving rank numbers its experts (e - r*E/R, or -1 for a
 * slot whose expert is on another rank) and the slot weights (0 where -1),
 * so a receiver expands its rows to its experts with moe_dispatch_layout +
 * moe_dispatch on a handle with E/R experts and 1 rank (the -1 slots are
 * skipped), reduces them locally with moe_combine, and the source adds the
 * per-rank partial rows with moe_combine_ranks. */

typedef struct {
  int32_t* rank_pos;  /* [num_tokens, R] row of each (token, rank) pair, -1 if none */
  int32_t* slot_row;  /* [num_tokens * topk] row a slot opens (first slot of its token on
                         that rank), else -1 */
  int32_t* src_idx;   /* [capacity] token of each row, -1 past the valid total */
  int32_t* counts_r;  /* [R] tokens per rank */
  int32_t* offsets_r; /* [R + 1] */
  int32_t* status;    /* [MOE_EP_STATUS_WORDS]; [0] = rows in use, [1] = num_tokens */
  int32_t num_tokens;
  int64_t capacity;   /* num_tokens * min(topk, R) */
} moe_rank_layout_view_t;

/* Rank layout: which ranks each token goes to and the row of every
 * (token, rank) pair (histogram, exclusive scan, stable placement over the
 * R ranks). Same arguments and conventions as moe_dispatch_layout; uses its
 * own workspace regions, so both layouts can coexist. */
int moe_rank_layout(moe_handle_t h, const int32_t* d_topk_idx, int32_t num_tokens,
                    hipStream_t stream);

/* Device pointers and sizes of the last rank layout (MOE_ERR_STATE before one). */
int moe_rank_layout_view(moe_handle_t h, moe_rank_layout_view_t* out);

/* Send side of the exchange: row rank_pos[t, r] receives x[t] (bf16 [num_tokens,
 * hidden]) for every rank r the token reaches, plus the receiver metadata
 * recv_idx int32 [out_rows, topk] and recv_w fp32 [out_rows, topk].
 * d_topk_idx / d_w: the same int32 / fp32 [num_tokens, topk] the rank layout
 * was built from. out_rows >= capacity; rows past the valid total are not
 * written. Requires a rank layout (MOE_ERR_STATE otherwise). */
int moe_dispatch_ranks(moe_handle_t h, const void* d_x, const int32_t* d_topk_idx,
                       const float* d_w, void* d_out, int32_t* d_recv_idx, float* d_recv_w,
                       int64_t out_rows, hipStream_t stream);

/* Source side of the return trip: out[t] = bf16_rne(sum over ranks r in
 * ascending order of y[rank_pos[t, r]]), fp32 accumulation; y bf16 [y_rows,
 * hidden] holds each (token, rank) row's partial result, y_rows >= capacity;
 * out bf16 [num_tokens, hidden]. */
int moe_combine_ranks(moe_handle_t h, const void* d_y, int64_t y_rows, void* d_out,
                      hipStream_t stream);

/* Cap the dispatch and combine calls at the wavefronts of max_workgroups
 * workgroups of 4 (combine launches 2 * max_workgroups workgroups of 2; the
 * standard bf16 dispatch, from 512 workgroups on, 4 * max_workgroups / W
 * workgroups that spread a token's slots over W = min(ceil(k/2), 8)
 * wavefronts, at least one, and below 512 one wavefront per item with all k
 * slots); 0 (the default) launches one wavefront per (token, column slice)
 * item (bf16 dispatch: one workgroup per item). With a cap, each
 * wavefront loops over several (token, column slice) items, so the exchange
 * keeps fewer wavefronts resident; which compute units they run on is not
 * chosen here (moe_stream_create_cu_limited does that). Related to the
 * pages' point that the exchange should fill the link with few compute
 * units (Hybrid-EP news item, "Efficiency Numbers"). Results are
 * bit-identical for every cap. Negative values are MOE_ERR_INVALID_ARG.
 * Host-side only; enqueues nothing. */
int moe_set_max_workgroups(moe_handle_t h, int32_t max_workgroups);

/* ---- Compute-unit-limited streams -------------------------------------------
 * The Hybrid-EP news item ("Efficiency Numbers") makes the point that the
 * exchange should need only a few SMs (4 fill NVLink), leaving the rest of
 * the GPU to the expert computation. Here the caller runs dispatch and
 * combine on a stream whose kernels may only use num_cus compute units, and
 * its other work (an expert GEMM) on a stream limited to the complement.
 *
 * The hardware spreads a kernel's workgroups over the MI355X's 8 XCDs in
 * turn, so a mask must leave every XCD some compute units (an XCD with none
 * would hold its share of the workgroups forever). moe_cu_mask gives each XCD
 * num_cus / MOE_EP_XCDS bits whether the driver maps mask bit b to XCD b % 8
 * or to XCD b / (total_cus / 8), and the complement likewise.
 *
 * Measured on MI355X (T=4096, H=7168, top-8, inputs from HBM): 32 units move
 * 1.35 TB/s of bf16 dispatch alone, but beside a bf16 GEMM on the other 224
 * units about 0.5 TB/s -- the compute units are disjoint, the memory path
 * beyond them (L2, fabric, last-level cache, HBM) is shared. The GEMM keeps
 * over 90% of its rate. */

/* Fill mask[0 .. mask_words) (bit b of word b/32 = compute unit b) with
 * num_cus compute units out of total_cus, an equal share of every XCD.
 * total_cus: MOE_EP_XCDS times a multiple of 8; num_cus: a multiple of
 * MOE_EP_XCDS in [MOE_EP_XCDS, total_cus]; mask_words * 32 >= total_cus.
 * Host only: touches no device. */
int moe_cu_mask(int32_t total_cus, int32_t num_cus, uint32_t* mask, int32_t mask_words);

/* Create a stream on the current device whose kernels may use only the
 * num_cus compute units of moe_cu_mask(device CU count, num_cus)
 * (hipExtStreamCreateWithCUMask; the stream has the default priority).
 * Release it with moe_stream_destroy. A CU-limited stream has a hardware
 * queue of its own, so keep few of them alive at once. */
int moe_stream_create_cu_limited(int32_t num_cus, hipStream_t* out);

/* Destroy a stream made by moe_stream_create_cu_limited (after its work is
 * done: hipStreamDestroy semantics). */
int moe_stream_destroy(hipStream_t stream);

/* Router: top-k expert selection and combine weights, the step that produces
 * topk_idx / topk_w for the layout calls. Each token activates the top-k of
 * the experts ("Inside the Nebius + PyTorch DeepSeek V3 recipe", section
 * "Mixture-of-experts and wide expert parallelism"); the pages fix no tie
 * rule or gate, so: the k largest logits in descending order, equal logits
 * to the lower expert id (-0 equals +0); weights by `score` (moe_score_t)
 * over the selected experts, computed in fp32 (expf, IEEE division).
 * d_logits fp32 [num_tokens, num_experts] row-major (finite values; a NaN
 * gives NaN weights, ids stay in range); d_topk_idx int32 and d_topk_w fp32
 * [num_tokens, topk], written by this call. num_tokens in [0, max_tokens]. */
int moe_route(moe_handle_t h, const float* d_logits, int32_t num_tokens, int score,
              int32_t* d_topk_idx, float* d_topk_w, hipStream_t stream);

/* Layout and dispatch in one launch, for small batches: exactly the results
 * of moe_dispatch_layout followed by moe_dispatch (the standard packed
 * layout: pos, src_idx, counts, offsets and status in the handle, the rows
 * in d_out), computed by one kernel in which every workgroup derives its
 * token's rows from the ids themselves -- a row is the number of valid slots
 * with a smaller expert id plus the number of earlier slots with the same id.
 * That count grows with num_tokens^2: from 640 tokens on the call enqueues
 * the layout of moe_dispatch_layout and the dispatch instead (same results,
 * faster there), and num_tokens must lie in [0, min(max_tokens,
 * MOE_EP_LL_MAX_TOKENS)]. dtype, d_out, d_scales and out_rows as in
 * moe_dispatch. Leaves the handle's layout ready, as moe_dispatch_layout does:
 * moe_layout_view, moe_dispatch and moe_combine follow as usual. */
int moe_layout_dispatch(moe_handle_t h, const int32_t* d_topk_idx, int32_t num_tokens,
                        const void* d_x, int dtype, void* d_out, void* d_scales,
                        int64_t out_rows, hipStream_t stream);

/* Decode-time dispatch: layout and payload in one launch, into a buffer whose
 * shape does not depend on the routing -- the regime of DeepEP's low-latency
 * kernel family ("Inside the Nebius + PyTorch DeepSeek V3 recipe", section
 * "DeepEP"). Expert e owns rows [e*capacity, (e+1)*capacity) of d_out; a
 * slot's row is e*capacity + its rank among the slots routed to e in (token,
 * slot) order; a slot ranked capacity or more is dropped (no row, no combine
 * term, counted in status[3]); ids outside [0, E) are skipped (status[0]).
 * num_tokens in [0, min(max_tokens, MOE_EP_LL_MAX_TOKENS)] (each wavefront
 * counts over all earlier slots, O(num_tokens * topk)); capacity >= 1;
 * out_rows >= num_experts * capacity. dtype, d_out and d_scales as in
 * moe_dispatch (scales rows = out_rows). Rows no slot maps to are not
 * written. Records the positions and per-expert counts in the handle (see
 * moe_ll_view) for moe_ll_combine; independent of moe_dispatch_layout. */
int moe_ll_dispatch(moe_handle_t h, const int32_t* d_topk_idx, int32_t num_tokens,
                    int32_t capacity, const void* d_x, int dtype, void* d_out, void* d_scales,
                    int64_t out_rows, hipStream_t stream);

typedef struct {
  int32_t* pos;    /* [num_tokens * topk] row of each slot, -1 if skipped or dropped */
  int32_t* counts; /* [num_experts] rows received per expert (<= capacity) */
  int32_t* status; /* [4] invalid slots, placed slots, num_tokens, dropped slots */
  int32_t num_tokens;
  int32_t capacity;
  int64_t rows;    /* num_experts * capacity */
} moe_ll_view_t;

/* Device pointers of the last moe_ll_dispatch (MOE_ERR_STATE before one). */
int moe_ll_view(moe_handle_t h, moe_ll_view_t* out);

/* Combine after moe_ll_dispatch: as moe_combine, over the fixed-capacity
 * rows; y bf16 [y_rows, hidden], y_rows >= num_experts * capacity. Dropped
 * and skipped slots contribute nothing. */
int moe_ll_combine(moe_handle_t h, const void* d_y, int64_t y_rows, const float* d_w,
                   void* d_out, hipStream_t stream);

/* Static text for a status code. */
const char* moe_status_string(int status);

/* This thread's message for the last failed call ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
