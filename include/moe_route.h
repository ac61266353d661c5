/*
 * moe_route.h - MoE token routing, dispatch and combine on one MI355X (gfx950).
 *
 * A plain C ABI over hand-written HIP kernels. Every pointer argument named
 * "device" is device memory owned by the caller; the library allocates
 * nothing, keeps no global mutable state and only enqueues work on `stream`
 * (a hipStream_t passed as void*; NULL means the default stream). Nothing is
 * copied back to the host: the number of rows dispatch produced stays on the
 * device (expert_offsets[E]) and buffers are sized by capacity.
 *
 * The path, after the Perplexity posts "Efficient and portable
 * mixture-of-experts communication" (sections Introduction, Dispatch,
 * Combine) and "Enabling trillion-parameter models on AWS EFA" (sections Send
 * and receive buffers, Dispatch and Combine, Evaluation), reduced to one GPU's
 * share of the work:
 *
 *   logits --moe_route_topk--> topk_idx, topk_w
 *   x, topk_idx --moe_dispatch--> per-expert contiguous rows (+ FP8 scales),
 *                                 counts, offsets, group offsets, row maps
 *   (or both in one call: logits, x --moe_route_dispatch--> all of the above)
 *   (experts run on the rows)
 *   expert rows, dst_row, topk_w --moe_combine--> y
 *
 * Error behaviour: every function returns a moe_status. All argument checks
 * run on the host before any HIP call, so an invalid call launches nothing
 * and needs no GPU. Among them: every kernel a call would enqueue must fit
 * one launch packet, i.e. its blocks times threads per block stay below 2^32
 * work-items (the packet's grid size is a 32-bit count of work-items), else
 * the call returns MOE_EINVAL before its first launch. MOE_EHIP reports a launch failure; faults inside kernels
 * surface at the caller's next synchronisation. Values are not validated:
 * logits must be finite, and each token's expert ids must be distinct.
 * Calls on one stream are ordered; calls that share a workspace must not run
 * concurrently on different streams.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,   /* a size, count or option is out of range */
    MOE_ENOSPC = -2,   /* workspace smaller than moe_dispatch_workspace_bytes */
    MOE_EALIGN = -3,   /* a pointer lacks the alignment stated below */
    MOE_EHIP = -4,     /* a kernel launch failed */
    MOE_ENULL = -5     /* a required pointer is NULL */
} moe_status;

typedef enum {
    MOE_OUT_BF16 = 0,      /* dispatch rows are bf16 copies of x */
    MOE_OUT_FP8_E4M3 = 1   /* dispatch rows are OCP E4M3 codes + 1x128 fp32 scales */
} moe_out_dtype;

/* Largest expert count the kernels accept. */
#define MOE_MAX_EXPERTS 1024

/*
 * Router gate: per token, softmax over E logits, the k experts with the
 * highest scores, and their probabilities renormalised over the chosen k
 * ("Efficient and portable mixture-of-experts communication", Introduction:
 * the router yields a probability distribution, the top-K experts are used
 * and the output is a weighted average; the DeepSeek-V3 excerpts keep gating
 * in its original precision, so this runs in fp32).
 *
 *   logits   device, fp32 [T, E] row-major, finite values, 4-byte aligned
 *   topk_idx device, int32 [T, k] out: slot j holds the j-th best expert;
 *            experts are ranked by logit, descending; equal logits (IEEE
 *            equality, so -0 == +0) rank the lower expert index first
 *   topk_w   device, fp32 [T, k] out: exp(l_j - l_max) / sum over the k
 *            chosen of exp(l_i - l_max), which equals the softmax weight
 *            renormalised over the chosen experts; k == 1 gives exactly 1
 *   1 <= k <= E <= MOE_MAX_EXPERTS, T >= 0 (T == 0 is a no-op).
 */
int moe_route_topk(const float* logits, int64_t T, int E, int k,
                   int32_t* topk_idx, float* topk_w, void* stream);

/*
 * Shared experts treated as routed ones (DeepSeek-V3 excerpt on the third
 * page: every token selects its routed experts plus the shared expert, a
 * heavy-load expert that is always chosen). Same as moe_route_topk for slots
 * 0..k-1; slots k..k+n_shared-1 hold experts E..E+n_shared-1 with weight
 * shared_w (the pages do not give the shared expert's weight; 1 adds its
 * output unweighted). Outputs are [T, k + n_shared]; dispatch them with
 * E + n_shared experts and k + n_shared slots.
 *   0 <= n_shared, E + n_shared <= MOE_MAX_EXPERTS; other limits as above.
 */
int moe_route_topk_shared(const float* logits, int64_t T, int E, int k, int n_shared,
                          float shared_w, int32_t* topk_idx, float* topk_w, void* stream);

/*
 * Redundant expert replicas (DeepSeek-V3 excerpts: heavily loaded experts get
 * extra copies hosted as separate experts). In place on topk_idx [T, k]:
 * logical expert e owns physical experts replica_base[e] ..
 * replica_base[e+1]-1 (device int32 [E+1], non-decreasing, each e with at
 * least one copy) and token t uses copy t mod (its number of copies). Ids
 * outside [0, E) are left unchanged. Choosing which experts to replicate
 * (from load statistics) is the caller's; dispatch the result with
 * replica_base[E] experts.
 */
int moe_route_replicas(int32_t* topk_idx, int64_t T, int k, int E,
                       const int32_t* replica_base, void* stream);

/* Rows dispatch may use: T*k + E*(row_align-1); -1 if the arguments are
 * invalid or the count does not fit in int32. */
int64_t moe_dispatch_max_rows(int64_t T, int E, int k, int row_align);

/* Workspace bytes moe_dispatch and moe_route_dispatch need (per-tile expert
 * counts and prefixes, in-tile ranks); 0 on invalid arguments. The
 * workspace holds nothing between calls and needs no initialisation; calls
 * sharing a workspace must not overlap. */
size_t moe_dispatch_workspace_bytes(int64_t T, int E, int k, int groups);

/*
 * Dispatch: count tokens per expert, turn the counts into segment offsets by
 * an exclusive running sum, and pack every (token, slot) pair into its
 * expert's contiguous segment ("Enabling trillion-parameter models on AWS
 * EFA", Dispatch and Combine: per-expert counts, then their cumulative sum as
 * the offsets for packing tokens into contiguous per-expert send buffers;
 * "Efficient and portable mixture-of-experts communication", Dispatch:
 * activations, block scales and the token index travel together and the
 * source and token index are stored per row). Within a segment rows are in
 * token order, so the layout is deterministic. With FP8, activations are
 * scaled per token per 128 channels (DeepSeek-V3 excerpt on 1x128 tiles):
 * s = amax / 448 in fp32, each code is the correctly rounded fp32 quotient
 * x / s rounded to nearest-even E4M3 and saturated to +-448; an all-zero
 * block has s = 0 and zero codes.
 *
 *   x              device, bf16 [T, H], 16-byte aligned
 *   topk_idx       device, int32 [T, k]; an id outside [0, E) drops that slot
 *                  (not counted, dst_row = -1, no row written)
 *   T, H, E, k     1 <= k <= E <= MOE_MAX_EXPERTS; H % 8 == 0 (bf16) or
 *                  H % 128 == 0 (FP8); 1 <= H <= 65536; T * k < 2^31; the
 *                  row kernel must fit a launch packet: 64 * T *
 *                  ceil(H / 512) < 2^32 for bf16 rows, T * 256 < 2^32 for FP8
 *                  rows up to H = 4096 (up to 1024 threads per token above)
 *   groups         destination groups (1 = none), E % groups == 0; group g
 *                  holds experts [g*E/groups, (g+1)*E/groups), so its rows
 *                  form one contiguous send buffer
 *   row_align      1..1024: every non-empty segment is padded to a multiple of
 *                  this many rows; pad rows have zero payload, zero scales and
 *                  row_src = -1 and sit at the end of the segment
 *   out_dtype      moe_out_dtype
 *   out            device [max_rows, H] bf16 or E4M3 bytes, 16-byte aligned
 *   out_scales     device fp32 [max_rows, H/128] for FP8 (4-byte aligned),
 *                  ignored for bf16
 *   expert_counts  device int32 [E] out: pairs routed to each expert
 *   expert_offsets device int32 [E+1] out: first row of each segment;
 *                  expert_offsets[E] is the number of rows used
 *   group_offsets  device int32 [groups+1] out, or NULL: first row of each
 *                  group's send buffer
 *   row_src        device int32 [max_rows] out: t*k+j of the pair in each
 *                  row, -1 for pad rows
 *   dst_row        device int32 [T, k] out: the row holding each pair
 *   workspace      device, >= moe_dispatch_workspace_bytes, 16-byte aligned
 * Rows at and beyond expert_offsets[E] are left untouched. max_rows is
 * moe_dispatch_max_rows(T, E, k, row_align). T == 0 writes zero counts and
 * offsets. Three kernels: per-tile counts and ranks, the scan into offsets,
 * the rows (two for batches of at most 64 count tiles, whose row kernel
 * does the scan). On a stream created with a CU mask the scan kernel runs
 * one block per CU of the mask (at most 128); the results do not depend on
 * the mask.
 */
int moe_dispatch(const void* x, const int32_t* topk_idx,
                 int64_t T, int H, int E, int k, int groups, int row_align,
                 int out_dtype, void* out, float* out_scales,
                 int32_t* expert_counts, int32_t* expert_offsets,
                 int32_t* group_offsets, int32_t* row_src, int32_t* dst_row,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_topk followed by moe_dispatch in one call, with the same results
 * as the two calls: the router's top-k and weights ("Efficient and portable
 * mixture-of-experts communication", Introduction) feed the counts, offsets
 * and packing of "Enabling trillion-parameter models on AWS EFA", Dispatch
 * and Combine. When k <= 8, E <= 768, E % 4 == 0 and logits is 16-byte
 * aligned, routing runs inside the counting kernel (three launches in all,
 * two for batches of at most 64 count tiles); if besides E <= 48, T <= 256
 * and T * k <= 1024, every block of the packing kernel routes the whole
 * batch itself and the call is one launch. Otherwise moe_route_topk's
 * kernel runs first (four launches).
 *
 *   logits         device fp32 [T, E], finite, 4-byte aligned
 *   topk_idx       device int32 [T, k] out (as moe_route_topk), then read by
 *                  the packing
 *   topk_w         device fp32 [T, k] out (as moe_route_topk)
 *   other arguments, limits and outputs as for moe_dispatch (workspace:
 *   moe_dispatch_workspace_bytes).
 */
int moe_route_dispatch(const float* logits, const void* x,
                       int64_t T, int H, int E, int k, int groups, int row_align,
                       int out_dtype, int32_t* topk_idx, float* topk_w,
                       void* out, float* out_scales,
                       int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* group_offsets, int32_t* row_src, int32_t* dst_row,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_dispatch for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call and results without a workspace argument. Its workspace is a static
 * device array of MOE_NO_ALLOC_SCRATCH_BYTES inside the library, one per
 * GPU, resident until the process ends; the call allocates nothing (no
 * hipMalloc, no allocating library routine). Its address is looked up once
 * per device, on the first call made with that device current.
 *   Arguments, limits and outputs as for moe_dispatch.
 *   Returns MOE_ENOSPC, before any HIP call, when the call needs more than
 *   MOE_NO_ALLOC_SCRATCH_BYTES of workspace (moe_dispatch_workspace_bytes).
 *   MOE_EHIP if the scratch address cannot be obtained or a launch fails.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (concurrent streams, or with a graph replay holding such a call) race
 * and give undefined results. Calls ordered on one stream are safe: each
 * call writes what it reads of the array before reading it.
 */
#define MOE_NO_ALLOC_SCRATCH_BYTES (16u << 20)

int moe_dispatch_no_alloc(const void* x, const int32_t* topk_idx,
                          int64_t T, int H, int E, int k, int groups, int row_align,
                          int out_dtype, void* out, float* out_scales,
                          int32_t* expert_counts, int32_t* expert_offsets,
                          int32_t* group_offsets, int32_t* row_src, int32_t* dst_row,
                          void* stream);

/*
 * Combine: each token's output is the weighted sum of the rows its experts
 * produced, y[t] = bf16(sum_j topk_w[t,j] * expert_out[dst_row[t,j]]),
 * accumulated in fp32 in slot order and rounded once to bf16 (nearest even).
 * This is the receiving side's weighted average ("Efficient and portable
 * mixture-of-experts communication", Combine: the routing table gives the
 * buffer to read and the weight of each expert; "Enabling trillion-parameter
 * models on AWS EFA", Evaluation: accumulation only on the receiving side;
 * the DeepSeek-V3 excerpts keep combine in BF16).
 *
 *   expert_out  device bf16 [rows, H], 16-byte aligned; rows named by dst_row
 *   dst_row     device int32 [T, k]; a negative entry contributes nothing
 *   topk_w      device fp32 [T, k]
 *   y           device bf16 [T, H] out, 16-byte aligned
 *   H % 8 == 0, 1 <= H <= 65536, 1 <= k <= MOE_MAX_EXPERTS, T >= 0,
 *   T * k < 2^31, 64 * T * ceil(H / 512) < 2^32 (one 64-lane wave per token
 *   and 512 columns must fit a launch packet).
 */
int moe_combine(const void* expert_out, const int32_t* dst_row,
                const float* topk_w, int64_t T, int H, int k,
                void* y, void* stream);

/*
 * Combine with partial sums on the sending side, as two halves. In the
 * expert-parallel setting each destination group is the rank hosting a range
 * of experts; that rank pre-sums, per token, the weighted rows of the token's
 * experts it hosts and sends one bf16 row per (token, group) instead of one
 * row per (token, expert); the token's owner then sums the partial rows
 * ("Enabling trillion-parameter models on AWS EFA", Evaluation: DeepEP
 * accumulates on the sender to cut transferred bytes, which may cost
 * accuracy; moe_combine is the receiver-only alternative).
 *
 * moe_combine_send
 *   expert_out, dst_row, topk_w  as for moe_combine
 *   topk_idx     device int32 [T, k]: the experts of the slots (as routed)
 *   E, groups    group of expert e is e / (E / groups); E % groups == 0
 *   partial      device bf16 [T, k, H] out, 16-byte aligned: token t's partial
 *                rows at [t, 0 .. partial_count[t]), one per distinct group of
 *                its live slots in ascending group order; each is the fp32 sum
 *                (slot order) of that group's weighted rows rounded to bf16
 *   partial_count device int32 [T] out: partial rows of each token
 * moe_combine_recv
 *   partial, partial_count  as written by moe_combine_send
 *   y            device bf16 [T, H] out: bf16 of the fp32 sum of the token's
 *                partial rows in order
 * Limits as for moe_combine; moe_combine_send also needs 1 <= k <= E <= 1024.
 */
int moe_combine_send(const void* expert_out, const int32_t* dst_row,
                     const float* topk_w, const int32_t* topk_idx,
                     int64_t T, int H, int E, int k, int groups,
                     void* partial, int32_t* partial_count, void* stream);

int moe_combine_recv(const void* partial, const int32_t* partial_count,
                     int64_t T, int H, int k, void* y, void* stream);

/*
 * Grouped GEMM consumer of the FP8 segments (DeepSeek-V3 report excerpts on
 * the fourth page: fine-grained quantisation with 1x128 activation tiles and
 * 128x128 weight blocks, and the promotion of each 128-element interval's
 * partial sum into higher-precision accumulators). For every expert e and
 * every row r in [expert_offsets[e], expert_offsets[e+1]):
 *
 *   y[r, n] = bf16_RNE( sum_b a_scales[r, b] * w_scales[e, n/128, b]
 *                       * sum_{k = 128b}^{128b+127} e4m3(a[r, k]) * e4m3(w[e, n, k]) )
 *
 * The partial of each interval comes from the matrix cores in fp32 (their
 * internal summation of an interval is not exact IEEE fp32); it is scaled by
 * the fp32 product of the two scales and added into an fp32 accumulator.
 * Pad rows of a moe_dispatch segment have zero codes and zero scales, so
 * their outputs are +0.
 *
 *   a               device E4M3 [max_rows, K]: moe_dispatch's out in FP8
 *                   mode; 16-byte aligned
 *   a_scales        device fp32 [max_rows, K/128]: moe_dispatch's out_scales
 *   expert_offsets  device int32 [E+1]: moe_dispatch's expert_offsets (any
 *                   row_align works; with 128 every 128-row tile is full).
 *                   Segment ends are clamped to max_rows.
 *   w               device E4M3 [E, N, K], K contiguous; 16-byte aligned
 *   w_scales        device fp32 [E, N/128, K/128]
 *   E, N, K         1 <= E <= 1024; 256 <= N <= 2^20 with N % 256 == 0;
 *                   128 <= K <= 2^20 with K % 128 == 0
 *   max_rows        rows of a, a_scales and y (the dispatch capacity,
 *                   moe_dispatch_max_rows); 0 <= max_rows < 2^31
 *   y               device bf16 [max_rows, N] out; 8-byte aligned. Rows at or
 *                   past expert_offsets[E] are not written.
 *   workspace       device, 16-byte aligned, at least
 *                   moe_grouped_gemm_workspace_bytes(max_rows, E) bytes
 *                   (the list of 128-row tiles, built on the device)
 * The caller owns every buffer; nothing is kept between calls. Errors:
 * MOE_EINVAL (limits), MOE_ENULL, MOE_EALIGN, MOE_ENOSPC (workspace),
 * MOE_EHIP (launch). max_rows == 0 returns MOE_OK without a launch.
 */
size_t moe_grouped_gemm_workspace_bytes(int64_t max_rows, int E);

int moe_grouped_gemm_fp8(const void* a, const float* a_scales, const int32_t* expert_offsets,
                         const void* w, const float* w_scales, int E, int N, int K,
                         int64_t max_rows, void* y, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Stand-in experts for tests and the benchmark (not part of the path):
 * expert_out[r] = bf16(v * c_e) with c_e = fp32(e+1) / fp32(E) (or 1 when
 * identity != 0), e the expert of row r, v the bf16 row or, for FP8 rows,
 * the code's value times its block scale in fp32. Pad rows become zero. Rows
 * from expert_offsets[E] up to max_rows are not written.
 *
 *   disp, disp_scales  moe_dispatch's out / out_scales
 *   row_src, topk_idx  moe_dispatch's row_src and its topk_idx input
 *   expert_offsets     moe_dispatch's expert_offsets
 *   expert_out         device bf16 [max_rows, H] out, 16-byte aligned
 */
int moe_harness_expert_scale(const void* disp, const float* disp_scales,
                             const int32_t* row_src, const int32_t* topk_idx,
                             const int32_t* expert_offsets, int64_t max_rows,
                             int H, int E, int out_dtype, int identity,
                             void* expert_out, void* stream);

/* Static text for a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
