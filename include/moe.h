/*
 * moe.h -- C ABI of libmoe: one GPU's share of a Mixture-of-Experts layer
 * forward on MI355X (gfx950), as hand-written HIP kernels.
 *
 * Sources for the operations declared here:
 *   [kucoin]   "Cursor's MoK logra un aumento del 2.37x en el rendimiento en
 *              NVIDIA GB300 NVL72" (kucoin.com/es news; same text in Vietnamese,
 *              Hindi and Chinese), sections 01, 02 and 03.
 *   [qubstore] "Смесь котят: как Cursor создал открытое ядро, ускоряющее обучение
 *              ИИ до 2,4 раз" (qubstore.ru): MoE primer, pull, ring buffer and
 *              megakernel paragraphs.
 *
 * Shapes: R source ranks (each with its own token and output buffers; on one GPU
 * the "remote" ranks are separate HBM allocations), T tokens per rank, hidden size
 * d, E global experts of which E_local live on this GPU, top-k = k, expert SwiGLU
 * width F.  A "pair" is one (rank, token, j) choice, j in [0, k); N is the number
 * of pairs whose expert is local (known on the device only, = offsets[E_local]).
 *
 * Conventions for every call below:
 *   - All buffer pointers are DEVICE pointers owned by the caller, except the
 *     per-rank pointer tables (`const T* const* p`), which are HOST arrays of R
 *     device pointers, read during the call only.  R <= MOE_MAX_RANKS.
 *   - The library allocates no memory and keeps no pointer after a call returns.
 *     Scratch lives in the caller's workspace `ws` of at least
 *     moe_workspace_bytes() bytes, 256-byte aligned.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL =
 *     the default stream)
 *     and make no host<->device copy or synchronisation; the only host-side work
 *     is argument checking and kernel launches.
 *   - Return 0 on success, a negative MOE_E* code otherwise; a failing call
 *     launches nothing (argument errors) or reports the HIP launch error.
 *     Errors detected on the device (invalid expert placement, watchdog) are
 *     written to a status word in the workspace, read by moe_read_status().
 *   - NaN or infinite logits are outside the contract.
 *   - Row storage: element type per moe_dtype_t, rows of d (or F) elements,
 *     densely packed; every row must be 16-byte aligned (d * elem_size % 16 == 0).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MAX_RANKS 64

/* error codes */
#define MOE_OK 0
#define MOE_EINVAL (-1)   /* bad shape, k, dtype, placement or NULL pointer */
#define MOE_EALIGN (-2)   /* row not 16-byte aligned, or d/F not a multiple the kernels need */
#define MOE_ENOSPC (-3)   /* workspace too small, or ring smaller than one slot */
#define MOE_EHIP (-4)     /* a HIP launch failed */
#define MOE_ETIMEOUT (-5) /* a device-side wait exceeded its watchdog budget */
#define MOE_EUNSUP (-6)   /* combination not built (e.g. dtype for this entry point) */
#define MOE_EINCOMPLETE (-7) /* the persistent kernel ended with work left undone (a pipeline
                                received no data-movement or no compute workgroup) */

typedef enum {
  MOE_F32 = 0,   /* fp32 rows and weights, fp32 arithmetic */
  MOE_BF16 = 1,  /* bf16 rows and weights, fp32 accumulation, bf16 h and outputs */
  MOE_MXFP8 = 2  /* bf16 token rows and outputs; the expert GEMMs in MXFP8: E4M3 elements
                    with one E8M0 scale per 32 consecutive K values (see moe_mx_quantize) */
} moe_dtype_t;

typedef struct {
  int32_t R, T, d, E, k, F;
  int32_t dtype; /* moe_dtype_t */
} moe_shape_t;

/* Expert placement: which global experts live on this GPU.
 * expert_to_local: DEVICE array [E] of int32, value in [0, E_local) or -1; the
 * local ids must be a bijection onto [0, E_local) (checked on the device: a bad
 * map sets MOE_EINVAL in the status word and the layout yields N = 0). */
typedef struct {
  const int32_t* expert_to_local;
  int32_t E_local;
} moe_placement_t;

/* MXFP8 scale layout (every scale array below): for a matrix of `rows` rows of K values
 * (K a multiple of 128), the E8M0 code of 32-value block b of row r is the byte at offset
 *     4 * (rows * (b / 4) + r) + b % 4,
 * i.e. one 32-bit word per (128-value K tile, row), K tiles outermost: [K/128][rows][4].
 * The grouped GEMM reads the words of 64 consecutive rows of one K tile at once.
 *
 * Block scales of MXFP8 expert weights (moe_mx_quantize of the bf16 weights), DEVICE
 * pointers, 4-byte aligned.  Used only when dtype is MOE_MXFP8, where the weight pointers
 * w1, w3, w2 hold E4M3 codes of the same [E_local][F][d] / [E_local][d][F] shapes (one byte
 * per value); each scale array covers the whole tensor as one matrix of E_local*F (or
 * E_local*d) rows. */
typedef struct {
  const uint8_t* w1;   /* [d/128][E_local*F][4] */
  const uint8_t* w3;   /* [d/128][E_local*F][4] */
  const uint8_t* w2;   /* [F/128][E_local*d][4] */
} moe_mx_scales_t;

/* Execution knobs.  Zero selects the default of each field. */
typedef struct {
  int32_t minibatch_rows;   /* rows of one expert released to compute at once (default 128;
                               the persistent path takes 64, 128 or 256) */
  int32_t comm_cus;         /* persistent path: workgroups doing data movement (default 16) */
  int32_t ring_slots;       /* persistent path: cap on ring slots (default: as many as ring_bytes holds) */
  int32_t trace;            /* persistent path: 1 = record a per-workgroup event trace into the
                               workspace (moe_persistent_trace_info); every other entry point
                               requires 0 (else MOE_EINVAL) */
  uint64_t watchdog_us;     /* persistent path: wall-clock budget of every device wait in
                               microseconds (default 2,000,000) */
  int32_t reverse_ring;     /* persistent path: 1 = walk each pipeline's row tiles in reverse
                               and keep every chunk's token rows and h rows in its ring slot
                               (the down GEMM stores the outputs straight to recv), so that
                               at the end the ring holds the activations of the first chunks,
                               which moe_backward_ring reads in place; 0 = layout order, the
                               outputs overwrite the token rows in the ring (in MXFP8 they always
                               go straight to recv).  Every other entry point requires 0 (else
                               MOE_EINVAL) */
} moe_exec_t;

/* Limits checked by every call: 1 <= k <= 16, k <= E <= 1024, 1 <= E_local <= E. */

/* Worst-case local pairs: R * T * min(k, E_local).  Sizes of xe/ye/pull_src below. */
int64_t moe_max_pairs(const moe_shape_t* s, const moe_placement_t* p);

/* Workspace bytes needed by every call below for this shape (a pure host function). */
size_t moe_workspace_bytes(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex);

/*
 * moe_mx_quantize -- MXFP8 quantisation of `rows` rows of K values [kucoin §02: MXFP8 in
 * the expert data path; the pages give no rule, the one used is OCP Microscaling v1.0]:
 * for every block of 32 consecutive values v of a row, amax = max |v|;
 *   amax == 0: scale code 0 and 32 zero codes;
 *   otherwise e = clamp(floor(log2 amax) - 8, -127, 127), scale code e + 127, and
 *   code_i = E4M3(v_i / 2^e) rounded to nearest (ties to even), saturated to +-448.
 * src: [rows][K] of src_dtype (MOE_BF16 or MOE_F32), 16-byte aligned; codes: [rows][K]
 * bytes, 16-byte aligned; scales: rows*K/32 bytes in the MXFP8 scale layout above
 * ([K/128][rows][4]).  K % 128 == 0 (else MOE_EALIGN).
 * Used offline on expert weights; moe_dispatch_pull and the GEMM1 epilogue apply the
 * same rule to token rows and h.  Bit-exact (integer decisions, exact power-of-two
 * scaling).
 */
int moe_mx_quantize(const void* src, int32_t src_dtype, int64_t rows, int32_t K, uint8_t* codes,
                    uint8_t* scales, void* stream);

/*
 * moe_layout -- routing and sort-free layout generation.
 *   [kucoin §01] the router picks several experts per token every step; the
 *   system counts each expert's tokens, decides where they land on the target and
 *   keeps one expert's tokens contiguous for the grouped GEMM.
 *   [kucoin §02] / [qubstore, pull] the puller needs only (source GPU, position in
 *   the source) -- a two-column schedule -- and decides local placement itself,
 *   without sorting.
 * Computes, for every rank r and token t (logits[r] is [T][E] fp32):
 *   topk_idx[r][t][j]: the k largest logits, ties to the lower expert id, listed
 *                      in descending logit order                    [R][T][k] int32
 *   topk_w[r][t][j]:   exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k kept  [R][T][k] fp32
 *   counts[e]:         pairs routed to global expert e, over all ranks       [E] int32
 *   offsets[l]:        exclusive prefix of counts over local ids; offsets[E_local] = N
 *                                                                   [E_local+1] int32
 *   pull_src[s]:       (source rank, source token) of local row s, rows of one
 *                      expert in ascending (r, t, j) order   [moe_max_pairs][2] int32
 *   slot_of[r][t][j]:  row s of the pair, or -1 if its expert is not local [R][T][k] int32
 * Also writes the chunk table (<= minibatch_rows rows of one expert per chunk)
 * into `ws`, used by the calls below.  All outputs are bit-exact (integer work;
 * the gate uses fp32 expf).
 */
int moe_layout(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
               const float* const* logits, int32_t* topk_idx, float* topk_w, int32_t* counts,
               int32_t* offsets, int32_t* pull_src, int32_t* slot_of, void* ws, size_t ws_bytes,
               void* stream);

/*
 * moe_dispatch_pull -- pull dispatch [kucoin §02: the expert side reads the
 * token rows it needs from their source; qubstore, pull paragraph].
 *   xe[s][:] = x[pull_src[s].rank][pull_src[s].token][:]  for s in [0, N)
 * x: R device pointers, each [T][d] rows.  xe: [moe_max_pairs][d] rows.
 * offsets/ws: from moe_layout (N is read on the device).  Bit-exact copy.
 * MOE_MXFP8 [kucoin §02: quantisation fused into the dispatch]: x is bf16 and each row
 * is quantised on its way (the moe_mx_quantize rule): xe receives [moe_max_pairs][d]
 * E4M3 codes and xe_scales their scale codes in the MXFP8 scale layout with
 * rows = moe_max_pairs ([d/128][moe_max_pairs][4], 4-byte aligned).
 * xe_scales is ignored for the other dtypes.
 */
int moe_dispatch_pull(const moe_shape_t* s, const moe_placement_t* p, const void* const* x,
                      const int32_t* pull_src, const int32_t* offsets, void* xe, uint8_t* xe_scales,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn -- grouped SwiGLU expert FFN [kucoin §01: grouped GEMM over
 * expert-contiguous rows; kucoin §02: SwiGLU in the expert data path].
 * For every local expert l and row s in [offsets[l], offsets[l+1]):
 *   h = silu(xe[s] W1[l]^T) * (xe[s] W3[l]^T)   (length F; stored as the row dtype)
 *   ye[s] = h W2[l]^T                             (length d; fp32 accumulate)
 * w1, w3: [E_local][F][d]; w2: [E_local][d][F]; xe, ye: [moe_max_pairs][d].
 * bf16: d and F must be multiples of 64.  Accuracy: see moe_forward tolerances
 * in the tests (bf16 max row-relative error <= 2e-2 against an fp64 oracle).
 * MOE_MXFP8 [kucoin §02: quantisation fused into the grouped GEMM and SwiGLU]: xe and
 * xe_scales as moe_dispatch_pull writes them, weights as E4M3 codes with w_scales
 * (moe_mx_quantize of the bf16 weights); h is quantised along F in GEMM1's epilogue
 * (fp32 h, the same rule); ye is bf16 with fp32 accumulation.  d and F must be
 * multiples of 128.  Accuracy against the fp64 forward on the dequantised operands (with
 * h quantised from its fp64 value): max row-relative error <= 6e-2 and relative Frobenius
 * error <= 5e-3; h is quantised from fp32, so an h code may differ from that reference's
 * by one E4M3 step where the value lies within fp32 rounding of the midpoint, and each
 * output element then lies within the effect of those steps plus one bf16 rounding.
 * xe_scales and w_scales are ignored for other dtypes.
 */
int moe_expert_ffn(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                   const void* xe, const uint8_t* xe_scales, const int32_t* offsets, const void* w1,
                   const void* w3, const void* w2, const moe_mx_scales_t* w_scales, void* ye, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn_push -- the expert FFN with the combine's push fused into the down GEMM's
 *   epilogue [kucoin §02: combine is a push because the destination of every result row is
 *   already known] and, for fp32 and bf16, optionally the pull fused into the gate/up GEMM's
 *   operand loads [kucoin §02: the expert side reads the token rows it needs from their
 *   source buffers].
 *   Same arithmetic as moe_expert_ffn.  Instead of ye[s] the down GEMM writes each result
 *   row straight to recv[r][t][j], where (r, t) = pull_src[s] and slot_of[r][t][j] == s.
 *   With x != NULL (fp32, bf16) the gate/up GEMM reads row s straight from x[r][t] instead
 *   of xe[s], so no dispatch (moe_dispatch_pull) is needed and xe is neither read nor
 *   written (may be NULL); with x == NULL it reads xe as moe_dispatch_pull wrote it.
 *   recv entries of local pairs are bit-identical to moe_dispatch_pull + moe_expert_ffn +
 *   the push of moe_combine_push; entries without a local pair are not written.  Per-pair
 *   address tables are built in the workspace first (16 bytes per pair, counted by
 *   moe_workspace_bytes).
 * x: NULL or R device pointers [T][d]; recv: R device pointers, each [T][k][d]; both
 *   16-byte aligned.  Other arguments, alignment and dtype rules as moe_expert_ffn.
 * Errors: MOE_EINVAL for a missing pull_src, slot_of or recv entry (or xe when x is NULL);
 *   MOE_EUNSUP for x != NULL with MOE_MXFP8 (its rows are quantised by the gather);
 *   otherwise as moe_expert_ffn.
 */
int moe_expert_ffn_push(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                        const void* const* x, const void* xe, const uint8_t* xe_scales, const int32_t* offsets,
                        const void* w1, const void* w3, const void* w2, const moe_mx_scales_t* w_scales,
                        const int32_t* pull_src, const int32_t* slot_of, void* const* recv, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * moe_weighted_merge -- the final weighted merge alone [kucoin §03: the final weighted merge
 *   is a step of its own]: y[r][t][:] = sum over ascending j with slot_of[r][t][j] >= 0 of
 *   topk_w[r][t][j] * recv[r][t][j][:], fp32 accumulation, rounded once to the row dtype;
 *   exactly 0 for a token with no local pair.  Deterministic.  Reads only the recv entries of
 *   local pairs.  recv: R pointers [T][k][d]; y: R pointers [T][d]; both 16-byte aligned.
 * Errors: MOE_EINVAL for a missing slot_of, topk_w or table entry; MOE_EALIGN for a
 *   misaligned row buffer.
 */
int moe_weighted_merge(const moe_shape_t* s, const moe_placement_t* p, const int32_t* slot_of,
                       const float* topk_w, void* const* recv, void* const* y, void* stream);

/*
 * moe_combine_push -- push combine then the final weighted merge
 *   [kucoin §01: combine returns each result to the token's original position;
 *   kucoin §02: combine is a push since the destination is known; kucoin §03: the
 *   final weighted merge is a step of its own].
 * Push: for s in [0, N): recv[r][t][j][:] = ye[s][:] where (r, t) = pull_src[s]
 *   and j is the pair with slot_of[r][t][j] == s (bit-exact copy, no atomics).
 * Merge: y[r][t][:] = sum over ascending j with slot_of[r][t][j] >= 0 of
 *   topk_w[r][t][j] * recv[r][t][j][:], fp32 accumulation, rounded once to the row
 *   dtype; exactly 0 for a token with no local pair.  Deterministic.
 * recv: R device pointers, each [T][k][d]; y: R device pointers, each [T][d].
 */
int moe_combine_push(const moe_shape_t* s, const moe_placement_t* p, const void* ye,
                     const int32_t* pull_src, const int32_t* slot_of, const float* topk_w,
                     const int32_t* offsets, void* const* recv, void* const* y, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * moe_forward -- the four calls above in order on one stream (the unfused,
 * multi-kernel path).  xe and ye are [moe_max_pairs][d] staging rows (xe holds E4M3
 * codes and xe_scales their scales for MOE_MXFP8; xe_scales and w_scales are ignored
 * for the other dtypes).
 */
int moe_forward(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                const float* const* logits, const void* const* x, const void* w1, const void* w3,
                const void* w2, const moe_mx_scales_t* w_scales, void* xe, uint8_t* xe_scales, void* ye,
                void* const* recv, void* const* y,
                int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                int32_t* pull_src, int32_t* slot_of, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_forward_fused -- moe_layout, moe_expert_ffn_push and moe_weighted_merge in order on one
 *   stream: for fp32 and bf16 the pull is fused into the gate/up GEMM and the push into the
 *   down GEMM, so neither the dispatched rows (xe) nor the expert outputs (ye) are staged;
 *   for MXFP8, moe_dispatch_pull (which quantises the rows) runs first and only the push is
 *   fused.  recv (local-pair entries) and y are bit-identical to moe_forward's.  Arguments
 *   as moe_forward without ye; xe and xe_scales are only used (and required) for MXFP8.
 *   moe_backward reads xe and ye, which this call does not write: a caller that runs the
 *   backward after it runs moe_forward instead, or moe_forward_persistent and then
 *   moe_backward_ring (which reads the expert outputs from recv and the token rows from the
 *   ring or the source buffers).
 */
int moe_forward_fused(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                      const float* const* logits, const void* const* x, const void* w1, const void* w3,
                      const void* w2, const moe_mx_scales_t* w_scales, void* xe, uint8_t* xe_scales,
                      void* const* recv, void* const* y, int32_t* topk_idx, float* topk_w, int32_t* counts,
                      int32_t* offsets, int32_t* pull_src, int32_t* slot_of, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * moe_forward_persistent -- the whole share with dispatch, expert FFN and combine in one
 * persistent kernel [kucoin §02: one megakernel; the SMs are split into a communication
 * part (dispatch, combine, state) and a compute part (expert FFN) that notify each other
 * through GPU-local counters; tokens reach the experts a minibatch at a time through a
 * fixed-size ring buffer whose slots are reused right after combine, so the combine of one
 * batch overlaps the dispatch of the next; qubstore, ring buffer and megakernel
 * paragraphs: no CPU in the loop, no worst-case buffers].
 * Same inputs and outputs as moe_forward (bf16 or MXFP8), plus:
 *   w_scales: MXFP8 only (else ignored): the weights' block scales, as for moe_forward
 *     (the weights are E4M3 codes, moe_mx_quantize).  [kucoin §02: MXFP8 quantisation fused
 *     into the dispatch, grouped-GEMM and SwiGLU data paths.]  The gather quantises each
 *     token row on its way into the ring, the gate/up GEMM's epilogue quantises h into the
 *     ring, and the down GEMM stores each bf16 output row straight to recv (a per-pair
 *     address table in the workspace); the push then only frees the slot.
 *   ring, ring_bytes: caller-owned device buffer, 256-byte aligned, of at least
 *     256 / minibatch_rows slots of moe_ring_slot_bytes() each.  A slot holds one
 *     minibatch of token rows (overwritten in place by their expert outputs) and their h
 *     rows; in MXFP8 the token rows' codes and scale words, then h's codes and scale words.
 *     Fewer slots mean more back-pressure, never a different result.
 *   ws: at least moe_persistent_workspace_bytes() bytes (no worst-case row staging).
 * Launch sequence on `stream`: the layout kernels, a preparation kernel (clears the control
 * words, builds the per-pipeline task tables), the persistent kernel (one 512-thread
 * workgroup per CU, ordinary launch), a completion check, the weighted merge.
 * Roles: in each pipeline the first comm_cus / pipelines workgroups to start move data --
 * they gather chunks of token rows from the source buffers into free ring slots and push
 * finished output rows to recv chunk by chunk, freeing the slots -- and the others take
 * GEMM tasks in ticket order (gathering claimable chunks themselves while a task waits for
 * its rows), then join the data movement once their pipeline has no task left -- with the
 * outputs stored straight to recv (reverse_ring = 1, or MXFP8) they first take down-tile
 * tasks of other pipelines' last groups while there are any (work stealing across XCDs).
 * Row tiles (256 rows of one expert) are split evenly over the pipelines:
 * eight (one per XCD, every hand-off inside one L2) when each XCD's share of the ring holds
 * two groups, else fewer, with agent-scope hand-offs.  Up to G consecutive row tiles of one
 * expert form a group whose GEMM tasks run weight-panel-major, so concurrent tasks share
 * each weight panel (G = slots per pipeline / (3 * chunks per row tile), or / 2 when three
 * groups do not fit, at most 8).
 * Every device wait is bounded by ex->watchdog_us; on expiry all workgroups exit and
 * moe_read_status() returns MOE_ETIMEOUT.  If a pipeline's work was left undone (no
 * workgroup reached it) moe_read_status() returns MOE_EINCOMPLETE.
 * recv (local-pair entries) and y are bit-identical to moe_forward's for the same inputs
 * (same quantisation and tile arithmetic, same merge order).
 * With ex->trace = 1 the kernel records one moe_trace_event_t per task and per workgroup
 * start / end into the workspace (moe_persistent_trace_info).
 * With ex->reverse_ring = 1 [qubstore, ring buffer paragraph: in the forward the ring is
 * walked in reverse order, so that at the end it holds the activations the gradient
 * computation needs and less is recomputed] each pipeline takes its row tiles from last to
 * first, and the down GEMM writes each output row straight to its recv slot (a per-pair
 * address table in the workspace), so a slot keeps its chunk's token rows and h rows until
 * the chunk S slots later (in the pipeline's order) is gathered into it.  At the end the
 * ring holds each pipeline's first chunks in layout order (all of them when the ring is large
 * enough), and the workspace records which slot holds which chunk, for moe_backward_ring.
 * Results are bit-identical to the layout order.
 * Errors: MOE_EUNSUP for an fp32 dtype, minibatch_rows not in {64, 128, 256}, or a device
 * where one workgroup per CU cannot be resident; MOE_EINVAL for a missing MXFP8 w_scales or
 * when comm_cus leaves no CU for compute; MOE_EALIGN for misaligned scales; MOE_ENOSPC for a
 * ring below one 256-row tile or a small workspace.
 */
int moe_forward_persistent(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                           const float* const* logits, const void* const* x, const void* w1, const void* w3,
                           const void* w2, const moe_mx_scales_t* w_scales, void* ring, size_t ring_bytes,
                           void* const* recv, void* const* y, int32_t* topk_idx, float* topk_w, int32_t* counts,
                           int32_t* offsets, int32_t* pull_src, int32_t* slot_of, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * moe_persistent_dispatch_ffn_combine -- the persistent kernel of moe_forward_persistent alone
 * (with its preparation and completion-check kernels): pull dispatch into the ring, the
 * grouped SwiGLU FFN and the push combine into recv, from the outputs of moe_layout (run
 * before, on the same stream, with the same shape, placement and ws).  recv's local-pair
 * entries are bit-identical to moe_dispatch_pull + moe_expert_ffn + the push of
 * moe_combine_push; the weighted merge (moe_weighted_merge) is not included.  Arguments,
 * errors and status as moe_forward_persistent.
 */
int moe_persistent_dispatch_ffn_combine(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                                        const void* const* x, const void* w1, const void* w3, const void* w2,
                                        const moe_mx_scales_t* w_scales, void* ring, size_t ring_bytes,
                                        const int32_t* pull_src, const int32_t* slot_of, const int32_t* offsets,
                                        void* const* recv, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_forward_persistent_noalloc -- for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_forward_persistent with its workspace and its ring in a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU, kept by every GPU the library runs on until the process
 * ends.  The first MOE_NOALLOC_WORKSPACE_BYTES of the array are the workspace, the rest the
 * ring (as many slots of moe_ring_slot_bytes() as fit, capped by ex->ring_slots).
 * Same inputs and outputs as moe_forward_persistent, minus ring and ws; the caller still
 * passes every input and output buffer.  The call makes no allocation (no hipMalloc, no
 * allocating library routine).
 * status: NULL, or a 4-byte-aligned DEVICE int32 that receives the device status word
 *   (what moe_read_status returns for moe_forward_persistent: 0, MOE_EINVAL, MOE_ETIMEOUT,
 *   MOE_EINCOMPLETE), written on `stream` after the merge.
 * Every call on one GPU shares that GPU's array and leaves its contents behind; each call
 * clears what must start at zero, but calls that overlap on one GPU (no ordering between
 * their streams) race on the array.
 * bf16 only: it takes no weight scales, so MXFP8 shapes return MOE_EUNSUP.
 * Errors: as moe_forward_persistent; MOE_ENOSPC when the shape's workspace
 * (moe_persistent_workspace_bytes) exceeds MOE_NOALLOC_WORKSPACE_BYTES or the ring part
 * holds less than one 256-row tile; MOE_EINVAL for ex->trace != 0; MOE_EHIP if the array's
 * address cannot be looked up.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (128u << 20)
#define MOE_NOALLOC_WORKSPACE_BYTES (8u << 20)
int moe_forward_persistent_noalloc(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                                   const float* const* logits, const void* const* x, const void* w1, const void* w3,
                                   const void* w2, void* const* recv, void* const* y, int32_t* topk_idx,
                                   float* topk_w, int32_t* counts, int32_t* offsets, int32_t* pull_src,
                                   int32_t* slot_of, int32_t* status, void* stream);

/* Bytes of one ring slot of moe_forward_persistent (0 if unsupported). */
size_t moe_ring_slot_bytes(const moe_shape_t* s, const moe_exec_t* ex);

/* Workspace bytes moe_forward_persistent needs (smaller than moe_workspace_bytes); includes
 * a per-pair recv address table (8 bytes per moe_max_pairs) when ex->reverse_ring is 1 or the
 * dtype is MXFP8, and the trace region after it when ex->trace is 1. */
size_t moe_persistent_workspace_bytes(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex);

/* One event of the persistent kernel's trace.  Times are wall-clock ticks of the GPU's
 * constant-rate counter (ticks_per_us from moe_persistent_trace_info). */
typedef struct {
  int64_t t_begin;   /* task start (after its waits) */
  int64_t t_end;     /* task end (its completion signal sent) */
  int32_t t_wait;    /* ticks spent waiting (or, for a mover, idle) before t_begin */
  int32_t index;     /* gather, push: pipeline-local chunk (in the pipeline's order, reversed
                        with reverse_ring); GEMM: row_tile * 256 + column tile (row tile in
                        layout order); start / end: 0 = data movement, 1 = compute */
  int32_t workgroup; /* blockIdx.x */
  int16_t kind;      /* MOE_TRACE_* */
  int16_t pipeline;
} moe_trace_event_t;

#define MOE_TRACE_START 0
#define MOE_TRACE_GATHER 1
#define MOE_TRACE_PUSH 2
#define MOE_TRACE_GATE_UP 3
#define MOE_TRACE_DOWN 4
#define MOE_TRACE_END 5

/* Where the trace of moe_forward_persistent (ex->trace = 1) lies in its workspace: an int32
 * event count at byte `offset`, then up to `capacity` events from byte offset + 256 (events
 * beyond the capacity are dropped; the count still counts them).  Also the wall-clock tick
 * rate of the current device (100 per us if it cannot be queried).  No kernel is launched;
 * MOE_EINVAL for a bad shape, a null pointer or ex->trace != 1. */
int moe_persistent_trace_info(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                              size_t* offset, int32_t* capacity, int32_t* ticks_per_us);

/* Where moe_forward_persistent records, in its workspace, which ring slot still holds which
 * chunk when it returns: `entries` int32 values from byte `offset`.  Entry 4 m + h is 1 + the
 * index of the ring slot (slot i starts at ring + i * moe_ring_slot_bytes()) that holds chunk
 * h (its rows minibatch_rows * h onward) of row tile m (256 rows of one expert, the layout's
 * tiles in expert order), or 0.  Every launch rewrites it: nonzero entries only with
 * ex->reverse_ring = 1 and a clean run.  No kernel is launched; MOE_EINVAL for a bad shape
 * or a null pointer. */
int moe_persistent_resident_info(const moe_shape_t* s, const moe_placement_t* p, size_t* offset, int32_t* entries);

/*
 * Backward of the share (bf16 only; other dtypes return MOE_EUNSUP)
 *   [kucoin §01: training adds a backward pass with two more communication rounds in the
 *   opposite direction; kucoin §02: the backward uses a pull reverse-combine and a push
 *   reverse-dispatch; kucoin §03: the backward is sped up as well].
 * The pages give the two rounds, not the arithmetic; what follows is the derivative of the
 * forward above for the loss L = sum over (r, t) of <dy[r][t], y[r][t]>.
 */

/* Bytes of the backward workspace `bws` for a bf16 or MXFP8 shape (0 otherwise). */
size_t moe_backward_workspace_bytes(const moe_shape_t* s, const moe_placement_t* p);

/*
 * The backward in three stages (moe_backward runs them in order).  Inputs common to all:
 * the forward's outputs (xe and ye as moe_forward left them, [moe_max_pairs][d];
 * topk_idx, topk_w, offsets, pull_src, slot_of from moe_layout), ws = the workspace the
 * forward ran with (read only: row count and row tiles), and bws, the backward workspace
 * (at least moe_backward_workspace_bytes(), 256-byte aligned), which carries the per-row
 * gradients from one stage to the next.  With g the pair's gate and, per row of a local
 * expert, a = x W1^T, b = x W3^T, h = silu(a) * b.  Deterministic.
 * Accuracy against the fp64 oracle: dx per token and every row of dw1, dw3, dw2 within
 * the bf16 row-relative 2e-2; dlogits of a token within 2e-2 of max_j g_j |dy| |o_j|.
 */

/*
 * moe_combine_pull_reverse -- pull reverse-combine [kucoin §02]: row s of pair (r, t, j)
 * pulls dO_s = g_j dy[r][t] (bf16, into bws) by the forward's pull schedule, and the
 * pair's gate gradient dg_s = <dy[r][t], ye[s]> (fp32 accumulation, into bws).
 * dy: R device pointers, each [T][d] bf16 (the incoming gradient of y).
 */
int moe_combine_pull_reverse(const moe_shape_t* s, const moe_placement_t* p, const void* const* dy, const void* ye,
                             const int32_t* pull_src, const int32_t* slot_of, const float* topk_w, const void* ws,
                             size_t ws_bytes, void* bws, size_t bws_bytes, void* stream);

/*
 * moe_expert_ffn_backward -- grouped SwiGLU backward of every local expert from the dO
 * rows in bws [kucoin §03: the backward is sped up as well].  Every operand is read as
 * stored (no transposed copies of weights or rows):
 *   dh = dO W2; da = dh * b * silu'(a); db = dh * silu(a), silu'(a) = sigma(a) (1 + a (1 - sigma(a)));
 *   dX = da W1 + db W3 (fp32 accumulate, bf16 rows, into bws);
 *   dw1[l] = sum_s da_s^T x_s, dw3[l] = sum_s db_s^T x_s ([E_local][F][d] bf16),
 *   dw2[l] = sum_s dO_s^T h_s ([E_local][d][F] bf16), summed over the expert's rows in
 *   ascending order; an expert with no rows gets zeros.
 * w1, w3: [E_local][F][d]; w2: [E_local][d][F] (the forward's bf16 weights).
 */
int moe_expert_ffn_backward(const moe_shape_t* s, const moe_placement_t* p, const void* xe, const int32_t* offsets,
                            const void* w1, const void* w3, const void* w2, const void* ws, size_t ws_bytes, void* dw1,
                            void* dw3, void* dw2, void* bws, size_t bws_bytes, void* stream);

/*
 * moe_dispatch_push_reverse -- push reverse-dispatch [kucoin §02], then the ordered sum and
 * the gate gradient:
 *   recv[r][t][j] = dX_s (R pointers, each [T][k][d] bf16; the forward's recv may be reused);
 *   dx[r][t] = sum over ascending j with a local expert of recv[r][t][j] (R pointers, each
 *     [T][d] bf16; exactly 0 for a token with no local pair);
 *   dlogits[r][t][e_j] = g_j (dg_j - sum_i g_i dg_i) for the k kept experts e_j, with
 *     dg = 0 for a pair whose expert is not local; 0 for every other e (R pointers,
 *     each [T][E] fp32).
 */
int moe_dispatch_push_reverse(const moe_shape_t* s, const moe_placement_t* p, const int32_t* pull_src,
                              const int32_t* slot_of, const int32_t* topk_idx, const float* topk_w, const void* ws,
                              size_t ws_bytes, void* const* recv, void* const* dx, float* const* dlogits, void* bws,
                              size_t bws_bytes, void* stream);

/*
 * moe_backward -- the three calls above in order on one stream, after moe_forward ran with
 * the same arguments: gradients of L with respect to the token rows (dx), the local
 * experts' weights (dw1, dw3, dw2) and the logits (dlogits).  Every stage's arguments are
 * checked before the first launch.  The results are bit-identical to the three calls; the
 * push of dX is fused into its GEMM here (each dX row is stored straight to recv[r][t][j]),
 * so bws's dX staging rows are not written (its first 8 N bytes hold the per-pair recv
 * addresses instead).
 */
int moe_backward(const moe_shape_t* s, const moe_placement_t* p, const void* const* dy, const void* xe,
                 const void* ye, const void* w1, const void* w3, const void* w2, const int32_t* topk_idx, const float* topk_w, const int32_t* offsets, const int32_t* pull_src,
                 const int32_t* slot_of, const void* ws, size_t ws_bytes, void* const* recv, void* const* dx,
                 float* const* dlogits, void* dw1, void* dw3, void* dw2, void* bws, size_t bws_bytes,
                 void* stream);

/*
 * moe_backward_ring -- moe_backward after moe_forward_persistent, reading the forward's
 * activations where that call left them [qubstore, ring buffer paragraph: the forward walks
 * the ring in reverse so that at its end the ring holds the activations the gradients need,
 * and less is recomputed; kucoin §02: pull reverse-combine, push reverse-dispatch].
 *   - The expert outputs o are read from recv, where the forward pushed them (no ye buffer);
 *     recv then receives the dX rows, as in moe_backward.
 *   - The expert-side token rows that the ring still holds (ex->reverse_ring = 1 in the
 *     forward) are read in place by the GEMMs; only the other rows are pulled again from the
 *     source buffers x, into xe at their rows.  ring = NULL pulls every row again.
 *   ex, ring, ring_bytes: exactly as passed to moe_forward_persistent.
 *   pws, pws_bytes: that call's workspace, unchanged since (its layout tables and the record
 *     of which ring slot holds which chunk).
 *   x: R device pointers, [T][d] bf16 (the forward's token rows).
 *   xe: [moe_max_pairs][d] bf16, rows not in the ring (contents on return unspecified).
 *   bws: at least moe_backward_workspace_bytes().
 * Other arguments and results as moe_backward; bit-identical to moe_backward given the same
 * token rows (xe) and expert outputs (ye).  bf16 only (else MOE_EUNSUP).  A ring that is not
 * the forward's, or a workspace changed since, gives wrong results, not an error.
 */
int moe_backward_ring(const moe_shape_t* s, const moe_placement_t* p, const moe_exec_t* ex,
                      const void* const* dy, const void* const* x, const void* ring, size_t ring_bytes,
                      const void* pws, size_t pws_bytes, const void* w1, const void* w3, const void* w2,
                      const int32_t* topk_idx, const float* topk_w, const int32_t* offsets,
                      const int32_t* pull_src, const int32_t* slot_of, void* const* recv, void* const* dx,
                      float* const* dlogits, void* dw1, void* dw3, void* dw2, void* xe, void* bws,
                      size_t bws_bytes, void* stream);

/*
 * MXFP8 backward [kucoin §02: MXFP8 in the expert data path; the pages give neither the
 * backward's quantisation points nor its rule].  Its two data-gradient GEMMs run in MXFP8 with
 * every operand quantised (the moe_mx_quantize rule) in blocks of 32 along that GEMM's K:
 *   dh = dO W2:           dO along d, W2 along d;
 *   dX = da W1 + db W3:   da and db along F, W1 and W3 along F;
 * a = x W1^T and b = x W3^T are recomputed from the forward's MXFP8 operands.  The weight
 * gradients contract over each expert's rows (32-row blocks would straddle experts) and
 * run in bf16 on bf16 dO, da, db, h and the bf16 token rows.
 */

/*
 * moe_backward_prepare_mx -- the weights in the backward's orientation, quantised from the
 * bf16 weights w1, w3 ([E_local][F][d]) and w2 ([E_local][d][F]), once per weight update:
 *   w2t:  [E_local][F][d] codes, row l*F + f = W2[l][:, f] quantised along d;
 *         w2t_scales: [d/128][E_local*F][4] (MXFP8 scale layout);
 *   w13t: [E_local][d][2F] codes, row l*d + n = [W1[l][:, n] | W3[l][:, n]] quantised along F;
 *         w13t_scales: [2F/128][E_local*d][4].
 * dtype must be MOE_MXFP8 (else MOE_EUNSUP).  Bit-exact (the moe_mx_quantize rule).
 */
int moe_backward_prepare_mx(const moe_shape_t* s, const moe_placement_t* p, const void* w1, const void* w3,
                            const void* w2, uint8_t* w2t, uint8_t* w2t_scales, uint8_t* w13t, uint8_t* w13t_scales,
                            void* stream);

/*
 * moe_backward_mx -- moe_backward for MOE_MXFP8, after moe_forward ran with the same
 * arguments.  Inputs as moe_backward, plus: x (R pointers, the bf16 token rows, for the
 * weight gradients), xe / xe_scales and w1q / w3q / w_scales as moe_forward read them, and
 * moe_backward_prepare_mx's outputs.  Outputs as moe_backward (dx, dlogits, and dw1, dw3,
 * dw2 in bf16).  bws: at least moe_backward_workspace_bytes() of this shape.
 * Accuracy against the MXFP8 backward oracle (the same quantisation points in fp64):
 * dx within 1e-1 of the largest row value per token and 2.5e-2 in Frobenius norm (rounding
 * decisions on fp32 / bf16 intermediates flip against fp64); weight gradients per row
 * within the bf16 row-relative 2e-2; dlogits as moe_backward.  As in moe_backward, the dX
 * GEMM stores each row straight to recv[r][t][j] (recv is written, then summed into dx).
 */
int moe_backward_mx(const moe_shape_t* s, const moe_placement_t* p, const void* const* dy, const void* const* x,
                    const uint8_t* xe, const uint8_t* xe_scales, const void* ye, const uint8_t* w1q, const uint8_t* w3q,
                    const moe_mx_scales_t* w_scales, const uint8_t* w2t, const uint8_t* w2t_scales, const uint8_t* w13t,
                    const uint8_t* w13t_scales, const int32_t* topk_idx, const float* topk_w, const int32_t* offsets,
                    const int32_t* pull_src, const int32_t* slot_of, const void* ws, size_t ws_bytes,
                    void* const* recv, void* const* dx, float* const* dlogits, void* dw1, void* dw3, void* dw2,
                    void* bws, size_t bws_bytes, void* stream);

/*
 * Inter-partition signal latency on one GPU -- the one-GPU analogue of the pages'
 * signalling measurement [kucoin §02: after a push the destination has to collect a
 * completion signal from every peer; Cursor's multi-node microbenchmark put that latency
 * near 103 us for push against about 18 us for pull].  Here 128 pairs of workgroups
 * hand a payload back and forth through device memory, `rounds` times each:
 *   the producer waits for the previous round's acknowledgement, writes payload_words
 *   32-bit words, makes them visible and raises a flag; the consumer waits for the flag,
 *   checks every word and acknowledges.
 *   cross_xcd: 0 = partners on the same XCD (workgroups w and w ^ 8; workgroup w runs on
 *     XCD w mod 8), 1 = on different XCDs (w and w ^ 1).
 *   scope: 0 = L2-local hand-off (stores waited for, relaxed flag, the consumer invalidates
 *     its L1 with buffer_inv sc1; not sufficient across XCDs), 1 = agent-scope release/acquire
 *     (writes back / invalidates the XCD's L2; correct anywhere), 2 = as 0 with a
 *     workgroup-scope invalidate (buffer_inv sc0), which leaves the consumer's L1 lines in
 *     place (shown stale with a payload that fits the L1), 3 = as 0 with no invalidate and the
 *     payload read by device-coherent sc1 loads (the persistent kernel's same-XCD form).
 *   scratch, scratch_bytes: caller-owned device memory, 256-byte aligned, at least
 *     moe_signal_probe_bytes(payload_words); cleared by the call.
 * Outputs (host): us_per_round = wall time of the launch / rounds (one round = one flag and
 * one acknowledgement per pair, all pairs concurrently); stale_words = payload words a
 * consumer read before they held the round's value (summed); timeouts = waits that hit the
 * 2 s budget; pairs_same_xcd = pairs whose two workgroups reported the same XCC id.
 * Synchronous: returns after the kernel and the copies of the counters finish.  Errors:
 * MOE_EINVAL (cross_xcd not 0/1, scope outside 0..3, payload_words outside [0, 2^20], rounds outside [1, 100000],
 * null pointer), MOE_EALIGN, MOE_ENOSPC, MOE_EHIP; MOE_ETIMEOUT if any wait expired.
 */
size_t moe_signal_probe_bytes(int32_t payload_words);
int moe_signal_probe(int32_t cross_xcd, int32_t scope, int32_t payload_words, int32_t rounds, void* scratch,
                     size_t scratch_bytes, float* us_per_round, int32_t* stale_words, int32_t* timeouts,
                     int32_t* pairs_same_xcd, void* stream);

/*
 * Hardware ceilings of this GPU -- a measurement utility, not an operation of the layer.  It
 * measures what the expert GEMMs' rooflines are read against: the bf16 and MXFP8 MFMA issue
 * rates [kucoin §02: the expert GEMMs in bf16 and MXFP8] and the bandwidth of the direct
 * global->LDS fills that feed their tiles.
 *   kind 0: v_mfma_f32_32x32x16_bf16, 8 independent accumulators per wave, operands in
 *     registers, one 4-wave workgroup per CU, `reps` iterations of 8 MFMAs per wave.
 *   kind 1: the same with v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, unit scales).
 *   kind 2: one 512-thread workgroup per CU streams its contiguous share of src (src_bytes /
 *     CUs, rounded down to 64 KiB) `reps` times through two 64 KiB LDS stages with
 *     global_load_lds_dwordx4 and one barrier per 64 KiB -- the tiles' fill pattern, missing
 *     the L2.
 *   kind 3: the same, each workgroup re-reading one 64 KiB window of the first 1 MiB of src
 *     (window = workgroup mod 16), 16 * reps times: fills that hit the L2.
 *   reps: [1, 1000000].  src, src_bytes: device memory, 16-byte aligned, read only (kinds 2
 *     and 3; kind 2 needs 64 KiB per CU, kind 3 1 MiB; ignored by kinds 0 and 1).
 *   scratch, scratch_bytes: caller-owned device memory, 256-byte aligned, at least
 *     moe_ceiling_probe_bytes(); each thread writes one 32-bit word: kinds 0 and 1 the first
 *     element of its first accumulator as fp32 (16 * reps, resp. 64 * reps: all operands are
 *     1.0); kinds 2 and 3 the int32 word at its index in the last LDS stage filled (thread t
 *     of workgroup b at index b * 512 + t; its word of src is the word t of the last 64 KiB
 *     round that workgroup read).
 * Outputs (host): work = FLOP (kinds 0, 1) or bytes read (kinds 2, 3) of the timed launch;
 * ms = its duration by HIP events on `stream`.  One untimed launch runs first.  Synchronous.
 * Errors: MOE_EINVAL (kind outside 0..3, reps out of range, null pointer), MOE_EALIGN,
 * MOE_ENOSPC (scratch or src too small), MOE_EHIP.
 */
size_t moe_ceiling_probe_bytes(void);
int moe_ceiling_probe(int32_t kind, int32_t reps, const void* src, size_t src_bytes, void* scratch,
                      size_t scratch_bytes, double* work, float* ms, void* stream);

/* Syncs `stream` and returns the device status word (0, MOE_EINVAL or MOE_ETIMEOUT). */
int moe_read_status(const void* ws, void* stream);

/* Static description of an error code. */
const char* moe_strerror(int code);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
