/*
 * moe.h -- C ABI of the MI355X (gfx950) single-GPU Mixture-of-Experts path:
 *
 *   moe_route       router softmax / top-k / renormalise / multihot map / counts
 *   moe_route_random the same over random logits (force-balanced benchmark mode)
 *   moe_dispatch    per-expert histogram + prefix sum, stable per-expert ordinals,
 *                   capacity drop/pad masks, row scatter into expert-contiguous rows
 *   moe_dispatch_noalloc the same with library-owned scratch (no workspace)
 *   moe_build_layout the dispatch layout alone (no row copy)
 *   moe_dispatch_mxfp8 the same, the permuted rows quantised to MXFP8 (E4M3 + E8M0)
 *   moe_expert_ffn  grouped SwiGLU expert GEMM (bf16 MFMA, fp32 accumulation)
 *   moe_expert_ffn_bwd backward of moe_expert_ffn (grads of rows and weights)
 *   moe_combine     probability-weighted unpermute / combine (fp32 accumulation)
 *   moe_combine_bwd backward of moe_combine (grad of expert rows, grad of weights)
 *   moe_dispatch_bwd backward of the row scatter (grad of the token rows)
 *   moe_mx_quantize / moe_expert_ffn_mxfp8
 *                   MXFP8 quantisation of a matrix; the expert FFN over MXFP8
 *                   rows and weights (scaled fp8 MFMA)
 *   moe_replica_plan / moe_replica_sync / moe_reroute / moe_expert_ffn_replicas /
 *   moe_expert_ffn_bwd_replicas / moe_replica_grad_reduce
 *                   hot-expert replication on one GPU (placement, weight sync,
 *                   logical -> physical reroute, FFN with replica weight slots,
 *                   replica gradient reduce)
 *
 * The steps follow the four stages of Megatron-Core's MoELayer.forward as laid
 * out on the page "Megatron MoE 实现" (router -> (probs, routing_map);
 * dispatch_preprocess / token_dispatch / dispatch_postprocess ->
 * (dispatched_input, tokens_per_expert, permuted_probs); experts;
 * combine_postprocess), restricted to one GPU: the expert-parallel all-to-all
 * between those stages is not part of this library.
 *
 * Conventions for every entry point:
 *  - Pointers to tensors are DEVICE pointers owned by the caller; the library
 *    never allocates or frees memory and keeps no state between calls.  Scratch
 *    space is a caller-provided device workspace of moe_workspace_size() bytes.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never reads device memory on the host, so it never blocks.
 *    Calls with distinct outputs and workspaces may be in flight on different
 *    streams at once.
 *  - Host-side validation runs before anything is enqueued; on error nothing is
 *    enqueued and a negative moe_status is returned.  A failed kernel launch
 *    returns MOE_ERR_HIP.  Device-side data errors (expert ids out of range) are
 *    never used as addresses: they are skipped and counted.
 *  - Tensors are dense row-major.  Activation rows must be 16-byte aligned and
 *    hold a multiple of 16 bytes (hidden * sizeof(dtype) % 16 == 0).
 *  - Logits and weights are fp32; activations are fp32 or bf16 (bf16 stored as
 *    raw 16-bit patterns); moe_expert_ffn is bf16 only.  Every bf16 result is
 *    rounded to nearest, ties to even, from fp32.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, negative or inconsistent size */
  MOE_ERR_MISALIGNED = -2,  /* pointer or row size breaks the 16-byte rule */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than moe_workspace_size */
  MOE_ERR_UNSUPPORTED = -4, /* valid but outside what the kernels implement */
  MOE_ERR_HIP = -5          /* a HIP launch failed */
} moe_status;

typedef enum moe_dtype { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 } moe_dtype;

/* Which assignments an over-full expert keeps when there is a capacity. */
typedef enum moe_drop_policy {
  MOE_DROP_POSITION = 0, /* the first C by assignment order */
  MOE_DROP_PROBS = 1     /* the C with the largest routing weights (Megatron's "probs" drop policy) */
} moe_drop_policy;

typedef enum moe_op {
  MOE_OP_ROUTE = 0,
  MOE_OP_DISPATCH = 1,
  MOE_OP_EXPERT_FFN = 2,
  MOE_OP_COMBINE = 3,
  MOE_OP_COMBINE_BWD = 4,
  MOE_OP_EXPERT_FFN_BWD = 5,
  MOE_OP_REROUTE = 6,
  MOE_OP_EXPERT_FFN_MXFP8 = 7
} moe_op;

/* Shapes and options; read on the host only, never kept. */
typedef struct moe_shape {
  int64_t n_tokens;  /* N >= 0: tokens (rows of logits, x, out, grad_out) */
  int64_t hidden;    /* H >= 1: activation row length */
  int32_t n_experts; /* E in [1, 1024]: experts on this GPU */
  int32_t top_k;     /* k >= 1: slots per token (route: k <= E) */
  int32_t capacity;  /* C: rows per expert; <= 0 means dropless */
  int32_t inter;     /* I: SwiGLU intermediate size (moe_expert_ffn only) */
  int64_t max_rows;  /* R: rows of the permuted buffer; 0 = default (E*C with a
                        capacity, else N*k).  With a capacity R must be E*C or 0. */
  int32_t act_dtype; /* moe_dtype of the activations */
  int32_t row_align; /* A: 0 or 1 = none; else a power of two <= 1024.  Without a
                        capacity, every expert segment is rounded up to a multiple
                        of A rows, so that each starts on an aligned row (the
                        padded routing maps of the MORI pull request, for
                        tile- or FP8-block-aligned expert GEMMs); the rows between
                        an expert's kept rows and the next segment are pad rows.
                        Default R becomes N*k + E*(A-1).  With a capacity, C must
                        be a multiple of A (segments are e*C already). */
  int32_t drop_policy; /* moe_drop_policy, used with a capacity only */
  int32_t reserved;    /* must be 0 */
} moe_shape;

/* The dispatch layout ("handle"): written by moe_dispatch, read by the other
 * calls.  All arrays are device int32/uint8 arrays of the stated lengths
 * (A = N*k assignments, a = t*k + j; R = rows of the permuted buffer). */
typedef struct moe_layout {
  int32_t *tokens_per_expert; /* [E]   rows kept per expert */
  int32_t *expert_offsets;    /* [E+1] first row of each expert segment; E*C
                                 spacing with a capacity, else the exclusive scan
                                 of the counts (rounded up to A when aligned)
                                 clipped to R; [E] = end of the last segment */
  int32_t *ordinal;           /* [A]   stable per-expert ordinal (number of earlier
                                 assignments to the same expert), -1 for -1 /
                                 invalid ids; dropped assignments keep theirs */
  int32_t *assign_row;        /* [A]   row of assignment a, -1 if not placed */
  int32_t *row_src;           /* [R]   assignment placed in the row, -1 if none */
  uint8_t *drop_mask;         /* [A]   1 = valid id but over capacity / R */
  uint8_t *pad_mask;          /* [R]   1 = row holds no assignment (capacity or
                                 alignment pad, or unused dropless tail) */
  int32_t *counters;          /* [4]   kept, dropped, pad rows (capacity or
                                 alignment: rows below expert_offsets[E] holding
                                 nothing), invalid ids */
} moe_layout;

/* Rows R of the permuted buffer for this shape (E*C, max_rows or N*k). */
int64_t moe_layout_rows(const moe_shape *s);

/* Bytes of device workspace `op` needs for shape `s` (0 is a valid answer).
 * Workspace must be 256-byte aligned.  The dispatch and reroute workspaces
 * (MOE_OP_DISPATCH, MOE_OP_REROUTE) hold the state of the single-pass layout
 * scan: a 256-byte header, then status words tagged with the header's call
 * counter.  Zero-fill the whole workspace once when it is allocated, before
 * its first use: a status word that an earlier workspace left in the same
 * memory carries a tag of that workspace's calls, and with only the header
 * cleared it could pass for a word of this call.  Every call leaves the
 * workspace ready for the next (the header zero again, its status words
 * tagged with a count the next call does not use), so it then serves any
 * number of calls in stream order, at any shape it is large enough for.  Two
 * calls in flight at once must not share a workspace.  No other workspace
 * needs initialisation.  A dispatch whose header was not zero does not hang or
 * write outside its arrays: its scan gives up after a bounded wait and reports
 * counters[3] = -1. */
moe_status moe_workspace_size(moe_op op, const moe_shape *s, size_t *bytes);

/* Router: the routing stage of MoELayer.forward ("Megatron MoE 实现",
 * router_and_preprocess: probs, routing_map = router(hidden_states)) with the
 * multihot [N, E] map of the MORI dispatcher's _indices_to_multihot and its
 * sync-free per-expert counting (ROCm/Megatron-LM "Add MORI as a Token
 * Dispatcher", commit log).  Per token t:
 *   topk_idx[t, 0..k-1] = the k experts with the largest logits, ties broken
 *     towards the lower index (-0.0 == +0.0, NaN ranks below every number),
 *     stored in that order;
 *   topk_w[t, j] = softmax(logits[t])[idx_j] / sum_j' softmax(logits[t])[idx_j']
 *     (fp32; equal to the softmax over the k chosen logits);
 *   routing_map[t, e] = 1 if e was chosen else 0 (nullable, uint8 [N, E]);
 *   tokens_per_expert[e] = number of tokens choosing e (nullable, int32 [E]).
 * expert_bias (nullable, fp32 [E]): a selection-only bias: experts are ranked by
 *   the fp32 sum logits[t, e] + expert_bias[e] (same order and tie rules), while
 *   topk_w stays the renormalised softmax of the chosen experts' logits (the
 *   load-balancing expert bias of Megatron's router, which the UltraEP pull
 *   request "Integrate UltraEP Runtime" lists as not yet supported there).
 * token_mask (nullable, uint8 [N]): a nonzero byte marks a padding token, which
 *   takes part in no routing (the pull request's router masks padding tokens out
 *   of routing and dispatch): its slots are -1 with weight 0, its map row is
 *   empty and it is not counted; moe_dispatch then skips it and moe_combine
 *   gives it a zero row.
 * Inputs: logits fp32 [N, E].  Outputs: topk_idx int32 [N, k], topk_w fp32 [N, k].
 * Infinite logits are unsupported (their weights are NaN).  k <= E <= 1024.
 * No workspace. */
moe_status moe_route(const moe_shape *s, const float *logits, const float *expert_bias, const uint8_t *token_mask,
                     int32_t *topk_idx, float *topk_w, uint8_t *routing_map, int32_t *tokens_per_expert,
                     void *stream);

/* Force-balanced router: moe_route with random instead of given logits (the
 * force-balanced router benchmark mode of the UltraEP pull request "Integrate
 * UltraEP Runtime": random-logits routing, so that every expert receives about
 * N*k/E assignments, the reference point of its throughput tables).  The logit
 * of token t and expert x is (w >> 8) * 2^-24, uniform in [0, 1) and exact in
 * fp32, where w is 32-bit word x % 4 of the Philox4x32-10 block (Salmon et al.,
 * "Parallel Random Numbers: As Easy as 1, 2, 3") of counter
 * (x / 4, t mod 2^32, t / 2^32, 0) under key (seed mod 2^32, seed / 2^32).
 * Everything else -- selection, weights, map, counts, expert_bias, token_mask,
 * errors -- is as moe_route. */
moe_status moe_route_random(const moe_shape *s, uint64_t seed, const float *expert_bias, const uint8_t *token_mask,
                            int32_t *topk_idx, float *topk_w, uint8_t *routing_map, int32_t *tokens_per_expert,
                            void *stream);

/* Dispatch: local permutation of token rows into expert-contiguous rows
 * ("Megatron MoE 实现", dispatch_preprocess / dispatch_postprocess ->
 * dispatched_input, tokens_per_expert, permuted_probs), with DeepSpeed's
 * per-assignment payload (ep_tp_dispatch.py RoutedAssignmentPayload:
 * capacity slots, drop and pad masks; assignment_ordinals_by_expert: stable
 * ordinals within each expert segment) and the MORI dispatcher's -1 sentinel
 * for non-local slots.
 * Inputs: x [N, H] activations; topk_idx int32 [N, k] expert ids (-1 = skip;
 *   < -1 or >= E: invalid, skipped, counted in counters[3]); topk_w fp32 [N, k].
 * Outputs: every array of *layout (see moe_layout); x_perm [R, H]: row
 *   assign_row[a] = x[a / k] bit for bit, pad rows (capacity or alignment)
 *   all-zero, unused dropless tail rows not written; w_perm fp32 [R]
 *   (nullable): topk_w[a] in row assign_row[a], 0 in every other row.
 * Stability: within an expert, rows follow assignment order a = t*k + j.
 * With a capacity C, MOE_DROP_POSITION keeps the first C assignments of each
 * expert (by ordinal); MOE_DROP_PROBS keeps the C with the largest topk_w
 * (ties to the earlier assignment, NaN below every number; topk_w required),
 * still placed in assignment order, so assign_row - offset is the rank among
 * the kept, and ordinal stays the position among all of the expert's
 * assignments.  Without a capacity, assignments past row R are dropped.
 * Workspace: moe_workspace_size(MOE_OP_DISPATCH). */
moe_status moe_dispatch(const moe_shape *s, const void *x, const int32_t *topk_idx, const float *topk_w,
                        const moe_layout *layout, void *x_perm, float *w_perm, void *workspace,
                        size_t workspace_bytes, void *stream);

/* The layout of moe_dispatch without the row copy: every array of *layout and
 * w_perm (nullable) exactly as moe_dispatch writes them, from topk_idx and
 * topk_w alone (the per-assignment payload of DeepSpeed's ep_tp_dispatch.py --
 * capacity slots, drop and pad masks, stable ordinals -- computed on its own,
 * for callers that move the rows themselves or only need the counts, offsets
 * and permutation).  s->hidden and s->act_dtype are checked as for
 * moe_dispatch but no activations are read.  Same options, workspace
 * (moe_workspace_size(MOE_OP_DISPATCH)) and errors as moe_dispatch. */
moe_status moe_build_layout(const moe_shape *s, const int32_t *topk_idx, const float *topk_w,
                            const moe_layout *layout, float *w_perm, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Bytes of the static scratch of moe_dispatch_noalloc (per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/* moe_dispatch for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It
 * takes no workspace: its scratch is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES owned by the library, one per GPU it runs on, held
 * until the process ends (found with hipGetSymbolAddress at the first call on
 * a device, which also enqueues the clearing of its header on `stream`; the
 * array is zero when the library is loaded, so its status words need no
 * clearing).  The
 * call allocates nothing: no hipMalloc, no hipFree, no allocating library
 * routine.  A shape whose dispatch workspace (moe_workspace_size with
 * MOE_OP_DISPATCH) exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_WORKSPACE
 * with nothing enqueued (8 MiB holds, for example, 2M assignments over 256
 * experts, or 1M assignments dropped by weight).  Every call on a GPU shares that
 * GPU's array, which keeps the last call's state: calls in stream order are
 * fine, calls that overlap in time on one GPU (several streams or threads)
 * race and must not be made.  Inputs, outputs, results and errors are
 * moe_dispatch's. */
moe_status moe_dispatch_noalloc(const moe_shape *s, const void *x, const int32_t *topk_idx, const float *topk_w,
                                const moe_layout *layout, void *x_perm, float *w_perm, void *stream);

/* MXFP8 dispatch: moe_dispatch with the permuted rows quantised to MXFP8 on the
 * way (the optional FP8 dispatch of the MORI token dispatcher, ROCm/Megatron-LM
 * "Add MORI as a Token Dispatcher": quantised rows plus a per-token scale
 * tensor; MXFP8 as in the ROCm Megatron MXFP8 training recipe).  The format is
 * the OCP "Microscaling (MX) Formats Specification" v1.0, blocks of 32
 * consecutive elements of a row:
 *   x_perm_scale[r, b] = s + 127 (E8M0), s = floor(log2(max_i |x_i|)) - 8
 *     clipped to [-127, 127]; an all-zero block has code 0;
 *   x_perm_q[r, 32b + i] = the FP8 E4M3 (OCP E4M3FN: bias 7, no infinities)
 *     code of x_i / 2^s, rounded to nearest, ties to even, magnitudes above
 *     448 clamped to 448 (the sign of x_i is kept, also for zero);
 * with x_i the elements of block b of token row assign_row^-1(r).  Every other
 * field, layout output, w_perm, stability and drop rule is as moe_dispatch.
 * Pad rows are all-zero bytes in both outputs (a zero row quantised); rows of
 * an unused dropless tail are not written.
 * Shapes: x bf16 [N, H] (act_dtype must be MOE_DT_BF16 and H % 32 == 0, else
 * MOE_ERR_UNSUPPORTED), 16-byte aligned; x_perm_q uint8 [R, H], 16-byte
 * aligned; x_perm_scale uint8 [R, H/32], any alignment.  Inputs must be finite
 * (a block holding an infinity or NaN gets unspecified codes).
 * Workspace: moe_workspace_size(MOE_OP_DISPATCH). */
moe_status moe_dispatch_mxfp8(const moe_shape *s, const void *x, const int32_t *topk_idx, const float *topk_w,
                              const moe_layout *layout, uint8_t *x_perm_q, uint8_t *x_perm_scale, float *w_perm,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Grouped SwiGLU expert FFN over the expert segments of a dispatch layout
 * ("Megatron MoE 实现", experts(dispatched_input, tokens_per_expert, ...), one
 * GEMM group per expert as in the grouped-GEMM paths of the MORI and UltraEP
 * pull requests, fed by device-resident counts with no host synchronisation).
 * For every row r of expert e's segment [offset_e, offset_e + kept_e):
 *   a[r, i] = bf16( silu(x_perm[r] . w_gate_up[e, i]) * (x_perm[r] . w_gate_up[e, I + i]) )
 *   y[r, c] = bf16( a[r] . w_down[e, c] )
 * bf16 operands, fp32 accumulation, no bias.  Rows outside the segments of y are
 * not written.  Shapes: x_perm bf16 [R, H]; w_gate_up bf16 [E, 2I, H] (gate rows
 * first); w_down bf16 [E, H, I]; y bf16 [R, H].  H and I must be multiples of 64
 * and 4*I*H < 2^32 (one expert's weights are addressed with 32-bit offsets).
 * gate_up (nullable) bf16 [R, 2I]: when given, the pre-activations are stored
 * there for moe_expert_ffn_bwd, gate_up[r, i] = bf16(x_perm[r] . w_gate_up[e, i])
 * for i < 2I (gate columns, then up columns), rows of the segments only.
 * Workspace: moe_workspace_size(MOE_OP_EXPERT_FFN) (holds a [R, I] bf16). */
moe_status moe_expert_ffn(const moe_shape *s, const void *x_perm, const moe_layout *layout,
                          const void *w_gate_up, const void *w_down, void *y, void *gate_up, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Expert FFN backward: the vector-Jacobian product of moe_expert_ffn (the
 * experts' backward of MoELayer on "Megatron MoE 实现", with the grouped-GEMM
 * weight gradients per expert of the MORI and UltraEP pull requests).  Per
 * expert e and the rows of its segment, with G = x_perm Wg^T, U = x_perm Wu^T
 * (Wg, Wu: gate and up halves of w_gate_up[e]), s = sigmoid(G), A = G s U and
 * the incoming grad_y (dY):
 *   dA = dY w_down[e];  dG = dA U s (1 + G (1 - s));  dU = dA G s
 *   grad_x_perm = dG Wg + dU Wu
 *   grad_w_down[e] = dY^T A;  grad_w_gate_up[e] = [dG^T x_perm ; dU^T x_perm]
 * bf16 operands, fp32 accumulation; G, U, dA, dG, dU and A are held in bf16
 * between the GEMMs.  gate_up (nullable): the pre-activations [G | U] that
 * moe_expert_ffn stored; when null they are recomputed (the same values, so
 * both ways give the same bits).  An expert with no rows gets zero weight
 * gradients; rows outside the segments of grad_x_perm are not written.
 * Shapes as moe_expert_ffn: x_perm, grad_y, grad_x_perm bf16 [R, H]; gate_up [R, 2I];
 * w_gate_up, grad_w_gate_up bf16 [E, 2I, H]; w_down, grad_w_down bf16 [E, H, I];
 * outputs must not alias inputs or each other.  Same shape limits as
 * moe_expert_ffn.  Deterministic: no atomics, fixed reduction order.
 * Workspace: moe_workspace_size(MOE_OP_EXPERT_FFN_BWD) (the [R, 3I] bf16
 * intermediates). */
moe_status moe_expert_ffn_bwd(const moe_shape *s, const void *x_perm, const void *grad_y, const void *gate_up,
                              const moe_layout *layout, const void *w_gate_up, const void *w_down, void *grad_x_perm,
                              void *grad_w_gate_up, void *grad_w_down, void *workspace, size_t workspace_bytes,
                              void *stream);

/* MXFP8 quantisation of a bf16 matrix along its rows (the format of
 * moe_dispatch_mxfp8): x bf16 [rows, cols] (16-byte aligned, cols % 32 == 0)
 * -> q uint8 [rows, cols] E4M3 codes (16-byte aligned), scale uint8
 * [rows, cols/32] E8M0 codes.  The expert weights of moe_expert_ffn_mxfp8 are
 * quantised with it along K: w_gate_up [E*2I, H] and w_down [E*H, I]. */
moe_status moe_mx_quantize(int64_t rows, int64_t cols, const void *x, uint8_t *q, uint8_t *scale, void *stream);

/* Grouped SwiGLU expert FFN over MXFP8 operands (the grouped expert GEMM with
 * FP8 grouped experts, which the UltraEP pull request lists as a follow-up, fed
 * by the MXFP8 dispatch; MXFP8 as in the ROCm Megatron MXFP8 recipe).  For every
 * row r of expert e's segment, every operand value being its E4M3 code times
 * its block's E8M0 scale:
 *   a[r, i] = bf16( silu(x[r] . w_gate_up[e, i]) * (x[r] . w_gate_up[e, I + i]) )
 *   a'      = MXFP8 of the row a[r] (blocks of 32 along I, as moe_mx_quantize)
 *   y[r, c] = bf16( a'[r] . w_down[e, c] )
 * with fp32 accumulation on the CDNA4 scaled MFMA (v_mfma_scale_f32_32x32x64_
 * f8f6f4).  Shapes: x_perm_q [R, H] + x_perm_scale [R, H/32] (from
 * moe_dispatch_mxfp8); w_gate_up_q [E, 2I, H] + w_gate_up_scale [E, 2I, H/32];
 * w_down_q [E, H, I] + w_down_scale [E, H, I/32]; y bf16 [R, H].  H and I must
 * be multiples of 512 (MOE_ERR_UNSUPPORTED otherwise); every array 16-byte
 * aligned.  Rows outside the segments of y are not written.  Forward only.
 * Workspace: moe_workspace_size(MOE_OP_EXPERT_FFN_MXFP8) (the MXFP8
 * intermediate). */
moe_status moe_expert_ffn_mxfp8(const moe_shape *s, const uint8_t *x_perm_q, const uint8_t *x_perm_scale,
                                const moe_layout *layout, const uint8_t *w_gate_up_q, const uint8_t *w_gate_up_scale,
                                const uint8_t *w_down_q, const uint8_t *w_down_scale, void *y, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Hot-expert replication, the part of one GPU (InternLM/xtuner pull request
 * "Integrate UltraEP Runtime": replicas of hot experts created from the current
 * load, part of their tokens rerouted to replica slots, master/replica weight
 * sync, one grouped GEMM over master and replica experts with the weights at
 * two storage bases, replica weight gradients in a replica buffer reduced into
 * the masters').  The router and its outputs keep logical expert ids; the
 * dispatch, FFN and combine run on physical ids: physical expert p < E is the
 * master of logical expert p, p = E + i is replica slot i, a copy of logical
 * expert replica_of[i].  Sequence: moe_route -> moe_replica_plan ->
 * moe_replica_sync -> moe_reroute -> moe_dispatch (E + R experts) ->
 * moe_expert_ffn_replicas -> moe_combine; backward moe_combine_bwd ->
 * moe_expert_ffn_bwd_replicas -> moe_replica_grad_reduce -> moe_dispatch_bwd.
 * Replica slot contents are device data: a slot naming no expert in [0, E) is
 * never used as an address (the sync and the reduce skip it; the reroute sends
 * nothing to it). */

/* Placement: replica_of[i] (int32 [n_replicas]) = the logical expert that slot
 * i copies.  Slots are filled in order, each going to the expert with the
 * largest load per copy tokens_per_expert[e] / (1 + slots given to e so far),
 * compared exactly, ties to the lower id.  s->n_experts = E (logical);
 * tokens_per_expert int32 [E] (moe_route's counts); 0 <= n_replicas <= 1024.
 * One wavefront; no workspace. */
moe_status moe_replica_plan(const moe_shape *s, const int32_t *tokens_per_expert, int32_t n_replicas,
                            int32_t *replica_of, void *stream);

/* Reroute: phys_idx [N, k] = the physical expert of every routed slot.  For a
 * logical expert e with c assignments (valid slots, in assignment order
 * a = t*k + j, ordinal o = its position among them) and m = 1 + (its number of
 * slots) copies, the assignment with ordinal o goes to run floor(o * m / c):
 * run 0 stays on the master e, run j >= 1 goes to e's j-th slot (slots in
 * increasing index), so every copy receives floor(c/m) or ceil(c/m) of them
 * in assignment order.  -1 stays -1; an id outside [0, E) becomes -2 (invalid
 * for the physical dispatch as well).  s->n_experts = E (logical), E +
 * n_replicas <= 1024; topk_idx and phys_idx int32 [N, k] (may be the same
 * array).  Workspace: moe_workspace_size(MOE_OP_REROUTE) (a dropless layout of
 * the logical ids, for the ordinals and counts). */
moe_status moe_reroute(const moe_shape *s, const int32_t *topk_idx, const int32_t *replica_of, int32_t n_replicas,
                       int32_t *phys_idx, void *workspace, size_t workspace_bytes, void *stream);

/* Replica weight sync: w_gate_up_replica[i] = w_gate_up[replica_of[i]] and
 * w_down_replica[i] = w_down[replica_of[i]] (bit copies).  s->n_experts = E
 * (logical), hidden, inter as moe_expert_ffn; replica buffers bf16
 * [R, 2I, H] and [R, H, I], 16-byte aligned, distinct from the masters. */
moe_status moe_replica_sync(const moe_shape *s, const int32_t *replica_of, int32_t n_replicas, const void *w_gate_up,
                            const void *w_down, void *w_gate_up_replica, void *w_down_replica, void *stream);

/* Replica gradient reduce: for every logical expert x with slots,
 *   grad_w_gate_up[x] = bf16(grad_w_gate_up[x] + sum over x's slots i, in slot
 *                       order, of grad_w_gate_up_replica[i])   (fp32 sum)
 * and the same for grad_w_down; experts without slots are untouched.  Shapes
 * as moe_replica_sync. */
moe_status moe_replica_grad_reduce(const moe_shape *s, const int32_t *replica_of, int32_t n_replicas,
                                   const void *grad_w_gate_up_replica, const void *grad_w_down_replica,
                                   void *grad_w_gate_up, void *grad_w_down, void *stream);

/* moe_expert_ffn over physical experts with replica slots: s->n_experts = P,
 * the layout's experts (E masters then n_replicas slots, 0 <= n_replicas < P);
 * physical expert p < P - n_replicas takes w_gate_up[p], w_down[p]; slot
 * p - (P - n_replicas) takes w_gate_up_replica[.], w_down_replica[.] (bf16
 * [R, 2I, H], [R, H, I]), in the same grouped GEMM launches.  Everything else
 * as moe_expert_ffn, whose workspace size it takes. */
moe_status moe_expert_ffn_replicas(const moe_shape *s, int32_t n_replicas, const void *x_perm, const moe_layout *layout,
                                   const void *w_gate_up, const void *w_down, const void *w_gate_up_replica,
                                   const void *w_down_replica, void *y, void *gate_up, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* moe_expert_ffn_bwd over physical experts with replica slots (as
 * moe_expert_ffn_replicas): the weight gradients of the slots go to
 * grad_w_gate_up_replica / grad_w_down_replica ([R, 2I, H], [R, H, I]), those
 * of the masters to grad_w_gate_up / grad_w_down ([P - R, ...]);
 * moe_replica_grad_reduce then adds the former into the latter. */
moe_status moe_expert_ffn_bwd_replicas(const moe_shape *s, int32_t n_replicas, const void *x_perm, const void *grad_y,
                                       const void *gate_up, const moe_layout *layout, const void *w_gate_up,
                                       const void *w_down, const void *w_gate_up_replica, const void *w_down_replica,
                                       void *grad_x_perm, void *grad_w_gate_up, void *grad_w_down,
                                       void *grad_w_gate_up_replica, void *grad_w_down_replica, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Combine: probability-weighted unpermute (DeepSpeed ep_tp_dispatch.py
 * restore_combined: weighted expert rows added into a zeroed [N, H] output by
 * token index, one top-k slot at a time in ascending slot order; "Megatron MoE
 * 实现", combine_postprocess).
 *   out[t, :] = sum over j = 0..k-1 with assign_row[t*k+j] >= 0, in that order,
 *               of topk_w[t, j] * y[assign_row[t*k+j], :]
 * accumulated in fp32 with one fused multiply-add per term and rounded once to
 * the activation type; a token with no kept slot gets a zero row.  Weights are
 * indexed like the assignments (receiver-side, as the MORI combine requires).
 * y [R, H] and out [N, H] have the activation type; out must not alias y.
 * For an identity expert pass x_perm as y.  No workspace. */
moe_status moe_combine(const moe_shape *s, const void *y, const float *topk_w, const moe_layout *layout,
                       void *out, void *stream);

/* Dispatch backward: the vector-Jacobian product of the row scatter of
 * moe_dispatch (the unpermute backward of the MORI pull request
 * ROCm/Megatron-LM "Add MORI as a Token Dispatcher"): for every token t,
 *   grad_x[t, :] = sum over kept slots j, in slot order, of
 *                  grad_x_perm[assign_row[t*k + j], :]
 * with an fp32 accumulator and one rounding to the activation type; a token with
 * no kept slot gets a zero row.  grad_x_perm: [max_rows, hidden] rows as laid
 * out by moe_dispatch; grad_x: [n_tokens, hidden]; both in act_dtype, 16-byte
 * aligned, grad_x must not alias grad_x_perm.  No workspace.  Errors as
 * moe_combine. */
moe_status moe_dispatch_bwd(const moe_shape *s, const void *grad_x_perm, const moe_layout *layout, void *grad_x,
                            void *stream);

/* Combine backward: the vector-Jacobian product of moe_combine (the MORI pull
 * request's combine backward, with receiver-side weights and indices).
 * For every kept assignment a = (t, j) in row r = assign_row[a]:
 *   grad_y[r, :] = topk_w[t, j] * grad_out[t, :]     (rounded to the activation type)
 *   grad_w[t, j] = sum_h grad_out[t, h] * y[r, h]    (fp32 accumulation)
 * grad_w = 0 for dropped, -1 and invalid slots; pad rows of grad_y (capacity or
 * alignment) are zero; unused dropless tail rows are not written.  grad_y must not alias y or
 * grad_out.  No workspace. */
moe_status moe_combine_bwd(const moe_shape *s, const void *grad_out, const void *y, const float *topk_w,
                           const moe_layout *layout, void *grad_y, float *grad_w, void *stream);

/* Static description of a status code. */
const char *moe_status_string(moe_status st);

/* Library version, "major.minor.patch". */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
