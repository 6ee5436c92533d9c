// C ABI of the MoE path (declared in include/moe.h): host-side validation,
// workspace carving and kernel launches on the caller's stream.  No device
// memory is read on the host and nothing is allocated.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <initializer_list>
#include <mutex>

#include "moe_kernels.hpp"

namespace {

constexpr int kMaxExperts = 1024;
constexpr int64_t kMaxIndex = 0x7FFFFFFFll;  // row and assignment indices are int32
constexpr int kMaxRowAlign = 1024;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int64_t elem_bytes(int32_t dt) { return dt == MOE_DT_F32 ? 4 : 2; }

// Checks every field common to all calls.
moe_status check_shape(const moe_shape *s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->n_tokens < 0 || s->hidden < 1 || s->n_experts < 1 || s->top_k < 1 || s->max_rows < 0) return MOE_ERR_INVALID_ARG;
  if (s->act_dtype != MOE_DT_F32 && s->act_dtype != MOE_DT_BF16) return MOE_ERR_INVALID_ARG;
  if (s->row_align < 0 || s->row_align > kMaxRowAlign || (s->row_align & (s->row_align - 1)) != 0)
    return MOE_ERR_INVALID_ARG;
  if ((s->drop_policy != MOE_DROP_POSITION && s->drop_policy != MOE_DROP_PROBS) || s->reserved != 0)
    return MOE_ERR_INVALID_ARG;
  if (s->n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (s->n_tokens > kMaxIndex / s->top_k) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Capacity drops by weight (else by position).
bool by_weight(const moe_shape *s) { return s->capacity > 0 && s->drop_policy == MOE_DROP_PROBS; }

int64_t rows_of(const moe_shape *s) {
  if (s->capacity > 0) return (int64_t)s->n_experts * s->capacity;
  if (s->max_rows > 0) return s->max_rows;
  // every aligned segment adds at most row_align - 1 pad rows
  return s->n_tokens * s->top_k + (s->row_align > 1 ? (int64_t)s->n_experts * (s->row_align - 1) : 0);
}

// Row geometry and the rows of the permuted buffer.
moe_status check_rows(const moe_shape *s, int64_t *row_bytes, int64_t *rows) {
  const int64_t rb = s->hidden * elem_bytes(s->act_dtype);
  if (rb % 16 != 0) return MOE_ERR_MISALIGNED;
  if (s->capacity > 0) {
    const int64_t ec = (int64_t)s->n_experts * s->capacity;
    if (s->max_rows != 0 && s->max_rows != ec) return MOE_ERR_INVALID_ARG;
    if (ec > kMaxIndex) return MOE_ERR_UNSUPPORTED;
    if (s->row_align > 1 && s->capacity % s->row_align != 0) return MOE_ERR_UNSUPPORTED;  // segments are e*C
  } else if (s->row_align > 1 &&
             s->n_tokens * s->top_k + (int64_t)s->n_experts * (s->row_align - 1) > kMaxIndex) {
    return MOE_ERR_UNSUPPORTED;  // the aligned offsets are int32
  }
  const int64_t r = rows_of(s);
  if (r > kMaxIndex) return MOE_ERR_UNSUPPORTED;
  *row_bytes = rb;
  *rows = r;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// A pointer the call dereferences must be non-null and aligned when its tensor
// is non-empty.
bool need(const void *p, int64_t elems, bool (*aligned)(const void *)) {
  return elems == 0 || p == nullptr || aligned(p);
}

// Checks shared by the forward and backward expert FFN.
moe_status check_ffn_shape(const moe_shape *s, int64_t *rows) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  int64_t row_bytes;
  if ((st = check_rows(s, &row_bytes, rows)) != MOE_OK) return st;
  if (s->act_dtype != MOE_DT_BF16) return MOE_ERR_UNSUPPORTED;
  if (s->inter < 1) return MOE_ERR_INVALID_ARG;
  if (s->inter % 64 != 0 || s->hidden % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (4 * (int64_t)s->inter * s->hidden >= (int64_t)1 << 32) return MOE_ERR_UNSUPPORTED;  // 32-bit weight offsets
  return MOE_OK;
}

}  // namespace

extern "C" {

int64_t moe_layout_rows(const moe_shape *s) {
  if (check_shape(s) != MOE_OK) return -1;
  return rows_of(s);
}

moe_status moe_workspace_size(moe_op op, const moe_shape *s, size_t *bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  switch (op) {
    case MOE_OP_ROUTE:
    case MOE_OP_COMBINE:
    case MOE_OP_COMBINE_BWD:
      *bytes = 0;
      return MOE_OK;
    case MOE_OP_DISPATCH:
      *bytes = moe::layout_workspace_bytes(s->n_tokens * s->top_k, s->n_experts, by_weight(s));
      return MOE_OK;
    case MOE_OP_EXPERT_FFN:
      if (s->inter < 1) return MOE_ERR_INVALID_ARG;
      *bytes = moe::ffn_workspace_bytes(rows_of(s), s->inter);
      return MOE_OK;
    case MOE_OP_EXPERT_FFN_MXFP8:
      if (s->inter < 1) return MOE_ERR_INVALID_ARG;
      *bytes = moe::ffn_mxfp8_workspace_bytes(rows_of(s), s->inter);
      return MOE_OK;
    case MOE_OP_REROUTE:
      *bytes = moe::reroute_workspace_bytes(s->n_tokens * s->top_k, s->n_experts);
      return MOE_OK;
    case MOE_OP_EXPERT_FFN_BWD:
      if (s->inter < 1) return MOE_ERR_INVALID_ARG;
      *bytes = moe::ffn_bwd_workspace_bytes(rows_of(s), s->inter, s->n_experts);
      return MOE_OK;
  }
  return MOE_ERR_INVALID_ARG;
}

moe_status moe_route(const moe_shape *s, const float *logits, const float *expert_bias, const uint8_t *token_mask,
                     int32_t *topk_idx, float *topk_w, uint8_t *routing_map, int32_t *tokens_per_expert,
                     void *stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->top_k > s->n_experts) return MOE_ERR_INVALID_ARG;
  const int64_t n = s->n_tokens;
  if (n > 0 && (!logits || !topk_idx || !topk_w)) return MOE_ERR_INVALID_ARG;
  if (n > 0 && (!aligned4(logits) || !aligned4(topk_idx) || !aligned4(topk_w))) return MOE_ERR_MISALIGNED;
  if (tokens_per_expert && !aligned4(tokens_per_expert)) return MOE_ERR_MISALIGNED;
  if (expert_bias && !aligned4(expert_bias)) return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_route(logits, 0, expert_bias, token_mask, n, s->n_experts, s->top_k, topk_idx, topk_w, routing_map,
                                      tokens_per_expert, as_stream(stream)));
}

moe_status moe_route_random(const moe_shape *s, uint64_t seed, const float *expert_bias, const uint8_t *token_mask,
                            int32_t *topk_idx, float *topk_w, uint8_t *routing_map, int32_t *tokens_per_expert,
                            void *stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->top_k > s->n_experts) return MOE_ERR_INVALID_ARG;
  const int64_t n = s->n_tokens;
  if (n > 0 && (!topk_idx || !topk_w)) return MOE_ERR_INVALID_ARG;
  if (n > 0 && (!aligned4(topk_idx) || !aligned4(topk_w))) return MOE_ERR_MISALIGNED;
  if (tokens_per_expert && !aligned4(tokens_per_expert)) return MOE_ERR_MISALIGNED;
  if (expert_bias && !aligned4(expert_bias)) return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_route(nullptr, seed, expert_bias, token_mask, n, s->n_experts, s->top_k, topk_idx,
                                      topk_w, routing_map, tokens_per_expert, as_stream(stream)));
}

}  // extern "C"

namespace {

// Validation and layout launch shared by the bf16 and MXFP8 dispatch; `outs`
// are the permuted-row outputs (each must be non-null when rows > 0).
moe_status dispatch_layout(const moe_shape *s, int64_t rows, const void *x, const int32_t *topk_idx,
                           const float *topk_w, const moe_layout *layout, std::initializer_list<const void *> outs,
                           float *w_perm, void *workspace, size_t workspace_bytes, hipStream_t hs,
                           bool place_in_scatter, bool needs_x = true) {
  if (!layout) return MOE_ERR_INVALID_ARG;
  const int64_t n = s->n_tokens, a = n * s->top_k;
  if (!layout->tokens_per_expert || !layout->expert_offsets || !layout->counters) return MOE_ERR_INVALID_ARG;
  if ((a > 0 && (!topk_idx || !layout->ordinal || !layout->assign_row || !layout->drop_mask)) ||
      (rows > 0 && (!layout->row_src || !layout->pad_mask)) || (needs_x && n > 0 && !x) ||
      (w_perm && a > 0 && !topk_w))
    return MOE_ERR_INVALID_ARG;
  for (const void *o : outs)
    if (rows > 0 && !o) return MOE_ERR_INVALID_ARG;
  if (!need(x, n, aligned16)) return MOE_ERR_MISALIGNED;
  if (by_weight(s) && a > 0 && !topk_w) return MOE_ERR_INVALID_ARG;  // the policy ranks the weights
  const size_t need_ws = moe::layout_workspace_bytes(a, s->n_experts, by_weight(s));
  if (workspace_bytes < need_ws || !workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return MOE_ERR_WORKSPACE;
  // the scan launch also reads the rows that the scatter after it copies
  const int64_t x_bytes = x ? n * s->hidden * elem_bytes(s->act_dtype) : 0;
  if (place_in_scatter)  // the scan alone; the scatter places the rows
    return hip_status(moe::launch_layout_scan(topk_idx, n, s->top_k, s->n_experts, s->capacity, s->row_align, rows,
                                              layout->tokens_per_expert, layout->expert_offsets, layout->ordinal,
                                              layout->counters, workspace, x, x_bytes, hs));
  return hip_status(moe::launch_layout(topk_idx, topk_w, n, s->top_k, s->n_experts, s->capacity, s->row_align,
                                       by_weight(s), rows, layout->tokens_per_expert, layout->expert_offsets,
                                       layout->ordinal, layout->assign_row, layout->row_src, layout->drop_mask,
                                       layout->pad_mask, layout->counters, w_perm, workspace, x, x_bytes, hs));
}

// Pad rows to zero: capacity pads (every row without an assignment), or the
// pads of aligned segments (those below the end of the last segment).
int64_t pad_rows_of(const moe_shape *s, int64_t rows) { return (s->capacity > 0 || s->row_align > 1) ? rows : 0; }
const int32_t *pad_limit_of(const moe_shape *s, const moe_layout *layout) {
  return s->capacity > 0 ? nullptr : layout->expert_offsets + s->n_experts;
}

}  // namespace

namespace {

// moe_dispatch with the workspace given (the caller's, or the no-allocation
// entry point's static scratch).
moe_status dispatch_impl(const moe_shape *s, const void *x, const int32_t *topk_idx, const float *topk_w,
                         const moe_layout *layout, void *x_perm, float *w_perm, void *workspace,
                         size_t workspace_bytes, void *stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  int64_t row_bytes, rows;
  if ((st = check_rows(s, &row_bytes, &rows)) != MOE_OK) return st;
  if (!need(x_perm, rows, aligned16)) return MOE_ERR_MISALIGNED;
  hipStream_t hs = as_stream(stream);
  // the position policy places rows in the scatter; dropping by weight selects first
  const bool place_in_scatter = !by_weight(s);
  if ((st = dispatch_layout(s, rows, x, topk_idx, topk_w, layout, {x_perm}, w_perm, workspace, workspace_bytes, hs,
                            place_in_scatter)) != MOE_OK)
    return st;
  if (place_in_scatter) {
    const moe::PlaceArgs p = moe::place_args(topk_idx, topk_w, layout->ordinal, layout->tokens_per_expert,
                                             layout->expert_offsets, s->n_experts, s->capacity, s->row_align, rows,
                                             layout->assign_row, layout->drop_mask, layout->row_src, layout->pad_mask,
                                             w_perm, workspace, layout->counters);
    return hip_status(moe::launch_scatter_placing(x, s->n_tokens, s->top_k, row_bytes, p, x_perm, hs));
  }
  return hip_status(moe::launch_scatter(x, s->n_tokens, s->top_k, row_bytes, layout->assign_row, x_perm,
                                        pad_rows_of(s, rows), pad_limit_of(s, layout), layout->row_src, hs));
}

// Scratch of moe_dispatch_noalloc: one array per GPU (each device holds its own
// copy at its own address), kept until the process ends.  Host code never uses
// the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, below.
constexpr size_t kNoallocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once known

// The current device's scratch address; on the first call on a device, look it
// up and zero the layout header at its start (the scan's state, which every
// call leaves zero again), enqueued on `hs` ahead of the call's kernels.
moe_status noalloc_scratch(hipStream_t hs, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    if (moe::clear_layout_header(ptr, hs) != hipSuccess) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_dispatch(const moe_shape *s, const void *x, const int32_t *topk_idx, const float *topk_w,
                        const moe_layout *layout, void *x_perm, float *w_perm, void *workspace,
                        size_t workspace_bytes, void *stream) {
  return dispatch_impl(s, x, topk_idx, topk_w, layout, x_perm, w_perm, workspace, workspace_bytes, stream);
}

moe_status moe_build_layout(const moe_shape *s, const int32_t *topk_idx, const float *topk_w,
                            const moe_layout *layout, float *w_perm, void *workspace, size_t workspace_bytes,
                            void *stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  int64_t row_bytes, rows;
  if ((st = check_rows(s, &row_bytes, &rows)) != MOE_OK) return st;
  return dispatch_layout(s, rows, nullptr, topk_idx, topk_w, layout, {}, w_perm, workspace, workspace_bytes,
                         as_stream(stream), false, false);
}

moe_status moe_dispatch_noalloc(const moe_shape *s, const void *x, const int32_t *topk_idx, const float *topk_w,
                                const moe_layout *layout, void *x_perm, float *w_perm, void *stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (moe::layout_workspace_bytes(s->n_tokens * s->top_k, s->n_experts, by_weight(s)) > kNoallocScratchBytes)
    return MOE_ERR_WORKSPACE;  // more scratch than the static array holds
  void *ws = nullptr;
  if ((st = noalloc_scratch(as_stream(stream), &ws)) != MOE_OK) return st;
  return dispatch_impl(s, x, topk_idx, topk_w, layout, x_perm, w_perm, ws, kNoallocScratchBytes, stream);
}

moe_status moe_dispatch_mxfp8(const moe_shape *s, const void *x, const int32_t *topk_idx, const float *topk_w,
                              const moe_layout *layout, uint8_t *x_perm_q, uint8_t *x_perm_scale, float *w_perm,
                              void *workspace, size_t workspace_bytes, void *stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  int64_t row_bytes, rows;
  if ((st = check_rows(s, &row_bytes, &rows)) != MOE_OK) return st;
  if (s->act_dtype != MOE_DT_BF16 || s->hidden % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (!need(x_perm_q, rows, aligned16)) return MOE_ERR_MISALIGNED;
  if (rows > 0 && x_perm_q && x_perm_q == x_perm_scale) return MOE_ERR_INVALID_ARG;
  hipStream_t hs = as_stream(stream);
  if ((st = dispatch_layout(s, rows, x, topk_idx, topk_w, layout, {x_perm_q, x_perm_scale}, w_perm, workspace,
                            workspace_bytes, hs, false)) != MOE_OK)
    return st;
  return hip_status(moe::launch_scatter_mxfp8(static_cast<const uint16_t *>(x), s->n_tokens, s->top_k, s->hidden,
                                              layout->assign_row, x_perm_q, x_perm_scale, pad_rows_of(s, rows),
                                              pad_limit_of(s, layout), layout->row_src, hs));
}

}  // extern "C"

namespace {

moe_status expert_ffn(const moe_shape *s, const void *x_perm, const moe_layout *layout, const void *w_gate_up,
                      const void *w_down, void *y, void *gate_up, const moe::ReplicaBases *rep, void *workspace,
                      size_t workspace_bytes, void *stream) {
  int64_t rows;
  moe_status st = check_ffn_shape(s, &rows);
  if (st != MOE_OK) return st;
  if (!layout || !layout->tokens_per_expert || !layout->expert_offsets || !w_gate_up || !w_down)
    return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!x_perm || !y)) return MOE_ERR_INVALID_ARG;
  if (!need(x_perm, rows, aligned16) || !need(y, rows, aligned16) || !need(gate_up, rows, aligned16) ||
      !aligned16(w_gate_up) || !aligned16(w_down))
    return MOE_ERR_MISALIGNED;
  if (gate_up && (gate_up == x_perm || gate_up == y || gate_up == w_gate_up || gate_up == w_down))
    return MOE_ERR_INVALID_ARG;
  const size_t need_ws = moe::ffn_workspace_bytes(rows, s->inter);
  if (workspace_bytes < need_ws || (need_ws > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_expert_ffn(static_cast<const uint16_t *>(x_perm), rows, s->hidden, s->inter,
                                           s->n_experts, s->capacity, layout->tokens_per_expert,
                                           layout->expert_offsets, static_cast<const uint16_t *>(w_gate_up),
                                           static_cast<const uint16_t *>(w_down), static_cast<uint16_t *>(y),
                                           static_cast<uint16_t *>(gate_up), rep, workspace, as_stream(stream)));
}

moe_status expert_ffn_bwd(const moe_shape *s, const void *x_perm, const void *grad_y, const void *gate_up,
                          const moe_layout *layout, const void *w_gate_up, const void *w_down, void *grad_x_perm,
                          void *grad_w_gate_up, void *grad_w_down, const moe::ReplicaBases *rep, void *workspace,
                          size_t workspace_bytes, void *stream) {
  int64_t rows;
  moe_status st = check_ffn_shape(s, &rows);
  if (st != MOE_OK) return st;
  if (!layout || !layout->tokens_per_expert || !layout->expert_offsets || !w_gate_up || !w_down || !grad_w_gate_up ||
      !grad_w_down)
    return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!x_perm || !grad_y || !grad_x_perm)) return MOE_ERR_INVALID_ARG;
  if (!need(x_perm, rows, aligned16) || !need(grad_y, rows, aligned16) || !need(grad_x_perm, rows, aligned16) ||
      !need(gate_up, rows, aligned16) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(grad_w_gate_up) ||
      !aligned16(grad_w_down))
    return MOE_ERR_MISALIGNED;
  const void *ins[] = {x_perm, grad_y, gate_up, w_gate_up, w_down};
  for (const void *in : ins)
    if (in && (in == grad_x_perm || in == grad_w_gate_up || in == grad_w_down)) return MOE_ERR_INVALID_ARG;
  if (grad_w_gate_up == grad_w_down || (grad_x_perm && (grad_x_perm == grad_w_gate_up || grad_x_perm == grad_w_down)))
    return MOE_ERR_INVALID_ARG;
  const size_t need_ws = moe::ffn_bwd_workspace_bytes(rows, s->inter, s->n_experts);
  if (workspace_bytes < need_ws || (need_ws > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_expert_ffn_bwd(
      static_cast<const uint16_t *>(x_perm), static_cast<const uint16_t *>(grad_y), rows, s->hidden, s->inter,
      s->n_experts, s->capacity, layout->tokens_per_expert, layout->expert_offsets,
      static_cast<const uint16_t *>(w_gate_up), static_cast<const uint16_t *>(w_down),
      static_cast<const uint16_t *>(gate_up), static_cast<uint16_t *>(grad_x_perm), static_cast<uint16_t *>(grad_w_gate_up),
      static_cast<uint16_t *>(grad_w_down), rep, workspace, as_stream(stream)));
}

// Replica slots of the grouped FFN: the last n_replicas of the shape's experts.
moe_status replica_bases(const moe_shape *s, int32_t n_replicas, const void *w_gate_up_replica,
                         const void *w_down_replica, void *grad_w_gate_up_replica, void *grad_w_down_replica,
                         bool backward, moe::ReplicaBases *out) {
  if (n_replicas < 0 || n_replicas >= s->n_experts) return MOE_ERR_INVALID_ARG;
  if (n_replicas > 0 && (!w_gate_up_replica || !w_down_replica ||
                         (backward && (!grad_w_gate_up_replica || !grad_w_down_replica))))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(w_gate_up_replica) || !aligned16(w_down_replica) || !aligned16(grad_w_gate_up_replica) ||
      !aligned16(grad_w_down_replica))
    return MOE_ERR_MISALIGNED;
  if (n_replicas > 0 && grad_w_gate_up_replica && grad_w_gate_up_replica == grad_w_down_replica)
    return MOE_ERR_INVALID_ARG;
  out->e_master = s->n_experts - n_replicas;
  out->w_gate_up = static_cast<const uint16_t *>(w_gate_up_replica);
  out->w_down = static_cast<const uint16_t *>(w_down_replica);
  out->grad_w_gate_up = static_cast<uint16_t *>(grad_w_gate_up_replica);
  out->grad_w_down = static_cast<uint16_t *>(grad_w_down_replica);
  return MOE_OK;
}

// Shape checks of the replication calls on logical experts: 0 <= R <= 1024.
moe_status check_replicas(const moe_shape *s, int32_t n_replicas, const int32_t *replica_of) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (n_replicas < 0) return MOE_ERR_INVALID_ARG;
  if (n_replicas > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (n_replicas > 0 && !replica_of) return MOE_ERR_INVALID_ARG;
  if (replica_of && !aligned4(replica_of)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_expert_ffn(const moe_shape *s, const void *x_perm, const moe_layout *layout, const void *w_gate_up,
                          const void *w_down, void *y, void *gate_up, void *workspace, size_t workspace_bytes,
                          void *stream) {
  return expert_ffn(s, x_perm, layout, w_gate_up, w_down, y, gate_up, nullptr, workspace, workspace_bytes, stream);
}

moe_status moe_expert_ffn_bwd(const moe_shape *s, const void *x_perm, const void *grad_y, const void *gate_up,
                              const moe_layout *layout, const void *w_gate_up, const void *w_down, void *grad_x_perm,
                              void *grad_w_gate_up, void *grad_w_down, void *workspace, size_t workspace_bytes,
                              void *stream) {
  return expert_ffn_bwd(s, x_perm, grad_y, gate_up, layout, w_gate_up, w_down, grad_x_perm, grad_w_gate_up,
                        grad_w_down, nullptr, workspace, workspace_bytes, stream);
}

moe_status moe_expert_ffn_replicas(const moe_shape *s, int32_t n_replicas, const void *x_perm, const moe_layout *layout,
                                   const void *w_gate_up, const void *w_down, const void *w_gate_up_replica,
                                   const void *w_down_replica, void *y, void *gate_up, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  if (!s) return MOE_ERR_INVALID_ARG;
  moe::ReplicaBases rep;
  moe_status st = replica_bases(s, n_replicas, w_gate_up_replica, w_down_replica, nullptr, nullptr, false, &rep);
  if (st != MOE_OK) return st;
  const void *ins[] = {x_perm, w_gate_up, w_down};
  for (const void *in : ins)
    if (n_replicas > 0 && in && (in == w_gate_up_replica || in == w_down_replica)) return MOE_ERR_INVALID_ARG;
  return expert_ffn(s, x_perm, layout, w_gate_up, w_down, y, gate_up, &rep, workspace, workspace_bytes, stream);
}

moe_status moe_expert_ffn_bwd_replicas(const moe_shape *s, int32_t n_replicas, const void *x_perm, const void *grad_y,
                                       const void *gate_up, const moe_layout *layout, const void *w_gate_up,
                                       const void *w_down, const void *w_gate_up_replica, const void *w_down_replica,
                                       void *grad_x_perm, void *grad_w_gate_up, void *grad_w_down,
                                       void *grad_w_gate_up_replica, void *grad_w_down_replica, void *workspace,
                                       size_t workspace_bytes, void *stream) {
  if (!s) return MOE_ERR_INVALID_ARG;
  moe::ReplicaBases rep;
  moe_status st = replica_bases(s, n_replicas, w_gate_up_replica, w_down_replica, grad_w_gate_up_replica,
                                grad_w_down_replica, true, &rep);
  if (st != MOE_OK) return st;
  if (n_replicas > 0) {
    const void *outs[] = {grad_w_gate_up_replica, grad_w_down_replica};
    const void *others[] = {x_perm, grad_y, gate_up, w_gate_up, w_down, w_gate_up_replica, w_down_replica, grad_x_perm,
                            grad_w_gate_up, grad_w_down};
    for (const void *o : outs)
      for (const void *in : others)
        if (in && in == o) return MOE_ERR_INVALID_ARG;
  }
  return expert_ffn_bwd(s, x_perm, grad_y, gate_up, layout, w_gate_up, w_down, grad_x_perm, grad_w_gate_up,
                        grad_w_down, &rep, workspace, workspace_bytes, stream);
}

moe_status moe_mx_quantize(int64_t rows, int64_t cols, const void *x, uint8_t *q, uint8_t *scale, void *stream) {
  if (rows < 0 || cols < 1) return MOE_ERR_INVALID_ARG;
  if (cols % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows > kMaxIndex) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scale || q == scale) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(q)) return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_scatter_mxfp8(static_cast<const uint16_t *>(x), rows, 1, cols, nullptr, q, scale, 0,
                                              nullptr, nullptr, as_stream(stream)));
}

moe_status moe_expert_ffn_mxfp8(const moe_shape *s, const uint8_t *x_perm_q, const uint8_t *x_perm_scale,
                                const moe_layout *layout, const uint8_t *w_gate_up_q, const uint8_t *w_gate_up_scale,
                                const uint8_t *w_down_q, const uint8_t *w_down_scale, void *y, void *workspace,
                                size_t workspace_bytes, void *stream) {
  int64_t rows;
  moe_status st = check_ffn_shape(s, &rows);
  if (st != MOE_OK) return st;
  if (s->hidden % 512 != 0 || s->inter % 512 != 0) return MOE_ERR_UNSUPPORTED;  // scale groups of 4 K steps
  if (!layout || !layout->tokens_per_expert || !layout->expert_offsets) return MOE_ERR_INVALID_ARG;
  if (!w_gate_up_q || !w_gate_up_scale || !w_down_q || !w_down_scale) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!x_perm_q || !x_perm_scale || !y)) return MOE_ERR_INVALID_ARG;
  // codes 16-byte aligned; scale rows are multiples of 16 bytes (H/32, I/32)
  const void *al[] = {x_perm_q, x_perm_scale, w_gate_up_q, w_gate_up_scale, w_down_q, w_down_scale, y};
  for (const void *ptr : al)
    if (ptr && !aligned16(ptr)) return MOE_ERR_MISALIGNED;
  const void *ins[] = {x_perm_q, x_perm_scale, w_gate_up_q, w_gate_up_scale, w_down_q, w_down_scale};
  for (const void *in : ins)
    if (in && in == y) return MOE_ERR_INVALID_ARG;
  const size_t need_ws = moe::ffn_mxfp8_workspace_bytes(rows, s->inter);
  if (workspace_bytes < need_ws || (need_ws > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_expert_ffn_mxfp8(x_perm_q, x_perm_scale, rows, s->hidden, s->inter, s->n_experts,
                                                 s->capacity, layout->tokens_per_expert, layout->expert_offsets,
                                                 w_gate_up_q, w_gate_up_scale, w_down_q, w_down_scale,
                                                 static_cast<uint16_t *>(y), workspace, as_stream(stream)));
}

moe_status moe_replica_plan(const moe_shape *s, const int32_t *tokens_per_expert, int32_t n_replicas,
                            int32_t *replica_of, void *stream) {
  moe_status st = check_replicas(s, n_replicas, replica_of);
  if (st != MOE_OK) return st;
  if (!tokens_per_expert) return MOE_ERR_INVALID_ARG;
  if (!aligned4(tokens_per_expert)) return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_replica_plan(tokens_per_expert, s->n_experts, n_replicas, replica_of,
                                             as_stream(stream)));
}

moe_status moe_reroute(const moe_shape *s, const int32_t *topk_idx, const int32_t *replica_of, int32_t n_replicas,
                       int32_t *phys_idx, void *workspace, size_t workspace_bytes, void *stream) {
  moe_status st = check_replicas(s, n_replicas, replica_of);
  if (st != MOE_OK) return st;
  if (s->n_experts + n_replicas > kMaxExperts) return MOE_ERR_UNSUPPORTED;  // the physical experts
  const int64_t a = s->n_tokens * s->top_k;
  if (a > 0 && (!topk_idx || !phys_idx)) return MOE_ERR_INVALID_ARG;
  if (a > 0 && (!aligned4(topk_idx) || !aligned4(phys_idx))) return MOE_ERR_MISALIGNED;
  const size_t need_ws = moe::reroute_workspace_bytes(a, s->n_experts);
  if (a > 0 && (workspace_bytes < need_ws || !workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_reroute(topk_idx, s->n_tokens, s->top_k, s->n_experts, replica_of, n_replicas,
                                        phys_idx, workspace, as_stream(stream)));
}

moe_status moe_replica_sync(const moe_shape *s, const int32_t *replica_of, int32_t n_replicas, const void *w_gate_up,
                            const void *w_down, void *w_gate_up_replica, void *w_down_replica, void *stream) {
  moe_status st = check_replicas(s, n_replicas, replica_of);
  if (st != MOE_OK) return st;
  int64_t rows;
  if ((st = check_ffn_shape(s, &rows)) != MOE_OK) return st;
  if (n_replicas == 0) return MOE_OK;
  if (!w_gate_up || !w_down || !w_gate_up_replica || !w_down_replica) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(w_gate_up_replica) || !aligned16(w_down_replica))
    return MOE_ERR_MISALIGNED;
  if (w_gate_up_replica == w_down_replica || w_gate_up_replica == w_gate_up || w_gate_up_replica == w_down ||
      w_down_replica == w_gate_up || w_down_replica == w_down)
    return MOE_ERR_INVALID_ARG;
  const int64_t hi = s->hidden * s->inter;
  hipStream_t hs = as_stream(stream);
  hipError_t e = moe::launch_replica_sync(w_gate_up, w_gate_up_replica, replica_of, n_replicas, s->n_experts,
                                          2 * hi * 2, hs);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_replica_sync(w_down, w_down_replica, replica_of, n_replicas, s->n_experts, hi * 2, hs));
}

moe_status moe_replica_grad_reduce(const moe_shape *s, const int32_t *replica_of, int32_t n_replicas,
                                   const void *grad_w_gate_up_replica, const void *grad_w_down_replica,
                                   void *grad_w_gate_up, void *grad_w_down, void *stream) {
  moe_status st = check_replicas(s, n_replicas, replica_of);
  if (st != MOE_OK) return st;
  int64_t rows;
  if ((st = check_ffn_shape(s, &rows)) != MOE_OK) return st;
  if (n_replicas == 0) return MOE_OK;
  if (!grad_w_gate_up_replica || !grad_w_down_replica || !grad_w_gate_up || !grad_w_down) return MOE_ERR_INVALID_ARG;
  if (!aligned16(grad_w_gate_up_replica) || !aligned16(grad_w_down_replica) || !aligned16(grad_w_gate_up) ||
      !aligned16(grad_w_down))
    return MOE_ERR_MISALIGNED;
  if (grad_w_gate_up == grad_w_down || grad_w_gate_up == grad_w_gate_up_replica ||
      grad_w_gate_up == grad_w_down_replica || grad_w_down == grad_w_gate_up_replica ||
      grad_w_down == grad_w_down_replica)
    return MOE_ERR_INVALID_ARG;
  const int64_t hi = s->hidden * s->inter;
  hipStream_t hs = as_stream(stream);
  hipError_t e = moe::launch_replica_grad_reduce(static_cast<uint16_t *>(grad_w_gate_up),
                                                 static_cast<const uint16_t *>(grad_w_gate_up_replica), replica_of,
                                                 n_replicas, s->n_experts, 2 * hi, hs);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_replica_grad_reduce(static_cast<uint16_t *>(grad_w_down),
                                                    static_cast<const uint16_t *>(grad_w_down_replica), replica_of,
                                                    n_replicas, s->n_experts, hi, hs));
}


moe_status moe_combine(const moe_shape *s, const void *y, const float *topk_w, const moe_layout *layout, void *out,
                       void *stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  int64_t row_bytes, rows;
  if ((st = check_rows(s, &row_bytes, &rows)) != MOE_OK) return st;
  const int64_t n = s->n_tokens;
  if (!layout) return MOE_ERR_INVALID_ARG;
  if (n > 0 && (!topk_w || !layout->assign_row || !out || (rows > 0 && !y))) return MOE_ERR_INVALID_ARG;
  if (!need(y, rows, aligned16) || !need(out, n, aligned16)) return MOE_ERR_MISALIGNED;
  if (n > 0 && y == out) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(s->act_dtype == MOE_DT_BF16, y, topk_w, layout->assign_row, n, s->top_k,
                                        row_bytes, out, as_stream(stream)));
}

moe_status moe_dispatch_bwd(const moe_shape *s, const void *grad_x_perm, const moe_layout *layout, void *grad_x,
                            void *stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  int64_t row_bytes, rows;
  if ((st = check_rows(s, &row_bytes, &rows)) != MOE_OK) return st;
  const int64_t n = s->n_tokens;
  if (!layout) return MOE_ERR_INVALID_ARG;
  if (n > 0 && (!layout->assign_row || !grad_x || (rows > 0 && !grad_x_perm))) return MOE_ERR_INVALID_ARG;
  if (!need(grad_x_perm, rows, aligned16) || !need(grad_x, n, aligned16)) return MOE_ERR_MISALIGNED;
  if (n > 0 && grad_x_perm == grad_x) return MOE_ERR_INVALID_ARG;
  // the combine with unit weights: same kernel, same slot order
  return hip_status(moe::launch_combine(s->act_dtype == MOE_DT_BF16, grad_x_perm, nullptr, layout->assign_row, n,
                                        s->top_k, row_bytes, grad_x, as_stream(stream)));
}

moe_status moe_combine_bwd(const moe_shape *s, const void *grad_out, const void *y, const float *topk_w,
                           const moe_layout *layout, void *grad_y, float *grad_w, void *stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  int64_t row_bytes, rows;
  if ((st = check_rows(s, &row_bytes, &rows)) != MOE_OK) return st;
  const int64_t n = s->n_tokens;
  if (!layout) return MOE_ERR_INVALID_ARG;
  if (n > 0 && (!grad_out || !topk_w || !layout->assign_row || !grad_w || (rows > 0 && (!y || !grad_y))))
    return MOE_ERR_INVALID_ARG;
  if ((s->capacity > 0 || s->row_align > 1) && rows > 0 && (!layout->row_src || !grad_y || !layout->expert_offsets))
    return MOE_ERR_INVALID_ARG;
  if (!need(grad_out, n, aligned16) || !need(y, rows, aligned16) || !need(grad_y, rows, aligned16) ||
      !need(grad_w, n, aligned4))
    return MOE_ERR_MISALIGNED;
  if (rows > 0 && grad_y && (grad_y == y || grad_y == grad_out)) return MOE_ERR_INVALID_ARG;
  const int64_t pad_rows = (s->capacity > 0 || s->row_align > 1) ? rows : 0;
  const int32_t *pad_limit = s->capacity > 0 ? nullptr : layout->expert_offsets + s->n_experts;
  return hip_status(moe::launch_combine_bwd(s->act_dtype == MOE_DT_BF16, grad_out, y, topk_w, layout->assign_row, n,
                                            s->top_k, row_bytes, grad_y, grad_w, pad_rows, pad_limit,
                                            layout->row_src, as_stream(stream)));
}

const char *moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_MISALIGNED: return "misaligned pointer or row size";
    case MOE_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char *moe_version(void) { return "0.2.0"; }

}  // extern "C"
