// Host launchers of the gfx950 kernels (internal; the public surface is moe.h).
// Each launcher enqueues on `stream` and returns the launch status; argument
// checking happens before, in moe_abi.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_place.hpp"

namespace moe {

// ---- route (moe_route.hip)
// logits == nullptr: uniform random logits drawn from `seed` (force-balanced mode)
hipError_t launch_route(const float *logits, uint64_t seed, const float *expert_bias, const uint8_t *token_mask,
                        int64_t n, int e, int k, int32_t *topk_idx, float *topk_w, uint8_t *routing_map,
                        int32_t *tokens_per_expert, hipStream_t stream);

// ---- layout (moe_layout.hip)
constexpr int kLayoutTile = 2048;  // assignments per layout tile
inline int64_t layout_tiles(int64_t assignments) {
  return assignments <= 0 ? 1 : (assignments + kLayoutTile - 1) / kLayoutTile;
}
// Workspace of the layout: a 256-byte header that must be zero before the
// workspace's first use (every call leaves it zero), then the scan's status
// words (and, dropping by weight, the per-expert assignment lists).
size_t layout_workspace_bytes(int64_t assignments, int e, bool drop_by_weight);
// zero the header of a layout workspace (a kernel, so that it can be captured)
hipError_t clear_layout_header(void *workspace, hipStream_t stream);
// the scan alone: ordinal, tokens_per_expert, expert_offsets, counters; rows
// are then placed by launch_scatter_placing (or not at all: the reroute).  The
// next kernel of the call must run finish_scan on the workspace header.
// warm, warm_bytes (both launches): the source rows that the call's scatter
// reads, which the scan launch reads alongside into the memory-side cache
// (nullptr, 0 where no rows follow).
hipError_t launch_layout_scan(const int32_t *topk_idx, int64_t n, int k, int e, int capacity, int row_align,
                              int64_t rows, int32_t *tokens_per_expert, int32_t *expert_offsets, int32_t *ordinal,
                              int32_t *counters, void *workspace, const void *warm, int64_t warm_bytes,
                              hipStream_t stream);
// the whole layout with the rows placed in a launch of their own;
// drop_by_weight (with a capacity): keep each expert's `capacity` largest weights
hipError_t launch_layout(const int32_t *topk_idx, const float *topk_w, int64_t n, int k, int e, int capacity,
                         int row_align, bool drop_by_weight, int64_t rows, int32_t *tokens_per_expert,
                         int32_t *expert_offsets, int32_t *ordinal, int32_t *assign_row, int32_t *row_src,
                         uint8_t *drop_mask, uint8_t *pad_mask, int32_t *counters, float *w_perm, void *workspace,
                         const void *warm, int64_t warm_bytes, hipStream_t stream);

// ---- row movement (moe_rows.hip); `row_bytes` is a multiple of 16.  Pad rows
// (row_src < 0) below pad_rows, and below *pad_limit when pad_limit is given,
// are zero-filled.
hipError_t launch_scatter(const void *x, int64_t n, int k, int64_t row_bytes, const int32_t *assign_row,
                          void *x_perm, int64_t pad_rows, const int32_t *pad_limit, const int32_t *row_src,
                          hipStream_t stream);
// The scatter that also places the rows after launch_layout_scan (the
// position policy): each slot's row from its ordinal, kept count and offset,
// the layout's row maps and masks written on the way, pad rows zeroed.
hipError_t launch_scatter_placing(const void *x, int64_t n, int k, int64_t row_bytes, const PlaceArgs &place,
                                  void *x_perm, hipStream_t stream);
// topk_w may be null: unit weights (the dispatch backward)
hipError_t launch_combine(bool bf16, const void *y, const float *topk_w, const int32_t *assign_row, int64_t n,
                          int k, int64_t row_bytes, void *out, hipStream_t stream);
hipError_t launch_combine_bwd(bool bf16, const void *grad_out, const void *y, const float *topk_w,
                              const int32_t *assign_row, int64_t n, int k, int64_t row_bytes, void *grad_y,
                              float *grad_w, int64_t pad_rows, const int32_t *pad_limit, const int32_t *row_src,
                              hipStream_t stream);

// ---- MXFP8 dispatch (moe_mxfp8.hip): x bf16 [n, h], h % 32 == 0; q [rows, h]
// E4M3 codes, scale [rows, h/32] E8M0 codes; pad rows as launch_scatter.
// assign_row null: row t of x goes to row t (k = 1), the plain quantisation.
hipError_t launch_scatter_mxfp8(const uint16_t *x, int64_t n, int k, int64_t h, const int32_t *assign_row,
                                uint8_t *q, uint8_t *scale, int64_t pad_rows, const int32_t *pad_limit,
                                const int32_t *row_src, hipStream_t stream);

// ---- grouped SwiGLU FFN (moe_ffn.hip, MXFP8 in moe_ffn_mx.hip); bf16 operands as uint16_t bit patterns
// Replica weight slots: experts from e_master on take their weights from (and
// write their weight gradients to) the replica buffers, slot e - e_master.
struct ReplicaBases {
  int e_master;
  const uint16_t *w_gate_up;  // [R, 2I, H]
  const uint16_t *w_down;     // [R, H, I]
  uint16_t *grad_w_gate_up;   // [R, 2I, H] (backward)
  uint16_t *grad_w_down;      // [R, H, I] (backward)
};
size_t ffn_workspace_bytes(int64_t rows, int inter);
// rep: nullable (no replica slots)
hipError_t launch_expert_ffn(const uint16_t *x_perm, int64_t rows, int64_t hidden, int inter, int e,
                             int capacity, const int32_t *tokens_per_expert, const int32_t *expert_offsets,
                             const uint16_t *w_gate_up, const uint16_t *w_down, uint16_t *y, uint16_t *gate_up,
                             const ReplicaBases *rep, void *workspace, hipStream_t stream);
size_t ffn_bwd_workspace_bytes(int64_t rows, int inter, int e);
hipError_t launch_expert_ffn_bwd(const uint16_t *x_perm, const uint16_t *grad_y, int64_t rows, int64_t hidden,
                                 int inter, int e, int capacity, const int32_t *tokens_per_expert,
                                 const int32_t *expert_offsets, const uint16_t *w_gate_up, const uint16_t *w_down,
                                 const uint16_t *gate_up, uint16_t *grad_x_perm, uint16_t *grad_w_gate_up,
                                 uint16_t *grad_w_down, const ReplicaBases *rep, void *workspace,
                                 hipStream_t stream);

// MXFP8 operands (E4M3 codes and E8M0 scales per 32 values along K; H and I
// multiples of 512): y bf16 [rows, H]; the workspace holds the MXFP8 intermediate
size_t ffn_mxfp8_workspace_bytes(int64_t rows, int inter);
hipError_t launch_expert_ffn_mxfp8(const uint8_t *x_q, const uint8_t *x_s, int64_t rows, int64_t hidden, int inter,
                                   int e, int capacity, const int32_t *tokens_per_expert,
                                   const int32_t *expert_offsets, const uint8_t *w_gate_up_q,
                                   const uint8_t *w_gate_up_s, const uint8_t *w_down_q, const uint8_t *w_down_s,
                                   uint16_t *y, void *workspace, hipStream_t stream);

// ---- hot-expert replication (moe_replica.hip)
// placement: replica_of[i] = logical expert of slot i (greedy by load per copy)
hipError_t launch_replica_plan(const int32_t *counts, int e, int r, int32_t *replica_of, hipStream_t stream);
size_t reroute_workspace_bytes(int64_t assignments, int e);
hipError_t launch_reroute(const int32_t *topk_idx, int64_t n, int k, int e, const int32_t *replica_of, int r,
                          int32_t *phys_idx, void *workspace, hipStream_t stream);
// replica[i] = master[replica_of[i]], `bytes` per expert (a multiple of 16);
// slots naming no expert in [0, e) are skipped
hipError_t launch_replica_sync(const void *master, void *replica, const int32_t *replica_of, int r, int e,
                               int64_t bytes, hipStream_t stream);
// grad_master[x] = bf16(fp32 sum of grad_master[x] and its slots' gradients in slot order)
hipError_t launch_replica_grad_reduce(uint16_t *grad_master, const uint16_t *grad_replica, const int32_t *replica_of,
                                      int r, int e, int64_t elems, hipStream_t stream);

}  // namespace moe
