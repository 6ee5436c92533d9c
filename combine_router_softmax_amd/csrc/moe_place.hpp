// Row placement of the dispatch layout, shared by the layout's own placement
// kernel and the scatter that places rows while it copies them.
//
// After the layout scan (moe_layout.hip) every valid assignment has its stable
// per-expert ordinal and every expert its kept count and segment start.  The
// row of assignment a with expert x follows from those alone (DeepSpeed
// ep_tp_dispatch.py: capacity slot = ordinal, dropped iff the slot is past the
// expert's rows):
//   row(a) = offset[x] + ordinal[a]  if ordinal[a] < kept[x]   (kept)
//          = -1                      otherwise                  (dropped)
// and every row that no assignment takes is a pad (inside a segment: a capacity
// or alignment pad, zero data) or part of the unused tail past the last
// segment (metadata only).  Segments never overlap and, without alignment or a
// capacity, follow one another with no gap, so there are pads below
// offset[E] only with a capacity or an alignment.
#pragma once

#include "moe_device.hpp"

namespace moe {

constexpr int kPlaceMaxExperts = 1024;

// State of the single-pass layout scan at the start of its workspace (256 bytes
// reserved): the next tile ticket, the epoch that tags this call's status
// words, and a flag set when a wait gave up.  Zero before the workspace's first
// use; the kernel that follows the scan in the same call (it runs after the
// scan has finished) reports a fault and resets the header with finish_scan.
struct ScanHeader {
  uint32_t ticket;
  uint32_t epoch;
  uint32_t fault;
  uint32_t unused;
};

// One thread of the kernel that follows the scan: a fault becomes
// counters[3] = -1; ticket and fault return to zero and the epoch advances,
// so the status words of this call never look ready to the next one.
__device__ __forceinline__ void finish_scan(ScanHeader *hdr, int32_t *counters) {
  volatile ScanHeader *h = hdr;
  if (h->fault) counters[3] = -1;
  h->fault = 0;
  h->ticket = 0;
  h->epoch = h->epoch + 1;
}

struct PlaceArgs {
  const int32_t *topk_idx;  // [A]
  const float *topk_w;      // [A] (nullable when w_perm is null)
  const int32_t *ordinal;   // [A] from the scan
  const int32_t *kept;      // [E] tokens_per_expert
  const int32_t *off;       // [E+1] expert_offsets
  int e;
  int capacity;             // > 0: segment x is [x*C, (x+1)*C)
  bool has_pads;            // capacity or alignment: pads below off[E]
  int64_t rows;             // R
  int32_t *assign_row;      // [A]
  uint8_t *drop_mask;       // [A]
  int32_t *row_src;         // [R]
  uint8_t *pad_mask;        // [R]
  float *w_perm;            // [R] (nullable)
  ScanHeader *hdr;          // the scan's header, reset by the placing kernel
  int32_t *counters;        // [4]
};

// `workspace`: the layout workspace, whose header the placing kernel resets.
inline PlaceArgs place_args(const int32_t *topk_idx, const float *topk_w, const int32_t *ordinal, const int32_t *kept,
                            const int32_t *off, int e, int capacity, int row_align, int64_t rows, int32_t *assign_row,
                            uint8_t *drop_mask, int32_t *row_src, uint8_t *pad_mask, float *w_perm, void *workspace,
                            int32_t *counters) {
  return PlaceArgs{topk_idx, topk_w,    ordinal,   kept,    off,      e,      capacity,
                   capacity > 0 || row_align > 1,       rows,    assign_row, drop_mask, row_src,
                   pad_mask, w_perm,    static_cast<ScanHeader *>(workspace), counters};
}

// Row of assignment a, -1 if it is not placed (sentinel, invalid id, dropped).
// The row is checked against [0, R) as well: a scan that gave up (a header that
// was not zeroed) leaves counts that cannot be trusted, and no write may leave
// the buffers then.
__device__ __forceinline__ int32_t placed_row(const PlaceArgs &p, int64_t a, bool *dropped) {
  const int32_t x = p.topk_idx[a];
  *dropped = false;
  if (x < 0 || x >= p.e) return -1;
  const int32_t o = p.ordinal[a];
  const int64_t r = (int64_t)p.off[x] + o;
  if (o >= 0 && o < p.kept[x] && r >= 0 && r < p.rows) return (int32_t)r;
  *dropped = true;
  return -1;
}

// End of the last segment, clamped into [0, R].
__device__ __forceinline__ int64_t used_rows(const PlaceArgs &p, int32_t end) {
  return end < 0 ? 0 : (end > p.rows ? p.rows : end);
}

// The metadata of assignment a placed in row r (r = -1: not placed).
__device__ __forceinline__ void write_assignment(const PlaceArgs &p, int64_t a, int32_t r, bool dropped) {
  p.assign_row[a] = r;
  p.drop_mask[a] = dropped ? 1 : 0;
  if (r >= 0) {
    p.row_src[r] = (int32_t)a;
    p.pad_mask[r] = 0;
    if (p.w_perm) p.w_perm[r] = p.topk_w[a];
  }
}

__device__ __forceinline__ void write_empty_row(const PlaceArgs &p, int64_t r) {
  p.row_src[r] = -1;
  p.pad_mask[r] = 1;
  if (p.w_perm) p.w_perm[r] = 0.0f;
}

// Segment holding row r < off[E]: the last expert whose segment starts at or
// before r (off[] in LDS, nondecreasing, off[0] == 0); r / C with a capacity.
__device__ __forceinline__ int segment_of(const int32_t *off_lds, int e, int capacity, int64_t r) {
  if (capacity > 0) return (int)(r / capacity);
  int lo = 0, hi = e - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off_lds[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

}  // namespace moe
