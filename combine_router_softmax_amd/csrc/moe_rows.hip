// Row-movement kernels of the MoE path, all HBM-bound:
//   scatter      token rows -> expert-contiguous rows (dispatch data move)
//   combine      probability-weighted gather of the k expert rows of a token
//   combine_bwd  its backward: grad of expert rows and grad of the weights
//
// Sources: "Megatron MoE 实现" (dispatch_preprocess permutes the hidden states;
// combine_postprocess unpermutes); DeepSpeed ep_tp_dispatch.py restore_combined
// (weighted rows added into a zeroed output one top-k slot at a time, in
// ascending slot order); the mscclpp high-throughput dispatch/combine commit
// (a direct-gather combine per token; exact dispatched copies).
//
// Design: one workgroup per source token, 16-byte vectors per lane.  The
// scatter reads each token row once and writes it to its k rows (source-major:
// HBM reads = N rows, writes = kept rows).  The combine gathers the token's k
// rows (destination-major: reads = kept rows, writes = N rows) and keeps one
// fp32 accumulator per element, updated with one fused multiply-add per slot in
// slot order j = 0..k-1, then rounds once.  Capacity pad rows are zero-filled
// by extra workgroups placed after the token workgroups.  Slots are handled in
// chunks of KC (compile-time) so the k row indices and weights of a chunk stay
// in scalar registers and the chunk's k loads are in flight together; the
// combine also takes two row segments per thread per round, so 2k loads are in
// flight (measured 3.8 % faster than one segment per round).  Rows
// written, and the expert rows the combines read, are touched once per call and
// use non-temporal (streaming) accesses; the scatter's source rows use plain
// loads, which measured faster for that 1-read / k-write pattern.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kRowThreads = 256;
constexpr int kMaxPadBlocks = 2048;
constexpr int kScatterAhead = 4;  // row segments per thread loaded ahead (a 14 KiB row at 256 threads)
constexpr int kStageIters = (kPlaceMaxExperts + 1 + kRowThreads - 1) / kRowThreads;  // expert table per thread

__device__ __forceinline__ char *row_ptr(void *base, int64_t row, int64_t row_bytes) {
  return static_cast<char *>(base) + row * row_bytes;
}
__device__ __forceinline__ const char *row_ptr(const void *base, int64_t row, int64_t row_bytes) {
  return static_cast<const char *>(base) + row * row_bytes;
}

// Zero-fill the pad rows: rows r < pad_rows (and r < *pad_limit when given: the
// end of the last expert segment) with row_src[r] < 0 -- capacity pads, or the
// pads of alignment-padded segments.
__device__ __forceinline__ void zero_pad_rows(void *dst, int64_t pad_rows, const int32_t *pad_limit,
                                              const int32_t *row_src, int64_t row_bytes, int64_t pad_block,
                                              int64_t pad_blocks) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  const int64_t vpr = row_bytes / 16;
  const int64_t lim = pad_limit && *pad_limit < pad_rows ? *pad_limit : pad_rows;
  for (int64_t r = pad_block; r < lim; r += pad_blocks) {
    if (row_src[r] >= 0) continue;
    char *d = row_ptr(dst, r, row_bytes);
    for (int64_t v = threadIdx.x; v < vpr; v += kRowThreads) st16_stream(d + v * 16, z);
  }
}

template <int KC>
__global__ __launch_bounds__(kRowThreads) void scatter_kernel(const void *__restrict__ x, int64_t n, int k,
                                                              int64_t row_bytes, const int32_t *__restrict__ assign_row,
                                                              void *__restrict__ x_perm, int64_t pad_rows,
                                                              const int32_t *__restrict__ pad_limit,
                                                              const int32_t *__restrict__ row_src, int64_t pad_blocks) {
  const int64_t b = blockIdx.x;
  if (b >= n) {
    zero_pad_rows(x_perm, pad_rows, pad_limit, row_src, row_bytes, b - n, pad_blocks);
    return;
  }
  const int64_t vpr = row_bytes / 16;
  const char *src = row_ptr(x, b, row_bytes);
  for (int j0 = 0; j0 < k; j0 += KC) {
    int32_t rows[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) rows[j] = j0 + j < k ? assign_row[b * k + j0 + j] : -1;
    for (int64_t v = threadIdx.x; v < vpr; v += kRowThreads) {
      const u32x4 val = ld16(src + v * 16);
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (rows[j] >= 0) st16_stream(row_ptr(x_perm, rows[j], row_bytes) + v * 16, val);
    }
  }
}

// The rows no assignment fills, for the scatter that places rows: pad rows
// (capacity or alignment, below the end of the last segment: zero data and
// metadata, one row per block and step) and the unused tail past it (metadata
// only, one row per thread).  Whether a row below the end is kept follows from
// its segment's kept count alone (moe_place.hpp).
__device__ __forceinline__ void place_empty_rows(const PlaceArgs &p, void *dst, int64_t row_bytes, int64_t pb,
                                                 int64_t pad_blocks) {
  __shared__ int32_t off_lds[kPlaceMaxExperts + 1];
  __shared__ int32_t kept_lds[kPlaceMaxExperts];
  for (int x = threadIdx.x; x <= p.e; x += kRowThreads) {
    off_lds[x] = p.off[x];
    if (x < p.e) kept_lds[x] = p.kept[x];
  }
  __syncthreads();
  const int64_t used = used_rows(p, off_lds[p.e]);
  if (p.has_pads) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int64_t vpr = row_bytes / 16;
    for (int64_t r = pb; r < used; r += pad_blocks) {
      const int x = segment_of(off_lds, p.e, p.capacity, r);
      if (r - off_lds[x] < kept_lds[x]) continue;  // block-uniform: a kept row
      char *d = row_ptr(dst, r, row_bytes);
      for (int64_t v = threadIdx.x; v < vpr; v += kRowThreads) st16_stream(d + v * 16, z);
      if (threadIdx.x == 0) write_empty_row(p, r);
    }
  }
  for (int64_t r = used + pb * kRowThreads + threadIdx.x; r < p.rows; r += pad_blocks * kRowThreads)
    write_empty_row(p, r);
}

// Scatter after the layout scan: token block t computes the row of each of its
// slots from the scan's ordinal, the expert's kept count and segment start,
// writes the slot's layout entries (assign_row, drop_mask, and for a kept slot
// row_src, pad_mask, w_perm) and copies the token row to the kept rows.  Blocks
// from n on write the rows no assignment fills.
// Latency: the slot ids and ordinals (scalar loads) and the token row's leading
// segments are requested together; the experts' kept counts and starts follow
// as scalar loads, so the rows are known about when the row data arrives.  The
// layout entries of a chunk of slots are one vector store per field from its
// first lanes.
// The read-only layout inputs are also passed as restrict-qualified pointers,
// which lets the uniform ids, ordinals, kept counts and starts come through
// scalar loads.
template <int KC>
__global__ __launch_bounds__(kRowThreads) void scatter_place_kernel(
    const void *__restrict__ x, int64_t n, int k, int64_t row_bytes, PlaceArgs p, const int32_t *__restrict__ topk_idx,
    const int32_t *__restrict__ ordinal, const int32_t *__restrict__ kept, const int32_t *__restrict__ off,
    const float *__restrict__ topk_w, int32_t *__restrict__ assign_row, uint8_t *__restrict__ drop_mask,
    int32_t *__restrict__ row_src, uint8_t *__restrict__ pad_mask, float *__restrict__ w_perm,
    void *__restrict__ x_perm, int64_t pad_blocks) {
  const int64_t b = blockIdx.x;
  if (b == 0 && threadIdx.x == 0) finish_scan(p.hdr, p.counters);
  if (b >= n) {
    place_empty_rows(p, x_perm, row_bytes, b - n, pad_blocks);
    return;
  }
  __shared__ int32_t off_lds[kPlaceMaxExperts + 1];
  __shared__ int32_t kept_lds[kPlaceMaxExperts];
  const int64_t vpr = row_bytes / 16;
  const char *src = row_ptr(x, b, row_bytes);
  const int lane = lane_id();
  const uint32_t n_rows = (uint32_t)p.rows;  // R < 2^31 (checked on the host)
  const float *w_src = w_perm ? topk_w : reinterpret_cast<const float *>(topk_idx);  // a valid address either way

  // Lane j of every wave holds slot j0 + j.  Its id, ordinal and weight are
  // requested first, then the expert's start and kept count; the layout
  // entries are written by the first wave; the rows are made uniform with
  // readlane.  Every address is clamped, so no branch separates the loads.
  struct Slot {
    int64_t a;
    int32_t id, ord;
    float w;
  };
  auto load_slot = [&](int j0) {
    const int js = j0 + (lane < KC ? lane : 0);
    Slot sl;
    sl.a = b * k + (js < k ? js : k - 1);
    sl.id = topk_idx[sl.a];
    sl.ord = ordinal[sl.a];
    sl.w = w_src[sl.a];
    return sl;
  };
  auto place_slots = [&](int j0, const Slot &sl, int32_t (&rows)[KC]) {
    const int js = j0 + lane;
    const int32_t ex = sl.id < 0 ? 0 : (sl.id >= p.e ? p.e - 1 : sl.id);
    const int32_t start = off_lds[ex];
    const int32_t cap = kept_lds[ex];
    const bool valid = (lane < KC) & (js < k) & (sl.id >= 0) & (sl.id < p.e);
    const uint32_t r = (uint32_t)start + (uint32_t)sl.ord;
    // checked against [0, R) too (see placed_row); an unsigned r >= R covers r < 0
    const bool keep = valid & (sl.ord >= 0) & (sl.ord < cap) & (r < n_rows);
    const int32_t my_row = keep ? (int32_t)r : -1;
    if (threadIdx.x < KC && js < k) {
      assign_row[sl.a] = my_row;
      drop_mask[sl.a] = (valid & !keep) ? 1 : 0;
      if (keep) {
        row_src[r] = (int32_t)sl.a;
        pad_mask[r] = 0;
        if (w_perm) w_perm[r] = sl.w;
      }
    }
#pragma unroll
    for (int j = 0; j < KC; ++j) rows[j] = __builtin_amdgcn_readlane(my_row, j);
  };
  auto copy_from = [&](int64_t v_first, const int32_t (&rows)[KC]) {
    for (int64_t v = v_first; v < vpr; v += kRowThreads) {
      const u32x4 val = ld16(src + v * 16);
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (rows[j] >= 0) st16_stream(row_ptr(x_perm, rows[j], row_bytes) + v * 16, val);
    }
  };

  // first chunk: the experts' starts and kept counts (into LDS), the slots and
  // the row's leading segments are all requested at once: one memory round
  // trip, then an LDS lookup, before the stores
  {
    int32_t st_v[kStageIters], kp_v[kStageIters];
#pragma unroll
    for (int i = 0; i < kStageIters; ++i) {
      const int x_ = threadIdx.x + i * kRowThreads;
      st_v[i] = off[x_ <= p.e ? x_ : p.e];
      kp_v[i] = kept[x_ < p.e ? x_ : p.e - 1];
    }
    const Slot sl = load_slot(0);
    u32x4 ahead[kScatterAhead];
#pragma unroll
    for (int i = 0; i < kScatterAhead; ++i) {
      const int64_t v = threadIdx.x + (int64_t)i * kRowThreads;
      ahead[i] = ld16(src + (v < vpr ? v : vpr - 1) * 16);
    }
#pragma unroll
    for (int i = 0; i < kStageIters; ++i) {
      const int x_ = threadIdx.x + i * kRowThreads;
      if (x_ <= p.e) off_lds[x_] = st_v[i];
      if (x_ < p.e) kept_lds[x_] = kp_v[i];
    }
    __syncthreads();
    int32_t rows[KC];
    place_slots(0, sl, rows);
#pragma unroll
    for (int i = 0; i < kScatterAhead; ++i) {
      const int64_t v = threadIdx.x + (int64_t)i * kRowThreads;
      if (v < vpr) {
#pragma unroll
        for (int j = 0; j < KC; ++j)
          if (rows[j] >= 0) st16_stream(row_ptr(x_perm, rows[j], row_bytes) + v * 16, ahead[i]);
      }
    }
    copy_from(threadIdx.x + (int64_t)kScatterAhead * kRowThreads, rows);
  }
  for (int j0 = KC; j0 < k; j0 += KC) {  // more than KC slots (the LDS stage stays)
    const Slot sl = load_slot(j0);
    int32_t rows[KC];
    place_slots(j0, sl, rows);
    copy_from(threadIdx.x, rows);
  }
}

template <bool BF16, int KC>
__global__ __launch_bounds__(kRowThreads) void combine_kernel(const void *__restrict__ y, const float *__restrict__ topk_w,
                                                              const int32_t *__restrict__ assign_row, int64_t n, int k,
                                                              int64_t row_bytes, void *__restrict__ out) {
  using V = Vec16<BF16>;
  constexpr int EL = V::kElems;
  const int64_t t = blockIdx.x;
  const int64_t vpr = row_bytes / 16;
  char *dst = row_ptr(out, t, row_bytes);
  // two row segments per thread per round: 2*KC loads in flight
  for (int64_t v0 = threadIdx.x; v0 < vpr; v0 += 2 * kRowThreads) {
    const int64_t v1 = v0 + kRowThreads;
    const bool has1 = v1 < vpr;
    float acc0[EL], acc1[EL];
#pragma unroll
    for (int i = 0; i < EL; ++i) acc0[i] = acc1[i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += KC) {
      int32_t rows[KC];
      float wts[KC];
      u32x4 vals0[KC], vals1[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        rows[j] = j0 + j < k ? assign_row[t * k + j0 + j] : -1;
        wts[j] = j0 + j < k ? (topk_w ? topk_w[t * k + j0 + j] : 1.0f) : 0.0f;  // no weights: unit weights
      }
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (rows[j] >= 0) {
          vals0[j] = ld16_stream(row_ptr(y, rows[j], row_bytes) + v0 * 16);
          if (has1) vals1[j] = ld16_stream(row_ptr(y, rows[j], row_bytes) + v1 * 16);
        }
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        if (rows[j] < 0) continue;
        float f[EL];
        V::unpack(vals0[j], f);
#pragma unroll
        for (int i = 0; i < EL; ++i) acc0[i] = __builtin_fmaf(wts[j], f[i], acc0[i]);
        if (has1) {
          V::unpack(vals1[j], f);
#pragma unroll
          for (int i = 0; i < EL; ++i) acc1[i] = __builtin_fmaf(wts[j], f[i], acc1[i]);
        }
      }
    }
    st16_stream(dst + v0 * 16, V::pack(acc0));
    if (has1) st16_stream(dst + v1 * 16, V::pack(acc1));
  }
}

template <bool BF16, int KC>
__global__ __launch_bounds__(kRowThreads) void combine_bwd_kernel(
    const void *__restrict__ grad_out, const void *__restrict__ y, const float *__restrict__ topk_w,
    const int32_t *__restrict__ assign_row, int64_t n, int k, int64_t row_bytes, void *__restrict__ grad_y,
    float *__restrict__ grad_w, int64_t pad_rows, const int32_t *__restrict__ pad_limit,
    const int32_t *__restrict__ row_src, int64_t pad_blocks) {
  using V = Vec16<BF16>;
  constexpr int EL = V::kElems;
  constexpr int kWaves = kRowThreads / kWave;
  __shared__ float part[kWaves][KC];
  const int64_t t = blockIdx.x;
  if (t >= n) {
    zero_pad_rows(grad_y, pad_rows, pad_limit, row_src, row_bytes, t - n, pad_blocks);
    return;
  }
  const int64_t vpr = row_bytes / 16;
  const char *g = row_ptr(grad_out, t, row_bytes);
  const int w = threadIdx.x / kWave;
  for (int j0 = 0; j0 < k; j0 += KC) {
    int32_t rows[KC];
    float wts[KC], dot[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      rows[j] = j0 + j < k ? assign_row[t * k + j0 + j] : -1;
      wts[j] = j0 + j < k ? topk_w[t * k + j0 + j] : 0.0f;
      dot[j] = 0.0f;
    }
    // two row segments per thread per round: 2*(KC+1) loads in flight
    for (int64_t v0 = threadIdx.x; v0 < vpr; v0 += 2 * kRowThreads) {
      const int64_t v1 = v0 + kRowThreads;
      const bool has1 = v1 < vpr;
      const u32x4 g0 = ld16_stream(g + v0 * 16);
      u32x4 g1 = {0u, 0u, 0u, 0u};
      if (has1) g1 = ld16_stream(g + v1 * 16);
      u32x4 y0[KC], y1[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j)
        if (rows[j] >= 0) {
          y0[j] = ld16_stream(row_ptr(y, rows[j], row_bytes) + v0 * 16);
          if (has1) y1[j] = ld16_stream(row_ptr(y, rows[j], row_bytes) + v1 * 16);
        }
      float gf0[EL], gf1[EL];
      V::unpack(g0, gf0);
      V::unpack(g1, gf1);
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        if (rows[j] < 0) continue;
        float yf[EL], o[EL];
        V::unpack(y0[j], yf);
#pragma unroll
        for (int i = 0; i < EL; ++i) {
          dot[j] = __builtin_fmaf(gf0[i], yf[i], dot[j]);
          o[i] = wts[j] * gf0[i];
        }
        st16_stream(row_ptr(grad_y, rows[j], row_bytes) + v0 * 16, V::pack(o));
        if (has1) {
          V::unpack(y1[j], yf);
#pragma unroll
          for (int i = 0; i < EL; ++i) {
            dot[j] = __builtin_fmaf(gf1[i], yf[i], dot[j]);
            o[i] = wts[j] * gf1[i];
          }
          st16_stream(row_ptr(grad_y, rows[j], row_bytes) + v1 * 16, V::pack(o));
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const float s = wave_sum_f32(dot[j]);
      if (lane_id() == 0) part[w][j] = s;
    }
    __syncthreads();
    if (threadIdx.x < KC && j0 + (int)threadIdx.x < k) {
      const int j = threadIdx.x;
      float s = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) s += part[ww][j];
      grad_w[t * k + j0 + j] = assign_row[t * k + j0 + j] >= 0 ? s : 0.0f;
    }
    __syncthreads();
  }
}

inline int slot_chunk(int k) { return k >= 8 ? 8 : (k >= 4 ? 4 : (k >= 2 ? 2 : 1)); }

inline int64_t pad_block_count(int64_t pad_rows) {
  return pad_rows <= 0 ? 0 : (pad_rows < kMaxPadBlocks ? pad_rows : kMaxPadBlocks);
}

}  // namespace

hipError_t launch_scatter(const void *x, int64_t n, int k, int64_t row_bytes, const int32_t *assign_row,
                          void *x_perm, int64_t pad_rows, const int32_t *pad_limit, const int32_t *row_src,
                          hipStream_t stream) {
  const int64_t pb = pad_block_count(pad_rows);
  const int64_t blocks = n + pb;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(kRowThreads);
  switch (slot_chunk(k)) {
    case 1: hipLaunchKernelGGL(scatter_kernel<1>, grid, block, 0, stream, x, n, k, row_bytes, assign_row, x_perm, pad_rows, pad_limit, row_src, pb); break;
    case 2: hipLaunchKernelGGL(scatter_kernel<2>, grid, block, 0, stream, x, n, k, row_bytes, assign_row, x_perm, pad_rows, pad_limit, row_src, pb); break;
    case 4: hipLaunchKernelGGL(scatter_kernel<4>, grid, block, 0, stream, x, n, k, row_bytes, assign_row, x_perm, pad_rows, pad_limit, row_src, pb); break;
    default: hipLaunchKernelGGL(scatter_kernel<8>, grid, block, 0, stream, x, n, k, row_bytes, assign_row, x_perm, pad_rows, pad_limit, row_src, pb); break;
  }
  return hipGetLastError();
}

hipError_t launch_scatter_placing(const void *x, int64_t n, int k, int64_t row_bytes, const PlaceArgs &place,
                                  void *x_perm, hipStream_t stream) {
  // empty-row blocks: one per pad row up to kMaxPadBlocks with pads, else enough
  // for one tail row per thread up to 256 blocks
  int64_t pb = place.has_pads ? pad_block_count(place.rows) : (place.rows + kRowThreads - 1) / kRowThreads;
  if (!place.has_pads && pb > 256) pb = 256;
  if (n + pb == 0) pb = 1;  // at least one block: block 0 resets the scan header
  const int64_t blocks = n + pb;
  const dim3 grid((unsigned)blocks), block(kRowThreads);
#define MOE_SCATTER_PLACE(KC)                                                                                     \
  hipLaunchKernelGGL(scatter_place_kernel<KC>, grid, block, 0, stream, x, n, k, row_bytes, place, place.topk_idx,     \
                     place.ordinal, place.kept, place.off, place.topk_w, place.assign_row, place.drop_mask,           \
                     place.row_src, place.pad_mask, place.w_perm, x_perm, pb)
  switch (slot_chunk(k)) {
    case 1: MOE_SCATTER_PLACE(1); break;
    case 2: MOE_SCATTER_PLACE(2); break;
    case 4: MOE_SCATTER_PLACE(4); break;
    default: MOE_SCATTER_PLACE(8); break;
  }
#undef MOE_SCATTER_PLACE
  return hipGetLastError();
}

template <bool BF16>
static hipError_t launch_combine_t(const void *y, const float *topk_w, const int32_t *assign_row, int64_t n, int k,
                                   int64_t row_bytes, void *out, hipStream_t stream) {
  const dim3 grid((unsigned)n), block(kRowThreads);
  switch (slot_chunk(k)) {
    case 1: hipLaunchKernelGGL((combine_kernel<BF16, 1>), grid, block, 0, stream, y, topk_w, assign_row, n, k, row_bytes, out); break;
    case 2: hipLaunchKernelGGL((combine_kernel<BF16, 2>), grid, block, 0, stream, y, topk_w, assign_row, n, k, row_bytes, out); break;
    case 4: hipLaunchKernelGGL((combine_kernel<BF16, 4>), grid, block, 0, stream, y, topk_w, assign_row, n, k, row_bytes, out); break;
    default: hipLaunchKernelGGL((combine_kernel<BF16, 8>), grid, block, 0, stream, y, topk_w, assign_row, n, k, row_bytes, out); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(bool bf16, const void *y, const float *topk_w, const int32_t *assign_row, int64_t n, int k,
                          int64_t row_bytes, void *out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  return bf16 ? launch_combine_t<true>(y, topk_w, assign_row, n, k, row_bytes, out, stream)
              : launch_combine_t<false>(y, topk_w, assign_row, n, k, row_bytes, out, stream);
}

template <bool BF16>
static hipError_t launch_combine_bwd_t(const void *grad_out, const void *y, const float *topk_w,
                                       const int32_t *assign_row, int64_t n, int k, int64_t row_bytes, void *grad_y,
                                       float *grad_w, int64_t pad_rows, const int32_t *pad_limit,
                                       const int32_t *row_src, hipStream_t stream) {
  const int64_t pb = pad_block_count(pad_rows);
  const dim3 grid((unsigned)(n + pb)), block(kRowThreads);
#define MOE_CBWD(KC)                                                                                         \
  hipLaunchKernelGGL((combine_bwd_kernel<BF16, KC>), grid, block, 0, stream, grad_out, y, topk_w, assign_row, n, \
                     k, row_bytes, grad_y, grad_w, pad_rows, pad_limit, row_src, pb)
  switch (slot_chunk(k)) {
    case 1: MOE_CBWD(1); break;
    case 2: MOE_CBWD(2); break;
    case 4: MOE_CBWD(4); break;
    default: MOE_CBWD(8); break;
  }
#undef MOE_CBWD
  return hipGetLastError();
}

hipError_t launch_combine_bwd(bool bf16, const void *grad_out, const void *y, const float *topk_w,
                              const int32_t *assign_row, int64_t n, int k, int64_t row_bytes, void *grad_y,
                              float *grad_w, int64_t pad_rows, const int32_t *pad_limit, const int32_t *row_src,
                              hipStream_t stream) {
  if (n + pad_block_count(pad_rows) == 0) return hipSuccess;
  return bf16 ? launch_combine_bwd_t<true>(grad_out, y, topk_w, assign_row, n, k, row_bytes, grad_y, grad_w, pad_rows,
                                           pad_limit, row_src, stream)
              : launch_combine_bwd_t<false>(grad_out, y, topk_w, assign_row, n, k, row_bytes, grad_y, grad_w,
                                            pad_rows, pad_limit, row_src, stream);
}

}  // namespace moe
