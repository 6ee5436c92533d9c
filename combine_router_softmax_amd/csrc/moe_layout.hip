// Dispatch layout kernels: per-expert histogram, prefix sums, stable
// per-expert ordinals, capacity drop / pad masks and the row maps.
//
// What is computed (DeepSpeed ep_tp_dispatch.py: RoutedAssignmentPayload with
// capacity_slots / drop_mask / pad_mask and assignment_ordinals_by_expert, the
// ordinal of an assignment inside its expert segment of the stably
// expert-sorted list; the MORI dispatcher's -1 sentinels and sync-free
// tokens_per_expert, ROCm/Megatron-LM "Add MORI as a Token Dispatcher"):
//   ordinal[a]    = #{a' < a : id[a'] = id[a]}          (stable counting sort)
//   expert offset = e*C with a capacity, else the exclusive scan of the counts
//                   (each rounded up to a multiple of the row alignment A, so
//                   that every segment starts on an aligned row: the padded
//                   routing maps of the MORI pull request) clipped to the row
//                   budget R
//   assign_row[a] = offset[id[a]] + ordinal[a] if kept, else -1
//
// How (two launches, no host synchronisation, no atomics on the ordering
// path, so the result does not depend on scheduling):
//   1. layout_count: one workgroup per tile of 512 assignments builds an LDS
//      histogram of the tile's ids -> tile_counts[tile][e] (a small matrix).
//   2. layout_place: every workgroup reads the whole tile_counts matrix once (a
//      single round of independent loads) and scans it in LDS: per expert, the
//      sum over earlier tiles (this tile's base) and over all tiles (the
//      expert's count); a block scan over experts gives the segment offsets.
//      Then each wave walks its 64-assignment chunks of the tile in order;
//      lanes holding the same expert find each other with one ballot per bit of
//      the expert id (a wave64 "match"), rank = popcount(peers below the lane);
//      the per-wave running count per expert lives in LDS and starts at the
//      tile's base plus the counts of the earlier waves of the tile.  The same
//      launch marks every row that receives no assignment (pad or tail), and
//      workgroup 0 writes the counts, offsets and counters.
// With a capacity and the drop-by-weight policy, layout_place lists every
// assignment by expert instead of placing it, and capacity_select_kernel keeps
// each expert's largest weights (see there).
// Re-scanning the count matrix in every workgroup replaces a separate scan
// launch: the matrix is tiles x E ints (64 x 256 for 4096 tokens, top-8, 256
// experts), and a dependent kernel-to-kernel round trip costs more than
// re-reading it.  Tiles of 512 assignments (one 64-assignment chunk per wave)
// give 64 placing workgroups at that shape; 2048-assignment tiles (16
// workgroups, four chunks per wave) measured 3 us slower.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kLayoutThreads = 512;
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kChunksPerWave = kLayoutTile / kLayoutThreads;  // 64-assignment chunks per wave
static_assert(kLayoutTile % kLayoutThreads == 0, "tile must be a multiple of the block");
constexpr int kMaxExperts = 1024;

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

__device__ __forceinline__ bool valid_id(int32_t x, int e) { return x >= 0 && x < e; }

__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t o = __shfl_up(v, off, kWave);
    if (l >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ int32_t wave_sum_i32(int32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Exclusive scan of in[0..n) (n <= 1024) into out[]; every thread of the block calls it.
__device__ void block_exclusive_scan(const int32_t *in, int32_t *out, int n) {
  __shared__ int32_t wave_tot[kLayoutWaves];
  constexpr int kPer = kMaxExperts / kLayoutThreads;
  const int t = threadIdx.x;
  int32_t v[kPer];
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int x = t * kPer + i;
    v[i] = x < n ? in[x] : 0;
    s += v[i];
  }
  const int32_t incl = wave_incl_scan(s);
  if (lane_id() == kWave - 1) wave_tot[t / kWave] = incl;
  __syncthreads();
  int32_t run = incl - s;
  for (int w = 0; w < t / kWave; ++w) run += wave_tot[w];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int x = t * kPer + i;
    if (x < n) out[x] = run;
    run += v[i];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kLayoutThreads) void layout_count(const int32_t *__restrict__ topk_idx, int64_t a_total,
                                                               int e, int32_t *__restrict__ tile_counts,
                                                               int32_t *__restrict__ tile_invalid) {
  extern __shared__ int32_t cnt[];  // [e + 1], cnt[e] = invalid ids
  for (int x = threadIdx.x; x <= e; x += kLayoutThreads) cnt[x] = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * kLayoutTile;
  int32_t ids[kChunksPerWave];
#pragma unroll
  for (int i = 0; i < kChunksPerWave; ++i) {
    const int64_t a = a0 + threadIdx.x + i * kLayoutThreads;
    ids[i] = a < a_total ? topk_idx[a] : -1;
  }
#pragma unroll
  for (int i = 0; i < kChunksPerWave; ++i) {
    if (valid_id(ids[i], e)) atomicAdd(&cnt[ids[i]], 1);
    else if (ids[i] != -1) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int x = threadIdx.x; x < e; x += kLayoutThreads) tile_counts[(int64_t)blockIdx.x * e + x] = cnt[x];
  if (threadIdx.x == 0) tile_invalid[blockIdx.x] = cnt[e];
}

__global__ __launch_bounds__(kLayoutThreads) void layout_place(
    const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_w, int64_t a_total, int64_t tiles, int e,
    int id_bits, int capacity, int row_align, int64_t rows, const int32_t *__restrict__ tile_counts,
    const int32_t *__restrict__ tile_invalid, int32_t *__restrict__ full_list, int32_t *__restrict__ full_off,
    int32_t *__restrict__ tokens_per_expert,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ counters, int32_t *__restrict__ ordinal,
    int32_t *__restrict__ assign_row, int32_t *__restrict__ row_src, uint8_t *__restrict__ drop_mask,
    uint8_t *__restrict__ pad_mask, float *__restrict__ w_perm) {
  extern __shared__ int32_t sm[];
  int32_t *run = sm;                      // [waves][e] running per-expert count of each wave
  int32_t *off = run + kLayoutWaves * e;  // [e + 1] segment starts
  int32_t *kept = off + e + 1;            // [e]
  int32_t *base = kept + e;               // [e] this tile's base (counts of earlier tiles)
  int32_t *total = base + e;              // [e] expert counts over all tiles
  int32_t *full = total + e;              // [e + 1] (drop by weight) starts of the experts' full lists
  __shared__ int32_t part[2][kLayoutThreads];
  __shared__ int32_t red[3][kLayoutWaves];
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();
  const int64_t tile = blockIdx.x;

  // this tile's expert ids, loaded first so they arrive while the count matrix is read
  const int64_t a_wave = tile * kLayoutTile + (int64_t)w * kChunksPerWave * kWave;
  int32_t ids[kChunksPerWave];
#pragma unroll
  for (int c = 0; c < kChunksPerWave; ++c) {
    const int64_t a = a_wave + c * kWave + l;
    ids[c] = (tile < tiles && a < a_total) ? topk_idx[a] : -1;
  }

  // ---- per-expert sums over tiles: before this tile, and over all tiles
  if (e <= kLayoutThreads) {
    // thread (g, x): expert x, tiles g, g+G, g+2G, ...  (G groups of e threads)
    const int groups = kLayoutThreads / e;
    const int g = tid / e, x = tid % e;
    if (g < groups) {
      int32_t before = 0, all = 0;
      for (int64_t t0 = g; t0 < tiles; t0 += 16 * (int64_t)groups) {
        int32_t c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int64_t t = t0 + (int64_t)u * groups;
          c[u] = t < tiles ? tile_counts[t * e + x] : 0;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          all += c[u];
          if (t0 + (int64_t)u * groups < tile) before += c[u];
        }
      }
      part[0][tid] = before;
      part[1][tid] = all;
    }
    __syncthreads();
    if (tid < e) {
      int32_t b = 0, a = 0;
      for (int gg = 0; gg < groups; ++gg) {
        b += part[0][gg * e + tid];
        a += part[1][gg * e + tid];
      }
      base[tid] = b;
      total[tid] = a;
    }
  } else {
    for (int x = tid; x < e; x += kLayoutThreads) {
      int32_t before = 0, all = 0;
      for (int64_t t0 = 0; t0 < tiles; t0 += 16) {
        int32_t c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) c[u] = t0 + u < tiles ? tile_counts[(t0 + u) * e + x] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          all += c[u];
          if (t0 + u < tile) before += c[u];
        }
      }
      base[x] = before;
      total[x] = all;
    }
  }
  __syncthreads();

  // drop by weight (full_list given): every assignment is listed, expert by
  // expert in assignment order, for capacity_select_kernel to choose from
  if (full_list) {
    block_exclusive_scan(total, full, e);
    if (tid == 0) full[e] = full[e - 1] + total[e - 1];
    __syncthreads();
    if (blockIdx.x == 0)
      for (int x = tid; x <= e; x += kLayoutThreads) full_off[x] = full[x];
  }

  // ---- segment offsets and kept counts
  if (capacity > 0) {
    for (int x = tid; x < e; x += kLayoutThreads) {
      off[x] = x * capacity;
      kept[x] = total[x] < capacity ? total[x] : capacity;
    }
    if (tid == 0) off[e] = (int32_t)rows;
    __syncthreads();
  } else {
    // segment lengths rounded up to the alignment (kept[] as scratch), their
    // exclusive scan, then each start and kept count clipped to the budget
    __shared__ int32_t used_end;
    for (int x = tid; x < e; x += kLayoutThreads) kept[x] = (total[x] + row_align - 1) / row_align * row_align;
    __syncthreads();
    block_exclusive_scan(kept, off, e);
    if (tid == 0) {
      const int64_t end = (int64_t)off[e - 1] + kept[e - 1];
      used_end = (int32_t)(end < rows ? end : rows);
    }
    __syncthreads();
    for (int x = tid; x < e; x += kLayoutThreads) {
      const int32_t s0 = off[x] < rows ? off[x] : (int32_t)rows;
      const int64_t room = rows - s0;
      kept[x] = (int32_t)(total[x] < room ? total[x] : room);
      off[x] = s0;
    }
    if (tid == 0) off[e] = used_end;
    __syncthreads();
  }

  if (blockIdx.x == 0) {  // the expert counts, offsets and counters
    int32_t k_sum = 0, t_sum = 0, inv = 0;
    for (int x = tid; x < e; x += kLayoutThreads) {
      tokens_per_expert[x] = kept[x];
      expert_offsets[x] = off[x];
      k_sum += kept[x];
      t_sum += total[x];
    }
    if (tid == 0) expert_offsets[e] = off[e];
    for (int64_t t = tid; t < tiles; t += kLayoutThreads) inv += tile_invalid[t];
    k_sum = wave_sum_i32(k_sum);
    t_sum = wave_sum_i32(t_sum);
    inv = wave_sum_i32(inv);
    if (l == 0) {
      red[0][w] = k_sum;
      red[1][w] = t_sum;
      red[2][w] = inv;
    }
    __syncthreads();
    if (tid == 0) {
      int32_t ks = 0, ts = 0, is = 0;
      for (int ww = 0; ww < kLayoutWaves; ++ww) {
        ks += red[0][ww];
        ts += red[1][ww];
        is += red[2][ww];
      }
      counters[0] = ks;
      counters[1] = ts - ks;
      counters[2] = off[e] - ks;  // rows below the end of the last segment holding nothing: pads
      counters[3] = is;
    }
  }

  if (tile < tiles) {  // block-uniform
    for (int x = tid; x < kLayoutWaves * e; x += kLayoutThreads) run[x] = 0;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c)
      if (valid_id(ids[c], e)) atomicAdd(&run[w * e + ids[c]], 1);
    __syncthreads();
    // exclusive prefix over the waves of this tile, on top of the tile's base
    for (int x = tid; x < e; x += kLayoutThreads) {
      int32_t b = base[x];
#pragma unroll
      for (int ww = 0; ww < kLayoutWaves; ++ww) {
        const int32_t c = run[ww * e + x];
        run[ww * e + x] = b;
        b += c;
      }
    }
    __syncthreads();
    const uint64_t below = lanes_below_mask();
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
      const int64_t a = a_wave + c * kWave + l;
      const int32_t x = ids[c];
      const bool valid = valid_id(x, e);
      uint64_t peers = ballot(valid);
      for (int b = 0; b < id_bits; ++b) {
        const bool bit = (x >> b) & 1;
        const uint64_t bal = ballot(valid && bit);
        peers &= bit ? bal : ~bal;
      }
      if (valid) {
        const int rank = __popcll(peers & below);
        const int32_t b = run[w * e + x];
        if (rank == 0) run[w * e + x] = b + __popcll(peers);
        const int32_t o = b + rank;
        ordinal[a] = o;
        if (full_list) {
          full_list[full[x] + o] = (int32_t)a;  // kept or dropped: capacity_select_kernel decides
        } else if (o < kept[x]) {
          const int32_t r = off[x] + o;
          assign_row[a] = r;
          drop_mask[a] = 0;
          row_src[r] = (int32_t)a;
          pad_mask[r] = 0;
          if (w_perm) w_perm[r] = topk_w[a];
        } else {
          assign_row[a] = -1;
          drop_mask[a] = 1;
        }
      } else if (a < a_total) {
        ordinal[a] = -1;
        assign_row[a] = -1;
        drop_mask[a] = 0;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }

  // rows that receive no assignment: capacity or alignment pads and the unused
  // dropless tail
  for (int64_t r = (int64_t)blockIdx.x * kLayoutThreads + tid; r < rows; r += (int64_t)gridDim.x * kLayoutThreads) {
    int x;
    if (capacity > 0) {
      x = (int)(r / capacity);
    } else {  // last expert whose segment starts at or before r
      int lo = 0, hi = e;  // off[lo] <= r always holds (off[0] == 0)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= r) lo = mid;
        else hi = mid - 1;
      }
      x = lo;
    }
    if (x < e && r - off[x] < kept[x]) continue;  // written by the assignment pass
    row_src[r] = -1;
    pad_mask[r] = 1;
    if (w_perm) w_perm[r] = 0.0f;
  }
}

// Order-preserving key of a weight for the drop-by-weight policy: a larger
// number gets a larger key, -0.0 == +0.0, NaN gets 0 (below every number).
__device__ __forceinline__ uint32_t weight_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelectThreads = 1024;
constexpr int kSelectWaves = kSelectThreads / kWave;
constexpr int kSelectLdsKeys = 32768;  // weight keys of an expert held in LDS (128 KiB); the rest re-read

// Exclusive prefix of a per-thread flag over the block in thread order, and the
// block total (every thread calls it; `wave_tot` holds kSelectWaves ints).
__device__ __forceinline__ int32_t block_flag_scan(bool f, int32_t *wave_tot, int32_t &total) {
  const int w = threadIdx.x / kWave;
  const uint64_t bal = ballot(f);
  const int32_t below = __popcll(bal & lanes_below_mask());
  if (lane_id() == 0) wave_tot[w] = __popcll(bal);
  __syncthreads();
  int32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kSelectWaves; ++i) {
    before += i < w ? wave_tot[i] : 0;
    all += wave_tot[i];
  }
  __syncthreads();
  total = all;
  return before + below;
}

// Drop by weight (Megatron's "probs" token-drop policy), one workgroup per
// expert: of the expert's assignments (full_list, in assignment order) keep the
// `capacity` with the largest weights -- ties to the earlier assignment, NaN
// below every number -- and place the kept ones in the expert's rows in
// assignment order.  The weight threshold comes from a radix select over the
// 32-bit weight keys (held in LDS), one byte per pass from the top: a
// histogram of the next byte among the keys that match the bytes chosen so far
// gives the byte of the C-th largest key (each of 256 threads sums the bins
// above its own) and how many keys above it are kept.  A last, ordered pass
// keeps every key above the threshold and the first `need` keys equal to it.
__global__ __launch_bounds__(kSelectThreads) void capacity_select_kernel(
    const int32_t *__restrict__ full_list, const int32_t *__restrict__ full_off, const float *__restrict__ topk_w,
    int capacity, int32_t *__restrict__ assign_row, uint8_t *__restrict__ drop_mask, int32_t *__restrict__ row_src,
    uint8_t *__restrict__ pad_mask, float *__restrict__ w_perm) {
  extern __shared__ uint32_t keys[];  // [kSelectLdsKeys]
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix;
  __shared__ int32_t sh_need;
  __shared__ int32_t wave_tot[kSelectWaves];
  const int x = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t c0 = full_off[x];
  const int32_t c = full_off[x + 1] - c0;
  const int32_t *list = full_list + c0;
  const bool select = c > capacity;
  auto key_of = [&](int32_t i) { return i < kSelectLdsKeys ? keys[i] : weight_key(topk_w[list[i]]); };
  uint32_t thr = 0;
  int32_t need = capacity;
  if (select) {
    const int32_t cached = c < kSelectLdsKeys ? c : kSelectLdsKeys;
    for (int32_t i = tid; i < cached; i += kSelectThreads) keys[i] = weight_key(topk_w[list[i]]);
    uint32_t prefix = 0, mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int32_t i = tid; i < c; i += kSelectThreads) {
        const uint32_t kk = key_of(i);
        if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
      }
      __syncthreads();
      // the bin holding the need-th largest matching key: thread t < 256 takes
      // bin b = 255 - t, an inclusive scan over those threads gives the number
      // of keys in bins b and above
      int32_t incl = 0;
      if (tid < 256) {
        const int32_t hb = (int32_t)hist[255 - tid];
        incl = wave_incl_scan(hb);
        if (lane_id() == kWave - 1) wave_tot[tid / kWave] = incl;
      }
      __syncthreads();
      if (tid < 256) {
        for (int i = 0; i < tid / kWave; ++i) incl += wave_tot[i];
        const int32_t hb = (int32_t)hist[255 - tid];
        if (incl - hb < need && incl >= need) {
          sh_need = need - (incl - hb);
          sh_prefix = prefix | ((uint32_t)(255 - tid) << shift);
        }
      }
      __syncthreads();
      need = sh_need;
      prefix = sh_prefix;
      mask |= 255u << shift;
      __syncthreads();
    }
    thr = prefix;
  }
  int32_t run_tie = 0, run_keep = 0;
  for (int32_t b0 = 0; b0 < c; b0 += kSelectThreads) {
    const int32_t i = b0 + tid;
    const bool valid = i < c;
    const int32_t a = valid ? list[i] : -1;
    const uint32_t kk = valid && select ? key_of(i) : 0u;
    const bool tie = valid && select && kk == thr;
    int32_t n_tie, n_keep;
    const int32_t tie_rank = run_tie + block_flag_scan(tie, wave_tot, n_tie);
    const bool keep = valid && (!select || kk > thr || (tie && tie_rank < need));
    const int32_t slot = run_keep + block_flag_scan(keep, wave_tot, n_keep);
    if (keep) {
      const int32_t r = x * capacity + slot;
      assign_row[a] = r;
      drop_mask[a] = 0;
      row_src[r] = a;
      pad_mask[r] = 0;
      if (w_perm) w_perm[r] = topk_w[a];
    } else if (valid) {
      assign_row[a] = -1;
      drop_mask[a] = 1;
    }
    run_tie += n_tie;
    run_keep += n_keep;
  }
}

}  // namespace

size_t layout_workspace_bytes(int64_t assignments, int e, bool drop_by_weight) {
  const int64_t tiles = layout_tiles(assignments);
  size_t b = align256(sizeof(int32_t) * (size_t)tiles * (size_t)e) + align256(sizeof(int32_t) * (size_t)tiles);
  if (drop_by_weight)  // every assignment listed by expert, and the list offsets
    b += align256(sizeof(int32_t) * (size_t)assignments) + align256(sizeof(int32_t) * (size_t)(e + 1));
  return b;
}

hipError_t launch_layout(const int32_t *topk_idx, const float *topk_w, int64_t n, int k, int e, int capacity,
                         int row_align, bool drop_by_weight, int64_t rows, int32_t *tokens_per_expert,
                         int32_t *expert_offsets, int32_t *ordinal, int32_t *assign_row, int32_t *row_src,
                         uint8_t *drop_mask, uint8_t *pad_mask, int32_t *counters, float *w_perm, void *workspace,
                         hipStream_t stream) {
  const int64_t a_total = n * k;
  const int64_t tiles = layout_tiles(a_total);
  char *ws = static_cast<char *>(workspace);
  int32_t *tile_counts = reinterpret_cast<int32_t *>(ws);
  ws += align256(sizeof(int32_t) * (size_t)tiles * (size_t)e);
  int32_t *tile_invalid = reinterpret_cast<int32_t *>(ws);
  ws += align256(sizeof(int32_t) * (size_t)tiles);
  const bool by_weight = drop_by_weight && capacity > 0;
  int32_t *full_list = nullptr, *full_off = nullptr;
  if (by_weight) {
    full_list = reinterpret_cast<int32_t *>(ws);
    ws += align256(sizeof(int32_t) * (size_t)a_total);
    full_off = reinterpret_cast<int32_t *>(ws);
  }
  if (tiles > 0) {
    hipLaunchKernelGGL(layout_count, dim3((unsigned)tiles), dim3(kLayoutThreads), sizeof(int32_t) * (e + 1), stream,
                       topk_idx, a_total, e, tile_counts, tile_invalid);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
  }
  int64_t row_blocks = (rows + kLayoutThreads - 1) / kLayoutThreads;
  if (row_blocks > 256) row_blocks = 256;
  int64_t blocks = tiles > row_blocks ? tiles : row_blocks;
  if (blocks == 0) blocks = 1;  // workgroup 0 still writes counts, offsets and counters
  const int id_bits = e <= 1 ? 0 : 32 - __builtin_clz((unsigned)(e - 1));
  const size_t lds = sizeof(int32_t) * ((size_t)kLayoutWaves * e + 5 * (size_t)e + 2);
  hipLaunchKernelGGL(layout_place, dim3((unsigned)blocks), dim3(kLayoutThreads), lds, stream, topk_idx, topk_w,
                     a_total, tiles, e, id_bits, capacity, row_align > 1 ? row_align : 1, rows, tile_counts,
                     tile_invalid, full_list, full_off, tokens_per_expert, expert_offsets, counters, ordinal,
                     assign_row, row_src, drop_mask, pad_mask, w_perm);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess || !by_weight) return st;
  hipLaunchKernelGGL(capacity_select_kernel, dim3((unsigned)e), dim3(kSelectThreads),
                     sizeof(uint32_t) * kSelectLdsKeys, stream, full_list, full_off, topk_w, capacity, assign_row,
                     drop_mask, row_src, pad_mask, w_perm);
  return hipGetLastError();
}

}  // namespace moe
