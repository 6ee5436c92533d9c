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
//                   clipped to the row budget R
//   assign_row[a] = offset[id[a]] + ordinal[a] if kept, else -1
//
// How (three launches, no host synchronisation, no atomics on the ordering
// path, so the result does not depend on scheduling):
//   1. layout_count: one workgroup per tile of 512 assignments builds an LDS
//      histogram of the tile's ids -> tile_counts[tile][e].
//   2. layout_scan: one workgroup turns tile_counts into per-expert exclusive
//      prefixes over tiles (in place), totals, offsets and counters.
//   3. layout_place: per tile, each wave walks its 64-assignment chunks in order;
//      lanes holding the same expert find each other with one ballot per bit of
//      the expert id (a wave64 "match"), rank = popcount(peers below the lane);
//      the per-wave running count per expert lives in LDS and starts at the
//      tile's prefix plus the counts of the earlier waves of the tile.  The same
//      launch marks every row that receives no assignment (pad or tail).
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kLayoutThreads = 256;
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kChunksPerWave = kLayoutTile / kLayoutThreads;  // 64-assignment chunks per wave
static_assert(kLayoutTile % kLayoutThreads == 0, "tile must be a multiple of the block");
constexpr int kScanThreads = 1024;

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

__device__ __forceinline__ bool valid_id(int32_t x, int e) { return x >= 0 && x < e; }

__global__ __launch_bounds__(kLayoutThreads) void layout_count(const int32_t *__restrict__ topk_idx, int64_t a_total,
                                                               int e, int32_t *__restrict__ tile_counts,
                                                               int32_t *__restrict__ tile_invalid) {
  extern __shared__ int32_t cnt[];  // [e + 1], cnt[e] = invalid ids
  for (int x = threadIdx.x; x <= e; x += kLayoutThreads) cnt[x] = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * kLayoutTile;
  for (int i = threadIdx.x; i < kLayoutTile; i += kLayoutThreads) {
    const int64_t a = a0 + i;
    if (a < a_total) {
      const int32_t x = topk_idx[a];
      if (valid_id(x, e)) atomicAdd(&cnt[x], 1);
      else if (x != -1) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < e; x += kLayoutThreads) tile_counts[(int64_t)blockIdx.x * e + x] = cnt[x];
  if (threadIdx.x == 0) tile_invalid[blockIdx.x] = cnt[e];
}

// Thread (x, g) owns expert x and a contiguous group g of tiles; the group sums
// are scanned in LDS, so every global load of the tile counts is independent.
__global__ __launch_bounds__(kScanThreads) void layout_scan(int32_t *__restrict__ tile_counts,
                                                            const int32_t *__restrict__ tile_invalid, int64_t tiles,
                                                            int e, int groups, int capacity, int64_t rows,
                                                            int32_t *__restrict__ tokens_per_expert,
                                                            int32_t *__restrict__ expert_offsets,
                                                            int32_t *__restrict__ counters) {
  __shared__ int64_t scan[kScanThreads];    // per expert: inclusive scan of totals
  __shared__ int32_t grp[kScanThreads];     // [groups][e] group sums, then group prefixes
  __shared__ unsigned long long sums[3];    // kept, dropped, invalid
  const int tid = threadIdx.x;
  const int x = tid % e;
  const int g = tid / e;
  const bool active = g < groups;
  const int64_t per_group = (tiles + groups - 1) / groups;
  const int64_t t0 = (int64_t)g * per_group;
  const int64_t t1 = t0 + per_group < tiles ? t0 + per_group : tiles;
  if (tid < 3) sums[tid] = 0;
  int32_t s = 0;
  if (active)
    for (int64_t t = t0; t < t1; ++t) s += tile_counts[t * e + x];
  if (active) grp[g * e + x] = s;
  __syncthreads();
  int32_t prefix = 0;
  int64_t total = 0;
  if (active) {
    for (int gg = 0; gg < groups; ++gg) {
      const int32_t v = grp[gg * e + x];
      if (gg < g) prefix += v;
      total += v;
    }
  }
  __syncthreads();
  if (active) {  // per-expert exclusive prefix over tiles, in place
    int32_t run = prefix;
    for (int64_t t = t0; t < t1; t += 8) {
      int32_t c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = t + u < t1 ? tile_counts[(t + u) * e + x] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (t + u < t1) {
          tile_counts[(t + u) * e + x] = run;
          run += c[u];
        }
    }
  }
  scan[tid] = (g == 0 && tid < e) ? total : 0;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {  // inclusive scan over experts
    const int64_t v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  if (g == 0 && tid < e) {
    int64_t start, kept;
    if (capacity > 0) {
      start = (int64_t)x * capacity;
      kept = total < capacity ? total : capacity;
    } else {
      const int64_t excl = scan[x] - total;
      const int64_t incl = scan[x];
      start = excl < rows ? excl : rows;
      kept = (incl < rows ? incl : rows) - start;
    }
    expert_offsets[x] = (int32_t)start;
    if (x == e - 1) expert_offsets[e] = (int32_t)(capacity > 0 ? rows : (scan[x] < rows ? scan[x] : rows));
    tokens_per_expert[x] = (int32_t)kept;
    atomicAdd(&sums[0], (unsigned long long)kept);
    atomicAdd(&sums[1], (unsigned long long)(total - kept));
  }
  for (int64_t t = tid; t < tiles; t += kScanThreads) atomicAdd(&sums[2], (unsigned long long)tile_invalid[t]);
  __syncthreads();
  if (tid == 0) {
    counters[0] = (int32_t)sums[0];
    counters[1] = (int32_t)sums[1];
    counters[2] = capacity > 0 ? (int32_t)(rows - (int64_t)sums[0]) : 0;
    counters[3] = (int32_t)sums[2];
  }
}

__global__ __launch_bounds__(kLayoutThreads) void layout_place(
    const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_w, int64_t a_total, int64_t tiles, int e,
    int id_bits, int capacity, int64_t rows, const int32_t *__restrict__ tile_base,
    const int32_t *__restrict__ expert_offsets, const int32_t *__restrict__ tokens_per_expert,
    int32_t *__restrict__ ordinal, int32_t *__restrict__ assign_row, int32_t *__restrict__ row_src,
    uint8_t *__restrict__ drop_mask, uint8_t *__restrict__ pad_mask, float *__restrict__ w_perm) {
  extern __shared__ int32_t sm[];
  int32_t *run = sm;                        // [waves][e] running per-expert count of each wave
  int32_t *off = sm + kLayoutWaves * e;     // [e + 1]
  int32_t *kept = off + e + 1;              // [e]
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  const int64_t tile = blockIdx.x;

  for (int x = threadIdx.x; x < e; x += kLayoutThreads) {
    off[x] = expert_offsets[x];
    kept[x] = tokens_per_expert[x];
#pragma unroll
    for (int ww = 0; ww < kLayoutWaves; ++ww) run[ww * e + x] = 0;
  }
  if (threadIdx.x == 0) off[e] = expert_offsets[e];
  __syncthreads();

  if (tile < tiles) {  // block-uniform
    const int64_t a_wave = tile * kLayoutTile + (int64_t)w * kChunksPerWave * kWave;
    int32_t ids[kChunksPerWave];
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
      const int64_t a = a_wave + c * kWave + l;
      ids[c] = a < a_total ? topk_idx[a] : -1;
      if (valid_id(ids[c], e)) atomicAdd(&run[w * e + ids[c]], 1);
    }
    __syncthreads();
    // exclusive prefix over the waves of this tile, on top of the tile's base
    for (int x = threadIdx.x; x < e; x += kLayoutThreads) {
      int32_t base = tile_base[tile * e + x];
#pragma unroll
      for (int ww = 0; ww < kLayoutWaves; ++ww) {
        const int32_t c = run[ww * e + x];
        run[ww * e + x] = base;
        base += c;
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
        const int32_t base = run[w * e + x];
        if (rank == 0) run[w * e + x] = base + __popcll(peers);
        const int32_t o = base + rank;
        ordinal[a] = o;
        if (o < kept[x]) {
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

  // rows that receive no assignment: capacity pads and the unused dropless tail
  for (int64_t r = (int64_t)blockIdx.x * kLayoutThreads + threadIdx.x; r < rows;
       r += (int64_t)gridDim.x * kLayoutThreads) {
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

}  // namespace

size_t layout_workspace_bytes(int64_t assignments, int e) {
  const int64_t tiles = layout_tiles(assignments);
  return align256(sizeof(int32_t) * (size_t)tiles * (size_t)e) + align256(sizeof(int32_t) * (size_t)tiles);
}

hipError_t launch_layout(const int32_t *topk_idx, const float *topk_w, int64_t n, int k, int e, int capacity,
                         int64_t rows, int32_t *tokens_per_expert, int32_t *expert_offsets, int32_t *ordinal,
                         int32_t *assign_row, int32_t *row_src, uint8_t *drop_mask, uint8_t *pad_mask,
                         int32_t *counters, float *w_perm, void *workspace, hipStream_t stream) {
  const int64_t a_total = n * k;
  const int64_t tiles = layout_tiles(a_total);
  int32_t *tile_counts = static_cast<int32_t *>(workspace);
  int32_t *tile_invalid = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                                      align256(sizeof(int32_t) * (size_t)tiles * (size_t)e));
  if (tiles > 0) {
    hipLaunchKernelGGL(layout_count, dim3((unsigned)tiles), dim3(kLayoutThreads), sizeof(int32_t) * (e + 1), stream,
                       topk_idx, a_total, e, tile_counts, tile_invalid);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
  }
  int groups = kScanThreads / e;
  if (groups > 64) groups = 64;
  if (groups > tiles) groups = tiles > 0 ? (int)tiles : 1;
  hipLaunchKernelGGL(layout_scan, dim3(1), dim3(kScanThreads), 0, stream, tile_counts, tile_invalid, tiles, e,
                     groups, capacity, rows, tokens_per_expert, expert_offsets, counters);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  int64_t row_blocks = (rows + kLayoutThreads - 1) / kLayoutThreads;
  if (row_blocks > 1024) row_blocks = 1024;
  const int64_t blocks = tiles > row_blocks ? tiles : row_blocks;
  if (blocks == 0) return hipSuccess;
  const int id_bits = e <= 1 ? 0 : 32 - __builtin_clz((unsigned)(e - 1));
  const size_t lds = sizeof(int32_t) * ((size_t)kLayoutWaves * e + 2 * (size_t)e + 1);
  hipLaunchKernelGGL(layout_place, dim3((unsigned)blocks), dim3(kLayoutThreads), lds, stream, topk_idx, topk_w,
                     a_total, tiles, e, id_bits, capacity, rows, tile_counts, expert_offsets, tokens_per_expert,
                     ordinal, assign_row, row_src, drop_mask, pad_mask, w_perm);
  return hipGetLastError();
}

}  // namespace moe
