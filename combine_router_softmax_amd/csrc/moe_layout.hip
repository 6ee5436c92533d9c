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
// How: one single-pass scan kernel, no host synchronisation.
//   layout_scan: one workgroup per tile of 2048 assignments.  A workgroup takes
//   its tile number from an atomic ticket, so every earlier tile belongs to a
//   workgroup that is already running (or done) and waiting on it cannot
//   deadlock.  It builds per-wave LDS histograms of its ids, publishes the
//   tile's per-expert counts, and ranks its assignments inside the tile: lanes
//   holding the same expert find each other with one ballot per bit of the
//   expert id (a wave64 match), local rank = earlier waves + peers below.  Then
//   it finds the counts of all earlier tiles by a decoupled look-back (Merrill
//   and Garland, "Single-pass Parallel Prefix Scan with Decoupled Look-back",
//   2016): walking back over the earlier tiles' published words -- a tile's own
//   count (AGG) or its inclusive prefix (INCL), which ends the walk -- sixteen
//   words in flight per round; publishes its inclusive prefix; and writes
//   ordinal = earlier tiles + local rank.  The tile with the last ticket holds
//   the totals and writes the counts, segment offsets and counters.  Ordinals
//   never depend on atomic order: the tiles are scanned in assignment order
//   whatever order they run in.
//   Rows are then placed from (ordinal, kept, offset) alone (moe_place.hpp):
//   by the scatter as it copies the rows, or by layout_finish where no scatter
//   follows.  In a dispatch, extra workgroups of the scan launch read the
//   source rows meanwhile, so that the scatter finds them in the memory-side
//   cache (layout_scan).
// Status words are 64-bit: [63:34] the call's epoch, [33:32] the flag, [31:0]
// the count, written and read with device-scope atomics, so one word carries
// flag and value together.  The workspace header holds the ticket and the
// epoch; the kernel that follows the scan in the same call resets the ticket
// and advances the epoch (finish_scan), so words left by an earlier call never
// look ready and the workspace needs no clearing between calls -- only the
// header must be zero before its first use.  A wait that runs past a bound (a
// header that was not zeroed, two calls sharing one workspace) gives up, and
// the call reports it with counters[3] = -1 instead of hanging.
// With a capacity and the drop-by-weight policy, layout_finish lists every
// assignment by expert and capacity_select_kernel keeps each expert's largest
// weights (see there).
#include "moe_device.hpp"
#include "moe_kernels.hpp"
#include "moe_place.hpp"

namespace moe {
namespace {

constexpr int kScanThreads = 512;
constexpr int kScanWaves = kScanThreads / kWave;
constexpr int kScanChunks = kLayoutTile / kScanThreads;  // 64-assignment chunks per wave
static_assert(kLayoutTile % kScanThreads == 0, "tile must be a multiple of the block");
constexpr int kMaxExperts = 1024;
constexpr int kLookback = 16;                // status words in flight per thread and round
constexpr uint32_t kSpinLimit = 1u << 17;    // polls of one word before giving up (~0.1 s)
constexpr uint64_t kFlagAgg = 1, kFlagIncl = 2;
constexpr uint32_t kEpochMask = 0x3FFFFFFFu;
constexpr int kWarmLoads = 8;                     // 16-byte loads in flight per thread
// row-reading workgroups beside the scan: one per compute unit (the scan's
// registers allow one 512-thread workgroup per unit); 64 and 128 measured
// 3-9 us slower cold
constexpr int64_t kWarmBlocks = 256;
// at most 64 MiB of rows, about what HBM delivers while the scan runs: reading
// more outlasts the scan and delays the scatter (measured: 128 MiB of a
// 235 MB source took a warm dispatch from 117 to 125 us and gained nothing
// cold; 64 MiB: 117 -> 119 us warm, 142 -> 140 us cold)
constexpr int64_t kWarmMaxBytes = 64ll << 20;

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

constexpr size_t kHeaderBytes = 256;  // ScanHeader (moe_place.hpp), padded

__device__ __forceinline__ bool valid_id(int32_t x, int e) { return x >= 0 && x < e; }

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations,
// then s_barrier (__syncthreads() also waits for every global store of the wave
// to be acknowledged).  The scan's status words, ordinals and totals are read
// by other workgroups or by the next kernel, never by this workgroup, so its
// barriers need not wait for them: measured, each such wait cost about a
// microsecond of the scan's critical path.  The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ void fill_u32(uint32_t *p, int64_t n, uint32_t v) {
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) p[i] = v;
}

__device__ __forceinline__ uint64_t status_word(uint32_t epoch, uint64_t flag, uint32_t v) {
  return ((uint64_t)(epoch & kEpochMask) << 34) | (flag << 32) | v;
}
__device__ __forceinline__ bool status_ready(uint64_t w, uint32_t epoch) {
  return (uint32_t)(w >> 34) == (epoch & kEpochMask) && ((w >> 32) & 3u) != 0;
}
__device__ __forceinline__ uint64_t ld_status(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_status(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The first kLookback status words of bin x before `tile` (nearest first).
__device__ __forceinline__ void look_back_first(const uint64_t *status, int64_t tile, int nbins, int x,
                                                uint64_t (&w)[kLookback]) {
#pragma unroll
  for (int i = 0; i < kLookback; ++i) w[i] = tile - 1 - i >= 0 ? ld_status(status + (tile - 1 - i) * nbins + x) : 0ull;
}

// Sum of bin x over the tiles before `tile`: walk back over their status words,
// kLookback at a time (`w` holds the first batch, look_back_first),
// adding each tile's count down to the nearest inclusive prefix, which is added
// and ends the walk.  A batch is summed once every word it needs -- those up to
// its nearest inclusive prefix -- carries this call's epoch; the words still
// missing are requested again together, so each round costs one memory round
// trip however many of them are missing.  Past the bound a wait records the
// fault and the walk ends (see the file comment).
__device__ __forceinline__ uint32_t look_back(const uint64_t *status, int64_t tile, int nbins, int x, uint32_t epoch,
                                              ScanHeader *hdr, uint64_t (&w)[kLookback]) {
  uint32_t sum = 0;
  for (int64_t p = tile - 1; p >= 0; p -= kLookback) {
    if (p != tile - 1) {
#pragma unroll
      for (int i = 0; i < kLookback; ++i) w[i] = p - i >= 0 ? ld_status(status + (p - i) * nbins + x) : 0ull;
    }
    const int n = p + 1 < kLookback ? (int)(p + 1) : kLookback;  // words of this batch (tile 0 is the last)
    for (uint32_t spin = 0;; ++spin) {
      uint32_t missing = 0, incl = 0;
#pragma unroll
      for (int i = 0; i < kLookback; ++i) {
        const bool ready = i < n && status_ready(w[i], epoch);
        missing |= (i < n && !ready ? 1u : 0u) << i;
        incl |= (ready && ((w[i] >> 32) & 3u) == kFlagIncl ? 1u : 0u) << i;
      }
      const int last = incl ? __builtin_ctz(incl) : n - 1;  // the batch's words that count: 0..last
      const uint32_t needed = last >= 31 ? ~0u : (2u << last) - 1u;
      if (!(missing & needed)) {
#pragma unroll
        for (int i = 0; i < kLookback; ++i)
          if (i <= last) sum += (uint32_t)w[i];
        if (incl) return sum;
        break;  // every word of the batch is a tile's own count: the next batch
      }
      if (spin == kSpinLimit) {
        __hip_atomic_store(&hdr->fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return sum;
      }
      __builtin_amdgcn_s_sleep(2);
#pragma unroll
      for (int i = 0; i < kLookback; ++i)
        if ((missing & needed) >> i & 1u) w[i] = ld_status(status + (p - i) * nbins + x);
    }
  }
  return sum;
}

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

// The last tile: from the expert totals (total[0..e), total[e] = invalid ids)
// the kept counts, segment starts and counters.  Each thread holds kPer
// consecutive experts; the segment lengths (C, or the count rounded up to the
// alignment) and the totals are scanned together across the block (one
// barrier), each start and kept count clipped to the row budget R, and the
// kept counts reduced (a second barrier).
__device__ void finalize_layout(const int32_t *total, int e, int capacity, int row_align, int64_t rows,
                                int32_t *__restrict__ tokens_per_expert, int32_t *__restrict__ expert_offsets,
                                int32_t *__restrict__ counters, int32_t *__restrict__ full_off) {
  constexpr int kPer = kMaxExperts / kScanThreads;
  __shared__ int32_t wsum[3][kScanWaves];
  const int t = threadIdx.x, w = t / kWave, l = lane_id();
  int32_t tot[kPer], len[kPer];
  int32_t s_len = 0, s_tot = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int x = t * kPer + i;
    tot[i] = x < e ? total[x] : 0;
    len[i] = x >= e ? 0 : (capacity > 0 ? capacity : (tot[i] + row_align - 1) / row_align * row_align);
    s_len += len[i];
    s_tot += tot[i];
  }
  const int32_t i_len = wave_incl_scan(s_len), i_tot = wave_incl_scan(s_tot);
  if (l == kWave - 1) {
    wsum[0][w] = i_len;
    wsum[1][w] = i_tot;
  }
  lds_barrier();
  int32_t off = i_len - s_len, foff = i_tot - s_tot, all_len = 0, all_tot = 0;
#pragma unroll
  for (int ww = 0; ww < kScanWaves; ++ww) {
    off += ww < w ? wsum[0][ww] : 0;
    foff += ww < w ? wsum[1][ww] : 0;
    all_len += wsum[0][ww];
    all_tot += wsum[1][ww];
  }
  const int32_t used_end = (int32_t)(all_len < rows ? all_len : rows);  // rows = E*C with a capacity
  int32_t k_sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int x = t * kPer + i;
    if (x < e) {
      const int32_t s0 = off < rows ? off : (int32_t)rows;
      const int64_t room = capacity > 0 ? capacity : rows - s0;
      const int32_t kept = (int32_t)(tot[i] < room ? tot[i] : room);
      tokens_per_expert[x] = kept;
      expert_offsets[x] = s0;
      if (full_off) full_off[x] = foff;  // drop by weight: where the expert's list starts
      k_sum += kept;
    }
    off += len[i];
    foff += tot[i];
  }
  if (t == 0) {
    expert_offsets[e] = used_end;
    if (full_off) full_off[e] = all_tot;
  }
  k_sum = wave_sum_i32(k_sum);
  if (l == 0) wsum[2][w] = k_sum;
  lds_barrier();
  if (t == 0) {
    int32_t ks = 0;
#pragma unroll
    for (int ww = 0; ww < kScanWaves; ++ww) ks += wsum[2][ww];
    counters[0] = ks;
    counters[1] = all_tot - ks;
    counters[2] = used_end - ks;  // rows below the end of the last segment holding nothing: pads
    counters[3] = total[e];
  }
}

// One workgroup per tile of kLayoutTile assignments (see the file comment).
// Wave w owns the tile's assignments w*256 .. w*256+255, in four 64-wide
// chunks; bin e (E + 1 bins) counts the invalid ids (neither -1 nor an expert).
// BITS: an upper bound of the expert id's bit count (a compile-time count keeps
// the ballot loop unrolled; bits above the ids' own are zero in every lane).
// Workgroups from `tiles` on take no ticket: they read the dispatch's source
// rows (the first `warm_vecs` 16-byte vectors) and exit.  The scan is bound by
// memory round trips and leaves HBM idle meanwhile; the reads bring the rows
// into the memory-side cache, where the scatter that follows finds them, and
// HBM still delivers each byte once.  The values are consumed by an empty asm
// statement, so the loads stay whole 16-byte loads.
template <int BITS>
__global__ __launch_bounds__(kScanThreads) void layout_scan(
    const int32_t *__restrict__ topk_idx, int64_t a_total, int64_t tiles, int e, int capacity,
    int row_align, int64_t rows, ScanHeader *hdr, uint64_t *status, int32_t *__restrict__ ordinal,
    int32_t *__restrict__ tokens_per_expert, int32_t *__restrict__ expert_offsets, int32_t *__restrict__ counters,
    int32_t *__restrict__ full_off, const u32x4 *__restrict__ warm, int64_t warm_vecs) {
  if (blockIdx.x >= tiles) {  // block-uniform
    const int64_t stride = (int64_t)(gridDim.x - tiles) * kScanThreads * kWarmLoads;
    uint32_t acc = 0;
    for (int64_t v0 = (blockIdx.x - tiles) * kScanThreads * kWarmLoads + threadIdx.x; v0 < warm_vecs;
         v0 += stride) {
      u32x4 r[kWarmLoads];
#pragma unroll
      for (int i = 0; i < kWarmLoads; ++i) {
        const int64_t v = v0 + i * kScanThreads;
        r[i] = warm[v < warm_vecs ? v : warm_vecs - 1];  // past the end: the last vector again
      }
#pragma unroll
      for (int i = 0; i < kWarmLoads; ++i) acc ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
    }
    asm volatile("" ::"v"(acc));
    return;
  }
  extern __shared__ int32_t sm[];
  const int nb = e + 1;
  int32_t *run = sm;                  // [waves][nb] per-wave counts, then running bases
  int32_t *agg = run + kScanWaves * nb;  // [nb] this tile's counts
  int32_t *base = agg + nb;           // [nb] counts of the earlier tiles
  __shared__ uint32_t sh_ticket, sh_epoch;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = lane_id();

  // the ids of tile blockIdx.x are requested first and the ticket and epoch
  // together while they are on their way, so the three cost one memory round
  // trip (tickets mostly follow dispatch order; another ticket reloads the
  // ids).  The epoch does not change during the call.
  const int64_t guess = blockIdx.x;
  int32_t ids[kScanChunks];
#pragma unroll
  for (int c = 0; c < kScanChunks; ++c) {
    const int64_t a = guess * kLayoutTile + (int64_t)w * kScanChunks * kWave + c * kWave + l;
    ids[c] = a < a_total ? topk_idx[a] : -1;
  }
  if (tid == 0) {
    const uint32_t ep = __hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t tk = __hip_atomic_fetch_add(&hdr->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_epoch = ep;
    sh_ticket = tk;
  }
  for (int x = tid; x < kScanWaves * nb; x += kScanThreads) run[x] = 0;
  lds_barrier();
  const int64_t tile = sh_ticket;
  const uint32_t epoch = sh_epoch;

  if (tile < tiles) {  // block-uniform; a larger ticket only comes from a header that was not zeroed
    const int64_t a_wave = tile * kLayoutTile + (int64_t)w * kScanChunks * kWave;
    if (tile != guess) {
#pragma unroll
      for (int c = 0; c < kScanChunks; ++c) {
        const int64_t a = a_wave + c * kWave + l;
        ids[c] = a < a_total ? topk_idx[a] : -1;
      }
    }
#pragma unroll
    for (int c = 0; c < kScanChunks; ++c) {
      if (valid_id(ids[c], e)) atomicAdd(&run[w * nb + ids[c]], 1);
      else if (ids[c] != -1) atomicAdd(&run[w * nb + e], 1);
    }
    lds_barrier();

    // this tile's counts, published at once (tile 0's are already inclusive),
    // and each wave's base inside the tile (its earlier waves' counts)
    uint64_t *mine = status + tile * nb;
    for (int x = tid; x < nb; x += kScanThreads) {
      int32_t c[kScanWaves];
#pragma unroll
      for (int ww = 0; ww < kScanWaves; ++ww) c[ww] = run[ww * nb + x];
      int32_t s = 0;
#pragma unroll
      for (int ww = 0; ww < kScanWaves; ++ww) {
        run[ww * nb + x] = s;
        s += c[ww];
      }
      agg[x] = s;
      st_status(mine + x, status_word(epoch, tile == 0 ? kFlagIncl : kFlagAgg, (uint32_t)s));
    }
    lds_barrier();

    // the first look-back batch of this thread's bin is requested now and
    // read after the ranking, which hides its memory round trip
    uint64_t first0[kLookback];
    if (tile > 0 && tid < nb) look_back_first(status, tile, nb, tid, first0);
    // stable ranks inside the tile: chunks in order, peers found by a ballot per
    // id bit; the earlier tiles' counts are added once the look-back has them
    const uint64_t below = lanes_below_mask();
    int32_t local[kScanChunks];
#pragma unroll
    for (int c = 0; c < kScanChunks; ++c) {
      const int32_t x = ids[c];
      const bool valid = valid_id(x, e);
      uint64_t peers = ballot(valid);
#pragma unroll
      for (int b = 0; b < BITS; ++b) {
        const bool bit = (x >> b) & 1;
        const uint64_t bal = ballot(valid && bit);
        peers &= bit ? bal : ~bal;
      }
      local[c] = 0;
      if (valid) {
        const int rank = __popcll(peers & below);
        const int32_t b = run[w * nb + x];
        if (rank == 0) run[w * nb + x] = b + __popcll(peers);
        local[c] = b + rank;
      }
      __builtin_amdgcn_wave_barrier();
    }

    // the earlier tiles' counts by look-back, then this tile's inclusive prefix
    // (agg becomes the inclusive prefix: the totals, in the last tile).  Words
    // of the first batch that were not ready when requested are requested
    // again by the walk.  (Requesting the batch before the ranking measured
    // slower while the tile's start took three round trips; with one, it is
    // 0.6-1 us faster at 4096 x 8 over 256 experts.)
    for (int x = tid; x < nb; x += kScanThreads) {
      uint64_t first[kLookback];
      if (tile > 0) {
        if (x == tid) {
#pragma unroll
          for (int i = 0; i < kLookback; ++i) first[i] = first0[i];
        } else {
          look_back_first(status, tile, nb, x, first);
        }
      }
      const int32_t b = tile == 0 ? 0 : (int32_t)look_back(status, tile, nb, x, epoch, hdr, first);
      base[x] = b;
      agg[x] += b;
      if (tile > 0) st_status(mine + x, status_word(epoch, kFlagIncl, (uint32_t)agg[x]));
    }
    lds_barrier();
#pragma unroll
    for (int c = 0; c < kScanChunks; ++c) {
      const int64_t a = a_wave + c * kWave + l;
      if (valid_id(ids[c], e)) ordinal[a] = base[ids[c]] + local[c];
      else if (a < a_total) ordinal[a] = -1;
    }

    if (tile == tiles - 1)  // the totals: counts, segment offsets, counters
      finalize_layout(agg, e, capacity, row_align, rows, tokens_per_expert, expert_offsets, counters, full_off);
  } else if (tid == 0) {
    __hip_atomic_store(&hdr->fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the header is reset by the kernel that follows (finish_scan)
}

// Placement where no scatter follows (the MXFP8 dispatch and the drop-by-weight
// policy place rows in their own launch): blocks below `assign_blocks` take 256
// assignments each, the others take the rows that no assignment fills.
// list_full (drop by weight): valid assignments are listed by expert for
// capacity_select_kernel instead of placed; their rows are written there.
__global__ __launch_bounds__(256) void layout_finish(PlaceArgs p, int64_t a_total, int64_t assign_blocks,
                                                     int32_t *__restrict__ full_list,
                                                     const int32_t *__restrict__ full_off) {
  __shared__ int32_t off_lds[kPlaceMaxExperts + 1];
  const int64_t b = blockIdx.x;
  if (b == 0 && threadIdx.x == 0) finish_scan(p.hdr, p.counters);
  if (b < assign_blocks) {
    const int64_t a = b * 256 + threadIdx.x;
    if (a >= a_total) return;
    if (full_list) {
      const int32_t x = p.topk_idx[a];
      if (valid_id(x, p.e)) {
        const int64_t i = (int64_t)full_off[x] + p.ordinal[a];
        if (i >= 0 && i < a_total) full_list[i] = (int32_t)a;  // always, unless the scan gave up
      } else {
        p.assign_row[a] = -1;
        p.drop_mask[a] = 0;
      }
      return;
    }
    bool dropped;
    const int32_t r = placed_row(p, a, &dropped);
    write_assignment(p, a, r, dropped);
    return;
  }
  for (int x = threadIdx.x; x <= p.e; x += 256) off_lds[x] = p.off[x];
  __syncthreads();
  const int64_t used = used_rows(p, off_lds[p.e]);
  const int64_t stride = (gridDim.x - assign_blocks) * 256;
  for (int64_t r = (b - assign_blocks) * 256 + threadIdx.x + (p.has_pads ? 0 : used); r < p.rows; r += stride) {
    if (r < used) {
      const int x = segment_of(off_lds, p.e, p.capacity, r);
      if (r - off_lds[x] < p.kept[x]) continue;  // a kept row: written by its assignment
    }
    write_empty_row(p, r);
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
    int64_t a_total, int capacity, int32_t *__restrict__ assign_row, uint8_t *__restrict__ drop_mask, int32_t *__restrict__ row_src,
    uint8_t *__restrict__ pad_mask, float *__restrict__ w_perm) {
  extern __shared__ uint32_t keys[];  // [kSelectLdsKeys]
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix;
  __shared__ int32_t sh_need;
  __shared__ int32_t wave_tot[kSelectWaves];
  const int x = blockIdx.x;
  const int tid = threadIdx.x;
  // list bounds and entries are checked, so that a scan that gave up (see
  // layout_scan) cannot send a read or write outside the arrays
  auto clamp_a = [&](int32_t v) { return v < 0 ? 0 : (v > a_total ? (int32_t)a_total : v); };
  const int32_t c0 = clamp_a(full_off[x]);
  const int32_t c1 = clamp_a(full_off[x + 1]);
  const int32_t c = c1 > c0 ? c1 - c0 : 0;
  const int32_t *list = full_list + c0;
  auto entry = [&](int32_t i) {
    const int32_t a = list[i];
    return a >= 0 && a < a_total ? a : -1;
  };
  auto key_at = [&](int32_t i) {
    const int32_t a = entry(i);
    return a >= 0 ? weight_key(topk_w[a]) : 0u;
  };
  const bool select = c > capacity;
  auto key_of = [&](int32_t i) { return i < kSelectLdsKeys ? keys[i] : key_at(i); };
  uint32_t thr = 0;
  int32_t need = capacity;
  if (select) {
    const int32_t cached = c < kSelectLdsKeys ? c : kSelectLdsKeys;
    for (int32_t i = tid; i < cached; i += kSelectThreads) keys[i] = key_at(i);
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
    const int32_t a = i < c ? entry(i) : -1;
    const bool valid = a >= 0;
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
  size_t b = kHeaderBytes + align256(sizeof(uint64_t) * (size_t)tiles * (size_t)(e + 1));
  if (drop_by_weight)  // every assignment listed by expert, and the list offsets
    b += align256(sizeof(int32_t) * (size_t)assignments) + align256(sizeof(int32_t) * (size_t)(e + 1));
  return b;
}

namespace {

struct LayoutWorkspace {
  ScanHeader *hdr;
  uint64_t *status;
  int32_t *full_list;  // drop by weight only
  int32_t *full_off;
};

LayoutWorkspace carve(void *workspace, int64_t a_total, int e, bool by_weight) {
  char *ws = static_cast<char *>(workspace);
  LayoutWorkspace w{};
  w.hdr = reinterpret_cast<ScanHeader *>(ws);
  ws += kHeaderBytes;
  w.status = reinterpret_cast<uint64_t *>(ws);
  ws += align256(sizeof(uint64_t) * (size_t)layout_tiles(a_total) * (size_t)(e + 1));
  if (by_weight) {
    w.full_list = reinterpret_cast<int32_t *>(ws);
    ws += align256(sizeof(int32_t) * (size_t)a_total);
    w.full_off = reinterpret_cast<int32_t *>(ws);
  }
  return w;
}

// warm, warm_bytes: the rows the next kernel reads (nullptr, 0: none); the
// scan launch reads up to kWarmMaxBytes of them alongside (see layout_scan)
hipError_t scan(const int32_t *topk_idx, int64_t a_total, int e, int capacity, int row_align, int64_t rows,
                int32_t *tokens_per_expert, int32_t *expert_offsets, int32_t *ordinal, int32_t *counters,
                const LayoutWorkspace &w, const void *warm, int64_t warm_bytes, hipStream_t stream) {
  const int64_t tiles = layout_tiles(a_total);
  const size_t lds = sizeof(int32_t) * (size_t)(kScanWaves + 2) * (e + 1);
  const int64_t warm_vecs = warm ? (warm_bytes < kWarmMaxBytes ? warm_bytes : kWarmMaxBytes) / 16 : 0;
  const int64_t per_block = (int64_t)kScanThreads * kWarmLoads;
  const int64_t warm_blocks = warm_vecs > 0 ? std::min<int64_t>(kWarmBlocks, (warm_vecs + per_block - 1) / per_block) : 0;
#define MOE_SCAN(B)                                                                                                  \
  hipLaunchKernelGGL(layout_scan<B>, dim3((unsigned)(tiles + warm_blocks)), dim3(kScanThreads), lds, stream,        \
                     topk_idx, a_total, tiles, e, capacity, row_align > 1 ? row_align : 1, rows, w.hdr, w.status,     \
                     ordinal, tokens_per_expert, expert_offsets, counters, w.full_off,                                \
                     static_cast<const u32x4 *>(warm), warm_vecs)
  if (e <= 16) MOE_SCAN(4);
  else if (e <= 64) MOE_SCAN(6);
  else if (e <= 256) MOE_SCAN(8);
  else MOE_SCAN(10);  // E <= 1024
#undef MOE_SCAN
  return hipGetLastError();
}

}  // namespace

hipError_t clear_layout_header(void *workspace, hipStream_t stream) {
  hipLaunchKernelGGL(fill_u32, dim3(1), dim3(64), 0, stream, static_cast<uint32_t *>(workspace),
                     (int64_t)(kHeaderBytes / 4), 0u);
  return hipGetLastError();
}

hipError_t launch_layout_scan(const int32_t *topk_idx, int64_t n, int k, int e, int capacity, int row_align,
                              int64_t rows, int32_t *tokens_per_expert, int32_t *expert_offsets, int32_t *ordinal,
                              int32_t *counters, void *workspace, const void *warm, int64_t warm_bytes,
                              hipStream_t stream) {
  const int64_t a_total = n * k;
  return scan(topk_idx, a_total, e, capacity, row_align, rows, tokens_per_expert, expert_offsets, ordinal, counters,
              carve(workspace, a_total, e, false), warm, warm_bytes, stream);
}

hipError_t launch_layout(const int32_t *topk_idx, const float *topk_w, int64_t n, int k, int e, int capacity,
                         int row_align, bool drop_by_weight, int64_t rows, int32_t *tokens_per_expert,
                         int32_t *expert_offsets, int32_t *ordinal, int32_t *assign_row, int32_t *row_src,
                         uint8_t *drop_mask, uint8_t *pad_mask, int32_t *counters, float *w_perm, void *workspace,
                         const void *warm, int64_t warm_bytes, hipStream_t stream) {
  const int64_t a_total = n * k;
  const bool by_weight = drop_by_weight && capacity > 0;
  const LayoutWorkspace w = carve(workspace, a_total, e, by_weight);
  hipError_t st = scan(topk_idx, a_total, e, capacity, row_align, rows, tokens_per_expert, expert_offsets, ordinal,
                       counters, w, warm, warm_bytes, stream);
  if (st != hipSuccess) return st;
  const PlaceArgs p = place_args(topk_idx, topk_w, ordinal, tokens_per_expert, expert_offsets, e, capacity,
                                 row_align, rows, assign_row, drop_mask, row_src, pad_mask, w_perm, workspace,
                                 counters);
  const int64_t assign_blocks = (a_total + 255) / 256;
  int64_t row_blocks = (rows + 255) / 256;
  if (row_blocks > 256) row_blocks = 256;
  if (row_blocks < 1) row_blocks = 1;  // at least one block: it resets the scan header
  hipLaunchKernelGGL(layout_finish, dim3((unsigned)(assign_blocks + row_blocks)), dim3(256), 0, stream, p, a_total,
                     assign_blocks, by_weight ? w.full_list : nullptr, by_weight ? w.full_off : nullptr);
  if ((st = hipGetLastError()) != hipSuccess) return st;
  if (!by_weight) return hipSuccess;
  hipLaunchKernelGGL(capacity_select_kernel, dim3((unsigned)e), dim3(kSelectThreads),
                     sizeof(uint32_t) * kSelectLdsKeys, stream, w.full_list, w.full_off, topk_w, a_total, capacity, assign_row,
                     drop_mask, row_src, pad_mask, w_perm);
  return hipGetLastError();
}

}  // namespace moe
