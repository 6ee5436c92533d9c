// Expert FFN in bf16: the forward (grouped SwiGLU GEMM1, then GEMM2) and the
// backward (dA and dX through the grouped GEMM with K-major weights, the
// SwiGLU backward, and the weight-gradient kernels below).  The grouped GEMM
// kernel itself is in moe_gemm.hpp.
#include "moe_gemm.hpp"

namespace moe {
namespace {

// ------------------------------------------------------------------ weight gradients

// The weight gradients C_e [M, N] = A_e^T B_e reduce over the rows of expert
// e's segment: K is the expert's row count (about 512 in a 128-expert layer of
// 65536 rows), so a 256 x 256 output tile has only a handful of K steps.
//
// Operand layouts.  One operand of each gradient is an input stored with its
// features contiguous (grad_y for dW_down, x_perm for dW_gate_up): K-major,
// read through the LDS transpose loads.  The other is made by the SwiGLU
// backward, which also writes it expert-major with K contiguous ("K-major
// copies" below): expert e's part is [features][kp_e] at element offset
// features * poff_e, where kp_e is the expert's row count rounded up to a
// multiple of 64 (zeros after the last row) and poff_e the sum of kp over the
// experts before e.  Measured on gfx950, a K step whose fragments all come
// through transpose loads takes about 1.5 times as long as one with half of
// them read as plain 16-byte rows.  The zero padding also makes the ragged last
// K step exact without masking: the K-major operand re-reads its last row
// there, which meets zeros.
//
// Work plan (a small kernel at the start of the backward).  A unit is a range
// of one expert's output tiles: the whole expert, or, when the expert holds
// more than 1/16 of all K steps, one of ceil(16 * steps / all steps) equal
// ranges.  Units are ranked by K steps per range, most first, and dealt to the
// 8 XCDs in snake order (0..7, 7..0, 0..7, ...), so each XCD works through
// whole experts or large parts of one: their operand panels are fetched into
// that XCD's L2 only.  Experts without rows are units too (their tiles are
// zero).  Each XCD's units form a list; a workgroup takes the next chain of
// tiles (kChain tiles of one unit, below) of its XCD's list (workgroup b runs
// on XCD b % 8 and takes chain b / 8), so the hardware's dispatch balances the
// chains over the XCD's CUs as they free up (simulated on the Zipf-loaded
// 32-expert layer with one tile per workgroup: the XCD finishing last ends 3 %
// after the mean; whole experts on fixed per-CU tile lists end 170 % after
// it).
// plan (int32): [0..8] first entry of each XCD's list; [9..16] and [17..24]
// chains of each XCD's list in dW_down and in dW_gate_up; [25] 64-row blocks
// of the K-major copies (poff_E / 64); entries of kEntryInts from kPlanEntries
// in XCD-list order: the unit (expert | part << 11 | parts << 21), the
// expert's rows, its segment start, its poff, its first chain in dW_down's
// list and in dW_gate_up's; poff_0 .. poff_E from kPlanPoff.
constexpr int kWgradDiv = 16;
constexpr int kMaxUnits = kMaxExperts + kWgradDiv;  // sum of ceil(16 steps_e / S) <= 16 + E
constexpr int kEntryInts = 8;
constexpr int kPlanEntries = 32;
constexpr int kPlanPoff = kPlanEntries + kEntryInts * kMaxUnits;
constexpr int kPlanInts = kPlanPoff + kMaxExperts + 16;
constexpr int kPlanThreads = 1024;
constexpr int kListLanes = 3;  // an XCD's list holds at most 3 * 64 entries
static_assert(kMaxExperts == kPlanThreads, "one plan thread per expert");
static_assert((kMaxUnits + kXcds - 1) / kXcds <= kListLanes * kWave, "an XCD's list fits the lookup");
static_assert(kMaxUnits <= 2 * kPlanThreads, "two units per plan thread");

// Tiles per workgroup: a workgroup runs a chain of kChain tiles of one unit
// one after the other (below).  Measured in one process against the kernel
// with one tile per workgroup (same output bits): both weight-gradient kernels
// 3 % faster at 512-row experts, the FFN backward 1.5 % faster on the
// Qwen3-like layer and 1.2 % on the Zipf-loaded 32-expert share.  Chains of 4
// made the kernels 5-6 % faster at 512-row experts but the share's backward
// 0.5 % slower than one tile per workgroup (its hot experts' tiles have about
// 160 K steps, so long chains leave the XCD's dispatcher coarse pieces to
// balance; chains of 8 were 26 % slower there).  A chain length chosen per
// expert from its K steps needs a grid sized for one tile per workgroup: the
// workgroups left without a chain each hold a CU (all of its LDS) while they
// start and exit, which cost that variant what its longer chains saved.
constexpr int kChain = 2;

// Upper bound of the workgroups of one XCD's list (the grid is 8 times that):
// at most ceil(units / 8) units, each of at most ceil(per_e / kChain) chains.
int64_t wgrad_list_bound(int e, int per_e) {
  return (int64_t)((e + kWgradDiv + kXcds - 1) / kXcds) * ((per_e + kChain - 1) / kChain);
}

// 64-row blocks of the K-major copies: at most one partial block per expert.
int64_t kmajor_blocks(int64_t rows, int e) { return rows / kBK + e + 1; }

// Tiles of part p of `parts` of an expert with per_e tiles.
__device__ __forceinline__ int part_tiles(int p, int parts, int per_e, int &first) {
  const int chunk = (per_e + parts - 1) / parts;
  first = p * chunk;
  const int last = first + chunk < per_e ? first + chunk : per_e;
  return last > first ? last - first : 0;
}

// Inclusive scan of v over the 1024-thread block (tmp: 16 LDS words); total out.
__device__ int block_scan(int v, int32_t *tmp, int &total) {
  const int l = lane_id(), wv = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (l >= off) incl += o;
  }
  if (l == kWave - 1) tmp[wv] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
  for (int i = 0; i < kPlanThreads / kWave; ++i) {
    base += i < wv ? tmp[i] : 0;
    total += tmp[i];
  }
  __syncthreads();
  return base + incl;
}

__global__ __launch_bounds__(kPlanThreads) void wgrad_plan_kernel(const int32_t *__restrict__ tokens_per_expert,
                                                                  const int32_t *__restrict__ expert_offsets, int e,
                                                                  int per_e_down, int per_e_gu,
                                                                  int32_t *__restrict__ plan,
                                                                  int32_t *__restrict__ block_expert) {
  __shared__ int32_t s_cost[kMaxUnits], s_unit[kMaxUnits], s_by_slot[kMaxUnits];
  __shared__ int32_t s_poff[kMaxExperts + 1];
  __shared__ int32_t tmp[kPlanThreads / kWave], count[kXcds], start[kXcds + 1];
  const int x = threadIdx.x, l = lane_id(), wv = x / kWave;
  const int rows = x < e ? tokens_per_expert[x] : 0;
  const int steps = (rows + kBK - 1) / kBK;
  int S = 0;
  const int s_incl = block_scan(steps, tmp, S);
  if (x < e) s_poff[x] = (s_incl - steps) * kBK;
  if (x == 0) s_poff[e] = S * kBK;
  if (x < kXcds) count[x] = 0;
  // the expert's parts and units
  const int parts = x >= e ? 0 : (rows > 0 ? ((steps * kWgradDiv + S - 1) / S > 1 ? (steps * kWgradDiv + S - 1) / S : 1)
                                           : 1);
  int U = 0;
  const int u_incl = block_scan(parts, tmp, U);
  for (int p = 0; p < parts; ++p) {
    const int u = u_incl - parts + p;
    s_unit[u] = x | (p << 11) | (parts << 21);
    const int64_t c = (((int64_t)2 * steps + 1) << 6) / parts;
    s_cost[u] = rows > 0 ? (int)(c < INT32_MAX ? c : INT32_MAX) : 0;
  }
  __syncthreads();
  // rank (most K steps per unit first, then unit order) and snake order
  int rank_of[2] = {0, 0}, xcd_of[2] = {0, 0};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = x + h * kPlanThreads;
    if (u < U) {
      const int c = s_cost[u];
      int r = 0;
      for (int v = 0; v < U; ++v) {
        const int cv = s_cost[v];
        r += (cv > c || (cv == c && v < u)) ? 1 : 0;
      }
      rank_of[h] = r;
      xcd_of[h] = ((r / kXcds) & 1) ? kXcds - 1 - r % kXcds : r % kXcds;
      atomicAdd(&count[xcd_of[h]], 1);
    }
  }
  __syncthreads();
  if (x == 0) {
    int s = 0;
    for (int i = 0; i < kXcds; ++i) {
      start[i] = s;
      s += count[i];
    }
    start[kXcds] = s;
  }
  __syncthreads();
  // each unit's entry (its rank r sits at position r / 8 of its XCD's list)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = x + h * kPlanThreads;
    if (u < U) {
      const int slot = start[xcd_of[h]] + rank_of[h] / kXcds;
      const int unit = s_unit[u], ex = unit & 2047;
      s_by_slot[slot] = unit;
      int32_t *en = plan + kPlanEntries + slot * kEntryInts;
      en[0] = unit;
      en[1] = tokens_per_expert[ex];
      en[2] = expert_offsets[ex];
      en[3] = s_poff[ex];
    }
  }
  if (x <= kXcds) plan[x] = start[x];
  if (x == kXcds + 1) plan[25] = S;
  if (x <= e) plan[kPlanPoff + x] = s_poff[x];
  __syncthreads();
  // first chain of every entry in its XCD's list, for both gradients: wave g
  // (0..7) scans list g for dW_down, wave 8 + g for dW_gate_up
  {
    const int g = wv % kXcds, gu = wv >= kXcds;
    const int per_e = gu ? per_e_gu : per_e_down;
    int carry = 0;
    for (int i0 = start[g]; i0 < start[g + 1]; i0 += kWave) {
      const int i = i0 + l;
      int nt = 0;
      if (i < start[g + 1]) {
        const int unit = s_by_slot[i];
        int first;
        nt = (part_tiles((unit >> 11) & 1023, unit >> 21, per_e, first) + kChain - 1) / kChain;
      }
      int incl = nt;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off, kWave);
        if (l >= off) incl += o;
      }
      if (i < start[g + 1]) plan[kPlanEntries + i * kEntryInts + 4 + gu] = carry + incl - nt;
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (l == 0) plan[9 + 8 * gu + g] = carry;
  }
  // the expert of each 64-row block: the last one whose first block is <= t
  for (int t = x; t < S; t += kPlanThreads) {
    int lo = 0, hi = e - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_poff[mid] <= t * kBK) lo = mid;
      else hi = mid - 1;
    }
    block_expert[t] = lo;
  }
}

// kAT: A is the K-major input and B the K-contiguous copy (dW_down = dy^T a);
// else A is the copy and B the input (dW_gate_up = [dG | dU]^T x).  kNFast: a
// unit's tiles run n-tile fastest (else m-tile fastest).  The workgroups of an
// XCD work on consecutive tiles side by side, so the faster index should be
// the operand with fewer tiles: each pass over it re-reads the smaller panel
// set.  `field`: which of the plan's two lists (0 dW_down, 1 dW_gate_up).
//
// Chains.  A unit of T tiles is covered by C = ceil(T / kChain) workgroups;
// workgroup c of the unit runs tiles c, c + C, c + 2C, ... (those below T) one
// after the other.  Every tile of the unit has the same K extent, so the load
// ring runs on across the tile boundary: the next tile's first two K steps are
// loaded during the current tile's last two, and the current tile's epilogue
// stages its output through the one ring slot that no load in flight targets.
// A chain pays the tile lookup, the wait for the first loads and the
// workgroup's launch once; the epilogue stays per tile (timing copies at
// 512-row experts: without its global stores each kernel ran 8 % faster,
// without its LDS staging 4-7 %).  The workgroups of an XCD still run
// consecutive tile numbers side by side, as without chains: first tiles
// c .. c+31 of the unit, then c+C .. c+C+31.
template <bool kNFast, bool kAT>
__global__ __launch_bounds__(kThreads, 1) void wgrad_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int M, int N, int m_tiles, int n_tiles, int field,
    const int32_t *__restrict__ plan, uint16_t *__restrict__ C, uint16_t *__restrict__ C_rep, int e_master) {
  constexpr bool kBT = !kAT;
  __shared__ __attribute__((aligned(1024))) char ring[kSlots * kOperandBytes];
  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = w >> 1, wn = w & 1;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  if (slot >= plan[9 + 8 * field + xcd]) return;

  // the entry of this chain: the last one of the XCD's list whose first chain
  // is <= slot, found by one ballot per 64 entries over all of them at once
  const int base = plan[xcd], n_ent = plan[xcd + 1] - base;
  const int32_t *ent = plan + kPlanEntries;
  int v_unit[kListLanes], v_rows[kListLanes], v_r0[kListLanes], v_poff[kListLanes], v_first[kListLanes];
  uint64_t hit[kListLanes];
#pragma unroll
  for (int h = 0; h < kListLanes; ++h) {
    const int i = h * kWave + l;
    const int32_t *en = ent + (int64_t)(base + (i < n_ent ? i : 0)) * kEntryInts;
    v_unit[h] = en[0];
    v_rows[h] = en[1];
    v_r0[h] = en[2];
    v_poff[h] = en[3];
    v_first[h] = en[4 + field];
    hit[h] = __ballot(i < n_ent && v_first[h] <= slot);
  }
  const int hsel = hit[2] ? 2 : (hit[1] ? 1 : 0);
  const uint64_t hm = hit[hsel];
  const int src = 63 - __builtin_clzll(hm);  // hm is not empty: the first entry starts at chain 0
  auto pick = [&](const int (&v)[kListLanes]) {
    const int a = __builtin_amdgcn_readlane(v[0], src), b = __builtin_amdgcn_readlane(v[1], src),
              c = __builtin_amdgcn_readlane(v[2], src);
    return hsel == 2 ? c : (hsel == 1 ? b : a);
  };
  const int unit = pick(v_unit), k_len = pick(v_rows), r0 = pick(v_r0), poff = pick(v_poff),
            first_slot = pick(v_first);
  const int x = unit & 2047;
  int first;
  const int unit_tiles = part_tiles((unit >> 11) & 1023, unit >> 21, m_tiles * n_tiles, first);
  const int KT = (k_len + kBK - 1) / kBK;
  const int chains = (unit_tiles + kChain - 1) / kChain;
  const int chain = slot - first_slot;
  // tiles of this chain: chain + i * chains for i < n_in (at least one)
  const int n_in = (unit_tiles - chain + chains - 1) / chains < kChain ? (unit_tiles - chain + chains - 1) / chains
                                                                       : kChain;
  auto tile_m0 = [&](int i) {
    const int loc = first + chain + i * chains;
    return (kNFast ? loc / n_tiles : loc % m_tiles) * kBM;
  };
  auto tile_n0 = [&](int i) {
    const int loc = first + chain + i * chains;
    return (kNFast ? loc % n_tiles : loc / m_tiles) * kBN;
  };
  uint16_t *cb = x < e_master ? C + (int64_t)x * M * N : C_rep + (int64_t)(x - e_master) * M * N;

  // Direct loads.  The K-major input: row k of a step holds 256 columns in 512
  // bytes; this wave fills rows w*16 .. w*16+15, two per instruction: lane l
  // fills row k = w*16 + 2i + l/32, 16-byte position l % 32 with chunk
  // position ^ swz_t(k); columns past the operand's end re-read its last
  // chunk, rows past the K extent its last row.  The K-contiguous copy: tile
  // row r (an output row or column) holds K step kt in 128 bytes; this wave
  // fills rows w*64 .. w*64+63, 8 per instruction: lane l fills row
  // w*64 + 8i + l/8, position l % 8 with chunk position ^ swz(r); rows past the
  // operand's end re-read its last row.  The offsets depend on the tile only
  // through those clamps at the matrix edges; they are set for the tile whose
  // K steps are being loaded (start_tile below).
  uint32_t a_off[kLoads], b_off[kLoads];
  const uint32_t kp2 = (uint32_t)KT * (uint32_t)kRowBytes;  // bytes per row of the copy
  auto set_offsets = [&](int m0_, int n0_) {
    const int rows_valid = M - m0_ < kBM ? M - m0_ : kBM;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int k = w * 16 + 2 * i + l / 32;
      const int ct8 = ((l % 32) ^ swz_t(k)) * 8;
      const int r = w * 64 + i * kLoadRows + l / kChunks;
      const uint32_t cc = (uint32_t)(((l % kChunks) ^ swz(r)) * 16);
      if constexpr (kAT) {
        a_off[i] = (uint32_t)(ct8 > rows_valid - 8 ? rows_valid - 8 : ct8) * 2u;
        b_off[i] = (uint32_t)(r < N - n0_ ? r : N - n0_ - 1) * kp2 + cc;
      } else {
        a_off[i] = (uint32_t)(r < rows_valid ? r : rows_valid - 1) * kp2 + cc;
        b_off[i] = (uint32_t)(ct8 > N - n0_ - 8 ? N - n0_ - 8 : ct8) * 2u;
      }
    }
  };
  // The load stream: the sources of the A and B tiles of the K step whose
  // loads are issued next, and that step's last valid K row (the K-major
  // operand clamps its rows to it), kept as running values so that a step
  // costs a few scalar adds (recomputing them from the tile and step numbers
  // put about 200 scalar instructions into every step, among the MFMAs).
  const char *ld_a, *ld_b;
  int ld_last;
  auto start_tile = [&](int i) {
    const int m0_ = tile_m0(i), n0_ = tile_n0(i);
    set_offsets(m0_, n0_);
    if constexpr (kAT) {
      ld_a = reinterpret_cast<const char *>(A + (int64_t)r0 * M + m0_);
      ld_b = reinterpret_cast<const char *>(B + (int64_t)N * poff + (int64_t)n0_ * KT * kBK);
    } else {
      ld_a = reinterpret_cast<const char *>(A + (int64_t)M * poff + (int64_t)m0_ * KT * kBK);
      ld_b = reinterpret_cast<const char *>(B + (int64_t)r0 * N + n0_);
    }
    ld_last = k_len - 1;
  };
  // bytes between consecutive K steps of the two operands
  const int64_t a_step = kAT ? (int64_t)kBK * M * 2 : (int64_t)kRowBytes;
  const int64_t b_step = kAT ? (int64_t)kRowBytes : (int64_t)kBK * N * 2;
  start_tile(0);
  const uint32_t ring_lds = lds_address(ring) + w * 64 * kRowBytes;  // = w * 16 * kTRowBytes
  auto load_a = [&](int slot_, int i) {
    const uint32_t dst = ring_lds + slot_ * kOperandBytes + i * 1024;
    if constexpr (kAT) {
      const int k = w * 16 + 2 * i + l / 32;
      dma16(ld_a, a_off[i] + (uint32_t)(k < ld_last ? k : ld_last) * (uint32_t)M * 2u, dst);
    } else {
      dma16(ld_a, a_off[i], dst);
    }
  };
  auto load_b = [&](int slot_, int i) {
    const uint32_t dst = ring_lds + slot_ * kOperandBytes + i * 1024;
    if constexpr (kBT) {
      const int k = w * 16 + 2 * i + l / 32;
      dma16(ld_b, b_off[i] + (uint32_t)(k < ld_last ? k : ld_last) * (uint32_t)N * 2u, dst);
    } else {
      dma16(ld_b, b_off[i], dst);
    }
  };
  uint32_t ta[4][2], tb[4][2];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ta[q][h] = kAT ? tr_off(l, 2 * q + wm, h) : 0u;
      tb[q][h] = kBT ? tr_off(l, 4 * wn + q, h) : 0u;
    }
  constexpr int kReads = 12;

  f32x16 acc[4][4];
  auto zero_acc = [&]() {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.0f;
  };

  // Epilogue of tile (m0, n0): each wave converts its 128 x 128 sub-tile to
  // bf16 and writes it out in four rounds of one 32-row block through its own
  // 8 KiB of `stage_slot` (16-byte chunks XOR-swizzled by row), as whole
  // 256-byte rows of 16-byte stores.  No load in flight targets that slot and
  // no wave still reads it.  The stores are non-temporal: the gradients (as
  // many bytes as the kernel reads) are not read again here, and streaming
  // them past the L2 leaves the operand panels there (dW_gate_up 2 % faster,
  // the backward 0.3-0.6 %, in one process against plain stores).
  auto epilogue = [&](int m0, int n0, char *stage_slot) __attribute__((always_inline)) {
    char *stage = stage_slot + w * (kOperandBytes / 4);
    const int rows_valid = M - m0 < kBM ? M - m0 : kBM;
    const bool whole = rows_valid == kBM && n0 + kBN <= N;
    const int ch = l % 16, col = n0 + wn * 128 + ch * 8;
    const int rr = l & 31;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16 &c = acc[mi][ni];
          const int f = ni * 32 + 8 * g + 4 * (l >> 5);
          *reinterpret_cast<uint2 *>(stage + rr * 256 + ((f >> 3) ^ (rr & 15)) * 16 + (f & 7) * 2) =
              make_uint2(pack_bf16x2(c[4 * g], c[4 * g + 1]), pack_bf16x2(c[4 * g + 2], c[4 * g + 3]));
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
      __builtin_amdgcn_wave_barrier();
      // all eight reads first, then the stores; a whole tile stores unconditionally
      u32x4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = l / 16 + 4 * q;
        v[q] = *reinterpret_cast<const u32x4 *>(stage + r * 256 + (ch ^ (r & 15)) * 16);
      }
      uint16_t *c_blk = cb + (int64_t)(m0 + (2 * mi + wm) * 32 + l / 16) * N + col;
      if (whole) {
#pragma unroll
        for (int q = 0; q < 8; ++q) st16_stream(c_blk + (int64_t)(4 * q) * N, v[q]);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int row = m0 + (2 * mi + wm) * 32 + l / 16 + 4 * q;
          if (row < M && col < N) st16_stream(c_blk + (int64_t)(4 * q) * N, v[q]);
        }
      }
    }
  };

  // K loop, as the grouped GEMM's, over the chain's n_in * KT steps: step s's
  // B and A tiles in slots sb, sa; slices 0 and 1 load step s+2's B tile into
  // slot pb, slice 3 its A tile into slot sb; after slice 2 every wave waits
  // for step s+1's tiles and passes a barrier.  (lt, lk) is the tile and K
  // step whose loads are issued next; (ct, ck) those of the MFMAs.  After the
  // last step of a tile its epilogue stages through slot sa, which holds only
  // that step's A tile, already read; a barrier then keeps step s+1's loads
  // into that slot (its pb) behind every wave's staging reads.
  const int total = n_in * KT;
  int lt = 0, lk = 0;
  auto advance = [&]() {
    if (++lk == KT) {
      lk = 0;
      if (++lt < n_in) start_tile(lt);
    } else {
      ld_a += a_step;
      ld_b += b_step;
      ld_last -= kBK;
    }
  };
  bf16x8 fa[2][4], fb[2][4];
  if (total > 0) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load_b(0, i);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load_a(1, i);
    advance();
    if (total > 1) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) load_b(2, i);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) load_a(3, i);
      advance();
      wait_vmcnt<2 * kLoads>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    load_frags<false, kAT, kBT>(ring + kOperandBytes, ring, 0, wm, wn, l, fa[0], fb[0], ta, tb);
    __builtin_amdgcn_sched_barrier(0);
  }
  int sb = 0, sa = 1;
  for (int ct = 0; ct < n_in; ++ct) {
    zero_acc();
    for (int ck = 0; ck < KT; ++ck) {
      const int nb = sb + 2 < kSlots ? sb + 2 : sb + 2 - kSlots;
      const int na = sa + 2 < kSlots ? sa + 2 : sa + 2 - kSlots;
      const int pb = na + 1 < kSlots ? na + 1 : na + 1 - kSlots;
      const bool ahead = ct * KT + ck + 2 < total;
      const char *as = ring + sa * kOperandBytes;
      const char *bs = ring + sb * kOperandBytes;
      load_frags<false, kAT, kBT>(as, bs, 1, wm, wn, l, fa[1], fb[1], ta, tb);
      slice<4, kReads>(fa[0], fb[0], acc, [&](int d) {
        if (ahead) load_b(pb, d);
      });
      load_frags<false, kAT, kBT>(as, bs, 2, wm, wn, l, fa[0], fb[0], ta, tb);
      slice<4, kReads>(fa[1], fb[1], acc, [&](int d) {
        if (ahead) load_b(pb, 4 + d);
      });
      load_frags<false, kAT, kBT>(as, bs, 3, wm, wn, l, fa[1], fb[1], ta, tb);
      slice<4, kReads>(fa[0], fb[0], acc, [&](int) {});
      if (ahead) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // step s+1's first fragments (after the last step: stale, unused)
      load_frags<false, kAT, kBT>(ring + na * kOperandBytes, ring + nb * kOperandBytes, 0, wm, wn, l, fa[0], fb[0],
                                  ta, tb);
      slice<4, kReads>(fa[1], fb[1], acc, [&](int d) {
        if (ahead) {
          load_a(sb, 2 * d);
          load_a(sb, 2 * d + 1);
        }
      });
      __builtin_amdgcn_sched_barrier(0);
      if (ahead) advance();
      sb = nb;
      sa = na;
    }
    // the last step's A slot, two behind the current one (an expert without
    // rows has no step: any slot)
    epilogue(tile_m0(ct), tile_n0(ct), ring + (sa + kSlots - 2) % kSlots * kOperandBytes);
    if (ct + 1 < n_in) {
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ------------------------------------------------------------------ backward

// SwiGLU backward, one 64-row block of an expert's padded K extent and up to
// kSwFeatures features per workgroup (blockIdx.y), 64 features at a time.  For row r and feature i, with
// g = gu[r, i], u = gu[r, I+i], da = d_act[r, i], s = sigmoid(g):
//   dgu[r, i]     = bf16(da * u * s * (1 + g * (1 - s)))   (silu'(g) = s (1 + g (1 - s)))
//   dgu[r, I + i] = bf16(da * g * s)
//   a[r, i]       = bf16(g * s * u)                         (the activation itself)
// fp32 arithmetic.  dgu is written [rows, 2I] (for dx); every element is read
// and written by the same thread, so dgu may be gu (in place).  a and
// [dG | dU] also go to the K-major copies aT ([I][kp_e] per expert) and gT
// ([2I][kp_e]) that the weight gradients read, with zeros at the padded K
// positions.  The transposition goes through LDS: a thread holds two rows x 8
// features and writes each feature's pair of values as one 32-bit word of the
// feature's 128-byte LDS row, word k/2 at position k/2 ^ 4*(feature/8) (the 32
// lanes of each half-wave then hit 32 distinct banks); each thread then reads
// 16 K values of one feature as two 16-byte reads and stores them.
constexpr int kSwThreads = 256;
constexpr int kSwFeatures = 256;
__global__ __launch_bounds__(kSwThreads) void swiglu_bwd_kernel(
    const uint16_t *gu, uint16_t *dgu, const uint16_t *__restrict__ d_act, int inter,
    const int32_t *__restrict__ tokens_per_expert, const int32_t *__restrict__ expert_offsets,
    const int32_t *__restrict__ plan, const int32_t *__restrict__ block_expert, uint16_t *__restrict__ aT,
    uint16_t *__restrict__ gT) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[3][64 * 32];  // a, dG, dU: [feature][k/2] words
  const int b = blockIdx.x;
  if (b >= plan[25]) return;
  const int x = block_expert[b];
  const int rows_x = tokens_per_expert[x];
  const int64_t kp = (int64_t)((rows_x + kBK - 1) / kBK) * kBK;
  const int64_t poff = plan[kPlanPoff + x];
  const int kb = b * kBK - (int)poff;  // the block's first K position inside the expert
  const int valid = rows_x - kb < kBK ? rows_x - kb : kBK;
  const int64_t r0 = (int64_t)expert_offsets[x] + kb;
  const int t = threadIdx.x;
  const int kpair = t / 8, fg = t % 8;  // rows 2*kpair, 2*kpair+1 of the block; features fg*8 .. fg*8+7
  const int tf = t / 4, tq = t % 4;     // transposed: feature tf, K positions 16*tq .. 16*tq+15
  const int swz_w = 4 * fg, swz_r = 4 * (tf / 8);
  uint16_t *a_row = aT + (int64_t)inter * poff + (int64_t)tf * kp + kb + 16 * tq;
  uint16_t *g_row = gT + (int64_t)2 * inter * poff + (int64_t)tf * kp + kb + 16 * tq;
  const int f_end = (int)blockIdx.y * kSwFeatures + kSwFeatures < inter ? (int)blockIdx.y * kSwFeatures + kSwFeatures
                                                                          : inter;
  for (int f0 = (int)blockIdx.y * kSwFeatures; f0 < f_end; f0 += 64) {
    uint32_t wa[8], wg[8], wu[8];  // per feature: the two rows' bf16 values, row 2*kpair low
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 2 * kpair + h;
      float dg[8], du[8], a[8];
      if (k < valid) {
        const int64_t r = r0 + k;
        const uint16_t *pg = gu + r * 2 * inter + f0 + fg * 8;
        float g[8], u[8], da[8];
        Vec16<true>::unpack(ld16(pg), g);
        Vec16<true>::unpack(ld16(pg + inter), u);
        Vec16<true>::unpack(ld16(d_act + r * inter + f0 + fg * 8), da);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float sg = 1.0f / (1.0f + __expf(-g[i]));
          const float gs = g[i] * sg;
          dg[i] = da[i] * u[i] * (sg * (1.0f + g[i] * (1.0f - sg)));
          du[i] = da[i] * gs;
          a[i] = gs * u[i];
        }
        uint16_t *qg = dgu + r * 2 * inter + f0 + fg * 8;
        st16(qg, Vec16<true>::pack(dg));
        st16(qg + inter, Vec16<true>::pack(du));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) dg[i] = du[i] = a[i] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t sh = 16 * h;
        const uint32_t ba = bf16_bits(a[i]), bg = bf16_bits(dg[i]), bu = bf16_bits(du[i]);
        wa[i] = h ? (wa[i] | (ba << sh)) : ba;
        wg[i] = h ? (wg[i] | (bg << sh)) : bg;
        wu[i] = h ? (wu[i] | (bu << sh)) : bu;
      }
    }
    __syncthreads();  // the previous feature block's transposed reads are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int wi = (fg * 8 + i) * 32 + (kpair ^ swz_w);
      tile[0][wi] = wa[i];
      tile[1][wi] = wg[i];
      tile[2][wi] = wu[i];
    }
    __syncthreads();
    const int w0 = tf * 32 + ((8 * tq) ^ swz_r), w1 = tf * 32 + ((8 * tq + 4) ^ swz_r);
    const int64_t fo = (int64_t)f0 * kp;
    st16(a_row + fo, *reinterpret_cast<const u32x4 *>(&tile[0][w0]));
    st16(a_row + fo + 8, *reinterpret_cast<const u32x4 *>(&tile[0][w1]));
    st16(g_row + fo, *reinterpret_cast<const u32x4 *>(&tile[1][w0]));
    st16(g_row + fo + 8, *reinterpret_cast<const u32x4 *>(&tile[1][w1]));
    st16(g_row + fo + (int64_t)inter * kp, *reinterpret_cast<const u32x4 *>(&tile[2][w0]));
    st16(g_row + fo + (int64_t)inter * kp + 8, *reinterpret_cast<const u32x4 *>(&tile[2][w1]));
  }
}

// Grouped GEMM over the expert segments, C [rows, N] = A [rows, K] B_e^T with
// B_e [N, K] (kBT false) or B_e [K, N] (kBT true).
template <bool kBT>
hipError_t launch_plain(const uint16_t *A, const uint16_t *B, const uint16_t *B_rep, int e_master, int64_t b_stride,
                        int K, int N, int64_t rows, int e, int capacity, const int32_t *tokens_per_expert,
                        const int32_t *expert_offsets, uint16_t *C, hipStream_t stream) {
  const int nt = (N + kBN - 1) / kBN;
  const int64_t g = tile_bound(rows, e, capacity, nt);
  if (g > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((grouped_gemm_kernel<kModePlain, kBT>), dim3((unsigned)g), dim3(kThreads), 0, stream, A, B,
                     b_stride, K, N, nt, tokens_per_expert, expert_offsets, e, C, (int64_t)N, nullptr, B_rep, e_master,
                     nullptr, nullptr, nullptr);
  return hipGetLastError();
}

// Weight-gradient GEMM: C_e [M, N] = A_e^T B_e for every expert over the rows of
// its segment, on the work plan `plan` (wgrad_plan_kernel over the same row
// counts; `field` 0 for dW_down, 1 for dW_gate_up).  kAT: A is the K-major
// input [rows, M] and B the K-contiguous copy ([N][kp_e] per expert); else A
// is the copy ([M][kp_e]) and B the input [rows, N].
template <bool kAT>
hipError_t launch_wgrad(const uint16_t *A, const uint16_t *B, int M, int N, int e, int field, const int32_t *plan,
                        uint16_t *C, uint16_t *C_rep, int e_master, hipStream_t stream) {
  const int mt = (M + kBM - 1) / kBM, nt = (N + kBN - 1) / kBN;
  const int64_t g = kXcds * wgrad_list_bound(e, mt * nt);
  if (g > INT32_MAX) return hipErrorInvalidConfiguration;
  if (nt <= mt)
    hipLaunchKernelGGL((wgrad_kernel<true, kAT>), dim3((unsigned)g), dim3(kThreads), 0, stream, A, B, M, N, mt, nt,
                       field, plan, C, C_rep, e_master);
  else
    hipLaunchKernelGGL((wgrad_kernel<false, kAT>), dim3((unsigned)g), dim3(kThreads), 0, stream, A, B, M, N, mt, nt,
                       field, plan, C, C_rep, e_master);
  return hipGetLastError();
}

// Workspace of the backward, in order: [dG | dU] [rows, 2I] (holding the
// recomputed [G | U] before, when the forward did not store them); dA [rows,
// I]; the weight gradients' work plan; the expert of each 64-row block of the
// K-major copies; the K-major copies of the activation (I features) and of
// [dG | dU] (2I features), each over at most kmajor_blocks * 64 K positions.
struct BwdWorkspace {
  uint16_t *gu, *dact;
  int32_t *plan, *block_expert;
  uint16_t *aT, *gT;
};

BwdWorkspace carve_bwd(void *workspace, int64_t rows, int inter, int e, size_t *total) {
  const size_t kb = (size_t)kmajor_blocks(rows, e);
  const size_t sizes[6] = {align256(4 * (size_t)rows * inter), align256(2 * (size_t)rows * inter),
                           align256(4 * (size_t)kPlanInts), align256(4 * kb),
                           align256(2 * (size_t)inter * kb * kBK), align256(4 * (size_t)inter * kb * kBK)};
  char *p[6];
  size_t off = 0;
  for (int i = 0; i < 6; ++i) {
    p[i] = static_cast<char *>(workspace) + off;
    off += sizes[i];
  }
  if (total) *total = off;
  return {reinterpret_cast<uint16_t *>(p[0]), reinterpret_cast<uint16_t *>(p[1]), reinterpret_cast<int32_t *>(p[2]),
          reinterpret_cast<int32_t *>(p[3]), reinterpret_cast<uint16_t *>(p[4]), reinterpret_cast<uint16_t *>(p[5])};
}

}  // namespace

size_t ffn_bwd_workspace_bytes(int64_t rows, int inter, int e) {
  size_t total = 0;
  carve_bwd(nullptr, rows, inter, e, &total);
  return total;
}

hipError_t launch_expert_ffn_bwd(const uint16_t *x_perm, const uint16_t *grad_y, int64_t rows, int64_t hidden,
                                 int inter, int e, int capacity, const int32_t *tokens_per_expert,
                                 const int32_t *expert_offsets, const uint16_t *w_gate_up, const uint16_t *w_down,
                                 const uint16_t *gate_up, uint16_t *grad_x_perm, uint16_t *grad_w_gate_up,
                                 uint16_t *grad_w_down, const ReplicaBases *rep, void *workspace,
                                 hipStream_t stream) {
  const int em = rep ? rep->e_master : e;
  const uint16_t *wgu_r = rep ? rep->w_gate_up : nullptr, *wd_r = rep ? rep->w_down : nullptr;
  uint16_t *gwgu_r = rep ? rep->grad_w_gate_up : nullptr, *gwd_r = rep ? rep->grad_w_down : nullptr;
  if (e < 1 || e > kMaxExperts) return hipErrorInvalidValue;
  const BwdWorkspace ws = carve_bwd(workspace, rows, inter, e, nullptr);
  const int H = (int)hidden, I = inter;
  hipError_t st;
#define MOE_TRY(x)                    \
  if ((st = (x)) != hipSuccess) return st;
  // the weight gradients' work plan, the padded K extents and their blocks' experts
  const int t_down = ((H + kBM - 1) / kBM) * ((I + kBN - 1) / kBN);
  const int t_gu = ((2 * I + kBM - 1) / kBM) * ((H + kBN - 1) / kBN);
  hipLaunchKernelGGL(wgrad_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, tokens_per_expert, expert_offsets, e,
                     t_down, t_gu, ws.plan, ws.block_expert);
  MOE_TRY(hipGetLastError());
  if (rows > 0) {
    // [G | U] = x W_gate_up^T unless saved by the forward; dA = dy W_down (W_down [H, I]: K-major)
    if (!gate_up)
      MOE_TRY(launch_plain<false>(x_perm, w_gate_up, wgu_r, em, (int64_t)2 * I * H, H, 2 * I, rows, e, capacity,
                                  tokens_per_expert, expert_offsets, ws.gu, stream));
    MOE_TRY(launch_plain<true>(grad_y, w_down, wd_r, em, (int64_t)I * H, H, I, rows, e, capacity, tokens_per_expert,
                               expert_offsets, ws.dact, stream));
    // [dG | dU] (in place of the recomputed [G | U]) and the K-major copies of a and [dG | dU]
    hipLaunchKernelGGL(swiglu_bwd_kernel,
                       dim3((unsigned)kmajor_blocks(rows, e), (unsigned)((I + kSwFeatures - 1) / kSwFeatures)),
                       dim3(kSwThreads), 0, stream,
                       gate_up ? gate_up : ws.gu, ws.gu, ws.dact, I, tokens_per_expert, expert_offsets, ws.plan,
                       ws.block_expert, ws.aT, ws.gT);
    MOE_TRY(hipGetLastError());
    // dx = [dG | dU] W_gate_up (W_gate_up [2I, H]: K-major)
    MOE_TRY(launch_plain<true>(ws.gu, w_gate_up, wgu_r, em, (int64_t)H * 2 * I, 2 * I, H, rows, e, capacity,
                               tokens_per_expert, expert_offsets, grad_x_perm, stream));
  }
  // dW_down_e = dy_e^T a_e;  [dW_gate; dW_up]_e = [dG | dU]_e^T x_e  (experts without rows: zeros)
  MOE_TRY(launch_wgrad<true>(grad_y, ws.aT, H, I, e, 0, ws.plan, grad_w_down, gwd_r, em, stream));
  MOE_TRY(launch_wgrad<false>(ws.gT, x_perm, 2 * I, H, e, 1, ws.plan, grad_w_gate_up, gwgu_r, em, stream));
#undef MOE_TRY
  return hipSuccess;
}

size_t ffn_workspace_bytes(int64_t rows, int inter) { return align256(sizeof(uint16_t) * (size_t)rows * (size_t)inter); }

hipError_t launch_expert_ffn(const uint16_t *x_perm, int64_t rows, int64_t hidden, int inter, int e, int capacity,
                             const int32_t *tokens_per_expert, const int32_t *expert_offsets,
                             const uint16_t *w_gate_up, const uint16_t *w_down, uint16_t *y, uint16_t *gate_up,
                             const ReplicaBases *rep, void *workspace, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int em = rep ? rep->e_master : e;
  uint16_t *act = static_cast<uint16_t *>(workspace);
  const int n1 = (inter + kBN / 2 - 1) / (kBN / 2);
  const int64_t g1 = tile_bound(rows, e, capacity, n1);
  const int64_t g2 = tile_bound(rows, e, capacity, (int)((hidden + kBN - 1) / kBN));
  if (g1 > INT32_MAX || g2 > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((grouped_gemm_kernel<kModeSwiGLU, false>), dim3((unsigned)g1), dim3(kThreads), 0, stream, x_perm,
                     w_gate_up, (int64_t)2 * inter * hidden, (int)hidden, inter, n1, tokens_per_expert, expert_offsets,
                     e, act, (int64_t)inter, gate_up, rep ? rep->w_gate_up : nullptr, em, nullptr, nullptr, nullptr);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  const int n2 = (int)((hidden + kBN - 1) / kBN);
  hipLaunchKernelGGL((grouped_gemm_kernel<kModePlain, false>), dim3((unsigned)g2), dim3(kThreads), 0, stream, act,
                     w_down, (int64_t)hidden * inter, inter, (int)hidden, n2, tokens_per_expert, expert_offsets, e, y,
                     hidden, nullptr, rep ? rep->w_down : nullptr, em, nullptr, nullptr, nullptr);
  return hipGetLastError();
}


}  // namespace moe
