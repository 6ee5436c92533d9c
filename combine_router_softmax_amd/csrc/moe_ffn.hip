// Grouped SwiGLU expert FFN on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// For expert e and the rows of its segment (expert_offsets[e] ..
// + tokens_per_expert[e]) of the expert-contiguous buffer:
//   GEMM1  [rows, H] x [H, 2I]: gate and up columns of the same index are
//          computed by the same workgroup, so the SwiGLU epilogue
//          a = bf16(silu(gate) * up) is applied in registers and only the [rows, I]
//          intermediate reaches memory.
//   GEMM2  [rows, I] x [I, H] -> y = bf16(acc).
// Both operands are K-contiguous (weights stored [out, in]), fp32 accumulation.
// ("Megatron MoE 实现": experts(dispatched_input, tokens_per_expert, ...); the
// grouped-GEMM paths of ROCm/Megatron-LM "Add MORI as a Token Dispatcher" and
// xtuner "Integrate UltraEP Runtime" take per-expert row counts; here the
// counts stay on the device: no host synchronisation.)
//
// Scheduling: the grid is an upper bound on the number of output tiles.  Every
// workgroup scans the per-expert tile counts (ceil(rows_e / BM) m-tiles times
// the n-tiles) in LDS and maps its id to (expert, n-tile, m-tile), m fastest,
// so the m-tiles that share a weight tile run side by side.  Ids are first
// remapped so that each of the 8 XCDs (workgroups are dealt to XCDs round-robin)
// receives one contiguous range of that order: weight and activation tiles are
// then re-read from the XCD's own L2.  Surplus workgroups exit at once.
//
// Tile: 256 rows x 256 columns (GEMM1: 128 gate + 128 up columns), 4 waves in
// a 2 x 2 arrangement of 128 x 128 sub-tiles (4 x 4 MFMA 32x32 blocks, 256 fp32
// accumulators per lane, held in AGPRs).  Operands go global -> LDS directly
// (global_load_lds_dwordx4, no register staging).  A K step is 64 wide, so every
// tile row of a step is one whole 128-byte line of the operand.  LDS holds a
// ring of five 32 KiB operand tiles (160 KiB): while one step's A and B tiles
// are read, the three other slots fill, 1.5 steps ahead.  A wave's load
// instruction fills 1 KiB (8 rows); each lane picks which 16-byte chunk of its
// row to fetch so that chunk c of row r lands at position c ^ swz(r), which
// keeps the MFMA fragment reads free of LDS bank conflicts.  Rows past the end
// of an expert's segment re-read its last row and are not stored.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;                          // K per step
constexpr int kRowBytes = kBK * 2;               // bytes of K per tile row: one 128-byte line
constexpr int kChunks = kRowBytes / 16;          // 16-byte chunks per tile row
constexpr int kLoadRows = 1024 / kRowBytes;      // tile rows one wave load instruction fills
constexpr int kLoads = kBM / kLoadRows / 4;      // load instructions per wave per operand tile
constexpr int kOperandBytes = kBM * kRowBytes;   // one operand tile of one K step: 32 KiB
constexpr int kSlots = 5;                        // ring of operand tiles
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kMaxExperts = 1024;
static_assert(kSlots * kOperandBytes <= 160 * 1024, "LDS budget");
static_assert(kLoads == 8, "load schedule below: 8 load instructions per wave per operand tile");

// LDS position of 16-byte chunk c of tile row r is c ^ swz(r).  A fragment
// read (ds_read_b128) has lane l read row l%32 of a 32-row block, chunk
// 2*slice + l/32.  Measured on gfx950, the permutation (r ^ r/4) % 8 of the
// eight chunks of a 128-byte row lets these reads run at the throughput of a
// linear 16-bytes-per-lane read; permuting by r % 8 alone, or by r/4 alone,
// reaches about 0.6 of it.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 2)) & 7; }

// Workgroup barrier for LDS: waits for this wave's LDS operations, then
// s_barrier; the memory clobber keeps the compiler from moving memory accesses
// across it.  Unlike __syncthreads() it does not wait for vector-memory loads.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 16 bytes per lane global -> LDS (global_load_lds_dwordx4): lane l reads
// base + off (base wave-uniform, in SGPRs; off a 32-bit per-lane byte offset)
// and its bytes land at LDS address lds_addr + 16*l (lds_addr is wave-uniform,
// passed in M0).  The instruction has no register result.  It is issued from
// inline asm so that the compiler's memory-counter bookkeeping does not see it:
// the compiler cannot tell which LDS stage such a load writes and would
// otherwise drain every load in flight before reading any stage; the K loop
// below waits for these loads itself with explicit vmcnt waits, and no other
// vector load is issued while they are in flight.  M0 is an input operand, so
// the compiler writes it and knows its value; the s_nop keeps one wait state
// between that write and the load that reads M0.
__device__ __forceinline__ void dma16(const void *base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"{m0}"(lds_addr), "v"(off), "s"(base) : "memory");
}

// LDS byte address of a pointer into a __shared__ array (the low 32 bits of its
// flat address).
__device__ __forceinline__ uint32_t lds_address(const void *p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }

// s_waitcnt on vector-memory operations only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct TileCoord {
  int e;
  int n_tile;
  int64_t row0;
  int64_t row_end;
};

// Maps blockIdx.x to an output tile; returns false for surplus workgroups.
// `scratch` (LDS) must hold kMaxExperts + kThreads int64 and is free again on
// return.
__device__ bool find_tile(const int32_t *__restrict__ tokens_per_expert, const int32_t *__restrict__ expert_offsets,
                          int e, int n_tiles, int64_t *scratch, TileCoord &tc) {
  constexpr int kPer = kMaxExperts / kThreads;  // experts per thread
  int64_t *part = scratch + kMaxExperts;
  const int tid = threadIdx.x;
  int64_t local[kPer];
  int64_t s = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int x = tid * kPer + i;
    const int64_t rows = x < e ? tokens_per_expert[x] : 0;
    local[i] = ((rows + kBM - 1) / kBM) * n_tiles;
    s += local[i];
  }
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int64_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int64_t run = part[tid] - s;  // exclusive prefix of this thread's experts
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    scratch[tid * kPer + i] = run;
    run += local[i];
  }
  const int64_t total = part[kThreads - 1];
  __syncthreads();

  const int64_t bid = blockIdx.x;
  const int64_t share = (total + kXcds - 1) / kXcds;
  const int64_t slot = bid / kXcds;
  const int64_t logical = (bid % kXcds) * share + slot;
  bool ok = slot < share && logical < total;
  if (ok) {
    int lo = 0, hi = e - 1;  // last expert whose first tile is <= logical
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (scratch[mid] <= logical) lo = mid;
      else hi = mid - 1;
    }
    const int64_t rows = tokens_per_expert[lo];
    const int64_t mt = (rows + kBM - 1) / kBM;
    const int64_t local_id = logical - scratch[lo];
    const int64_t m_tile = local_id % mt;
    tc.e = lo;
    tc.n_tile = (int)(local_id / mt);
    tc.row0 = expert_offsets[lo] + m_tile * kBM;
    tc.row_end = (int64_t)expert_offsets[lo] + rows;
  }
  __syncthreads();
  return ok;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ uint16_t bf16_bits(float v) { return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu); }

// Fragments of one 16-wide K slice ks from the A tile `as` and the B tile `bs`:
// A rows (2*mi + wm)*32 + l%32, B rows as below, k-chunk 2*ks + l/32.
template <bool kSwiGLU>
__device__ __forceinline__ void load_frags(const char *__restrict__ as, const char *__restrict__ bs, int ks, int wm,
                                           int wn, int l, bf16x8 (&a)[4], bf16x8 (&b)[4]) {
  const int r32 = l & 31;
  const int pos = ((2 * ks + (l >> 5)) ^ swz(r32)) * 16;  // every row read is r32 plus a multiple of 32
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    // SwiGLU: blocks 0,1 are gate columns wn*64 + ni*32, blocks 2,3 the matching up columns
    const int brow = kSwiGLU ? ((ni >> 1) * (kBN / 2) + wn * 64 + (ni & 1) * 32 + r32) : (wn * 128 + ni * 32 + r32);
    b[ni] = *reinterpret_cast<const bf16x8 *>(bs + brow * kRowBytes + pos);
  }
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
    a[mi] = *reinterpret_cast<const bf16x8 *>(as + ((2 * mi + wm) * 32 + r32) * kRowBytes + pos);
}

// MFMAs FIRST .. FIRST+COUNT-1 of one 16-wide K slice, numbered row block
// major (i = 4*mi + ni).  The weight fragment is the MFMA's first operand, so
// block (mi, ni) of the result holds, in lane l, activation row l%32 of the
// wave's row block mi and output features ni*32 + 8*(q/4) + 4*(l/32) + q%4 for
// accumulator element q: four consecutive features per group of four elements.
template <int FIRST, int COUNT>
__device__ __forceinline__ void mfma_range(const bf16x8 (&a)[4], const bf16x8 (&b)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = FIRST; i < FIRST + COUNT; ++i)
    acc[i / 4][i % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[i % 4], a[i / 4], acc[i / 4][i % 4], 0, 0, 0);
}

// The 4*MI MFMAs of one K slice for the wave's first MI row blocks.  The
// fragment reads of the following slice (issued just before, in the same
// scheduling region) are paired with the first half of the MFMAs; the slice's
// four direct-load instructions (dma(0..3)) sit between the MFMAs of the
// second half.  A run of load instructions would stall the wave -- and with it
// the matrix pipe -- while the address unit works through them; spread out,
// each load issues while the previous MFMAs run.
template <int MI, typename Dma>
__device__ __forceinline__ void slice(const bf16x8 (&a)[4], const bf16x8 (&b)[4], f32x16 (&acc)[4][4],
                                      Dma &&dma) {
  constexpr int kPart = MI / 2;                  // MFMAs between two load slots (MI = 1: none)
  constexpr int kHead = 4 * MI - 4 * kPart;      // MFMAs paired with the fragment reads
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  mfma_range<0, kHead>(a, b, acc);
#pragma unroll
  for (int i = 0; i < kHead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 8 / kHead, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  mfma_range<kHead, kPart>(a, b, acc);
  __builtin_amdgcn_sched_barrier(0);
  dma(0);
  __builtin_amdgcn_sched_barrier(0);
  mfma_range<kHead + kPart, kPart>(a, b, acc);
  __builtin_amdgcn_sched_barrier(0);
  dma(1);
  __builtin_amdgcn_sched_barrier(0);
  mfma_range<kHead + 2 * kPart, kPart>(a, b, acc);
  __builtin_amdgcn_sched_barrier(0);
  dma(2);
  __builtin_amdgcn_sched_barrier(0);
  mfma_range<kHead + 3 * kPart, kPart>(a, b, acc);
  __builtin_amdgcn_sched_barrier(0);
  dma(3);
  __builtin_amdgcn_sched_barrier(0);
}

// Modes of the grouped GEMM.  kModePlain: per expert segment, C = A B_e^T
// (y = act W_down^T; also the GEMMs of the backward with pre-transposed
// weights).  kModeSwiGLU: B tile rows 0..127 are gate rows n0.., rows 128..255
// the up rows I+n0..; output the [rows, I] SwiGLU intermediate.  kModeWGrad:
// per expert e, C_e [M, N] = A[:, seg_e] B[:, seg_e]^T, where A [M, ld] and B
// [N, ld] hold the experts' rows transposed, each expert's segment starting at
// seg_offp[e] and padded with zero columns to a multiple of 64 -- the weight
// gradients, the reduction running over the expert's rows.
constexpr int kModePlain = 0, kModeSwiGLU = 1, kModeWGrad = 2;

template <int kMode>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int64_t b_expert_stride, int K, int N,
    int n_tiles, const int32_t *__restrict__ tokens_per_expert, const int32_t *__restrict__ expert_offsets, int e,
    uint16_t *__restrict__ C, int64_t ldc, int M, int ld, const int32_t *__restrict__ seg_offp, int m_tiles) {
  constexpr bool kSwiGLU = kMode == kModeSwiGLU, kWGrad = kMode == kModeWGrad;
  // ring of operand tiles; also find_tile's scratch before the K loop and the
  // output staging after it
  __shared__ __attribute__((aligned(1024))) char ring[kSlots * kOperandBytes];

  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = w >> 1, wn = w & 1;
  // tile coordinates (the same in every lane: kept in scalar registers), the
  // operand bases and row stride, the K steps and the output base
  int te, n0, rows_valid, KT, n_lim;
  uint32_t lda;
  const char *a_base, *b_base;
  uint16_t *c_base;
  int64_t c_ld;
  if constexpr (kWGrad) {
    // each XCD (workgroup b runs on XCD b % 8) takes one eighth of every
    // expert's tiles, m fastest, expert after expert: the experts' different
    // row counts (the K of these GEMMs) load the XCDs evenly
    const int per_e = m_tiles * n_tiles, chunk = (per_e + kXcds - 1) / kXcds;
    const int slot = (int)blockIdx.x / kXcds;
    te = slot / chunk;
    const int local = ((int)blockIdx.x % kXcds) * chunk + slot % chunk;
    if (te >= e || local >= per_e) return;
    const int m0 = (local % m_tiles) * kBM;
    n0 = (local / m_tiles) * kBN;
    rows_valid = M - m0 < kBM ? M - m0 : kBM;
    const int koff = __builtin_amdgcn_readfirstlane(seg_offp[te]);
    KT = (__builtin_amdgcn_readfirstlane(seg_offp[te + 1]) - koff) / kBK;
    lda = (uint32_t)ld;
    a_base = reinterpret_cast<const char *>(A + (int64_t)m0 * ld + koff);
    b_base = reinterpret_cast<const char *>(B + (int64_t)n0 * ld + koff);
    c_ld = N;
    c_base = C + ((int64_t)te * M + m0) * N;
    n_lim = N - n0;
  } else {
    TileCoord tc;
    if (!find_tile(tokens_per_expert, expert_offsets, e, n_tiles, reinterpret_cast<int64_t *>(ring), tc)) return;
    te = __builtin_amdgcn_readfirstlane(tc.e);
    n0 = __builtin_amdgcn_readfirstlane(tc.n_tile) * (kSwiGLU ? kBN / 2 : kBN);
    const int64_t row0 = ((int64_t)__builtin_amdgcn_readfirstlane((int)(tc.row0 >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)tc.row0);
    rows_valid = __builtin_amdgcn_readfirstlane((int)(tc.row_end - tc.row0 < kBM ? tc.row_end - tc.row0 : kBM));
    KT = K / kBK;
    lda = (uint32_t)K;
    a_base = reinterpret_cast<const char *>(A + row0 * K);
    b_base = reinterpret_cast<const char *>(B + (int64_t)te * b_expert_stride);
    c_ld = ldc;
    c_base = C + row0 * ldc;
    n_lim = N;
  }

  // the tile's 32-row blocks 0..7 alternate between the two row groups of waves
  // (block 2*mi + wm is this wave's block mi); count this wave's blocks that
  // hold rows of the segment
  const int blocks_valid = (rows_valid + 31) / 32;
  const int mi_count = blocks_valid > wm ? (blocks_valid - wm + 1) / 2 : 0;

  // direct-load sources: this wave fills tile rows w*64 .. w*64+63 of each
  // operand tile, kLoadRows rows per instruction; lane l writes LDS bytes
  // l*16..l*16+15 of the instruction's 1 KiB, i.e. row l / kChunks, position
  // l % kChunks, so it fetches global chunk position ^ swz(row).  Addresses are
  // a per-tile scalar base plus a 32-bit per-lane byte offset.
  uint32_t a_off[kLoads], b_off[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = w * 64 + i * kLoadRows + l / kChunks;
    const int c = (l % kChunks) ^ swz(r);
    const int ar = r < rows_valid ? r : rows_valid - 1;  // ragged tail: re-read the last row
    a_off[i] = ((uint32_t)ar * lda + (uint32_t)(c * 8)) * 2u;
    int br;
    if (kSwiGLU) {
      int col = n0 + (r & (kBN / 2 - 1));
      if (col > N - 1) col = N - 1;  // N = I: up rows start at I
      br = (r >= kBN / 2 ? N : 0) + col;
    } else if (kWGrad) {
      br = r < n_lim ? r : n_lim - 1;  // the base already points at row n0
    } else {
      br = n0 + r < N ? n0 + r : N - 1;
    }
    b_off[i] = ((uint32_t)br * lda + (uint32_t)(c * 8)) * 2u;  // < 2^32: checked by the launcher
  }
  const uint32_t ring_lds = lds_address(ring) + w * 64 * kRowBytes;
  // load instruction i (0..7) of this wave for the A (B) tile of step kt into ring slot `slot`
  auto load_a = [&](int slot, int kt, int i) {
    dma16(a_base + 2 * kt * kBK, a_off[i], ring_lds + slot * kOperandBytes + i * 1024);
  };
  auto load_b = [&](int slot, int kt, int i) {
    dma16(b_base + 2 * kt * kBK, b_off[i], ring_lds + slot * kOperandBytes + i * 1024);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // K loop.  The tiles of step kt sit in ring slots 2kt % 5 (B) and
  // (2kt+1) % 5 (A).  Step kt multiplies them in four 16-wide slices, reading
  // the fragments of the next slice under the MFMAs of the current one.
  // Slices 0 and 1 also load the B tile of step kt+2 (into the slot step kt-1's
  // A tile held).  After slice 2 every wave waits for its own loads of step
  // kt+1 (only step kt+2's B tile may stay in flight) and passes a barrier:
  // then every wave's loads of step kt+1 are visible and no wave reads step
  // kt's tiles any more (the last slice's fragments are in registers).  Slice
  // 3 reads the first fragments of step kt+1 and loads the A tile of step kt+2
  // into the slot of step kt's B tile.  So B tiles are requested about 1.5
  // steps and A tiles about one step before use; no LDS read latency is
  // exposed; and the load instructions are spread over the MFMA stream.  The
  // barrier orders LDS accesses only (a full workgroup fence would also wait
  // for the loads in flight).
  // (a weight-gradient tile of an expert without rows has no K step: its
  // accumulators stay zero)
  if (KT > 0) {
  bf16x8 fa[2][4], fb[2][4];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) load_b(0, 0, i);
#pragma unroll
  for (int i = 0; i < kLoads; ++i) load_a(1, 0, i);
  if (KT > 1) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load_b(2, 1, i);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load_a(3, 1, i);
    wait_vmcnt<2 * kLoads>();
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  load_frags<kSwiGLU>(ring + kOperandBytes, ring, 0, wm, wn, l, fa[0], fb[0]);
  __builtin_amdgcn_sched_barrier(0);

  // one K step with MI row blocks per wave; sb, sa: slots of step kt's B and A
  // tiles; nb, na: of step kt+1's; pb: slot for step kt+2's B tile
#define MOE_K_STEP(MI)                                                                                   \
  {                                                                                                     \
    const int nb = sb + 2 < kSlots ? sb + 2 : sb + 2 - kSlots;                                          \
    const int na = sa + 2 < kSlots ? sa + 2 : sa + 2 - kSlots;                                          \
    const int pb = na + 1 < kSlots ? na + 1 : na + 1 - kSlots;                                          \
    const bool ahead = kt + 2 < KT;                                                                     \
    const char *as = ring + sa * kOperandBytes;                                                         \
    const char *bs = ring + sb * kOperandBytes;                                                         \
    load_frags<kSwiGLU>(as, bs, 1, wm, wn, l, fa[1], fb[1]);                                            \
    slice<MI>(fa[0], fb[0], acc, [&](int d) {                                                           \
      if (ahead) load_b(pb, kt + 2, d);                                                                 \
    });                                                                                                 \
    load_frags<kSwiGLU>(as, bs, 2, wm, wn, l, fa[0], fb[0]);                                            \
    slice<MI>(fa[1], fb[1], acc, [&](int d) {                                                           \
      if (ahead) load_b(pb, kt + 2, 4 + d);                                                             \
    });                                                                                                 \
    load_frags<kSwiGLU>(as, bs, 3, wm, wn, l, fa[1], fb[1]);                                            \
    slice<MI>(fa[0], fb[0], acc, [&](int) {});                                                          \
    if (ahead) wait_vmcnt<kLoads>();                                                                    \
    else wait_vmcnt<0>();                                                                               \
    lds_barrier();                                                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                                  \
    load_frags<kSwiGLU>(ring + na * kOperandBytes, ring + nb * kOperandBytes, 0, wm, wn, l, fa[0], fb[0]); \
    slice<MI>(fa[1], fb[1], acc, [&](int d) {                                                           \
      if (ahead) {                                                                                      \
        load_a(sb, kt + 2, 2 * d);                                                                      \
        load_a(sb, kt + 2, 2 * d + 1);                                                                  \
      }                                                                                                 \
    });                                                                                                 \
    sb = nb;                                                                                            \
    sa = na;                                                                                            \
  }
  // the ragged last tile of an expert runs the loop with the MFMAs of the row
  // blocks that hold rows: a quarter or half of them when the waves hold at
  // most one or two such blocks
  int sb = 0, sa = 1;
  if (mi_count > 2) {
    for (int kt = 0; kt < KT; ++kt) MOE_K_STEP(4)
  } else if (mi_count == 2) {
    for (int kt = 0; kt < KT; ++kt) MOE_K_STEP(2)
  } else {
    for (int kt = 0; kt < KT; ++kt) MOE_K_STEP(1)
  }
#undef MOE_K_STEP
  wait_vmcnt<0>();  // no direct load may still be writing LDS when the wave ends
  }

  // epilogue: every real LDS read is done (the last barrier has passed), so
  // each wave stages its bf16 sub-tile in its own LDS buffer -- 128 rows x
  // (64 SwiGLU features or 128 output columns), 16-byte chunks XOR-swizzled by
  // row -- and writes it out as whole rows of 16-byte stores.
  constexpr int kCols = kSwiGLU ? 64 : 128;     // output columns of this wave
  constexpr int kPitch = kCols * 2;             // LDS bytes per staged row
  constexpr int kChunksPerRow = kPitch / 16;
  static_assert(128 * kPitch <= kOperandBytes, "staging fits one ring slot");
  auto out_pos = [](int r, int c) {             // LDS chunk position of chunk c of staged row r
    return kChunksPerRow == 16 ? (c ^ (r & 15)) : (c ^ ((r & 7) ^ ((r >> 3) & 1)));
  };
  char *stage = ring + w * kOperandBytes;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int r = mi * 32 + (l & 31);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (kSwiGLU) {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = silu_f(acc[mi][ni][4 * g + i]) * acc[mi][ni + 2][4 * g + i];
          const int f = ni * 32 + 8 * g + 4 * (l >> 5);
          *reinterpret_cast<uint2 *>(stage + r * kPitch + out_pos(r, f >> 3) * 16 + (f & 7) * 2) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      } else {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const f32x16 &c = acc[mi][ni];
          const int f = ni * 32 + 8 * g + 4 * (l >> 5);
          *reinterpret_cast<uint2 *>(stage + r * kPitch + out_pos(r, f >> 3) * 16 + (f & 7) * 2) =
              make_uint2(pack_bf16x2(c[4 * g], c[4 * g + 1]), pack_bf16x2(c[4 * g + 2], c[4 * g + 3]));
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
  __builtin_amdgcn_wave_barrier();
  constexpr int kRowsPerPass = kWave / kChunksPerRow;
  const int col0 = n0 + wn * kCols;
  const int ch = l % kChunksPerRow;
#pragma unroll 4
  for (int r = l / kChunksPerRow; r < 128; r += kRowsPerPass) {
    const int row = (2 * (r >> 5) + wm) * 32 + (r & 31);  // staged row r is row r%32 of block r/32
    const int col = col0 + ch * 8;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + r * kPitch + out_pos(r, ch) * 16);
    if (row < rows_valid && col < N) st16(c_base + (int64_t)row * c_ld + col, v);
  }
}

int64_t tile_bound(int64_t rows, int e, int capacity, int n_tiles) {
  int64_t m = (rows + kBM - 1) / kBM + e;
  if (capacity > 0) {
    const int64_t cap_m = (int64_t)e * ((capacity + kBM - 1) / kBM);
    if (cap_m < m) m = cap_m;
  }
  const int64_t t = m * n_tiles;
  return (t + kXcds - 1) / kXcds * kXcds;
}

// ------------------------------------------------------------------ backward
//
// The weight gradients reduce over an expert's rows, so their GEMM operands
// (dy, x and the two intermediates) are used transposed: [features, rows], each
// expert's rows a segment of columns padded with zeros to a multiple of kBK and
// starting at seg_offp[e].  The activation-gradient GEMMs take the weights
// transposed ([E, I, H] and [E, H, 2I]) so that their operands are K-contiguous
// like every other operand of the grouped GEMM.

// seg_offp[x] = sum over experts x' < x of tokens_per_expert[x'] rounded up to
// kBK; seg_offp[e] = the columns in use.
__global__ __launch_bounds__(kThreads) void seg_offsets_kernel(const int32_t *__restrict__ tokens_per_expert, int e,
                                                               int32_t *__restrict__ seg_offp) {
  constexpr int kPer = kMaxExperts / kThreads;
  __shared__ int32_t part[kThreads];
  const int tid = threadIdx.x;
  int32_t local[kPer];
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int x = tid * kPer + i;
    const int32_t c = x < e ? tokens_per_expert[x] : 0;
    local[i] = (c + kBK - 1) / kBK * kBK;
    s += local[i];
  }
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - s;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int x = tid * kPer + i;
    if (x < e) seg_offp[x] = run;
    run += local[i];
  }
  if (tid == kThreads - 1) seg_offp[e] = part[kThreads - 1];
}

// One 64 x 64 bf16 transpose through LDS: source rows 0..63 (rows >= nv read
// as zeros), columns 0..63 of `src` (row stride src_ld) become destination rows
// 0..63, columns 0..63 of `dst` (row stride dst_ld).  The tile is held as
// 32-bit column pairs, 33 words per source row, so that both the 16-byte row
// writes and the column reads spread over the LDS banks.
__device__ __forceinline__ void transpose_tile64(const uint16_t *__restrict__ src, int64_t src_ld, int nv,
                                                 uint16_t *__restrict__ dst, int64_t dst_ld) {
  constexpr int kPitch = 33;
  __shared__ uint32_t tile[64 * kPitch];
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int j = t / 8 + 32 * p, q = t % 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j < nv) v = ld16(src + (int64_t)j * src_ld + 8 * q);
#pragma unroll
    for (int d = 0; d < 4; ++d) tile[j * kPitch + 4 * q + d] = v[d];
  }
  __syncthreads();
  const int jg = t % 8, cp = t / 8;  // source rows 8*jg .. 8*jg+7, source columns 2*cp, 2*cp+1
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = tile[(8 * jg + i) * kPitch + cp];
  u32x4 lo, hi;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo[i] = (w[2 * i] & 0xFFFFu) | (w[2 * i + 1] << 16);
    hi[i] = (w[2 * i] >> 16) | (w[2 * i + 1] & 0xFFFF0000u);
  }
  st16(dst + (int64_t)(2 * cp) * dst_ld + 8 * jg, lo);
  st16(dst + (int64_t)(2 * cp + 1) * dst_ld + 8 * jg, hi);
}

// Batched transpose of expert weights: src [batch, P, Q] -> dst [batch, Q, P];
// P and Q multiples of 64; grid (P/64, Q/64, batch).
__global__ __launch_bounds__(kThreads) void weight_transpose_kernel(const uint16_t *__restrict__ src, int P, int Q,
                                                                    uint16_t *__restrict__ dst) {
  const int64_t b = blockIdx.z;
  const int j0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  transpose_tile64(src + (b * P + j0) * Q + c0, Q, 64, dst + (b * Q + c0) * P + j0, P);
}

// Segment transpose of expert rows: dst [C, ld] column seg_offp[x] + i holds
// row expert_offsets[x] + i of src [*, C] for i < tokens_per_expert[x] and zero
// up to the next multiple of 64.  C is a multiple of 64; grid (ld/64, C/64).
// Every 64-column block lies inside one expert's padded segment.
__global__ __launch_bounds__(kThreads) void seg_transpose_kernel(
    const uint16_t *__restrict__ src, int C, const int32_t *__restrict__ seg_offp,
    const int32_t *__restrict__ tokens_per_expert, const int32_t *__restrict__ expert_offsets, int e,
    uint16_t *__restrict__ dst, int ld) {
  const int j0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  if (j0 >= seg_offp[e]) return;
  int lo = 0, hi = e - 1;  // the last expert whose segment starts at or before j0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg_offp[mid] <= j0) lo = mid;
    else hi = mid - 1;
  }
  const int i0 = j0 - seg_offp[lo];
  const int nv = tokens_per_expert[lo] - i0;
  transpose_tile64(src + ((int64_t)expert_offsets[lo] + i0) * C + c0, C, nv, dst + (int64_t)c0 * ld + j0, ld);
}

// SwiGLU backward, in place, 8 features per thread.  For row r and feature i,
// with g = gu[r, i], u = gu[r, I+i], da = d_act[r, i], s = sigmoid(g):
//   gu[r, i]     <- bf16(da * u * s * (1 + g * (1 - s)))   (silu'(g) = s (1 + g (1 - s)))
//   gu[r, I + i] <- bf16(da * g * s)
//   d_act[r, i]  <- bf16(g * s * u)                          (the activation itself)
// fp32 arithmetic.  Every element is read and written by the same thread.
__global__ __launch_bounds__(kThreads) void swiglu_bwd_kernel(uint16_t *__restrict__ gu, uint16_t *__restrict__ d_act,
                                                              int64_t rows, int inter) {
  const int per_row = inter / 8;
  const int64_t n = rows * per_row;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * kThreads) {
    const int64_t r = idx / per_row;
    const int c = (int)(idx % per_row) * 8;
    uint16_t *pg = gu + r * 2 * inter + c;
    uint16_t *pu = pg + inter;
    uint16_t *pa = d_act + r * inter + c;
    float g[8], u[8], da[8], dg[8], du[8], a[8];
    Vec16<true>::unpack(ld16(pg), g);
    Vec16<true>::unpack(ld16(pu), u);
    Vec16<true>::unpack(ld16(pa), da);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float sg = 1.0f / (1.0f + __expf(-g[i]));
      const float gs = g[i] * sg;
      dg[i] = da[i] * u[i] * (sg * (1.0f + g[i] * (1.0f - sg)));
      du[i] = da[i] * gs;
      a[i] = gs * u[i];
    }
    st16(pg, Vec16<true>::pack(dg));
    st16(pu, Vec16<true>::pack(du));
    st16(pa, Vec16<true>::pack(a));
  }
}

int64_t seg_ld(int64_t rows, int e) { return ((rows + kBK - 1) / kBK + e) * kBK; }

struct BwdWorkspace {
  int32_t *seg_offp;
  uint16_t *wd_t, *wgu_t, *gu, *dact, *t_h, *t_i;
};

// Carves the backward workspace; with base == nullptr only counts bytes.
size_t carve_bwd(char *base, int64_t rows, int64_t hidden, int inter, int e, BwdWorkspace *w) {
  const int64_t ld = seg_ld(rows, e);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  BwdWorkspace v;
  v.seg_offp = reinterpret_cast<int32_t *>(take(sizeof(int32_t) * (size_t)(e + 1)));
  v.wd_t = reinterpret_cast<uint16_t *>(take(2 * (size_t)e * inter * hidden));
  v.wgu_t = reinterpret_cast<uint16_t *>(take(4 * (size_t)e * inter * hidden));
  v.gu = reinterpret_cast<uint16_t *>(take(4 * (size_t)rows * inter));
  v.dact = reinterpret_cast<uint16_t *>(take(2 * (size_t)rows * inter));
  v.t_h = reinterpret_cast<uint16_t *>(take(2 * (size_t)hidden * ld));
  v.t_i = reinterpret_cast<uint16_t *>(take(4 * (size_t)inter * ld));
  if (w) *w = v;
  return off;
}

// Plain grouped GEMM over the expert segments: C [rows, N] = A [rows, K] B_e^T.
hipError_t launch_plain(const uint16_t *A, const uint16_t *B, int64_t b_stride, int K, int N, int64_t rows, int e,
                        int capacity, const int32_t *tokens_per_expert, const int32_t *expert_offsets, uint16_t *C,
                        hipStream_t stream) {
  const int nt = (N + kBN - 1) / kBN;
  const int64_t g = tile_bound(rows, e, capacity, nt);
  hipLaunchKernelGGL(grouped_gemm_kernel<kModePlain>, dim3((unsigned)g), dim3(kThreads), 0, stream, A, B, b_stride,
                     K, N, nt, tokens_per_expert, expert_offsets, e, C, (int64_t)N, 0, 0, nullptr, 0);
  return hipGetLastError();
}

// Weight-gradient GEMM: C_e [M, N] = A[:, seg_e] B[:, seg_e]^T for every expert.
hipError_t launch_wgrad(const uint16_t *A, const uint16_t *B, int M, int N, int ld, const int32_t *seg_offp, int e,
                        uint16_t *C, hipStream_t stream) {
  const int mt = (M + kBM - 1) / kBM, nt = (N + kBN - 1) / kBN;
  const int chunk = (mt * nt + kXcds - 1) / kXcds;
  hipLaunchKernelGGL(grouped_gemm_kernel<kModeWGrad>, dim3((unsigned)(kXcds * e * chunk)), dim3(kThreads), 0, stream,
                     A, B, (int64_t)0, 0, N, nt, nullptr, nullptr, e, C, (int64_t)N, M, ld, seg_offp, mt);
  return hipGetLastError();
}

hipError_t launch_seg_transpose(const uint16_t *src, int cols, const BwdWorkspace &w, int ld,
                                const int32_t *tokens_per_expert, const int32_t *expert_offsets, int e,
                                uint16_t *dst, hipStream_t stream) {
  hipLaunchKernelGGL(seg_transpose_kernel, dim3((unsigned)(ld / 64), (unsigned)(cols / 64)), dim3(kThreads), 0,
                     stream, src, cols, w.seg_offp, tokens_per_expert, expert_offsets, e, dst, ld);
  return hipGetLastError();
}

}  // namespace

size_t ffn_bwd_workspace_bytes(int64_t rows, int64_t hidden, int inter, int e) {
  return carve_bwd(nullptr, rows, hidden, inter, e, nullptr);
}

int64_t ffn_bwd_seg_ld(int64_t rows, int e) { return seg_ld(rows, e); }

hipError_t launch_expert_ffn_bwd(const uint16_t *x_perm, const uint16_t *grad_y, int64_t rows, int64_t hidden,
                                 int inter, int e, int capacity, const int32_t *tokens_per_expert,
                                 const int32_t *expert_offsets, const uint16_t *w_gate_up, const uint16_t *w_down,
                                 uint16_t *grad_x_perm, uint16_t *grad_w_gate_up, uint16_t *grad_w_down,
                                 void *workspace, hipStream_t stream) {
  BwdWorkspace w;
  carve_bwd(static_cast<char *>(workspace), rows, hidden, inter, e, &w);
  const int ld = (int)seg_ld(rows, e);
  const int H = (int)hidden, I = inter;
  hipError_t st;
#define MOE_TRY(x)                    \
  if ((st = (x)) != hipSuccess) return st;
  hipLaunchKernelGGL(seg_offsets_kernel, dim3(1), dim3(kThreads), 0, stream, tokens_per_expert, e, w.seg_offp);
  MOE_TRY(hipGetLastError());
  // W_down^T [E, I, H] and W_gate_up^T [E, H, 2I]
  hipLaunchKernelGGL(weight_transpose_kernel, dim3((unsigned)(H / 64), (unsigned)(I / 64), (unsigned)e),
                     dim3(kThreads), 0, stream, w_down, H, I, w.wd_t);
  MOE_TRY(hipGetLastError());
  hipLaunchKernelGGL(weight_transpose_kernel, dim3((unsigned)(2 * I / 64), (unsigned)(H / 64), (unsigned)e),
                     dim3(kThreads), 0, stream, w_gate_up, 2 * I, H, w.wgu_t);
  MOE_TRY(hipGetLastError());
  if (rows > 0) {
    // [G | U] = x W_gate_up^T (recomputed), dA = dy W_down
    MOE_TRY(launch_plain(x_perm, w_gate_up, (int64_t)2 * I * H, H, 2 * I, rows, e, capacity, tokens_per_expert,
                         expert_offsets, w.gu, stream));
    MOE_TRY(launch_plain(grad_y, w.wd_t, (int64_t)I * H, H, I, rows, e, capacity, tokens_per_expert, expert_offsets,
                         w.dact, stream));
    // [dG | dU] in place of [G | U]; the activation in place of dA
    const int64_t chunks = rows * (I / 8);
    int64_t blocks = (chunks + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, w.gu, w.dact, rows, I);
    MOE_TRY(hipGetLastError());
    // dx = [dG | dU] W_gate_up
    MOE_TRY(launch_plain(w.gu, w.wgu_t, (int64_t)H * 2 * I, 2 * I, H, rows, e, capacity, tokens_per_expert,
                         expert_offsets, grad_x_perm, stream));
  }
  // dW_down_e = dy_e^T a_e
  MOE_TRY(launch_seg_transpose(grad_y, H, w, ld, tokens_per_expert, expert_offsets, e, w.t_h, stream));
  MOE_TRY(launch_seg_transpose(w.dact, I, w, ld, tokens_per_expert, expert_offsets, e, w.t_i, stream));
  MOE_TRY(launch_wgrad(w.t_h, w.t_i, H, I, ld, w.seg_offp, e, grad_w_down, stream));
  // [dW_gate; dW_up]_e = [dG | dU]_e^T x_e
  MOE_TRY(launch_seg_transpose(x_perm, H, w, ld, tokens_per_expert, expert_offsets, e, w.t_h, stream));
  MOE_TRY(launch_seg_transpose(w.gu, 2 * I, w, ld, tokens_per_expert, expert_offsets, e, w.t_i, stream));
  MOE_TRY(launch_wgrad(w.t_i, w.t_h, 2 * I, H, ld, w.seg_offp, e, grad_w_gate_up, stream));
#undef MOE_TRY
  return hipSuccess;
}

size_t ffn_workspace_bytes(int64_t rows, int inter) { return align256(sizeof(uint16_t) * (size_t)rows * (size_t)inter); }

hipError_t launch_expert_ffn(const uint16_t *x_perm, int64_t rows, int64_t hidden, int inter, int e, int capacity,
                             const int32_t *tokens_per_expert, const int32_t *expert_offsets,
                             const uint16_t *w_gate_up, const uint16_t *w_down, uint16_t *y, void *workspace,
                             hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  uint16_t *act = static_cast<uint16_t *>(workspace);
  const int n1 = (inter + kBN / 2 - 1) / (kBN / 2);
  const int64_t g1 = tile_bound(rows, e, capacity, n1);
  hipLaunchKernelGGL(grouped_gemm_kernel<kModeSwiGLU>, dim3((unsigned)g1), dim3(kThreads), 0, stream, x_perm,
                     w_gate_up, (int64_t)2 * inter * hidden, (int)hidden, inter, n1, tokens_per_expert, expert_offsets,
                     e, act, (int64_t)inter, 0, 0, nullptr, 0);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  const int n2 = (int)((hidden + kBN - 1) / kBN);
  const int64_t g2 = tile_bound(rows, e, capacity, n2);
  hipLaunchKernelGGL(grouped_gemm_kernel<kModePlain>, dim3((unsigned)g2), dim3(kThreads), 0, stream, act, w_down,
                     (int64_t)hidden * inter, inter, (int)hidden, n2, tokens_per_expert, expert_offsets, e, y, hidden,
                     0, 0, nullptr, 0);
  return hipGetLastError();
}

}  // namespace moe
