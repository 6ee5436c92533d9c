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
// The backward (moe_expert_ffn_bwd) runs the same kernel with K-major operands
// -- the weights as stored, for dA and dx, and the expert's rows themselves for
// the weight gradients, which reduce over the rows of each segment -- read
// through LDS transpose loads, plus one elementwise SwiGLU-backward kernel.
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
// then re-read from the XCD's own L2.  Surplus workgroups exit at once.  An
// expert's rows are split evenly over its ceil(rows / 256) m-tiles in whole
// 32-row blocks (520 rows: 192 + 192 + 136, not 256 + 256 + 8), so the m-tiles
// that share a weight tile run the same MFMA loop and stay in step: a short
// last tile ran ahead of its partners through the weights, which they then
// fetched from HBM again (measured at 520 rows per expert: GEMM1 read 8.8 GB
// of HBM against 4.0 GB at 512).  The MFMA work is the same either way: each
// wave runs the MFMAs of its row blocks that hold rows.
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
//
// This header holds the kernel and its helpers; moe_ffn.hip (bf16 forward
// and backward) and moe_ffn_mx.hip (MXFP8 forward) instantiate it.
#pragma once

#include "moe_device.hpp"
#include "moe_kernels.hpp"
#include "moe_mx.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

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
// MXFP8 operands (E4M3 codes, 128 per K step in the same 128-byte tile rows):
// a ring of four operand tiles and the E8M0 scales of two groups of four K
// steps, each group 16 bytes per tile row for each operand.
constexpr int kSlots8 = 4;
constexpr int kScaleGroupBytes = 2 * kBM * 16;  // A and B scales of one group of 4 K steps
static_assert(kSlots8 * kOperandBytes + 2 * kScaleGroupBytes <= 160 * 1024, "LDS budget (MXFP8)");
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
  int64_t row0;     // the tile's first row
  int64_t row_end;  // one past its last row (at most row0 + 256)
};

// Maps blockIdx.x to an output tile; returns false for surplus workgroups.
// `scratch` (LDS) must hold kThreads / kWave + 4 int32 and is free again on
// return.  The experts' row counts and offsets are read in one round of loads
// (kPer experts per thread, in registers); the tile counts are scanned with
// wave scans and one barrier, after which each thread knows the first tile of
// each of its experts, and the thread whose expert holds the workgroup's tile
// publishes the tile's coordinates for a second barrier.  Tile counts fit in
// int32: their total bounds the grid.
__device__ bool find_tile(const int32_t *__restrict__ tokens_per_expert, const int32_t *__restrict__ expert_offsets,
                          int e, int n_tiles, int32_t *scratch, TileCoord &tc) {
  constexpr int kPer = kMaxExperts / kThreads;  // experts per thread
  int32_t *wave_tot = scratch;                  // [kThreads / kWave]
  int32_t *found = wave_tot + kThreads / kWave; // [4]: expert, n-tile, first row, one past the last
  const int tid = threadIdx.x;
  int32_t rows[kPer], offs[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int x = tid * kPer + i;
    rows[i] = x < e ? tokens_per_expert[x] : 0;
    offs[i] = x < e ? expert_offsets[x] : 0;
  }
  int32_t local[kPer];
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    local[i] = ((rows[i] + kBM - 1) / kBM) * n_tiles;
    s += local[i];
  }
  const int l = lane_id(), wv = tid / kWave;
  int32_t incl = s;  // inclusive scan over the wave
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t o = __shfl_up(incl, off, kWave);
    if (l >= off) incl += o;
  }
  if (l == kWave - 1) wave_tot[wv] = incl;
  __syncthreads();
  int32_t run = incl - s, total = 0;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) {
    run += i < wv ? wave_tot[i] : 0;
    total += wave_tot[i];
  }
  const int32_t bid = blockIdx.x;
  const int32_t share = (total + kXcds - 1) / kXcds;
  const int32_t slot = bid / kXcds;
  const int32_t logical = (bid % kXcds) * share + slot;
  const bool ok = slot < share && logical < total;  // block-uniform
  if (ok) {
    // exactly one expert's tile range [run, run + local) holds `logical`
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (logical >= run && logical < run + local[i]) {
        const int32_t nrows = rows[i];
        const int32_t mt = (nrows + kBM - 1) / kBM;
        const int32_t local_id = logical - run;
        const int32_t m_tile = local_id % mt;
        // the expert's 32-row blocks split evenly over its m-tiles (q blocks
        // each, the last one fewer; q <= 8 and every tile holds rows)
        const int32_t blocks = (nrows + 31) / 32;
        const int32_t q = (blocks + mt - 1) / mt;
        const int32_t first = m_tile * q * 32;
        const int32_t last = first + q * 32 < nrows ? first + q * 32 : nrows;
        found[0] = tid * kPer + i;
        found[1] = local_id / mt;
        found[2] = offs[i] + first;  // row offsets are int32 (the layout's row maps are)
        found[3] = offs[i] + last;
      }
      run += local[i];
    }
  }
  __syncthreads();
  if (ok) {
    tc.e = found[0];
    tc.n_tile = found[1];
    tc.row0 = found[2];
    tc.row_end = found[3];
  }
  __syncthreads();
  return ok;
}

// silu(g) = g * sigmoid(g), with the hardware reciprocal (v_rcp_f32, about one
// ulp) in place of a correctly rounded division: the result is rounded to bf16.
__device__ __forceinline__ float silu_f(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

__device__ __forceinline__ uint16_t bf16_bits(float v) { return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu); }

// K-major operand tiles (the source stores K as its row index, the tile's 256
// columns contiguous): 64 rows of 512 bytes per K step, the same 32 KiB as a
// K-contiguous tile.  The fragments are read with ds_read_b64_tr_b16, which
// transposes 16-bit elements across each group of 16 lanes: lane i of a group
// receives, for j = 0..3, element i % 4 of the 8-byte row that lane 4*j + i/4
// of the group addressed.  When lane r of a group addresses row kb + r/4,
// columns nb + 4*(r % 4) .. +3, lane i thus receives column nb + i, rows
// kb .. kb+3: four consecutive K values of one column, half of an MFMA operand.
constexpr int kTRowBytes = kBN * 2;  // bytes per row of a K-major tile

// LDS position of 16-byte chunk c of row k of a K-major tile is c ^ swz_t(k).
// Measured on gfx950, the fragment reads below then run as fast as linear
// 8-byte-per-lane reads; without the permutation they run at about half that.
__device__ __forceinline__ int swz_t(int k) { return ((k & 3) << 2) | (((k >> 2) & 1) << 4); }

// Byte offset, within a K-major tile, of this lane's transposed read h (K values
// 4h .. 4h+3 of its eight) of the fragment of 32-column block blk in slice 0;
// slice ks adds 16*ks rows, which leaves swz_t unchanged.
__device__ __forceinline__ uint32_t tr_off(int l, int blk, int h) {
  const int g = l >> 4, i = l & 15;
  const int k = 8 * (g >> 1) + (i >> 2) + 4 * h;  // lanes 32..63 hold K values 8..15
  const int n = blk * 32 + 16 * (g & 1) + 4 * (i & 3);
  return (uint32_t)(k * kTRowBytes + (((n >> 3) ^ swz_t(k)) << 4) + (n & 7) * 2);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One MFMA operand (8 consecutive K values of one column) from a K-major tile.
__device__ __forceinline__ bf16x8 tr_frag(const char *tile, uint32_t off0, uint32_t off1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + off0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + off1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Fragments of one 16-wide K slice ks from the A tile `as` and the B tile `bs`:
// A rows (2*mi + wm)*32 + l%32, B rows as below, k-chunk 2*ks + l/32.  A K-major
// operand (kAT, kBT) is read through its per-lane offsets ta / tb (block, half).
template <bool kSwiGLU, bool kAT, bool kBT>
__device__ __forceinline__ void load_frags(const char *__restrict__ as, const char *__restrict__ bs, int ks, int wm,
                                           int wn, int l, bf16x8 (&a)[4], bf16x8 (&b)[4],
                                           const uint32_t (&ta)[4][2], const uint32_t (&tb)[4][2]) {
  const int r32 = l & 31;
  const int pos = ((2 * ks + (l >> 5)) ^ swz(r32)) * 16;  // every row read is r32 plus a multiple of 32
  const int tks = ks * 16 * kTRowBytes;
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    if constexpr (kBT) {
      b[ni] = tr_frag(bs + tks, tb[ni][0], tb[ni][1]);
    } else {
      // SwiGLU: blocks 0,1 are gate columns wn*64 + ni*32, blocks 2,3 the matching up columns
      const int brow = kSwiGLU ? ((ni >> 1) * (kBN / 2) + wn * 64 + (ni & 1) * 32 + r32) : (wn * 128 + ni * 32 + r32);
      b[ni] = *reinterpret_cast<const bf16x8 *>(bs + brow * kRowBytes + pos);
    }
  }
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    if constexpr (kAT) a[mi] = tr_frag(as + tks, ta[mi][0], ta[mi][1]);
    else a[mi] = *reinterpret_cast<const bf16x8 *>(as + ((2 * mi + wm) * 32 + r32) * kRowBytes + pos);
  }
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
// fragment reads of the following slice (kReads LDS reads, issued just before,
// in the same scheduling region) are paired with the first half of the MFMAs;
// the slice's four direct-load instructions (dma(0..3)) sit between the MFMAs
// of the second half.  A run of load instructions would stall the wave -- and
// with it the matrix pipe -- while the address unit works through them; spread
// out, each load issues while the previous MFMAs run.
template <int MI, int kReads, typename Dma>
__device__ __forceinline__ void slice(const bf16x8 (&a)[4], const bf16x8 (&b)[4], f32x16 (&acc)[4][4],
                                      Dma &&dma) {
  constexpr int kPart = MI / 2;                  // MFMAs between two load slots (MI = 1: none)
  constexpr int kHead = 4 * MI - 4 * kPart;      // MFMAs paired with the fragment reads
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  mfma_range<0, kHead>(a, b, acc);
#pragma unroll
  for (int i = 0; i < kHead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, (kReads + kHead - 1) / kHead, 0);
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

// MXFP8 fragments: the MFMA v_mfma_scale_f32_32x32x64_f8f6f4 takes, in lane l
// (h = l/32), K values 16h .. 16h+15 and 32+16h .. 32+16h+15 of row l%32 as its
// 32 operand bytes (measured with an in-bounds probe) -- in a tile row of 128
// codes, slice i's chunks 4i+h and 4i+2+h, which are the chunks the bf16
// fragment reads of slices 2i and 2i+1 fetch.  So a slice-i MXFP8 fragment is
// those two bf16 reads side by side.
template <bool kSwiGLU>
__device__ __forceinline__ void load_frags_fp8(const char *__restrict__ as, const char *__restrict__ bs, int i, int wm,
                                               int wn, int l, i32x8 (&a)[4], i32x8 (&b)[4]) {
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  const uint32_t none[4][2] = {};
  load_frags<kSwiGLU, false, false>(as, bs, 2 * i, wm, wn, l, a0, b0, none, none);
  load_frags<kSwiGLU, false, false>(as, bs, 2 * i + 1, wm, wn, l, a1, b1, none, none);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const i32x4 x0 = __builtin_bit_cast(i32x4, a0[j]), x1 = __builtin_bit_cast(i32x4, a1[j]);
    const i32x4 y0 = __builtin_bit_cast(i32x4, b0[j]), y1 = __builtin_bit_cast(i32x4, b1[j]);
    a[j] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    b[j] = __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// MXFP8 MFMAs FIRST .. FIRST+COUNT-1 of one 64-wide K slice, numbered as in
// mfma_range.  Lane l's scale operand covers its row and 32-value block l/32 of
// the slice: the lane's scale words hold the K step's four block codes shifted
// right by 8*(l/32), so byte 2*slice (the op_sel) is its block.
template <int FIRST, int COUNT, int kOpsel>
__device__ __forceinline__ void mfma8_range(const i32x8 (&a)[4], const i32x8 (&b)[4], const uint32_t (&sa)[4],
                                            const uint32_t (&sb)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = FIRST; i < FIRST + COUNT; ++i)
    acc[i / 4][i % 4] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        b[i % 4], a[i / 4], acc[i / 4][i % 4], 0, 0, kOpsel, (int)sb[i % 4], kOpsel, (int)sa[i / 4]);
}

// One MXFP8 K slice (as slice(): the reads of what comes next paired with the
// first MFMAs, the four load slots between the later ones).
template <int MI, int kReads, int kOpsel, typename Dma>
__device__ __forceinline__ void slice_fp8(const i32x8 (&a)[4], const i32x8 (&b)[4], const uint32_t (&sa)[4],
                                          const uint32_t (&sb)[4], f32x16 (&acc)[4][4], Dma &&dma) {
  constexpr int kPart = MI / 2;
  constexpr int kHead = 4 * MI - 4 * kPart;
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  mfma8_range<0, kHead, kOpsel>(a, b, sa, sb, acc);
#pragma unroll
  for (int i = 0; i < kHead; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, (kReads + kHead - 1) / kHead, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  mfma8_range<kHead, kPart, kOpsel>(a, b, sa, sb, acc);
  __builtin_amdgcn_sched_barrier(0);
  dma(0);
  __builtin_amdgcn_sched_barrier(0);
  mfma8_range<kHead + kPart, kPart, kOpsel>(a, b, sa, sb, acc);
  __builtin_amdgcn_sched_barrier(0);
  dma(1);
  __builtin_amdgcn_sched_barrier(0);
  mfma8_range<kHead + 2 * kPart, kPart, kOpsel>(a, b, sa, sb, acc);
  __builtin_amdgcn_sched_barrier(0);
  dma(2);
  __builtin_amdgcn_sched_barrier(0);
  mfma8_range<kHead + 3 * kPart, kPart, kOpsel>(a, b, sa, sb, acc);
  __builtin_amdgcn_sched_barrier(0);
  dma(3);
  __builtin_amdgcn_sched_barrier(0);
}

// Modes of the grouped GEMM.  kModePlain: per expert segment, C = A B_e^T
// (y = act W_down^T, and the backward's products with the weights).
// kModeSwiGLU: B tile rows 0..127 are gate rows n0.., rows 128..255 the up rows
// I+n0..; output the [rows, I] SwiGLU intermediate.  kBT: B is K-major (a
// weight [K, N] of each expert, row length N) instead of K-contiguous ([N, K]);
// plain mode only.
// gate_up (SwiGLU mode, nullable): also store the pre-activations [rows, 2I],
// gate columns then up columns, for the backward.
// kFp8: A and B are MXFP8 (E4M3 codes [.., K] with E8M0 scales A_scale [rows,
// K/32], B_scale [E, N rows, K/32]; K a multiple of 512); plain mode writes
// bf16 C, SwiGLU mode writes the intermediate as MXFP8 (codes into C as bytes
// [rows, ldc], scales into C_scale [rows, ldc/32]).
constexpr int kModePlain = 0, kModeSwiGLU = 1;

template <int kMode, bool kBT, bool kFp8 = false>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int64_t b_expert_stride, int K, int N,
    int n_tiles, const int32_t *__restrict__ tokens_per_expert, const int32_t *__restrict__ expert_offsets, int e,
    uint16_t *__restrict__ C, int64_t ldc, uint16_t *__restrict__ gate_up, const uint16_t *__restrict__ B_rep,
    int e_master, const uint8_t *__restrict__ A_scale, const uint8_t *__restrict__ B_scale,
    uint8_t *__restrict__ C_scale) {
  constexpr bool kSwiGLU = kMode == kModeSwiGLU;
  static_assert(!(kSwiGLU && kBT), "the SwiGLU pairing reads K-contiguous weights");
  static_assert(!kFp8 || !kBT, "MXFP8 operands: K-contiguous forward GEMMs");
  constexpr int kEsz = kFp8 ? 1 : 2;            // bytes per operand element
  constexpr int kStepK = kRowBytes / kEsz;      // K values per step
  // ring of operand tiles (MXFP8: and the scale groups after it); also
  // find_tile's scratch before the K loop and the output staging after it
  __shared__ __attribute__((aligned(1024))) char ring[kFp8 ? kSlots8 * kOperandBytes + 2 * kScaleGroupBytes
                                                            : kSlots * kOperandBytes];

  const int l = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = w >> 1, wn = w & 1;
  // tile coordinates (the same in every lane: kept in scalar registers): n0 the
  // first output column, rows_valid the output rows of the tile, KT the K
  // steps, the operand bases at K = 0 and the output base
  int n0, rows_valid, KT;
  const char *a_base, *b_base;
  const uint8_t *as_base = nullptr, *bs_base = nullptr;  // MXFP8 scale rows of the tile at K = 0
  uint8_t *q_base = nullptr, *qs_base = nullptr;        // MXFP8 intermediate: codes and scales of row0
  uint16_t *c_base, *gu_base = nullptr;
  {
    TileCoord tc;
    if (!find_tile(tokens_per_expert, expert_offsets, e, n_tiles, reinterpret_cast<int32_t *>(ring), tc)) return;
    const int te = __builtin_amdgcn_readfirstlane(tc.e);
    n0 = __builtin_amdgcn_readfirstlane(tc.n_tile) * (kSwiGLU ? kBN / 2 : kBN);
    const int64_t row0 = ((int64_t)__builtin_amdgcn_readfirstlane((int)(tc.row0 >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)tc.row0);
    rows_valid = __builtin_amdgcn_readfirstlane((int)(tc.row_end - tc.row0 < kBM ? tc.row_end - tc.row0 : kBM));
    KT = K / kStepK;
    a_base = reinterpret_cast<const char *>(A) + row0 * K * kEsz;
    // replica slots (experts from e_master on) read the replica weights
    const char *b_e = te < e_master
                          ? reinterpret_cast<const char *>(B) + (int64_t)te * b_expert_stride * kEsz
                          : reinterpret_cast<const char *>(B_rep) + (int64_t)(te - e_master) * b_expert_stride * kEsz;
    b_base = b_e + (kBT ? n0 * 2 : 0);
    if constexpr (kFp8) {
      as_base = A_scale + row0 * (K / 32);
      bs_base = B_scale + (int64_t)te * (b_expert_stride / 32);
      if constexpr (kSwiGLU) {
        q_base = reinterpret_cast<uint8_t *>(C) + row0 * ldc;
        qs_base = C_scale + row0 * (ldc / 32);
      }
    }
    c_base = C + row0 * ldc;
    if (kSwiGLU && gate_up) gu_base = gate_up + row0 * 2 * N;
  }
  // bytes between the operand tiles of consecutive K steps
  const int64_t a_step = kRowBytes;
  const int64_t b_step = kBT ? (int64_t)kBK * N * 2 : kRowBytes;

  // the tile's 32-row blocks 0..7 alternate between the two row groups of waves
  // (block 2*mi + wm is this wave's block mi); count this wave's blocks that
  // hold rows of the segment
  const int blocks_valid = (rows_valid + 31) / 32;
  const int mi_count = blocks_valid > wm ? (blocks_valid - wm + 1) / 2 : 0;

  // direct-load sources: a K-contiguous tile's row r (an output row or column)
  // holds K step kt in 128 bytes (64 bf16 or 128 E4M3 values); this wave fills rows w*64 ..
  // w*64+63, kLoadRows rows per instruction; lane l writes LDS bytes
  // l*16..l*16+15 of the instruction's 1 KiB, i.e. row l / kChunks, position
  // l % kChunks, so it fetches global chunk position ^ swz(row).  A K-major
  // tile's row k holds 256 columns in 512 bytes; this wave fills rows w*16 ..
  // w*16+15, two per instruction: lane l fills row l / 32, position l % 32 with
  // chunk position ^ swz_t(row); columns past the operand's end re-read its last
  // chunk.  Addresses are a per-step scalar base plus a 32-bit per-lane offset.
  uint32_t a_off[kLoads], b_off[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    {
      const int r = w * 64 + i * kLoadRows + l / kChunks;
      const int c = (l % kChunks) ^ swz(r);
      const int ar = r < rows_valid ? r : rows_valid - 1;  // ragged tail: re-read the last row
      a_off[i] = (uint32_t)ar * (uint32_t)(K * kEsz) + (uint32_t)(c * 16);
    }
    if constexpr (kBT) {
      const int k = w * 16 + 2 * i + l / 32;
      const int n_lim = N - n0;  // columns of the operand from n0 on
      int col = ((l % 32) ^ swz_t(k)) * 8;
      if (col > n_lim - 8) col = n_lim - 8;
      b_off[i] = (uint32_t)col * 2u + (uint32_t)k * (uint32_t)N * 2u;
    } else {
      const int r = w * 64 + i * kLoadRows + l / kChunks;
      const int c = (l % kChunks) ^ swz(r);
      int br;
      if (kSwiGLU) {
        int col = n0 + (r & (kBN / 2 - 1));
        if (col > N - 1) col = N - 1;  // N = I: up rows start at I
        br = (r >= kBN / 2 ? N : 0) + col;
      } else {
        br = n0 + r < N ? n0 + r : N - 1;
      }
      b_off[i] = (uint32_t)br * (uint32_t)(K * kEsz) + (uint32_t)(c * 16);  // < 4*I*H bytes
    }
  }
  const uint32_t ring_lds = lds_address(ring) + w * 64 * kRowBytes;  // = w * 16 * kTRowBytes
  // load instruction i (0..7) of this wave for the A (B) tile of step kt into
  // ring slot `slot`.  A wave whose 64 A rows all lie past the segment's end
  // (a tile of at most 192 rows) issues no A loads: no wave multiplies those
  // row blocks, so their stale LDS rows are never used; such a wave's waits
  // count its B loads only.
  const bool a_live = w * 64 < rows_valid;
  auto load_a = [&](int slot, int kt, int i) {
    if (a_live) dma16(a_base + kt * a_step, a_off[i], ring_lds + slot * kOperandBytes + i * 1024);
  };
  auto load_b = [&](int slot, int kt, int i) {
    dma16(b_base + kt * b_step, b_off[i], ring_lds + slot * kOperandBytes + i * 1024);
  };
  // per-lane offsets of the transposed fragment reads (A is never K-major here)
  uint32_t ta[4][2], tb[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ta[j][h] = 0u;
      tb[j][h] = kBT ? tr_off(l, 4 * wn + j, h) : 0u;
    }
  constexpr int kReads = 4 + (kBT ? 8 : 4);

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
  if constexpr (kFp8) {
    // MXFP8 K loop: 128 codes per step in two 64-wide slices.  Four ring slots:
    // step kt's B and A tiles in slots (2kt) % 4 and (2kt) % 4 + 1.  Slice 0
    // runs under the reads of slice 1's fragments; once they have arrived,
    // every wave holds all of step kt's fragments, so an LDS barrier there
    // frees step kt's slots and the rest of slice 0 loads step kt+2's B tile
    // into its B slot (two loads per load slot).  Then every wave waits for its
    // loads of step kt+1 (step kt+2's B tile may stay in flight) and passes a
    // barrier; slice 1 runs under the reads of step kt+1's first fragments and
    // scales and loads step kt+2's A tile (two per load slot).  Issuing all
    // sixteen loads in slice 1 (after the second barrier, the first point at
    // which the slots were known free) had the loads' address processing hold
    // the waves' MFMA issue: slice 1 took about twice its MFMA time (in-kernel
    // clock stamps), and the extra barrier made the MXFP8 FFN 12-13 % faster.
    // The E8M0 scales come in groups of four K steps (16 bytes per tile row per
    // operand) into two LDS buffers: group g+1 is loaded in step 4g, after its
    // buffer's previous group was last read (in step 4g-2), and is waited for
    // with the tiles before its first read (in step 4g+3).
    if (KT > 0) {
      char *sbuf = ring + kSlots8 * kOperandBytes;
      const int sr = w * 64 + l;  // the tile row whose scales this lane fetches
      const int sar = sr < rows_valid ? sr : rows_valid - 1;
      int sbr;
      if (kSwiGLU) {
        int col = n0 + (sr & (kBN / 2 - 1));
        if (col > N - 1) col = N - 1;
        sbr = (sr >= kBN / 2 ? N : 0) + col;
      } else {
        sbr = n0 + sr < N ? n0 + sr : N - 1;
      }
      const uint32_t sa_off = (uint32_t)sar * (uint32_t)(K / 32), sb_off = (uint32_t)sbr * (uint32_t)(K / 32);
      const uint32_t sbuf_lds = lds_address(sbuf) + w * 1024;
      auto load_scales = [&](int g) {
        const uint32_t dst = sbuf_lds + (g & 1) * kScaleGroupBytes;
        dma16(as_base + g * 16, sa_off, dst);
        dma16(bs_base + g * 16, sb_off, dst + kBM * 16);
      };
      const int r32 = l & 31, half = l >> 5;
      // step kt's scale words of the lane's four A and four B fragment rows,
      // shifted so that byte 2*slice is the lane's block (op_sel 0 and 2)
      auto read_scales = [&](int kt, uint32_t (&sa)[4], uint32_t (&sb)[4]) {
        const char *base = sbuf + ((kt >> 2) & 1) * kScaleGroupBytes + (kt & 3) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int brow = kSwiGLU ? ((j >> 1) * (kBN / 2) + wn * 64 + (j & 1) * 32 + r32) : (wn * 128 + j * 32 + r32);
          sa[j] = *reinterpret_cast<const uint32_t *>(base + ((2 * j + wm) * 32 + r32) * 16) >> (8 * half);
          sb[j] = *reinterpret_cast<const uint32_t *>(base + kBM * 16 + brow * 16) >> (8 * half);
        }
      };
      i32x8 fa[2][4], fb[2][4];
      uint32_t sa_c[4], sb_c[4], sa_n[4], sb_n[4];
      load_scales(0);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) load_b(0, 0, i);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) load_a(1, 0, i);
      if (KT > 1) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) load_b(2, 1, i);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) load_a(3, 1, i);
        if (a_live) wait_vmcnt<2 * kLoads>();  // step 0's tiles (and the scales) have landed
        else wait_vmcnt<kLoads>();
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      load_frags_fp8<kSwiGLU>(ring + kOperandBytes, ring, 0, wm, wn, l, fa[0], fb[0]);
      read_scales(0, sa_c, sb_c);
      __builtin_amdgcn_sched_barrier(0);
#define MOE_K_STEP8(MI)                                                                               \
  {                                                                                                   \
    const int sbt = (2 * kt) & 3; /* step kt's B tile; its A tile is in the next slot */              \
    const char *bs = ring + sbt * kOperandBytes;                                                      \
    const char *nbs = ring + (sbt ^ 2) * kOperandBytes;                                               \
    const bool ahead = kt + 2 < KT;                                                                   \
    const bool scales_ahead = (kt & 3) == 0 && kt + 4 < KT;                                           \
    load_frags_fp8<kSwiGLU>(bs + kOperandBytes, bs, 1, wm, wn, l, fa[1], fb[1]);                      \
    slice_fp8<MI, 16, 0>(fa[0], fb[0], sa_c, sb_c, acc, [&](int d) {                                  \
      /* once every wave holds step kt's last fragments, its B slot takes step kt+2's B tile */        \
      if (d == 0) lds_barrier();                                                                      \
      if (ahead) {                                                                                    \
        load_b(sbt, kt + 2, 2 * d);                                                                   \
        load_b(sbt, kt + 2, 2 * d + 1);                                                               \
      }                                                                                               \
    });                                                                                               \
    if (ahead) wait_vmcnt<kLoads>(); /* all but step kt+2's B tile */                                 \
    else wait_vmcnt<0>();                                                                             \
    lds_barrier();                                                                                    \
    __builtin_amdgcn_sched_barrier(0);                                                                \
    /* the last step reads stale slots here; those values are not used */                           \
    load_frags_fp8<kSwiGLU>(nbs + kOperandBytes, nbs, 0, wm, wn, l, fa[0], fb[0]);                    \
    read_scales(kt + 1, sa_n, sb_n);                                                                  \
    slice_fp8<MI, 24, 2>(fa[1], fb[1], sa_c, sb_c, acc, [&](int d) {                                  \
      if (ahead) {                                                                                    \
        load_a(sbt + 1, kt + 2, 2 * d);                                                               \
        load_a(sbt + 1, kt + 2, 2 * d + 1);                                                           \
      }                                                                                               \
      if (d == 0 && scales_ahead) load_scales((kt >> 2) + 1);                                         \
    });                                                                                               \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                                   \
      sa_c[j] = sa_n[j];                                                                              \
      sb_c[j] = sb_n[j];                                                                              \
    }                                                                                                 \
  }
      if (mi_count > 3) {
        for (int kt = 0; kt < KT; ++kt) MOE_K_STEP8(4)
      } else if (mi_count == 3) {
        for (int kt = 0; kt < KT; ++kt) MOE_K_STEP8(3)
      } else if (mi_count == 2) {
        for (int kt = 0; kt < KT; ++kt) MOE_K_STEP8(2)
      } else {
        for (int kt = 0; kt < KT; ++kt) MOE_K_STEP8(1)
      }
#undef MOE_K_STEP8
      wait_vmcnt<0>();  // no direct load may still be writing LDS when the wave ends
    }
  } else if (KT > 0) {
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
    if (a_live) wait_vmcnt<2 * kLoads>();  // step 0's tiles have landed
    else wait_vmcnt<kLoads>();
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  load_frags<kSwiGLU, false, kBT>(ring + kOperandBytes, ring, 0, wm, wn, l, fa[0], fb[0], ta, tb);
  __builtin_amdgcn_sched_barrier(0);

  // one K step with MI row blocks per wave; sb, sa: slots of step kt's B and A
  // tiles; nb, na: of step kt+1's; pb: slot for step kt+2's B tile.
#define MOE_K_STEP(MI)                                                                                 \
  {                                                                                                    \
    const int nb = sb + 2 < kSlots ? sb + 2 : sb + 2 - kSlots;                                         \
    const int na = sa + 2 < kSlots ? sa + 2 : sa + 2 - kSlots;                                         \
    const int pb = na + 1 < kSlots ? na + 1 : na + 1 - kSlots;                                         \
    const bool ahead = kt + 2 < KT;                                                                    \
    const char *as = ring + sa * kOperandBytes;                                                        \
    const char *bs = ring + sb * kOperandBytes;                                                        \
    load_frags<kSwiGLU, false, kBT>(as, bs, 1, wm, wn, l, fa[1], fb[1], ta, tb);                       \
    slice<MI, kReads>(fa[0], fb[0], acc, [&](int d) {                                                  \
      if (ahead) load_b(pb, kt + 2, d);                                                                \
    });                                                                                                \
    load_frags<kSwiGLU, false, kBT>(as, bs, 2, wm, wn, l, fa[0], fb[0], ta, tb);                       \
    slice<MI, kReads>(fa[1], fb[1], acc, [&](int d) {                                                  \
      if (ahead) load_b(pb, kt + 2, 4 + d);                                                            \
    });                                                                                                \
    load_frags<kSwiGLU, false, kBT>(as, bs, 3, wm, wn, l, fa[1], fb[1], ta, tb);                       \
    slice<MI, kReads>(fa[0], fb[0], acc, [&](int) {});                                                 \
    if (ahead) wait_vmcnt<kLoads>();                                                                   \
    else wait_vmcnt<0>();                                                                              \
    lds_barrier();                                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                                 \
    load_frags<kSwiGLU, false, kBT>(ring + na * kOperandBytes, ring + nb * kOperandBytes, 0, wm, wn, l,\
                                  fa[0], fb[0], ta, tb);                                               \
    slice<MI, kReads>(fa[1], fb[1], acc, [&](int d) {                                                  \
      if (ahead) {                                                                                     \
        load_a(sb, kt + 2, 2 * d);                                                                     \
        load_a(sb, kt + 2, 2 * d + 1);                                                                 \
      }                                                                                                \
    });                                                                                                \
    sb = nb;                                                                                           \
    sa = na;                                                                                           \
  }
  // a tile of fewer than 256 rows runs the loop with the MFMAs of the row
  // blocks that hold rows: one to four of each wave's four
  int sb = 0, sa = 1;
  if (mi_count > 3) {
    for (int kt = 0; kt < KT; ++kt) MOE_K_STEP(4)
  } else if (mi_count == 3) {
    for (int kt = 0; kt < KT; ++kt) MOE_K_STEP(3)
  } else if (mi_count == 2) {
    for (int kt = 0; kt < KT; ++kt) MOE_K_STEP(2)
  } else {
    for (int kt = 0; kt < KT; ++kt) MOE_K_STEP(1)
  }
#undef MOE_K_STEP
  wait_vmcnt<0>();  // no direct load may still be writing LDS when the wave ends
  }

  // epilogue: every real LDS read is done (the last barrier has passed), so
  // each wave stages its bf16 sub-tile in its own LDS buffer -- 128 rows x 128
  // columns (the four accumulator blocks side by side) or, for the SwiGLU
  // intermediate, 128 rows x 64 features; 16-byte chunks XOR-swizzled by row --
  // and writes it out as whole rows of 16-byte stores.
  char *stage = ring + w * kOperandBytes;
  auto pos16 = [](int r, int c) { return c ^ (r & 15); };               // rows of 16 chunks
  auto pos8 = [](int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); };  // rows of 8 chunks
  auto stage_acc = [&]() {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int r = mi * 32 + (l & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const f32x16 &c = acc[mi][ni];
          const int f = ni * 32 + 8 * g + 4 * (l >> 5);
          *reinterpret_cast<uint2 *>(stage + r * 256 + pos16(r, f >> 3) * 16 + (f & 7) * 2) =
              make_uint2(pack_bf16x2(c[4 * g], c[4 * g + 1]), pack_bf16x2(c[4 * g + 2], c[4 * g + 3]));
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
    __builtin_amdgcn_wave_barrier();
  };
  // staged row r is row r%32 of the wave's block r/32
  auto tile_row = [&](int r) { return (2 * (r >> 5) + wm) * 32 + (r & 31); };
  if constexpr (kSwiGLU) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int r = mi * 32 + (l & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = silu_f(acc[mi][ni][4 * g + i]) * acc[mi][ni + 2][4 * g + i];
          const int f = ni * 32 + 8 * g + 4 * (l >> 5);
          *reinterpret_cast<uint2 *>(stage + r * 128 + pos8(r, f >> 3) * 16 + (f & 7) * 2) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    const int ch = l % 8;
    const int col = n0 + wn * 64 + ch * 8;
    if constexpr (kFp8) {
      // the bf16 intermediate quantised to MXFP8 on the way out: the four lanes
      // ch 0..3 (4..7) of a row hold one 32-feature block (N % 512 == 0, so
      // every column exists); all lanes quantise, the rows inside the tile store
#pragma unroll
      for (int b = 0; b < 16; b += 8) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = l / 8 + 8 * (b + j);
          v[j] = *reinterpret_cast<const u32x4 *>(stage + r * 128 + pos8(r, ch) * 16);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int row = tile_row(l / 8 + 8 * (b + j));
          u32x2 q;
          const uint32_t code = mx_quad(v[j], q);
          if (row < rows_valid) {
            *reinterpret_cast<u32x2 *>(q_base + (int64_t)row * ldc + col) = q;
            if ((ch & 3) == 0) qs_base[(int64_t)row * (ldc / 32) + col / 32] = (uint8_t)code;
          }
        }
      }
    } else {
#pragma unroll
      for (int b = 0; b < 16; b += 8) {
        u32x4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = l / 8 + 8 * (b + q);
          v[q] = *reinterpret_cast<const u32x4 *>(stage + r * 128 + pos8(r, ch) * 16);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int row = tile_row(l / 8 + 8 * (b + q));
          if (row < rows_valid && col < N) st16(c_base + (int64_t)row * ldc + col, v[q]);
        }
      }
    }
    if (gu_base) {
      // the pre-activations too: staged columns 0..63 are gate features
      // n0 + wn*64 .., columns 64..127 the matching up features
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads of the staged intermediate are done
      __builtin_amdgcn_wave_barrier();
      stage_acc();
      const int ch16 = l % 16;
      const int feat = n0 + wn * 64 + (ch16 & 7) * 8;
      const int gcol = (ch16 >= 8 ? N : 0) + feat;
#pragma unroll
      for (int b = 0; b < 32; b += 8) {
        u32x4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = l / 16 + 4 * (b + q);
          v[q] = *reinterpret_cast<const u32x4 *>(stage + r * 256 + pos16(r, ch16) * 16);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int row = tile_row(l / 16 + 4 * (b + q));
          if (row < rows_valid && feat < N) st16(gu_base + (int64_t)row * 2 * N + gcol, v[q]);
        }
      }
    }
  } else {
    stage_acc();
    const int ch = l % 16;
    const int col = n0 + wn * 128 + ch * 8;
    const int64_t c_ld = ldc;
    // eight staged vectors read (unconditionally: the stage is in bounds), then
    // their stores, so that one LDS wait serves eight stores
#pragma unroll
    for (int b = 0; b < 32; b += 8) {
      u32x4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = l / 16 + 4 * (b + q);
        v[q] = *reinterpret_cast<const u32x4 *>(stage + r * 256 + pos16(r, ch) * 16);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int row = tile_row(l / 16 + 4 * (b + q));
        if (row < rows_valid && col < N) st16(c_base + (int64_t)row * c_ld + col, v[q]);
      }
    }
  }
}

int64_t tile_bound(int64_t rows, int e, int capacity, int n_tiles) {
  int64_t m = (rows + kBM - 1) / kBM + e;
  if (capacity > 0) {
    const int64_t cap_m = (int64_t)e * ((capacity + kBM - 1) / kBM);
    if (cap_m < m) m = cap_m;
  }
  const int64_t t = m * n_tiles;
  return (t + kXcds - 1) / kXcds * kXcds;  // the launchers reject a grid past INT32_MAX (tile ids are int32)
}

}  // namespace
}  // namespace moe
