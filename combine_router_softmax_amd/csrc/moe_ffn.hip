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
// Tile: 128 rows x 128 columns (GEMM1: 64 gate + 64 up columns), K step 64,
// 4 waves in a 2 x 2 arrangement of 64 x 64 sub-tiles (2 x 2 MFMA 32x32 blocks),
// LDS double buffer fed through registers (one barrier per K step), 16-byte
// padded LDS rows.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kLds = kBK + 8;  // bf16 per LDS row
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kMaxExperts = 1024;
constexpr int kTileElems = kBM * kLds;  // per operand per buffer

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct TileCoord {
  int e;
  int n_tile;
  int64_t row0;
  int64_t row_end;
};

// Maps blockIdx.x to an output tile; returns false for surplus workgroups.
// `scratch` must hold kMaxExperts + 1 int64 and is free again on return.
__device__ bool find_tile(const int32_t *__restrict__ tokens_per_expert, const int32_t *__restrict__ expert_offsets,
                          int e, int n_tiles, int64_t *scratch, TileCoord &tc) {
  constexpr int kPer = kMaxExperts / kThreads;  // experts per thread
  __shared__ int64_t part[kThreads];
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
  if (tid == 0) scratch[kMaxExperts] = total;
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

// kSwiGLU: B rows 0..63 are gate rows n0.., 64..127 are up rows I+n0..; output
// the [rows, I] SwiGLU intermediate.  Otherwise a plain 128-column tile of y.
template <bool kSwiGLU>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int64_t b_expert_stride, int K, int N,
    int n_tiles, const int32_t *__restrict__ tokens_per_expert, const int32_t *__restrict__ expert_offsets, int e,
    uint16_t *__restrict__ C, int64_t ldc, int inter) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * kTileElems];
  TileCoord tc;
  if (!find_tile(tokens_per_expert, expert_offsets, e, n_tiles, reinterpret_cast<int64_t *>(lds), tc)) return;

  const int tid = threadIdx.x;
  const int l = lane_id();
  const int w = tid / kWave;
  const int wm = w >> 1, wn = w & 1;
  const int n0 = tc.n_tile * (kSwiGLU ? kBN / 2 : kBN);
  const uint16_t *Be = B + (int64_t)tc.e * b_expert_stride;

  // global -> register staging: 4 x 16 B per operand per thread
  const uint16_t *a_src[4];
  const uint16_t *b_src[4];
  int lds_off[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int v = tid + kThreads * p;
    const int r = v >> 3, kc = v & 7;
    int64_t ar = tc.row0 + r;
    if (ar > tc.row_end - 1) ar = tc.row_end - 1;
    a_src[p] = A + ar * K + kc * 8;
    int64_t br;
    if (kSwiGLU) br = r < kBN / 2 ? n0 + r : inter + n0 + (r - kBN / 2);
    else br = n0 + r < N ? n0 + r : N - 1;
    b_src[p] = Be + br * K + kc * 8;
    lds_off[p] = r * kLds + kc * 8;
  }
  u32x4 ra[4], rb[4];
  auto load_regs = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      ra[p] = ld16(a_src[p] + k0);
      rb[p] = ld16(b_src[p] + k0);
    }
  };
  auto store_lds = [&](int buf) {
    uint16_t *as = lds + buf * 2 * kTileElems;
    uint16_t *bs = as + kTileElems;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      *reinterpret_cast<u32x4 *>(as + lds_off[p]) = ra[p];
      *reinterpret_cast<u32x4 *>(bs + lds_off[p]) = rb[p];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const int KT = K / kBK;
  load_regs(0);
  store_lds(0);
  __syncthreads();
  const int frag_row = l & 31;
  const int frag_k = (l >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_regs((kt + 1) * kBK);
    const uint16_t *as = lds + cur * 2 * kTileElems;
    const uint16_t *bs = as + kTileElems;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kk = ks * 16 + frag_k;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        a[mi] = *reinterpret_cast<const bf16x8 *>(as + (wm * 64 + mi * 32 + frag_row) * kLds + kk);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        // SwiGLU: ni = 0 gate columns wn*32.., ni = 1 the matching up columns
        const int brow = kSwiGLU ? (ni * (kBN / 2) + wn * 32 + frag_row) : (wn * 64 + ni * 32 + frag_row);
        b[ni] = *reinterpret_cast<const bf16x8 *>(bs + brow * kLds + kk);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < KT) store_lds(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column (l & 31) of each 32x32 block, rows
  // 8*(q/4) + 4*(l/32) + q%4 for accumulator element q
  const int col_in = l & 31;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int rl = wm * 64 + mi * 32 + 8 * (q >> 2) + 4 * (l >> 5) + (q & 3);
      const int64_t row = tc.row0 + rl;
      if (row >= tc.row_end) continue;
      if (kSwiGLU) {
        const int col = n0 + wn * 32 + col_in;
        const float g = acc[mi][0][q], u = acc[mi][1][q];
        const float a = silu_f(g) * u;
        C[row * ldc + col] = (uint16_t)(pack_bf16x2(a, 0.0f) & 0xFFFFu);
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = n0 + wn * 64 + ni * 32 + col_in;
          if (col < N) C[row * ldc + col] = (uint16_t)(pack_bf16x2(acc[mi][ni][q], 0.0f) & 0xFFFFu);
        }
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
  return (t + kXcds - 1) / kXcds * kXcds;
}

}  // namespace

size_t ffn_workspace_bytes(int64_t rows, int inter) { return align256(sizeof(uint16_t) * (size_t)rows * (size_t)inter); }

hipError_t launch_expert_ffn(const uint16_t *x_perm, int64_t rows, int64_t hidden, int inter, int e, int capacity,
                             const int32_t *tokens_per_expert, const int32_t *expert_offsets,
                             const uint16_t *w_gate_up, const uint16_t *w_down, uint16_t *y, void *workspace,
                             hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  uint16_t *act = static_cast<uint16_t *>(workspace);
  const int n1 = inter / (kBN / 2);
  const int64_t g1 = tile_bound(rows, e, capacity, n1);
  hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3((unsigned)g1), dim3(kThreads), 0, stream, x_perm, w_gate_up,
                     (int64_t)2 * inter * hidden, (int)hidden, inter, n1, tokens_per_expert, expert_offsets, e, act,
                     (int64_t)inter, inter);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  const int n2 = (int)((hidden + kBN - 1) / kBN);
  const int64_t g2 = tile_bound(rows, e, capacity, n2);
  hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3((unsigned)g2), dim3(kThreads), 0, stream, act, w_down,
                     (int64_t)hidden * inter, inter, (int)hidden, n2, tokens_per_expert, expert_offsets, e, y,
                     hidden, inter);
  return hipGetLastError();
}

}  // namespace moe
