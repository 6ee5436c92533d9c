// Hot-expert replication, the one-GPU part of InternLM/xtuner "Integrate UltraEP
// Runtime": replicas of hot experts placed from the current load, part of each
// hot expert's assignments rerouted to its replica slots (logical -> physical
// expert ids), replica weights synchronised from the masters, and the replica
// weight gradients reduced into the masters'.  The grouped FFN over master and
// replica experts (weights from two storage bases) is the grouped GEMM of
// moe_gemm.hpp with replica bases.
//
// Physical expert p < E is the master of logical expert p; p = E + i is
// replica slot i, holding a copy of logical expert replica_of[i].
//   placement: slots filled one at a time, each to the logical expert with the
//     largest load per copy count_e / (1 + slots_e), ties to the lower id;
//   reroute: expert e's count_e assignments, in assignment order (ordinal o),
//     are cut into m_e = 1 + slots_e runs as equal as possible: o goes to run
//     floor(o * m_e / count_e); run 0 stays on the master, run j >= 1 goes to
//     e's j-th slot in slot order.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kMaxExperts = 1024;
constexpr int kMaxSlots = 1024;
constexpr int kPerLane = kMaxExperts / kWave;
constexpr int kThreads = 256;

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// (c1 / m1, expert x1) ranks before (c2 / m2, x2): larger load per copy,
// compared exactly by cross-multiplication, then the lower expert id.
__device__ __forceinline__ bool ranks_before(int c1, int m1, int x1, int c2, int m2, int x2) {
  const int64_t a = (int64_t)c1 * m2, b = (int64_t)c2 * m1;
  return a > b || (a == b && x1 < x2);
}

// One wave: lane l holds experts l, l + 64, ... with their counts and copy
// numbers in registers; each slot is one wave-wide arg-max.
__global__ __launch_bounds__(kWave) void replica_plan_kernel(const int32_t *__restrict__ counts, int e, int r,
                                                             int32_t *__restrict__ replica_of) {
  const int l = lane_id();
  int c[kPerLane], m[kPerLane];
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int x = l + kWave * j;
    c[j] = x < e ? counts[x] : -1;
    m[j] = 1;
  }
  for (int i = 0; i < r; ++i) {
    int bc = -1, bm = 1, bx = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      const int x = l + kWave * j;
      if (x < e && ranks_before(c[j], m[j], x, bc, bm, bx)) bc = c[j], bm = m[j], bx = x;
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
      const int oc = __shfl_xor(bc, off, kWave), om = __shfl_xor(bm, off, kWave), ox = __shfl_xor(bx, off, kWave);
      if (ranks_before(oc, om, ox, bc, bm, bx)) bc = oc, bm = om, bx = ox;
    }
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
      if (l + kWave * j == bx) ++m[j];
    if (l == 0) replica_of[i] = bx;
  }
}

// Physical id of every assignment from its logical id, its ordinal among the
// expert's assignments and the expert's count (a dropless layout of the
// logical ids).  -1 stays -1; ids outside [0, E) become -2.
__global__ __launch_bounds__(kThreads) void reroute_kernel(const int32_t *__restrict__ idx, int64_t a_n, int e,
                                                           const int32_t *__restrict__ ordinal,
                                                           const int32_t *__restrict__ count,
                                                           const int32_t *__restrict__ replica_of, int r,
                                                           int32_t *__restrict__ phys, ScanHeader *hdr,
                                                           int32_t *counters) {
  __shared__ int32_t slots[kMaxSlots];
  if (blockIdx.x == 0 && threadIdx.x == 0) finish_scan(hdr, counters);  // the layout scan's header
  for (int i = threadIdx.x; i < r; i += kThreads) slots[i] = replica_of[i];
  __syncthreads();
  for (int64_t a = (int64_t)blockIdx.x * kThreads + threadIdx.x; a < a_n; a += (int64_t)gridDim.x * kThreads) {
    const int32_t x = idx[a];
    int32_t p;
    if (x == -1) {
      p = -1;
    } else if (x < 0 || x >= e) {
      p = -2;
    } else {
      int m = 1;
      for (int i = 0; i < r; ++i) m += slots[i] == x;
      const int64_t run = (int64_t)ordinal[a] * m / count[x];
      p = x;
      for (int i = 0, found = 0; i < r && run > 0; ++i)
        if (slots[i] == x && ++found == run) {
          p = e + i;
          break;
        }
    }
    phys[a] = p;
  }
}

// replica[i] = master[replica_of[i]]; slots naming no expert are skipped.
__global__ __launch_bounds__(kThreads) void replica_sync_kernel(const char *__restrict__ master,
                                                                char *__restrict__ replica,
                                                                const int32_t *__restrict__ replica_of, int e,
                                                                int64_t bytes) {
  const int i = blockIdx.y;
  const int x = replica_of[i];
  if (x < 0 || x >= e) return;
  const char *src = master + (int64_t)x * bytes;
  char *dst = replica + (int64_t)i * bytes;
  for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < bytes / 16; v += (int64_t)gridDim.x * kThreads)
    st16_stream(dst + v * 16, ld16_stream(src + v * 16));
}

// The first slot of each replicated expert adds, in slot order, every slot's
// gradient to the master's (fp32 sum, one rounding to bf16).
__global__ __launch_bounds__(kThreads) void replica_grad_reduce_kernel(uint16_t *__restrict__ grad_master,
                                                                       const uint16_t *__restrict__ grad_replica,
                                                                       const int32_t *__restrict__ replica_of, int r,
                                                                       int e, int64_t elems) {
  __shared__ int32_t slots[kMaxSlots];
  for (int i = threadIdx.x; i < r; i += kThreads) slots[i] = replica_of[i];
  __syncthreads();
  const int first = blockIdx.y;
  const int x = slots[first];
  if (x < 0 || x >= e) return;
  for (int i = 0; i < first; ++i)
    if (slots[i] == x) return;  // an earlier slot of the same expert does the sum
  uint16_t *dst = grad_master + (int64_t)x * elems;
  for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < elems / 8; v += (int64_t)gridDim.x * kThreads) {
    float acc[8], g[8];
    Vec16<true>::unpack(ld16(dst + v * 8), acc);
    for (int i = first; i < r; ++i) {
      if (slots[i] != x) continue;
      Vec16<true>::unpack(ld16(grad_replica + (int64_t)i * elems + v * 8), g);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += g[q];
    }
    st16(dst + v * 8, Vec16<true>::pack(acc));
  }
}

unsigned grid_for(int64_t work, int64_t cap) {
  const int64_t b = (work + kThreads - 1) / kThreads;
  return (unsigned)(b < 1 ? 1 : (b > cap ? cap : b));
}

}  // namespace

hipError_t launch_replica_plan(const int32_t *counts, int e, int r, int32_t *replica_of, hipStream_t stream) {
  if (r == 0) return hipSuccess;
  hipLaunchKernelGGL(replica_plan_kernel, dim3(1), dim3(kWave), 0, stream, counts, e, r, replica_of);
  return hipGetLastError();
}

// Workspace: a dropless layout of the logical ids (counts, offsets, ordinals,
// rows, row sources, masks, counters) and that layout's own workspace.
// The layout workspace comes first, so that its header (zero before first use)
// is the reroute workspace's header.
size_t reroute_workspace_bytes(int64_t a, int e) {
  return layout_workspace_bytes(a, e, false) + 2 * align256(4 * (size_t)(e + 1)) + align256(4 * (size_t)a) +
         align256(16);
}

hipError_t launch_reroute(const int32_t *topk_idx, int64_t n, int k, int e, const int32_t *replica_of, int r,
                          int32_t *phys_idx, void *workspace, hipStream_t stream) {
  const int64_t a = n * k;
  if (a == 0) return hipSuccess;
  char *w = static_cast<char *>(workspace) + layout_workspace_bytes(a, e, false);
  auto take = [&](size_t bytes) {
    char *p = w;
    w += align256(bytes);
    return p;
  };
  int32_t *tpe = reinterpret_cast<int32_t *>(take(4 * (size_t)(e + 1)));
  int32_t *off = reinterpret_cast<int32_t *>(take(4 * (size_t)(e + 1)));
  int32_t *ord = reinterpret_cast<int32_t *>(take(4 * (size_t)a));
  int32_t *ctr = reinterpret_cast<int32_t *>(take(16));
  // the layout scan alone gives the ordinals and counts of the logical ids
  hipError_t st = launch_layout_scan(topk_idx, n, k, e, 0, 0, a, tpe, off, ord, ctr, workspace, nullptr, 0, stream);
  if (st != hipSuccess) return st;
  hipLaunchKernelGGL(reroute_kernel, dim3(grid_for(a, 4096)), dim3(kThreads), 0, stream, topk_idx, a, e, ord, tpe,
                     replica_of, r, phys_idx, static_cast<ScanHeader *>(workspace), ctr);
  return hipGetLastError();
}

hipError_t launch_replica_sync(const void *master, void *replica, const int32_t *replica_of, int r, int e,
                               int64_t bytes, hipStream_t stream) {
  if (r == 0 || bytes == 0) return hipSuccess;
  hipLaunchKernelGGL(replica_sync_kernel, dim3(grid_for(bytes / 16, 1024), (unsigned)r), dim3(kThreads), 0, stream,
                     static_cast<const char *>(master), static_cast<char *>(replica), replica_of, e, bytes);
  return hipGetLastError();
}

hipError_t launch_replica_grad_reduce(uint16_t *grad_master, const uint16_t *grad_replica, const int32_t *replica_of,
                                      int r, int e, int64_t elems, hipStream_t stream) {
  if (r == 0 || elems == 0) return hipSuccess;
  hipLaunchKernelGGL(replica_grad_reduce_kernel, dim3(grid_for(elems / 8, 1024), (unsigned)r), dim3(kThreads), 0,
                     stream, grad_master, grad_replica, replica_of, r, e, elems);
  return hipGetLastError();
}

}  // namespace moe
