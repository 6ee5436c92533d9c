// Router kernel: per-token top-k over fp32 logits with a lowest-index
// tie-break, softmax renormalised over the chosen k, the multihot routing map
// and per-expert token counts (the routing stage of MoELayer.forward on the
// page "Megatron MoE 实现"; the multihot map and the host-sync-free counting of
// ROCm/Megatron-LM "Add MORI as a Token Dispatcher").
//
// One wave64 per token.  Lane l holds experts l, l+64, l+128, ... as 64-bit
// keys (ordered logit bits << 32 | ~expert), so one unsigned max picks the
// largest logit and, among equal logits, the lowest expert.  k rounds of a
// wave max-reduction select the top-k in order; the chosen key is zeroed.
// Weights use the identity softmax(l)[i] / sum_chosen softmax(l) =
// exp(l_i - l_max) / sum_chosen exp(l_j - l_max), with l_max the slot-0 logit.
// Counts go through an LDS histogram per block, then global atomics (integer
// adds commute, so the counts are exact and order-independent).
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteTokensPerBlock = kRouteThreads / kWave;

// Order-preserving key of a logit: a larger number gets a larger key; -0.0 and
// +0.0 share one key; NaN gets 0, below every number (whose keys are >= 1).
__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t key) {
  if (key == 0u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

__global__ void fill_i32(int32_t *p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <int VPL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float *__restrict__ logits, int64_t n, int e,
                                                              int k, int32_t *__restrict__ topk_idx,
                                                              float *__restrict__ topk_w,
                                                              uint8_t *__restrict__ routing_map,
                                                              int32_t *__restrict__ tokens_per_expert) {
  extern __shared__ uint32_t smem[];
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  uint32_t *sel_key = smem + w * k;                                        // [4][k]
  int32_t *sel_idx = reinterpret_cast<int32_t *>(smem + kRouteTokensPerBlock * k) + w * k;  // [4][k]
  int32_t *hist = reinterpret_cast<int32_t *>(smem + 2 * kRouteTokensPerBlock * k);         // [e]

  if (tokens_per_expert)
    for (int x = threadIdx.x; x < e; x += kRouteThreads) hist[x] = 0;
  __syncthreads();

  const int64_t t = (int64_t)blockIdx.x * kRouteTokensPerBlock + w;
  if (t < n) {
    const float *row = logits + t * e;
    uint64_t key[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int x = l + kWave * i;
      key[i] = x < e ? ((uint64_t)logit_key(row[x]) << 32) | (uint32_t)~(uint32_t)x : 0ull;
    }
    uint32_t taken = 0;
    for (int j = 0; j < k; ++j) {
      uint64_t best = key[0];
#pragma unroll
      for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const uint32_t x = ~(uint32_t)best;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if ((uint32_t)(l + kWave * i) == x) {
          key[i] = 0ull;
          taken |= 1u << i;
        }
      if (l == 0) {
        sel_key[j] = (uint32_t)(best >> 32);
        sel_idx[j] = (int32_t)x;
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const float lmax = key_logit(sel_key[0]);
    float part = 0.0f;
    for (int j = l; j < k; j += kWave) part += expf(key_logit(sel_key[j]) - lmax);
    const float denom = wave_sum_f32(part);
    for (int j = l; j < k; j += kWave) {
      topk_idx[t * k + j] = sel_idx[j];
      topk_w[t * k + j] = expf(key_logit(sel_key[j]) - lmax) / denom;
    }
    if (routing_map) {
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int x = l + kWave * i;
        if (x < e) routing_map[t * e + x] = (uint8_t)((taken >> i) & 1u);
      }
    }
    if (tokens_per_expert) {
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if ((taken >> i) & 1u) atomicAdd(&hist[l + kWave * i], 1);
    }
  }
  if (tokens_per_expert) {
    __syncthreads();
    for (int x = threadIdx.x; x < e; x += kRouteThreads)
      if (hist[x]) atomicAdd(&tokens_per_expert[x], hist[x]);
  }
}

template <int VPL>
hipError_t launch_route_vpl(const float *logits, int64_t n, int e, int k, int32_t *topk_idx, float *topk_w,
                            uint8_t *routing_map, int32_t *tokens_per_expert, hipStream_t stream) {
  const int64_t blocks = (n + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock;
  const size_t lds = sizeof(uint32_t) * (2 * kRouteTokensPerBlock * (size_t)k + (size_t)e);
  hipLaunchKernelGGL(route_kernel<VPL>, dim3((unsigned)blocks), dim3(kRouteThreads), lds, stream, logits, n, e, k,
                     topk_idx, topk_w, routing_map, tokens_per_expert);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float *logits, int64_t n, int e, int k, int32_t *topk_idx, float *topk_w,
                        uint8_t *routing_map, int32_t *tokens_per_expert, hipStream_t stream) {
  if (tokens_per_expert) {
    hipLaunchKernelGGL(fill_i32, dim3((unsigned)((e + 255) / 256)), dim3(256), 0, stream, tokens_per_expert,
                       (int64_t)e, 0);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
  }
  if (n == 0) return hipSuccess;
  if (e <= 64) return launch_route_vpl<1>(logits, n, e, k, topk_idx, topk_w, routing_map, tokens_per_expert, stream);
  if (e <= 128) return launch_route_vpl<2>(logits, n, e, k, topk_idx, topk_w, routing_map, tokens_per_expert, stream);
  if (e <= 256) return launch_route_vpl<4>(logits, n, e, k, topk_idx, topk_w, routing_map, tokens_per_expert, stream);
  if (e <= 512) return launch_route_vpl<8>(logits, n, e, k, topk_idx, topk_w, routing_map, tokens_per_expert, stream);
  return launch_route_vpl<16>(logits, n, e, k, topk_idx, topk_w, routing_map, tokens_per_expert, stream);
}

}  // namespace moe
