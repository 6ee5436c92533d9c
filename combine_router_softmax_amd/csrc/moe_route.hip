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
// A token marked in the optional padding mask routes nowhere (the router of
// "Add MORI as a Token Dispatcher" masks padding tokens out of routing and
// dispatch).  An optional per-expert bias enters the selection only: experts
// are ranked by logit + bias, the weights come from the logits (Megatron's
// load-balancing expert bias, which "Integrate UltraEP Runtime" lists as not
// yet supported there).  Without logits, the force-balanced benchmark mode of
// "Integrate UltraEP Runtime" routes by uniform random logits drawn from a
// counter-based generator (Philox4x32-10) keyed by a seed.
// Counts: when the routing map is written (E % 16 == 0), a second kernel takes
// its column sums in a few dozen workgroups, one global atomic per expert and
// workgroup; otherwise each router workgroup adds its LDS histogram with global
// atomics.  Integer adds commute, so the counts are exact either way.
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

// Wave-wide max of a 32-bit value with DPP row operations instead of LDS
// permutes: four row_shr steps leave each row's max in its lane 15, two row
// broadcasts carry it to lane 63, which is read back into every lane.  The
// top-k loop makes k of these reductions in a row, so their latency matters.
// A lane without a source (or outside ROW_MASK) reads 0, which leaves an
// unsigned max unchanged; so the move and the max fuse into one DPP max.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
  return t > v ? t : v;
}

__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  v = dpp_max_u32<0x111, 0xF>(v);
  v = dpp_max_u32<0x112, 0xF>(v);
  v = dpp_max_u32<0x114, 0xF>(v);
  v = dpp_max_u32<0x118, 0xF>(v);
  v = dpp_max_u32<0x142, 0xA>(v);
  v = dpp_max_u32<0x143, 0xC>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

__device__ __forceinline__ float key_logit(uint32_t key) {
  if (key == 0u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC 2011): ten rounds of two 32x32 -> 64-bit products, the
// key bumped by two Weyl constants between rounds.  Returns word `word` of the
// output block of counter (c0, c1, c2, 0) under key (k0, k1).
__device__ __forceinline__ uint32_t philox_word(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t k0, uint32_t k1,
                                                int word) {
  uint32_t c3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return word == 0 ? c0 : word == 1 ? c1 : word == 2 ? c2 : c3;
}

// Force-balanced mode: the logit of token t and expert x is the uniform number
// (w >> 8) * 2^-24 in [0, 1), exact in fp32, w = word x % 4 of the Philox block
// of counter (x / 4, t mod 2^32, t / 2^32) under the 64-bit seed.
__device__ __forceinline__ float random_logit(int64_t t, int x, uint64_t seed) {
  const uint32_t w = philox_word((uint32_t)(x >> 2), (uint32_t)t, (uint32_t)((uint64_t)t >> 32), (uint32_t)seed,
                                 (uint32_t)(seed >> 32), x & 3);
  return (float)(w >> 8) * (1.0f / 16777216.0f);
}

__global__ void fill_i32(int32_t *p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Column sums of the [N, E] uint8 routing map (E % 16 == 0, 16-byte rows): a
// thread owns one 16-byte column slice and a strided set of rows of the block's
// row range; a few dozen workgroups each add their partial counts with one
// atomic per expert, which keeps same-address atomic traffic small.
constexpr int kCountRows = 8;  // routing-map rows a thread requests at once

__global__ __launch_bounds__(kRouteThreads) void count_map_kernel(const uint8_t *__restrict__ routing_map, int64_t n,
                                                                  int e, int64_t rows_per_block,
                                                                  int32_t *__restrict__ tokens_per_expert) {
  extern __shared__ int32_t red[];  // [e]
  const int vpr = e / 16;
  const int row_lanes = kRouteThreads / vpr;
  const int v = threadIdx.x % vpr;
  const int rl = threadIdx.x / vpr;
  for (int x = threadIdx.x; x < e; x += kRouteThreads) red[x] = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < n ? r0 + rows_per_block : n;
  if (rl < row_lanes) {
    uint32_t c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = 0;
    // kCountRows rows per round, all requested before any is added (a row at a
    // time costs a memory round trip per row); rows past the range re-read the
    // first row and add nothing
    for (int64_t r = r0 + rl; r < r1; r += (int64_t)kCountRows * row_lanes) {
      u32x4 m[kCountRows];
#pragma unroll
      for (int u = 0; u < kCountRows; ++u) {
        const int64_t rr = r + (int64_t)u * row_lanes;
        m[u] = ld16(routing_map + (rr < r1 ? rr : r0) * e + v * 16);
      }
#pragma unroll
      for (int u = 0; u < kCountRows; ++u) {
        const uint32_t keep = r + (int64_t)u * row_lanes < r1 ? 0xFFu : 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i) c[i] += (m[u][i / 4] >> (8 * (i % 4))) & keep;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (c[i]) atomicAdd(&red[v * 16 + i], (int32_t)c[i]);
  }
  __syncthreads();
  for (int x = threadIdx.x; x < e; x += kRouteThreads)
    if (red[x]) atomicAdd(&tokens_per_expert[x], red[x]);
}

template <int VPL>
// logits == nullptr: the force-balanced mode, logits drawn from `seed`.
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float *__restrict__ logits, uint64_t seed,
                                                              const float *__restrict__ expert_bias,
                                                              const uint8_t *__restrict__ token_mask, int64_t n, int e,
                                                              int k, int32_t *__restrict__ topk_idx,
                                                              float *__restrict__ topk_w,
                                                              uint8_t *__restrict__ routing_map,
                                                              int32_t *__restrict__ tokens_per_expert,
                                                              int32_t *__restrict__ zero_counts) {
  extern __shared__ uint32_t smem[];
  // counts taken later from the routing map start from zero (a later launch adds them)
  if (zero_counts && blockIdx.x == 0)
    for (int x = threadIdx.x; x < e; x += kRouteThreads) zero_counts[x] = 0;
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  uint32_t *sel_key = smem + w * k;                                        // [4][k]
  int32_t *sel_idx = reinterpret_cast<int32_t *>(smem + kRouteTokensPerBlock * k) + w * k;  // [4][k]
  int32_t *hist = reinterpret_cast<int32_t *>(smem + 2 * kRouteTokensPerBlock * k);         // [e]

  if (tokens_per_expert)
    for (int x = threadIdx.x; x < e; x += kRouteThreads) hist[x] = 0;
  __syncthreads();

  const int64_t t = (int64_t)blockIdx.x * kRouteTokensPerBlock + w;
  // a padding token (nonzero mask byte) takes part in no routing: -1 slots,
  // weight 0, an empty map row, no count
  const bool pad = t < n && token_mask && token_mask[t];
  if (pad) {
    for (int j = l; j < k; j += kWave) {
      topk_idx[t * k + j] = -1;
      topk_w[t * k + j] = 0.0f;
    }
    if (routing_map)
      for (int x = l; x < e; x += kWave) routing_map[t * e + x] = 0;
  } else if (t < n) {
    const float *row = logits ? logits + t * e : nullptr;
    auto logit = [&](int x) { return row ? row[x] : random_logit(t, x, seed); };
    // the lane's logits (and biases) are all requested before any is used: one
    // memory round trip per token (loading them one by one, each behind the
    // branch on the logit source, took one round trip each)
    float lx[VPL];
    if (row) {
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int x = l + kWave * i;
        lx[i] = row[x < e ? x : e - 1];
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPL; ++i) lx[i] = random_logit(t, l + kWave * i, seed);
    }
    if (expert_bias) {  // selection score: the logit plus the expert's bias
      float bx[VPL];
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int x = l + kWave * i;
        bx[i] = expert_bias[x < e ? x : e - 1];
      }
#pragma unroll
      for (int i = 0; i < VPL; ++i) lx[i] += bx[i];
    }
    uint64_t key[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int x = l + kWave * i;
      key[i] = x < e ? ((uint64_t)logit_key(lx[i]) << 32) | (uint32_t)~(uint32_t)x : 0ull;
    }
    // Each round takes the largest remaining 64-bit key.  Every lane keeps its
    // own largest key; the wave's largest logit key (the high words) comes from
    // one 32-bit reduction, and only when several lanes hold it does a second
    // reduction over their low words (~expert) pick the lowest expert.  The
    // lane holding the chosen expert (x mod 64, slot x / 64) clears it.  (One
    // 64-bit reduction per round, a compare and two selects per step, took
    // about 930 cycles a round.)
    uint32_t taken = 0;
    uint64_t lbest = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) lbest = key[i] > lbest ? key[i] : lbest;
    for (int j = 0; j < k; ++j) {
      const uint32_t hi = (uint32_t)(lbest >> 32), lo = (uint32_t)lbest;
      const uint32_t m_hi = wave_max_u32_dpp(hi);
      const uint64_t cand = ballot(hi == m_hi);
      const uint32_t m_lo = __popcll(cand) == 1 ? (uint32_t)__builtin_amdgcn_readlane((int)lo, __builtin_ctzll(cand))
                                                : wave_max_u32_dpp(hi == m_hi ? lo : 0u);
      const uint32_t x = ~m_lo;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if ((uint32_t)(l + kWave * i) == x) {
          key[i] = 0ull;
          taken |= 1u << i;
        }
      lbest = key[0];
#pragma unroll
      for (int i = 1; i < VPL; ++i) lbest = key[i] > lbest ? key[i] : lbest;
      if (l == 0) {
        sel_key[j] = m_hi;
        sel_idx[j] = (int32_t)x;
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (!expert_bias) {
      // the chosen logits are the selection keys; slot 0 holds the largest
      const float lmax = key_logit(sel_key[0]);
      float part = 0.0f;
      for (int j = l; j < k; j += kWave) part += expf(key_logit(sel_key[j]) - lmax);
      const float denom = wave_sum_f32(part);
      for (int j = l; j < k; j += kWave) {
        topk_idx[t * k + j] = sel_idx[j];
        topk_w[t * k + j] = expf(key_logit(sel_key[j]) - lmax) / denom;
      }
    } else {
      // the bias only selects: the weights come from the chosen experts' logits,
      // relative to the largest of them
      float lmax = -INFINITY;
      for (int j = l; j < k; j += kWave) lmax = fmaxf(lmax, logit(sel_idx[j]));
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off, kWave));
      float part = 0.0f;
      for (int j = l; j < k; j += kWave) part += expf(logit(sel_idx[j]) - lmax);
      const float denom = wave_sum_f32(part);
      for (int j = l; j < k; j += kWave) {
        topk_idx[t * k + j] = sel_idx[j];
        topk_w[t * k + j] = expf(logit(sel_idx[j]) - lmax) / denom;
      }
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
hipError_t launch_route_vpl(const float *logits, uint64_t seed, const float *expert_bias, const uint8_t *token_mask,
                            int64_t n, int e, int k, int32_t *topk_idx, float *topk_w, uint8_t *routing_map,
                            int32_t *tokens_per_expert, int32_t *zero_counts, hipStream_t stream) {
  const int64_t blocks = (n + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock;
  const size_t lds = sizeof(uint32_t) * (2 * kRouteTokensPerBlock * (size_t)k + (size_t)e);
  hipLaunchKernelGGL(route_kernel<VPL>, dim3((unsigned)blocks), dim3(kRouteThreads), lds, stream, logits, seed,
                     expert_bias, token_mask, n, e, k, topk_idx, topk_w, routing_map, tokens_per_expert, zero_counts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float *logits, uint64_t seed, const float *expert_bias, const uint8_t *token_mask,
                        int64_t n, int e, int k, int32_t *topk_idx, float *topk_w, uint8_t *routing_map,
                        int32_t *tokens_per_expert, hipStream_t stream) {
  const bool map_counts = n > 0 && tokens_per_expert && routing_map && e % 16 == 0 &&
                          (reinterpret_cast<uintptr_t>(routing_map) & 15u) == 0;
  if (tokens_per_expert && !map_counts) {  // the router kernel adds into zeroed counts
    hipLaunchKernelGGL(fill_i32, dim3((unsigned)((e + 255) / 256)), dim3(256), 0, stream, tokens_per_expert,
                       (int64_t)e, 0);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
  }
  if (n == 0) return hipSuccess;
  int32_t *kernel_counts = map_counts ? nullptr : tokens_per_expert;
  int32_t *zero_counts = map_counts ? tokens_per_expert : nullptr;
  hipError_t st;
#define MOE_ROUTE(V) \
  launch_route_vpl<V>(logits, seed, expert_bias, token_mask, n, e, k, topk_idx, topk_w, routing_map, kernel_counts, \
                      zero_counts, stream)
  if (e <= 64) st = MOE_ROUTE(1);
  else if (e <= 128) st = MOE_ROUTE(2);
  else if (e <= 256) st = MOE_ROUTE(4);
  else if (e <= 512) st = MOE_ROUTE(8);
  else st = MOE_ROUTE(16);
#undef MOE_ROUTE
  if (st != hipSuccess || !map_counts) return st;
  int64_t blocks = (n + 63) / 64;
  if (blocks > 32) blocks = 32;
  const int64_t rows_per_block = (n + blocks - 1) / blocks;
  hipLaunchKernelGGL(count_map_kernel, dim3((unsigned)blocks), dim3(kRouteThreads), sizeof(int32_t) * e, stream,
                     routing_map, n, e, rows_per_block, tokens_per_expert);
  return hipGetLastError();
}

}  // namespace moe
