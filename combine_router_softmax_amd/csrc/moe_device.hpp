// Device helpers shared by the gfx950 kernels of the MoE path: wave64
// primitives, bf16 <-> fp32 conversion, 16-byte vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// Unpack 16 bytes of activations (8 bf16 or 4 fp32) into fp32.
template <bool kBf16>
struct Vec16;

template <>
struct Vec16<true> {
  static constexpr int kElems = 8;
  __device__ __forceinline__ static void unpack(const u32x4 &v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(v[i]);
      f[2 * i + 1] = bf16_hi(v[i]);
    }
  }
  __device__ __forceinline__ static u32x4 pack(const float (&f)[8]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
  }
};

template <>
struct Vec16<false> {
  static constexpr int kElems = 4;
  __device__ __forceinline__ static void unpack(const u32x4 &v, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  __device__ __forceinline__ static u32x4 pack(const float (&f)[4]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    return v;
  }
};

// 16-byte global load / store (global_load_dwordx4 / global_store_dwordx4).
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, const u32x4 &v) { *reinterpret_cast<u32x4 *>(p) = v; }
// Streaming load: the source is read once by this kernel.
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
// Streaming store: the destination is not re-read by this kernel.
__device__ __forceinline__ void st16_stream(void *p, const u32x4 &v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanes_below_mask() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe
