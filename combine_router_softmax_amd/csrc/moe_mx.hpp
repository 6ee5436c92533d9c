// MXFP8 (OCP "Microscaling (MX) Formats Specification" v1.0) quantisation on
// the device, shared by the MXFP8 dispatch and the MXFP8 expert FFN: blocks of
// 32 consecutive elements of a row share one E8M0 scale 2^s with
// s = floor(log2(amax)) - 8 clipped to [-127, 127] (code 0 for an all-zero
// block); each element is the FP8 E4M3 code of x / 2^s, rounded to nearest with
// ties to even and clamped to +-448.
#pragma once

#include "moe_device.hpp"

namespace moe {

// E4M3 codes of four scaled values (|q| < 2^10, finite), code of a in byte 0
// up to d in byte 3.  Each value is first clamped to +-448, E4M3's largest
// finite magnitude (without the clamp the conversion turns a value that
// rounds past 448 into the NaN code 0x7F); the hardware pair conversion then
// rounds to nearest with ties to even, subnormal range (step 2^-9 below 2^-6)
// included.  Checked on gfx950 against the round-to-nearest-even definition
// for every bf16 value times every E8M0 scale inside that range: identical
// codes throughout.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  auto clamp = [](float q) { return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(a), clamp(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp(c), clamp(d), lo, true);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Four lanes per MX block, 8 bf16 elements per lane (element 2i in the low
// half of word i of `in`): the block maximum is taken on the integer bit
// patterns (for non-negative finite floats their order is the order of the
// values) and shared within the aligned group of four lanes by two xor
// shuffles, so all four lanes must execute this together.  Returns the block's
// E8M0 scale code and the lane's 8 E4M3 codes (element i in byte i % 4 of word
// i / 4 of out).
__device__ __forceinline__ uint32_t mx_quad(const u32x4 &in, u32x2 &out) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) m = max(m, max(in[j] & 0x7FFFu, (in[j] >> 16) & 0x7FFFu));
  m = max(m, (uint32_t)__shfl_xor((int)m, 1, kWave));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2, kWave));
  // bf16 exponent field f = floor(log2 amax) + 127 for a normal amax, so the
  // scale code (s + 127) is f - 8; zero and subnormal maxima (f = 0) and every
  // f < 8 give the clipped code 0.
  const int code = max((int)(m >> 7) - 8, 0);
  const float inv = __uint_as_float((uint32_t)(254 - code) << 23);  // 2^-s, exact
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w0 = in[2 * h], w1 = in[2 * h + 1];
    out[h] = e4m3x4(bf16_lo(w0) * inv, bf16_hi(w0) * inv, bf16_lo(w1) * inv, bf16_hi(w1) * inv);
  }
  return (uint32_t)code;
}

}  // namespace moe
