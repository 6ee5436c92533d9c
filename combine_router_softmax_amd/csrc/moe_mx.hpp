// MXFP8 (OCP "Microscaling (MX) Formats Specification" v1.0) quantisation on
// the device, shared by the MXFP8 dispatch and the MXFP8 expert FFN: blocks of
// 32 consecutive elements of a row share one E8M0 scale 2^s with
// s = floor(log2(amax)) - 8 clipped to [-127, 127] (code 0 for an all-zero
// block); each element is the FP8 E4M3 code of x / 2^s, rounded to nearest with
// ties to even and clamped to +-448.
#pragma once

#include "moe_device.hpp"

namespace moe {

// E4M3 code of q (|q| < 2^10, finite).  Magnitudes below 2^-6 sit on the
// subnormal grid of step 2^-9: a * 512 is exact and rintf rounds it to the
// nearest integer, ties to even -- the code itself (8 = 0x08 = 2^-6 when it
// rounds up into the normal range).  From 2^-6 up, rounding the fp32 mantissa
// to its top 3 bits with ties to even (add 0x7FFFF plus the lowest kept bit,
// then shift) gives exponent field and mantissa together, a carry moving into
// the exponent; the fp32 exponent bias 127 becomes E4M3's 7 by subtracting
// 120 << 3.  The clamp to 448 (0x7E) comes first, so no code reaches 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fminf(fabsf(q), 448.0f);
  const uint32_t ab = __float_as_uint(a);
  const uint32_t normal = ((ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20) - (120u << 3);
  const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
  return (a < 0x1p-6f ? sub : normal) | sign;
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
    out[h] = e4m3_code(bf16_lo(w0) * inv) | (e4m3_code(bf16_hi(w0) * inv) << 8) |
             (e4m3_code(bf16_lo(w1) * inv) << 16) | (e4m3_code(bf16_hi(w1) * inv) << 24);
  }
  return (uint32_t)code;
}

}  // namespace moe
