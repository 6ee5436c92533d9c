// MXFP8 dispatch: the row scatter of the dispatch with each token row quantised
// on the way to MXFP8 (FP8 dispatch with per-token scales, as the MORI token
// dispatcher of ROCm/Megatron-LM "Add MORI as a Token Dispatcher" offers it;
// MXFP8 as in the ROCm Megatron MXFP8 training recipe).  The format is the OCP
// "Microscaling (MX) Formats Specification" v1.0: every 32 consecutive
// elements of a row share one E8M0 scale 2^s, s = floor(log2(amax)) - 8
// clipped to [-127, 127] (an all-zero block takes the smallest scale, code 0);
// element i is the FP8 E4M3 code of x_i / 2^s, rounded to nearest with ties to
// even and clamped to +-448.
//
// Design: one workgroup per source token as in the bf16 scatter; two lanes
// per MX block (mx_half).  Each token row is read and quantised once, in
// registers, and its codes and scales are stored to each of the token's kept
// rows.  HBM traffic per token: one bf16 row read, (H + H/32) bytes written
// per kept copy -- about half the bytes the bf16 scatter writes.
#include "moe_device.hpp"
#include "moe_kernels.hpp"
#include "moe_mx.hpp"

namespace moe {
namespace {

constexpr int kMxThreads = 256;
constexpr int kMxBlock = 32;  // elements per MX block
constexpr int kMaxPadBlocks = 2048;

// Lane l of a row pass owns 16 consecutive elements, half an MX block, read
// as two 16-byte vectors; the two lanes of a block exchange their maxima with
// one xor shuffle, and each lane's 16 codes form one 16-byte store, so a
// wave's store instruction writes 1 KiB of contiguous codes.  The block
// maximum is taken on the integer bit patterns (for non-negative finite floats
// their order is the order of the values).  Returns the block's E8M0 scale
// code and the lane's 16 E4M3 codes (element i in byte i % 4 of word i / 4).
__device__ __forceinline__ uint32_t mx_half(const u32x4 (&in)[2], u32x4 &out) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(in[i][j] & 0x7FFFu, (in[i][j] >> 16) & 0x7FFFu));
  m = max(m, (uint32_t)__shfl_xor((int)m, 1, kWave));
  // bf16 exponent field f = floor(log2 amax) + 127 for a normal amax, so the
  // scale code (s + 127) is f - 8; zero and subnormal maxima (f = 0) and every
  // f < 8 give the clipped code 0.
  const int code = max((int)(m >> 7) - 8, 0);
  const float inv = __uint_as_float((uint32_t)(254 - code) << 23);  // 2^-s, exact
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w0 = in[i][2 * h], w1 = in[i][2 * h + 1];
      out[2 * i + h] = e4m3x4(bf16_lo(w0) * inv, bf16_hi(w0) * inv, bf16_lo(w1) * inv, bf16_hi(w1) * inv);
    }
  return (uint32_t)code;
}

template <int KC>
__global__ __launch_bounds__(kMxThreads) void scatter_mxfp8_kernel(
    const uint16_t *__restrict__ x, int64_t n, int k, int64_t h, const int32_t *__restrict__ assign_row,
    uint8_t *__restrict__ q, uint8_t *__restrict__ scale, int64_t pad_rows, const int32_t *__restrict__ pad_limit,
    const int32_t *__restrict__ row_src, int64_t pad_blocks) {
  const int64_t b = blockIdx.x;
  const int64_t nblk = h / kMxBlock;
  if (b >= n) {  // zero the pad rows: codes and scales (code 0 = the scale of a zero block)
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int64_t lim = pad_limit && *pad_limit < pad_rows ? *pad_limit : pad_rows;
    for (int64_t r = b - n; r < lim; r += pad_blocks) {
      if (row_src[r] >= 0) continue;
      for (int64_t v = threadIdx.x; v < h / 16; v += kMxThreads) st16_stream(q + r * h + v * 16, z);
      for (int64_t v = threadIdx.x; v < nblk; v += kMxThreads) __builtin_nontemporal_store((uint8_t)0, scale + r * nblk + v);
    }
    return;
  }
  const char *src = reinterpret_cast<const char *>(x + b * h);
  // h / 16 half blocks per row, an even number (h % 32 == 0), and kMxThreads is
  // even: the two lanes of a block always run the same iterations.
  for (int64_t v = threadIdx.x; v < h / 16; v += kMxThreads) {
    u32x4 in[2];
    in[0] = ld16(src + v * 32);
    in[1] = ld16(src + v * 32 + 16);
    u32x4 out;
    const uint8_t code = (uint8_t)mx_half(in, out);
    for (int j0 = 0; j0 < k; j0 += KC) {
      int32_t rows[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j) rows[j] = j0 + j < k ? (assign_row ? assign_row[b * k + j0 + j] : (int32_t)b) : -1;
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        if (rows[j] < 0) continue;
        st16_stream(q + (int64_t)rows[j] * h + v * 16, out);
        if ((v & 1) == 0) __builtin_nontemporal_store(code, scale + (int64_t)rows[j] * nblk + v / 2);
      }
    }
  }
}

inline int slot_chunk(int k) { return k >= 8 ? 8 : (k >= 4 ? 4 : (k >= 2 ? 2 : 1)); }

}  // namespace

hipError_t launch_scatter_mxfp8(const uint16_t *x, int64_t n, int k, int64_t h, const int32_t *assign_row,
                                uint8_t *q, uint8_t *scale, int64_t pad_rows, const int32_t *pad_limit,
                                const int32_t *row_src, hipStream_t stream) {
  const int64_t pb = pad_rows <= 0 ? 0 : (pad_rows < kMaxPadBlocks ? pad_rows : kMaxPadBlocks);
  const int64_t blocks = n + pb;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(kMxThreads);
#define MOE_MXS(KC)                                                                                             \
  hipLaunchKernelGGL(scatter_mxfp8_kernel<KC>, grid, block, 0, stream, x, n, k, h, assign_row, q, scale, pad_rows, \
                     pad_limit, row_src, pb)
  switch (slot_chunk(k)) {
    case 1: MOE_MXS(1); break;
    case 2: MOE_MXS(2); break;
    case 4: MOE_MXS(4); break;
    default: MOE_MXS(8); break;
  }
#undef MOE_MXS
  return hipGetLastError();
}

}  // namespace moe
