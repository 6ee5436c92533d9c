// Expert FFN over MXFP8 operands: the grouped SwiGLU GEMM1 and GEMM2 of
// moe_gemm.hpp on the scaled fp8 MFMA, the intermediate re-quantised to
// MXFP8 in GEMM1's epilogue.  This file is built with LLVM's machine-sinking
// pass off: the pass moved the first slice's MFMAs of each K step below the
// step's load wait and barrier (measured: 9 % slower forward).
#include "moe_gemm.hpp"

namespace moe {

size_t ffn_mxfp8_workspace_bytes(int64_t rows, int inter) {
  return align256((size_t)rows * (size_t)inter) + align256((size_t)rows * (size_t)(inter / 32));
}

hipError_t launch_expert_ffn_mxfp8(const uint8_t *x_q, const uint8_t *x_s, int64_t rows, int64_t hidden, int inter,
                                   int e, int capacity, const int32_t *tokens_per_expert,
                                   const int32_t *expert_offsets, const uint8_t *w_gate_up_q,
                                   const uint8_t *w_gate_up_s, const uint8_t *w_down_q, const uint8_t *w_down_s,
                                   uint16_t *y, void *workspace, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  // workspace: the MXFP8 intermediate, codes [rows, I] then scales [rows, I/32]
  uint8_t *act_q = static_cast<uint8_t *>(workspace);
  uint8_t *act_s = act_q + align256((size_t)rows * (size_t)inter);
  const int n1 = (inter + kBN / 2 - 1) / (kBN / 2);
  const int n2 = (int)((hidden + kBN - 1) / kBN);
  const int64_t g1 = tile_bound(rows, e, capacity, n1);
  const int64_t g2 = tile_bound(rows, e, capacity, n2);
  if (g1 > INT32_MAX || g2 > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((grouped_gemm_kernel<kModeSwiGLU, false, true>), dim3((unsigned)g1), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint16_t *>(x_q), reinterpret_cast<const uint16_t *>(w_gate_up_q),
                     (int64_t)2 * inter * hidden, (int)hidden, inter, n1, tokens_per_expert, expert_offsets, e,
                     reinterpret_cast<uint16_t *>(act_q), (int64_t)inter, nullptr, nullptr, e, x_s, w_gate_up_s,
                     act_s);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  hipLaunchKernelGGL((grouped_gemm_kernel<kModePlain, false, true>), dim3((unsigned)g2), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint16_t *>(act_q), reinterpret_cast<const uint16_t *>(w_down_q),
                     (int64_t)hidden * inter, inter, (int)hidden, n2, tokens_per_expert, expert_offsets, e, y, hidden,
                     nullptr, nullptr, e, act_s, w_down_s, nullptr);
  return hipGetLastError();
}

}  // namespace moe
