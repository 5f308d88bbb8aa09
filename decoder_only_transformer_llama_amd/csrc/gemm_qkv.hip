// Instances of the bf16 GEMM with the Q/K/V epilogue (norm fold + RoPE).
#include "gemm_kernel.h"

namespace llama {
hipError_t gemm_launch_qkv(const GemmKey &key, const GemmArgs &a, hipStream_t s) {
  GEMM_CASE(256, ASRC_BF16, 0, 1, EPI_QKV)
  GEMM_CASE(256, ASRC_BF16, 1, 1, EPI_QKV)
  GEMM_CASE(256, ASRC_F32, 0, 1, EPI_QKV)
  GEMM_CASE(256, ASRC_F32, 1, 1, EPI_QKV)
  return hipErrorInvalidValue;
}
}  // namespace llama
