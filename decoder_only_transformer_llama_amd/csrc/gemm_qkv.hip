// Instances of the bf16 GEMM with the Q/K/V epilogue (row scale + RoPE).
#include "gemm_kernel.h"

namespace llama {
hipError_t gemm_launch_qkv(const GemmKey &key, const GemmArgs &a, hipStream_t s) {
  GEMM_CASE(256, 0, EPI_QKV)
  GEMM_CASE(256, 1, EPI_QKV)
  GEMM_CASE(128, 0, EPI_QKV)
  GEMM_CASE(128, 1, EPI_QKV)
  GEMM_CASE_F16(256, EPI_QKV)
  GEMM_CASE_F16(128, EPI_QKV)
  return hipErrorInvalidValue;
}
}  // namespace llama
