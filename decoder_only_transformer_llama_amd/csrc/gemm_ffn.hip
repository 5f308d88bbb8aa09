// Instances of the bf16 GEMM with the SiLU(gate)*up epilogue.
#include "gemm_kernel.h"

namespace llama {
hipError_t gemm_launch_ffn(const GemmKey &key, const GemmArgs &a, hipStream_t s) {
  GEMM_CASE(256, 0, EPI_SILU)
  GEMM_CASE(256, 1, EPI_SILU)
  GEMM_CASE_F16(256, EPI_SILU)
  GEMM_CASE_192(EPI_SILU)
  return hipErrorInvalidValue;
}
}  // namespace llama
