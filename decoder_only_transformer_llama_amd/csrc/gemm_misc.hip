// Instances of the bf16 GEMM with plain-store, residual-add and split-K
// partial epilogues, and the dispatcher over every instance.
#include "gemm_kernel.h"

namespace llama {
hipError_t gemm_launch_misc(const GemmKey &key, const GemmArgs &a, hipStream_t s) {
  GEMM_CASE_F16(256, EPI_PARTIAL)
  GEMM_CASE_F16(256, EPI_RESID)
  GEMM_CASE_F16(128, EPI_RESID)
  GEMM_CASE_F16(256, EPI_STORE)
  GEMM_CASE(256, 0, EPI_PARTIAL)
  GEMM_CASE(256, 1, EPI_PARTIAL)
  GEMM_CASE(256, 0, EPI_RESID)
  GEMM_CASE(256, 1, EPI_RESID)
  GEMM_CASE(128, 0, EPI_RESID)
  GEMM_CASE(128, 1, EPI_RESID)
  GEMM_CASE(128, 0, EPI_STORE)
  GEMM_CASE(128, 1, EPI_STORE)
  GEMM_CASE(256, 0, EPI_STORE)
  GEMM_CASE(256, 1, EPI_STORE)
  return hipErrorInvalidValue;
}

hipError_t gemm_launch(const GemmKey &key, const GemmArgs &a, hipStream_t s) {
  if (key.epi == EPI_QKV) return gemm_launch_qkv(key, a, s);
  if (key.epi == EPI_SILU) return gemm_launch_ffn(key, a, s);
  return gemm_launch_misc(key, a, s);
}
}  // namespace llama
