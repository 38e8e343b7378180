// fp32 GEMM launcher (the fp32 path of the layer): same contraction, layouts and
// epilogues as the bf16 MFMA path, computed with fp32 fused multiply-adds.
#include "gemm_kernels.hpp"

namespace mt {

namespace {
template <bool AK, bool BK, int KIND>
hipError_t run(const GemmArgs& g, int batch, hipStream_t s) {
  const int tiles = ((g.M + 63) / 64) * ((g.N + 63) / 64);
  hipLaunchKernelGGL((gemm_f32_kernel<AK, BK, KIND>), dim3(tiles, batch), dim3(256), 0, s, g);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& g, bool a_k, bool b_k, int kind, int batch, hipStream_t s) {
  if (g.colsum) return hipErrorInvalidValue;  // the fused column sums are a bf16-launcher feature
  if (g.M <= 0 || g.N <= 0 || batch <= 0) return hipSuccess;
  if (a_k && b_k) {
    switch (kind) {
      case EPI_STORE: return run<true, true, EPI_STORE>(g, batch, s);
      case EPI_STORE_F32: return run<true, true, EPI_STORE_F32>(g, batch, s);
      case EPI_BIAS: return run<true, true, EPI_BIAS>(g, batch, s);
      case EPI_BIAS_GELU: return run<true, true, EPI_BIAS_GELU>(g, batch, s);
      case EPI_DSOFTMAX: return run<true, true, EPI_DSOFTMAX>(g, batch, s);
      case EPI_BIAS_RESID: return run<true, true, EPI_BIAS_RESID>(g, batch, s);
    }
  } else if (a_k && !b_k) {
    switch (kind) {
      case EPI_STORE: return run<true, false, EPI_STORE>(g, batch, s);
      case EPI_DGELU: return run<true, false, EPI_DGELU>(g, batch, s);
    }
  } else if (!a_k && !b_k) {
    switch (kind) {
      case EPI_STORE: return run<false, false, EPI_STORE>(g, batch, s);
      case EPI_STORE_F32: return run<false, false, EPI_STORE_F32>(g, batch, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace mt
