// fp32 GEMM launcher (the fp32 path of the layer): the same LDS-DMA MFMA tile kernel as
// the bf16 path (gemm_dma.hpp) instantiated for fp32 operands and outputs, on the
// v_mfma_f32_32x32x2_f32 instruction: same contraction, operand layouts, causal modes,
// loaders, schedule and epilogue arithmetic. Problems the DMA kernel cannot address
// (dimensions or strides not multiples of 4, unaligned bases) run on a 64x64 SIMT tile
// kernel with fp32 fused multiply-adds.
#include "gemm_dma.hpp"

namespace mt {

namespace {
template <bool AK, bool BK, int KIND>
hipError_t run(const GemmArgs& g, int batch, hipStream_t s) {
  if (dma_addressable(g, AK, BK, 4)) {
    // 128x128 tiles (4 waves, 32-deep k-steps): the fp32 path runs small problems, and
    // the causal attention products need a tile side that divides the written chunk.
    const int tiles = ((g.M + 127) / 128) * ((g.N + 127) / 128);
    hipLaunchKernelGGL((gemm_dma_kernel<float, AK, BK, 128, 128, 32, 2, 2, 2, KIND>), dim3(tiles, batch), dim3(256),
                       0, s, g);
    return hipGetLastError();
  }
  const int tiles = ((g.M + 63) / 64) * ((g.N + 63) / 64);
  hipLaunchKernelGGL((gemm_f32_kernel<AK, BK, KIND>), dim3(tiles, batch), dim3(256), 0, s, g);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& g, bool a_k, bool b_k, int kind, int batch, hipStream_t s) {
  if (g.colsum) return hipErrorInvalidValue;  // the fused column sums are a bf16-launcher feature
  if (g.nseg != 1) return hipErrorInvalidValue;  // K segments are a bf16-launcher feature
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
