// bf16 MFMA GEMM launcher: picks a tile shape for the problem and the instantiation
// for (operand layouts, epilogue).
#include "gemm_kernels.hpp"

namespace mt {

namespace {

constexpr int kNumCUs = 256;

struct TileCfg {
  int bm, bn, wm, wn;
  float eff;  // relative per-tile throughput, measured on the layer's shapes
};
// Candidates per operand layout: forward (A, B k-contiguous), input gradient (B
// n-contiguous), weight gradient (both token-strided).
constexpr TileCfg kFwd[] = {{256, 256, 2, 4, 1.0f}, {128, 128, 2, 2, 0.85f}};
constexpr TileCfg kDgrad[] = {{256, 128, 2, 4, 1.0f}, {256, 256, 2, 4, 0.95f}, {128, 128, 2, 2, 0.8f}};
constexpr TileCfg kWgrad[] = {{256, 256, 2, 2, 1.0f}, {128, 256, 2, 2, 0.9f}, {128, 128, 2, 2, 0.8f}};

// Pick the candidate with the least estimated time: whole waves of tiles over the CUs
// times tile area over the candidate's throughput.
template <int N>
int pick(const TileCfg (&c)[N], const GemmArgs& g, int batch) {
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < N; ++i) {
    const long tiles = (long)((g.M + c[i].bm - 1) / c[i].bm) * ((g.N + c[i].bn - 1) / c[i].bn) * batch;
    const long waves = (tiles + kNumCUs - 1) / kNumCUs;
    const double cost = (double)waves * c[i].bm * c[i].bn / c[i].eff;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = i;
    }
  }
  return best;
}

template <bool AK, bool BK, int BM, int BN, int WM, int WN, int KIND>
hipError_t run(const GemmArgs& g, int batch, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<AK, BK, BM, BN, WM, WN, KIND>), dim3(tiles, batch), dim3(64 * WM * WN), 0, s,
                     g);
  return hipGetLastError();
}

template <bool AK, bool BK, int KIND>
hipError_t run_tile(const GemmArgs& g, int batch, hipStream_t s) {
  // Attention products (causal) use 128x128 tiles: every causal tile size must divide
  // the 256-column chunk the probability rows are written in.
  if (g.causal != CAUSAL_NONE) return run<AK, BK, 128, 128, 2, 2, KIND>(g, batch, s);
  if constexpr (AK && BK) {
    switch (pick(kFwd, g, batch)) {
      case 0: return run<AK, BK, 256, 256, 2, 4, KIND>(g, batch, s);
      default: return run<AK, BK, 128, 128, 2, 2, KIND>(g, batch, s);
    }
  } else if constexpr (AK) {
    switch (pick(kDgrad, g, batch)) {
      case 0: return run<AK, BK, 256, 128, 2, 4, KIND>(g, batch, s);
      case 1: return run<AK, BK, 256, 256, 2, 4, KIND>(g, batch, s);
      default: return run<AK, BK, 128, 128, 2, 2, KIND>(g, batch, s);
    }
  } else {
    switch (pick(kWgrad, g, batch)) {
      case 0: return run<AK, BK, 256, 256, 2, 2, KIND>(g, batch, s);
      case 1: return run<AK, BK, 128, 256, 2, 2, KIND>(g, batch, s);
      default: return run<AK, BK, 128, 128, 2, 2, KIND>(g, batch, s);
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, bool a_k, bool b_k, int kind, int batch, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || batch <= 0) return hipSuccess;
  if (g.nseg < 1 || g.nseg > kMaxSeg || (g.nseg > 1 && g.causal != CAUSAL_NONE && g.causal != CAUSAL_SKIP_UPPER))
    return hipErrorInvalidValue;
  if (a_k && b_k) {  // forward products (X W^T, Q K^T, dctx V^T)
    switch (kind) {
      case EPI_STORE: return run_tile<true, true, EPI_STORE>(g, batch, s);
      case EPI_STORE_F32: return run_tile<true, true, EPI_STORE_F32>(g, batch, s);
      case EPI_BIAS: return run_tile<true, true, EPI_BIAS>(g, batch, s);
      case EPI_BIAS_SPLIT: return run_tile<true, true, EPI_BIAS_SPLIT>(g, batch, s);
      case EPI_BIAS_GELU: return run_tile<true, true, EPI_BIAS_GELU>(g, batch, s);
      case EPI_DSOFTMAX: return run_tile<true, true, EPI_DSOFTMAX>(g, batch, s);
    }
  } else if (a_k && !b_k) {  // input gradients (dY W), P V, dS K
    switch (kind) {
      case EPI_STORE: return run_tile<true, false, EPI_STORE>(g, batch, s);
      case EPI_DGELU: return run_tile<true, false, EPI_DGELU>(g, batch, s);
    }
  } else if (!a_k && !b_k) {  // weight gradients (dY^T X), P^T dC, dS^T Q
    switch (kind) {
      case EPI_STORE: return run_tile<false, false, EPI_STORE>(g, batch, s);
      case EPI_STORE_F32: return run_tile<false, false, EPI_STORE_F32>(g, batch, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace mt
