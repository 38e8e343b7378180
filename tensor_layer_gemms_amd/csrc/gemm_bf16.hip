// bf16 MFMA GEMM launcher: picks a tile shape for the problem and the instantiation
// for (operand layouts, epilogue).
#include "gemm_kernels.hpp"

namespace mt {

namespace {

constexpr int kNumCUs = 256;

struct TileCfg {
  int bm, bn;
  float eff;  // relative per-tile MFMA efficiency (bigger tiles reuse LDS operands more)
};
// 256x256: 8 waves (2 x 4), wave tile 128x64; 256x128: 4 waves (2 x 2), 128x64;
// 128x128: 4 waves, 64x64.
constexpr TileCfg kTiles[] = {{256, 256, 1.0f}, {256, 128, 0.9f}, {128, 128, 0.75f}};

int pick_tile(const GemmArgs& g, int batch) {
  if (g.causal != CAUSAL_NONE) return 2;  // attention products: small square tiles
  int best = 0;
  double best_cost = 1e300;
  for (int c = 0; c < 3; ++c) {
    const long tiles = (long)((g.M + kTiles[c].bm - 1) / kTiles[c].bm) * ((g.N + kTiles[c].bn - 1) / kTiles[c].bn) * batch;
    const long waves = (tiles + kNumCUs - 1) / kNumCUs;
    const double cost = (double)waves * kTiles[c].bm * kTiles[c].bn / kTiles[c].eff;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = c;
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
  switch (pick_tile(g, batch)) {
    case 0: return run<AK, BK, 256, 256, 2, 4, KIND>(g, batch, s);
    case 1: return run<AK, BK, 256, 128, 2, 2, KIND>(g, batch, s);
    default: return run<AK, BK, 128, 128, 2, 2, KIND>(g, batch, s);
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, bool a_k, bool b_k, int kind, int batch, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || batch <= 0) return hipSuccess;
  if (a_k && b_k) {  // forward products (X W^T, Q K^T, dctx V^T)
    switch (kind) {
      case EPI_STORE: return run_tile<true, true, EPI_STORE>(g, batch, s);
      case EPI_STORE_F32: return run_tile<true, true, EPI_STORE_F32>(g, batch, s);
      case EPI_BIAS: return run_tile<true, true, EPI_BIAS>(g, batch, s);
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
