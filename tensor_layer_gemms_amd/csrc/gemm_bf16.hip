// bf16 MFMA GEMM launcher: picks a kernel and tile shape for the problem and the
// instantiation for (operand layouts, epilogue).
//
// The LDS-DMA kernel (gemm_dma.hpp) runs every problem whose operands it can address:
// 16-byte aligned bases and strides, M, N, K multiples of 8, and every byte offset an
// operand tile needs below 4 GiB (its buffer resource takes 32-bit offsets). Anything
// else runs on the register-staged kernel (gemm_kernels.hpp).
#include <algorithm>

#include "gemm_dma.hpp"

namespace mt {

namespace {

constexpr int kNumCUs = 256;

struct TileCfg {
  int bm, bn, per_cu;  // tile, work-groups resident per CU (LDS- or register-limited)
  float eff;           // relative throughput of a CU running per_cu such tiles
};
// DMA kernel candidates (k-step 64; measured on the layer's shapes). Both k-contiguous:
// 256x256 (8 waves), 256x192 (8 waves), 128x128 (4 waves, two per CU). With an
// m-contiguous operand the tile side along it must be a power of two: 256x256 or
// 128x128.
constexpr TileCfg kDmaNT[] = {{256, 256, 1, 1.0f}, {256, 192, 1, 0.95f}, {128, 128, 2, 0.82f}};
constexpr TileCfg kDmaT[] = {{256, 256, 1, 1.0f}, {128, 128, 2, 0.85f}};
// Register-staged kernel candidates per operand layout.
constexpr TileCfg kFwd[] = {{256, 256, 1, 1.0f}, {128, 128, 1, 0.85f}};
constexpr TileCfg kDgrad[] = {{256, 128, 1, 1.0f}, {256, 256, 1, 0.95f}, {128, 128, 1, 0.8f}};
constexpr TileCfg kWgrad[] = {{256, 256, 1, 1.0f}, {128, 256, 1, 0.9f}, {128, 128, 1, 0.8f}};

// Pick the candidate with the least estimated time: whole rounds of tiles over the
// resident slots, each round costing the tile area of one CU's tiles over the
// candidate's throughput.
template <int N>
int pick(const TileCfg (&c)[N], const GemmArgs& g, int batch) {
  int best = 0;
  double best_cost = 1e300;
  for (int i = 0; i < N; ++i) {
    const long tiles = (long)((g.M + c[i].bm - 1) / c[i].bm) * ((g.N + c[i].bn - 1) / c[i].bn) * batch;
    const long slots = (long)kNumCUs * c[i].per_cu;
    const long rounds = (tiles + slots - 1) / slots;
    const double cost = (double)rounds * c[i].bm * c[i].bn * c[i].per_cu / c[i].eff;
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

template <bool AK, bool BK, int BM, int BN, int KT, int WM, int WN, int KIND>
hipError_t run_dma(const GemmArgs& g, int batch, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_dma_kernel<bf16, AK, BK, BM, BN, KT, 2, WM, WN, KIND>), dim3(tiles, batch), dim3(64 * WM * WN),
                     0, s, g);
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

template <bool AK, bool BK, int KIND>
hipError_t run_dma_tile(const GemmArgs& g, int batch, hipStream_t s) {
  if (g.causal != CAUSAL_NONE) return run_dma<AK, BK, 128, 128, 64, 2, 2, KIND>(g, batch, s);
  if constexpr (AK && BK) {
    switch (pick(kDmaNT, g, batch)) {
      case 0: return run_dma<AK, BK, 256, 256, 64, 2, 4, KIND>(g, batch, s);
      case 1: return run_dma<AK, BK, 256, 192, 64, 4, 2, KIND>(g, batch, s);
      default: return run_dma<AK, BK, 128, 128, 64, 2, 2, KIND>(g, batch, s);
    }
  } else {
    switch (pick(kDmaT, g, batch)) {
      case 0: return run_dma<AK, BK, 256, 256, 64, 2, 4, KIND>(g, batch, s);
      default: return run_dma<AK, BK, 128, 128, 64, 2, 2, KIND>(g, batch, s);
    }
  }
}

// Whether the DMA kernel can address the problem (see the file comment).
bool dma_ok(const GemmArgs& g, bool a_k, bool b_k) { return dma_addressable(g, a_k, b_k, 2); }

// Column sums of C over each 128-row block (the register-staged kernel's epilogue does
// not form them): thread = one column, rows in order, fp32.
__global__ __launch_bounds__(256) void colsum_rows_kernel(const bf16* __restrict__ c, int64_t ldc, int M, int N,
                                                          float* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x, rb = blockIdx.y;
  if (n >= N) return;
  const int r1 = min(M, (rb + 1) * kColsumRows);
  float sum = 0.f;
  for (int r = rb * kColsumRows; r < r1; ++r) sum += (float)c[(int64_t)r * ldc + n];
  out[(int64_t)rb * N + n] = sum;
}

template <bool AK, bool BK, int KIND>
hipError_t dispatch(const GemmArgs& g, int batch, hipStream_t s) {
  if (dma_ok(g, AK, BK)) return run_dma_tile<AK, BK, KIND>(g, batch, s);
  const hipError_t e = run_tile<AK, BK, KIND>(g, batch, s);
  if constexpr (KIND == EPI_DGELU) {
    if (e == hipSuccess && g.colsum) {
      hipLaunchKernelGGL(colsum_rows_kernel, dim3((unsigned)((g.N + 255) / 256), (unsigned)((g.M + kColsumRows - 1) / kColsumRows)),
                         dim3(256), 0, s, static_cast<const bf16*>(g.C), g.ldc, g.M, g.N, g.colsum);
      return hipGetLastError();
    }
  }
  return e;
}

// Paired launch; either problem may be batched (batch0 / batch1 entries, e.g. k slices).
template <class P0, class P1>
hipError_t run_pair(const GemmArgs& g0, const GemmArgs& g1, hipStream_t s, int batch0 = 1, int batch1 = 1) {
  const int z0 = ((g0.M + P0::kBM - 1) / P0::kBM) * ((g0.N + P0::kBN - 1) / P0::kBN);
  const int z1 = ((g1.M + P1::kBM - 1) / P1::kBM) * ((g1.N + P1::kBN - 1) / P1::kBN);
  const int t0 = z0 * batch0, t1 = z1 * batch1;
  const int first = g1.K > g0.K ? 1 : 0;  // deeper contraction first
  hipLaunchKernelGGL((gemm_dma_pair_kernel<P0, P1>), dim3(t0 + t1), dim3(P0::kThreads), 0, s, g0, g1, first,
                     first ? t1 : t0, z0, z1);
  return hipGetLastError();
}

// Estimated time of a paired launch (problem i batched b_i times): the larger of the mean
// work per resident slot and the deepest single tile, in tile-k-steps, times the CU's
// share of tile area over the candidate's throughput.
double pair_cost(const TileCfg& c, const GemmArgs& g0, const GemmArgs& g1, int b0 = 1, int b1 = 1) {
  auto tiles = [&](const GemmArgs& g) { return (double)((g.M + c.bm - 1) / c.bm) * ((g.N + c.bn - 1) / c.bn); };
  const double s0 = (g0.K + 63) / 64, s1 = (g1.K + 63) / 64;
  const double slots = (double)kNumCUs * c.per_cu;
  const double t = std::max((tiles(g0) * b0 * s0 + tiles(g1) * b1 * s1) / slots, std::max(s0, s1));
  return t * c.bm * c.bn * c.per_cu / c.eff;
}

// pair_cost in microseconds: one k-step of a 256x256 tile on a CU takes ~2.1 us (the
// backward pairs of the 175B shard).
constexpr double kUsPerCostUnit = 2.1 / (256.0 * 256.0);

// C = sum over `splits` fp32 slices of part (each [M, N] dense) in slice order, stored as
// T (bf16 input gradient or fp32 weight gradient), C strided by ldc.
template <typename T>
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, T* __restrict__ C, int M,
                                                        int N, int splits, int64_t ldc, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int cpr = N / 8;
  const int m = (int)(i / cpr), n = (int)(i % cpr) * 8;
  float acc[8];
  load8(part + (int64_t)m * N + n, acc);
  for (int z = 1; z < splits; ++z) {
    float v[8];
    load8(part + ((int64_t)z * M + m) * N + n, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += v[e];
  }
  store8(C + (int64_t)m * ldc + n, acc);
}

// dgrad (A k-contiguous, B n-contiguous) + wgrad (both token-strided, fp32 out).
template <int KIND0>
hipError_t pair_dispatch(const GemmArgs& g0, const GemmArgs& g1, hipStream_t s) {
  if (pair_cost(kDmaT[0], g0, g1) <= pair_cost(kDmaT[1], g0, g1))
    return run_pair<DmaProblem<true, false, 256, 256, 64, 2, 4, KIND0>,
                    DmaProblem<false, false, 256, 256, 64, 2, 4, EPI_STORE_F32>>(g0, g1, s);
  return run_pair<DmaProblem<true, false, 128, 128, 64, 2, 2, KIND0>,
                  DmaProblem<false, false, 128, 128, 64, 2, 2, EPI_STORE_F32>>(g0, g1, s);
}

// Two both-k-contiguous problems, fp32 out.
hipError_t pair_dispatch_nt(const GemmArgs& g0, const GemmArgs& g1, hipStream_t s) {
  if (pair_cost(kDmaNT[0], g0, g1) <= pair_cost(kDmaNT[2], g0, g1))
    return run_pair<DmaProblem<true, true, 256, 256, 64, 2, 4, EPI_STORE_F32>,
                    DmaProblem<true, true, 256, 256, 64, 2, 4, EPI_STORE_F32>>(g0, g1, s);
  return run_pair<DmaProblem<true, true, 128, 128, 64, 2, 2, EPI_STORE_F32>,
                  DmaProblem<true, true, 128, 128, 64, 2, 2, EPI_STORE_F32>>(g0, g1, s);
}

}  // namespace

int gemm_dgrad_splits(int64_t N, int64_t K) {
  int best = 1;
  for (int sp = 2; sp <= 4; sp *= 2) {
    if (K / (sp / 2) <= 2 * N || K % (64 * sp) != 0) break;  // already shallow enough, or not divisible
    best = sp;
  }
  return best;
}

void gemm_pair_splits(const GemmArgs& dg, int dkind, const GemmArgs& wg, int* sd, int* sw) {
  *sd = dkind == EPI_STORE ? gemm_dgrad_splits(dg.N, dg.K) : 1;
  *sw = 1;
  if (*sd > 1 || dkind != EPI_STORE) return;
  // Weight gradient in k slices (the token dimension) where its tiles are the long pole of
  // the pair: estimated time with sw slices plus the slices' extra traffic (written and
  // read back beyond the direct store, at ~4 TB/s) and the summing launch, taken when it
  // saves at least a tenth.
  auto best_us = [&](const GemmArgs& g1, int b1) {
    return std::min(pair_cost(kDmaT[0], dg, g1, 1, b1), pair_cost(kDmaT[1], dg, g1, 1, b1)) * kUsPerCostUnit;
  };
  double t_best = best_us(wg, 1);
  for (int sp = 2; sp <= 4; sp *= 2) {
    if (wg.K % (64 * sp) != 0) break;
    GemmArgs g1 = wg;
    g1.K = wg.K / sp;
    const double extra_us = (2.0 * sp - 1.0) * 4.0 * (double)wg.M * (double)wg.N / 4.0e6 + 3.0;
    const double t = best_us(g1, sp) + extra_us;
    if (t < 0.9 * t_best) {
      t_best = t;
      *sw = sp;
    }
  }
}

int64_t gemm_pair_split_floats(const GemmArgs& dg, int dkind, const GemmArgs& wg) {
  int sd, sw;
  gemm_pair_splits(dg, dkind, wg, &sd, &sw);
  if (sd > 1) return (int64_t)sd * dg.M * dg.N;
  if (sw > 1) return (int64_t)sw * wg.M * wg.N;
  return 0;
}

namespace {

// The weight gradient of an EPI_STORE pair as sw k slices into part, then summed into wg.C.
hipError_t pair_wgrad_split(const GemmArgs& dg, const GemmArgs& wg, int sw, float* part, hipStream_t s) {
  if (wg.N % 8 || wg.zdiv != 1 || dg.colsum || wg.colsum) return hipErrorNotSupported;
  // slice z contracts the tokens k in [z K/sw, (z + 1) K/sw) into part[z]
  GemmArgs g1 = wg;
  const int64_t ks = wg.K / sw;
  g1.K = (int)ks;
  g1.a_so = ks * wg.lda;  // A(m, k) at k lda + m
  g1.b_so = ks * wg.ldb;  // B(n, k) at k ldb + n
  g1.C = part;
  g1.ldc = wg.N;
  g1.c_so = (int64_t)wg.M * wg.N;
  g1.a_si = g1.b_si = g1.c_si = 0;
  g1.alpha = 1.0f;
  if (!dma_ok(g1, false, false)) return hipErrorNotSupported;
  hipError_t e;
  if (pair_cost(kDmaT[0], dg, g1, 1, sw) <= pair_cost(kDmaT[1], dg, g1, 1, sw))
    e = run_pair<DmaProblem<true, false, 256, 256, 64, 2, 4, EPI_STORE>,
                 DmaProblem<false, false, 256, 256, 64, 2, 4, EPI_STORE_F32>>(dg, g1, s, 1, sw);
  else
    e = run_pair<DmaProblem<true, false, 128, 128, 64, 2, 2, EPI_STORE>,
                 DmaProblem<false, false, 128, 128, 64, 2, 2, EPI_STORE_F32>>(dg, g1, s, 1, sw);
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)wg.M * (wg.N / 8);
  hipLaunchKernelGGL(split_sum_kernel<float>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part,
                     static_cast<float*>(wg.C), wg.M, wg.N, sw, wg.ldc, total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16_pair_split(const GemmArgs& dg, int dkind, const GemmArgs& wg, float* part,
                                       hipStream_t s) {
  int sp, sw;
  gemm_pair_splits(dg, dkind, wg, &sp, &sw);
  if ((sp <= 1 && sw <= 1) || !part || dg.causal != CAUSAL_NONE || dg.nseg != 1 || dg.zdiv != 1)
    return hipErrorNotSupported;
  for (const GemmArgs* g : {&dg, &wg})
    if (g->causal != CAUSAL_NONE || g->nseg != 1 || g->M <= 0 || g->N <= 0) return hipErrorNotSupported;
  if (!dma_ok(dg, true, false) || !dma_ok(wg, false, false)) return hipErrorNotSupported;
  if (sw > 1) return pair_wgrad_split(dg, wg, sw, part, s);
  if (dg.N % 8) return hipErrorNotSupported;
  // dgrad as `sp` k slices: slice z contracts k in [z K/sp, (z + 1) K/sp) into part[z].
  GemmArgs g0 = dg;
  const int64_t ks = dg.K / sp;
  g0.K = (int)ks;
  g0.a_so = ks;             // A(m, k) at m lda + k
  g0.b_so = ks * dg.ldb;    // B(n, k) at k ldb + n
  g0.C = part;
  g0.ldc = dg.N;
  g0.c_so = (int64_t)dg.M * dg.N;
  g0.a_si = g0.b_si = g0.c_si = 0;
  g0.zdiv = 1;
  g0.alpha = 1.0f;
  hipError_t e;
  if (pair_cost(kDmaT[0], g0, wg) <= pair_cost(kDmaT[1], g0, wg))
    e = run_pair<DmaProblem<true, false, 256, 256, 64, 2, 4, EPI_STORE_F32>,
                 DmaProblem<false, false, 256, 256, 64, 2, 4, EPI_STORE_F32>>(g0, wg, s, sp);
  else
    e = run_pair<DmaProblem<true, false, 128, 128, 64, 2, 2, EPI_STORE_F32>,
                 DmaProblem<false, false, 128, 128, 64, 2, 2, EPI_STORE_F32>>(g0, wg, s, sp);
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)dg.M * (dg.N / 8);
  hipLaunchKernelGGL(split_sum_kernel<bf16>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part,
                     static_cast<bf16*>(dg.C), dg.M, dg.N, sp, dg.ldc, total);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_pair(const GemmArgs& g0, bool a_k0, bool b_k0, int kind0, const GemmArgs& g1, bool a_k1,
                                 bool b_k1, int kind1, hipStream_t s) {
  for (const GemmArgs* g : {&g0, &g1})
    if (g->causal != CAUSAL_NONE || g->nseg != 1 || g->M <= 0 || g->N <= 0) return hipErrorNotSupported;
  if (!dma_ok(g0, a_k0, b_k0) || !dma_ok(g1, a_k1, b_k1)) return hipErrorNotSupported;
  if (a_k0 && b_k0 && a_k1 && b_k1) {
    if (kind0 != EPI_STORE_F32 || kind1 != EPI_STORE_F32) return hipErrorNotSupported;
    return pair_dispatch_nt(g0, g1, s);
  }
  if (!(a_k0 && !b_k0 && !a_k1 && !b_k1 && kind1 == EPI_STORE_F32)) return hipErrorNotSupported;
  if (kind0 != EPI_STORE && kind0 != EPI_DGELU) return hipErrorNotSupported;
  if ((g0.colsum && kind0 != EPI_DGELU) || g1.colsum) return hipErrorInvalidValue;
  return kind0 == EPI_DGELU ? pair_dispatch<EPI_DGELU>(g0, g1, s) : pair_dispatch<EPI_STORE>(g0, g1, s);
}

hipError_t launch_gemm_bf16(const GemmArgs& g, bool a_k, bool b_k, int kind, int batch, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || batch <= 0) return hipSuccess;
  if (g.colsum && (kind != EPI_DGELU || batch != 1)) return hipErrorInvalidValue;
  if (g.nseg < 1 || g.nseg > kMaxSeg || (g.nseg > 1 && g.causal != CAUSAL_NONE && g.causal != CAUSAL_SKIP_UPPER))
    return hipErrorInvalidValue;
  if (a_k && b_k) {  // forward products (X W^T, Q K^T, dctx V^T)
    switch (kind) {
      case EPI_STORE: return dispatch<true, true, EPI_STORE>(g, batch, s);
      case EPI_STORE_F32: return dispatch<true, true, EPI_STORE_F32>(g, batch, s);
      case EPI_BIAS: return dispatch<true, true, EPI_BIAS>(g, batch, s);
      case EPI_BIAS_SPLIT: return dispatch<true, true, EPI_BIAS_SPLIT>(g, batch, s);
      case EPI_BIAS_GELU: return dispatch<true, true, EPI_BIAS_GELU>(g, batch, s);
      case EPI_DSOFTMAX: return dispatch<true, true, EPI_DSOFTMAX>(g, batch, s);
      case EPI_BIAS_RESID: return dispatch<true, true, EPI_BIAS_RESID>(g, batch, s);
    }
  } else if (a_k && !b_k) {  // input gradients (dY W), P V, dS K
    switch (kind) {
      case EPI_STORE: return dispatch<true, false, EPI_STORE>(g, batch, s);
      case EPI_DGELU: return dispatch<true, false, EPI_DGELU>(g, batch, s);
    }
  } else if (!a_k && !b_k) {  // weight gradients (dY^T X), P^T dC, dS^T Q
    switch (kind) {
      case EPI_STORE: return dispatch<false, false, EPI_STORE>(g, batch, s);
      case EPI_STORE_F32: return dispatch<false, false, EPI_STORE_F32>(g, batch, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace mt
