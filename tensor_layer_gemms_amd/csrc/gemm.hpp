// GEMM family of the layer shard: C[m, n] = epilogue(sum_k A(m, k) B(n, k)).
//
// Every linear layer, its input-gradient (dgrad) and weight-gradient (wgrad), and the
// four attention products are instances of this one contraction; they differ in which
// index of each operand is contiguous in memory and in the fused epilogue:
//   forward  Y = X W^T          A = X  [M, K] (K-contiguous), B = W [N, K] (K-contiguous)
//   dgrad    dX = dY W          A = dY [M, K] (K-contiguous), B(n, k) = W[k, n] (N-contiguous)
//   wgrad    dW = dY^T X        A(n, m) = dY[m, n], B(k, m) = X[m, k]: both token-strided
// The split of the weights (columns of the first GEMM of a block, rows of the second)
// follows the "Megatron-LM" concept report (compassingai.com), section 4.1; only the
// operand layouts, not the arithmetic, depend on which side of the split a GEMM is.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mt {

enum EpiKind : int {
  EPI_STORE = 0,      // C = alpha * acc, stored in the activation type
  EPI_STORE_F32 = 1,  // C = alpha * acc, stored as fp32 (weight gradients, scores)
  EPI_BIAS = 2,       // C = acc + bias[n]
  EPI_BIAS_GELU = 3,  // C = a = acc + bias[n] (pre-activation, kept for backward); C2 = GeLU(a)
  EPI_DGELU = 4,      // C = acc * GeLU'(aux[m, n])            (aux = saved pre-activation)
  EPI_DSOFTMAX = 5,   // C = aux[m, n] * (acc - vec[m])        (aux = P, vec = rowsum(P * dP))
  EPI_BIAS_SPLIT = 6, // v = acc + bias[n]; C = bf16(v); for n < seg_n also C2 = bf16(v - bf16(v))
  EPI_BIAS_RESID = 7, // C = acc + bias[n] + aux[m, n]              (aux = fp32 residual, layout of C)
};

enum Causal : int {
  CAUSAL_NONE = 0,
  CAUSAL_SKIP_UPPER = 1,  // output tiles entirely above the diagonal (n0 > last m) are skipped
  CAUSAL_K_LE_M = 2,      // contraction limited to k < m0 + BM   (A = P or dS, row-major)
  CAUSAL_K_GE_M = 3,      // contraction starts at k = m0          (A = P^T or dS^T)
};

// Rows of the probability matrices (P, dS) are written for columns
// [0, min(s, roundup(q + 1, kCausalChunk))), with zeros right of the diagonal, so every
// causal consumer whose tile sizes divide kCausalChunk reads only written entries.
constexpr int kCausalChunk = 256;

// K segments (bf16 path): the contraction may run over nseg segments of K each, segment s
// reading A from seg_a[s] and B from seg_b[s] with the strides of A and B (segment 0 is
// A and B). Tiles whose first column is >= seg_n run segment 0 only, and the later
// segments read zeros for the B rows (output columns) >= seg_n of a tile that straddles
// seg_n, so no column's arithmetic depends on the tile shape. This forms
// hi/lo-compensated products, e.g. (U_hi + U_lo) W^T or Q_hi K_hi^T + Q_hi K_lo^T +
// Q_lo K_hi^T, with bf16 MFMA operands.
constexpr int kMaxSeg = 3;

struct GemmArgs {
  const void* A;
  const void* B;
  const void* seg_a[kMaxSeg];
  const void* seg_b[kMaxSeg];
  int nseg, seg_n;
  void* C;
  void* C2;         // EPI_BIAS_GELU / EPI_BIAS_SPLIT second output, same layout as C
  const void* aux;  // EPI_DGELU / EPI_DSOFTMAX input, same layout as C
  const void* vec;  // bias [N] (activation type) or fp32 row vector [M] per batch
  int64_t lda, ldb, ldc;
  // batch z = blockIdx.y; offsets (z / zdiv) * so + (z % zdiv) * si, in elements
  int64_t a_so, a_si, b_so, b_si, c_so, c_si;
  int64_t vec_bs;   // row-vector batch stride (EPI_DSOFTMAX)
  // EPI_DGELU, unbatched, bf16 launchers: if set, also the column sums of the stored
  // (bf16) C over each 128-row block of the M rows, fp32 [ceil(M / 128)][N] (the bias
  // gradient of the layer whose pre-activation gradient C is, before its final sum).
  float* colsum;
  int M, N, K, zdiv, causal;
  float alpha;
};
constexpr int kColsumRows = 128;  // rows per partial column-sum row of GemmArgs::colsum
inline size_t gemm_colsum_floats(int rows, int cols) {
  return (size_t)((rows + kColsumRows - 1) / kColsumRows) * (size_t)cols;
}

// Host launchers (gemm_*.hip). a_kcontig / b_kcontig: whether A(m, k) / B(n, k) is
// contiguous along k. Return the launch status.
hipError_t launch_gemm_bf16(const GemmArgs& g, bool a_kcontig, bool b_kcontig, int kind, int batch,
                            hipStream_t stream);
hipError_t launch_gemm_f32(const GemmArgs& g, bool a_kcontig, bool b_kcontig, int kind, int batch,
                           hipStream_t stream);
// Two independent unbatched, non-causal bf16 problems in one launch (an input gradient
// and a weight gradient of the same layer): the tiles of the deeper contraction first,
// then the other problem's, which fill the CUs the first leaves idle. Supported pairs,
// each problem addressable by the DMA kernel: (A k-contiguous, B n-contiguous; EPI_STORE
// or EPI_DGELU) with (both token-strided; EPI_STORE_F32), and two both-k-contiguous
// EPI_STORE_F32 problems. Returns hipErrorNotSupported for anything else, without
// launching; the caller then runs the two one after the other.
hipError_t launch_gemm_bf16_pair(const GemmArgs& g0, bool a_k0, bool b_k0, int kind0, const GemmArgs& g1, bool a_k1,
                                 bool b_k1, int kind1, hipStream_t stream);

// Input gradient with a deep, narrow contraction (K > 2 N): the number of k slices it is
// split into (1, 2 or 4; depends on N and K only, so every token is computed the same way
// at any batch size).
int gemm_dgrad_splits(int64_t N, int64_t K);
// k slices of a paired input gradient dg (epilogue dkind) and weight gradient wg: at most
// one of them splits (*sd or *sw > 1). An EPI_STORE input gradient splits as
// gemm_dgrad_splits says; otherwise an EPI_STORE pair's weight gradient splits its
// token dimension where its tiles are the long pole of the pair and the estimated time
// saved exceeds the slices' extra traffic (the small, deep weight gradients of narrow
// layers). Depends on the shapes only.
void gemm_pair_splits(const GemmArgs& dg, int dkind, const GemmArgs& wg, int* sd, int* sw);
// fp32 floats of `part` that launch_gemm_bf16_pair_split needs for the pair (0: no split).
int64_t gemm_pair_split_floats(const GemmArgs& dg, int dkind, const GemmArgs& wg);
// The same pairing as above for an input gradient dg (A k-contiguous, B n-contiguous,
// unbatched; epilogue dkind) and a weight gradient wg, with the problem that
// gemm_pair_splits names split into k slices written as fp32 to part ([splits, M, N])
// and summed in slice order into its C by a second pass (bf16 dg.C, fp32 wg.C).
// Returns hipErrorNotSupported (nothing launched) if neither splits or the pair does not
// qualify.
hipError_t launch_gemm_bf16_pair_split(const GemmArgs& dg, int dkind, const GemmArgs& wg, float* part,
                                       hipStream_t stream);

}  // namespace mt
