// Host launchers of the HBM-bound kernels: LayerNorm forward/backward (with the fused
// bias + residual add), causal softmax, column sums (bias and LayerNorm parameter
// gradients), the final bias + residual add and the attention row dot.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mt {

// Largest row LayerNorm keeps in registers: 512 threads x 8 chunks of 8 elements.
constexpr int kLnThreads = 512;
constexpr int kLnChunksPerThread = 8;
constexpr int kLnMaxH = kLnThreads * kLnChunksPerThread * 8;
// Longest causal softmax row kept in registers (64 lanes x 4 x 16 values).
constexpr int kSoftmaxMaxSeq = 4096;

// T below is the activation type: bf16 (is_bf16) or fp32. The residual stream X2 and
// its gradient dX2 are kept in fp32 whatever T is.

// y = LN(x); saves the row mean and 1/sqrt(var + eps) (fp32). With y_lo (bf16 only),
// also writes the rounding remainder y_lo = bf16(y - bf16(y)).
hipError_t launch_ln_fwd(bool is_bf16, const void* x, const void* gamma, const void* beta, void* y, void* y_lo,
                         float* mean, float* rstd, int rows, int h, float eps, hipStream_t s);

// x2 = x + o + bias (fp32, unrounded), y = LN(x2).
hipError_t launch_add_ln_fwd(bool is_bf16, const void* x, const void* o, const void* bias, const void* gamma,
                             const void* beta, float* x2, void* y, float* mean, float* rstd, int rows, int h,
                             float eps, hipStream_t s);

// dx = resid + LN-backward(dy; x, gamma, mean, rstd). x / resid are fp32 when the
// matching flag is set (else type T). dx is T; dx_f32 (optional) receives an fp32 copy.
hipError_t launch_ln_bwd(bool is_bf16, const void* dy, const void* x, bool x_f32, const void* gamma,
                         const float* mean, const float* rstd, const void* resid, bool resid_f32, void* dx,
                         float* dx_f32, int rows, int h, hipStream_t s);

// LayerNorm backward (as launch_ln_bwd) fused with its column sums: dgamma[c] =
// sum_r dy[r, c] xhat[r, c], dbeta[c] = sum_r dy[r, c], when dsum is not null
// dsum[c] = sum_r dx[r, c] (the fp32 values before rounding) and when rsum is not null
// rsum[c] = sum_r resid[r, c]. `part` holds ln_bwd_sums_partial_floats(rows, h, 4) floats
// (and at least colsum_partial_floats(rows, h, 0)); fixed reduction order.
// Supported when ln_bwd_sums_supported(h) (h / 8 chunks over at most 4 per thread).
bool ln_bwd_sums_supported(int h);
size_t ln_bwd_sums_partial_floats(int rows, int h, int nsum);
hipError_t launch_ln_bwd_sums(bool is_bf16, const void* dy, const void* x, bool x_f32, const void* gamma,
                              const float* mean, const float* rstd, const void* resid, bool resid_f32, void* dx,
                              float* dx_f32, float* part, float* dgamma, float* dbeta, float* dsum, float* rsum,
                              int rows, int h, hipStream_t s);

// Column sums over `rows` rows, deterministic two-stage reduction through `partial`.
// mode 0: out0[c] = sum_r a[r, c].
// mode 1: out0[c] = sum_r a[r, c] * (x[r, c] - mean[r]) * rstd[r], out1[c] = sum_r a[r, c].
// a / x are fp32 when a_f32 / x_f32, else type T.
size_t colsum_partial_floats(int rows, int cols, int mode);
hipError_t launch_colsum(bool is_bf16, int mode, const void* a, bool a_f32, const void* x, bool x_f32,
                         const float* mean, const float* rstd, float* out0, float* out1, float* partial, int rows,
                         int cols, hipStream_t s);

// out[c] = sum over the nrb partial rows part[r, c] (fp32 [nrb][cols]), in row order.
hipError_t launch_colsum_final(const float* part, float* out, int nrb, int cols, hipStream_t s);

// out = x2 + y + bias (x2 fp32, bias broadcast over rows).
hipError_t launch_add_bias_residual(bool is_bf16, const float* x2, const void* y, const void* bias, void* out,
                                    int rows, int h, hipStream_t s);

// bf16 QKV projection from two fp32 partial products (hi: [rows, n] of U_hi W^T, lo:
// [rows, seg_n] of U_lo W^T for the first seg_n columns): v = hi + lo + bias (lo only
// for c < seg_n); qkv = bf16(v) and, for c < seg_n, qkv_lo = bf16(v - bf16(v)).
hipError_t launch_qkv_finish(const float* hi, const float* lo, const void* bias, void* qkv, void* qkv_lo, int rows,
                             int n, int seg_n, hipStream_t s);

// P = softmax over keys j <= q of S (fp32) for each of `nmat` [seq, seq] matrices;
// row q is written for j < min(seq, roundup(q + 1, 256)), zeros right of the diagonal.
hipError_t launch_softmax_causal(bool is_bf16, const float* S, void* P, int nmat, int seq, hipStream_t s);

// D[(b * heads + k) * seq + q] = sum_c dctx[b*seq+q, k*d+c] * ctx[b*seq+q, k*d+c]
// (= rowsum(P * dP) of head k, since ctx = P V and dP = dctx V^T).
hipError_t launch_attn_rowdot(bool is_bf16, const void* dctx, const void* ctx, float* D, int batch, int seq,
                              int heads, int d, hipStream_t s);

}  // namespace mt
