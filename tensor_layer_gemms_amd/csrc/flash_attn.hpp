// Fused causal attention of the layer shard's heads (bf16 path, head dim 64, 128 or 160).
//
// Forward: a work-group owns 64 query rows of one (sequence, head); four (two) groups of
// two waves stream consecutive runs of the visible keys in blocks of 32 through their own
// LDS rings (DMA loads, two stages) and merge their partial results at the end. Per block
// the logits S = Q K^T / sqrt(d) — with qkv_lo given, in the compensated form
// (Q_hi K_hi^T + Q_hi K_lo^T + Q_lo K_hi^T) / sqrt(d) — are formed on the matrix cores,
// the causal mask is applied, the running row maximum and exponential sum are updated
// (online softmax) and O += P V is accumulated with P taken straight from the logit
// accumulators (rounded to bf16 as the matrix-core operand). S and P never reach
// HBM. The forward writes ctx = O / l and the row log-sum-exp L = m + ln(l), from which
// the backward recomputes P = exp(S - L).
//
// Attention and its causal mask follow the layer definition of the "Megatron-LM" concept
// report (compassingai.com), section 4.1 (the attention heads of a rank); the fused,
// tiled form is the FlashAttention approach the same pages cite for long sequences.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mt {

struct FlashArgs {
  const void* qkv;     // [B seq, ldq] bf16: Q of head k at column k d, K at hs + k d, V at 2 hs + k d
  const void* qkv_lo;  // same layout: rounding remainders of Q and K, or null (plain Q K^T)
  void* ctx;           // [B seq, ldc] bf16: head k at column k d
  float* lse;          // [B, heads, seq] fp32 natural-log row log-sum-exp
  const void* dctx;    // backward: dL/dctx, layout of ctx
  const float* D;      // backward: rowsum(dctx * ctx) [B, heads, seq]
  void* dqkv;          // backward: layout of qkv (dQ, dK, dV of every head)
  // backward, optional: column sums of the stored (bf16) dQ, dK, dV over each block of
  // 32 rows of a sequence, fp32 [flash_dbias_rows(batch, seq)][3 hs] (row
  // b flash_dbias_rows(1, seq) + j: rows 32 j .. of sequence b, zeros past its end), for
  // the QKV bias gradient's fixed-order final sum
  float* dbias_part;
  int64_t ldq, ldc;
  int batch, heads, seq, hs;
  float scale;         // 1 / sqrt(d)
};

// Head dims the fused kernels handle (forward and backward).
inline bool flash_supported(int d) { return d == 64 || d == 128 || d == 160; }

// Forward: ctx and lse from qkv, qkv_lo (d = 64, 128 or 160).
hipError_t launch_flash_fwd(const FlashArgs& a, int d, hipStream_t s);
// Backward: dQ, dK, dV into dqkv from qkv, qkv_lo, dctx, lse and D (d = 64, 128 or 160),
// and, if dbias_part is set, their per-32-row column sums.
hipError_t launch_flash_bwd(const FlashArgs& a, int d, hipStream_t s);
// Rows of dbias_part: two per 64-row block of every sequence.
__host__ __device__ inline int64_t flash_dbias_rows(int batch, int seq) { return (int64_t)batch * 2 * ((seq + 63) / 64); }

}  // namespace mt
