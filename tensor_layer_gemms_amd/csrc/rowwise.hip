// HBM-bound kernels of the layer shard. Every row kernel reads and writes with 16-byte
// vectors along the contiguous hidden dimension and reduces with wavefront shuffles
// plus one LDS exchange per block; reductions have a fixed order (no atomics), so the
// results are bitwise reproducible.
#include <type_traits>

#include "device_common.hpp"
#include "rowwise.hpp"

namespace mt {

namespace {

// ------------------------------------------------------------------ LayerNorm forward
// LayerNorm is one of the fused element-wise operations ("In-Depth Analysis of
// Distributed Training Frameworks ... Megatron-LM", oreateai.com, section 2.2). One
// block per row, 8-element chunks; the row stays in registers between the mean,
// variance and output passes. With ADD the residual sum x + o + bias is formed in fp32,
// written to the fp32 residual stream x2, and normalised without rounding.
template <typename T, bool ADD, int CPT, int NT>
__global__ __launch_bounds__(NT) void ln_fwd_kernel(const T* __restrict__ x, const T* __restrict__ o,
                                                            const T* __restrict__ bias, const T* __restrict__ gamma,
                                                            const T* __restrict__ beta, float* __restrict__ x2,
                                                            T* __restrict__ y, T* __restrict__ ylo,
                                                            float* __restrict__ mean, float* __restrict__ rstd, int h,
                                                            float eps) {
  constexpr int NW = NT / 64;
  __shared__ float red[NW];
  const int64_t row = blockIdx.x;
  const int nch = h / 8;
  float v[CPT][8], ov[CPT][8], bv[CPT][8];
  float s = 0.f;
  // every load first (clamped chunk indices keep idle chunks' loads in bounds)
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int chc = min((int)threadIdx.x + c * NT, nch - 1);
    const int64_t off = row * h + (int64_t)chc * 8;
    load8(x + off, v[c]);
    if constexpr (ADD) {
      load8(o + off, ov[c]);
      load8(bias + chc * 8, bv[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * NT;
    if (ch < nch) {
      if constexpr (ADD) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[c][e] += ov[c][e] + bv[c][e];
        store8(x2 + row * h + (int64_t)ch * 8, v[c]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[c][e];
    }
  }
  block_sum<1, NW>(&s, red);
  const float mu = s / (float)h;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * NT;
    if (ch < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dlt = v[c][e] - mu;
        q += dlt * dlt;
      }
    }
  }
  block_sum<1, NW>(&q, red);
  const float rs = 1.0f / sqrtf(q / (float)h + eps);
  if (threadIdx.x == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * NT;
    if (ch < nch) {
      float gv[8], bv[8], out[8];
      load8(gamma + ch * 8, gv);
      load8(beta + ch * 8, bv);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = (v[c][e] - mu) * rs * gv[e] + bv[e];
      store8(y + row * h + (int64_t)ch * 8, out);
      if (ylo) {
        float lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = out[e] - to_f32(from_f32<T>(out[e]));
        store8(ylo + row * h + (int64_t)ch * 8, lo);
      }
    }
  }
}

// ------------------------------------------------------------------ LayerNorm backward
// dx = resid + rstd * (g - mean(g) - xhat * mean(g * xhat)), g = dy * gamma.
template <typename T, typename TX, typename TR, int CPT, int NT>
__global__ __launch_bounds__(NT) void ln_bwd_kernel(const T* __restrict__ dy, const TX* __restrict__ x,
                                                            const T* __restrict__ gamma,
                                                            const float* __restrict__ mean,
                                                            const float* __restrict__ rstd,
                                                            const TR* __restrict__ resid, T* __restrict__ dx,
                                                            float* __restrict__ dxf, int h) {
  constexpr int NW = NT / 64;
  __shared__ float red[2 * NW];
  const int64_t row = blockIdx.x;
  const int nch = h / 8;
  const float mu = mean[row], rs = rstd[row];
  // Every load first (clamped chunk indices keep idle chunks' loads in bounds); above 4
  // chunks per thread the residual is loaded after the reduction, to stay in registers.
  constexpr bool kResidFirst = CPT <= 4;
  float g[CPT][8], xh[CPT][8], gv[CPT][8], rv[CPT][8];
  float s[2] = {0.f, 0.f};
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int chc = min((int)threadIdx.x + c * NT, nch - 1);
    const int64_t off = row * h + (int64_t)chc * 8;
    load8(dy + off, g[c]);
    load8(x + off, xh[c]);
    load8(gamma + chc * 8, gv[c]);
    if constexpr (kResidFirst) load8(resid + off, rv[c]);
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * NT;
    if (ch < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        g[c][e] *= gv[c][e];
        xh[c][e] = (xh[c][e] - mu) * rs;
        s[0] += g[c][e];
        s[1] += g[c][e] * xh[c][e];
      }
    }
  }
  block_sum<2, NW>(s, red);
  const float mg = s[0] / (float)h, mgx = s[1] / (float)h;
  if constexpr (!kResidFirst) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      load8(resid + row * h + (int64_t)min((int)threadIdx.x + c * NT, nch - 1) * 8, rv[c]);
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * NT;
    if (ch < nch) {
      const int64_t off = row * h + (int64_t)ch * 8;
      float out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = rv[c][e] + rs * (g[c][e] - mg - xh[c][e] * mgx);
      store8(dx + off, out);
      if (dxf) store8(dxf + off, out);
    }
  }
}

// LayerNorm backward fused with its column reductions. A block walks `rpb` consecutive
// rows (the row math is ln_bwd_kernel's) and keeps, per thread and column, the sums
// over its rows of dy * xhat (d gamma), dy (d beta), with DSUM dx (the bias gradient of
// the sublayer whose output dx is) and with RSUM the residual input resid (the bias
// gradient of the sublayer whose output gradient resid is: dOut for LayerNorm 2); it
// writes them as one partial row per sum and block, which colsum_final_kernel adds in a
// fixed order. The rows' inputs are read once, where separate column-sum launches would
// read dy, x, dx and resid again.
template <typename T, typename TX, typename TR, int CPT, bool DSUM, bool RSUM, int NT>
__global__ __launch_bounds__(NT) void ln_bwd_sums_kernel(const T* __restrict__ dy, const TX* __restrict__ x,
                                                                 const T* __restrict__ gamma,
                                                                 const float* __restrict__ mean,
                                                                 const float* __restrict__ rstd,
                                                                 const TR* __restrict__ resid, T* __restrict__ dx,
                                                                 float* __restrict__ dxf, float* __restrict__ part,
                                                                 int rows, int h, int rpb) {
  constexpr int NW = NT / 64;
  constexpr int NS = 2 + (DSUM ? 1 : 0) + (RSUM ? 1 : 0);
  __shared__ float red[2 * NW];
  const int nch = h / 8;
  const int r0 = blockIdx.x * rpb, r1 = min(rows, r0 + rpb);
  float acc[NS][CPT][8];
#pragma unroll
  for (int k = 0; k < NS; ++k)
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[k][c][e] = 0.f;
  // Every load of a row is issued before any of its arithmetic (clamped chunk indices
  // keep the loads of idle chunks in bounds); gamma is loaded once per block where the
  // registers allow (up to 3 chunks per thread), else with each row.
  constexpr bool kGammaOnce = CPT <= 3;
  static_assert(CPT <= 3 || !RSUM, "the residual's column sum rides along up to 3 chunks per thread");
  float gv[CPT][8];
  if constexpr (kGammaOnce) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) load8(gamma + min((int)threadIdx.x + c * NT, nch - 1) * 8, gv[c]);
  }
  for (int row = r0; row < r1; ++row) {
    const float mu = mean[row], rs = rstd[row];
    float g[CPT][8], xh[CPT][8], rv[CPT][8];
    float s[2] = {0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chc = min((int)threadIdx.x + c * NT, nch - 1);
      const int64_t off = (int64_t)row * h + (int64_t)chc * 8;
      load8(dy + off, g[c]);
      load8(x + off, xh[c]);
      if constexpr (kGammaOnce) load8(resid + off, rv[c]);  // else after the reduction
      else load8(gamma + chc * 8, gv[c]);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = threadIdx.x + c * NT;
      if (ch < nch) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xh[c][e] = (xh[c][e] - mu) * rs;
          acc[0][c][e] += g[c][e] * xh[c][e];
          acc[1][c][e] += g[c][e];
          if constexpr (RSUM) acc[NS - 1][c][e] += rv[c][e];
          g[c][e] *= gv[c][e];
          s[0] += g[c][e];
          s[1] += g[c][e] * xh[c][e];
        }
      }
    }
    block_sum<2, NW>(s, red);
    const float mg = s[0] / (float)h, mgx = s[1] / (float)h;
    if constexpr (!kGammaOnce) {
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        load8(resid + (int64_t)row * h + (int64_t)min((int)threadIdx.x + c * NT, nch - 1) * 8, rv[c]);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = threadIdx.x + c * NT;
      if (ch < nch) {
        const int64_t off = (int64_t)row * h + (int64_t)ch * 8;
        float out[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = rv[c][e] + rs * (g[c][e] - mg - xh[c][e] * mgx);
        store8(dx + off, out);
        if (dxf) store8(dxf + off, out);
        if constexpr (DSUM) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[2][c][e] += out[e];
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NS; ++k)
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = threadIdx.x + c * NT;
      if (ch < nch) store8(part + ((int64_t)k * gridDim.x + blockIdx.x) * h + (int64_t)ch * 8, acc[k][c]);
    }
}

// ------------------------------------------------------------------ column sums
// Stage 1: block (64 column chunks of 8 x 4 row lanes) sums a slab of rows per column.
template <typename TA, typename TX, int MODE>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const TA* __restrict__ a, const TX* __restrict__ x,
                                                             const float* __restrict__ mean,
                                                             const float* __restrict__ rstd,
                                                             float* __restrict__ part, int rows, int cols,
                                                             int rows_per_block, int nrb) {
  constexpr int NS = MODE == 1 ? 2 : 1;
  __shared__ float red[NS][4][64][8];
  const int lane = threadIdx.x & 63, rl = threadIdx.x >> 6;
  const int chunk = blockIdx.x * 64 + lane;
  const int nch = cols / 8;
  const int r0 = blockIdx.y * rows_per_block, r1 = min(rows, r0 + rows_per_block);
  float acc[NS][8];
#pragma unroll
  for (int k = 0; k < NS; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
  if (chunk < nch) {
#pragma unroll 4
    for (int r = r0 + rl; r < r1; r += 4) {
      const int64_t off = (int64_t)r * cols + (int64_t)chunk * 8;
      float av[8];
      load8(a + off, av);
      if constexpr (MODE == 1) {
        float xv[8];
        load8(x + off, xv);
        const float mu = mean[r], rs = rstd[r];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[0][e] += av[e] * ((xv[e] - mu) * rs);
          acc[1][e] += av[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[0][e] += av[e];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NS; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[k][rl][lane][e] = acc[k][e];
  __syncthreads();
  if (rl == 0 && chunk < nch) {
#pragma unroll
    for (int k = 0; k < NS; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = red[k][0][lane][e] + red[k][1][lane][e] + red[k][2][lane][e] + red[k][3][lane][e];
        part[((int64_t)k * nrb + blockIdx.y) * cols + (int64_t)chunk * 8 + e] = t;
      }
  }
}

// Stage 2: sum the row-slab partials of `nsum` (1 to 4) column sums, partial k of slab b
// at part[(k nrb + b) cols + c] (cols a multiple of 4, 16-byte aligned rows). A block owns
// 256 columns of one sum, 4 per lane (16-byte loads); its 16 waves take slabs w, w + 16,
// ..., in eight interleaved chains (eight loads in flight per lane: the pass is bound by
// load latency, not bandwidth), then the waves' sums are added in wave order. The order
// depends on the geometry only.
constexpr int kFinalWaves = 16;
__global__ __launch_bounds__(64 * kFinalWaves) void colsum_final_kernel(const float* __restrict__ part,
                                                                        float* __restrict__ out0,
                                                                        float* __restrict__ out1,
                                                                        float* __restrict__ out2,
                                                                        float* __restrict__ out3, int nrb, int cols) {
  constexpr int W = kFinalWaves;
  __shared__ f32x4 red[W][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int k = blockIdx.y;
  const int c = (blockIdx.x * 64 + lane) * 4;
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (c < cols) {
    const float* p = part + (int64_t)k * nrb * cols + c;
    int b = w;
    for (; b + 7 * W < nrb; b += 8 * W) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += *reinterpret_cast<const f32x4*>(p + (int64_t)(b + j * W) * cols);
    }
    for (; b < nrb; b += W) acc[0] += *reinterpret_cast<const f32x4*>(p + (int64_t)b * cols);
  }
  red[w][lane] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  if (w == 0 && c < cols) {
    f32x4 t = red[0][lane];
#pragma unroll
    for (int i = 1; i < W; ++i) t += red[i][lane];
    float* out = k == 0 ? out0 : k == 1 ? out1 : k == 2 ? out2 : out3;
    *reinterpret_cast<f32x4*>(out + c) = t;
  }
}

// Grid of colsum_final_kernel: 256 columns per block along x, one sum per y.
dim3 colsum_final_grid(int cols, int nsum) { return dim3((unsigned)((cols / 4 + 63) / 64), (unsigned)nsum); }

// ------------------------------------------------------------------ bias + residual
template <typename T>
__global__ __launch_bounds__(256) void add_bias_residual_kernel(const float* __restrict__ x2, const T* __restrict__ y,
                                                                const T* __restrict__ bias, T* __restrict__ out,
                                                                int64_t nchunks, int hch) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nchunks) return;
  float a[8], b[8], c[8];
  load8(x2 + i * 8, a);
  load8(y + i * 8, b);
  load8(bias + (i % hch) * 8, c);
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] += b[e] + c[e];
  store8(out + i * 8, a);
}

// ------------------------------------------------------------------ QKV finish
// One thread per 8 consecutive columns of one row (n and seg_n multiples of 8).
__global__ __launch_bounds__(256) void qkv_finish_kernel(const float* __restrict__ hi, const float* __restrict__ lo,
                                                         const bf16* __restrict__ bias, bf16* __restrict__ qkv,
                                                         bf16* __restrict__ qkv_lo, int64_t nchunks, int n,
                                                         int seg_n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nchunks) return;
  const int cpr = n / 8;
  const int64_t r = i / cpr;
  const int c = (int)(i % cpr) * 8;
  float v[8], b[8];
  load8(hi + r * n + c, v);
  load8(bias + c, b);
  if (c < seg_n) {
    float l[8];
    load8(lo + r * seg_n + c, l);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (v[e] + l[e]) + b[e];
    float h8[8], r8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h8[e] = to_f32(from_f32<bf16>(v[e]));
      r8[e] = v[e] - h8[e];
    }
    store8(qkv + r * n + c, h8);
    store8(qkv_lo + r * n + c, r8);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += b[e];
    store8(qkv + r * n + c, v);
  }
}

// ------------------------------------------------------------------ causal softmax
// One wavefront per score row; row q keeps keys j <= q. The row max and the sum of
// exponentials are wavefront reductions; all arithmetic is fp32.
template <typename TP, int NV>
__global__ __launch_bounds__(256) void softmax_causal_kernel(const float* __restrict__ S, TP* __restrict__ P,
                                                             int seq, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int q = (int)(row % seq);
  const float* sr = S + row * seq;
  TP* pr = P + row * seq;
  const int W = min(seq, ((q + 1 + 255) / 256) * 256);
  float v[NV][4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c <= q) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(sr + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[i][e] = (c + e <= q) ? t[e] : -INFINITY;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[i][e] = -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) mx = fmaxf(mx, v[i][e]);
  }
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[i][e] = __expf(v[i][e] - mx);  // masked entries: exp(-inf) = 0
      sum += v[i][e];
    }
  sum = wave_sum(sum);
  const float inv = 1.0f / sum;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = (i * 64 + lane) * 4;
    if (c < W) {
      if constexpr (sizeof(TP) == 2) {
        u32x2 w;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const bf16 lo = (bf16)(v[i][2 * e] * inv), hi = (bf16)(v[i][2 * e + 1] * inv);
          w[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *reinterpret_cast<u32x2*>(pr + c) = w;
      } else {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = v[i][e] * inv;
        *reinterpret_cast<f32x4*>(pr + c) = w;
      }
    }
  }
}

// ------------------------------------------------------------------ attention row dot
// D[b, k, q] = sum_c dctx[r, k, c] ctx[r, k, c], r = b seq + q. The (row, head) pairs are
// the rows of a contiguous [rows * heads, d] matrix; 16 lanes share a pair, each summing
// its 16-byte chunks c = lane, lane + 16, ..., so a wave reads 4 pairs' elements
// contiguously; the 16 lanes' sums are added by shuffles in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void attn_rowdot_kernel(const T* __restrict__ dctx, const T* __restrict__ ctx,
                                                          float* __restrict__ D, int64_t nrows, int seq, int heads,
                                                          int d) {
  const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  const bool ok = t < nrows * heads;  // no early exit: every lane takes part in the shuffles
  float s = 0.f;
  if (ok) {
    const int64_t base = t * d;
    for (int c = sub * 8; c < d; c += 128) {
      float a[8], b[8];
      load8(dctx + base + c, a);
      load8(ctx + base + c, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += a[e] * b[e];
    }
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (ok && sub == 0) {
    const int64_t r = t / heads;
    const int k = (int)(t % heads);
    const int64_t b = r / seq, q = r % seq;
    D[(b * heads + k) * seq + q] = s;
  }
}

// Threads per row block of the LayerNorm forward and the unfused backward: 512, or 128 /
// 256 where the row has no more 8-element chunks than that (narrow rows, one chunk per
// thread; at h = 1024 the LN1 forward 13.9 -> 8.9 us, add + LN2 15.8 -> 12.7 us).
int ln_threads(int h) {
  const int nch = h / 8;
  return nch <= 128 ? 128 : nch <= 256 ? 256 : kLnThreads;
}

int ln_cpt(int h) {
  const int nch = h / 8;
  const int need = (nch + kLnThreads - 1) / kLnThreads;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
}

void colsum_geometry(int rows, int cols, int& xblocks, int& rpb, int& nrb) {
  const int nch = cols / 8;
  xblocks = (nch + 63) / 64;
  int want = (2048 + xblocks - 1) / xblocks;
  const int cap = (rows + 15) / 16;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  rpb = (rows + want - 1) / want;
  nrb = (rows + rpb - 1) / rpb;
}

template <typename T, bool ADD, int CPT, int NT>
void ln_fwd_launch(const void* x, const void* o, const void* bias, const void* gamma, const void* beta, float* x2,
                   void* y, void* ylo, float* mean, float* rstd, int rows, int h, float eps, hipStream_t s) {
  hipLaunchKernelGGL((ln_fwd_kernel<T, ADD, CPT, NT>), dim3(rows), dim3(NT), 0, s, (const T*)x, (const T*)o,
                     (const T*)bias, (const T*)gamma, (const T*)beta, x2, (T*)y, (T*)ylo, mean, rstd, h, eps);
}

template <typename T, bool ADD>
hipError_t ln_fwd_t(const void* x, const void* o, const void* bias, const void* gamma, const void* beta, float* x2,
                    void* y, void* ylo, float* mean, float* rstd, int rows, int h, float eps, hipStream_t s) {
  switch (ln_threads(h) < kLnThreads ? -ln_threads(h) : ln_cpt(h)) {
    case -128: ln_fwd_launch<T, ADD, 1, 128>(x, o, bias, gamma, beta, x2, y, ylo, mean, rstd, rows, h, eps, s); break;
    case -256: ln_fwd_launch<T, ADD, 1, 256>(x, o, bias, gamma, beta, x2, y, ylo, mean, rstd, rows, h, eps, s); break;
    case 1: ln_fwd_launch<T, ADD, 1, kLnThreads>(x, o, bias, gamma, beta, x2, y, ylo, mean, rstd, rows, h, eps, s); break;
    case 2: ln_fwd_launch<T, ADD, 2, kLnThreads>(x, o, bias, gamma, beta, x2, y, ylo, mean, rstd, rows, h, eps, s); break;
    case 4: ln_fwd_launch<T, ADD, 4, kLnThreads>(x, o, bias, gamma, beta, x2, y, ylo, mean, rstd, rows, h, eps, s); break;
    default: ln_fwd_launch<T, ADD, 8, kLnThreads>(x, o, bias, gamma, beta, x2, y, ylo, mean, rstd, rows, h, eps, s); break;
  }
  return hipGetLastError();
}

template <typename T, typename TX, typename TR, int CPT, int NT>
void ln_bwd_launch(const void* dy, const void* x, const void* gamma, const float* mean, const float* rstd,
                   const void* resid, void* dx, float* dxf, int rows, int h, hipStream_t s) {
  hipLaunchKernelGGL((ln_bwd_kernel<T, TX, TR, CPT, NT>), dim3(rows), dim3(NT), 0, s, (const T*)dy,
                     (const TX*)x, (const T*)gamma, mean, rstd, (const TR*)resid, (T*)dx, dxf, h);
}

template <typename T, typename TX, typename TR>
hipError_t ln_bwd_t(const void* dy, const void* x, const void* gamma, const float* mean, const float* rstd,
                    const void* resid, void* dx, float* dxf, int rows, int h, hipStream_t s) {
  switch (ln_threads(h) < kLnThreads ? -ln_threads(h) : ln_cpt(h)) {
    case -128: ln_bwd_launch<T, TX, TR, 1, 128>(dy, x, gamma, mean, rstd, resid, dx, dxf, rows, h, s); break;
    case -256: ln_bwd_launch<T, TX, TR, 1, 256>(dy, x, gamma, mean, rstd, resid, dx, dxf, rows, h, s); break;
    case 1: ln_bwd_launch<T, TX, TR, 1, kLnThreads>(dy, x, gamma, mean, rstd, resid, dx, dxf, rows, h, s); break;
    case 2: ln_bwd_launch<T, TX, TR, 2, kLnThreads>(dy, x, gamma, mean, rstd, resid, dx, dxf, rows, h, s); break;
    case 4: ln_bwd_launch<T, TX, TR, 4, kLnThreads>(dy, x, gamma, mean, rstd, resid, dx, dxf, rows, h, s); break;
    default: ln_bwd_launch<T, TX, TR, 8, kLnThreads>(dy, x, gamma, mean, rstd, resid, dx, dxf, rows, h, s); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t ln_bwd_dispatch(const void* dy, const void* x, bool x_f32, const void* gamma, const float* mean,
                           const float* rstd, const void* resid, bool resid_f32, void* dx, float* dxf, int rows,
                           int h, hipStream_t s) {
  if (x_f32 && !resid_f32) return ln_bwd_t<T, float, T>(dy, x, gamma, mean, rstd, resid, dx, dxf, rows, h, s);
  if (!x_f32 && resid_f32) return ln_bwd_t<T, T, float>(dy, x, gamma, mean, rstd, resid, dx, dxf, rows, h, s);
  if (x_f32 && resid_f32) return ln_bwd_t<T, float, float>(dy, x, gamma, mean, rstd, resid, dx, dxf, rows, h, s);
  return ln_bwd_t<T, T, T>(dy, x, gamma, mean, rstd, resid, dx, dxf, rows, h, s);
}

// Rows per block of the fused LayerNorm backward: about 256 blocks (one per CU).
int ln_sums_rpb(int rows) { return rows <= 256 ? 1 : (rows + 255) / 256; }

template <typename T, typename TX, typename TR, int CPT, int NT>
hipError_t ln_bwd_sums_launch(const void* dy, const void* x, const void* gamma, const float* mean, const float* rstd,
                              const void* resid, void* dx, float* dxf, float* part, float* dgamma, float* dbeta,
                              float* dsum, float* rsum, int rows, int h, hipStream_t s) {
  const int rpb = ln_sums_rpb(rows), nblk = (rows + rpb - 1) / rpb;
  // The residual's column sum rides along up to 3 chunks per thread (h <= 12288); with 4
  // its accumulators would spill, and it runs as a separate column sum after the pass.
  constexpr bool kFuseR = CPT <= 3;
  const bool fr = kFuseR && rsum != nullptr;
  auto go = [&](auto dflag, auto rflag) {
    hipLaunchKernelGGL((ln_bwd_sums_kernel<T, TX, TR, CPT, decltype(dflag)::value, decltype(rflag)::value, NT>),
                       dim3(nblk), dim3(NT), 0, s, (const T*)dy, (const TX*)x, (const T*)gamma, mean, rstd,
                       (const TR*)resid, (T*)dx, dxf, part, rows, h, rpb);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if constexpr (kFuseR) {
    if (dsum && fr) go(T_{}, T_{});
    else if (dsum) go(T_{}, F_{});
    else if (fr) go(F_{}, T_{});
    else go(F_{}, F_{});
  } else {
    if (dsum) go(T_{}, F_{});
    else go(F_{}, F_{});
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* out2 = dsum ? dsum : (fr ? rsum : nullptr);
  float* out3 = dsum && fr ? rsum : nullptr;
  hipLaunchKernelGGL(colsum_final_kernel, colsum_final_grid(h, 2 + (dsum ? 1 : 0) + (fr ? 1 : 0)),
                     dim3(64 * kFinalWaves), 0, s, part, dgamma, dbeta, out2, out3, nblk, h);
  e = hipGetLastError();
  if (e != hipSuccess || !rsum || fr) return e;
  return launch_colsum(std::is_same<T, bf16>::value, 0, resid, std::is_same<TR, float>::value, nullptr, false, nullptr,
                       nullptr, rsum, nullptr, part, rows, h, s);
}

template <typename T, typename TX, typename TR>
hipError_t ln_bwd_sums_t(const void* dy, const void* x, const void* gamma, const float* mean, const float* rstd,
                         const void* resid, void* dx, float* dxf, float* part, float* dgamma, float* dbeta, float* dsum,
                         float* rsum, int rows, int h, hipStream_t s) {
  // 512 threads at every width: narrower blocks (128 threads, 1024 blocks of 4 rows at
  // h = 1024) ran the row pass faster but left the fixed-order final pass 4x the partial
  // rows, and the two together slower.
  const int need = (h / 8 + kLnThreads - 1) / kLnThreads;
  switch (need) {
    case 1: return ln_bwd_sums_launch<T, TX, TR, 1, kLnThreads>(dy, x, gamma, mean, rstd, resid, dx, dxf, part, dgamma, dbeta, dsum, rsum, rows, h, s);
    case 2: return ln_bwd_sums_launch<T, TX, TR, 2, kLnThreads>(dy, x, gamma, mean, rstd, resid, dx, dxf, part, dgamma, dbeta, dsum, rsum, rows, h, s);
    case 3: return ln_bwd_sums_launch<T, TX, TR, 3, kLnThreads>(dy, x, gamma, mean, rstd, resid, dx, dxf, part, dgamma, dbeta, dsum, rsum, rows, h, s);
    case 4: return ln_bwd_sums_launch<T, TX, TR, 4, kLnThreads>(dy, x, gamma, mean, rstd, resid, dx, dxf, part, dgamma, dbeta, dsum, rsum, rows, h, s);
    default: return hipErrorNotSupported;
  }
}

template <typename T>
hipError_t ln_bwd_sums_dispatch(const void* dy, const void* x, bool x_f32, const void* gamma, const float* mean,
                                const float* rstd, const void* resid, bool resid_f32, void* dx, float* dxf,
                                float* part, float* dgamma, float* dbeta, float* dsum, float* rsum, int rows, int h,
                                hipStream_t s) {
  if (x_f32 && !resid_f32)
    return ln_bwd_sums_t<T, float, T>(dy, x, gamma, mean, rstd, resid, dx, dxf, part, dgamma, dbeta, dsum, rsum, rows,
                                      h, s);
  if (!x_f32 && resid_f32)
    return ln_bwd_sums_t<T, T, float>(dy, x, gamma, mean, rstd, resid, dx, dxf, part, dgamma, dbeta, dsum, rsum, rows,
                                      h, s);
  if (x_f32 && resid_f32)
    return ln_bwd_sums_t<T, float, float>(dy, x, gamma, mean, rstd, resid, dx, dxf, part, dgamma, dbeta, dsum, rsum,
                                          rows, h, s);
  return ln_bwd_sums_t<T, T, T>(dy, x, gamma, mean, rstd, resid, dx, dxf, part, dgamma, dbeta, dsum, rsum, rows, h, s);
}

template <typename TA, typename TX>
hipError_t colsum_t(int mode, const void* a, const void* x, const float* mean, const float* rstd, float* out0,
                    float* out1, float* partial, int rows, int cols, hipStream_t s) {
  int xb, rpb, nrb;
  colsum_geometry(rows, cols, xb, rpb, nrb);
  if (mode == 1)
    hipLaunchKernelGGL((colsum_partial_kernel<TA, TX, 1>), dim3(xb, nrb), dim3(256), 0, s, (const TA*)a,
                       (const TX*)x, mean, rstd, partial, rows, cols, rpb, nrb);
  else
    hipLaunchKernelGGL((colsum_partial_kernel<TA, TX, 0>), dim3(xb, nrb), dim3(256), 0, s, (const TA*)a,
                       (const TX*)x, mean, rstd, partial, rows, cols, rpb, nrb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colsum_final_kernel, colsum_final_grid(cols, mode == 1 ? 2 : 1), dim3(64 * kFinalWaves), 0, s,
                     partial, out0, out1, nullptr, nullptr, nrb, cols);
  return hipGetLastError();
}

template <typename TP>
hipError_t softmax_t(const float* S, void* P, int nmat, int seq, hipStream_t s) {
  const int64_t rows = (int64_t)nmat * seq;
  const dim3 grid((unsigned)((rows + 3) / 4));
  TP* p = (TP*)P;
  if (seq <= 256) hipLaunchKernelGGL((softmax_causal_kernel<TP, 1>), grid, dim3(256), 0, s, S, p, seq, rows);
  else if (seq <= 512) hipLaunchKernelGGL((softmax_causal_kernel<TP, 2>), grid, dim3(256), 0, s, S, p, seq, rows);
  else if (seq <= 1024) hipLaunchKernelGGL((softmax_causal_kernel<TP, 4>), grid, dim3(256), 0, s, S, p, seq, rows);
  else if (seq <= 2048) hipLaunchKernelGGL((softmax_causal_kernel<TP, 8>), grid, dim3(256), 0, s, S, p, seq, rows);
  else hipLaunchKernelGGL((softmax_causal_kernel<TP, 16>), grid, dim3(256), 0, s, S, p, seq, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ln_fwd(bool is_bf16, const void* x, const void* gamma, const void* beta, void* y, void* y_lo,
                         float* mean, float* rstd, int rows, int h, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return is_bf16
             ? ln_fwd_t<bf16, false>(x, nullptr, nullptr, gamma, beta, nullptr, y, y_lo, mean, rstd, rows, h, eps, s)
             : ln_fwd_t<float, false>(x, nullptr, nullptr, gamma, beta, nullptr, y, nullptr, mean, rstd, rows, h, eps,
                                      s);
}

hipError_t launch_add_ln_fwd(bool is_bf16, const void* x, const void* o, const void* bias, const void* gamma,
                             const void* beta, float* x2, void* y, float* mean, float* rstd, int rows, int h,
                             float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return is_bf16 ? ln_fwd_t<bf16, true>(x, o, bias, gamma, beta, x2, y, nullptr, mean, rstd, rows, h, eps, s)
                 : ln_fwd_t<float, true>(x, o, bias, gamma, beta, x2, y, nullptr, mean, rstd, rows, h, eps, s);
}

hipError_t launch_ln_bwd(bool is_bf16, const void* dy, const void* x, bool x_f32, const void* gamma,
                         const float* mean, const float* rstd, const void* resid, bool resid_f32, void* dx,
                         float* dx_f32, int rows, int h, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return is_bf16 ? ln_bwd_dispatch<bf16>(dy, x, x_f32, gamma, mean, rstd, resid, resid_f32, dx, dx_f32, rows, h, s)
                 : ln_bwd_dispatch<float>(dy, x, x_f32, gamma, mean, rstd, resid, resid_f32, dx, dx_f32, rows, h, s);
}

bool ln_bwd_sums_supported(int h) { return h % 8 == 0 && (h / 8 + kLnThreads - 1) / kLnThreads <= 4; }

size_t ln_bwd_sums_partial_floats(int rows, int h, int nsum) {
  const int rpb = ln_sums_rpb(rows);
  return (size_t)nsum * ((rows + rpb - 1) / rpb) * h;
}

hipError_t launch_ln_bwd_sums(bool is_bf16, const void* dy, const void* x, bool x_f32, const void* gamma,
                              const float* mean, const float* rstd, const void* resid, bool resid_f32, void* dx,
                              float* dx_f32, float* part, float* dgamma, float* dbeta, float* dsum, float* rsum,
                              int rows, int h, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (!ln_bwd_sums_supported(h)) return hipErrorNotSupported;
  return is_bf16 ? ln_bwd_sums_dispatch<bf16>(dy, x, x_f32, gamma, mean, rstd, resid, resid_f32, dx, dx_f32, part,
                                              dgamma, dbeta, dsum, rsum, rows, h, s)
                 : ln_bwd_sums_dispatch<float>(dy, x, x_f32, gamma, mean, rstd, resid, resid_f32, dx, dx_f32, part,
                                               dgamma, dbeta, dsum, rsum, rows, h, s);
}

size_t colsum_partial_floats(int rows, int cols, int mode) {
  int xb, rpb, nrb;
  colsum_geometry(rows, cols, xb, rpb, nrb);
  return (size_t)nrb * cols * (mode == 1 ? 2 : 1);
}

hipError_t launch_colsum_final(const float* part, float* out, int nrb, int cols, hipStream_t s) {
  if (nrb <= 0 || cols <= 0) return hipSuccess;
  if (cols % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(colsum_final_kernel, colsum_final_grid(cols, 1), dim3(64 * kFinalWaves), 0, s, part, out, nullptr,
                     nullptr, nullptr, nrb, cols);
  return hipGetLastError();
}

hipError_t launch_colsum(bool is_bf16, int mode, const void* a, bool a_f32, const void* x, bool x_f32,
                         const float* mean, const float* rstd, float* out0, float* out1, float* partial, int rows,
                         int cols, hipStream_t s) {
  if (cols <= 0) return hipSuccess;
  if (cols % 8 != 0) return hipErrorInvalidValue;  // 8-column chunks in both passes
  if (!is_bf16 || (a_f32 && (mode == 0 || x_f32)))
    return colsum_t<float, float>(mode, a, x, mean, rstd, out0, out1, partial, rows, cols, s);
  if (a_f32) return colsum_t<float, bf16>(mode, a, x, mean, rstd, out0, out1, partial, rows, cols, s);
  if (mode == 1 && x_f32) return colsum_t<bf16, float>(mode, a, x, mean, rstd, out0, out1, partial, rows, cols, s);
  return colsum_t<bf16, bf16>(mode, a, x, mean, rstd, out0, out1, partial, rows, cols, s);
}

hipError_t launch_add_bias_residual(bool is_bf16, const float* x2, const void* y, const void* bias, void* out,
                                    int rows, int h, hipStream_t s) {
  const int64_t n = (int64_t)rows * h / 8;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (is_bf16)
    hipLaunchKernelGGL(add_bias_residual_kernel<bf16>, grid, dim3(256), 0, s, x2, (const bf16*)y, (const bf16*)bias,
                       (bf16*)out, n, h / 8);
  else
    hipLaunchKernelGGL(add_bias_residual_kernel<float>, grid, dim3(256), 0, s, x2, (const float*)y,
                       (const float*)bias, (float*)out, n, h / 8);
  return hipGetLastError();
}

hipError_t launch_softmax_causal(bool is_bf16, const float* S, void* P, int nmat, int seq, hipStream_t s) {
  if (nmat <= 0) return hipSuccess;
  return is_bf16 ? softmax_t<bf16>(S, P, nmat, seq, s) : softmax_t<float>(S, P, nmat, seq, s);
}

hipError_t launch_qkv_finish(const float* hi, const float* lo, const void* bias, void* qkv, void* qkv_lo, int rows,
                             int n, int seg_n, hipStream_t s) {
  if (n % 8 || seg_n % 8 || seg_n > n) return hipErrorInvalidValue;
  const int64_t nchunks = (int64_t)rows * (n / 8);
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(qkv_finish_kernel, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, s, hi, lo,
                     (const bf16*)bias, (bf16*)qkv, (bf16*)qkv_lo, nchunks, n, seg_n);
  return hipGetLastError();
}

hipError_t launch_attn_rowdot(bool is_bf16, const void* dctx, const void* ctx, float* D, int batch, int seq, int heads,
                              int d, hipStream_t s) {
  const int64_t nrows = (int64_t)batch * seq;
  const int64_t n = nrows * heads;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 15) / 16));  // 16 lanes per (row, head)
  if (is_bf16)
    hipLaunchKernelGGL(attn_rowdot_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)dctx, (const bf16*)ctx, D, nrows,
                       seq, heads, d);
  else
    hipLaunchKernelGGL(attn_rowdot_kernel<float>, grid, dim3(256), 0, s, (const float*)dctx, (const float*)ctx, D,
                       nrows, seq, heads, d);
  return hipGetLastError();
}

}  // namespace mt
