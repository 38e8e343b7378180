// HBM-bound kernels of the layer shard. Every row kernel reads and writes with 16-byte
// vectors along the contiguous hidden dimension and reduces with wavefront shuffles
// plus one LDS exchange per block; reductions have a fixed order (no atomics), so the
// results are bitwise reproducible.
#include "device_common.hpp"
#include "rowwise.hpp"

namespace mt {

namespace {

template <typename T>
using V = Vec16<T>;

// ------------------------------------------------------------------ LayerNorm forward
// LayerNorm is one of the fused element-wise operations ("In-Depth Analysis of
// Distributed Training Frameworks ... Megatron-LM", oreateai.com, section 2.2). One
// block per row; the row stays in registers between the mean, variance and output passes.
template <typename T, bool ADD, int CPT>
__global__ __launch_bounds__(kLnThreads) void ln_fwd_kernel(const T* __restrict__ x, const T* __restrict__ o,
                                                            const T* __restrict__ bias, const T* __restrict__ gamma,
                                                            const T* __restrict__ beta, T* __restrict__ x2,
                                                            T* __restrict__ y, float* __restrict__ mean,
                                                            float* __restrict__ rstd, int h, float eps) {
  constexpr int VE = V<T>::N, NW = kLnThreads / 64;
  __shared__ float red[NW];
  const int64_t row = blockIdx.x;
  const int nch = h / VE;
  float v[CPT][VE];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * kLnThreads;
    if (ch < nch) {
      const int64_t off = row * h + (int64_t)ch * VE;
      load16(x + off, v[c]);
      if constexpr (ADD) {
        float ov[VE], bv[VE];
        load16(o + off, ov);
        load16(bias + ch * VE, bv);
#pragma unroll
        for (int e = 0; e < VE; ++e) v[c][e] = to_f32(from_f32<T>(v[c][e] + ov[e] + bv[e]));
        store16(x2 + off, v[c]);  // the stored (rounded) residual is what LN and backward see
      }
#pragma unroll
      for (int e = 0; e < VE; ++e) s += v[c][e];
    }
  }
  block_sum<1, NW>(&s, red);
  const float mu = s / (float)h;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * kLnThreads;
    if (ch < nch) {
#pragma unroll
      for (int e = 0; e < VE; ++e) {
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
    const int ch = threadIdx.x + c * kLnThreads;
    if (ch < nch) {
      float gv[VE], bv[VE], out[VE];
      load16(gamma + ch * VE, gv);
      load16(beta + ch * VE, bv);
#pragma unroll
      for (int e = 0; e < VE; ++e) out[e] = (v[c][e] - mu) * rs * gv[e] + bv[e];
      store16(y + row * h + (int64_t)ch * VE, out);
    }
  }
}

// ------------------------------------------------------------------ LayerNorm backward
// dx = resid + rstd * (g - mean(g) - xhat * mean(g * xhat)), g = dy * gamma.
template <typename T, int CPT>
__global__ __launch_bounds__(kLnThreads) void ln_bwd_kernel(const T* __restrict__ dy, const T* __restrict__ x,
                                                            const T* __restrict__ gamma,
                                                            const float* __restrict__ mean,
                                                            const float* __restrict__ rstd,
                                                            const T* __restrict__ resid, T* __restrict__ dx, int h) {
  constexpr int VE = V<T>::N, NW = kLnThreads / 64;
  __shared__ float red[2 * NW];
  const int64_t row = blockIdx.x;
  const int nch = h / VE;
  const float mu = mean[row], rs = rstd[row];
  float g[CPT][VE], xh[CPT][VE];
  float s[2] = {0.f, 0.f};
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * kLnThreads;
    if (ch < nch) {
      const int64_t off = row * h + (int64_t)ch * VE;
      float gv[VE];
      load16(dy + off, g[c]);
      load16(x + off, xh[c]);
      load16(gamma + ch * VE, gv);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        g[c][e] *= gv[e];
        xh[c][e] = (xh[c][e] - mu) * rs;
        s[0] += g[c][e];
        s[1] += g[c][e] * xh[c][e];
      }
    }
  }
  block_sum<2, NW>(s, red);
  const float mg = s[0] / (float)h, mgx = s[1] / (float)h;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = threadIdx.x + c * kLnThreads;
    if (ch < nch) {
      const int64_t off = row * h + (int64_t)ch * VE;
      float rv[VE], out[VE];
      load16(resid + off, rv);
#pragma unroll
      for (int e = 0; e < VE; ++e) out[e] = rv[e] + rs * (g[c][e] - mg - xh[c][e] * mgx);
      store16(dx + off, out);
    }
  }
}

// ------------------------------------------------------------------ column sums
// Stage 1: block (64 column chunks x 4 row lanes) sums a slab of rows per column.
template <typename T, int MODE>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T* __restrict__ a, const T* __restrict__ x,
                                                             const float* __restrict__ mean,
                                                             const float* __restrict__ rstd,
                                                             float* __restrict__ part, int rows, int cols,
                                                             int rows_per_block, int nrb) {
  constexpr int VE = V<T>::N;
  constexpr int NS = MODE == 1 ? 2 : 1;
  __shared__ float red[NS][4][64][VE];
  const int lane = threadIdx.x & 63, rl = threadIdx.x >> 6;
  const int chunk = blockIdx.x * 64 + lane;
  const int nch = cols / VE;
  const int r0 = blockIdx.y * rows_per_block, r1 = min(rows, r0 + rows_per_block);
  float acc[NS][VE];
#pragma unroll
  for (int k = 0; k < NS; ++k)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[k][e] = 0.f;
  if (chunk < nch) {
    for (int r = r0 + rl; r < r1; r += 4) {
      const int64_t off = (int64_t)r * cols + (int64_t)chunk * VE;
      float av[VE];
      load16(a + off, av);
      if constexpr (MODE == 1) {
        float xv[VE];
        load16(x + off, xv);
        const float mu = mean[r], rs = rstd[r];
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          acc[0][e] += av[e] * ((xv[e] - mu) * rs);
          acc[1][e] += av[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[0][e] += av[e];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NS; ++k)
#pragma unroll
    for (int e = 0; e < VE; ++e) red[k][rl][lane][e] = acc[k][e];
  __syncthreads();
  if (rl == 0 && chunk < nch) {
#pragma unroll
    for (int k = 0; k < NS; ++k)
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const float t = red[k][0][lane][e] + red[k][1][lane][e] + red[k][2][lane][e] + red[k][3][lane][e];
        part[((int64_t)k * nrb + blockIdx.y) * cols + (int64_t)chunk * VE + e] = t;
      }
  }
}

// Stage 2: sum the row-slab partials in slab order.
__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ part, float* __restrict__ out0,
                                                           float* __restrict__ out1, int nrb, int cols, int mode) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  float s = 0.f;
  for (int b = 0; b < nrb; ++b) s += part[(int64_t)b * cols + c];
  out0[c] = s;
  if (mode == 1) {
    float t = 0.f;
    for (int b = 0; b < nrb; ++b) t += part[((int64_t)nrb + b) * cols + c];
    out1[c] = t;
  }
}

// ------------------------------------------------------------------ bias + residual
template <typename T>
__global__ __launch_bounds__(256) void add_bias_residual_kernel(const T* __restrict__ x2, const T* __restrict__ y,
                                                                const T* __restrict__ bias, T* __restrict__ out,
                                                                int64_t nchunks, int hch) {
  constexpr int VE = V<T>::N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nchunks) return;
  float a[VE], b[VE], c[VE];
  load16(x2 + i * VE, a);
  load16(y + i * VE, b);
  load16(bias + (i % hch) * VE, c);
#pragma unroll
  for (int e = 0; e < VE; ++e) a[e] += b[e] + c[e];
  store16(out + i * VE, a);
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
template <typename T>
__global__ __launch_bounds__(256) void attn_rowdot_kernel(const T* __restrict__ dctx, const T* __restrict__ ctx,
                                                          float* __restrict__ D, int64_t nrows, int seq, int heads,
                                                          int d) {
  constexpr int VE = V<T>::N;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= nrows * heads) return;
  const int64_t r = t / heads;
  const int k = (int)(t % heads);
  const int64_t base = r * (int64_t)heads * d + (int64_t)k * d;
  float s = 0.f;
  for (int c = 0; c < d; c += VE) {
    float a[VE], b[VE];
    load16(dctx + base + c, a);
    load16(ctx + base + c, b);
#pragma unroll
    for (int e = 0; e < VE; ++e) s += a[e] * b[e];
  }
  const int64_t b = r / seq, q = r % seq;
  D[(b * heads + k) * seq + q] = s;
}

int ln_cpt(int h, int ve) {
  const int nch = h / ve;
  const int need = (nch + kLnThreads - 1) / kLnThreads;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
}

void colsum_geometry(int rows, int cols, int ve, int& xblocks, int& rpb, int& nrb) {
  const int nch = cols / ve;
  xblocks = (nch + 63) / 64;
  int want = (2048 + xblocks - 1) / xblocks;
  const int cap = (rows + 15) / 16;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  rpb = (rows + want - 1) / want;
  nrb = (rows + rpb - 1) / rpb;
}

template <typename T, bool ADD>
hipError_t ln_fwd_t(const void* x, const void* o, const void* bias, const void* gamma, const void* beta, void* x2,
                    void* y, float* mean, float* rstd, int rows, int h, float eps, hipStream_t s) {
  const T *px = (const T*)x, *po = (const T*)o, *pb = (const T*)bias, *pg = (const T*)gamma, *pbe = (const T*)beta;
  T *px2 = (T*)x2, *py = (T*)y;
  switch (ln_cpt(h, V<T>::N)) {
    case 1: hipLaunchKernelGGL((ln_fwd_kernel<T, ADD, 1>), dim3(rows), dim3(kLnThreads), 0, s, px, po, pb, pg, pbe, px2, py, mean, rstd, h, eps); break;
    case 2: hipLaunchKernelGGL((ln_fwd_kernel<T, ADD, 2>), dim3(rows), dim3(kLnThreads), 0, s, px, po, pb, pg, pbe, px2, py, mean, rstd, h, eps); break;
    case 4: hipLaunchKernelGGL((ln_fwd_kernel<T, ADD, 4>), dim3(rows), dim3(kLnThreads), 0, s, px, po, pb, pg, pbe, px2, py, mean, rstd, h, eps); break;
    default: hipLaunchKernelGGL((ln_fwd_kernel<T, ADD, 8>), dim3(rows), dim3(kLnThreads), 0, s, px, po, pb, pg, pbe, px2, py, mean, rstd, h, eps); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t ln_bwd_t(const void* dy, const void* x, const void* gamma, const float* mean, const float* rstd,
                    const void* resid, void* dx, int rows, int h, hipStream_t s) {
  const T *pdy = (const T*)dy, *px = (const T*)x, *pg = (const T*)gamma, *pr = (const T*)resid;
  T* pdx = (T*)dx;
  switch (ln_cpt(h, V<T>::N)) {
    case 1: hipLaunchKernelGGL((ln_bwd_kernel<T, 1>), dim3(rows), dim3(kLnThreads), 0, s, pdy, px, pg, mean, rstd, pr, pdx, h); break;
    case 2: hipLaunchKernelGGL((ln_bwd_kernel<T, 2>), dim3(rows), dim3(kLnThreads), 0, s, pdy, px, pg, mean, rstd, pr, pdx, h); break;
    case 4: hipLaunchKernelGGL((ln_bwd_kernel<T, 4>), dim3(rows), dim3(kLnThreads), 0, s, pdy, px, pg, mean, rstd, pr, pdx, h); break;
    default: hipLaunchKernelGGL((ln_bwd_kernel<T, 8>), dim3(rows), dim3(kLnThreads), 0, s, pdy, px, pg, mean, rstd, pr, pdx, h); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t colsum_t(int mode, const void* a, const void* x, const float* mean, const float* rstd, float* out0,
                    float* out1, float* partial, int rows, int cols, hipStream_t s) {
  int xb, rpb, nrb;
  colsum_geometry(rows, cols, V<T>::N, xb, rpb, nrb);
  if (mode == 1)
    hipLaunchKernelGGL((colsum_partial_kernel<T, 1>), dim3(xb, nrb), dim3(256), 0, s, (const T*)a, (const T*)x, mean,
                       rstd, partial, rows, cols, rpb, nrb);
  else
    hipLaunchKernelGGL((colsum_partial_kernel<T, 0>), dim3(xb, nrb), dim3(256), 0, s, (const T*)a, (const T*)x, mean,
                       rstd, partial, rows, cols, rpb, nrb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colsum_final_kernel, dim3((cols + 255) / 256), dim3(256), 0, s, partial, out0, out1, nrb, cols,
                     mode);
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

hipError_t launch_ln_fwd(bool is_bf16, bool add, const void* x, const void* o, const void* bias, const void* gamma,
                         const void* beta, void* x2, void* y, float* mean, float* rstd, int rows, int h, float eps,
                         hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (is_bf16)
    return add ? ln_fwd_t<bf16, true>(x, o, bias, gamma, beta, x2, y, mean, rstd, rows, h, eps, s)
               : ln_fwd_t<bf16, false>(x, o, bias, gamma, beta, x2, y, mean, rstd, rows, h, eps, s);
  return add ? ln_fwd_t<float, true>(x, o, bias, gamma, beta, x2, y, mean, rstd, rows, h, eps, s)
             : ln_fwd_t<float, false>(x, o, bias, gamma, beta, x2, y, mean, rstd, rows, h, eps, s);
}

hipError_t launch_ln_bwd(bool is_bf16, const void* dy, const void* x, const void* gamma, const float* mean,
                         const float* rstd, const void* resid, void* dx, int rows, int h, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return is_bf16 ? ln_bwd_t<bf16>(dy, x, gamma, mean, rstd, resid, dx, rows, h, s)
                 : ln_bwd_t<float>(dy, x, gamma, mean, rstd, resid, dx, rows, h, s);
}

size_t colsum_partial_floats(int rows, int cols, int mode) {
  int xb, rpb, nrb;
  colsum_geometry(rows, cols, 4, xb, rpb, nrb);  // fp32 chunks give the most slabs
  int xb2, rpb2, nrb2;
  colsum_geometry(rows, cols, 8, xb2, rpb2, nrb2);
  const int n = nrb > nrb2 ? nrb : nrb2;
  return (size_t)n * cols * (mode == 1 ? 2 : 1);
}

hipError_t launch_colsum(bool is_bf16, int mode, const void* a, const void* x, const float* mean, const float* rstd,
                         float* out0, float* out1, float* partial, int rows, int cols, hipStream_t s) {
  if (cols <= 0) return hipSuccess;
  return is_bf16 ? colsum_t<bf16>(mode, a, x, mean, rstd, out0, out1, partial, rows, cols, s)
                 : colsum_t<float>(mode, a, x, mean, rstd, out0, out1, partial, rows, cols, s);
}

hipError_t launch_add_bias_residual(bool is_bf16, const void* x2, const void* y, const void* bias, void* out, int rows,
                                    int h, hipStream_t s) {
  const int ve = is_bf16 ? 8 : 4;
  const int64_t n = (int64_t)rows * h / ve;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (is_bf16)
    hipLaunchKernelGGL(add_bias_residual_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)x2, (const bf16*)y,
                       (const bf16*)bias, (bf16*)out, n, h / ve);
  else
    hipLaunchKernelGGL(add_bias_residual_kernel<float>, grid, dim3(256), 0, s, (const float*)x2, (const float*)y,
                       (const float*)bias, (float*)out, n, h / ve);
  return hipGetLastError();
}

hipError_t launch_softmax_causal(bool is_bf16, const float* S, void* P, int nmat, int seq, hipStream_t s) {
  if (nmat <= 0) return hipSuccess;
  return is_bf16 ? softmax_t<bf16>(S, P, nmat, seq, s) : softmax_t<float>(S, P, nmat, seq, s);
}

hipError_t launch_attn_rowdot(bool is_bf16, const void* dctx, const void* ctx, float* D, int batch, int seq, int heads,
                              int d, hipStream_t s) {
  const int64_t nrows = (int64_t)batch * seq;
  const int64_t n = nrows * heads;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (is_bf16)
    hipLaunchKernelGGL(attn_rowdot_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)dctx, (const bf16*)ctx, D, nrows,
                       seq, heads, d);
  else
    hipLaunchKernelGGL(attn_rowdot_kernel<float>, grid, dim3(256), 0, s, (const float*)dctx, (const float*)ctx, D,
                       nrows, seq, heads, d);
  return hipGetLastError();
}

}  // namespace mt
