// Fused AdamW step (see adamw.hpp). HBM-bound streaming kernel: a wave owns 1024
// consecutive parameters per grid-stride iteration and reads and writes them as four
// 1 KB-contiguous sweeps of 16-byte lane accesses (4 parameters per lane per sweep), so
// each vector instruction covers whole cache lines and 16 loads per lane are in flight. Loads and stores are nontemporal:
// every byte is touched once and should not displace the L2 and MALL contents of the
// work around the step. 30 bytes of HBM traffic per parameter with the bf16 copy, 28
// without.
#include "adamw.hpp"
#include "device_common.hpp"

namespace mt {
namespace {

constexpr int kThreads = 256;
constexpr int kSweeps = 4;            // 1 KB-contiguous sweeps per array and iteration
constexpr int kPer = 4 * kSweeps;     // parameters per lane and iteration

__device__ __forceinline__ f32x4 ld4(const float* p) { return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)); }
__device__ __forceinline__ void st4(float* p, f32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p)); }

// One parameter: moments, bias-corrected step, decoupled decay.
__device__ __forceinline__ void adamw_one(const AdamwArgs& a, float& p, float g, float& m, float& v) {
  g *= a.grad_scale;
  m = fmaf(a.beta1, m, a.one_minus_beta1 * g);
  v = fmaf(a.beta2, v, a.one_minus_beta2 * (g * g));
  const float denom = fmaf(sqrtf(v), a.inv_sqrt_bc2, a.eps);
  p = fmaf(-a.lr_wd, p, p) - a.step_size * (m / denom);
}

__global__ __launch_bounds__(kThreads) void adamw_kernel(AdamwArgs a) {
  constexpr int kWaves = kThreads / 64, kChunk = 64 * kPer;  // parameters per wave and iteration
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t chunks = a.n / kChunk;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  for (int64_t c = (int64_t)blockIdx.x * kWaves + wave; c < chunks; c += stride) {
    f32x4 p[kSweeps], g[kSweeps], m[kSweeps], v[kSweeps];
#pragma unroll
    for (int h = 0; h < kSweeps; ++h) {
      const int64_t i = c * kChunk + h * 256 + 4 * lane;
      p[h] = ld4(a.p + i);
      g[h] = ld4(a.g + i);
      m[h] = ld4(a.m + i);
      v[h] = ld4(a.v + i);
    }
#pragma unroll
    for (int h = 0; h < kSweeps; ++h) {
      const int64_t i = c * kChunk + h * 256 + 4 * lane;
      bf16x4 q;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pe = p[h][e], me = m[h][e], ve = v[h][e];
        adamw_one(a, pe, g[h][e], me, ve);
        p[h][e] = pe;
        m[h][e] = me;
        v[h][e] = ve;
        q[e] = from_f32<bf16>(pe);
      }
      st4(a.p + i, p[h]);
      st4(a.m + i, m[h]);
      st4(a.v + i, v[h]);
      if (a.p16) __builtin_nontemporal_store(q, reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.p16) + i));
    }
  }
  // the last n % 1024 parameters, by the first block
  if (blockIdx.x == 0) {
    for (int64_t t = chunks * kChunk + threadIdx.x; t < a.n; t += kThreads) {
      float pe = a.p[t], me = a.m[t], ve = a.v[t];
      adamw_one(a, pe, a.g[t], me, ve);
      a.p[t] = pe;
      a.m[t] = me;
      a.v[t] = ve;
      if (a.p16) static_cast<bf16*>(a.p16)[t] = from_f32<bf16>(pe);
    }
  }
}

}  // namespace

hipError_t launch_adamw(const AdamwArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  // one chunk per wave, at most 64 work-groups per CU (each wave loops; measured best)
  const int64_t chunks = (a.n + 64 * kPer - 1) / (64 * kPer);
  const int64_t want = (chunks + kThreads / 64 - 1) / (kThreads / 64);
  const int blocks = (int)(want < 16384 ? (want > 0 ? want : 1) : 16384);
  hipLaunchKernelGGL(adamw_kernel, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mt
