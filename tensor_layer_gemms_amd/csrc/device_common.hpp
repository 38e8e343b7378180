// Device-side helpers shared by the HIP kernels of the layer shard (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
// fp32 -> bf16 round-to-nearest-even (gfx950 lowers this to v_cvt_pk_bf16_f32).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

// 16-byte vectors of T: 8 bf16 or 4 fp32.
template <typename T> struct Vec16 { static constexpr int N = 16 / sizeof(T); };

template <typename T>
__device__ __forceinline__ void load16(const T* p, float* out) {
  u32x4 raw = *reinterpret_cast<const u32x4*>(p);
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(raw[i] << 16);
      out[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(raw[i]);
  }
}

template <typename T>
__device__ __forceinline__ void store16(T* p, const float* v) {
  u32x4 raw;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16 lo = (bf16)v[2 * i], hi = (bf16)v[2 * i + 1];
      raw[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = __float_as_uint(v[i]);
  }
  *reinterpret_cast<u32x4*>(p) = raw;
}

// 8 consecutive elements of T <-> 8 floats (one 16-byte access for bf16, two for fp32).
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out) {
  if constexpr (sizeof(T) == 2) {
    load16(p, out);
  } else {
    load16(p, out);
    load16(p + 4, out + 4);
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    store16(p, v);
  } else {
    store16(p, v);
    store16(p + 4, v + 4);
  }
}

// Wavefront (64 lanes) reductions.
// Wavefront reductions without LDS: DPP exchanges within rows of 16 lanes (lane ^ 1,
// lane ^ 2, then the 8- and 16-lane mirrors, which pair up the partial groups), then the
// gfx950 permlane swaps across rows (rows 0<->1 and 2<->3) and halves. At every step both
// partners combine the same two operands in the same order, so all 64 lanes end with the
// same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float swap16_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  return swap32_pair_sum(swap16_pair_sum(v));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Block-wide sum of NV values (every thread gets the totals). `red` holds
// NV * (blockDim/64) floats of LDS.
template <int NV, int NWAVES>
__device__ __forceinline__ void block_sum(float* v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = wave_sum(v[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) red[i * NWAVES + wave] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) s += red[i * NWAVES + w];
    v[i] = s;
  }
  __syncthreads();
}

// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2), t = 1 / (1 + p x)
// for x >= 0 (odd extension below), absolute error <= 1.5e-7. Branch-free, about a
// dozen VALU operations; the device library's erff is piecewise and a wave with mixed
// arguments runs both of its pieces (~33 operations), which made the GeLU epilogues
// ~10% of their GEMM tiles. Also returns exp(-x^2), which GeLU' reuses.
__device__ __forceinline__ float erf_as(float x, float& ex2) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  ex2 = __expf(-ax * ax);
  return copysignf(1.0f - poly * ex2, x);
}

// Exact (erf-form) GeLU a * Phi(a) = a/2 (1 + erf(a / sqrt 2)) and its derivative
// Phi(a) + a phi(a), phi(a) = exp(-a^2 / 2) / sqrt(2 pi) = exp(-x^2) / sqrt(2 pi) at
// x = a / sqrt 2.
__device__ __forceinline__ float gelu_f(float a) {
  float e;
  return 0.5f * a * (1.0f + erf_as(a * 0.70710678118654752f, e));
}
__device__ __forceinline__ float gelu_grad_f(float a) {
  float e;
  const float erf = erf_as(a * 0.70710678118654752f, e);
  return 0.5f * (1.0f + erf) + a * 0.39894228040143268f * e;
}
