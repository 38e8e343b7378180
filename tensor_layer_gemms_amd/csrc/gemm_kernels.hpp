// Device code of the GEMM family (see gemm.hpp for the contraction and layouts).
#pragma once

#include "device_common.hpp"
#include "gemm.hpp"

namespace mt {

// ---------------------------------------------------------------------------- epilogue
// Per-element epilogue (fp32 outputs: the fp32 DMA MFMA path and the SIMT fallback).
template <typename T, int KIND>
__device__ __forceinline__ void epi_store(const GemmArgs& g, int64_t coff, int64_t voff, int m, int n, float v) {
  const int64_t idx = coff + (int64_t)m * g.ldc + n;
  if constexpr (KIND == EPI_STORE) {
    static_cast<T*>(g.C)[idx] = from_f32<T>(g.alpha * v);
  } else if constexpr (KIND == EPI_STORE_F32) {
    static_cast<float*>(g.C)[idx] = g.alpha * v;
  } else if constexpr (KIND == EPI_BIAS) {
    static_cast<T*>(g.C)[idx] = from_f32<T>(v + to_f32(static_cast<const T*>(g.vec)[n]));
  } else if constexpr (KIND == EPI_BIAS_GELU) {
    const float a = v + to_f32(static_cast<const T*>(g.vec)[n]);
    static_cast<T*>(g.C)[idx] = from_f32<T>(a);
    static_cast<T*>(g.C2)[idx] = from_f32<T>(gelu_f(a));
  } else if constexpr (KIND == EPI_DGELU) {
    const float a = to_f32(static_cast<const T*>(g.aux)[idx]);
    static_cast<T*>(g.C)[idx] = from_f32<T>(v * gelu_grad_f(a));
  } else if constexpr (KIND == EPI_DSOFTMAX) {
    const float p = to_f32(static_cast<const T*>(g.aux)[idx]);
    const float d = static_cast<const float*>(g.vec)[voff + m];
    static_cast<T*>(g.C)[idx] = from_f32<T>(p * (g.alpha * v - d));
  } else if constexpr (KIND == EPI_BIAS_RESID) {
    const float r = static_cast<const float*>(g.aux)[idx];
    static_cast<T*>(g.C)[idx] = from_f32<T>(v + to_f32(static_cast<const T*>(g.vec)[n]) + r);
  }
}

// 4 consecutive bf16 <-> 4 floats (8-byte accesses).
__device__ __forceinline__ void load4_bf16(const bf16* p, float* v) {
  const u32x2 r = *reinterpret_cast<const u32x2*>(p);
  v[0] = __uint_as_float(r[0] << 16);
  v[1] = __uint_as_float(r[0] & 0xffff0000u);
  v[2] = __uint_as_float(r[1] << 16);
  v[3] = __uint_as_float(r[1] & 0xffff0000u);
}
__device__ __forceinline__ void store4_bf16(bf16* p, const float* v) {
  u32x2 r;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const bf16 lo = (bf16)v[2 * e], hi = (bf16)v[2 * e + 1];
    r[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  *reinterpret_cast<u32x2*>(p) = r;
}

// Epilogue of the MFMA path for 4 consecutive columns n..n+3 of row m (bf16 operands;
// the activation type is bf16). Inputs are loaded before anything is stored.
template <int KIND>
__device__ __forceinline__ void epi_store4(const GemmArgs& g, int64_t coff, int64_t voff, int m, int n,
                                           const float* acc) {
  const int64_t idx = coff + (int64_t)m * g.ldc + n;
  float v[4];
  if constexpr (KIND == EPI_STORE_F32) {
    f32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = g.alpha * acc[e];
    *reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + idx) = w;
    return;
  } else if constexpr (KIND == EPI_STORE) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = g.alpha * acc[e];
  } else if constexpr (KIND == EPI_BIAS || KIND == EPI_BIAS_GELU) {
    float b[4];
    load4_bf16(static_cast<const bf16*>(g.vec) + n, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = acc[e] + b[e];
    if constexpr (KIND == EPI_BIAS_GELU) {
      float z[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) z[e] = gelu_f(v[e]);
      store4_bf16(static_cast<bf16*>(g.C2) + idx, z);
    }
  } else if constexpr (KIND == EPI_BIAS_SPLIT) {
    float b[4];
    load4_bf16(static_cast<const bf16*>(g.vec) + n, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = acc[e] + b[e];
    if (n < g.seg_n) {
      float lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) lo[e] = v[e] - (float)(bf16)v[e];
      store4_bf16(static_cast<bf16*>(g.C2) + idx, lo);
    }
  } else if constexpr (KIND == EPI_DGELU) {
    float a[4];
    load4_bf16(static_cast<const bf16*>(g.aux) + idx, a);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = acc[e] * gelu_grad_f(a[e]);
  } else if constexpr (KIND == EPI_DSOFTMAX) {
    float p[4];
    load4_bf16(static_cast<const bf16*>(g.aux) + idx, p);
    const float d = static_cast<const float*>(g.vec)[voff + m];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = p[e] * (g.alpha * acc[e] - d);
  } else if constexpr (KIND == EPI_BIAS_RESID) {
    float b[4];
    load4_bf16(static_cast<const bf16*>(g.vec) + n, b);
    const f32x4 r = *reinterpret_cast<const f32x4*>(static_cast<const float*>(g.aux) + idx);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = acc[e] + b[e] + r[e];
  }
  store4_bf16(static_cast<bf16*>(g.C) + idx, v);
}

__device__ __forceinline__ void causal_k_range(const GemmArgs& g, int m0, int bm, int& kbeg, int& kend) {
  kbeg = 0;
  kend = g.K;
  if (g.causal == CAUSAL_K_LE_M) kend = min(g.K, m0 + bm);
  if (g.causal == CAUSAL_K_GE_M) kbeg = m0;
}

// Logical tile for workgroup `bid`. Workgroups are handed to the 8 XCDs round-robin
// (id mod 8); each XCD is given a contiguous range of logical tiles, and inside it
// GROUP_M tile-rows are walked together so neighbouring tiles share A and B panels in
// that XCD's L2.
template <int GROUP_M>
__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int NXCD = 8;
  const int total = tiles_m * tiles_n;
  int logical = bid;
  if (total >= NXCD) {
    const int per = (total + NXCD - 1) / NXCD, rem = total % NXCD;
    const int xcd = bid % NXCD, local = bid / NXCD;
    logical = (rem == 0 || xcd < rem) ? xcd * per + local : rem * per + (xcd - rem) * (per - 1) + local;
  }
  const int group = GROUP_M * tiles_n;
  const int first_m = (logical / group) * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int r = logical % group;
  tm = first_m + r % gm;
  tn = r / gm;
}

// ---------------------------------------------------------------------------- bf16 MFMA
// LDS tile: ROWS x 64 bf16, row = 128 bytes = 8 chunks of 16 bytes. The 64 banks of 4
// bytes span 256 bytes = two rows, and a 16-byte read is served 16 lanes at a time. An
// MFMA operand read has 16 lanes on 16 consecutive rows at the same chunk, so chunk c of
// row r lives at position c ^ ((r >> 1) & 7): the eight even rows then use eight distinct
// chunks of the lower bank half and the eight odd rows those of the upper half.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3); }

template <int ROWS, int NT, bool KCONTIG>
struct TileLoader {
  // K-contiguous: one 16-byte chunk per item. Token-strided: one 8x8 block per item
  // (8 loads of 8 consecutive rows at 8 consecutive k, transposed in registers).
  static constexpr int ITEMS = KCONTIG ? ROWS * 8 : ROWS;
  static constexpr int PER = (ITEMS + NT - 1) / NT;
  static constexpr int NREG = KCONTIG ? PER : PER * 8;
  static constexpr int NDSW = KCONTIG ? PER : PER * 8;  // LDS writes per tile
  static_assert(NREG <= 32, "validity mask holds 32 loads");
  u32x4 r[NREG];
  uint32_t ok = 0;  // bit q: load q was in range (zeroed at store time otherwise)

  // Issues the global loads of one k tile. Out-of-range items read the (always valid)
  // tile origin; their bit in `ok` is clear and store() writes zeros instead. Nothing
  // here consumes the loaded data, so the loads stay in flight until store().
  __device__ __forceinline__ void load(const bf16* base, int64_t ld, int row0, int rows_valid, int k0, int kend,
                                       int tid) {
    ok = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = tid + i * NT;
      if (ITEMS % NT != 0 && it >= ITEMS) break;
      if constexpr (KCONTIG) {
        const int row = it >> 3, kc = it & 7;
        const int gr = row0 + row, gk = k0 + kc * 8;
        const bool v = gr < rows_valid && gk < kend;
        r[i] = *reinterpret_cast<const u32x4*>(base + (v ? (int64_t)gr * ld + gk : 0));
        ok |= (uint32_t)v << i;
      } else {
        const int kb = it & 7, rb = it >> 3;
        const int gr = row0 + rb * 8;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int gk = k0 + kb * 8 + kk;
          const bool v = gr < rows_valid && gk < kend;
          r[i * 8 + kk] = *reinterpret_cast<const u32x4*>(base + (v ? (int64_t)gk * ld + gr : 0));
          ok |= (uint32_t)v << (i * 8 + kk);
        }
      }
    }
  }

  __device__ __forceinline__ u32x4 val(int q) const {
    return ((ok >> q) & 1u) ? r[q] : u32x4{0u, 0u, 0u, 0u};
  }

  __device__ __forceinline__ void store(bf16* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = tid + i * NT;
      if (ITEMS % NT != 0 && it >= ITEMS) break;
      if constexpr (KCONTIG) {
        const int row = it >> 3, kc = it & 7;
        *reinterpret_cast<u32x4*>(lds + swz(row, kc)) = val(i);
      } else {
        const int kb = it & 7, rb = it >> 3;
        u32x4 v[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) v[kk] = val(i * 8 + kk);
        // v[kk] holds rows rb*8..rb*8+7 at k = kb*8+kk (two rows per dword); output
        // row rr gathers its 8 k values (two k per dword). Lanes 8..15 hold the next
        // row block; they write the rows in the order rr ^ 1 so that each 16-lane store
        // covers one even and one odd row (both bank halves).
        const bool odd = rb & 1;
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          u32x4 wa, wb;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            wa[j] = __builtin_amdgcn_perm(v[2 * j + 1][rr >> 1], v[2 * j][rr >> 1],
                                          (rr & 1) ? 0x07060302u : 0x05040100u);
            wb[j] = __builtin_amdgcn_perm(v[2 * j + 1][(rr ^ 1) >> 1], v[2 * j][(rr ^ 1) >> 1],
                                          ((rr ^ 1) & 1) ? 0x07060302u : 0x05040100u);
          }
          const int row = rb * 8 + (odd ? (rr ^ 1) : rr);
          *reinterpret_cast<u32x4*>(lds + swz(row, kb)) = odd ? wb : wa;
        }
      }
    }
  }
};

template <bool A_K, bool B_K, int BM, int BN, int WM, int WN, int KIND>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int NT = 64 * WM * WN, BK = 64;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold 32x32 MFMA blocks");
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (BM + BN) * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WN) * (BM / WM), wn0 = (wave % WN) * (BN / WN);
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  int tm, tn;
  map_tile<4>(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  if (g.causal == CAUSAL_SKIP_UPPER && n0 > m0 + BM - 1) return;
  int kbeg, kend;
  causal_k_range(g, m0, BM, kbeg, kend);
  const int z = blockIdx.y, zo = z / g.zdiv, zi = z % g.zdiv;
  const int64_t aoff = zo * g.a_so + zi * g.a_si, boff = zo * g.b_so + zi * g.b_si;
  const int nseg = n0 < g.seg_n ? g.nseg : 1;

  TileLoader<BM, NT, A_K> la;
  TileLoader<BN, NT, B_K> lb;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk1 = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;  // k steps per segment
  const int nk = nk1 * nseg;
  // Step t reads segment t / nk1 at k = kbeg + (t % nk1) * BK.
  auto issue = [&](int t) {
    const int sg = (t >= nk1) + (t >= 2 * nk1);
    const int k0 = kbeg + (t - sg * nk1) * BK;
    la.load(static_cast<const bf16*>(g.seg_a[sg]) + aoff, g.lda, m0, g.M, k0, kend, tid);
    lb.load(static_cast<const bf16*>(g.seg_b[sg]) + boff, g.ldb, n0, sg ? min(g.N, g.seg_n) : g.N, k0, kend, tid);
  };
  // Three-stage pipeline: LDS buffer t & 1 holds the tile being multiplied, the other
  // buffer receives tile t + 1 (loaded into registers during step t - 1), and the
  // registers receive tile t + 2. A step's body has no branches (loads past the end of
  // the k range are masked to zero like any other out-of-range load), so it is one
  // scheduling region in which the hints below interleave the LDS reads of the next
  // fragments, the LDS writes of tile t + 1 and the global loads of tile t + 2 between
  // the MFMAs.
  if (nk > 0) {
    issue(0);
    la.store(smem, tid);
    lb.store(smem + BM * BK, tid);
    issue(nk > 1 ? 1 : 0);
    __syncthreads();
    constexpr int KS = BK / 16;
    constexpr int NMF = KS * TM * TN;                  // MFMAs per step
    constexpr int NDR = (KS - 1) * (TM + TN);          // fragment reads issued inside the step
    constexpr int NDW = TileLoader<BM, NT, A_K>::NDSW + TileLoader<BN, NT, B_K>::NDSW;  // LDS writes
    constexpr int NVM = TileLoader<BM, NT, A_K>::NREG + TileLoader<BN, NT, B_K>::NREG;  // global loads
    for (int t = 0; t < nk; ++t) {
      const int cur = t & 1;
      const bf16* sA = smem + cur * (BM + BN) * BK;
      const bf16* sB = sA + BM * BK;
      bf16* nxt = smem + (cur ^ 1) * (BM + BN) * BK;
      // 32x32x16 operands: lane l supplies row (l & 31) and 8 consecutive k starting
      // at 8 * (l >> 5) of the 16-wide k step.
      bf16x8 af[2][TM], bfr[2][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(sA + swz(wm0 + i * 32 + (lane & 31), lane >> 5));
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[0][j] = *reinterpret_cast<const bf16x8*>(sB + swz(wn0 + j * 32 + (lane & 31), lane >> 5));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int cb = ks & 1, nb = cb ^ 1;
        if (ks + 1 < KS) {
          const int ch = (ks + 1) * 2 + (lane >> 5);
#pragma unroll
          for (int i = 0; i < TM; ++i) af[nb][i] = *reinterpret_cast<const bf16x8*>(sA + swz(wm0 + i * 32 + (lane & 31), ch));
#pragma unroll
          for (int j = 0; j < TN; ++j) bfr[nb][j] = *reinterpret_cast<const bf16x8*>(sB + swz(wn0 + j * 32 + (lane & 31), ch));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cb][j], af[cb][i], acc[i][j], 0, 0, 0);
        if (ks == 0) {
          la.store(nxt, tid);
          lb.store(nxt + BM * BK, tid);
          issue(t + 2 < nk ? t + 2 : nk - 1);  // past the last step: a harmless reload
        }
      }
      // Interleave: every MFMA is followed by one fragment read while they last, and
      // the LDS writes and global loads are spread over the remaining MFMA slots.
#pragma unroll
      for (int q = 0; q < NMF; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (q < NDR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (q >= NMF / 4 && q < NMF / 4 + NDW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        if (q >= NMF / 8 && q < NMF / 8 + NVM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __syncthreads();
    }
  }

  // The MFMA computes the transposed block (B rows as its first operand), so in the
  // 32x32 accumulator layout lane l holds row (l & 31) and, in registers 4g..4g+3, the
  // four consecutive columns 8g + 4 (l >> 5) + 0..3. N is a multiple of 8, so a group
  // is either wholly inside or wholly outside the matrix.
  const int64_t coff = zo * g.c_so + zi * g.c_si;
  const int64_t voff = (int64_t)z * g.vec_bs;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm0 + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn0 + j * 32 + q * 8 + (lane >> 5) * 4;
        float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if (m < g.M && n < g.N) epi_store4<KIND>(g, coff, voff, m, n, v);
      }
    }
  }
}

// ---------------------------------------------------------------------------- fp32 SIMT (fallback)
// fp32 problems the DMA kernel cannot address: 64x64 tiles, 16-deep k steps through LDS, 4x4 outputs per thread, fp32
// fused multiply-add. Same operand layouts, causal modes and epilogues as the MFMA path.
template <bool A_K, bool B_K, int KIND>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[BK][BN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int tiles_n = (g.N + BN - 1) / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  if (g.causal == CAUSAL_SKIP_UPPER && n0 > m0 + BM - 1) return;
  int kbeg, kend;
  causal_k_range(g, m0, BM, kbeg, kend);
  const int z = blockIdx.y, zo = z / g.zdiv, zi = z % g.zdiv;
  const float* A = static_cast<const float*>(g.A) + zo * g.a_so + zi * g.a_si;
  const float* B = static_cast<const float*>(g.B) + zo * g.b_so + zi * g.b_si;
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * 256;
      int r, k;
      if (A_K) { r = e >> 4; k = e & 15; } else { k = e >> 6; r = e & 63; }
      int gr = m0 + r, gk = k0 + k;
      sA[k][r] = (gr < g.M && gk < kend) ? A[A_K ? (int64_t)gr * g.lda + gk : (int64_t)gk * g.lda + gr] : 0.f;
      if (B_K) { r = e >> 4; k = e & 15; } else { k = e >> 6; r = e & 63; }
      gr = n0 + r;
      gk = k0 + k;
      sB[k][r] = (gr < g.N && gk < kend) ? B[B_K ? (int64_t)gr * g.ldb + gk : (int64_t)gk * g.ldb + gr] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int64_t coff = zo * g.c_so + zi * g.c_si;
  const int64_t voff = (int64_t)z * g.vec_bs;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < g.M && n < g.N) epi_store<float, KIND>(g, coff, voff, m, n, acc[i][j]);
    }
}

}  // namespace mt
