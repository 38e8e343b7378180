// Fused causal attention kernels (see flash_attn.hpp).
#include "flash_attn.hpp"

#include "gemm_dma.hpp"

namespace mt {

namespace {

constexpr int kFlashRows = 64;  // query rows per work-group (waves of 32 rows)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Head dim 160: rows of 20 chunks (320 bytes) take no XOR swizzle; rotating row r's
// chunks by (r >> 2) & 3 keeps 16 consecutive rows at one chunk, and 4 consecutive rows
// at 4 consecutive chunks, on distinct bank groups (every fragment read of the kernels
// below is conflict-free).
__device__ __forceinline__ int rot20(int row, int chunk) {
  const int c = chunk + ((row >> 2) & 3);
  return c >= 20 ? c - 20 : c;
}
__device__ __forceinline__ int unrot20(int row, int p) {
  const int c = p - ((row >> 2) & 3);
  return c < 0 ? c + 20 : c;
}

// LDS placement of 16-byte chunks in a [32 keys][D] tile.
// K (read with ds_read_b128, 16 lanes on 16 consecutive keys at one chunk): spread the 16
// rows over the 64 banks.
template <int D>
__device__ __forceinline__ int kswz(int row, int chunk) {
  if constexpr (D == 160) return rot20(row, chunk);
  else if constexpr (D == 128) return chunk ^ (row & 15);
  else return chunk ^ ((row >> 1) & 7);
}
// V (read with ds_read_b64_tr_b16, a half-wave on 4 consecutive keys x 32 columns): put
// the 4 rows in 4 different 64-byte bank groups.
template <int D>
__device__ __forceinline__ int vswz(int row, int chunk) {
  if constexpr (D == 160) return rot20(row, chunk);
  else if constexpr (D == 128) return chunk ^ ((row & 3) << 2);
  else return chunk ^ (((row >> 1) & 1) << 2);
}
// Logical chunk held by stored chunk p of a row (the XOR swizzles are their own inverse).
template <int D, bool VTILE>
__device__ __forceinline__ int tile_unswz(int row, int p) {
  if constexpr (D == 160) return unrot20(row, p);
  else return VTILE ? vswz<D>(row, p) : kswz<D>(row, p);
}

// DMA of one [32][D] tile whose rows are key rows kb.. of a head's column slice. `rsrc`
// covers the sequence's rows, so rows past it read zeros (the byte offset of row kb + r
// is at least the resource size once kb + r >= seq; the host keeps that size below
// 4 GiB). A wave instruction fills 1 KB of LDS: lane L writes bytes [16 L, +16) of it =
// tile row q * RPI + L / CPR, stored chunk L % CPR, which holds the logical chunk the
// swizzle maps there. The lane's byte offset within the tile is the same for every key
// block, so it is computed once (TileOffsets) and each block adds kb * ld * 2 (the
// kernels issue the loads themselves).
template <int D, bool VTILE, int NW>
struct TileOffsets {
  static constexpr int CPR = D / 8, INSTR = 32 * D / 512, PER = INSTR / NW;
  static_assert(INSTR % NW == 0, "tile instructions split over the waves");
  uint32_t off[PER];
  __device__ __forceinline__ void init(int64_t ld, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int pos = (wave + i * NW) * 64 + lane;  // stored chunk of the tile
      const int r = pos / CPR, c = tile_unswz<D, VTILE>(r, pos % CPR);
      off[i] = (uint32_t)(((int64_t)r * ld + c * 8) * 2);
    }
  }
};

// One 16-byte LDS-DMA load per lane into dst (the wave's 512-element slot of a tile).
// The kernels' loader lambdas call this instead of the builtin: a lambda is compiled for
// the host too, and there the target builtin would drop the kernel's host stub.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, bf16* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, off, 0, 0, 0);
}

// Work-groups are handed to the 8 XCDs round-robin by linear id. Maps a grid of
// `per_z` blocks per (sequence, head) to (z, block) so that each XCD gets a contiguous
// run of the (z, block) list: one to two heads per XCD, whose K/V (or Q/dO) panels then
// stay in that XCD's L2, instead of every XCD streaming every head. Within a run the
// blocks keep their order (the deepest first).
__device__ __forceinline__ void xcd_block(int per_z, int& z, int& blk) {
  constexpr int NXCD = 8;
  const int total = (int)(gridDim.x * gridDim.y);
  const int lin = (int)(blockIdx.x + gridDim.x * blockIdx.y);
  int logical = lin;
  if (total >= NXCD) {
    const int per = (total + NXCD - 1) / NXCD, rem = total % NXCD;
    const int xcd = lin % NXCD, local = lin / NXCD;
    logical = (rem == 0 || xcd < rem) ? xcd * per + local : rem * per + (xcd - rem) * (per - 1) + local;
  }
  z = logical / per_z;
  blk = logical % per_z;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t seq_rsrc(const bf16* base, int64_t ld, int seq) {
  const uint64_t bytes = (uint64_t)seq * (uint64_t)ld * 2u;
  const uint32_t n = bytes < 0xFFFFFFF0ull ? (uint32_t)bytes : 0xFFFFFFF0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), (short)0, (int)n, 0x00020000);
}

// ---------------------------------------------------------------------------- forward
// Combination of a value with the one in lane l ^ 32 (v_permlane32_swap: no LDS round
// trip). Both halves compute the same expression on the same operands.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work-group: 64 query rows of sequence b, head k, and 2 NG waves; wave w works on rows
// q0 + 32 (w & 1) and key group w >> 1. The row block's visible key blocks (32 keys) are
// split into NG contiguous runs, one per group, so the longest chain of dependent key
// steps (the deepest row block walks every key of the sequence) is 1 / NG of the
// sequence. Each group streams its run through its own two-stage LDS ring. At the end
// groups 1..NG-1 park their running (O, m, l) in LDS and group 0 merges them in group
// order and writes. Lane l of a wave owns query row (l & 31); the logit accumulator of a
// 32-key block holds keys 8 q + 4 (l >> 5) + j in register 4 q + j (the operand-swapped
// MFMA layout). COMP: the logits take the compensated form Q_hi K_hi^T + Q_hi K_lo^T +
// Q_lo K_hi^T (a.qkv_lo holds the remainders); otherwise Q K^T with the bf16 Q and K.
template <int D, bool COMP, int NG>
__global__ __launch_bounds__(128 * NG) void flash_fwd_kernel(FlashArgs a) {
  constexpr int KB = 32, NSTG = 2;
  constexpr int KS = D / 16, NB = D / 32, TILE = KB * D, NT = COMP ? 3 : 2, RING = NSTG * NT * TILE;
  constexpr int NV = NB * 16 + 2;  // parked floats per lane
  static_assert((NG - 1) * NV * 128 * 4 <= NG * RING * 2, "parked partials fit the rings");
  __shared__ __attribute__((aligned(1024))) bf16 smem[NG * RING];
  dma_lds_escape(smem);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 1, wv = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  const int nqb = (a.seq + kFlashRows - 1) / kFlashRows;
  int z, qbi;
  xcd_block(nqb, z, qbi);
  const int qb = nqb - 1 - qbi;
  const int b = z / a.heads, hd = z % a.heads;
  const int row = qb * kFlashRows + wv * 32 + r32;
  const bool row_ok = row < a.seq;

  const bf16* qkv = static_cast<const bf16*>(a.qkv) + (int64_t)b * a.seq * a.ldq;
  const bf16* qlo = static_cast<const bf16*>(a.qkv_lo) + (int64_t)b * a.seq * a.ldq;
  const int cq = hd * D, ck = a.hs + hd * D, cv = 2 * a.hs + hd * D;

  bf16x8 qh[KS], ql[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (row_ok) {
      qh[ks] = *reinterpret_cast<const bf16x8*>(qkv + (int64_t)row * a.ldq + cq + 16 * ks + 8 * h);
      if constexpr (COMP) ql[ks] = *reinterpret_cast<const bf16x8*>(qlo + (int64_t)row * a.ldq + cq + 16 * ks + 8 * h);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qh[ks][e] = ql[ks][e] = (bf16)0.f;
    }
  }

  const __amdgpu_buffer_rsrc_t rk = seq_rsrc(qkv + ck, a.ldq, a.seq);
  const __amdgpu_buffer_rsrc_t rkl = seq_rsrc(COMP ? qlo + ck : qkv + ck, a.ldq, a.seq);
  const __amdgpu_buffer_rsrc_t rv = seq_rsrc(qkv + cv, a.ldq, a.seq);
  const int kend = min(a.seq, (qb + 1) * kFlashRows);
  const int nsteps = (kend + KB - 1) / KB;
  const int per = (nsteps + NG - 1) / NG;                 // steps of every group (barrier count)
  const int tb = min(grp * per, nsteps), cnt = min(per, nsteps - tb);
  bf16* ring = smem + grp * RING;
  TileOffsets<D, false, 2> ok;
  TileOffsets<D, true, 2> ov;
  ok.init(a.ldq, wv, lane);
  ov.init(a.ldq, wv, lane);
  auto issue = [&](int j) {
    bf16* st = ring + (j % NSTG) * NT * TILE;
    const uint32_t rb = (uint32_t)((tb + j) * KB) * (uint32_t)a.ldq * 2u;
#pragma unroll
    for (int i = 0; i < TileOffsets<D, false, 2>::PER; ++i) {
      const int q = (wv + i * 2) * 512;
      lds_dma16(rk, st + q, ok.off[i] + rb);
      if (COMP) lds_dma16(rkl, st + 2 * TILE + q, ok.off[i] + rb);
      lds_dma16(rv, st + TILE + q, ov.off[i] + rb);
    }
  };

  const float scale2 = a.scale * kLog2e;
  f32x16 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[nb][r] = 0.f;
  float m = -__builtin_inff(), l = 0.f;

  if (cnt > 0) issue(0);
  for (int j = 0; j < per; ++j) {
    wait_vmcnt<0>();  // this wave's loads of block j
    dma_barrier();
    if (j + 1 < cnt) issue(j + 1);  // into the stage read in step j - 1
    const bf16* sK = ring + (j % NSTG) * NT * TILE;
    const bf16* sV = sK + TILE;
    const bf16* sKl = sK + 2 * TILE;
    const int kb = (tb + j) * KB, r0 = qb * kFlashRows + wv * 32;
    if (j >= cnt || kb > r0) continue;
    const bool diag = kb == r0;

    // two accumulation chains over the head dim (even and odd 16-wide steps)
    f32x16 sa, sb;
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[r] = sb[r] = 0.f;
    // all K fragments of the block first, then the MFMAs
    bf16x8 kf[KS], klf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = r32 * D + (kswz<D>(r32, 2 * ks + h) << 3);
      kf[ks] = *reinterpret_cast<const bf16x8*>(sK + off);
      if constexpr (COMP) klf[ks] = *reinterpret_cast<const bf16x8*>(sKl + off);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f32x16& s = (ks & 1) ? sb : sa;
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qh[ks], s, 0, 0, 0);
      if constexpr (COMP) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klf[ks], qh[ks], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], ql[ks], s, 0, 0, 0);
      }
    }
    f32x16 sv;
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = sa[r] + sb[r];
    if (diag) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb + 8 * (r >> 2) + 4 * h + (r & 3) > row) sv[r] = -__builtin_inff();
    }
    float mloc = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, sv[r]);
    const float mblk = xor32_max(mloc) * scale2;
    if (__any(mblk > m + 8.f)) {
      const float mnew = fmaxf(m, mblk);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[nb][r] *= alpha;
    }
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sv[r] = __builtin_amdgcn_exp2f(fmaf(sv[r], scale2, -m));
      lsum += sv[r];
    }
    l += xor32_sum(lsum);

#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      bf16x8 p;
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = (bf16)sv[8 * sl + e];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = 32 * nb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        s16x4 v2[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const int krow = 16 * sl + 8 * rr + 4 * h + ((lane & 15) >> 2);
          const bf16* pv = sV + krow * D + (vswz<D>(krow, col >> 3) << 3) + (col & 7);
          v2[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(pv));
        }
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v2[0], v2[1], 0, 1, 2, 3, 4, 5, 6, 7));
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p, o[nb], 0, 0, 0);
      }
    }
  }

  // Merge: groups 1..NG-1 park (O, m, l) as [group - 1][value][wave-in-group, lane] floats;
  // group 0 combines all groups in order: M = max m_g, O = sum O_g 2^(m_g - M), l likewise
  // (a group that saw no key of a row has m = -inf, l = 0, O = 0 and adds nothing).
  float* park = reinterpret_cast<float*>(smem);
  const int slot = wv * 64 + lane;
  dma_barrier();  // every ring is done with
  if (grp > 0) {
    float* pg = park + (grp - 1) * NV * 128;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pg[(nb * 16 + r) * 128 + slot] = o[nb][r];
    pg[(NV - 2) * 128 + slot] = m;
    pg[(NV - 1) * 128 + slot] = l;
  }
  dma_barrier();
  if (grp > 0) {
    return;
  }
  float mm = m;
#pragma unroll
  for (int g = 1; g < NG; ++g) mm = fmaxf(mm, park[((g - 1) * NV + NV - 2) * 128 + slot]);
  const float w0 = __builtin_amdgcn_exp2f(m - mm);
  l *= w0;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[nb][r] *= w0;
#pragma unroll
  for (int g = 1; g < NG; ++g) {
    const float* pg = park + (g - 1) * NV * 128;
    const float wg = __builtin_amdgcn_exp2f(pg[(NV - 2) * 128 + slot] - mm);
    l += pg[(NV - 1) * 128 + slot] * wg;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[nb][r] += pg[(nb * 16 + r) * 128 + slot] * wg;
  }

  if (row_ok) {
    const float inv = 1.f / l;
    bf16* out = static_cast<bf16*>(a.ctx) + ((int64_t)b * a.seq + row) * a.ldc + hd * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4] = {o[nb][4 * q] * inv, o[nb][4 * q + 1] * inv, o[nb][4 * q + 2] * inv, o[nb][4 * q + 3] * inv};
        store4_bf16(out + 32 * nb + 8 * q + 4 * h, v);
      }
    if (h == 0) a.lse[(int64_t)z * a.seq + row] = mm * kLn2 + logf(l);
  }
}

// ---------------------------------------------------------------------------- backward
// Head dim D = 64, 128 or 160. Tiles [32 rows][D] that serve both row reads
// (ds_read_b128, 16 lanes on 16 consecutive rows at one chunk) and transposing reads (a
// half-wave on 4 consecutive rows x 4 chunks) permute the chunks of each row so that 16
// consecutive rows land on 16 different 16-byte bank positions and 4 consecutive rows in 4
// different 64-byte bank groups: D = 128 (256-byte rows) chunk ^ (4 (r & 3) | ((r >> 2) &
// 3)); D = 64 (128-byte rows, two per bank window) chunk ^ (4 ((r >> 1) & 1) | ((r >> 2) &
// 3)); D = 160 (320-byte rows) the rotation rot20.
template <int D>
__device__ __forceinline__ int dswz(int row, int chunk) {
  static_assert(D == 64 || D == 128 || D == 160, "backward head dims");
  if constexpr (D == 160) return rot20(row, chunk);
  else if constexpr (D == 128) return chunk ^ (((row & 3) << 2) | ((row >> 2) & 3));
  else return chunk ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int dunswz(int row, int p) {
  if constexpr (D == 160) return unrot20(row, p);
  else return dswz<D>(row, p);
}

// Per-lane byte offsets of the DMA loads of a [32][D] tile (dual swizzle) relative to the
// tile's first row, computed once per leading dimension; a block adds its row offset, and
// rows past the sequence read zeros through the resource's range (as for dma_tile).
template <int D>
struct DualOffsets {
  static constexpr int CPR = D / 8, PER = 32 * D / 512 / 2;  // per wave, 2 waves
  uint32_t off[PER];
  __device__ __forceinline__ void init(int64_t ld, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int pos = (wave + i * 2) * 64 + lane;  // stored chunk of the tile
      const int r = pos / CPR, c = dunswz<D>(r, pos % CPR);
      off[i] = (uint32_t)(((int64_t)r * ld + c * 8) * 2);
    }
  }
};

// Row read of a dual-swizzled tile: lane's row r32, 16-k step ks (B operand).
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const bf16* t, int r32, int ks, int h) {
  return *reinterpret_cast<const bf16x8*>(t + r32 * D + (dswz<D>(r32, 2 * ks + h) << 3));
}
// Transposing read of a dual-swizzled tile for output column block nb and 16-row slice
// sl, matching the A operand taken from an accumulator (rows 16 sl + 4 h + 0..3 and
// 16 sl + 8 + 4 h + 0..3 of the tile).
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const bf16* t, int sl, int nb, int lane) {
  const int h = lane >> 5;
  const int col = 32 * nb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  s16x4 v[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int r = 16 * sl + 8 * rr + 4 * h + ((lane & 15) >> 2);
    v[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(t + r * D + (dswz<D>(r, col >> 3) << 3) + (col & 7)));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// bf16 operand of a 16-wide slice from accumulator registers 8 sl .. 8 sl + 7.
__device__ __forceinline__ bf16x8 acc_operand(const float* v, int sl) {
  bf16x8 p;
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = (bf16)v[8 * sl + e];
  return p;
}

template <int D>
__device__ __forceinline__ void store_rows(bf16* out, const f32x16* acc, float scale, int h) {
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4] = {acc[nb][4 * q] * scale, acc[nb][4 * q + 1] * scale, acc[nb][4 * q + 2] * scale,
                    acc[nb][4 * q + 3] * scale};
      store4_bf16(out + 32 * nb + 8 * q + 4 * h, v);
    }
}

// Stores a wave's 32 rows of a gradient (acc * scale, rounded to bf16) where `store`
// holds, and, if t is set, puts the rounded values (0 for rows past the sequence, given
// by ok) as fp32 in the wave's own LDS region t (32 rows of D + 4 floats) for
// wave_colsum. One conversion serves both.
template <int D>
__device__ __forceinline__ void store_stage_rows(bf16* out, bool store, const f32x16* acc, float scale, int h,
                                                 float* t, bool ok, int lane) {
  float* rowp = t ? t + (lane & 31) * (D + 4) + 4 * h : nullptr;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4] = {acc[nb][4 * q] * scale, acc[nb][4 * q + 1] * scale, acc[nb][4 * q + 2] * scale,
                    acc[nb][4 * q + 3] * scale};
      u32x2 r;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bf16 lo = (bf16)v[2 * e], hi = (bf16)v[2 * e + 1];
        r[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      if (store) *reinterpret_cast<u32x2*>(out + 32 * nb + 8 * q + 4 * h) = r;
      if (rowp) {
        f32x4 w;
        w[0] = ok ? __uint_as_float(r[0] << 16) : 0.f;
        w[1] = ok ? __uint_as_float(r[0] & 0xffff0000u) : 0.f;
        w[2] = ok ? __uint_as_float(r[1] << 16) : 0.f;
        w[3] = ok ? __uint_as_float(r[1] & 0xffff0000u) : 0.f;
        *reinterpret_cast<f32x4*>(rowp + 32 * nb + 8 * q) = w;
      }
    }
}

// Column sums of the 32 rows a wave staged in t (store_stage_rows) into out[0 .. D): lane
// l adds 4 consecutive columns over a run of rows (RS runs of 32 / RS rows per column
// group, as many as the 64 lanes allow) and the runs' sums are added across lanes, run 0
// first. LDS operations of one wave complete in order, so the exchange needs no barrier.
template <int D>
__device__ __forceinline__ void wave_colsum(float* out, const float* t, int lane) {
  constexpr int LD = D + 4, G = D / 4;  // row pitch, column groups
  constexpr int RS = G <= 16 ? 4 : G <= 32 ? 2 : 1, RPL = 32 / RS;
  const int g = lane % G, run = lane / G;
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  if (run < RS) {
    const float* p = t + run * RPL * LD + 4 * g;
#pragma unroll 8
    for (int r = 0; r < RPL; ++r) sum += *reinterpret_cast<const f32x4*>(p + r * LD);
  }
  if constexpr (RS == 4) {  // G = 16: runs in lanes g, g + 16, g + 32, g + 48
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = sum[e] + __shfl_xor(sum[e], 16);  // run 0 + run 1 (run 2 + run 3)
      sum[e] = x + __shfl_xor(x, 32);
    }
  } else if constexpr (RS == 2) {  // G = 32: runs in lanes g, g + 32
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[e] += __shfl_xor(sum[e], 32);
  }
  if (lane < G) *reinterpret_cast<f32x4*>(out + 4 * g) = sum;
}

// LDS floats of the parked partials of groups 1 .. NG - 1 (placed first in the rings), and
// the column-sum region of wave wv of group 0 after them.
template <int D, int NG>
constexpr int park_floats() { return (NG - 1) * (D / 32) * 16 * 128; }
template <int D, int NG>
__device__ __forceinline__ float* colsum_region(bf16* smem, int wv) {
  return reinterpret_cast<float*>(smem) + park_floats<D, NG>() + wv * 32 * (D + 4);
}

// Stage layouts of the backward rings (elements): NT tiles of [32][D] (Q or K first, then
// dO or V, then the Q or K remainders when compensated), and for the key part 1 KB for L
// and 1 KB for D of the stage's 32 queries (one DMA instruction each; the first 128 bytes
// carry the values).
template <int D, bool COMP>
constexpr int kv_stage() { return (COMP ? 3 : 2) * 32 * D + 1024; }
template <int D, bool COMP>
constexpr int q_stage() { return (COMP ? 3 : 2) * 32 * D; }
// Ring depth per group: two stages (loads one block ahead) with several groups, three
// (two blocks ahead) for a single group.
template <int NG>
constexpr int bwd_stages() { return NG == 1 ? 3 : 2; }

// dK and dV. Work-group: 64 keys of sequence b, head k, and NG groups of two waves (wave
// w: keys 64 kb + 32 (w & 1) .., group w >> 1). The query blocks (32 queries) that see the
// keys are split into NG consecutive runs; each group streams its run through its own
// two-stage LDS ring and accumulates partial dK, dV, which groups 1..NG-1 park in LDS at
// the end for group 0 to add in group order. Lane l owns key (l & 31); the accumulators
// of S^T and dP^T hold queries 8 q + 4 (l >> 5) + j in register 4 q + j.
//   P^T = exp(S^T / sqrt(d) - L[q]) (0 above the diagonal), dV += P^T dO,
//   dS^T = P^T * (dP^T - D[q]) with dP^T = V dO^T, dK += dS^T Q / sqrt(d).
template <int D, bool COMP, int NG>
__device__ __forceinline__ void flash_bwd_kv(const FlashArgs& a, int kblk, int z, bf16* smem) {
  constexpr int KS = D / 16, NB = D / 32, TILE = 32 * D, NT = COMP ? 3 : 2, STAGE = kv_stage<D, COMP>();
  constexpr int NSTG = bwd_stages<NG>();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 1, wv = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  const int b = z / a.heads, hd = z % a.heads;
  const int key = kblk * 64 + wv * 32 + r32;
  const bool key_ok = key < a.seq;

  const bf16* qkv = static_cast<const bf16*>(a.qkv) + (int64_t)b * a.seq * a.ldq;
  const bf16* qlo = static_cast<const bf16*>(a.qkv_lo) + (int64_t)b * a.seq * a.ldq;
  const bf16* dO = static_cast<const bf16*>(a.dctx) + (int64_t)b * a.seq * a.ldc + hd * D;
  const int cq = hd * D, ck = a.hs + hd * D, cv = 2 * a.hs + hd * D;

  bf16x8 kh[KS], kl[KS], vv[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (key_ok) {
      const int64_t o = (int64_t)key * a.ldq + 16 * ks + 8 * h;
      kh[ks] = *reinterpret_cast<const bf16x8*>(qkv + o + ck);
      if constexpr (COMP) kl[ks] = *reinterpret_cast<const bf16x8*>(qlo + o + ck);
      vv[ks] = *reinterpret_cast<const bf16x8*>(qkv + o + cv);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kh[ks][e] = kl[ks][e] = vv[ks][e] = (bf16)0.f;
    }
  }
  const __amdgpu_buffer_rsrc_t rq = seq_rsrc(qkv + cq, a.ldq, a.seq);
  const __amdgpu_buffer_rsrc_t rql = seq_rsrc(COMP ? qlo + cq : qkv + cq, a.ldq, a.seq);
  const __amdgpu_buffer_rsrc_t rdo = seq_rsrc(dO, a.ldc, a.seq);
  // L and D rows of this (sequence, head): seq floats each; reads past them return 0.
  const __amdgpu_buffer_rsrc_t rl =
      __builtin_amdgcn_make_buffer_rsrc(a.lse + (int64_t)z * a.seq, (short)0, a.seq * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.D) + (int64_t)z * a.seq, (short)0, a.seq * 4, 0x00020000);
  const int qb0 = (kblk * 64) / 32, nqb = (a.seq + 31) / 32;
  const int nsteps = nqb - qb0;
  const int per = (nsteps + NG - 1) / NG;
  const int tb = min(grp * per, nsteps), cnt = min(per, nsteps - tb);
  bf16* ring = smem + grp * NSTG * STAGE;
  DualOffsets<D> oq, oo;
  oq.init(a.ldq, wv, lane);
  oo.init(a.ldc, wv, lane);
  // lanes 0..7 of one instruction fetch the 32 floats; the others read past the range
  // (2^31 plus a row offset below 2^20 stays past it)
  const uint32_t lane_ld = lane < 8 ? 16u * lane : 0x80000000u;
  auto issue = [&](int j) {
    bf16* st = ring + (j % NSTG) * STAGE;
    const uint32_t r0 = (uint32_t)((qb0 + tb + j) * 32);
    const uint32_t rbq = r0 * (uint32_t)a.ldq * 2u, rbo = r0 * (uint32_t)a.ldc * 2u;
#pragma unroll
    for (int i = 0; i < DualOffsets<D>::PER; ++i) {  // Q_hi, dO (and Q_lo) tiles of the block
      const int q = (wv + i * 2) * 512;
      lds_dma16(rq, st + q, oq.off[i] + rbq);
      lds_dma16(rdo, st + TILE + q, oo.off[i] + rbo);
      if (COMP) lds_dma16(rql, st + 2 * TILE + q, oq.off[i] + rbq);
    }
    lds_dma16(wv == 0 ? rl : rd, st + NT * TILE + wv * 512, lane_ld + r0 * 4u);
  };

  const float scale2 = a.scale * kLog2e;
  f32x16 dv[NB], dk[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[nb][r] = dk[nb][r] = 0.f;

  // per wave and block: NT tiles of DualOffsets::PER instructions, and one for L or D
  constexpr int LOADS = NT * DualOffsets<D>::PER + 1;
  for (int j = 0; j < NSTG - 1; ++j)
    if (j < cnt) issue(j);
  for (int j = 0; j < per; ++j) {
    // this wave's loads of block j are done when at most those of the NSTG - 2 blocks
    // after it are pending
    if (NSTG == 3 && j + 1 < cnt) wait_vmcnt<(NSTG - 2) * LOADS>();
    else wait_vmcnt<0>();
    dma_barrier();
    if (j + NSTG - 1 < cnt) issue(j + NSTG - 1);  // into the stage read in step j - 1
    if (j >= cnt) continue;
    const bf16* sQ = ring + (j % NSTG) * STAGE;
    const bf16* sO = sQ + TILE;
    const bf16* sQl = sQ + 2 * TILE;
    const int q0 = (qb0 + tb + j) * 32, k0 = kblk * 64 + wv * 32;
    // Queries of this block vs this wave's keys (starts are multiples of 32): all see
    // them, the diagonal block, or none.
    const bool masked = q0 == k0 || q0 + 32 > a.seq;
    if (q0 < k0) continue;
    // L and D of this lane's 16 query columns (4 runs of 4 consecutive queries).
    const float* sL = reinterpret_cast<const float*>(sQ + NT * TILE);
    float l2[16], dq[16];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const f32x4 lv = *reinterpret_cast<const f32x4*>(sL + 8 * qq + 4 * h);
      const f32x4 dv4 = *reinterpret_cast<const f32x4*>(sL + 256 + 8 * qq + 4 * h);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        l2[4 * qq + jj] = lv[jj] * kLog2e;
        dq[4 * qq + jj] = dv4[jj];
      }
    }
    f32x16 st, dpt;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = dpt[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 qf = row_frag<D>(sQ, r32, ks, h), of = row_frag<D>(sO, r32, ks, h);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kh[ks], st, 0, 0, 0);
      dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(of, vv[ks], dpt, 0, 0, 0);
      if constexpr (COMP) {
        const bf16x8 qfl = row_frag<D>(sQl, r32, ks, h);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kl[ks], st, 0, 0, 0);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfl, kh[ks], st, 0, 0, 0);
      }
    }
    float p[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(st[r], scale2, -l2[r]));
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key > q || q >= a.seq) p[r] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = p[r] * (dpt[r] - dq[r]);
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const bf16x8 pp = acc_operand(p, sl), dd = acc_operand(ds, sl);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        dv[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(sO, sl, nb, lane), pp, dv[nb], 0, 0, 0);
        dk[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(sQ, sl, nb, lane), dd, dk[nb], 0, 0, 0);
      }
    }
  }
  // Merge dK, then dV: groups 1..NG-1 park [group - 1][value][wave-in-group, lane] floats,
  // group 0 adds them in group order.
  float* park = reinterpret_cast<float*>(smem);
  const int slot = wv * 64 + lane;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    f32x16* acc = which ? dv : dk;
    dma_barrier();  // the rings (or the previous round) are done with
    if (grp > 0) {
      float* pg = park + (grp - 1) * NB * 16 * 128;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) pg[(nb * 16 + r) * 128 + slot] = acc[nb][r];
    }
    dma_barrier();
    if (grp == 0) {
#pragma unroll
      for (int g = 1; g < NG; ++g) {
        const float* pg = park + (g - 1) * NB * 16 * 128;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[nb][r] += pg[(nb * 16 + r) * 128 + slot];
      }
    }
  }
  if (grp == 0) {
    bf16* out = static_cast<bf16*>(a.dqkv) + ((int64_t)b * a.seq + key) * a.ldq;
    if (!a.dbias_part) {  // uniform
      if (key_ok) {
        store_rows<D>(out + ck, dk, a.scale, h);
        store_rows<D>(out + cv, dv, 1.f, h);
      }
    } else {  // the rings and the parked partials are done with
      float* prow = a.dbias_part + (flash_dbias_rows(b, a.seq) + 2 * kblk + wv) * (3 * (int64_t)a.hs);
      float* t = colsum_region<D, NG>(smem, wv);
      store_stage_rows<D>(out + ck, key_ok, dk, a.scale, h, t, key_ok, lane);
      wave_colsum<D>(prow + ck, t, lane);
      store_stage_rows<D>(out + cv, key_ok, dv, 1.f, h, t, key_ok, lane);
      wave_colsum<D>(prow + cv, t, lane);
    }
  }
}

// dQ. Work-group: 64 query rows of sequence b, head k, and NG groups of two waves (wave w:
// rows 64 qb + 32 (w & 1) .., group w >> 1); the key blocks (32 keys) the rows see are
// split into NG consecutive runs, one per group, and group 0 adds the parked partial dQ
// of the others in group order. Lane l owns query row (l & 31).
//   P = exp(S / sqrt(d) - L), dS = P * (dO V^T - D), dQ += dS K / sqrt(d).
template <int D, bool COMP, int NG>
__device__ __forceinline__ void flash_bwd_q(const FlashArgs& a, int qb, int z, bf16* smem) {
  constexpr int KS = D / 16, NB = D / 32, TILE = 32 * D, STAGE = q_stage<D, COMP>();
  constexpr int NSTG = bwd_stages<NG>();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 1, wv = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  const int b = z / a.heads, hd = z % a.heads;
  const int row = qb * kFlashRows + wv * 32 + r32;
  const bool row_ok = row < a.seq;

  const bf16* qkv = static_cast<const bf16*>(a.qkv) + (int64_t)b * a.seq * a.ldq;
  const bf16* qlo = static_cast<const bf16*>(a.qkv_lo) + (int64_t)b * a.seq * a.ldq;
  const bf16* dO = static_cast<const bf16*>(a.dctx) + (int64_t)b * a.seq * a.ldc + hd * D;
  const int cq = hd * D, ck = a.hs + hd * D, cv = 2 * a.hs + hd * D;
  const int rc = min(row, a.seq - 1);
  const float l2 = a.lse[(int64_t)z * a.seq + rc] * kLog2e;
  const float drow = a.D[(int64_t)z * a.seq + rc];

  bf16x8 qh[KS], ql[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (row_ok) {
      const int64_t o = (int64_t)row * a.ldq + 16 * ks + 8 * h;
      qh[ks] = *reinterpret_cast<const bf16x8*>(qkv + o + cq);
      if constexpr (COMP) ql[ks] = *reinterpret_cast<const bf16x8*>(qlo + o + cq);
      of[ks] = *reinterpret_cast<const bf16x8*>(dO + (int64_t)row * a.ldc + 16 * ks + 8 * h);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qh[ks][e] = ql[ks][e] = of[ks][e] = (bf16)0.f;
    }
  }
  const __amdgpu_buffer_rsrc_t rk = seq_rsrc(qkv + ck, a.ldq, a.seq);
  const __amdgpu_buffer_rsrc_t rkl = seq_rsrc(COMP ? qlo + ck : qkv + ck, a.ldq, a.seq);
  const __amdgpu_buffer_rsrc_t rv = seq_rsrc(qkv + cv, a.ldq, a.seq);
  const int kend = min(a.seq, (qb + 1) * kFlashRows);
  const int nsteps = (kend + 31) / 32;
  const int per = (nsteps + NG - 1) / NG;
  const int tb = min(grp * per, nsteps), cnt = min(per, nsteps - tb);
  bf16* ring = smem + grp * NSTG * STAGE;
  DualOffsets<D> koff;
  koff.init(a.ldq, wv, lane);
  auto issue = [&](int j) {
    bf16* st = ring + (j % NSTG) * STAGE;
    const uint32_t rb = (uint32_t)((tb + j) * 32) * (uint32_t)a.ldq * 2u;
#pragma unroll
    for (int i = 0; i < DualOffsets<D>::PER; ++i) {  // K_hi, V (and K_lo) tiles of the key block
      const int q = (wv + i * 2) * 512;
      const uint32_t off = koff.off[i] + rb;
      lds_dma16(rk, st + q, off);
      lds_dma16(rv, st + TILE + q, off);
      if (COMP) lds_dma16(rkl, st + 2 * TILE + q, off);
    }
  };

  const float scale2 = a.scale * kLog2e;
  f32x16 dq[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[nb][r] = 0.f;

  constexpr int LOADS = (COMP ? 3 : 2) * DualOffsets<D>::PER;  // per wave and block
  for (int j = 0; j < NSTG - 1; ++j)
    if (j < cnt) issue(j);
  for (int j = 0; j < per; ++j) {
    if (NSTG == 3 && j + 1 < cnt) wait_vmcnt<(NSTG - 2) * LOADS>();
    else wait_vmcnt<0>();
    dma_barrier();
    if (j + NSTG - 1 < cnt) issue(j + NSTG - 1);  // into the stage read in step j - 1
    if (j >= cnt) continue;
    const bf16* sK = ring + (j % NSTG) * STAGE;
    const bf16* sV = sK + TILE;
    const bf16* sKl = sK + 2 * TILE;
    // Keys of this block vs this wave's rows (starts are multiples of 32): all visible,
    // the diagonal block, or none.
    const int kb = (tb + j) * 32, r0 = qb * kFlashRows + wv * 32;
    if (kb > r0) continue;
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kf = row_frag<D>(sK, r32, ks, h), vf = row_frag<D>(sV, r32, ks, h);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qh[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, of[ks], dp, 0, 0, 0);
      if constexpr (COMP) {
        const bf16x8 kfl = row_frag<D>(sKl, r32, ks, h);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfl, qh[ks], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, ql[ks], s, 0, 0, 0);
      }
    }
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = __builtin_amdgcn_exp2f(fmaf(s[r], scale2, -l2));
    if (kb == r0) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb + 8 * (r >> 2) + 4 * h + (r & 3) > row) ds[r] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] *= dp[r] - drow;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const bf16x8 dd = acc_operand(ds, sl);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        dq[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(sK, sl, nb, lane), dd, dq[nb], 0, 0, 0);
    }
  }
  float* park = reinterpret_cast<float*>(smem);
  const int slot = wv * 64 + lane;
  dma_barrier();  // the rings are done with
  if (grp > 0) {
    float* pg = park + (grp - 1) * NB * 16 * 128;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pg[(nb * 16 + r) * 128 + slot] = dq[nb][r];
  }
  dma_barrier();
  if (grp > 0) return;
#pragma unroll
  for (int g = 1; g < NG; ++g) {
    const float* pg = park + (g - 1) * NB * 16 * 128;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[nb][r] += pg[(nb * 16 + r) * 128 + slot];
  }
  bf16* out = static_cast<bf16*>(a.dqkv) + ((int64_t)b * a.seq + row) * a.ldq + cq;
  if (!a.dbias_part) {  // uniform
    if (row_ok) store_rows<D>(out, dq, a.scale, h);
  } else {
    float* t = colsum_region<D, NG>(smem, wv);
    store_stage_rows<D>(out, row_ok, dq, a.scale, h, t, row_ok, lane);
    wave_colsum<D>(a.dbias_part + (flash_dbias_rows(b, a.seq) + 2 * qb + wv) * (3 * (int64_t)a.hs) + cq, t, lane);
  }
}

// Both backward parts in one grid, each walking its deepest blocks first: blockIdx.x
// interleaves them (even: key block x / 2 of dK, dV; odd: row block of dQ, deepest
// first), so the grid's critical path is the longer of the two chains, not their sum.
template <int D, bool COMP, int NG>
__global__ __launch_bounds__(128 * NG) void flash_bwd_kernel(FlashArgs a) {
  constexpr int KVS = kv_stage<D, COMP>(), QS = q_stage<D, COMP>();
  constexpr int SMEM = NG * bwd_stages<NG>() * (KVS > QS ? KVS : QS);
  static_assert((NG - 1) * (D / 32) * 16 * 128 * 4 <= SMEM * 2, "parked partials fit the rings");
  static_assert((park_floats<D, NG>() + 64 * (D + 4)) * 4 <= SMEM * 2, "the column-sum regions fit the rings");
  __shared__ __attribute__((aligned(1024))) bf16 smem[SMEM];
  dma_lds_escape(smem);
  int z, x;
  xcd_block((int)gridDim.x, z, x);
  const int nqb = (a.seq + kFlashRows - 1) / kFlashRows, nkb = (a.seq + 63) / 64;
  if ((x & 1) == 0) {
    if (x / 2 < nkb) flash_bwd_kv<D, COMP, NG>(a, x / 2, z, smem);
  } else {
    if (x / 2 < nqb) flash_bwd_q<D, COMP, NG>(a, nqb - 1 - x / 2, z, smem);
  }
}

}  // namespace

// The kernels address a sequence's rows with 32-bit byte offsets and rely on the buffer
// range check for the rows of a last partial block past the sequence: the rows up to one
// block beyond it must span < 4 GiB in every column slice.
static bool flash_extents_ok(const FlashArgs& a) {
  const uint64_t lim = 0xFFFFFFF0ull, rows = (uint64_t)a.seq + 64u;
  return rows * (uint64_t)a.ldq * 2u < lim && rows * (uint64_t)a.ldc * 2u < lim && rows * 4u < (1ull << 20);
}

hipError_t launch_flash_bwd(const FlashArgs& a, int d, hipStream_t s) {
  if (a.seq <= 0 || a.batch <= 0 || a.heads <= 0) return hipSuccess;
  if (!flash_extents_ok(a)) return hipErrorInvalidValue;
  const int nqb = (a.seq + kFlashRows - 1) / kFlashRows, nkb = (a.seq + 63) / 64;
  const int n = 2 * (nqb > nkb ? nqb : nkb);
  const dim3 grid(n, a.batch * a.heads);
  const bool comp = a.qkv_lo != nullptr;
  // Two groups of two waves per work-group; one group (three-stage ring) for the plain
  // head dim 128, where a work-group per CU leaves three rounds of work-groups either
  // way and the split only adds the merge (more groups spill registers at head dim 128
  // and ran slower at 64).
  if (d == 160 && comp) hipLaunchKernelGGL((flash_bwd_kernel<160, true, 2>), grid, dim3(256), 0, s, a);
  else if (d == 160) hipLaunchKernelGGL((flash_bwd_kernel<160, false, 1>), grid, dim3(128), 0, s, a);
  else if (d == 128 && comp) hipLaunchKernelGGL((flash_bwd_kernel<128, true, 2>), grid, dim3(256), 0, s, a);
  else if (d == 128) hipLaunchKernelGGL((flash_bwd_kernel<128, false, 1>), grid, dim3(128), 0, s, a);
  else if (d == 64 && comp) hipLaunchKernelGGL((flash_bwd_kernel<64, true, 2>), grid, dim3(256), 0, s, a);
  else if (d == 64) hipLaunchKernelGGL((flash_bwd_kernel<64, false, 2>), grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_flash_fwd(const FlashArgs& a, int d, hipStream_t s) {
  if (a.seq <= 0 || a.batch <= 0 || a.heads <= 0) return hipSuccess;
  if (!flash_extents_ok(a)) return hipErrorInvalidValue;
  const dim3 grid((a.seq + kFlashRows - 1) / kFlashRows, a.batch * a.heads);
  const bool comp = a.qkv_lo != nullptr;
  // four key groups (8 waves) where their rings fit the LDS; two for the compensated
  // head dim 128 (three tiles per stage) and for head dim 160
  if (d == 160 && comp) hipLaunchKernelGGL((flash_fwd_kernel<160, true, 2>), grid, dim3(256), 0, s, a);
  else if (d == 160) hipLaunchKernelGGL((flash_fwd_kernel<160, false, 2>), grid, dim3(256), 0, s, a);
  else if (d == 128 && comp) hipLaunchKernelGGL((flash_fwd_kernel<128, true, 2>), grid, dim3(256), 0, s, a);
  else if (d == 128) hipLaunchKernelGGL((flash_fwd_kernel<128, false, 4>), grid, dim3(512), 0, s, a);
  else if (d == 64 && comp) hipLaunchKernelGGL((flash_fwd_kernel<64, true, 4>), grid, dim3(512), 0, s, a);
  else if (d == 64) hipLaunchKernelGGL((flash_fwd_kernel<64, false, 4>), grid, dim3(512), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mt
