// MFMA GEMM fed by LDS-DMA loads, for every operand layout of the layer, in bf16
// (v_mfma_f32_32x32x16_bf16, k-step 64) or fp32 (v_mfma_f32_32x32x2_f32, k-step 32).
//
// Each lane's 16-byte global load is written by the memory system straight into LDS
// (buffer_load ... lds): no staging registers, no LDS store instructions, no register
// transposes. A k-contiguous operand tile is kept in LDS as rows of k ([rows][BK]) and
// read with ds_read_b128; an m-contiguous operand tile (token-strided wgrad operands,
// the weight of a dgrad, V in P V) is kept as it lies in memory ([BK][rows]) and read
// with the transposing ds_read_b64_tr_b16 (bf16), which hands each lane 4 consecutive k
// of one m, or with one ds_read_b32 per k (fp32). Out-of-range rows and the k tail read
// zeros through the buffer resource's range check. Two LDS stages alternate: one is
// multiplied while the loads of the next fill the other. Both element types use the same
// LDS geometry in 16-byte chunks (a k-contiguous row is 128 bytes: 64 bf16 or 32 fp32),
// the same loaders, schedule and accumulator layout; they differ in the fragment reads,
// the MFMA instruction and the epilogue (bf16 outputs are staged through LDS, fp32
// outputs stored by each lane).
#pragma once

#include "gemm_kernels.hpp"

namespace mt {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

// s_waitcnt with vmcnt <= n and the other counters left alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt with vmcnt and lgkmcnt both 0 (expcnt left alone).
__device__ __forceinline__ void wait_lgkm_vm0() { __builtin_amdgcn_s_waitcnt(7 << 4); }

// LDS filled by DMA loads. The compiler does not see those loads as writes of the LDS
// they fill; if the LDS array's address never escapes it even concludes that nothing
// writes the array, and moves reads of a freshly filled stage above the barrier and
// above the wait for the loads. dma_lds_escape hands the array's address to an opaque
// asm once, so every later memory clobber may write it; dma_barrier puts memory
// clobbers and scheduling barriers around the work-group barrier, which pins every LDS
// access on its side.
__device__ __forceinline__ void dma_lds_escape(void* lds) { asm volatile("" : : "v"(lds) : "memory"); }

__device__ __forceinline__ void dma_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// LDS placement of 16-byte chunks.
// k-contiguous tile [rows][BK] (KCH = 8 or 4 chunks per row): chunk c of row r sits at
// c ^ f(r); f spreads the 16 rows one ds_read_b128 quarter-wave touches (same chunk) over
// the 64 banks.
template <int KCH>
__device__ __forceinline__ int kc_swz(int row, int chunk) {
  static_assert(KCH == 8 || KCH == 4, "k-contiguous rows of 128 or 64 bytes");
  if constexpr (KCH == 8) return chunk ^ ((row >> 1) & 7);
  else return chunk ^ ((row >> 2) & 3);
}
// m-contiguous tile [BK][rows] (rows a power of two >= 128): chunk c of k-row r sits at
// c ^ 4 (r & 3). A half-wave transposing read covers 4 consecutive k-rows x 32
// consecutive m = 4 rows x 4 chunks; the XOR moves the 4 rows to 4 different 64-byte
// bank groups.
__device__ __forceinline__ int mc_swz(int krow, int chunk) { return chunk ^ ((krow & 3) << 2); }

// DMA loads of one ROWS x BK operand tile (ROWS along m or n) of element type T. The
// tile is ROWS BK sizeof(T) bytes = INSTR wave instructions of 1 KB. Lane L of
// instruction q fills LDS bytes [q 1024 + 16 L, +16): LDS row q RPI + L / CPR, stored
// chunk L % CPR, which holds the logical chunk the swizzle maps there.
// Loader waves: with 8 waves (two per SIMD) only waves 0-3, one per SIMD, issue the
// loads (wave w instructions w, w + 4, ...), so the other wave of every SIMD never waits
// for loads of its own and runs its MFMAs while its partner issues and waits; measured on
// the layer's shapes: forward GEMMs 4-15% faster, input and weight gradients 3-6%, than
// with every wave issuing an equal share at the same point of the step. With 4 waves
// every wave issues (instructions w, w + 4, ...).
template <typename T, int ROWS, int BK, int NW, bool KC>
struct DmaLoader {
  static constexpr int ES = sizeof(T), EPC = 16 / ES;  // bytes per element, elements per chunk
  static constexpr int ROW_ELEMS = KC ? BK : ROWS;     // elements per LDS row
  static constexpr int CPR = ROW_ELEMS / EPC;          // 16-byte chunks per LDS row
  static constexpr int KCH = BK / EPC;                 // chunks per k-contiguous row
  static constexpr int RPI = 64 / CPR;                 // LDS rows per wave instruction
  static constexpr int INSTR = ROWS * BK * ES / 1024;  // instructions per tile
  static constexpr int IEL = 1024 / ES;                // elements per instruction
  static constexpr int LW = NW == 8 ? 4 : NW;        // loader waves
  static constexpr int PER_WAVE = INSTR / LW;        // instructions per loader wave
  static_assert(INSTR % LW == 0, "tile must split evenly over the loader waves");
  static_assert(KC || (ROWS >= 128 && (ROWS & (ROWS - 1)) == 0), "m-contiguous tiles: power of two >= 128");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t invalid;  // an offset at the end of the range: reads zeros
  int64_t ld;
  int rows_valid;

  // KC: base = element (row0, 0), rows_valid rows left; the range ends after them.
  // !KC: base = element (k = 0, row0); the range is the K x ld block; rows past
  // rows_valid are masked per lane.
  __device__ __forceinline__ void init(const T* base, int64_t ld_, int rows_valid_, int kdim) {
    ld = ld_;
    rows_valid = rows_valid_;
    uint64_t bytes;
    if constexpr (KC) bytes = rows_valid_ > 0 ? (uint64_t)rows_valid_ * (uint64_t)ld_ * ES : 0u;
    else bytes = (uint64_t)kdim * (uint64_t)ld_ * ES;
    invalid = bytes < 0xFFFFFFF0ull ? (uint32_t)bytes : 0xFFFFFFF0u;
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, (int)invalid, 0x00020000);
  }

  // Fast path of a full k-step (k0 + BK <= kend, every lane's k in range): the lane's byte
  // offset of instruction i at k = 0 is a per-tile constant (vo[i], from offsets()), and
  // the step's advance, uniform over the work-group, goes in the instruction's SGPR
  // offset. Masked lanes (an m-contiguous operand's columns past rows_valid) carry
  // `invalid`; k-contiguous rows past rows_valid lie past the range by themselves. Both
  // read zeros whether or not the hardware's range check counts the SGPR offset, as long
  // as no sum wraps 32 bits: fast() requires twice the range to stay below 4 GiB.
  __device__ __forceinline__ bool fast() const { return (uint64_t)invalid * 2u < 0xFFFFFFF0ull; }
  __device__ __forceinline__ void offsets(int wave, int lane, uint32_t (&vo)[PER_WAVE]) const {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = (wave < LW ? wave : 0) + i * LW;
      const int r = q * RPI + lane / CPR;
      const int p = lane % CPR;
      if constexpr (KC) {
        vo[i] = (uint32_t)(r * ld + kc_swz<KCH>(r, p) * EPC) * ES;
      } else {
        const int m = mc_swz(r, p) * EPC;
        vo[i] = m < rows_valid ? (uint32_t)(r * ld + m) * ES : invalid;
      }
    }
  }
  __device__ __forceinline__ void issue_full(T* lds_stage, int k0, const uint32_t* vo, int wave) const {
    if (wave >= LW) return;  // wave-uniform
    const uint32_t soff = KC ? (uint32_t)k0 * ES : (uint32_t)k0 * (uint32_t)ld * ES;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = wave + i * LW;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds_stage + q * IEL), 16, vo[i], soff, 0, 0);
    }
  }

  // General path (tail steps, causal k ranges, segmented m-contiguous operands): every
  // lane checks its k against kend (and its m against rows_valid) each step.
  __device__ __forceinline__ void issue(T* lds_stage, int k0, int kend, int wave, int lane) const {
    if (wave >= LW) return;  // wave-uniform
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = wave + i * LW;
      const int r = q * RPI + lane / CPR;
      const int p = lane % CPR;
      uint32_t off;
      if constexpr (KC) {
        const int k = k0 + kc_swz<KCH>(r, p) * EPC;
        off = k < kend ? (uint32_t)(r * ld + k) * ES : invalid;
      } else {
        const int k = k0 + r, m = mc_swz(r, p) * EPC;
        off = (k < kend && m < rows_valid) ? (uint32_t)(k * ld + m) * ES : invalid;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds_stage + q * IEL), 16, off, 0, 0, 0);
    }
  }
};

// Operand fragment reads, one slice (16 k of bf16, 8 k of fp32) per call.
// bf16, for the 32x32x16 MFMA: lane l gets row (l & 31) of the 32-row block and
// k = 8 (l >> 5) + 0..7 of the slice.
// fp32, for four 32x32x2 MFMAs: lane l gets row (l & 31) and k = 4 (l >> 5) + 0..3 of
// the slice; MFMA e takes value e, i.e. contracts the slice's k = e and k = 4 + e (the
// two lane halves), the same pairing for both operands, so the four cover the slice.
template <typename T, int ROWS, int BK, bool KC>
struct FragReader;

template <int ROWS, int BK, bool KC>
struct FragReader<bf16, ROWS, BK, KC> {
  using Frag = bf16x8;
  static constexpr int READS = KC ? 1 : 2;  // LDS read instructions per call
  int off;  // per-lane element offset of the block at k-step 0
  int row;  // KC: this lane's tile row
  __device__ __forceinline__ void init(int row0, int lane) {
    if constexpr (KC) {
      row = row0 + (lane & 31);
      off = row * BK;
    } else {
      // Transposing read: within a 16-lane group, lane L addresses 4 consecutive m at
      // k-row (L >> 2), m offset 4 (L & 3); lane j of the group then receives the
      // 4 k-rows of m offset j. Two reads (k-rows 0..3 and 4..7) give the 8 k.
      const int kr = 8 * (lane >> 5) + ((lane >> 2) & 3);
      const int m = row0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      off = kr * ROWS + (mc_swz(kr, m >> 3) << 3) + (m & 7);
    }
  }
  __device__ __forceinline__ bf16x8 read(const bf16* tile, int ks, int lane) const {
    if constexpr (KC) {
      return *reinterpret_cast<const bf16x8*>(tile + off + (kc_swz<BK / 8>(row, 2 * ks + (lane >> 5)) << 3));
    } else {
      const bf16* p = tile + off + ks * 16 * ROWS;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p + 4 * ROWS));
      const auto v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, v);
    }
  }
};

template <int ROWS, int BK, bool KC>
struct FragReader<float, ROWS, BK, KC> {
  using Frag = f32x4;
  static constexpr int READS = KC ? 1 : 4;
  int off[KC ? 1 : 4];  // per-lane element offsets at k-step 0 (m-contiguous: one per k-row)
  int row;
  __device__ __forceinline__ void init(int row0, int lane) {
    if constexpr (KC) {
      row = row0 + (lane & 31);
      off[0] = row * BK;
    } else {
      // k-row 4 (l >> 5) + e of the slice, column m = row0 + (l & 31); chunk m / 4 of
      // k-row r sits at mc_swz(r, m / 4), and r & 3 = e for every slice.
      const int m = row0 + (lane & 31), kr = 4 * (lane >> 5);
#pragma unroll
      for (int e = 0; e < 4; ++e) off[e] = (kr + e) * ROWS + (mc_swz(kr + e, m >> 2) << 2) + (m & 3);
    }
  }
  __device__ __forceinline__ f32x4 read(const float* tile, int ks, int lane) const {
    if constexpr (KC) {
      return *reinterpret_cast<const f32x4*>(tile + off[0] + (kc_swz<BK / 4>(row, 2 * ks + (lane >> 5)) << 2));
    } else {
      const float* p = tile + ks * 8 * ROWS;
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = p[off[e]];
      return v;
    }
  }
};

// acc += the slice's product: bf16 one 32x32x16 MFMA, fp32 four 32x32x2 MFMAs. The B
// fragment goes first, so lane l holds accumulator row (l & 31) of the A side.
__device__ __forceinline__ void mfma_frag(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_frag(f32x16& acc, const f32x4& a, const f32x4& b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(b[e], a[e], acc, 0, 0, 0);
}
template <typename T>
constexpr int kMfmaPerFrag = sizeof(T) == 2 ? 1 : 4;

// LDS placement of the 16-byte chunks of a staged bf16 output tile [BM][BN]: chunk c of
// row r sits at c ^ f(r), so the 16 consecutive rows that one accumulator write covers
// fall in 16 different 16-byte bank groups (row pitch 0 mod 256 bytes for BN = 128, 256;
// 128 mod 256 for BN = 192).
template <int BN>
__device__ __forceinline__ int epi_swz(int row, int chunk) {
  static_assert(BN == 128 || BN == 192 || BN == 256, "staged tile widths");
  if constexpr (BN == 192) return chunk ^ ((row >> 1) & 7);
  else return chunk ^ (row & 15);
}

// Epilogue through LDS for bf16 outputs: the element-wise epilogue runs on the
// accumulators, the values go to LDS (free once the last k-step has been read), and the
// work-group then writes whole row segments with 16-byte stores, so every output cache
// line is written at once instead of in 16-byte pieces from 32 rows per store.
// One-output epilogues stage the whole tile in one round. Two-output epilogues (bias +
// GeLU: a and GeLU(a); the bias split: hi and remainder) stage both outputs of one
// 32-row accumulator block per wave at a time, TM rounds, so no value outlives its
// round. Requires ldc, the batch strides and seg_n to be multiples of 8 and C, C2 to be
// 16-byte aligned (checked on the host).
template <int BM, int BN, int TM, int TN, int WM, int WN, int KIND>
__device__ __forceinline__ void epi_staged(const GemmArgs& g, f32x16 (&acc)[TM][TN], bf16* smem, int m0, int n0,
                                           int wm0, int wn0, int64_t coff, int64_t voff) {
  constexpr bool TWO = KIND == EPI_BIAS_GELU || KIND == EPI_BIAS_SPLIT;
  constexpr int NT = 64 * WM * WN, CPR = BN / 8;
  constexpr int ROUNDS = TWO ? TM : 1, TR = TM / ROUNDS;  // accumulator blocks per round
  constexpr int RROWS = BM / ROUNDS;                      // staged tile rows per round
  constexpr int REGION = RROWS * BN;                      // elements per staged output
  static_assert(RROWS * CPR % NT == 0, "drain splits evenly");
  const int tid = threadIdx.x, lane = tid & 63, wr = wm0 / (BM / WM);
  bf16* s0 = smem;
  bf16* s1 = smem + REGION;
  auto put = [&](bf16* region, int rho, int c, const float* v) {  // 4 values, staged row rho, columns c..c+3
    store4_bf16(region + rho * BN + (epi_swz<BN>(rho, c >> 3) << 3) + (c & 7), v);
  };
  // EPI_DGELU with g.colsum: each thread drains one 8-column chunk (NT is a multiple of
  // CPR) of several rows and adds the stored bf16 values per 128-row half of the tile.
  constexpr bool CSUM = KIND == EPI_DGELU;
  constexpr int HALVES = BM / kColsumRows;
  static_assert(!CSUM || (NT % CPR == 0 && BM % kColsumRows == 0 && ROUNDS == 1), "column-sum drain layout");
  const bool csum = CSUM && g.colsum != nullptr;
  float cs[CSUM ? HALVES : 1][8];
#pragma unroll
  for (int hh = 0; hh < (CSUM ? HALVES : 1); ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) cs[hh][e] = 0.f;
  auto drain = [&](const bf16* region, void* dst, int round, int ncols) {
#pragma unroll 2
    for (int it = 0; it < RROWS * CPR / NT; ++it) {
      const int id = it * NT + tid, rho = id / CPR, c = id % CPR;
      const int r = (rho / (32 * TR)) * (BM / WM) + round * TR * 32 + rho % (32 * TR);
      const int m = m0 + r, n = n0 + 8 * c;
      const u32x4 w = *reinterpret_cast<const u32x4*>(region + rho * BN + (epi_swz<BN>(rho, c) << 3));
      if (m < g.M && n < ncols) {
        *reinterpret_cast<u32x4*>(static_cast<bf16*>(dst) + coff + (int64_t)m * g.ldc + n) = w;
        if constexpr (CSUM) {
          if (csum) {
            const bf16x8 v = __builtin_bit_cast(bf16x8, w);
#pragma unroll
            for (int hh = 0; hh < HALVES; ++hh)
              if (r / kColsumRows == hh) {
#pragma unroll
                for (int e = 0; e < 8; ++e) cs[hh][e] += (float)v[e];
              }
          }
        }
      }
    }
  };

#pragma unroll
  for (int round = 0; round < ROUNDS; ++round) {
    dma_barrier();  // the operand stages, or the previous round, have been read
#pragma unroll
    for (int ii = 0; ii < TR; ++ii) {
      const int i = round * TR + ii;
      const int rho = (wr * TR + ii) * 32 + (lane & 31);
      const int m = m0 + wm0 + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn0 + j * 32 + q * 8 + (lane >> 5) * 4, n = n0 + c;
          const bool ok = m < g.M && n < g.N;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          if constexpr (KIND == EPI_STORE) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= g.alpha;
          } else if constexpr (KIND == EPI_BIAS || KIND == EPI_BIAS_GELU || KIND == EPI_BIAS_SPLIT) {
            float b[4] = {0.f, 0.f, 0.f, 0.f};
            if (ok) load4_bf16(static_cast<const bf16*>(g.vec) + n, b);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += b[e];
          } else if constexpr (KIND == EPI_DGELU) {
            float a[4] = {0.f, 0.f, 0.f, 0.f};
            if (ok) load4_bf16(static_cast<const bf16*>(g.aux) + coff + (int64_t)m * g.ldc + n, a);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= gelu_grad_f(a[e]);
          } else if constexpr (KIND == EPI_DSOFTMAX) {
            float p[4] = {0.f, 0.f, 0.f, 0.f};
            float d = 0.f;
            if (ok) {
              load4_bf16(static_cast<const bf16*>(g.aux) + coff + (int64_t)m * g.ldc + n, p);
              d = static_cast<const float*>(g.vec)[voff + m];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = p[e] * (g.alpha * v[e] - d);
          } else if constexpr (KIND == EPI_BIAS_RESID) {
            float b[4] = {0.f, 0.f, 0.f, 0.f};
            f32x4 r = {0.f, 0.f, 0.f, 0.f};
            if (ok) {
              load4_bf16(static_cast<const bf16*>(g.vec) + n, b);
              r = *reinterpret_cast<const f32x4*>(static_cast<const float*>(g.aux) + coff + (int64_t)m * g.ldc + n);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += b[e] + r[e];
          }
          put(s0, rho, c, v);
          if constexpr (TWO) {
            float w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = KIND == EPI_BIAS_GELU ? gelu_f(v[e]) : v[e] - (float)(bf16)v[e];
            put(s1, rho, c, w);
          }
        }
      }
    }
    dma_barrier();
    drain(s0, g.C, round, g.N);
    if constexpr (TWO) drain(s1, g.C2, round, KIND == EPI_BIAS_SPLIT ? min(g.N, g.seg_n) : g.N);
  }
  if constexpr (CSUM) {
    if (csum) {  // wave-uniform: the threads of a chunk column add their rows in slot order
      constexpr int TPC = NT / CPR;
      float* red = reinterpret_cast<float*>(smem);  // [TPC][HALVES][BN]
      const int c = tid % CPR, slot = tid / CPR;
      dma_barrier();  // the drain's reads of the staged tile are done
#pragma unroll
      for (int hh = 0; hh < HALVES; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[(slot * HALVES + hh) * BN + c * 8 + e] = cs[hh][e];
      dma_barrier();
      for (int t = tid; t < HALVES * BN; t += NT) {
        const int hh = t / BN, col = t % BN, n = n0 + col, mrow = m0 + hh * kColsumRows;
        if (n < g.N && mrow < g.M) {
          float sum = 0.f;
#pragma unroll
          for (int sl = 0; sl < TPC; ++sl) sum += red[(sl * HALVES + hh) * BN + col];
          g.colsum[(int64_t)(mrow / kColsumRows) * g.N + n] = sum;
        }
      }
    }
  }
}

// One output tile: bid = tile index of the problem, z = batch index, smem = the
// launch's LDS ring (at least NS (BM + BN) BK elements). T = bf16 or float: the type of
// the operands and of the outputs the epilogue writes (fp32 weight gradients aside).
template <typename T, bool A_K, bool B_K, int BM, int BN, int BK, int NS, int WM, int WN, int KIND>
__device__ __forceinline__ void gemm_dma_tile(const GemmArgs& g, int bid, int z, T* smem) {
  constexpr bool F32 = sizeof(T) == 4;
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  constexpr int STAGE = (BM + BN) * BK;  // elements per stage
  static_assert(BK * sizeof(T) == 128, "k-contiguous LDS rows of 128 bytes");
  static_assert(TM >= 1 && TN >= 1 && BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "wave tile of 32x32 blocks");
  static_assert(F32 || KIND == EPI_STORE_F32 ||
                    ((KIND == EPI_BIAS_GELU || KIND == EPI_BIAS_SPLIT) ? 2 * (BM / TM) * BN : BM * BN) <= NS * STAGE,
                "the staged epilogue fits the LDS ring");
  static_assert(!F32 || KIND != EPI_BIAS_SPLIT, "the hi/lo split is a bf16 epilogue");

  dma_lds_escape(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave / WN) * (BM / WM), wn0 = (wave % WN) * (BN / WN);
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  int tm, tn;
  map_tile<4>(bid, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  if (g.causal == CAUSAL_SKIP_UPPER && n0 > m0 + BM - 1) return;
  int kbeg, kend;
  causal_k_range(g, m0, BM, kbeg, kend);
  const int zo = z / g.zdiv, zi = z % g.zdiv;
  const int64_t aoff = zo * g.a_so + zi * g.a_si + (A_K ? (int64_t)m0 * g.lda : (int64_t)m0);
  const int64_t boff = zo * g.b_so + zi * g.b_si + (B_K ? (int64_t)n0 * g.ldb : (int64_t)n0);
  const int nseg = n0 < g.seg_n ? g.nseg : 1;

  using LA = DmaLoader<T, BM, BK, NW, A_K>;
  using LB = DmaLoader<T, BN, BK, NW, B_K>;
  LA la[kMaxSeg];
  LB lb[kMaxSeg];
#pragma unroll
  for (int s = 0; s < kMaxSeg; ++s) {
    if (s < nseg) {
      la[s].init(static_cast<const T*>(g.seg_a[s]) + aoff, g.lda, g.M - m0, g.K);
      lb[s].init(static_cast<const T*>(g.seg_b[s]) + boff, g.ldb, (s ? min(g.N, g.seg_n) : g.N) - n0, g.K);
    }
  }
  using RA = FragReader<T, BM, BK, A_K>;
  using RB = FragReader<T, BN, BK, B_K>;
  RA ra[TM];
  RB rb[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) ra[i].init(wm0 + i * 32, lane);
#pragma unroll
  for (int j = 0; j < TN; ++j) rb[j].init(wn0 + j * 32, lane);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk1 = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const int nk = nk1 * nseg;
  // per-lane offsets of the full-step loads (shared by the segments, whose operands have
  // the same strides; an m-contiguous operand masks per lane, so with several segments,
  // whose ranges differ, it stays on the general path)
  uint32_t va[LA::PER_WAVE], vb[LB::PER_WAVE];
  la[0].offsets(wave, lane, va);
  lb[0].offsets(wave, lane, vb);
  bool full_ok = (A_K || nseg == 1) && (B_K || nseg == 1);
#pragma unroll
  for (int s = 0; s < kMaxSeg; ++s)
    if (s < nseg) full_ok = full_ok && la[s].fast() && lb[s].fast();
  auto issue = [&](int t) {  // loads of step t into stage t % NS
    const int sg = (t >= nk1) + (t >= 2 * nk1);
    const int k0 = kbeg + (t - sg * nk1) * BK;
    T* st = smem + (t % NS) * STAGE;
    if (full_ok && k0 + BK <= kend) {
      if (sg == 0) {
        la[0].issue_full(st, k0, va, wave);
        lb[0].issue_full(st + BM * BK, k0, vb, wave);
      } else if (sg == 1) {
        la[1].issue_full(st, k0, va, wave);
        lb[1].issue_full(st + BM * BK, k0, vb, wave);
      } else {
        la[2].issue_full(st, k0, va, wave);
        lb[2].issue_full(st + BM * BK, k0, vb, wave);
      }
      return;
    }
    if (sg == 0) {
      la[0].issue(st, k0, kend, wave, lane);
      lb[0].issue(st + BM * BK, k0, kend, wave, lane);
    } else if (sg == 1) {
      la[1].issue(st, k0, kend, wave, lane);
      lb[1].issue(st + BM * BK, k0, kend, wave, lane);
    } else {
      la[2].issue(st, k0, kend, wave, lane);
      lb[2].issue(st + BM * BK, k0, kend, wave, lane);
    }
  };

  // Two-stage ring. The fragments of slice ks + 1 are read while slice ks is multiplied
  // (the reads spread over the slice's first MFMAs). Where the step boundary sits
  // depends on the operand layout, by measurement on the layer's shapes:
  // - both operands k-contiguous (the forward GEMMs): the boundary opens the step. The
  //   wave waits for its loads of step t, the barrier publishes every wave's loads and
  //   frees the stage of step t - 1; the first fragment reads go out, then the loads of
  //   step t + 1 into the freed stage.
  // - otherwise (dgrad and wgrad, with transposing reads): the boundary sits inside the
  //   last slice of step t, whose fragments are already in registers. The wave waits for
  //   its loads of step t + 1 and its own LDS reads, the barrier frees the stage of step
  //   t, the first fragment reads of step t + 1 and the loads of step t + 2 go out, and
  //   the last slice's MFMAs run under them, so the barrier's latency is covered by
  //   matrix work (5-7% on the paired backward launches; 2-3% slower on the forward ones).
  static_assert(NS == 2, "two-stage ring");
  constexpr int KS = BK * sizeof(T) / 32;  // slices per step (16 k of bf16, 8 k of fp32)
  static_assert(KS % 2 == 0, "slice buffers alternate; every step starts in buffer 0");
  constexpr int NM = TM * TN * kMfmaPerFrag<T>;            // MFMAs per slice
  constexpr int NR = TM * RA::READS + TN * RB::READS;      // LDS read instructions per slice
  typename RA::Frag af[2][TM];
  typename RB::Frag bfr[2][TN];
  auto read_slice = [&](const T* sA, int ks, int b) {
#pragma unroll
    for (int i = 0; i < TM; ++i) af[b][i] = ra[i].read(sA, ks, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[b][j] = rb[j].read(sA + BM * BK, ks, lane);
  };
  auto mfma_slice = [&](int b) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) mfma_frag(acc[i][j], af[b][i], bfr[b][j]);
  };
  auto interleave = [&]() {  // instruction order: next slice's reads between the first MFMAs
    constexpr int q = NR / NM, r = NR % NM;
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      if (j < r) __builtin_amdgcn_sched_group_barrier(0x100, q + 1, 0);
      else if constexpr (q > 0) __builtin_amdgcn_sched_group_barrier(0x100, q > 0 ? q : 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };
  auto inner_slices = [&](const T* sA) {  // slices 0 .. KS - 2, each reading the next
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      read_slice(sA, ks + 1, (ks + 1) & 1);
      mfma_slice(ks & 1);
      interleave();
    }
  };
  if (nk > 0) {
    issue(0);
    if constexpr (A_K && B_K) {
      for (int t = 0; t < nk; ++t) {
        wait_vmcnt<0>();
        dma_barrier();
        const T* sA = smem + (t & 1) * STAGE;
        read_slice(sA, 0, 0);
        if (t + 1 < nk) issue(t + 1);  // after the first reads, which fly under the issue
        inner_slices(sA);
        mfma_slice((KS - 1) & 1);
      }
    } else {
      wait_vmcnt<0>();
      dma_barrier();
      read_slice(smem, 0, 0);
      if (nk > 1) issue(1);
      for (int t = 0; t < nk; ++t) {
        inner_slices(smem + (t & 1) * STAGE);
        wait_lgkm_vm0();
        dma_barrier();
        read_slice(smem + ((t + 1) & 1) * STAGE, 0, 0);  // past the last step: read, unused
        if (t + 2 < nk) issue(t + 2);
        mfma_slice((KS - 1) & 1);
      }
      wait_lgkm_vm0();  // those reads land before the epilogue reuses the LDS
    }
  }

  const int64_t coff = zo * g.c_so + zi * g.c_si;
  const int64_t voff = (int64_t)z * g.vec_bs;
  if constexpr (KIND == EPI_STORE_F32 || F32) {
    // fp32 tiles do not fit the LDS ring; each lane stores its 16-byte row pieces (fp32
    // outputs of the other epilogues value by value; N is a multiple of 4 here).
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm0 + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn0 + j * 32 + q * 8 + (lane >> 5) * 4;
          float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          if (m < g.M && n < g.N) {
            if constexpr (KIND == EPI_STORE_F32) {
              epi_store4<KIND>(g, coff, voff, m, n, v);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) epi_store<float, KIND>(g, coff, voff, m, n + e, v[e]);
            }
          }
        }
      }
    }
  } else {
    epi_staged<BM, BN, TM, TN, WM, WN, KIND>(g, acc, smem, m0, n0, wm0, wn0, coff, voff);
  }
}

template <typename T, bool A_K, bool B_K, int BM, int BN, int BK, int NS, int WM, int WN, int KIND>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) T smem[NS * (BM + BN) * BK];
  gemm_dma_tile<T, A_K, B_K, BM, BN, BK, NS, WM, WN, KIND>(g, blockIdx.x, blockIdx.y, smem);
}

// Whether the DMA kernel can address the problem with elements of es bytes (2 or 4):
// every contiguous dimension, stride and batch offset a whole number of 16-byte chunks,
// 16-byte aligned bases (the bf16 epilogue writes 16-byte row chunks of C and C2, the
// fp32 one 16-byte pieces), and every byte offset from a tile's base below 4 GiB (the
// buffer resource's 32-bit range): k-contiguous 256 rows of ld, m-contiguous K rows.
inline bool dma_addressable(const GemmArgs& g, bool a_k, bool b_k, int es) {
  const int64_t epc = 16 / es;
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  if (g.M % epc || g.N % epc || g.K % epc || g.lda % epc || g.ldb % epc) return false;
  if (g.a_so % epc || g.a_si % epc || g.b_so % epc || g.b_si % epc) return false;
  if (g.ldc % epc || g.c_so % epc || g.c_si % epc || g.seg_n % epc || !a16(g.C) || !a16(g.C2)) return false;
  for (int s = 0; s < g.nseg; ++s)
    if (!a16(g.seg_a[s]) || !a16(g.seg_b[s])) return false;
  const uint64_t lim = 0xFFFFFFF0ull;
  const uint64_t a_span = (uint64_t)(a_k ? 256 : g.K) * (uint64_t)g.lda * (uint64_t)es;
  const uint64_t b_span = (uint64_t)(b_k ? 256 : g.K) * (uint64_t)g.ldb * (uint64_t)es;
  return a_span < lim && b_span < lim;
}

// Compile-time description of one problem of a paired launch.
template <bool A_K, bool B_K, int BM, int BN, int BK, int WM, int WN, int KIND>
struct DmaProblem {
  static constexpr int kBM = BM, kBN = BN, kThreads = 64 * WM * WN, kSmem = 2 * (BM + BN) * BK;
  static __device__ __forceinline__ void tile(const GemmArgs& g, int bid, int z, bf16* smem) {
    gemm_dma_tile<bf16, A_K, B_K, BM, BN, BK, 2, WM, WN, KIND>(g, bid, z, smem);
  }
};

// Two independent problems in one launch; problem i has per_z[i] tiles per batch entry.
// Blocks [0, tiles_first) run the problem named by `first` (0 or 1), the remaining
// blocks the other one, so the second problem's tiles fill the CUs the first one leaves
// idle.
template <class P0, class P1>
__global__ __launch_bounds__(P0::kThreads) void gemm_dma_pair_kernel(GemmArgs g0, GemmArgs g1, int first,
                                                                      int tiles_first, int per_z0, int per_z1) {
  static_assert(P0::kThreads == P1::kThreads, "paired problems share the work-group size");
  constexpr int SMEM = P0::kSmem > P1::kSmem ? P0::kSmem : P1::kSmem;
  __shared__ __attribute__((aligned(1024))) bf16 smem[SMEM];
  const int bid = blockIdx.x;
  const bool in_first = bid < tiles_first;
  const int local = in_first ? bid : bid - tiles_first;
  if (in_first == (first == 0)) P0::tile(g0, local % per_z0, local / per_z0, smem);
  else P1::tile(g1, local % per_z1, local / per_z1, smem);
}

}  // namespace mt
