// lce_gemm.hpp -- MFMA-tiled GEMM core for gfx950 (CDNA4) with fused epilogues.
//
// Computes, per workgroup tile, C[m][n] = sum_k A(m,k) * B(n,k) and hands the
// accumulators to an epilogue functor.  Each operand is either K-major
// (X[row][k], k contiguous) or MN-major (X[k][row], row contiguous); MN-major
// tiles are transposed in registers on their way into LDS, so the LDS layout
// and the MFMA operand reads are the same for both.
//
// LDS layout: every tile row holds 128 bytes of K (8 chunks of 16 bytes); the
// chunk c of row r sits in slot c ^ ((r ^ (r >> 3)) & 7), which keeps the
// 16-byte MFMA operand reads and both kinds of tile stores free of bank
// conflicts.
//
// bf16 / fp16: v_mfma_f32_32x32x16_bf16 / _f16, tile 256x256x64, 4 waves
//       (2 x 2), wave tile 128x128, fp32 accumulators (256 per lane, held in
//       AGPRs).
// fp64: v_mfma_f64_16x16x4_f64, tile 128x128x16, 4 waves (2 x 2), wave tile
//       64x64, fp64 accumulators.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

struct Control;

// ---------------------------------------------------------------- traits --

// 16-bit float inputs held as their bits (F16: IEEE half, else bf16) with
// fp32 accumulation.
template <bool F16_>
struct TraitsH16 {
  static constexpr bool F16 = F16_;
  typedef uint16_t E;        // bf16 or fp16 bits
  typedef float Acc;
  typedef f32x16 AccBlock;
  static constexpr int BM = 256, BN = 256, BK = 64;
  static constexpr int WAVES_M = 2, WAVES_N = 2;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int MF = 32;                 // MFMA output block edge
  static constexpr int FM = WTM / MF, FN = WTN / MF;
  static constexpr int R = 16;                  // accumulators per lane per block
  static constexpr int MIN_BLOCKS = 1;          // workgroups per CU the registers allow
  static constexpr int CE = 8;                  // elements per 16-byte chunk
  // Row of accumulator r of `lane` inside a 32x32 block; its column is lane & 31.
  __device__ static inline int row_of(int r, int lane) {
    return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
  }
  __device__ static inline int col_of(int lane) { return lane & 31; }
};
typedef TraitsH16<false> TraitsBF16;
typedef TraitsH16<true> TraitsF16;

template <class TR> struct IsH16 { static constexpr bool value = false; };
template <bool F> struct IsH16<TraitsH16<F>> { static constexpr bool value = true; };

// The 32x32x16 MFMA of the 16-bit input type.
template <class TR>
__device__ inline f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (TR::F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

struct TraitsF64 {
  static constexpr bool F16 = false;
  typedef double E;
  typedef double Acc;
  typedef f64x4 AccBlock;
  static constexpr int BM = 128, BN = 128, BK = 16;
  static constexpr int WAVES_M = 2, WAVES_N = 2;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int MF = 16;
  static constexpr int FM = WTM / MF, FN = WTN / MF;
  static constexpr int R = 4;
  static constexpr int CE = 2;
  // Two workgroups per CU (at most 256 registers per lane): with one, every
  // k-step's two barriers and LDS stores leave the matrix cores idle.
  static constexpr int MIN_BLOCKS = 2;
  // Row of accumulator r of `lane` inside a 16x16 block (v_mfma_f64_16x16x4_f64
  // interleaves the four lane groups row by row); its column is lane & 15.
  __device__ static inline int row_of(int r, int lane) { return (lane >> 4) + 4 * r; }
  __device__ static inline int col_of(int lane) { return lane & 15; }
};

__device__ inline int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical tiles so tiles that share an operand tile share
// that XCD's L2.
__device__ inline int64_t xcd_remap(int64_t b, int64_t nb) {
  const int64_t X = 8;
  const int64_t xcd = b % X, idx = b / X;
  const int64_t q = nb / X, r = nb % X;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// ------------------------------------------------------------ bf16 / f64 --

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN).
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
// fp16: v_cvt_f16_f32 rounds to nearest even.
__device__ inline uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
__device__ inline float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

template <class TR> struct Elem;
template <bool F> struct Elem<TraitsH16<F>> {
  __device__ static inline u32x4 pack(const uint16_t *v) {
    u32x4 r;
    r[0] = uint32_t(v[0]) | (uint32_t(v[1]) << 16);
    r[1] = uint32_t(v[2]) | (uint32_t(v[3]) << 16);
    r[2] = uint32_t(v[4]) | (uint32_t(v[5]) << 16);
    r[3] = uint32_t(v[6]) | (uint32_t(v[7]) << 16);
    return r;
  }
  __device__ static inline uint16_t zero() { return 0; }
};
template <> struct Elem<TraitsF64> {
  __device__ static inline u32x4 pack(const double *v) {
    u32x4 r;
    uint64_t a = __double_as_longlong(v[0]), b = __double_as_longlong(v[1]);
    r[0] = uint32_t(a); r[1] = uint32_t(a >> 32);
    r[2] = uint32_t(b); r[3] = uint32_t(b >> 32);
    return r;
  }
  __device__ static inline double zero() { return 0.0; }
};

// One 16-byte chunk of CE consecutive elements starting at p[off], elements
// whose index is not below `valid` read as zero.
template <class TR>
__device__ inline u32x4 load_chunk_elems(const typename TR::E *p, int64_t off, int valid) {
  typename TR::E v[TR::CE];
#pragma unroll
  for (int e = 0; e < TR::CE; ++e) v[e] = e < valid ? p[off + e] : Elem<TR>::zero();
  return Elem<TR>::pack(v);
}

// ------------------------------------------------------------ loaders --

// K-major operand X[row][k]: tile rows [row0, row0+ROWS), k in [k0, k0+BK).
// Rows at or past row_lim are clamped to the last row: they only feed output
// rows or columns that the epilogues never store.  Only the K tail is
// zero-filled, because it would otherwise enter every sum.
template <class TR, int ROWS, bool VEC>
struct KMajorTile {
  static constexpr int UNITS = ROWS * 8;
  static constexpr int PER_T = (UNITS + TR::NT - 1) / TR::NT;
  u32x4 reg[PER_T];
  const typename TR::E *ptr[PER_T];

  __device__ inline void init(const typename TR::E *p, int64_t ld, int64_t row0, int64_t row_lim,
                              int64_t /*row_read*/, int tid) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int u = tid + i * TR::NT;
      const int r = (u >> 3) % ROWS, c = u & 7;
      int64_t row = row0 + r;
      if (row >= row_lim) row = row_lim - 1;
      ptr[i] = p + row * ld + c * TR::CE;
    }
  }
  // Full step: every element of k0 .. k0+BK is inside the K range.
  __device__ inline void load(int64_t k0) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      if (UNITS % TR::NT != 0 && int(threadIdx.x) + i * TR::NT >= UNITS) break;
      if (VEC) {
        reg[i] = *reinterpret_cast<const u32x4 *>(ptr[i] + k0);
      } else {
        reg[i] = load_chunk_elems<TR>(ptr[i], k0, TR::CE);
      }
    }
  }
  // Tail step: elements at k >= k_lim read as zero.
  __device__ inline void load_tail(int64_t k0, int64_t k_lim) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int u = int(threadIdx.x) + i * TR::NT;
      if (UNITS % TR::NT != 0 && u >= UNITS) break;
      const int64_t k = k0 + (u & 7) * TR::CE;
      const int64_t avail = k_lim - k;
      const int valid = avail <= 0 ? 0 : (avail >= TR::CE ? TR::CE : int(avail));
      reg[i] = load_chunk_elems<TR>(ptr[i], k0, valid);
    }
  }
  __device__ inline void store(u32x4 *lds) const {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int u = int(threadIdx.x) + i * TR::NT;
      if (UNITS % TR::NT != 0 && u >= UNITS) break;
      const int r = u >> 3, c = u & 7;
      lds[r * 8 + (c ^ swz(r))] = reg[i];
    }
  }
};

// MN-major operand X[k][row] (row contiguous): each unit is a CE x CE block
// (CE k-rows by CE tile rows) that is transposed in registers.  k rows past
// k_lim read as zero.  Tile rows past row_lim feed outputs that are never
// stored: with VEC the whole 16-byte vector is clamped to end at row_read
// (the readable extent, a multiple of CE, so no vector straddles the valid
// edge); without VEC each element index is clamped to row_lim - 1.
template <class TR, int ROWS, bool VEC>
struct MNMajorTile {
  static constexpr int MB = ROWS / TR::CE;              // blocks along the tile rows
  static constexpr int UNITS = (TR::BK / TR::CE) * MB;  // = 8 * MB
  static constexpr int PER_T = (UNITS + TR::NT - 1) / TR::NT;
  u32x4 reg[PER_T][TR::CE];
  const typename TR::E *ptr[PER_T];
  int64_t ld_;
  int edge[PER_T];   // non-VEC only: valid rows in this unit's block

  __device__ inline void init(const typename TR::E *p, int64_t ld, int64_t row0, int64_t row_lim,
                              int64_t row_read, int tid) {
    ld_ = ld;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int u = (tid + i * TR::NT) % UNITS;
      const int mb = u % MB, kb = u / MB;
      int64_t mn = row0 + int64_t(mb) * TR::CE;
      if (VEC) {
        if (mn + TR::CE > row_read) mn = row_read - TR::CE;
        edge[i] = TR::CE;
      } else {
        const int64_t avail = row_lim - mn;
        edge[i] = avail >= TR::CE ? TR::CE : (avail < 1 ? 0 : int(avail));
        if (mn >= row_lim) mn = row_lim - 1;
      }
      ptr[i] = p + int64_t(kb) * TR::CE * ld + mn;
    }
  }
  __device__ inline void load_rows(int i, int64_t k0, int krows) {
    const typename TR::E *q = ptr[i] + k0 * ld_;
#pragma unroll
    for (int j = 0; j < TR::CE; ++j) {
      if (j >= krows) {
        reg[i][j] = u32x4{0u, 0u, 0u, 0u};
      } else if (VEC) {
        reg[i][j] = *reinterpret_cast<const u32x4 *>(q + j * ld_);
      } else {
        typename TR::E v[TR::CE];
        const int last = edge[i] > 0 ? edge[i] - 1 : 0;
#pragma unroll
        for (int e = 0; e < TR::CE; ++e) v[e] = q[j * ld_ + (e <= last ? e : last)];
        reg[i][j] = Elem<TR>::pack(v);
      }
    }
  }
  __device__ inline void load(int64_t k0) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      if (UNITS % TR::NT != 0 && int(threadIdx.x) + i * TR::NT >= UNITS) break;
      load_rows(i, k0, TR::CE);
    }
  }
  __device__ inline void load_tail(int64_t k0, int64_t k_lim) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int u = int(threadIdx.x) + i * TR::NT;
      if (UNITS % TR::NT != 0 && u >= UNITS) break;
      const int kb = u / MB;
      const int64_t avail = k_lim - (k0 + int64_t(kb) * TR::CE);
      load_rows(i, k0, avail <= 0 ? 0 : (avail >= TR::CE ? TR::CE : int(avail)));
    }
  }
  __device__ inline void store(u32x4 *lds) const;
};

template <class TR>
__device__ inline void transpose_block(const u32x4 *in, u32x4 *out);

// 16-bit: 8x8 transpose.  in[r] holds k = r with tile rows 0..7 in dword
// pairs; out[j] gets tile row j with k = 0..7.
__device__ inline void transpose_block16(const u32x4 *in, u32x4 *out) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = j >> 1;
#pragma unroll
    for (int pw = 0; pw < 4; ++pw) {
      const uint32_t a = in[2 * pw][w], b = in[2 * pw + 1][w];
      out[j][pw] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}
template <>
__device__ inline void transpose_block<TraitsBF16>(const u32x4 *in, u32x4 *out) {
  transpose_block16(in, out);
}
template <>
__device__ inline void transpose_block<TraitsF16>(const u32x4 *in, u32x4 *out) {
  transpose_block16(in, out);
}

template <>
__device__ inline void transpose_block<TraitsF64>(const u32x4 *in, u32x4 *out) {
  // in[0] = (k0: row0, row1), in[1] = (k1: row0, row1)
  out[0][0] = in[0][0]; out[0][1] = in[0][1]; out[0][2] = in[1][0]; out[0][3] = in[1][1];
  out[1][0] = in[0][2]; out[1][1] = in[0][3]; out[1][2] = in[1][2]; out[1][3] = in[1][3];
}

template <class TR, int ROWS, bool VEC>
__device__ inline void MNMajorTile<TR, ROWS, VEC>::store(u32x4 *lds) const {
#pragma unroll
  for (int i = 0; i < PER_T; ++i) {
    const int u = int(threadIdx.x) + i * TR::NT;
    if (UNITS % TR::NT != 0 && u >= UNITS) break;
    const int mb = u % MB, kb = u / MB;
    u32x4 out[TR::CE];
    transpose_block<TR>(reg[i], out);
#pragma unroll
    for (int j = 0; j < TR::CE; ++j) {
      const int r = mb * TR::CE + j;
      lds[r * 8 + (kb ^ swz(r))] = out[j];
    }
  }
}

template <class TR, int ROWS, bool KMAJOR, bool VEC>
struct TileLoader;
template <class TR, int ROWS, bool VEC>
struct TileLoader<TR, ROWS, true, VEC> : KMajorTile<TR, ROWS, VEC> {};
template <class TR, int ROWS, bool VEC>
struct TileLoader<TR, ROWS, false, VEC> : MNMajorTile<TR, ROWS, VEC> {};

// ------------------------------------------------------------- MFMA steps --

template <class TR> struct Mma;

template <bool F> struct Mma<TraitsH16<F>> {
  typedef TraitsH16<F> TR;
  // One BK = 64 slab from LDS: 4 MFMA k-steps of 16.
  __device__ static inline void step(const u32x4 *As, const u32x4 *Bs, int wm, int wn, int lane,
                                     typename TR::AccBlock (&acc)[TR::FM][TR::FN]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 a[TR::FM], b[TR::FN];
      const int c = kk * 2 + (lane >> 5);
#pragma unroll
      for (int fm = 0; fm < TR::FM; ++fm) {
        const int r = wm * TR::WTM + fm * 32 + (lane & 31);
        a[fm] = As[r * 8 + (c ^ swz(r))];
      }
#pragma unroll
      for (int fn = 0; fn < TR::FN; ++fn) {
        const int r = wn * TR::WTN + fn * 32 + (lane & 31);
        b[fn] = Bs[r * 8 + (c ^ swz(r))];
      }
#pragma unroll
      for (int fm = 0; fm < TR::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < TR::FN; ++fn)
          acc[fm][fn] = mfma32<TR>(a[fm], b[fn], acc[fm][fn]);
      // Bound how far the scheduler hoists operand reads of later k-steps:
      // one step of operands in flight keeps the arch VGPRs for staging.
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

template <> struct Mma<TraitsF64> {
  typedef TraitsF64 TR;
  // One BK = 16 slab: each 16-byte read feeds two MFMA k-steps of 4.  Lane
  // group g = lane/16 reads chunk pp*4+g, so step (pp, e) of group g covers
  // k = 8*pp + 2*g + e: the same bijection on both operands.
  __device__ static inline void step(const u32x4 *As, const u32x4 *Bs, int wm, int wn, int lane,
                                     TR::AccBlock (&acc)[TR::FM][TR::FN]) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      u32x4 a[TR::FM], b[TR::FN];
      const int c = pp * 4 + (lane >> 4);
#pragma unroll
      for (int fm = 0; fm < TR::FM; ++fm) {
        const int r = wm * TR::WTM + fm * 16 + (lane & 15);
        a[fm] = As[r * 8 + (c ^ swz(r))];
      }
#pragma unroll
      for (int fn = 0; fn < TR::FN; ++fn) {
        const int r = wn * TR::WTN + fn * 16 + (lane & 15);
        b[fn] = Bs[r * 8 + (c ^ swz(r))];
      }
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int fm = 0; fm < TR::FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < TR::FN; ++fn) {
            const uint64_t ab = (uint64_t(a[fm][2 * e + 1]) << 32) | a[fm][2 * e];
            const uint64_t bb = (uint64_t(b[fn][2 * e + 1]) << 32) | b[fn][2 * e];
            acc[fm][fn] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                __longlong_as_double(ab), __longlong_as_double(bb), acc[fm][fn], 0, 0, 0);
          }
    }
  }
};

// ------------------------------------------------------------- the kernel --

struct GemmParams {
  const void *A;
  int64_t lda;
  const void *B;
  int64_t ldb;
  int64_t M, N, K;
  int64_t M_read, N_read;  // readable extents of MN-major operands (multiples of CE)
  int64_t k_per_split;     // multiple of BK
  int64_t tiles_n;
  const int32_t *bad;    // when *bad != 0 the kernel exits before any write
};

// Grid: x = tiles_m * tiles_n (logical order n fastest, XCD-remapped),
//       y = number of K splits.
template <class TR, bool AK, bool BKM, bool VEC, class Epi>
__global__ void __launch_bounds__(TR::NT, TR::MIN_BLOCKS) gemm_kernel(GemmParams g, Epi epi) {
  if (g.bad && *g.bad) return;
  __shared__ u32x4 smem[(TR::BM + TR::BN) * 8];
  u32x4 *As = smem;
  u32x4 *Bs = smem + TR::BM * 8;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / TR::WAVES_N, wn = wave % TR::WAVES_N;

  const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t m0 = (L / g.tiles_n) * TR::BM;
  const int64_t n0 = (L % g.tiles_n) * TR::BN;
  const int split = blockIdx.y;
  const int64_t k_begin = int64_t(split) * g.k_per_split;
  int64_t k_end = k_begin + g.k_per_split;
  if (k_end > g.K) k_end = g.K;

  typename TR::AccBlock acc[TR::FM][TR::FN];
#pragma unroll
  for (int fm = 0; fm < TR::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < TR::FN; ++fn)
#pragma unroll
      for (int r = 0; r < TR::R; ++r) acc[fm][fn][r] = 0;

  const typename TR::E *Ap = static_cast<const typename TR::E *>(g.A);
  const typename TR::E *Bp = static_cast<const typename TR::E *>(g.B);
  TileLoader<TR, TR::BM, AK, VEC> la;
  TileLoader<TR, TR::BN, BKM, VEC> lb;
  la.init(Ap, g.lda, m0, g.M, g.M_read, tid);
  lb.init(Bp, g.ldb, n0, g.N, g.N_read, tid);

  // Full BK steps first, then at most one zero-filled tail step.
  const int64_t k_full_end = k_begin + (k_end > k_begin ? (k_end - k_begin) / TR::BK * TR::BK : 0);
  if (k_begin < k_full_end) {
    la.load(k_begin);
    lb.load(k_begin);
  }
  for (int64_t k0 = k_begin; k0 < k_full_end; k0 += TR::BK) {
    __syncthreads();
    la.store(As);
    lb.store(Bs);
    __syncthreads();
    if (k0 + TR::BK < k_full_end) {
      la.load(k0 + TR::BK);
      lb.load(k0 + TR::BK);
    }
    Mma<TR>::step(As, Bs, wm, wn, lane, acc);
  }
  if (k_full_end < k_end) {
    la.load_tail(k_full_end, k_end);
    lb.load_tail(k_full_end, k_end);
    __syncthreads();
    la.store(As);
    lb.store(Bs);
    __syncthreads();
    Mma<TR>::step(As, Bs, wm, wn, lane, acc);
  }
  // Launder the coordinates the epilogue derives its addresses from, so the
  // compiler cannot hoist that address math above the main loop (where it
  // would stay live next to the accumulators).
  int lane_e = lane, wm_e = wm, wn_e = wn;
  int64_t m0_e = m0, n0_e = n0;
  asm volatile("" : "+v"(lane_e), "+v"(wm_e), "+v"(wn_e), "+v"(m0_e), "+v"(n0_e));
  epi(acc, m0_e, n0_e, wm_e, wn_e, lane_e, split);
}

}  // namespace lce
