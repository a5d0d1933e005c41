// lce_gemm2.hpp -- pipelined 16-bit (bf16 / fp16) GEMM core for gfx950 (CDNA4).
//
// Same contract as gemm_kernel in lce_gemm.hpp (C = A(m,k) B(n,k) per
// 256x256 tile, accumulators handed to an epilogue in the 32x32x16 MFMA
// layout), built for throughput:
//   * operands go global -> LDS with buffer_load_dwordx4 ... lds (no staging
//     registers); the buffer descriptor's record count zero-fills every
//     element past the operand's valid extent, which handles the M/N edges and
//     the K tail of MN-major operands without branches;
//   * a ring of LDS stages (PipeCfg: STAGES x BK; the library runs 2 x 64,
//     128 KB) keeps the next k-steps' loads in flight; each stage ends with one
//     s_barrier after a vmcnt wait that only covers the stage about to be read;
//   * K-major tiles keep BK * 2-byte rows and are read with ds_read_b128; MN-major
//     tiles keep their global orientation (512-byte k-rows) and are read with
//     ds_read_b64_tr_b16, which hands each lane four consecutive k of one row.
//     XOR swizzles of the 16-byte chunks keep the DMA writes and both kinds of
//     operand reads free of LDS bank conflicts;
//   * operand fragments are double-buffered in registers: the MFMAs of one
//     k-substep run while the next substep's fragments are read, and the
//     stage barrier sits between the last two substeps, so LDS latency and the
//     DMA issue hide behind MFMA work;
//   * an epilogue with kStaged set gets the LDS ring (after a barrier) as
//     staging space for its output tile (staged()); otherwise operator() runs
//     straight from the accumulators.  kPrefetchBytes lets it load per-tile
//     constants before the first stages issue and write them to LDS after
//     the main loop.
// Requirements (checked by the host): 16-byte aligned bases, leading
// dimensions multiple of 8, K-major operands zero-padded (or exact) to a
// multiple of the k-step along K, 256 * ld * 2 bytes below 2^31.
#pragma once

#include <type_traits>

#include "lce_gemm.hpp"
#include "lce_internal.h"

namespace lce {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4_t;

template <int BK_, int STAGES_, int AUX_ = 0>
struct PipeCfg {
  static constexpr int BM = 256, BN = 256, BK = BK_, STAGES = STAGES_;
  static constexpr int AUX = AUX_;                    // cache-policy bits of the operand loads
  static constexpr int KSUB = BK / 16;                // MFMA k-substeps per stage
  static constexpr int ROWB = BK * 2;                  // bytes per K-major tile row
  static constexpr int OP_BYTES = 256 * BK * 2;       // per operand per stage
  static constexpr int STAGE_BYTES = 2 * OP_BYTES;
};

// 256x256 tile on 8 waves (two per SIMD), each 128 x 64: while one wave of a
// SIMD waits on LDS or the stage barrier the other keeps the matrix core busy.
template <bool F16_>
struct TraitsH16W8 : TraitsH16<F16_> {
  typedef TraitsH16<F16_> Base;
  static constexpr int WAVES_M = 2, WAVES_N = 4;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int WTM = Base::BM / WAVES_M, WTN = Base::BN / WAVES_N;
  static constexpr int FM = WTM / Base::MF, FN = WTN / Base::MF;
};
typedef TraitsH16W8<false> TraitsBF16W8;
typedef TraitsH16W8<true> TraitsF16W8;

// The 8-wave traits of a 16-bit input type.
template <class TR> struct W8Of;
template <bool F> struct W8Of<TraitsH16<F>> { typedef TraitsH16W8<F> type; };

// Chunk swizzles.  K-major rows of 64 bytes (BK 32) or 128 bytes (BK 64): the
// rows read by 16 consecutive lanes land in 16 distinct 16-byte bank groups of
// a 256-byte window, and any 8 consecutive rows in 8 distinct groups of a
// 128-byte window.  MN-major (512-byte k-rows): the four k-rows x 32 bytes read
// by a 16-lane group of ds_read_b64_tr_b16, and the two such groups reading
// the same k-rows, never share a bank.
template <int ROWB>
__device__ inline int kswz(int r) {
  if (ROWB == 64) return ((r >> 1) & 3) ^ ((r >> 3) & 1);
  return ((r >> 1) & 7) ^ ((r & 1) << 2);
}
__device__ inline int mswz2(int q) { return (q & 3) << 2; }

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7fffffff) bytes = 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), 0x00020000);
}

// One 16-byte-per-lane load from the buffer `rs` at byte offset `voff` into
// LDS at `dst` + 16 * lane.
template <int AUX>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, char *dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)dst, 16, voff, 0, 0, AUX);
}

// One operand of one stage: OP_BYTES / 1 KB wave-instructions, INSTR per wave.
template <class CFG, int NWAVES, bool KMAJOR>
struct PipeOperand {
  static constexpr int INSTR = CFG::OP_BYTES / 1024 / NWAVES;
  const uint16_t *p;   // operand base (element 0 of row/k-row 0)
  int64_t ld;          // leading dimension in elements
  int64_t row0;        // first tile row (M or N index)
  int64_t row_lim;     // valid rows (K-major) / readable row length (MN-major)
  int64_t k_lim;       // valid k (MN-major zero-fill)
  uint32_t voff[INSTR];  // per-lane byte offsets
  __amdgpu_buffer_rsrc_t rs;

  __device__ inline void init(const uint16_t *p_, int64_t ld_, int64_t row0_, int64_t row_lim_,
                              int64_t k_lim_, int wave, int lane) {
    p = p_; ld = ld_; row0 = row0_; row_lim = row_lim_; k_lim = k_lim_;
    constexpr int CPR = CFG::ROWB / 16;   // 16-byte chunks per K-major row
    if (KMAJOR) {
      rs = make_rsrc(p + row0 * ld, (row_lim - row0) * ld * 2);
#pragma unroll
      for (int i = 0; i < INSTR; ++i) {
        const int j = wave * INSTR + i;
        const int r = (64 / CPR) * j + lane / CPR;
        const int c = (lane % CPR) ^ kswz<CFG::ROWB>(r);
        voff[i] = uint32_t(r) * uint32_t(ld * 2) + uint32_t(c * 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < INSTR; ++i) {
        const int j = wave * INSTR + i;
        const int q = 2 * j + (lane >> 5);
        const int c = (lane & 31) ^ mswz2(q);
        voff[i] = uint32_t(q) * uint32_t(ld * 2) + uint32_t(c * 16);
      }
    }
  }

  // K-major: point the loads at the tile whose first row is row0_.
  __device__ inline void retarget(int64_t row0_) {
    row0 = row0_;
    rs = make_rsrc(p + row0 * ld, (row_lim - row0) * ld * 2);
  }

  // Issue this wave's loads of k-step k0 into the operand region `dst`.
  __device__ inline void issue(int64_t k0, char *dst, int wave) const {
    if (KMAJOR) {
#pragma unroll
      for (int i = 0; i < INSTR; ++i) {
        const int j = wave * INSTR + i;
        dma16<CFG::AUX>(rs, dst + j * 1024, voff[i] + uint32_t(k0 * 2));
      }
    } else {
      // base at (k0, row0): bytes up to the end of row k_lim-1's readable part
      const int64_t rows = k_lim - k0;
      const int64_t bytes = rows > 0 ? ((rows - 1) * ld + (row_lim - row0)) * 2 : 0;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(p + k0 * ld + row0, bytes);
#pragma unroll
      for (int i = 0; i < INSTR; ++i) {
        const int j = wave * INSTR + i;
        dma16<CFG::AUX>(r, dst + j * 1024, voff[i]);
      }
    }
  }

  // MN-major reads issued by hand (mn_frag_addr, mn_reads, mn_substep): the
  // LDS address of the fragment of tile rows base..base+31 at k-substep 0 of
  // the stage at `src`; substep kk adds kk * 16 k-rows of 512 bytes, the
  // second half of the fragment 4 k-rows more (both fit the instruction's
  // offset).
  __device__ inline uint32_t mn_frag_addr(const char *src, int base, int lane) const {
    static_assert(!KMAJOR, "MN-major operands only");
    const int g = lane >> 4, i = lane & 15;
    const int mn = base + 16 * (g & 1) + 4 * (i & 3);
    const int krow = 8 * (g >> 1) + (i >> 2);
    const char *a = src + krow * 512 + (((mn >> 3) ^ mswz2(krow)) << 4) + (mn & 7) * 2;
    // generic -> LDS address space: the 32-bit LDS byte address
    return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)a));
  }

  // The 32x32x16 MFMA operand of tile rows base..base+31 for k-substep kk.
  __device__ inline u32x4 frag(const char *src, int base, int kk, int lane) const {
    if (KMAJOR) {
      const int r = base + (lane & 31);
      const int c = kk * 2 + (lane >> 5);
      return *reinterpret_cast<const u32x4 *>(src + r * CFG::ROWB +
                                              ((c ^ kswz<CFG::ROWB>(r)) << 4));
    } else {
      const int g = lane >> 4, i = lane & 15;
      const int mn = base + 16 * (g & 1) + 4 * (i & 3);
      const int kb = kk * 16 + 8 * (g >> 1) + (i >> 2);
      u32x4 out;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int krow = kb + 4 * q;
        const char *a = src + krow * 512 + (((mn >> 3) ^ mswz2(krow)) << 4) + (mn & 7) * 2;
        const shortx4 h = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t *)(a));
        out[2 * q] = uint32_t(uint16_t(h[0])) | (uint32_t(uint16_t(h[1])) << 16);
        out[2 * q + 1] = uint32_t(uint16_t(h[2])) | (uint32_t(uint16_t(h[3])) << 16);
      }
      return out;
    }
  }
};

struct Gemm2Params {
  const void *A;
  int64_t lda;
  const void *B;
  int64_t ldb;
  int64_t M, N, K;          // K: valid depth (K-major operands are zero-padded past it)
  int64_t M_read, N_read;   // readable row lengths of MN-major operands
  int64_t k_per_split;      // multiple of the configuration's k-step
  int64_t tiles_n;
  const int32_t *bad;
};

// f(std::integral_constant<int, I>) for I = B .. E-1, in order.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Hand-issued MN-major fragment reads (ds_read_b64_tr_b16) for the 8-wave
// 128 x 64 wave tile: four A fragments and two B fragments per k-substep,
// each two 8-byte transposing reads (k-rows +0 and +4).  Every block below
// ends with its own s_waitcnt lgkmcnt(0), so no read is in flight once the
// asm statement is over and the compiler may use the output registers freely.
// (The builtin form of these reads makes the compiler wait for every operand
// DMA in flight first, which exposes a whole stage load per k-step.)
#define LCE_MN_RD(LO, HI, AD, OL, OH)                         \
  "ds_read_b64_tr_b16 %" #LO ", %" #AD " offset:" OL "\n\t"   \
  "ds_read_b64_tr_b16 %" #HI ", %" #AD " offset:" OH "\n\t"
// Operands: %0..%11 the six fragments' low / high halves (outputs), %12..%17
// their addresses.
#define LCE_MN_READS(OL, OH)                                                         \
  LCE_MN_RD(0, 1, 12, OL, OH) LCE_MN_RD(2, 3, 13, OL, OH) LCE_MN_RD(4, 5, 14, OL, OH)   \
  LCE_MN_RD(6, 7, 15, OL, OH) LCE_MN_RD(8, 9, 16, OL, OH) LCE_MN_RD(10, 11, 17, OL, OH) \
  "s_waitcnt lgkmcnt(0)"
// One k-substep: the eight MFMAs acc[fm][fn] += A[fm] B[fn] on the current
// fragments, with the next substep's six fragments read between them.
// Operands: %0..%7 acc[0][0], acc[0][1], .. acc[3][1]; %8..%19 the next
// fragments' halves (outputs); %20..%23 A[0..3]; %24, %25 B[0..1]; %26..%31
// the next fragments' addresses.
#define LCE_MN_SUBSTEP(MF, OL, OH)                                           \
  MF " %0, %20, %24, %0\n\t" LCE_MN_RD(8, 9, 26, OL, OH)                     \
  MF " %1, %20, %25, %1\n\t" LCE_MN_RD(10, 11, 27, OL, OH)                   \
  MF " %2, %21, %24, %2\n\t" LCE_MN_RD(12, 13, 28, OL, OH)                   \
  MF " %3, %21, %25, %3\n\t" LCE_MN_RD(14, 15, 29, OL, OH)                   \
  MF " %4, %22, %24, %4\n\t" LCE_MN_RD(16, 17, 30, OL, OH)                   \
  MF " %5, %22, %25, %5\n\t" LCE_MN_RD(18, 19, 31, OL, OH)                   \
  MF " %6, %23, %24, %6\n\t"                                                 \
  MF " %7, %23, %25, %7\n\t"                                                 \
  "s_waitcnt lgkmcnt(0)"

__device__ __forceinline__ void mn_join(u32x4 &f, u32x2 lo, u32x2 hi) {
  f = u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// The six fragments of substep KK at the addresses ad[0..5] (A[0..3], B[0..1]).
template <int KK>
__device__ __forceinline__ void mn_reads(u32x4 (&fa)[4], u32x4 (&fb)[2], const uint32_t (&ad)[6]) {
  static_assert(KK >= 0 && KK < 4, "k-substep");
  u32x2 h[12];
#define LCE_MN_READS_ASM(OL, OH)                                                       \
  asm volatile(LCE_MN_READS(OL, OH)                                                      \
               : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3]), "=&v"(h[4]),        \
                 "=&v"(h[5]), "=&v"(h[6]), "=&v"(h[7]), "=&v"(h[8]), "=&v"(h[9]),        \
                 "=&v"(h[10]), "=&v"(h[11])                                              \
               : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]))
  if constexpr (KK == 0) LCE_MN_READS_ASM("0", "2048");
  else if constexpr (KK == 1) LCE_MN_READS_ASM("8192", "10240");
  else if constexpr (KK == 2) LCE_MN_READS_ASM("16384", "18432");
  else LCE_MN_READS_ASM("24576", "26624");
#undef LCE_MN_READS_ASM
#pragma unroll
  for (int i = 0; i < 4; ++i) mn_join(fa[i], h[2 * i], h[2 * i + 1]);
#pragma unroll
  for (int i = 0; i < 2; ++i) mn_join(fb[i], h[8 + 2 * i], h[9 + 2 * i]);
}

// One k-substep on fragments (a, b) while reading the next substep's
// fragments (substep KK of the stage the addresses ad[] point into) into
// (na, nb).  F16: fp16 inputs (else bf16).
template <bool F16, int KK>
__device__ __forceinline__ void mn_substep(f32x16 (&acc)[4][2], const u32x4 (&a)[4],
                                           const u32x4 (&b)[2], const uint32_t (&ad)[6],
                                           u32x4 (&na)[4], u32x4 (&nb)[2]) {
  static_assert(KK >= 0 && KK < 4, "k-substep");
  u32x2 h[12];
#define LCE_MN_SUBSTEP_ASM(MF, OL, OH)                                                  \
  asm volatile(LCE_MN_SUBSTEP(MF, OL, OH)                                                 \
               : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]),      \
                 "+v"(acc[2][0]), "+v"(acc[2][1]), "+v"(acc[3][0]), "+v"(acc[3][1]),      \
                 "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3]), "=&v"(h[4]),         \
                 "=&v"(h[5]), "=&v"(h[6]), "=&v"(h[7]), "=&v"(h[8]), "=&v"(h[9]),         \
                 "=&v"(h[10]), "=&v"(h[11])                                               \
               : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]),        \
                 "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]))
#define LCE_MN_SUBSTEP_KK(MF)                                       \
  if constexpr (KK == 0) LCE_MN_SUBSTEP_ASM(MF, "0", "2048");             \
  else if constexpr (KK == 1) LCE_MN_SUBSTEP_ASM(MF, "8192", "10240");    \
  else if constexpr (KK == 2) LCE_MN_SUBSTEP_ASM(MF, "16384", "18432");   \
  else LCE_MN_SUBSTEP_ASM(MF, "24576", "26624");
  if constexpr (F16) {
    LCE_MN_SUBSTEP_KK("v_mfma_f32_32x32x16_f16")
  } else {
    LCE_MN_SUBSTEP_KK("v_mfma_f32_32x32x16_bf16")
  }
#undef LCE_MN_SUBSTEP_KK
#undef LCE_MN_SUBSTEP_ASM
#pragma unroll
  for (int i = 0; i < 4; ++i) mn_join(na[i], h[2 * i], h[2 * i + 1]);
#pragma unroll
  for (int i = 0; i < 2; ++i) mn_join(nb[i], h[8 + 2 * i], h[9 + 2 * i]);
}

// s_waitcnt lgkmcnt(0) vmcnt(N) followed by a bare s_barrier: unlike
// __syncthreads this leaves the N most recent loads in flight.
template <int N>
__device__ inline void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt lgkmcnt(0) vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
// The same with the count chosen at run time among 0, L, 2L, ... (L loads per
// stage, up to S stages).
template <int L, int S>
__device__ inline void wait_vm_barrier_stages(int stages) {
  if constexpr (S > 0) {
    if (stages >= S) { wait_vm_barrier<L * S>(); return; }
    wait_vm_barrier_stages<L, S - 1>(stages);
  } else {
    wait_vm_barrier<0>();
  }
}

// Optional epilogue hooks: kStaged (staged() gets the LDS ring after the main
// loop) and kPrefetchBytes (pre_load() runs before the first operand load and
// its values stay in registers through the main loop, so their latency hides
// behind it; pre_store() then writes per-tile constants to an LDS area of that
// size past the ring, which staged() reads).
template <class E, class = void> struct EpiStaged { static constexpr bool value = false; };
template <class E>
struct EpiStaged<E, std::void_t<decltype(E::kStaged)>> { static constexpr bool value = E::kStaged; };
template <class E, class = void> struct EpiPrefetch { static constexpr int bytes = 0; };
template <class E>
struct EpiPrefetch<E, std::void_t<decltype(E::kPrefetchBytes)>> {
  static constexpr int bytes = E::kPrefetchBytes;
};

// LDS bytes a product needs (ring + epilogue prefetch table).
template <class CFG, class Epi> constexpr int gemm2_lds_bytes() {
  return CFG::STAGES * CFG::STAGE_BYTES + EpiPrefetch<Epi>::bytes;
}

// One tile of a product: logical index LS (split-major over (split, tile));
// `smem` at least gemm2_lds_bytes<CFG, Epi>() bytes (1 KB aligned).
template <class CFG, class TR, bool AK, bool BKM, class Epi>
__device__ __forceinline__ void gemm2_tile(const Gemm2Params &g, const Epi &epi, int64_t LS,
                                           char *smem) {
  constexpr int BK = CFG::BK, STAGES = CFG::STAGES, KSUB = CFG::KSUB;
  constexpr int NWAVES = TR::NT / 64;
  typedef PipeOperand<CFG, NWAVES, AK> OpA;
  typedef PipeOperand<CFG, NWAVES, BKM> OpB;
  constexpr int LPS = OpA::INSTR + OpB::INSTR;          // loads per stage per wave
  constexpr int NMF = TR::FM * TR::FN;                   // MFMAs per substep
  constexpr int NDS = TR::FM * (AK ? 1 : 2) + TR::FN * (BKM ? 1 : 2);  // LDS reads per substep
  static_assert(KSUB % 2 == 0 && KSUB >= 2, "fragment double-buffer parity");
  static_assert(TR::BM == CFG::BM && TR::BN == CFG::BN, "tile");
  if (g.bad && *g.bad) return;
  constexpr int PRE = EpiPrefetch<Epi>::bytes;
  char *const pre_lds = smem + STAGES * CFG::STAGE_BYTES;

  // (opaque: a workgroup running several tiles recomputes its per-lane set-up
  // per tile instead of holding every product's across the whole loop)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / TR::WAVES_N, wn = wave % TR::WAVES_N;

  const int64_t tiles = (g.M + CFG::BM - 1) / CFG::BM * g.tiles_n;
  const int split = int(LS / tiles);
  const int64_t L = LS % tiles;
  const int64_t m0 = (L / g.tiles_n) * CFG::BM;
  const int64_t n0 = (L % g.tiles_n) * CFG::BN;
  const int64_t k_begin = int64_t(split) * g.k_per_split;
  int64_t k_end = k_begin + g.k_per_split;
  if (k_end > g.K) k_end = g.K;
  const int n_k = k_end > k_begin ? int((k_end - k_begin + BK - 1) / BK) : 0;

  typename TR::AccBlock acc[TR::FM][TR::FN];
#pragma unroll
  for (int fm = 0; fm < TR::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < TR::FN; ++fn)
#pragma unroll
      for (int r = 0; r < TR::R; ++r) acc[fm][fn][r] = 0;

  OpA pa;
  OpB pb;
  pa.init(static_cast<const uint16_t *>(g.A), g.lda, m0, AK ? g.M : g.M_read, g.K, wave, lane);
  pb.init(static_cast<const uint16_t *>(g.B), g.ldb, n0, BKM ? g.N : g.N_read, g.K, wave, lane);

  // Epilogue constants: loaded before the operands, consumed after the main
  // loop (the last stage wait covers them).
  [[maybe_unused]] auto pre = [&] {
    if constexpr (PRE > 0) return epi.pre_load(m0, n0, tid);
    else return 0;
  }();

  // Prologue: every stage of the ring in flight; wait for stage 0 and read its
  // first k-substep fragments.
#pragma unroll
  for (int s = 0; s < STAGES; ++s) {
    if (s < n_k) {
      char *st = smem + s * CFG::STAGE_BYTES;
      pa.issue(k_begin + int64_t(s) * BK, st, wave);
      pb.issue(k_begin + int64_t(s) * BK, st + CFG::OP_BYTES, wave);
    }
  }
  wait_vm_barrier_stages<LPS, STAGES - 1>(n_k - 1);
  u32x4 fa[2][TR::FM], fb[2][TR::FN];
  // Both operands MN-major: fragments come from hand-issued transposing reads
  // (see mn_step); their lane addresses within a stage are fixed.
  constexpr bool MNMN = !AK && !BKM;
  uint32_t a_off[TR::FM], b_off[TR::FN];
  if constexpr (MNMN) {
#pragma unroll
    for (int f = 0; f < TR::FM; ++f) a_off[f] = pa.mn_frag_addr(smem, wm * TR::WTM + f * 32, lane);
#pragma unroll
    for (int f = 0; f < TR::FN; ++f)
      b_off[f] = pb.mn_frag_addr(smem + CFG::OP_BYTES, wn * TR::WTN + f * 32, lane);
  }
  if (n_k > 0) {
    if constexpr (MNMN) {
      const uint32_t ad[6] = {a_off[0], a_off[1], a_off[2], a_off[3], b_off[0], b_off[1]};
      mn_reads<0>(fa[0], fb[0], ad);
    } else {
#pragma unroll
      for (int f = 0; f < TR::FM; ++f) fa[0][f] = pa.frag(smem, wm * TR::WTM + f * 32, 0, lane);
#pragma unroll
      for (int f = 0; f < TR::FN; ++f)
        fb[0][f] = pb.frag(smem + CFG::OP_BYTES, wn * TR::WTN + f * 32, 0, lane);
    }
  }

  // One k-step of an MN-major x MN-major product.  Same dataflow as `step`
  // below, in a fixed instruction order: each substep is one asm block that
  // alternates one MFMA with one fragment (two transposing reads) of the next
  // substep and ends waiting for those reads.  The compiler does not see
  // these reads, so it does not hold them until the next stage's loads have
  // landed (which would expose the whole load latency each step).
  auto mn_step = [&](const int it, auto steady_tag) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    static_assert(TR::FM == 4 && TR::FN == 2 && CFG::KSUB == 4 && CFG::BM == 256 &&
                      CFG::BN == 256,
                  "the asm substeps assume 128 x 64 wave tiles, k64 stages and 512-byte k-rows");
    const uint32_t sa = uint32_t((it % CFG::STAGES) * CFG::STAGE_BYTES);
    const uint32_t sn = uint32_t(((it + 1) % CFG::STAGES) * CFG::STAGE_BYTES);
    char *sa_p = smem + sa;
    static_for<0, CFG::KSUB>([&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      constexpr int cur = kk & 1, nxt = cur ^ 1;
      constexpr bool last = kk == CFG::KSUB - 1;
      constexpr int ks = last ? 0 : kk + 1;
      // (the last substep of the last k-step also reads: the next stage's
      // slot holds stale data then, read and discarded, which keeps one
      // straight-line register schedule for every k-step)
      const uint32_t so = last ? sn : sa;
      const uint32_t ad[6] = {a_off[0] + so, a_off[1] + so, a_off[2] + so,
                              a_off[3] + so, b_off[0] + so, b_off[1] + so};
      mn_substep<TR::F16, ks>(acc, fa[cur], fb[cur], ad, fa[nxt], fb[nxt]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kk == CFG::KSUB - 2) {
        if (STEADY) wait_vm_barrier<LPS * (CFG::STAGES - 2)>();
        else wait_vm_barrier_stages<LPS, CFG::STAGES - 2>(n_k - 2 - it);
        if (STEADY || it + CFG::STAGES < n_k) {
          pa.issue(k_begin + int64_t(it + CFG::STAGES) * CFG::BK, sa_p, wave);
          pb.issue(k_begin + int64_t(it + CFG::STAGES) * CFG::BK, sa_p + CFG::OP_BYTES, wave);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  };

  // One k-step of BK = KSUB MFMA k-substeps.  Substep kk computes on the
  // fragments read during substep kk-1 while reading those of kk+1 (of the
  // next stage for the last substep).  Between the last two substeps: stage
  // it+1 has landed in every wave's view and stage it is in registers
  // everywhere, so its buffer is refilled with stage it+STAGES.  STEADY: a
  // refill is due and STAGES-2 later stages are in flight.
  auto step = [&](const int it, auto steady_tag) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    char *sa = smem + (it % CFG::STAGES) * CFG::STAGE_BYTES;
    const char *sn = smem + ((it + 1) % CFG::STAGES) * CFG::STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < CFG::KSUB; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      const bool last = kk == CFG::KSUB - 1;
      if (!last || STEADY || it + 1 < n_k) {
        const char *src = last ? sn : sa;
        const int ks = last ? 0 : kk + 1;
#pragma unroll
        for (int f = 0; f < TR::FM; ++f) fa[nxt][f] = pa.frag(src, wm * TR::WTM + f * 32, ks, lane);
#pragma unroll
        for (int f = 0; f < TR::FN; ++f)
          fb[nxt][f] = pb.frag(src + CFG::OP_BYTES, wn * TR::WTN + f * 32, ks, lane);
      }
#pragma unroll
      for (int fm = 0; fm < TR::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < TR::FN; ++fn)
          acc[fm][fn] = mfma32<TR>(fa[cur][fm], fb[cur][fn], acc[fm][fn]);
      // Interleave: one MFMA, then (while any remain) one refill load and one
      // LDS read.
      constexpr int NDS_I = NDS < NMF ? NDS : NMF;
      if (last && STEADY) {
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < LPS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          if (i < NDS_I) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else if (!last) {
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < NDS_I) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      if (kk == CFG::KSUB - 2) {
        if (STEADY) wait_vm_barrier<LPS * (CFG::STAGES - 2)>();
        else wait_vm_barrier_stages<LPS, CFG::STAGES - 2>(n_k - 2 - it);
        if (STEADY || it + CFG::STAGES < n_k) {
          pa.issue(k_begin + int64_t(it + CFG::STAGES) * CFG::BK, sa, wave);
          pb.issue(k_begin + int64_t(it + CFG::STAGES) * CFG::BK, sa + CFG::OP_BYTES, wave);
        }
      }
    }
  };
  int it = 0;
  if constexpr (MNMN) {
    for (; it + STAGES < n_k; ++it) mn_step(it, std::true_type{});
    for (; it < n_k; ++it) mn_step(it, std::false_type{});
    // The accumulators were last written by MFMAs inside asm blocks, which the
    // compiler's hazard tracking does not see: give the matrix core's result
    // latency (at most 16 passes) before any other instruction reads them
    // (the accumulators are operands, so no read moves above the wait).
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]),
                   "+v"(acc[2][0]), "+v"(acc[2][1]), "+v"(acc[3][0]), "+v"(acc[3][1])
                 :
                 : "memory");
  } else {
    for (; it + STAGES < n_k; ++it) step(it, std::true_type{});
    for (; it < n_k; ++it) step(it, std::false_type{});
  }

  int lane_e = lane, wm_e = wm, wn_e = wn;
  int64_t m0_e = m0, n0_e = n0;
  asm volatile("" : "+v"(lane_e), "+v"(wm_e), "+v"(wn_e), "+v"(m0_e), "+v"(n0_e));
  if constexpr (EpiStaged<Epi>::value) {
    // The epilogue reuses the stage ring as staging space: every wave must be
    // done reading its operand fragments first.
    __syncthreads();
    if constexpr (PRE > 0) {
      if (tid < CFG::BN) epi.pre_store(pre, m0_e, n0_e, tid, pre_lds);
      __syncthreads();
    }
    epi.staged(acc, m0_e, n0_e, wm_e, wn_e, lane_e, split, smem, pre_lds);
  } else {
    epi(acc, m0_e, n0_e, wm_e, wn_e, lane_e, split);
  }
}

// One workgroup of a product: `bid` of `nb` workgroups of this product, of
// which the first `nreal` logical ones carry work (nb may be padded to a
// multiple of the XCD count so that a following product keeps its XCD
// mapping).  One flat grid over (split, tile), split-major, dealt to the XCDs
// in contiguous ranges: an XCD's workgroups share whole K-splits, so each
// split's operand rows are fetched into one L2 only.
template <class CFG, class TR, bool AK, bool BKM, class Epi>
__device__ __forceinline__ void gemm2_block(const Gemm2Params &g, const Epi &epi, int64_t bid,
                                            int64_t nb, int64_t nreal, char *smem) {
  const int64_t LS = xcd_remap(bid, nb);
  if (LS >= nreal) return;   // padding
  gemm2_tile<CFG, TR, AK, BKM, Epi>(g, epi, LS, smem);
}

template <class CFG, class TR, bool AK, bool BKM, class Epi>
__global__ void __launch_bounds__(TR::NT) gemm2_kernel(Gemm2Params g, Epi epi) {
  __shared__ __attribute__((aligned(1024))) char smem[gemm2_lds_bytes<CFG, Epi>()];
  gemm2_block<CFG, TR, AK, BKM, Epi>(g, epi, blockIdx.x, gridDim.x, gridDim.x, smem);
}

// Persistent form for K-major x K-major products with one K-split and a
// register-only epilogue (the forward's online LSE): one workgroup per CU
// walks its tiles as a single stream of k-steps, so the operand ring keeps
// loading the next tile's first stages while the current tile finishes its
// last k-steps and its epilogue, and no tile starts on an empty pipeline.
// Tiles are dealt as xcd_remap does: each XCD owns a contiguous range of
// logical tiles and its workgroups take consecutive tiles of it in rounds.
template <class CFG, class TR, class Epi>
__global__ void __launch_bounds__(TR::NT) gemm2_persistent_kernel(Gemm2Params g, Epi epi) {
  constexpr int BK = CFG::BK, STAGES = CFG::STAGES, KSUB = CFG::KSUB;
  constexpr int NWAVES = TR::NT / 64;
  typedef PipeOperand<CFG, NWAVES, true> Op;
  constexpr int LPS = 2 * Op::INSTR;
  constexpr int NMF = TR::FM * TR::FN;
  constexpr int NDS = TR::FM + TR::FN;
  static_assert(KSUB % 2 == 0 && KSUB >= 2, "fragment double-buffer parity");
  static_assert(!EpiStaged<Epi>::value && EpiPrefetch<Epi>::bytes == 0, "register epilogue");
  if (g.bad && *g.bad) return;
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * CFG::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / TR::WAVES_N, wn = wave % TR::WAVES_N;

  // this workgroup's tiles: lo + slot + j * per_xcd, j = 0.., below hi
  const int64_t tiles = (g.M + CFG::BM - 1) / CFG::BM * g.tiles_n;
  const int64_t X = 8, nb = gridDim.x;
  const int64_t xcd = blockIdx.x % X, slot = blockIdx.x / X;
  const int64_t per_xcd = nb / X + (xcd < nb % X ? 1 : 0);
  const int64_t q8 = tiles / X, r8 = tiles % X;
  const int64_t lo = xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8;
  const int64_t hi = lo + q8 + (xcd < r8 ? 1 : 0);
  const int64_t my_tiles = lo + slot < hi ? (hi - lo - slot + per_xcd - 1) / per_xcd : 0;
  const int n_k = int((g.K + BK - 1) / BK);
  if (my_tiles == 0 || n_k == 0) return;
  const int64_t total = my_tiles * n_k;
  auto tile_m0 = [&](int64_t j) { return ((lo + slot + j * per_xcd) / g.tiles_n) * CFG::BM; };
  auto tile_n0 = [&](int64_t j) { return ((lo + slot + j * per_xcd) % g.tiles_n) * CFG::BN; };

  typename TR::AccBlock acc[TR::FM][TR::FN];
#pragma unroll
  for (int fm = 0; fm < TR::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < TR::FN; ++fn)
#pragma unroll
      for (int r = 0; r < TR::R; ++r) acc[fm][fn][r] = 0;

  // Load stream: the next global k-step to load is k-step ld_k of tile
  // ld_t; stage slots rotate with the global step.
  Op pa, pb;
  pa.init(static_cast<const uint16_t *>(g.A), g.lda, tile_m0(0), g.M, g.K, wave, lane);
  pb.init(static_cast<const uint16_t *>(g.B), g.ldb, tile_n0(0), g.N, g.K, wave, lane);
  int64_t ld_t = 0;
  int ld_k = 0;
  auto issue = [&](int64_t q) {
    if (ld_k == n_k) {
      ld_k = 0;
      ++ld_t;
      pa.retarget(tile_m0(ld_t));
      pb.retarget(tile_n0(ld_t));
    }
    char *st = smem + (q % STAGES) * CFG::STAGE_BYTES;
    const int64_t k0 = int64_t(ld_k) * BK;
    pa.issue(k0, st, wave);
    pb.issue(k0, st + CFG::OP_BYTES, wave);
    ++ld_k;
  };
  int64_t cp_t = 0;   // tile being computed
  int cp_k = 0;       // its k-step

#pragma unroll
  for (int s2 = 0; s2 < STAGES; ++s2)
    if (s2 < total) issue(s2);
  wait_vm_barrier_stages<LPS, STAGES - 1>(int(total - 1 < STAGES - 1 ? total - 1 : STAGES - 1));
  u32x4 fa[2][TR::FM], fb[2][TR::FN];
#pragma unroll
  for (int f = 0; f < TR::FM; ++f) fa[0][f] = pa.frag(smem, wm * TR::WTM + f * 32, 0, lane);
#pragma unroll
  for (int f = 0; f < TR::FN; ++f)
    fb[0][f] = pb.frag(smem + CFG::OP_BYTES, wn * TR::WTN + f * 32, 0, lane);

  auto step = [&](const int64_t q, auto steady_tag) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    char *sa = smem + (q % STAGES) * CFG::STAGE_BYTES;
    const char *sn = smem + ((q + 1) % STAGES) * CFG::STAGE_BYTES;
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      const bool last = kk == KSUB - 1;
      if (!last || STEADY || q + 1 < total) {
        const char *src = last ? sn : sa;
        const int ks = last ? 0 : kk + 1;
#pragma unroll
        for (int f = 0; f < TR::FM; ++f) fa[nxt][f] = pa.frag(src, wm * TR::WTM + f * 32, ks, lane);
#pragma unroll
        for (int f = 0; f < TR::FN; ++f)
          fb[nxt][f] = pb.frag(src + CFG::OP_BYTES, wn * TR::WTN + f * 32, ks, lane);
      }
#pragma unroll
      for (int fm = 0; fm < TR::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < TR::FN; ++fn)
          acc[fm][fn] = mfma32<TR>(fa[cur][fm], fb[cur][fn], acc[fm][fn]);
      constexpr int NDS_I = NDS < NMF ? NDS : NMF;
      if (last && STEADY) {
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < LPS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          if (i < NDS_I) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else if (!last) {
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < NDS_I) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      if (kk == KSUB - 2) {
        if (STEADY) wait_vm_barrier<LPS * (STAGES - 2)>();
        else wait_vm_barrier_stages<LPS, STAGES - 2>(int(total - 2 - q));
        if (STEADY || q + STAGES < total) issue(q + STAGES);
      }
    }
    if (++cp_k == n_k) {   // tile cp_t is complete
      cp_k = 0;
      const int64_t j = cp_t++;
      int lane_e = lane, wm_e = wm, wn_e = wn;
      int64_t m0_e = tile_m0(j), n0_e = tile_n0(j);
      asm volatile("" : "+v"(lane_e), "+v"(wm_e), "+v"(wn_e), "+v"(m0_e), "+v"(n0_e));
      epi(acc, m0_e, n0_e, wm_e, wn_e, lane_e, 0);
#pragma unroll
      for (int fm = 0; fm < TR::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < TR::FN; ++fn)
#pragma unroll
          for (int r = 0; r < TR::R; ++r) acc[fm][fn][r] = 0;
    }
  };
  int64_t q = 0;
  for (; q + STAGES < total; ++q) step(q, std::true_type{});
  for (; q < total; ++q) step(q, std::false_type{});
}

// One product of a multi-product launch.
template <class CFG_, bool AK_, bool BKM_, class Epi_>
struct Gemm2Job {
  typedef CFG_ CFG;
  typedef Epi_ Epi;
  static constexpr bool AK = AK_, BKM = BKM_;
  Gemm2Params g;
  Epi e;
  int64_t nb;      // workgroups launched, a multiple of 8 (0: absent from this launch)
  int64_t nreal;   // workgroups with work (tiles x splits)
};

// Three independent products in one grid: workgroups [0, j0.nb) run j0, the
// next j1.nb run j1, then j2.  Longer-running products go first so that the
// store-bound epilogues of early finishers overlap later products' main loops.
template <class TR, class J0, class J1, class J2>
__global__ void __launch_bounds__(TR::NT) gemm2_multi_kernel(J0 j0, J1 j1, J2 j2) {
  constexpr int B0 = gemm2_lds_bytes<typename J0::CFG, typename J0::Epi>();
  constexpr int B1 = gemm2_lds_bytes<typename J1::CFG, typename J1::Epi>();
  constexpr int B2 = gemm2_lds_bytes<typename J2::CFG, typename J2::Epi>();
  constexpr int B01 = B0 > B1 ? B0 : B1;
  __shared__ __attribute__((aligned(1024))) char smem[B01 > B2 ? B01 : B2];
  int64_t b = blockIdx.x;
  if (b < j0.nb) {
    gemm2_block<typename J0::CFG, TR, J0::AK, J0::BKM>(j0.g, j0.e, b, j0.nb, j0.nreal,
                                                                     smem);
    return;
  }
  b -= j0.nb;
  if (b < j1.nb) {
    gemm2_block<typename J1::CFG, TR, J1::AK, J1::BKM>(j1.g, j1.e, b, j1.nb, j1.nreal,
                                                                     smem);
    return;
  }
  b -= j1.nb;
  gemm2_block<typename J2::CFG, TR, J2::AK, J2::BKM>(j2.g, j2.e, b, j2.nb, j2.nreal,
                                                                     smem);
}

// A packed launch (PackCounts): slot b = 8 s + x (slot s of XCD x) runs
// c[b][j] tiles of product j, taken in order from the XCD's contiguous range
// of that product's logical tiles, after the tiles of the same product that
// the XCD's earlier slots run.
// First logical tile of XCD x's range when n tiles are dealt to 8 XCDs in
// contiguous ranges (the larger ranges first).
__device__ inline int64_t xcd_range_lo(int64_t n, int x) {
  const int64_t q = n / 8, r = n % 8;
  return x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
}

// Three independent products, packed: each workgroup (one per compute unit)
// runs the list of tiles its slot holds, so that long and short tiles share
// compute units as a host-side bin packing decided instead of in dispatch
// order.  Every logical tile of every product is run exactly once when the
// counts of each XCD sum to that XCD's range; indices past a range are
// skipped.
template <class TR, class J0, class J1, class J2>
__global__ void __launch_bounds__(TR::NT) gemm2_packed_kernel(J0 j0, J1 j1, J2 j2,
                                                              PackCounts pc) {
  constexpr int B0 = gemm2_lds_bytes<typename J0::CFG, typename J0::Epi>();
  constexpr int B1 = gemm2_lds_bytes<typename J1::CFG, typename J1::Epi>();
  constexpr int B2 = gemm2_lds_bytes<typename J2::CFG, typename J2::Epi>();
  constexpr int B01 = B0 > B1 ? B0 : B1;
  __shared__ __attribute__((aligned(1024))) char smem[B01 > B2 ? B01 : B2];
  const int b = blockIdx.x, x = b % 8, s = b / 8;
  int off0 = 0, off1 = 0, off2 = 0;
  for (int t = 0; t < s; ++t) {
    off0 += pc.c[8 * t + x][0];
    off1 += pc.c[8 * t + x][1];
    off2 += pc.c[8 * t + x][2];
  }
  bool first = true;
  auto run = [&](const auto &job, int n_here, int off) {
    typedef typename std::remove_reference<decltype(job)>::type J;
    const int64_t n = job.nreal;
    const int64_t lo = xcd_range_lo(n, x), hi = xcd_range_lo(n, x + 1);
    for (int i = 0; i < n_here; ++i) {
      const int64_t LS = lo + off + i;
      if (LS >= hi) break;
      if (!first) __syncthreads();   // the previous tile's epilogue is done with the LDS
      first = false;
      gemm2_tile<typename J::CFG, TR, J::AK, J::BKM>(job.g, job.e, LS, smem);
    }
  };
  run(j0, pc.c[b][0], off0);
  run(j1, pc.c[b][1], off1);
  run(j2, pc.c[b][2], off2);
}

}  // namespace lce
