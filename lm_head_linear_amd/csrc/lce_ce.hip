// lce_ce.hip -- fused linear cross-entropy forward and backward on gfx950.
//
// Forward (lossk table, fused_linear_ce_flat, and "lossk: the loss is where
// the memory goes", on "Loss functions and resident-context kernels"):
//   one MFMA GEMM launch per token pass computes logit tiles Z^T = W H^T in
//   registers and reduces each (token, 128-row vocabulary block) at once to an
//   online (max, sum-of-exp) pair; no logit is stored.  The target logits
//   <H_t, W_{y_t}> come from one small dot-product kernel.
//   A merge kernel folds the pairs in a fixed order into lse_t, and one
//   fixed-tree reduction sums the counted tokens' losses and lse_t^2 in fp64.
// Backward (lossk table, fused_linear_ce_bwd_flat; the one-hot superposition
// and the z-loss coefficient of "Fuse distillation + z-loss in the triton
// monolithic path", section "What it does"):
//   the vocabulary is cut into slabs whose logit gradient for every token fits
//   the chunk*vocab cell budget.  Per slab: a GEMM recomputes the logits and
//   turns them into d = (g + 2 g_z lse) p - g [v == y] in its epilogue
//   (stored bf16 / fp64); a GEMM forms that slab's d_weight rows = d^T H in one
//   pass over all tokens (written once); a split-K GEMM adds d W_slab into
//   fp32 / fp64 d_hidden accumulators.  A last kernel folds the splits.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <type_traits>

#include "lce_gemm.hpp"
#include "lce_gemm2.hpp"
#include "lce_internal.h"

namespace lce {

// ---------------------------------------------------------- small kernels --

// keep_loss (a backward after a forward on this workspace): leave the
// forward's loss scalars for lce_loss_fetch and carry the guard verdicts met
// since that forward into seen_bad; otherwise (a forward) start afresh.
__global__ void ctl_init_kernel(Control *ctl, int keep_loss) {
  if (threadIdx.x == 0) {
    ctl->seen_bad = keep_loss ? (ctl->seen_bad | ctl->bad) : 0;
    ctl->bad = 0;
    ctl->first_bad = LLONG_MAX;
    ctl->count = 0;
    ctl->pad1 = 0;
    if (!keep_loss) {
      ctl->loss_sum = 0.0;
      ctl->z_sum = 0.0;
    }
  }
}

// Target-range guard (lossk table, loss_targets_in_range) and the count of
// counted tokens (y == nullptr: the count only).  Integer work only, so the
// atomics are order-free.
// Block `bid` of `nblk` (blockDim 256).
__device__ __forceinline__ void guard_block(const int64_t *y, const uint8_t *mask, int64_t n,
                                            int64_t V, Control *ctl, int64_t bid, int64_t nblk) {
  __shared__ unsigned long long s_first[4];
  __shared__ unsigned long long s_count[4];
  unsigned long long first = ULLONG_MAX, count = 0;
  for (int64_t t = bid * blockDim.x + threadIdx.x; t < n; t += nblk * blockDim.x) {
    const int64_t v = y ? y[t] : 0;
    if (v < 0 || v >= V) first = first < (unsigned long long)t ? first : (unsigned long long)t;
    count += mask ? (mask[t] != 0) : 1;
  }
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long f2 = __shfl_xor(first, o);
    first = f2 < first ? f2 : first;
    count += __shfl_xor(count, o);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) { s_first[wave] = first; s_count[wave] = count; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < int(blockDim.x >> 6); ++w) {
      first = s_first[w] < first ? s_first[w] : first;
      count += s_count[w];
    }
    if (count) atomicAdd(reinterpret_cast<unsigned long long *>(&ctl->count), count);
    if (first != ULLONG_MAX) {
      atomicMin(reinterpret_cast<unsigned long long *>(&ctl->first_bad), first);
      atomicExch(&ctl->bad, 1);
    }
  }
}

// The same check by one workgroup that also starts the control block afresh
// (what ctl_init_kernel does before a multi-workgroup guard): it writes the
// verdict and the count instead of accumulating them, so no separate clearing
// launch has to run first.
__device__ __forceinline__ void guard_init_block(const int64_t *y, const uint8_t *mask, int64_t n,
                                                 int64_t V, Control *ctl, int keep_loss) {
  __shared__ unsigned long long s_first[16];
  __shared__ unsigned long long s_count[16];
  unsigned long long first = ULLONG_MAX, count = 0;
  for (int64_t t = threadIdx.x; t < n; t += blockDim.x) {
    const int64_t v = y ? y[t] : 0;
    if (v < 0 || v >= V) first = first < (unsigned long long)t ? first : (unsigned long long)t;
    count += mask ? (mask[t] != 0) : 1;
  }
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long f2 = __shfl_xor(first, o);
    first = f2 < first ? f2 : first;
    count += __shfl_xor(count, o);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) { s_first[wave] = first; s_count[wave] = count; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < int(blockDim.x >> 6); ++w) {
      first = s_first[w] < first ? s_first[w] : first;
      count += s_count[w];
    }
    const int32_t old_bad = ctl->bad;   // the previous call's verdict
    ctl->seen_bad = keep_loss ? (ctl->seen_bad | old_bad) : 0;
    ctl->bad = first != ULLONG_MAX ? 1 : 0;
    ctl->first_bad = first != ULLONG_MAX ? int64_t(first) : LLONG_MAX;
    ctl->count = int64_t(count);
    ctl->pad1 = 0;
    if (!keep_loss) {
      ctl->loss_sum = 0.0;
      ctl->z_sum = 0.0;
    }
  }
}

__global__ void guard_kernel(const int64_t *y, const uint8_t *mask, int64_t n, int64_t V,
                             Control *ctl) {
  guard_block(y, mask, n, V, ctl, blockIdx.x, gridDim.x);
}

template <class T> __device__ inline T fexp(T x);
template <> __device__ inline float fexp<float>(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
template <> __device__ inline double fexp<double>(double x) { return exp(x); }
template <class T> __device__ inline T flog(T x);
template <> __device__ inline float flog<float>(float x) { return logf(x); }
template <> __device__ inline double flog<double>(double x) { return log(x); }

template <class T> __device__ inline T neg_inf();
template <> __device__ inline float neg_inf<float>() { return -INFINITY; }
template <> __device__ inline double neg_inf<double>() { return -INFINITY; }

// Reduce over the lanes that hold the same output column of an MFMA block.
// Keyed on the accumulator type, which fixes the MFMA layout: fp32 = the
// 32x32 bf16 block (a column's rows sit in lanes l and l ^ 32), fp64 = the
// 16x16 fp64 block (lanes l, l ^ 16, l ^ 32, l ^ 48).
template <class TR, class T> __device__ inline T col_max(T x) {
  if constexpr (std::is_same<T, float>::value) {
    return fmaxf(x, __shfl_xor(x, 32));
  } else {
    x = fmax(x, __shfl_xor(x, 16));
    return fmax(x, __shfl_xor(x, 32));
  }
}
template <class TR, class T> __device__ inline T col_sum(T x) {
  if constexpr (std::is_same<T, float>::value) {
    return x + __shfl_xor(x, 32);
  } else {
    x = x + __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
  }
}

template <class TR> __device__ inline typename TR::E to_elem(typename TR::Acc x) {
  if constexpr (std::is_same<typename TR::Acc, float>::value)
    return TR::F16 ? f32_to_f16_rne(x) : f32_to_bf16_rne(x);
  else return x;
}
template <class TR> __device__ inline typename TR::Acc to_acc(typename TR::E x) {
  if constexpr (std::is_same<typename TR::Acc, float>::value)
    return TR::F16 ? f16_to_f32(x) : bf16_to_f32(x);
  else return x;
}

// ------------------------------------------------------ forward epilogue --

// exp(x - m) with the shift folded into one FMA for fp32 (exp2 of a base-2
// exponent); plain exp for fp64.
template <class T> __device__ inline T shift_exp(T x, T m);
template <> __device__ inline float shift_exp<float>(float x, float m) {
  const float L2E = 1.4426950408889634f;
  return __builtin_amdgcn_exp2f(fmaf(x, L2E, -m * L2E));
}
template <> __device__ inline double shift_exp<double>(double x, double m) { return exp(x - m); }

// Z^T tile: rows = vocabulary ids, columns = tokens of the pass.  For every
// token column and every wave (WTM consecutive vocabulary rows) write
// (max, sum exp(z - max)).  (The target logits come from target_logit_block.)
template <class TR>
struct FwdLseEpi {
  typedef typename TR::Acc Acc;
  static constexpr bool kStaged = false;
  int64_t n_cols;          // tokens in the pass
  int64_t V;
  int64_t n_vparts;
  Acc *partials;           // [n_cols][n_vparts][2]

  // With CHECK only rows below `lim` (relative to the wave's first row)
  // count; row 0 always does, so every column max is finite.
  template <bool CHECK>
  __device__ __forceinline__ void body(const typename TR::AccBlock (&acc)[TR::FM][TR::FN],
                                       int64_t tcol, int64_t vpart, int lane, int lim) const {
#pragma unroll
    for (int fn = 0; fn < TR::FN; ++fn) {
      Acc x[TR::FM * TR::R];
#pragma unroll
      for (int fm = 0; fm < TR::FM; ++fm)
#pragma unroll
        for (int r = 0; r < TR::R; ++r)
          x[fm * TR::R + r] = (!CHECK || fm * TR::MF + TR::row_of(r, lane) < lim)
                                  ? acc[fm][fn][r] : neg_inf<Acc>();
      Acc mx = x[0];
#pragma unroll
      for (int i = 1; i < TR::FM * TR::R; ++i) mx = fmax(mx, x[i]);
      mx = col_max<TR, Acc>(mx);
      Acc sm = 0;
#pragma unroll
      for (int i = 0; i < TR::FM * TR::R; ++i) sm += shift_exp<Acc>(x[i], mx);
      sm = col_sum<TR, Acc>(sm);
      const int64_t t = tcol + fn * TR::MF;
      if (lane < TR::MF && t < n_cols) {
        Acc *p = partials + (t * n_vparts + vpart) * 2;
        p[0] = mx;
        p[1] = sm;
      }
    }
  }

  __device__ __forceinline__ void operator()(typename TR::AccBlock (&acc)[TR::FM][TR::FN], int64_t m0, int64_t n0,
                             int wm, int wn, int lane, int) const {
    const int64_t vrow0 = m0 + int64_t(wm) * TR::WTM;
    if (vrow0 >= V) return;  // wave-uniform
    const int64_t vpart = vrow0 / TR::WTM;
    const int lim = V - vrow0 < TR::WTM ? int(V - vrow0) : TR::WTM;
    const int64_t tcol = n0 + int64_t(wn) * TR::WTN + TR::col_of(lane);
    if (lim == TR::WTM) body<false>(acc, tcol, vpart, lane, lim);
    else body<true>(acc, tcol, vpart, lane, lim);
  }
};

// zy[t] = <H[t], W[y_t]> for every token: one wave per token, lane-strided
// partial sums in the accumulator type and a fixed shuffle tree.
// Block `bid` (blockDim 256, four tokens per block).  W holds head rows
// [offset, offset + rows); a target outside them (another vocabulary shard's
// row, or an id the guard refuses) gives 0.
template <class TR>
__device__ __forceinline__ void target_logit_block(const typename TR::E *H,
                                                   const typename TR::E *W, const int64_t *y,
                                                   int64_t offset, int64_t rows, int64_t n,
                                                   int64_t D, typename TR::Acc *zy, int vec8,
                                                   int64_t bid) {
  typedef typename TR::Acc Acc;
  const int lane = threadIdx.x & 63;
  const int64_t t = bid * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= n) return;
  const int64_t v = y[t] - offset;
  if (v < 0 || v >= rows) {
    if (lane == 0) zy[t] = 0;
    return;
  }
  const typename TR::E *h = H + t * D;
  const typename TR::E *w = W + v * D;
  Acc s = 0;
  if constexpr (std::is_same<typename TR::E, uint16_t>::value) {
    // 16-byte chunks of 8 elements (rows 16-byte aligned and D % 8 == 0: the
    // host passes vec8 only then), lane-strided, then the scalar remainder
    if (vec8) {
      for (int64_t c = lane; c < D / 8; c += 64) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(h + 8 * c);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(w + 8 * c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s = fmaf(to_acc<TR>(uint16_t(a[j])), to_acc<TR>(uint16_t(b[j])), s);
          s = fmaf(to_acc<TR>(uint16_t(a[j] >> 16)), to_acc<TR>(uint16_t(b[j] >> 16)), s);
        }
      }
    } else {
      for (int64_t d = lane; d < D; d += 64) s += to_acc<TR>(h[d]) * to_acc<TR>(w[d]);
    }
  } else {
    for (int64_t d = lane; d < D; d += 64) s += to_acc<TR>(h[d]) * to_acc<TR>(w[d]);
  }
  for (int o = 32; o > 0; o >>= 1) s += __shfl_down(s, o);
  if (lane == 0) zy[t] = s;
}

// One wave per token: fold the token's (max, sum) pairs in a fixed order.
// stats == nullptr: lse and the per-token loss; otherwise the vocabulary
// shard's exchange record {m, s, z_target} at stats[0/1/2][t] (row stride
// stride).
template <class Acc>
__global__ void fwd_merge_kernel(const Acc *partials, const Acc *zy, int64_t n_vparts,
                                 int64_t ntok, Acc *lse_out, double *loss_tok,
                                 const int32_t *bad, Acc *stats, int64_t stride) {
  if (*bad) return;
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const Acc *p = partials + t * n_vparts * 2;
  Acc m = neg_inf<Acc>();
  Acc s = 0;
  constexpr int CAP = sizeof(Acc) == 4 ? 32 : 16;   // partials per lane held in registers
  if (n_vparts <= 64 * CAP) {
    // every partial of the lane loaded at once (one memory latency), then
    // the same arithmetic in the same order as the loop below
    Acc pm[CAP], ps[CAP];
#pragma unroll
    for (int k = 0; k < CAP; ++k) {
      const int64_t i = lane + 64 * k;
      pm[k] = i < n_vparts ? p[2 * i] : neg_inf<Acc>();
      ps[k] = i < n_vparts ? p[2 * i + 1] : Acc(0);
    }
#pragma unroll
    for (int k = 0; k < CAP; ++k) m = pm[k] > m ? pm[k] : m;
    for (int o = 32; o > 0; o >>= 1) {
      Acc o2 = __shfl_xor(m, o);
      m = o2 > m ? o2 : m;
    }
#pragma unroll
    for (int k = 0; k < CAP; ++k)
      if (lane + 64 * k < n_vparts) s += ps[k] * fexp<Acc>(pm[k] - m);
  } else {
    for (int64_t i = lane; i < n_vparts; i += 64) m = p[2 * i] > m ? p[2 * i] : m;
    for (int o = 32; o > 0; o >>= 1) {
      Acc o2 = __shfl_xor(m, o);
      m = o2 > m ? o2 : m;
    }
    for (int64_t i = lane; i < n_vparts; i += 64) s += p[2 * i + 1] * fexp<Acc>(p[2 * i] - m);
  }
  // Fixed tree; lane 0 holds the result.
  for (int o = 32; o > 0; o >>= 1) s += __shfl_down(s, o);
  if (lane == 0) {
    if (stats) {
      stats[t] = m;
      stats[stride + t] = s;
      stats[2 * stride + t] = zy[t];
    } else {
      const Acc lse = m + flog<Acc>(s);
      lse_out[t] = lse;
      loss_tok[t] = double(lse) - double(zy[t]);
    }
  }
}

// Exchange of vocabulary shards: per token, fold the shards' {m, s, z}
// records (stats[p][0/1/2][t], shards in ascending order):
//   M = max m_p,  lse = M + log sum_p s_p exp(m_p - M),  z_y = sum_p z_p
// (z_p is 0 except in the shard that holds the target row).
template <class Acc>
__global__ void shard_merge_kernel(const Acc *stats, int64_t n_shards, int64_t n, Acc *lse_out,
                                   double *loss_tok) {
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < n;
       t += int64_t(gridDim.x) * blockDim.x) {
    Acc M = neg_inf<Acc>();
    for (int64_t q = 0; q < n_shards; ++q) {
      const Acc mq = stats[q * 3 * n + t];
      M = mq > M ? mq : M;
    }
    Acc S = 0, Z = 0;
    for (int64_t q = 0; q < n_shards; ++q) {
      const Acc *r = stats + q * 3 * n;
      S += r[n + t] * fexp<Acc>(r[t] - M);
      Z += r[2 * n + t];
    }
    const Acc lse = M + flog<Acc>(S);
    lse_out[t] = lse;
    loss_tok[t] = double(lse) - double(Z);
  }
}

// Sums over counted tokens in fp64 with a fixed thread-to-token map and a
// fixed reduction tree, so the result is independent of the chunk size.
template <class Acc>
__global__ void fwd_final_kernel(const double *loss_tok, const Acc *lse, const uint8_t *mask,
                                 int64_t n, Control *ctl) {
  if (ctl->bad) return;
  __shared__ double s_l[1024], s_z[1024];
  double ls = 0.0, zs = 0.0;
  for (int64_t t = threadIdx.x; t < n; t += blockDim.x) {
    if (mask && !mask[t]) continue;
    const double l = double(lse[t]);
    ls += loss_tok[t];
    zs += l * l;
  }
  s_l[threadIdx.x] = ls;
  s_z[threadIdx.x] = zs;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if (int(threadIdx.x) < w) {
      s_l[threadIdx.x] += s_l[threadIdx.x + w];
      s_z[threadIdx.x] += s_z[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    ctl->loss_sum = s_l[0];
    ctl->z_sum = s_z[0];
  }
}

// ----------------------------------------------------- backward epilogues --

// LDS-staged output of one wave's fp32-accumulated tile (16-bit core; the wave
// tile is TR::WTM x TR::WTN, 32x32 MFMA blocks).  Rows of the accumulator
// layout are spread over lanes in steps of four, so storing straight from
// registers costs one narrow access per value.  Instead each 32-row block goes
// to a private LDS region (value xf(fm, fn, r, row) at [row][col]) and comes
// back as 16-byte row chunks, which are stored (or added to memory) with one
// dwordx4 access each: consecutive lanes cover contiguous bytes of one output
// row.  Staged rows are unpadded; chunk c of row R sits at c ^ sw(R), which
// moves rows R+4..R+7 (written by lanes 32..63 together with rows R..R+3 by
// lanes 0..31) to the other half of the banks, so neither the writes nor the
// row-chunk reads conflict.
//   ptr(row, col): destination of the chunk at wave-tile (row, col), or
//                  nullptr to skip it (outside the output);
//   patch(fm, region): runs after block fm is written, before it is read
//                  back (may overwrite single staged values, staged_at()).
template <class T, class TR> struct Staging {
  static constexpr int ES = int(sizeof(T));
  static constexpr int PITCH = TR::WTN * ES;           // bytes per staged row
  static constexpr int CPR = PITCH / 16;                // 16-byte chunks per row
  static constexpr int SW = CPR / 2 < 8 ? CPR / 2 : 8;  // swizzle span
  static constexpr int BYTES = 32 * PITCH;              // one wave's region
  __device__ static inline int chunk_at(int row, int c) {
    return row * PITCH + ((c ^ (((row >> 2) & 1) * SW)) << 4);
  }
  // byte offset of value (row, col) of a staged block
  __device__ static inline int at(int row, int col) {
    return chunk_at(row, (col * ES) >> 4) + ((col * ES) & 15);
  }
};

template <class T, class TR, bool ACCUM, bool NT = true, class Xf, class Ptr, class Patch>
__device__ __forceinline__ void staged_tile(const typename TR::AccBlock (&acc)[TR::FM][TR::FN],
                                            char *region, int lane, const Xf &xf, const Ptr &ptr,
                                            const Patch &patch) {
  typedef Staging<T, TR> S;
  constexpr int NR = 32 * S::CPR / 64;            // chunk reads per lane per block
  constexpr int EPC = 16 / S::ES;                 // values per chunk
  static_assert(!ACCUM || S::ES == 4, "accumulation is fp32");
  static_assert(NR >= 1, "staged block");
#pragma unroll
  for (int fm = 0; fm < TR::FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < TR::FN; ++fn)
#pragma unroll
      for (int r = 0; r < TR::R; ++r) {
        const int row = TR::row_of(r, lane);
        const int col = fn * TR::MF + TR::col_of(lane);
        *reinterpret_cast<T *>(region + S::at(row, col)) = xf(fm, fn, r, fm * TR::MF + row);
      }
    patch(fm, region);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    u32x4 d[NR];
    T *dst[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int q = i * 64 + lane;
      const int row = q / S::CPR, c = q % S::CPR;
      d[i] = *reinterpret_cast<const u32x4 *>(region + S::chunk_at(row, c));
      dst[i] = ptr(fm * TR::MF + row, c * EPC);
    }
    if constexpr (ACCUM) {
      u32x4 old[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i)
        old[i] = dst[i] ? *reinterpret_cast<const u32x4 *>(dst[i]) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if (!dst[i]) continue;
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = __float_as_uint(__uint_as_float(old[i][j]) + __uint_as_float(d[i][j]));
        *reinterpret_cast<u32x4 *>(dst[i]) = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NR; ++i)
        if (dst[i]) {
          // fp32 results written once (d_weight rows, kept logits, split
          // partials) stream past the caches: keeping them there evicts the
          // operands the next tiles read (the 512-token heads run 4-7% faster)
          if constexpr (S::ES == 4 && NT)
            __builtin_nontemporal_store(d[i], reinterpret_cast<u32x4 *>(dst[i]));
          else *reinterpret_cast<u32x4 *>(dst[i]) = d[i];
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);   // one block's registers at a time
  }
}

// Recomputed Z^T tile of a vocabulary slab -> logit gradient, stored
// [slab row][token] in the input dtype.
template <class TR>
struct DlogitEpi {
  typedef typename TR::Acc Acc;
  const int64_t *targets;
  const uint8_t *mask;
  const Acc *lse;
  int64_t n;
  int64_t vs0;     // first vocabulary row of the slab
  int64_t rows;    // rows in the slab
  const Control *ctl;
  double grad_out, z_coef;
  typename TR::E *dbuf;
  int64_t d_ld;
  const Acc *zy;   // target logits (staged path)

  template <bool CHECK>
  __device__ __forceinline__ void body(const typename TR::AccBlock (&acc)[TR::FM][TR::FN],
                                       int64_t vw0, int64_t tw0, int lane, Acc g, Acc gz) const {
#pragma unroll
    for (int fn = 0; fn < TR::FN; ++fn) {
      const int64_t t = tw0 + fn * TR::MF + TR::col_of(lane);
      if (CHECK && t >= d_ld) continue;
      if (CHECK && t >= n) {  // K padding of the d_weight product
#pragma unroll
        for (int fm = 0; fm < TR::FM; ++fm)
#pragma unroll
          for (int r = 0; r < TR::R; ++r) {
            const int vr = fm * TR::MF + TR::row_of(r, lane);
            if (vw0 + vr < rows) dbuf[(vw0 + vr) * d_ld + t] = to_elem<TR>(Acc(0));
          }
        continue;
      }
      const Acc l = lse[t];
      const bool counted = !mask || mask[t];
      const Acc coef = counted ? g + Acc(2) * gz * l : Acc(0);
      const Acc gy = counted ? g : Acc(0);
      const int64_t yr = targets[t] - (vs0 + vw0);
      const int yl = (yr >= 0 && yr < TR::WTM) ? int(yr) : -1;
      typename TR::E *col = dbuf + t;
#pragma unroll
      for (int fm = 0; fm < TR::FM; ++fm)
#pragma unroll
        for (int r = 0; r < TR::R; ++r) {
          const int vr = fm * TR::MF + TR::row_of(r, lane);
          if (CHECK && vw0 + vr >= rows) continue;
          Acc d = coef * shift_exp<Acc>(acc[fm][fn][r], l);
          d -= (vr == yl) ? gy : Acc(0);
          col[(vw0 + vr) * d_ld] = to_elem<TR>(d);
        }
    }
  }

  __device__ __forceinline__ void operator()(typename TR::AccBlock (&acc)[TR::FM][TR::FN], int64_t m0, int64_t n0,
                             int wm, int wn, int lane, int) const {
    const int64_t C = ctl->count;
    const Acc g = C ? Acc(grad_out / double(C)) : Acc(0);
    const Acc gz = C ? Acc(z_coef * grad_out / double(C)) : Acc(0);
    const int64_t vw0 = m0 + int64_t(wm) * TR::WTM;
    const int64_t tw0 = n0 + int64_t(wn) * TR::WTN;
    if (vw0 >= rows || tw0 >= n) return;
    if (vw0 + TR::WTM <= rows && tw0 + TR::WTN <= n) body<false>(acc, vw0, tw0, lane, g, gz);
    else body<true>(acc, vw0, tw0, lane, g, gz);
  }

  // 16-bit core: the same values through LDS.  Token columns in [n, d_ld) get
  // zeros (they are the K padding of the d_weight GEMM).
  //   d = coef * exp(z - lse) - g [v == y] = s exp2(z log2(e) + c2) - g [v == y]
  // with c2 = log2|coef| - lse log2(e) and s the sign of coef (coef 0 gives
  // exp2(-inf) = 0; a negative coef needs grad_out < 0 or lse < -1/(2 z)).
  // The target element comes from the separately computed target logit.
  // Per-token inputs are loaded before the main loop; after it, per-token
  // constants {c2, sign bit, target row - tile row, d at the target} go
  // through LDS to the lanes that hold each column.
  static constexpr bool kStaged = true;
  static constexpr int kPrefetchBytes = 256 * 16;
  struct Pre {
    float l, z;
    int32_t y;    // targets < 2^24
    uint32_t mk;  // mask byte (any value when there is no mask)
  };
  __device__ __forceinline__ Pre pre_load(int64_t, int64_t n0, int tid) const {
    // unconditional loads (index clamped; pre_store ignores columns >= n) so
    // that nothing waits on them before the operand loads issue
    const int64_t t = n0 + tid < n ? n0 + tid : n - 1;
    // without a mask any readable byte will do (pre_store ignores it)
    const uint8_t *mp = mask ? mask : reinterpret_cast<const uint8_t *>(lse);
    Pre q;
    q.l = lse[t];
    q.z = zy[t];
    q.y = int32_t(targets[t]);
    q.mk = mp[t];
    return q;
  }
  __device__ __forceinline__ void pre_store(const Pre &q, int64_t m0, int64_t n0, int tid,
                                            char *pre) const {
    const float L2E = 1.4426950408889634f;
    const int64_t C = ctl->count;
    const float g = C ? float(grad_out / double(C)) : 0.f;
    const float gz = C ? float(z_coef * grad_out / double(C)) : 0.f;
    const bool live = n0 + tid < n;
    const bool counted = live && (!mask || q.mk != 0);
    const float coef = counted ? g + 2.f * gz * q.l : 0.f;
    const float c2 = __builtin_amdgcn_logf(fabsf(coef)) - q.l * L2E;
    const uint32_t sb = __float_as_uint(coef) & 0x80000000u;
    const int64_t yr = live ? int64_t(q.y) - (vs0 + m0) : -1;
    const float ey = __uint_as_float(__float_as_uint(__builtin_amdgcn_exp2f(fmaf(q.z, L2E, c2))) ^ sb);
    u32x4 v;
    v[0] = __float_as_uint(c2);
    v[1] = sb;
    v[2] = uint32_t(int32_t(yr >= 0 && yr < 256 ? yr : -1));
    v[3] = __float_as_uint(ey - (counted ? g : 0.f));
    *reinterpret_cast<u32x4 *>(pre + tid * 16) = v;
  }
  __device__ __forceinline__ void staged(typename TR::AccBlock (&acc)[TR::FM][TR::FN], int64_t m0,
                                         int64_t n0, int wm, int wn, int lane, int,
                                         char *lds, const char *pre) const {
    static_assert(std::is_same<typename TR::Acc, float>::value, "staged epilogue is bf16");
    const float L2E = 1.4426950408889634f;
    const int64_t vw0 = m0 + int64_t(wm) * TR::WTM;
    const int64_t tw0 = n0 + int64_t(wn) * TR::WTN;
    if (vw0 >= rows || tw0 >= d_ld) return;  // wave-uniform
    float c2[TR::FN], gy[TR::FN];
    uint32_t sb[TR::FN];
    int yl[TR::FN];
#pragma unroll
    for (int fn = 0; fn < TR::FN; ++fn) {
      const u32x4 q = *reinterpret_cast<const u32x4 *>(
          pre + (wn * TR::WTN + fn * TR::MF + TR::col_of(lane)) * 16);
      c2[fn] = __uint_as_float(q[0]);
      sb[fn] = q[1];
      const int yr = int(q[2]) - wm * TR::WTM;   // row within this wave's 128
      yl[fn] = (int(q[2]) >= 0 && yr >= 0 && yr < TR::WTM && vw0 + yr < rows) ? yr : -1;
      gy[fn] = __uint_as_float(q[3]);
    }
    typedef Staging<uint16_t, TR> S;
    char *region = lds + (wm * TR::WAVES_N + wn) * S::BYTES;
    auto store = [&](auto neg_tag) {
      // NEG: some column of this wave has a negative coefficient (its sign
      // goes onto every value by XOR); otherwise every value is positive
      constexpr bool NEG = decltype(neg_tag)::value;
      staged_tile<uint16_t, TR, false>(
          acc, region, lane,
          [&](int fm, int fn, int r, int) -> uint16_t {
            const float e = __builtin_amdgcn_exp2f(fmaf(acc[fm][fn][r], L2E, c2[fn]));
            if constexpr (NEG) return to_elem<TR>(__uint_as_float(__float_as_uint(e) ^ sb[fn]));
            else return to_elem<TR>(e);
          },
          [&](int vr, int tc) -> uint16_t * {
            const int64_t v = vw0 + vr, t = tw0 + tc;
            return (v < rows && t < d_ld) ? dbuf + v * d_ld + t : nullptr;
          },
          [&](int fm, char *blk) {
            // overwrite the target element of each column that has it here
#pragma unroll
            for (int fn = 0; fn < TR::FN; ++fn)
              if (lane < TR::MF && yl[fn] >= fm * TR::MF && yl[fn] < fm * TR::MF + TR::MF)
                *reinterpret_cast<uint16_t *>(blk + S::at(yl[fn] - fm * TR::MF, fn * TR::MF + lane)) =
                    to_elem<TR>(gy[fn]);
          });
    };
    uint32_t any_sb = 0;
#pragma unroll
    for (int fn = 0; fn < TR::FN; ++fn) any_sb |= sb[fn];
    if (__builtin_amdgcn_ballot_w64(any_sb != 0) != 0)   // wave-uniform
      store(std::true_type{});
    else
      store(std::false_type{});
  }
};

// out[split][row_off + row][col] = C (ACCUM false) or += C (ACCUM true).
// NT: stored values stream past the caches (written once, read much later);
// otherwise they stay cached for a reader that follows soon.
template <class TR, bool ACCUM, bool NT = true>
struct StoreEpi {
  typedef typename TR::Acc Acc;
  Acc *out;
  int64_t ldo;
  int64_t row_off;
  int64_t rows, cols;
  int64_t split_stride;

  template <bool CHECK>
  __device__ __forceinline__ void body(const typename TR::AccBlock (&acc)[TR::FM][TR::FN], Acc *o,
                                       int64_t rw0, int64_t cw0, int lane) const {
#pragma unroll
    for (int fn = 0; fn < TR::FN; ++fn) {
      const int64_t c = cw0 + fn * TR::MF + TR::col_of(lane);
      if (CHECK && c >= cols) continue;
      Acc *colp = o + c;
#pragma unroll
      for (int fm = 0; fm < TR::FM; ++fm) {
#pragma unroll
        for (int r = 0; r < TR::R; ++r) {
          const int64_t row = rw0 + fm * TR::MF + TR::row_of(r, lane);
          if (CHECK && row >= rows) continue;
          Acc *q = colp + (row_off + row) * ldo;
          if (ACCUM) *q += acc[fm][fn][r];
          else *q = acc[fm][fn][r];
        }
        // keep the read-modify-write of one block in flight at a time
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  __device__ __forceinline__ void operator()(typename TR::AccBlock (&acc)[TR::FM][TR::FN], int64_t m0, int64_t n0,
                             int wm, int wn, int lane, int split) const {
    Acc *o = out + int64_t(split) * split_stride;
    const int64_t rw0 = m0 + int64_t(wm) * TR::WTM;
    const int64_t cw0 = n0 + int64_t(wn) * TR::WTN;
    if (rw0 >= rows || cw0 >= cols) return;
    if (rw0 + TR::WTM <= rows && cw0 + TR::WTN <= cols) body<false>(acc, o, rw0, cw0, lane);
    else body<true>(acc, o, rw0, cw0, lane);
  }

  // 16-bit core: through LDS, 16-byte accesses (cols and ldo multiples of 4,
  // `out` 16-byte aligned; the host checks).
  static constexpr bool kStaged = true;
  __device__ __forceinline__ void staged(typename TR::AccBlock (&acc)[TR::FM][TR::FN], int64_t m0,
                                         int64_t n0, int wm, int wn, int lane, int split,
                                         char *lds, const char *) const {
    static_assert(std::is_same<typename TR::Acc, float>::value, "staged epilogue is bf16");
    Acc *o = out + int64_t(split) * split_stride;
    const int64_t rw0 = m0 + int64_t(wm) * TR::WTM;
    const int64_t cw0 = n0 + int64_t(wn) * TR::WTN;
    if (rw0 >= rows || cw0 >= cols) return;  // wave-uniform
    char *region = lds + (wm * TR::WAVES_N + wn) * Staging<float, TR>::BYTES;
    staged_tile<float, TR, ACCUM, NT>(
        acc, region, lane, [&](int fm, int fn, int r, int) -> float { return acc[fm][fn][r]; },
        [&](int rr, int cc) -> float * {
          const int64_t row = rw0 + rr, c = cw0 + cc;
          return (row < rows && c < cols) ? o + (row_off + row) * ldo + c : nullptr;
        },
        [](int, char *) {});
  }
};

// Ht[d][t] = H[t][d] for t < n, 0 for n <= t < ld (16-bit values).  64x64
// tiles through LDS; blockDim 256; block (bt, bd) of the tile grid.
template <class E>
__device__ __forceinline__ void transpose_h_block(const E *H, int64_t n, int64_t D, E *Ht,
                                                  int64_t ld, int64_t bt, int64_t bd) {
  __shared__ E tile[64][66];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t t0 = bt * 64, d0 = bd * 64;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int64_t t = t0 + ty + 4 * j, d = d0 + tx;
    tile[ty + 4 * j][tx] = (t < n && d < D) ? H[t * D + d] : E(0);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int64_t d = d0 + ty + 4 * j, t = t0 + tx;
    if (d < D && t < ld) Ht[d * ld + t] = tile[tx][ty + 4 * j];
  }
}


// Forward of the single-call path: the online-LSE partials (FwdLseEpi) and
// the fp32 tile itself, kept at Z[v][t] (StoreEpi, row stride `ldo`).
template <class TR>
struct FwdKeepEpi {
  FwdLseEpi<TR> lse;
  StoreEpi<TR, false> keep;
  static constexpr bool kStaged = true;
  __device__ __forceinline__ void staged(typename TR::AccBlock (&acc)[TR::FM][TR::FN], int64_t m0,
                                         int64_t n0, int wm, int wn, int lane, int,
                                         char *lds, const char *pre) const {
    lse(acc, m0, n0, wm, wn, lane, 0);
    keep.staged(acc, m0, n0, wm, wn, lane, 0, lds, pre);
  }
};

// Single-call path: row v of the kept logits Z (fp32, row stride ld) becomes
// row v of the logit gradient, written over the same bytes as 16-bit values
// with row stride 2 * ld.  Each value is formed as DlogitEpi forms it
// (d = s * exp2(z log2(e) + c2), the target element from the target logit),
// so the gradient equals the recomputing backward's; token columns
// [n, round_up(n, 64)) get zeros (the d_weight product's K padding).  A wave
// takes kDlogitRows consecutive rows and walks the tokens in ascending
// segments of 64 * K: it forms the segment's per-token constants once, reads
// the segment of every row, and only then writes them (the 16-bit values of
// tokens [t0, t1) land on the fp32 bytes of tokens [t0 / 2, t1 / 2), all read
// by then).
constexpr int kDlogitRows = 4;
// Workgroups of dlogit_rows4_kernel (4 waves each): about six waves per SIMD.
constexpr int64_t kDlogit4Blocks = 1536;
template <class TR>
__global__ void dlogit_rows_kernel(float *Z, int64_t V, int64_t n, int64_t ld,
                                   const int64_t *y, const uint8_t *mask, const float *lse,
                                   const float *zy, const Control *ctl, double grad_out,
                                   double z_coef) {
  if (ctl->bad) return;
  constexpr int K = 8;
  const float L2E = 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const int64_t v0 = (int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6)) * kDlogitRows;
  if (v0 >= V) return;
  const int64_t C = ctl->count;
  const float g = C ? float(grad_out / double(C)) : 0.f;
  const float gz = C ? float(z_coef * grad_out / double(C)) : 0.f;
  const int64_t tpad = (n + 63) / 64 * 64;
  for (int64_t t0 = 0; t0 < tpad; t0 += 64 * K) {
    float c2[K], gy[K];
    uint32_t sb[K];
    int64_t yt[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t t = t0 + 64 * k + lane;
      c2[k] = -INFINITY;   // tokens >= n: exp2(-inf) = 0
      sb[k] = 0;
      gy[k] = 0.f;
      yt[k] = -1;
      if (t < n) {
        const float l = lse[t];
        const bool counted = !mask || mask[t] != 0;
        const float coef = counted ? g + 2.f * gz * l : 0.f;
        c2[k] = __builtin_amdgcn_logf(fabsf(coef)) - l * L2E;
        sb[k] = __float_as_uint(coef) & 0x80000000u;
        yt[k] = y[t];
        const float ey = __uint_as_float(
            __float_as_uint(__builtin_amdgcn_exp2f(fmaf(zy[t], L2E, c2[k]))) ^ sb[k]);
        gy[k] = ey - (counted ? g : 0.f);
      }
    }
    // every row's segment in flight at once, then written
    float z[kDlogitRows][K];
#pragma unroll
    for (int r = 0; r < kDlogitRows; ++r) {
      const float *zr = Z + (v0 + r) * ld;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t t = t0 + 64 * k + lane;
        z[r][k] = (t < n && v0 + r < V) ? zr[t] : 0.f;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the segment of every row is read
#pragma unroll
    for (int r = 0; r < kDlogitRows; ++r) {
      const int64_t v = v0 + r;
      if (v >= V) break;
      typename TR::E *dr = reinterpret_cast<typename TR::E *>(Z) + v * 2 * ld;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t t = t0 + 64 * k + lane;
        if (t >= tpad) continue;
        const float e = __uint_as_float(
            __float_as_uint(__builtin_amdgcn_exp2f(fmaf(z[r][k], L2E, c2[k]))) ^ sb[k]);
        dr[t] = to_elem<TR>(yt[k] == v ? gy[k] : e);
      }
    }
  }
}

// The same values for a token count that is a multiple of 4 (16-byte rows):
// each lane forms four consecutive tokens per 16-byte load, so a wave's
// access to a row is one 1 KB load and one 512-byte store per 256 tokens.
// A segment is 512 tokens (two loads per lane and row).  Each wave takes
// groups of kDlogitRows rows in a grid stride and forms a segment's
// per-token constants once for all its groups; a group's segment is read for
// every row before any is written, in ascending order as above.
template <class TR>
__global__ void dlogit_rows4_kernel(float *Z, int64_t V, int64_t n, int64_t ld,
                                    const int64_t *y, const uint8_t *mask, const float *lse,
                                    const float *zy, const Control *ctl, double grad_out,
                                    double z_coef) {
  if (ctl->bad) return;
  const float L2E = 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const int64_t wave = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t n_waves = int64_t(gridDim.x) * (blockDim.x >> 6);
  const int64_t groups = (V + kDlogitRows - 1) / kDlogitRows;
  if (wave >= groups) return;
  const int64_t C = ctl->count;
  const float g = C ? float(grad_out / double(C)) : 0.f;
  const float gz = C ? float(z_coef * grad_out / double(C)) : 0.f;
  const int64_t tpad = (n + 63) / 64 * 64;
  typedef typename TR::E E;
  for (int64_t t0 = 0; t0 < tpad; t0 += 512) {
    float c2[2][4], gy[2][4];
    uint32_t sb[2][4];
    int32_t yt[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t tb = t0 + 256 * k + 4 * lane;
      // n % 4 == 0: the four tokens of a lane are all below n or all past it
      if (tb < n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t t = tb + e;
          const float l = lse[t];
          const bool counted = !mask || mask[t] != 0;
          const float coef = counted ? g + 2.f * gz * l : 0.f;
          c2[k][e] = __builtin_amdgcn_logf(fabsf(coef)) - l * L2E;
          sb[k][e] = __float_as_uint(coef) & 0x80000000u;
          yt[k][e] = int32_t(y[t]);
          const float ey = __uint_as_float(
              __float_as_uint(__builtin_amdgcn_exp2f(fmaf(zy[t], L2E, c2[k][e]))) ^ sb[k][e]);
          gy[k][e] = ey - (counted ? g : 0.f);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c2[k][e] = -INFINITY;   // tokens >= n: exp2(-inf) = 0
          sb[k][e] = 0;
          gy[k][e] = 0.f;
          yt[k][e] = -1;
        }
      }
    }
    for (int64_t grp = wave; grp < groups; grp += n_waves) {
      const int64_t v0 = grp * kDlogitRows;
      float4 z[kDlogitRows][2];
#pragma unroll
      for (int r = 0; r < kDlogitRows; ++r)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int64_t t = t0 + 256 * k + 4 * lane;
          z[r][k] = (t < n && v0 + r < V) ? *reinterpret_cast<const float4 *>(Z + (v0 + r) * ld + t)
                                          : float4{0.f, 0.f, 0.f, 0.f};
        }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the segment of every row is read
#pragma unroll
      for (int r = 0; r < kDlogitRows; ++r) {
        const int64_t v = v0 + r;
        if (v >= V) break;
        E *dr = reinterpret_cast<E *>(Z) + v * 2 * ld;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int64_t t = t0 + 256 * k + 4 * lane;
          if (t >= tpad) continue;
          const float zz[4] = {z[r][k].x, z[r][k].y, z[r][k].z, z[r][k].w};
          E o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float d = __uint_as_float(
                __float_as_uint(__builtin_amdgcn_exp2f(fmaf(zz[e], L2E, c2[k][e]))) ^ sb[k][e]);
            o[e] = to_elem<TR>(yt[k][e] == int32_t(v) ? gy[k][e] : d);
          }
          uint2 w;
          w.x = uint32_t(o[0]) | (uint32_t(o[1]) << 16);
          w.y = uint32_t(o[2]) | (uint32_t(o[3]) << 16);
          *reinterpret_cast<uint2 *>(dr + t) = w;
        }
      }
    }
  }
}

// Per-call preparation in one launch.  Its parts do not read each other's
// results, so they share a grid: blocks [0, nb_guard) run the target guard
// and token count (one block that also starts the control block, or several
// after ctl_init), then nb_local blocks the shard-local target ids, nb_zy
// blocks the target logits and nb_tr blocks H^T (the d_weight product's
// K-major operand).  A part with no blocks is absent.  blockDim 256.
template <class TR>
struct Prep {
  const int64_t *y;
  const uint8_t *mask;
  int64_t n, v_check;       // guard: ids must lie in [0, v_check)
  Control *ctl;
  int64_t offset, rows;     // W holds head rows [offset, offset + rows)
  int64_t *yl;              // shard-local ids (shard calls): y - offset, or -1
                            // when another shard holds the target row
  const typename TR::E *H, *W;
  int64_t D;
  typename TR::Acc *zy;
  int vec8;
  typename TR::E *Ht;       // [D][ld] (16-bit inputs)
  int64_t ld, tr_cols;      // tr_cols = ceil(ld / 64) tile columns
  int64_t nb_guard, nb_local, nb_zy, nb_tr;
  int guard_init;           // one guard workgroup that also starts the control block
  int keep_loss;            // (as ctl_init_kernel's argument)
  int64_t blocks() const { return nb_guard + nb_local + nb_zy + nb_tr; }
};

template <class TR>
__global__ void prep_kernel(Prep<TR> a) {
  int64_t b = blockIdx.x;
  if (b < a.nb_guard) {
    if (a.guard_init) guard_init_block(a.y, a.mask, a.n, a.v_check, a.ctl, a.keep_loss);
    else guard_block(a.y, a.mask, a.n, a.v_check, a.ctl, b, a.nb_guard);
    return;
  }
  b -= a.nb_guard;
  if (b < a.nb_local) {
    for (int64_t t = b * blockDim.x + threadIdx.x; t < a.n; t += a.nb_local * blockDim.x) {
      const int64_t v = a.y[t] - a.offset;
      a.yl[t] = (v >= 0 && v < a.rows) ? v : -1;
    }
    return;
  }
  b -= a.nb_local;
  if (b < a.nb_zy) {
    target_logit_block<TR>(a.H, a.W, a.y, a.offset, a.rows, a.n, a.D, a.zy, a.vec8, b);
    return;
  }
  b -= a.nb_zy;
  transpose_h_block(a.H, a.n, a.D, a.Ht, a.ld, b % a.tr_cols, b / a.tr_cols);
}

// d_hidden = sum over splits (ascending) of the split accumulators, in the
// input dtype (OUT = TR::E) or unrounded (OUT = TR::Acc, a vocabulary shard's
// partial).
template <class TR, class OUT>
__global__ void dh_final_kernel(const typename TR::Acc *P, int64_t splits, int64_t count,
                                OUT *out, const int32_t *bad, int vec4) {
  if (*bad) return;
  int64_t begin = 0;
  if constexpr (std::is_same<typename TR::Acc, float>::value &&
                std::is_same<OUT, typename TR::E>::value) {
    // four consecutive elements per thread: 16-byte loads, one 8-byte store
    // (count % 4 == 0 and out 8-byte aligned: the host passes vec4 only then)
    if (vec4) {
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count / 4;
           i += int64_t(gridDim.x) * blockDim.x) {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int64_t j = 0; j < splits; ++j)
          s += *reinterpret_cast<const f32x4_t *>(P + j * count + 4 * i);
        uint2 o;
        o.x = uint32_t(to_elem<TR>(s[0])) | (uint32_t(to_elem<TR>(s[1])) << 16);
        o.y = uint32_t(to_elem<TR>(s[2])) | (uint32_t(to_elem<TR>(s[3])) << 16);
        *reinterpret_cast<uint2 *>(out + 4 * i) = o;
      }
      begin = count / 4 * 4;
    }
  }
  for (int64_t i = begin + int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
       i += int64_t(gridDim.x) * blockDim.x) {
    typename TR::Acc s = 0;
    for (int64_t j = 0; j < splits; ++j) s += P[j * count + i];
    if constexpr (std::is_same<OUT, typename TR::Acc>::value) out[i] = s;
    else out[i] = to_elem<TR>(s);
  }
}

// ------------------------------------------------------------- host side --

TimedLaunch::TimedLaunch(lce_timers *t, int kind, void *st) : slot(nullptr), stream(st), idx(-1) {
  if (t && t->slot[kind].capacity > t->slot[kind].used) {
    slot = &t->slot[kind];
    idx = slot->used;
    (void)hipEventRecord(static_cast<hipEvent_t>(slot->start[idx]), static_cast<hipStream_t>(st));
  }
}
TimedLaunch::~TimedLaunch() {
  if (slot) {
    (void)hipEventRecord(static_cast<hipEvent_t>(slot->stop[idx]), static_cast<hipStream_t>(stream));
    slot->used = idx + 1;
  }
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static int64_t round_up8(int64_t x) { return (x + 7) / 8 * 8; }
// the d_hidden fold may use 4-element chunks
static int fold_vec4(int64_t count, const void *out) {
  return count % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & 7u) == 0;
}

static uint8_t *ws_base(const lce_tensor *ws) {
  uintptr_t p = reinterpret_cast<uintptr_t>(ws->data);
  return reinterpret_cast<uint8_t *>((p + 255) & ~uintptr_t(255));
}

template <class TR, bool AK, bool BKM, class Epi>
static void launch_gemm(bool vec, const GemmParams &g, int64_t splits, const Epi &epi,
                        hipStream_t st) {
  const int64_t tiles = cdiv(g.M, TR::BM) * g.tiles_n;
  const dim3 grid{unsigned(tiles), unsigned(splits), 1u};
  if (vec)
    hipLaunchKernelGGL((gemm_kernel<TR, AK, BKM, true, Epi>), grid, dim3(TR::NT), 0, st, g, epi);
  else
    hipLaunchKernelGGL((gemm_kernel<TR, AK, BKM, false, Epi>), grid, dim3(TR::NT), 0, st, g, epi);
}

// Pipelined-core stage configurations.  With 8 waves per tile two stages of
// k 64 measured faster than four of k 32 for both operand kinds (K-major rows
// become whole 128-byte lines; half the barriers per k).
typedef PipeCfg<64, 2> PipeKK;
typedef PipeCfg<64, 2> PipeMN;

// The pipelined core runs 8 waves per tile (TraitsH16W8); its epilogues are
// the same structs instantiated on those traits (same members, so the fields
// carry over bit for bit).
template <class TR2, class TR> FwdLseEpi<TR2> retrait(const FwdLseEpi<TR> &e) {
  return __builtin_bit_cast(FwdLseEpi<TR2>, e);
}
template <class TR2, class TR> DlogitEpi<TR2> retrait(const DlogitEpi<TR> &e) {
  return __builtin_bit_cast(DlogitEpi<TR2>, e);
}
template <class TR2, class TR, bool A> StoreEpi<TR2, A> retrait(const StoreEpi<TR, A> &e) {
  return __builtin_bit_cast(StoreEpi<TR2, A>, e);
}

template <class CFG> static Gemm2Params to_gemm2(const GemmParams &g0) {
  Gemm2Params g;
  g.A = g0.A; g.lda = g0.lda; g.B = g0.B; g.ldb = g0.ldb;
  g.M = g0.M; g.N = g0.N; g.K = g0.K; g.M_read = g0.M_read; g.N_read = g0.N_read;
  g.k_per_split = (g0.k_per_split + CFG::BK - 1) / CFG::BK * CFG::BK;
  g.tiles_n = g0.tiles_n; g.bad = g0.bad;
  return g;
}

template <class CFG, class TR, bool AK, bool BKM, class Epi>
static void launch_gemm2(const GemmParams &g0, int64_t splits, const Epi &epi, hipStream_t st) {
  const Gemm2Params g = to_gemm2<CFG>(g0);
  const int64_t tiles = cdiv(g.M, CFG::BM) * g.tiles_n;
  const dim3 grid{unsigned(tiles * splits), 1u, 1u};
  typedef typename W8Of<TR>::type TRP;
  const auto e = retrait<TRP>(epi);
  hipLaunchKernelGGL((gemm2_kernel<CFG, TRP, AK, BKM, decltype(e)>), grid, dim3(TRP::NT), 0, st, g,
                     e);
}

// The pipelined 16-bit core applies when every operand is 16-byte aligned with
// leading dimensions that are multiples of 8, d_model is a multiple of the
// K-major configuration's k-step (K-major operands are read in whole steps)
// and 256 rows of any operand span less than 2 GiB (buffer offsets are 32-bit).
template <class TR> struct UsePipe { static bool ok(bool, int64_t, int64_t) { return false; } };
template <bool F> struct UsePipe<TraitsH16<F>> {
  static bool ok(bool vec, int64_t D, int64_t d_ld) {
    return vec && D % PipeKK::BK == 0 && 256 * D * 2 < (int64_t(1) << 31) &&
           256 * d_ld * 2 < (int64_t(1) << 31);
  }
};

// 16-bit inputs with `pipe`: the pipelined core (both operands K-major:
// PipeKK, else PipeMN); otherwise the generic one.
template <class TR, bool AK, bool BKM, class Epi>
static void launch_any(bool pipe, bool vec, const GemmParams &g, int64_t splits, const Epi &epi,
                       hipStream_t st) {
  if constexpr (IsH16<TR>::value) {
    if (pipe) {
      if constexpr (AK && BKM) launch_gemm2<PipeKK, TR, AK, BKM>(g, splits, epi, st);
      else launch_gemm2<PipeMN, TR, AK, BKM>(g, splits, epi, st);
      return;
    }
  }
  launch_gemm<TR, AK, BKM>(vec, g, splits, epi, st);
}

static void launch_guard(const int64_t *y, const uint8_t *mask, int64_t n, int64_t V,
                         Control *ctl, hipStream_t st, lce_timers *tm, int keep_loss) {
  TimedLaunch tl(tm, LCE_K_GUARD, st);
  hipLaunchKernelGGL(ctl_init_kernel, dim3(1), dim3(64), 0, st, ctl, keep_loss);
  int64_t blocks = cdiv(n, 256);
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(guard_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, y, mask, n, V, ctl);
}

void launch_target_guard(const int64_t *targets, const uint8_t *mask, int64_t n, int64_t V,
                         Control *ctl, void *stream, lce_timers *tm) {
  launch_guard(targets, mask, n, V, ctl, static_cast<hipStream_t>(stream), tm, 0);
}

// A vocabulary-shard call covers rows [offset, offset + V) of a head of
// `total` rows (total == 0: the whole head).  Targets are checked against
// `total` and used relative to the shard; the forward then ends with the
// shard's exchange records instead of the loss.
template <class Acc>
struct Shard {
  int64_t offset = 0, total = 0;
  Acc *stats = nullptr;   // forward: {m, s, z_target} rows of n tokens
};

// The per-call preparation: one prep_kernel with the guard (against the
// head's rows; for up to 32768 tokens one workgroup that also starts the
// control block, else after a ctl_init launch), the shard-local ids (shard
// calls), the target logits (zy; absent when null) and H^T (Ht; absent when
// null).  Returns the target ids the later kernels use.
template <class TR>
static const int64_t *prepare(const CEPlan &p, const int64_t *y, const uint8_t *mask,
                              const Shard<typename TR::Acc> &sh, Control *ctl, uint8_t *ws,
                              const typename TR::E *H, const typename TR::E *W,
                              typename TR::Acc *zy, bool vec, typename TR::E *Ht,
                              hipStream_t st, lce_timers *tm, int keep_loss) {
  TimedLaunch tl(tm, LCE_K_GUARD, st);
  // Up to kGuardOneBlock tokens one guard workgroup also starts the control
  // block; beyond, ctl_init runs first and the guard is spread out.
  constexpr int64_t kGuardOneBlock = 32768;
  const bool one = p.n <= kGuardOneBlock;
  if (!one) hipLaunchKernelGGL(ctl_init_kernel, dim3(1), dim3(64), 0, st, ctl, keep_loss);
  const int64_t row_blocks = cdiv(p.n, 256) < 1024 ? cdiv(p.n, 256) : 1024;
  Prep<TR> a{};
  a.guard_init = one ? 1 : 0;
  a.keep_loss = keep_loss;
  a.y = y;
  a.mask = mask;
  a.n = p.n;
  a.v_check = sh.total ? sh.total : p.V;
  a.ctl = ctl;
  a.offset = sh.total ? sh.offset : 0;
  a.rows = p.V;
  a.yl = sh.total ? reinterpret_cast<int64_t *>(ws + p.off_yloc) : nullptr;
  a.H = H;
  a.W = W;
  a.D = p.D;
  a.zy = zy;
  a.vec8 = vec ? 1 : 0;
  a.Ht = Ht;
  a.ld = p.d_ld;
  a.tr_cols = cdiv(p.d_ld, 64);
  a.nb_guard = one ? 1 : row_blocks;
  a.nb_local = sh.total ? row_blocks : 0;
  a.nb_zy = zy ? cdiv(p.n, 4) : 0;
  a.nb_tr = Ht ? a.tr_cols * cdiv(p.D, 64) : 0;
  hipLaunchKernelGGL(prep_kernel<TR>, dim3(unsigned(a.blocks())), dim3(256), 0, st, a);
  return sh.total ? a.yl : y;
}

template <class TR>
static void forward_impl(const CEPlan &p, const void *H, const void *W, const int64_t *y_in,
                         const uint8_t *mask, typename TR::Acc *lse_out, uint8_t *ws, bool vec,
                         hipStream_t st, lce_timers *tm, const Shard<typename TR::Acc> &sh) {
  typedef typename TR::Acc Acc;
  Control *ctl = reinterpret_cast<Control *>(ws);
  Acc *partials = reinterpret_cast<Acc *>(ws + p.off_partials);
  Acc *zy = reinterpret_cast<Acc *>(ws + p.off_zy);
  double *loss_tok = reinterpret_cast<double *>(ws + p.off_losstok);
  const typename TR::E *Hp = static_cast<const typename TR::E *>(H);
  // (the forward needs no target ids after the preparation: the target
  // logits come from it)
  prepare<TR>(p, y_in, mask, sh, ctl, ws, Hp, static_cast<const typename TR::E *>(W), zy, vec,
              nullptr, st, tm, 0);
  for (int64_t tok0 = 0; tok0 < p.n; tok0 += p.tok_per_pass) {
    const int64_t ntok = p.tok_per_pass < p.n - tok0 ? p.tok_per_pass : p.n - tok0;
    GemmParams g;
    g.A = W; g.lda = p.D;
    g.B = Hp + tok0 * p.D; g.ldb = p.D;
    g.M = p.V; g.N = ntok; g.K = p.D;
    g.M_read = p.V; g.N_read = ntok;
    g.k_per_split = cdiv(p.D, TR::BK) * TR::BK;
    g.tiles_n = cdiv(ntok, TR::BN);
    g.bad = &ctl->bad;
    FwdLseEpi<TR> epi{ntok, p.V, p.n_vparts, partials};
    {
      TimedLaunch tl(tm, LCE_K_FWD_GEMM, st);
      bool done = false;
      if constexpr (IsH16<TR>::value) {
        if (UsePipe<TR>::ok(vec, p.D, p.d_ld)) {  // persistent: one workgroup per CU
          typedef typename W8Of<TR>::type TRP;
          const int64_t tiles = cdiv(g.M, PipeKK::BM) * g.tiles_n;
          const int64_t grid = tiles < kComputeUnits ? tiles : kComputeUnits;
          const auto e = retrait<TRP>(epi);
          hipLaunchKernelGGL((gemm2_persistent_kernel<PipeKK, TRP, decltype(e)>),
                             dim3(unsigned(grid)), dim3(TRP::NT), 0, st, to_gemm2<PipeKK>(g), e);
          done = true;
        }
      }
      if (!done) launch_any<TR, true, true>(false, vec, g, 1, epi, st);
    }
    TimedLaunch tl(tm, LCE_K_FWD_MERGE, st);
    hipLaunchKernelGGL(fwd_merge_kernel<Acc>, dim3(unsigned(cdiv(ntok, 4))), dim3(256), 0, st,
                       (const Acc *)partials, (const Acc *)(zy + tok0), p.n_vparts, ntok,
                       lse_out ? lse_out + tok0 : nullptr, loss_tok + tok0,
                       (const int32_t *)&ctl->bad, sh.stats ? sh.stats + tok0 : nullptr, p.n);
  }
  if (sh.stats) return;   // a shard's records; the exchange forms the loss
  TimedLaunch tl(tm, LCE_K_REDUCE, st);
  hipLaunchKernelGGL(fwd_final_kernel<Acc>, dim3(1), dim3(1024), 0, st, (const double *)loss_tok,
                     (const Acc *)lse_out, mask, p.n, ctl);
}

// 16-bit backward as a slab pipeline: launch k runs d_hidden and d_weight of
// slab k-1 (from slab buffer (k-1) % 2) together with the logit gradient of
// slab k (into buffer k % 2), longest products first.  Slab 0 may be shorter
// than the rest (the plan sizes it to one round of CUs).  The first launch
// with d_hidden work stores the split accumulators and every later launch adds
// to them.
template <class TR, bool ACC_DW>
static void backward_pipelined(const CEPlan &p, const uint16_t *Hp, const uint16_t *Wp,
                               const int64_t *y, const uint8_t *mask, const float *lse,
                               double z_coef, double grad_out, float *dW, uint16_t *dbuf,
                               float *dhacc, const uint16_t *Ht, const float *zyb, Control *ctl,
                               hipStream_t st, lce_timers *tm) {
  typedef typename W8Of<TR>::type TRP;
  typedef Gemm2Job<PipeMN, false, false, StoreEpi<TRP, true>> JH;
  // the first slab's d_hidden partials are stored, not added (nothing to
  // clear), and kept in the caches for the next launch's additions
  typedef Gemm2Job<PipeMN, false, false, StoreEpi<TRP, false, false>> JH0;
  typedef Gemm2Job<PipeKK, true, true, StoreEpi<TRP, ACC_DW>> JW;
  typedef Gemm2Job<PipeKK, true, true, DlogitEpi<TRP>> JL;
  const int64_t n = p.n, D = p.D, V = p.V, S = p.pslab, sp = p.pdh_splits;
  const int64_t tiles_d = cdiv(D, 256), tiles_t = cdiv(n, 256);
  // first vocabulary row and row count of slab j
  auto slab_at = [&](int64_t j, int64_t &rows) {
    const int64_t v0 = j == 0 ? 0 : p.pslab0 + (j - 1) * S;
    const int64_t cap = j == 0 ? p.pslab0 : S;
    rows = cap < V - v0 ? cap : V - v0;
    return v0;
  };
  struct Packed {
    int64_t key[3];
    double d0;
    bool ok;
    PackCounts pc;
    int slots;
  } packs[4];
  int n_packs = 0;
  for (int64_t k = 0; k <= p.pn_slabs; ++k) {
    JH jh{};
    JW jw{};
    JL jl{};
    if (k >= 1) {  // slab k-1: d_hidden += d W_slab, d_weight rows = d H
      int64_t rows;
      const int64_t vs0 = slab_at(k - 1, rows);
      const uint16_t *buf = dbuf + ((k - 1) & 1) * S * p.d_ld;
      GemmParams g;
      g.A = buf; g.lda = p.d_ld;
      g.B = Wp + vs0 * D; g.ldb = D;
      g.M = n; g.N = D; g.K = rows;
      g.M_read = p.d_ld; g.N_read = D;
      g.k_per_split = cdiv(cdiv(rows, sp), PipeMN::BK) * PipeMN::BK;
      g.tiles_n = tiles_d;
      g.bad = &ctl->bad;
      jh.g = to_gemm2<PipeMN>(g);
      jh.e = StoreEpi<TRP, true>{dhacc, D, 0, n, D, n * D};
      jh.nreal = tiles_t * tiles_d * sp;
      jh.nb = round_up8(jh.nreal);
      GemmParams h;
      h.A = buf; h.lda = p.d_ld;
      h.B = Ht; h.ldb = p.d_ld;
      h.M = rows; h.N = D; h.K = n;
      h.M_read = rows; h.N_read = D;
      h.k_per_split = cdiv(n, PipeKK::BK) * PipeKK::BK;
      h.tiles_n = tiles_d;
      h.bad = &ctl->bad;
      jw.g = to_gemm2<PipeKK>(h);
      jw.e = StoreEpi<TRP, ACC_DW>{dW, D, vs0, rows, D, 0};
      jw.nreal = cdiv(rows, 256) * tiles_d;
      jw.nb = round_up8(jw.nreal);
    }
    if (k < p.pn_slabs) {  // slab k: recomputed logits -> logit gradient
      int64_t rows;
      const int64_t vs0 = slab_at(k, rows);
      uint16_t *buf = dbuf + (k & 1) * S * p.d_ld;
      GemmParams g;
      g.A = Wp + vs0 * D; g.lda = D;
      g.B = Hp; g.ldb = D;
      g.M = rows; g.N = n; g.K = D;
      g.M_read = rows; g.N_read = n;
      g.k_per_split = cdiv(D, PipeKK::BK) * PipeKK::BK;
      g.tiles_n = tiles_t;
      g.bad = &ctl->bad;
      jl.g = to_gemm2<PipeKK>(g);
      jl.e = DlogitEpi<TRP>{y, mask, lse, n, vs0, rows, ctl, grad_out, z_coef, buf, p.d_ld, zyb};
      jl.nreal = cdiv(rows, 256) * tiles_t;
      jl.nb = round_up8(jl.nreal);
    }
    TimedLaunch tl(tm, LCE_K_BWD_GEMM, st);
    // Packed onto the compute units by the host with the tile-duration model
    // the planner chose the slabs with; hardware dispatch in product order
    // when the packing does not apply.
    const int64_t nt[3] = {jh.nreal, jw.nreal, jl.nreal};
    const double dur[3] = {tile_us_dhidden(jh.g.k_per_split), tile_us_dweight(n),
                           tile_us_dlogit(D)};
    // launches with the same tile counts and durations share one packing
    int m = -1;
    for (int i = 0; i < n_packs; ++i)
      if (packs[i].key[0] == nt[0] && packs[i].key[1] == nt[1] && packs[i].key[2] == nt[2] &&
          packs[i].d0 == dur[0])
        m = i;
    if (m < 0 && n_packs < 4 && p.ppacked) {
      m = n_packs++;
      packs[m].key[0] = nt[0]; packs[m].key[1] = nt[1]; packs[m].key[2] = nt[2];
      packs[m].d0 = dur[0];
      packs[m].ok = pack_tiles(nt, dur, &packs[m].pc, &packs[m].slots);
    }
    auto launch = [&](const auto &jhx) {
      typedef typename std::decay<decltype(jhx)>::type JHX;
      if (m >= 0 && packs[m].ok) {
        const PackCounts &pack = packs[m].pc;
        const int pack_slots = packs[m].slots;
        hipLaunchKernelGGL((gemm2_packed_kernel<TRP, JHX, JW, JL>),
                           dim3(unsigned(kPackXcds * pack_slots)), dim3(TRP::NT), 0, st, jhx, jw,
                           jl, pack);
      } else {
        const int64_t total = jhx.nb + jw.nb + jl.nb;
        hipLaunchKernelGGL((gemm2_multi_kernel<TRP, JHX, JW, JL>), dim3(unsigned(total)),
                           dim3(TRP::NT), 0, st, jhx, jw, jl);
      }
    };
    if (k == 1) {
      JH0 jh0{};
      jh0.g = jh.g;
      jh0.e = StoreEpi<TRP, false, false>{jh.e.out, jh.e.ldo, jh.e.row_off, jh.e.rows, jh.e.cols,
                                   jh.e.split_stride};
      jh0.nb = jh.nb;
      jh0.nreal = jh.nreal;
      launch(jh0);
    } else {
      launch(jh);
    }
  }
}

template <class TR>
static void launch_dh_final(const typename TR::Acc *P, int64_t splits, int64_t count, void *dH,
                            bool acc_out, const int32_t *bad, hipStream_t st, lce_timers *tm) {
  int64_t blocks = cdiv(count, 256);
  if (blocks > 4096) blocks = 4096;
  TimedLaunch tl(tm, LCE_K_DH_FINAL, st);
  typedef typename TR::Acc Acc;
  typedef typename TR::E E;
  if (acc_out)
    hipLaunchKernelGGL((dh_final_kernel<TR, Acc>), dim3(unsigned(blocks)), dim3(256), 0, st, P,
                       splits, count, static_cast<Acc *>(dH), bad, 0);
  else
    hipLaunchKernelGGL((dh_final_kernel<TR, E>), dim3(unsigned(blocks)), dim3(256), 0, st, P,
                       splits, count, static_cast<E *>(dH), bad, fold_vec4(count, dH));
}

template <class TR>
static void backward_impl(const CEPlan &p, const void *H, const void *W, const int64_t *y_in,
                          const uint8_t *mask, const typename TR::Acc *lse, double z_coef,
                          double grad_out, void *dH, bool dh_acc, typename TR::Acc *dW,
                          int accumulate, uint8_t *ws, bool vec, hipStream_t st,
                          lce_timers *tm, const Shard<typename TR::Acc> &sh) {
  typedef typename TR::Acc Acc;
  typedef typename TR::E E;
  Control *ctl = reinterpret_cast<Control *>(ws);
  E *dbuf = reinterpret_cast<E *>(ws + p.off_dbuf);
  Acc *dhacc = reinterpret_cast<Acc *>(ws + p.off_dhacc);
  const E *Hp = static_cast<const E *>(H);
  const E *Wp = static_cast<const E *>(W);
  const bool pipe = UsePipe<TR>::ok(vec, p.D, p.d_ld);
  E *Ht = nullptr;
  Acc *zyb = nullptr;
  if constexpr (IsH16<TR>::value) {
    if (pipe) {
      // K-major operands of the d_weight product: H^T and the slab buffer,
      // both zero in token columns [n, d_ld) (the staged logit-gradient
      // epilogue writes the slab buffer's zeros); the target logits for that
      // epilogue.  (The d_hidden accumulators need no clearing: the first
      // slab's launch stores them.)
      Ht = reinterpret_cast<E *>(ws + p.off_ht);
      zyb = reinterpret_cast<Acc *>(ws + p.off_zyb);
    }
  } else {
    // fp64: H^T too, so that the d_weight product reads both operands
    // K-major instead of transposing H's 8 x 8 blocks in registers
    Ht = reinterpret_cast<E *>(ws + p.off_ht);
  }
  const int64_t *y = prepare<TR>(p, y_in, mask, sh, ctl, ws, Hp, Wp, zyb, vec, Ht, st, tm, 1);
  if constexpr (IsH16<TR>::value) {
    if (pipe) {
      if (p.pslab > 0) {
        if (accumulate)
          backward_pipelined<TR, true>(p, Hp, Wp, y, mask, lse, z_coef, grad_out, dW, dbuf,
                                       dhacc, Ht, zyb, ctl, st, tm);
        else
          backward_pipelined<TR, false>(p, Hp, Wp, y, mask, lse, z_coef, grad_out, dW, dbuf,
                                        dhacc, Ht, zyb, ctl, st, tm);
        launch_dh_final<TR>(dhacc, p.pdh_splits, p.n * p.D, dH, dh_acc,
                            (const int32_t *)&ctl->bad, st, tm);
        return;
      }
    }
  }
  for (int64_t s = 0; s < p.n_slabs; ++s) {
    const int64_t vs0 = s * p.slab;
    const int64_t rows = p.slab < p.V - vs0 ? p.slab : p.V - vs0;
    const E *Wslab = Wp + vs0 * p.D;
    {  // logits of the slab -> logit gradient
      GemmParams g;
      g.A = Wslab; g.lda = p.D;
      g.B = Hp; g.ldb = p.D;
      g.M = rows; g.N = p.n; g.K = p.D;
      g.M_read = rows; g.N_read = p.n;
      g.k_per_split = cdiv(p.D, TR::BK) * TR::BK;
      g.tiles_n = cdiv(p.n, TR::BN);
      g.bad = &ctl->bad;
      DlogitEpi<TR> epi{y, mask, lse, p.n, vs0, rows, ctl, grad_out, z_coef, dbuf, p.d_ld, zyb};
      TimedLaunch tl(tm, LCE_K_DLOGIT_GEMM, st);
      launch_any<TR, true, true>(pipe, vec, g, 1, epi, st);
    }
    {  // d_weight rows of the slab = d^T H over all tokens
      GemmParams g;
      g.A = dbuf; g.lda = p.d_ld;
      g.M = rows; g.N = p.D; g.K = p.n;
      g.M_read = rows;
      g.k_per_split = cdiv(p.n, TR::BK) * TR::BK;
      g.tiles_n = cdiv(p.D, TR::BN);
      g.bad = &ctl->bad;
      TimedLaunch tl(tm, LCE_K_DW_GEMM, st);
      const StoreEpi<TR, true> e_acc{dW, p.D, vs0, rows, p.D, 0};
      const StoreEpi<TR, false> e_set{dW, p.D, vs0, rows, p.D, 0};
      if (Ht) {    // B = H^T, K-major like the slab buffer
        g.B = Ht; g.ldb = p.d_ld;
        g.N_read = p.D;
        if (accumulate) launch_any<TR, true, true>(pipe, vec, g, 1, e_acc, st);
        else launch_any<TR, true, true>(pipe, vec, g, 1, e_set, st);
      } else {     // B = H read MN-major (rows D long)
        g.B = Hp; g.ldb = p.D;
        g.N_read = p.D;
        if (accumulate) launch_gemm<TR, true, false>(vec, g, 1, e_acc, st);
        else launch_gemm<TR, true, false>(vec, g, 1, e_set, st);
      }
    }
    {  // d_hidden split accumulators += d W_slab
      const int64_t kps = cdiv(cdiv(rows, p.dh_splits), TR::BK) * TR::BK;
      GemmParams g;
      g.A = dbuf; g.lda = p.d_ld;
      g.B = Wslab; g.ldb = p.D;
      g.M = p.n; g.N = p.D; g.K = rows;
      g.M_read = p.d_ld; g.N_read = p.D;  // slab rows are d_ld long; W rows D long
      g.k_per_split = kps;
      g.tiles_n = cdiv(p.D, TR::BN);
      g.bad = &ctl->bad;
      TimedLaunch tl(tm, LCE_K_DH_GEMM, st);
      const StoreEpi<TR, true> e_acc{dhacc, p.D, 0, p.n, p.D, p.n * p.D};
      const StoreEpi<TR, false> e_set{dhacc, p.D, 0, p.n, p.D, p.n * p.D};
      if (s > 0) launch_any<TR, false, false>(pipe, vec, g, p.dh_splits, e_acc, st);
      else launch_any<TR, false, false>(pipe, vec, g, p.dh_splits, e_set, st);
    }
  }
  launch_dh_final<TR>(dhacc, p.dh_splits, p.n * p.D, dH, dh_acc, (const int32_t *)&ctl->bad,
                      st, tm);
}


// Forward and backward in one pass over the logits (16-bit inputs, the whole
// batch in one chunk): the forward GEMM keeps its fp32 tiles in Z besides the
// (max, sum) partials; after the merge gives lse, dlogit_rows_kernel turns Z
// in place into the logit gradient, and one launch runs d_hidden (split over
// the vocabulary) and d_weight from it.  6 n D V flops instead of 8.
template <class TR>
static void forward_backward_single(const CEPlan &p, const void *H, const void *W,
                                    const int64_t *y, const uint8_t *mask, float *lse_out,
                                    double z_coef, double grad_out, void *dH, float *dW,
                                    int accumulate, uint8_t *ws, bool vec, hipStream_t st,
                                    lce_timers *tm) {
  typedef typename W8Of<TR>::type TRP;
  typedef typename TR::E E;
  const int64_t n = p.n, D = p.D, V = p.V, sp = p.f_sp;
  Control *ctl = reinterpret_cast<Control *>(ws);
  float *partials = reinterpret_cast<float *>(ws + p.off_partials);
  float *zy = reinterpret_cast<float *>(ws + p.off_zy);
  double *loss_tok = reinterpret_cast<double *>(ws + p.off_losstok);
  float *Z = reinterpret_cast<float *>(ws + p.off_fz);
  float *dhacc = reinterpret_cast<float *>(ws + p.off_fdh);
  E *Ht = reinterpret_cast<E *>(ws + p.off_fht);
  const E *Hp = static_cast<const E *>(H);
  const E *Wp = static_cast<const E *>(W);
  const Shard<float> whole;
  // (every d_hidden split partial is written whole by its own workgroup:
  // nothing to clear)
  prepare<TR>(p, y, mask, whole, ctl, ws, Hp, Wp, zy, vec, Ht, st, tm, 0);
  const int64_t tiles_t = cdiv(n, 256), tiles_d = cdiv(D, 256);
  {
    GemmParams g;
    g.A = Wp; g.lda = D;
    g.B = Hp; g.ldb = D;
    g.M = V; g.N = n; g.K = D;
    g.M_read = V; g.N_read = n;
    g.k_per_split = cdiv(D, PipeKK::BK) * PipeKK::BK;
    g.tiles_n = tiles_t;
    g.bad = &ctl->bad;
    const FwdKeepEpi<TRP> e{FwdLseEpi<TRP>{n, V, p.n_vparts, partials},
                            StoreEpi<TRP, false>{Z, p.f_ld, 0, V, n, 0}};
    TimedLaunch tl(tm, LCE_K_FWD_GEMM, st);
    // (the persistent form, with these stores from the registers, measured
    // slower: 2.63 against 2.32 ms for the whole call at 512 x 4096 x 151936)
    hipLaunchKernelGGL((gemm2_kernel<PipeKK, TRP, true, true, FwdKeepEpi<TRP>>),
                       dim3(unsigned(cdiv(V, 256) * tiles_t)), dim3(TRP::NT), 0, st,
                       to_gemm2<PipeKK>(g), e);
  }
  {
    TimedLaunch tl(tm, LCE_K_FWD_MERGE, st);
    hipLaunchKernelGGL(fwd_merge_kernel<float>, dim3(unsigned(cdiv(n, 4))), dim3(256), 0, st,
                       (const float *)partials, (const float *)zy, p.n_vparts, n, lse_out,
                       loss_tok, (const int32_t *)&ctl->bad, (float *)nullptr, n);
  }
  {
    TimedLaunch tl(tm, LCE_K_REDUCE, st);
    hipLaunchKernelGGL(fwd_final_kernel<float>, dim3(1), dim3(1024), 0, st,
                       (const double *)loss_tok, (const float *)lse_out, mask, n, ctl);
  }
  {
    TimedLaunch tl(tm, LCE_K_DLOGIT_ROWS, st);
    if (n % 4 == 0)
      hipLaunchKernelGGL(dlogit_rows4_kernel<TR>,
                         dim3(unsigned(std::min<int64_t>(cdiv(V, 4 * kDlogitRows), kDlogit4Blocks))),
                         dim3(256), 0, st, Z, V, n, p.f_ld, y, mask, (const float *)lse_out,
                         (const float *)zy, (const Control *)ctl, grad_out, z_coef);
    else
      hipLaunchKernelGGL(dlogit_rows_kernel<TR>, dim3(unsigned(cdiv(V, 4 * kDlogitRows))),
                         dim3(256), 0, st, Z, V, n, p.f_ld, y, mask, (const float *)lse_out,
                         (const float *)zy, (const Control *)ctl, grad_out, z_coef);
  }
  // d_hidden += d W over the whole vocabulary (split-K), d_weight = d^T H:
  // the two products of a slab-pipeline launch, with the logit gradient in Z
  // (16-bit values, row stride 2 * f_ld) as the one slab.
  const uint16_t *buf = reinterpret_cast<const uint16_t *>(Z);
  const int64_t ldd = 2 * p.f_ld;
  auto launch = [&](auto acc_tag) {
    constexpr bool ACC = decltype(acc_tag)::value;
    typedef Gemm2Job<PipeMN, false, false, StoreEpi<TRP, false>> JH;
    typedef Gemm2Job<PipeKK, true, true, StoreEpi<TRP, ACC>> JW;
    typedef Gemm2Job<PipeKK, true, true, DlogitEpi<TRP>> JL;
    JH jh{};
    JW jw{};
    JL jl{};
    GemmParams g;
    g.A = buf; g.lda = ldd;
    g.B = Wp; g.ldb = D;
    g.M = n; g.N = D; g.K = V;
    g.M_read = p.d_ld; g.N_read = D;
    g.k_per_split = cdiv(cdiv(V, sp), PipeMN::BK) * PipeMN::BK;
    g.tiles_n = tiles_d;
    g.bad = &ctl->bad;
    jh.g = to_gemm2<PipeMN>(g);
    jh.e = StoreEpi<TRP, false>{dhacc, D, 0, n, D, n * D};
    jh.nreal = tiles_t * tiles_d * sp;
    jh.nb = round_up8(jh.nreal);
    GemmParams h;
    h.A = buf; h.lda = ldd;
    h.B = Ht; h.ldb = p.d_ld;
    h.M = V; h.N = D; h.K = n;
    h.M_read = V; h.N_read = D;
    h.k_per_split = cdiv(n, PipeKK::BK) * PipeKK::BK;
    h.tiles_n = tiles_d;
    h.bad = &ctl->bad;
    jw.g = to_gemm2<PipeKK>(h);
    jw.e = StoreEpi<TRP, ACC>{dW, D, 0, V, D, 0};
    jw.nreal = cdiv(V, 256) * tiles_d;
    jw.nb = round_up8(jw.nreal);
    TimedLaunch tl(tm, LCE_K_BWD_GEMM, st);
    hipLaunchKernelGGL((gemm2_multi_kernel<TRP, JH, JW, JL>), dim3(unsigned(jh.nb + jw.nb)),
                       dim3(TRP::NT), 0, st, jh, jw, jl);
  };
  if (accumulate) launch(std::true_type{});
  else launch(std::false_type{});
  launch_dh_final<TR>(dhacc, sp, n * D, dH, false, (const int32_t *)&ctl->bad, st, tm);
}

}  // namespace lce

using namespace lce;

namespace {

bool has(const lce_tensor *t) { return t && t->data; }

// Dtype and length checks shared by forward and backward.
int32_t check_ce_tensors(const lce_tensor *hidden, const lce_tensor *weight,
                         const lce_tensor *targets, const lce_tensor *loss_mask, int64_t n,
                         int64_t D, int64_t V, int32_t *dtype) {
  if (!hidden || !weight || !targets) return LCE_LENGTH_MISMATCH;
  const int32_t dt = hidden->dtype;
  if (dt != LCE_BF16 && dt != LCE_F16 && dt != LCE_F64) return LCE_DTYPE_MISMATCH;
  if (weight->dtype != dt || targets->dtype != LCE_I64) return LCE_DTYPE_MISMATCH;
  if (has(loss_mask) && loss_mask->dtype != LCE_U8) return LCE_DTYPE_MISMATCH;
  *dtype = dt;
  return LCE_OK;
}

int32_t check_ce_lengths(const lce_tensor *hidden, const lce_tensor *weight,
                         const lce_tensor *targets, const lce_tensor *loss_mask, int64_t n,
                         int64_t D, int64_t V) {
  if (!has(hidden) || hidden->numel < n * D) return LCE_LENGTH_MISMATCH;
  if (!has(weight) || weight->numel < V * D) return LCE_LENGTH_MISMATCH;
  if (!has(targets) || targets->numel < n) return LCE_LENGTH_MISMATCH;
  if (has(loss_mask) && loss_mask->numel < n) return LCE_LENGTH_MISMATCH;
  return LCE_OK;
}

// A vocabulary shard: rows [offset, offset + vocab) inside a head of `total`
// rows (total == 0: the call covers the whole head).
int32_t check_shard(int64_t vocab, int64_t offset, int64_t total) {
  if (total == 0) return LCE_OK;
  if (total < 0) return LCE_EMPTY_DIMENSION;
  if (total > LCE_MAX_VOCAB) return LCE_DIMENSION_TOO_LARGE;
  if (offset < 0 || offset > total - vocab) return LCE_LENGTH_MISMATCH;
  return LCE_OK;
}

int32_t forward_call(const lce_tensor *hidden, const lce_tensor *weight,
                     const lce_tensor *targets, const lce_tensor *loss_mask, int64_t n_tok,
                     int64_t d_model, int64_t vocab, int64_t chunk, double z_coef,
                     lce_tensor *lse_out, lce_tensor *workspace, lce_loss *out, void *stream,
                     lce_timers *timers, int64_t offset, int64_t total, lce_tensor *stats);
int32_t backward_call(const lce_tensor *hidden, const lce_tensor *weight,
                      const lce_tensor *targets, const lce_tensor *loss_mask,
                      const lce_tensor *lse, int64_t n_tok, int64_t d_model, int64_t vocab,
                      int64_t chunk, double z_coef, double grad_out, lce_tensor *d_hidden,
                      lce_tensor *d_weight, int32_t accumulate_d_weight,
                      lce_tensor *workspace, void *stream, lce_timers *timers, int64_t offset,
                      int64_t total);

int32_t finish(hipStream_t st, Control *dev_ctl, Control *host_ctl) {
  if (hipGetLastError() != hipSuccess) return LCE_DEVICE_ERROR;
  if (hipMemcpyAsync(host_ctl, dev_ctl, sizeof(Control), hipMemcpyDeviceToHost, st) != hipSuccess)
    return LCE_DEVICE_ERROR;
  if (hipStreamSynchronize(st) != hipSuccess) return LCE_DEVICE_ERROR;
  return (host_ctl->bad || host_ctl->seen_bad) ? LCE_TARGET_OUT_OF_RANGE : LCE_OK;
}

// An asynchronous call's status: only launch errors are known on return.
int32_t enqueued() { return hipGetLastError() == hipSuccess ? LCE_OK : LCE_DEVICE_ERROR; }

void fill_loss(const Control &hc, lce_loss *out) {
  out->loss_sum = hc.loss_sum;
  out->z_sum = hc.z_sum;
  out->n_counted = hc.count;
  out->loss_mean = hc.count ? hc.loss_sum / double(hc.count) : 0.0;
  out->z_mean = hc.count ? hc.z_sum / double(hc.count) : 0.0;
}

}  // namespace

extern "C" {

int32_t lce_forward(const lce_tensor *hidden, const lce_tensor *weight,
                    const lce_tensor *targets, const lce_tensor *loss_mask, int64_t n_tok,
                    int64_t d_model, int64_t vocab, int64_t chunk, double z_coef,
                    lce_tensor *lse_out, lce_tensor *workspace, lce_loss *out, void *stream) {
  return lce_forward_timed(hidden, weight, targets, loss_mask, n_tok, d_model, vocab, chunk,
                           z_coef, lse_out, workspace, out, stream, nullptr);
}

int32_t lce_forward_timed(const lce_tensor *hidden, const lce_tensor *weight,
                          const lce_tensor *targets, const lce_tensor *loss_mask, int64_t n_tok,
                          int64_t d_model, int64_t vocab, int64_t chunk, double z_coef,
                          lce_tensor *lse_out, lce_tensor *workspace, lce_loss *out,
                          void *stream, lce_timers *timers) {
  return forward_call(hidden, weight, targets, loss_mask, n_tok, d_model, vocab, chunk, z_coef,
                      lse_out, workspace, out, stream, timers, 0, 0, nullptr);
}

int32_t lce_shard_forward(const lce_tensor *hidden, const lce_tensor *weight_shard,
                          const lce_tensor *targets, int64_t n_tok, int64_t d_model,
                          int64_t vocab_shard, int64_t vocab_offset, int64_t vocab_total,
                          int64_t chunk, lce_tensor *stats, lce_tensor *workspace, void *stream) {
  // asynchronous: a target out of range shows in lce_loss_fetch(workspace)
  return forward_call(hidden, weight_shard, targets, nullptr, n_tok, d_model, vocab_shard, chunk,
                      0.0, nullptr, workspace, nullptr, stream, nullptr, vocab_offset, vocab_total,
                      stats);
}

int32_t lce_shard_merge(const lce_tensor *stats, int32_t n_shards, const lce_tensor *loss_mask,
                        int64_t n_tok, lce_tensor *lse_out, lce_tensor *workspace, lce_loss *out,
                        void *stream) {
  if (n_tok < 1 || n_shards < 1) return LCE_EMPTY_DIMENSION;
  if (n_tok > LCE_MAX_N_TOK) return LCE_DIMENSION_TOO_LARGE;
  if (!stats || !lse_out || !workspace) return LCE_LENGTH_MISMATCH;
  const int32_t adt = stats->dtype;
  if (adt != LCE_F32 && adt != LCE_F64) return LCE_DTYPE_MISMATCH;
  if (lse_out->dtype != adt) return LCE_DTYPE_MISMATCH;
  if (has(loss_mask) && loss_mask->dtype != LCE_U8) return LCE_DTYPE_MISMATCH;
  if (workspace->dtype != LCE_U8) return LCE_DTYPE_MISMATCH;
  DistillPlan p;   // {control | n per-token doubles | ...} fits the same layout
  int32_t st = plan_distill(n_tok, 1, &p);
  if (st != LCE_OK) return st;
  if (!has(stats) || stats->numel / 3 / n_shards < n_tok) return LCE_LENGTH_MISMATCH;
  if (!has(lse_out) || lse_out->numel < n_tok) return LCE_LENGTH_MISMATCH;
  if (has(loss_mask) && loss_mask->numel < n_tok) return LCE_LENGTH_MISMATCH;
  if (!has(workspace) || workspace->numel < int64_t(p.total) + 256) return LCE_LENGTH_MISMATCH;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *ws = ws_base(workspace);
  Control *ctl = reinterpret_cast<Control *>(ws);
  double *loss_tok = reinterpret_cast<double *>(ws + p.off_rows);
  const uint8_t *mask = has(loss_mask) ? static_cast<const uint8_t *>(loss_mask->data) : nullptr;
  (void)hipGetLastError();
  launch_guard(nullptr, mask, n_tok, 1, ctl, s, nullptr, 0);   // counted tokens
  int64_t blocks = cdiv(n_tok, 256);
  if (blocks > 1024) blocks = 1024;
  if (adt == LCE_F32) {
    hipLaunchKernelGGL(shard_merge_kernel<float>, dim3(unsigned(blocks)), dim3(256), 0, s,
                       static_cast<const float *>(stats->data), int64_t(n_shards), n_tok,
                       static_cast<float *>(lse_out->data), loss_tok);
    hipLaunchKernelGGL(fwd_final_kernel<float>, dim3(1), dim3(1024), 0, s,
                       (const double *)loss_tok, static_cast<const float *>(lse_out->data), mask,
                       n_tok, ctl);
  } else {
    hipLaunchKernelGGL(shard_merge_kernel<double>, dim3(unsigned(blocks)), dim3(256), 0, s,
                       static_cast<const double *>(stats->data), int64_t(n_shards), n_tok,
                       static_cast<double *>(lse_out->data), loss_tok);
    hipLaunchKernelGGL(fwd_final_kernel<double>, dim3(1), dim3(1024), 0, s,
                       (const double *)loss_tok, static_cast<const double *>(lse_out->data), mask,
                       n_tok, ctl);
  }
  if (!out) return enqueued();   // the scalars: lce_loss_fetch(workspace)
  Control hc;
  st = finish(s, ctl, &hc);
  if (st != LCE_OK) return st;
  fill_loss(hc, out);
  return LCE_OK;
}

}  // extern "C"

namespace {

// The whole head (total == 0) or a vocabulary shard of rows [offset, offset
// + vocab) of a `total`-row head (exchange records to `stats`).
int32_t forward_call(const lce_tensor *hidden, const lce_tensor *weight,
                     const lce_tensor *targets, const lce_tensor *loss_mask, int64_t n_tok,
                     int64_t d_model, int64_t vocab, int64_t chunk, double z_coef,
                     lce_tensor *lse_out, lce_tensor *workspace, lce_loss *out, void *stream,
                     lce_timers *timers, int64_t offset, int64_t total, lce_tensor *stats) {
  int32_t st = lce_dims_check(n_tok, d_model, vocab);
  if (st != LCE_OK) return st;
  st = check_shard(vocab, offset, total);
  if (st != LCE_OK) return st;
  st = lce_chunk_check(chunk, vocab);
  if (st != LCE_OK) return st;
  if (!finite_scalar(z_coef)) return LCE_NON_FINITE_SCALAR;
  int32_t dt = 0;
  st = check_ce_tensors(hidden, weight, targets, loss_mask, n_tok, d_model, vocab, &dt);
  if (st != LCE_OK) return st;
  lce_tensor *res = total ? stats : lse_out;   // [3 n] records or [n] lse
  if (!res || !workspace) return LCE_LENGTH_MISMATCH;
  if (res->dtype != (dt == LCE_F64 ? LCE_F64 : LCE_F32)) return LCE_DTYPE_MISMATCH;
  if (workspace->dtype != LCE_U8) return LCE_DTYPE_MISMATCH;
  CEPlan p;
  st = plan_ce(n_tok, d_model, vocab, chunk, dt, &p);
  if (st != LCE_OK) return st;
  st = check_ce_lengths(hidden, weight, targets, loss_mask, n_tok, d_model, vocab);
  if (st != LCE_OK) return st;
  if (!has(res) || res->numel < (total ? 3 : 1) * n_tok) return LCE_LENGTH_MISMATCH;
  if (!has(workspace) || workspace->numel < int64_t(p.total) + 256) return LCE_LENGTH_MISMATCH;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *ws = ws_base(workspace);
  const uint8_t *mask = has(loss_mask) ? static_cast<const uint8_t *>(loss_mask->data) : nullptr;
  const int64_t *y = static_cast<const int64_t *>(targets->data);
  (void)hipGetLastError();
  if (dt != LCE_F64) {
    const bool vec = d_model % 8 == 0 && aligned16(hidden->data) && aligned16(weight->data);
    Shard<float> sh;
    sh.offset = offset; sh.total = total;
    sh.stats = total ? static_cast<float *>(stats->data) : nullptr;
    float *lo = total ? nullptr : static_cast<float *>(lse_out->data);
    if (dt == LCE_F16)
      forward_impl<TraitsF16>(p, hidden->data, weight->data, y, mask, lo, ws, vec, s, timers, sh);
    else
      forward_impl<TraitsBF16>(p, hidden->data, weight->data, y, mask, lo, ws, vec, s, timers, sh);
  } else {
    const bool vec = d_model % 2 == 0 && aligned16(hidden->data) && aligned16(weight->data);
    Shard<double> sh;
    sh.offset = offset; sh.total = total;
    sh.stats = total ? static_cast<double *>(stats->data) : nullptr;
    forward_impl<TraitsF64>(p, hidden->data, weight->data, y, mask,
                            total ? nullptr : static_cast<double *>(lse_out->data), ws, vec, s,
                            timers, sh);
  }
  if (!out) return enqueued();   // the scalars stay in the workspace (lce_loss_fetch)
  Control hc;
  st = finish(s, reinterpret_cast<Control *>(ws), &hc);
  if (st != LCE_OK) return st;
  if (!total) fill_loss(hc, out);
  return LCE_OK;
}

}  // namespace

extern "C" {

int32_t lce_loss_fetch(const lce_tensor *workspace, lce_loss *out, void *stream) {
  if (!out || !has(workspace) || workspace->numel < int64_t(kControlBytes) + 256)
    return LCE_LENGTH_MISMATCH;
  if (workspace->dtype != LCE_U8) return LCE_DTYPE_MISMATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Control hc;
  const int32_t st = finish(s, reinterpret_cast<Control *>(ws_base(workspace)), &hc);
  if (st != LCE_OK) return st;
  fill_loss(hc, out);
  return LCE_OK;
}

int32_t lce_backward(const lce_tensor *hidden, const lce_tensor *weight,
                     const lce_tensor *targets, const lce_tensor *loss_mask,
                     const lce_tensor *lse, int64_t n_tok, int64_t d_model, int64_t vocab,
                     int64_t chunk, double z_coef, double grad_out, lce_tensor *d_hidden,
                     lce_tensor *d_weight, int32_t accumulate_d_weight,
                     lce_tensor *workspace, void *stream) {
  return lce_backward_timed(hidden, weight, targets, loss_mask, lse, n_tok, d_model, vocab, chunk,
                            z_coef, grad_out, d_hidden, d_weight, accumulate_d_weight, workspace,
                            stream, nullptr);
}

int32_t lce_backward_timed(const lce_tensor *hidden, const lce_tensor *weight,
                           const lce_tensor *targets, const lce_tensor *loss_mask,
                           const lce_tensor *lse, int64_t n_tok, int64_t d_model, int64_t vocab,
                           int64_t chunk, double z_coef, double grad_out, lce_tensor *d_hidden,
                           lce_tensor *d_weight, int32_t accumulate_d_weight,
                           lce_tensor *workspace, void *stream, lce_timers *timers) {
  return backward_call(hidden, weight, targets, loss_mask, lse, n_tok, d_model, vocab, chunk,
                       z_coef, grad_out, d_hidden, d_weight, accumulate_d_weight, workspace,
                       stream, timers, 0, 0);
}

int32_t lce_shard_backward(const lce_tensor *hidden, const lce_tensor *weight_shard,
                           const lce_tensor *targets, const lce_tensor *loss_mask,
                           const lce_tensor *lse, int64_t n_tok, int64_t d_model,
                           int64_t vocab_shard, int64_t vocab_offset, int64_t vocab_total,
                           int64_t chunk, double z_coef, double grad_out,
                           lce_tensor *d_hidden_partial, lce_tensor *d_weight_shard,
                           int32_t accumulate_d_weight, lce_tensor *workspace, void *stream) {
  return backward_call(hidden, weight_shard, targets, loss_mask, lse, n_tok, d_model, vocab_shard,
                       chunk, z_coef, grad_out, d_hidden_partial, d_weight_shard,
                       accumulate_d_weight, workspace, stream, nullptr, vocab_offset,
                       vocab_total);
}

}  // extern "C"

namespace {

int32_t backward_call(const lce_tensor *hidden, const lce_tensor *weight,
                      const lce_tensor *targets, const lce_tensor *loss_mask,
                      const lce_tensor *lse, int64_t n_tok, int64_t d_model, int64_t vocab,
                      int64_t chunk, double z_coef, double grad_out, lce_tensor *d_hidden,
                      lce_tensor *d_weight, int32_t accumulate_d_weight,
                      lce_tensor *workspace, void *stream, lce_timers *timers, int64_t offset,
                      int64_t total) {
  int32_t st = lce_dims_check(n_tok, d_model, vocab);
  if (st != LCE_OK) return st;
  st = check_shard(vocab, offset, total);
  if (st != LCE_OK) return st;
  st = lce_chunk_check(chunk, vocab);
  if (st != LCE_OK) return st;
  if (!finite_scalar(z_coef) || !finite_scalar(grad_out)) return LCE_NON_FINITE_SCALAR;
  int32_t dt = 0;
  st = check_ce_tensors(hidden, weight, targets, loss_mask, n_tok, d_model, vocab, &dt);
  if (st != LCE_OK) return st;
  if (!lse || !d_hidden || !d_weight || !workspace) return LCE_LENGTH_MISMATCH;
  const int32_t acc_dt = dt == LCE_F64 ? LCE_F64 : LCE_F32;
  // a shard's d_hidden is its unrounded partial (the shards' sum is the gradient)
  if (lse->dtype != acc_dt || d_weight->dtype != acc_dt ||
      d_hidden->dtype != (total ? acc_dt : dt))
    return LCE_DTYPE_MISMATCH;
  if (workspace->dtype != LCE_U8) return LCE_DTYPE_MISMATCH;
  CEPlan p;
  st = plan_ce(n_tok, d_model, vocab, chunk, dt, &p);
  if (st != LCE_OK) return st;
  st = check_ce_lengths(hidden, weight, targets, loss_mask, n_tok, d_model, vocab);
  if (st != LCE_OK) return st;
  if (!has(lse) || lse->numel < n_tok) return LCE_LENGTH_MISMATCH;
  if (!has(d_hidden) || d_hidden->numel < n_tok * d_model) return LCE_LENGTH_MISMATCH;
  if (!has(d_weight) || d_weight->numel < vocab * d_model) return LCE_LENGTH_MISMATCH;
  if (!has(workspace) || workspace->numel < int64_t(p.total) + 256) return LCE_LENGTH_MISMATCH;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *ws = ws_base(workspace);
  const uint8_t *mask = has(loss_mask) ? static_cast<const uint8_t *>(loss_mask->data) : nullptr;
  const int64_t *y = static_cast<const int64_t *>(targets->data);
  (void)hipGetLastError();
  if (dt != LCE_F64) {
    Shard<float> sh;
    sh.offset = offset; sh.total = total;
    // the staged d_weight epilogue writes 16-byte chunks
    const bool vec = d_model % 8 == 0 && aligned16(hidden->data) && aligned16(weight->data) &&
                     aligned16(d_weight->data);
    const float *l = static_cast<const float *>(lse->data);
    float *dw = static_cast<float *>(d_weight->data);
    if (dt == LCE_F16)
      backward_impl<TraitsF16>(p, hidden->data, weight->data, y, mask, l, z_coef, grad_out,
                               d_hidden->data, total != 0, dw, accumulate_d_weight != 0, ws, vec,
                               s, timers, sh);
    else
      backward_impl<TraitsBF16>(p, hidden->data, weight->data, y, mask, l, z_coef, grad_out,
                                d_hidden->data, total != 0, dw, accumulate_d_weight != 0, ws,
                                vec, s, timers, sh);
  } else {
    Shard<double> sh;
    sh.offset = offset; sh.total = total;
    const bool vec = d_model % 2 == 0 && aligned16(hidden->data) && aligned16(weight->data);
    backward_impl<TraitsF64>(p, hidden->data, weight->data, y, mask,
                             static_cast<const double *>(lse->data), z_coef, grad_out,
                             d_hidden->data, total != 0, static_cast<double *>(d_weight->data),
                             accumulate_d_weight != 0, ws, vec, s, timers, sh);
  }
  // No wait: a failed target guard makes every later kernel of the call exit
  // before writing, and lce_loss_fetch reports it.
  return enqueued();
}

}  // namespace

namespace {

int32_t forward_backward_call(const lce_tensor *hidden, const lce_tensor *weight,
                              const lce_tensor *targets, const lce_tensor *loss_mask,
                              int64_t n_tok, int64_t d_model, int64_t vocab, int64_t chunk,
                              double z_coef, double grad_out, lce_tensor *lse_out,
                              lce_tensor *d_hidden, lce_tensor *d_weight,
                              int32_t accumulate_d_weight, lce_tensor *workspace, lce_loss *out,
                              void *stream, lce_timers *timers) {
  int32_t st = lce_dims_check(n_tok, d_model, vocab);
  if (st != LCE_OK) return st;
  st = lce_chunk_check(chunk, vocab);
  if (st != LCE_OK) return st;
  if (!finite_scalar(z_coef) || !finite_scalar(grad_out)) return LCE_NON_FINITE_SCALAR;
  int32_t dt = 0;
  st = check_ce_tensors(hidden, weight, targets, loss_mask, n_tok, d_model, vocab, &dt);
  if (st != LCE_OK) return st;
  if (!lse_out || !d_hidden || !d_weight || !workspace) return LCE_LENGTH_MISMATCH;
  const int32_t acc_dt = dt == LCE_F64 ? LCE_F64 : LCE_F32;
  if (lse_out->dtype != acc_dt || d_weight->dtype != acc_dt || d_hidden->dtype != dt)
    return LCE_DTYPE_MISMATCH;
  if (workspace->dtype != LCE_U8) return LCE_DTYPE_MISMATCH;
  CEPlan p;
  st = plan_ce(n_tok, d_model, vocab, chunk, dt, &p);
  if (st != LCE_OK) return st;
  st = check_ce_lengths(hidden, weight, targets, loss_mask, n_tok, d_model, vocab);
  if (st != LCE_OK) return st;
  if (!has(lse_out) || lse_out->numel < n_tok) return LCE_LENGTH_MISMATCH;
  if (!has(d_hidden) || d_hidden->numel < n_tok * d_model) return LCE_LENGTH_MISMATCH;
  if (!has(d_weight) || d_weight->numel < vocab * d_model) return LCE_LENGTH_MISMATCH;
  if (!has(workspace) || workspace->numel < int64_t(p.f_total) + 256) return LCE_LENGTH_MISMATCH;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *ws = ws_base(workspace);
  const uint8_t *mask = has(loss_mask) ? static_cast<const uint8_t *>(loss_mask->data) : nullptr;
  const int64_t *y = static_cast<const int64_t *>(targets->data);
  const bool acc = accumulate_d_weight != 0;
  (void)hipGetLastError();
  if (dt != LCE_F64) {
    const bool vec = d_model % 8 == 0 && aligned16(hidden->data) && aligned16(weight->data) &&
                     aligned16(d_weight->data);
    float *l = static_cast<float *>(lse_out->data);
    float *dw = static_cast<float *>(d_weight->data);
    const Shard<float> whole;
    // the kept logits' 16-bit rows (stride 2 f_ld) must suit the pipelined core
    const bool single = p.f_ok && UsePipe<TraitsBF16>::ok(vec, d_model, 2 * p.f_ld) &&
                        UsePipe<TraitsBF16>::ok(vec, d_model, p.d_ld);
    if (single) {
      if (dt == LCE_F16)
        forward_backward_single<TraitsF16>(p, hidden->data, weight->data, y, mask, l, z_coef,
                                           grad_out, d_hidden->data, dw, acc, ws, vec, s, timers);
      else
        forward_backward_single<TraitsBF16>(p, hidden->data, weight->data, y, mask, l, z_coef,
                                            grad_out, d_hidden->data, dw, acc, ws, vec, s, timers);
    } else if (dt == LCE_F16) {
      forward_impl<TraitsF16>(p, hidden->data, weight->data, y, mask, l, ws, vec, s, timers, whole);
      backward_impl<TraitsF16>(p, hidden->data, weight->data, y, mask, l, z_coef, grad_out,
                               d_hidden->data, false, dw, acc, ws, vec, s, timers, whole);
    } else {
      forward_impl<TraitsBF16>(p, hidden->data, weight->data, y, mask, l, ws, vec, s, timers,
                               whole);
      backward_impl<TraitsBF16>(p, hidden->data, weight->data, y, mask, l, z_coef, grad_out,
                                d_hidden->data, false, dw, acc, ws, vec, s, timers, whole);
    }
  } else {
    const bool vec = d_model % 2 == 0 && aligned16(hidden->data) && aligned16(weight->data);
    double *l = static_cast<double *>(lse_out->data);
    const Shard<double> whole;
    forward_impl<TraitsF64>(p, hidden->data, weight->data, y, mask, l, ws, vec, s, timers, whole);
    backward_impl<TraitsF64>(p, hidden->data, weight->data, y, mask, l, z_coef, grad_out,
                             d_hidden->data, false, static_cast<double *>(d_weight->data), acc,
                             ws, vec, s, timers, whole);
  }
  if (!out) return enqueued();   // the scalars and the guard's verdict: lce_loss_fetch
  Control hc;
  st = finish(s, reinterpret_cast<Control *>(ws), &hc);
  if (st != LCE_OK) return st;
  fill_loss(hc, out);
  return LCE_OK;
}

}  // namespace

extern "C" {

int32_t lce_forward_backward(const lce_tensor *hidden, const lce_tensor *weight,
                             const lce_tensor *targets, const lce_tensor *loss_mask,
                             int64_t n_tok, int64_t d_model, int64_t vocab, int64_t chunk,
                             double z_coef, double grad_out, lce_tensor *lse_out,
                             lce_tensor *d_hidden, lce_tensor *d_weight,
                             int32_t accumulate_d_weight, lce_tensor *workspace, lce_loss *out,
                             void *stream) {
  return forward_backward_call(hidden, weight, targets, loss_mask, n_tok, d_model, vocab, chunk,
                               z_coef, grad_out, lse_out, d_hidden, d_weight, accumulate_d_weight,
                               workspace, out, stream, nullptr);
}

int32_t lce_forward_backward_timed(const lce_tensor *hidden, const lce_tensor *weight,
                                   const lce_tensor *targets, const lce_tensor *loss_mask,
                                   int64_t n_tok, int64_t d_model, int64_t vocab, int64_t chunk,
                                   double z_coef, double grad_out, lce_tensor *lse_out,
                                   lce_tensor *d_hidden, lce_tensor *d_weight,
                                   int32_t accumulate_d_weight, lce_tensor *workspace,
                                   lce_loss *out, void *stream, lce_timers *timers) {
  return forward_backward_call(hidden, weight, targets, loss_mask, n_tok, d_model, vocab, chunk,
                               z_coef, grad_out, lse_out, d_hidden, d_weight, accumulate_d_weight,
                               workspace, out, stream, timers);
}

}  // extern "C"
