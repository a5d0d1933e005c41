// lce_distill.hip -- logit distillation against a full teacher distribution,
// fused forward + backward, with z-loss over the same student softmax.
//
// Source: "Fuse distillation + z-loss in the triton monolithic path"
// (Fast-LLM pull request 566), sections "What it does" and "Changes": the
// from-distribution kernels return loss, z-loss and the logit gradient; the
// z term adds lse^2 to the forward and 2*grad_z*lse*p to the gradient and
// shares the distillation loss mask and divisor.
//
// One workgroup per CU walks token rows, streaming each row twice (HBM-bound):
//   pass 1 reads student s and teacher u once, keeping online (max, sum exp)
//          for x = s/T and y = u/T plus one objective accumulator tied to one
//          of the two running maxima:
//            0 cross-entropy  A = sum e^(y-my) x      L = lse_x - A/sy
//            1 forward KL     A = sum e^(y-my) (y-x)  L = A/sy + lse_x - lse_y
//            2 reverse KL     A = sum e^(x-mx) (x-y)  L = A/sx + lse_y - lse_x
//   pass 2 re-reads the row and writes grad = (grad_out/C)(dL/dx + 2 z lse_x p)/T
//          with dL/dx = p - q (0, 1) or p (ls - lq - L) (2).
// With one 1024-thread workgroup per CU only ~256 rows are in flight (155 MB
// at a 151936 vocabulary), so the re-read is served by the 256 MB Infinity
// Cache; gradient stores are non-temporal so they do not evict those rows.
// Masked rows only write zeros.  Per-row L and lse_x go to the workspace; a
// fixed-order fp64 reduction forms the means.
//
// Label cross-entropy from materialized logits (the lossk page's
// ce_from_logits reference function on the device, with the loss mask and the
// z term of Fast-LLM 566) runs the same row walk with a one-hot target:
// pass 1 keeps (max, sum exp) of z and reads z[y_t] once, L = lse - z[y_t];
// pass 2, when a gradient is asked for, writes
// (grad_out/C)((1 + 2 z_coef lse) p - onehot(y_t)).  Without a gradient the
// row is read once.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include <climits>
#include <cmath>

#include "lce_internal.h"

namespace lce {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class T> struct IO;
template <> struct IO<uint16_t> {  // bf16 bits
  typedef float C;
  __device__ static inline void load8(const uint16_t *p, float *o) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(v[i] << 16);
      o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ static inline float load1(const uint16_t *p) { return __uint_as_float(uint32_t(*p) << 16); }
  __device__ static inline void unpack8(const u32x4 v, float *o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(v[i] << 16);
      o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ static inline u32x4 pack8(const float *g) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2_t h = {static_cast<__bf16>(g[2 * i]), static_cast<__bf16>(g[2 * i + 1])};
      v[i] = __builtin_bit_cast(uint32_t, h);
    }
    return v;
  }
  // round to nearest even (v_cvt_pk_bf16_f32; NaN stays NaN)
  __device__ static inline uint16_t cvt(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
  }
  __device__ static inline void store8(uint16_t *p, const float *g) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2_t h = {static_cast<__bf16>(g[2 * i]), static_cast<__bf16>(g[2 * i + 1])};
      v[i] = __builtin_bit_cast(uint32_t, h);
    }
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
  }
  __device__ static inline void store1(uint16_t *p, float g) { *p = cvt(g); }
};
template <> struct IO<_Float16> {  // IEEE half; v_cvt_f16_f32 rounds to nearest even
  typedef float C;
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  __device__ static inline void load8(const _Float16 *p, float *o) {
    const h8 v = *reinterpret_cast<const h8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = static_cast<float>(v[i]);
  }
  __device__ static inline float load1(const _Float16 *p) { return static_cast<float>(*p); }
  __device__ static inline void unpack8(const u32x4 v, float *o) {
    const h8 h = __builtin_bit_cast(h8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = static_cast<float>(h[i]);
  }
  __device__ static inline u32x4 pack8(const float *g) {
    h8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = static_cast<_Float16>(g[i]);
    return __builtin_bit_cast(u32x4, v);
  }
  __device__ static inline void store8(_Float16 *p, const float *g) {
    h8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = static_cast<_Float16>(g[i]);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
  }
  __device__ static inline void store1(_Float16 *p, float g) { *p = static_cast<_Float16>(g); }
};
template <> struct IO<float> {
  typedef float C;
  __device__ static inline void load8(const float *p, float *o) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
  __device__ static inline float load1(const float *p) { return *p; }
  __device__ static inline void store8(float *p, const float *g) {
    reinterpret_cast<float4 *>(p)[0] = make_float4(g[0], g[1], g[2], g[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(g[4], g[5], g[6], g[7]);
  }
  __device__ static inline void store1(float *p, float g) { *p = g; }
};
template <> struct IO<double> {
  typedef double C;
  __device__ static inline void load8(const double *p, double *o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double2 a = reinterpret_cast<const double2 *>(p)[i];
      o[2 * i] = a.x;
      o[2 * i + 1] = a.y;
    }
  }
  __device__ static inline double load1(const double *p) { return *p; }
  __device__ static inline void store8(double *p, const double *g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) reinterpret_cast<double2 *>(p)[i] = make_double2(g[2 * i], g[2 * i + 1]);
  }
  __device__ static inline void store1(double *p, double g) { *p = g; }
};

template <class C> __device__ inline C dexp(C x);
template <> __device__ inline float dexp<float>(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
template <> __device__ inline double dexp<double>(double x) { return exp(x); }
template <class C> __device__ inline C dlog(C x);
template <> __device__ inline float dlog<float>(float x) { return logf(x); }
template <> __device__ inline double dlog<double>(double x) { return log(x); }

// Running (max, sum of exp(v - max)) with a weighted sum tied to the same max.
template <class C>
struct Online {
  C m, s, a;
  __device__ inline void init() { m = -INFINITY; s = 0; a = 0; }
  __device__ inline void merge(const Online &o) {
    const C M = m > o.m ? m : o.m;
    if (M == -INFINITY) return;
    const C f1 = dexp<C>(m - M), f2 = dexp<C>(o.m - M);
    s = s * f1 + o.s * f2;
    a = a * f1 + o.a * f2;
    m = M;
  }
};

template <class C>
__device__ inline Online<C> shfl_xor_online(const Online<C> &v, int o) {
  Online<C> r;
  r.m = __shfl_xor(v.m, o);
  r.s = __shfl_xor(v.s, o);
  r.a = __shfl_xor(v.a, o);
  return r;
}

constexpr int kBlock = 1024;
constexpr int64_t kRowGrid = 256;   // workgroups: one per compute unit
// Row-resident kernels: 512 threads (8 waves of up to 256 registers) keep
// kResidentChunks 16-byte chunks each, rows up to 8 * 38 * 512 = 155648 values.
constexpr int kResBlock = 512;
constexpr int kResidentChunks = 38;

// f(std::integral_constant<int, I>) for I = B .. E-1, in order.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Reduce within the block (NT threads) in a fixed order; thread 0 gets the
// result.
template <class C, int NT = kBlock>
__device__ inline void block_merge(Online<C> &v, Online<C> *sh) {
  for (int o = 1; o < 64; o <<= 1) {
    Online<C> w = shfl_xor_online(v, o);
    v.merge(w);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < NT / 64; ++w) v.merge(sh[w]);
}

template <class T, int OBJ, bool VEC>
__device__ __forceinline__ void distill_row(const T *S, const T *U, const uint8_t *mask, int64_t t,
                                            int64_t V, double inv_T, double z_coef,
                                            double grad_out, const Control *ctl, T *grad,
                                            double *row_out);

// The 16-byte chunks i = tid, tid + NT, ... (below nvec) of one row (b ==
// nullptr) or of two rows at once, with kStreamBatch chunks per row and
// thread in flight before any is consumed (a load per thread and row at a
// time leaves the memory system too few bytes in flight to reach its
// bandwidth); f(i, chunk of a, chunk of b) runs for ascending i.
constexpr int kStreamBatch = 4;
template <int NT = kBlock, class T, class F>
__device__ __forceinline__ void stream_chunks(const T *a, const T *b, int64_t nvec, int tid,
                                              F &&f) {
  constexpr int B = kStreamBatch;
  const int64_t step = int64_t(B) * NT;
  const int64_t n_batches = nvec > tid ? (nvec - tid + step - 1) / step : 0;
  for (int64_t bi = 0; bi < n_batches; ++bi) {
    const int64_t i0 = tid + bi * step;
    u32x4 va[B], vb[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int64_t i = i0 + int64_t(k) * NT;
      va[k] = vb[k] = u32x4{0u, 0u, 0u, 0u};
      if (i < nvec) {
        va[k] = *reinterpret_cast<const u32x4 *>(a + i * 8);
        if (b) vb[k] = *reinterpret_cast<const u32x4 *>(b + i * 8);
      }
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int64_t i = i0 + int64_t(k) * NT;
      if (i < nvec) f(i, va[k], vb[k]);
    }
  }
}

template <class T, int OBJ>
__device__ __forceinline__ void distill_row16(const T *S, const T *U, const uint8_t *mask,
                                              int64_t t, int64_t V, double inv_T, double z_coef,
                                              double grad_out, const Control *ctl, T *grad,
                                              double *row_out);

template <class T, int OBJ, bool VEC>
__global__ void __launch_bounds__(kBlock)
distill_row_kernel(const T *S, const T *U, const uint8_t *mask, int64_t n, int64_t V,
                   double inv_T, double z_coef, double grad_out, const Control *ctl, T *grad,
                   double *row_out) {
  for (int64_t t = blockIdx.x; t < n; t += gridDim.x) {
    if constexpr (sizeof(T) == 2 && VEC)
      distill_row16<T, OBJ>(S, U, mask, t, V, inv_T, z_coef, grad_out, ctl, grad, row_out);
    else
      distill_row<T, OBJ, VEC>(S, U, mask, t, V, inv_T, z_coef, grad_out, ctl, grad, row_out);
  }
}

// 16-bit rows, vocabulary a multiple of 8 and 16-byte aligned rows: the same
// statistics, objective and gradient as distill_row with the arithmetic
// arranged to issue fewer vector instructions (the row is streamed twice, so
// the work per element bounds the kernel as much as the memory does):
//   * running maxima are kept in raw input units (T > 0 preserves the order),
//     so each exponential is one fma and one exp2 with c = log2(e) / T folded
//     in: e^(x - m_x) = 2^(s c - m_s c);
//   * the maximum is updated, and the sums rescaled, once per batch of
//     kStreamBatch chunks rather than once per chunk;
//   * the gradient's scale, sign and z term fold into the exponent:
//     objectives 0 and 1: g = kA 2^(s c + A) - kB 2^(u c + B) with
//     A = log2|scale (1 + zc)| - lse_x log2(e), B = log2|scale| - lse_y log2(e);
//     objective 2: g = kB 2^(s c + B') ((s - u) / T + K), B' = log2|scale| -
//     lse_x log2(e), K = lse_y - lse_x - L + zc.
struct OnlineRaw {
  float m, s, a;   // raw-unit max, sum of 2^((v - m) c), weighted sum on the same max
};

// max(a, b, c) in one instruction.  (fmaxf on values loaded from memory costs
// an extra canonicalizing instruction per value; these are finite logits, and
// a NaN among them makes the row's statistics NaN either way.)
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ inline void raw_merge(OnlineRaw &v, const OnlineRaw &o, float c) {
  const float M = fmaxf(v.m, o.m);
  if (M == -INFINITY) return;
  const float f1 = __builtin_amdgcn_exp2f((v.m - M) * c), f2 = __builtin_amdgcn_exp2f((o.m - M) * c);
  v.s = v.s * f1 + o.s * f2;
  v.a = v.a * f1 + o.a * f2;
  v.m = M;
}

// Fixed-order block reduction of raw-unit statistics (NT threads); thread 0
// gets the result.
template <int NT = kBlock>
__device__ inline void block_merge_raw(OnlineRaw &v, OnlineRaw *sh, float c) {
  for (int o = 1; o < 64; o <<= 1) {
    OnlineRaw w;
    w.m = __shfl_xor(v.m, o);
    w.s = __shfl_xor(v.s, o);
    w.a = __shfl_xor(v.a, o);
    raw_merge(v, w, c);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < NT / 64; ++w) raw_merge(v, sh[w], c);
}

template <class T, int OBJ>
__device__ __forceinline__ void distill_row16(const T *S, const T *U, const uint8_t *mask,
                                              int64_t t, int64_t V, double inv_T, double z_coef,
                                              double grad_out, const Control *ctl, T *grad,
                                              double *row_out) {
  constexpr int B = kStreamBatch;
  const float L2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
  const T *s_row = S + t * V;
  const T *u_row = U + t * V;
  T *g_row = grad + t * V;
  const int tid = threadIdx.x;
  const int64_t nvec = V / 8;
  const float iT = float(inv_T);
  const float c = float(inv_T * 1.4426950408889634);

  if (mask && !mask[t]) {
    const float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t i = tid; i < nvec; i += kBlock) IO<T>::store8(g_row + i * 8, z);
    if (tid == 0) { row_out[2 * t] = 0.0; row_out[2 * t + 1] = 0.0; }
    return;
  }
  __syncthreads();   // the previous row's statistics are no longer read

  // Pass 1: batches of B chunks per thread, loads first.
  OnlineRaw fx{-INFINITY, 0.f, 0.f}, fy{-INFINITY, 0.f, 0.f};
  for (int64_t i0 = tid; i0 < nvec; i0 += int64_t(B) * kBlock) {
    u32x4 vs[B], vu[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int64_t i = i0 + int64_t(k) * kBlock;
      vs[k] = vu[k] = u32x4{0u, 0u, 0u, 0u};
      if (i < nvec) {
        vs[k] = *reinterpret_cast<const u32x4 *>(s_row + i * 8);
        vu[k] = *reinterpret_cast<const u32x4 *>(u_row + i * 8);
      }
    }
    float xs[B][8], ys[B][8];
    float bmx = fx.m, bmy = fy.m;   // running max, then this batch's values
#pragma unroll
    for (int k = 0; k < B; ++k) {
      IO<T>::unpack8(vs[k], xs[k]);
      IO<T>::unpack8(vu[k], ys[k]);
      if (i0 + int64_t(k) * kBlock < nvec) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          bmx = max3_raw(bmx, xs[k][j], xs[k][j + 1]);
          bmy = max3_raw(bmy, ys[k][j], ys[k][j + 1]);
        }
      }
    }
    const float nmx = bmx, nmy = bmy;
    const float rx = __builtin_amdgcn_exp2f((fx.m - nmx) * c);
    const float ry = __builtin_amdgcn_exp2f((fy.m - nmy) * c);
    fx.s *= rx; fx.a *= rx; fx.m = nmx;
    fy.s *= ry; fy.a *= ry; fy.m = nmy;
    const float bx = -nmx * c, by = -nmy * c;
#pragma unroll
    for (int k = 0; k < B; ++k) {
      if (i0 + int64_t(k) * kBlock >= nvec) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ex = __builtin_amdgcn_exp2f(fmaf(xs[k][j], c, bx));
        const float ey = __builtin_amdgcn_exp2f(fmaf(ys[k][j], c, by));
        fx.s += ex;
        fy.s += ey;
        if constexpr (OBJ == 0) fy.a = fmaf(ey, xs[k][j], fy.a);
        else if constexpr (OBJ == 1) fy.a = fmaf(ey, ys[k][j] - xs[k][j], fy.a);
        else fx.a = fmaf(ex, xs[k][j] - ys[k][j], fx.a);
      }
    }
  }

  __shared__ OnlineRaw sh_x[kBlock / 64], sh_y[kBlock / 64];
  __shared__ float sh_stats[4];
  block_merge_raw(fx, sh_x, c);
  block_merge_raw(fy, sh_y, c);
  if (tid == 0) {
    // natural-log statistics of x = s / T and y = u / T
    const float lse_x = (fx.m * c + __builtin_amdgcn_logf(fx.s)) * LN2;
    const float lse_y = (fy.m * c + __builtin_amdgcn_logf(fy.s)) * LN2;
    float L;
    if constexpr (OBJ == 0) L = lse_x - iT * fy.a / fy.s;
    else if constexpr (OBJ == 1) L = iT * fy.a / fy.s + lse_x - lse_y;
    else L = iT * fx.a / fx.s + lse_y - lse_x;
    sh_stats[0] = lse_x;
    sh_stats[1] = lse_y;
    sh_stats[2] = L;
    row_out[2 * t] = double(L);
    row_out[2 * t + 1] = double(lse_x);
  }
  __syncthreads();
  const float lse_x = sh_stats[0], lse_y = sh_stats[1], L = sh_stats[2];
  const int64_t cnt = ctl->count;
  const float scale = cnt ? float(grad_out / double(cnt) * inv_T) : 0.f;
  const float zc = float(2.0 * z_coef) * lse_x;
  // exponent offsets and signs of the gradient's terms (log2 of 0 is -inf,
  // which makes the term 0)
  const float aA = scale * (1.f + zc);
  const float offA = __builtin_amdgcn_logf(fabsf(aA)) - lse_x * L2E;
  const float kA = aA < 0.f ? -1.f : 1.f;
  const float offB = __builtin_amdgcn_logf(fabsf(scale)) - (OBJ == 2 ? lse_x : lse_y) * L2E;
  const float kB = scale < 0.f ? -1.f : 1.f;
  const float K = lse_y - lse_x - L + zc;

  // Pass 2: gradient.  With a positive scale and 1 + zc > 0 (the usual case)
  // the two terms combine with one subtraction.
  auto pass2 = [&](auto plain_tag) {
    constexpr bool PLAIN = decltype(plain_tag)::value;
    stream_chunks(s_row, u_row, nvec, tid, [&](int64_t i, u32x4 cs, u32x4 cu) {
      float xs[8], ys[8], gs[8];
      IO<T>::unpack8(cs, xs);
      IO<T>::unpack8(cu, ys);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (OBJ == 2) {
          const float p = __builtin_amdgcn_exp2f(fmaf(xs[j], c, offB));
          const float f = fmaf(xs[j] - ys[j], iT, K);
          gs[j] = PLAIN ? p * f : kB * p * f;
        } else {
          const float pa = __builtin_amdgcn_exp2f(fmaf(xs[j], c, offA));
          const float qb = __builtin_amdgcn_exp2f(fmaf(ys[j], c, offB));
          gs[j] = PLAIN ? pa - qb : fmaf(kA, pa, -kB * qb);
        }
      }
      IO<T>::store8(g_row + i * 8, gs);
    });
  };
  if (kB > 0.f && (OBJ == 2 || kA > 0.f)) pass2(std::true_type{});
  else pass2(std::false_type{});
}

// 16-bit rows of at most 8 * CPT * kResBlock values, vocabulary a multiple
// of 8, 16-byte aligned rows: the same statistics, objective and gradient as
// distill_row16, with the student row read from memory once.  Each thread
// keeps its CPT 16-byte chunks of the student row in registers; the teacher
// row streams through a ring of kDRing chunk-steps in LDS that direct
// buffer-to-LDS loads keep full (no registers held by loads in flight), once
// for the statistics and once more for the gradient.  512 threads, one
// workgroup per CU.  Every load and store is issued for every chunk index,
// with indices past the row dropped by the buffer's range check, so that
// each wave's count of memory operations in flight is known at compile time
// and the ring's waits can name it.
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kDRing = 16;   // chunk-steps in flight (16 x 8 KB of LDS)

// Vector memory operations issued after the ring load of step q and before
// the wait at the start of step q (steps [0, 2 CPT): the statistics pass,
// then the gradient pass, which stores one chunk per step).  The ring loads
// of steps [0, kDRing) go first; step s then waits, reads its chunk, loads
// step s + kDRing (if any) and, in the gradient pass, stores its chunk.
template <int CPT>
constexpr int ring_ops_after(int q) {
  int n = 0;
  bool seen = false;
  for (int r = 0; r < kDRing && r < 2 * CPT; ++r) {
    if (seen) ++n;
    if (r == q) seen = true;
  }
  for (int st = 0; st < q; ++st) {
    if (st + kDRing < 2 * CPT) {
      if (seen) ++n;
      if (st + kDRing == q) seen = true;
    }
    if (st >= CPT && seen) ++n;
  }
  return n;
}

template <class T, int OBJ, int CPT>
__device__ __forceinline__ void distill_row_resident(const T *S, const T *U, const uint8_t *mask,
                                                     int64_t t, int64_t V, double inv_T,
                                                     double z_coef, double grad_out,
                                                     const Control *ctl, T *grad,
                                                     double *row_out, char *ring) {
  const float L2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
  const T *s_row = S + t * V;
  const T *u_row = U + t * V;
  T *g_row = grad + t * V;
  const int tid = threadIdx.x;
  const int64_t nvec = V / 8;
  const float iT = float(inv_T);
  const float c = float(inv_T * 1.4426950408889634);
  const uint32_t voff = uint32_t(tid) * 16u;
  const int rbytes = int(V * int64_t(sizeof(T)));
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(g_row, 0, rbytes, 0x00020000);
  if (mask && !mask[t]) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(zero, ro, voff, i * kResBlock * 16, 2);
    if (tid == 0) { row_out[2 * t] = 0.0; row_out[2 * t + 1] = 0.0; }
    return;
  }
  __syncthreads();   // the previous row's statistics are no longer read
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(s_row), 0, rbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ru =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(u_row), 0, rbytes, 0x00020000);
  u32x4 xr[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    xr[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, i * kResBlock * 16, 0);
  // this wave's 1 KB of every ring slot; lane l's chunk lands at + 16 l
  char *const wring = ring + (tid >> 6) * 1024;
  auto ring_load = [&](int q) {   // step q: teacher chunk q mod CPT
    const int i = q % CPT;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (lds_void_t *)(wring + (q % kDRing) * (kResBlock * 16)),
                                             16, voff + uint32_t(i * kResBlock * 16), 0, 0, 0);
  };
#pragma unroll
  for (int q = 0; q < kDRing && q < 2 * CPT; ++q) ring_load(q);
  auto ring_wait_read = [&](auto q_tag) {
    constexpr int q = decltype(q_tag)::value;
    constexpr int N = ring_ops_after<CPT>(q);
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    u32x4 u = *reinterpret_cast<const u32x4 *>(wring + (q % kDRing) * (kResBlock * 16) +
                                               (tid & 63) * 16);
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(u) : : "memory");
    if constexpr (q + kDRing < 2 * CPT) ring_load(q + kDRing);
    // no later memory operation (this step's store) moves above this load:
    // the counts of ring_ops_after rely on the issue order
    asm volatile("" ::: "memory");
    return u;
  };

  // Statistics pass: the raw running maxima are updated, and the sums
  // rescaled, once per chunk; even and odd chunks add into separate partial
  // sums (independent add chains).
  float mx = -INFINITY, my = -INFINITY;
  float sx[2] = {0.f, 0.f}, sy[2] = {0.f, 0.f}, sa[2] = {0.f, 0.f};
  static_for<0, CPT>([&](auto q_tag) {
    constexpr int i = decltype(q_tag)::value;
    constexpr int k = i & 1;
    const u32x4 uu = ring_wait_read(q_tag);
    do {
      if (tid + int64_t(i) * kResBlock >= nvec) break;
      float xs[8], ys[8];
      IO<T>::unpack8(xr[i], xs);
      IO<T>::unpack8(uu, ys);
      float bmx = mx, bmy = my;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        bmx = max3_raw(bmx, xs[j], xs[j + 1]);
        bmy = max3_raw(bmy, ys[j], ys[j + 1]);
      }
      if (bmx == -INFINITY || bmy == -INFINITY) break;
      const float rx = __builtin_amdgcn_exp2f((mx - bmx) * c);
      const float ry = __builtin_amdgcn_exp2f((my - bmy) * c);
      const float ra = OBJ == 2 ? rx : ry;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        sx[h] *= rx;
        sy[h] *= ry;
        sa[h] *= ra;
      }
      mx = bmx;
      my = bmy;
      const float bx = -bmx * c, by = -bmy * c;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ex = __builtin_amdgcn_exp2f(fmaf(xs[j], c, bx));
        const float ey = __builtin_amdgcn_exp2f(fmaf(ys[j], c, by));
        sx[k] += ex;
        sy[k] += ey;
        if constexpr (OBJ == 0) sa[k] = fmaf(ey, xs[j], sa[k]);
        else if constexpr (OBJ == 1) sa[k] = fmaf(ey, ys[j] - xs[j], sa[k]);
        else sa[k] = fmaf(ex, xs[j] - ys[j], sa[k]);
      }
    } while (false);
  });
  OnlineRaw fx{mx, sx[0] + sx[1], 0.f}, fy{my, sy[0] + sy[1], 0.f};
  (OBJ == 2 ? fx : fy).a = sa[0] + sa[1];
  __shared__ OnlineRaw sh_x[kResBlock / 64], sh_y[kResBlock / 64];
  __shared__ float sh_stats[3];
  block_merge_raw<kResBlock>(fx, sh_x, c);
  block_merge_raw<kResBlock>(fy, sh_y, c);
  if (tid == 0) {
    const float lse_x = (fx.m * c + __builtin_amdgcn_logf(fx.s)) * LN2;
    const float lse_y = (fy.m * c + __builtin_amdgcn_logf(fy.s)) * LN2;
    float L;
    if constexpr (OBJ == 0) L = lse_x - iT * fy.a / fy.s;
    else if constexpr (OBJ == 1) L = iT * fy.a / fy.s + lse_x - lse_y;
    else L = iT * fx.a / fx.s + lse_y - lse_x;
    sh_stats[0] = lse_x;
    sh_stats[1] = lse_y;
    sh_stats[2] = L;
    row_out[2 * t] = double(L);
    row_out[2 * t + 1] = double(lse_x);
  }
  __syncthreads();
  const float lse_x = sh_stats[0], lse_y = sh_stats[1], L = sh_stats[2];
  const int64_t cnt = ctl->count;
  const float scale = cnt ? float(grad_out / double(cnt) * inv_T) : 0.f;
  const float zc = float(2.0 * z_coef) * lse_x;
  const float aA = scale * (1.f + zc);
  const float offA = __builtin_amdgcn_logf(fabsf(aA)) - lse_x * L2E;
  const float kA = aA < 0.f ? -1.f : 1.f;
  const float offB = __builtin_amdgcn_logf(fabsf(scale)) - (OBJ == 2 ? lse_x : lse_y) * L2E;
  const float kB = scale < 0.f ? -1.f : 1.f;
  const float K = lse_y - lse_x - L + zc;
#pragma unroll
  for (int i = 0; i < CPT; ++i) asm volatile("" : "+v"(xr[i]));

  // Gradient pass (the same exponent folds as distill_row16).
  auto pass2 = [&](auto plain_tag) {
    constexpr bool PLAIN = decltype(plain_tag)::value;
    static_for<CPT, 2 * CPT>([&](auto q_tag) {
      constexpr int i = decltype(q_tag)::value - CPT;
      const u32x4 uu = ring_wait_read(q_tag);
      float xs[8], ys[8], gs[8];
      IO<T>::unpack8(xr[i], xs);
      IO<T>::unpack8(uu, ys);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (OBJ == 2) {
          const float p = __builtin_amdgcn_exp2f(fmaf(xs[j], c, offB));
          const float f = fmaf(xs[j] - ys[j], iT, K);
          gs[j] = PLAIN ? p * f : kB * p * f;
        } else {
          const float pa = __builtin_amdgcn_exp2f(fmaf(xs[j], c, offA));
          const float qb = __builtin_amdgcn_exp2f(fmaf(ys[j], c, offB));
          gs[j] = PLAIN ? pa - qb : fmaf(kA, pa, -kB * qb);
        }
      }
      __builtin_amdgcn_raw_buffer_store_b128(IO<T>::pack8(gs), ro, voff, i * kResBlock * 16, 2);
    });
  };
  if (kB > 0.f && (OBJ == 2 || kA > 0.f)) pass2(std::true_type{});
  else pass2(std::false_type{});
}

template <class T, int OBJ, int CPT>
__global__ void __launch_bounds__(kResBlock)
distill_resident_kernel(const T *S, const T *U, const uint8_t *mask, int64_t n, int64_t V,
                        double inv_T, double z_coef, double grad_out, const Control *ctl, T *grad,
                        double *row_out) {
  __shared__ __attribute__((aligned(1024))) char ring[kDRing * kResBlock * 16];
  for (int64_t t = blockIdx.x; t < n; t += gridDim.x)
    distill_row_resident<T, OBJ, CPT>(S, U, mask, t, V, inv_T, z_coef, grad_out, ctl, grad,
                                      row_out, ring);
}

template <class T, int OBJ, bool VEC>
__device__ __forceinline__ void distill_row(const T *S, const T *U, const uint8_t *mask, int64_t t,
                                            int64_t V, double inv_T, double z_coef,
                                            double grad_out, const Control *ctl, T *grad,
                                            double *row_out) {
  typedef typename IO<T>::C C;
  const T *s_row = S + t * V;
  const T *u_row = U + t * V;
  T *g_row = grad + t * V;
  const C iT = C(inv_T);
  const int tid = threadIdx.x;
  const int64_t nvec = VEC ? V / 8 : 0;
  const int64_t tail0 = nvec * 8;

  if (mask && !mask[t]) {
    const C z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t i = tid; i < nvec; i += kBlock) IO<T>::store8(g_row + i * 8, z);
    for (int64_t v = tail0 + tid; v < V; v += kBlock) IO<T>::store1(g_row + v, C(0));
    if (tid == 0) { row_out[2 * t] = 0.0; row_out[2 * t + 1] = 0.0; }
    return;
  }
  __syncthreads();   // the previous row's statistics are no longer read

  // Pass 1: online statistics.  fx tracks x; fy tracks y.  The objective
  // accumulator rides on fy (objectives 0, 1) or fx (objective 2).
  Online<C> fx, fy;
  fx.init();
  fy.init();
  auto consume = [&](const C *xs, const C *ys, int cnt) {
    C lmx = -INFINITY, lmy = -INFINITY;
    for (int i = 0; i < cnt; ++i) {
      lmx = xs[i] > lmx ? xs[i] : lmx;
      lmy = ys[i] > lmy ? ys[i] : lmy;
    }
    const C nmx = fx.m > lmx ? fx.m : lmx;
    const C nmy = fy.m > lmy ? fy.m : lmy;
    const C rx = dexp<C>(fx.m - nmx), ry = dexp<C>(fy.m - nmy);
    fx.s *= rx; fx.a *= rx; fx.m = nmx;
    fy.s *= ry; fy.a *= ry; fy.m = nmy;
    for (int i = 0; i < cnt; ++i) {
      const C ex = dexp<C>(xs[i] - nmx), ey = dexp<C>(ys[i] - nmy);
      fx.s += ex;
      fy.s += ey;
      if (OBJ == 0) fy.a += ey * xs[i];
      else if (OBJ == 1) fy.a += ey * (ys[i] - xs[i]);
      else fx.a += ex * (xs[i] - ys[i]);
    }
  };
  if constexpr (sizeof(T) == 2) {
    stream_chunks(s_row, u_row, nvec, tid, [&](int64_t, u32x4 cs, u32x4 cu) {
      C xs[8], ys[8];
      IO<T>::unpack8(cs, xs);
      IO<T>::unpack8(cu, ys);
#pragma unroll
      for (int j = 0; j < 8; ++j) { xs[j] *= iT; ys[j] *= iT; }
      consume(xs, ys, 8);
    });
  } else {
    for (int64_t i = tid; i < nvec; i += kBlock) {
      C xs[8], ys[8];
      IO<T>::load8(s_row + i * 8, xs);
      IO<T>::load8(u_row + i * 8, ys);
#pragma unroll
      for (int j = 0; j < 8; ++j) { xs[j] *= iT; ys[j] *= iT; }
      consume(xs, ys, 8);
    }
  }
  for (int64_t v = tail0 + tid; v < V; v += kBlock) {
    C xs[1] = {IO<T>::load1(s_row + v) * iT}, ys[1] = {IO<T>::load1(u_row + v) * iT};
    consume(xs, ys, 1);
  }

  __shared__ Online<C> sh_x[kBlock / 64], sh_y[kBlock / 64];
  __shared__ C sh_stats[3];
  block_merge(fx, sh_x);
  block_merge(fy, sh_y);
  if (tid == 0) {
    const C lse_x = fx.m + dlog<C>(fx.s);
    const C lse_y = fy.m + dlog<C>(fy.s);
    C L;
    if (OBJ == 0) L = lse_x - fy.a / fy.s;
    else if (OBJ == 1) L = fy.a / fy.s + lse_x - lse_y;
    else L = fx.a / fx.s + lse_y - lse_x;
    sh_stats[0] = lse_x;
    sh_stats[1] = lse_y;
    sh_stats[2] = L;
    row_out[2 * t] = double(L);
    row_out[2 * t + 1] = double(lse_x);
  }
  __syncthreads();
  const C lse_x = sh_stats[0], lse_y = sh_stats[1], L = sh_stats[2];
  const int64_t cnt = ctl->count;
  const C scale = cnt ? C(grad_out / double(cnt) * inv_T) : C(0);
  const C zc = C(2.0 * z_coef) * lse_x;

  // Pass 2: gradient.
  auto grad_of = [&](C x, C y) -> C {
    const C ls = x - lse_x;
    const C p = dexp<C>(ls);
    C d;
    if (OBJ == 2) d = p * (ls - (y - lse_y) - L);
    else d = p - dexp<C>(y - lse_y);
    return scale * (d + zc * p);
  };
  if constexpr (sizeof(T) == 2) {
    stream_chunks(s_row, u_row, nvec, tid, [&](int64_t i, u32x4 cs, u32x4 cu) {
      C xs[8], ys[8], gs[8];
      IO<T>::unpack8(cs, xs);
      IO<T>::unpack8(cu, ys);
#pragma unroll
      for (int j = 0; j < 8; ++j) gs[j] = grad_of(xs[j] * iT, ys[j] * iT);
      IO<T>::store8(g_row + i * 8, gs);
    });
  } else {
    for (int64_t i = tid; i < nvec; i += kBlock) {
      C xs[8], ys[8], gs[8];
      IO<T>::load8(s_row + i * 8, xs);
      IO<T>::load8(u_row + i * 8, ys);
#pragma unroll
      for (int j = 0; j < 8; ++j) gs[j] = grad_of(xs[j] * iT, ys[j] * iT);
      IO<T>::store8(g_row + i * 8, gs);
    }
  }
  for (int64_t v = tail0 + tid; v < V; v += kBlock)
    IO<T>::store1(g_row + v, grad_of(IO<T>::load1(s_row + v) * iT, IO<T>::load1(u_row + v) * iT));
}

template <class T, bool VEC, bool GRAD, int NT>
__device__ __forceinline__ void label_row(const T *Z, const int64_t *y, const uint8_t *mask,
                                          int64_t t, int64_t V, double z_coef, double grad_out,
                                          const Control *ctl, T *grad, double *row_out) {
  typedef typename IO<T>::C C;
  const T *z_row = Z + t * V;
  const int tid = threadIdx.x;
  const int64_t nvec = VEC ? V / 8 : 0;
  const int64_t tail0 = nvec * 8;

  if (mask && !mask[t]) {
    if constexpr (GRAD) {
      T *g_row = grad + t * V;
      const C z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int64_t i = tid; i < nvec; i += NT) IO<T>::store8(g_row + i * 8, z);
      for (int64_t v = tail0 + tid; v < V; v += NT) IO<T>::store1(g_row + v, C(0));
    }
    if (tid == 0) { row_out[2 * t] = 0.0; row_out[2 * t + 1] = 0.0; }
    return;
  }
  __syncthreads();   // the previous row's statistics are no longer read

  Online<C> f;
  f.init();
  auto consume = [&](const C *xs, int cnt) {
    C lm = -INFINITY;
    for (int i = 0; i < cnt; ++i) lm = xs[i] > lm ? xs[i] : lm;
    const C nm = f.m > lm ? f.m : lm;
    f.s *= dexp<C>(f.m - nm);
    f.m = nm;
    for (int i = 0; i < cnt; ++i) f.s += dexp<C>(xs[i] - nm);
  };
  if constexpr (sizeof(T) == 2) {
    stream_chunks<NT>(z_row, static_cast<const T *>(nullptr), nvec, tid,
                  [&](int64_t, u32x4 cz, u32x4) {
                    C xs[8];
                    IO<T>::unpack8(cz, xs);
                    consume(xs, 8);
                  });
  } else {
    for (int64_t i = tid; i < nvec; i += NT) {
      C xs[8];
      IO<T>::load8(z_row + i * 8, xs);
      consume(xs, 8);
    }
  }
  for (int64_t v = tail0 + tid; v < V; v += NT) {
    const C xs[1] = {IO<T>::load1(z_row + v)};
    consume(xs, 1);
  }
  __shared__ Online<C> sh_f[NT / 64];
  __shared__ C sh_lse;
  block_merge<C, NT>(f, sh_f);
  const int64_t yt = y[t];
  if (tid == 0) {
    const C lse = f.m + dlog<C>(f.s);
    sh_lse = lse;
    row_out[2 * t] = double(lse - IO<T>::load1(z_row + yt));
    row_out[2 * t + 1] = double(lse);
  }
  if constexpr (GRAD) {
    __syncthreads();
    T *g_row = grad + t * V;
    const C lse = sh_lse;
    const int64_t cnt = ctl->count;
    const C g = cnt ? C(grad_out / double(cnt)) : C(0);
    const C a = g * (C(1) + C(2.0 * z_coef) * lse);
    auto grad8 = [&](int64_t i, const C *xs) {
      C gs[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) gs[j] = a * dexp<C>(xs[j] - lse) - (i * 8 + j == yt ? g : C(0));
      IO<T>::store8(g_row + i * 8, gs);
    };
    if constexpr (sizeof(T) == 2) {
      stream_chunks<NT>(z_row, static_cast<const T *>(nullptr), nvec, tid,
                          [&](int64_t i, u32x4 cz, u32x4) {
                            C xs[8];
                            IO<T>::unpack8(cz, xs);
                            grad8(i, xs);
                          });
    } else {
      for (int64_t i = tid; i < nvec; i += NT) {
        C xs[8];
        IO<T>::load8(z_row + i * 8, xs);
        grad8(i, xs);
      }
    }
    for (int64_t v = tail0 + tid; v < V; v += NT)
      IO<T>::store1(g_row + v, a * dexp<C>(IO<T>::load1(z_row + v) - lse) - (v == yt ? g : C(0)));
  }
}

// 16-bit logits with the gradient, rows of at most 8 * CPT * kResBlock values:
// each thread keeps its CPT 16-byte chunks of the row in registers, so the row
// is read from memory once (pass 2 computes from the registers).  512 threads,
// one workgroup per CU: 8 waves of up to 256 registers each.
template <class T, int CPT>
__device__ __forceinline__ void label_row_resident(const T *Z, const int64_t *y,
                                                   const uint8_t *mask, int64_t t, int64_t V,
                                                   double z_coef, double grad_out,
                                                   const Control *ctl, T *grad, double *row_out) {
  const T *z_row = Z + t * V;
  T *g_row = grad + t * V;
  const int tid = threadIdx.x;
  const int64_t nvec = V / 8;
  // Buffer accesses: one lane offset, the chunk index in the scalar offset;
  // every access is predicated on its chunk lying inside the row.
  const uint32_t voff = uint32_t(tid) * 16u;
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(g_row, 0, int(V * int64_t(sizeof(T))), 0x00020000);
  if (mask && !mask[t]) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (tid + int64_t(i) * kResBlock < nvec)
        __builtin_amdgcn_raw_buffer_store_b128(zero, ro, voff, i * kResBlock * 16, 2);
    if (tid == 0) { row_out[2 * t] = 0.0; row_out[2 * t + 1] = 0.0; }
    return;
  }
  __syncthreads();   // the previous row's statistics are no longer read
  const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T *>(z_row), 0, int(V * int64_t(sizeof(T))), 0x00020000);
  u32x4 xr[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    if (tid + int64_t(i) * kResBlock < nvec)
      xr[i] = __builtin_amdgcn_raw_buffer_load_b128(ri, voff, i * kResBlock * 16, 0);
  // Pass 1 from the registers, in batches of four chunks: the raw running
  // maximum is updated and the sums rescaled once per batch, each chunk of a
  // batch adds into its own partial sum (independent add chains), and every
  // exponential is one fma and one exp2 with log2(e) folded in.
  const float L2E = 1.4426950408889634f;
  constexpr int BB = 4;
  float m = -INFINITY, ps[BB] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i0 = 0; i0 < CPT; i0 += BB) {
    float xs[BB][8];
    float bm = m;
#pragma unroll
    for (int k = 0; k < BB; ++k) {
      if (i0 + k >= CPT) continue;
      IO<T>::unpack8(xr[i0 + k], xs[k]);
      if (tid + int64_t(i0 + k) * kResBlock < nvec) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) bm = max3_raw(bm, xs[k][j], xs[k][j + 1]);
      }
    }
    if (bm == -INFINITY) continue;   // nothing but -inf so far
    const float r = __builtin_amdgcn_exp2f((m - bm) * L2E);
#pragma unroll
    for (int k = 0; k < BB; ++k) ps[k] *= r;
    m = bm;
    const float b = -bm * L2E;
#pragma unroll
    for (int k = 0; k < BB; ++k) {
      if (i0 + k >= CPT || tid + int64_t(i0 + k) * kResBlock >= nvec) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) ps[k] += __builtin_amdgcn_exp2f(fmaf(xs[k][j], L2E, b));
    }
  }
  Online<float> f;
  f.m = m;
  f.s = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  f.a = 0.f;
  __shared__ Online<float> sh_f[kResBlock / 64];
  __shared__ float sh_lse;
  block_merge<float, kResBlock>(f, sh_f);
  const int64_t yt = y[t];
  if (tid == 0) {
    const float lse = f.m + dlog<float>(f.s);
    sh_lse = lse;
    row_out[2 * t] = double(lse - IO<T>::load1(z_row + yt));
    row_out[2 * t + 1] = double(lse);
  }
  __syncthreads();
  const float lse = sh_lse;
  const int64_t cnt = ctl->count;
  const float g = cnt ? float(grad_out / double(cnt)) : 0.f;
  const float a = g * (1.f + float(2.0 * z_coef) * lse);
  // a exp(x - lse) = sign(a) 2^(x log2(e) + c2), c2 = log2|a| - lse log2(e)
  // (a = 0 gives exp2(-inf) = 0)
  const float c2 = __builtin_amdgcn_logf(fabsf(a)) - lse * L2E;
  const bool neg = a < 0.f;
  // the target element: chunk it of this thread (-1: another thread's), and
  // g at its place within the chunk
  const int64_t ty = yt - int64_t(tid) * 8;
  const int64_t span = int64_t(kResBlock) * 8;
  const int it = (ty >= 0 && ty % span < 8) ? int(ty / span) : -1;
  float gp[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) gp[j] = (it >= 0 && ty % span == j) ? g : 0.f;
  // Pass 2 unpacks the packed chunks again: holding pass 1's floats (8 per
  // chunk) across the reduction would not fit the registers.
#pragma unroll
  for (int i = 0; i < CPT; ++i) asm volatile("" : "+v"(xr[i]));
  auto pass2 = [&](auto neg_tag) {
    constexpr bool NEG = decltype(neg_tag)::value;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      if (tid + int64_t(i) * kResBlock >= nvec) continue;
      float xs[8], gs[8];
      IO<T>::unpack8(xr[i], xs);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float e = __builtin_amdgcn_exp2f(fmaf(xs[j], L2E, c2));
        gs[j] = NEG ? -e : e;
      }
      if (i == it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) gs[j] -= gp[j];
      }
      __builtin_amdgcn_raw_buffer_store_b128(IO<T>::pack8(gs), ro, voff, i * kResBlock * 16, 2);
    }
  };
  if (neg) pass2(std::true_type{});
  else pass2(std::false_type{});
}

template <class T, int CPT>
__global__ void __launch_bounds__(kResBlock)
label_resident_kernel(const T *Z, const int64_t *y, const uint8_t *mask, int64_t n, int64_t V,
                      double z_coef, double grad_out, const Control *ctl, T *grad,
                      double *row_out) {
  if (ctl->bad) return;
  for (int64_t t = blockIdx.x; t < n; t += gridDim.x)
    label_row_resident<T, CPT>(Z, y, mask, t, V, z_coef, grad_out, ctl, grad, row_out);
}

// Rows t = blockIdx.x, + gridDim.x, ...; nothing runs when the guard found
// an out-of-range target (the outputs stay untouched).
// NT threads per workgroup: 1024 (one per CU) when the row is read twice,
// so the second read finds it in the Infinity Cache; 512 (two per CU, their
// rows' phases interleaving) for the single read of the loss alone.
template <class T, bool VEC, bool GRAD, int NT = kBlock>
__global__ void __launch_bounds__(NT)
label_row_kernel(const T *Z, const int64_t *y, const uint8_t *mask, int64_t n, int64_t V,
                 double z_coef, double grad_out, const Control *ctl, T *grad, double *row_out) {
  if (ctl->bad) return;
  for (int64_t t = blockIdx.x; t < n; t += gridDim.x)
    label_row<T, VEC, GRAD, NT>(Z, y, mask, t, V, z_coef, grad_out, ctl, grad, row_out);
}

__global__ void distill_init_kernel(Control *ctl) {
  if (threadIdx.x == 0) {
    ctl->bad = 0;
    ctl->seen_bad = 0;
    ctl->first_bad = LLONG_MAX;
    ctl->count = 0;
    ctl->loss_sum = 0.0;
    ctl->z_sum = 0.0;
  }
}

__global__ void distill_count_kernel(const uint8_t *mask, int64_t n, Control *ctl) {
  __shared__ unsigned long long sh[4];
  unsigned long long c = 0;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < n;
       t += int64_t(gridDim.x) * blockDim.x)
    c += mask ? (mask[t] != 0) : 1;
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < int(blockDim.x >> 6); ++w) c += sh[w];
    if (c) atomicAdd(reinterpret_cast<unsigned long long *>(&ctl->count), c);
  }
}

// Fixed-order fp64 sums of the per-row loss and lse^2 over counted rows.
__global__ void distill_final_kernel(const double *row_out, const uint8_t *mask, int64_t n,
                                     Control *ctl) {
  __shared__ double s_l[1024], s_z[1024];
  double l = 0.0, z = 0.0;
  for (int64_t t = threadIdx.x; t < n; t += blockDim.x) {
    if (mask && !mask[t]) continue;
    l += row_out[2 * t];
    z += row_out[2 * t + 1] * row_out[2 * t + 1];
  }
  s_l[threadIdx.x] = l;
  s_z[threadIdx.x] = z;
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

template <class T, int OBJ>
void launch_rows(bool vec, const T *S, const T *U, const uint8_t *mask, int64_t n, int64_t V,
                 double inv_T, double z, double go, const Control *ctl, T *grad, double *rows,
                 hipStream_t st) {
  const unsigned grid = unsigned(n < kRowGrid ? n : kRowGrid);
  if constexpr (sizeof(T) == 2) {   // student rows that fit the registers: read once
    if (vec && V / 8 <= int64_t(kResidentChunks) * kResBlock) {
      hipLaunchKernelGGL((distill_resident_kernel<T, OBJ, kResidentChunks>), dim3(grid),
                         dim3(kResBlock), 0, st, S, U, mask, n, V, inv_T, z, go, ctl, grad, rows);
      return;
    }
  }
  if (vec)
    hipLaunchKernelGGL((distill_row_kernel<T, OBJ, true>), dim3(grid), dim3(kBlock), 0, st, S, U,
                       mask, n, V, inv_T, z, go, ctl, grad, rows);
  else
    hipLaunchKernelGGL((distill_row_kernel<T, OBJ, false>), dim3(grid), dim3(kBlock), 0, st, S, U,
                       mask, n, V, inv_T, z, go, ctl, grad, rows);
}

template <class T>
void distill_impl(int objective, bool vec, const T *S, const T *U, const uint8_t *mask,
                  int64_t n, int64_t V, double T_, double z, double go, Control *ctl, T *grad,
                  double *rows, hipStream_t st, lce_timers *tm) {
  {
    TimedLaunch tl(tm, LCE_K_GUARD, st);
    hipLaunchKernelGGL(distill_init_kernel, dim3(1), dim3(64), 0, st, ctl);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(distill_count_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, mask, n,
                       ctl);
  }
  const double inv_T = 1.0 / T_;
  {
    TimedLaunch tl(tm, LCE_K_DISTILL, st);
    if (objective == 0) launch_rows<T, 0>(vec, S, U, mask, n, V, inv_T, z, go, ctl, grad, rows, st);
    else if (objective == 1) launch_rows<T, 1>(vec, S, U, mask, n, V, inv_T, z, go, ctl, grad, rows, st);
    else launch_rows<T, 2>(vec, S, U, mask, n, V, inv_T, z, go, ctl, grad, rows, st);
  }
  TimedLaunch tl(tm, LCE_K_REDUCE, st);
  hipLaunchKernelGGL(distill_final_kernel, dim3(1), dim3(1024), 0, st, (const double *)rows, mask,
                     n, ctl);
}

template <class T>
void label_impl(bool vec, bool want_grad, const T *Z, const int64_t *y, const uint8_t *mask,
                int64_t n, int64_t V, double z, double go, Control *ctl, T *grad, double *rows,
                hipStream_t st, lce_timers *tm) {
  launch_target_guard(y, mask, n, V, ctl, st, tm);
  const unsigned grid = unsigned(n < kRowGrid ? n : kRowGrid);
  {
    TimedLaunch tl(tm, LCE_K_LABEL_CE, st);
    bool done = false;
    if constexpr (sizeof(T) == 2) {   // 16-bit rows that fit the registers: read once
      if (vec && want_grad && V / 8 <= int64_t(kResidentChunks) * kResBlock) {
        hipLaunchKernelGGL((label_resident_kernel<T, kResidentChunks>), dim3(grid),
                           dim3(kResBlock), 0, st, Z, y, mask, n, V, z, go, ctl, grad, rows);
        done = true;
      }
    }
    if (done) {
    } else if (vec && want_grad)
      hipLaunchKernelGGL((label_row_kernel<T, true, true>), dim3(grid), dim3(kBlock), 0, st, Z, y,
                         mask, n, V, z, go, ctl, grad, rows);
    else if (vec)
      hipLaunchKernelGGL((label_row_kernel<T, true, false, kBlock / 2>),
                         dim3(unsigned(n < 2 * kRowGrid ? n : 2 * kRowGrid)), dim3(kBlock / 2), 0,
                         st, Z, y, mask, n, V, z, go, ctl, grad, rows);
    else if (want_grad)
      hipLaunchKernelGGL((label_row_kernel<T, false, true>), dim3(grid), dim3(kBlock), 0, st, Z,
                         y, mask, n, V, z, go, ctl, grad, rows);
    else
      hipLaunchKernelGGL((label_row_kernel<T, false, false>), dim3(grid), dim3(kBlock), 0, st, Z,
                         y, mask, n, V, z, go, ctl, grad, rows);
  }
  TimedLaunch tl(tm, LCE_K_REDUCE, st);
  hipLaunchKernelGGL(distill_final_kernel, dim3(1), dim3(1024), 0, st, (const double *)rows, mask,
                     n, ctl);
}

bool has(const lce_tensor *t) { return t && t->data; }
bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace
}  // namespace lce

using namespace lce;

extern "C" int32_t lce_distill_fwd_bwd(const lce_tensor *student, const lce_tensor *teacher,
                                       const lce_tensor *loss_mask, int64_t n_tok, int64_t vocab,
                                       int32_t objective, double temperature, double z_coef,
                                       double grad_out, lce_tensor *grad_logits,
                                       lce_tensor *workspace, lce_loss *out, void *stream) {
  return lce_distill_fwd_bwd_timed(student, teacher, loss_mask, n_tok, vocab, objective,
                                   temperature, z_coef, grad_out, grad_logits, workspace, out,
                                   stream, nullptr);
}

namespace lce {
namespace {

// The distillation call on a resolved scratch region: `ws` (256-byte aligned)
// holds at least `ws_bytes` bytes of device memory for the control block and
// the per-row results (DistillPlan).  ws == nullptr: the caller's workspace
// descriptor `workspace` supplies it.
int32_t distill_call(const lce_tensor *student, const lce_tensor *teacher,
                     const lce_tensor *loss_mask, int64_t n_tok, int64_t vocab,
                     int32_t objective, double temperature, double z_coef, double grad_out,
                     lce_tensor *grad_logits, const lce_tensor *workspace, uint8_t *ws,
                     int64_t ws_bytes, lce_loss *out, void *stream, lce_timers *timers) {
  DistillPlan p;
  int32_t st = plan_distill(n_tok, vocab, &p);
  if (st != LCE_OK) return st;
  if (!finite_scalar(z_coef) || !finite_scalar(grad_out) || !finite_scalar(temperature) ||
      !(temperature > 0.0))
    return LCE_NON_FINITE_SCALAR;
  if (!student || !teacher || !grad_logits || (!ws && !workspace)) return LCE_LENGTH_MISMATCH;
  const int32_t dt = student->dtype;
  if (dt != LCE_BF16 && dt != LCE_F16 && dt != LCE_F32 && dt != LCE_F64)
    return LCE_DTYPE_MISMATCH;
  if (teacher->dtype != dt || grad_logits->dtype != dt) return LCE_DTYPE_MISMATCH;
  if (has(loss_mask) && loss_mask->dtype != LCE_U8) return LCE_DTYPE_MISMATCH;
  if (!ws && workspace->dtype != LCE_U8) return LCE_DTYPE_MISMATCH;
  const int64_t cells = n_tok * vocab;
  if (!has(student) || student->numel < cells || !has(teacher) || teacher->numel < cells ||
      !has(grad_logits) || grad_logits->numel < cells)
    return LCE_LENGTH_MISMATCH;
  if (has(loss_mask) && loss_mask->numel < n_tok) return LCE_LENGTH_MISMATCH;
  if (ws) {
    if (ws_bytes < int64_t(p.total)) return LCE_LENGTH_MISMATCH;
  } else if (!has(workspace) || workspace->numel < int64_t(p.total) + 256) {
    return LCE_LENGTH_MISMATCH;
  }
  if (objective < 0 || objective > 2) return LCE_UNKNOWN_OBJECTIVE;
  // out == NULL: asynchronous, the scalars stay in the caller's workspace for
  // lce_loss_fetch; the static scratch has no such handle
  if (!out && ws) return LCE_LENGTH_MISMATCH;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!ws) {
    const uintptr_t base = (reinterpret_cast<uintptr_t>(workspace->data) + 255) & ~uintptr_t(255);
    ws = reinterpret_cast<uint8_t *>(base);
  }
  Control *ctl = reinterpret_cast<Control *>(ws);
  double *rows = reinterpret_cast<double *>(ws + p.off_rows);
  const uint8_t *mask = has(loss_mask) ? static_cast<const uint8_t *>(loss_mask->data) : nullptr;
  const size_t esz = dtype_size(dt);
  const bool vec = (vocab % 8 == 0) && aligned(student->data, 16) && aligned(teacher->data, 16) &&
                   aligned(grad_logits->data, 16) && (esz * 8) % 16 == 0;
  (void)hipGetLastError();
  if (dt == LCE_F16)
    distill_impl<_Float16>(objective, vec, static_cast<const _Float16 *>(student->data),
                           static_cast<const _Float16 *>(teacher->data), mask, n_tok, vocab,
                           temperature, z_coef, grad_out, ctl,
                           static_cast<_Float16 *>(grad_logits->data), rows, s, timers);
  else if (dt == LCE_BF16)
    distill_impl<uint16_t>(objective, vec, static_cast<const uint16_t *>(student->data),
                           static_cast<const uint16_t *>(teacher->data), mask, n_tok, vocab,
                           temperature, z_coef, grad_out, ctl,
                           static_cast<uint16_t *>(grad_logits->data), rows, s, timers);
  else if (dt == LCE_F32)
    distill_impl<float>(objective, vec, static_cast<const float *>(student->data),
                        static_cast<const float *>(teacher->data), mask, n_tok, vocab,
                        temperature, z_coef, grad_out, ctl, static_cast<float *>(grad_logits->data),
                        rows, s, timers);
  else
    distill_impl<double>(objective, vec, static_cast<const double *>(student->data),
                         static_cast<const double *>(teacher->data), mask, n_tok, vocab,
                         temperature, z_coef, grad_out, ctl,
                         static_cast<double *>(grad_logits->data), rows, s, timers);
  if (hipGetLastError() != hipSuccess) return LCE_DEVICE_ERROR;
  if (!out) return LCE_OK;   // enqueued; lce_loss_fetch(workspace) reads the scalars
  Control hc;
  if (hipMemcpyAsync(&hc, ctl, sizeof(Control), hipMemcpyDeviceToHost, s) != hipSuccess)
    return LCE_DEVICE_ERROR;
  if (hipStreamSynchronize(s) != hipSuccess) return LCE_DEVICE_ERROR;
  out->loss_sum = hc.loss_sum;
  out->z_sum = hc.z_sum;
  out->n_counted = hc.count;
  out->loss_mean = hc.count ? hc.loss_sum / double(hc.count) : 0.0;
  out->z_mean = hc.count ? hc.z_sum / double(hc.count) : 0.0;
  return LCE_OK;
}

// Scratch of the allocation-free distillation call: one control block and
// the per-row results of up to kNoAllocMaxTok tokens.  Each device holds its
// own copy for the life of the process; host code reaches it only through
// the per-device address hipGetSymbolAddress returns.
constexpr int64_t kNoAllocMaxTok = 65536;
constexpr size_t kNoAllocScratchBytes = kControlBytes + size_t(kNoAllocMaxTok) * 2 * sizeof(double);
__device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up once per device.
uint8_t *scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return static_cast<uint8_t *>(g_scratch_ptr[dev]);
}

}  // namespace
}  // namespace lce

extern "C" int32_t lce_distill_fwd_bwd_timed(const lce_tensor *student, const lce_tensor *teacher,
                                             const lce_tensor *loss_mask, int64_t n_tok,
                                             int64_t vocab, int32_t objective, double temperature,
                                             double z_coef, double grad_out,
                                             lce_tensor *grad_logits, lce_tensor *workspace,
                                             lce_loss *out, void *stream, lce_timers *timers) {
  return distill_call(student, teacher, loss_mask, n_tok, vocab, objective, temperature, z_coef,
                      grad_out, grad_logits, workspace, nullptr, 0, out, stream, timers);
}

extern "C" int32_t lce_distill_fwd_bwd_noalloc(const lce_tensor *student,
                                               const lce_tensor *teacher,
                                               const lce_tensor *loss_mask, int64_t n_tok,
                                               int64_t vocab, int32_t objective,
                                               double temperature, double z_coef, double grad_out,
                                               lce_tensor *grad_logits, lce_loss *out,
                                               void *stream) {
  // more than kNoAllocMaxTok tokens: the scratch-length check refuses (582)
  uint8_t *ws = scratch_for_current_device();
  if (!ws) return LCE_DEVICE_ERROR;
  return distill_call(student, teacher, loss_mask, n_tok, vocab, objective, temperature, z_coef,
                      grad_out, grad_logits, nullptr, ws, int64_t(kNoAllocScratchBytes), out,
                      stream, nullptr);
}

extern "C" int32_t lce_ce_logits_fwd_bwd(const lce_tensor *logits, const lce_tensor *targets,
                                         const lce_tensor *loss_mask, int64_t n_tok,
                                         int64_t vocab, double z_coef, double grad_out,
                                         lce_tensor *grad_logits, lce_tensor *workspace,
                                         lce_loss *out, void *stream) {
  return lce_ce_logits_fwd_bwd_timed(logits, targets, loss_mask, n_tok, vocab, z_coef, grad_out,
                                     grad_logits, workspace, out, stream, nullptr);
}

extern "C" int32_t lce_ce_logits_fwd_bwd_timed(const lce_tensor *logits,
                                               const lce_tensor *targets,
                                               const lce_tensor *loss_mask, int64_t n_tok,
                                               int64_t vocab, double z_coef, double grad_out,
                                               lce_tensor *grad_logits, lce_tensor *workspace,
                                               lce_loss *out, void *stream, lce_timers *timers) {
  DistillPlan p;
  int32_t st = plan_distill(n_tok, vocab, &p);
  if (st != LCE_OK) return st;
  if (!finite_scalar(z_coef) || !finite_scalar(grad_out)) return LCE_NON_FINITE_SCALAR;
  if (!logits || !targets || !workspace) return LCE_LENGTH_MISMATCH;
  const int32_t dt = logits->dtype;
  const bool want_grad = has(grad_logits);
  if (dt != LCE_BF16 && dt != LCE_F16 && dt != LCE_F32 && dt != LCE_F64)
    return LCE_DTYPE_MISMATCH;
  if (targets->dtype != LCE_I64) return LCE_DTYPE_MISMATCH;
  if (want_grad && grad_logits->dtype != dt) return LCE_DTYPE_MISMATCH;
  if (has(loss_mask) && loss_mask->dtype != LCE_U8) return LCE_DTYPE_MISMATCH;
  if (workspace->dtype != LCE_U8) return LCE_DTYPE_MISMATCH;
  const int64_t cells = n_tok * vocab;
  if (!has(logits) || logits->numel < cells || !has(targets) || targets->numel < n_tok)
    return LCE_LENGTH_MISMATCH;
  if (want_grad && grad_logits->numel < cells) return LCE_LENGTH_MISMATCH;
  if (has(loss_mask) && loss_mask->numel < n_tok) return LCE_LENGTH_MISMATCH;
  if (!has(workspace) || workspace->numel < int64_t(p.total) + 256) return LCE_LENGTH_MISMATCH;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uintptr_t base = (reinterpret_cast<uintptr_t>(workspace->data) + 255) & ~uintptr_t(255);
  uint8_t *ws = reinterpret_cast<uint8_t *>(base);
  Control *ctl = reinterpret_cast<Control *>(ws);
  double *rows = reinterpret_cast<double *>(ws + p.off_rows);
  const uint8_t *mask = has(loss_mask) ? static_cast<const uint8_t *>(loss_mask->data) : nullptr;
  const int64_t *y = static_cast<const int64_t *>(targets->data);
  const size_t esz = dtype_size(dt);
  const bool vec = (vocab % 8 == 0) && aligned(logits->data, 16) &&
                   (!want_grad || aligned(grad_logits->data, 16)) && (esz * 8) % 16 == 0;
  (void)hipGetLastError();
  if (dt == LCE_F16)
    label_impl<_Float16>(vec, want_grad, static_cast<const _Float16 *>(logits->data), y, mask,
                         n_tok, vocab, z_coef, grad_out, ctl,
                         want_grad ? static_cast<_Float16 *>(grad_logits->data) : nullptr, rows,
                         s, timers);
  else if (dt == LCE_BF16)
    label_impl<uint16_t>(vec, want_grad, static_cast<const uint16_t *>(logits->data), y, mask,
                         n_tok, vocab, z_coef, grad_out, ctl,
                         want_grad ? static_cast<uint16_t *>(grad_logits->data) : nullptr, rows,
                         s, timers);
  else if (dt == LCE_F32)
    label_impl<float>(vec, want_grad, static_cast<const float *>(logits->data), y, mask, n_tok,
                      vocab, z_coef, grad_out, ctl,
                      want_grad ? static_cast<float *>(grad_logits->data) : nullptr, rows, s,
                      timers);
  else
    label_impl<double>(vec, want_grad, static_cast<const double *>(logits->data), y, mask, n_tok,
                       vocab, z_coef, grad_out, ctl,
                       want_grad ? static_cast<double *>(grad_logits->data) : nullptr, rows, s,
                       timers);
  if (hipGetLastError() != hipSuccess) return LCE_DEVICE_ERROR;
  // out == NULL: enqueued; lce_loss_fetch(workspace) reads the scalars, or 586
  if (!out) return LCE_OK;
  Control hc;
  if (hipMemcpyAsync(&hc, ctl, sizeof(Control), hipMemcpyDeviceToHost, s) != hipSuccess)
    return LCE_DEVICE_ERROR;
  if (hipStreamSynchronize(s) != hipSuccess) return LCE_DEVICE_ERROR;
  if (hc.bad) return LCE_TARGET_OUT_OF_RANGE;
  out->loss_sum = hc.loss_sum;
  out->z_sum = hc.z_sum;
  out->n_counted = hc.count;
  out->loss_mean = hc.count ? hc.loss_sum / double(hc.count) : 0.0;
  out->z_mean = hc.count ? hc.z_sum / double(hc.count) : 0.0;
  return LCE_OK;
}
