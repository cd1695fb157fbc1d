// Device-side helpers shared by the attention forward kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernel.h"

namespace fa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994531f;

// ------------------------------------------------------------------------ //
// 16-bit element types: MFMA 32x32x16 and packed conversion from fp32.
// ------------------------------------------------------------------------ //
template <typename T> struct Half16;
template <> struct Half16<__bf16> {
  using v8 = bf16x8;
  using v2 = bf16x2;
  static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Half16<_Float16> {
  using v8 = f16x8;
  using v2 = f16x2;
  static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Two fp32 -> two T (round to nearest even), packed lo | hi << 16, as one
// packed conversion.
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typename Half16<T>::v2 v = {(T)lo, (T)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// max / sum of x[lane] and x[lane ^ 32] via v_permlane32_swap.
// NaN-propagating maximum. Unlike fmaxf it needs no NaN-quieting copy of an
// operand that is not known to be canonical (an MFMA result), and nested
// pairs of it become single v_maximum3_f32 instructions.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// x if bit p of the kept-key word w (keep_word) is set, else the float with
// bits `fill`: a signed 1-bit extract (0 or all ones) and one bit select --
// two instructions per score instead of three compares and two lane-mask
// operations.
__device__ __forceinline__ float keep_or(float x, uint32_t w, int p, uint32_t fill) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)w, p, 1);
  return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x) & m) | (fill & ~m));
}

// Visible-key test of the mask (see flash_attn.h), written without
// short-circuit branches so it lowers to compares and one v_cndmask.
__device__ __forceinline__ bool keep_ij(int i, int j, int S, int causal, int window, int n_sink) {
  const bool in_range = j < S;
  const bool in_window = (window == 0) | ((i - j) < window) | (j < n_sink);
  return in_range & ((causal == 0) | ((j <= i) & in_window));
}

// Key-block range a query block [q_lo, q_lo + BR) visits: sink blocks
// [0, n_sinkb) then [kb_lo, kb_hi]. Blocks outside hold no key visible to
// any of its rows, so they are never loaded.
struct BlockRange {
  int n_sinkb, kb_lo, kb_hi;
  __device__ __forceinline__ int count() const { return n_sinkb + (kb_hi - kb_lo + 1); }
  __device__ __forceinline__ int kb(int it) const { return it < n_sinkb ? it : kb_lo + (it - n_sinkb); }
};

template <int BR, int BC>
__device__ __forceinline__ BlockRange block_range(int q_lo, int S, int causal, int window, int n_sink) {
  BlockRange r;
  r.n_sinkb = 0;
  r.kb_lo = 0;
  if (causal) {
    const int q_last = min(q_lo + BR, S) - 1;
    r.kb_hi = q_last / BC;
    if (window > 0) {
      r.kb_lo = max(0, q_lo - window + 1) / BC;
      r.n_sinkb = min(r.kb_lo, (n_sink + BC - 1) / BC);
    }
  } else {
    r.kb_hi = (S - 1) / BC;
  }
  return r;
}

// True when every (query row of the block, key of the K block) pair is visible.
template <int BR, int BC>
__device__ __forceinline__ bool block_full(int q_lo, int k0, int S, int causal, int window, int n_sink) {
  bool full = (k0 + BC <= S);
  if (causal) {
    full = full && (k0 + BC - 1 <= q_lo);
    if (window > 0) full = full && ((q_lo + BR - 1 - k0 < window) || (k0 + BC <= n_sink));
  }
  return full;
}

// True when no key of the block [k0, k0 + BC) is visible to any of the query
// rows [r0, r1]: past the rows under the causal mask, or wholly before every
// row's window and holding no sink. The diagonal block of a 128-row query block
// is like this for the waves of its upper rows.
template <int BC>
__device__ __forceinline__ bool block_hidden(int r0, int r1, int k0, int causal, int window,
                                             int n_sink) {
  if (!causal) return false;
  if (k0 > r1) return true;
  const int k1 = k0 + BC - 1;
  return window > 0 && k0 >= n_sink && k1 < r0 && r0 - k1 >= window;
}

// Work-group -> (query block, batch*head): the order wg_tile describes.
__device__ __forceinline__ void wg_coords(const FwdParams& p, int id, int& qb, int& bh) {
  const Tile t = wg_tile(id, p.BH, p.nqb, p.causal != 0, p.window > 0);
  qb = t.qb;
  bh = t.bh;
}
// The work-group's position in dispatch order, or its mirror image when the
// host asks for the reverse order (a testing aid: no work-group depends on
// another, so the results must not change).
__device__ __forceinline__ int wg_id(const FwdParams& p) {
  return p.reverse ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
}
__device__ __forceinline__ void wg_coords(const FwdParams& p, int& qb, int& bh) {
  wg_coords(p, wg_id(p), qb, bh);
}

// ALiBi bias in the base-2 logit domain: turns raw (sign-folded) scores into
// t = c * s - b2 * |i - j| for keys j = jb + e, e = 32 t + 8 (r >> 2) + (r & 3),
// with b2 = slope * log2(e). The softmax then runs on t with a unit scale.
// Only the first NTU of the NT sub-tiles are touched.
template <int NTU, int NT>
__device__ __forceinline__ void alibi_logits(f32x16 (&acc)[NT], float c, float b2, int i, int jb) {
  static_assert(NTU <= NT, "sub-tiles");
  const float d0 = (float)(i - jb);
#pragma unroll
  for (int t = 0; t < NTU; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = (float)(32 * t + 8 * (r >> 2) + (r & 3));
      acc[t][r] = __builtin_fmaf(acc[t][r], c, -b2 * fabsf(d0 - e));
    }
}

// The ALiBi bias in raw score units (base-2 logit / c) under the causal mask,
// where j <= i for every visible key: -beta |i - j| = beta (j - i), with
// beta = slope log2(e) / c and key j = jb + 4h + e. This adds the per-key part beta e (e a compile-time
// constant, one FMA per score); the per-row part beta (jb + 4h - i) is one
// number per lane and block, applied in the softmax.
template <int NTU, int NT>
__device__ __forceinline__ void alibi_ramp(f32x16 (&acc)[NT], float beta) {
  static_assert(NTU <= NT, "sub-tiles");
#pragma unroll
  for (int t = 0; t < NTU; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      acc[t][r] = __builtin_fmaf((float)(32 * t + 8 * (r >> 2) + (r & 3)), beta, acc[t][r]);
}

// Smallest softmax scale (|scale| log2 e) for which the linear ALiBi form is
// used: beta = slope log2(e) / c stays far from overflow.
constexpr float kAlibiMinScale = 1e-6f;
// Largest |slope log2 e| for the linear form: the ramp and offset then stay
// below 16 * 2^8 log2 units in the blocks that carry the row's weight, so
// the scores keep all but a few of their bits (the error in an exponent is
// about 2^-24 of that size).
constexpr float kAlibiLinMaxB2 = 16.f;

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace fa
