// Merge of key-split partial results (the NumPy tiled-block guide closes on
// reducing partial outputs across workers; Lesson 91's online-softmax update,
// slide 11, applied once per partial instead of once per key block). For
// every row r with partials (O_s, LSE_s), s < n:
//     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s,
// computed against the largest LSE_s so no exponential overflows; partials
// with LSE_s = -inf (rows that saw no key of that split) weigh zero, and a row
// with no finite partial becomes (0, -inf).
//
// Memory-bound: each lane owns 4 consecutive elements of one row (16-byte
// loads of every partial, one store); D / 4 lanes share a row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_kernel.h"

namespace fa {

namespace {

template <typename T> struct Store4;
template <> struct Store4<float> {
  static __device__ __forceinline__ void put(float* dst, f32x4 v) {
    *reinterpret_cast<f32x4*>(dst) = v;
  }
};
template <typename T> struct Store4 {
  static __device__ __forceinline__ void put(T* dst, f32x4 v) {
    u32x2 w;
    w[0] = pack2<T>(v[0], v[1]);
    w[1] = pack2<T>(v[2], v[3]);
    *reinterpret_cast<u32x2*>(dst) = w;
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void fa_merge_kernel(const float* __restrict__ o_part,
                                                       const float* __restrict__ lse_part, int n,
                                                       int64_t rows, T* __restrict__ o,
                                                       float* __restrict__ lse) {
  constexpr int LPR = D / 4;       // lanes per row
  constexpr int RPB = 256 / LPR;   // rows per work-group
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = (threadIdx.x % LPR) * 4;
  if (r >= rows) return;
  float m = kNegInf;
  for (int s = 0; s < n; ++s) m = fmaxf(m, lse_part[(int64_t)s * rows + r]);
  const float ms = (m == kNegInf) ? 0.f : m;
  float tot = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < n; ++s) {
    const int64_t sr = (int64_t)s * rows + r;
    const float w = fast_exp2((lse_part[sr] - ms) * kLog2e);   // -inf -> 0
    const f32x4 x = *reinterpret_cast<const f32x4*>(o_part + sr * D + c);
    tot += w;
    acc[0] = __builtin_fmaf(w, x[0], acc[0]);
    acc[1] = __builtin_fmaf(w, x[1], acc[1]);
    acc[2] = __builtin_fmaf(w, x[2], acc[2]);
    acc[3] = __builtin_fmaf(w, x[3], acc[3]);
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const f32x4 out = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  Store4<T>::put(o + r * D + c, out);
  if (c == 0) lse[r] = tot > 0.f ? ms + fast_log2(tot) * kLn2 : kNegInf;
}

template <typename T>
static hipError_t launch_merge_t(const float* o_part, const float* lse_part, int n, int64_t rows,
                                 int D, T* o, float* lse, hipStream_t st) {
  const int rpb = 256 / (D / 4);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  switch (D) {
    case 16:
      hipLaunchKernelGGL((fa_merge_kernel<T, 16>), dim3(grid), dim3(256), 0, st, o_part, lse_part,
                         n, rows, o, lse);
      break;
    case 32:
      hipLaunchKernelGGL((fa_merge_kernel<T, 32>), dim3(grid), dim3(256), 0, st, o_part, lse_part,
                         n, rows, o, lse);
      break;
    case 64:
      hipLaunchKernelGGL((fa_merge_kernel<T, 64>), dim3(grid), dim3(256), 0, st, o_part, lse_part,
                         n, rows, o, lse);
      break;
    case 128:
      hipLaunchKernelGGL((fa_merge_kernel<T, 128>), dim3(grid), dim3(256), 0, st, o_part, lse_part,
                         n, rows, o, lse);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const float* o_part, const float* lse_part, int n_split, int64_t rows,
                        int D, void* o, float* lse, int dtype, hipStream_t st) {
  switch (dtype) {
    case kDtypeF32:
      return launch_merge_t(o_part, lse_part, n_split, rows, D, static_cast<float*>(o), lse, st);
    case kDtypeF16:
      return launch_merge_t(o_part, lse_part, n_split, rows, D, static_cast<_Float16*>(o), lse, st);
    case kDtypeBF16:
      return launch_merge_t(o_part, lse_part, n_split, rows, D, static_cast<__bf16*>(o), lse, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fa
