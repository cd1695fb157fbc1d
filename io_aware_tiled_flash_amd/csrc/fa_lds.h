// LDS staging helpers shared by the bf16/f16 attention kernels (gfx950):
// the swizzled K / V tile layouts, the direct-to-LDS buffer loads that fill
// them, and the transposing LDS read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"

namespace fa {

constexpr int kBCf = 64;     // keys per streamed block
constexpr float kTau = 8.f;  // lazy-rescale threshold (base-2 exponent)
// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data format,
// no swizzle, no stride): offsets at or past the size read as zero.
constexpr int kBufferFlags = 0x00020000;

typedef short s16x4 __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// 16-byte chunk swizzle of the K layout.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
// 64-byte segment swizzle of the V layout.
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? (row & 3) : ((row >> 1) & 1);
}

// Direct HBM -> LDS copy of one BC x D tile (K if IS_V is false, else V)
// with buffer loads: wave w fills LDS 16-byte positions [w*NI*64,
// (w+1)*NI*64); position pos is (row, physical chunk) = divmod(pos, D/8) and
// receives the logical chunk the swizzle maps there. The per-lane byte
// offsets are fixed for the whole kernel; the buffer descriptor is rebuilt per
// block with its base at the block's first key and its size ending at the
// sequence end, so rows past the end read as zeros (every such key is masked
// out).
template <typename T, int D, int NW, bool IS_V>
struct TileDma {
  static constexpr int CPR = D / 8;                    // 16-byte chunks per row
  static constexpr int NI = kBCf * CPR / (64 * NW);    // instructions per wave per tile
  static_assert(NI >= 1 && NI * 64 * NW == kBCf * CPR, "tile / wave split");
  uint32_t voff[NI];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int pos = (wave * NI + n) * 64 + lane;
      const int row = pos / CPR;
      const int pc = pos % CPR;
      int d;
      if (IS_V) {
        const int seg = (pc >> 2) ^ v_swz<D>(row);
        d = 32 * seg + 8 * (pc & 3);
      } else {
        d = 8 * (pc ^ k_swz<D>(row));
      }
      voff[n] = (uint32_t)((row * D + d) * (int)sizeof(T));
    }
  }

  __device__ __forceinline__ void load(T* lds_tile, const T* __restrict__ g, int k0, int S,
                                       int wave) const {
    // Base and size are wave-uniform and the descriptor must sit in scalar
    // registers: the head pointer goes through readfirstlane before the
    // block offset is added, so the per-block address arithmetic is scalar.
    const uint64_t g64 = reinterpret_cast<uint64_t>(g);
    const uint32_t glo = __builtin_amdgcn_readfirstlane((uint32_t)g64);
    const uint32_t ghi = __builtin_amdgcn_readfirstlane((uint32_t)(g64 >> 32));
    const uint64_t base = (((uint64_t)ghi << 32) | glo) + (uint64_t)(uint32_t)k0 * (D * sizeof(T));
    // The descriptor covers this tile only (rows past the sequence end read
    // as zero), so its 32-bit size cannot overflow however long S is.
    const int bytes = min(S - k0, kBCf) * D * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(base), (short)0, bytes, kBufferFlags);
#pragma unroll
    for (int n = 0; n < NI; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_tile + (wave * NI + n) * 512),
                                               16, voff[n], 0, 0, 0);
  }
};

// A wave-uniform pointer moved to scalar registers.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left at their maxima (gfx9 encoding:
// vmcnt low bits [3:0], high bits [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <typename T>
__device__ __forceinline__ u32x2 lds_tr_read(const T* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

}  // namespace fa
