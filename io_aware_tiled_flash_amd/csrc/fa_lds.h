// LDS staging helpers shared by the bf16/f16 attention kernels (gfx950):
// the swizzled K / V tile layouts, the direct-to-LDS buffer loads that fill
// them, and the transposing LDS read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"

namespace fa {

constexpr int kBCf = kFastBC;  // keys per streamed block
constexpr float kTau = 8.f;  // lazy-rescale threshold (base-2 exponent)
// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data format,
// no swizzle, no stride): offsets at or past the size read as zero.
constexpr int kBufferFlags = 0x00020000;

typedef short s16x4 __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// The K layout's chunk swizzle k_swz and the V layout's segment swizzle
// v_swz are in fa_shapes.h (constexpr, so the host unit can check that every
// read pattern below is free of bank conflicts).

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

// A wave's 32 rows of X from a 32x32 accumulator layout (lane (r, h), r =
// lane & 31, holds X[r][32 dt + 8 g + 4 h + e] in acc[dt][4 g + e]), times
// `scale`, packed to T and written to dst (row-major, D elements a row; rows
// r >= nrows are not written) through the wave's LDS slice `stage` (32 D
// elements). Each lane writes its 8-byte pieces to the slice, then the wave
// reads whole 16-byte chunks row by row and writes full rows with 16-byte
// stores, instead of every store instruction touching 32 rows. The slice's
// 8-byte slot of (row r, chunk c, half e) is ((c ^ sw(r)) << 1) | (e ^ r bit
// 4), with sw(r) = r & 15 (D = 128) or (r >> 1) & 7 (D = 64): the 32 rows of a
// write cycle meet every bank once, and each read instruction (4 rows at
// D = 128, 8 at D = 64) sees one value of r bit 4.
template <typename T, int D>
__device__ __forceinline__ void rows_out_staged(T* __restrict__ dst, int nrows,
                                                const f32x16 (&acc)[D / 32], float scale,
                                                T* stage, int lane) {
  static_assert(sizeof(T) == 2 && (D == 64 || D == 128), "16-bit rows of 64 or 128");
  constexpr int RB = 2 * D;        // row bytes
  constexpr int CPR = RB / 16;     // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;   // rows per read instruction
  auto sw = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  char* const st = reinterpret_cast<char*>(stage);
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack2<T>(acc[dt][4 * g + 0] * scale, acc[dt][4 * g + 1] * scale);
      w[1] = pack2<T>(acc[dt][4 * g + 2] * scale, acc[dt][4 * g + 3] * scale);
      const int slot = (((4 * dt + g) ^ sw(r)) << 1) | (h ^ ((r >> 4) & 1));
      *reinterpret_cast<u32x2*>(st + r * RB + slot * 8) = w;
    }
#pragma unroll
  for (int ii = 0; ii < 32 / RPI; ++ii) {
    const int lr = ii * RPI + lane / CPR;
    const int pc = lane % CPR;
    u32x4 v = *reinterpret_cast<const u32x4*>(st + lr * RB + pc * 16);
    if (((ii * RPI) >> 4) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
    if (lr < nrows) *reinterpret_cast<u32x4*>(dst + (size_t)lr * D + 8 * (pc ^ sw(lr))) = v;
  }
}

// The same for fp32 rows (the key split's partial outputs): lane (r, h)
// holds the 16-byte chunk 8 dt + 2 g + h of row r. A 16-byte write serves 16
// lanes (16 rows) a cycle, so the chunk is placed at c ^ (r & 15); a read
// instruction covers 2 rows (D = 128) or 4 (D = 64) with whole chunks. The
// slice is 32 rows of D floats.
template <int D>
__device__ __forceinline__ void rows_out_staged_f32(float* __restrict__ dst, int nrows,
                                                    const f32x16 (&acc)[D / 32], float scale,
                                                    float* stage, int lane) {
  static_assert(D == 64 || D == 128, "rows of 64 or 128 floats");
  constexpr int RB = 4 * D;        // row bytes
  constexpr int CPR = RB / 16;     // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;   // rows per read instruction
  char* const st = reinterpret_cast<char*>(stage);
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 w = {acc[dt][4 * g + 0] * scale, acc[dt][4 * g + 1] * scale,
                       acc[dt][4 * g + 2] * scale, acc[dt][4 * g + 3] * scale};
      const int c = 8 * dt + 2 * g + h;
      *reinterpret_cast<f32x4*>(st + r * RB + 16 * (c ^ (r & 15))) = w;
    }
#pragma unroll
  for (int ii = 0; ii < 32 / RPI; ++ii) {
    const int lr = ii * RPI + lane / CPR;
    const int pc = lane % CPR;
    const f32x4 v = *reinterpret_cast<const f32x4*>(st + lr * RB + pc * 16);
    if (lr < nrows) *reinterpret_cast<f32x4*>(dst + (size_t)lr * D + 4 * (pc ^ (lr & 15))) = v;
  }
}

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
