// Backward pass of the tiled attention for gfx950 (bf16 / f16, head dim 64
// or 128): dQ, dK, dV by recomputation from the forward's logsumexp, without
// storing the S x S probability matrix (the Lesson 91 deck, slide 12 and its
// closing note: the tile loop keeps only m, l and O, and the backward
// recomputes the tiles; the gradients themselves are those of ordinary
// attention). With P = exp(scale Q K^T + bias - LSE) on the visible pairs,
// dP = dO V^T and delta_i = sum_d dO_id O_id (= sum_j P_ij dP_ij):
//     dV = P^T dO,   dS = P * (dP - delta),   dQ = scale dS K,   dK = scale dS^T Q.
//
// Two kernels, both on v_mfma_f32_32x32x16 for every product:
//  * dq kernel: one work-group per (query block of 32 * NW rows, query head),
//    two work-groups per CU.
//    Each wave holds 32 rows of Q and dO in registers, computes its rows'
//    delta (written to the workspace for the second kernel) and streams the
//    visible key blocks: S^T = K Q^T and dP^T = V dO^T (K, V rows read from
//    LDS), P and dS in registers, dQ^T += K^T dS^T with K^T read from LDS by
//    transposing reads.
//  * dkv kernel: one work-group per (key block of 32 * NW keys, key/value
//    head). Each wave holds 32 keys of K and V in registers and accumulates
//    dK^T and dV^T over the query heads of its group and the query blocks
//    that see its keys: S = Q K^T and dP = dO V^T (Q, dO rows from LDS), then
//    dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T read transposed.
// Tiles are staged HBM -> LDS with direct-to-LDS buffer loads in the K layout
// of the forward kernel (16-byte chunks XOR-swizzled by row), which serves
// both the row reads and the transposing reads without bank conflicts.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "fa_device.h"
#include "fa_kernel.h"
#include "fa_lds.h"

#include <type_traits>

namespace fa {

namespace {

constexpr int kBwdWaves = 4;

// Per-lane element offsets of the transposing reads of a tile in the K
// layout, relative to a 16-row chunk: lane 32h + 16grp + r16 fetches 4
// elements of row 4h + (r16 >> 2) (lo) or that + 8 (hi), columns
// 32 dt + 16 grp + 4 (r16 & 3) .., so that lane m of each half receives
// column 32 dt + (m & 31) of rows {4h .. 4h+3} and {8 + 4h .. 8 + 4h+3} --
// the k-slot order in which the C layout of a 32x32 MFMA holds its rows.
template <int D>
struct TrOffsets {
  static constexpr int NDT = D / 32;
  int lo[NDT], hi[NDT];
  __device__ __forceinline__ void init(int lane) {
    const int h = lane >> 5, grp = (lane >> 4) & 1, r16 = lane & 15;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const int row = 4 * h + (r16 >> 2) + 8 * part;
      const int sw = k_swz<D>(row);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int chunk = 4 * dt + 2 * grp + ((r16 & 3) >> 1);
        const int off = row * D + ((chunk ^ sw) << 3) + 4 * (r16 & 1);
        if (part == 0)
          lo[dt] = off;
        else
          hi[dt] = off;
      }
    }
  }
};

// Row-read offsets (the A operand of an MFMA over d): lane (col, h) reads 8
// elements of row col of a 32-row tile, columns 16 s + 8 h .. +7.
template <int D>
struct RowOffsets {
  static constexpr int NS = D / 16;
  int off[NS];
  __device__ __forceinline__ void init(int lane) {
    const int h = lane >> 5, col = lane & 31;
    const int sw = k_swz<D>(col);
#pragma unroll
    for (int s = 0; s < NS; ++s) off[s] = col * D + (((2 * s + h) ^ sw) << 3);
  }
};

template <typename T>
__device__ __forceinline__ typename Half16<T>::v8 lds_row8(const T* p) {
  return __builtin_bit_cast(typename Half16<T>::v8, *reinterpret_cast<const u32x4*>(p));
}

template <typename T>
__device__ __forceinline__ typename Half16<T>::v8 lds_tr8(const T* lo, const T* hi) {
  const u32x2 a = lds_tr_read(lo);
  const u32x2 b = lds_tr_read(hi);
  const u32x4 w = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(typename Half16<T>::v8, w);
}

// 8 elements of a global row (16-byte aligned) as an MFMA operand; zeros
// when the row is past the end.
template <typename T>
__device__ __forceinline__ typename Half16<T>::v8 load_frag(const T* __restrict__ base, int row,
                                                            int S, int D, int d0) {
  u32x4 w = {0u, 0u, 0u, 0u};
  if (row < S) w = *reinterpret_cast<const u32x4*>(base + (size_t)row * D + d0);
  return __builtin_bit_cast(typename Half16<T>::v8, w);
}

// Pack 8 accumulator values (k-slots of one 16-row chunk) into a B operand.
template <typename T>
__device__ __forceinline__ typename Half16<T>::v8 pack8(const f32x16& acc, int u) {
  u32x4 w;
  w[0] = pack2<T>(acc[8 * u + 0], acc[8 * u + 1]);
  w[1] = pack2<T>(acc[8 * u + 2], acc[8 * u + 3]);
  w[2] = pack2<T>(acc[8 * u + 4], acc[8 * u + 5]);
  w[3] = pack2<T>(acc[8 * u + 6], acc[8 * u + 7]);
  return __builtin_bit_cast(typename Half16<T>::v8, w);
}

// Query-block range [first, last] whose rows see some key of [k_lo, k_hi].
__device__ __forceinline__ void query_range(const BwdParams& p, int k_lo, int k_hi, int BQ,
                                            int& first, int& last) {
  const int nqb = (p.S + BQ - 1) / BQ;
  first = 0;
  last = nqb - 1;
  if (p.causal) {
    first = k_lo / BQ;
    if (p.window > 0 && k_lo >= p.n_sink) {
      const int last_row = min(p.S - 1, k_hi + p.window - 1);
      last = last_row / BQ;
    }
  }
}

// Scheduling groups for a run of N MFMAs fed by LDS reads (PER reads per
// MFMA): AHEAD MFMAs' worth of reads first, then one MFMA and its successor's
// reads in turn, then the last MFMAs. With one wave per SIMD nothing else
// hides the LDS latency, and left to itself the scheduler issues each read
// right before the MFMA that consumes it. Mask bits: 0x100 LDS read, 0x008
// MFMA.
template <int N, int PER, int AHEAD>
__device__ __forceinline__ void lds_mfma_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, PER * AHEAD, 0);
#pragma unroll
  for (int u = 0; u < N - AHEAD; ++u) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// Direct-to-LDS copy of 64 consecutive fp32 values (one per lane, 4 bytes
// each) from g to the LDS array lds: issued by one wave.
__device__ __forceinline__ void rows_to_lds(float* lds, const float* g, int lane) {
  const uint64_t g64 = reinterpret_cast<uint64_t>(g);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)g64);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(g64 >> 32));
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, 64 * 4, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds, 4, (uint32_t)lane * 4u, 0, 0, 0);
}

// Row reads (the A operand of an MFMA over d) in byte form, for 2-byte
// elements: lane (col, h) reads chunk (2 s + h) ^ k_swz(row) of row
// row0 + col. The row's offset, the swizzled chunk h ^ k_swz and the
// k-step's chunk bits 2 s occupy disjoint bit fields once the low two are
// XORed, so the byte offset of k-step s is b ^ (32 s): one XOR per k-step.
// Rows 32 apart share the swizzle, and 32 rows of D elements span a
// multiple of 256 bytes, so another wave's rows are b + 64 D wave.
template <int D>
struct RowXor {
  uint32_t b;
  __device__ __forceinline__ void init(int lane) {
    const int h = lane >> 5, col = lane & 31;
    b = (uint32_t)(2 * (col * D + ((h ^ k_swz<D>(col)) << 3)));
  }
  __device__ __forceinline__ uint32_t at(int s) const { return b ^ (32u * (uint32_t)s); }
};

// Transposing reads (see TrOffsets) in byte form, by the same argument:
// chunk (4 dt + c) ^ k_swz(row) with c < 4, so lo / hi (dt) = b[0] / b[1]
// ^ (64 dt).
template <int D>
struct TrXor {
  uint32_t b[2];
  __device__ __forceinline__ void init(int lane) {
    const int h = lane >> 5, grp = (lane >> 4) & 1, r16 = lane & 15;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const int row = 4 * h + (r16 >> 2) + 8 * part;
      const int c = 2 * grp + ((r16 & 3) >> 1);
      b[part] = (uint32_t)(2 * (row * D + ((c ^ k_swz<D>(row)) << 3) + 4 * (r16 & 1)));
    }
  }
  __device__ __forceinline__ uint32_t lo(int dt) const { return b[0] ^ (64u * (uint32_t)dt); }
  __device__ __forceinline__ uint32_t hi(int dt) const { return b[1] ^ (64u * (uint32_t)dt); }
};

// p advanced by b bytes
template <typename T>
__device__ __forceinline__ const T* at_bytes(const T* p, uint32_t b) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(p) + b);
}

// Direct-to-LDS copy of ROWS rows of D elements (K layout: 16-byte chunks
// XOR-swizzled by row, as TileDma) by NW waves. Rows past the sequence end
// read as zeros (the descriptor ends there).
template <typename T, int D, int ROWS, int NW>
struct RowsDma {
  static constexpr int CPR = D / 8;                   // 16-byte chunks per row
  static constexpr int NI = ROWS * CPR / (64 * NW);   // instructions per wave
  static_assert(NI >= 1 && NI * 64 * NW == ROWS * CPR, "tile / wave split");
  uint32_t voff[NI];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int pos = (wave * NI + n) * 64 + lane;
      const int row = pos / CPR;
      const int pc = pos % CPR;
      voff[n] = (uint32_t)((row * D + 8 * (pc ^ k_swz<D>(row))) * (int)sizeof(T));
    }
  }

  // rows [r0, r0 + ROWS) of g (r0 < S) into lds
  __device__ __forceinline__ void load(T* lds, const T* __restrict__ g, int r0, int S,
                                       int wave) const {
    const uint64_t g64 = reinterpret_cast<uint64_t>(g);
    const uint32_t glo = __builtin_amdgcn_readfirstlane((uint32_t)g64);
    const uint32_t ghi = __builtin_amdgcn_readfirstlane((uint32_t)(g64 >> 32));
    const uint64_t base = (((uint64_t)ghi << 32) | glo) + (uint64_t)(uint32_t)r0 * (D * sizeof(T));
    const int bytes = min(S - r0, ROWS) * D * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(base), (short)0, bytes, kBufferFlags);
#pragma unroll
    for (int n = 0; n < NI; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + (wave * NI + n) * 512), 16,
                                               voff[n], 0, 0, 0);
  }
};

// Direct-to-LDS copy of 32 consecutive fp32 values from g to lds[0..31],
// issued by one wave (lanes 32..63 fall outside the descriptor and read 0
// into lds[32..63]).
__device__ __forceinline__ void rows32_to_lds(float* lds, const float* g, int lane) {
  const uint64_t g64 = reinterpret_cast<uint64_t>(g);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)g64);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(g64 >> 32));
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, 32 * 4, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds, 4, (uint32_t)lane * 4u, 0, 0, 0);
}

}  // namespace

// ------------------------------------------------------------------------ //
// dq kernel
// ------------------------------------------------------------------------ //
// Besides dQ, it writes the two per-row arrays the dkv kernel reads, padded to
// Sp rows per head so that the dkv kernel's 16-byte loads need no bounds
// checks: delta (0 past the sequence end) and lse * log2(e) (+inf there, so
// that rows past the end get P = 0 without a mask).
//
// Waves per SIMD: two at D = 128 (256 registers). At D = 64 the kernel fits in
// 168 registers without spilling, so a third work-group per CU (96 KiB of LDS
// in all) adds a third wave per SIMD: same-process A/B +2.3 % on a causal
// B4 H32 S4096 D64 backward, +3.8 % with a 256-key window, +0.9 % unmasked.
// (The dK/dV kernel at D = 64 needs 175 and spills at 168; it stays at two.)
template <int D>
constexpr int dq_waves_per_simd() {
  return D == 64 ? 3 : 2;
}

template <typename T, int D, bool ALIBI>
__global__ __launch_bounds__(64 * kBwdWaves) __attribute__((amdgpu_waves_per_eu(
    dq_waves_per_simd<D>(), dq_waves_per_simd<D>())))
void fa_bwd_dq_kernel(BwdParams p) {
  constexpr int NW = kBwdWaves;
  constexpr int BR = 32 * NW;
  constexpr int BC = kBCf;
  constexpr int NT = BC / 32;
  constexpr int NS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int TILE = BC * D;
  using Tr = Half16<T>;
  using v8 = typename Tr::v8;

  // two K/V buffer pairs: block it+1 lands while block it is computed
  __shared__ __attribute__((aligned(1024))) T k0s[TILE];
  __shared__ __attribute__((aligned(1024))) T v0s[TILE];
  __shared__ __attribute__((aligned(1024))) T k1s[TILE];
  __shared__ __attribute__((aligned(1024))) T v1s[TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  // the forward's work-group order (wg_tile): the XCD's heads in groups of
  // four under the causal mask, heaviest query blocks first
  const Tile tq = wg_tile((int)blockIdx.x, p.BH, p.nqb, p.causal != 0, p.window > 0);
  const int bh = tq.bh;
  const int qb = tq.qb;
  const int S = p.S;
  const int q_lo = qb * BR;
  const int i = q_lo + 32 * wave + col;   // < nqb * BR = Sp
  const size_t head = (size_t)bh * S * D;
  const size_t kv_head = (size_t)(bh / p.G) * S * D;
  const T* __restrict__ Qh = reinterpret_cast<const T*>(p.q) + head;
  const T* __restrict__ Oh = reinterpret_cast<const T*>(p.o) + head;
  const T* __restrict__ dOh = reinterpret_cast<const T*>(p.dout) + head;
  const T* __restrict__ Kh = reinterpret_cast<const T*>(p.k) + kv_head;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(p.v) + kv_head;

  // Q and dO rows as B operands; delta_i = dO_i . O_i
  v8 qf[NS], df[NS];
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = load_frag<T>(Qh, i, S, D, 16 * s + 8 * h);
    df[s] = load_frag<T>(dOh, i, S, D, 16 * s + 8 * h);
    const v8 of = load_frag<T>(Oh, i, S, D, 16 * s + 8 * h);
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf((float)df[s][e], (float)of[e], dpart);
  }
  const bool row_ok = i < S;
  const float delta = row_ok ? xhalf_sum(dpart) : 0.f;
  const float lse2 = row_ok ? p.lse[(size_t)bh * S + i] * kLog2e : __builtin_inff();
  if (h == 0) {
    p.delta[(size_t)bh * p.Sp + i] = delta;
    p.lse2[(size_t)bh * p.Sp + i] = lse2;
  }
  const float b2 = ALIBI ? p.alibi[bh % p.H] * kLog2e : 0.f;

  RowOffsets<D> ro;
  ro.init(lane);
  TrOffsets<D> tro;
  tro.init(lane);
  TileDma<T, D, NW, false> dma;
  dma.init(wave, lane);

  f32x16 dq[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

  // Per-lane mask bounds in units of e = 32 t + 8 g + r4 (key j = k0 + 4 h + e),
  // as in the forward kernel: keep iff e <= hi and (e >= lo or e <= sk).
  const int big = 1 << 30;
  const int hi0 = p.causal ? min(i, S - 1) : S - 1;
  const int lo0 = p.window > 0 ? i - p.window + 1 : -big;
  const int sk0 = p.window > 0 ? p.n_sink - 1 : -big;

  const BlockRange br = block_range<BR, BC>(q_lo, S, p.causal, p.window, p.n_sink);
  const int n_iter = br.count();
  if (n_iter > 0) {
    dma.load(k0s, Kh, br.kb(0) * BC, S, wave);
    dma.load(v0s, Vh, br.kb(0) * BC, S, wave);
  }
  wait_vmem<0>();
  __syncthreads();
  // Block `it` from buffer pair PAR while block it+1 loads into the other;
  // MASK selects the masked variant at compile time (partially visible
  // blocks sit at the two ends of the visiting order, as in the forward).
  auto step = [&](auto par, auto mask, int it) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    constexpr bool MASK = decltype(mask)::value;
    const T* ks = PAR == 0 ? k0s : k1s;
    const T* vs = PAR == 0 ? v0s : v1s;
    if (it + 1 < n_iter) {
      const int k1 = br.kb(it + 1) * BC;
      dma.load(PAR == 0 ? k1s : k0s, Kh, k1, S, wave);
      dma.load(PAR == 0 ? v1s : v0s, Vh, k1, S, wave);
    }
    const int k0 = br.kb(it) * BC;
    const int jb = k0 + 4 * h;
    const int hi = hi0 - jb, lo = lo0 - jb, sk = sk0 - jb;
    // One 32-key half at a time (scores, dS, then its share of dQ), with
    // short read lookaheads: that keeps the kernel within 256 registers, so
    // two work-groups share a CU and one wave's vector work overlaps the
    // other's MFMAs (8 % faster than one wave per SIMD with both halves'
    // scores held at once).
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // dP^T accumulates from -delta (a per-lane constant here), so the
      // subtraction of dS = P (dP - delta) happens in the MFMA chain (not with
      // ALiBi, whose bias terms need the 16 registers that constant takes)
      f32x16 sT, pT;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sT[r] = 0.f;
        pT[r] = ALIBI ? 0.f : -delta;
      }
      v8 ka[NS], va[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        ka[s] = lds_row8(ks + 32 * t * D + ro.off[s]);
        va[s] = lds_row8(vs + 32 * t * D + ro.off[s]);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sT = Tr::mma(ka[s], qf[s], sT);
        pT = Tr::mma(va[s], df[s], pT);
      }
      lds_mfma_pipeline<2 * NS, 1, 4>();
      // kept iff e <= hi and (e >= lo or e <= sk), as one bit word
      const uint32_t mw = MASK ? keep_word(lo, hi, min(sk, hi), 32 * t) : 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = 32 * t + 8 * (r >> 2) + (r & 3);
        float x;
        if (ALIBI)
          x = __builtin_fmaf(sT[r], p.c, -b2 * fabsf((float)(i - jb - e))) - lse2;
        else
          x = __builtin_fmaf(sT[r], p.c, -lse2);
        float pr = fast_exp2(x);
        if (MASK) pr = keep_or(pr, mw, 8 * (r >> 2) + (r & 3), 0u);
        sT[r] = pr * (ALIBI ? pT[r] - delta : pT[r]);   // dS^T
      }
      v8 dsb[2];
      dsb[0] = pack8<T>(sT, 0);
      dsb[1] = pack8<T>(sT, 1);
      // dQ^T += K^T dS^T
      v8 kT[2][NDT];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const T* kk = ks + (32 * t + 16 * u) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) kT[u][dt] = lds_tr8(kk + tro.lo[dt], kk + tro.hi[dt]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) dq[dt] = Tr::mma(kT[u][dt], dsb[u], dq[dt]);
      lds_mfma_pipeline<2 * NDT, 2, 2>();
    }
    wait_vmem<0>();
    __syncthreads();
  };
  auto segment = [&](auto mask, int b, int e) __attribute__((always_inline)) {
    int it = b;
    if (it < e && (it & 1)) step(std::integral_constant<int, 1>{}, mask, it++);
    for (; it + 2 <= e; it += 2) {
      step(std::integral_constant<int, 0>{}, mask, it);
      step(std::integral_constant<int, 1>{}, mask, it + 1);
    }
    if (it < e) step(std::integral_constant<int, 0>{}, mask, it);
  };
  const StepRange fr = local_steps(
      full_key_steps(q_lo, BR, BC, S, p.causal, p.window, br.n_sinkb, br.kb_lo, br.kb_hi), 0,
      n_iter, false);
  const int f0 = fr.lo, f1 = fr.hi;
  segment(std::true_type{}, 0, f0);
  segment(std::false_type{}, f0, f1);
  segment(std::true_type{}, f1, n_iter);
  // dQ rows through the idle K/V tiles (every wave is past the last barrier)
  rows_out_staged<T, D>(reinterpret_cast<T*>(p.dq) + head + (size_t)(q_lo + 32 * wave) * D,
                        S - (q_lo + 32 * wave), dq, p.scale,
                        ((wave >> 1) == 0 ? k0s : v0s) + (wave & 1) * 32 * D, lane);
}

// ------------------------------------------------------------------------ //
// dkv kernel
// ------------------------------------------------------------------------ //
template <typename T, int D, bool ALIBI>
__global__ __launch_bounds__(64 * kBwdWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bwd_dkv_kernel(BwdParams p) {
  constexpr int NW = kBwdWaves;
  constexpr int BK = 32 * NW;    // keys per work-group
  constexpr int BQ = 2 * kBCf;   // query rows per streamed block (two tile loads)
  constexpr int NT = BQ / 32;
  constexpr int NS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int TILE = BQ * D;
  using Tr = Half16<T>;
  using v8 = typename Tr::v8;

  // two Q/dO buffer pairs: the next query block lands while this one is computed
  __shared__ __attribute__((aligned(1024))) T q0s[TILE];
  __shared__ __attribute__((aligned(1024))) T d0s[TILE];
  __shared__ __attribute__((aligned(1024))) T q1s[TILE];
  __shared__ __attribute__((aligned(1024))) T d1s[TILE];
  // the block's lse * log2(e) and delta rows, staged with the tiles
  __shared__ __attribute__((aligned(16))) float r0s[2 * BQ];
  __shared__ __attribute__((aligned(16))) float r1s[2 * BQ];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int BHkv = p.BH / p.G;
  // the order of wg_tile over key blocks, as in fa_bwd_dkv2_kernel below
  const Tile tk = wg_tile((int)blockIdx.x, BHkv, p.nkb, p.causal != 0, false);
  const int bkv = tk.bh;
  const int kb = p.causal ? p.nkb - 1 - tk.qb : tk.qb;
  const int S = p.S;
  const int k_lo = kb * BK;
  const int j = k_lo + 32 * wave + col;   // this lane's key
  const size_t kv_head = (size_t)bkv * S * D;
  const T* __restrict__ Kh = reinterpret_cast<const T*>(p.k) + kv_head;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(p.v) + kv_head;

  v8 kf[NS], vf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kf[s] = load_frag<T>(Kh, j, S, D, 16 * s + 8 * h);
    vf[s] = load_frag<T>(Vh, j, S, D, 16 * s + 8 * h);
  }

  RowOffsets<D> ro;
  ro.init(lane);
  TrOffsets<D> tro;
  tro.init(lane);
  TileDma<T, D, NW, false> dma;
  dma.init(wave, lane);

  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }

  int qfirst, qlast;
  query_range(p, k_lo, min(k_lo + BK, S) - 1, BQ, qfirst, qlast);
  // Mask of a partially visible (query block, key block) pair, for row
  // i = q0 + 4 h + e (e = 32 t + 8 g + r4) and this lane's key j: keep iff
  // i >= j and (i - j < window or j < n_sink). Rows past the sequence end
  // need no mask (their lse * log2(e) is +inf), nor do keys past it (their
  // K / V rows are zero and their dK, dV are never stored).
  const int big = 1 << 30;
  const bool sinkj = p.window > 0 && j < p.n_sink;
  const int wlen = p.window > 0 ? p.window : big;

  // steps: (query head of the group gi, query block qb) in order, n_q blocks per head
  const int n_q = qlast - qfirst + 1;
  const int n_iter = n_q > 0 ? p.G * n_q : 0;
  auto tile_src = [&](int it, const T*& Qh, const T*& dOh, int& bh, int& q0)
      __attribute__((always_inline)) {
    const int gi = it / n_q;
    bh = bkv * p.G + gi;   // query head (b * H + h)
    q0 = (qfirst + it - gi * n_q) * BQ;
    const size_t head = (size_t)bh * S * D;
    Qh = reinterpret_cast<const T*>(p.q) + head;
    dOh = reinterpret_cast<const T*>(p.dout) + head;
  };
  // a BQ-row tile as kBCf-row loads; a part wholly past the sequence end
  // loads row S - 1 and zeros (finite data; those rows carry P = 0)
  auto tile_load = [&](T* dst, const T* src, int q0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < BQ / kBCf; ++u)
      dma.load(dst + u * kBCf * D, src, min(q0 + u * kBCf, S - 1), S, wave);
  };
  // rows [q0, q0 + BQ) of the padded per-row arrays (no bounds checks: q0 +
  // BQ <= Sp) into dst = [lse * log2(e) | delta]
  auto rows_dma = [&](float* dst, int bh, int q0) __attribute__((always_inline)) {
    if (wave == 0) {
      const size_t rb = (size_t)bh * p.Sp + q0;
#pragma unroll
      for (int u = 0; u < BQ / 64; ++u) {
        rows_to_lds(dst + 64 * u, p.lse2 + rb + 64 * u, lane);
        rows_to_lds(dst + BQ + 64 * u, p.delta + rb + 64 * u, lane);
      }
    }
  };
  if (n_iter > 0) {
    const T *Qh, *dOh;
    int bh0, q00;
    tile_src(0, Qh, dOh, bh0, q00);
    tile_load(q0s, Qh, q00);
    tile_load(d0s, dOh, q00);
    rows_dma(r0s, bh0, q00);
  }
  wait_vmem<0>();
  __syncthreads();
  auto step = [&](auto par, auto mask, int it) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    constexpr bool MASK = decltype(mask)::value;
    const T* qs = PAR == 0 ? q0s : q1s;
    const T* dos = PAR == 0 ? d0s : d1s;
    const float* rs = PAR == 0 ? r0s : r1s;
    const T *Qh_, *dOh_;
    int bh, q0;
    tile_src(it, Qh_, dOh_, bh, q0);
    if (it + 1 < n_iter) {
      const T *Qn, *dOn;
      int bhn, qn;
      tile_src(it + 1, Qn, dOn, bhn, qn);
      tile_load(PAR == 0 ? q1s : q0s, Qn, qn);
      tile_load(PAR == 0 ? d1s : d0s, dOn, qn);
      rows_dma(PAR == 0 ? r1s : r0s, bhn, qn);
    }
    const float b2 = ALIBI ? p.alibi[bh % p.H] * kLog2e : 0.f;
    const int emin = j - q0 - 4 * h;   // keep iff e >= emin and (e < emin + wlen or sinkj)
    const int ehi = sinkj ? big : emin + wlen - 1;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[r] = 0.f;
        dp[r] = 0.f;
      }
      // operands read into arrays first: with the reads inline the register
      // allocator gave every read the same registers, serialising them
      v8 qa[NS], da[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        qa[s] = lds_row8(qs + 32 * t * D + ro.off[s]);
        da[s] = lds_row8(dos + 32 * t * D + ro.off[s]);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sc = Tr::mma(qa[s], kf[s], sc);
        dp = Tr::mma(da[s], vf[s], dp);
      }
      lds_mfma_pipeline<2 * NS, 1, 6>();
      // this lane's rows of the block: 32 t + 8 g + 4 h + (0..3); read after
      // the operand reads above (one more scheduling group of 8 LDS reads)
      f32x4 l2[4], dd[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        l2[g] = *reinterpret_cast<const f32x4*>(rs + 32 * t + 8 * g + 4 * h);
        dd[g] = *reinterpret_cast<const f32x4*>(rs + BQ + 32 * t + 8 * g + 4 * h);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      f32x16 pm, ds;
      const uint32_t mw = MASK ? keep_word(emin, ehi, -1, 32 * t) : 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int g = r >> 2, e4 = r & 3;
        const int e = 32 * t + 8 * g + e4;
        float x;
        if (ALIBI)
          x = __builtin_fmaf(sc[r], p.c, -b2 * fabsf((float)(e - emin))) - l2[g][e4];
        else
          x = __builtin_fmaf(sc[r], p.c, -l2[g][e4]);
        float pr = fast_exp2(x);
        if (MASK) pr = keep_or(pr, mw, 8 * g + e4, 0u);
        pm[r] = pr;
        ds[r] = pr * (dp[r] - dd[g][e4]);
      }
      v8 oT[2][NDT], qT[2][NDT];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const T* qq = qs + (32 * t + 16 * u) * D;
        const T* oo = dos + (32 * t + 16 * u) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          oT[u][dt] = lds_tr8(oo + tro.lo[dt], oo + tro.hi[dt]);
          qT[u][dt] = lds_tr8(qq + tro.lo[dt], qq + tro.hi[dt]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const v8 pb = pack8<T>(pm, u);
        const v8 db = pack8<T>(ds, u);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          dv[dt] = Tr::mma(oT[u][dt], pb, dv[dt]);
          dk[dt] = Tr::mma(qT[u][dt], db, dk[dt]);
        }
      }
      lds_mfma_pipeline<4 * NDT, 2, 4>();
      // keep the two 32-row halves apart: hoisting the second half's LDS
      // reads into the first runs the register file out
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmem<0>();
    __syncthreads();
  };
  // Steps [b, e) of one segment; the buffer pair alternates with it & 1.
  auto segment = [&](auto mask, int b, int e) __attribute__((always_inline)) {
    int it = b;
    if (it < e && (it & 1)) step(std::integral_constant<int, 1>{}, mask, it++);
    for (; it + 2 <= e; it += 2) {
      step(std::integral_constant<int, 0>{}, mask, it);
      step(std::integral_constant<int, 1>{}, mask, it + 1);
    }
    if (it < e) step(std::integral_constant<int, 0>{}, mask, it);
  };
  // Per query head, the query blocks run [partially visible][fully
  // visible][partially visible] (the causal diagonal first, the window's end
  // last), so each head is three segments and the common step carries no mask
  // code and no branch: a branch per step would make the compiler copy the
  // dK / dV accumulators at every join.
  if (n_q > 0) {
    const StepRange fr = local_steps(
        full_query_steps(k_lo, BK, BQ, p.causal, p.window, p.n_sink, qfirst, qlast), 0, n_q, false);
    const int f0 = fr.lo, f1 = fr.hi;
    for (int gi = 0; gi < p.G; ++gi) {
      const int b = gi * n_q;
      segment(std::true_type{}, b, b + f0);
      segment(std::false_type{}, b + f0, b + f1);
      segment(std::true_type{}, b + f1, b + n_q);
    }
  }
  // dK / dV rows through the idle Q / dO tiles (every wave is past the last
  // barrier)
  {
    const int row0 = k_lo + 32 * wave;
    rows_out_staged<T, D>(reinterpret_cast<T*>(p.dk) + kv_head + (size_t)row0 * D, S - row0, dk,
                          p.scale, q0s + 32 * wave * D, lane);
    rows_out_staged<T, D>(reinterpret_cast<T*>(p.dv) + kv_head + (size_t)row0 * D, S - row0, dv,
                          1.f, d0s + 32 * wave * D, lane);
  }
}

// ------------------------------------------------------------------------ //
// dkv kernel, two independent work-groups per CU
// ------------------------------------------------------------------------ //
// 4 waves x 32 keys per work-group. K of a wave's keys stays in registers
// (the B operand of S), V of the block is staged once in LDS and 32-row Q /
// dO tiles are double-buffered: about 65 KiB of LDS, so two work-groups share
// a CU and each SIMD holds one wave of each, out of step with each other.
template <typename T, int D, bool ALIBI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkv2_kernel(BwdParams p) {
  constexpr int BK = 128;   // keys per work-group: 4 waves of 32
  constexpr int BQ = 32;    // query rows per streamed block
  constexpr int NS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int KT = BK * D;
  constexpr int QT = BQ * D;
  using Tr = Half16<T>;
  using v8 = typename Tr::v8;

  __shared__ __attribute__((aligned(1024))) T vs[KT];
  // two stages of Q and dO: the stage being read and the stage being loaded
  // are distinct objects, so the compiler needs no wait on the loads in
  // flight before its LDS reads
  __shared__ __attribute__((aligned(1024))) T q0s[QT];
  __shared__ __attribute__((aligned(1024))) T q1s[QT];
  __shared__ __attribute__((aligned(1024))) T d0s[QT];
  __shared__ __attribute__((aligned(1024))) T d1s[QT];
  // [lse * log2(e) (64) | delta (64)] per stage (32 rows used of each)
  __shared__ __attribute__((aligned(16))) float r0s[128];
  __shared__ __attribute__((aligned(16))) float r1s[128];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int BHkv = p.BH / p.G;
  // the order of wg_tile over key blocks. Under the causal mask the first key
  // blocks are the heaviest, with a window too (the sink block is seen by
  // every query block), so every causal grid takes the grouped heaviest-first
  // order; the XCD's K/V heads go in groups of four, so the work-groups on an
  // XCD stream the query tiles of at most four heads (L2 fetches of the
  // headline backward 1669 -> 1061 MB, +0.4 % there, +3.9 % on B4 H32 S4096).
  const Tile tk = wg_tile((int)blockIdx.x, BHkv, p.nkb, p.causal != 0, false);
  const int bkv = tk.bh;
  const int kb = p.causal ? p.nkb - 1 - tk.qb : tk.qb;
  const int S = p.S;
  const int k_lo = kb * BK;
  const int j = k_lo + 32 * wave + col;   // this lane's key
  const size_t kv_head = (size_t)bkv * S * D;
  const T* __restrict__ Kh = reinterpret_cast<const T*>(p.k) + kv_head;
  const T* __restrict__ Vh = uniform_ptr(reinterpret_cast<const T*>(p.v) + kv_head);

  static_assert(sizeof(T) == 2, "byte-form LDS offsets assume 2-byte elements");
  RowXor<D> ro;
  ro.init(lane);
  const uint32_t vo = ro.b + (uint32_t)(64 * D * wave);   // this wave's 32 rows of V
  TrXor<D> tro;
  tro.init(lane);
  RowsDma<T, D, BK, 4> vdma;
  vdma.init(wave, lane);
  RowsDma<T, D, BQ, 4> qdma;
  qdma.init(wave, lane);

  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[dt][r] = 0.f;
      dv[dt][r] = 0.f;
    }
  v8 kf[NS];
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) kf[s2] = load_frag<T>(Kh, j, S, D, 16 * s2 + 8 * h);

  int qfirst, qlast;
  query_range(p, k_lo, min(k_lo + BK, S) - 1, BQ, qfirst, qlast);
  // mask of a partially visible pair for row i = q0 + 4 h + e (e = 8 g + r4)
  // and this lane's key j: keep iff i >= j and (i - j < window or j < n_sink)
  const int big = 1 << 30;
  const bool sinkj = p.window > 0 && j < p.n_sink;
  const int wlen = p.window > 0 ? p.window : big;

  // steps: (query head gi, query block) in order, n_q blocks per head
  const int n_q = qlast - qfirst + 1;
  const int n_iter = n_q > 0 ? p.G * n_q : 0;
  auto tile_src = [&](int it, int& bh, int& q0) __attribute__((always_inline)) {
    const int gi = it / n_q;
    bh = bkv * p.G + gi;   // query head (b * H + h)
    q0 = (qfirst + it - gi * n_q) * BQ;
  };
  // the Q / dO tiles and the lse2 / delta rows of step `it` into one stage
  auto tile_load = [&](T* qd, T* dd, float* rd, int it) __attribute__((always_inline)) {
    int bh, q0;
    tile_src(it, bh, q0);
    const size_t head = (size_t)bh * S * D;
    qdma.load(qd, reinterpret_cast<const T*>(p.q) + head, q0, S, wave);
    qdma.load(dd, reinterpret_cast<const T*>(p.dout) + head, q0, S, wave);
    if (wave == 0) {
      const size_t rb = (size_t)bh * p.Sp + q0;
      rows32_to_lds(rd, p.lse2 + rb, lane);
      rows32_to_lds(rd + 64, p.delta + rb, lane);
    }
  };
  vdma.load(vs, Vh, k_lo, S, wave);
  if (n_iter > 0) tile_load(q0s, d0s, r0s, 0);
  wait_vmem<0>();
  __syncthreads();

  auto step = [&](auto par, auto mask, int it) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    constexpr bool MASK = decltype(mask)::value;
    const T* qs = PAR == 0 ? q0s : q1s;
    const T* dos = PAR == 0 ? d0s : d1s;
    const float* rs = PAR == 0 ? r0s : r1s;
    int bh, q0;
    tile_src(it, bh, q0);
    if (it + 1 < n_iter) {
      if (PAR == 0)
        tile_load(q1s, d1s, r1s, it + 1);
      else
        tile_load(q0s, d0s, r0s, it + 1);
    }
    // Under the causal mask a tile whose rows all precede this wave's keys adds
    // nothing to them (its weights are exact zeros): the wave skips its products.
    if (!MASK || !p.causal || q0 + BQ - 1 >= k_lo + 32 * wave) {
      const float b2 = ALIBI ? p.alibi[bh % p.H] * kLog2e : 0.f;
      const int emin = j - q0 - 4 * h;   // keep iff e >= emin and (e < emin + wlen or sinkj)
      const int ehi = sinkj ? big : emin + wlen - 1;
      // The LDS offsets pass through an empty asm each step, so the read
      // addresses are formed here (one add each) instead of being hoisted out
      // of the loop, where 30-odd of them do not fit the register budget.
      RowXor<D> rl = ro;
      uint32_t vl = vo;
      TrXor<D> tl = tro;
      asm volatile("" : "+v"(rl.b), "+v"(vl), "+v"(tl.b[0]), "+v"(tl.b[1]));
      auto vrow = [&](int s) __attribute__((always_inline)) {
        return at_bytes(vs, vl ^ (32u * s));
      };
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[r] = 0.f;
        dp[r] = 0.f;
      }
      // S = Q K^T (K in registers) and dP = dO V^T (dO, V from LDS), reads
      // pinned two k-steps ahead of their MFMAs (one with ALiBi, whose bias
      // terms need the registers): left free, the scheduler hoists every read
      // and the kernel spills; the other work-group's wave on the SIMD covers
      // the read latency.
      if constexpr (!ALIBI) {
        v8 qa[2], da[2], va[2];
        qa[0] = lds_row8(at_bytes(qs, rl.at(0)));
        qa[1] = lds_row8(at_bytes(qs, rl.at(1)));
        da[0] = lds_row8(at_bytes(dos, rl.at(0)));
        va[0] = lds_row8(vrow(0));
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s + 1 < NS) {
            da[(s + 1) & 1] = lds_row8(at_bytes(dos, rl.at(s + 1)));
            va[(s + 1) & 1] = lds_row8(vrow(s + 1));
          }
          sc = Tr::mma(qa[s & 1], kf[s], sc);
          __builtin_amdgcn_sched_barrier(0);
          if (s + 2 < NS) qa[s & 1] = lds_row8(at_bytes(qs, rl.at(s + 2)));
          dp = Tr::mma(da[s & 1], va[s & 1], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        v8 qa = lds_row8(at_bytes(qs, rl.at(0)));
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const v8 da = lds_row8(at_bytes(dos, rl.at(s))), va = lds_row8(vrow(s));
          sc = Tr::mma(qa, kf[s], sc);
          __builtin_amdgcn_sched_barrier(0);
          if (s + 1 < NS) qa = lds_row8(at_bytes(qs, rl.at(s + 1)));
          dp = Tr::mma(da, va, dp);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // this lane's rows of the block: 8 g + 4 h + (0..3); with ALiBi their
      // lse2 / delta are read one group of four at a time, pinned (all 32 at
      // once ran that build out of registers)
      const uint32_t mw = MASK ? keep_word(emin, ehi, -1, 0) : 0u;
      f32x4 l2[4], dd[4];
      const auto read_rows = [&](int g) {
        l2[g] = *reinterpret_cast<const f32x4*>(rs + 8 * g + 4 * h);
        dd[g] = *reinterpret_cast<const f32x4*>(rs + 64 + 8 * g + 4 * h);
      };
      if constexpr (!ALIBI) {
#pragma unroll
        for (int g = 0; g < 4; ++g) read_rows(g);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if constexpr (ALIBI) read_rows(g);
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int r = 4 * g + e4;
          const int e = 8 * g + e4;
          float x;
          if (ALIBI)
            x = __builtin_fmaf(sc[r], p.c, -b2 * fabsf((float)(e - emin))) - l2[g][e4];
          else
            x = __builtin_fmaf(sc[r], p.c, -l2[g][e4]);
          float pr = fast_exp2(x);
          if (MASK) pr = keep_or(pr, mw, e, 0u);
          sc[r] = pr;                        // P
          dp[r] = pr * (dp[r] - dd[g][e4]);  // dS
        }
        if constexpr (ALIBI) __builtin_amdgcn_sched_barrier(0);
      }
      // P and dS as MFMA B operands (16 rows each half); the fp32 tiles die here
      const v8 pb[2] = {pack8<T>(sc, 0), pack8<T>(sc, 1)};
      const v8 db[2] = {pack8<T>(dp, 0), pack8<T>(dp, 1)};
      __builtin_amdgcn_sched_barrier(0);
      // dV^T += dO^T P and dK^T += Q^T dS: per (16-row half u, 32-wide d tile)
      // the two transposed operands, one pair ahead of its MFMAs
      auto tr_reads = [&](int u, int dt, v8& o, v8& q) __attribute__((always_inline)) {
        const T* qq = qs + 16 * u * D;
        const T* oo = dos + 16 * u * D;
        o = lds_tr8(at_bytes(oo, tl.lo(dt)), at_bytes(oo, tl.hi(dt)));
        q = lds_tr8(at_bytes(qq, tl.lo(dt)), at_bytes(qq, tl.hi(dt)));
      };
      v8 oT, qT;
      tr_reads(0, 0, oT, qT);
#pragma unroll
      for (int x = 0; x < 2 * NDT; ++x) {
        const int u = x / NDT, dt = x % NDT;
        v8 on = oT, qn = qT;
        if (x + 1 < 2 * NDT) tr_reads((x + 1) / NDT, (x + 1) % NDT, on, qn);
        dv[dt] = Tr::mma(oT, pb[u], dv[dt]);
        dk[dt] = Tr::mma(qT, db[u], dk[dt]);
        __builtin_amdgcn_sched_barrier(0);
        oT = on;
        qT = qn;
      }
    }
    wait_vmem<0>();
    __syncthreads();
  };
  auto segment = [&](auto mask, int b, int e) __attribute__((always_inline)) {
    int it = b;
    if (it < e && (it & 1)) step(std::integral_constant<int, 1>{}, mask, it++);
    for (; it + 2 <= e; it += 2) {
      step(std::integral_constant<int, 0>{}, mask, it);
      step(std::integral_constant<int, 1>{}, mask, it + 1);
    }
    if (it < e) step(std::integral_constant<int, 0>{}, mask, it);
  };
  // Per query head [partially visible][fully visible][partially visible]
  // query blocks (the causal diagonal first, the window's end last).
  if (n_q > 0) {
    const StepRange fr = local_steps(
        full_query_steps(k_lo, BK, BQ, p.causal, p.window, p.n_sink, qfirst, qlast), 0, n_q, false);
    const int f0 = fr.lo, f1 = fr.hi;
    for (int gi = 0; gi < p.G; ++gi) {
      const int b = gi * n_q;
      segment(std::true_type{}, b, b + f0);
      segment(std::false_type{}, b + f0, b + f1);
      segment(std::true_type{}, b + f1, b + n_q);
    }
  }
  // dK rows through this wave's own V rows, dV rows through one Q / dO tile
  // (every wave is past the last barrier)
  {
    const int row0 = k_lo + 32 * wave;
    rows_out_staged<T, D>(reinterpret_cast<T*>(p.dk) + kv_head + (size_t)row0 * D, S - row0, dk,
                          p.scale, vs + 32 * wave * D, lane);
    T* const st = wave == 0 ? q0s : wave == 1 ? d0s : wave == 2 ? q1s : d1s;
    rows_out_staged<T, D>(reinterpret_cast<T*>(p.dv) + kv_head + (size_t)row0 * D, S - row0, dv,
                          1.f, st, lane);
  }
}

#define FA_BWD_INST(T, D)                                                \
  template __global__ void fa_bwd_dq_kernel<T, D, false>(BwdParams);     \
  template __global__ void fa_bwd_dq_kernel<T, D, true>(BwdParams);      \
  template __global__ void fa_bwd_dkv_kernel<T, D, false>(BwdParams);    \
  template __global__ void fa_bwd_dkv_kernel<T, D, true>(BwdParams);     \
  template __global__ void fa_bwd_dkv2_kernel<T, D, false>(BwdParams);   \
  template __global__ void fa_bwd_dkv2_kernel<T, D, true>(BwdParams);
FA_BWD_INST(__bf16, 128)
FA_BWD_INST(__bf16, 64)
FA_BWD_INST(_Float16, 128)
FA_BWD_INST(_Float16, 64)
#undef FA_BWD_INST

static_assert(32 * kBwdWaves == kBwdRows && 2 * kBCf == kBwdRows, "tile sizes of the plan");

// ------------------------------------------------------------------------ //
// Scratch of the allocation-free backward: the two per-row arrays (delta and
// lse * log2 e) of flash_attn_bwd_noalloc live in this file-scope device
// array instead of a caller workspace. Every GPU the library runs on holds its
// own copy until the process ends. Host code never passes the array's name to
// a kernel (on the host it is only a stand-in for the device symbol): the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current, and that address is what the kernels receive.
// All calls on one GPU share the array; calls that overlap in time on one GPU
// race on it. Nothing in it needs clearing: the dq kernel writes every padded
// row before the dkv kernel reads it.
// ------------------------------------------------------------------------ //
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

hipError_t bwd_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  constexpr int kMaxDevices = 64;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

template <typename T, int D, bool ALIBI>
static hipError_t launch_bwd_a(const BwdParams& p, hipStream_t st) {
  const unsigned g1 = (unsigned)p.nqb * (unsigned)p.BH;
  hipLaunchKernelGGL((fa_bwd_dq_kernel<T, D, ALIBI>), dim3(g1), dim3(64 * kBwdWaves), 0, st, p);
  const unsigned g2 = (unsigned)p.nkb * (unsigned)(p.BH / p.G);
  // dK/dV: two 4-wave work-groups per CU, or one 4-wave work-group per CU
  // (the host's choice, bwd_dkv_pair)
  if (p.dkv_pair)
    hipLaunchKernelGGL((fa_bwd_dkv2_kernel<T, D, ALIBI>), dim3(g2), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((fa_bwd_dkv_kernel<T, D, ALIBI>), dim3(g2), dim3(64 * kBwdWaves), 0, st, p);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t st) {
  return p.alibi ? launch_bwd_a<T, D, true>(p, st) : launch_bwd_a<T, D, false>(p, st);
}

hipError_t launch_bwd(const BwdParams& p, int D, int dtype, hipStream_t st) {
  if (dtype == kDtypeBF16) {
    if (D == 128) return launch_bwd_t<__bf16, 128>(p, st);
    if (D == 64) return launch_bwd_t<__bf16, 64>(p, st);
  } else if (dtype == kDtypeF16) {
    if (D == 128) return launch_bwd_t<_Float16, 128>(p, st);
    if (D == 64) return launch_bwd_t<_Float16, 64>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
