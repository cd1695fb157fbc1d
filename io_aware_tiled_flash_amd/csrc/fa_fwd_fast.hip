// Fast tiled online-softmax attention forward pass for gfx950: bf16 / f16,
// head dim 64 or 128.
//
// Same algorithm as the generic kernels (Lab 3 page "Tiled attention with
// online softmax"; Lesson 91 deck, slide 11): a query block streams over
// key/value blocks under the online-softmax rescale and writes O / l and the
// logsumexp once. What differs is how the work is fed to the matrix cores:
//
//  * K and V tiles go HBM -> LDS with direct-to-LDS buffer loads
//    (buffer_load_dwordx4 ... lds): no staging registers and, since the
//    per-lane offsets are fixed and the block's position lives in the scalar
//    buffer descriptor, no per-block address arithmetic. The descriptor's
//    size ends at the sequence end, so a ragged last block reads zeros past
//    it. Each wave fills a contiguous 1 KiB run of LDS per instruction, so
//    the XOR swizzles of the LDS layouts are applied on the global side.
//  * K is stored row-major with its 16-byte chunks XOR-swizzled by row, so
//    the 32 lanes reading one chunk column of 32 keys (the A operand of
//    S^T = K Q^T on v_mfma_f32_32x32x16) hit distinct LDS banks.
//  * V is stored row-major (no transpose on the way in) with its 64-byte
//    segments XOR-swizzled by row. The A operand of O^T = V^T P^T needs, per
//    lane, 8 keys of one column d; ds_read_b64_tr_b16 delivers exactly that:
//    in each group of 16 lanes, lane o receives element o%4 of the rows that
//    lanes o/4 + 4k fetched, so lanes fetching V[key0 + r/4][d0 + 4(r%4)..]
//    leave V[key0 + k][d0 + o] in lane o. Two such reads give 8 keys.
//  * P never leaves registers: the S^T accumulator, rounded to the input
//    type, is the B operand of the PV MFMA (key = contraction index, both
//    operands enumerate the keys of a 16-key chunk in the same order).
//  * Lazy rescale: a row's running max only moves (and O, l are only
//    rescaled) when the new block max exceeds it by more than 2^8 in the
//    base-2 exponent; otherwise the stale max is kept and exp2 arguments stay
//    <= 8. The result O / l does not depend on the reference max, and fp32
//    holds the <= 256x larger partial sums without loss. The decision is
//    wave-uniform, so the rescale of O is skipped as a branch.
//  * Masks are applied only to partially visible blocks, with per-lane
//    bounds and compile-time key offsets (two VALU ops per score). The
//    partially visible blocks sit at the two ends of the visiting order, so
//    the loop runs in three segments and only the end segments carry mask
//    code. In those blocks a wave whose rows see none of the keys skips them.
//  * ALiBi (template AL): under the causal mask the bias is linear in the key
//    (AL == 1): one FMA with a compile-time ramp per score and one offset per
//    lane and block, with the block walk running from the diagonal. Without
//    the mask, or for steep slopes, the bias is formed per score (AL == 2).
//
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_kernel.h"
#include "fa_lds.h"

namespace fa {

namespace {

// Per-lane state and block operations shared by both schedules. One wave
// owns 32 query rows; lane (col, h) = (lane & 31, lane >> 5) owns query row
// i = q_lo + 32 * wave_in_block + col and, in every 32-key sub-tile, the keys
// 8 g + 4 h + r (g, r < 4) of the S^T accumulator.
template <typename T, int D, int BR, int AL>
struct Core {
  using Tr = Half16<T>;
  using v8 = typename Tr::v8;
  static constexpr int BC = kBCf;
  static constexpr int NT = BC / 32;   // 32-key sub-tiles
  static constexpr int NDT = D / 32;   // 32-wide d tiles of O^T
  static constexpr int NS = D / 16;    // k-steps of QK^T

  v8 qf[NS];         // Q fragment (B operand of S^T = K Q^T)
  int koff[NS];      // LDS offsets of the K fragment per k-step
  int vdt[NDT];      // LDS offsets of the V^T fragment reads per d tile
  f32x16 oacc[NDT];  // O^T accumulator
  float m_run;       // running max (raw sign-folded score units)
  float mc;          // m_run * c, or 0 while nothing is visible
  float l[4];        // this lane half's running sum, in 4 parts
  float c, tau_raw;  // softmax scale (1 for AL == 2, whose logits come scaled)
  float b2;          // ALiBi slope in base 2 (AL != 0)
  float beta;        // b2 / c: the ALiBi slope in raw score units (AL == 1)
  int i, h, col;

  __device__ __forceinline__ void init(const FwdParams& p, const T* __restrict__ Qh, int q_row,
                                       int lane, int bh) {
    b2 = AL ? p.alibi[bh % p.H] * kLog2e : 0.f;
    h = lane >> 5;
    col = lane & 31;
    i = q_row;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (i < p.S) w = *reinterpret_cast<const u32x4*>(Qh + (size_t)i * D + 16 * s + 8 * h);
      if (p.neg) w ^= 0x80008000u;
      qf[s] = __builtin_bit_cast(v8, w);
    }
    const int sw = k_swz<D>(col);
#pragma unroll
    for (int s = 0; s < NS; ++s) koff[s] = col * D + (((2 * s + h) ^ sw) << 3);
    const int r16 = lane & 15;
    const int grp = (lane >> 4) & 1;
    const int vsw = D == 128 ? ((r16 >> 2) & 3) : ((r16 >> 3) & 1);
    const int vbase = (4 * h + (r16 >> 2)) * D + 16 * grp + 4 * (r16 & 3);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vdt[dt] = vbase + ((dt ^ vsw) << 5);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    m_run = kNegInf;
    mc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) l[k] = 0.f;
    c = (AL == 2) ? 1.f : p.c;
    beta = (AL == 1) ? b2 / p.c : 0.f;
    tau_raw = kTau / c;
  }

  // S^T = K Q^T for the K tile at ks. The two 32-key sub-tiles alternate
  // (independent accumulators back to back), and the K fragment reads run
  // kQkAhead MFMAs ahead of their use: left to itself the scheduler keeps only
  // one or two reads in flight, and each MFMA then waits out an LDS latency.
  static constexpr int kQkAhead = 4;
  __device__ __forceinline__ void qk(f32x16 (&acc)[NT], const T* ks) const {
    v8 a[NS][NT];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        a[s][t] = __builtin_bit_cast(v8, *reinterpret_cast<const u32x4*>(ks + 32 * t * D + koff[s]));
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = Tr::mma(a[s][t], qf[s], acc[t]);
    // Schedule: kQkAhead reads, then (one MFMA, one read) pairs, then the
    // last MFMAs. Mask bits: 0x100 LDS read, 0x008 MFMA.
    __builtin_amdgcn_sched_group_barrier(0x100, kQkAhead, 0);
#pragma unroll
    for (int u = 0; u < NS * NT - kQkAhead; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kQkAhead, 0);
  }

  // Mask the scores of a partially visible block: key j = k0 + 4h + e,
  // e = 32t + 8g + r.
  __device__ __forceinline__ void mask(f32x16 (&acc)[NT], const FwdParams& p, int k0) const {
    const int jb = k0 + 4 * h;
    const int hi = (p.causal ? min(i, p.S - 1) : p.S - 1) - jb;
    if (p.window > 0) {
      const int lo = i - p.window + 1 - jb;
      const int sk = p.n_sink - 1 - jb;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = 32 * t + 8 * (r >> 2) + (r & 3);
          const bool keep = (e <= hi) & ((e >= lo) | (e <= sk));
          acc[t][r] = keep ? acc[t][r] : kNegInf;
        }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = 32 * t + 8 * (r >> 2) + (r & 3);
          acc[t][r] = (e <= hi) ? acc[t][r] : kNegInf;
        }
    }
  }

  // Online softmax with lazy rescale: turns the (masked) scores into p,
  // adds them to l and packs them into the B operands of the PV MFMA.
  // off (AL == 1 only): this lane's ALiBi offset for the block, added to
  // every score the lane holds after the per-key ramp (see alibi_ramp).
  __device__ __forceinline__ void softmax(f32x16 (&acc)[NT], v8 (&pb)[NT][2], float off = 0.f) {
    // Row max: one chain of three-input maxima per 32-key sub-tile, the
    // first seeded with the running max (the lane pair holding a row shares
    // it), then the exchange across the half-waves.
    // Sub-tile 0: the running max and 16 scores (8 v_maximum3); later
    // sub-tiles: 15 scores (7), their 16th joins the final maximum3. With
    // the ALiBi offset the running max joins after the offset is added.
    float mj = (AL == 1) ? vmax(acc[0][0], acc[0][1]) : vmax(vmax(m_run, acc[0][0]), acc[0][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mj = vmax(vmax(mj, acc[0][r]), acc[0][r + 1]);
#pragma unroll
    for (int t = 1; t < NT; ++t) {
      float a = vmax(vmax(acc[t][0], acc[t][1]), acc[t][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) a = vmax(vmax(a, acc[t][r]), acc[t][r + 1]);
      mj = vmax(vmax(mj, a), acc[t][15]);
    }
    // (each half-wave adds its own offset, 4 beta apart, before the exchange)
    const float m_new = (AL == 1) ? vmax(m_run, xhalf_max(mj + off)) : xhalf_max(mj);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + tau_raw)) {
      const float mc_new = (m_new == kNegInf) ? 0.f : m_new * c;
      const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(mc - mc_new);
      m_run = m_new;
      mc = mc_new;
#pragma unroll
      for (int k = 0; k < 4; ++k) l[k] *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    const float bo = (AL == 1) ? __builtin_fmaf(off, c, -mc) : -mc;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(__builtin_fmaf(acc[t][r], c, bo));
        acc[t][r] = e;
        l[r & 3] += e;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 w;
        w[0] = pack2<T>(acc[t][8 * u + 0], acc[t][8 * u + 1]);
        w[1] = pack2<T>(acc[t][8 * u + 2], acc[t][8 * u + 3]);
        w[2] = pack2<T>(acc[t][8 * u + 4], acc[t][8 * u + 5]);
        w[3] = pack2<T>(acc[t][8 * u + 6], acc[t][8 * u + 7]);
        pb[t][u] = __builtin_bit_cast(v8, w);
      }
    }
  }

  // O^T += V^T P^T for the V tile at vs (two transposed reads per operand).
  __device__ __forceinline__ void pv(const T* vs, const v8 (&pb)[NT][2]) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const T* vk = vs + (32 * t + 16 * u) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const u32x2 lo = lds_tr_read(vk + vdt[dt]);
          const u32x2 hi = lds_tr_read(vk + 8 * D + vdt[dt]);
          const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
          oacc[dt] = Tr::mma(__builtin_bit_cast(v8, w), pb[t][u], oacc[dt]);
        }
      }
  }

  // Partial result of a key split: O_r = O / l in fp32 and LSE_r into the
  // workspace ([split][B*H][S][D] and [split][B*H][S]); a row that saw no key
  // of this split gets (0, -inf).
  __device__ __forceinline__ void epilogue_partial(const FwdParams& p, int split, int bh) {
    const float l_tot = xhalf_sum((l[0] + l[1]) + (l[2] + l[3]));
    if (i < p.S) {
      const size_t row = ((size_t)split * p.BH + bh) * (size_t)p.S + i;
      const bool any = l_tot > 0.f;
      const float inv = any ? 1.f / l_tot : 0.f;
      float* __restrict__ Op = p.o_part + row * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * dt + 8 * g + 4 * h;
          f32x4 w = {oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv,
                     oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(Op + d) = w;
        }
      if (h == 0) p.lse_part[row] = any ? (mc + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
  }

  // O = O / l (both lane halves' partial sums), LSE = (mc + log2 l) ln 2.
  __device__ __forceinline__ void epilogue(const FwdParams& p, size_t head, int bh) {
    const float l_tot = xhalf_sum((l[0] + l[1]) + (l[2] + l[3]));
    if (i < p.S) {
      const float inv = 1.f / l_tot;
      T* __restrict__ Oh = reinterpret_cast<T*>(p.o) + head + (size_t)i * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * dt + 8 * g + 4 * h;
          u32x2 w;
          w[0] = pack2<T>(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv);
          w[1] = pack2<T>(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(Oh + d) = w;
        }
      if (h == 0) p.lse[(size_t)bh * p.S + i] = (mc + fast_log2(l_tot)) * kLn2;
    }
  }
};

}  // namespace

// ------------------------------------------------------------------------ //
// The kernel. Every wave runs QK^T, mask, softmax and PV for block j while
// the direct-to-LDS loads of block j+1 land in the other K/V buffer pair; one
// barrier per block. The two buffer pairs are distinct __shared__ objects and
// the block loop is unrolled by two, so every LDS access names its buffer at
// compile time: the compiler can then tell the DMA target from the buffer
// being read and does not wait for the in-flight loads before each read (it
// would have to if both were slots of one array picked at run time).
// ------------------------------------------------------------------------ //
template <typename T, int D, int NW, int AL>
__device__ __forceinline__ void fwd_body(const FwdParams& p, T* k0s, T* v0s, T* k1s, T* v1s) {
  constexpr int BR = 32 * NW;
  constexpr int BC = kBCf;
  using C = Core<T, D, BR, AL>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform: LDS destinations of the tile loads (m0) stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // With a key split, work-group id = split * (nqb * BH) + (the id of the
  // unsplit launch); each split takes a contiguous share of the key blocks.
  const int per = p.nqb * p.BH;
  const int split = (int)blockIdx.x / per;
  int qb, bh;
  wg_coords(p, (int)blockIdx.x - split * per, qb, bh);
  const int S = p.S;
  const int q_lo = qb * BR;
  const size_t head = (size_t)bh * (size_t)S * D;
  const size_t kv_head = (size_t)(bh / p.G) * (size_t)S * D;
  const T* __restrict__ Qh = reinterpret_cast<const T*>(p.q) + head;
  // K/V head bases are wave-uniform; moved to scalar registers once here, the
  // per-block descriptor arithmetic of the tile loads stays scalar.
  const T* __restrict__ Kh = uniform_ptr(reinterpret_cast<const T*>(p.k) + kv_head);
  const T* __restrict__ Vh = uniform_ptr(reinterpret_cast<const T*>(p.v) + kv_head);

  const BlockRange br = block_range<BR, BC>(q_lo, S, p.causal, p.window, p.n_sink);
  const int n_all = br.count();
  const int it_b = (int)((int64_t)split * n_all / p.n_split);
  const int n_iter = (int)((int64_t)(split + 1) * n_all / p.n_split) - it_b;
  // key block of the t-th step of this work-group. With ALiBi under the
  // causal mask the walk runs backwards, from the diagonal: the bias only
  // falls with distance, so the first blocks hold the row maximum and the
  // running max seldom moves afterwards (forwards, it would move, and O be
  // rescaled, at nearly every block of the steeper heads).
  auto kb = [&](int t) __attribute__((always_inline)) {
    return br.kb(it_b + (AL == 1 ? n_iter - 1 - t : t));
  };
  if (p.block_pairs && tid == 0) atomicAdd(p.block_pairs, (unsigned long long)n_iter);

  TileDma<T, D, NW, false> kdma;
  TileDma<T, D, NW, true> vdma;
  kdma.init(wave, lane);
  vdma.init(wave, lane);

  C core;
  if (n_iter > 0) {
    // Block 0 in flight while Q is fetched.
    kdma.load(k0s, Kh, kb(0) * BC, S, wave);
    vdma.load(v0s, Vh, kb(0) * BC, S, wave);
  }
  core.init(p, Qh, q_lo + 32 * wave + (lane & 31), lane, bh);
  wait_vmem<0>();
  __syncthreads();

  // Step `it` computed from buffer pair PAR while step it+1 loads into the other.
  // MASK selects the masked variant at compile time: the visiting order is
  // [partially visible blocks][fully visible blocks][partially visible
  // blocks] (sinks and the window's first blocks, the interior, the causal
  // diagonal), and each segment runs its own copy of the loop, so the common
  // fully visible step carries no mask code and no branch around it.
  auto step = [&](auto par, auto mask, int it) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    T* kc = PAR == 0 ? k0s : k1s;
    T* vc = PAR == 0 ? v0s : v1s;
    T* kn = PAR == 0 ? k1s : k0s;
    T* vn = PAR == 0 ? v1s : v0s;
    if (it + 1 < n_iter) {
      const int k1 = kb(it + 1) * BC;
      kdma.load(kn, Kh, k1, S, wave);
      vdma.load(vn, Vh, k1, S, wave);
    }
    // In a partially visible block, a wave whose 32 rows see none of its keys
    // (above the causal diagonal, or before the window) skips the block.
    const int k0 = kb(it) * BC;
    if (!decltype(mask)::value ||
        !block_hidden<BC>(q_lo + 32 * wave, q_lo + 32 * wave + 31, k0, p.causal, p.window,
                          p.n_sink)) {
      f32x16 sacc[C::NT];
      core.qk(sacc, kc);
      if (decltype(mask)::value) core.mask(sacc, p, k0);
      if (AL == 2) alibi_logits<C::NT>(sacc, p.c, core.b2, core.i, k0 + 4 * core.h);
      if (AL == 1) alibi_ramp<C::NT>(sacc, core.beta);
      typename C::v8 pb[C::NT][2];
      core.softmax(sacc, pb, AL == 1 ? core.beta * (float)(k0 + 4 * core.h - core.i) : 0.f);
      core.pv(vc, pb);
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
  int f0 = 0;
  while (f0 < n_iter && !block_full<BR, BC>(q_lo, kb(f0) * BC, S, p.causal, p.window, p.n_sink))
    ++f0;
  int f1 = f0;
  while (f1 < n_iter && block_full<BR, BC>(q_lo, kb(f1) * BC, S, p.causal, p.window, p.n_sink))
    ++f1;
  segment(std::true_type{}, 0, f0);
  segment(std::false_type{}, f0, f1);
  segment(std::true_type{}, f1, n_iter);
  if (p.o_part)
    core.epilogue_partial(p, split, bh);
  else
    core.epilogue(p, head, bh);
}

template <typename T, int D, int NW, int AL>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fa_fwd_fast_kernel(FwdParams p) {
  constexpr int TILE = kBCf * D;
  __shared__ __attribute__((aligned(1024))) T k0s[TILE];
  __shared__ __attribute__((aligned(1024))) T v0s[TILE];
  __shared__ __attribute__((aligned(1024))) T k1s[TILE];
  __shared__ __attribute__((aligned(1024))) T v1s[TILE];
  if constexpr (AL == 1) {
    // The linear ALiBi form adds the bias as beta (j - i) in parts of size up
    // to beta * 64 and more; for steep slopes those parts would swamp the
    // score's own bits, so such heads take the per-score |i - j| form.
    const int per = p.nqb * p.BH;
    int qb, bh;
    wg_coords(p, (int)blockIdx.x % per, qb, bh);
    if (fabsf(p.alibi[bh % p.H] * kLog2e) <= kAlibiLinMaxB2)
      fwd_body<T, D, NW, 1>(p, k0s, v0s, k1s, v1s);
    else
      fwd_body<T, D, NW, 2>(p, k0s, v0s, k1s, v1s);
  } else {
    fwd_body<T, D, NW, AL>(p, k0s, v0s, k1s, v1s);
  }
}

// ------------------------------------------------------------------------ //
// Host side.
// ------------------------------------------------------------------------ //
bool fast_supported(int D, int dtype) {
  return (dtype == kDtypeBF16 || dtype == kDtypeF16) && (D == 64 || D == 128);
}
int fast_tile_keys() { return kBCf; }

// Explicit instantiations: with several instantiations of the kernel template
// in one translation unit, the host pass emitted launch stubs only for the
// first boolean variant it met; naming each one here makes all of them exist.
#define FA_FAST_INST(T, D, NW)                                         \
  template __global__ void fa_fwd_fast_kernel<T, D, NW, 0>(FwdParams); \
  template __global__ void fa_fwd_fast_kernel<T, D, NW, 1>(FwdParams); \
  template __global__ void fa_fwd_fast_kernel<T, D, NW, 2>(FwdParams);
FA_FAST_INST(__bf16, 128, 8)
FA_FAST_INST(__bf16, 128, 4)
FA_FAST_INST(__bf16, 64, 8)
FA_FAST_INST(__bf16, 64, 4)
FA_FAST_INST(_Float16, 128, 8)
FA_FAST_INST(_Float16, 128, 4)
FA_FAST_INST(_Float16, 64, 8)
FA_FAST_INST(_Float16, 64, 4)
#undef FA_FAST_INST

template <typename T, int D, int AL>
static void launch_fast_a(const FwdParams& p, int nw, hipStream_t st) {
  const unsigned grid = (unsigned)p.nqb * (unsigned)p.BH * (unsigned)p.n_split;
  if (nw == 8)
    hipLaunchKernelGGL((fa_fwd_fast_kernel<T, D, 8, AL>), dim3(grid), dim3(512), 0, st, p);
  else
    hipLaunchKernelGGL((fa_fwd_fast_kernel<T, D, 4, AL>), dim3(grid), dim3(256), 0, st, p);
}

// ALiBi variants: under the causal mask every visible key has j <= i, so the
// bias -slope |i - j| = slope (j - i) is linear in the key and costs one FMA
// per score (AL = 1). Without the mask, or with a scale so small that
// slope / scale would not be a usable number, the bias is formed per score
// with its absolute value (AL = 2).
template <typename T, int D>
static hipError_t launch_fast_t(const FwdParams& p, int nw, hipStream_t st) {
  if (!p.alibi)
    launch_fast_a<T, D, 0>(p, nw, st);
  else if (p.causal && p.c >= kAlibiMinScale)
    launch_fast_a<T, D, 1>(p, nw, st);
  else
    launch_fast_a<T, D, 2>(p, nw, st);
  return hipGetLastError();
}

hipError_t launch_fast(const FwdParams& p, int D, int dtype, int nw, hipStream_t st) {
  if (dtype == kDtypeBF16) {
    if (D == 128) return launch_fast_t<__bf16, 128>(p, nw, st);
    if (D == 64) return launch_fast_t<__bf16, 64>(p, nw, st);
  } else if (dtype == kDtypeF16) {
    if (D == 128) return launch_fast_t<_Float16, 128>(p, nw, st);
    if (D == 64) return launch_fast_t<_Float16, 64>(p, nw, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
