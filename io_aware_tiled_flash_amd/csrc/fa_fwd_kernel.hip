// Tiled online-softmax attention forward pass for gfx950 (MI355X, CDNA4).
//
// What is computed (Lab 3 page "Tiled attention with online softmax", its
// tiled loop; Lesson 91 deck, slide 11 "Online softmax: tiled update
// equations"): a block of query rows streams over key/value blocks keeping a
// running max m, a running denominator l and an output accumulator O; each
// new block rescales the old state by exp(m_old - m_new) and adds
// exp(S - m_new) V; O / l and the row logsumexp are written once at the end.
// Blocks the causal / window mask hides entirely are never loaded (Lab 3,
// its causal block bound and the block-pair exercise); partially hidden
// blocks are masked per element, fully visible ones pay no mask work.
//
// gfx950 mapping
//  * One work-group = 4 waves = 128 query rows of one (batch, head); each
//    wave owns 32 query rows. Keys stream in blocks of BC = 64.
//  * Scores are formed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16
//    (bf16/f16) or v_mfma_f32_32x32x2f32 (f32): the K tile (from LDS) is the
//    A operand and the wave's Q rows, held in registers for the whole kernel,
//    are the B operand. In the 32x32 accumulator layout each lane then holds
//    one query row (its column, lane & 31) and 16 keys per 32-key sub-tile,
//    the other 16 sitting in lane ^ 32. Row max / row sum are in-lane
//    reductions plus one v_permlane32_swap exchange.
//  * The same accumulator registers, rounded to the input type, are directly
//    the B operand of O^T += V^T P^T (the key index is the contraction index;
//    both operands enumerate keys in the same permuted order), so P never
//    leaves registers. V is stored transposed in LDS in that key order so
//    each lane fetches its A fragment with one 16-byte LDS read.
//  * K / V tiles are double-buffered in LDS: the next tile's global loads
//    are issued before the current tile's math and written to the other
//    buffer afterwards; one barrier per tile.
//  * exp is the hardware base-2 exponential with log2(e) folded into the
//    scale; the running max and LSE are kept in that base-2 domain.
//  * Work-groups are ordered heaviest-first under the causal mask, and all
//    query blocks of one (batch, head) land on the same XCD (work-group id
//    modulo 8 picks the XCD; B*H consecutive ids hold distinct heads).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_kernel.h"

namespace fa {

namespace {
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;   // query rows per work-group
constexpr int kBC = 64;            // keys per streamed block
}  // namespace

// ------------------------------------------------------------------------ //
// Online-softmax update for one K block, shared by both element paths.
// sacc[t][r] holds raw scores (sign-folded Q . K) for keys
//   j = k0 + 32 t + 8 (r >> 2) + 4 h + (r & 3)   of query row i.
// Turns them into p = exp2(c s - m2) in place and returns alpha. With ALIBI
// the scores first become base-2 logits c s - b2 |i - j| and the rest runs
// with a unit scale.
// ------------------------------------------------------------------------ //
template <int NT, bool ALIBI>
__device__ __forceinline__ float softmax_step(f32x16 (&sacc)[NT], bool full, int i, int k0, int h,
                                              const FwdParams& p, float b2, float& m2, float& l) {
  if (!full) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = k0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
        const float x = sacc[t][r];
        sacc[t][r] = keep_ij(i, j, p.S, p.causal, p.window, p.n_sink) ? x : kNegInf;
      }
  }
  if (ALIBI) alibi_logits<NT>(sacc, p.c, b2, i, k0 + 4 * h);
  float mt = sacc[0][0];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[t][r]);
  mt = xhalf_max(mt);
  const float c = ALIBI ? 1.f : p.c;
  float m2_new = fmaxf(m2, mt * c);                 // c > 0, so c*max = max of c*s
  float m2_use = (m2_new == kNegInf) ? 0.f : m2_new;
  float alpha = fast_exp2(m2 - m2_use);             // m2 = -inf (nothing seen) -> 0
  float rs = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float e = fast_exp2(__builtin_fmaf(sacc[t][r], c, -m2_use));
      sacc[t][r] = e;
      rs += e;
    }
  l = l * alpha + rs;
  m2 = m2_new;
  return alpha;
}

// ------------------------------------------------------------------------ //
// bf16 / f16 kernel.
// ------------------------------------------------------------------------ //
// Waves per SIMD the kernel is built for. At D <= 32 it needs at most 115
// registers and 19 KiB of LDS per work-group, so four work-groups share a CU
// (four waves per SIMD). Built for two, the kernel descriptor reserved 169
// registers and only two fit. Same-process A/B (bitwise equal): +27 % causal
// B4 H32 S4096 D32, +25 % unmasked B4 H32 S2048 D16, +36 % with a 512-key
// window at D32.
template <int D>
constexpr int half_waves_per_simd() {
  return D <= 32 ? 4 : 2;
}

template <typename T, int D, bool ALIBI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    half_waves_per_simd<D>(), half_waves_per_simd<D>()))) void fa_fwd_half_kernel(FwdParams p) {
  using Tr = Half16<T>;
  using v8 = typename Tr::v8;
  constexpr int DP = D < 32 ? 32 : D;     // M extent of the O^T accumulator
  constexpr int KSTR = D + 8;             // K tile row stride (elements), +16 B pad
  constexpr int VSTR = kBC + 8;           // V^T tile row stride (elements), +16 B pad
  constexpr int NT = kBC / 32;            // 32-key sub-tiles per block
  constexpr int NDT = DP / 32;            // 32-wide d tiles of O^T
  constexpr int NS = D / 16;              // k-steps of the QK contraction
  constexpr int KCH = kBC * D / 8;        // 16-byte chunks in a K tile
  constexpr int KPT = (KCH + kThreads - 1) / kThreads;
  constexpr int VUN = (kBC / 4) * (D / 8);  // 4-key x 8-d units in a V tile
  constexpr int VPT = (VUN + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) T Ks[2][kBC * KSTR];
  __shared__ __attribute__((aligned(16))) T Vt[2][DP * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  int qb, bh;
  wg_coords(p, qb, bh);
  const int S = p.S;
  const int q_lo = qb * kBR;
  const int i = q_lo + 32 * wave + col;   // this lane's query row
  const size_t head = (size_t)bh * (size_t)S * D;
  const size_t kv_head = (size_t)(bh / p.G) * (size_t)S * D;
  const T* __restrict__ Qh = reinterpret_cast<const T*>(p.q) + head;
  const T* __restrict__ Kh = reinterpret_cast<const T*>(p.k) + kv_head;
  const T* __restrict__ Vh = reinterpret_cast<const T*>(p.v) + kv_head;
  const float b2 = ALIBI ? p.alibi[bh % p.H] * kLog2e : 0.f;

  if (D < 32) {   // O^T rows d >= D read zeros from V^T
    for (int e = tid; e < 2 * DP * VSTR; e += kThreads) (&Vt[0][0])[e] = T(0.f);
  }

  // Q fragment: lane holds Q[i][16 s + 8 h .. +7] for s < D/16, sign-folded.
  v8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (i < S) w = *reinterpret_cast<const u32x4*>(Qh + (size_t)i * D + 16 * s + 8 * h);
    if (p.neg) w ^= 0x80008000u;
    qf[s] = __builtin_bit_cast(v8, w);
  }

  const BlockRange br = block_range<kBR, kBC>(q_lo, S, p.causal, p.window, p.n_sink);
  const int n_iter = br.count();
  if (p.block_pairs && tid == 0) atomicAdd(p.block_pairs, (unsigned long long)n_iter);

  u32x4 kreg[KPT];
  u32x4 vreg[VPT][4];

  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      int c = tid + kThreads * r;
      int row = c / (D / 8), c8 = c % (D / 8);
      u32x4 w = {0u, 0u, 0u, 0u};
      if ((KCH % kThreads == 0 || c < KCH) && k0 + row < S)
        w = *reinterpret_cast<const u32x4*>(Kh + (size_t)(k0 + row) * D + 8 * c8);
      kreg[r] = w;
    }
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      int u = tid + kThreads * r;
      int jq = u / (D / 8), dq = u % (D / 8);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        int j = k0 + 4 * jq + a;
        u32x4 w = {0u, 0u, 0u, 0u};
        if ((VUN % kThreads == 0 || u < VUN) && j < S)
          w = *reinterpret_cast<const u32x4*>(Vh + (size_t)j * D + 8 * dq);
        vreg[r][a] = w;
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      int c = tid + kThreads * r;
      if (KCH % kThreads == 0 || c < KCH) {
        int row = c / (D / 8), c8 = c % (D / 8);
        *reinterpret_cast<u32x4*>(&Ks[buf][row * KSTR + 8 * c8]) = kreg[r];
      }
    }
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      int u = tid + kThreads * r;
      if (VUN % kThreads == 0 || u < VUN) {
        int jq = u / (D / 8), dq = u % (D / 8);
        // keys 4jq..4jq+3 -> permuted position inside their 16-key chunk:
        // key quad a (0..3) goes to [0, 8, 4, 12][a], so that MFMA lane half h
        // finds its keys {4h..4h+3, 8+4h..8+4h+3} at 8h..8h+7.
        int j4 = 4 * jq;
        int a = (j4 & 15) >> 2;
        int pos = (j4 & ~15) + ((a & 1) << 3) + ((a >> 1) << 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          int wsel = e >> 1;
          uint32_t x0 = vreg[r][0][wsel], x1 = vreg[r][1][wsel];
          uint32_t x2 = vreg[r][2][wsel], x3 = vreg[r][3][wsel];
          u32x2 out;
          if (e & 1) {
            out[0] = (x0 >> 16) | (x1 & 0xffff0000u);
            out[1] = (x2 >> 16) | (x3 & 0xffff0000u);
          } else {
            out[0] = (x0 & 0xffffu) | (x1 << 16);
            out[1] = (x2 & 0xffffu) | (x3 << 16);
          }
          *reinterpret_cast<u32x2*>(&Vt[buf][(8 * dq + e) * VSTR + pos]) = out;
        }
      }
    }
  };

  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m2 = kNegInf, l = 0.f;

  gload(br.kb(0) * kBC);
  if (D < 32) __syncthreads();   // zero-fill of V^T before the first tile store
  lstore(0);
  __syncthreads();

  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    const int k0 = br.kb(it) * kBC;
    if (it + 1 < n_iter) gload(br.kb(it + 1) * kBC);

    // S^T = K Q^T
    f32x16 sacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        v8 a = __builtin_bit_cast(v8, *reinterpret_cast<const u32x4*>(
                                          &Ks[buf][(32 * t + col) * KSTR + 16 * s + 8 * h]));
        sacc[t] = Tr::mma(a, qf[s], sacc[t]);
      }
    }

    const bool full = block_full<kBR, kBC>(q_lo, k0, S, p.causal, p.window, p.n_sink);
    const float alpha = softmax_step<NT, ALIBI>(sacc, full, i, k0, h, p, b2, m2, l);

#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;

    // P^T as B operands: keys {4h+r, 8+4h+r} of each 16-key chunk (t, u).
    v8 pb[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 w;
        w[0] = pack2<T>(sacc[t][8 * u + 0], sacc[t][8 * u + 1]);
        w[1] = pack2<T>(sacc[t][8 * u + 2], sacc[t][8 * u + 3]);
        w[2] = pack2<T>(sacc[t][8 * u + 4], sacc[t][8 * u + 5]);
        w[3] = pack2<T>(sacc[t][8 * u + 6], sacc[t][8 * u + 7]);
        pb[t][u] = __builtin_bit_cast(v8, w);
      }

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          v8 a = __builtin_bit_cast(v8, *reinterpret_cast<const u32x4*>(
                                            &Vt[buf][(32 * dt + col) * VSTR + 32 * t + 16 * u + 8 * h]));
          oacc[dt] = Tr::mma(a, pb[t][u], oacc[dt]);
        }

    if (it + 1 < n_iter) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O / l (both lane halves' partial sums), LSE = (m2 + log2 l) ln 2.
  const float l_tot = xhalf_sum(l);
  if (i < S) {
    const float inv = 1.f / l_tot;
    T* __restrict__ Oh = reinterpret_cast<T*>(p.o) + head + (size_t)i * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        int d = 32 * dt + 8 * g + 4 * h;
        if (d < D) {
          u32x2 w;
          w[0] = pack2<T>(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv);
          w[1] = pack2<T>(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(Oh + d) = w;
        }
      }
    if (h == 0) p.lse[(size_t)bh * S + i] = (m2 + fast_log2(l_tot)) * kLn2;
  }
}

// ------------------------------------------------------------------------ //
// f32 kernel: v_mfma_f32_32x32x2f32, same structure.
// K = 2 per MFMA: lane half h supplies contraction slot h.
//  * QK: step s pairs d = s (h = 0) with d = D/2 + s (h = 1), so each lane
//    reads a contiguous run of its K row / Q row.
//  * PV: step (t, g, r) pairs key 32t + 8g + r (h = 0) with key +4 (h = 1),
//    exactly the accumulator's own key for that register; V^T keeps, per
//    32-key chunk, keys {8g + 4h + r} of half h at 16h + 4g + r.
// ------------------------------------------------------------------------ //
template <int D, bool ALIBI>
__global__ __launch_bounds__(kThreads) void fa_fwd_f32_kernel(FwdParams p) {
  constexpr int DP = D < 32 ? 32 : D;
  constexpr int KSTR = D + 4;
  constexpr int VSTR = kBC + 4;
  constexpr int NT = kBC / 32;
  constexpr int NDT = DP / 32;
  constexpr int DH = D / 2;
  constexpr int KCH = kBC * D / 4;          // 16-byte chunks in a K tile
  constexpr int KPT = (KCH + kThreads - 1) / kThreads;
  constexpr int VUN = (kBC / 4) * (D / 4);  // 4-key x 4-d units in a V tile
  constexpr int VPT = (VUN + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) float Ks[2][kBC * KSTR];
  __shared__ __attribute__((aligned(16))) float Vt[2][DP * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  int qb, bh;
  wg_coords(p, qb, bh);
  const int S = p.S;
  const int q_lo = qb * kBR;
  const int i = q_lo + 32 * wave + col;
  const size_t head = (size_t)bh * (size_t)S * D;
  const size_t kv_head = (size_t)(bh / p.G) * (size_t)S * D;
  const float* __restrict__ Qh = reinterpret_cast<const float*>(p.q) + head;
  const float* __restrict__ Kh = reinterpret_cast<const float*>(p.k) + kv_head;
  const float* __restrict__ Vh = reinterpret_cast<const float*>(p.v) + kv_head;
  const float b2 = ALIBI ? p.alibi[bh % p.H] * kLog2e : 0.f;

  if (D < 32) {
    for (int e = tid; e < 2 * DP * VSTR; e += kThreads) (&Vt[0][0])[e] = 0.f;
  }

  float qf[DH];
#pragma unroll
  for (int s4 = 0; s4 < DH / 4; ++s4) {
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    if (i < S) w = *reinterpret_cast<const f32x4*>(Qh + (size_t)i * D + h * DH + 4 * s4);
    if (p.neg) w = -w;
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[4 * s4 + e] = w[e];
  }

  const BlockRange br = block_range<kBR, kBC>(q_lo, S, p.causal, p.window, p.n_sink);
  const int n_iter = br.count();
  if (p.block_pairs && tid == 0) atomicAdd(p.block_pairs, (unsigned long long)n_iter);

  f32x4 kreg[KPT];
  f32x4 vreg[VPT][4];

  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      int c = tid + kThreads * r;
      int row = c / (D / 4), c4 = c % (D / 4);
      f32x4 w = {0.f, 0.f, 0.f, 0.f};
      if ((KCH % kThreads == 0 || c < KCH) && k0 + row < S)
        w = *reinterpret_cast<const f32x4*>(Kh + (size_t)(k0 + row) * D + 4 * c4);
      kreg[r] = w;
    }
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      int u = tid + kThreads * r;
      int jq = u / (D / 4), dq = u % (D / 4);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        int j = k0 + 4 * jq + a;
        f32x4 w = {0.f, 0.f, 0.f, 0.f};
        if ((VUN % kThreads == 0 || u < VUN) && j < S)
          w = *reinterpret_cast<const f32x4*>(Vh + (size_t)j * D + 4 * dq);
        vreg[r][a] = w;
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      int c = tid + kThreads * r;
      if (KCH % kThreads == 0 || c < KCH) {
        int row = c / (D / 4), c4 = c % (D / 4);
        *reinterpret_cast<f32x4*>(&Ks[buf][row * KSTR + 4 * c4]) = kreg[r];
      }
    }
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      int u = tid + kThreads * r;
      if (VUN % kThreads == 0 || u < VUN) {
        int jq = u / (D / 4), dq = u % (D / 4);
        int j4 = 4 * jq;                       // keys j4..j4+3 share (g, h)
        int g = (j4 & 31) >> 3, hh = (j4 & 7) >> 2;
        int pos = (j4 & ~31) + 16 * hh + 4 * g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f32x4 out = {vreg[r][0][e], vreg[r][1][e], vreg[r][2][e], vreg[r][3][e]};
          *reinterpret_cast<f32x4*>(&Vt[buf][(4 * dq + e) * VSTR + pos]) = out;
        }
      }
    }
  };

  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m2 = kNegInf, l = 0.f;

  gload(br.kb(0) * kBC);
  if (D < 32) __syncthreads();
  lstore(0);
  __syncthreads();

  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    const int k0 = br.kb(it) * kBC;
    if (it + 1 < n_iter) gload(br.kb(it + 1) * kBC);

    f32x16 sacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
      const float* krow = &Ks[buf][(32 * t + col) * KSTR + h * DH];
#pragma unroll
      for (int s4 = 0; s4 < DH / 4; ++s4) {
        f32x4 a = *reinterpret_cast<const f32x4*>(krow + 4 * s4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[4 * s4 + e], sacc[t], 0, 0, 0);
      }
    }

    const bool full = block_full<kBR, kBC>(q_lo, k0, S, p.causal, p.window, p.n_sink);
    const float alpha = softmax_step<NT, ALIBI>(sacc, full, i, k0, h, p, b2, m2, l);

#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;

#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float* vrow = &Vt[buf][(32 * dt + col) * VSTR + 32 * t + 16 * h];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 a = *reinterpret_cast<const f32x4*>(vrow + 4 * g);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[r], sacc[t][4 * g + r], oacc[dt], 0, 0, 0);
        }
      }

    if (it + 1 < n_iter) lstore(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = xhalf_sum(l);
  if (i < S) {
    const float inv = 1.f / l_tot;
    float* __restrict__ Oh = reinterpret_cast<float*>(p.o) + head + (size_t)i * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        int d = 32 * dt + 8 * g + 4 * h;
        if (d < D) {
          f32x4 w = {oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv,
                     oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(Oh + d) = w;
        }
      }
    if (h == 0) p.lse[(size_t)bh * S + i] = (m2 + fast_log2(l_tot)) * kLn2;
  }
}

// ------------------------------------------------------------------------ //
// Host-side launch.
// ------------------------------------------------------------------------ //
static_assert(kBR == kGenericBR && kBC == kGenericBC, "tile sizes of the plan");

template <typename K>
static hipError_t launch_kernel(K kernel, const FwdParams& p, unsigned grid, hipStream_t st) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <typename T, bool ALIBI>
static hipError_t launch_half(const FwdParams& p, int D, unsigned grid, hipStream_t st) {
  switch (D) {
    case 16: return launch_kernel(fa_fwd_half_kernel<T, 16, ALIBI>, p, grid, st);
    case 32: return launch_kernel(fa_fwd_half_kernel<T, 32, ALIBI>, p, grid, st);
    case 64: return launch_kernel(fa_fwd_half_kernel<T, 64, ALIBI>, p, grid, st);
    case 128: return launch_kernel(fa_fwd_half_kernel<T, 128, ALIBI>, p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool ALIBI>
static hipError_t launch_f32(const FwdParams& p, int D, unsigned grid, hipStream_t st) {
  switch (D) {
    case 16: return launch_kernel(fa_fwd_f32_kernel<16, ALIBI>, p, grid, st);
    case 32: return launch_kernel(fa_fwd_f32_kernel<32, ALIBI>, p, grid, st);
    case 64: return launch_kernel(fa_fwd_f32_kernel<64, ALIBI>, p, grid, st);
    case 128: return launch_kernel(fa_fwd_f32_kernel<128, ALIBI>, p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool ALIBI>
static hipError_t launch_generic_a(const FwdParams& p, int D, int dtype, unsigned grid,
                                   hipStream_t st) {
  switch (dtype) {
    case kDtypeBF16: return launch_half<__bf16, ALIBI>(p, D, grid, st);
    case kDtypeF16: return launch_half<_Float16, ALIBI>(p, D, grid, st);
    case kDtypeF32: return launch_f32<ALIBI>(p, D, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_generic(const FwdParams& p, int D, int dtype, hipStream_t st) {
  const unsigned grid = (unsigned)p.nqb * (unsigned)p.BH;
  return p.alibi ? launch_generic_a<true>(p, D, dtype, grid, st)
                 : launch_generic_a<false>(p, D, dtype, grid, st);
}

}  // namespace fa
