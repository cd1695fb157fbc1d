// Host-only driver of the C ABI's argument validation (fa_validate.cpp),
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_validate_host.py. It runs the invalid-argument table of the ABI
// tests, checks the normalised parameters of valid calls, and then pushes
// random extreme arguments (sizes near the int64 limits, addresses near the
// top of the address space) through every entry so the sanitizers see any
// overflow or out-of-bounds access. No GPU and no HIP runtime is involved.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <functional>
#include <limits>
#include <string>
#include <vector>
#include <type_traits>

#include "../../include/flash_attn.h"
#include "../../io_aware_tiled_flash_amd/csrc/fa_validate.h"

namespace {

int g_failures = 0;

void expect(bool ok, const std::string& what) {
  if (!ok) {
    std::printf("FAIL %s\n", what.c_str());
    ++g_failures;
  }
}

template <typename T>
T* addr(uintptr_t a) {
  return reinterpret_cast<T*>(a);
}

constexpr uintptr_t Q = 0x100000, K = 0x200000, V = 0x300000, O = 0x400000, L = 0x500000;

fa::FwdCall base_fwd() {
  fa::FwdCall a;
  a.q = addr<const void>(Q);
  a.k = addr<const void>(K);
  a.v = addr<const void>(V);
  a.o = addr<void>(O);
  a.lse = addr<float>(L);
  a.B = 1;
  a.H = 1;
  a.H_kv = 1;
  a.S = 64;
  a.D = 64;
  a.scale = 0.125f;
  a.dtype = FA_BF16;
  return a;
}

void fwd_case(const char* name, int want, const std::function<void(fa::FwdCall&)>& edit) {
  fa::FwdCall a = base_fwd();
  edit(a);
  fa::FwdLaunch l;
  std::string err;
  const int rc = fa::prepare_fwd(a, &l, &err);
  expect(rc == want, std::string("fwd ") + name + ": rc " + std::to_string(rc));
  expect(rc == FA_OK || !err.empty(), std::string("fwd ") + name + ": empty message");
}

fa::BwdCall base_bwd() {
  fa::BwdCall a;
  a.q = addr<const void>(0x100000);
  a.k = addr<const void>(0x200000);
  a.v = addr<const void>(0x300000);
  a.o = addr<const void>(0x400000);
  a.dout = addr<const void>(0x500000);
  a.lse = addr<const float>(0x600000);
  a.dq = addr<void>(0x700000);
  a.dk = addr<void>(0x800000);
  a.dv = addr<void>(0x900000);
  a.workspace = addr<void>(0xa00000);
  a.workspace_bytes = 1 << 20;
  a.B = 1;
  a.H = 2;
  a.H_kv = 1;
  a.S = 64;
  a.D = 64;
  a.causal = 1;
  a.scale = 0.125f;
  a.dtype = FA_BF16;
  return a;
}

void bwd_case(const char* name, int want, const std::function<void(fa::BwdCall&)>& edit) {
  fa::BwdCall a = base_bwd();
  edit(a);
  fa::BwdParams p;
  std::string err;
  const int rc = fa::prepare_bwd(a, &p, &err);
  expect(rc == want, std::string("bwd ") + name + ": rc " + std::to_string(rc));
  expect(rc == FA_OK || !err.empty(), std::string("bwd ") + name + ": empty message");
}

// Deterministic 64-bit generator (SplitMix64) for the fuzz.
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  // A size drawn from a mix of small values, powers of two near the int32 and
  // int64 limits, and negatives.
  int64_t size() {
    const uint64_t r = next();
    switch (r % 8) {
      case 0: return (int64_t)(next() % 9) - 2;
      case 1: return (int64_t)(next() % 5000);
      case 2: return (int64_t)1 << (next() % 63);
      case 3: return std::numeric_limits<int64_t>::max() - (int64_t)(next() % 3);
      case 4: return std::numeric_limits<int64_t>::min() + (int64_t)(next() % 3);
      case 5: return (int64_t)INT32_MAX - (int64_t)(next() % 300);
      case 6: return (int64_t)(next() >> 1);
      default: return 128;
    }
  }
  uintptr_t address() {
    const uint64_t r = next();
    switch (r % 4) {
      case 0: return 0;
      case 1: return (uintptr_t)(next() & ~(uint64_t)15);
      case 2: return ~(uintptr_t)0 - (uintptr_t)(next() % 4096);
      default: return (uintptr_t)(0x100000 * (1 + next() % 16) + 16 * (next() % 4));
    }
  }
  float scale() {
    const uint64_t r = next() % 6;
    if (r == 0) return std::numeric_limits<float>::infinity();
    if (r == 1) return std::nanf("");
    if (r == 2) return 0.f;
    if (r == 3) return -0.0883883f;
    if (r == 4) return std::numeric_limits<float>::max();
    return 0.0883883f;
  }
};

}  // namespace

int main() {
  // ---- forward: each precondition of flash_attn.h ----
  fwd_case("valid", FA_OK, [](fa::FwdCall&) {});
  fwd_case("null_q", FA_ERR_INVALID, [](fa::FwdCall& a) { a.q = nullptr; });
  fwd_case("null_k", FA_ERR_INVALID, [](fa::FwdCall& a) { a.k = nullptr; });
  fwd_case("null_v", FA_ERR_INVALID, [](fa::FwdCall& a) { a.v = nullptr; });
  fwd_case("null_o", FA_ERR_INVALID, [](fa::FwdCall& a) { a.o = nullptr; });
  fwd_case("null_lse", FA_ERR_INVALID, [](fa::FwdCall& a) { a.lse = nullptr; });
  fwd_case("B0", FA_ERR_INVALID, [](fa::FwdCall& a) { a.B = 0; });
  fwd_case("H0", FA_ERR_INVALID, [](fa::FwdCall& a) { a.H = 0; });
  fwd_case("S0", FA_ERR_INVALID, [](fa::FwdCall& a) { a.S = 0; });
  fwd_case("S_negative", FA_ERR_INVALID, [](fa::FwdCall& a) { a.S = -5; });
  fwd_case("D0", FA_ERR_INVALID, [](fa::FwdCall& a) { a.D = 0; });
  fwd_case("causal_2", FA_ERR_INVALID, [](fa::FwdCall& a) { a.causal = 2; });
  fwd_case("window_negative", FA_ERR_INVALID, [](fa::FwdCall& a) { a.causal = 1; a.window = -1; });
  fwd_case("window_without_causal", FA_ERR_INVALID, [](fa::FwdCall& a) { a.window = 16; });
  fwd_case("n_sink_negative", FA_ERR_INVALID,
           [](fa::FwdCall& a) { a.causal = 1; a.window = 16; a.n_sink = -1; });
  fwd_case("scale_nan", FA_ERR_INVALID, [](fa::FwdCall& a) { a.scale = std::nanf(""); });
  fwd_case("scale_inf", FA_ERR_INVALID,
           [](fa::FwdCall& a) { a.scale = std::numeric_limits<float>::infinity(); });
  fwd_case("dtype_unknown", FA_ERR_INVALID, [](fa::FwdCall& a) { a.dtype = 3; });
  fwd_case("q_misaligned", FA_ERR_INVALID, [](fa::FwdCall& a) { a.q = addr<const void>(Q + 8); });
  fwd_case("lse_misaligned", FA_ERR_INVALID, [](fa::FwdCall& a) { a.lse = addr<float>(L + 2); });
  fwd_case("o_overlaps_q", FA_ERR_INVALID, [](fa::FwdCall& a) { a.o = addr<void>(Q + 64); });
  fwd_case("lse_overlaps_o", FA_ERR_INVALID, [](fa::FwdCall& a) { a.lse = addr<float>(O + 128); });
  fwd_case("size_overflow", FA_ERR_INVALID,
           [](fa::FwdCall& a) { a.B = (int64_t)1 << 40; a.H = (int64_t)1 << 20; a.S = 1024; });
  fwd_case("kv_heads_not_dividing", FA_ERR_INVALID, [](fa::FwdCall& a) { a.H = 6; a.H_kv = 4; });
  fwd_case("alibi_overlaps_lse", FA_ERR_INVALID,
           [](fa::FwdCall& a) { a.alibi = addr<const float>(L); });
  fwd_case("counter_misaligned", FA_ERR_INVALID,
           [](fa::FwdCall& a) { a.block_pairs = addr<uint64_t>(0x600004); });
  fwd_case("split_no_workspace", FA_ERR_INVALID, [](fa::FwdCall& a) { a.n_split = 2; });
  fwd_case("split_too_many", FA_ERR_INVALID, [](fa::FwdCall& a) { a.n_split = 257; });
  fwd_case("split_small_workspace", FA_ERR_INVALID, [](fa::FwdCall& a) {
    a.n_split = 2;
    a.workspace = addr<void>(0x800000);
    a.workspace_bytes = 16;
  });
  fwd_case("split_f32", FA_ERR_UNSUPPORTED, [](fa::FwdCall& a) {
    a.n_split = 2;
    a.dtype = FA_F32;
    a.workspace = addr<void>(0x800000);
    a.workspace_bytes = 1 << 20;
  });
  fwd_case("head_dim_96", FA_ERR_UNSUPPORTED, [](fa::FwdCall& a) { a.D = 96; });
  fwd_case("index_range", FA_ERR_UNSUPPORTED, [](fa::FwdCall& a) {
    a.S = (int64_t)1 << 31;
    a.D = 16;
    a.o = addr<void>((uintptr_t)1 << 44);
    a.lse = addr<float>((uintptr_t)1 << 45);
  });
  fwd_case("grid_range", FA_ERR_UNSUPPORTED, [](fa::FwdCall& a) {
    a.B = (int64_t)1 << 20;
    a.S = 1 << 20;
    a.D = 16;
    a.k = addr<const void>((uintptr_t)1 << 46);
    a.v = addr<const void>((uintptr_t)1 << 47);
    a.o = addr<void>((uintptr_t)1 << 48);
    a.lse = addr<float>((uintptr_t)1 << 49);
  });

  // ---- forward: normalisation of a valid call ----
  {
    fa::FwdCall a = base_fwd();
    a.B = 2;
    a.H = 8;
    a.H_kv = 2;
    a.S = 1000;
    a.D = 128;
    a.causal = 1;
    a.window = 5000;   // wider than S: no window
    a.n_sink = 9;
    a.scale = -0.25f;
    a.q = addr<const void>(0x10000000);
    a.k = addr<const void>(0x20000000);
    a.v = addr<const void>(0x30000000);
    a.o = addr<void>(0x40000000);
    a.lse = addr<float>(0x50000000);
    fa::FwdLaunch l;
    std::string err;
    expect(fa::prepare_fwd(a, &l, &err) == FA_OK, "normalise: rc");
    expect(l.p.window == 0 && l.p.n_sink == 0, "normalise: window folded");
    expect(l.p.neg == 1 && std::fabs(l.p.c - 0.25f * 1.4426950408889634f) < 1e-6f, "normalise: scale");
    expect(l.p.G == 4 && l.p.BH == 16 && l.p.S == 1000, "normalise: heads");
    expect(l.plan.fast && l.p.nqb == (1000 + l.plan.block_q - 1) / l.plan.block_q, "normalise: plan");
    expect(l.rows == 16000, "normalise: rows");
    a.window = 100;
    a.n_sink = 5000;
    expect(fa::prepare_fwd(a, &l, &err) == FA_OK && l.p.window == 100 && l.p.n_sink == 1000,
           "normalise: sinks clamped to S");
    a.scale = 0.f;
    expect(fa::prepare_fwd(a, &l, &err) == FA_OK && l.p.c > 0.f && l.p.neg == 0,
           "normalise: zero scale");
  }

  // ---- backward ----
  bwd_case("valid", FA_OK, [](fa::BwdCall&) {});
  bwd_case("null_dq", FA_ERR_INVALID, [](fa::BwdCall& a) { a.dq = nullptr; });
  bwd_case("null_workspace", FA_ERR_INVALID, [](fa::BwdCall& a) { a.workspace = nullptr; });
  bwd_case("small_workspace", FA_ERR_INVALID, [](fa::BwdCall& a) { a.workspace_bytes = 8; });
  bwd_case("dk_overlaps_k", FA_ERR_INVALID,
           [](fa::BwdCall& a) { a.dk = addr<void>(0x200000 + 16); });
  bwd_case("dq_overlaps_dv", FA_ERR_INVALID, [](fa::BwdCall& a) { a.dq = addr<void>(0x900000); });
  bwd_case("misaligned_dout", FA_ERR_INVALID,
           [](fa::BwdCall& a) { a.dout = addr<const void>(0x500008); });
  bwd_case("f32", FA_ERR_UNSUPPORTED, [](fa::BwdCall& a) { a.dtype = FA_F32; });
  bwd_case("d32", FA_ERR_UNSUPPORTED, [](fa::BwdCall& a) { a.D = 32; });
  bwd_case("window_no_causal", FA_ERR_INVALID, [](fa::BwdCall& a) { a.causal = 0; a.window = 4; });
  // the library's own scratch (no workspace pointer): valid within its size,
  // FA_ERR_UNSUPPORTED past it, and the workspace binds afterwards
  bwd_case("internal_ws", FA_OK, [](fa::BwdCall& a) {
    a.workspace = nullptr;
    a.internal_workspace = true;
    a.workspace_bytes = fa::kBwdScratchBytes;
  });
  bwd_case("internal_ws_too_big", FA_ERR_UNSUPPORTED, [](fa::BwdCall& a) {
    a.workspace = nullptr;
    a.internal_workspace = true;
    a.workspace_bytes = fa::kBwdScratchBytes;
    a.H = 2050;
    a.H_kv = 2050;
    a.S = 2048;
    for (const void** t : {&a.q, &a.k, &a.v, &a.o, &a.dout})
      *t = reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(*t) << 20);
    a.lse = reinterpret_cast<const float*>(reinterpret_cast<uintptr_t>(a.lse) << 20);
    for (void** t : {&a.dq, &a.dk, &a.dv})
      *t = reinterpret_cast<void*>(reinterpret_cast<uintptr_t>(*t) << 20);
  });
  {
    fa::BwdCall a = base_bwd();
    a.workspace = nullptr;
    a.internal_workspace = true;
    a.workspace_bytes = fa::kBwdScratchBytes;
    fa::BwdParams p;
    std::string err;
    expect(fa::prepare_bwd(a, &p, &err) == FA_OK && p.delta == nullptr && p.lse2 == nullptr,
           "internal workspace unbound after validation");
    fa::bwd_bind_workspace(&p, addr<void>(0x40000000));
    expect(p.delta == addr<float>(0x40000000) &&
               p.lse2 == addr<float>(0x40000000) + (int64_t)p.BH * p.Sp && p.Sp == 128,
           "internal workspace bound");
  }

  // ---- merge and sizes ----
  {
    std::string err;
    const float* op = addr<const float>(0x100000);
    const float* lp = addr<const float>(0x200000);
    expect(fa::check_merge(op, lp, 4, 64, 64, addr<void>(0x300000), addr<float>(0x400000), FA_BF16,
                           &err) == FA_OK, "merge valid");
    expect(fa::check_merge(op, lp, 4, 64, 64, addr<void>(0x100010), addr<float>(0x400000), FA_BF16,
                           &err) == FA_ERR_INVALID, "merge overlap");
    expect(fa::check_merge(op, lp, 0, 64, 64, addr<void>(0x300000), addr<float>(0x400000), FA_BF16,
                           &err) == FA_ERR_INVALID, "merge n_parts");
    expect(fa::split_workspace_bytes(1, 8, 4096, 128, 1, &err) == 0, "split ws n=1");
    expect(fa::split_workspace_bytes(1, 8, 4096, 128, 4, &err) ==
               (int64_t)4 * 8 * 4096 * 128 * 4 + 4 * 8 * 4096 * 4, "split ws size");
    expect(fa::bwd_workspace_bytes(4, 16, 4096, &err) == 2 * 64 * 4096 * 4, "bwd ws size");
    expect(fa::bwd_workspace_bytes(1, 1, 0, &err) == -1, "bwd ws invalid");
    int bq = 0, bk = 0;
    expect(fa::tile_shape(1, 1, 64, 48, FA_BF16, 0, &bq, &bk, &err) == FA_ERR_UNSUPPORTED, "tile d48");
    expect(fa::tile_shape(4, 16, 4096, 128, FA_BF16, 0, &bq, &bk, &err) == FA_OK && bk == fa::kFastBC,
           "tile c3");
    expect(fa::tile_shape(4, 16, 4096, 128, FA_BF16, -1, &bq, &bk, &err) == FA_ERR_INVALID,
           "tile window < 0");
  }

  // ---- LDS layouts: every read pattern free of bank conflicts ----
  // gfx950 LDS: 64 banks of 4 bytes, 256 bytes a clock; a 16-byte read serves
  // 16 lanes a cycle, an 8-byte read 32. An instruction is conflict-free when
  // no bank holds two different dwords within a cycle's lanes. The lane
  // addresses restate the kernels' offsets: K-layout row reads (forward QK,
  // every backward operand over d), K-layout transposing reads (dQ's K^T,
  // dK/dV's Q^T and dO^T) and the forward's V-layout transposing reads.
  {
    auto cycles = [](const std::vector<long>& byte_addr, int width) {
      const int per = 256 / width;
      int tot = 0;
      for (int g0 = 0; g0 < 64; g0 += per) {
        std::vector<std::vector<long>> bank(64);
        for (int l = g0; l < g0 + per; ++l)
          for (int w = 0; w < width / 4; ++w) {
            const long dw = byte_addr[l] / 4 + w;
            auto& b = bank[dw % 64];
            if (std::find(b.begin(), b.end(), dw) == b.end()) b.push_back(dw);
          }
        size_t worst = 0;
        for (auto& b : bank) worst = std::max(worst, b.size());
        tot += (int)worst;
      }
      return tot;
    };
    auto check = [&](auto dc) {
      constexpr int D = decltype(dc)::value;
      const long E = 2;   // bf16 / f16 bytes
      std::vector<long> a(64);
      for (int t = 0; t < 4; ++t)          // row reads: lane (col, h), rows 32 t + col
        for (int s = 0; s < D / 16; ++s) {
          for (int l = 0; l < 64; ++l) {
            const int row = 32 * t + (l & 31), h = l >> 5;
            a[l] = E * (row * D + (((2 * s + h) ^ fa::k_swz<D>(row)) << 3));
          }
          expect(cycles(a, 16) == 4, "k_swz row read conflicts, D " + std::to_string(D));
        }
      for (int u = 0; u < 8; ++u)          // transposing reads of the K layout
        for (int part = 0; part < 2; ++part)
          for (int dt = 0; dt < D / 32; ++dt) {
            for (int l = 0; l < 64; ++l) {
              const int h = l >> 5, grp = (l >> 4) & 1, r16 = l & 15;
              const int row = 16 * u + 4 * h + (r16 >> 2) + 8 * part;
              const int chunk = 4 * dt + 2 * grp + ((r16 & 3) >> 1);
              a[l] = E * (row * D + ((chunk ^ fa::k_swz<D>(row)) << 3) + 4 * (r16 & 1));
            }
            expect(cycles(a, 8) == 2, "k_swz transposing read conflicts, D " + std::to_string(D));
          }
      for (int tu = 0; tu < 4; ++tu)       // transposing reads of the V layout
        for (int part = 0; part < 2; ++part)
          for (int dt = 0; dt < D / 32; ++dt) {
            for (int l = 0; l < 64; ++l) {
              const int h = l >> 5, grp = (l >> 4) & 1, r16 = l & 15;
              const int row = 16 * tu + 4 * h + (r16 >> 2) + 8 * part;
              a[l] = E * (row * D + 16 * grp + 4 * (r16 & 3) + ((dt ^ fa::v_swz<D>(row)) << 5));
            }
            expect(cycles(a, 8) == 2, "v_swz transposing read conflicts, D " + std::to_string(D));
          }
      // each swizzle is a permutation of a row's chunks / segments
      for (int row = 0; row < 128; ++row) {
        std::vector<int> seen(D / 8, 0), segs(D / 32, 0);
        for (int c = 0; c < D / 8; ++c) {
          const int p = c ^ fa::k_swz<D>(row);
          expect(0 <= p && p < D / 8 && !seen[p]++, "k_swz not a permutation");
        }
        for (int sg = 0; sg < D / 32; ++sg) {
          const int p = sg ^ fa::v_swz<D>(row);
          expect(0 <= p && p < D / 32 && !segs[p]++, "v_swz not a permutation");
        }
      }
    };
    check(std::integral_constant<int, 128>{});
    check(std::integral_constant<int, 64>{});
    // the model itself: a plain row & 15 swizzle gives the 4-way conflicts
    // the counters showed on the transposing reads
    {
      std::vector<long> a(64);
      for (int l = 0; l < 64; ++l) {
        const int h = l >> 5, grp = (l >> 4) & 1, r16 = l & 15;
        const int row = 4 * h + (r16 >> 2), chunk = 2 * grp + ((r16 & 3) >> 1);
        a[l] = 2 * (row * 128 + ((chunk ^ (row & 15)) << 3) + 4 * (r16 & 1));
      }
      expect(cycles(a, 8) == 8, "bank model: row & 15 should give 4-way conflicts");
    }
    std::printf("LDS layouts: row and transposing reads conflict-free at D 64 and 128\n");
  }

  // ---- kept-key bit words of the masks with a window ----
  // keep_word bit by bit against the set it stands for, and the two masks the
  // kernels build from it: forward / dQ (key offset e kept iff e <= hi and
  // (e >= lo or e <= sk)) with skh = min(sk, hi), and dK/dV (row offset e kept
  // iff e >= emin and (e < emin + wlen or the key is a sink)) with
  // hi = sink ? 2^30 : emin + wlen - 1.
  {
    Rng g{4242};
    const int big = 1 << 30;
    int words = 0;
    auto near = [&](int base) {   // bounds around the word, now and then far away
      switch (g.next() % 8) {
        case 0: return -big;
        case 1: return big;
        case 2: return base + (int)(g.next() % 4000) - 2000;
        default: return base + (int)(g.next() % 80) - 24;
      }
    };
    for (int trial = 0; trial < 200000; ++trial) {
      const int base = 32 * ((int)(g.next() % 64) - 32);
      const int lo = near(base), hi = near(base), sk = near(base);
      const uint32_t w = fa::keep_word(lo, hi, sk, base);
      const uint32_t wf = fa::keep_word(lo, hi, std::min(sk, hi), base);
      const int emin = near(base), wlen = 1 + (int)(g.next() % 300);
      const bool sink = g.next() % 2;
      const uint32_t wk = fa::keep_word(emin, sink ? big : emin + wlen - 1, -big, base);
      bool ok = true;
      for (int p = 0; p < 32; ++p) {
        const long e = (long)base + p;
        ok = ok && (((w >> p) & 1u) == (uint32_t)((lo <= e && e <= hi) || e <= sk));
        ok = ok && (((wf >> p) & 1u) == (uint32_t)(e <= hi && (e >= lo || e <= sk)));
        ok = ok && (((wk >> p) & 1u) == (uint32_t)(e >= emin && (e < (long)emin + wlen || sink)));
      }
      expect(ok, "keep_word (lo " + std::to_string(lo) + ", hi " + std::to_string(hi) + ", sk " +
                     std::to_string(sk) + ", base " + std::to_string(base) + ", emin " +
                     std::to_string(emin) + ", wlen " + std::to_string(wlen) + ")");
      ++words;
    }
    std::printf("keep_word: %d words checked bit by bit\n", words);
  }

  // ---- closed-form mask segments against a scan of the blocks ----
  // The kernels take their fully visible run of blocks from full_key_steps /
  // full_query_steps. Every step of that run must be fully visible, and
  // without sink keys it must be exactly the first fully visible run (what a
  // scan of the walk finds). The walk and the visibility test restate the mask
  // geometry: sink blocks first, then the window's blocks (forward, dQ); the
  // query blocks that see a key block (dK/dV).
  {
    Rng g{777};
    int checked = 0, exact = 0;
    for (int trial = 0; trial < 200000; ++trial) {
      const int BC = 64;
      const int BR = (int[]){64, 128, 256}[g.next() % 3];
      const int S = 1 + (int)(g.next() % 3000);
      const int causal = (int)(g.next() % 4 != 0);
      const int window = causal && (g.next() % 2) ? 1 + (int)(g.next() % 600) : 0;
      const int n_sink = window ? (int)(g.next() % 200) : 0;
      const int q_lo = BR * (int)(g.next() % ((S + BR - 1) / BR));
      // the walk
      int n_sinkb = 0, kb_lo = 0, kb_hi;
      if (causal) {
        kb_hi = (std::min(q_lo + BR, S) - 1) / BC;
        if (window > 0) {
          kb_lo = std::max(0, q_lo - window + 1) / BC;
          n_sinkb = std::min(kb_lo, (n_sink + BC - 1) / BC);
        }
      } else {
        kb_hi = (S - 1) / BC;
      }
      const int n_all = n_sinkb + kb_hi - kb_lo + 1;
      auto kb_of = [&](int it) { return it < n_sinkb ? it : kb_lo + it - n_sinkb; };
      auto full = [&](int kb) {
        const int k0 = kb * BC;
        bool f = k0 + BC <= S;
        if (causal) {
          f = f && k0 + BC - 1 <= q_lo;
          if (window > 0) f = f && (q_lo + BR - 1 - k0 < window || k0 + BC <= n_sink);
        }
        return f;
      };
      // a sub-walk (a key split's share), forwards or in reverse
      const int it_b = (int)(g.next() % n_all);
      const int n = 1 + (int)(g.next() % (n_all - it_b));
      const bool rev = g.next() % 2;
      const fa::StepRange F = fa::full_key_steps(q_lo, BR, BC, S, causal, window, n_sinkb, kb_lo, kb_hi);
      const fa::StepRange r = fa::local_steps(F, it_b, n, rev);
      auto step_kb = [&](int t) { return kb_of(rev ? it_b + n - 1 - t : it_b + t); };
      bool ok = 0 <= r.lo && r.lo <= r.hi && r.hi <= n;
      for (int t = r.lo; ok && t < r.hi; ++t) ok = full(step_kb(t));
      expect(ok, "full_key_steps: a step of the run is not fully visible (S " + std::to_string(S) +
                     ", q_lo " + std::to_string(q_lo) + ", window " + std::to_string(window) + ")");
      if (n_sink == 0) {
        int f0 = 0;
        while (f0 < n && !full(step_kb(f0))) ++f0;
        int f1 = f0;
        while (f1 < n && full(step_kb(f1))) ++f1;
        const bool same = f1 == f0 ? r.lo == r.hi : (r.lo == f0 && r.hi == f1);
        expect(same, "full_key_steps: not the scanned run (S " + std::to_string(S) + ", q_lo " +
                         std::to_string(q_lo) + ", BR " + std::to_string(BR) + ", window " +
                         std::to_string(window) + ", rev " + std::to_string(rev) + ")");
        ++exact;
      }
      ++checked;
      // dK/dV: key block [k_lo, k_lo + BK), query blocks of BQ rows
      const int BK = 128, BQ = (g.next() % 2) ? 32 : 128;
      const int k_lo = BK * (int)(g.next() % ((S + BK - 1) / BK));
      const int k_hi = std::min(k_lo + BK, S) - 1;
      const int nqb = (S + BQ - 1) / BQ;
      int qfirst = 0, qlast = nqb - 1;
      if (causal) {
        qfirst = k_lo / BQ;
        if (window > 0 && k_lo >= n_sink) qlast = std::min(S - 1, k_hi + window - 1) / BQ;
      }
      if (qfirst > qlast) continue;
      const int nq = qlast - qfirst + 1;
      auto qfull = [&](int qb) {
        const int q0 = qb * BQ;
        bool f = true;
        if (causal) {
          f = q0 >= k_lo + BK - 1;
          if (window > 0) f = f && (q0 + BQ - 1 - k_lo < window || k_lo + BK <= n_sink);
        }
        return f;
      };
      const fa::StepRange rq = fa::local_steps(
          fa::full_query_steps(k_lo, BK, BQ, causal, window, n_sink, qfirst, qlast), 0, nq, false);
      bool okq = 0 <= rq.lo && rq.lo <= rq.hi && rq.hi <= nq;
      for (int t = rq.lo; okq && t < rq.hi; ++t) okq = qfull(qfirst + t);
      int q0 = 0;
      while (q0 < nq && !qfull(qfirst + q0)) ++q0;
      int q1 = q0;
      while (q1 < nq && qfull(qfirst + q1)) ++q1;
      const bool sameq = q1 == q0 ? rq.lo == rq.hi : (rq.lo == q0 && rq.hi == q1);
      expect(okq && sameq, "full_query_steps (S " + std::to_string(S) + ", k_lo " +
                               std::to_string(k_lo) + ", BQ " + std::to_string(BQ) + ", window " +
                               std::to_string(window) + ", sinks " + std::to_string(n_sink) + ")");
    }
    std::printf("mask segments: %d walks checked, %d against the scanned run\n", checked, exact);
  }

  // ---- fuzz: random extreme arguments through every entry ----
  Rng rng{12345};
  int ok_fwd = 0, ok_bwd = 0;
  for (int it = 0; it < 200000; ++it) {
    fa::FwdCall a;
    a.q = addr<const void>(rng.address());
    a.k = addr<const void>(rng.address());
    a.v = addr<const void>(rng.address());
    a.o = addr<void>(rng.address());
    a.lse = addr<float>(rng.address());
    a.B = rng.size();
    a.H = rng.size();
    a.H_kv = (rng.next() & 1) ? a.H : rng.size();
    a.S = rng.size();
    a.D = (rng.next() & 1) ? (int64_t)16 << (rng.next() % 4) : rng.size();
    a.causal = (int)(rng.next() % 3);
    a.window = rng.size();
    a.n_sink = rng.size();
    a.scale = rng.scale();
    a.alibi = (rng.next() & 1) ? nullptr : addr<const float>(rng.address());
    a.dtype = (int)(rng.next() % 4);
    a.block_pairs = (rng.next() & 3) ? nullptr : addr<uint64_t>(rng.address());
    a.n_split = (rng.next() & 1) ? 1 : rng.size();
    a.workspace = addr<void>(rng.address());
    a.workspace_bytes = rng.size();
    if (it & 1) {
      // mostly valid: disjoint, aligned tensors 2^40 bytes apart and sizes
      // that fit, with the random mask, scale, dtype and split kept
      a.q = addr<const void>((uintptr_t)1 << 40);
      a.k = addr<const void>((uintptr_t)2 << 40);
      a.v = addr<const void>((uintptr_t)3 << 40);
      a.o = addr<void>((uintptr_t)4 << 40);
      a.lse = addr<float>((uintptr_t)5 << 40);
      a.alibi = (rng.next() & 1) ? nullptr : addr<const float>((uintptr_t)6 << 40);
      a.block_pairs = nullptr;
      a.workspace = addr<void>((uintptr_t)7 << 40);
      a.workspace_bytes = (int64_t)1 << 40;
      a.B = 1 + (int64_t)(rng.next() % 8);
      a.H_kv = 1 + (int64_t)(rng.next() % 4);
      a.H = a.H_kv * (1 + (int64_t)(rng.next() % 4));
      a.S = 1 + (int64_t)(rng.next() % 70000);
      a.D = (int64_t)16 << (rng.next() % 4);
      a.n_split = 1 + (int64_t)(rng.next() % 8);
      a.window = (int64_t)(rng.next() % 3) * (int64_t)(rng.next() % 100000);
      a.n_sink = (int64_t)(rng.next() % 9);
      if (a.window > 0) a.causal = 1;
    }
    fa::FwdLaunch l;
    std::string err;
    if (fa::prepare_fwd(a, &l, &err) == FA_OK) {
      ++ok_fwd;
      expect(l.p.S >= 1 && l.p.BH >= 1 && l.p.nqb >= 1 && l.p.c > 0.f, "fuzz fwd accepted sanely");
      expect(l.p.window >= 0 && l.p.window < l.p.S + (l.p.window == 0) && l.p.n_sink <= l.p.S &&
                 (l.p.window > 0 || l.p.n_sink == 0) && (int64_t)l.p.nqb * l.plan.block_q >= l.p.S,
             "fuzz fwd normalised mask and grid");
    }
    fa::BwdCall b;
    b.q = addr<const void>(rng.address());
    b.k = addr<const void>(rng.address());
    b.v = addr<const void>(rng.address());
    b.o = addr<const void>(rng.address());
    b.dout = addr<const void>(rng.address());
    b.lse = addr<const float>(rng.address());
    b.dq = addr<void>(rng.address());
    b.dk = addr<void>(rng.address());
    b.dv = addr<void>(rng.address());
    b.workspace = addr<void>(rng.address());
    b.workspace_bytes = rng.size();
    b.B = rng.size();
    b.H = rng.size();
    b.H_kv = (rng.next() & 1) ? b.H : rng.size();
    b.S = rng.size();
    b.D = (rng.next() & 1) ? 64 : rng.size();
    b.causal = (int)(rng.next() % 3);
    b.window = rng.size();
    b.n_sink = rng.size();
    b.scale = rng.scale();
    b.dtype = (int)(rng.next() % 4);
    fa::BwdParams bp;
    if (fa::prepare_bwd(b, &bp, &err) == FA_OK) ++ok_bwd;
    (void)fa::check_merge(addr<const float>(rng.address()), addr<const float>(rng.address()),
                          rng.size(), rng.size(), rng.size(), addr<void>(rng.address()),
                          addr<float>(rng.address()), (int)(rng.next() % 4), &err);
    (void)fa::split_workspace_bytes(rng.size(), rng.size(), rng.size(), rng.size(), rng.size(),
                                    &err);
    (void)fa::bwd_workspace_bytes(rng.size(), rng.size(), rng.size(), &err);
    int bq, bk;
    (void)fa::tile_shape(rng.size(), rng.size(), rng.size(), rng.size(), (int)(rng.next() % 4),
                         rng.size(), &bq, &bk, &err);
    std::string kname;
    (void)fa::fwd_kernel_name(rng.size(), rng.size(), rng.size(), rng.size(), (int)(rng.next() % 4),
                              (int)(rng.next() % 2), rng.size(), rng.size(), &kname, &err);
    (void)fa::bwd_kernel_name(rng.size(), rng.size(), rng.size(), rng.size(), rng.size(),
                              (int)(rng.next() % 4), (int)(rng.next() % 2), rng.size(),
                              (int)(rng.next() % 2), &kname, &err);
  }
  // ---- the forward work-group order ----
  // wg_tile must visit every (query block, head) of the grid exactly once; with
  // BH a multiple of 8 every work-group of an XCD (id & 7) must stay in that
  // XCD's run of heads; under the causal mask each head's query blocks must
  // come heaviest first, and the work-groups of an XCD must cover at most
  // kOrderGroupHeads heads within any kOrderGroupHeads * nqb consecutive ids.
  {
    int grids = 0;
    for (int BH : {1, 2, 3, 5, 7, 8, 16, 24, 40, 64, 96, 128, 256}) {
      for (int nqb : {1, 2, 3, 7, 16, 32, 33, 64, 128}) {
        for (int mode = 0; mode < 3; ++mode) {
          const bool causal = mode > 0, window = mode == 2;
          std::vector<int> seen((size_t)BH * nqb, 0);
          std::vector<int> last_qb(BH, 1 << 30);
          bool ok = true;
          for (int id = 0; id < BH * nqb; ++id) {
            const fa::Tile t = fa::wg_tile(id, BH, nqb, causal, window);
            if (t.qb < 0 || t.qb >= nqb || t.bh < 0 || t.bh >= BH) { ok = false; break; }
            ++seen[(size_t)t.bh * nqb + t.qb];
            if (BH % 8 == 0 && t.bh / (BH / 8) != (id & 7)) ok = false;
            if (causal && !window) {
              if (t.qb >= last_qb[t.bh]) ok = false;   // heaviest first, per head
              last_qb[t.bh] = t.qb;
            }
          }
          for (int c : seen) ok = ok && c == 1;
          if (ok && BH % 8 == 0 && causal && !window) {
            // heads per XCD within each window of kOrderGroupHeads * nqb ids of that XCD
            const int HX = BH / 8, W = fa::kOrderGroupHeads * nqb;
            for (int xcd = 0; xcd < 8 && ok; ++xcd)
              for (int k0 = 0; k0 < HX * nqb && ok; k0 += W) {
                std::vector<int> heads;
                for (int kk = k0; kk < std::min(k0 + W, HX * nqb); ++kk) {
                  const int bh = fa::wg_tile(8 * kk + xcd, BH, nqb, true, false).bh;
                  if (std::find(heads.begin(), heads.end(), bh) == heads.end()) heads.push_back(bh);
                }
                ok = (int)heads.size() <= fa::kOrderGroupHeads;
              }
          }
          expect(ok, "wg_tile (BH " + std::to_string(BH) + ", nqb " + std::to_string(nqb) +
                         ", mode " + std::to_string(mode) + ")");
          ++grids;
        }
      }
    }
    std::printf("wg_tile: %d grids checked\n", grids);
  }

  std::printf("fuzz: %d forward and %d backward calls accepted of 200000 each\n", ok_fwd, ok_bwd);
  if (g_failures) {
    std::printf("%d FAILURES\n", g_failures);
    return 1;
  }
  std::printf("ALL OK\n");
  return 0;
}
