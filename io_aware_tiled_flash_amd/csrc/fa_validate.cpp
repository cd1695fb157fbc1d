// Host-side argument validation of the C ABI; see fa_validate.h. Mirrors the
// contract in include/flash_attn.h line by line: each rejected condition there
// has its check here, in the order the header lists them.
#include "fa_validate.h"

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "../../include/flash_attn.h"

namespace fa {

namespace {

int fail(std::string* err, int code, const char* msg) {
  if (err) *err = msg;
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Half-open byte ranges [a, a + na) and [b, b + nb) intersect. Sizes are
// bounded by the callers' overflow checks; the sums are taken in unsigned
// arithmetic, so they wrap instead of overflowing (an address near the top
// of the space then reads as overlapping, which only rejects a call).
bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uint64_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

int elem_bytes(int dtype) {
  switch (dtype) {
    case FA_F32: return 4;
    case FA_F16: return 2;
    case FA_BF16: return 2;
    default: return 0;
  }
}

bool supported_d(int64_t D) { return D == 16 || D == 32 || D == 64 || D == 128; }

// Bytes of the key-split workspace: fp32 partial outputs [n_split][B*H][S][D]
// then, 256-byte aligned, partial LSE [n_split][B*H][S]. -1 if it overflows.
int64_t split_ws(int64_t rows, int64_t D, int64_t n_split, int64_t* lse_offset) {
  // rows * n_split * (D + 1) <= INT64_MAX / 8, tested without forming an
  // overflowing intermediate (D + 1 itself may not be representable).
  const int64_t lim = INT64_MAX / 8;
  if (rows > lim / n_split) return -1;
  const int64_t rn = rows * n_split;
  if (D > lim / rn - 1) return -1;
  const int64_t o_bytes = rows * n_split * D * 4;
  const int64_t off = (o_bytes + 255) / 256 * 256;
  if (lse_offset) *lse_offset = off;
  return off + rows * n_split * 4;
}

// Testing aid: FLASH_ATTN_REVERSE_ORDER=1 makes the forward work-groups take
// their tiles in reverse dispatch order (results must not change).
int reverse_order() {
  const char* e = std::getenv("FLASH_ATTN_REVERSE_ORDER");
  return (e && e[0] == '1') ? 1 : 0;
}

}  // namespace

// Kernel choice. bf16/f16 with D = 64 or 128 take the fast kernel. Its
// work-group holds 4 waves (128 query rows), so two work-groups share a CU (three
// at D = 64) and run out of step with each other: one's softmax (vector ALU)
// overlaps the other's matrix products. With at least two 8-wave work-groups
// per CU, 8 waves (256 rows, one work-group per CU) halve the K/V tile traffic
// per query row. They win for S >= 16384, and at D = 128 without a window from
// S = 2048 on (same-process A/B with the grouped work-group order: +1.9 % on
// causal B4 H16 S4096, +2.4 % with grouped heads, +5 % at S 2048 and
// unmasked, +1.3 % at S 8192; -4 % at S 1024, -2.8 % with a 1024-key window,
// -16 % with a 256-key one, -1.7 % at D = 64). window is the call's window (0,
// or >= S, for none). FLASH_ATTN_WAVES=4|8 overrides the wave count (tuning
// only).
//
// Grids of fewer than two 4-wave work-groups of 128 rows per CU (256 CUs)
// leave SIMDs with one wave or none. Without ALiBi and a key split they take
// the small-grid schedule: 8-wave work-groups whose waves split each query
// block's key blocks into key parts, so that every SIMD holds two waves and
// each wave takes 1/parts of the steps. Two parts keep 128-row blocks; four
// parts (D = 64, where the tiles of four parts fit in LDS) use 64-row blocks,
// which doubles the work-group count of a grid that covers at most half the
// CUs. FLASH_ATTN_PARTS=0|2|4 overrides (tuning).
Plan plan_fwd(int64_t BH, int64_t S, int64_t D, int dtype, bool plain, int64_t window) {
  Plan pl;
  pl.parts = 0;
  if (fast_supported(D, dtype)) {
    pl.fast = true;
    // 8-wave work-groups (256 rows) for S >= 16384 when there are at least 512
    // of them; the product BH * ceil(S / 256) is only formed when both factors
    // are small, so it cannot overflow for any argument.
    const int64_t nb8 = S / 256 + (S % 256 != 0);
    const bool many8 = BH >= 512 || nb8 >= 512 || BH * nb8 >= 512;
    const bool no_window = window <= 0 || window >= S;
    pl.nw = (many8 && (S >= 16384 || (D == 128 && no_window && S >= 2048))) ? 8 : 4;
    if (const char* e = std::getenv("FLASH_ATTN_WAVES")) {
      const int v = std::atoi(e);
      if (v == 4 || v == 8) pl.nw = v;
    }
    pl.block_q = 32 * pl.nw;
    pl.block_k = kFastBC;
    if (plain && pl.nw == 4) {
      const int64_t nb = S / 128 + (S % 128 != 0);
      if (BH < 512 && nb < 512 && BH * nb < 512) pl.parts = (D == 64 && BH * nb <= 128) ? 4 : 2;
      if (const char* e = std::getenv("FLASH_ATTN_PARTS")) {
        if (e[0] == '0') pl.parts = 0;
        if (e[0] == '2') pl.parts = 2;
        if (e[0] == '4') pl.parts = D == 64 ? 4 : 2;
      }
      if (pl.parts == 4) pl.block_q = 64;
    }
  } else {
    pl.fast = false;
    pl.nw = 4;
    pl.block_q = kGenericBR;
    pl.block_k = kGenericBC;
  }
  return pl;
}

int prepare_fwd(const FwdCall& a, FwdLaunch* out, std::string* err) {
  const int64_t B = a.B, H = a.H, Hkv = a.H_kv, S = a.S, D = a.D;
  if (!a.q || !a.k || !a.v || !a.o || !a.lse) return fail(err, FA_ERR_INVALID, "null tensor pointer");
  if (B < 1 || H < 1 || S < 1) return fail(err, FA_ERR_INVALID, "B, H and S must be >= 1");
  if (Hkv < 1 || H % Hkv != 0)
    return fail(err, FA_ERR_INVALID, "key/value heads must be >= 1 and divide the query heads");
  if (D < 1) return fail(err, FA_ERR_INVALID, "D must be >= 1");
  if (a.causal != 0 && a.causal != 1) return fail(err, FA_ERR_INVALID, "causal must be 0 or 1");
  if (a.window < 0) return fail(err, FA_ERR_INVALID, "window must be >= 0");
  if (a.window > 0 && !a.causal)
    return fail(err, FA_ERR_INVALID, "a sliding window needs causal = 1");
  if (a.n_sink < 0) return fail(err, FA_ERR_INVALID, "n_sink must be >= 0");
  if (!std::isfinite(a.scale)) return fail(err, FA_ERR_INVALID, "scale must be finite");
  const int e = elem_bytes(a.dtype);
  if (e == 0) return fail(err, FA_ERR_INVALID, "unknown dtype");
  if (!aligned(a.q, 16) || !aligned(a.k, 16) || !aligned(a.v, 16) || !aligned(a.o, 16))
    return fail(err, FA_ERR_INVALID, "q, k, v and o must be 16-byte aligned");
  if (!aligned(a.lse, 4)) return fail(err, FA_ERR_INVALID, "lse must be 4-byte aligned");
  if (a.block_pairs && !aligned(a.block_pairs, 8))
    return fail(err, FA_ERR_INVALID, "block_pairs must be 8-byte aligned");
  if (a.alibi && !aligned(a.alibi, 4))
    return fail(err, FA_ERR_INVALID, "alibi_slopes must be 4-byte aligned");
  // Byte sizes must fit in int64: B*H*S*D*e.
  const int64_t lim = INT64_MAX;
  if (B > lim / H) return fail(err, FA_ERR_INVALID, "B*H overflows");
  const int64_t bh = B * H;
  if (bh > lim / S) return fail(err, FA_ERR_INVALID, "B*H*S overflows");
  const int64_t rows = bh * S;
  if (rows > lim / D || rows * D > lim / e) return fail(err, FA_ERR_INVALID, "tensor size overflows");
  const uint64_t tbytes = (uint64_t)(rows * D * e);            // q and o
  const uint64_t kvbytes = tbytes / (uint64_t)(H / Hkv);        // k and v
  const uint64_t lbytes = (uint64_t)rows * 4;
  if (overlaps(a.o, tbytes, a.q, tbytes) || overlaps(a.o, tbytes, a.k, kvbytes) ||
      overlaps(a.o, tbytes, a.v, kvbytes))
    return fail(err, FA_ERR_INVALID, "o overlaps q, k or v");
  if (overlaps(a.lse, lbytes, a.o, tbytes) || overlaps(a.lse, lbytes, a.q, tbytes) ||
      overlaps(a.lse, lbytes, a.k, kvbytes) || overlaps(a.lse, lbytes, a.v, kvbytes))
    return fail(err, FA_ERR_INVALID, "lse overlaps o, q, k or v");
  if (a.alibi && (overlaps(a.alibi, (uint64_t)H * 4, a.o, tbytes) ||
                  overlaps(a.alibi, (uint64_t)H * 4, a.lse, lbytes)))
    return fail(err, FA_ERR_INVALID, "alibi_slopes overlaps o or lse");

  const int64_t n_split = a.n_split;
  if (n_split < 1 || n_split > 256) return fail(err, FA_ERR_INVALID, "n_split must be in [1, 256]");
  int64_t lse_off = 0;
  if (n_split > 1) {
    const int64_t need = split_ws(rows, D, n_split, &lse_off);
    if (need < 0) return fail(err, FA_ERR_INVALID, "workspace size overflows");
    if (!a.workspace) return fail(err, FA_ERR_INVALID, "null workspace");
    if (!aligned(a.workspace, 16))
      return fail(err, FA_ERR_INVALID, "workspace must be 16-byte aligned");
    if (a.workspace_bytes < need) return fail(err, FA_ERR_INVALID, "workspace too small");
    const uint64_t wb = (uint64_t)need;
    if (overlaps(a.workspace, wb, a.q, tbytes) || overlaps(a.workspace, wb, a.k, kvbytes) ||
        overlaps(a.workspace, wb, a.v, kvbytes) || overlaps(a.workspace, wb, a.o, tbytes) ||
        overlaps(a.workspace, wb, a.lse, lbytes) ||
        (a.alibi && overlaps(a.workspace, wb, a.alibi, (uint64_t)H * 4)))
      return fail(err, FA_ERR_INVALID, "workspace overlaps a tensor");
  }

  if (!supported_d(D)) return fail(err, FA_ERR_UNSUPPORTED, "head dim must be 16, 32, 64 or 128");
  if (n_split > 1 && !fast_supported(D, a.dtype))
    return fail(err, FA_ERR_UNSUPPORTED,
                "key splitting needs bf16 / f16 with head dim 64 or 128");
  const Plan plan = plan_fwd(bh, S, D, a.dtype, !a.alibi && n_split == 1, a.window);
  const int64_t br = plan.block_q;
  const int64_t nqb = (S + br - 1) / br;
  // grid = nqb * bh * n_split work-groups (times 256 threads at most) in 32 bits;
  // the product is bounded factor by factor so that it cannot overflow.
  const int64_t grid_lim = (int64_t)INT32_MAX / 256;
  if (S > INT32_MAX - 2 * br || bh > INT32_MAX || nqb > grid_lim / bh ||
      nqb * bh > grid_lim / n_split)
    return fail(err, FA_ERR_UNSUPPORTED, "S, B*H or the grid exceed the 32-bit index range");

  FwdParams& p = out->p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.block_pairs = reinterpret_cast<unsigned long long*>(a.block_pairs);
  p.alibi = a.alibi;
  p.n_split = (int)n_split;
  p.o_part = nullptr;
  p.lse_part = nullptr;
  if (n_split > 1) {
    p.o_part = static_cast<float*>(a.workspace);
    p.lse_part = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + lse_off);
  }
  p.S = (int)S;
  p.BH = (int)bh;
  p.H = (int)H;
  p.G = (int)(H / Hkv);
  p.nqb = (int)nqb;
  p.causal = a.causal;
  // A window as wide as the sequence hides nothing: fold it to "no window".
  p.window = (a.window >= S) ? 0 : (int)a.window;
  p.n_sink = (p.window == 0) ? 0 : (int)(a.n_sink < S ? a.n_sink : S);
  // scores are used as exp2(c * s - m2) with c = |scale| log2(e) > 0; a
  // negative scale flips the sign of Q instead. A zero scale uses the
  // smallest normal float, whose products with finite scores round exp2 to
  // exactly 1, the result of a zero scale, while -inf masked scores stay -inf.
  const double c = std::fabs((double)a.scale) * 1.4426950408889634;
  float cf = (float)c;
  if (!(cf >= FLT_MIN)) cf = FLT_MIN;
  p.c = cf;
  p.neg = a.scale < 0.f ? 1 : 0;
  p.reverse = reverse_order();
  p.parts = plan.parts;
  out->plan = plan;
  out->rows = rows;
  return FA_OK;
}

int check_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, int64_t rows,
                int64_t D, const void* o, const float* lse, int dtype, std::string* err) {
  if (!o_parts || !lse_parts || !o || !lse) return fail(err, FA_ERR_INVALID, "null pointer");
  if (n_parts < 1 || n_parts > 4096 || rows < 1 || D < 1)
    return fail(err, FA_ERR_INVALID, "n_parts in [1, 4096], rows and D must be >= 1");
  const int e = elem_bytes(dtype);
  if (e == 0) return fail(err, FA_ERR_INVALID, "unknown dtype");
  if (!aligned(o_parts, 16) || !aligned(o, 16))
    return fail(err, FA_ERR_INVALID, "o_parts and o must be 16-byte aligned");
  if (!aligned(lse_parts, 4) || !aligned(lse, 4))
    return fail(err, FA_ERR_INVALID, "lse_parts and lse must be 4-byte aligned");
  const int64_t lim = INT64_MAX / 8;
  if (rows > lim / n_parts || rows * n_parts > lim / D)
    return fail(err, FA_ERR_INVALID, "size overflows");
  const uint64_t pb = (uint64_t)(rows * n_parts * D * 4), lb = (uint64_t)(rows * n_parts * 4);
  const uint64_t ob = (uint64_t)(rows * D * e), ol = (uint64_t)(rows * 4);
  if (overlaps(o, ob, o_parts, pb) || overlaps(o, ob, lse_parts, lb) ||
      overlaps(lse, ol, o_parts, pb) || overlaps(lse, ol, lse_parts, lb) || overlaps(o, ob, lse, ol))
    return fail(err, FA_ERR_INVALID, "outputs overlap the partials or each other");
  if (!supported_d(D)) return fail(err, FA_ERR_UNSUPPORTED, "head dim must be 16, 32, 64 or 128");
  if (rows > (int64_t)UINT32_MAX) return fail(err, FA_ERR_UNSUPPORTED, "too many rows");
  return FA_OK;
}

int64_t split_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D, int64_t n_split,
                              std::string* err) {
  if (B < 1 || H < 1 || S < 1 || D < 1 || n_split < 1 || n_split > 256) {
    fail(err, FA_ERR_INVALID, "B, H, S, D must be >= 1 and n_split in [1, 256]");
    return -1;
  }
  if (B > INT64_MAX / H || B * H > INT64_MAX / S) {
    fail(err, FA_ERR_INVALID, "B*H*S overflows");
    return -1;
  }
  if (n_split == 1) return 0;
  const int64_t r = split_ws(B * H * S, D, n_split, nullptr);
  if (r < 0) fail(err, FA_ERR_INVALID, "workspace size overflows");
  return r;
}

int64_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t S, std::string* err) {
  if (B < 1 || H < 1 || S < 1) {
    fail(err, FA_ERR_INVALID, "B, H and S must be >= 1");
    return -1;
  }
  // two fp32 arrays [B*H][Sp] (per-row delta and lse * log2(e)), Sp = S
  // rounded up to the dq kernel's block of rows
  const int64_t br = kBwdRows;
  if (S > INT64_MAX / 16 || B > INT64_MAX / 16 / H || B * H > INT64_MAX / 16 / (S + br)) {
    fail(err, FA_ERR_INVALID, "B*H*S overflows");
    return -1;
  }
  const int64_t sp = (S + br - 1) / br * br;
  return (2 * B * H * sp * 4 + 255) / 256 * 256;
}

int prepare_bwd(const BwdCall& a, BwdParams* out, std::string* err) {
  const int64_t B = a.B, H = a.H, H_kv = a.H_kv, S = a.S, D = a.D;
  if (!a.q || !a.k || !a.v || !a.o || !a.dout || !a.lse || !a.dq || !a.dk || !a.dv ||
      (!a.workspace && !a.internal_workspace))
    return fail(err, FA_ERR_INVALID, "null pointer");
  if (B < 1 || H < 1 || S < 1 || D < 1)
    return fail(err, FA_ERR_INVALID, "B, H, S and D must be >= 1");
  if (H_kv < 1 || H % H_kv != 0)
    return fail(err, FA_ERR_INVALID, "key/value heads must be >= 1 and divide the query heads");
  if (a.causal != 0 && a.causal != 1) return fail(err, FA_ERR_INVALID, "causal must be 0 or 1");
  if (a.window < 0) return fail(err, FA_ERR_INVALID, "window must be >= 0");
  if (a.window > 0 && !a.causal)
    return fail(err, FA_ERR_INVALID, "a sliding window needs causal = 1");
  if (a.n_sink < 0) return fail(err, FA_ERR_INVALID, "n_sink must be >= 0");
  if (!std::isfinite(a.scale)) return fail(err, FA_ERR_INVALID, "scale must be finite");
  const int e = elem_bytes(a.dtype);
  if (e == 0) return fail(err, FA_ERR_INVALID, "unknown dtype");
  const void* al16[] = {a.q, a.k, a.v, a.o, a.dout, a.dq, a.dk, a.dv, a.workspace};
  for (const void* ptr : al16)
    if (!aligned(ptr, 16))
      return fail(err, FA_ERR_INVALID, "tensors and workspace must be 16-byte aligned");
  if (!aligned(a.lse, 4)) return fail(err, FA_ERR_INVALID, "lse must be 4-byte aligned");
  if (a.alibi && !aligned(a.alibi, 4))
    return fail(err, FA_ERR_INVALID, "alibi_slopes must be 4-byte aligned");
  const int64_t lim = INT64_MAX / 8;
  if (B > lim / H || B * H > lim / S || B * H * S > lim / D / e)
    return fail(err, FA_ERR_INVALID, "tensor size overflows");
  const int64_t rows = B * H * S;
  const uint64_t tb = (uint64_t)(rows * D * e), kvb = tb / (uint64_t)(H / H_kv);
  const uint64_t lb = (uint64_t)rows * 4;
  const int64_t need = bwd_workspace_bytes(B, H, S, err);
  if (need < 0) return FA_ERR_INVALID;
  if (!a.internal_workspace && a.workspace_bytes < need)
    return fail(err, FA_ERR_INVALID, "workspace too small");
  struct Region {
    const void* p;
    uint64_t n;
  };
  // (the library's scratch array is its own allocation and overlaps nothing)
  const Region outs[] = {{a.dq, tb}, {a.dk, kvb}, {a.dv, kvb},
                         {a.workspace, a.internal_workspace ? 0 : (uint64_t)need}};
  const Region ins[] = {{a.q, tb},    {a.k, kvb},   {a.v, kvb}, {a.o, tb},
                        {a.dout, tb}, {a.lse, lb}, {a.alibi, a.alibi ? (uint64_t)H * 4 : 0}};
  for (const Region& x : outs) {
    for (const Region& y : ins)
      if (x.n && y.p && overlaps(x.p, x.n, y.p, y.n))
        return fail(err, FA_ERR_INVALID, "an output or the workspace overlaps an input");
    for (const Region& y : outs)
      if (&x != &y && x.n && y.n && overlaps(x.p, x.n, y.p, y.n))
        return fail(err, FA_ERR_INVALID, "outputs overlap each other or the workspace");
  }
  if (!supported_d(D)) return fail(err, FA_ERR_UNSUPPORTED, "head dim must be 16, 32, 64 or 128");
  if (!bwd_supported(D, a.dtype))
    return fail(err, FA_ERR_UNSUPPORTED,
                "the backward pass needs bf16 / f16 with head dim 64 or 128");
  const int64_t br = kBwdRows;
  const int64_t nb = (S + br - 1) / br;
  if (S > INT32_MAX - 2 * br || B * H > INT32_MAX || nb * B * H > (int64_t)INT32_MAX / 256)
    return fail(err, FA_ERR_UNSUPPORTED, "S, B*H or the grid exceed the 32-bit index range");
  if (a.internal_workspace && need > a.workspace_bytes)
    return fail(err, FA_ERR_UNSUPPORTED,
                "the allocation-free backward keeps at most 32 MiB of per-row state "
                "(8 bytes per row of B*H*S, S rounded up to 128): use flash_attn_bwd "
                "with a workspace");

  BwdParams& p = *out;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.dout = a.dout;
  p.lse = a.lse;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  const int64_t sp = nb * br;   // rows per head of the two workspace arrays
  p.Sp = (int)sp;
  p.BH = (int)(B * H);
  bwd_bind_workspace(&p, a.workspace);
  p.alibi = a.alibi;
  p.S = (int)S;
  p.BH = (int)(B * H);
  p.H = (int)H;
  p.G = (int)(H / H_kv);
  p.nqb = (int)nb;
  p.nkb = (int)nb;
  p.causal = a.causal;
  p.window = (a.window >= S) ? 0 : (int)a.window;
  p.n_sink = (p.window == 0) ? 0 : (int)(a.n_sink < S ? a.n_sink : S);
  p.scale = a.scale;
  p.c = (float)((double)a.scale * 1.4426950408889634);
  p.dkv_pair = bwd_dkv_pair(nb * (B * H_kv), a.causal != 0, p.window > 0);
  return FA_OK;
}

int bwd_kernel_name(int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D, int dtype, int causal,
                    int64_t window, int alibi, std::string* name, std::string* err) {
  if (!name) return fail(err, FA_ERR_INVALID, "null output pointer");
  if (B < 1 || H < 1 || S < 1) return fail(err, FA_ERR_INVALID, "B, H and S must be >= 1");
  if (H_kv < 1 || H % H_kv != 0)
    return fail(err, FA_ERR_INVALID, "key/value heads must be >= 1 and divide the query heads");
  if (elem_bytes(dtype) == 0) return fail(err, FA_ERR_INVALID, "unknown dtype");
  if (window < 0) return fail(err, FA_ERR_INVALID, "window must be >= 0");
  if (!bwd_supported(D, dtype))
    return fail(err, FA_ERR_UNSUPPORTED,
                "the backward pass needs bf16 / f16 with head dim 64 or 128");
  if (B > INT64_MAX / H) return fail(err, FA_ERR_INVALID, "B*H overflows");
  const int64_t nb = S / kBwdRows + (S % kBwdRows != 0);
  const int64_t kv = B * H_kv;
  const int64_t grid = kv > INT64_MAX / nb ? INT64_MAX : nb * kv;
  const bool pair = bwd_dkv_pair(grid, causal != 0, window > 0 && window < S);
  const std::string t = std::string("<") + (dtype == kDtypeF16 ? "f16" : "bf16") + ",D=" +
                        std::to_string(D) + (alibi ? ",alibi" : "") + ">";
  *name = "fa_bwd_dq_kernel" + t + " (128 rows, 4 waves) + " +
          (pair ? "fa_bwd_dkv2_kernel" + t + " (128 keys, 4 waves, 2 work-groups per CU)"
                : "fa_bwd_dkv_kernel" + t + " (128 keys, 4 waves, 1 work-group per CU)");
  return FA_OK;
}

bool bwd_dkv_pair(int64_t grid, bool causal, bool window) {
  bool pair = grid >= 1024 || ((!causal || window) && grid >= 512);
  if (const char* e = std::getenv("FLASH_ATTN_DKV")) {
    if (e[0] == '1') pair = false;
    if (e[0] == '2') pair = true;
  }
  return pair;
}

void bwd_bind_workspace(BwdParams* p, void* ws) {
  p->delta = static_cast<float*>(ws);
  p->lse2 = ws ? static_cast<float*>(ws) + (int64_t)p->BH * p->Sp : nullptr;
}

int tile_shape(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int64_t window, int* block_q,
               int* block_k, std::string* err) {
  if (!block_q || !block_k) return fail(err, FA_ERR_INVALID, "null output pointer");
  if (B < 1 || H < 1 || S < 1) return fail(err, FA_ERR_INVALID, "B, H and S must be >= 1");
  if (window < 0) return fail(err, FA_ERR_INVALID, "window must be >= 0");
  if (elem_bytes(dtype) == 0) return fail(err, FA_ERR_INVALID, "unknown dtype");
  if (!supported_d(D)) return fail(err, FA_ERR_UNSUPPORTED, "head dim must be 16, 32, 64 or 128");
  if (B > INT64_MAX / H) return fail(err, FA_ERR_INVALID, "B*H overflows");
  const Plan plan = plan_fwd(B * H, S, D, dtype, true, window);
  *block_q = plan.block_q;
  *block_k = plan.block_k;
  return FA_OK;
}

int fwd_kernel_name(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int alibi,
                    int64_t n_split, int64_t window, std::string* name, std::string* err) {
  if (!name) return fail(err, FA_ERR_INVALID, "null output pointer");
  if (B < 1 || H < 1 || S < 1) return fail(err, FA_ERR_INVALID, "B, H and S must be >= 1");
  if (window < 0) return fail(err, FA_ERR_INVALID, "window must be >= 0");
  const int e = elem_bytes(dtype);
  if (e == 0) return fail(err, FA_ERR_INVALID, "unknown dtype");
  if (n_split < 1 || n_split > 256) return fail(err, FA_ERR_INVALID, "n_split must be in [1, 256]");
  if (!supported_d(D)) return fail(err, FA_ERR_UNSUPPORTED, "head dim must be 16, 32, 64 or 128");
  if (n_split > 1 && !fast_supported(D, dtype))
    return fail(err, FA_ERR_UNSUPPORTED, "key splitting needs bf16 / f16 with head dim 64 or 128");
  if (B > INT64_MAX / H) return fail(err, FA_ERR_INVALID, "B*H overflows");
  const Plan plan = plan_fwd(B * H, S, D, dtype, !alibi && n_split == 1, window);
  const char* ty = dtype == kDtypeF32 ? "f32" : dtype == kDtypeF16 ? "f16" : "bf16";
  const std::string d = std::to_string(D);
  const std::string tile = " (" + std::to_string(plan.block_q) + "x" + std::to_string(plan.block_k) + " tile)";
  if (!plan.fast)
    *name = std::string(dtype == kDtypeF32 ? "fa_fwd_f32_kernel<D=" : "fa_fwd_half_kernel<D=") + d +
            ">" + tile;
  else if (plan.parts)
    *name = std::string("fa_fwd_parts_kernel<") + ty + ",D=" + d + ",parts=" +
            std::to_string(plan.parts) + "> (8 waves, " + tile.substr(2);
  else
    *name = std::string("fa_fwd_fast_kernel<") + ty + ",D=" + d + ",waves=" +
            std::to_string(plan.nw) + (alibi ? ",alibi" : "") + ">" + tile;
  if (n_split > 1) *name += " + fa_merge_kernel";
  return FA_OK;
}

}  // namespace fa
