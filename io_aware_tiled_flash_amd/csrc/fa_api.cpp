// C ABI of the attention forward pass: host-side validation, normalisation of
// the mask arguments and dispatch to the gfx950 kernels. See flash_attn.h for
// the contract.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "../../include/flash_attn.h"
#include "fa_kernel.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* msg) {
  g_last_error = msg;
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
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
int64_t split_ws_bytes(int64_t rows, int64_t D, int64_t n_split, int64_t* lse_offset) {
  const int64_t lim = INT64_MAX / 8;
  if (rows > lim / n_split || rows * n_split > lim / (D + 1)) return -1;
  const int64_t o_bytes = rows * n_split * D * 4;
  const int64_t off = (o_bytes + 255) / 256 * 256;
  if (lse_offset) *lse_offset = off;
  return off + rows * n_split * 4;
}

int forward(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
            int64_t Hkv, int64_t S, int64_t D, int causal, int64_t window, int64_t n_sink,
            float scale, const float* alibi, void* stream, int dtype, uint64_t* block_pairs,
            int64_t n_split = 1, void* workspace = nullptr, int64_t workspace_bytes = 0) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID, "null tensor pointer");
  if (B < 1 || H < 1 || S < 1) return fail(FA_ERR_INVALID, "B, H and S must be >= 1");
  if (Hkv < 1 || H % Hkv != 0)
    return fail(FA_ERR_INVALID, "key/value heads must be >= 1 and divide the query heads");
  if (D < 1) return fail(FA_ERR_INVALID, "D must be >= 1");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID, "causal must be 0 or 1");
  if (window < 0) return fail(FA_ERR_INVALID, "window must be >= 0");
  if (window > 0 && !causal) return fail(FA_ERR_INVALID, "a sliding window needs causal = 1");
  if (n_sink < 0) return fail(FA_ERR_INVALID, "n_sink must be >= 0");
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID, "scale must be finite");
  const int e = elem_bytes(dtype);
  if (e == 0) return fail(FA_ERR_INVALID, "unknown dtype");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID, "q, k, v and o must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(FA_ERR_INVALID, "lse must be 4-byte aligned");
  if (block_pairs && !aligned(block_pairs, 8))
    return fail(FA_ERR_INVALID, "block_pairs must be 8-byte aligned");
  if (alibi && !aligned(alibi, 4)) return fail(FA_ERR_INVALID, "alibi_slopes must be 4-byte aligned");
  // Byte sizes must fit in int64: B*H*S*D*e.
  const int64_t lim = INT64_MAX;
  if (B > lim / H) return fail(FA_ERR_INVALID, "B*H overflows");
  const int64_t bh = B * H;
  if (bh > lim / S) return fail(FA_ERR_INVALID, "B*H*S overflows");
  const int64_t rows = bh * S;
  if (rows > lim / D || rows * D > lim / e) return fail(FA_ERR_INVALID, "tensor size overflows");
  const uint64_t tbytes = (uint64_t)(rows * D * e);            // q and o
  const uint64_t kvbytes = tbytes / (uint64_t)(H / Hkv);        // k and v
  if (overlaps(o, tbytes, q, tbytes) || overlaps(o, tbytes, k, kvbytes) ||
      overlaps(o, tbytes, v, kvbytes))
    return fail(FA_ERR_INVALID, "o overlaps q, k or v");
  if (overlaps(lse, (uint64_t)rows * 4, o, tbytes) || overlaps(lse, (uint64_t)rows * 4, q, tbytes) ||
      overlaps(lse, (uint64_t)rows * 4, k, kvbytes) || overlaps(lse, (uint64_t)rows * 4, v, kvbytes))
    return fail(FA_ERR_INVALID, "lse overlaps o, q, k or v");
  if (alibi && (overlaps(alibi, (uint64_t)H * 4, o, tbytes) ||
                overlaps(alibi, (uint64_t)H * 4, lse, (uint64_t)rows * 4)))
    return fail(FA_ERR_INVALID, "alibi_slopes overlaps o or lse");

  if (n_split < 1 || n_split > 256) return fail(FA_ERR_INVALID, "n_split must be in [1, 256]");
  int64_t lse_off = 0;
  if (n_split > 1) {
    const int64_t need = split_ws_bytes(rows, D, n_split, &lse_off);
    if (need < 0) return fail(FA_ERR_INVALID, "workspace size overflows");
    if (!workspace) return fail(FA_ERR_INVALID, "null workspace");
    if (!aligned(workspace, 16)) return fail(FA_ERR_INVALID, "workspace must be 16-byte aligned");
    if (workspace_bytes < need) return fail(FA_ERR_INVALID, "workspace too small");
    const uint64_t wb = (uint64_t)need;
    if (overlaps(workspace, wb, q, tbytes) || overlaps(workspace, wb, k, kvbytes) ||
        overlaps(workspace, wb, v, kvbytes) || overlaps(workspace, wb, o, tbytes) ||
        overlaps(workspace, wb, lse, (uint64_t)rows * 4) ||
        (alibi && overlaps(workspace, wb, alibi, (uint64_t)H * 4)))
      return fail(FA_ERR_INVALID, "workspace overlaps a tensor");
  }

  if (!supported_d(D)) return fail(FA_ERR_UNSUPPORTED, "head dim must be 16, 32, 64 or 128");
  if (n_split > 1 && !fa::fast_supported((int)D, dtype))
    return fail(FA_ERR_UNSUPPORTED, "key splitting needs bf16 / f16 with head dim 64 or 128");
  const fa::Plan plan = fa::plan_fwd(B * H, S, D, dtype);
  const int64_t br = plan.block_q;
  const int64_t nqb = (S + br - 1) / br;
  if (S > INT32_MAX - 2 * br || bh > INT32_MAX || nqb * bh * n_split > (int64_t)INT32_MAX / 256)
    return fail(FA_ERR_UNSUPPORTED, "S, B*H or the grid exceed the 32-bit index range");

  fa::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.block_pairs = reinterpret_cast<unsigned long long*>(block_pairs);
  p.alibi = alibi;
  p.n_split = (int)n_split;
  p.o_part = nullptr;
  p.lse_part = nullptr;
  if (n_split > 1) {
    p.o_part = static_cast<float*>(workspace);
    p.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + lse_off);
  }
  p.S = (int)S;
  p.BH = (int)bh;
  p.H = (int)H;
  p.G = (int)(H / Hkv);
  p.nqb = (int)nqb;
  p.causal = causal;
  // A window as wide as the sequence hides nothing: fold it to "no window".
  p.window = (window >= S) ? 0 : (int)window;
  p.n_sink = (p.window == 0) ? 0 : (int)(n_sink < S ? n_sink : S);
  // scores are used as exp2(c * s - m2) with c = |scale| log2(e) > 0; a
  // negative scale flips the sign of Q instead. A zero scale uses the
  // smallest normal float, whose products with finite scores round exp2 to
  // exactly 1, the result of a zero scale, while -inf masked scores stay -inf.
  double c = std::fabs((double)scale) * 1.4426950408889634;
  float cf = (float)c;
  if (!(cf >= FLT_MIN)) cf = FLT_MIN;
  p.c = cf;
  p.neg = scale < 0.f ? 1 : 0;

  hipError_t err = fa::launch_plan(plan, p, (int)D, dtype, reinterpret_cast<hipStream_t>(stream));
  if (err == hipSuccess && n_split > 1)
    err = fa::launch_merge(p.o_part, p.lse_part, (int)n_split, rows, (int)D, o, lse, dtype,
                           reinterpret_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    g_last_error = std::string("HIP launch failed: ") + hipGetErrorString(err);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

}  // namespace

namespace fa {

// Kernel choice. bf16/f16 with D = 64 or 128 take the fast kernel. Its
// work-group holds 4 waves (128 query rows), so two work-groups share a CU and
// run out of step with each other: one's softmax (vector ALU) overlaps the
// other's matrix products. Only for very long sequences (S >= 16384, with at
// least two 8-wave work-groups per CU) do 8 waves win, by halving the K/V
// tile traffic per query row. FLASH_ATTN_WAVES=4|8 overrides the wave count
// (tuning only).
Plan plan_fwd(int64_t BH, int64_t S, int64_t D, int dtype) {
  Plan pl;
  if (fast_supported((int)D, dtype)) {
    pl.fast = true;
    const int64_t wgs8 = BH * ((S + 255) / 256);
    pl.nw = (S >= 16384 && wgs8 >= 512) ? 8 : 4;
    if (const char* e = std::getenv("FLASH_ATTN_WAVES")) {
      const int v = std::atoi(e);
      if (v == 4 || v == 8) pl.nw = v;
    }
    pl.block_q = 32 * pl.nw;
    pl.block_k = fast_tile_keys();
  } else {
    pl.fast = false;
    pl.nw = 4;
    pl.block_q = generic_tile_rows();
    pl.block_k = generic_tile_keys();
  }
  return pl;
}

hipError_t launch_plan(const Plan& plan, const FwdParams& p, int D, int dtype, hipStream_t st) {
  if (plan.fast) return launch_fast(p, D, dtype, plan.nw, st);
  return launch_generic(p, D, dtype, st);
}

}  // namespace fa

extern "C" {

int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                   int64_t H, int64_t S, int64_t D, int causal, int64_t window, int64_t n_sink,
                   float scale, void* stream, int dtype) {
  return forward(q, k, v, o, lse, B, H, H, S, D, causal, window, n_sink, scale, nullptr, stream,
                 dtype, nullptr);
}

int flash_attn_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                       int64_t H, int64_t H_kv, int64_t S, int64_t D, int causal, int64_t window,
                       int64_t n_sink, float scale, const float* alibi_slopes, void* stream,
                       int dtype) {
  return forward(q, k, v, o, lse, B, H, H_kv, S, D, causal, window, n_sink, scale, alibi_slopes,
                 stream, dtype, nullptr);
}

int flash_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D, int causal,
                         int64_t window, int64_t n_sink, float scale, const float* alibi_slopes,
                         int64_t n_split, void* workspace, int64_t workspace_bytes, void* stream,
                         int dtype) {
  return forward(q, k, v, o, lse, B, H, H_kv, S, D, causal, window, n_sink, scale, alibi_slopes,
                 stream, dtype, nullptr, n_split, workspace, workspace_bytes);
}

int64_t flash_attn_split_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D,
                                         int64_t n_split) {
  g_last_error.clear();
  if (B < 1 || H < 1 || S < 1 || D < 1 || n_split < 1 || n_split > 256) {
    fail(FA_ERR_INVALID, "B, H, S, D must be >= 1 and n_split in [1, 256]");
    return -1;
  }
  if (B > INT64_MAX / H || B * H > INT64_MAX / S) {
    fail(FA_ERR_INVALID, "B*H*S overflows");
    return -1;
  }
  if (n_split == 1) return 0;
  const int64_t r = split_ws_bytes(B * H * S, D, n_split, nullptr);
  if (r < 0) fail(FA_ERR_INVALID, "workspace size overflows");
  return r;
}

int flash_attn_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, int64_t rows,
                     int64_t D, void* o, float* lse, void* stream, int dtype) {
  g_last_error.clear();
  if (!o_parts || !lse_parts || !o || !lse) return fail(FA_ERR_INVALID, "null pointer");
  if (n_parts < 1 || n_parts > 4096 || rows < 1 || D < 1)
    return fail(FA_ERR_INVALID, "n_parts in [1, 4096], rows and D must be >= 1");
  const int e = elem_bytes(dtype);
  if (e == 0) return fail(FA_ERR_INVALID, "unknown dtype");
  if (!aligned(o_parts, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID, "o_parts and o must be 16-byte aligned");
  if (!aligned(lse_parts, 4) || !aligned(lse, 4))
    return fail(FA_ERR_INVALID, "lse_parts and lse must be 4-byte aligned");
  const int64_t lim = INT64_MAX / 8;
  if (rows > lim / n_parts || rows * n_parts > lim / D) return fail(FA_ERR_INVALID, "size overflows");
  const uint64_t pb = (uint64_t)(rows * n_parts * D * 4), lb = (uint64_t)(rows * n_parts * 4);
  const uint64_t ob = (uint64_t)(rows * D * e), ol = (uint64_t)(rows * 4);
  if (overlaps(o, ob, o_parts, pb) || overlaps(o, ob, lse_parts, lb) ||
      overlaps(lse, ol, o_parts, pb) || overlaps(lse, ol, lse_parts, lb) || overlaps(o, ob, lse, ol))
    return fail(FA_ERR_INVALID, "outputs overlap the partials or each other");
  if (!supported_d(D)) return fail(FA_ERR_UNSUPPORTED, "head dim must be 16, 32, 64 or 128");
  if (rows > (int64_t)UINT32_MAX) return fail(FA_ERR_UNSUPPORTED, "too many rows");
  hipError_t err = fa::launch_merge(o_parts, lse_parts, (int)n_parts, rows, (int)D, o, lse, dtype,
                                    reinterpret_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    g_last_error = std::string("HIP launch failed: ") + hipGetErrorString(err);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                   int64_t H_kv, int64_t S, int64_t D, int causal, int64_t window, int64_t n_sink,
                   float scale, const float* alibi_slopes, void* workspace,
                   int64_t workspace_bytes, void* stream, int dtype) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
    return fail(FA_ERR_INVALID, "null pointer");
  if (B < 1 || H < 1 || S < 1 || D < 1) return fail(FA_ERR_INVALID, "B, H, S and D must be >= 1");
  if (H_kv < 1 || H % H_kv != 0)
    return fail(FA_ERR_INVALID, "key/value heads must be >= 1 and divide the query heads");
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID, "causal must be 0 or 1");
  if (window < 0) return fail(FA_ERR_INVALID, "window must be >= 0");
  if (window > 0 && !causal) return fail(FA_ERR_INVALID, "a sliding window needs causal = 1");
  if (n_sink < 0) return fail(FA_ERR_INVALID, "n_sink must be >= 0");
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID, "scale must be finite");
  const int e = elem_bytes(dtype);
  if (e == 0) return fail(FA_ERR_INVALID, "unknown dtype");
  const void* al16[] = {q, k, v, o, dout, dq, dk, dv, workspace};
  for (const void* ptr : al16)
    if (!aligned(ptr, 16)) return fail(FA_ERR_INVALID, "tensors and workspace must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(FA_ERR_INVALID, "lse must be 4-byte aligned");
  if (alibi_slopes && !aligned(alibi_slopes, 4))
    return fail(FA_ERR_INVALID, "alibi_slopes must be 4-byte aligned");
  const int64_t lim = INT64_MAX / 8;
  if (B > lim / H || B * H > lim / S || B * H * S > lim / D / e)
    return fail(FA_ERR_INVALID, "tensor size overflows");
  const int64_t rows = B * H * S;
  const uint64_t tb = (uint64_t)(rows * D * e), kvb = tb / (uint64_t)(H / H_kv);
  const uint64_t lb = (uint64_t)rows * 4;
  const int64_t need = flash_attn_bwd_workspace_bytes(B, H, S);
  if (need < 0) return FA_ERR_INVALID;
  if (workspace_bytes < need) return fail(FA_ERR_INVALID, "workspace too small");
  struct Region { const void* p; uint64_t n; };
  const Region outs[] = {{dq, tb}, {dk, kvb}, {dv, kvb}, {workspace, (uint64_t)need}};
  const Region ins[] = {{q, tb}, {k, kvb}, {v, kvb}, {o, tb}, {dout, tb}, {lse, lb},
                        {alibi_slopes, alibi_slopes ? (uint64_t)H * 4 : 0}};
  for (const Region& a : outs) {
    for (const Region& b : ins)
      if (b.p && overlaps(a.p, a.n, b.p, b.n))
        return fail(FA_ERR_INVALID, "an output or the workspace overlaps an input");
    for (const Region& b : outs)
      if (&a != &b && overlaps(a.p, a.n, b.p, b.n))
        return fail(FA_ERR_INVALID, "outputs overlap each other or the workspace");
  }
  if (!supported_d(D)) return fail(FA_ERR_UNSUPPORTED, "head dim must be 16, 32, 64 or 128");
  if (!fa::bwd_supported((int)D, dtype))
    return fail(FA_ERR_UNSUPPORTED, "the backward pass needs bf16 / f16 with head dim 64 or 128");
  const int64_t br = fa::bwd_tile_rows();
  const int64_t nb = (S + br - 1) / br;
  if (S > INT32_MAX - 2 * br || B * H > INT32_MAX || nb * B * H > (int64_t)INT32_MAX / 256)
    return fail(FA_ERR_UNSUPPORTED, "S, B*H or the grid exceed the 32-bit index range");

  fa::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  const int64_t sp = nb * br;   // rows per head of the two workspace arrays
  p.delta = static_cast<float*>(workspace);
  p.lse2 = static_cast<float*>(workspace) + B * H * sp;
  p.Sp = (int)sp;
  p.alibi = alibi_slopes;
  p.S = (int)S;
  p.BH = (int)(B * H);
  p.H = (int)H;
  p.G = (int)(H / H_kv);
  p.nqb = (int)nb;
  p.nkb = (int)nb;
  p.causal = causal;
  p.window = (window >= S) ? 0 : (int)window;
  p.n_sink = (p.window == 0) ? 0 : (int)(n_sink < S ? n_sink : S);
  p.scale = scale;
  p.c = (float)((double)scale * 1.4426950408889634);
  hipError_t err = fa::launch_bwd(p, (int)D, dtype, reinterpret_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    g_last_error = std::string("HIP launch failed: ") + hipGetErrorString(err);
    return FA_ERR_HIP;
  }
  return FA_OK;
}

int64_t flash_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S) {
  g_last_error.clear();
  if (B < 1 || H < 1 || S < 1) {
    fail(FA_ERR_INVALID, "B, H and S must be >= 1");
    return -1;
  }
  // two fp32 arrays [B*H][Sp] (per-row delta and lse * log2(e)), Sp = S
  // rounded up to the dq kernel's block of rows
  const int64_t br = fa::bwd_tile_rows();
  if (S > INT64_MAX / 16 || B > INT64_MAX / 16 / H || B * H > INT64_MAX / 16 / (S + br)) {
    fail(FA_ERR_INVALID, "B*H*S overflows");
    return -1;
  }
  const int64_t sp = (S + br - 1) / br * br;
  return (2 * B * H * sp * 4 + 255) / 256 * 256;
}

int flash_attn_fwd_counted(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t S, int64_t D, int causal, int64_t window,
                           int64_t n_sink, float scale, void* stream, int dtype,
                           uint64_t* block_pairs) {
  return forward(q, k, v, o, lse, B, H, H, S, D, causal, window, n_sink, scale, nullptr, stream,
                 dtype, block_pairs);
}

int flash_attn_tile_shape(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int* block_q,
                          int* block_k) {
  g_last_error.clear();
  if (!block_q || !block_k) return fail(FA_ERR_INVALID, "null output pointer");
  if (B < 1 || H < 1 || S < 1) return fail(FA_ERR_INVALID, "B, H and S must be >= 1");
  if (elem_bytes(dtype) == 0) return fail(FA_ERR_INVALID, "unknown dtype");
  if (!supported_d(D)) return fail(FA_ERR_UNSUPPORTED, "head dim must be 16, 32, 64 or 128");
  if (B > INT64_MAX / H) return fail(FA_ERR_INVALID, "B*H overflows");
  const fa::Plan plan = fa::plan_fwd(B * H, S, D, dtype);
  *block_q = plan.block_q;
  *block_k = plan.block_k;
  return FA_OK;
}

const char* flash_attn_last_error(void) { return g_last_error.c_str(); }

const char* flash_attn_version(void) { return "io_aware_tiled_flash_amd 0.1 (gfx950)"; }

}  // extern "C"
