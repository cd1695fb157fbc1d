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

int forward(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
            int64_t Hkv, int64_t S, int64_t D, int causal, int64_t window, int64_t n_sink,
            float scale, const float* alibi, void* stream, int dtype, uint64_t* block_pairs) {
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
  if (overlaps(lse, (uint64_t)rows * 4, o, tbytes))
    return fail(FA_ERR_INVALID, "lse overlaps o");
  if (alibi && (overlaps(alibi, (uint64_t)H * 4, o, tbytes) ||
                overlaps(alibi, (uint64_t)H * 4, lse, (uint64_t)rows * 4)))
    return fail(FA_ERR_INVALID, "alibi_slopes overlaps o or lse");

  if (!supported_d(D)) return fail(FA_ERR_UNSUPPORTED, "head dim must be 16, 32, 64 or 128");
  const fa::Plan plan = fa::plan_fwd(B * H, S, D, dtype);
  const int64_t br = plan.block_q;
  const int64_t nqb = (S + br - 1) / br;
  if (S > INT32_MAX - 2 * br || bh > INT32_MAX || nqb * bh > (int64_t)UINT32_MAX / 256)
    return fail(FA_ERR_UNSUPPORTED, "S, B*H or the grid exceed the 32-bit index range");

  fa::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.block_pairs = reinterpret_cast<unsigned long long*>(block_pairs);
  p.alibi = alibi;
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
