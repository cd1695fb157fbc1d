// C ABI of the attention library: argument validation (fa_validate.cpp) then
// the launches on the caller's stream. See include/flash_attn.h for the
// contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>

#include "../../include/flash_attn.h"
#include "fa_kernel.h"
#include "fa_validate.h"

namespace {

thread_local std::string g_last_error;

int launch_failed(hipError_t err) {
  g_last_error = std::string("HIP launch failed: ") + hipGetErrorString(err);
  return FA_ERR_HIP;
}

int forward(const fa::FwdCall& a, void* stream) {
  g_last_error.clear();
  fa::FwdLaunch l;
  const int rc = fa::prepare_fwd(a, &l, &g_last_error);
  if (rc != FA_OK) return rc;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t err = fa::launch_plan(l.plan, l.p, (int)a.D, a.dtype, st);
  if (err == hipSuccess && l.p.n_split > 1)
    err = fa::launch_merge(l.p.o_part, l.p.lse_part, l.p.n_split, l.rows, (int)a.D, a.o, a.lse,
                           a.dtype, st);
  return err == hipSuccess ? FA_OK : launch_failed(err);
}

fa::FwdCall fwd_call(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                     int64_t H, int64_t H_kv, int64_t S, int64_t D, int causal, int64_t window,
                     int64_t n_sink, float scale, const float* alibi, int dtype) {
  fa::FwdCall a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.S = S;
  a.D = D;
  a.causal = causal;
  a.window = window;
  a.n_sink = n_sink;
  a.scale = scale;
  a.alibi = alibi;
  a.dtype = dtype;
  return a;
}

}  // namespace

extern "C" {

int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                   int64_t H, int64_t S, int64_t D, int causal, int64_t window, int64_t n_sink,
                   float scale, void* stream, int dtype) {
  return forward(fwd_call(q, k, v, o, lse, B, H, H, S, D, causal, window, n_sink, scale, nullptr,
                          dtype),
                 stream);
}

int flash_attn_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                       int64_t H, int64_t H_kv, int64_t S, int64_t D, int causal, int64_t window,
                       int64_t n_sink, float scale, const float* alibi_slopes, void* stream,
                       int dtype) {
  return forward(fwd_call(q, k, v, o, lse, B, H, H_kv, S, D, causal, window, n_sink, scale,
                          alibi_slopes, dtype),
                 stream);
}

int flash_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D, int causal,
                         int64_t window, int64_t n_sink, float scale, const float* alibi_slopes,
                         int64_t n_split, void* workspace, int64_t workspace_bytes, void* stream,
                         int dtype) {
  fa::FwdCall a = fwd_call(q, k, v, o, lse, B, H, H_kv, S, D, causal, window, n_sink, scale,
                           alibi_slopes, dtype);
  a.n_split = n_split;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  return forward(a, stream);
}

int64_t flash_attn_split_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D,
                                         int64_t n_split) {
  g_last_error.clear();
  return fa::split_workspace_bytes(B, H, S, D, n_split, &g_last_error);
}

int flash_attn_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, int64_t rows,
                     int64_t D, void* o, float* lse, void* stream, int dtype) {
  g_last_error.clear();
  const int rc = fa::check_merge(o_parts, lse_parts, n_parts, rows, D, o, lse, dtype, &g_last_error);
  if (rc != FA_OK) return rc;
  const hipError_t err = fa::launch_merge(o_parts, lse_parts, (int)n_parts, rows, (int)D, o, lse,
                                          dtype, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : launch_failed(err);
}

int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                   int64_t H_kv, int64_t S, int64_t D, int causal, int64_t window, int64_t n_sink,
                   float scale, const float* alibi_slopes, void* workspace,
                   int64_t workspace_bytes, void* stream, int dtype) {
  g_last_error.clear();
  fa::BwdCall a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.S = S;
  a.D = D;
  a.causal = causal;
  a.window = window;
  a.n_sink = n_sink;
  a.scale = scale;
  a.alibi = alibi_slopes;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  a.dtype = dtype;
  fa::BwdParams p;
  const int rc = fa::prepare_bwd(a, &p, &g_last_error);
  if (rc != FA_OK) return rc;
  const hipError_t err = fa::launch_bwd(p, (int)D, dtype, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : launch_failed(err);
}

int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D, int causal,
                           int64_t window, int64_t n_sink, float scale, const float* alibi_slopes,
                           void* stream, int dtype) {
  g_last_error.clear();
  fa::BwdCall a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.S = S;
  a.D = D;
  a.causal = causal;
  a.window = window;
  a.n_sink = n_sink;
  a.scale = scale;
  a.alibi = alibi_slopes;
  a.internal_workspace = true;
  a.workspace_bytes = fa::kBwdScratchBytes;
  a.dtype = dtype;
  fa::BwdParams p;
  const int rc = fa::prepare_bwd(a, &p, &g_last_error);
  if (rc != FA_OK) return rc;
  void* ws = nullptr;
  hipError_t err = fa::bwd_scratch(&ws);
  if (err != hipSuccess) {
    g_last_error = std::string("scratch lookup failed: ") + hipGetErrorString(err);
    return FA_ERR_HIP;
  }
  fa::bwd_bind_workspace(&p, ws);
  err = fa::launch_bwd(p, (int)D, dtype, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : launch_failed(err);
}

int64_t flash_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t S) {
  g_last_error.clear();
  return fa::bwd_workspace_bytes(B, H, S, &g_last_error);
}

int flash_attn_fwd_counted(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t S, int64_t D, int causal, int64_t window,
                           int64_t n_sink, float scale, void* stream, int dtype,
                           uint64_t* block_pairs) {
  fa::FwdCall a = fwd_call(q, k, v, o, lse, B, H, H, S, D, causal, window, n_sink, scale, nullptr,
                           dtype);
  a.block_pairs = block_pairs;
  return forward(a, stream);
}

int flash_attn_tile_shape(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int64_t window,
                          int* block_q, int* block_k) {
  g_last_error.clear();
  return fa::tile_shape(B, H, S, D, dtype, window, block_q, block_k, &g_last_error);
}

int flash_attn_fwd_kernel(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int alibi,
                          int64_t n_split, int64_t window, char* buf, int64_t buf_bytes) {
  g_last_error.clear();
  if (!buf || buf_bytes < 1) {
    g_last_error = "null or empty output buffer";
    return FA_ERR_INVALID;
  }
  std::string name;
  const int rc = fa::fwd_kernel_name(B, H, S, D, dtype, alibi, n_split, window, &name,
                                     &g_last_error);
  const size_t n = rc == FA_OK ? std::min(name.size(), (size_t)(buf_bytes - 1)) : 0;
  std::memcpy(buf, name.data(), n);
  buf[n] = '\0';
  return rc;
}

int flash_attn_bwd_kernel(int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D, int dtype,
                          int causal, int64_t window, int alibi, char* buf, int64_t buf_bytes) {
  g_last_error.clear();
  if (!buf || buf_bytes < 1) {
    g_last_error = "null or empty output buffer";
    return FA_ERR_INVALID;
  }
  std::string name;
  const int rc =
      fa::bwd_kernel_name(B, H, H_kv, S, D, dtype, causal, window, alibi, &name, &g_last_error);
  const size_t n = rc == FA_OK ? std::min(name.size(), (size_t)(buf_bytes - 1)) : 0;
  std::memcpy(buf, name.data(), n);
  buf[n] = '\0';
  return rc;
}

const char* flash_attn_last_error(void) { return g_last_error.c_str(); }

const char* flash_attn_version(void) { return "io_aware_tiled_flash_amd 0.2 (gfx950)"; }

}  // extern "C"
