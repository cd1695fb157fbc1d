// Host-side argument validation of the C ABI (include/flash_attn.h): every
// precondition check, the normalisation of the mask and scale arguments, the
// workspace sizes and the kernel plan. Plain C++ with no HIP dependency, so it
// can be built and exercised on the host alone (the library links it with the
// launches in fa_api.cpp). Each function returns FA_OK or the FA_ERR_* code
// the ABI documents, with the reason in *err; nothing here touches memory
// behind the pointers it is given.
#pragma once

#include <stdint.h>

#include <string>

#include "fa_shapes.h"

namespace fa {

// The arguments of flash_attn_fwd / _ext / _split / _counted, as passed.
struct FwdCall {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  void* o = nullptr;
  float* lse = nullptr;
  int64_t B = 0, H = 0, H_kv = 0, S = 0, D = 0;
  int causal = 0;
  int64_t window = 0, n_sink = 0;
  float scale = 0.f;
  const float* alibi = nullptr;
  int dtype = 0;
  uint64_t* block_pairs = nullptr;
  int64_t n_split = 1;
  void* workspace = nullptr;
  int64_t workspace_bytes = 0;
};

// What a valid forward call launches: the kernel parameters, the plan, the
// number of output rows (B*H*S) and, with a key split, the merge's inputs.
struct FwdLaunch {
  FwdParams p;
  Plan plan;
  int64_t rows = 0;
};

int prepare_fwd(const FwdCall& a, FwdLaunch* out, std::string* err);

// The arguments of flash_attn_bwd, as passed.
struct BwdCall {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  const void* o = nullptr;
  const void* dout = nullptr;
  const float* lse = nullptr;
  void* dq = nullptr;
  void* dk = nullptr;
  void* dv = nullptr;
  int64_t B = 0, H = 0, H_kv = 0, S = 0, D = 0;
  int causal = 0;
  int64_t window = 0, n_sink = 0;
  float scale = 0.f;
  const float* alibi = nullptr;
  void* workspace = nullptr;
  int64_t workspace_bytes = 0;
  int dtype = 0;
  // The library's own scratch array holds the per-row state instead of a
  // caller workspace (the allocation-free entry point): the workspace pointer
  // is then bound after validation, and workspace_bytes is the array's size;
  // a shape that needs more is FA_ERR_UNSUPPORTED.
  bool internal_workspace = false;
};

int prepare_bwd(const BwdCall& a, BwdParams* out, std::string* err);

// Points the backward's two per-row arrays into the workspace ws.
void bwd_bind_workspace(BwdParams* p, void* ws);

// flash_attn_merge's checks.
int check_merge(const float* o_parts, const float* lse_parts, int64_t n_parts, int64_t rows,
                int64_t D, const void* o, const float* lse, int dtype, std::string* err);

// Workspace sizes (-1 with *err set for invalid sizes).
int64_t split_workspace_bytes(int64_t B, int64_t H, int64_t S, int64_t D, int64_t n_split,
                              std::string* err);
int64_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t S, std::string* err);

// flash_attn_tile_shape.
int tile_shape(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int64_t window, int* block_q,
               int* block_k, std::string* err);

// flash_attn_bwd_kernel: writes the kernels' description to *name.
int bwd_kernel_name(int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t D, int dtype, int causal,
                    int64_t window, int alibi, std::string* name, std::string* err);

// flash_attn_fwd_kernel: writes the kernel's description to *name.
int fwd_kernel_name(int64_t B, int64_t H, int64_t S, int64_t D, int dtype, int alibi,
                    int64_t n_split, int64_t window, std::string* name, std::string* err);

}  // namespace fa
