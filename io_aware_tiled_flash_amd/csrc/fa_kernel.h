// Internal interface between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum { kDtypeF32 = 0, kDtypeF16 = 1, kDtypeBF16 = 2 };

// Arguments of one forward launch, already validated and normalised on the
// host: window >= S is folded to 0 (no window), n_sink is clamped to S, and a
// negative scale is folded into the sign of Q (neg = 1) so that c > 0.
// Query head bh (= b * H + h) reads key/value head bh / G.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  unsigned long long* block_pairs;  // optional instrumentation counter (may be null)
  const float* alibi;  // per-query-head ALiBi slopes [H], or null (no bias)
  float* o_part;       // key-split partial outputs [n_split][BH][S][D] fp32, or null
  float* lse_part;     // key-split partial LSE [n_split][BH][S] (with o_part)
  int n_split;         // key-block ranges per query block (1: no split)
  int S;        // sequence length
  int BH;       // batch * query heads
  int H;        // query heads
  int G;        // query heads per key/value head
  int nqb;      // query blocks per head = ceil(S / block_q of the chosen kernel)
  int causal;   // 0 / 1
  int window;   // 0 = none
  int n_sink;   // leading always-visible keys (only with window > 0)
  float c;      // |scale| * log2(e), at least FLT_MIN
  int neg;      // scale < 0
};

// Arguments of one backward launch (validated on the host). c = scale * log2(e)
// keeps the sign of scale here: the backward kernels use the logits directly.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;    // forward logsumexp [BH][S]
  void* dq;
  void* dk;
  void* dv;
  float* delta;        // workspace: rowsum(dO * O) [BH][Sp], 0 past S
  float* lse2;         // workspace: lse * log2(e) [BH][Sp], +inf past S
  const float* alibi;  // per-query-head slopes [H], or null
  int S, BH, H, G;     // G = query heads per key/value head
  int Sp;              // rows per head of the workspace arrays (S rounded up to the dq block)
  int nqb, nkb;        // query blocks of the dq kernel, key blocks of the dkv kernel
  int causal, window, n_sink;
  float c, scale;
};

// Backward kernels: bf16 / f16 with D in {64, 128}.
bool bwd_supported(int D, int dtype);
int bwd_tile_rows();
hipError_t launch_bwd(const BwdParams& p, int D, int dtype, hipStream_t st);

// Generic kernels: every dtype, D in {16, 32, 64, 128}.
int generic_tile_rows();
int generic_tile_keys();
hipError_t launch_generic(const FwdParams& p, int D, int dtype, hipStream_t st);

// Merge of key-split partials: o[r] = sum_s exp(lse_part[s][r] - lse[r]) o_part[s][r],
// lse[r] = log sum_s exp(lse_part[s][r]); rows = number of rows r; dtype of o.
hipError_t launch_merge(const float* o_part, const float* lse_part, int n_split, int64_t rows,
                        int D, void* o, float* lse, int dtype, hipStream_t st);

// Fast kernels: bf16 / f16 with D in {64, 128}; nw = waves per work-group (4 or 8).
bool fast_supported(int D, int dtype);
int fast_tile_keys();
hipError_t launch_fast(const FwdParams& p, int D, int dtype, int nw, hipStream_t st);

// Which kernel and tile a problem runs with (host-only, pure function of the shape).
struct Plan {
  bool fast;
  int nw;        // waves per work-group of the fast kernel
  int block_q;   // query rows per work-group
  int block_k;   // keys per streamed block
};
Plan plan_fwd(int64_t BH, int64_t S, int64_t D, int dtype);
hipError_t launch_plan(const Plan& plan, const FwdParams& p, int D, int dtype, hipStream_t st);

}  // namespace fa
