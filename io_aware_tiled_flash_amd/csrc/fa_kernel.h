// Internal interface between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum { kDtypeF32 = 0, kDtypeF16 = 1, kDtypeBF16 = 2 };

// Arguments of one forward launch, already validated and normalised on the
// host: window >= S is folded to 0 (no window), n_sink is clamped to S, and a
// negative scale is folded into the sign of Q (neg = 1) so that c > 0.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  unsigned long long* block_pairs;  // optional instrumentation counter (may be null)
  int S;        // sequence length
  int BH;       // batch * heads
  int nqb;      // query blocks per head = ceil(S / tile_rows())
  int causal;   // 0 / 1
  int window;   // 0 = none
  int n_sink;   // leading always-visible keys (only with window > 0)
  float c;      // |scale| * log2(e), at least FLT_MIN
  int neg;      // scale < 0
};

int tile_rows();   // query rows per work-group
int tile_keys();   // keys per streamed block

// Enqueues the kernel for (D, dtype) on `st`; returns the launch status.
hipError_t launch_fwd(const FwdParams& p, int D, int dtype, hipStream_t st);

}  // namespace fa
