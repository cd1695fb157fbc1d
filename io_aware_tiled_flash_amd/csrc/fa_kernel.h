// Internal interface between the C-ABI layer and the gfx950 kernels: the
// launch functions. The parameter blocks, tile sizes and plan they use are in
// fa_shapes.h (host-only C++).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_shapes.h"

namespace fa {

// Backward kernels: bf16 / f16 with D in {64, 128}.
hipError_t launch_bwd(const BwdParams& p, int D, int dtype, hipStream_t st);
// Device address of the allocation-free backward's scratch array on the
// current device (kBwdScratchBytes bytes; looked up once per device).
hipError_t bwd_scratch(void** out);

// Generic forward kernels: every dtype, D in {16, 32, 64, 128}.
hipError_t launch_generic(const FwdParams& p, int D, int dtype, hipStream_t st);

// Merge of key-split partials: o[r] = sum_s exp(lse_part[s][r] - lse[r]) o_part[s][r],
// lse[r] = log sum_s exp(lse_part[s][r]); rows = number of rows r; dtype of o.
hipError_t launch_merge(const float* o_part, const float* lse_part, int n_split, int64_t rows,
                        int D, void* o, float* lse, int dtype, hipStream_t st);

// Fast forward kernels: bf16 / f16 with D in {64, 128}; nw = waves per work-group (4 or 8).
hipError_t launch_fast(const FwdParams& p, int D, int dtype, int nw, hipStream_t st);

inline hipError_t launch_plan(const Plan& plan, const FwdParams& p, int D, int dtype,
                              hipStream_t st) {
  if (plan.fast) return launch_fast(p, D, dtype, plan.nw, st);
  return launch_generic(p, D, dtype, st);
}

}  // namespace fa
