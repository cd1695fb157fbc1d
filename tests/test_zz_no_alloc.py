"""The allocation-free backward (flash_attn_bwd_noalloc) against flash_attn_bwd.

Both run the same kernels; the allocation-free call keeps the per-row state in
the library's static device scratch instead of a caller workspace. Two calls
in a row through the C ABI, the second on a smaller input (so the second reads
nothing the first left behind), each compared with flash_attn_bwd on the same
inputs: the gradients must be bitwise equal, and within the backward's
normwise tolerance of the fp64 oracle.
"""
from __future__ import annotations

import ctypes
import math
import sys

import numpy as np
import pytest
import torch

import fa_inputs
import io_aware_tiled_flash_amd as fa
from oracle import attention as ORACLE

pytestmark = pytest.mark.gpu

TOL_GRAD = {"bf16": 2.5e-2, "f16": 4e-3}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bwd_pair(B, H, H_kv, S, D, dtype, seed, causal, window, n_sink):
    q, k, v = fa_inputs.make_qkv(B, H, S, D, dtype, seed=seed, H_kv=H_kv)
    dout = fa_inputs.make_qkv(B, H, S, D, dtype, seed=seed + 1)[0]
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, dout))
    scale = 1.0 / math.sqrt(D)
    o, lse = fa.flash_attn_fwd(qd, kd, vd, causal=causal, window=window, n_sink=n_sink,
                               scale=scale)
    ref = fa.flash_attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, window=window,
                            n_sink=n_sink, scale=scale)
    # the allocation-free call straight through the C ABI, into outputs
    # filled with NaN beforehand (every element must be written)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (qd, kd, vd))
    torch.cuda.synchronize()
    code = {"bf16": fa.FA_BF16, "f16": fa.FA_F16}[dtype]
    stream = torch.cuda.current_stream().cuda_stream
    rc = fa.capi().flash_attn_bwd_noalloc(
        qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), dod.data_ptr(),
        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, H_kv, S, D,
        int(causal), window, n_sink, ctypes.c_float(scale), None, ctypes.c_void_p(stream), code)
    assert rc == fa.FA_OK, fa.flash_attn_last_error()
    torch.cuda.synchronize()
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        assert torch.equal(got, want), name
    g = ORACLE.attention_bwd(fa_inputs.to_f64(q), fa_inputs.to_f64(k), fa_inputs.to_f64(v),
                             fa_inputs.to_f64(dout), causal=causal, scale=scale, window=window,
                             n_sink=n_sink)
    errs = [float(np.abs(t.float().cpu().double().numpy() - r).max() / max(1.0, np.abs(r).max()))
            for t, r in zip((dq, dk, dv), g)]
    _say(f"  noalloc B{B} H{H}/{H_kv} S{S} D{D} {dtype}: bitwise equal to flash_attn_bwd; "
         f"normwise vs oracle {errs}")
    assert max(errs) <= TOL_GRAD[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_bwd_noalloc_matches_workspace_call(dtype):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _bwd_pair(2, 4, 2, 700, 128, dtype, seed=31, causal=True, window=0, n_sink=0)
    _bwd_pair(1, 2, 2, 300, 64, dtype, seed=32, causal=True, window=120, n_sink=2)


def test_bwd_noalloc_rejects_oversized_shape():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # B*H*S past the 32 MiB scratch (4,194,304 padded rows): rejected before
    # anything is launched, with tensors that are never touched
    H = (32 << 20) // 8 // 4096 + 1
    q = torch.empty((1, 1, 4096, 128), dtype=torch.bfloat16, device="cuda")
    rc = fa.capi().flash_attn_bwd_noalloc(
        q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
        1 << 44, 2 << 44, 3 << 44, 1, H, H, 4096, 128, 1, 0, 0, ctypes.c_float(0.1), None, None,
        fa.FA_BF16)
    assert rc == fa.FA_ERR_UNSUPPORTED, fa.flash_attn_last_error()
