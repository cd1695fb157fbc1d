"""MI355X (gfx950) tiled online-softmax attention forward pass.

Thin Python binding over the C ABI in include/flash_attn.h (libflashattn.so,
built in-tree by `io_aware_tiled_flash_amd.build`). Python only marshals
arguments: torch supplies device memory and the current stream, every step of
the computation runs in the library's HIP kernels. There is no CPU fallback:
if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["flash_attn_fwd", "flash_attn_bwd", "flash_attn_bwd_noalloc", "flash_attn_fwd_counted",
           "flash_attn_fwd_split",
           "flash_attn_merge", "flash_attn_bwd_workspace_bytes",
           "flash_attn_split_workspace_bytes", "flash_attn_tile_shape", "flash_attn_fwd_kernel",
           "flash_attn_bwd_kernel",
           "flash_attn_last_error", "flash_attn_version", "capi", "library_path",
           "FA_F32", "FA_F16", "FA_BF16", "FA_OK", "FA_ERR_INVALID", "FA_ERR_UNSUPPORTED",
           "FA_ERR_HIP"]

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, -1, -2, -3

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashattn.so")


class _CAPI:
    """ctypes view of the exported symbols, with the C names and argument order."""

    def __init__(self, path: str):
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build the gfx950 library first "
                "(python -m io_aware_tiled_flash_amd.build); there is no fallback path")
        self.lib = ctypes.CDLL(path)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        fwd_args = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i64, i64, f32, vp, i32]
        self.flash_attn_fwd = self._fn("flash_attn_fwd", fwd_args, i32)
        self.flash_attn_fwd_counted = self._fn("flash_attn_fwd_counted", fwd_args + [vp], i32)
        self.flash_attn_fwd_ext = self._fn(
            "flash_attn_fwd_ext",
            [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i64, i64, f32, vp, vp, i32], i32)
        self.flash_attn_fwd_split = self._fn(
            "flash_attn_fwd_split",
            [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i64, i64, f32, vp, i64, vp, i64, vp,
             i32], i32)
        self.flash_attn_split_workspace_bytes = self._fn(
            "flash_attn_split_workspace_bytes", [i64, i64, i64, i64, i64], i64)
        self.flash_attn_merge = self._fn(
            "flash_attn_merge", [vp, vp, i64, i64, i64, vp, vp, vp, i32], i32)
        self.flash_attn_bwd = self._fn(
            "flash_attn_bwd",
            [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i64, i64, f32, vp,
             vp, i64, vp, i32], i32)
        self.flash_attn_bwd_noalloc = self._fn(
            "flash_attn_bwd_noalloc",
            [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i64, i64, f32, vp,
             vp, i32], i32)
        self.flash_attn_bwd_workspace_bytes = self._fn(
            "flash_attn_bwd_workspace_bytes", [i64, i64, i64], i64)
        self.flash_attn_tile_shape = self._fn(
            "flash_attn_tile_shape",
            [i64, i64, i64, i64, i32, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)], i32)
        self.flash_attn_fwd_kernel = self._fn(
            "flash_attn_fwd_kernel",
            [i64, i64, i64, i64, i32, i32, i64, i64, ctypes.c_char_p, i64], i32)
        self.flash_attn_bwd_kernel = self._fn(
            "flash_attn_bwd_kernel",
            [i64, i64, i64, i64, i64, i32, i32, i64, i32, ctypes.c_char_p, i64], i32)
        self.flash_attn_last_error = self._fn("flash_attn_last_error", [], ctypes.c_char_p)
        self.flash_attn_version = self._fn("flash_attn_version", [], ctypes.c_char_p)

    def _fn(self, name, argtypes, restype):
        f = getattr(self.lib, name)
        f.argtypes = argtypes
        f.restype = restype
        return f


_capi = None


def capi() -> _CAPI:
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _capi
    if _capi is None:
        _capi = _CAPI(library_path)
    return _capi


def flash_attn_last_error() -> str:
    return capi().flash_attn_last_error().decode()


def flash_attn_version() -> str:
    return capi().flash_attn_version().decode()


def flash_attn_tile_shape(B: int, H: int, S: int, D: int, dtype: int, *,
                          window: int = 0) -> tuple[int, int]:
    """(query rows per work-group, keys per streamed block) flash_attn_fwd uses
    for a [B, H, S, D] problem of this dtype and sliding window (0: none)."""
    bq, bk = ctypes.c_int(0), ctypes.c_int(0)
    rc = capi().flash_attn_tile_shape(B, H, S, D, dtype, window, ctypes.byref(bq),
                                      ctypes.byref(bk))
    _check(rc)
    return bq.value, bk.value


def flash_attn_fwd_kernel(B: int, H: int, S: int, D: int, dtype: int, *, alibi: bool = False,
                          n_split: int = 1, window: int = 0) -> str:
    """Description of the kernel a forward call would launch for this problem."""
    buf = ctypes.create_string_buffer(128)
    _check(capi().flash_attn_fwd_kernel(B, H, S, D, dtype, int(bool(alibi)), n_split, window,
                                        buf, 128))
    return buf.value.decode()


def flash_attn_bwd_kernel(B: int, H: int, S: int, D: int, dtype: int, *, H_kv: int | None = None,
                          causal: bool = False, window: int = 0, alibi: bool = False) -> str:
    """Description of the kernels a backward call would launch for this problem."""
    buf = ctypes.create_string_buffer(256)
    _check(capi().flash_attn_bwd_kernel(B, H, H if H_kv is None else H_kv, S, D, dtype,
                                        int(bool(causal)), window, int(bool(alibi)), buf, 256))
    return buf.value.decode()


def _check(rc: int):
    if rc == FA_OK:
        return
    msg = flash_attn_last_error()
    if rc == FA_ERR_INVALID:
        raise ValueError(msg)
    if rc == FA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(f"flash_attn error {rc}: {msg}")


def _check_device_tensor(name, t, device, dtype=None, shape=None):
    """t must be a contiguous torch tensor on `device` (and of dtype / shape
    when given): the library receives only its address, so nothing below
    this line could catch a host tensor or a short buffer."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}")


def _check_workspace(t, device, need: int):
    _check_device_tensor("workspace", t, device)
    if t.numel() * t.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes")


_codes = None
_raw_stream = None


def _dtype_code(t) -> int:
    global _codes
    if _codes is None:
        import torch
        _codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    code = _codes.get(t.dtype)
    if code is None:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return code


def _stream_handle(index: int) -> int:
    """Handle of torch's current stream on device `index` (the caller has
    made that device current). torch's raw-stream query returns the handle
    without building a Stream object; the public call is the fallback."""
    global _raw_stream
    if _raw_stream is None:
        import torch
        fn = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _raw_stream = fn if fn is not None else (
            lambda i: torch.cuda.current_stream(i).cuda_stream)
    return _raw_stream(index)


def _on_device(index: int, call):
    """Run call() with device `index` current (switching only when another
    device is current)."""
    import torch
    if torch.cuda.current_device() == index:
        return call()
    with torch.cuda.device(index):
        return call()


def _forward(q, k, v, causal, window, n_sink, scale, out, lse, block_pairs, alibi_slopes=None,
             n_split=None, workspace=None):
    import torch
    # (device checks compare get_device() indices: -1 for a host tensor)
    Tensor = torch.Tensor
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D torch tensor [B, H, S, D]")
        if t.get_device() < 0:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, H, S, D]")
    B, H, S, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H_kv, S, D] with q's B, S, D")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    dev = q.get_device()
    if k.get_device() != dev or v.get_device() != dev:
        raise ValueError("q, k, v must be on one device")
    if alibi_slopes is not None:
        if not isinstance(alibi_slopes, Tensor) or alibi_slopes.dtype != torch.float32 \
                or alibi_slopes.shape != (H,) or not alibi_slopes.is_contiguous() \
                or alibi_slopes.get_device() != dev:
            raise ValueError("alibi_slopes must be a contiguous float32 tensor [H] on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if lse is None else lse
    if not isinstance(o, Tensor) or o.shape != q.shape or o.dtype != q.dtype \
            or not o.is_contiguous() or o.get_device() != dev:
        raise ValueError("out must be a contiguous tensor like q")
    if not isinstance(l, Tensor) or l.shape != (B, H, S) or l.dtype != torch.float32 \
            or not l.is_contiguous() or l.get_device() != dev:
        raise ValueError("lse must be a contiguous float32 tensor [B, H, S] on q's device")
    code = _dtype_code(q)
    mask = (int(bool(causal)), int(window), int(n_sink), float(scale))
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr())
    slopes = None if alibi_slopes is None else alibi_slopes.data_ptr()
    lib = capi()
    if n_split is not None:
        need = lib.flash_attn_split_workspace_bytes(B, H, S, D, int(n_split))
        if need < 0:
            _check(FA_ERR_INVALID)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        elif workspace is not None:
            _check_workspace(workspace, q.device, need)
        ws_ptr = None if workspace is None else workspace.data_ptr()
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()

        def call():
            return lib.flash_attn_fwd_split(*ptrs, B, H, Hkv, S, D, *mask, slopes, int(n_split),
                                            ws_ptr, ws_bytes, _stream_handle(dev), code)
    elif Hkv != H or alibi_slopes is not None:
        if block_pairs is not None:
            raise ValueError("the block counter is available for plain multi-head calls only")

        def call():
            return lib.flash_attn_fwd_ext(*ptrs, B, H, Hkv, S, D, *mask, slopes,
                                          _stream_handle(dev), code)
    elif block_pairs is None:
        def call():
            return lib.flash_attn_fwd(*ptrs, B, H, S, D, *mask, _stream_handle(dev), code)
    else:
        if not isinstance(block_pairs, Tensor) or block_pairs.dtype not in (torch.int64, torch.uint64) \
                or block_pairs.numel() < 1 or block_pairs.get_device() != dev:
            raise ValueError("block_pairs must be an int64 tensor on q's device")

        def call():
            return lib.flash_attn_fwd_counted(*ptrs, B, H, S, D, *mask, _stream_handle(dev), code,
                                              block_pairs.data_ptr())
    _check(_on_device(dev, call))
    return o, l


def flash_attn_fwd(q, k, v, *, causal: bool = False, window: int = 0, n_sink: int = 0,
                   scale: float | None = None, alibi_slopes=None, out=None, lse=None):
    """Attention forward on the GPU: returns (o [B,H,S,D] in q's dtype, lse [B,H,S] fp32).

    q: contiguous GPU tensor [B, H, S, D]; k, v: [B, H_kv, S, D] with H_kv
    dividing H (query head h reads key/value head h // (H // H_kv); H_kv = 1 is
    multi-query attention); one dtype (float32, float16, bfloat16). scale
    defaults to 1/sqrt(D); window/n_sink need causal=True. alibi_slopes: an
    optional contiguous float32 GPU tensor [H]; the logit of (i, j) in head h
    then gains -alibi_slopes[h] * |i - j| (the Lesson 91 deck's slopes are
    2^(-8 (h + 1) / H)). Enqueued on torch's current stream; no
    synchronisation happens here.
    """
    return _forward(q, k, v, causal, window, n_sink, scale, out, lse, None, alibi_slopes)


def flash_attn_fwd_split(q, k, v, *, n_split: int, causal: bool = False, window: int = 0,
                         n_sink: int = 0, scale: float | None = None, alibi_slopes=None,
                         workspace=None, out=None, lse=None):
    """flash_attn_fwd with the keys of every query block split into n_split
    ranges (separate work-groups) whose partial results are then merged.
    workspace: optional GPU tensor of at least flash_attn_split_workspace_bytes
    bytes (allocated here through torch when None)."""
    return _forward(q, k, v, causal, window, n_sink, scale, out, lse, None, alibi_slopes,
                    n_split, workspace)


def flash_attn_split_workspace_bytes(B: int, H: int, S: int, D: int, n_split: int) -> int:
    n = capi().flash_attn_split_workspace_bytes(B, H, S, D, n_split)
    if n < 0:
        _check(FA_ERR_INVALID)
    return n


def flash_attn_merge(o_parts, lse_parts, *, dtype=None, out=None, lse=None):
    """Merge partial results: o_parts fp32 [n, ..., D], lse_parts fp32 [n, ...]
    (GPU, contiguous) -> (o [..., D] in dtype (default float32), lse [...])."""
    import torch
    if not (isinstance(o_parts, torch.Tensor) and isinstance(lse_parts, torch.Tensor)):
        raise ValueError("o_parts and lse_parts must be torch tensors")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise ValueError("partials must be float32")
    if not (o_parts.is_cuda and lse_parts.is_cuda and o_parts.is_contiguous()
            and lse_parts.is_contiguous()):
        raise ValueError("partials must be contiguous GPU tensors")
    if o_parts.dim() < 2 or o_parts.shape[:-1] != lse_parts.shape:
        raise ValueError("o_parts must be [n, ..., D] and lse_parts [n, ...]")
    if lse_parts.device != o_parts.device:
        raise ValueError("o_parts and lse_parts must be on one device")
    n, D = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts[0].numel()
    dev = o_parts.device
    dtype = torch.float32 if dtype is None else dtype
    o = torch.empty(o_parts.shape[1:], dtype=dtype, device=dev) if out is None else out
    l = torch.empty(lse_parts.shape[1:], dtype=torch.float32, device=dev) if lse is None else lse
    _check_device_tensor("out", o, dev, dtype=dtype, shape=o_parts.shape[1:])
    _check_device_tensor("lse", l, dev, dtype=torch.float32, shape=lse_parts.shape[1:])
    idx = o_parts.get_device()
    code = _dtype_code(o)
    _check(_on_device(idx, lambda: capi().flash_attn_merge(
        o_parts.data_ptr(), lse_parts.data_ptr(), n, rows, D, o.data_ptr(), l.data_ptr(),
        _stream_handle(idx), code)))
    return o, l


def flash_attn_bwd_workspace_bytes(B: int, H: int, S: int) -> int:
    n = capi().flash_attn_bwd_workspace_bytes(B, H, S)
    if n < 0:
        _check(FA_ERR_INVALID)
    return n


def _bwd_args(q, k, v, o, lse, dout, scale, alibi_slopes, dq, dk, dv):
    """Checks of the backward's tensors; returns (B, H, Hkv, S, D, scale, dq, dk, dv)."""
    import torch
    ts = {"q": q, "k": k, "v": v, "o": o, "dout": dout}
    for name, t in ts.items():
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or not t.is_cuda \
                or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D GPU tensor")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError("all tensors must share q's dtype and device")
    B, H, S, D = q.shape
    Hkv = k.shape[1]
    if o.shape != q.shape or dout.shape != q.shape or k.shape != (B, Hkv, S, D) \
            or v.shape != k.shape:
        raise ValueError("q, o, dout: [B, H, S, D]; k, v: [B, H_kv, S, D]")
    _check_device_tensor("lse", lse, q.device, dtype=torch.float32, shape=(B, H, S))
    if alibi_slopes is not None:
        _check_device_tensor("alibi_slopes", alibi_slopes, q.device, dtype=torch.float32,
                             shape=(H,))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_device_tensor(name, t, q.device, dtype=ref.dtype, shape=ref.shape)
    return B, H, Hkv, S, D, scale, dq, dk, dv


def flash_attn_bwd(q, k, v, o, lse, dout, *, causal: bool = False, window: int = 0,
                   n_sink: int = 0, scale: float | None = None, alibi_slopes=None,
                   workspace=None, dq=None, dk=None, dv=None):
    """Gradients (dq, dk, dv) of flash_attn_fwd on the GPU, recomputed from the
    forward's o and lse. q, o, dout: [B, H, S, D]; k, v: [B, H_kv, S, D]; lse:
    fp32 [B, H, S]; bf16 / f16 with D 64 or 128. workspace: optional GPU tensor
    of at least flash_attn_bwd_workspace_bytes(B, H, S) bytes."""
    import torch
    B, H, Hkv, S, D, scale, dq, dk, dv = _bwd_args(q, k, v, o, lse, dout, scale, alibi_slopes,
                                                   dq, dk, dv)
    need = flash_attn_bwd_workspace_bytes(B, H, S)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, q.device, need)
    idx = q.get_device()
    code = _dtype_code(q)
    _check(_on_device(idx, lambda: capi().flash_attn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, S, D,
        int(bool(causal)), int(window), int(n_sink), float(scale),
        None if alibi_slopes is None else alibi_slopes.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(idx), code)))
    return dq, dk, dv


def flash_attn_bwd_noalloc(q, k, v, o, lse, dout, *, causal: bool = False, window: int = 0,
                           n_sink: int = 0, scale: float | None = None, alibi_slopes=None,
                           dq=None, dk=None, dv=None):
    """flash_attn_bwd with its per-row state in the library's static device
    scratch instead of a workspace: the library call allocates nothing (pass
    dq, dk, dv to allocate nothing here either). Shapes whose state exceeds
    the scratch (B*H*S above about 4.19 million rows) raise NotImplementedError;
    calls that overlap in time on one GPU race on the scratch."""
    B, H, Hkv, S, D, scale, dq, dk, dv = _bwd_args(q, k, v, o, lse, dout, scale, alibi_slopes,
                                                   dq, dk, dv)
    idx = q.get_device()
    code = _dtype_code(q)
    _check(_on_device(idx, lambda: capi().flash_attn_bwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, S, D,
        int(bool(causal)), int(window), int(n_sink), float(scale),
        None if alibi_slopes is None else alibi_slopes.data_ptr(), _stream_handle(idx), code)))
    return dq, dk, dv


def flash_attn_fwd_counted(q, k, v, block_pairs, *, causal: bool = False, window: int = 0,
                           n_sink: int = 0, scale: float | None = None, out=None, lse=None):
    """flash_attn_fwd that also adds the number of (query-block, key-block) tile
    pairs the kernel computed to block_pairs[0] (a GPU int64 tensor)."""
    return _forward(q, k, v, causal, window, n_sink, scale, out, lse, block_pairs)
