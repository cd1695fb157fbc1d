"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects every invalid argument before touching the GPU.

No call here reaches a kernel launch: each one fails host-side validation
(pointers are fake but never dereferenced), so the suite runs without a GPU.
"""
from __future__ import annotations

import ctypes
import pathlib
import re
import subprocess

import pytest

import io_aware_tiled_flash_amd as fa

ROOT = pathlib.Path(__file__).resolve().parents[1]
HEADERS = sorted((ROOT / "include").glob("*.h"))

# fake but aligned, disjoint "device" addresses; validation never dereferences them
Q, K, V, O, L = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", h.read_text(), flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\**\s*(flash_attn_\w+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


def test_headers_declare_the_abi():
    names = _declared_functions()
    assert {"flash_attn_fwd", "flash_attn_fwd_ext", "flash_attn_fwd_split", "flash_attn_bwd",
            "flash_attn_bwd_workspace_bytes",
            "flash_attn_split_workspace_bytes", "flash_attn_merge", "flash_attn_fwd_counted",
            "flash_attn_tile_shape", "flash_attn_last_error", "flash_attn_version"} <= names


def test_library_exports_every_declared_symbol():
    assert pathlib.Path(fa.library_path).exists(), "build the library first"
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = _declared_functions() - exported
    assert not missing, missing
    lib = ctypes.CDLL(fa.library_path)
    for name in _declared_functions():
        getattr(lib, name)


def test_version_and_tile_shape():
    assert "gfx950" in fa.flash_attn_version()
    for D in (16, 32, 64, 128):
        for dt in (fa.FA_F32, fa.FA_F16, fa.FA_BF16):
            bq, bk = fa.flash_attn_tile_shape(1, 1, 4096, D, dt)
            assert bq >= 32 and bk >= 32 and bq % 32 == 0 and bk % 32 == 0
    with pytest.raises(NotImplementedError):
        fa.flash_attn_tile_shape(1, 1, 64, 48, fa.FA_BF16)
    with pytest.raises(ValueError):
        fa.flash_attn_tile_shape(1, 1, 64, 64, 7)


def test_small_grid_tile_choice(monkeypatch):
    """The plan behind flash_attn_tile_shape: a D = 64 grid of at most 128
    work-groups of 128 rows (half the CUs) takes four key parts on 64-row
    blocks; other grids of fewer than 512 keep 128-row blocks (two parts, or
    8 waves at S >= 16384); D = 128 without a window takes 8 waves from
    S = 2048 once there are 512 such work-groups; FLASH_ATTN_PARTS=0|2|4
    overrides."""
    monkeypatch.delenv("FLASH_ATTN_PARTS", raising=False)
    monkeypatch.delenv("FLASH_ATTN_WAVES", raising=False)
    for dt in (fa.FA_F16, fa.FA_BF16):
        assert fa.flash_attn_tile_shape(2, 8, 1024, 64, dt) == (64, 64)       # 128 work-groups
        assert fa.flash_attn_tile_shape(1, 1, 1, 64, dt) == (64, 64)
        assert fa.flash_attn_tile_shape(1, 16, 2048, 64, dt) == (128, 64)    # 256: two parts
        assert fa.flash_attn_tile_shape(1, 32, 2048, 64, dt) == (128, 64)    # 512: 4 waves
        assert fa.flash_attn_tile_shape(2, 8, 1024, 128, dt) == (128, 64)    # D = 128: two parts
        assert fa.flash_attn_tile_shape(4, 16, 4096, 128, dt) == (256, 64)  # 8 waves
        assert fa.flash_attn_tile_shape(4, 16, 4096, 128, dt, window=1024) == (128, 64)
        assert fa.flash_attn_tile_shape(4, 16, 4096, 128, dt, window=4096) == (256, 64)
        assert fa.flash_attn_tile_shape(4, 16, 4096, 64, dt) == (128, 64)    # D = 64: 4 waves
        assert fa.flash_attn_tile_shape(16, 16, 1024, 128, dt) == (128, 64)  # S < 2048
        assert fa.flash_attn_tile_shape(1, 16, 4096, 128, dt) == (128, 64)  # 256 groups of 8
        assert fa.flash_attn_tile_shape(1, 32, 16384, 128, dt) == (256, 64)  # 8 waves
        assert fa.flash_attn_tile_shape(1, 32, 16384, 64, dt) == (256, 64)
    c2 = fa.flash_attn_fwd_kernel(2, 8, 1024, 64, fa.FA_F16)
    assert c2 == "fa_fwd_parts_kernel<f16,D=64,parts=4> (8 waves, 64x64 tile)", c2
    assert "parts=2" in fa.flash_attn_fwd_kernel(2, 8, 1024, 128, fa.FA_BF16)
    assert "waves=8" in fa.flash_attn_fwd_kernel(4, 16, 4096, 128, fa.FA_BF16)
    assert "waves=8" in fa.flash_attn_fwd_kernel(4, 16, 4096, 128, fa.FA_BF16, alibi=True)
    assert "waves=4" in fa.flash_attn_fwd_kernel(4, 16, 4096, 128, fa.FA_BF16, window=1024)
    assert "waves=8" in fa.flash_attn_fwd_kernel(1, 32, 16384, 128, fa.FA_BF16)
    # ALiBi and key splits never take the small-grid schedule
    assert "fast_kernel" in fa.flash_attn_fwd_kernel(2, 8, 1024, 64, fa.FA_F16, alibi=True)
    assert fa.flash_attn_fwd_kernel(2, 8, 1024, 64, fa.FA_F16, n_split=4).endswith("fa_merge_kernel")
    assert fa.flash_attn_fwd_kernel(1, 1, 64, 16, fa.FA_F32).startswith("fa_fwd_f32_kernel<D=16>")
    with pytest.raises(NotImplementedError):
        fa.flash_attn_fwd_kernel(1, 1, 64, 48, fa.FA_BF16)
    with pytest.raises(NotImplementedError):
        fa.flash_attn_fwd_kernel(1, 1, 64, 32, fa.FA_BF16, n_split=2)
    with pytest.raises(ValueError):
        fa.flash_attn_fwd_kernel(1, 1, 64, 64, fa.FA_BF16, n_split=0)
    with pytest.raises(ValueError):
        fa.flash_attn_fwd_kernel(1, 1, 64, 64, fa.FA_BF16, window=-1)
    with pytest.raises(ValueError):
        fa.flash_attn_tile_shape(1, 1, 64, 64, fa.FA_BF16, window=-1)
    buf = ctypes.create_string_buffer(8)   # truncated to fit, NUL-terminated
    assert fa.capi().flash_attn_fwd_kernel(2, 8, 1024, 64, fa.FA_F16, 0, 1, 0, buf, 8) == fa.FA_OK
    assert buf.value == b"fa_fwd_"
    monkeypatch.setenv("FLASH_ATTN_PARTS", "0")
    assert fa.flash_attn_tile_shape(2, 8, 1024, 64, fa.FA_F16) == (128, 64)
    assert "waves=4" in fa.flash_attn_fwd_kernel(2, 8, 1024, 64, fa.FA_F16)
    monkeypatch.setenv("FLASH_ATTN_PARTS", "4")
    assert fa.flash_attn_tile_shape(1, 32, 2048, 64, fa.FA_F16) == (64, 64)
    assert fa.flash_attn_tile_shape(2, 8, 1024, 128, fa.FA_F16) == (128, 64)
    assert fa.flash_attn_tile_shape(1, 1, 1024, 64, fa.FA_F32)[0] == 128   # generic kernel


def _call(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, S=64, D=64, causal=0, window=0, n_sink=0,
          scale=0.125, stream=None, dtype=fa.FA_BF16, counter=None):
    c = fa.capi()
    args = (q, k, v, o, lse, B, H, S, D, causal, window, n_sink, scale, stream, dtype)
    if counter is None:
        rc = c.flash_attn_fwd(*args)
    else:
        rc = c.flash_attn_fwd_counted(*args, counter)
    return rc, fa.flash_attn_last_error()


INVALID = {
    "null_q": dict(q=None),
    "null_k": dict(k=None),
    "null_v": dict(v=None),
    "null_o": dict(o=None),
    "null_lse": dict(lse=None),
    "B0": dict(B=0),
    "H0": dict(H=0),
    "S0": dict(S=0),
    "S_negative": dict(S=-5),
    "D0": dict(D=0),
    "causal_2": dict(causal=2),
    "causal_negative": dict(causal=-1),
    "window_negative": dict(causal=1, window=-1),
    "window_without_causal": dict(causal=0, window=16),
    "n_sink_negative": dict(causal=1, window=16, n_sink=-1),
    "scale_nan": dict(scale=float("nan")),
    "scale_inf": dict(scale=float("inf")),
    "scale_neg_inf": dict(scale=float("-inf")),
    "dtype_unknown": dict(dtype=3),
    "dtype_negative": dict(dtype=-1),
    "q_misaligned": dict(q=Q + 8),
    "k_misaligned": dict(k=K + 2),
    "v_misaligned": dict(v=V + 4),
    "o_misaligned": dict(o=O + 8),
    "lse_misaligned": dict(lse=L + 2),
    "o_overlaps_q": dict(o=Q + 64),
    "o_overlaps_v": dict(o=V - 64),
    "lse_overlaps_o": dict(lse=O + 128),
    "lse_overlaps_q": dict(lse=Q + 256),
    "lse_overlaps_k": dict(lse=K),
    "size_overflow": dict(B=1 << 40, H=1 << 20, S=1 << 10),
    "counter_misaligned": dict(counter=0x600004),
}


@pytest.mark.parametrize("case", sorted(INVALID))
def test_invalid_arguments_rejected(case):
    rc, msg = _call(**INVALID[case])
    assert rc == fa.FA_ERR_INVALID, (case, rc, msg)
    assert msg


def _call_ext(q=Q, k=K, v=V, o=O, lse=L, B=1, H=4, H_kv=2, S=64, D=64, causal=1, window=0,
              n_sink=0, scale=0.125, alibi=None, stream=None, dtype=fa.FA_BF16):
    rc = fa.capi().flash_attn_fwd_ext(q, k, v, o, lse, B, H, H_kv, S, D, causal, window, n_sink,
                                      scale, alibi, stream, dtype)
    return rc, fa.flash_attn_last_error()


INVALID_EXT = {
    "kv_heads_zero": dict(H_kv=0),
    "kv_heads_negative": dict(H_kv=-2),
    "kv_heads_not_dividing": dict(H=6, H_kv=4),
    "kv_heads_above_heads": dict(H=2, H_kv=4),
    "alibi_misaligned": dict(alibi=0x600002),
    "alibi_overlaps_o": dict(alibi=O + 64),
    "alibi_overlaps_lse": dict(alibi=L),
    "null_k_ext": dict(k=None),
    "window_without_causal_ext": dict(causal=0, window=8),
}


@pytest.mark.parametrize("case", sorted(INVALID_EXT))
def test_invalid_ext_arguments_rejected(case):
    rc, msg = _call_ext(**INVALID_EXT[case])
    assert rc == fa.FA_ERR_INVALID, (case, rc, msg)
    assert msg


def test_ext_unsupported_head_dim():
    rc, msg = _call_ext(D=96)
    assert rc == fa.FA_ERR_UNSUPPORTED and "head dim" in msg


@pytest.mark.parametrize("D", [8, 48, 96, 256, 512])
def test_unsupported_head_dim(D):
    rc, msg = _call(D=D)
    assert rc == fa.FA_ERR_UNSUPPORTED and "head dim" in msg


def test_index_range_limit():
    rc, msg = _call(S=1 << 31, D=64, o=1 << 44, lse=1 << 46, v=1 << 42, k=1 << 41, q=1 << 40)
    assert rc == fa.FA_ERR_UNSUPPORTED, msg


def test_error_text_clears_on_success_path_queries():
    _call(q=None)
    assert fa.flash_attn_last_error()
    fa.flash_attn_tile_shape(1, 1, 64, 64, fa.FA_F16)
    assert fa.flash_attn_last_error() == ""


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 16)
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(x, x, x)


# --------------------------------------------------------------------------- #
# Key splitting and the merge
# --------------------------------------------------------------------------- #

WS = 0x10000000   # fake workspace address, far from the tensors


def _call_split(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, H_kv=2, S=64, D=64, causal=1, window=0,
                n_sink=0, scale=0.125, alibi=None, n_split=2, ws=WS, ws_bytes=1 << 30,
                stream=None, dtype=fa.FA_BF16):
    rc = fa.capi().flash_attn_fwd_split(q, k, v, o, lse, B, H, H_kv, S, D, causal, window,
                                        n_sink, scale, alibi, n_split, ws, ws_bytes, stream,
                                        dtype)
    return rc, fa.flash_attn_last_error()


INVALID_SPLIT = {
    "n_split_zero": dict(n_split=0),
    "n_split_too_large": dict(n_split=257),
    "null_workspace": dict(ws=None),
    "workspace_misaligned": dict(ws=WS + 8),
    "workspace_too_small": dict(ws_bytes=1024),
    "workspace_overlaps_o": dict(ws=O),
    "workspace_overlaps_q": dict(ws=Q - 4096),
}


@pytest.mark.parametrize("case", sorted(INVALID_SPLIT))
def test_invalid_split_arguments_rejected(case):
    rc, msg = _call_split(**INVALID_SPLIT[case])
    assert rc == fa.FA_ERR_INVALID, (case, rc, msg)
    assert msg


def test_split_needs_fast_path():
    for kw in (dict(dtype=fa.FA_F32), dict(D=16), dict(D=32)):
        rc, msg = _call_split(**kw)
        assert rc == fa.FA_ERR_UNSUPPORTED, (kw, msg)


def test_split_workspace_bytes():
    c = fa.capi()
    rows, D = 2 * 8 * 1024, 64
    n = c.flash_attn_split_workspace_bytes(2, 8, 1024, 64, 4)
    o_bytes = 4 * rows * D * 4
    assert n == (o_bytes + 255) // 256 * 256 + 4 * rows * 4
    assert c.flash_attn_split_workspace_bytes(2, 8, 1024, 64, 1) == 0
    assert c.flash_attn_split_workspace_bytes(2, 8, 1024, 64, 0) == -1
    assert fa.flash_attn_last_error()
    assert c.flash_attn_split_workspace_bytes(1 << 40, 1 << 20, 1 << 10, 64, 2) == -1


def _call_merge(op=WS, lp=WS + (1 << 26), n=3, rows=100, D=64, o=O, lse=L, dtype=fa.FA_BF16):
    rc = fa.capi().flash_attn_merge(op, lp, n, rows, D, o, lse, None, dtype)
    return rc, fa.flash_attn_last_error()


INVALID_MERGE = {
    "null_parts": dict(op=None),
    "null_lse": dict(lse=None),
    "n_zero": dict(n=0),
    "rows_zero": dict(rows=0),
    "parts_misaligned": dict(op=WS + 4),
    "o_misaligned": dict(o=O + 8),
    "lse_misaligned": dict(lse=L + 2),
    "o_overlaps_parts": dict(o=WS + 64),
    "lse_overlaps_o": dict(lse=O + 16),
    "dtype_unknown": dict(dtype=9),
}


@pytest.mark.parametrize("case", sorted(INVALID_MERGE))
def test_invalid_merge_arguments_rejected(case):
    rc, msg = _call_merge(**INVALID_MERGE[case])
    assert rc == fa.FA_ERR_INVALID, (case, rc, msg)


def test_merge_unsupported_head_dim():
    rc, msg = _call_merge(D=48)
    assert rc == fa.FA_ERR_UNSUPPORTED


# --------------------------------------------------------------------------- #
# Backward
# --------------------------------------------------------------------------- #

DO, DQ, DK, DV, BWS = 0x700000, 0x800000, 0x900000, 0xA00000, 0xB00000


def _call_bwd(q=Q, k=K, v=V, o=O, dout=DO, lse=L, dq=DQ, dk=DK, dv=DV, B=1, H=2, H_kv=2, S=64,
              D=64, causal=1, window=0, n_sink=0, scale=0.125, alibi=None, ws=BWS,
              ws_bytes=1 << 20, dtype=fa.FA_BF16):
    rc = fa.capi().flash_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, S, D, causal,
                                  window, n_sink, scale, alibi, ws, ws_bytes, None, dtype)
    return rc, fa.flash_attn_last_error()


INVALID_BWD = {
    "null_dout": dict(dout=None),
    "null_dk": dict(dk=None),
    "null_workspace": dict(ws=None),
    "workspace_small": dict(ws_bytes=16),
    "dq_misaligned": dict(dq=DQ + 8),
    "dk_overlaps_q": dict(dk=Q + 1024),
    "dv_overlaps_dk": dict(dv=DK + 64),
    "workspace_overlaps_dq": dict(ws=DQ),
    "kv_heads_not_dividing": dict(H=3, H_kv=2),
    "window_without_causal": dict(causal=0, window=4),
    "scale_nan": dict(scale=float("nan")),
    "dtype_unknown": dict(dtype=5),
}


@pytest.mark.parametrize("case", sorted(INVALID_BWD))
def test_invalid_bwd_arguments_rejected(case):
    rc, msg = _call_bwd(**INVALID_BWD[case])
    assert rc == fa.FA_ERR_INVALID, (case, rc, msg)
    assert msg


def test_bwd_unsupported_types():
    for kw in (dict(dtype=fa.FA_F32), dict(D=32), dict(D=96)):
        rc, msg = _call_bwd(**kw)
        assert rc == fa.FA_ERR_UNSUPPORTED, (kw, msg)


def test_bwd_workspace_bytes():
    # two fp32 arrays of B*H rows, each padded to a multiple of 128 per head
    assert fa.capi().flash_attn_bwd_workspace_bytes(2, 3, 100) == 2 * 2 * 3 * 128 * 4
    assert fa.capi().flash_attn_bwd_workspace_bytes(1, 1, 129) == (2 * 256 * 4 + 255) // 256 * 256
    assert fa.capi().flash_attn_bwd_workspace_bytes(0, 3, 100) == -1


# --------------------------------------------------------------------------- #
# Allocation-free backward: same validation, then the size limit of the
# library's scratch (all of this fails before any HIP call)
# --------------------------------------------------------------------------- #

def _call_bwd_noalloc(q=Q, k=K, v=V, o=O, dout=DO, lse=L, dq=DQ, dk=DK, dv=DV, B=1, H=2, H_kv=2,
                      S=64, D=64, causal=1, window=0, n_sink=0, scale=0.125, alibi=None,
                      dtype=fa.FA_BF16):
    rc = fa.capi().flash_attn_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, S, D,
                                          causal, window, n_sink, scale, alibi, None, dtype)
    return rc, fa.flash_attn_last_error()


INVALID_BWD_NOALLOC = {k: v for k, v in INVALID_BWD.items()
                       if k not in ("null_workspace", "workspace_small", "workspace_overlaps_dq")}


@pytest.mark.parametrize("case", sorted(INVALID_BWD_NOALLOC))
def test_invalid_bwd_noalloc_arguments_rejected(case):
    rc, msg = _call_bwd_noalloc(**INVALID_BWD_NOALLOC[case])
    assert rc == fa.FA_ERR_INVALID, (case, rc, msg)
    assert msg


def test_bwd_noalloc_size_limit():
    """The scratch holds 32 MiB: 8 bytes per padded row of B*H*S. One row past
    it is rejected with a message naming the way out (a caller workspace);
    tensors are placed far apart so that only the limit is in question."""
    far = 1 << 40
    ptrs = dict(q=1 * far, k=2 * far, v=3 * far, o=4 * far, dout=5 * far, lse=6 * far,
                dq=7 * far, dk=8 * far, dv=9 * far)
    rows_max = (32 << 20) // 8            # 4,194,304 padded rows
    H = rows_max // 4096 + 1              # B*H*4096 rows, one head too many
    rc, msg = _call_bwd_noalloc(**ptrs, B=1, H=H, H_kv=H, S=4096, D=128)
    assert rc == fa.FA_ERR_UNSUPPORTED and "flash_attn_bwd" in msg, (rc, msg)
    assert fa.capi().flash_attn_bwd_workspace_bytes(1, H, 4096) > (32 << 20)
    assert fa.capi().flash_attn_bwd_workspace_bytes(1, H - 1, 4096) <= (32 << 20)


def test_bwd_noalloc_unsupported_types():
    for kw in (dict(dtype=fa.FA_F32), dict(D=32)):
        rc, msg = _call_bwd_noalloc(**kw)
        assert rc == fa.FA_ERR_UNSUPPORTED, (kw, msg)


def test_backward_kernel_choice(monkeypatch):
    """The dK/dV kernel of a backward: two 4-wave work-groups per CU on grids
    of at least 1024 work-groups of 128 keys (512 without the causal mask or
    with a window); else one per CU. FLASH_ATTN_DKV=1|2 overrides."""
    monkeypatch.delenv("FLASH_ATTN_DKV", raising=False)
    bk = fa.flash_attn_bwd_kernel
    head = bk(4, 16, 4096, 128, fa.FA_BF16, causal=True)
    assert head.startswith("fa_bwd_dq_kernel<bf16,D=128>") and "fa_bwd_dkv2_kernel" in head, head
    assert "dkv2" in bk(2, 16, 2048, 128, fa.FA_BF16, causal=False)          # 512, no mask
    assert "dkv2" not in bk(1, 16, 4096, 128, fa.FA_BF16, causal=True)       # 512, causal
    assert "dkv2" not in bk(4, 16, 4096, 128, fa.FA_BF16, H_kv=2, causal=True)   # 256
    al = bk(4, 16, 4096, 128, fa.FA_BF16, causal=True, alibi=True)
    assert "fa_bwd_dq_kernel<bf16,D=128,alibi>" in al and "fa_bwd_dkv2_kernel<bf16,D=128,alibi>" in al, al
    assert "dkv2" not in bk(1, 16, 4096, 128, fa.FA_BF16, causal=True, alibi=True)   # 512
    assert "dkv2" in bk(2, 16, 8192, 128, fa.FA_BF16, causal=True, window=1024)    # 2048
    assert "dkv2" in bk(1, 8, 8192, 128, fa.FA_BF16, causal=True, window=4096)     # 512
    assert "dkv2" not in bk(1, 4, 8192, 128, fa.FA_BF16, causal=True, window=1024)  # 256
    assert "dkv2" not in bk(1, 8, 8192, 128, fa.FA_BF16, causal=True, window=8192)  # no-op window
    monkeypatch.setenv("FLASH_ATTN_DKV", "2")
    assert "dkv2" in bk(1, 1, 64, 64, fa.FA_F16, causal=True)
    monkeypatch.setenv("FLASH_ATTN_DKV", "1")
    assert "dkv2" not in bk(4, 16, 4096, 128, fa.FA_BF16, causal=True)
    with pytest.raises(NotImplementedError):
        bk(1, 1, 64, 32, fa.FA_BF16)
    with pytest.raises(NotImplementedError):
        bk(1, 1, 64, 64, fa.FA_F32)
    with pytest.raises(ValueError):
        bk(1, 3, 64, 64, fa.FA_BF16, H_kv=2)
