"""Blockwise-scaled FP8 GEMM for AMD MI355X (gfx950): Python binding of libbfp8.so.

Thin layer over the C ABI in include/bfp8.h: it allocates outputs with torch on
the current device and stream, passes pointers, sizes and the stream handle,
and maps status codes to exceptions (ValueError for invalid or misaligned
arguments, NotImplementedError for unsupported requests, RuntimeError for device
and launch failures). Every step of the computation runs in the HIP kernels;
there is no fallback path.

    q, s = quant_act(x)                 # x: [M, K] fp32 or bf16 (cuda)
    c = gemm(q, s, w_q, w_s)            # c: [M, N] bf16
    c = grouped_gemm_contiguous(q, s, w_q, w_s, layout)
    y = linear(x_bf16, w_q, w_s, bias)  # quantize + GEMM (+ bias), bf16 out
"""

from __future__ import annotations

import ctypes

import torch

from . import _native
from ._native import SCHEDULES, LibraryMissing  # noqa: F401

__all__ = [
    "quant_act", "gemm", "gemm_f16", "grouped_gemm_contiguous", "grouped_gemm_gathered", "linear", "linear_workspace_bytes", "linear_fuses",
    "quant_act_1x64", "gemm_1x64",
    "quant_act_ue8m0", "gemm_ue8m0", "grouped_gemm_contiguous_ue8m0", "ue8m0_scales",
    "moe_padded_rows", "moe_dispatch", "quant_act_gather", "quant_act_scatter", "swiglu_quant", "swiglu", "moe_combine", "moe_forward",
    "moe_forward_workspace_bytes", "nn_to_nt_weights", "pad_k", "expand_act_scales", "expand_weight_scale", "set_schedule", "get_schedule", "schedule_for",
    "abi_version", "BfpError", "LibraryMissing",
]


class BfpError(RuntimeError):
    pass


def _raise(status: int, what: str):
    lib = _native.lib()
    msg = lib.bfp8_last_error_message().decode()
    name = lib.bfp8_status_string(status).decode()
    text = f"{what}: {name}: {msg}"
    if status in (_native.BFP8_ERR_INVALID_ARGUMENT, _native.BFP8_ERR_MISALIGNED, _native.BFP8_ERR_WORKSPACE):
        raise ValueError(text)
    if status == _native.BFP8_ERR_UNSUPPORTED:
        raise NotImplementedError(text)
    raise BfpError(text)


def _check(status: int, what: str):
    if status != _native.BFP8_OK:
        _raise(status, what)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _require(t: torch.Tensor, name: str, dtype, dims: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dims:
        raise ValueError(f"{name} must be {dims}-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")


def _as_u8(t: torch.Tensor, name: str) -> torch.Tensor:
    """FP8 codes may be passed as uint8 or float8_e4m3fn (same bytes)."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    return t


_workspaces: dict = {}


def _workspace(device: torch.device, nbytes: int) -> tuple[int, int]:
    """(pointer, size) of a workspace for the current stream, grown on demand.

    Its contents do not persist between calls (the linear layer's quantized activations are
    written and read within one call), so one buffer per (device, stream) serves every call
    ordered on that stream."""
    if nbytes == 0:
        return 0, 0
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf.data_ptr(), buf.numel()


_IN_DTYPES = {torch.float32: _native.BFP8_IN_F32, torch.bfloat16: _native.BFP8_IN_BF16,
              torch.float16: _native.BFP8_IN_F16}


def _in_dtype(x: torch.Tensor, what: str) -> int:
    if x.dtype not in _IN_DTYPES:
        raise NotImplementedError(f"{what} takes float32, bfloat16 or float16 input, got {x.dtype}")
    return _IN_DTYPES[x.dtype]


def abi_version() -> int:
    return _native.lib().bfp8_abi_version()


def quant_act(x: torch.Tensor, q: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Per-token-group FP8 quantization of x [M, K] (fp32, bf16 or fp16; K a multiple of 16; row
    stride may exceed K).

    Returns (q, s): q uint8 e4m3fn codes [M, K], a view of rows padded to ceil(K/128) * 128 bytes
    (the GEMMs read whole 128-byte blocks; the padding is never written); s float32
    [M, ceil(K/128)], stored group-major (s.stride() == (1, M)), i.e. the "column-major"
    activation scales the GEMM reads.
    """
    dt = _in_dtype(x, "quant_act")
    _require(x, "x", x.dtype, 2)
    if x.stride(1) != 1:
        raise ValueError("x must be K-contiguous")
    m, k = x.shape
    if q is None:  # rows of whole 128-byte blocks, as the GEMMs read them
        q = torch.empty((m, -(-k // 128) * 128), dtype=torch.uint8, device=x.device)[:, :k]
    if scales is None:
        scales = torch.empty((-(-k // 128), m), dtype=torch.float32, device=x.device).t()
    _require(q, "q", torch.uint8, 2)
    _require(scales, "scales", torch.float32, 2)
    if q.stride(1) != 1 or scales.stride(0) != 1:
        raise ValueError("q must be K-contiguous and scales group-major (stride(0) == 1)")
    st = _native.lib().bfp8_quant_act(x.data_ptr(), dt, m, k, x.stride(0), q.data_ptr(), q.stride(0),
                                      scales.data_ptr(), scales.stride(1) if scales.dim() == 2 else m,
                                      _stream(x.device))
    _check(st, "bfp8_quant_act")
    return q, scales


def _scale_ld_as(a_s: torch.Tensor, m: int) -> int:
    if a_s.stride(0) != 1 and m > 1:
        raise ValueError("activation scales must be group-major: a_s.stride(0) == 1 (as quant_act returns)")
    return a_s.stride(1) if a_s.size(1) > 1 else max(m, 1)


def pad_k(codes: torch.Tensor) -> torch.Tensor:
    """A [..., K] view of the uint8 codes whose rows are padded with zeros to ceil(K/128) * 128
    bytes, the row length the GEMMs read (a copy unless they already are laid out so)."""
    codes = _as_u8(codes, "codes")
    *lead, k = codes.shape
    kp = -(-k // 128) * 128
    want, span = [1], kp
    for d in reversed(lead):  # strides of a contiguous [..., Kp] buffer
        want.insert(0, span)
        span *= d
    if codes.stride() == tuple(want) and codes.data_ptr() % 16 == 0:
        return codes
    buf = torch.zeros((*lead, kp), dtype=torch.uint8, device=codes.device)
    buf[..., :k] = codes
    return buf[..., :k]


def _check_expert_codes(b_q: torch.Tensor):
    """Expert weights [G, N, K]: K-contiguous rows, ldb apart, matrices N * ldb apart."""
    if b_q.stride(2) != 1 or b_q.stride(0) != b_q.shape[1] * b_q.stride(1):
        raise ValueError("b_q must be [G, N, K] with contiguous rows (padded rows from pad_k are fine)")


def gemm(a_q: torch.Tensor, a_s: torch.Tensor, b_q: torch.Tensor, b_s: torch.Tensor,
         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """C[M, N] (bf16) = blockwise FP8 product of a_q [M, K] and b_q [N, K] with scales a_s
    [M, ceil(K/128)] (group-major) and b_s [ceil(N/128), ceil(K/128)]. K is a multiple of 16; the
    row strides of a_q and b_q must be at least ceil(K/128) * 128 (what quant_act and pad_k give).

    workspace: optional caller-owned uint8 buffer on the same device (at least
    bfp8_gemm_workspace_bytes(M, N, K) bytes); by default one buffer per (device, stream) is kept."""
    return _gemm(a_q, a_s, b_q, b_s, out, workspace, torch.bfloat16)


def quant_act_1x64(x: torch.Tensor):
    """quant_act with 1x64 groups: returns (q [M, K] codes in rows padded to ceil(K/128) * 128
    bytes, s float32 [M, ceil(K/64)] stored group-major)."""
    dt = _in_dtype(x, "quant_act_1x64")
    _require(x, "x", x.dtype, 2)
    if x.stride(1) != 1:
        raise ValueError("x must be K-contiguous")
    m, k = x.shape
    q = torch.empty((m, -(-k // 128) * 128), dtype=torch.uint8, device=x.device)[:, :k]
    scales = torch.empty((-(-k // 64), m), dtype=torch.float32, device=x.device).t()
    st = _native.lib().bfp8_quant_act_1x64(x.data_ptr(), dt, m, k, x.stride(0), q.data_ptr(), q.stride(0),
                                           scales.data_ptr(), m if m > 0 else 1, _stream(x.device))
    _check(st, "bfp8_quant_act_1x64")
    return q, scales


def gemm_1x64(a_q: torch.Tensor, a_s: torch.Tensor, b_q: torch.Tensor, b_s: torch.Tensor,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """C[M, N] (bf16) with 1x64 activation groups and 128x64 weight blocks: a_s [M, ceil(K/64)]
    (group-major, as quant_act_1x64 returns), b_s [ceil(N/128), ceil(K/64)]; operands as for gemm."""
    a_q, b_q = _as_u8(a_q, "a_q"), _as_u8(b_q, "b_q")
    _require(a_q, "a_q", torch.uint8, 2)
    _require(b_q, "b_q", torch.uint8, 2)
    _require(a_s, "a_s", torch.float32, 2)
    _require(b_s, "b_s", torch.float32, 2)
    m, k = a_q.shape
    n = b_q.shape[0]
    if b_q.shape[1] != k:
        raise ValueError(f"a_q and b_q disagree on K: {k} vs {b_q.shape[1]}")
    if a_q.stride(1) != 1 or b_q.stride(1) != 1 or b_s.stride(1) != 1:
        raise ValueError("a_q, b_q and b_s must be contiguous along K")
    if tuple(a_s.shape) != (m, -(-k // 64)) or tuple(b_s.shape) != (-(-n // 128), -(-k // 64)):
        raise ValueError(f"scale shapes {tuple(a_s.shape)}, {tuple(b_s.shape)} do not match M={m}, N={n}, K={k} "
                         "with 1x64 / 128x64 blocks")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    _require(out, "out", torch.bfloat16, 2)
    st = _native.lib().bfp8_gemm_1x64(a_q.data_ptr(), a_q.stride(0), a_s.data_ptr(), _scale_ld_as(a_s, m),
                                      b_q.data_ptr(), b_q.stride(0), b_s.data_ptr(), b_s.stride(0), out.data_ptr(),
                                      out.stride(0), m, n, k, _stream(a_q.device))
    _check(st, "bfp8_gemm_1x64")
    return out


def gemm_f16(a_q: torch.Tensor, a_s: torch.Tensor, b_q: torch.Tensor, b_s: torch.Tensor,
             out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """gemm with an fp16 output."""
    return _gemm(a_q, a_s, b_q, b_s, out, workspace, torch.float16)


def _gemm(a_q, a_s, b_q, b_s, out, workspace, out_dtype):
    a_q, b_q = _as_u8(a_q, "a_q"), _as_u8(b_q, "b_q")
    _require(a_q, "a_q", torch.uint8, 2)
    _require(b_q, "b_q", torch.uint8, 2)
    _require(a_s, "a_s", torch.float32, 2)
    _require(b_s, "b_s", torch.float32, 2)
    m, k = a_q.shape
    n = b_q.shape[0]
    if b_q.shape[1] != k:
        raise ValueError(f"a_q and b_q disagree on K: {k} vs {b_q.shape[1]}")
    if a_q.stride(1) != 1 or b_q.stride(1) != 1 or b_s.stride(1) != 1:
        raise ValueError("a_q, b_q and b_s must be contiguous along K")
    if tuple(a_s.shape) != (m, -(-k // 128)) or tuple(b_s.shape) != (-(-n // 128), -(-k // 128)):
        raise ValueError(f"scale shapes {tuple(a_s.shape)}, {tuple(b_s.shape)} do not match M={m}, N={n}, K={k}")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a_q.device)
    _require(out, "out", out_dtype, 2)
    if out.stride(1) != 1:
        raise ValueError("out must be contiguous along N")
    lib = _native.lib()
    if workspace is None:
        ws_ptr, ws_bytes = _workspace(a_q.device, lib.bfp8_gemm_workspace_bytes(m, n, k))
    else:
        _require(workspace, "workspace", torch.uint8, 1)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    entry, name = (lib.bfp8_gemm, "bfp8_gemm") if out_dtype == torch.bfloat16 else (lib.bfp8_gemm_f16, "bfp8_gemm_f16")
    st = entry(a_q.data_ptr(), a_q.stride(0), a_s.data_ptr(), _scale_ld_as(a_s, m),
               b_q.data_ptr(), b_q.stride(0), b_s.data_ptr(), b_s.stride(0),
               out.data_ptr(), out.stride(0), m, n, k, ws_ptr or None, ws_bytes, _stream(a_q.device))
    _check(st, name)
    return out


def grouped_gemm_contiguous(a_q: torch.Tensor, a_s: torch.Tensor, b_q: torch.Tensor, b_s: torch.Tensor,
                            layout: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """M-grouped contiguous product: row m uses expert layout[m] (int32; -1 = padding, not written).

    a_q [M, K] (M % 128 == 0), a_s [M, ceil(K/128)] group-major, b_q [G, N, K] (rows of whole
    128-byte blocks, as for gemm), b_s [G, ceil(N/128), ceil(K/128)]."""
    a_q, b_q = _as_u8(a_q, "a_q"), _as_u8(b_q, "b_q")
    _require(a_q, "a_q", torch.uint8, 2)
    _require(b_q, "b_q", torch.uint8, 3)
    _require(a_s, "a_s", torch.float32, 2)
    _require(b_s, "b_s", torch.float32, 3)
    _require(layout, "layout", torch.int32, 1)
    m, k = a_q.shape
    g, n, k2 = b_q.shape
    if k2 != k or layout.shape[0] != m:
        raise ValueError("shape mismatch between a_q, b_q and layout")
    _check_expert_codes(b_q)
    if not (b_s.is_contiguous() and layout.is_contiguous()):
        raise ValueError("b_s and layout must be contiguous")
    if tuple(b_s.shape) != (g, -(-n // 128), -(-k // 128)) or tuple(a_s.shape) != (m, -(-k // 128)):
        raise ValueError("scale shapes do not match")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    _require(out, "out", torch.bfloat16, 2)
    st = _native.lib().bfp8_grouped_gemm_contiguous(
        a_q.data_ptr(), a_q.stride(0), a_s.data_ptr(), _scale_ld_as(a_s, m), b_q.data_ptr(), b_q.stride(1),
        b_s.data_ptr(), b_s.stride(1), layout.data_ptr(), g, out.data_ptr(), out.stride(0), m, n, k, None, 0,
        _stream(a_q.device))
    _check(st, "bfp8_grouped_gemm_contiguous")
    return out


def grouped_gemm_gathered(a_q: torch.Tensor, a_s: torch.Tensor, b_q: torch.Tensor, b_s: torch.Tensor,
                          layout: torch.Tensor, row_src: torch.Tensor, src_div: int = 1,
                          out: torch.Tensor | None = None) -> torch.Tensor:
    """grouped_gemm_contiguous with gathered activation codes: row m of the [M, N] product uses
    expert layout[m], reads its codes from row row_src[m] // src_div of a_q [rows, K] and its
    scales from row m of a_s [M, ceil(K/128)] (group-major, as quant_act_scatter writes them);
    rows with row_src < 0 are padding (layout -1, not written). With moe_dispatch: row_src =
    pair_of_row, src_div = top_k."""
    a_q, b_q = _as_u8(a_q, "a_q"), _as_u8(b_q, "b_q")
    _require(a_q, "a_q", torch.uint8, 2)
    _require(b_q, "b_q", torch.uint8, 3)
    _require(a_s, "a_s", torch.float32, 2)
    _require(b_s, "b_s", torch.float32, 3)
    _require(layout, "layout", torch.int32, 1)
    _require(row_src, "row_src", torch.int32, 1)
    rows, k = a_q.shape
    g, n, k2 = b_q.shape
    m = layout.shape[0]
    if k2 != k or row_src.shape[0] != m:
        raise ValueError("shape mismatch between a_q, b_q, layout and row_src")
    _check_expert_codes(b_q)
    if not (b_s.is_contiguous() and layout.is_contiguous() and row_src.is_contiguous()):
        raise ValueError("b_s, layout and row_src must be contiguous")
    if tuple(b_s.shape) != (g, -(-n // 128), -(-k // 128)) or tuple(a_s.shape) != (m, -(-k // 128)):
        raise ValueError("scale shapes do not match")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    _require(out, "out", torch.bfloat16, 2)
    st = _native.lib().bfp8_grouped_gemm_gathered(
        a_q.data_ptr(), a_q.stride(0), a_s.data_ptr(), _scale_ld_as(a_s, m), rows, row_src.data_ptr(), src_div,
        b_q.data_ptr(), b_q.stride(1), b_s.data_ptr(), b_s.stride(1), layout.data_ptr(), g, out.data_ptr(),
        out.stride(0), m, n, k, _stream(a_q.device))
    _check(st, "bfp8_grouped_gemm_gathered")
    return out


def linear(x: torch.Tensor, w_q: torch.Tensor, w_s: torch.Tensor, bias: torch.Tensor | None = None,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """FP8 linear layer, bf16 (or fp16) in and out: per-1x128-group quantization of x [M, K], the
    blockwise FP8 product with w_q [N, K] / w_s [ceil(N/128), K/128], then out + bias, the output
    and bias having x's dtype.

    workspace: optional uint8 buffer of at least bfp8_linear_workspace_bytes(M, N, K) bytes
    (holds the quantized activations); by default one buffer per (device, stream) is kept."""
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise NotImplementedError(f"linear takes bfloat16 or float16 activations (the output has their dtype), "
                                  f"got {x.dtype}")
    _require(x, "x", x.dtype, 2)
    w_q = _as_u8(w_q, "w_q")
    _require(w_q, "w_q", torch.uint8, 2)
    _require(w_s, "w_s", torch.float32, 2)
    if x.stride(1) != 1 or w_q.stride(1) != 1 or w_s.stride(1) != 1:
        raise ValueError("x, w_q and w_s must be contiguous along K")
    m, k = x.shape
    n = w_q.shape[0]
    if w_q.shape[1] != k:
        raise ValueError(f"x and w_q disagree on K: {k} vs {w_q.shape[1]}")
    if tuple(w_s.shape) != (-(-n // 128), -(-k // 128)):
        raise ValueError(f"w_s shape {tuple(w_s.shape)} does not match N={n}, K={k}")
    if bias is not None:
        _require(bias, "bias", x.dtype, 1)
        if bias.shape[0] != n or bias.stride(0) != 1:
            raise ValueError("bias must be a contiguous bf16 vector of length N")
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    _require(out, "out", x.dtype, 2)
    if out.stride(1) != 1:
        raise ValueError("out must be contiguous along N")
    lib = _native.lib()
    if workspace is None:
        ws_ptr, ws_bytes = _workspace(x.device, lib.bfp8_linear_workspace_bytes(m, n, k))
    else:
        _require(workspace, "workspace", torch.uint8, 1)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = lib.bfp8_linear(x.data_ptr(), _IN_DTYPES[x.dtype], m, k, x.stride(0), w_q.data_ptr(), w_q.stride(0),
                         w_s.data_ptr(), w_s.stride(0), bias.data_ptr() if bias is not None else None,
                         out.data_ptr(), out.stride(0), n, ws_ptr or None, ws_bytes, _stream(x.device))
    _check(st, "bfp8_linear")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # BFP8_NOALLOC_SCRATCH_BYTES


def linear_noalloc(x: torch.Tensor, w_q: torch.Tensor, w_s: torch.Tensor, out: torch.Tensor,
                   bias: torch.Tensor | None = None) -> torch.Tensor:
    """linear() through bfp8_linear_noalloc: no workspace, the quantized activations are staged in
    the library's fixed device array (at most NOALLOC_SCRATCH_BYTES of staging). The caller passes
    the output, so the call allocates nothing; calls that overlap in time on one device race on the
    array."""
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise NotImplementedError(f"linear takes bfloat16 or float16 activations, got {x.dtype}")
    _require(x, "x", x.dtype, 2)
    w_q = _as_u8(w_q, "w_q")
    _require(w_q, "w_q", torch.uint8, 2)
    _require(w_s, "w_s", torch.float32, 2)
    _require(out, "out", x.dtype, 2)
    if x.stride(1) != 1 or w_q.stride(1) != 1 or w_s.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("x, w_q, w_s and out must be contiguous along their last dimension")
    m, k = x.shape
    n = w_q.shape[0]
    if w_q.shape[1] != k or tuple(out.shape) != (m, n):
        raise ValueError(f"shapes disagree: x {tuple(x.shape)}, w_q {tuple(w_q.shape)}, out {tuple(out.shape)}")
    if tuple(w_s.shape) != (-(-n // 128), -(-k // 128)):
        raise ValueError(f"w_s shape {tuple(w_s.shape)} does not match N={n}, K={k}")
    if bias is not None:
        _require(bias, "bias", x.dtype, 1)
        if bias.shape[0] != n or bias.stride(0) != 1:
            raise ValueError("bias must be a contiguous vector of length N")
    st = _native.lib().bfp8_linear_noalloc(
        x.data_ptr(), _IN_DTYPES[x.dtype], m, k, x.stride(0), w_q.data_ptr(), w_q.stride(0), w_s.data_ptr(),
        w_s.stride(0), bias.data_ptr() if bias is not None else None, out.data_ptr(), out.stride(0), n,
        _stream(x.device))
    _check(st, "bfp8_linear_noalloc")
    return out


def _codes(t: torch.Tensor, name: str) -> torch.Tensor:
    """UE8M0 scale codes as uint8 (float8_e8m0fnu tensors are viewed as their bytes)."""
    if t.dtype == torch.float8_e8m0fnu:
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise NotImplementedError(f"{name}: UE8M0 scale codes are uint8 or float8_e8m0fnu, got {t.dtype}")
    return t


def _check_padded_rows(t: torch.Tensor, name: str, ld: int, rows: int, cols: int):
    """The UE8M0 kernels read codes four at a time: rows of ld bytes (a multiple of 4), all allocated."""
    if ld % 4:
        raise ValueError(f"{name}: rows of UE8M0 codes must be a multiple of 4 bytes apart (got {ld}); "
                         "ue8m0_scales() and quant_act_ue8m0() lay them out so")
    span = (rows - 1) * ld + (-(-cols // 4) * 4)
    if t.untyped_storage().nbytes() - t.storage_offset() < span:
        raise ValueError(f"{name}: the last row of UE8M0 codes must be padded to a multiple of 4 bytes")


def ue8m0_scales(codes: torch.Tensor) -> torch.Tensor:
    """UE8M0 scale codes [..., R, C] copied into rows padded to a multiple of 4 bytes, the layout
    the UE8M0 GEMMs read (weights are prepared once); returns a view of the same shape."""
    codes = _codes(codes, "codes")
    *lead, r, c = codes.shape
    buf = torch.zeros((*lead, r, -(-c // 4) * 4), dtype=torch.uint8, device=codes.device)
    buf[..., :c] = codes
    return buf[..., :c]


def quant_act_ue8m0(x: torch.Tensor, q: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """quant_act with power-of-two scales: returns (q, e) with e the UE8M0 codes [M, K/128]
    (uint8), stored group-major with a row of codes padded to a multiple of 4 bytes."""
    dt = _in_dtype(x, "quant_act_ue8m0")
    _require(x, "x", x.dtype, 2)
    if x.stride(1) != 1:
        raise ValueError("x must be K-contiguous")
    m, k = x.shape
    if q is None:  # rows of whole 128-byte blocks, as the GEMMs read them
        q = torch.empty((m, -(-k // 128) * 128), dtype=torch.uint8, device=x.device)[:, :k]
    if scales is None:
        ld = max(-(-m // 4) * 4, 4)
        scales = torch.empty((-(-k // 128), ld), dtype=torch.uint8, device=x.device)[:, :m].t()
    scales = _codes(scales, "scales")
    _require(q, "q", torch.uint8, 2)
    _require(scales, "scales", torch.uint8, 2)
    if q.stride(1) != 1 or (scales.stride(0) != 1 and m > 1):
        raise ValueError("q must be K-contiguous and scales group-major (stride(0) == 1)")
    st = _native.lib().bfp8_quant_act_ue8m0(x.data_ptr(), dt, m, k, x.stride(0), q.data_ptr(), q.stride(0),
                                            scales.data_ptr(), scales.stride(1), _stream(x.device))
    _check(st, "bfp8_quant_act_ue8m0")
    return q, scales


def gemm_ue8m0(a_q: torch.Tensor, a_e: torch.Tensor, b_q: torch.Tensor, b_e: torch.Tensor,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """gemm with UE8M0 scale codes: a_e [M, K/128] group-major (as quant_act_ue8m0 returns) and
    b_e [ceil(N/128), K/128] with rows padded to a multiple of 4 bytes (ue8m0_scales)."""
    a_q, b_q = _as_u8(a_q, "a_q"), _as_u8(b_q, "b_q")
    a_e, b_e = _codes(a_e, "a_e"), _codes(b_e, "b_e")
    _require(a_q, "a_q", torch.uint8, 2)
    _require(b_q, "b_q", torch.uint8, 2)
    _require(a_e, "a_e", torch.uint8, 2)
    _require(b_e, "b_e", torch.uint8, 2)
    m, k = a_q.shape
    n = b_q.shape[0]
    kb = -(-k // 128)
    if b_q.shape[1] != k:
        raise ValueError(f"a_q and b_q disagree on K: {k} vs {b_q.shape[1]}")
    if a_q.stride(1) != 1 or b_q.stride(1) != 1 or b_e.stride(1) != 1:
        raise ValueError("a_q, b_q and b_e must be contiguous along K")
    if tuple(a_e.shape) != (m, kb) or tuple(b_e.shape) != (-(-n // 128), kb):
        raise ValueError(f"scale shapes {tuple(a_e.shape)}, {tuple(b_e.shape)} do not match M={m}, N={n}, K={k}")
    if a_e.stride(0) != 1 and m > 1:
        raise ValueError("a_e must be group-major: a_e.stride(0) == 1 (as quant_act_ue8m0 returns)")
    ld_as = a_e.stride(1)
    if m > 0:
        _check_padded_rows(a_e, "a_e", ld_as, kb, m)
    _check_padded_rows(b_e, "b_e", b_e.stride(0), b_e.shape[0], kb)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    _require(out, "out", torch.bfloat16, 2)
    if out.stride(1) != 1:
        raise ValueError("out must be contiguous along N")
    lib = _native.lib()
    if workspace is None:
        ws_ptr, ws_bytes = _workspace(a_q.device, lib.bfp8_gemm_workspace_bytes(m, n, k))
    else:
        _require(workspace, "workspace", torch.uint8, 1)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = lib.bfp8_gemm_ue8m0(a_q.data_ptr(), a_q.stride(0), a_e.data_ptr(), ld_as, b_q.data_ptr(), b_q.stride(0),
                             b_e.data_ptr(), b_e.stride(0), out.data_ptr(), out.stride(0), m, n, k, ws_ptr or None,
                             ws_bytes, _stream(a_q.device))
    _check(st, "bfp8_gemm_ue8m0")
    return out


def grouped_gemm_contiguous_ue8m0(a_q: torch.Tensor, a_e: torch.Tensor, b_q: torch.Tensor, b_e: torch.Tensor,
                                  layout: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """grouped_gemm_contiguous with UE8M0 scale codes: b_e [G, ceil(N/128), K/128] with rows padded
    to a multiple of 4 bytes (ue8m0_scales), a_e as for gemm_ue8m0."""
    a_q, b_q = _as_u8(a_q, "a_q"), _as_u8(b_q, "b_q")
    a_e, b_e = _codes(a_e, "a_e"), _codes(b_e, "b_e")
    _require(a_q, "a_q", torch.uint8, 2)
    _require(b_q, "b_q", torch.uint8, 3)
    _require(a_e, "a_e", torch.uint8, 2)
    _require(b_e, "b_e", torch.uint8, 3)
    _require(layout, "layout", torch.int32, 1)
    m, k = a_q.shape
    g, n, k2 = b_q.shape
    kb = -(-k // 128)
    nb = -(-n // 128)
    if k2 != k or layout.shape[0] != m:
        raise ValueError("shape mismatch between a_q, b_q and layout")
    _check_expert_codes(b_q)
    if not layout.is_contiguous():
        raise ValueError("layout must be contiguous")
    if tuple(b_e.shape) != (g, nb, kb) or tuple(a_e.shape) != (m, kb):
        raise ValueError("scale shapes do not match")
    if b_e.stride(2) != 1 or b_e.stride(0) != nb * b_e.stride(1):
        raise ValueError("b_e must be [G][ceil(N/128)][ld] with consecutive experts (ue8m0_scales)")
    if a_e.stride(0) != 1 and m > 1:
        raise ValueError("a_e must be group-major: a_e.stride(0) == 1 (as quant_act_ue8m0 returns)")
    if m > 0:
        _check_padded_rows(a_e, "a_e", a_e.stride(1), kb, m)
    _check_padded_rows(b_e, "b_e", b_e.stride(1), g * nb, kb)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a_q.device)
    _require(out, "out", torch.bfloat16, 2)
    st = _native.lib().bfp8_grouped_gemm_contiguous_ue8m0(
        a_q.data_ptr(), a_q.stride(0), a_e.data_ptr(), a_e.stride(1), b_q.data_ptr(), b_q.stride(1),
        b_e.data_ptr(), b_e.stride(1), layout.data_ptr(), g, out.data_ptr(), out.stride(0), m, n, k, None, 0,
        _stream(a_q.device))
    _check(st, "bfp8_grouped_gemm_contiguous_ue8m0")
    return out


def moe_padded_rows(s: int, e: int, align: int = 128) -> int:
    """Rows of the padded MoE buffer for s (token, expert) pairs and e experts."""
    return _native.lib().bfp8_moe_padded_rows(s, e, align)


def moe_dispatch(topk_ids: torch.Tensor, num_experts: int, align: int = 128):
    """Routing layout on the device: (row_of_pair [S], pair_of_row [R], layout [R], expert_start [E+1]),
    int32, for topk_ids [T, top_k] (ids outside [0, E) are sentinels)."""
    _require(topk_ids, "topk_ids", torch.int32, 2)
    ids = topk_ids.contiguous()
    s_pairs = ids.numel()
    lib = _native.lib()
    rows = lib.bfp8_moe_padded_rows(s_pairs, num_experts, align)
    dev = ids.device
    row_of_pair = torch.empty(s_pairs, dtype=torch.int32, device=dev)
    pair_of_row = torch.empty(rows, dtype=torch.int32, device=dev)
    layout = torch.empty(rows, dtype=torch.int32, device=dev)
    expert_start = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    scratch = torch.empty(max(lib.bfp8_moe_dispatch_workspace_bytes(s_pairs, num_experts), 4), dtype=torch.uint8,
                          device=dev)
    st = lib.bfp8_moe_dispatch(ids.data_ptr(), s_pairs, num_experts, align, row_of_pair.data_ptr(),
                               pair_of_row.data_ptr(), layout.data_ptr(), expert_start.data_ptr(), scratch.data_ptr(),
                               scratch.numel(), _stream(dev))
    _check(st, "bfp8_moe_dispatch")
    return row_of_pair, pair_of_row, layout, expert_start


def quant_act_gather(x: torch.Tensor, row_src: torch.Tensor, src_div: int = 1):
    """quant_act of the gathered rows: output row m quantizes x[row_src[m] // src_div]; rows with
    row_src[m] < 0 are left unwritten. Returns (q [M, K], s [M, K/128] group-major)."""
    dt = _in_dtype(x, "quant_act_gather")
    _require(x, "x", x.dtype, 2)
    _require(row_src, "row_src", torch.int32, 1)
    if x.stride(1) != 1 or not row_src.is_contiguous():
        raise ValueError("x must be K-contiguous and row_src contiguous")
    m, k = row_src.numel(), x.shape[1]
    q = torch.empty((m, -(-k // 128) * 128), dtype=torch.uint8, device=x.device)[:, :k]
    s = torch.empty((-(-k // 128), m), dtype=torch.float32, device=x.device).t()
    st = _native.lib().bfp8_quant_act_gather(x.data_ptr(), dt, x.shape[0], k, x.stride(0), row_src.data_ptr(),
                                             src_div, m, q.data_ptr(), q.stride(0), s.data_ptr(), max(m, 1),
                                             _stream(x.device))
    _check(st, "bfp8_quant_act_gather")
    return q, s


def quant_act_scatter(x: torch.Tensor, scale_dst: torch.Tensor, scale_fan: int, rows: int):
    """quant_act of x [M, K] with each row's scales written to rows scale_dst[m * scale_fan + j] of
    a [rows, ceil(K/128)] group-major scale matrix (entries < 0 skipped; rows no entry names are
    left unwritten). Returns (q [M, K], s [rows, ceil(K/128)]). With moe_dispatch: scale_dst =
    row_of_pair, scale_fan = top_k, rows = len(layout)."""
    _require(x, "x", x.dtype, 2)
    _require(scale_dst, "scale_dst", torch.int32, 1)
    m, k = x.shape
    if scale_dst.numel() != m * scale_fan or not scale_dst.is_contiguous():
        raise ValueError("scale_dst must be a contiguous int32 vector of M * scale_fan entries")
    if x.stride(1) != 1:
        raise ValueError("x must be contiguous along K")
    q = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    s = torch.empty((-(-k // 128), max(rows, 1)), dtype=torch.float32, device=x.device).t()[:rows]
    st = _native.lib().bfp8_quant_act_scatter(x.data_ptr(), _in_dtype(x, "x"), m, k, x.stride(0), q.data_ptr(),
                                              q.stride(0), s.data_ptr(), max(rows, 1), scale_dst.data_ptr(), scale_fan,
                                              _stream(x.device))
    _check(st, "bfp8_quant_act_scatter")
    return q, s


def swiglu_quant(proj: torch.Tensor, layout: torch.Tensor | None = None):
    """h = bf16(bf16(silu(gate)) * up) of proj [M, 2I] (bf16, gate first) quantized per 1x128 group:
    returns (q [M, I], s [M, I/128] group-major); rows with layout == -1 are left unwritten."""
    _require(proj, "proj", torch.bfloat16, 2)
    if proj.stride(1) != 1:
        raise ValueError("proj must be contiguous along its columns")
    m, two_i = proj.shape
    i = two_i // 2
    if layout is not None:
        _require(layout, "layout", torch.int32, 1)
        if layout.numel() != m or not layout.is_contiguous():
            raise ValueError("layout must be a contiguous int32 vector of M entries")
    q = torch.empty((m, i), dtype=torch.uint8, device=proj.device)
    s = torch.empty((i // 128, m), dtype=torch.float32, device=proj.device).t()
    st = _native.lib().bfp8_swiglu_quant(proj.data_ptr(), m, i, proj.stride(0),
                                         layout.data_ptr() if layout is not None else None, q.data_ptr(), q.stride(0),
                                         s.data_ptr(), max(m, 1), _stream(proj.device))
    _check(st, "bfp8_swiglu_quant")
    return q, s


def swiglu(proj: torch.Tensor, layout: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """h = bf16(bf16(silu(gate)) * up) of proj [M, 2I] (bf16, gate first) as bf16 [M, I], the values
    swiglu_quant quantizes; rows with layout == -1 are left unwritten."""
    _require(proj, "proj", torch.bfloat16, 2)
    if proj.stride(1) != 1:
        raise ValueError("proj must be contiguous along its columns")
    m, two_i = proj.shape
    i = two_i // 2
    if layout is not None:
        _require(layout, "layout", torch.int32, 1)
        if layout.numel() != m or not layout.is_contiguous():
            raise ValueError("layout must be a contiguous int32 vector of M entries")
    if out is None:
        out = torch.empty((m, i), dtype=torch.bfloat16, device=proj.device)
    _require(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (m, i) or out.stride(1) != 1:
        raise ValueError(f"out must be [{m}, {i}] and contiguous along its columns")
    st = _native.lib().bfp8_swiglu(proj.data_ptr(), m, i, proj.stride(0),
                                   layout.data_ptr() if layout is not None else None, out.data_ptr(), out.stride(0),
                                   _stream(proj.device))
    _check(st, "bfp8_swiglu")
    return out


def moe_combine(out: torch.Tensor, row_of_pair: torch.Tensor, topk_weights: torch.Tensor) -> torch.Tensor:
    """y [T, H] = per token, sum_j bf16(out[row_of_pair[t, j]] * bf16(w[t, j])) (float32 sum, in order j)."""
    _require(out, "out", torch.bfloat16, 2)
    _require(topk_weights, "topk_weights", torch.float32, 2)
    _require(row_of_pair, "row_of_pair", torch.int32, row_of_pair.dim())
    t, k = topk_weights.shape
    if row_of_pair.numel() != t * k or not row_of_pair.is_contiguous() or not topk_weights.is_contiguous():
        raise ValueError("row_of_pair and topk_weights must be contiguous with T * top_k entries")
    h = out.shape[1]
    y = torch.empty((t, h), dtype=torch.bfloat16, device=out.device)
    st = _native.lib().bfp8_moe_combine(out.data_ptr(), out.stride(0), row_of_pair.data_ptr(), topk_weights.data_ptr(),
                                        t, k, h, y.data_ptr(), y.stride(0), _stream(out.device))
    _check(st, "bfp8_moe_combine")
    return y


def moe_forward_workspace_bytes(t: int, top_k: int, e: int, h: int, i: int) -> int:
    return _native.lib().bfp8_moe_forward_workspace_bytes(t, top_k, e, h, i)


def moe_forward(hidden: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor, w_up: torch.Tensor,
                s_up: torch.Tensor, w_down: torch.Tensor, s_down: torch.Tensor, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """FP8 experts forward: hidden [T, H] bf16, topk_ids [T, k] int32, topk_weights [T, k] float32,
    w_up [E, 2I, H] e4m3 with s_up [E, 2I/128, H/128], w_down [E, H, I] with s_down [E, H/128, I/128]."""
    _require(hidden, "hidden", torch.bfloat16, 2)
    _require(topk_ids, "topk_ids", torch.int32, 2)
    _require(topk_weights, "topk_weights", torch.float32, 2)
    w_up, w_down = _as_u8(w_up, "w_up"), _as_u8(w_down, "w_down")
    _require(w_up, "w_up", torch.uint8, 3)
    _require(w_down, "w_down", torch.uint8, 3)
    _require(s_up, "s_up", torch.float32, 3)
    _require(s_down, "s_down", torch.float32, 3)
    t, h = hidden.shape
    e, two_i, h2 = w_up.shape
    i = two_i // 2
    if h2 != h or tuple(w_down.shape) != (e, h, i) or topk_ids.shape != topk_weights.shape or topk_ids.shape[0] != t:
        raise ValueError("shape mismatch between hidden, routing and expert weights")
    if tuple(s_up.shape) != (e, -(-two_i // 128), h // 128) or tuple(s_down.shape) != (e, -(-h // 128), i // 128):
        raise ValueError("scale shapes do not match the expert weights")
    for name, ten in (("w_up", w_up), ("w_down", w_down), ("s_up", s_up), ("s_down", s_down),
                      ("topk_ids", topk_ids), ("topk_weights", topk_weights)):
        if not ten.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if hidden.stride(1) != 1:
        raise ValueError("hidden must be contiguous along H")
    if out is None:
        out = torch.empty((t, h), dtype=torch.bfloat16, device=hidden.device)
    _require(out, "out", torch.bfloat16, 2)
    lib = _native.lib()
    need = lib.bfp8_moe_forward_workspace_bytes(t, topk_ids.shape[1], e, h, i)
    if workspace is None:
        ws_ptr, ws_bytes = _workspace(hidden.device, need)
    else:
        _require(workspace, "workspace", torch.uint8, 1)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = lib.bfp8_moe_forward(hidden.data_ptr(), t, h, hidden.stride(0), topk_ids.data_ptr(), topk_weights.data_ptr(),
                              topk_ids.shape[1], e, w_up.data_ptr(), s_up.data_ptr(), w_down.data_ptr(),
                              s_down.data_ptr(), i, out.data_ptr(), out.stride(0), ws_ptr or None, ws_bytes,
                              _stream(hidden.device))
    _check(st, "bfp8_moe_forward")
    return out


def nn_to_nt_weights(w_nn: torch.Tensor, s_nn: torch.Tensor):
    """NN expert weights w_nn [E, K, N] (e4m3) and scales s_nn [E, K/128, ceil(N/128)] converted once
    to the NT layout the grouped GEMM reads: (w [E, N, K], s [E, ceil(N/128), K/128])."""
    w_nn = _as_u8(w_nn, "w_nn")
    _require(w_nn, "w_nn", torch.uint8, 3)
    _require(s_nn, "s_nn", torch.float32, 3)
    if not (w_nn.is_contiguous() and s_nn.is_contiguous()):
        raise ValueError("w_nn and s_nn must be contiguous")
    e, k, n = w_nn.shape
    if tuple(s_nn.shape) != (e, -(-k // 128), -(-n // 128)):
        raise ValueError("s_nn shape does not match w_nn")
    kp = -(-k // 128) * 128  # rows of whole 128-byte blocks, as the GEMMs read them
    w = torch.empty((e, n, kp), dtype=torch.uint8, device=w_nn.device)[..., :k]
    s = torch.empty((e, s_nn.shape[2], s_nn.shape[1]), dtype=torch.float32, device=w_nn.device)
    lib = _native.lib()
    _check(lib.bfp8_transpose_weights(w_nn.data_ptr(), e, k, n, n, w.data_ptr(), kp, _stream(w_nn.device)),
           "bfp8_transpose_weights")
    _check(lib.bfp8_transpose_scales(s_nn.data_ptr(), e, s_nn.shape[1], s_nn.shape[2], s.data_ptr(),
                                     _stream(w_nn.device)), "bfp8_transpose_scales")
    return w, s


def expand_act_scales(s: torch.Tensor, m: int, k: int) -> torch.Tensor:
    """Block activation scales [M, ceil(K/128)] (group-major, as quant_act returns them) from one
    per-tensor scale (a 0-d or 1-element float32 tensor) or per-token scales s [M], on s's device."""
    _require(s, "s", torch.float32, s.dim())
    if s.dim() > 1 or (s.numel() != m and s.numel() != 1):
        raise ValueError(f"s must hold one scale or one per row (M = {m}), got shape {tuple(s.shape)}")
    s = s.contiguous()
    g = -(-k // 128)
    out = torch.empty((g, max(m, 1)), dtype=torch.float32, device=s.device)[:, :m].t()
    stride = 1 if s.numel() == m and m != 1 else 0
    _check(_native.lib().bfp8_expand_act_scales(s.data_ptr(), stride, m, k, out.data_ptr(), max(m, 1),
                                                _stream(s.device)), "bfp8_expand_act_scales")
    return out


def expand_weight_scale(s: torch.Tensor, n: int, k: int) -> torch.Tensor:
    """Block weight scales [ceil(N/128), ceil(K/128)] from one per-tensor scale (float32 tensor of
    one element), on s's device."""
    _require(s, "s", torch.float32, s.dim())
    if s.numel() != 1:
        raise ValueError("a per-tensor weight scale has one element (per-channel scales have no block form)")
    s = s.contiguous()
    out = torch.empty((-(-n // 128), -(-k // 128)), dtype=torch.float32, device=s.device)
    _check(_native.lib().bfp8_expand_weight_scale(s.data_ptr(), n, k, out.data_ptr(), out.stride(0),
                                                  _stream(s.device)), "bfp8_expand_weight_scale")
    return out


def linear_workspace_bytes(m: int, n: int, k: int) -> int:
    """Bytes of device workspace that linear() needs for an [m, k] x [n, k] layer."""
    return _native.lib().bfp8_linear_workspace_bytes(m, n, k)


def linear_fuses(m: int, n: int, k: int, ldx: int | None = None) -> bool:
    """Whether linear() with these sizes runs one kernel that quantizes the activations inside
    the GEMM (small M), rather than the quantizer and then the GEMM."""
    return bool(_native.lib().bfp8_linear_fuses(m, n, k, k if ldx is None else ldx))


def set_schedule(name: str) -> None:
    """Force a GEMM schedule ('small_m', 'tiled', 'persistent') or restore the automatic choice
    ('auto'). 'persistent' is the tiled schedule with its 256 x 256 launches on the persistent
    kernel; the automatic choice never takes it (it measured slower)."""
    if name not in SCHEDULES:
        raise ValueError(f"unknown schedule {name!r}; choose from {sorted(SCHEDULES)}")
    _check(_native.lib().bfp8_set_schedule(SCHEDULES[name]), "bfp8_set_schedule")


def get_schedule() -> str:
    v = _native.lib().bfp8_get_schedule()
    return {v_: k_ for k_, v_ in SCHEDULES.items()}[v]


def schedule_for(m: int, n: int, k: int) -> str:
    v = _native.lib().bfp8_gemm_schedule_for(m, n, k)
    return {v_: k_ for k_, v_ in SCHEDULES.items()}[v]
