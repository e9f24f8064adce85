"""AWQ W4A16 hot path on AMD Instinct MI355X (gfx950).

Thin Python binding of the C ABI declared in include/awq.h.  Each function has
the name of the C entry point it calls and only marshals arguments: torch
provides device memory (outputs and workspaces are allocated with torch when
the caller does not pass them) and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback: the
functions raise if the library is missing or a tensor is not on the GPU.
"""
from __future__ import annotations

import ctypes

import torch

from . import _abi
from ._abi import (AWQ_BF16, AWQ_F16, AWQ_F32, AWQ_GROUP, AWQ_OP_ACT_STATS, AWQ_OP_GEMM,  # noqa: F401
                   AWQ_OP_QUANTIZE, AWQ_OP_SEARCH, AwqError, lib)

__all__ = ["awq_act_stats", "awq_search_scales", "awq_search_scales_ex", "awq_quantize_pack", "awq_quantize_codes",
           "awq_w4a16_gemm", "awq_w4a16_gemm_noalloc", "awq_read_stream", "awq_fold_scales", "awq_salient_channels", "awq_workspace_bytes",
           "AwqError", "lib"]

_DT = {torch.float16: AWQ_F16, torch.bfloat16: AWQ_BF16, torch.float32: AWQ_F32}


def _dev(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a tensor on the GPU")


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p | None:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _rows(x: torch.Tensor, name: str) -> tuple[int, int, int]:
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return x.shape[0], x.shape[1], x.stride(0)


def _workspace(nbytes: int, device, ws: torch.Tensor | None) -> tuple[torch.Tensor | None, int]:
    if nbytes == 0:
        return ws, 0 if ws is None else ws.numel() * ws.element_size()
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def awq_workspace_bytes(op: int, M: int = 0, N: int = 0, K: int = 0, T: int = 0, n_alpha: int = 0) -> int:
    return int(lib().awq_workspace_bytes(op, M, N, K, T, n_alpha))


def awq_act_stats(x: torch.Tensor, mean_abs: torch.Tensor | None = None,
                  ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mean |x[:, j]| over rows, float32 [K]."""
    _dev(x, "x")
    T, K, ldx = _rows(x, "x")
    if mean_abs is None:
        mean_abs = torch.empty(K, dtype=torch.float32, device=x.device)
    ws, wsb = _workspace(awq_workspace_bytes(AWQ_OP_ACT_STATS, 0, 0, K, T, 0), x.device, ws)
    st = lib().awq_act_stats(_ptr(x), _DT.get(x.dtype, -1), T, K, ldx, _ptr(mean_abs), _ptr(ws),
                             wsb, _stream(x.device, stream))
    _abi.check("awq_act_stats", st)
    return mean_abs


def awq_search_scales(w: torch.Tensor, x_calib: torch.Tensor, mean_abs: torch.Tensor,
                      alphas: torch.Tensor, group_size: int = AWQ_GROUP,
                      s_out: torch.Tensor | None = None, inv_s_out: torch.Tensor | None = None,
                      loss_out: torch.Tensor | None = None, best_idx_out: torch.Tensor | None = None,
                      ws: torch.Tensor | None = None, stream=None, *, bits: int = 4,
                      symmetric: bool = False, kept: torch.Tensor | None = None):
    """Returns (s [K] f32, inv_s [K] f32, losses [n] f64, best index int32 [1]).
    With the defaults this calls awq_search_scales (the 4-bit asymmetric grid);
    bits / symmetric (another grid) or kept (uint8 [K]: channels kept in
    16-bit, the mixed-precision baseline) call awq_search_scales_ex."""
    ex = bits != 4 or bool(symmetric) or kept is not None
    return _search(w, x_calib, mean_abs, alphas, group_size, s_out, inv_s_out, loss_out,
                   best_idx_out, ws, stream, (bits, symmetric, kept) if ex else None)


def awq_search_scales_ex(w: torch.Tensor, x_calib: torch.Tensor, mean_abs: torch.Tensor,
                         alphas: torch.Tensor, group_size: int = AWQ_GROUP, bits: int = 4,
                         symmetric: bool = False, kept: torch.Tensor | None = None,
                         s_out: torch.Tensor | None = None, inv_s_out: torch.Tensor | None = None,
                         loss_out: torch.Tensor | None = None,
                         best_idx_out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                         stream=None):
    """awq_search_scales_ex: the search under the grid (bits, symmetric) with
    the channels marked in kept (uint8 [K] or None) left in 16-bit."""
    return _search(w, x_calib, mean_abs, alphas, group_size, s_out, inv_s_out, loss_out,
                   best_idx_out, ws, stream, (bits, symmetric, kept))


def _search(w, x_calib, mean_abs, alphas, group_size, s_out, inv_s_out, loss_out, best_idx_out,
            ws, stream, variant):
    for t, n in ((w, "w"), (x_calib, "x_calib"), (mean_abs, "mean_abs"), (alphas, "alphas")):
        _dev(t, n)
    if not w.is_contiguous() or w.dim() != 2:
        raise ValueError("w must be a contiguous [N, K] tensor")
    if alphas.dtype != torch.float64:
        raise ValueError("alphas must be float64")
    N, K = w.shape
    T, Kx, ldx = _rows(x_calib, "x_calib")
    if Kx != K or x_calib.dtype != w.dtype:
        raise ValueError("x_calib must be [T, K] with w's dtype")
    n_alpha = alphas.numel()
    dev = w.device
    s_out = torch.empty(K, dtype=torch.float32, device=dev) if s_out is None else s_out
    inv_s_out = torch.empty(K, dtype=torch.float32, device=dev) if inv_s_out is None else inv_s_out
    loss_out = torch.empty(n_alpha, dtype=torch.float64, device=dev) if loss_out is None else loss_out
    best_idx_out = torch.empty(1, dtype=torch.int32, device=dev) if best_idx_out is None else best_idx_out
    ws, wsb = _workspace(awq_workspace_bytes(AWQ_OP_SEARCH, 0, N, K, T, n_alpha), dev, ws)
    head = (_ptr(w), _DT.get(w.dtype, -1), N, K, _ptr(x_calib), T, ldx, _ptr(mean_abs),
            _ptr(alphas), n_alpha, group_size)
    tail = (_ptr(s_out), _ptr(inv_s_out), _ptr(loss_out), _ptr(best_idx_out), _ptr(ws), wsb,
            _stream(dev, stream))
    if variant is None:
        st = lib().awq_search_scales(*head, *tail)
        _abi.check("awq_search_scales", st)
    else:
        bits, symmetric, kept = variant
        st = lib().awq_search_scales_ex(*head, bits, int(bool(symmetric)), _ptr(kept), *tail)
        _abi.check("awq_search_scales_ex", st)
    return s_out, inv_s_out, loss_out, best_idx_out


def awq_quantize_pack(w: torch.Tensor, s: torch.Tensor | None = None, group_size: int = AWQ_GROUP,
                      qweight: torch.Tensor | None = None, scales: torch.Tensor | None = None,
                      zeros: torch.Tensor | None = None, scales_f32_dbg: torch.Tensor | None = None,
                      stream=None):
    """Returns (qweight int32 [N, K/8], scales fp16 [N, K/g], zeros uint8 [N, K/g])."""
    _dev(w, "w")
    if not w.is_contiguous() or w.dim() != 2:
        raise ValueError("w must be a contiguous [N, K] tensor")
    N, K = w.shape
    dev = w.device
    G = K // group_size if group_size > 0 else 0
    qweight = torch.empty((N, K // 8), dtype=torch.int32, device=dev) if qweight is None else qweight
    scales = torch.empty((N, G), dtype=torch.float16, device=dev) if scales is None else scales
    zeros = torch.empty((N, G), dtype=torch.uint8, device=dev) if zeros is None else zeros
    st = lib().awq_quantize_pack(_ptr(w), _DT.get(w.dtype, -1), N, K, _ptr(s), group_size,
                                 _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(scales_f32_dbg),
                                 _stream(dev, stream))
    _abi.check("awq_quantize_pack", st)
    return qweight, scales, zeros


def awq_quantize_codes(w: torch.Tensor, s: torch.Tensor | None = None, group_size: int = AWQ_GROUP,
                       bits: int = 4, symmetric: bool = False, codes: torch.Tensor | None = None,
                       scales: torch.Tensor | None = None, zeros: torch.Tensor | None = None,
                       stream=None):
    """Returns (codes uint8 [N, K], scales fp16 [N, K/g], zeros uint8 [N, K/g])."""
    _dev(w, "w")
    if not w.is_contiguous() or w.dim() != 2:
        raise ValueError("w must be a contiguous [N, K] tensor")
    N, K = w.shape
    dev = w.device
    G = K // group_size if group_size > 0 else 0
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev) if codes is None else codes
    scales = torch.empty((N, G), dtype=torch.float16, device=dev) if scales is None else scales
    zeros = torch.empty((N, G), dtype=torch.uint8, device=dev) if zeros is None else zeros
    st = lib().awq_quantize_codes(_ptr(w), _DT.get(w.dtype, -1), N, K, _ptr(s), group_size, bits,
                                  int(bool(symmetric)), _ptr(codes), _ptr(scales), _ptr(zeros),
                                  _stream(dev, stream))
    _abi.check("awq_quantize_codes", st)
    return codes, scales, zeros


def awq_salient_channels(mean_abs: torch.Tensor, n_keep: int, kept: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """uint8 [K]: 1 for the n_keep channels of largest mean |x| (ties: lower index)."""
    _dev(mean_abs, "mean_abs")
    if mean_abs.dtype != torch.float32 or mean_abs.dim() != 1 or not mean_abs.is_contiguous():
        raise ValueError("mean_abs must be a contiguous float32 vector")
    K = mean_abs.numel()
    kept = torch.empty(K, dtype=torch.uint8, device=mean_abs.device) if kept is None else kept
    st = lib().awq_salient_channels(_ptr(mean_abs), K, n_keep, _ptr(kept), _stream(mean_abs.device, stream))
    _abi.check("awq_salient_channels", st)
    return kept


def awq_w4a16_gemm(x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor,
                   zeros: torch.Tensor, inv_s: torch.Tensor | None = None,
                   out_dtype: torch.dtype | None = None, y: torch.Tensor | None = None,
                   group_size: int = AWQ_GROUP, ws: torch.Tensor | None = None, stream=None):
    """y = x (dequant W)^T, [M, N] of out_dtype (default x.dtype)."""
    _dev(x, "x")
    _dev(qweight, "qweight")
    M, K, ldx = _rows(x, "x")
    N = qweight.shape[0]
    if qweight.shape[1] * 8 != K:
        raise ValueError("qweight must be [N, K/8]")
    dev = x.device
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype or x.dtype, device=dev)
    ldy = y.stride(0) if y.dim() == 2 else N
    ws, wsb = _workspace(awq_workspace_bytes(AWQ_OP_GEMM, M, N, K, 0, 0), dev, ws)
    st = lib().awq_w4a16_gemm(_ptr(x), _DT.get(x.dtype, -1), M, K, ldx, _ptr(qweight), _ptr(scales),
                              _ptr(zeros), N, group_size, _ptr(inv_s), _ptr(y), _DT.get(y.dtype, -1),
                              ldy, _ptr(ws), wsb, _stream(dev, stream))
    _abi.check("awq_w4a16_gemm", st)
    return y


def awq_w4a16_gemm_noalloc(x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor,
                           zeros: torch.Tensor, inv_s: torch.Tensor | None = None,
                           y: torch.Tensor | None = None, out_dtype: torch.dtype | None = None,
                           group_size: int = AWQ_GROUP, stream=None):
    """awq_w4a16_gemm without a workspace: the library's own per-GPU scratch
    array serves the product (calls that overlap on one GPU race).  Pass y to
    call it without any allocation."""
    _dev(x, "x")
    _dev(qweight, "qweight")
    M, K, ldx = _rows(x, "x")
    N = qweight.shape[0]
    if qweight.shape[1] * 8 != K:
        raise ValueError("qweight must be [N, K/8]")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype or x.dtype, device=x.device)
    ldy = y.stride(0) if y.dim() == 2 else N
    st = lib().awq_w4a16_gemm_noalloc(_ptr(x), _DT.get(x.dtype, -1), M, K, ldx, _ptr(qweight),
                                      _ptr(scales), _ptr(zeros), N, group_size, _ptr(inv_s), _ptr(y),
                                      _DT.get(y.dtype, -1), ldy, _stream(x.device, stream))
    _abi.check("awq_w4a16_gemm_noalloc", st)
    return y


def awq_read_stream(buf: torch.Tensor, blocks: int, unroll: int = 4, block_xor: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """A plain streaming read of buf's bytes (a multiple of 1024); returns the
    per-block XOR of the 32-bit words read (int32 [blocks]).  The rate the
    products are measured against."""
    _dev(buf, "buf")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if block_xor is None:
        block_xor = torch.empty(blocks, dtype=torch.int32, device=buf.device)
    st = lib().awq_read_stream(_ptr(buf), buf.numel() * buf.element_size(), blocks, unroll,
                               _ptr(block_xor), _stream(buf.device, stream))
    _abi.check("awq_read_stream", st)
    return block_xor


def awq_fold_scales(v: torch.Tensor, s: torch.Tensor, axis: int = 1, stream=None) -> torch.Tensor:
    """In place: v[i][j] /= s[j] (axis 1) or s[i] (axis 0); a 1-D v is one row."""
    _dev(v, "v")
    _dev(s, "s")
    if s.dtype != torch.float32 or s.dim() != 1 or not s.is_contiguous():
        raise ValueError("s must be a contiguous float32 vector")
    v2 = v.view(1, -1) if v.dim() == 1 else v
    rows, cols, ld = _rows(v2, "v")
    if s.numel() != (cols if axis == 1 else rows):
        raise ValueError("s must have one entry per column (axis 1) or per row (axis 0)")
    st = lib().awq_fold_scales(_ptr(v2), _DT.get(v.dtype, -1), rows, cols, ld, _ptr(s), axis,
                               _stream(v.device, stream))
    _abi.check("awq_fold_scales", st)
    return v
