"""MI355X-native SVDQuant W4A4 + low-rank linear.

Thin Python binding over libsvdq.so (C ABI: include/svdq.h).  Every step of
the hot path runs in the library's HIP kernels; this module only marshals
arguments: it checks dtypes, shapes and devices of inputs and of caller-given
outputs, allocates outputs and device workspaces with torch on the current
device, and passes raw pointers and the current HIP stream.

Workspaces.  Calls 1 and 2 may need a device workspace (the C ABI's
svdq_*_workspace_size).  Pass ``workspace=`` (a zero-filled uint8 device
tensor, reused across calls ordered on one stream) or let the binding keep one
per (device, stream): it is allocated zero-filled by torch on first need and
replaced by a larger one when a call needs more.  A replaced buffer stays
alive until ``release_workspaces()``, because a HIP graph captured earlier may
still point at it.  While the stream is being captured the binding never
allocates: make one eager call of the largest shape before capturing.

Two online calls (the charmloop.ai news item on Nunchaku in Diffusers,
paragraph on the 16-bit branch, names the two fusions):

    codes, scales, lora_act = quantize_act_lora_down(x, smooth, lora_down)
    y = w4a4_gemm_lora_up(codes, scales, w_codes, w_scales, lora_act, lora_up, bias)

and the offline host packer (``smooth_from_absmax``, ``pack_weights``).
"""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import SvdqError, check, lib

__all__ = ["SvdqError", "lib", "check_device", "quantize_act_lora_down", "w4a4_gemm_lora_up",
           "mlp_pair", "w4a4_gemm_lora_up_noalloc", "w4a4_gemm_qkv_norm_rope", "w4a4_group_acc_debug", "debug_set_quant_plan", "debug_set_quant_waves", "debug_set_gemm_path", "debug_set_gemm_splits",
           "debug_set_fp4_tile",
           "EPILOGUES", "smooth_from_absmax", "pack_weights", "awq_w4a16_gemm", "awq_w4a16_gemm_stacked",
           "awq_pack_weights",
           "quantize_act_lora_down_fp4", "fp4_gemm_lora_up", "pack_weights_fp4",
           "release_workspaces", "GROUP_SIZE"]

GROUP_SIZE = 64


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, shape, name):
    torch = _torch()
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() and t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    del torch


def _need_out(t, dtype, shape, device, name):
    """A caller-given output: exact dtype and shape, contiguous, on the inputs' device."""
    _need(t, dtype, shape, name)
    if t.numel() and t.device != device:
        raise ValueError(f"{name}: must be on {device}, got {t.device}")


_WS: dict = {}        # (device index, stream handle) -> zero-filled uint8 tensor
_WS_RETIRED: list = []


def release_workspaces() -> None:
    """Drop the binding's cached workspaces (and the replaced ones kept for
    graphs captured earlier); later calls allocate afresh."""
    _WS.clear()
    _WS_RETIRED.clear()


def _workspace(need: int, device, stream, given):
    """(pointer, bytes) of a workspace of at least `need` bytes for a call on `stream`."""
    torch = _torch()
    if given is not None:
        if given.dtype != torch.uint8 or not given.is_contiguous() or given.device != device:
            raise ValueError("workspace: must be a contiguous uint8 tensor on the call's device")
        return ctypes.c_void_p(given.data_ptr()), given.numel()
    if need == 0:
        return None, 0
    s = torch.cuda.current_stream(device) if stream is None else stream
    key = (device.index, s.cuda_stream)
    buf = _WS.get(key)
    if buf is None or buf.numel() < need:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(f"the call needs a workspace of {need} bytes and the stream is being "
                               "captured: make one eager call of this shape before capturing")
        with torch.cuda.stream(s):
            nb = max(need + need // 4, 0 if buf is None else buf.numel())
            new = torch.zeros(nb, dtype=torch.uint8, device=device)
        if buf is not None:
            _WS_RETIRED.append(buf)
        _WS[key] = buf = new
    return ctypes.c_void_p(buf.data_ptr()), buf.numel()


def check_device(device: int = 0) -> None:
    """Raise unless HIP device ``device`` is a gfx950."""
    check(lib().svdq_check_device(int(device)), "svdq_check_device")


def quantize_act_lora_down(x, smooth, lora_down=None, out=None, stream=None, workspace=None):
    """Call 1: smoothing + int4 quantization + packing + fused lora_down.

    x bf16 [M, K], smooth fp32 [K], lora_down bf16 [r, K] or None (r = 0).
    Returns (act_codes uint8 [M, K/2], act_scales bf16 [M, K/64], lora_act bf16 [M, r]).
    """
    torch = _torch()
    M, K = x.shape
    r = 0 if lora_down is None else lora_down.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(smooth, torch.float32, (K,), "smooth")
    if r:
        _need(lora_down, torch.bfloat16, (r, K), "lora_down")
    dev = x.device
    if out is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((M, K // GROUP_SIZE), dtype=torch.bfloat16, device=dev)
        lora_act = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    else:
        codes, scales, lora_act = out
        _need_out(codes, torch.uint8, (M, K // 2), dev, "act_codes")
        _need_out(scales, torch.bfloat16, (M, K // GROUP_SIZE), dev, "act_scales")
        _need_out(lora_act, torch.bfloat16, (M, r), dev, "lora_act")
    ws, wsb = _workspace(lib().svdq_quantize_act_workspace_size(M, K, r), dev, stream, workspace)
    st = lib().svdq_quantize_act_lora_down(
        _ptr(x), _ptr(smooth), _ptr(lora_down) if r else None, M, K, r, GROUP_SIZE,
        _ptr(codes), _ptr(scales), _ptr(lora_act) if r else None, ws, wsb, _stream(stream))
    check(st, "svdq_quantize_act_lora_down")
    return codes, scales, lora_act


def debug_set_quant_plan(k_blocks: int = 0, tiles_per_wg: int = 0) -> None:
    """Test hook: force call 1's work split for later calls (0 = automatic)."""
    check(lib().svdq_debug_set_quant_plan(int(k_blocks), int(tiles_per_wg)), "svdq_debug_set_quant_plan")


def debug_set_quant_waves(waves: int = 0) -> None:
    """Test hook: call 1's kernel (0 by shape, 1 one wave per row tile, 2..8 the
    row-tile kernel with that many waves per K-block)."""
    check(lib().svdq_debug_set_quant_waves(int(waves)), "svdq_debug_set_quant_waves")


def debug_set_gemm_path(path: int = 0) -> None:
    """Test hook: 0 = kernel chosen by shape, 1 = tiled kernel, 2 = K-split (few-token) kernel."""
    check(lib().svdq_debug_set_gemm_path(int(path)), "svdq_debug_set_gemm_path")


def debug_set_gemm_splits(splits: int = 0) -> None:
    """Test hook: K-splits per tile of the tiled kernel (0 = chosen by shape)."""
    check(lib().svdq_debug_set_gemm_splits(int(splits)), "svdq_debug_set_gemm_splits")


def debug_set_fp4_tile(tile: int = 0) -> None:
    """Test hook: output tile edge of the MXFP4 GEMM (0 = chosen by shape, 128, 256)."""
    check(lib().svdq_debug_set_fp4_tile(int(tile)), "svdq_debug_set_fp4_tile")


EPILOGUES = {"none": 0, "gelu_tanh": 1}


def _out_y(out, M, N, device, lead=()):
    torch = _torch()
    if out is None:
        return torch.empty((*lead, M, N), dtype=torch.bfloat16, device=device)
    _need_out(out, torch.bfloat16, (*lead, M, N), device, "y")
    return out


def w4a4_gemm_lora_up(act_codes, act_scales, w_codes, w_scales, lora_act=None, lora_up=None,
                      bias=None, out=None, stream=None, epilogue="none", workspace=None):
    """Call 2: W4A4 GEMM + per-group dequant + fused lora_up + bias -> Y bf16 [M, N].

    epilogue "gelu_tanh" applies GELU (tanh form) to y + b before the rounding.
    """
    torch = _torch()
    M = act_codes.shape[0]
    K = act_codes.shape[1] * 2
    N = w_codes.shape[0]
    r = 0 if lora_up is None else lora_up.shape[1]
    _need(act_codes, torch.uint8, (M, K // 2), "act_codes")
    _need(act_scales, torch.bfloat16, (M, K // GROUP_SIZE), "act_scales")
    _need(w_codes, torch.uint8, (N, K // 2), "w_codes")
    _need(w_scales, torch.bfloat16, (N, K // GROUP_SIZE), "w_scales")
    if r:
        _need(lora_act, torch.bfloat16, (M, r), "lora_act")
        _need(lora_up, torch.bfloat16, (N, r), "lora_up")
    if bias is not None:
        _need(bias, torch.bfloat16, (N,), "bias")
    dev = act_codes.device
    y = _out_y(out, M, N, dev)
    ws, wsb = _workspace(lib().svdq_w4a4_gemm_workspace_size(M, N, K, r), dev, stream, workspace)
    st = lib().svdq_w4a4_gemm_lora_up_ex(
        _ptr(act_codes), _ptr(act_scales), _ptr(w_codes), _ptr(w_scales),
        _ptr(lora_act) if r else None, _ptr(lora_up) if r else None, _ptr(bias),
        M, N, K, r, GROUP_SIZE, EPILOGUES[epilogue], _ptr(y), ws, wsb, _stream(stream))
    check(st, "svdq_w4a4_gemm_lora_up_ex")
    return y


def w4a4_gemm_lora_up_noalloc(act_codes, act_scales, w_codes, w_scales, lora_act=None, lora_up=None,
                              bias=None, out=None, stream=None, epilogue="none"):
    """Call 2 through the library's fixed device scratch: no workspace and no
    allocation by the library (``out`` must then be given by a caller that may
    not allocate either).  Calls on one device must not overlap in time."""
    torch = _torch()
    M = act_codes.shape[0]
    K = act_codes.shape[1] * 2
    N = w_codes.shape[0]
    r = 0 if lora_up is None else lora_up.shape[1]
    _need(act_codes, torch.uint8, (M, K // 2), "act_codes")
    _need(act_scales, torch.bfloat16, (M, K // GROUP_SIZE), "act_scales")
    _need(w_codes, torch.uint8, (N, K // 2), "w_codes")
    _need(w_scales, torch.bfloat16, (N, K // GROUP_SIZE), "w_scales")
    if r:
        _need(lora_act, torch.bfloat16, (M, r), "lora_act")
        _need(lora_up, torch.bfloat16, (N, r), "lora_up")
    if bias is not None:
        _need(bias, torch.bfloat16, (N,), "bias")
    y = _out_y(out, M, N, act_codes.device)
    st = lib().svdq_w4a4_gemm_lora_up_noalloc(
        _ptr(act_codes), _ptr(act_scales), _ptr(w_codes), _ptr(w_scales),
        _ptr(lora_act) if r else None, _ptr(lora_up) if r else None, _ptr(bias),
        M, N, K, r, GROUP_SIZE, EPILOGUES[epilogue], _ptr(y), _stream(stream))
    check(st, "svdq_w4a4_gemm_lora_up_noalloc")
    return y


def w4a4_gemm_qkv_norm_rope(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias,
                            q_norm, k_norm, rope_cos, rope_sin, eps=1e-6, head_dim=128, out=None,
                            stream=None):
    """Call 2 with the fused QKV epilogue -> bf16 [M, N] = [Q | K | V]: per-head
    RMSNorm (scales q_norm / k_norm, bf16 [head_dim]) and the rotary turn of
    adjacent channel pairs (rope_cos / rope_sin fp32 [M, head_dim/2]) on Q and
    K; V as in call 2."""
    torch = _torch()
    M = act_codes.shape[0]
    K = act_codes.shape[1] * 2
    N = w_codes.shape[0]
    r = 0 if lora_up is None else lora_up.shape[1]
    _need(act_codes, torch.uint8, (M, K // 2), "act_codes")
    _need(act_scales, torch.bfloat16, (M, K // GROUP_SIZE), "act_scales")
    _need(w_codes, torch.uint8, (N, K // 2), "w_codes")
    _need(w_scales, torch.bfloat16, (N, K // GROUP_SIZE), "w_scales")
    if r:
        _need(lora_act, torch.bfloat16, (M, r), "lora_act")
        _need(lora_up, torch.bfloat16, (N, r), "lora_up")
    if bias is not None:
        _need(bias, torch.bfloat16, (N,), "bias")
    _need(q_norm, torch.bfloat16, (head_dim,), "q_norm")
    _need(k_norm, torch.bfloat16, (head_dim,), "k_norm")
    _need(rope_cos, torch.float32, (M, head_dim // 2), "rope_cos")
    _need(rope_sin, torch.float32, (M, head_dim // 2), "rope_sin")
    y = _out_y(out, M, N, act_codes.device)
    st = lib().svdq_w4a4_gemm_qkv_norm_rope(
        _ptr(act_codes), _ptr(act_scales), _ptr(w_codes), _ptr(w_scales),
        _ptr(lora_act) if r else None, _ptr(lora_up) if r else None, _ptr(bias),
        M, N, K, r, GROUP_SIZE, int(head_dim), _ptr(q_norm), _ptr(k_norm), float(eps),
        _ptr(rope_cos), _ptr(rope_sin), _ptr(y), _stream(stream))
    check(st, "svdq_w4a4_gemm_qkv_norm_rope")
    return y


def mlp_pair(x, up: dict, down: dict, h_out=None, out=None, stream=None):
    """An MLP pair on one stream: the up-projection (calls 1 and 2) with the GELU
    epilogue writes H bf16 [M, N_up], which stays in device memory as the input
    of the down-projection (calls 1 and 2 again).

    ``up`` and ``down`` hold the packed layer as device tensors: smooth,
    lora_down (or None), w_codes, w_scales, lora_up (or None), bias (or None).
    Returns (y bf16 [M, N_down], h)."""
    codes, scales, la = quantize_act_lora_down(x, up["smooth"], up["lora_down"], stream=stream)
    h = w4a4_gemm_lora_up(codes, scales, up["w_codes"], up["w_scales"], la if up["lora_up"] is not None
                          else None, up["lora_up"], up["bias"], out=h_out, stream=stream,
                          epilogue="gelu_tanh")
    codes, scales, la = quantize_act_lora_down(h, down["smooth"], down["lora_down"], stream=stream)
    y = w4a4_gemm_lora_up(codes, scales, down["w_codes"], down["w_scales"], la if down["lora_up"] is not None
                          else None, down["lora_up"], down["bias"], out=out, stream=stream)
    return y, h


def w4a4_group_acc_debug(act_codes, w_codes, rows=None, cols=None, stream=None):
    """Test hook: the exact int32 group accumulators of call 2's main loop for the
    window rows = (m0, mc), cols = (n0, nc) (default: everything) -> [mc, nc, K/64]."""
    torch = _torch()
    M = act_codes.shape[0]
    K = act_codes.shape[1] * 2
    N = w_codes.shape[0]
    _need(act_codes, torch.uint8, (M, K // 2), "act_codes")
    _need(w_codes, torch.uint8, (N, K // 2), "w_codes")
    m0, mc = (0, M) if rows is None else rows
    n0, nc = (0, N) if cols is None else cols
    acc = torch.empty((max(mc, 0), max(nc, 0), K // GROUP_SIZE), dtype=torch.int32, device=act_codes.device)
    st = lib().svdq_w4a4_group_acc_debug(_ptr(act_codes), _ptr(w_codes), M, N, K, m0, mc, n0, nc,
                                         _ptr(acc), _stream(stream))
    check(st, "svdq_w4a4_group_acc_debug")
    return acc


def quantize_act_lora_down_fp4(x, smooth, lora_down=None, out=None, stream=None, workspace=None):
    """Call 1, FP4 variant: -> (act_codes u8 [M, K/2] E2M1, act_scales u8 [M, K/32] E8M0,
    lora_act bf16 [M, r])."""
    torch = _torch()
    M, K = x.shape
    r = 0 if lora_down is None else lora_down.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(smooth, torch.float32, (K,), "smooth")
    if r:
        _need(lora_down, torch.bfloat16, (r, K), "lora_down")
    if out is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
        lora_act = torch.empty((M, r), dtype=torch.bfloat16, device=x.device)
    else:
        codes, scales, lora_act = out
        _need_out(codes, torch.uint8, (M, K // 2), x.device, "act_codes")
        _need_out(scales, torch.uint8, (M, K // 32), x.device, "act_scales")
        _need_out(lora_act, torch.bfloat16, (M, r), x.device, "lora_act")
    ws, wsb = _workspace(lib().svdq_quantize_act_workspace_size(M, K, r), x.device, stream, workspace)
    st = lib().svdq_quantize_act_lora_down_fp4(_ptr(x), _ptr(smooth), _ptr(lora_down) if r else None, M, K, r,
                                                _ptr(codes), _ptr(scales), _ptr(lora_act) if r else None,
                                                ws, wsb, _stream(stream))
    check(st, "svdq_quantize_act_lora_down_fp4")
    return codes, scales, lora_act


def fp4_gemm_lora_up(act_codes, act_scales, w_codes, w_scales, lora_act=None, lora_up=None, bias=None,
                     out=None, stream=None, epilogue="none", workspace=None):
    """Call 2, FP4 variant: MXFP4 GEMM (block scales in the matrix core) + lora_up + bias -> Y bf16."""
    torch = _torch()
    M = act_codes.shape[0]
    K = act_codes.shape[1] * 2
    N = w_codes.shape[0]
    r = 0 if lora_up is None else lora_up.shape[1]
    _need(act_codes, torch.uint8, (M, K // 2), "act_codes")
    _need(act_scales, torch.uint8, (M, K // 32), "act_scales")
    _need(w_codes, torch.uint8, (N, K // 2), "w_codes")
    _need(w_scales, torch.uint8, (N, K // 32), "w_scales")
    if r:
        _need(lora_act, torch.bfloat16, (M, r), "lora_act")
        _need(lora_up, torch.bfloat16, (N, r), "lora_up")
    if bias is not None:
        _need(bias, torch.bfloat16, (N,), "bias")
    y = _out_y(out, M, N, act_codes.device)
    ws, wsb = _workspace(lib().svdq_fp4_gemm_workspace_size(M, N, K, r), act_codes.device, stream, workspace)
    st = lib().svdq_fp4_gemm_lora_up(_ptr(act_codes), _ptr(act_scales), _ptr(w_codes), _ptr(w_scales),
                                     _ptr(lora_act) if r else None, _ptr(lora_up) if r else None, _ptr(bias),
                                     M, N, K, r, EPILOGUES[epilogue], _ptr(y), ws, wsb, _stream(stream))
    check(st, "svdq_fp4_gemm_lora_up")
    return y


def pack_weights_fp4(w_bf16: np.ndarray, smooth: np.ndarray, rank: int, seed: int = 0) -> dict:
    """Host packer, FP4 variant: -> w_codes u8 [N, K/2], w_scales u8 [N, K/32] (E8M0),
    lora_down, lora_up (bf16 bits)."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    lam = np.ascontiguousarray(smooth, dtype=np.float32)
    N, K = w.shape
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 32), dtype=np.uint8)
    down = np.empty((rank, K), dtype=np.uint16)
    up = np.empty((N, rank), dtype=np.uint16)
    vp = ctypes.c_void_p
    st = lib().svdq_pack_weights_fp4(w.ctypes.data_as(vp), lam.ctypes.data_as(vp), N, K, int(rank), int(seed),
                                     codes.ctypes.data_as(vp), scales.ctypes.data_as(vp),
                                     down.ctypes.data_as(vp) if rank else None,
                                     up.ctypes.data_as(vp) if rank else None)
    check(st, "svdq_pack_weights_fp4")
    return {"w_codes": codes, "w_scales": scales, "lora_down": down, "lora_up": up}


def awq_w4a16_gemm(x, smooth, w_codes, w_scales, w_zeros, bias=None, out=None, stream=None):
    """AWQ W4A16 linear: x bf16 [M, K], smooth fp32 [K], codes u8 [N, K/2], scales bf16 [N, K/64],
    zeros u8 [N, K/64], bias bf16 [N] or None -> Y bf16 [M, N]."""
    torch = _torch()
    M, K = x.shape
    N = w_codes.shape[0]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(smooth, torch.float32, (K,), "smooth")
    _need(w_codes, torch.uint8, (N, K // 2), "w_codes")
    _need(w_scales, torch.bfloat16, (N, K // GROUP_SIZE), "w_scales")
    _need(w_zeros, torch.uint8, (N, K // GROUP_SIZE), "w_zeros")
    if bias is not None:
        _need(bias, torch.bfloat16, (N,), "bias")
    y = _out_y(out, M, N, x.device)
    st = lib().svdq_awq_w4a16_gemm(_ptr(x), _ptr(smooth), _ptr(w_codes), _ptr(w_scales), _ptr(w_zeros),
                                   _ptr(bias), M, N, K, GROUP_SIZE, _ptr(y), _stream(stream))
    check(st, "svdq_awq_w4a16_gemm")
    return y


def awq_w4a16_gemm_stacked(x, smooth, w_codes, w_scales, w_zeros, bias=None, out=None, stream=None):
    """L AWQ W4A16 linears sharing x: x bf16 [M, K], smooth fp32 [L, K], codes u8 [L, N, K/2],
    scales bf16 [L, N, K/64], zeros u8 [L, N, K/64], bias bf16 [L, N] or None -> Y bf16 [L, M, N]."""
    torch = _torch()
    M, K = x.shape
    L, N = w_codes.shape[0], w_codes.shape[1]
    _need(x, torch.bfloat16, (M, K), "x")
    _need(smooth, torch.float32, (L, K), "smooth")
    _need(w_codes, torch.uint8, (L, N, K // 2), "w_codes")
    _need(w_scales, torch.bfloat16, (L, N, K // GROUP_SIZE), "w_scales")
    _need(w_zeros, torch.uint8, (L, N, K // GROUP_SIZE), "w_zeros")
    if bias is not None:
        _need(bias, torch.bfloat16, (L, N), "bias")
    y = _out_y(out, M, N, x.device, lead=(L,))
    st = lib().svdq_awq_w4a16_gemm_stacked(_ptr(x), _ptr(smooth), _ptr(w_codes), _ptr(w_scales), _ptr(w_zeros),
                                           _ptr(bias), L, M, N, K, GROUP_SIZE, _ptr(y), _stream(stream))
    check(st, "svdq_awq_w4a16_gemm_stacked")
    return y


def awq_pack_weights(w_bf16: np.ndarray, x_calib_bf16: np.ndarray, n_grid: int = 20) -> dict:
    """Host AWQ packer: W bf16 bits [N, K] + calibration activations bf16 bits [Mc, K] ->
    smooth fp32 [K], codes u8 [N, K/2], scales (bf16 bits) [N, K/64], zeros u8 [N, K/64], alpha."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    xc = np.ascontiguousarray(x_calib_bf16, dtype=np.uint16)
    N, K = w.shape
    Mc = xc.shape[0]
    smooth = np.empty(K, dtype=np.float32)
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // GROUP_SIZE), dtype=np.uint16)
    zeros = np.empty((N, K // GROUP_SIZE), dtype=np.uint8)
    alpha = ctypes.c_float(0.0)
    vp = ctypes.c_void_p
    st = lib().svdq_awq_pack_weights(w.ctypes.data_as(vp), xc.ctypes.data_as(vp), Mc, N, K, GROUP_SIZE,
                                     int(n_grid), smooth.ctypes.data_as(vp), codes.ctypes.data_as(vp),
                                     scales.ctypes.data_as(vp), zeros.ctypes.data_as(vp),
                                     ctypes.cast(ctypes.pointer(alpha), vp))
    check(st, "svdq_awq_pack_weights")
    return {"smooth": smooth, "codes": codes, "scales": scales, "zeros": zeros, "alpha": float(alpha.value)}


def smooth_from_absmax(x_absmax: np.ndarray, w_bf16: np.ndarray) -> np.ndarray:
    """Host packer step 1: lambda (fp32 [K]) from activation absmax fp32 [K] and W bf16 bits [N, K]."""
    a = np.ascontiguousarray(x_absmax, dtype=np.float32)
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    N, K = w.shape
    out = np.empty(K, dtype=np.float32)
    st = lib().svdq_smooth_from_absmax(a.ctypes.data_as(ctypes.c_void_p), w.ctypes.data_as(ctypes.c_void_p),
                                       N, K, out.ctypes.data_as(ctypes.c_void_p))
    check(st, "svdq_smooth_from_absmax")
    return out


def pack_weights(w_bf16: np.ndarray, smooth: np.ndarray, rank: int, seed: int = 0) -> dict:
    """Host packer step 2: W bf16 bits [N, K] + lambda -> packed residual and low-rank factors.

    Returns numpy arrays: w_codes uint8 [N, K/2], w_scales uint16 (bf16 bits) [N, K/64],
    lora_down uint16 [r, K], lora_up uint16 [N, r].
    """
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    lam = np.ascontiguousarray(smooth, dtype=np.float32)
    N, K = w.shape
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // GROUP_SIZE), dtype=np.uint16)
    down = np.empty((rank, K), dtype=np.uint16)
    up = np.empty((N, rank), dtype=np.uint16)
    vp = ctypes.c_void_p
    st = lib().svdq_pack_weights(
        w.ctypes.data_as(vp), lam.ctypes.data_as(vp), N, K, int(rank), GROUP_SIZE, int(seed),
        codes.ctypes.data_as(vp), scales.ctypes.data_as(vp),
        down.ctypes.data_as(vp) if rank else None, up.ctypes.data_as(vp) if rank else None)
    check(st, "svdq_pack_weights")
    return {"w_codes": codes, "w_scales": scales, "lora_down": down, "lora_up": up}
