"""ctypes loader of libsvdq.so: signatures of the C ABI declared in include/svdq.h.

The library is loaded from this package directory (built in-tree by
``bit_diffusion_transformer_svdq_amd.build``).  A missing or unloadable library
is an error: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsvdq.so")

SUCCESS, INVALID_VALUE, NOT_SUPPORTED, ARCH_MISMATCH, NO_DEVICE, HIP_ERROR, INTERNAL = range(7)

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_size = ctypes.c_size_t

# name -> (restype, argtypes), in the order of include/svdq.h
SIGNATURES = {
    "svdq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "svdq_last_error": (ctypes.c_char_p, []),
    "svdq_version": (ctypes.c_int, []),
    "svdq_check_device": (ctypes.c_int, [ctypes.c_int]),
    "svdq_quantize_act_lora_down": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i64,
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_quantize_act_workspace_size": (_size, [_i64, _i64, _i64]),
    "svdq_debug_set_quant_plan": (ctypes.c_int, [ctypes.c_int, ctypes.c_int]),
    "svdq_debug_set_quant_waves": (ctypes.c_int, [ctypes.c_int]),
    "svdq_debug_set_gemm_path": (ctypes.c_int, [ctypes.c_int]),
    "svdq_debug_set_gemm_splits": (ctypes.c_int, [ctypes.c_int]),
    "svdq_debug_set_fp4_tile": (ctypes.c_int, [ctypes.c_int]),
    "svdq_w4a4_gemm_lora_up": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
        _i64, _i64, _i64, _i64, _i64, _c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_w4a4_gemm_workspace_size": (_size, [_i64, _i64, _i64, _i64]),
    "svdq_w4a4_gemm_lora_up_ex": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
        _i64, _i64, _i64, _i64, _i64, ctypes.c_int, _c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_w4a4_gemm_lora_up_noalloc": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
        _i64, _i64, _i64, _i64, _i64, ctypes.c_int, _c_void_p, _c_void_p]),
    "svdq_w4a4_gemm_qkv_norm_rope": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
        _i64, _i64, _i64, _i64, _i64, _i64, _c_void_p, _c_void_p, ctypes.c_float,
        _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "svdq_quantize_act_lora_down_fp4": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
        _c_void_p, _size, _c_void_p]),
    "svdq_fp4_gemm_lora_up": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
        _i64, _i64, _i64, _i64, ctypes.c_int, _c_void_p, _c_void_p, _size, _c_void_p]),
    "svdq_fp4_gemm_workspace_size": (_size, [_i64, _i64, _i64, _i64]),
    "svdq_awq_w4a16_gemm": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i64,
        _c_void_p, _c_void_p]),
    "svdq_awq_w4a16_gemm_stacked": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _i64, _i64,
        _c_void_p, _c_void_p]),
    "svdq_w4a4_group_acc_debug": (ctypes.c_int, [
        _c_void_p, _c_void_p, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _c_void_p, _c_void_p]),
    "svdq_smooth_from_absmax": (ctypes.c_int, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p]),
    "svdq_pack_weights": (ctypes.c_int, [
        _c_void_p, _c_void_p, _i64, _i64, _i64, _i64, _u64,
        _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "svdq_pack_weights_fp4": (ctypes.c_int, [
        _c_void_p, _c_void_p, _i64, _i64, _i64, _u64, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "svdq_awq_pack_weights": (ctypes.c_int, [
        _c_void_p, _c_void_p, _i64, _i64, _i64, _i64, ctypes.c_int, _c_void_p, _c_void_p, _c_void_p,
        _c_void_p, _c_void_p]),
}

_lib = None
_lock = threading.Lock()


class SvdqError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(message)


def lib() -> ctypes.CDLL:
    """Load libsvdq.so once; raises if it is missing (build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m bit_diffusion_transformer_svdq_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def check(status: int, what: str) -> None:
    """Raise SvdqError with the library's message on a non-success status."""
    if status != SUCCESS:
        L = lib()
        name = L.svdq_status_string(status).decode()
        msg = L.svdq_last_error().decode()
        raise SvdqError(status, f"{what}: {name}: {msg}")
