"""C ABI checks that need no GPU: exports, status strings, argument validation.

Argument errors must be reported before any HIP call, so they are testable on a
machine without a GPU; a well-formed call there must report NO_DEVICE rather
than crash.
"""
import ctypes
import os
import re
import subprocess

import pytest

from bit_diffusion_transformer_svdq_amd import _lib
from bit_diffusion_transformer_svdq_amd._lib import (ARCH_MISMATCH, INVALID_VALUE, NO_DEVICE,
                                                     NOT_SUPPORTED, SUCCESS, lib)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")
FAKE = ctypes.c_void_p(0x10000)     # non-null, 16-byte aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x10008)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svdq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    names = _declared_functions()
    for must in ("svdq_quantize_act_lora_down", "svdq_w4a4_gemm_lora_up", "svdq_pack_weights",
                 "svdq_smooth_from_absmax", "svdq_check_device", "svdq_w4a4_group_acc_debug"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = lib()
    names = _declared_functions()
    assert set(names) == set(_lib.SIGNATURES)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(svdq_\w+)", out))
    assert set(names) <= exported


def test_status_strings_and_version():
    L = lib()
    assert L.svdq_status_string(SUCCESS) == b"SVDQ_STATUS_SUCCESS"
    assert L.svdq_status_string(NOT_SUPPORTED) == b"SVDQ_STATUS_NOT_SUPPORTED"
    assert L.svdq_status_string(99) == b"SVDQ_STATUS_UNKNOWN"
    assert L.svdq_version() >= 100


def _quant(**kw):
    a = dict(x=FAKE, smooth=FAKE, lora_down=FAKE, M=64, K=256, r=16, g=64,
             codes=FAKE, scales=FAKE, la=FAKE, stream=None)
    a.update(kw)
    return lib().svdq_quantize_act_lora_down(a["x"], a["smooth"], a["lora_down"], a["M"], a["K"], a["r"],
                                             a["g"], a["codes"], a["scales"], a["la"], a["stream"])


def _gemm(**kw):
    a = dict(ac=FAKE, asc=FAKE, wc=FAKE, ws=FAKE, la=FAKE, lu=FAKE, bias=FAKE, M=64, N=256, K=256,
             r=16, g=64, y=FAKE, stream=None)
    a.update(kw)
    return lib().svdq_w4a4_gemm_lora_up(a["ac"], a["asc"], a["wc"], a["ws"], a["la"], a["lu"], a["bias"],
                                        a["M"], a["N"], a["K"], a["r"], a["g"], a["y"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID_VALUE),
    (dict(smooth=None), INVALID_VALUE),
    (dict(codes=None), INVALID_VALUE),
    (dict(scales=None), INVALID_VALUE),
    (dict(lora_down=None), INVALID_VALUE),
    (dict(la=None), INVALID_VALUE),
    (dict(M=-1), INVALID_VALUE),
    (dict(K=0), INVALID_VALUE),
    (dict(K=96), NOT_SUPPORTED),
    (dict(g=32), NOT_SUPPORTED),
    (dict(r=8), NOT_SUPPORTED),
    (dict(r=144), NOT_SUPPORTED),
    (dict(x=FAKE_ODD), INVALID_VALUE),
    (dict(M=0), SUCCESS),                       # empty batch: a no-op
    (dict(r=0, lora_down=None, la=None, M=0), SUCCESS),
    (dict(M=0, x=None, codes=None, scales=None), SUCCESS),   # empty tensors may be null
    (dict(M=0, K=96), NOT_SUPPORTED),           # dimensions are still validated
])
def test_quantize_argument_errors(kw, status):
    assert _quant(**kw) == status
    if status != SUCCESS:
        assert len(lib().svdq_last_error()) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(ac=None), INVALID_VALUE),
    (dict(wc=None), INVALID_VALUE),
    (dict(asc=None), INVALID_VALUE),
    (dict(ws=None), INVALID_VALUE),
    (dict(y=None), INVALID_VALUE),
    (dict(la=None), INVALID_VALUE),
    (dict(lu=None), INVALID_VALUE),
    (dict(N=96), NOT_SUPPORTED),
    (dict(N=0), INVALID_VALUE),
    (dict(K=100), NOT_SUPPORTED),
    (dict(r=20), NOT_SUPPORTED),
    (dict(g=128), NOT_SUPPORTED),
    (dict(bias=FAKE_ODD), INVALID_VALUE),
    (dict(M=0), SUCCESS),
    (dict(M=0, bias=None, r=0, la=None, lu=None), SUCCESS),
    (dict(M=0, ac=None, asc=None, la=None, y=None), SUCCESS),
    (dict(M=0, N=96), NOT_SUPPORTED),
])
def test_gemm_argument_errors(kw, status):
    assert _gemm(**kw) == status


def test_gemm_epilogue_argument():
    """The _ex entry point accepts the declared epilogues and rejects others
    before any device call; the plain entry point is the no-epilogue case."""
    L = lib()

    def ex(ep, **kw):
        a = dict(M=64)
        a.update(kw)
        return L.svdq_w4a4_gemm_lora_up_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["M"], 256, 256,
                                           16, 64, ep, FAKE, None)
    for bad in (-1, 2, 7):
        assert ex(bad) == INVALID_VALUE
        assert b"epilogue" in L.svdq_last_error()
        assert ex(bad, M=0) == INVALID_VALUE
    for good in (0, 1):
        assert ex(good, M=0) == SUCCESS
        if not _gpu_visible():
            assert ex(good) == NO_DEVICE


def test_qkv_entry_point_argument_errors():
    L = lib()

    def qkv(M=64, N=768, head_dim=128, eps=1e-6, qn=FAKE, cos=FAKE):
        return L.svdq_w4a4_gemm_qkv_norm_rope(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, M, N, 256, 16, 64,
                                              head_dim, qn, FAKE, eps, cos, FAKE, FAKE, None)
    assert qkv(head_dim=64) == NOT_SUPPORTED
    assert qkv(N=512) == NOT_SUPPORTED
    assert qkv(N=96) == NOT_SUPPORTED
    assert qkv(eps=float("nan")) == INVALID_VALUE
    assert qkv(eps=-1.0) == INVALID_VALUE
    assert qkv(qn=None) == INVALID_VALUE
    assert qkv(cos=FAKE_ODD) == INVALID_VALUE
    assert qkv(M=0, qn=None, cos=None) == SUCCESS
    assert qkv(M=0, N=512) == NOT_SUPPORTED
    if not _gpu_visible():
        assert qkv() == NO_DEVICE


def test_awq_entry_points_argument_errors():
    L = lib()

    def awq(M=4, N=64, K=256, g=64, x=FAKE, zeros=FAKE, bias=FAKE):
        return L.svdq_awq_w4a16_gemm(x, FAKE, FAKE, FAKE, zeros, bias, M, N, K, g, FAKE, None)
    assert awq(N=48) == NOT_SUPPORTED
    assert awq(K=96) == NOT_SUPPORTED
    assert awq(g=128) == NOT_SUPPORTED
    assert awq(K=64 * 700) == NOT_SUPPORTED          # x_hat staging beyond the LDS
    assert awq(M=1, K=16384 + 64) == NOT_SUPPORTED
    assert awq(M=5, K=4096 + 64) == NOT_SUPPORTED
    assert awq(M=-1) == INVALID_VALUE
    assert awq(x=None) == INVALID_VALUE
    assert awq(zeros=None) == INVALID_VALUE
    assert awq(bias=FAKE_ODD) == INVALID_VALUE
    assert awq(M=0, x=None, zeros=None) == SUCCESS
    if not _gpu_visible():
        assert awq() == NO_DEVICE
        assert awq(M=1, K=16384) == NO_DEVICE            # the largest staged shapes pass validation
        assert awq(M=4, K=8192) == NO_DEVICE
        assert awq(M=40, K=4096) == NO_DEVICE

    def stacked(Ls=3, M=4, N=64, K=256, g=64, x=FAKE, bias=FAKE):
        return L.svdq_awq_w4a16_gemm_stacked(x, FAKE, FAKE, FAKE, FAKE, bias, Ls, M, N, K, g, FAKE, None)
    assert stacked(Ls=-1) == INVALID_VALUE
    assert stacked(Ls=65536) == NOT_SUPPORTED
    assert stacked(N=48) == NOT_SUPPORTED
    assert stacked(M=5, K=4096 + 64) == NOT_SUPPORTED
    assert stacked(x=None) == INVALID_VALUE
    assert stacked(bias=FAKE_ODD) == INVALID_VALUE
    assert stacked(Ls=0, x=None) == SUCCESS
    assert stacked(M=0, x=None) == SUCCESS
    if not _gpu_visible():
        assert stacked() == NO_DEVICE
        assert stacked(Ls=65535, M=1, K=16384) == NO_DEVICE
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.cast(buf, ctypes.c_void_p)
    assert L.svdq_awq_pack_weights(None, p, 4, 8, 64, 64, 20, p, p, p, p, None) == INVALID_VALUE
    assert L.svdq_awq_pack_weights(p, p, 4, 8, 96, 64, 20, p, p, p, p, None) == NOT_SUPPORTED
    assert L.svdq_awq_pack_weights(p, p, 4, 8, 64, 64, 0, p, p, p, p, None) == INVALID_VALUE


def test_fp4_entry_points_argument_errors():
    L = lib()

    def q(M=64, K=256, r=16, x=FAKE):
        return L.svdq_quantize_act_lora_down_fp4(x, FAKE, FAKE, M, K, r, FAKE, FAKE, FAKE, None)

    def g(M=64, N=256, K=256, r=16, ep=0, asc=FAKE):
        return L.svdq_fp4_gemm_lora_up(FAKE, asc, FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, r, ep, FAKE, None)
    assert q(K=192) == NOT_SUPPORTED and g(K=192) == NOT_SUPPORTED
    assert q(x=None) == INVALID_VALUE and g(asc=None) == INVALID_VALUE
    assert g(ep=2) == INVALID_VALUE and g(N=96) == NOT_SUPPORTED
    assert q(M=0, x=None) == SUCCESS and g(M=0, asc=None) == SUCCESS
    if not _gpu_visible():
        assert q() == NO_DEVICE and g() == NO_DEVICE and g(ep=1) == NO_DEVICE
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.cast(buf, ctypes.c_void_p)
    assert L.svdq_pack_weights_fp4(p, p, 8, 192, 0, 0, p, p, None, None) == NOT_SUPPORTED
    assert L.svdq_pack_weights_fp4(None, p, 8, 128, 0, 0, p, p, None, None) == INVALID_VALUE


def test_debug_hook_argument_errors():
    L = lib()
    assert L.svdq_w4a4_group_acc_debug(FAKE, FAKE, 4, 64, 64, 64, None, None) == INVALID_VALUE
    assert L.svdq_w4a4_group_acc_debug(FAKE, FAKE, 4, 64, 96, 64, FAKE, None) == NOT_SUPPORTED
    assert L.svdq_w4a4_group_acc_debug(FAKE, FAKE, 0, 64, 64, 64, FAKE, None) == SUCCESS


def test_quant_plan_hook_arguments():
    L = lib()
    assert L.svdq_debug_set_quant_plan(-1, 0) == INVALID_VALUE
    assert L.svdq_debug_set_quant_plan(0, -2) == INVALID_VALUE
    assert L.svdq_debug_set_quant_plan(2, 13) == INVALID_VALUE
    assert L.svdq_debug_set_quant_plan(3, 12) == SUCCESS
    assert L.svdq_debug_set_quant_plan(0, 0) == SUCCESS


def test_gemm_path_hook_arguments():
    L = lib()
    assert L.svdq_debug_set_gemm_path(-1) == INVALID_VALUE
    assert L.svdq_debug_set_gemm_path(3) == INVALID_VALUE
    for p in (1, 2, 0):
        assert L.svdq_debug_set_gemm_path(p) == SUCCESS


def test_gemm_splits_hook_arguments():
    L = lib()
    assert L.svdq_debug_set_gemm_splits(-1) == INVALID_VALUE
    assert L.svdq_debug_set_gemm_splits(65) == INVALID_VALUE
    for v in (3, 64, 0):
        assert L.svdq_debug_set_gemm_splits(v) == SUCCESS


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="checks the no-GPU path")
def test_well_formed_calls_without_a_gpu_report_no_device():
    assert lib().svdq_check_device(0) in (NO_DEVICE, ARCH_MISMATCH)
    assert _quant() == NO_DEVICE
    assert _gemm() == NO_DEVICE
    assert lib().svdq_check_device(-1) == INVALID_VALUE


def test_packer_argument_errors():
    L = lib()
    assert L.svdq_pack_weights(None, FAKE, 4, 64, 0, 64, 0, FAKE, FAKE, None, None) == INVALID_VALUE
    assert L.svdq_smooth_from_absmax(None, FAKE, 4, 64, FAKE) == INVALID_VALUE
    import numpy as np
    w = np.zeros((4, 96), np.uint16)
    lam = np.ones(96, np.float32)
    codes = np.zeros((4, 48), np.uint8)
    sc = np.zeros((4, 2), np.uint16)
    vp = ctypes.c_void_p
    st = L.svdq_pack_weights(w.ctypes.data_as(vp), lam.ctypes.data_as(vp), 4, 96, 0, 64, 0,
                             codes.ctypes.data_as(vp), sc.ctypes.data_as(vp), None, None)
    assert st == NOT_SUPPORTED
    w = np.zeros((4, 64), np.uint16)
    lam = np.ones(64, np.float32)
    st = L.svdq_pack_weights(w.ctypes.data_as(vp), lam.ctypes.data_as(vp), 4, 64, 4, 64, 0,
                             codes.ctypes.data_as(vp), sc.ctypes.data_as(vp), None, None)
    assert st == INVALID_VALUE   # r > 0 needs the factor outputs
    st = L.svdq_pack_weights(w.ctypes.data_as(vp), lam.ctypes.data_as(vp), 4, 64, 8, 64, 0,
                             codes.ctypes.data_as(vp), sc.ctypes.data_as(vp), FAKE, FAKE)
    assert st == NOT_SUPPORTED   # rank larger than min(N, K)
