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
# Fake device pointers, never dereferenced: 16-byte aligned and far apart, so
# buffers of any tested size stay disjoint (the entry points reject overlapping
# outputs).  FAKE_ODD is misaligned.
_SPACING = 1 << 40


def P(i: int) -> ctypes.c_void_p:
    return ctypes.c_void_p((i + 1) * _SPACING)


FAKE = P(0)
FAKE_ODD = ctypes.c_void_p(P(30).value + 8)


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
    a = dict(x=P(1), smooth=P(2), lora_down=P(3), M=64, K=256, r=16, g=64,
             codes=P(4), scales=P(5), la=P(6), ws=P(9), wsb=1 << 30, stream=None)
    a.update(kw)
    return lib().svdq_quantize_act_lora_down(a["x"], a["smooth"], a["lora_down"], a["M"], a["K"], a["r"],
                                             a["g"], a["codes"], a["scales"], a["la"], a["ws"], a["wsb"],
                                             a["stream"])


def _gemm(**kw):
    a = dict(ac=P(1), asc=P(2), wc=P(3), ws_=P(4), la=P(5), lu=P(6), bias=P(7), M=64, N=256, K=256,
             r=16, g=64, y=P(8), ws=P(9), wsb=1 << 30, stream=None)
    a.update(kw)
    return lib().svdq_w4a4_gemm_lora_up(a["ac"], a["asc"], a["wc"], a["ws_"], a["la"], a["lu"], a["bias"],
                                        a["M"], a["N"], a["K"], a["r"], a["g"], a["y"], a["ws"], a["wsb"],
                                        a["stream"])


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
    (dict(ws_=None), INVALID_VALUE),
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
        return L.svdq_w4a4_gemm_lora_up_ex(P(1), P(2), P(3), P(4), P(5), P(6), P(7), a["M"], 256, 256,
                                           16, 64, ep, P(8), P(9), 1 << 30, None)
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

    def qkv(M=64, N=768, head_dim=128, eps=1e-6, qn=P(8), cos=P(10), y=P(12)):
        return L.svdq_w4a4_gemm_qkv_norm_rope(P(1), P(2), P(3), P(4), P(5), P(6), P(7), M, N, 256, 16, 64,
                                              head_dim, qn, P(9), eps, cos, P(11), y, None)
    assert qkv(head_dim=64) == NOT_SUPPORTED
    assert qkv(N=512) == NOT_SUPPORTED
    assert qkv(N=96) == NOT_SUPPORTED
    assert qkv(eps=float("nan")) == INVALID_VALUE
    assert qkv(eps=-1.0) == INVALID_VALUE
    assert qkv(qn=None) == INVALID_VALUE
    assert qkv(cos=FAKE_ODD) == INVALID_VALUE
    assert qkv(M=0, qn=None, cos=None) == SUCCESS
    assert qkv(M=0, N=512) == NOT_SUPPORTED
    assert qkv(y=P(10)) == INVALID_VALUE            # output over an input table
    assert b"overlap" in L.svdq_last_error()
    if not _gpu_visible():
        assert qkv() == NO_DEVICE


def test_awq_entry_points_argument_errors():
    L = lib()

    def awq(M=4, N=64, K=256, g=64, x=P(1), zeros=P(5), bias=P(6), y=P(7)):
        return L.svdq_awq_w4a16_gemm(x, P(2), P(3), P(4), zeros, bias, M, N, K, g, y, None)
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
    assert awq(y=P(3)) == INVALID_VALUE                # output over the codes
    if not _gpu_visible():
        assert awq() == NO_DEVICE
        assert awq(M=1, K=16384) == NO_DEVICE            # the largest staged shapes pass validation
        assert awq(M=4, K=8192) == NO_DEVICE
        assert awq(M=40, K=4096) == NO_DEVICE

    def stacked(Ls=3, M=4, N=64, K=256, g=64, x=P(1), bias=P(6)):
        return L.svdq_awq_w4a16_gemm_stacked(x, P(2), P(3), P(4), P(5), bias, Ls, M, N, K, g, P(7), None)
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

    def q(M=64, K=256, r=16, x=P(1)):
        return L.svdq_quantize_act_lora_down_fp4(x, P(2), P(3), M, K, r, P(4), P(5), P(6), P(9), 1 << 30, None)

    def g(M=64, N=256, K=256, r=16, ep=0, asc=P(2)):
        return L.svdq_fp4_gemm_lora_up(P(1), asc, P(3), P(4), P(5), P(6), P(7), M, N, K, r, ep, P(8),
                                       P(9), 1 << 30, None)
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

    def dump(M=4, N=64, K=64, m0=0, mc=4, n0=0, nc=64, acc=P(3), ac=P(1)):
        return L.svdq_w4a4_group_acc_debug(ac, P(2), M, N, K, m0, mc, n0, nc, acc, None)
    assert dump(acc=None) == INVALID_VALUE
    assert dump(K=96) == NOT_SUPPORTED
    assert dump(M=0, mc=0) == SUCCESS
    assert dump(m0=1) == INVALID_VALUE                 # window beyond the rows
    assert dump(n0=60, nc=5) == INVALID_VALUE          # window beyond the columns
    assert dump(mc=-1) == INVALID_VALUE
    assert dump(mc=0) == SUCCESS                       # empty window: nothing to do
    assert dump(acc=P(1)) == INVALID_VALUE             # window output over the codes
    if not _gpu_visible():
        assert dump() == NO_DEVICE
        assert dump(M=100, N=256, m0=37, mc=5, n0=70, nc=3) == NO_DEVICE


def test_quant_plan_hook_arguments():
    L = lib()
    assert L.svdq_debug_set_quant_plan(-1, 0) == INVALID_VALUE
    assert L.svdq_debug_set_quant_plan(0, -2) == INVALID_VALUE
    assert L.svdq_debug_set_quant_plan(2, 13) == INVALID_VALUE
    assert L.svdq_debug_set_quant_plan(3, 12) == SUCCESS
    assert L.svdq_debug_set_quant_plan(0, 0) == SUCCESS
    assert L.svdq_debug_set_quant_waves(-1) == INVALID_VALUE
    assert L.svdq_debug_set_quant_waves(9) == INVALID_VALUE
    assert L.svdq_debug_set_quant_waves(8) == SUCCESS
    assert L.svdq_debug_set_quant_waves(0) == SUCCESS


def test_gemm_path_hook_arguments():
    L = lib()
    assert L.svdq_debug_set_gemm_path(-1) == INVALID_VALUE
    assert L.svdq_debug_set_gemm_path(3) == INVALID_VALUE
    for p in (1, 2, 0):
        assert L.svdq_debug_set_gemm_path(p) == SUCCESS


def test_fp4_tile_hook_arguments():
    L = lib()
    for bad in (-1, 1, 64, 129, 512):
        assert L.svdq_debug_set_fp4_tile(bad) == INVALID_VALUE
    for t in (128, 256, 0):
        assert L.svdq_debug_set_fp4_tile(t) == SUCCESS


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
    # inputs may share memory (only outputs must be disjoint)
    assert _gemm(asc=P(1), wc=P(1)) == NO_DEVICE
    assert _quant(smooth=P(1), lora_down=P(1)) == NO_DEVICE
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


# ---- outputs that overlap, the caller's workspace, size limits ----

@pytest.mark.parametrize("kw", [
    dict(y=P(1)),                                        # Y over the activation codes
    dict(y=ctypes.c_void_p(P(3).value + 4096)),          # Y starting inside the weight codes
    dict(bias=ctypes.c_void_p(P(8).value + 64 * 256 * 2 - 16)),   # bias under Y's last bytes
])
def test_gemm_overlapping_output_is_rejected(kw):
    assert _gemm(**kw) == INVALID_VALUE
    assert b"overlap" in lib().svdq_last_error()


@pytest.mark.parametrize("kw", [
    dict(codes=P(1)),                                    # codes over x
    dict(la=P(5)),                                       # two outputs on one buffer
    dict(scales=ctypes.c_void_p(P(4).value + 64 * 128 - 16)),    # scales overlap the codes' tail
])
def test_quantize_overlapping_outputs_are_rejected(kw):
    assert _quant(**kw) == INVALID_VALUE
    assert b"overlap" in lib().svdq_last_error()


def test_buffers_that_only_touch_are_accepted():
    """codes [64, 128] end exactly where the scales begin: no overlap."""
    if _gpu_visible():
        pytest.skip("checks the no-GPU path")
    assert _quant(scales=ctypes.c_void_p(P(4).value + 64 * 128)) == NO_DEVICE


def test_workspace_size_queries_and_checks():
    L = lib()
    assert L.svdq_w4a4_gemm_workspace_size(4608, 12288, 3072, 32) == 0       # many tiles: no split
    # 864 tiles on the 256 CUs assumed without a device (768 slots): one round
    # runs whole, the last 96 tiles as 2 K-splits each (2 x 4 waves x 16 KB)
    assert L.svdq_w4a4_gemm_workspace_size(4608, 3072, 3072, 32) == (1 << 20) + 96 * 2 * 4 * 16384
    assert L.svdq_w4a4_gemm_workspace_size(0, 256, 256, 16) == 0
    assert L.svdq_w4a4_gemm_workspace_size(64, 96, 256, 16) == 0             # rejected shape
    assert L.svdq_quantize_act_workspace_size(64, 100, 16) == 0
    # MXFP4 on 256 x 256 tiles (864 of them fill every CU): no K-split, no workspace
    assert L.svdq_fp4_gemm_workspace_size(4608, 12288, 3072, 32) == 0
    L.svdq_debug_set_fp4_tile(256)
    try:
        assert L.svdq_fp4_gemm_workspace_size(64, 256, 1024, 16) == 0
    finally:
        L.svdq_debug_set_fp4_tile(0)
    L.svdq_debug_set_gemm_path(1)
    L.svdq_debug_set_gemm_splits(2)
    L.svdq_debug_set_quant_plan(4, 0)
    try:
        need_g = L.svdq_w4a4_gemm_workspace_size(64, 256, 256, 16)
        need_q = L.svdq_quantize_act_workspace_size(64, 256, 16)
        need_f = L.svdq_fp4_gemm_workspace_size(64, 256, 256, 16)
        # the fixed 1 MiB counter region, then 2 tiles x 2 splits x 4 fp32 sub-tiles of 64 x 64
        assert need_g == (1 << 20) + 2 * 2 * 4 * 4096 * 4
        assert need_f == need_g
        # 4 row tiles; partials [4 K-blocks][4 tiles][1][4][64] fp32
        assert need_q == (1 << 20) + 4 * 4 * 1 * 4 * 64 * 4
        assert L.svdq_quantize_act_workspace_size(64, 256, 0) == 0          # rank 0: nothing to reduce
        assert _gemm(ws=None, wsb=0) == INVALID_VALUE and b"workspace" in L.svdq_last_error()
        assert _gemm(ws=P(9), wsb=need_g - 1) == INVALID_VALUE
        assert _gemm(ws=ctypes.c_void_p(P(9).value + 8), wsb=need_g) == INVALID_VALUE   # misaligned
        assert _gemm(ws=ctypes.c_void_p(P(8).value + 1024), wsb=need_g) == INVALID_VALUE  # inside Y
        assert _quant(ws=None, wsb=0) == INVALID_VALUE and b"workspace" in L.svdq_last_error()
        assert _quant(ws=P(9), wsb=need_q - 16) == INVALID_VALUE
        assert _quant(ws=P(1), wsb=need_q) == INVALID_VALUE                  # over the input x
        if not _gpu_visible():
            assert _gemm(ws=P(9), wsb=need_g) == NO_DEVICE
            assert _gemm(ws=P(9), wsb=need_g + 4096) == NO_DEVICE
            assert _quant(ws=P(9), wsb=need_q) == NO_DEVICE
    finally:
        L.svdq_debug_set_gemm_splits(0)
        L.svdq_debug_set_gemm_path(0)
        L.svdq_debug_set_quant_plan(0, 0)


def test_call1_plan_choice_through_the_workspace_query():
    """Call 1's plan shows in its workspace: 1 MiB of counters, then K-blocks x
    row tiles x r/16 KB of fp32 partials when K is split.  The row-tile
    kernel's plan for a few thousand tokens or fewer (K-blocks from its cost
    model on the 256 CUs assumed without a device: 8 blocks of 6 groups for
    64-512 tokens at K = 3072, 24 blocks of 10 groups for 64 tokens at
    K = 15360), the one-wave kernel's plan past the 96 MB read cap (2048 x 12288:
    16 blocks) and at the headline (6 blocks), and both test hooks."""
    L = lib()
    part = lambda kb, M, r: (1 << 20) + kb * ((M + 15) // 16) * (r // 16) * 1024
    assert L.svdq_quantize_act_workspace_size(64, 3072, 32) == part(8, 64, 32)
    assert L.svdq_quantize_act_workspace_size(512, 3072, 32) == part(8, 512, 32)
    assert L.svdq_quantize_act_workspace_size(300, 3072, 16) == part(8, 300, 16)
    assert L.svdq_quantize_act_workspace_size(64, 15360, 32) == part(24, 64, 32)
    assert L.svdq_quantize_act_workspace_size(1024, 12288, 32) == part(4, 1024, 32)
    assert L.svdq_quantize_act_workspace_size(2048, 12288, 32) == part(16, 2048, 32)
    assert L.svdq_quantize_act_workspace_size(4608, 3072, 32) == part(6, 4608, 32)
    try:
        assert L.svdq_debug_set_quant_waves(1) == SUCCESS        # the one-wave kernel's own plan
        assert L.svdq_quantize_act_workspace_size(64, 3072, 32) == part(24, 64, 32)
        assert L.svdq_debug_set_quant_waves(8) == SUCCESS        # row-tile kernel, 2 forced K-blocks
        assert L.svdq_debug_set_quant_plan(2, 0) == SUCCESS
        assert L.svdq_quantize_act_workspace_size(200, 448, 32) == part(2, 200, 32)
        assert L.svdq_debug_set_quant_plan(0, 0) == SUCCESS      # one K-block: nothing to add up
        assert L.svdq_quantize_act_workspace_size(200, 448, 32) == 0
    finally:
        L.svdq_debug_set_quant_waves(0)
        L.svdq_debug_set_quant_plan(0, 0)


@pytest.mark.skipif(_gpu_visible(), reason="checks the no-GPU path")
def test_large_shapes_pass_validation_up_to_the_limits():
    """Codes of 2^32 bytes and more (rows * K / 2) are addressed from 64-bit row
    bases, so they pass validation; the stated limits are exact."""
    big_k = 1 << 20
    assert _gemm(M=1 << 13, N=1 << 13, K=big_k, r=0, la=None, lu=None) == NO_DEVICE     # 4 GiB codes each
    assert _gemm(M=1 << 24, N=64, K=1024, r=0, la=None, lu=None) == NO_DEVICE         # 2^33 bytes of codes
    assert _gemm(M=(1 << 24) + 1, N=64, K=1024, r=0, la=None, lu=None) == NOT_SUPPORTED
    assert _gemm(M=64, N=(1 << 20) + 64, K=256) == NOT_SUPPORTED
    assert _gemm(M=64, N=256, K=big_k + 64) == NOT_SUPPORTED
    assert _quant(M=1 << 20, K=big_k, r=0, lora_down=None, la=None) == NO_DEVICE     # M * K = 2^40
    assert _quant(M=(1 << 20) + 1, K=big_k, r=0, lora_down=None, la=None) == NOT_SUPPORTED
    # K beyond 4096 is split over workgroups, one workspace counter per 16 rows (2^18 counters)
    assert _quant(M=1 << 22, K=8192, r=16, wsb=1 << 40) == NO_DEVICE
    assert _quant(M=(1 << 22) + 1, K=8192, r=16, wsb=1 << 40) == NOT_SUPPORTED
    assert _quant(M=(1 << 22) + 1, K=4096, r=16, wsb=1 << 40) == NO_DEVICE
