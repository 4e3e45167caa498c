"""The no-allocation variant of call 2 (svdq_w4a4_gemm_lora_up_noalloc), through
the C ABI.  Needs an MI355X.

It must give exactly what svdq_w4a4_gemm_lora_up_ex gives on the same inputs
(the same kernels and plan, its K-split partial sums going through the
library's fixed device scratch instead of a caller's workspace), on two calls
in a row whose second is smaller, and stay within the oracle's bar."""
import ctypes

import numpy as np
import pytest

import oracle as O
from tests.gpu_util import bf16_bits, check_y, custom_case, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_diffusion_transformer_svdq_amd import check_device
    check_device(0)


def _inputs(case):
    d, lam, p = case
    ref = O.quantize_act_lora_down(d["x"], lam, p["lora_down"])
    return ref, dict(ac=to_dev(ref["act_codes"]), asc=to_dev_bf16(ref["act_scales"]), wc=to_dev(p["w_codes"]),
                     wsc=to_dev_bf16(p["w_scales"]), la=to_dev_bf16(ref["lora_act"]), lu=to_dev_bf16(p["lora_up"]),
                     b=to_dev_bf16(d["bias"]))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _call_noalloc(t, M, N, K, r, y, epilogue=0):
    import torch
    from bit_diffusion_transformer_svdq_amd import _lib
    L = _lib.lib()
    st = L.svdq_w4a4_gemm_lora_up_noalloc(_ptr(t["ac"]), _ptr(t["asc"]), _ptr(t["wc"]), _ptr(t["wsc"]), _ptr(t["la"]),
                                          _ptr(t["lu"]), _ptr(t["b"]), M, N, K, r, 64, epilogue, _ptr(y),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check(st, "svdq_w4a4_gemm_lora_up_noalloc")


def _call_ws(t, M, N, K, r, y, epilogue=0):
    import torch
    from bit_diffusion_transformer_svdq_amd import _lib
    L = _lib.lib()
    need = L.svdq_w4a4_gemm_workspace_size(M, N, K, r)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    st = L.svdq_w4a4_gemm_lora_up_ex(_ptr(t["ac"]), _ptr(t["asc"]), _ptr(t["wc"]), _ptr(t["wsc"]), _ptr(t["la"]),
                                     _ptr(t["lu"]), _ptr(t["b"]), M, N, K, r, 64, epilogue, _ptr(y),
                                     _ptr(ws) if need else None, need, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check(st, "svdq_w4a4_gemm_lora_up_ex")
    return need


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    import torch
    from bit_diffusion_transformer_svdq_amd import _lib
    # a text-stream sized projection (K split over workgroups, partials in the scratch),
    # then a smaller one with a different split
    cases = [(512, 3072, 3072, 32, 101), (200, 1024, 192, 16, 102)]
    for i, (M, K, N, r, seed) in enumerate(cases):
        case = custom_case(M, K, N, r, seed=seed)
        ref, t = _inputs(case)
        y0 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        y1 = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
        print(f"noalloc call {i}: M={M} K={K} N={N} r={r}", flush=True)
        need = _call_ws(t, M, N, K, r, y0)
        assert need > 0, "the case must split K to exercise the scratch"
        _call_noalloc(t, M, N, K, r, y1)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1), i
        check_y(bf16_bits(y1), case[0], case[1], case[2], ref)
    # the GELU epilogue through the same scratch, after the calls above
    M, K, N, r, seed = cases[1]
    case = custom_case(M, K, N, r, seed=seed)
    ref, t = _inputs(case)
    y0 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    _call_ws(t, M, N, K, r, y0, epilogue=1)
    _call_noalloc(t, M, N, K, r, y1, epilogue=1)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    del _lib


def test_noalloc_rejects_a_plan_beyond_the_fixed_scratch():
    import torch
    from bit_diffusion_transformer_svdq_amd import _lib
    L = _lib.lib()
    case = custom_case(256, 3072, 3072, 16, seed=103)
    ref, t = _inputs(case)
    y = torch.empty((256, 3072), dtype=torch.bfloat16, device="cuda")
    L.svdq_debug_set_gemm_path(1)
    L.svdq_debug_set_gemm_splits(48)   # 48 tiles x 48 splits x 64 KiB > 64 MiB
    try:
        assert L.svdq_w4a4_gemm_workspace_size(256, 3072, 3072, 16) > 64 << 20
        with pytest.raises(_lib.SvdqError, match="scratch"):
            _call_noalloc(t, 256, 3072, 3072, 16, y)
    finally:
        L.svdq_debug_set_gemm_splits(0)
        L.svdq_debug_set_gemm_path(0)


def test_noalloc_binding_matches_call_2():
    """The Python binding of the same entry point (argument marshalling only)."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    case = custom_case(384, 2048, 1024, 32, seed=104)
    ref, t = _inputs(case)
    y0 = K.w4a4_gemm_lora_up(t["ac"], t["asc"], t["wc"], t["wsc"], t["la"], t["lu"], t["b"])
    y1 = K.w4a4_gemm_lora_up_noalloc(t["ac"], t["asc"], t["wc"], t["wsc"], t["la"], t["lu"], t["b"])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    check_y(bf16_bits(y1), case[0], case[1], case[2], ref)
