"""Call 2 with the fused QKV epilogue (per-head RMSNorm + rotary turn on Q and
K, V plain) against the oracle.  Needs an MI355X.

Bar: each third of Y (Q, K, V) is within relative Frobenius 5e-3 and max-abs
1e-2 * max|.| of the float64 oracle, which normalizes and rotates the unrounded
Y* and rounds once, as the kernel does in fp32.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from tests.gpu_util import (Y_MAX_ABS, Y_REL_FRO, bf16_bits, custom_case, oracle_case, to_dev,
                            to_dev_bf16, y_errors)

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_diffusion_transformer_svdq_amd import check_device
    check_device(0)


def _run_qkv(d, lam, packed, cos, sin, qn, kn, path=0):
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    r = packed["lora_down"].shape[0]
    codes, scales, la = K.quantize_act_lora_down(to_dev_bf16(d["x"]), to_dev(np.asarray(lam, np.float32)),
                                                 to_dev_bf16(packed["lora_down"]) if r else None)
    K.debug_set_gemm_path(path)
    try:
        y = K.w4a4_gemm_qkv_norm_rope(codes, scales, to_dev(packed["w_codes"]), to_dev_bf16(packed["w_scales"]),
                                      la if r else None, to_dev_bf16(packed["lora_up"]) if r else None,
                                      to_dev_bf16(d["bias"]), to_dev_bf16(qn), to_dev_bf16(kn),
                                      to_dev(cos), to_dev(sin), eps=EPS)
        torch.cuda.synchronize()
    finally:
        K.debug_set_gemm_path(0)
    return bf16_bits(y)


def _check(got, d, lam, packed, cos, sin, qn, kn, rows=None):
    a = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    want, _ = O.qkv_output(a["act_codes"], a["act_scales"], packed["w_codes"], packed["w_scales"],
                           a["lora_act"], packed["lora_up"], d["bias"], 128, qn, kn, EPS, cos, sin, rows=rows)
    g = got if rows is None else got[np.asarray(rows)]
    sec = want.shape[1] // 3
    for t, name in enumerate("QKV"):
        rel, mx = y_errors(g[:, t * sec:(t + 1) * sec], want[:, t * sec:(t + 1) * sec])
        assert rel <= Y_REL_FRO and mx <= Y_MAX_ABS, (name, rel, mx)
    return want


@pytest.mark.parametrize("path", [0, 2])
@pytest.mark.parametrize("M,K,heads,r", [(1, 256, 1, 16), (37, 256, 2, 16), (200, 448, 2, 32),
                                          (300, 192, 1, 0), (130, 3072, 3, 32)])
def test_qkv_epilogue_small(path, M, K, heads, r):
    """Several heads per third, ragged token counts, rank 0; path 2 asks for
    the few-token kernel, which this epilogue never takes (same result)."""
    d, lam, packed = custom_case(M, K, 3 * 128 * heads, r, seed=5 * M + heads)
    cos, sin = S.make_rope_tables(M, 128, n_text=min(8, M), grid_w=16)
    qn, kn = S.make_norm_weight(d["spec"], 0), S.make_norm_weight(d["spec"], 1)
    got = _run_qkv(d, lam, packed, cos, sin, qn, kn, path)
    want = _check(got, d, lam, packed, cos, sin, qn, kn)
    # the normalization really ran: every Q head of every token has RMS ~ |w|
    q = O.bf16_to_f64(got[:, :128 * heads]).reshape(M, heads, 128)
    wq = np.sqrt((O.bf16_to_f64(qn) ** 2).mean())
    assert np.allclose(np.sqrt((q ** 2).mean(-1)), wq, rtol=0.15)
    assert np.isfinite(want).all()


def test_qkv_epilogue_full_shape_sampled_rows():
    """The fused QKV projection at its full size (M=4608, K=3072, N=9216: 24
    heads per third, r=32) with the FLUX-like rotary tables of 512 text + 64x64
    image tokens, in the launch configuration the benchmark times."""
    d, lam, packed = oracle_case("qkv")
    M = d["spec"].M
    cos, sin = S.make_rope_tables(M, 128)
    qn, kn = S.make_norm_weight(d["spec"], 0), S.make_norm_weight(d["spec"], 1)
    got = _run_qkv(d, lam, packed, cos, sin, qn, kn)
    rows = [0, 1, 127, 128, 511, 512, 513, 2047, 4095, 4096, 4607]
    _check(got, d, lam, packed, cos, sin, qn, kn, rows=rows)
