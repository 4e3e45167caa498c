"""FP4 (MXFP4) variant of calls 1 and 2 against the oracle.  Needs an MI355X.

Bar: call 1's E2M1 codes and E8M0 exponents bit-exact; lora_act within one
bf16 ulp as for the int4 path; Y within relative Frobenius 5e-3 and max-abs
1e-2 * max|Y*| of the float64 oracle (products of E2M1 values and power-of-two
scales are exact; the matrix core accumulates in fp32).  Weights are packed by
the oracle."""
import numpy as np
import pytest

import oracle as O
import oracle.mxfp4_oracle as X
import synthetic as S
from tests.gpu_util import (Y_MAX_ABS, Y_REL_FRO, bf16_bits, to_dev, to_dev_bf16, ulp_distance, y_errors)

pytestmark = pytest.mark.gpu
_CASES = {}


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_diffusion_transformer_svdq_amd import check_device
    check_device(0)


def _case(spec):
    if spec not in _CASES:
        d = S.make_linear(spec)
        lam = O.smooth_factors(O.activation_absmax(d["x"]), d["w"])
        _CASES[spec] = (d, lam, X.pack_weights_fp4(d["w"], lam, spec.r))
    return _CASES[spec]


def _spec(M, K, N, r, seed):
    return S.LinearSpec(f"fp4_{M}x{K}x{N}r{r}", 10, M, K, N, r, outlier_frac=0.02, outlier_scale=30.0,
                        heavy_tail=True, layer_id=seed)


def _run(d, lam, pk, x_bits=None, epilogue="none"):
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    r = pk["lora_down"].shape[0]
    x = d["x"] if x_bits is None else x_bits
    codes, scales, la = K.quantize_act_lora_down_fp4(to_dev_bf16(x), to_dev(np.asarray(lam, np.float32)),
                                                     to_dev_bf16(pk["lora_down"]) if r else None)
    y = K.fp4_gemm_lora_up(codes, scales, to_dev(pk["w_codes"]), to_dev(pk["w_scales"]), la if r else None,
                           to_dev_bf16(pk["lora_up"]) if r else None, to_dev_bf16(d["bias"]), epilogue=epilogue)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), bf16_bits(la), bf16_bits(y)


def _check(got, d, lam, pk, x_bits=None, rows=None, epilogue="none"):
    codes, scales, la, y = got
    x = d["x"] if x_bits is None else x_bits
    ref = X.quantize_act_lora_down_fp4(x, lam, pk["lora_down"])
    assert np.array_equal(scales, ref["act_scales"]), np.argwhere(scales != ref["act_scales"])[:5]
    assert np.array_equal(codes, ref["act_codes"]), np.argwhere(codes != ref["act_codes"])[:5]
    if ref["lora_act"].size:
        assert (ulp_distance(la, ref["lora_act"]) <= 1).mean() >= 0.999
    want, _ = X.linear_output_fp4(ref["act_codes"], ref["act_scales"], pk["w_codes"], pk["w_scales"],
                                  ref["lora_act"], pk["lora_up"], d["bias"], rows=rows)
    if epilogue == "gelu_tanh":
        want = O.gelu_tanh(want)
    g = y if rows is None else y[np.asarray(rows)]
    rel, mx = y_errors(g, want)
    assert rel <= Y_REL_FRO and mx <= Y_MAX_ABS, (rel, mx)


@pytest.mark.parametrize("M,K,N,r", [(64, 256, 256, 16), (37, 384, 192, 32), (200, 1024, 320, 48),
                                     (300, 128, 64, 0), (129, 640, 128, 16), (1, 128, 64, 16)])
def test_fp4_small_shapes(M, K, N, r):
    d, lam, pk = _case(_spec(M, K, N, r, M + K + N))
    _check(_run(d, lam, pk), d, lam, pk)


@pytest.mark.parametrize("splits", [2, 3])
def test_fp4_forced_splits_and_gelu(splits):
    import bit_diffusion_transformer_svdq_amd as K
    d, lam, pk = _case(_spec(160, 1536, 192, 32, 5))
    K.debug_set_gemm_splits(splits)
    try:
        got = _run(d, lam, pk, epilogue="gelu_tanh")
    finally:
        K.debug_set_gemm_splits(0)
    _check(got, d, lam, pk, epilogue="gelu_tanh")


def test_fp4_quantizer_edge_blocks():
    """Zero rows (exponent code 0, zero codes), huge and tiny magnitudes, and a
    block whose maximum sits exactly on a power of two and on a midpoint."""
    d, lam, pk = _case(_spec(48, 256, 64, 16, 7))
    x = d["x"].copy()
    x[0] = 0
    x[1] = S.to_bf16_bits(O.bf16_to_f64(x[1]) * 1e30)
    x[2] = S.to_bf16_bits(O.bf16_to_f64(x[2]) * 1e-30)
    x[3] = S.to_bf16_bits(np.tile(np.array([4.0, 5.0, 1.25, -0.75, 2.5, 3.5, 0.25, -6.0]), 32))
    ones = np.ones_like(np.asarray(lam, np.float32))
    got = _run(d, ones, pk, x_bits=x)
    ref = X.quantize_act_lora_down_fp4(x, ones, pk["lora_down"])
    assert np.array_equal(got[1], ref["act_scales"]) and np.array_equal(got[0], ref["act_codes"])
    assert np.all(got[1][0] == 0) and np.all(got[0][0] == 0)


def test_fp4_forced_quant_plans():
    import bit_diffusion_transformer_svdq_amd as K
    d, lam, pk = _case(_spec(130, 1152, 64, 32, 9))
    for plan in [(3, 2), (1, 5), (9, 1)]:
        K.debug_set_quant_plan(*plan)
        try:
            got = _run(d, lam, pk)
        finally:
            K.debug_set_quant_plan(0, 0)
        _check(got, d, lam, pk)


def test_fp4_headline_shape_sampled_rows():
    """The headline linear (M=4608, K=3072, N=12288, r=32) in the FP4 variant,
    codes and scales of every token, Y on sampled rows."""
    d, lam, pk = _case(S.SPECS["mlp_up"])
    rows = [0, 1, 127, 128, 2047, 4095, 4096, 4607]
    _check(_run(d, lam, pk), d, lam, pk, rows=rows)
