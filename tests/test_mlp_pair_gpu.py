"""GELU epilogue of call 2 and the GPU-chained MLP pair against the oracle.  Needs an MI355X.

Bar: as for the single linear.  Codes and scales of call 1 are bit-exact on
the oracle's inputs; H and Y are within relative Frobenius 5e-3 and max-abs
1e-2 * max|.| of the float64 oracle.  In the chain each side quantizes its own
H, and the two H differ by rounding, so the down-projection's codes there are
checked to differ by at most one step (a one-ulp change of an element or of a
group maximum moves a code by at most one).
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from tests.gpu_util import (Y_MAX_ABS, Y_REL_FRO, bf16_bits, custom_case, to_dev, to_dev_bf16,
                            ulp_distance, y_errors)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_diffusion_transformer_svdq_amd import check_device
    check_device(0)


def _layer_dev(lam, packed, bias):
    r = packed["lora_down"].shape[0]
    return {"smooth": to_dev(np.asarray(lam, np.float32)),
            "lora_down": to_dev_bf16(packed["lora_down"]) if r else None,
            "lora_up": to_dev_bf16(packed["lora_up"]) if r else None,
            "w_codes": to_dev(packed["w_codes"]), "w_scales": to_dev_bf16(packed["w_scales"]),
            "bias": None if bias is None else to_dev_bf16(bias)}


def _assert_bar(got_bits, want_f64, what):
    rel, mx = y_errors(got_bits, want_f64)
    assert rel <= Y_REL_FRO and mx <= Y_MAX_ABS, (what, rel, mx)


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("M,K,N,r", [
    (1, 64, 64, 16), (37, 448, 192, 32), (130, 640, 448, 48), (300, 192, 320, 16), (64, 3072, 1024, 32),
])
def test_gelu_epilogue_both_kernels(path, M, K, N, r):
    import torch
    import bit_diffusion_transformer_svdq_amd as K_
    d, lam, packed = custom_case(M, K, N, r, seed=3 * M + N)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    L = _layer_dev(lam, packed, d["bias"])
    codes, scales, la = K_.quantize_act_lora_down(to_dev_bf16(d["x"]), L["smooth"], L["lora_down"])
    K_.debug_set_gemm_path(path)
    try:
        y = K_.w4a4_gemm_lora_up(codes, scales, L["w_codes"], L["w_scales"], la, L["lora_up"], L["bias"],
                                 epilogue="gelu_tanh")
        torch.cuda.synchronize()
    finally:
        K_.debug_set_gemm_path(0)
    assert np.array_equal(codes.cpu().numpy(), ref["act_codes"])
    y_ref, _ = O.linear_output(ref["act_codes"], ref["act_scales"], packed["w_codes"], packed["w_scales"],
                               ref["lora_act"], packed["lora_up"], d["bias"], epilogue="gelu_tanh")
    _assert_bar(bf16_bits(y), y_ref, "gelu")
    # the epilogue really ran: negative pre-activations are squashed towards 0
    assert O.bf16_to_f64(bf16_bits(y)).min() > -0.2


def _pair_case(M, K, N_up, N_dn, r, seed, full=False):
    if full:
        su, sd = S.SPECS["pair_up"], S.SPECS["pair_down"]
    else:
        su = S.LinearSpec(f"pair_up{M}", 9, M, K, N_up, r, outlier_frac=0.02, outlier_scale=30.0,
                          heavy_tail=True, row_outlier_frac=0.02, layer_id=seed)
        sd = S.LinearSpec(f"pair_dn{M}", 9, M, N_up, N_dn, r, heavy_tail=True, layer_id=seed + 1)
    du = S.make_linear(su)
    wd, bd = S.make_w(sd), S.make_bias(sd)
    lam_u = O.smooth_factors(O.activation_absmax(du["x"]), du["w"])
    pu = O.pack_weights(du["w"], lam_u, su.r)
    # lambda of the down-projection: calibrated on the float model's GELU output
    lam_d = O.smooth_factors(O.activation_absmax(O.float_mlp_hidden(du["x"], du["w"], du["bias"])), wd)
    pd = O.pack_weights(wd, lam_d, sd.r)
    return du, (lam_u, pu, du["bias"]), (lam_d, pd, bd)


def _check_pair(du, up, dn, rows=None):
    import torch
    import bit_diffusion_transformer_svdq_amd as K_
    (lam_u, pu, bu), (lam_d, pd, bd) = up, dn
    Lu, Ld = _layer_dev(lam_u, pu, bu), _layer_dev(lam_d, pd, bd)
    x = to_dev_bf16(du["x"])
    y, h = K_.mlp_pair(x, Lu, Ld)
    # the down-projection's call 1 on the chained H, kept for the code check
    codes_d, _, _ = K_.quantize_act_lora_down(h, Ld["smooth"], Ld["lora_down"])
    torch.cuda.synchronize()
    ref = O.mlp_pair(du["x"], lam_u, pu, bu, lam_d, pd, bd, rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    hb, yb = bf16_bits(h)[sel], bf16_bits(y)[sel]
    a = ref["a_up"]
    h_star, _ = O.linear_output(a["act_codes"], a["act_scales"], pu["w_codes"], pu["w_scales"],
                                a["lora_act"], pu["lora_up"], bu, epilogue="gelu_tanh")
    _assert_bar(hb, h_star, "H")
    _assert_bar(yb, ref["y"], "Y")
    dq = np.abs(O.unpack_int4(codes_d.cpu().numpy())[sel].astype(int)
                - O.unpack_int4(ref["a_down"]["act_codes"]).astype(int))
    assert dq.max() <= 1 and (dq == 0).mean() >= 0.99, (dq.max(), (dq == 0).mean())
    # call 1 of the down-projection on the oracle's H: bit-exact
    c2, s2, la2 = K_.quantize_act_lora_down(to_dev_bf16(ref["h"]), Ld["smooth"], Ld["lora_down"])
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy(), ref["a_down"]["act_codes"])
    assert np.array_equal(bf16_bits(s2), ref["a_down"]["act_scales"])
    assert (ulp_distance(bf16_bits(la2), ref["a_down"]["lora_act"]) <= 1).mean() >= 0.999


@pytest.mark.parametrize("M", [40, 300])
def test_mlp_pair_chain_small(M):
    """Up 256 -> 512 with GELU, down 512 -> 192 (M=40 takes the few-token GEMM
    kernel, M=300 the tiled one)."""
    du, up, dn = _pair_case(M, 256, 512, 192, 16, seed=M)
    _check_pair(du, up, dn)


def test_mlp_pair_full_size_sampled_rows():
    """The MLP pair at its full size (M=4608, 3072 -> 12288 -> 3072, r=32) in the
    launch configuration the benchmark times; the oracle follows sampled token
    rows through the whole chain (every step is per token once lambda is fixed)."""
    du, up, dn = _pair_case(0, 0, 0, 0, 0, 0, full=True)
    rows = [0, 1, 63, 64, 1000, 2047, 4095, 4096, 4607]
    _check_pair(du, up, dn, rows=rows)
