"""Host packer of the FP4 variant (svdq_pack_weights_fp4) against the oracle.  CPU only.

Its factors are those of svdq_pack_weights (same split, same seed); its MXFP4
residual codes are checked against the oracle's MXFP4 quantizer applied to the
packer's own factors (the residual's summation order may move an element
sitting exactly on a rounding midpoint, and a block maximum sitting exactly on
a power of two, nothing else)."""
import numpy as np

import oracle as O
import oracle.mxfp4_oracle as X
import synthetic as S
from bit_diffusion_transformer_svdq_amd import pack_weights, pack_weights_fp4, smooth_from_absmax


def _lam(d):
    return smooth_from_absmax(O.activation_absmax(d["x"]).astype(np.float32), d["w"])


def _check(d, r, seed=0):
    lam = _lam(d)
    pk = pack_weights_fp4(d["w"], lam, r, seed=seed)
    i4 = pack_weights(d["w"], lam, r, seed=seed)
    assert np.array_equal(pk["lora_down"], i4["lora_down"]) and np.array_equal(pk["lora_up"], i4["lora_up"])
    resid = O.smoothed_weight(d["w"], lam) - O.bf16_to_f64(pk["lora_up"]) @ O.bf16_to_f64(pk["lora_down"])
    codes, exps = X.mx_quantize_blocks(resid)
    assert (pk["w_scales"] == exps).mean() >= 1 - 1e-4
    mism = X.unpack_fp4(pk["w_codes"]) != codes
    same_e = np.repeat(pk["w_scales"] == exps, 32, axis=1)
    if mism.any():
        t = np.abs(resid) / np.exp2(np.repeat(exps.astype(np.float64), 32, axis=1) - 127)
        near = np.min(np.abs(t[..., None] - np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])), axis=-1) < 1e-9
        assert not (mism & same_e & ~near).any()
        assert mism.mean() <= 1e-4


def test_fp4_pack_tiny():
    _check(S.make_linear("tiny"), 16)


def test_fp4_pack_rank0_equals_oracle_exactly():
    d = S.make_linear("tiny")
    lam = _lam(d)
    pk = pack_weights_fp4(d["w"], lam, 0)
    ref = X.pack_weights_fp4(d["w"], lam, 0)
    assert np.array_equal(pk["w_codes"], ref["w_codes"]) and np.array_equal(pk["w_scales"], ref["w_scales"])


def test_fp4_pack_larger_rank32():
    spec = S.LinearSpec("fp4pk", 9, 64, 512, 256, 32, outlier_frac=0.01, outlier_scale=30.0, heavy_tail=True)
    _check(S.make_linear(spec), 32)
