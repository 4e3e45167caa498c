"""Host packer (C++, in libsvdq) against the oracle.  CPU only.

The SVD is not unique (signs, near-equal singular values), so the packer's
factors are compared through invariants, and its codes and scales are checked
against the oracle's quantizer applied to the packer's own factors.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from bit_diffusion_transformer_svdq_amd import pack_weights, smooth_from_absmax


def _lam(d):
    return smooth_from_absmax(O.activation_absmax(d["x"]).astype(np.float32), d["w"])


def test_smoothing_vector_is_bit_exact():
    d = S.make_linear("tiny")
    ours = _lam(d)
    ref = O.smooth_factors(O.activation_absmax(d["x"]), d["w"])
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def _check_pack(w_bits, lam, r, seed=0, tail_slack=1e-3, code_mismatch_frac=1e-4):
    packed = pack_weights(w_bits, lam, r, seed=seed)
    ws = O.smoothed_weight(w_bits, lam)
    N, K = ws.shape
    up = O.bf16_to_f64(packed["lora_up"])
    down = O.bf16_to_f64(packed["lora_down"])
    resid = ws - up @ down
    # codes and scales: the oracle's residual quantizer applied to the packer's factors
    q_ref, s_ref = O.quantize_weight_groups(resid)
    s_eq = packed["w_scales"] == s_ref
    assert s_eq.mean() >= 1 - 1e-4, (s_eq.size - s_eq.sum())
    q_pk = O.unpack_int4(packed["w_codes"])
    mism = q_pk != q_ref
    if mism.any():
        # only near-ties (summation order of the residual) may differ
        s = np.repeat(O.bf16_to_f64(s_ref), 64, axis=1)
        ratio = np.abs(resid / np.where(s > 0, s, 1.0))
        frac = np.abs(ratio - np.floor(ratio) - 0.5)
        bad = mism & (frac > 1e-9) & np.repeat(s_eq, 64, axis=1)
        assert not bad.any(), np.argwhere(bad)[:5]
        assert mism.mean() <= code_mismatch_frac
    # low-rank quality: close to the Eckart-Young optimum of the exact SVD
    sv = np.linalg.svd(ws, compute_uv=False)
    tail = np.sqrt((sv[r:] ** 2).sum())
    _, _, resid_o, _ = O.lowrank_split(ws, r)
    assert np.linalg.norm(resid) <= np.linalg.norm(resid_o) * (1 + tail_slack) + 1e-12
    assert np.linalg.norm(resid) >= tail * (1 - 1e-9)
    return packed, sv


def test_pack_tiny_rank16():
    d = S.make_linear("tiny")
    _check_pack(d["w"], _lam(d), 16)


def test_pack_rank0_equals_oracle_exactly():
    d = S.make_linear("tiny")
    lam = _lam(d)
    packed = pack_weights(d["w"], lam, 0)
    ref = O.pack_weights(d["w"], lam, 0)
    assert np.array_equal(packed["w_codes"], ref["w_codes"])
    assert np.array_equal(packed["w_scales"], ref["w_scales"])


def test_pack_top_singular_values_recovered():
    """Strong, well separated directions are found to high accuracy."""
    rng = np.random.default_rng(3)
    N, K, r = 192, 320, 16
    base = rng.standard_normal((N, K)) * 0.01
    u = np.linalg.qr(rng.standard_normal((N, r)))[0]
    v = np.linalg.qr(rng.standard_normal((K, r)))[0]
    base += (u * np.geomspace(4.0, 1.0, r)) @ v.T
    w_bits = O.f64_to_bf16(base)
    lam = np.ones(K, np.float32)
    packed, sv = _check_pack(w_bits, lam, r, tail_slack=1e-6)
    lowrank = O.bf16_to_f64(packed["lora_up"]) @ O.bf16_to_f64(packed["lora_down"])
    got = np.linalg.svd(lowrank, compute_uv=False)[:r]
    assert np.allclose(got, sv[:r], rtol=1e-2)


def test_pack_is_deterministic_and_seeded():
    d = S.make_linear("tiny")
    lam = _lam(d)
    a = pack_weights(d["w"], lam, 16, seed=5)
    b = pack_weights(d["w"], lam, 16, seed=5)
    for k in a:
        assert np.array_equal(a[k], b[k])


@pytest.mark.slow
def test_pack_dit_shape_rank32():
    """Config shape of the attention-out linear (K = N = 3072) with heavy tails and outliers."""
    spec = S.SPECS["attn_out"].with_m(256)
    d = S.make_linear(spec)
    _check_pack(d["w"], _lam(d), 32, tail_slack=2e-3)
