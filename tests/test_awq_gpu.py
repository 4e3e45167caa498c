"""The AWQ W4A16 kernel (svdq_awq_w4a16_gemm) against the oracle.  Needs an MI355X.

Bar: as for the W4A4 linear, Y within relative Frobenius 5e-3 and max-abs
1e-2 * max|Y*| of the float64 oracle (the kernel's products are exact; it
accumulates in fp32).  Weights are quantized by the oracle."""
import numpy as np
import pytest

import oracle as O
import oracle.awq_oracle as A
import synthetic as S
from tests.gpu_util import Y_MAX_ABS, Y_REL_FRO, bf16_bits, to_dev, to_dev_bf16, y_errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_diffusion_transformer_svdq_amd import check_device
    check_device(0)


def _case(spec, search=True, alpha=0.5):
    x = S.make_x(spec)
    w = S.make_w(spec)
    b = S.make_bias(spec)
    if search:
        pk = A.awq_pack(S.make_calibration(spec, 32), w)
    else:   # full-size case: the kernel does not depend on how s was chosen
        s = A.awq_scales(A.activation_mean_abs(S.make_calibration(spec, 32)), alpha)
        q, d, z = A.quantize_asym_groups(O.bf16_to_f64(w) * s.astype(np.float64)[None, :])
        pk = {"smooth": s, "codes": A.pack_uint4(q), "scales": d, "zeros": z}
    return x, b, pk


def _run(x, b, pk, bias=True):
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    y = K.awq_w4a16_gemm(to_dev_bf16(x), to_dev(np.asarray(pk["smooth"], np.float32)), to_dev(pk["codes"]),
                         to_dev_bf16(pk["scales"]), to_dev(pk["zeros"]), to_dev_bf16(b) if bias else None)
    torch.cuda.synchronize()
    return bf16_bits(y)


def _check(got, x, b, pk, bias=True):
    want, _ = A.awq_linear(x, pk["smooth"], pk["codes"], pk["scales"], pk["zeros"], b if bias else None)
    rel, mx = y_errors(got, want)
    assert rel <= Y_REL_FRO and mx <= Y_MAX_ABS, (rel, mx)


@pytest.mark.parametrize("M,K,N", [(1, 64, 32), (3, 192, 96), (16, 256, 64), (17, 320, 96), (40, 1024, 160),
                                   (2, 6144, 64), (20, 3072, 96), (1, 16384, 32), (4, 8192, 64), (5, 4096, 32),
                                   (1, 320, 96), (1, 4096, 64)])
def test_awq_small_shapes(M, K, N):
    """Ragged token tiles, K of one group (three of the four waves idle), an
    odd number of groups per wave, and the largest K of each staged class
    (one token: 16384, up to four: 8192, more: 4096)."""
    spec = S.LinearSpec(f"awq{M}x{K}x{N}", 8, M, K, N, 0, outlier_frac=0.03, outlier_scale=10.0,
                        heavy_tail=True, silu_input=True, layer_id=M + K + N)
    x, b, pk = _case(spec)
    _check(_run(x, b, pk), x, b, pk)
    _check(_run(x, b, pk, bias=False), x, b, pk, bias=False)


@pytest.mark.parametrize("name,M", [("mod_double", 1), ("mod_single", 4), ("mod_final", 2), ("mod_double", 4),
                                    ("mod_double", 3), ("mod_single", 1), ("mod_final", 1)])
def test_awq_modulation_shapes(name, M):
    """The modulation projections of a 12B DiT at their full size (3072 ->
    18432 / 9216 / 6144) for 1 to 4 images (3072 -> 18432 at 3 and 4 images
    runs three n-tiles per workgroup)."""
    spec = S.MOD_SPECS[name].with_m(M)
    x, b, pk = _case(spec, search=False)
    _check(_run(x, b, pk), x, b, pk)


def test_awq_three_tiles_per_workgroup_ragged():
    """770 n-tiles at 3 per workgroup: the last workgroup has a missing tile
    (its loads repeat the last tile, nothing is stored for it)."""
    spec = S.LinearSpec("awq_wide", 8, 2, 3072, 12320, 0, outlier_frac=0.03, outlier_scale=10.0,
                        heavy_tail=True, silu_input=True, layer_id=91)
    x, b, pk = _case(spec, search=False)
    _check(_run(x, b, pk), x, b, pk)


def test_awq_repeated_launches_are_bit_identical():
    spec = S.LinearSpec("awqrep", 8, 5, 512, 96, 0, outlier_frac=0.03, outlier_scale=10.0, silu_input=True)
    x, b, pk = _case(spec)
    assert np.array_equal(_run(x, b, pk), _run(x, b, pk))


def _stack(packs, key):
    return np.ascontiguousarray(np.stack([pk[key] for pk in packs]))


@pytest.mark.parametrize("M,K,N,L", [(1, 512, 96, 3), (4, 320, 64, 2), (20, 256, 32, 3), (1, 3072, 18432, 4),
                                     (4, 3072, 18432, 2)])
def test_awq_stacked_matches_single_layers(M, K, N, L):
    """L layers sharing x in one launch: every layer's output is bit-identical
    to the one-layer call on its own arrays, and layer 0 matches the oracle
    (3072 -> 18432 at four tokens: three n-tiles per workgroup)."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K_
    cases = []
    for l in range(L):
        spec = S.LinearSpec(f"awqst{M}x{K}x{N}", 8, M, K, N, 0, outlier_frac=0.03, outlier_scale=10.0,
                            heavy_tail=True, silu_input=True, layer_id=300 + l)
        cases.append(_case(spec, search=K * N <= 512 * 96))
    x = cases[0][0]                      # the shared input
    packs = [c[2] for c in cases]
    biases = [c[1] for c in cases]
    xd = to_dev_bf16(x)
    sm = to_dev(np.asarray(_stack(packs, "smooth"), np.float32))
    codes, scales, zeros = to_dev(_stack(packs, "codes")), to_dev_bf16(_stack(packs, "scales")), \
        to_dev(_stack(packs, "zeros"))
    bias = to_dev_bf16(np.ascontiguousarray(np.stack(biases)))
    for b in (bias, None):
        ys = K_.awq_w4a16_gemm_stacked(xd, sm, codes, scales, zeros, b)
        torch.cuda.synchronize()
        for l in range(L):
            y1 = K_.awq_w4a16_gemm(xd, sm[l], codes[l], scales[l], zeros[l], None if b is None else b[l])
            torch.cuda.synchronize()
            assert torch.equal(ys[l], y1), l
    _check(bf16_bits(ys[0]), x, None, packs[0], bias=False)
