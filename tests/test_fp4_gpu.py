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
from tests.gpu_util import (Y_MAX_ABS, Y_REL_FRO, bf16_bits, check_lora_act, to_dev, to_dev_bf16, ulp_distance,
                            y_errors)

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
        check_lora_act(la, ref, pk["lora_down"])
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


def test_fp4_row_tile_quant_kernel():
    """MXFP4 call 1 through the row-tile kernel (one workgroup per row tile,
    waves splitting K; one and two K-blocks)."""
    import bit_diffusion_transformer_svdq_amd as K
    d, lam, pk = _case(_spec(130, 1152, 64, 32, 11))
    for waves, kb in [(8, 0), (4, 2)]:
        K.debug_set_quant_waves(waves)
        K.debug_set_quant_plan(kb, 0)
        try:
            got = _run(d, lam, pk)
        finally:
            K.debug_set_quant_waves(0)
            K.debug_set_quant_plan(0, 0)
        _check(got, d, lam, pk)


def _tile_rows(M, tile):
    """One row of every row tile at an offset that walks through the tile,
    plus the first and the last two rows."""
    rows = {0, M - 2, M - 1}
    for t in range((M + tile - 1) // tile):
        rows.add(min(M - 1, t * tile + (37 * t + 5) % tile))
    return sorted(r for r in rows if r >= 0)


def test_fp4_headline_shape_sampled_rows():
    """The headline linear (M=4608, K=3072, N=12288, r=32) in the FP4 variant
    (864 tiles of 256 x 256: the 256 x 256 kernel), codes and scales of every
    token, Y on one row of every 256-row tile (every column)."""
    d, lam, pk = _case(S.SPECS["mlp_up"])
    _check(_run(d, lam, pk), d, lam, pk, rows=_tile_rows(4608, 256))


@pytest.mark.parametrize("M,K,N,r,epi", [(300, 1024, 320, 32, "none"), (64, 1024, 64, 0, "none"),
                                         (257, 2048, 576, 16, "gelu_tanh"), (513, 3072, 512, 48, "none"),
                                         (1, 1024, 256, 32, "none"), (256, 4096, 256, 128, "gelu_tanh")])
def test_fp4_256_tile_kernel_forced(M, K, N, r, epi):
    """The 256 x 256 kernel forced at small shapes, every element of Y:
    partial tiles in m and in n, rank chunks of 32 with and without a
    trailing 16, no low-rank branch, one token, the largest rank, GELU."""
    import bit_diffusion_transformer_svdq_amd as K_
    print(f"fp4 256-tile M={M} K={K} N={N} r={r} {epi}", flush=True)
    d, lam, pk = _case(_spec(M, K, N, r, 3 * M + N))
    K_.debug_set_fp4_tile(256)
    try:
        got = _run(d, lam, pk, epilogue=epi)
    finally:
        K_.debug_set_fp4_tile(0)
    _check(got, d, lam, pk, epilogue=epi)


def test_fp4_256_tile_kernel_long_k_sampled_rows():
    """The MLP down-projection shape (M=4608, K=12288, N=3072, r=32) on the
    256 x 256 kernel (forced: its 216 tiles would pick the 128 x 128 kernel
    with K-splits), Y on one row of every 256-row tile."""
    import bit_diffusion_transformer_svdq_amd as K_
    d, lam, pk = _case(S.SPECS["mlp_down"])
    K_.debug_set_fp4_tile(256)
    try:
        got = _run(d, lam, pk)
    finally:
        K_.debug_set_fp4_tile(0)
    _check(got, d, lam, pk, rows=_tile_rows(4608, 256))


def test_fp4_256_tile_kernel_several_tiles_per_workgroup():
    """More 256 x 256 tiles than compute units (M=4000, N=4160: 16 x 17 = 272
    tiles, ragged in m and in n), so workgroups run several tiles one after
    another, the last ones partial; Y on one row of every 256-row tile and the
    last rows, every column."""
    import bit_diffusion_transformer_svdq_amd as K_
    M, K, N, r = 4000, 1024, 4160, 16
    print(f"fp4 256-tile persistent M={M} K={K} N={N} r={r}", flush=True)
    d, lam, pk = _case(_spec(M, K, N, r, 11))
    K_.debug_set_fp4_tile(256)
    try:
        got = _run(d, lam, pk)
    finally:
        K_.debug_set_fp4_tile(0)
    _check(got, d, lam, pk, rows=_tile_rows(M, 256))


def _bf16_ladder_blocks(s: int) -> np.ndarray:
    """Blocks of 32 bf16 patterns whose maximum 6 * 2^s fixes the shared
    exponent at s (elements divide by 2^s exactly), filled with every E2M1
    rounding midpoint times 2^s, its two bf16 neighbours, and their negatives."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * 2.0 ** s
    base = S.to_bf16_bits(mids).astype(np.int64)
    vals = np.concatenate([base - 1, base, base + 1])            # one bf16 ulp below / above
    vals = np.concatenate([vals, vals | 0x8000]).astype(np.uint16)  # and the negatives
    top = S.to_bf16_bits(np.array([6.0 * 2.0 ** s]))
    pad = np.concatenate([top, vals])                             # 43 values
    out = np.resize(pad, 64)                                      # two blocks, each holding 6 * 2^s
    out[32] = top[0]
    return out


def test_fp4_quantizer_midpoint_neighbours_and_signs():
    """The hardware E2M1 converter plus the sign-of-zero fixup against the
    oracle's midpoint ladder (MX specification rounding: nearest, midpoints to
    the even code, saturation above 6, zero unsigned) on every bf16 input that
    borders a midpoint, at several block exponents; negatives that round to
    zero (small values, -0.25 * 2^s exactly, -0.0) must give code 0;
    maxima in (6, 8) * 2^s saturate; blocks whose exponent clamps at -127."""
    d, lam, pk = _case(_spec(48, 256, 64, 16, 7))
    x = np.zeros((16, 256), dtype=np.uint16)
    for i, s in enumerate([-40, -9, -1, 0, 3, 17, 60, 100]):
        x[i, :64] = _bf16_ladder_blocks(s)
        x[i, 64:128] = _bf16_ladder_blocks(s + 1)[::-1]
        # negatives rounding to zero, negative zero, and saturating maxima
        neg_small = -np.array([0.25, 0.2, 0.125, 2.0 ** -6, 0.249])
        blk = np.concatenate([[7.0, -7.5, 7.96875, 6.5], neg_small, [0.0] * 23]) * 2.0 ** s
        x[i, 128:160] = S.to_bf16_bits(blk)
        x[i, 128 + 9] = 0x8000                                   # -0.0
        x[i, 160:192] = S.to_bf16_bits(np.resize(np.array([-7.9375, 6.25, -0.75, 0.0]), 32) * 2.0 ** s)
    # exponent clamped at -127: normal values just above 2^-126
    tiny = np.array([1.0, 1.25, 1.5, 1.75, 1.125, -1.5, -1.0, 1.875]) * 2.0 ** -126
    x[8:16, :32] = S.to_bf16_bits(np.resize(tiny, 32))
    x[8:16, 192:256] = x[0:8, 0:64]
    ones = np.ones(256, dtype=np.float32)
    got = _run(d, ones, pk, x_bits=np.tile(x, (3, 1)))
    ref = X.quantize_act_lora_down_fp4(np.tile(x, (3, 1)), ones, pk["lora_down"])
    assert np.array_equal(got[1], ref["act_scales"]), np.argwhere(got[1] != ref["act_scales"])[:5]
    assert np.array_equal(got[0], ref["act_codes"]), np.argwhere(got[0] != ref["act_codes"])[:5]
    # the clamped blocks really clamp, and no code 8 (negative zero) appears
    assert np.all(ref["act_scales"][8:16, 0] == 0)
    codes = X.unpack_fp4(got[0])
    assert not np.any(codes == 8)
