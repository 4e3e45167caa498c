"""Pins of the MXFP4 oracle (oracle/mxfp4_oracle.py)."""
import numpy as np

import oracle as O
import oracle.mxfp4_oracle as X
import synthetic as S


def test_fp4_code_table():
    """E2M1: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0; code 1 is
    the subnormal 0.5 (OCP MX v1.0, FP4 E2M1 element format)."""
    for c in range(16):
        e, m, sgn = (c >> 1) & 3, c & 1, -1.0 if c & 8 else 1.0
        want = sgn * (m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))
        assert X.fp4_value(c) == want


def test_fp4_round_is_nearest_with_even_ties():
    """Against brute force over all 8 magnitudes on a dense grid with every
    midpoint: the nearest value wins, an exact tie takes the even code, above 6
    saturates."""
    vals = np.concatenate([np.linspace(-8, 8, 16001), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0],
                           -np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])])
    got = X.fp4_round(vals)
    for v, c in zip(vals, got):
        a = abs(v)
        d = np.abs(X.FP4_MAG - a)
        cands = np.flatnonzero(d == d.min())
        best = 7 if a > 6 else (cands[cands % 2 == 0][0] if len(cands) > 1 else cands[0])
        want = best | (8 if v < 0 and best != 0 else 0)
        assert c == want, (v, c, want)


def test_mx_block_scale_rule():
    """Shared exponent floor(log2 amax) - 2: the block maximum lands in [4, 8)
    before rounding (so it may saturate to 6); scaling a block by 2^k shifts the
    exponent by k and leaves the codes; an all-zero block is exponent -127 with
    zero codes; every element's error is at most half a step of its binade or
    the saturation error at the top."""
    rng = np.random.default_rng(0)
    v = rng.standard_normal((5, 128)) * rng.uniform(1e-3, 1e3, size=(5, 1))
    v[2, 32:64] = 0.0
    codes, e = X.mx_quantize_blocks(v)
    amax = np.abs(v.reshape(5, 4, 32)).max(-1)
    nz = amax > 0
    assert np.all(e[nz] == np.floor(np.log2(amax[nz])) - 2 + 127)
    assert e[2, 1] == 0 and np.all(codes[2, 32:64] == 0)
    c2, e2 = X.mx_quantize_blocks(v * 2.0 ** 5)
    assert np.array_equal(c2, codes) and np.array_equal(e2[nz], e[nz] + 5)
    deq = X.mx_dequantize(codes, e)
    scale = np.exp2(e.astype(np.float64) - 127).repeat(32, axis=1)
    err = np.abs(deq - v) / scale
    a = np.abs(v) / scale
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    assert np.all((err <= step / 2 + 1e-12) | (a > 6))


def test_fp4_packing_golden():
    """Hand-derived: values (0.5, -6, 1.5, 0) in a block with exponent 0 ->
    codes (1, 15, 3, 0) -> bytes 0xF1, 0x03."""
    v = np.zeros((1, 32))
    v[0, :4] = [0.5, -6.0, 1.5, 0.0]
    v[0, 4] = 4.0                                   # amax 6 -> e = floor(log2 6) - 2 = 0
    codes, e = X.mx_quantize_blocks(v)
    assert e[0, 0] == 127 and codes[0, :5].tolist() == [1, 15, 3, 0, 6]
    assert X.pack_fp4(codes)[0, :2].tolist() == [0xF1, 0x03]


def test_fp4_linear_exact_sum():
    """linear_output_fp4 is the dequantized product in float64: on a tiny case
    every product of two E2M1 values with power-of-two scales is exact, so the
    oracle equals a plain integer-scaled sum written out per element."""
    rng = np.random.default_rng(1)
    a = rng.integers(0, 16, (2, 64)).astype(np.uint8)
    w = rng.integers(0, 16, (3, 64)).astype(np.uint8)
    ea = rng.integers(120, 134, (2, 2)).astype(np.uint8)
    ew = rng.integers(120, 134, (3, 2)).astype(np.uint8)
    y, _ = X.linear_output_fp4(X.pack_fp4(a), ea, X.pack_fp4(w), ew, np.zeros((2, 0), np.uint16),
                               np.zeros((3, 0), np.uint16), None)
    for m in range(2):
        for n in range(3):
            tot = 0.0
            for k in range(64):
                tot += (X.fp4_value(a[m, k]) * 2.0 ** (int(ea[m, k // 32]) - 127)) * \
                       (X.fp4_value(w[n, k]) * 2.0 ** (int(ew[n, k // 32]) - 127))
            assert y[m, n] == tot


def test_fp4_whole_layer_reduces_to_plain_mxfp4_and_tracks_the_dense_layer():
    """Rank 0 with lambda = 1 is plain MXFP4 (dequantize both operands, one
    float64 matmul, written out here); with the real split and smoothing the
    layer is closer to the dense X W^T + b than plain MXFP4 on outlier inputs."""
    spec = S.LinearSpec("fp4pin", 9, 32, 256, 64, 16, outlier_channels=4, outlier_scale=50.0)
    d = S.make_linear(spec)
    ones = np.ones(256, dtype=np.float32)
    p0 = X.pack_weights_fp4(d["w"], ones, 0)
    a0 = X.quantize_act_lora_down_fp4(d["x"], ones, p0["lora_down"])
    y0, _ = X.linear_output_fp4(a0["act_codes"], a0["act_scales"], p0["w_codes"], p0["w_scales"],
                                a0["lora_act"], p0["lora_up"], d["bias"])
    xq = X.mx_dequantize(*X.mx_quantize_blocks(O.bf16_to_f64(d["x"])))
    wq = X.mx_dequantize(*X.mx_quantize_blocks(O.bf16_to_f64(d["w"])))
    assert np.allclose(y0, xq @ wq.T + O.bf16_to_f64(d["bias"]), rtol=1e-12, atol=1e-12)
    lam = O.smooth_factors(O.activation_absmax(d["x"]), d["w"])
    p = X.pack_weights_fp4(d["w"], lam, 16)
    a = X.quantize_act_lora_down_fp4(d["x"], lam, p["lora_down"])
    y, _ = X.linear_output_fp4(a["act_codes"], a["act_scales"], p["w_codes"], p["w_scales"], a["lora_act"],
                               p["lora_up"], d["bias"])
    dense = O.bf16_to_f64(d["x"]) @ O.bf16_to_f64(d["w"]).T + O.bf16_to_f64(d["bias"])
    assert np.linalg.norm(y - dense) < 0.7 * np.linalg.norm(y0 - dense)
