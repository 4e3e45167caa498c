"""Pins of the AWQ W4A16 oracle (oracle/awq_oracle.py) against closed forms,
textbook reductions and exact rationals."""
from fractions import Fraction

import numpy as np

import oracle as O
import oracle.awq_oracle as A
import synthetic as S


def _rng(seed):
    return np.random.default_rng(seed)


def test_uint4_packing_golden():
    """Hand-derived: codes (1, 2, 15, 0) -> bytes 0x21, 0x0F (element 2i low)."""
    q = np.array([[1, 2, 15, 0]], dtype=np.uint8)
    assert A.pack_uint4(q).tolist() == [[0x21, 0x0F]]
    assert np.array_equal(A.unpack_uint4(A.pack_uint4(q)), q)


def test_asym_quantizer_closed_forms():
    """Codes stay in 0..15; where the value is inside the grid's range the
    reconstruction error is at most Delta/2; a group whose minimum is 0 has
    z = 0 and q = rint(w / Delta); a constant positive group has its range
    clamped to 1e-5 and, the zero point being clamped to the code range, lies
    above the grid [0, 15 Delta]: every code clips to 15."""
    rng = _rng(1)
    w = rng.standard_normal((6, 256)) * rng.uniform(0.01, 3, size=(6, 1))
    w[1] = np.abs(w[1]); w[1, 0::64] = 0.0                     # min 0 in every group
    w[2] = 0.37                                                # constant row
    w[3] = -np.abs(w[3])                                       # all non-positive
    q, dbits, z = A.quantize_asym_groups(w)
    assert q.max() <= 15 and z.max() <= 15
    d = O.bf16_to_f64(dbits)
    rec = A.dequantize_asym(q, dbits, z)
    lo = (0.0 - z) * d
    hi = (15.0 - z) * d
    wg = w.reshape(6, 4, 64)
    inside = (wg >= lo[..., None]) & (wg <= hi[..., None])
    err = np.abs(rec.reshape(6, 4, 64) - wg)
    assert np.all(err[inside] <= (d[..., None] / 2 * (1 + 1e-12)).repeat(64, -1)[inside])
    assert np.all(z[1] == 0)
    assert np.array_equal(q[1].reshape(4, 64), np.clip(np.rint(wg[1] / d[1][:, None]), 0, 15))
    assert np.all(dbits[2] == O.f64_to_bf16(np.array([1e-5 / 15]))[0]) and np.all(z[2] == 0)
    assert np.all(q[2] == 15)


def test_awq_alpha_zero_is_plain_round_to_nearest():
    """alpha = 0 gives s = 1 exactly, and the layer error of the search's first
    grid point equals that of textbook min/max round-to-nearest group
    quantization, written out here per group with scalar loops."""
    rng = _rng(2)
    w = S.to_bf16_bits(rng.standard_normal((3, 128)) * 0.05)
    x = S.to_bf16_bits(rng.standard_normal((5, 128)))
    s = A.awq_scales(A.activation_mean_abs(x), 0.0)
    assert np.all(s == 1.0)
    wf, xf = O.bf16_to_f64(w), O.bf16_to_f64(x)
    rtn = np.empty_like(wf)
    for n in range(3):
        for g in range(2):
            v = wf[n, 64 * g:64 * g + 64]
            step = float(O.bf16_to_f64(O.f64_to_bf16(np.array([max(v.max() - v.min(), 1e-5) / 15]))[0]))
            zero = min(max(round(-v.min() / step), 0), 15)   # Python round: half to even
            for j in range(64):
                code = min(max(round(v[j] / step) + zero, 0), 15)
                rtn[n, 64 * g + j] = (code - zero) * step
    want = float((((xf @ wf.T) - (xf @ rtn.T)) ** 2).mean())
    assert abs(A.awq_loss(x, w, s) - want) <= 1e-15 * max(want, 1e-300)


def test_awq_scales_normalization_and_power():
    """max(s) * min(s) = 1 (up to the fp32 rounding) and s_i / s_j = (a_i / a_j)^alpha."""
    a = _rng(3).uniform(0.01, 5.0, 64)
    for alpha in (0.25, 0.5, 0.95):
        s = A.awq_scales(a, alpha).astype(np.float64)
        assert abs(s.max() * s.min() - 1.0) < 1e-6
        assert np.allclose(s / s[0], (a / a[0]) ** alpha, rtol=1e-6)


def test_awq_search_is_never_worse_than_rtn_and_helps_salient_channels():
    """The grid holds alpha = 0, so the chosen error is at most plain RTN's; with
    a few activation channels 10x larger than the rest (salient channels) the
    activation-aware scale cuts the error clearly."""
    spec = S.LinearSpec("awqpin", 9, 48, 256, 96, 0, outlier_frac=0.03, outlier_scale=10.0,
                        silu_input=True)
    x = S.make_calibration(spec, 48)
    w = S.make_w(spec)
    alpha, s, losses = A.awq_search(x, w)
    assert losses.min() <= losses[0]
    assert alpha > 0 and losses.min() < 0.8 * losses[0], (alpha, losses.min() / losses[0])


def test_awq_linear_exact_rationals():
    """The whole layer on a tiny case in exact rationals (smoothing rounded as
    the definition says, then the dequantized sum) against the float64 oracle."""
    rng = _rng(4)
    M, N, K = 2, 3, 128
    x = S.to_bf16_bits(rng.standard_normal((M, K)))
    w = S.to_bf16_bits(rng.standard_normal((N, K)) * 0.1)
    b = S.to_bf16_bits(rng.standard_normal(N) * 0.01)
    pk = A.awq_pack(x, w)
    y, _ = A.awq_linear(x, pk["smooth"], pk["codes"], pk["scales"], pk["zeros"], b)
    xh = O.bf16_to_f64(O.smooth_activations(x, pk["smooth"]))
    q = A.unpack_uint4(pk["codes"])
    d = O.bf16_to_f64(pk["scales"])
    for m in range(M):
        for n in range(N):
            tot = Fraction(float(O.bf16_to_f64(b)[n]))
            for k in range(K):
                g = k // 64
                tot += Fraction(float(xh[m, k])) * (int(q[n, k]) - int(pk["zeros"][n, g])) * Fraction(float(d[n, g]))
            assert abs(float(tot) - y[m, n]) <= 1e-14 * max(abs(float(tot)), 1e-300)


def test_awq_linear_rows_select():
    rng = _rng(5)
    x = S.to_bf16_bits(rng.standard_normal((7, 64)))
    w = S.to_bf16_bits(rng.standard_normal((32, 64)) * 0.1)
    pk = A.awq_pack(x, w)
    full, fb = A.awq_linear(x, pk["smooth"], pk["codes"], pk["scales"], pk["zeros"], None)
    sub, sb = A.awq_linear(x, pk["smooth"], pk["codes"], pk["scales"], pk["zeros"], None, rows=[6, 0])
    assert np.array_equal(sb, fb[[6, 0]])
