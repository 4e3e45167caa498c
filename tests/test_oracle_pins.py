"""Pins of the oracle against things other than itself.

Closed forms, invariants, reductions to library routines, brute force in exact
rationals, and hand-derived examples (tests/golden).  CPU only.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.exact import bf16 as ex_bf16
from tests.exact import fl32 as ex_fl32
from tests.exact import rne_int

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- rounding ---

def test_f32_to_bf16_equals_torch_cast_including_ties():
    rng = np.random.default_rng(1)
    a = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    u = a.view(np.uint32).copy()
    # exact ties: lower 16 bits = 0x8000, both parities of bit 16
    ties = (u[:4000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    below = (u[4000:6000] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    above = (u[6000:8000] & np.uint32(0xFFFF0000)) | np.uint32(0x8001)
    allv = np.concatenate([a, ties.view(np.float32), below.view(np.float32), above.view(np.float32),
                           np.array([0.0, -0.0, 1.0, -1.0], np.float32)])
    ours = O.f32_to_bf16(allv)
    ref = torch.from_numpy(allv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_is_single_rounding():
    rng = np.random.default_rng(2)
    v = rng.standard_normal(3000) * np.exp(rng.uniform(-10, 10, 3000))
    # near-ties where float64->float32->bf16 double rounding would go wrong
    base = O.bf16_to_f64(O.f64_to_bf16(v[:500]))
    ulp = np.abs(base) * 2.0 ** -7
    near = base + ulp / 2 + np.sign(base) * ulp * 2.0 ** -30
    near2 = base + ulp / 2 - np.sign(base) * ulp * 2.0 ** -30
    exact_tie = base + ulp / 2
    vals = np.concatenate([v, near, near2, exact_tie])
    got = O.bf16_to_f64(O.f64_to_bf16(vals))
    for x, g in zip(vals, got):
        assert Fraction(float(g)) == ex_bf16(Fraction(float(x))), x


def test_f64_to_f32_matches_exact_rounding():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(2000) * np.exp(rng.uniform(-20, 20, 2000))
    got = O.f64_to_f32(v)
    for x, g in zip(v, got):
        assert Fraction(float(g)) == ex_fl32(Fraction(float(x)))


# ----------------------------------------------------------------- packing ---

def test_packing_golden_and_roundtrip():
    gold = json.load(open(os.path.join(GOLD, "int4_packing.json")))
    q = np.array([gold["codes"]], dtype=np.int8)
    assert O.pack_int4(q)[0].tolist() == gold["bytes"]
    allq = np.arange(-8, 8, dtype=np.int8)
    grid = np.array(np.meshgrid(allq, allq)).reshape(2, -1).T.reshape(1, -1)
    assert np.array_equal(O.unpack_int4(O.pack_int4(grid)), grid)
    # every byte value decodes and re-encodes to itself
    b = np.arange(256, dtype=np.uint8)[None, :]
    assert np.array_equal(O.pack_int4(O.unpack_int4(b)), b)


def test_storage_order_golden():
    """Rows 8-15 of every 16 hold their 8-byte halves exchanged; a hand-derived
    9-row example (rows 0-7 plain, row 8 exchanged) and the round trip over 40
    rows of random codes."""
    gold = json.load(open(os.path.join(GOLD, "int4_storage_order.json")))
    q = np.tile(np.array(gold["codes_every_row"], dtype=np.int8), (gold["rows"], 1))
    b = O.pack_int4(q)
    for r in range(8):
        assert b[r].tolist() == gold["bytes_row0"], r
    assert b[8].tolist() == gold["bytes_row8"]
    rq = np.random.default_rng(5).integers(-8, 8, size=(40, 128)).astype(np.int8)
    assert np.array_equal(O.unpack_int4(O.pack_int4(rq)), rq)
    with pytest.raises(ValueError):
        O.pack_int4(np.zeros((9, 8), np.int8))  # 4-byte rows cannot hold the order


# ------------------------------------------------------ golden quantization ---

def _golden_act_inputs(gold):
    K = 256
    x = np.zeros((1, K))
    for gi, key in enumerate(["group0", "group1", "group2", "group3"]):
        for k, v in gold["x_nonzero"][key]:
            x[0, gi * 64 + k] = v
    lam = np.repeat(np.array(gold["lambda_groups"], np.float32), 64)
    return O.f64_to_bf16(x), lam


def test_activation_quant_golden():
    gold = json.load(open(os.path.join(GOLD, "act_quant_example.json")))
    x_bits, lam = _golden_act_inputs(gold)
    out = O.quantize_act_lora_down(x_bits, lam, np.zeros((0, 256), np.uint16))
    assert out["act_scales"][0].tolist() == gold["scale_bits"]
    for gi, key in enumerate(["group0", "group1", "group2", "group3"]):
        want = np.zeros(64, np.int8)
        for k, v in gold["q_nonzero"][key]:
            want[k] = v
        assert np.array_equal(out["q_x"][0, gi * 64:(gi + 1) * 64], want), key
        nb = len(gold["packed_first_bytes"][key])
        got = out["act_codes"][0, gi * 32: gi * 32 + nb].tolist()
        assert got == gold["packed_first_bytes"][key], key


def test_weight_quant_and_linear_golden():
    gold = json.load(open(os.path.join(GOLD, "weight_quant_example.json")))
    R = np.zeros((1, 64))
    for k, v in gold["residual_nonzero"]:
        R[0, k] = v
    q, s_bits = O.quantize_weight_groups(R)
    assert int(s_bits[0, 0]) == gold["scale_bits"]
    want = np.zeros(64, np.int8)
    for k, v in gold["q_nonzero"]:
        want[k] = v
    assert np.array_equal(q[0], want)
    assert O.pack_int4(q)[0, :4].tolist() == gold["packed_first_bytes"]
    # the 1x64x1 linear with rank 0 and lambda = 1 (R = W)
    lin = gold["linear"]
    x = np.zeros((1, 64))
    for k, v in lin["x_nonzero"]:
        x[0, k] = v
    w_bits = O.f64_to_bf16(R)
    lam = np.ones(64, np.float32)
    packed = O.pack_weights(w_bits, lam, r=0)
    bias = O.f64_to_bf16(np.array([lin["bias"]]))
    a, y, y_bits = O.forward(O.f64_to_bf16(x), lam, packed, bias)
    acc = O.group_accumulators(a["act_codes"], packed["w_codes"])
    assert int(acc[0, 0, 0]) == lin["acc"]
    assert float(y[0, 0]) == lin["y"]
    assert int(y_bits[0, 0]) == lin["y_bits"]


# ----------------------------------------------------------- smoothing (O1) ---

def test_smoothing_preserves_the_product_exactly():
    """X diag(1/lambda) (W diag(lambda))^T = X W^T in exact arithmetic."""
    d = S.make_linear("tiny")
    lam = O.smooth_factors(O.activation_absmax(d["x"]), d["w"])
    x = O.bf16_to_f64(d["x"])
    w = O.bf16_to_f64(d["w"])
    lhs = (x / lam.astype(np.float64)) @ O.smoothed_weight(d["w"], lam).T
    rhs = x @ w.T
    assert np.linalg.norm(lhs - rhs) <= 1e-14 * np.linalg.norm(rhs)


def test_smoothing_factor_definition_and_outlier_channels():
    d = S.make_linear("tiny")
    a = O.activation_absmax(d["x"])
    lam = O.smooth_factors(a, d["w"])
    wmax = np.abs(O.bf16_to_f64(d["w"])).max(axis=0)
    # lambda^2 * max|W_j| = max|X_j| up to float32 rounding of lambda
    assert np.allclose(lam.astype(np.float64) ** 2 * wmax, a, rtol=3e-7)
    # after smoothing, the activation and weight channel maxima are balanced
    xs = a / lam
    ws = wmax * lam
    assert np.allclose(xs, ws, rtol=3e-7)
    # the outlier channels (x50) get the largest lambdas
    top = np.argsort(a)[-4:]
    assert set(top) == set(np.argsort(lam)[-4:])
    # zero channel is clamped, not 0 or inf
    lam0 = O.smooth_factors(np.zeros(4), np.zeros((2, 4), np.uint16))
    assert np.all(lam0 == np.float32(1.0))


# ----------------------------------------------------- low-rank split (O3/4) ---

def _spiky_matrix(N, K, r_spikes, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K)) * 0.02
    u = rng.standard_normal((N, r_spikes))
    v = rng.standard_normal((r_spikes, K))
    w += (u * np.linspace(0.5, 0.1, r_spikes)) @ v * 0.05
    return O.f64_to_bf16(w)


@pytest.mark.parametrize("r", [1, 4, 16])
def test_lowrank_split_eckart_young(r):
    """The unrounded factors reach the Eckart-Young bound; sigma from eigvalsh of W'W'^T."""
    w_bits = _spiky_matrix(96, 128, 8, 4)
    lam = np.exp(np.random.default_rng(5).uniform(-1, 1, 128)).astype(np.float32)
    ws = O.smoothed_weight(w_bits, lam)
    down, up, resid, sv = O.lowrank_split(ws, r)
    eig = np.sort(np.linalg.eigvalsh(ws @ ws.T))[::-1]
    tail = eig[r:].sum()
    # rounded factors: residual energy is the tail plus the factor-rounding error
    lowrank = O.bf16_to_f64(up) @ O.bf16_to_f64(down)
    assert np.linalg.norm(ws - lowrank - resid) <= 1e-13 * np.linalg.norm(ws)
    # the product of the factors approximates the best rank-r part to bf16 precision
    best = ws - 0.0
    uu, ss, vv = np.linalg.svd(ws)
    best = (uu[:, :r] * ss[:r]) @ vv[:r]
    assert np.linalg.norm(lowrank - best) <= 2.0 ** -7 * np.linalg.norm(best)
    # the residual energy matches the tail of the spectrum up to that error
    err = np.linalg.norm(lowrank - best)
    assert abs(np.linalg.norm(resid) - np.sqrt(tail)) <= err + 1e-12
    # split convention: singular values shared evenly between the factors
    up_n = np.linalg.norm(O.bf16_to_f64(up), axis=0)
    down_n = np.linalg.norm(O.bf16_to_f64(down), axis=1)
    assert np.allclose(up_n, np.sqrt(np.sqrt(eig[:r])), rtol=1e-2)
    assert np.allclose(down_n, np.sqrt(np.sqrt(eig[:r])), rtol=1e-2)


def test_lowrank_split_rank0_is_identity():
    w_bits = _spiky_matrix(32, 64, 4, 6)
    ws = O.smoothed_weight(w_bits, np.ones(64, np.float32))
    down, up, resid, _ = O.lowrank_split(ws, 0)
    assert down.shape == (0, 64) and up.shape == (32, 0)
    assert np.array_equal(resid, ws)


# -------------------------------------------------------- quantizers (O5/O7) ---

def _quant_props(v, q, s, group, slack):
    M, K = v.shape
    vg = v.reshape(M, K // group, group)
    qg = q.reshape(M, K // group, group).astype(np.float64)
    assert np.all(np.abs(qg) <= 7)
    err = np.abs(vg - qg * s[:, :, None])
    assert np.all(err <= s[:, :, None] / 2 * (1 + slack) + 0.0)
    nz = s > 0
    assert np.all(np.abs(qg).max(axis=2)[nz] == 7)
    assert np.all(qg[~nz] == 0)


def test_activation_quantizer_properties():
    d = S.make_linear("tiny")
    lam = O.smooth_factors(O.activation_absmax(d["x"]), d["w"])
    xh_bits = O.smooth_activations(d["x"], lam)
    q, s_bits = O.quantize_activation_groups(xh_bits)
    _quant_props(O.bf16_to_f64(xh_bits), q, O.bf16_to_f64(s_bits), 64, 2.0 ** -20)
    # sign symmetry
    neg = xh_bits ^ np.uint16(0x8000)
    qn, sn = O.quantize_activation_groups(neg)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s_bits)
    # power-of-two covariance: codes unchanged, scales scale
    xh4 = O.f64_to_bf16(O.bf16_to_f64(xh_bits) * 4.0)
    q4, s4 = O.quantize_activation_groups(xh4)
    assert np.array_equal(q4, q)
    assert np.array_equal(O.bf16_to_f64(s4), 4.0 * O.bf16_to_f64(s_bits))


def test_weight_quantizer_properties():
    rng = np.random.default_rng(7)
    R = rng.standard_normal((16, 256)) * 0.03
    R[3, 64:128] = 0.0
    q, s_bits = O.quantize_weight_groups(R)
    _quant_props(R, q, O.bf16_to_f64(s_bits), 64, 2.0 ** -40)
    qn, sn = O.quantize_weight_groups(-R)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s_bits)
    q8, s8 = O.quantize_weight_groups(R * 8.0)
    assert np.array_equal(q8, q) and np.array_equal(O.bf16_to_f64(s8), 8 * O.bf16_to_f64(s_bits))


def test_quantizer_is_nearest_code_by_brute_force():
    rng = np.random.default_rng(8)
    R = rng.standard_normal((8, 64))
    q, s_bits = O.quantize_weight_groups(R)
    s = O.bf16_to_f64(s_bits)
    for i in range(8):
        for k in range(64):
            cands = np.arange(-7, 8)
            d = np.abs(R[i, k] - cands * s[i, 0])
            best = cands[d == d.min()]
            if len(best) == 1:
                assert q[i, k] == best[0]
            else:  # exact tie: even code
                assert q[i, k] in best and q[i, k] % 2 == 0


# ------------------------------------------- brute force in exact rationals ---

def _exact_pipeline(x_bits, lam, down_bits, w_codes, w_scale_bits, up_bits, bias_bits):
    """Whole call-1 + call-2 computation in Fractions, every rounding exact."""
    M, K = x_bits.shape
    N = w_codes.shape[0]
    r = down_bits.shape[0]
    G = K // 64
    X = [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(x_bits)]
    L = [Fraction(float(v)) for v in lam]
    D = [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(down_bits)]
    U = [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(up_bits)]
    B = [Fraction(float(v)) for v in O.bf16_to_f64(bias_bits)]
    SW = [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(w_scale_bits)]
    # decode weight codes bit by bit
    QW = []
    for row in w_codes:
        vals = []
        for byte in row:
            for nib in (int(byte) & 15, int(byte) >> 4):
                vals.append(nib - 16 if nib >= 8 else nib)
        QW.append(vals)
    mu = [ex_fl32(1 / l) for l in L]
    xh = [[ex_bf16(ex_fl32(X[m][k] * mu[k])) for k in range(K)] for m in range(M)]
    qx, sx = [], []
    for m in range(M):
        qrow, srow = [], []
        for g in range(G):
            seg = xh[m][g * 64:(g + 1) * 64]
            A = max(abs(v) for v in seg)
            s = ex_bf16(ex_fl32(A / 7))
            srow.append(s)
            if s == 0:
                qrow += [0] * 64
            else:
                io = ex_fl32(1 / s)
                qrow += [max(-7, min(7, rne_int(v * io))) for v in seg]
        qx.append(qrow)
        sx.append(srow)
    la = [[ex_bf16(sum(xh[m][k] * D[j][k] for k in range(K))) for j in range(r)] for m in range(M)]
    Y = []
    for m in range(M):
        yrow = []
        for n in range(N):
            y = Fraction(0)
            for g in range(G):
                acc = sum(qx[m][k] * QW[n][k] for k in range(g * 64, (g + 1) * 64))
                y += sx[m][g] * SW[n][g] * acc
            y += sum(la[m][j] * U[n][j] for j in range(r))
            y += B[n]
            yrow.append(y)
        Y.append(yrow)
    return qx, sx, la, Y


@pytest.mark.parametrize("K,r", [(64, 0), (64, 1), (128, 1), (128, 0)])
def test_whole_layer_against_exact_rationals(K, r):
    rng = np.random.default_rng(100 + K + r)
    M, N = 2, 2
    x = rng.standard_normal((M, K))
    x[:, 3] *= 40
    x_bits = O.f64_to_bf16(x)
    w_bits = O.f64_to_bf16(rng.standard_normal((N, K)) * 0.02)
    lam = O.smooth_factors(O.activation_absmax(x_bits), w_bits)
    packed = O.pack_weights(w_bits, lam, r)
    bias = O.f64_to_bf16(rng.standard_normal(N) * 0.01)
    a, y, _ = O.forward(x_bits, lam, packed, bias)
    qx, sx, la, Y = _exact_pipeline(x_bits, lam, packed["lora_down"], packed["w_codes"],
                                    packed["w_scales"], packed["lora_up"], bias)
    assert a["q_x"].astype(int).tolist() == qx
    assert [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(a["act_scales"])] == sx
    assert [[Fraction(float(v)) for v in row] for row in O.bf16_to_f64(a["lora_act"])] == la
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(y[m, n])) - Y[m][n]) <= abs(Y[m][n]) * Fraction(1, 10 ** 15)


def test_weight_quantization_against_exact_rationals():
    rng = np.random.default_rng(9)
    w_bits = O.f64_to_bf16(rng.standard_normal((3, 128)) * 0.02)
    lam = np.exp(rng.uniform(-1, 1, 128)).astype(np.float32)
    packed = O.pack_weights(w_bits, lam, 2)
    W = O.bf16_to_f64(w_bits)
    U = O.bf16_to_f64(packed["lora_up"])
    D = O.bf16_to_f64(packed["lora_down"])
    qw = O.unpack_int4(packed["w_codes"])
    sw = O.bf16_to_f64(packed["w_scales"])
    for n in range(3):
        for g in range(2):
            Rg = [Fraction(float(W[n, k])) * Fraction(float(lam[k]))
                  - sum(Fraction(float(U[n, j])) * Fraction(float(D[j, k])) for j in range(2))
                  for k in range(g * 64, (g + 1) * 64)]
            A = max(abs(v) for v in Rg)
            s = ex_bf16(A / 7)
            assert Fraction(float(sw[n, g])) == s
            for i, v in enumerate(Rg):
                assert qw[n, g * 64 + i] == max(-7, min(7, rne_int(v / s)))


# ------------------------------------------------- method-level reductions ---

def _textbook_w4a4(act_codes, act_scales, w_codes, w_scales, bias):
    """Dequantize both operands, then one matmul (written independently)."""
    def deq(codes, scales):
        q = O.unpack_int4(codes).astype(np.float64)
        s = O.bf16_to_f64(scales)
        return q * np.repeat(s, 64, axis=1)
    return deq(act_codes, act_scales) @ deq(w_codes, w_scales).T + O.bf16_to_f64(bias)[None, :]


def test_rank0_unit_smoothing_is_plain_w4a4():
    d = S.make_linear("tiny")
    lam = np.ones(d["spec"].K, np.float32)
    packed = O.pack_weights(d["w"], lam, 0)
    a, y, _ = O.forward(d["x"], lam, packed, d["bias"])
    # lambda = 1: x_hat is X itself; rank 0: the residual is W itself
    assert np.array_equal(a["xhat"], d["x"])
    qw, sw = O.quantize_weight_groups(O.bf16_to_f64(d["w"]))
    assert np.array_equal(packed["w_codes"], O.pack_int4(qw))
    ref = _textbook_w4a4(a["act_codes"], a["act_scales"], packed["w_codes"], packed["w_scales"], d["bias"])
    assert np.linalg.norm(y - ref) <= 1e-12 * np.linalg.norm(ref)


def test_zero_residual_is_the_bf16_lowrank_gemm():
    rng = np.random.default_rng(11)
    M, K, N, r = 8, 128, 16, 4
    down = O.f64_to_bf16(rng.standard_normal((r, K)) * 0.1)
    up = O.f64_to_bf16(rng.standard_normal((N, r)) * 0.1)
    ws = O.bf16_to_f64(up) @ O.bf16_to_f64(down)          # exactly representable W'
    resid = ws - O.bf16_to_f64(up) @ O.bf16_to_f64(down)
    assert not resid.any()
    qw, sw = O.quantize_weight_groups(resid)
    assert not qw.any() and not sw.any()
    x_bits = O.f64_to_bf16(rng.standard_normal((M, K)))
    lam = np.ones(K, np.float32)
    a = O.quantize_act_lora_down(x_bits, lam, down)
    bias = O.f64_to_bf16(rng.standard_normal(N) * 0.01)
    y, _ = O.linear_output(a["act_codes"], a["act_scales"], O.pack_int4(qw), sw, a["lora_act"], up, bias)
    exact = O.bf16_to_f64(a["lora_act"]) @ O.bf16_to_f64(up).T + O.bf16_to_f64(bias)
    assert np.array_equal(y, exact)
    dense = O.bf16_to_f64(x_bits) @ ws.T + O.bf16_to_f64(bias)
    assert np.linalg.norm(y - dense) <= 2.0 ** -8 * np.linalg.norm(dense)


def test_group_accumulator_bound_and_group_permutation_invariance():
    d = S.make_linear("tiny")
    K = d["spec"].K
    lam = O.smooth_factors(O.activation_absmax(d["x"]), d["w"])
    packed = O.pack_weights(d["w"], lam, 0)
    a, y, _ = O.forward(d["x"], lam, packed, d["bias"])
    acc = O.group_accumulators(a["act_codes"], packed["w_codes"])
    assert np.abs(acc).max() <= 64 * 49
    perm_g = np.array([2, 0, 3, 1])
    perm_k = np.concatenate([np.arange(g * 64, (g + 1) * 64) for g in perm_g])
    x2, w2, lam2 = d["x"][:, perm_k], d["w"][:, perm_k], lam[perm_k]
    packed2 = O.pack_weights(w2, lam2, 0)
    a2, y2, _ = O.forward(x2, lam2, packed2, d["bias"])
    acc2 = O.group_accumulators(a2["act_codes"], packed2["w_codes"])
    assert np.array_equal(acc2, acc[:, :, perm_g])
    assert np.allclose(y2, y, rtol=0, atol=1e-12 * np.abs(y).max())


def test_svdquant_beats_plain_w4a4_on_outlier_inputs():
    """Method-level sanity: smoothing + low rank lowers the layer error (soft pin)."""
    d = S.make_linear("tiny")
    x = O.bf16_to_f64(d["x"])
    ref = x @ O.bf16_to_f64(d["w"]).T + O.bf16_to_f64(d["bias"])
    errs = {}
    lam1 = np.ones(d["spec"].K, np.float32)
    _, y0, _ = O.forward(d["x"], lam1, O.pack_weights(d["w"], lam1, 0), d["bias"])
    errs["plain"] = np.linalg.norm(y0 - ref) / np.linalg.norm(ref)
    lam = O.smooth_factors(O.activation_absmax(d["x"]), d["w"])
    for r in (0, 16, 32):
        _, y, _ = O.forward(d["x"], lam, O.pack_weights(d["w"], lam, r), d["bias"])
        errs[r] = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert errs[0] < errs["plain"]
    assert errs[16] < errs[0] and errs[32] < errs[16]


def test_weight_scale_is_one_rounding_at_a_constructed_near_tie():
    """A/7 just above a bf16 midpoint whose lower neighbour is even: one rounding
    from float64 goes up; a detour through float32 would land on the tie and go
    down to the even neighbour."""
    b_lo = O.bf16_to_f64(np.array([0x3C10], np.uint16))[0]      # even mantissa
    b_hi = O.bf16_to_f64(np.array([0x3C11], np.uint16))[0]
    tie = (b_lo + b_hi) / 2
    target = tie * (1 + 2.0 ** -35)
    R = np.zeros((1, 64))
    R[0, 0] = 7.0 * target
    R[0, 1] = -0.3 * target
    q, s_bits = O.quantize_weight_groups(R)
    assert Fraction(float(O.bf16_to_f64(s_bits)[0, 0])) == ex_bf16(Fraction(float(R[0, 0])) / 7)
    assert int(s_bits[0, 0]) == 0x3C11


def test_activation_quantizer_tiny_groups_reading():
    """Reading for a case the pages leave open: a group whose scale s is so small
    that fl32(1/s) overflows (s < 2^-128) quantizes to zero, like s = 0.  Just
    above that, s = 2^-127 gives iota = 2^127 and the exact codes."""
    xh = np.zeros((1, 128))
    xh[0, :64] = np.linspace(-1.0, 1.0, 64) * 7.0 * 2.0 ** -127      # s = 2^-127
    xh[0, 64:] = np.linspace(-1.0, 1.0, 64) * 7.0 * 2.0 ** -130      # s < 2^-128
    bits = O.f64_to_bf16(xh)
    q, s_bits = O.quantize_activation_groups(bits)
    s = O.bf16_to_f64(s_bits)[0]
    assert s[0] == 2.0 ** -127 and 0 < s[1] < 2.0 ** -128
    xv = O.bf16_to_f64(bits)[0]
    assert np.array_equal(q[0, :64], np.clip(np.rint(xv[:64] / s[0]), -7, 7))
    assert q[0, 0] == -7 and q[0, 63] == 7
    assert not np.any(q[0, 64:])


def test_gelu_tanh_pins():
    """The tanh-form GELU against closed forms: g(x) - g(-x) = x exactly (the
    tanh terms cancel), g(0) = 0, g -> x for large x and -> 0 for large -x, and
    the exact GELU x*Phi(x) (math.erf) within the approximation's error."""
    import math
    x = np.linspace(-8, 8, 4001)
    g = O.gelu_tanh(x)
    assert np.allclose(g - O.gelu_tanh(-x), x, rtol=0, atol=1e-13)
    assert O.gelu_tanh(0.0) == 0.0
    assert abs(O.gelu_tanh(12.0) - 12.0) < 1e-12 and abs(O.gelu_tanh(-12.0)) < 1e-12
    exact = np.array([v * 0.5 * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x])
    err = np.abs(g - exact).max()
    assert 1e-5 < err < 1e-3, err


def test_mlp_pair_chains_the_two_calls():
    """mlp_pair is call 1 + call 2 (GELU) on the up weights, then call 1 + call 2
    on the bf16 GELU output with the down weights, each step as defined above;
    a row subset gives the same rows (every step is per token once lambda is fixed)."""
    up = S.LinearSpec("pair_up", 9, 48, 128, 192, 16, outlier_channels=3, outlier_scale=20.0,
                      row_outlier_frac=0.05)
    dn = S.LinearSpec("pair_dn", 9, 48, 192, 128, 16, layer_id=1)
    du = S.make_linear(up)
    wd, bd = S.make_w(dn), S.make_bias(dn)
    lam_u = O.smooth_factors(O.activation_absmax(du["x"]), du["w"])
    pu = O.pack_weights(du["w"], lam_u, 16)
    a_u, y_u, _ = O.forward(du["x"], lam_u, pu, du["bias"])
    h = O.f64_to_bf16(O.gelu_tanh(y_u))
    lam_d = O.smooth_factors(O.activation_absmax(O.float_mlp_hidden(du["x"], du["w"], du["bias"])), wd)
    pd = O.pack_weights(wd, lam_d, 16)
    res = O.mlp_pair(du["x"], lam_u, pu, du["bias"], lam_d, pd, bd)
    assert np.array_equal(res["h"], h)
    _, y_d, yb_d = O.forward(h, lam_d, pd, bd)
    assert np.array_equal(res["y_bits"], yb_d) and np.array_equal(res["y"], y_d)
    rows = [0, 5, 47]
    sub = O.mlp_pair(du["x"], lam_u, pu, du["bias"], lam_d, pd, bd, rows=rows)
    assert np.array_equal(sub["y_bits"], res["y_bits"][rows]) and np.array_equal(sub["h"], h[rows])


def test_float_mlp_hidden_brute_force():
    """The calibration activations against scalar loops in exact rationals on a
    tiny case (the tanh itself in float64)."""
    import math
    from fractions import Fraction
    rng = np.random.default_rng(3)
    x = S.to_bf16_bits(rng.standard_normal((3, 5)))
    w = S.to_bf16_bits(rng.standard_normal((4, 5)) * 0.5)
    b = S.to_bf16_bits(rng.standard_normal(4) * 0.1)
    got = O.float_mlp_hidden(x, w, b)
    xf, wf, bf = (S.bf16_bits_to_f32(a).astype(np.float64) for a in (x, w, b))
    for m in range(3):
        for n in range(4):
            z = float(sum(Fraction(xf[m, k]) * Fraction(wf[n, k]) for k in range(5)) + Fraction(bf[n]))
            g = 0.5 * z * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))
            want = O.f64_to_bf16(np.array([g]))[0]
            assert abs(int(got[m, n]) - int(want)) <= 1, (m, n, got[m, n], want)


def test_pair_up_rows_carry_outliers():
    """The synthetic up-projection of the chained pair scales round(1 % of N)
    output channels by 30 (rows of W and the bias), the rest as the plain spec."""
    spec = S.LinearSpec("rows", 9, 8, 64, 300, 16, row_outlier_frac=0.01, outlier_scale=30.0)
    plain = S.LinearSpec("rows", 9, 8, 64, 300, 16, outlier_scale=30.0)
    w, w0 = S.bf16_bits_to_f32(S.make_w(spec)), S.bf16_bits_to_f32(S.make_w(plain))
    ratio = np.abs(w).max(axis=1) / np.abs(w0).max(axis=1)
    big = np.flatnonzero(np.abs(ratio - 30.0) < 0.5)
    assert big.size == 3 and np.all(np.abs(ratio[np.setdiff1d(np.arange(300), big)] - 1.0) < 1e-6)


def test_rms_norm_heads_closed_forms():
    """With unit scales each head row of the output has mean square ms/(ms+eps)
    (exactly 1 for eps = 0) and the direction of the input; a positive factor on
    the input cancels when eps = 0; the scale multiplies channel-wise."""
    rng = np.random.default_rng(5)
    y = rng.standard_normal((7, 3 * 16)) * rng.uniform(0.1, 10, size=(7, 1))
    ones = O.f64_to_bf16(np.ones(16))
    for eps in (0.0, 1e-6, 0.5):
        z = O.rms_norm_heads(y, 16, ones, eps).reshape(7, 3, 16)
        h = y.reshape(7, 3, 16)
        ms = (h * h).mean(-1)
        assert np.allclose((z * z).mean(-1), ms / (ms + eps), rtol=1e-12, atol=0)
        cosang = (z * h).sum(-1) / np.linalg.norm(z, axis=-1) / np.linalg.norm(h, axis=-1)
        assert np.allclose(cosang, 1.0, rtol=0, atol=1e-12)
    assert np.allclose(O.rms_norm_heads(37.5 * y, 16, ones, 0.0), O.rms_norm_heads(y, 16, ones, 0.0),
                       rtol=1e-12, atol=1e-14)
    w = O.f64_to_bf16(rng.uniform(0.5, 2, 16))
    ratio = O.rms_norm_heads(y, 16, w, 1e-6) / O.rms_norm_heads(y, 16, ones, 1e-6)
    assert np.allclose(ratio, np.tile(O.bf16_to_f64(w), 3)[None, :], rtol=1e-12)


def test_rope_pairs_rotation_properties():
    """Each channel pair is turned by its angle: zero angle is the identity, a
    quarter turn maps (a, b) to (-b, a), pair norms are kept, and turns compose:
    <R(t1) q, R(t2) k> = <R(t1 - t2) q, k> per pair (the relative-position
    property of the rotary embedding)."""
    rng = np.random.default_rng(6)
    m, hd = 5, 8
    q, k = rng.standard_normal((m, 2 * hd)), rng.standard_normal((m, 2 * hd))
    zero = np.zeros((m, hd // 2))
    assert np.array_equal(O.rope_pairs(q, hd, np.cos(zero), np.sin(zero)), q)
    quarter = O.rope_pairs(q, hd, np.zeros((m, hd // 2)), np.ones((m, hd // 2)))
    qp = q.reshape(m, 2, hd // 2, 2)
    assert np.array_equal(quarter.reshape(m, 2, hd // 2, 2), np.stack([-qp[..., 1], qp[..., 0]], -1))
    t1, t2 = rng.uniform(-7, 7, (m, hd // 2)), rng.uniform(-7, 7, (m, hd // 2))
    r1 = O.rope_pairs(q, hd, np.cos(t1), np.sin(t1)).reshape(m, 2, hd // 2, 2)
    r2 = O.rope_pairs(k, hd, np.cos(t2), np.sin(t2)).reshape(m, 2, hd // 2, 2)
    assert np.allclose(np.linalg.norm(r1, axis=-1), np.linalg.norm(qp, axis=-1), rtol=1e-13)
    d = O.rope_pairs(q, hd, np.cos(t1 - t2), np.sin(t1 - t2)).reshape(m, 2, hd // 2, 2)
    kp = k.reshape(m, 2, hd // 2, 2)
    assert np.allclose((r1 * r2).sum(-1), (d * kp).sum(-1), rtol=1e-10, atol=1e-12)


def test_qkv_output_composition():
    """qkv_output is call 2's Y* followed by the per-third epilogue: the V third
    is Y* itself (bit for bit after rounding), Q and K are norm-then-rotate of
    their thirds with their own scales; rows select token rows and table rows."""
    spec = S.LinearSpec("qkvpin", 9, 24, 128, 3 * 32, 16, outlier_channels=2, outlier_scale=20.0)
    d = S.make_linear(spec)
    lam = O.smooth_factors(O.activation_absmax(d["x"]), d["w"])
    pk = O.pack_weights(d["w"], lam, 16)
    a = O.quantize_act_lora_down(d["x"], lam, pk["lora_down"])
    cos, sin = S.make_rope_tables(24, 16, n_text=4, grid_w=4, axes=(4, 6, 6))
    qn, kn = S.make_norm_weight(spec, 0, 16), S.make_norm_weight(spec, 1, 16)
    args = (a["act_codes"], a["act_scales"], pk["w_codes"], pk["w_scales"], a["lora_act"], pk["lora_up"],
            d["bias"])
    y, yb = O.linear_output(*args)
    out, ob = O.qkv_output(*args, 16, qn, kn, 1e-6, cos, sin)
    assert np.array_equal(ob[:, 64:], yb[:, 64:])
    assert np.allclose(out[:, :32], O.rope_pairs(O.rms_norm_heads(y[:, :32], 16, qn, 1e-6), 16, cos, sin),
                       rtol=0, atol=0)
    assert np.allclose(out[:, 32:64], O.rope_pairs(O.rms_norm_heads(y[:, 32:64], 16, kn, 1e-6), 16, cos, sin),
                       rtol=0, atol=0)
    rows = [3, 0, 23]
    sub, subb = O.qkv_output(*args, 16, qn, kn, 1e-6, cos, sin, rows=rows)
    assert np.array_equal(subb, ob[rows])


def test_rope_tables_positions():
    """Text tokens get zero angles; image token t turns its height-axis pairs by
    t // grid_w and its width-axis pairs by t % grid_w times the pair frequency."""
    cos, sin = S.make_rope_tables(10, 16, n_text=2, grid_w=3, axes=(4, 6, 6))
    assert np.all(cos[:2] == 1) and np.all(sin[:2] == 0) and np.all(cos[:, :2] == 1)
    t = 2 + 7   # image token 7: row 2, col 1
    f6 = 10000.0 ** (-np.arange(0, 6, 2) / 6)
    assert np.allclose(np.arctan2(sin[t, 2:5], cos[t, 2:5]), np.angle(np.exp(1j * 2 * f6)), atol=1e-6)
    assert np.allclose(np.arctan2(sin[t, 5:8], cos[t, 5:8]), np.angle(np.exp(1j * 1 * f6)), atol=1e-6)
