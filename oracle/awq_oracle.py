"""Reference oracle for the AWQ W4A16 linear (4-bit weights, 16-bit activations).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
``__graft_entry__.smoke()`` and the CPU baseline leg of ``bench.py`` use it; it
shares nothing with the HIP kernels, the C ABI or the host packer.

What is computed.  The Nunchaku Lite integration runs two kernel families; the
second, awq_w4a16, keeps 4-bit weights with 16-bit activations for the
adaptive-normalization and modulation projections, which are memory-heavy and
sensitive to precision (mind-verse.de, "Effiziente Optimierung von
Diffusionsmodellen durch Nunchaku 4-Bit-Quantisierung", section "Nunchaku Lite:
Nahtlose Integration in Diffusers"); its config block gives precision int4 and
group_size 64 (same page, section "Native Ladefunktion in Diffusers").  The page
names the scheme only; the algorithm is AWQ as published (Lin et al., 2023,
"AWQ: Activation-aware Weight Quantization for LLM Compression and
Acceleration"): per input channel a scale s = mean|x|^alpha (normalized by the
geometric mean of its extremes) multiplies the weights and divides the
activations, alpha taken from a grid that minimizes the layer's output error on
calibration activations, and the scaled weights are quantized per group to
unsigned 4-bit codes with a scale and a zero point.

Readings (listed with reasons in the design notes): grid alpha = i/20,
i = 0..19; s clamped to >= 1e-4 before normalizing, stored as fp32; group
scale Delta = bf16(max(max - min, 1e-5) / 15) rounded once from float64, zero
point z = clamp(rint(-min / Delta), 0, 15), code q = clamp(rint(w / Delta) + z,
0, 15) with the rounded Delta; activations x_hat = bf16(fl32(x * fl32(1/s))) as
in the W4A4 smoothing; Y* = x_hat . ((q - z) Delta)^T + b in float64.

Layouts: W [N, K]; codes u8 [N, K/2] (element 2i in the low nibble, unsigned);
scales bf16 bits [N, K/64]; zeros u8 [N, K/64]; smoothing fp32 [K].
"""
from __future__ import annotations

import numpy as np

from .svdq_oracle import bf16_to_f64, f64_to_bf16, f64_to_f32, smooth_activations

AWQ_GROUP = 64
AWQ_QMAX = 15
AWQ_GRID = 20
AWQ_SCALE_MIN = 1e-4
AWQ_RANGE_MIN = 1e-5


def activation_mean_abs(x_bits) -> np.ndarray:
    """s_x[k] = mean over calibration tokens of |x[m, k]| (float64)."""
    return np.abs(bf16_to_f64(x_bits)).mean(axis=0)


def awq_scales(s_x, alpha: float) -> np.ndarray:
    """s = clamp(s_x^alpha, 1e-4) / sqrt(max * min), rounded to fp32."""
    s = np.maximum(np.power(np.asarray(s_x, dtype=np.float64), alpha), AWQ_SCALE_MIN)
    s = s / np.sqrt(s.max() * s.min())
    return f64_to_f32(s)


def quantize_asym_groups(w_prime, group: int = AWQ_GROUP):
    """Per (row, group): Delta, z, q as defined in the module header.

    Returns (q uint8 [N, K] in 0..15, Delta bf16 bits [N, G], z uint8 [N, G])."""
    w = np.asarray(w_prime, dtype=np.float64)
    N, K = w.shape
    G = K // group
    wg = w.reshape(N, G, group)
    mx, mn = wg.max(axis=-1), wg.min(axis=-1)
    dbits = f64_to_bf16(np.maximum(mx - mn, AWQ_RANGE_MIN) / AWQ_QMAX)
    d = bf16_to_f64(dbits)
    z = np.clip(np.rint(-mn / d), 0, AWQ_QMAX)
    q = np.clip(np.rint(wg / d[..., None]) + z[..., None], 0, AWQ_QMAX)
    return q.reshape(N, K).astype(np.uint8), dbits, z.astype(np.uint8)


def dequantize_asym(q, dbits, z, group: int = AWQ_GROUP) -> np.ndarray:
    """(q - z) * Delta per group, float64 [N, K]."""
    q = np.asarray(q, dtype=np.float64)
    N, K = q.shape
    qg = q.reshape(N, K // group, group)
    return ((qg - np.asarray(z, dtype=np.float64)[..., None]) * bf16_to_f64(dbits)[..., None]).reshape(N, K)


def pack_uint4(q) -> np.ndarray:
    """Two unsigned 4-bit codes per byte along K, element 2i in the low nibble."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def unpack_uint4(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty((c.shape[0], c.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = c & 0x0F
    out[:, 1::2] = c >> 4
    return out


def awq_loss(x_calib_bits, w_bits, s32, group: int = AWQ_GROUP) -> float:
    """Mean squared output error of the layer quantized with scales s (float64)."""
    x = bf16_to_f64(x_calib_bits)
    w = bf16_to_f64(w_bits)
    s = np.asarray(s32, dtype=np.float64)
    q, dbits, z = quantize_asym_groups(w * s[None, :], group)
    w_eff = dequantize_asym(q, dbits, z, group) / s[None, :]
    d = x @ w.T - x @ w_eff.T
    return float((d * d).mean())


def awq_search(x_calib_bits, w_bits, group: int = AWQ_GROUP, n_grid: int = AWQ_GRID):
    """alpha on the grid i / n_grid with the least output error (the first one on ties).

    Returns (alpha, s fp32 [K], losses [n_grid])."""
    s_x = activation_mean_abs(x_calib_bits)
    losses = np.array([awq_loss(x_calib_bits, w_bits, awq_scales(s_x, i / n_grid), group)
                       for i in range(n_grid)])
    best = int(np.argmin(losses))
    return best / n_grid, awq_scales(s_x, best / n_grid), losses


def awq_pack(x_calib_bits, w_bits, group: int = AWQ_GROUP, n_grid: int = AWQ_GRID) -> dict:
    """The offline step: search s, quantize W * s.  Returns smooth (fp32 [K]),
    codes, scales (bf16 bits), zeros, alpha and the grid's losses."""
    alpha, s, losses = awq_search(x_calib_bits, w_bits, group, n_grid)
    w = bf16_to_f64(w_bits) * np.asarray(s, dtype=np.float64)[None, :]
    q, dbits, z = quantize_asym_groups(w, group)
    return {"smooth": s, "codes": pack_uint4(q), "scales": dbits, "zeros": z, "alpha": alpha,
            "losses": losses, "q": q}


def awq_linear(x_bits, smooth, codes, scales_bits, zeros, bias_bits, group: int = AWQ_GROUP, rows=None):
    """Y* = x_hat . ((q - z) Delta)^T + b (float64), x_hat = bf16(fl32(x * fl32(1/s))).

    Returns (Y* float64 [m, N], bf16 bits); ``rows`` selects token rows."""
    x = np.asarray(x_bits) if rows is None else np.asarray(x_bits)[np.asarray(rows)]
    xh = bf16_to_f64(smooth_activations(x, smooth))
    w = dequantize_asym(unpack_uint4(codes), scales_bits, zeros, group)
    y = xh @ w.T
    if bias_bits is not None:
        y = y + bf16_to_f64(bias_bits)[None, :]
    return y, f64_to_bf16(y)
