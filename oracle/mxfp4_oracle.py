"""Reference oracle for the FP4 variant of the SVDQuant W4A4 linear.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
``__graft_entry__.smoke()`` and the CPU baseline leg of ``bench.py`` use it; it
shares nothing with the HIP kernels, the C ABI or the host packer.

What is computed.  The svdq_w4a4 family also comes in a 4-bit floating-point
precision ("nvfp4", group size 16 in the config example, for Blackwell GPUs:
mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch Nunchaku
4-Bit-Quantisierung", sections "Nunchaku Lite: Nahtlose Integration in
Diffusers", "Native Ladefunktion in Diffusers" and "Hardware-Unterstützung").
The pages do not define that format beyond its name.  The 4-bit floating-point
format that CDNA4's matrix cores compute on natively is the OCP Microscaling
format MXFP4 (OCP "Microscaling Formats (MX) Specification" v1.0, 2023): blocks
of 32 elements along K share one power-of-two scale (E8M0), each element is an
FP4 E2M1 number (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).  The FP4 variant here
is SVDQuant with that element format in place of int4: the same smoothing, the
same rank-r low-rank branch (16-bit), and the residual R and the smoothed
activations quantized to MXFP4 per 32-block of K.

Conversion of a block (the MX specification's rule): shared exponent
e = floor(log2(max |v|)) - 2 (2 is the largest exponent of E2M1), scale X =
2^e with e clamped to the E8M0 range [-127, 127]; each element is v / X rounded
to the nearest E2M1 value, ties to the even code, with magnitudes above 6
saturating to 6; an all-zero block has e = -127 and all elements 0.

Layouts: codes u8 [rows, K/2], element 2i in the low nibble, E2M1 code = sign
bit 3, exponent bits 2-1, mantissa bit 0; scales u8 [rows, K/32] holding the
biased exponent e + 127.
"""
from __future__ import annotations

import numpy as np

from .svdq_oracle import (bf16_to_f64, f64_to_bf16, lora_down_project, lowrank_split,
                          smooth_activations, smoothed_weight)

MX_BLOCK = 32
FP4_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def fp4_value(codes) -> np.ndarray:
    """E2M1 code (0..15) -> float64 value."""
    c = np.asarray(codes, dtype=np.int64)
    v = FP4_MAG[c & 7]
    return np.where(c & 8, -v, v)


def fp4_round(v) -> np.ndarray:
    """Nearest E2M1 code of each float64 value, ties to the even code (the
    even mantissa), magnitudes above 6 saturating to 6.  Reading: a value that
    rounds to zero gets code 0 (no negative zero).

    On magnitudes the rule is a ladder of thresholds at the midpoints
    0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; a midpoint goes to the even code,
    i.e. down at 0.25, 1.25, 2.5, 5 and up at 0.75, 1.75, 3.5."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    code = np.select([a <= 0.25, a < 0.75, a <= 1.25, a < 1.75, a <= 2.5, a < 3.5, a <= 5.0],
                     [0, 1, 2, 3, 4, 5, 6], default=7)
    neg = (v < 0) & (code != 0)
    return (code | np.where(neg, 8, 0)).astype(np.uint8)


def mx_quantize_blocks(v, block: int = MX_BLOCK):
    """MXFP4 of each row of v (float64 [rows, K]) per block of 32 along K.

    Returns (codes uint8 [rows, K] in 0..15, biased exponents uint8 [rows, K/32])."""
    v = np.asarray(v, dtype=np.float64)
    R, K = v.shape
    vb = v.reshape(R, K // block, block)
    amax = np.abs(vb).max(axis=-1)
    # floor(log2 amax) exactly, from the binary exponent (frexp: amax = f 2^x, f in [0.5, 1))
    _, x = np.frexp(amax)
    e = np.where(amax > 0, x.astype(np.float64) - 1 - 2, -127)
    e = np.clip(e, -127, 127)
    codes = fp4_round(vb / np.exp2(e)[..., None])
    return codes.reshape(R, K), (e + 127).astype(np.uint8)


def mx_dequantize(codes, exps, block: int = MX_BLOCK) -> np.ndarray:
    c = np.asarray(codes)
    R, K = c.shape
    x = np.exp2(np.asarray(exps, dtype=np.float64) - 127)
    return (fp4_value(c).reshape(R, K // block, block) * x[..., None]).reshape(R, K)


def pack_fp4(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0x0F
    out[:, 1::2] = p >> 4
    return out


def quantize_residual_fp4(residual) -> dict:
    """The residual R (float64 [N, K]) to MXFP4: packed codes and exponents."""
    codes, exps = mx_quantize_blocks(residual)
    return {"w_codes": pack_fp4(codes), "w_scales": exps}


def pack_weights_fp4(w_bits, lam, r: int) -> dict:
    """Offline packing of the FP4 variant: the same smoothing and rank-r split as
    the int4 path, the residual to MXFP4."""
    ws = smoothed_weight(w_bits, lam)
    down, up, resid, sv = lowrank_split(ws, r)
    out = quantize_residual_fp4(resid)
    out.update({"lora_down": down, "lora_up": up, "residual": resid})
    return out


def quantize_act_lora_down_fp4(x_bits, lam, lora_down_bits) -> dict:
    """Call 1 of the FP4 variant: x_hat as in the int4 path, MXFP4 codes and
    exponents per token and 32-block, lora_act = bf16(x_hat L1)."""
    xh = smooth_activations(x_bits, lam)
    codes, exps = mx_quantize_blocks(bf16_to_f64(xh))
    la = lora_down_project(xh, lora_down_bits) if np.asarray(lora_down_bits).shape[0] else \
        np.zeros((xh.shape[0], 0), dtype=np.uint16)
    return {"xhat": xh, "act_codes": pack_fp4(codes), "act_scales": exps, "lora_act": la, "codes": codes}


def linear_output_fp4(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias, rows=None):
    """Y* = deq(act) . deq(w)^T + lora_act . lora_up^T + b (float64); (Y*, bf16 bits)."""
    ac = np.asarray(act_codes) if rows is None else np.asarray(act_codes)[np.asarray(rows)]
    asc = np.asarray(act_scales) if rows is None else np.asarray(act_scales)[np.asarray(rows)]
    xa = mx_dequantize(unpack_fp4(ac), asc)
    wd = mx_dequantize(unpack_fp4(w_codes), w_scales)
    y = xa @ wd.T
    la = np.asarray(lora_act) if rows is None else np.asarray(lora_act)[np.asarray(rows)]
    if la.shape[1] > 0:
        y = y + bf16_to_f64(la) @ bf16_to_f64(lora_up).T
    if bias is not None:
        y = y + bf16_to_f64(bias)[None, :]
    return y, f64_to_bf16(y)
