"""Helpers for the GPU parity tests: host <-> device conversion and comparisons."""
from __future__ import annotations

import numpy as np

import oracle as O
import synthetic as S

_CASES: dict = {}


def to_dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place (monotone integer order of the patterns)."""
    def order(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(order(a_bits) - order(b_bits))


def y_errors(y_bits: np.ndarray, y_ref: np.ndarray):
    y = O.bf16_to_f64(y_bits)
    rel_fro = np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    max_abs = np.abs(y - y_ref).max() / max(np.abs(y_ref).max(), 1e-300)
    return rel_fro, max_abs


# tolerance on Y against the float64 oracle: relative Frobenius and max-abs / max|Y*|
Y_REL_FRO = 5e-3
Y_MAX_ABS = 1e-2


def oracle_case(spec, M=None, r=None):
    """Inputs plus the oracle's own packing of the weights (cached per shape)."""
    if isinstance(spec, str):
        spec = S.SPECS[spec]
    key = (spec, M, r)
    if key not in _CASES:
        d = S.make_linear(spec, M=M)
        lam = O.smooth_factors(O.activation_absmax(d["x"]), d["w"])
        rr = spec.r if r is None else r
        packed = O.pack_weights(d["w"], lam, rr)
        for k in ("residual", "w_smooth", "q_w"):
            packed.pop(k, None)
        _CASES[key] = (d, lam, packed)
    return _CASES[key]


def custom_case(M, K, N, r, seed=0, outliers=4):
    spec = S.LinearSpec(f"custom{M}x{K}x{N}r{r}", 9, M, K, N, r, outlier_channels=min(outliers, K),
                        outlier_scale=30.0, heavy_tail=True, layer_id=seed)
    return oracle_case(spec)


def check_quant(got, ref, lora_down=None):
    assert np.array_equal(got["act_scales"], ref["act_scales"]), \
        np.argwhere(got["act_scales"] != ref["act_scales"])[:5]
    assert np.array_equal(got["act_codes"], ref["act_codes"]), \
        np.argwhere(got["act_codes"] != ref["act_codes"])[:5]
    if ref["lora_act"].size:
        check_lora_act(got["lora_act"], ref, lora_down)


def check_lora_act(got_bits, ref, lora_down):
    """lora_act = bf16(x_hat @ L1) with fp32 accumulation on the GPU.

    Bound from the arithmetic: both sides round to bf16 once (half an ulp each),
    and an fp32 sum of K products (exact bf16 x bf16 products) is off by at most
    K * 2^-24 * sum_k |x_hat_k L1_k|.  Where the sum does not cancel this is
    below one ulp, and almost every element must be within one ulp."""
    d = ulp_distance(got_bits, ref["lora_act"])
    assert (d <= 1).mean() >= 0.999, (d > 1).sum()
    if lora_down is None:
        assert d.max() <= 1
        return
    xh = np.abs(O.bf16_to_f64(ref["xhat"]))
    mag = xh @ np.abs(O.bf16_to_f64(lora_down)).T
    K = xh.shape[1]
    got = O.bf16_to_f64(got_bits)
    want = O.bf16_to_f64(ref["lora_act"])
    ulp = np.maximum(np.abs(want), np.abs(got)) * 2.0 ** -7
    assert np.all(np.abs(got - want) <= ulp + K * 2.0 ** -24 * mag)


def check_y(y_bits, d, lam, packed, ref_a, rows=None, bias=True):
    y_ref, _ = O.linear_output(ref_a["act_codes"], ref_a["act_scales"], packed["w_codes"],
                               packed["w_scales"], ref_a["lora_act"], packed["lora_up"],
                               d["bias"] if bias else None, rows=rows)
    got = y_bits if rows is None else y_bits[np.asarray(rows)]
    rel, mx = y_errors(got, y_ref)
    assert rel <= Y_REL_FRO and mx <= Y_MAX_ABS, (rel, mx)
    return rel, mx
