"""Reference oracle for the SVDQuant W4A4 + low-rank linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only the test suite, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  It is a plain, slow, CPU implementation in
numpy (float64 unless a step names float32 or bfloat16 rounding) and shares no
code, table or helper with the HIP kernels, the C ABI or the host packer.

What the method computes (sources, cited by page title and section):

* "Effiziente Optimierung von Diffusionsmodellen durch Nunchaku
  4-Bit-Quantisierung" (mind-verse.de), section "Nunchaku und SVDQuant": the
  main transformer layers run with 4-bit weights and 4-bit activations; outliers
  of the activations are shifted into the weights; the hardest part of each
  weight matrix is kept in a small 16-bit low-rank branch; the remainder is
  quantized to 4 bits.
* "AI-Bildmodelle auf normalen GPUs ausführen: Hugging Face bringt 4-Bit-Diffusion
  für alle" (ai2day.live), section "Was ist Nunchaku Lite und was macht es
  genau?": 4-bit precision both for stored weights and for the live activations;
  the method name expands to singular value decomposition quantization.
* mind-verse.de, section "Native Ladefunktion in Diffusers": the quantization
  config names ``group_size``, ``rank`` (32 in the example) and a bfloat16
  compute dtype.
* charmloop.ai news item on Nunchaku in Diffusers, paragraph on the 16-bit
  branch: the low-rank down-projection is fused with the activation
  quantization, the low-rank up-projection with the 4-bit compute kernel.  The
  fusion changes where the work runs, not what is computed, so the oracle
  computes both projections unfused.

The pages print no formula.  Every convention below (smoothing factor, SVD split,
scale dtype, rounding, int4 range and packing) is a reading; each is listed with
its reason in the design notes.  Notation: ``bf16(v)`` rounds to nearest-even
bfloat16 (8 significant bits), ``fl32(v)`` rounds to nearest-even binary32,
``rint`` rounds half to even.

Layouts (nn.Linear convention, the module tree is unchanged by the swap described
in mind-verse.de § "Native Ladefunktion in Diffusers"): X [M, K], W [N, K],
lora_down = L1^T [r, K], lora_up = L2^T [N, r], Y [M, N].  int4 codes are packed
two per byte along K, element 2i in the low nibble, two's complement, the rows
in the boundary's storage order (``storage_order``); scales are row-major
[rows, K / group].
"""
from __future__ import annotations

import numpy as np

GROUP = 64          # quant group along K (int4 variant; config field group_size)
QMAX = 7            # symmetric int4 range [-7, 7]
SMOOTH_EPS = 1e-5   # clamp of the per-channel maxima in the smoothing factor


# ---------------------------------------------------------------------------
# Number formats (own implementations; no shared helpers with the GPU path)
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def f64_to_f32(v) -> np.ndarray:
    """fl32: round float64 to float32, nearest-even (numpy's cast)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def f64_to_bf16(v) -> np.ndarray:
    """Round float64 values to bfloat16 with ONE rounding (nearest, ties to even).

    float64 -> float32 is done with round-to-odd (truncate, then set the sticky
    bit when inexact); 24 bits >= 8 + 2, so the following nearest-even rounding to
    8 bits equals a single rounding of the float64 value.  Returns uint16 bits.
    """
    v = np.asarray(v, dtype=np.float64)
    t = v.astype(np.float32)
    back = t.astype(np.float64)
    over = np.abs(back) > np.abs(v)
    t = np.where(over, np.nextafter(t, np.float32(0)), t).astype(np.float32)
    bits = np.ascontiguousarray(t).view(np.uint32)
    inexact = t.astype(np.float64) != v
    bits = np.where(inexact, bits | np.uint32(1), bits).astype(np.uint32)
    return f32_to_bf16(bits.view(np.float32))


# ---------------------------------------------------------------------------
# int4 packing (two's complement nibbles, element 2i low, 2i+1 high)
# ---------------------------------------------------------------------------

def storage_order(b) -> np.ndarray:
    """The storage order of packed int4 rows at the library's C boundary
    (include/svdq.h, "Layouts"): in every row whose index in the array has bit 3
    set (rows 8-15 of each 16), the two 8-byte halves of every 16-byte piece of
    the row are exchanged, i.e. byte j of the row is stored at j ^ 8.  Rows
    0-7 of each 16 keep the plain order.  The exchange is its own inverse.  It
    is a layout convention of the boundary, not part of the method."""
    b = np.array(b, dtype=np.uint8, copy=True)
    swapped = (np.arange(b.shape[0]) & 8) != 0
    if swapped.any():
        if b.shape[1] % 16:
            raise ValueError("packed rows of 9 or more rows need a multiple of 16 bytes")
        b[swapped] = b[swapped][:, np.arange(b.shape[1]) ^ 8]
    return b


def pack_int4(q) -> np.ndarray:
    """Pack int codes in [-8, 7] of shape [rows, K] (K even) into uint8 [rows, K/2]:
    element 2i in the low nibble of byte i, then the rows in ``storage_order``."""
    q = np.asarray(q, dtype=np.int64)
    lo = q[:, 0::2] & 0xF
    hi = q[:, 1::2] & 0xF
    return storage_order((lo | (hi << 4)).astype(np.uint8))


def unpack_int4(codes) -> np.ndarray:
    """Decode uint8 [rows, K/2] into int8 [rows, K] (inverse of ``pack_int4``)."""
    c = storage_order(codes).astype(np.int64)
    nib = np.empty((c.shape[0], c.shape[1] * 2), dtype=np.int64)
    nib[:, 0::2] = c & 0xF
    nib[:, 1::2] = c >> 4
    nib = np.where(nib >= 8, nib - 16, nib)
    return nib.astype(np.int8)


# ---------------------------------------------------------------------------
# Offline side: smoothing, low-rank split, residual quantization
# (mind-verse.de § "Nunchaku und SVDQuant"; ai2day.live § "Was ist Nunchaku Lite")
# ---------------------------------------------------------------------------

def smooth_factors(x_absmax, w_bits, eps: float = SMOOTH_EPS) -> np.ndarray:
    """Per-input-channel smoothing factor lambda (float32 [K]).

    lambda_j = fl32(sqrt(max(a_j, eps) / max(w_j, eps))) with a_j the activation
    absmax of channel j and w_j = max_n |W_nj|; computed in float64, rounded once.
    Dividing X by lambda and multiplying W by lambda moves activation outliers
    into the weights (mind-verse.de § "Nunchaku und SVDQuant").  The square-root
    balance is the smoothing rule of the tiny workload definition.
    """
    a = np.maximum(np.asarray(x_absmax, dtype=np.float64), eps)
    w = np.maximum(np.abs(bf16_to_f64(w_bits)).max(axis=0), eps)
    return f64_to_f32(np.sqrt(a / w))


def activation_absmax(x_bits) -> np.ndarray:
    """a_j = max_m |X_mj| (float64 [K]); the calibration statistic of lambda."""
    return np.abs(bf16_to_f64(x_bits)).max(axis=0)


def smoothed_weight(w_bits, lam) -> np.ndarray:
    """W' = W diag(lambda) in float64 (exact: 8 + 24 significant bits)."""
    return bf16_to_f64(w_bits) * np.asarray(lam, dtype=np.float32).astype(np.float64)[None, :]


def lowrank_split(w_smooth, r: int):
    """Split W' [N, K] into a rank-r branch and a residual.

    SVD W' = U S V^T (LAPACK, float64).  The singular values are shared evenly:
    lora_up* = U_r S_r^(1/2) [N, r], lora_down* = S_r^(1/2) V_r^T [r, K].  The
    stored factors are bf16 (the 16-bit branch); the residual is taken against the
    ROUNDED factors, R = W' - lora_up @ lora_down, so W' = L1 L2 + R holds up to
    float64 rounding (mind-verse.de § "Nunchaku und SVDQuant": low-rank branch for
    the hardest part, 4 bits for the rest).

    Returns (lora_down_bits [r,K] uint16, lora_up_bits [N,r] uint16,
             residual [N,K] float64, singular_values [min(N,K)] float64).
    """
    w_smooth = np.asarray(w_smooth, dtype=np.float64)
    N, K = w_smooth.shape
    u, s, vt = np.linalg.svd(w_smooth, full_matrices=False)
    if r == 0:
        down = np.zeros((0, K), dtype=np.uint16)
        up = np.zeros((N, 0), dtype=np.uint16)
        return down, up, w_smooth.copy(), s
    root = np.sqrt(s[:r])
    up = f64_to_bf16(u[:, :r] * root[None, :])
    down = f64_to_bf16(root[:, None] * vt[:r, :])
    lowrank = bf16_to_f64(up) @ bf16_to_f64(down)
    return down, up, w_smooth - lowrank, s


def quantize_weight_groups(resid, group: int = GROUP):
    """Symmetric per-group int4 quantization of the residual R [N, K].

    Per row n and group g of ``group`` consecutive k: A = max |R|, scale
    s = bf16(A / 7) (float64 quotient, one rounding), q = clamp(rint(R / s), -7, 7)
    with a float64 quotient; an all-zero group has s = 0 and q = 0.
    Returns (q int8 [N, K], scale bits uint16 [N, K/group]).
    """
    R = np.asarray(resid, dtype=np.float64)
    N, K = R.shape
    Rg = R.reshape(N, K // group, group)
    amax = np.abs(Rg).max(axis=2)
    s_bits = f64_to_bf16(amax / float(QMAX))
    s = bf16_to_f64(s_bits)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(Rg / s[:, :, None])
    q = np.where(s[:, :, None] > 0, q, 0.0)
    q = np.clip(q, -QMAX, QMAX).astype(np.int8)
    return q.reshape(N, K), s_bits


def pack_weights(w_bits, lam, r: int, group: int = GROUP):
    """Offline packing of one linear: smoothing, low-rank split, residual quantization.

    Returns a dict with w_codes uint8 [N,K/2], w_scales uint16 [N,K/group],
    lora_down uint16 [r,K], lora_up uint16 [N,r] and, for checks, the residual and
    the singular values of W'.
    """
    ws = smoothed_weight(w_bits, lam)
    down, up, resid, sv = lowrank_split(ws, r)
    q, s_bits = quantize_weight_groups(resid, group)
    return {
        "w_codes": pack_int4(q),
        "w_scales": s_bits,
        "lora_down": down,
        "lora_up": up,
        "residual": resid,
        "w_smooth": ws,
        "singular_values": sv,
        "q_w": q,
    }


# ---------------------------------------------------------------------------
# Online side, call 1: smoothing + per-token per-group int4 quantization + lora_down
# (ai2day.live § "Was ist Nunchaku Lite"; charmloop.ai fusion paragraph)
# ---------------------------------------------------------------------------

def smooth_activations(x_bits, lam) -> np.ndarray:
    """x_hat = bf16(fl32(X * mu)), mu = fl32(1 / lambda).  Returns uint16 bits [M, K].

    One canonical bf16 x_hat feeds both the quantizer and the low-rank
    down-projection (compute dtype bfloat16, mind-verse.de § "Native Ladefunktion
    in Diffusers").  The float64 product of a bf16 and a float32 is exact, so the
    cast to float32 is the single fl32 rounding; 1/lambda in float64 rounded to
    float32 is the correctly rounded float32 reciprocal (53 >= 2*24 + 2).
    """
    mu = f64_to_f32(1.0 / np.asarray(lam, dtype=np.float32).astype(np.float64))
    p = f64_to_f32(bf16_to_f64(x_bits) * mu.astype(np.float64)[None, :])
    return f32_to_bf16(p)


def quantize_activation_groups(xhat_bits, group: int = GROUP):
    """Per-token, per-group symmetric int4 quantization of x_hat [M, K].

    A = max |x_hat| over the group; s = bf16(fl32(A / 7)); iota = fl32(1 / s);
    q = clamp(rint(x_hat * iota), -7, 7), the product taken exactly (8 + 24 bits
    fit float64); s = 0 gives q = 0.  Reading (the pages are silent): when
    fl32(1 / s) overflows (s < 2^-128, a group maximum below about 2e-38) the
    group is treated like s = 0, q = 0.  Returns (q int8 [M, K], scale bits
    uint16 [M, K/group]).
    """
    xh = bf16_to_f64(xhat_bits)
    M, K = xh.shape
    g = xh.reshape(M, K // group, group)
    amax = np.abs(g).max(axis=2)
    s_bits = f32_to_bf16(f64_to_f32(amax / float(QMAX)))
    s = bf16_to_f64(s_bits)
    with np.errstate(divide="ignore", over="ignore"):
        iota = f64_to_f32(1.0 / s).astype(np.float64)
    iota = np.where((s > 0) & np.isfinite(iota), iota, 0.0)
    q = np.rint(g * iota[:, :, None])
    q = np.clip(q, -QMAX, QMAX).astype(np.int8)
    return q.reshape(M, K), s_bits


def lora_down_project(xhat_bits, lora_down_bits) -> np.ndarray:
    """lora_act = bf16(x_hat @ L1), L1 = lora_down^T; float64 sum, one rounding.

    Returns uint16 bits [M, r].
    """
    r = np.asarray(lora_down_bits).shape[0]
    xh = bf16_to_f64(xhat_bits)
    if r == 0:
        return np.zeros((xh.shape[0], 0), dtype=np.uint16)
    return f64_to_bf16(xh @ bf16_to_f64(lora_down_bits).T)


def quantize_act_lora_down(x_bits, lam, lora_down_bits, group: int = GROUP):
    """What the first fused call returns: packed codes, scales and x_hat @ L1.

    Returns dict(act_codes uint8 [M,K/2], act_scales uint16 [M,K/group],
    lora_act uint16 [M,r], xhat uint16 [M,K], q_x int8 [M,K]).
    """
    xh = smooth_activations(x_bits, lam)
    q, s_bits = quantize_activation_groups(xh, group)
    return {
        "act_codes": pack_int4(q),
        "act_scales": s_bits,
        "lora_act": lora_down_project(xh, lora_down_bits),
        "xhat": xh,
        "q_x": q,
    }


# ---------------------------------------------------------------------------
# Online side, call 2: W4A4 group products + dequantization + lora_up + bias
# (mind-verse.de § "Nunchaku und SVDQuant"; charmloop.ai fusion paragraph)
# ---------------------------------------------------------------------------

def group_accumulators(act_codes, w_codes, group: int = GROUP, rows=None, cols=None) -> np.ndarray:
    """acc[m, n, g] = sum over k in group g of q_x[m,k] * q_w[n,k] (exact integers).

    |acc| <= 64 * 49.  ``rows`` / ``cols`` select a window.  Returns int64 [m, n, G].
    """
    qx = unpack_int4(act_codes).astype(np.int64)
    qw = unpack_int4(w_codes).astype(np.int64)
    if rows is not None:
        qx = qx[np.asarray(rows)]
    if cols is not None:
        qw = qw[np.asarray(cols)]
    M, K = qx.shape
    N = qw.shape[0]
    G = K // group
    out = np.empty((M, N, G), dtype=np.int64)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        out[:, :, g] = qx[:, sl] @ qw[:, sl].T
    return out


def linear_output(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias,
                  group: int = GROUP, rows=None, epilogue=None):
    """Y* = sum_g s_x[m,g] s_w[n,g] acc_g[m,n] + lora_act @ lora_up^T + b (float64).

    Returns (Y* float64 [m, N], bf16(Y*) uint16 [m, N]); ``rows`` selects rows.
    ``bias`` may be None.  ``epilogue="gelu_tanh"`` applies gelu_tanh to Y*
    before the rounding.
    """
    rows_idx = np.arange(np.asarray(act_codes).shape[0]) if rows is None else np.asarray(rows)
    acc = group_accumulators(act_codes, w_codes, group, rows=rows_idx)
    sx = bf16_to_f64(np.asarray(act_scales)[rows_idx])          # [m, G]
    sw = bf16_to_f64(w_scales)                                  # [N, G]
    y = np.zeros(acc.shape[:2], dtype=np.float64)
    for g in range(acc.shape[2]):
        y += sx[:, g][:, None] * sw[:, g][None, :] * acc[:, :, g]
    la = np.asarray(lora_act)
    if la.shape[1] > 0:
        y += bf16_to_f64(la[rows_idx]) @ bf16_to_f64(lora_up).T
    if bias is not None:
        y += bf16_to_f64(bias)[None, :]
    if epilogue == "gelu_tanh":
        y = gelu_tanh(y)
    elif epilogue is not None:
        raise ValueError(f"unknown epilogue {epilogue!r}")
    return y, f64_to_bf16(y)


def forward(x_bits, lam, packed: dict, bias, group: int = GROUP, rows=None):
    """Whole layer: call 1 then call 2 on the oracle's own intermediates."""
    a = quantize_act_lora_down(x_bits, lam, packed["lora_down"], group)
    y, y_bits = linear_output(a["act_codes"], a["act_scales"], packed["w_codes"],
                              packed["w_scales"], a["lora_act"], packed["lora_up"],
                              bias, group, rows=rows)
    return a, y, y_bits


# ---------------------------------------------------------------------------
# Output epilogue and the MLP pair.  The W4A4 layer serves the attention and
# MLP projections of the transformer (mind-verse.de, "Effiziente Optimierung
# von Diffusionsmodellen durch Nunchaku 4-Bit-Quantisierung", section "Nunchaku
# Lite: Nahtlose Integration in Diffusers"); in an MLP the up-projection's
# output goes through GELU before the down-projection.
# ---------------------------------------------------------------------------

GELU_C = 0.7978845608028654   # sqrt(2 / pi)
GELU_A = 0.044715


def gelu_tanh(v):
    """GELU, tanh approximation (Hendrycks and Gimpel, 2016), float64:
    0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + np.tanh(GELU_C * (v + GELU_A * v ** 3)))


def float_mlp_hidden(x_bits, w_bits, bias_bits, rows=None):
    """bf16(gelu_tanh(X W^T + b)) of the unquantized up-projection, float64.

    The smoothing factors of a layer are calibrated on the activations that
    reach it; for the down-projection of an MLP these are the GELU outputs of
    the floating-point model, so its lambda comes from this array's absmax."""
    x = bf16_to_f64(x_bits)
    if rows is not None:
        x = x[np.asarray(rows)]
    y = x @ bf16_to_f64(w_bits).T + bf16_to_f64(bias_bits)[None, :]
    return f64_to_bf16(gelu_tanh(y))


def mlp_pair(x_bits, lam_up, packed_up: dict, bias_up, lam_down, packed_down: dict, bias_down,
             group: int = GROUP, rows=None):
    """Up-projection with the GELU epilogue, its bf16 output H as the input of
    the down-projection (call 1 then call 2 again).  Every step is local to a
    token row once lambda is fixed, so ``rows`` computes just those rows.

    Returns dict(h uint16 [m, N_up], y float64 [m, N_down], y_bits uint16, and
    the intermediates a_up, a_down of call 1)."""
    x = np.asarray(x_bits) if rows is None else np.asarray(x_bits)[np.asarray(rows)]
    a_up = quantize_act_lora_down(x, lam_up, packed_up["lora_down"], group)
    _, h = linear_output(a_up["act_codes"], a_up["act_scales"], packed_up["w_codes"],
                         packed_up["w_scales"], a_up["lora_act"], packed_up["lora_up"], bias_up,
                         group, epilogue="gelu_tanh")
    a_dn = quantize_act_lora_down(h, lam_down, packed_down["lora_down"], group)
    y, y_bits = linear_output(a_dn["act_codes"], a_dn["act_scales"], packed_down["w_codes"],
                              packed_down["w_scales"], a_dn["lora_act"], packed_down["lora_up"],
                              bias_down, group)
    return {"h": h, "y": y, "y_bits": y_bits, "a_up": a_up, "a_down": a_dn}


# ---------------------------------------------------------------------------
# Fused QKV epilogue.  For FLUX.1-dev the engine merges the Q, K and V
# projections into one quantized to_qkv module because its fused operator
# handles the QKV projection, the Q/K normalization and the rotary embeddings
# together (mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch
# Nunchaku 4-Bit-Quantisierung", section "Quantisierung von Modellen mit
# strukturellen Umschreibungen").  The page names the three steps only; their
# definitions here are the textbook ones: RMSNorm (Zhang and Sennrich, 2019)
# over each head's channels with a learned scale, then the rotary position
# embedding of RoFormer (Su et al., 2021), which turns each pair of adjacent
# channels (2i, 2i+1) of a head by a per-token angle.  Y = [Q | K | V] along N.
# ---------------------------------------------------------------------------

def rms_norm_heads(y, head_dim: int, weight_bits, eps: float):
    """z = y / sqrt(mean over the head's channels of y^2 + eps) * w, float64."""
    y = np.asarray(y, dtype=np.float64)
    m, n = y.shape
    h = y.reshape(m, n // head_dim, head_dim)
    ms = (h * h).mean(axis=-1, keepdims=True)
    w = bf16_to_f64(weight_bits)[None, None, :]
    return (h / np.sqrt(ms + eps) * w).reshape(m, n)


def rope_pairs(z, head_dim: int, cos, sin):
    """Rotate each adjacent pair (2i, 2i+1) of every head by the token's angle i:
    (a, b) -> (a cos - b sin, a sin + b cos).  cos, sin: [m, head_dim/2]."""
    z = np.asarray(z, dtype=np.float64)
    m, n = z.shape
    h = z.reshape(m, n // head_dim, head_dim // 2, 2)
    c = np.asarray(cos, dtype=np.float64)[:, None, :]
    s_ = np.asarray(sin, dtype=np.float64)[:, None, :]
    a, b = h[..., 0], h[..., 1]
    out = np.stack([a * c - b * s_, a * s_ + b * c], axis=-1)
    return out.reshape(m, n)


def qkv_norm_rope(y_star, head_dim: int, q_norm_bits, k_norm_bits, eps: float, cos, sin):
    """Q and K thirds of Y*: RMSNorm per head, then the rotary embedding; the V
    third unchanged.  Returns (float64 [m, N], bf16 bits)."""
    y = np.asarray(y_star, dtype=np.float64)
    sec = y.shape[1] // 3
    q = rope_pairs(rms_norm_heads(y[:, :sec], head_dim, q_norm_bits, eps), head_dim, cos, sin)
    k = rope_pairs(rms_norm_heads(y[:, sec:2 * sec], head_dim, k_norm_bits, eps), head_dim, cos, sin)
    out = np.concatenate([q, k, y[:, 2 * sec:]], axis=1)
    return out, f64_to_bf16(out)


def qkv_output(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias, head_dim: int,
               q_norm_bits, k_norm_bits, eps: float, cos, sin, group: int = GROUP, rows=None):
    """Call 2 with the fused QKV epilogue: linear_output, then qkv_norm_rope on
    the unrounded Y* (the fused operator rounds once, at the end)."""
    y, _ = linear_output(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias, group,
                         rows=rows)
    sel = slice(None) if rows is None else np.asarray(rows)
    return qkv_norm_rope(y, head_dim, q_norm_bits, k_norm_bits, eps, np.asarray(cos)[sel],
                         np.asarray(sin)[sel])
