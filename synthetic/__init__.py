"""Seeded synthetic inputs for the SVDQuant W4A4 + low-rank linear.

This module only draws and rounds inputs; it holds none of the method's
arithmetic (no smoothing, SVD, quantization or packing).  Both the oracle side
and the GPU side of every test and of the benchmark take their inputs from here.

The pages measure trained diffusion transformers at 1024x1024 (FLUX.1-dev,
ERNIE-Image-Turbo: mind-verse.de § "Benchmarks"; dailytechsnack.ch § "Wo der
Speicher tatsächlich steckt").  No weights or prompts exist here, so random
tensors with the shapes of a 12B-class DiT linear stand in for them:

* tokens: 4096 image + 512 text = 4608 rows per 1024x1024 image;
* X ~ N(0, 1) with a fraction of whole input channels carrying outliers;
* W ~ N(0, 0.02) (standard deviation), optionally with a 0.1 % share of
  entries replaced by 0.02 * t(3) (heavy tails);
* bias ~ N(0, 0.01);
* for the up-projection of a chained MLP pair, a fraction of whole output
  channels (rows of W and entries of the bias) scaled by the outlier factor, so
  that the GELU output feeding the down-projection carries outlier channels of
  its own.

All values are drawn in float64 from ``numpy.random.default_rng(SeedSequence(
[config_id, layer_id, tensor_id]))`` and rounded to bfloat16 once (through
float32, by torch's cast).  Arrays are returned as uint16 bf16 bit patterns.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = ["LinearSpec", "SPECS", "PAIRS", "MOD_SPECS", "make_linear", "make_w", "make_bias",
           "make_calibration", "stack_specs",
           "make_rope_tables", "make_norm_weight", "to_bf16_bits", "bf16_bits_to_f32"]

# tensor ids inside one (config, layer) seed sequence
_T_X, _T_XOUT, _T_W, _T_WTAIL, _T_BIAS, _T_WROW, _T_NORM = 0, 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class LinearSpec:
    name: str
    config_id: int
    M: int
    K: int
    N: int
    r: int
    outlier_channels: int | None = None   # fixed count (tiny case)
    outlier_frac: float = 0.0             # fraction of K (rounded) otherwise
    outlier_scale: float = 1.0
    heavy_tail: bool = False
    gelu_input: bool = False
    silu_input: bool = False              # modulation input: SiLU of the conditioning vector
    row_outlier_frac: float = 0.0         # fraction of N output channels scaled (rounded)
    layer_id: int = 0
    note: str = field(default="", compare=False)

    def with_m(self, M: int) -> "LinearSpec":
        d = dict(self.__dict__)
        d["M"] = int(M)
        return LinearSpec(**d)

    def n_outliers(self) -> int:
        if self.outlier_channels is not None:
            return int(self.outlier_channels)
        return int(round(self.outlier_frac * self.K))


SPECS = {
    # small case the oracle finishes in well under a second
    "tiny": LinearSpec("tiny", 0, 64, 256, 256, 16, outlier_channels=4, outlier_scale=50.0,
                       note="M=64 K=256 N=256 r=16; 4 outlier channels x50"),
    # one attention-output projection of a 12B-class DiT at 1024^2
    "attn_out": LinearSpec("attn_out", 1, 4608, 3072, 3072, 32, outlier_frac=0.01,
                           outlier_scale=30.0, heavy_tail=True),
    # fused QKV projection
    "qkv": LinearSpec("qkv", 2, 4608, 3072, 9216, 32, outlier_frac=0.01,
                      outlier_scale=30.0, heavy_tail=True),
    # MLP up-projection: the headline shape M=4608 K=3072 N=12288
    "mlp_up": LinearSpec("mlp_up", 3, 4608, 3072, 12288, 32, outlier_frac=0.01,
                         outlier_scale=30.0, heavy_tail=True, layer_id=0),
    # MLP down-projection; its input is a GELU(tanh) output with its own outliers
    "mlp_down": LinearSpec("mlp_down", 3, 4608, 12288, 3072, 32, outlier_frac=0.01,
                           outlier_scale=30.0, heavy_tail=True, gelu_input=True, layer_id=1),
    # chained MLP pair: up 3072 -> 12288 whose GELU output (123 channels x30 from
    # scaled rows of W_up) is the input of down 12288 -> 3072
    "pair_up": LinearSpec("pair_up", 3, 4608, 3072, 12288, 32, outlier_frac=0.01,
                          outlier_scale=30.0, heavy_tail=True, row_outlier_frac=0.01, layer_id=2),
    "pair_down": LinearSpec("pair_down", 3, 4608, 12288, 3072, 32, heavy_tail=True, layer_id=3),
}

# modulation projections of a FLUX-like 12B DiT (AWQ W4A16): one conditioning
# vector per image, SiLU of a pre-activation with 1 % of its channels x10;
# double blocks 3072 -> 6 x 3072 (image and text stream), single blocks
# 3072 -> 3 x 3072, the final layer 3072 -> 2 x 3072
MOD_SPECS = {
    "mod_double": LinearSpec("mod_double", 6, 1, 3072, 18432, 0, outlier_frac=0.01, outlier_scale=10.0,
                             heavy_tail=True, silu_input=True, layer_id=0),
    "mod_single": LinearSpec("mod_single", 6, 1, 3072, 9216, 0, outlier_frac=0.01, outlier_scale=10.0,
                             heavy_tail=True, silu_input=True, layer_id=1),
    "mod_final": LinearSpec("mod_final", 6, 1, 3072, 6144, 0, outlier_frac=0.01, outlier_scale=10.0,
                            heavy_tail=True, silu_input=True, layer_id=2),
}


def make_calibration(spec: LinearSpec, rows: int = 32) -> np.ndarray:
    """Calibration activations for an offline packer: rows drawn like the
    layer's input, from a seed stream of their own (bf16 bits [rows, K])."""
    d = dict(spec.__dict__)
    d.update(M=int(rows), layer_id=spec.layer_id + 100000)
    return make_x(LinearSpec(**d))


# chained pairs: name -> (up spec, down spec)
PAIRS = {"mlp_pair": ("pair_up", "pair_down")}


def stack_specs(batch: int = 1):
    """The linears of one denoising step of a FLUX-like 12B DiT (228 layers).

    19 double-stream blocks, each with an image stream (4096*batch rows) and a text
    stream (512*batch rows) holding QKV (3072->9216), out (3072->3072), MLP up
    (3072->12288) and MLP down (12288->3072); 38 single-stream blocks (4608*batch
    rows) with fused QKV+MLP-in (3072->21504) and out (15360->3072).
    """
    out = []
    lid = 0
    shapes_double = [(3072, 9216), (3072, 3072), (3072, 12288), (12288, 3072)]
    for blk in range(19):
        for stream, m in (("img", 4096), ("txt", 512)):
            for (k, n) in shapes_double:
                out.append(LinearSpec(f"double{blk}.{stream}.{k}x{n}", 4, m * batch, k, n, 32,
                                      outlier_frac=0.01, outlier_scale=30.0, heavy_tail=True,
                                      gelu_input=(k == 12288), layer_id=lid))
                lid += 1
    for blk in range(38):
        for (k, n) in ((3072, 21504), (15360, 3072)):
            out.append(LinearSpec(f"single{blk}.{k}x{n}", 4, 4608 * batch, k, n, 32,
                                  outlier_frac=0.01, outlier_scale=30.0, heavy_tail=True,
                                  layer_id=lid))
            lid += 1
    return out


def _rng(spec: LinearSpec, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([spec.config_id, spec.layer_id, tensor_id]))


def to_bf16_bits(a64: np.ndarray) -> np.ndarray:
    """Round float64 -> float32 -> bfloat16 with torch's casts; uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 view of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _gelu_tanh(z: np.ndarray) -> np.ndarray:
    # textbook tanh form (Hendrycks & Gimpel): input generation for the down-projection
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def make_x(spec: LinearSpec) -> np.ndarray:
    """Activations [M, K] as bf16 bits."""
    g = _rng(spec, _T_X)
    x = g.standard_normal((spec.M, spec.K))
    if spec.gelu_input:
        x = _gelu_tanh(x)
    n_out = spec.n_outliers()
    if n_out:
        ch = _rng(spec, _T_XOUT).choice(spec.K, size=n_out, replace=False)
        x[:, ch] *= spec.outlier_scale
    if spec.silu_input:
        x = x / (1.0 + np.exp(-x))
    return to_bf16_bits(x)


def _outlier_rows(spec: LinearSpec) -> np.ndarray:
    cnt = int(round(spec.row_outlier_frac * spec.N))
    return _rng(spec, _T_WROW).choice(spec.N, size=cnt, replace=False) if cnt else np.zeros(0, np.int64)


def make_w(spec: LinearSpec) -> np.ndarray:
    """Weights [N, K] as bf16 bits."""
    w = _rng(spec, _T_W).standard_normal((spec.N, spec.K)) * 0.02
    if spec.heavy_tail:
        g = _rng(spec, _T_WTAIL)
        cnt = int(round(0.001 * spec.N * spec.K))
        idx = g.choice(spec.N * spec.K, size=cnt, replace=False)
        w.reshape(-1)[idx] = 0.02 * g.standard_t(3.0, size=cnt)
    w[_outlier_rows(spec)] *= spec.outlier_scale
    return to_bf16_bits(w)


def make_bias(spec: LinearSpec) -> np.ndarray:
    b = _rng(spec, _T_BIAS).standard_normal(spec.N) * 0.01
    b[_outlier_rows(spec)] *= spec.outlier_scale
    return to_bf16_bits(b)


def make_linear(spec: LinearSpec | str, M: int | None = None) -> dict:
    """X, W and bias for one linear; ``M`` overrides the row count."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    if M is not None:
        spec = spec.with_m(M)
    return {"spec": spec, "x": make_x(spec), "w": make_w(spec), "bias": make_bias(spec)}


def make_rope_tables(M: int, head_dim: int = 128, n_text: int = 512, grid_w: int = 64,
                     axes=(16, 56, 56), theta: float = 10000.0):
    """Per-token rotary tables cos, sin (fp32 [M, head_dim/2]) of a FLUX-like
    DiT: the first n_text tokens (text) sit at position (0, 0, 0), image token t
    at (0, t // grid_w, t % grid_w); the head's channel pairs are split over the
    three position axes (16 + 56 + 56 = 128 channels), pair i of an axis of
    d channels turning at pos * theta^(-2i/d).  Positions and frequencies are
    inputs of the rotary step, not part of it."""
    assert sum(axes) == head_dim
    t = np.arange(M)
    img = np.maximum(t - n_text, 0)
    pos = np.stack([np.zeros(M), np.where(t < n_text, 0, img // grid_w),
                    np.where(t < n_text, 0, img % grid_w)], axis=1).astype(np.float64)
    ang = []
    for a, d in enumerate(axes):
        freq = theta ** (-np.arange(0, d, 2, dtype=np.float64) / d)
        ang.append(pos[:, a:a + 1] * freq[None, :])
    ang = np.concatenate(ang, axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make_norm_weight(spec: LinearSpec, which: int, head_dim: int = 128) -> np.ndarray:
    """Learned RMSNorm scale of Q (which=0) or K (which=1): 1 + 0.1 N(0,1), bf16 bits."""
    g = np.random.default_rng(np.random.SeedSequence([spec.config_id, spec.layer_id, _T_NORM, which]))
    return to_bf16_bits(1.0 + 0.1 * g.standard_normal(head_dim))
