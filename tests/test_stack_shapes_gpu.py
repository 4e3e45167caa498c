"""Parity at the shapes of one denoising step, with weights from the product packer.

The W4A4 layer replaces the attention and MLP projections of the transformer
(mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch Nunchaku
4-Bit-Quantisierung", section "Nunchaku Lite: Nahtlose Integration in
Diffusers").  A FLUX-like 12B step has, besides the single-layer shapes of
test_kernels_gpu.py, the single blocks' fused QKV + MLP-in (3072 -> 21504) and
output (15360 -> 3072) projections, the 512-token text stream, and four images
at once (18432 tokens).  Every case runs the whole product chain:

    svdq_smooth_from_absmax -> svdq_pack_weights (host, C++)
    -> svdq_quantize_act_lora_down -> svdq_w4a4_gemm_lora_up (GPU),

and the oracle is evaluated on the packer's own lora_down, lora_up, w_codes and
w_scales (SVD factors are not unique, so the GEMM is judged on identical
inputs).  Bar: activation codes and scales bit-exact on every row; lora_act
within the fp32 summation bound; Y within relative Frobenius 5e-3 and max-abs
1e-2 * max|Y*| on one row of every 128-row tile (a different row offset in each
tile) plus the last rows, so every output tile of the launch is compared.
Shapes run in the launch configuration the benchmark times (kernel and K-split
chosen by shape)."""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from tests.gpu_util import bf16_bits, check_quant, check_y, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_diffusion_transformer_svdq_amd import check_device
    check_device(0)


def product_pack(d, r, seed=7):
    """Smoothing and packing by the library's host packer (calibration on the
    layer's own input, as the benchmark does)."""
    import bit_diffusion_transformer_svdq_amd as K
    lam = K.smooth_from_absmax(O.activation_absmax(d["x"]).astype(np.float32), d["w"])
    return lam, K.pack_weights(d["w"], lam, r, seed=seed)


def run_chain(d, lam, pk):
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    r = pk["lora_down"].shape[0]
    print(f"chain M={d['x'].shape[0]} K={d['x'].shape[1]} N={pk['w_codes'].shape[0]} r={r}", flush=True)
    codes, scales, la = K.quantize_act_lora_down(to_dev_bf16(d["x"]), to_dev(np.asarray(lam, np.float32)),
                                                 to_dev_bf16(pk["lora_down"]) if r else None)
    y = K.w4a4_gemm_lora_up(codes, scales, to_dev(pk["w_codes"]), to_dev_bf16(pk["w_scales"]),
                            la if r else None, to_dev_bf16(pk["lora_up"]) if r else None,
                            to_dev_bf16(d["bias"]))
    torch.cuda.synchronize()
    return {"act_codes": codes.cpu().numpy(), "act_scales": bf16_bits(scales), "lora_act": bf16_bits(la),
            "y": bf16_bits(y)}


def tile_rows(M, tile=128):
    """One row of every row tile, at an offset that walks through the tile,
    plus the first and the last two rows."""
    rows = {0, M - 2, M - 1}
    for t in range((M + tile - 1) // tile):
        rows.add(min(M - 1, t * tile + (37 * t + 5) % tile))
    return sorted(r for r in rows if r >= 0)


def _stack_spec(tag, M, K, N):
    return S.LinearSpec(f"stack_{tag}", 4, M, K, N, 32, outlier_frac=0.01, outlier_scale=30.0,
                        heavy_tail=True, gelu_input=(K == 12288), layer_id=700 + len(tag))


STACK_SHAPES = [
    ("single_qkv_mlp_in", 4608, 3072, 21504),
    ("single_out", 4608, 15360, 3072),
    ("text_qkv", 512, 3072, 9216),
    ("text_mlp_up", 512, 3072, 12288),
    ("batch4_mlp_up", 18432, 3072, 12288),
]


@pytest.mark.parametrize("tag,M,K,N", STACK_SHAPES, ids=[s[0] for s in STACK_SHAPES])
def test_step_stack_shape_packer_fed(tag, M, K, N):
    d = S.make_linear(_stack_spec(tag, M, K, N))
    lam, pk = product_pack(d, 32)
    got = run_chain(d, lam, pk)
    ref = O.quantize_act_lora_down(d["x"], lam, pk["lora_down"])
    check_quant(got, ref, pk["lora_down"])
    check_y(got["y"], d, lam, pk, ref, rows=tile_rows(M))


@pytest.mark.parametrize("M,K,N,r", [(300, 1024, 448, 32), (129, 3072, 640, 16), (64, 256, 256, 0)])
def test_packer_fed_chain_full_output(M, K, N, r):
    """Small shapes: every element of Y against the oracle on the packer's output."""
    spec = S.LinearSpec(f"pk{M}x{K}x{N}r{r}", 9, M, K, N, r, outlier_frac=0.01, outlier_scale=30.0,
                        heavy_tail=True, layer_id=800 + M)
    d = S.make_linear(spec)
    lam, pk = product_pack(d, r)
    got = run_chain(d, lam, pk)
    ref = O.quantize_act_lora_down(d["x"], lam, pk["lora_down"])
    check_quant(got, ref, pk["lora_down"] if r else None)
    check_y(got["y"], d, lam, pk, ref)


def test_headline_every_tile_packer_fed():
    """The headline linear (M=4608, K=3072, N=12288, r=32) on the packer's
    weights, Y on one row of every 128-row tile."""
    d = S.make_linear(S.SPECS["mlp_up"])
    lam, pk = product_pack(d, 32)
    got = run_chain(d, lam, pk)
    ref = O.quantize_act_lora_down(d["x"], lam, pk["lora_down"])
    check_quant(got, ref, pk["lora_down"])
    check_y(got["y"], d, lam, pk, ref, rows=tile_rows(4608))
