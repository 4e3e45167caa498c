"""Seeded random shapes through the automatic plans of both calls (int4 and MXFP4).

Kernel choice, work splits, K-splits and tail splits are all picked by the
host's cost models from the shape, so a plan that no hand-picked test forces
could still be wrong.  Each shape runs calls 1 and 2 with every plan left
automatic and is checked against the CPU oracle: codes and scales bit-exact,
lora_act within its fp32 summation bound, Y within relative Frobenius 5e-3 and
max-abs 1e-2 * max|Y*| on every row.  Shapes: M in [1, 700), K a multiple of 64
up to 2496 (of 128 up to 2560 for MXFP4, the ABI's rule), N a multiple of 64 (the
ABI's rule) up to 768, r in {0, 16, 32, 48, 64}.
"""
import numpy as np
import pytest

import oracle as O
from tests.gpu_util import bf16_bits, check_quant, check_y, custom_case, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _shapes(n, seed, kq=64):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 700))
        K = kq * int(rng.integers(1, 2560 // kq))
        N = 64 * int(rng.integers(1, 13))
        r = int(rng.choice([0, 16, 32, 48, 64]))
        out.append((M, K, N, r))
    return out


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_diffusion_transformer_svdq_amd import check_device
    check_device(0)


@pytest.mark.parametrize("M,K,N,r", _shapes(24, 20261203))
def test_random_shape_automatic_plans(M, K, N, r):
    import torch
    import bit_diffusion_transformer_svdq_amd as KK
    d, lam, packed = custom_case(M, K, N, r, seed=M * 7 + K + N + r)
    x = to_dev_bf16(d["x"])
    lam_t = to_dev(np.asarray(lam, np.float32))
    down = to_dev_bf16(packed["lora_down"]) if r else None
    up = to_dev_bf16(packed["lora_up"]) if r else None
    codes, scales, la = KK.quantize_act_lora_down(x, lam_t, down)
    y = KK.w4a4_gemm_lora_up(codes, scales, to_dev(packed["w_codes"]), to_dev_bf16(packed["w_scales"]),
                             la if r else None, up, to_dev_bf16(d["bias"]))
    torch.cuda.synchronize()
    got = {"act_codes": codes.cpu().numpy(), "act_scales": bf16_bits(scales), "lora_act": bf16_bits(la)}
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    check_quant(got, ref, packed["lora_down"])
    check_y(bf16_bits(y), d, lam, packed, ref)


@pytest.mark.parametrize("M,K,N,r", _shapes(12, 20261204, kq=128))
def test_random_shape_automatic_plans_mxfp4(M, K, N, r):
    from tests.test_fp4_gpu import _case, _check, _run, _spec
    d, lam, pk = _case(_spec(M, K, N, r, M + K + N + r))
    _check(_run(d, lam, pk), d, lam, pk)
