"""The two calls inside a captured HIP graph.  Needs an MI355X.

A chain of layers (an MLP pair and a third linear whose call 1 splits K over
workgroups, so the binding's per-stream workspace is used) is run eagerly,
then captured on the same stream and replayed several times with eager work in
between; every replay must reproduce the eager outputs bit for bit (the
kernels are the same and deterministic).  A call whose workspace the binding
would have to allocate during capture fails cleanly instead.
"""
import numpy as np
import pytest

import oracle as O
from tests.gpu_util import custom_case, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_diffusion_transformer_svdq_amd import check_device
    check_device(0)


def _layer(case):
    d, lam, packed = case
    r = packed["lora_down"].shape[0]
    return {"smooth": to_dev(np.asarray(lam, np.float32)),
            "lora_down": to_dev_bf16(packed["lora_down"]) if r else None,
            "lora_up": to_dev_bf16(packed["lora_up"]) if r else None,
            "w_codes": to_dev(packed["w_codes"]), "w_scales": to_dev_bf16(packed["w_scales"]),
            "bias": to_dev_bf16(d["bias"])}


def test_graph_replays_match_eager():
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    M = 200
    up_c, dn_c, third_c = custom_case(M, 256, 512, 16, seed=71), custom_case(M, 512, 256, 16, seed=72), \
        custom_case(M, 1024, 192, 32, seed=73)
    up, dn, third = _layer(up_c), _layer(dn_c), _layer(third_c)
    x = to_dev_bf16(up_c[0]["x"])
    x3 = to_dev_bf16(third_c[0]["x"])
    h = torch.empty((M, 512), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, 256), dtype=torch.bfloat16, device="cuda")
    y3 = torch.empty((M, 192), dtype=torch.bfloat16, device="cuda")
    q3 = (torch.empty((M, 512), dtype=torch.uint8, device="cuda"),
          torch.empty((M, 16), dtype=torch.bfloat16, device="cuda"),
          torch.empty((M, 32), dtype=torch.bfloat16, device="cuda"))
    s = torch.cuda.Stream()

    def chain():
        K.mlp_pair(x, up, dn, h_out=h, out=y)
        c, sc, la = K.quantize_act_lora_down(x3, third["smooth"], third["lora_down"], out=q3)
        K.w4a4_gemm_lora_up(c, sc, third["w_codes"], third["w_scales"], la, third["lora_up"], third["bias"],
                            out=y3)

    K.debug_set_quant_plan(3, 0)   # call 1 splits K into 3 blocks: partials go through the workspace
    try:
        with torch.cuda.stream(s):
            chain()                  # eager, on the capture stream (allocates its workspace)
        torch.cuda.synchronize()
        want = [t.clone() for t in (h, y, y3, *q3)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            chain()
        torch.cuda.synchronize()
        for rep in range(3):
            # everything on the capture stream: the graph's launches use that
            # stream's workspace, like the eager calls on it
            with torch.cuda.stream(s):
                for t in (h, y, y3, *q3):
                    t.zero_()
                chain()              # eager work on the same stream between replays
                for t in (h, y, y3, *q3):
                    t.fill_(7)
                g.replay()
            torch.cuda.synchronize()
            for got, w in zip((h, y, y3, *q3), want):
                assert torch.equal(got, w), rep
    finally:
        K.debug_set_quant_plan(0, 0)
    # the chain's codes of the third layer are still the oracle's
    ref = O.quantize_act_lora_down(third_c[0]["x"], third_c[1], third_c[2]["lora_down"])
    assert np.array_equal(q3[0].cpu().numpy(), ref["act_codes"])


def test_workspace_growth_during_capture_is_refused():
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    d, lam, packed = custom_case(64, 1024, 64, 16, seed=74)
    L = _layer((d, lam, packed))
    x = to_dev_bf16(d["x"])
    out = (torch.empty((64, 512), dtype=torch.uint8, device="cuda"),
           torch.empty((64, 16), dtype=torch.bfloat16, device="cuda"),
           torch.empty((64, 16), dtype=torch.bfloat16, device="cuda"))
    s = torch.cuda.Stream()        # fresh stream: no workspace yet
    K.debug_set_quant_plan(4, 0)
    g = torch.cuda.CUDAGraph()
    err = None
    try:
        with torch.cuda.graph(g, stream=s):
            try:
                K.quantize_act_lora_down(x, L["smooth"], L["lora_down"], out=out)
            except RuntimeError as e:
                err = str(e)
    finally:
        K.debug_set_quant_plan(0, 0)
    torch.cuda.synchronize()
    assert err is not None and "captur" in err.lower(), err
    # outside capture the same call allocates and works
    with torch.cuda.stream(s):
        c, _, _ = K.quantize_act_lora_down(x, L["smooth"], L["lora_down"], out=out)
    torch.cuda.synchronize()
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    assert np.array_equal(c.cpu().numpy(), ref["act_codes"])


def test_graph_replays_awq_and_fp4_match_eager():
    """The AWQ W4A16 linear (one layer and a stack) and both MXFP4 calls inside one captured graph:
    every replay (with eager work on the stream in between) reproduces the
    eager outputs bit for bit, and those match the oracle."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    import oracle.awq_oracle as A
    import oracle.mxfp4_oracle as X
    import synthetic as S
    # MXFP4 linear, K split over workgroups in call 1 (workspace on the stream)
    fspec = S.LinearSpec("graph_fp4", 10, 200, 512, 256, 16, outlier_frac=0.02, outlier_scale=30.0,
                         heavy_tail=True, layer_id=81)
    fd = S.make_linear(fspec)
    flam = O.smooth_factors(O.activation_absmax(fd["x"]), fd["w"])
    fpk = X.pack_weights_fp4(fd["w"], flam, fspec.r)
    fx, fl = to_dev_bf16(fd["x"]), to_dev(np.asarray(flam, np.float32))
    fld, flu = to_dev_bf16(fpk["lora_down"]), to_dev_bf16(fpk["lora_up"])
    fwc, fws, fb = to_dev(fpk["w_codes"]), to_dev(fpk["w_scales"]), to_dev_bf16(fd["bias"])
    fq = (torch.empty((200, 256), dtype=torch.uint8, device="cuda"),
          torch.empty((200, 16), dtype=torch.uint8, device="cuda"),
          torch.empty((200, 16), dtype=torch.bfloat16, device="cuda"))
    fy = torch.empty((200, 256), dtype=torch.bfloat16, device="cuda")
    # AWQ linear at one and at four tokens
    aspec = S.LinearSpec("graph_awq", 8, 4, 1024, 256, 0, outlier_frac=0.03, outlier_scale=10.0,
                         heavy_tail=True, silu_input=True, layer_id=82)
    ax, aw = S.make_x(aspec), S.make_w(aspec)
    apk = A.awq_pack(S.make_calibration(aspec, 16), aw)
    adev = [to_dev(np.asarray(apk["smooth"], np.float32)), to_dev(apk["codes"]), to_dev_bf16(apk["scales"]),
            to_dev(apk["zeros"]), to_dev_bf16(S.make_bias(aspec))]
    ax4, ax1 = to_dev_bf16(ax), to_dev_bf16(ax[:1])
    ay4 = torch.empty((4, 256), dtype=torch.bfloat16, device="cuda")
    ay1 = torch.empty((1, 256), dtype=torch.bfloat16, device="cuda")
    # the same layer twice as a stack of 2 sharing x
    sdev = [torch.stack([t, t]).contiguous() for t in adev]
    ays = torch.empty((2, 4, 256), dtype=torch.bfloat16, device="cuda")
    outs = (*fq, fy, ay4, ay1, ays)
    s = torch.cuda.Stream()

    def chain():
        c, sc, la = K.quantize_act_lora_down_fp4(fx, fl, fld, out=fq)
        K.fp4_gemm_lora_up(c, sc, fwc, fws, la, flu, fb, out=fy)
        K.awq_w4a16_gemm(ax4, *adev, out=ay4)
        K.awq_w4a16_gemm(ax1, *adev, out=ay1)
        K.awq_w4a16_gemm_stacked(ax4, *sdev, out=ays)

    K.debug_set_quant_plan(2, 0)
    try:
        with torch.cuda.stream(s):
            chain()
        torch.cuda.synchronize()
        want = [t.clone() for t in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            chain()
        torch.cuda.synchronize()
        for rep in range(3):
            with torch.cuda.stream(s):
                for t in outs:
                    t.zero_()
                chain()
                for t in outs:
                    t.fill_(7)
                g.replay()
            torch.cuda.synchronize()
            for got, w in zip(outs, want):
                assert torch.equal(got, w), rep
    finally:
        K.debug_set_quant_plan(0, 0)
    ref = X.quantize_act_lora_down_fp4(fd["x"], flam, fpk["lora_down"])
    assert np.array_equal(fq[0].cpu().numpy(), ref["act_codes"])
    assert np.array_equal(fq[1].cpu().numpy(), ref["act_scales"])
    want4, _ = A.awq_linear(ax, apk["smooth"], apk["codes"], apk["scales"], apk["zeros"], S.make_bias(aspec))
    from tests.gpu_util import Y_MAX_ABS, Y_REL_FRO, bf16_bits, y_errors
    rel, mx = y_errors(bf16_bits(ay4), want4)
    assert rel <= Y_REL_FRO and mx <= Y_MAX_ABS, (rel, mx)
    assert torch.equal(ay1[0], ay4[0])
    assert torch.equal(ays[0], ay4) and torch.equal(ays[1], ay4)
