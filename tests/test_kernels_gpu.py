"""Parity of the HIP path (through the C ABI) with the CPU oracle.  Needs an MI355X.

Bar: activation codes, activation scales and the int32 group accumulators are
bit-exact; lora_act is within one bf16 ulp (fp32 vs float64 summation order);
Y is within relative Frobenius 5e-3 and max-abs 1e-2 * max|Y*| of the float64
oracle.  Weights are packed by the oracle, so the kernels are checked on the
oracle's own inputs; the C++ packer is checked separately on the CPU.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from tests.gpu_util import (Y_MAX_ABS, Y_REL_FRO, bf16_bits, check_quant as _check_quant, check_y as _check_y,
                            custom_case, oracle_case, to_dev, to_dev_bf16, y_errors)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_diffusion_transformer_svdq_amd import check_device
    check_device(0)


def _run(d, lam, packed, bias=True):
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    r = packed["lora_down"].shape[0]
    x = to_dev_bf16(d["x"])
    lam_t = to_dev(np.asarray(lam, np.float32))
    down = to_dev_bf16(packed["lora_down"]) if r else None
    up = to_dev_bf16(packed["lora_up"]) if r else None
    wc = to_dev(packed["w_codes"])
    ws = to_dev_bf16(packed["w_scales"])
    b = to_dev_bf16(d["bias"]) if bias else None
    codes, scales, la = K.quantize_act_lora_down(x, lam_t, down)
    y = K.w4a4_gemm_lora_up(codes, scales, wc, ws, la if r else None, up, b)
    torch.cuda.synchronize()
    return {"act_codes": codes.cpu().numpy(), "act_scales": bf16_bits(scales),
            "lora_act": bf16_bits(la), "y": bf16_bits(y)}


def test_tiny_config_full_parity():
    d, lam, packed = oracle_case("tiny")
    got = _run(d, lam, packed)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    _check_quant(got, ref, packed["lora_down"])
    _check_y(got["y"], d, lam, packed, ref)


def test_group_accumulators_bit_exact_tiny():
    import bit_diffusion_transformer_svdq_amd as K
    d, lam, packed = oracle_case("tiny")
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    acc = K.w4a4_group_acc_debug(to_dev(ref["act_codes"]), to_dev(packed["w_codes"])).cpu().numpy()
    want = O.group_accumulators(ref["act_codes"], packed["w_codes"])
    assert np.array_equal(acc, want), np.argwhere(acc != want)[:5]


@pytest.mark.parametrize("M,K,N,r", [
    (1, 64, 64, 0), (17, 128, 192, 16), (127, 320, 64, 48), (129, 256, 320, 64),
    (255, 192, 128, 32), (300, 512, 448, 16), (64, 1024, 256, 128), (513, 64, 64, 16),
])
def test_edge_shapes(M, K, N, r):
    d, lam, packed = custom_case(M, K, N, r, seed=M + N)
    got = _run(d, lam, packed)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    _check_quant(got, ref, packed["lora_down"])
    _check_y(got["y"], d, lam, packed, ref)


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("M,K,N,r", [
    (1, 64, 64, 16), (37, 448, 192, 32), (64, 3072, 1024, 32), (130, 640, 448, 48), (256, 256, 256, 128),
    (300, 192, 320, 16),
])
def test_both_gemm_kernels_parity(path, M, K, N, r):
    """The tiled kernel (path 1) and the K-split few-token kernel (path 2) on the
    same shapes: same codes, accumulators and Y within the bar."""
    import bit_diffusion_transformer_svdq_amd as K_
    d, lam, packed = custom_case(M, K, N, r, seed=M + K + N)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    K_.debug_set_gemm_path(path)
    try:
        got = _run(d, lam, packed)
        acc = K_.w4a4_group_acc_debug(to_dev(ref["act_codes"]), to_dev(packed["w_codes"])).cpu().numpy()
    finally:
        K_.debug_set_gemm_path(0)
    _check_quant(got, ref, packed["lora_down"])
    _check_y(got["y"], d, lam, packed, ref)
    want = O.group_accumulators(ref["act_codes"], packed["w_codes"])
    assert np.array_equal(acc, want), np.argwhere(acc != want)[:5]


@pytest.mark.parametrize("M,K,N", [(37, 192, 320), (200, 128, 64)])
def test_group_accumulators_bit_exact_ragged(M, K, N):
    import bit_diffusion_transformer_svdq_amd as K_
    d, lam, packed = custom_case(M, K, N, 0, seed=3)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    acc = K_.w4a4_group_acc_debug(to_dev(ref["act_codes"]), to_dev(packed["w_codes"])).cpu().numpy()
    want = O.group_accumulators(ref["act_codes"], packed["w_codes"])
    assert np.array_equal(acc, want)


def test_no_bias_and_rank0():
    d, lam, packed = custom_case(96, 256, 128, 0, seed=11)
    got = _run(d, lam, packed, bias=False)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    _check_quant(got, ref, packed["lora_down"])
    _check_y(got["y"], d, lam, packed, ref, bias=False)


def test_extreme_groups_zero_and_saturated():
    """All-zero groups (s = 0, q = 0) and single-spike groups (one code at +-7)."""
    d, lam, packed = custom_case(48, 256, 128, 16, seed=21)
    x = d["x"].copy()
    x[:, 64:128] = 0                     # a whole zero group in every row
    x[5, :] = 0                          # an all-zero row
    x[7, 130] = 0x4700                   # a lone spike
    d = dict(d, x=x)
    got = _run(d, lam, packed)
    ref = O.quantize_act_lora_down(x, lam, packed["lora_down"])
    _check_quant(got, ref, packed["lora_down"])
    assert np.all(got["act_scales"][:, 1] == 0)
    _check_y(got["y"], d, lam, packed, ref)


def test_bf16_rounding_ties_in_smoothing():
    """mu = 1.5 and 2.5 exactly: x * mu needs 9-10 significant bits, so the bf16
    rounding of x_hat hits exact ties often (round half to even decides)."""
    d, lam, packed = custom_case(64, 128, 64, 16, seed=5)
    lam2 = np.full_like(lam, np.float32(1.0))
    lam2[::3] = np.float32(2.0 / 3.0)    # fl32(1 / lambda) = 1.5
    lam2[1::3] = np.float32(0.4)         # fl32(1 / lambda) = 2.5
    p = O.f64_to_f32(O.bf16_to_f64(d["x"]) * (1.0 / lam2.astype(np.float64)).astype(np.float32))
    ties = (p.view(np.uint32) & 0xFFFF) == 0x8000
    assert ties.sum() > 100
    got = _run(d, lam2, packed)
    ref = O.quantize_act_lora_down(d["x"], lam2, packed["lora_down"])
    _check_quant(got, ref, packed["lora_down"])


def test_empty_batch_is_a_noop():
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    d, lam, packed = oracle_case("tiny")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    codes, scales, la = K.quantize_act_lora_down(x, to_dev(lam), to_dev_bf16(packed["lora_down"]))
    y = K.w4a4_gemm_lora_up(codes, scales, to_dev(packed["w_codes"]), to_dev_bf16(packed["w_scales"]),
                            la, to_dev_bf16(packed["lora_up"]), None)
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


def test_outputs_do_not_write_outside_their_buffers():
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    d, lam, packed = custom_case(77, 256, 192, 32, seed=8)
    M, Kd, N, r = 77, 256, 192, 32
    pad = 4096
    sent = 0x5A

    def guarded(n, dtype):
        buf = torch.full((n + 2 * pad,), sent, dtype=torch.uint8, device="cuda")
        return buf

    cb = guarded(M * Kd // 2, torch.uint8)
    sb = guarded(M * (Kd // 64) * 2, torch.uint8)
    lb = guarded(M * r * 2, torch.uint8)
    yb = guarded(M * N * 2, torch.uint8)
    codes = cb[pad:pad + M * Kd // 2].view(M, Kd // 2)
    scales = sb[pad:pad + M * (Kd // 64) * 2].view(torch.bfloat16).view(M, Kd // 64)
    la = lb[pad:pad + M * r * 2].view(torch.bfloat16).view(M, r)
    y = yb[pad:pad + M * N * 2].view(torch.bfloat16).view(M, N)
    K.quantize_act_lora_down(to_dev_bf16(d["x"]), to_dev(lam), to_dev_bf16(packed["lora_down"]),
                             out=(codes, scales, la))
    K.w4a4_gemm_lora_up(codes, scales, to_dev(packed["w_codes"]), to_dev_bf16(packed["w_scales"]), la,
                        to_dev_bf16(packed["lora_up"]), to_dev_bf16(d["bias"]), out=y)
    torch.cuda.synchronize()
    for buf, n in ((cb, M * Kd // 2), (sb, M * (Kd // 64) * 2), (lb, M * r * 2), (yb, M * N * 2)):
        h = buf.cpu().numpy()
        assert np.all(h[:pad] == sent) and np.all(h[pad + n:] == sent)


def test_repeated_launches_are_bit_identical():
    d, lam, packed = custom_case(257, 512, 384, 32, seed=4)
    first = _run(d, lam, packed)
    for _ in range(5):
        again = _run(d, lam, packed)
        for k in first:
            assert np.array_equal(first[k], again[k]), k


def _quant(d, lam, packed, stream=None):
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    r = packed["lora_down"].shape[0]
    codes, scales, la = K.quantize_act_lora_down(
        to_dev_bf16(d["x"]), to_dev(np.asarray(lam, np.float32)),
        to_dev_bf16(packed["lora_down"]) if r else None, stream=stream)
    torch.cuda.synchronize()
    return {"act_codes": codes.cpu().numpy(), "act_scales": bf16_bits(scales), "lora_act": bf16_bits(la)}


@pytest.mark.parametrize("plan,M,K,r", [
    ((1, 1), 200, 448, 32), ((3, 2), 200, 448, 32), ((7, 5), 200, 448, 32), ((2, 12), 200, 448, 32),
    ((0, 1), 200, 448, 32), ((5, 0), 200, 448, 32), ((4, 3), 61, 1024, 128), ((3, 4), 130, 576, 48),
    ((6, 7), 33, 384, 0), ((40, 2), 40, 3072, 16),
])
def test_forced_work_splits(plan, M, K, r):
    """Every split of call 1 (K-blocks, row tiles per workgroup) gives the oracle's
    codes and scales bit for bit and lora_act within its bound; ragged M and a
    ragged last K-block (K = 448 is 7 groups)."""
    import bit_diffusion_transformer_svdq_amd as K_
    d, lam, packed = custom_case(M, K, 64, r, seed=M + K)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    K_.debug_set_quant_plan(*plan)
    try:
        got = _quant(d, lam, packed)
        again = _quant(d, lam, packed)
    finally:
        K_.debug_set_quant_plan(0, 0)
    _check_quant(got, ref, packed["lora_down"] if r else None)
    for k in got:  # the K-block partials are added in a fixed order
        assert np.array_equal(got[k], again[k]), k


@pytest.mark.parametrize("waves,kb,M,K,r", [
    (8, 0, 200, 448, 32),    # 7 groups: one group per wave, 7 waves (ragged last row tile)
    (8, 2, 200, 448, 32),    # blocks of 4 and 3 groups: a wave of the last block has none
    (8, 1, 64, 3072, 32),    # 48 groups over 8 waves, 6 each: pairs only
    (8, 0, 61, 3072, 128),   # 8 rank tiles, one K-block
    (5, 3, 130, 1344, 48),   # 21 groups in 3 blocks of 7 over 5 waves: odd runs, K-block partials
    (3, 0, 33, 384, 0),      # no low-rank branch
    (2, 4, 40, 3072, 16),    # 4 blocks of 12 over 2 waves
    (8, 0, 16, 15360, 32),   # 240 groups: 4 blocks of 60 (LDS bound), one row tile
])
def test_row_tile_kernel_forced(waves, kb, M, K, r):
    """Call 1's row-tile kernel (a workgroup per row tile, its waves splitting
    each K-block, partials added in LDS in wave order): the oracle's codes and
    scales bit for bit, lora_act within its bound, the same bits on a repeat."""
    import bit_diffusion_transformer_svdq_amd as K_
    d, lam, packed = custom_case(M, K, 64, r, seed=M + K + waves)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    K_.debug_set_quant_waves(waves)
    K_.debug_set_quant_plan(kb, 0)
    try:
        got = _quant(d, lam, packed)
        again = _quant(d, lam, packed)
    finally:
        K_.debug_set_quant_waves(0)
        K_.debug_set_quant_plan(0, 0)
    _check_quant(got, ref, packed["lora_down"] if r else None)
    for k in got:
        assert np.array_equal(got[k], again[k]), k


def test_quantizer_scale_sweep_covers_every_scale():
    """One group per bf16 group maximum A whose scale s = bf16(A/7) lies in
    [2^-100, 2^100], i.e. every scale that reaches the kernel's fast reciprocal
    (so that path is checked exhaustively), plus maxima outside that range
    (IEEE division path; below 7 * 2^-128 fl32(1/s) overflows and the group
    quantizes to zero) and all-zero groups.  lambda = 1, so x_hat = x; each
    group holds +-A and 63 values drawn from [-A, A]."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K_
    rng = np.random.default_rng(7)
    a_bits = np.arange(0, 0x7F80, dtype=np.uint32)
    a_all = (a_bits << 16).view(np.float32).astype(np.float64)
    s_all = O.bf16_to_f64(O.f32_to_bf16((a_all / 7.0).astype(np.float32)))
    in_rng = (s_all >= 2.0 ** -100) & (s_all <= 2.0 ** 100)
    assert in_rng.sum() > 25000
    extra = np.concatenate([2.0 ** rng.uniform(-126, -99, 150), 2.0 ** rng.uniform(101, 127, 150)])
    A = np.concatenate([a_all[in_rng], extra, np.zeros(64)])
    G, Kd = len(A), 4096
    M = -(-G // (Kd // 64))
    A = np.concatenate([A, np.ones(M * (Kd // 64) - G)])
    A_bits = O.f64_to_bf16(A)
    Ab = O.bf16_to_f64(A_bits)
    vals = rng.uniform(-1.0, 1.0, (len(Ab), 64)) * Ab[:, None]
    pos = rng.integers(0, 64, len(Ab))
    vals[np.arange(len(Ab)), pos] = Ab * np.where(rng.random(len(Ab)) < 0.5, -1.0, 1.0)
    x_bits = O.f64_to_bf16(vals).reshape(M, Kd)
    lam = np.ones(Kd, np.float32)
    ref = O.quantize_act_lora_down(x_bits, lam, np.zeros((0, Kd), np.uint16))
    codes, scales, _ = K_.quantize_act_lora_down(to_dev_bf16(x_bits), to_dev(lam), None)
    torch.cuda.synchronize()
    got_s = bf16_bits(scales)
    assert np.array_equal(got_s, ref["act_scales"]), np.argwhere(got_s != ref["act_scales"])[:5]
    got_c = codes.cpu().numpy()
    assert np.array_equal(got_c, ref["act_codes"]), np.argwhere(got_c != ref["act_codes"])[:5]


def test_two_streams_use_separate_workspaces():
    """Split-K calls on two streams at once, then a larger problem on one of them
    (the workspace grows), then the first size again."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K_
    cases = [custom_case(300, 512, 64, 32, seed=s) for s in (31, 32)]
    big = custom_case(900, 1024, 64, 32, seed=33)
    refs = [O.quantize_act_lora_down(d["x"], lam, p["lora_down"]) for d, lam, p in cases]
    ref_big = O.quantize_act_lora_down(big[0]["x"], big[1], big[2]["lora_down"])
    ins = [(to_dev_bf16(d["x"]), to_dev(np.asarray(lam, np.float32)), to_dev_bf16(p["lora_down"]))
           for d, lam, p in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    K_.debug_set_quant_plan(4, 2)
    try:
        outs = [None, None]
        for _ in range(3):
            for i in (0, 1):
                outs[i] = K_.quantize_act_lora_down(*ins[i], stream=streams[i])
        torch.cuda.synchronize()
        got = [{"act_codes": c.cpu().numpy(), "act_scales": bf16_bits(s), "lora_act": bf16_bits(l)}
               for c, s, l in outs]
        got_big = _quant(*big, stream=streams[0])
        got_small = _quant(*cases[0], stream=streams[0])
    finally:
        K_.debug_set_quant_plan(0, 0)
    for g, ref, (d, lam, p) in zip(got, refs, cases):
        _check_quant(g, ref, p["lora_down"])
    _check_quant(got_big, ref_big, big[2]["lora_down"])
    _check_quant(got_small, refs[0], cases[0][2]["lora_down"])


# ---- DiT-scale shapes, in the launch configuration the benchmark times ----

def _full_case(name):
    d, lam, packed = oracle_case(name)
    got = _run(d, lam, packed)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    _check_quant(got, ref, packed["lora_down"])     # codes and scales: every row, bit-exact
    M = d["spec"].M
    rows = sorted(set([0, 1, 63, 64, 127, 128, 129, 1000, 2047, 2048, 4095, 4096, 4097, M - 2, M - 1]))
    rows = [r for r in rows if r < M]
    _check_y(got["y"], d, lam, packed, ref, rows=rows)
    return d, packed, ref


@pytest.mark.parametrize("name", ["attn_out", "qkv", "mlp_up", "mlp_down"])
def test_dit_shapes_parity(name):
    _full_case(name)


def test_headline_group_accumulators_on_a_row_window():
    import bit_diffusion_transformer_svdq_amd as K
    d, lam, packed = oracle_case("mlp_up")
    ref = O.quantize_act_lora_down(d["x"][4544:4608], lam, packed["lora_down"])
    acc = K.w4a4_group_acc_debug(to_dev(ref["act_codes"]), to_dev(packed["w_codes"])).cpu().numpy()
    want = O.group_accumulators(ref["act_codes"], packed["w_codes"])
    assert np.array_equal(acc, want)


# ---- K-split of the tiled kernel ----

@pytest.mark.parametrize("splits", [1, 2, 3, 8])
@pytest.mark.parametrize("M,K,N,r", [(200, 1024, 192, 32), (300, 3072, 320, 16), (129, 640, 128, 0)])
def test_forced_gemm_splits(splits, M, K, N, r):
    """Each split count gives Y within the bar (partials added in split order),
    the same bits on a second launch, and the same codes."""
    import bit_diffusion_transformer_svdq_amd as K_
    d, lam, packed = custom_case(M, K, N, r, seed=11 * M + splits)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    K_.debug_set_gemm_path(1)
    K_.debug_set_gemm_splits(splits)
    try:
        got = _run(d, lam, packed)
        again = _run(d, lam, packed)
    finally:
        K_.debug_set_gemm_splits(0)
        K_.debug_set_gemm_path(0)
    _check_quant(got, ref, packed["lora_down"])
    _check_y(got["y"], d, lam, packed, ref)
    assert np.array_equal(got["y"], again["y"])


@pytest.mark.parametrize("M,K,N", [(512, 3072, 3072), (256, 3072, 12288), (512, 12288, 3072),
                                   (128, 3072, 12288), (100, 3072, 12288)])
def test_split_shapes_parity(M, K, N):
    """Token counts of the text stream and the small-M sweep, where the tiled
    kernel splits K automatically (96 to 192 tiles), at their full size; 100
    and 128 tokens of a large layer take the tiled kernel rather than the
    few-token one (the 100-token tile is ragged)."""
    spec = S.LinearSpec(f"split{M}x{K}x{N}", 5, M, K, N, 32, outlier_frac=0.01, outlier_scale=30.0,
                        heavy_tail=True, gelu_input=(K == 12288))
    d, lam, packed = oracle_case(spec)
    got = _run(d, lam, packed)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    _check_quant(got, ref, packed["lora_down"])
    rows = [0, 1, 63, 64, 127, 128, 255, M - 2, M - 1]
    _check_y(got["y"], d, lam, packed, ref, rows=sorted(set(r for r in rows if r < M)))


# ---- the boundary: accumulator windows and caller-owned workspaces ----

@pytest.mark.parametrize("path", [1, 2])
def test_row_views_at_multiples_of_16(path):
    """Codes arrays are in the boundary's storage order (rows 8-15 of every 16
    with their 8-byte halves exchanged), so a view starting at a multiple of 16
    rows is a valid input of call 2: rows 48.. of call 1's outputs give the
    oracle's Y of those rows, on both kernels."""
    import bit_diffusion_transformer_svdq_amd as K
    import torch
    d, lam, packed = custom_case(150, 256, 192, 16, seed=17)
    codes, scales, la = K.quantize_act_lora_down(to_dev_bf16(d["x"]), to_dev(lam), to_dev_bf16(packed["lora_down"]))
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    K.debug_set_gemm_path(path)
    try:
        y = K.w4a4_gemm_lora_up(codes[48:], scales[48:], to_dev(packed["w_codes"]), to_dev_bf16(packed["w_scales"]),
                                la[48:], to_dev_bf16(packed["lora_up"]), to_dev_bf16(d["bias"]))
        torch.cuda.synchronize()
    finally:
        K.debug_set_gemm_path(0)
    y_ref, _ = O.linear_output(ref["act_codes"], ref["act_scales"], packed["w_codes"], packed["w_scales"],
                               ref["lora_act"], packed["lora_up"], d["bias"], rows=np.arange(48, 150))
    rel, mx = y_errors(bf16_bits(y), y_ref)
    assert rel <= Y_REL_FRO and mx <= Y_MAX_ABS, (rel, mx)


@pytest.mark.parametrize("path", [1, 2])
def test_group_accumulator_window(path):
    """The dump hook's window: rows and columns at offsets that are not tile
    or 64 aligned, on both kernels."""
    import bit_diffusion_transformer_svdq_amd as K
    d, lam, packed = custom_case(300, 320, 448, 16, seed=91)
    ref = O.quantize_act_lora_down(d["x"], lam, packed["lora_down"])
    K.debug_set_gemm_path(path)
    try:
        acc = K.w4a4_group_acc_debug(to_dev(ref["act_codes"]), to_dev(packed["w_codes"]),
                                     rows=(37, 100), cols=(70, 129)).cpu().numpy()
    finally:
        K.debug_set_gemm_path(0)
    want = O.group_accumulators(ref["act_codes"], packed["w_codes"], rows=np.arange(37, 137),
                                cols=np.arange(70, 199))
    assert np.array_equal(acc, want), np.argwhere(acc != want)[:5]


def test_caller_workspace_reused_across_shapes():
    """One zero-filled workspace given by the caller serves call 1 and call 2 of
    several shapes in turn (forced K splits, so both use it); the results are
    bit-identical to the calls with the binding's own workspace and match the
    oracle."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    cases = [custom_case(200, 1024, 192, 32, seed=92), custom_case(96, 3072, 320, 16, seed=93)]
    K.debug_set_gemm_path(1)
    K.debug_set_gemm_splits(3)
    K.debug_set_quant_plan(4, 0)
    try:
        need = max(max(K.lib().svdq_quantize_act_workspace_size(d["spec"].M, d["spec"].K, p["lora_down"].shape[0]),
                       K.lib().svdq_w4a4_gemm_workspace_size(d["spec"].M, d["spec"].N, d["spec"].K,
                                                             p["lora_down"].shape[0]))
                   for d, _, p in cases)
        assert need > 0
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        for rep in range(2):
            for d, lam, p in cases:
                x, lam_t = to_dev_bf16(d["x"]), to_dev(np.asarray(lam, np.float32))
                down, up = to_dev_bf16(p["lora_down"]), to_dev_bf16(p["lora_up"])
                wc, wsc, b = to_dev(p["w_codes"]), to_dev_bf16(p["w_scales"]), to_dev_bf16(d["bias"])
                c1, s1, l1 = K.quantize_act_lora_down(x, lam_t, down, workspace=ws)
                y1 = K.w4a4_gemm_lora_up(c1, s1, wc, wsc, l1, up, b, workspace=ws)
                c2, s2, l2 = K.quantize_act_lora_down(x, lam_t, down)
                y2 = K.w4a4_gemm_lora_up(c2, s2, wc, wsc, l2, up, b)
                torch.cuda.synchronize()
                assert torch.equal(c1, c2) and torch.equal(s1, s2) and torch.equal(l1, l2)
                assert torch.equal(y1, y2), rep
                ref = O.quantize_act_lora_down(d["x"], lam, p["lora_down"])
                _check_quant({"act_codes": c1.cpu().numpy(), "act_scales": bf16_bits(s1),
                              "lora_act": bf16_bits(l1)}, ref, p["lora_down"])
                _check_y(bf16_bits(y1), d, lam, p, ref)
        # every counter is back at zero after the calls
        torch.cuda.synchronize()
        assert int(ws[:1 << 20].view(torch.int32).abs().sum()) == 0
    finally:
        K.debug_set_quant_plan(0, 0)
        K.debug_set_gemm_splits(0)
        K.debug_set_gemm_path(0)


def test_too_small_caller_workspace_is_refused():
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    d, lam, p = custom_case(200, 1024, 192, 32, seed=94)
    K.debug_set_gemm_path(1)
    K.debug_set_gemm_splits(2)
    try:
        ref = O.quantize_act_lora_down(d["x"], lam, p["lora_down"])
        need = K.lib().svdq_w4a4_gemm_workspace_size(200, 192, 1024, 32)
        small = torch.zeros(need - 256, dtype=torch.uint8, device="cuda")
        with pytest.raises(K.SvdqError, match="workspace"):
            K.w4a4_gemm_lora_up(to_dev(ref["act_codes"]), to_dev_bf16(ref["act_scales"]), to_dev(p["w_codes"]),
                                to_dev_bf16(p["w_scales"]), to_dev_bf16(ref["lora_act"]),
                                to_dev_bf16(p["lora_up"]), None, workspace=small)
    finally:
        K.debug_set_gemm_splits(0)
        K.debug_set_gemm_path(0)
