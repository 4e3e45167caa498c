"""Benchmark of the SVDQuant W4A4 + low-rank linear on one MI355X.

One step = the whole per-inference hot path on one batch: call 1
(svdq_quantize_act_lora_down: smoothing, int4 quantization, packing, fused
lora_down) followed by call 2 (svdq_w4a4_gemm_lora_up: W4A4 GEMM, group dequant,
fused lora_up, bias), back to back on one stream, inputs resident in HBM.
Weight packing is offline (once per layer) and is not part of a step; its host
time is reported separately.

Workload (default): the MLP up-projection of a 12B-class DiT at 1024x1024,
M = 4608 tokens (4096 image + 512 text), K = 3072, N = 12288, rank 32, group 64,
synthetic seeded inputs (see the ``synthetic`` module).  Four input/output
buffer sets (> 512 MB) rotate so the 256 MB last-level cache cannot hold the
working set between steps.

Prints ONE JSON line.  ``value`` = effective TOPS = 2*M*N*K / step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TOPS + % int8-MFMA peak, W4A4+LoRA linear M=4608 K=3072 N=12288"
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
SETTLE_S = 0.3     # untimed steps before the warmup steps (clock ramp), seconds
NSETS = 4          # at least this many rotating input/weight/output sets ...
ROTATE_BYTES = 512e6  # ... and enough of them to exceed the 256 MB last-level cache twice
GEMM_SRC = os.path.join(ROOT, "bit_diffusion_transformer_svdq_amd", "csrc", "w4a4_gemm_lora_up.hip")
QUANT_SRC = os.path.join(ROOT, "bit_diffusion_transformer_svdq_amd", "csrc", "quant_lora_down.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_mlp_up.json")


def gemm_min_bytes(M, N, K, r):
    """Algorithmic HBM bytes of call 2 (every operand read once, Y written once)."""
    return (M * K // 2 + N * K // 2 + 2 * M * K // 64 + 2 * N * K // 64 + 2 * M * r + 2 * N * r
            + 2 * N + 2 * M * N)


def quant_min_bytes(M, K, r):
    """Algorithmic HBM bytes of call 1."""
    return 2 * M * K + 4 * K + 2 * K * r + M * K // 2 + 2 * M * K // 64 + 2 * M * r


def _sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _bf(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def measure_gpu(spec_name, M, steps, warmup, seed=0):
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    import synthetic as S

    spec = S.SPECS[spec_name].with_m(M) if M else S.SPECS[spec_name]
    d = S.make_linear(spec)
    Mv, Kd, N, r = spec.M, spec.K, spec.N, spec.r
    # host-side packer (offline step of the product path)
    absmax = np.abs(S.bf16_bits_to_f32(d["x"])).max(axis=0).astype(np.float32)
    t0 = time.perf_counter()
    lam = K.smooth_from_absmax(absmax, d["w"])
    packed = K.pack_weights(d["w"], lam, r, seed=seed)
    pack_s = time.perf_counter() - t0

    dev = torch.device("cuda:0")
    K.check_device(0)
    per_set = (2 * Mv * Kd + 4 * Kd + 2 * r * Kd + 2 * r * N + N * Kd // 2 + 2 * N * Kd // 64 + 2 * N
               + Mv * Kd // 2 + 2 * Mv * Kd // 64 + 2 * Mv * r + 2 * Mv * N)
    nsets = int(min(32, max(NSETS, -(-ROTATE_BYTES // per_set))))
    sets = []
    for _ in range(nsets):
        sets.append(dict(
            x=_bf(d["x"], dev), lam=torch.from_numpy(lam).to(dev),
            down=_bf(packed["lora_down"], dev), up=_bf(packed["lora_up"], dev),
            wc=torch.from_numpy(packed["w_codes"]).to(dev), ws=_bf(packed["w_scales"], dev),
            bias=_bf(d["bias"], dev),
            codes=torch.empty((Mv, Kd // 2), dtype=torch.uint8, device=dev),
            scales=torch.empty((Mv, Kd // 64), dtype=torch.bfloat16, device=dev),
            la=torch.empty((Mv, r), dtype=torch.bfloat16, device=dev),
            y=torch.empty((Mv, N), dtype=torch.bfloat16, device=dev)))
    stream = torch.cuda.current_stream()

    def step(s, evs=None):
        if evs is not None:
            evs[0].record(stream)
        K.quantize_act_lora_down(s["x"], s["lam"], s["down"], out=(s["codes"], s["scales"], s["la"]),
                                 stream=stream)
        if evs is not None:
            evs[1].record(stream)
        K.w4a4_gemm_lora_up(s["codes"], s["scales"], s["wc"], s["ws"], s["la"], s["up"], s["bias"],
                            out=s["y"], stream=stream)
        if evs is not None:
            evs[2].record(stream)

    # The engine clock ramps up over the first ~0.2 s of sustained load: before
    # the W warmup steps the same step runs untimed for SETTLE_S seconds
    # (reported as settle_s), so short runs time the clock a server runs at.
    t_settle, n_settle = time.perf_counter(), 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(8):
            step(sets[n_settle % nsets])
            n_settle += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    # wall clock over exactly `steps` steps
    t0 = time.perf_counter()
    for i in range(steps):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-kernel durations with HIP events on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(sets[i % nsets], evs[i])
    torch.cuda.synchronize()
    tq = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    tg = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    return dict(spec=spec, M=Mv, K=Kd, N=N, r=r, wall_s=wall, steps=steps, t_quant=tq, t_gemm=tg,
                pack_s=pack_s, nsets=nsets)


def measure_gpu_graph(spec_name, M, reps, seed=0):
    """Calls 1 and 2 of one linear timed from HIP graph replays: per set one
    launch of each call is captured (all rotating sets in one graph), and the
    graph of call 1 alone, of call 2 alone and of both are replayed `reps`
    times between HIP events.  A few-token call is shorter than the host's
    launch path, so timing eager launches one by one would count host gaps;
    the replays run back to back on the GPU."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    import synthetic as S

    spec = S.SPECS[spec_name].with_m(M)
    d = S.make_linear(spec)
    Mv, Kd, N, r = spec.M, spec.K, spec.N, spec.r
    absmax = np.abs(S.bf16_bits_to_f32(d["x"])).max(axis=0).astype(np.float32)
    lam = K.smooth_from_absmax(absmax, d["w"])
    packed = K.pack_weights(d["w"], lam, r, seed=seed)
    dev = torch.device("cuda:0")
    per_set = N * Kd // 2 + 2 * N * Kd // 64 + 2 * r * N + 2 * Mv * Kd + 2 * Mv * N
    nsets = int(min(64, max(NSETS, -(-ROTATE_BYTES // per_set))))
    sets = []
    for _ in range(nsets):
        sets.append(dict(
            x=_bf(d["x"], dev), lam=torch.from_numpy(lam).to(dev),
            down=_bf(packed["lora_down"], dev), up=_bf(packed["lora_up"], dev),
            wc=torch.from_numpy(packed["w_codes"]).to(dev), ws=_bf(packed["w_scales"], dev),
            bias=_bf(d["bias"], dev),
            codes=torch.empty((Mv, Kd // 2), dtype=torch.uint8, device=dev),
            scales=torch.empty((Mv, Kd // 64), dtype=torch.bfloat16, device=dev),
            la=torch.empty((Mv, r), dtype=torch.bfloat16, device=dev),
            y=torch.empty((Mv, N), dtype=torch.bfloat16, device=dev)))
    stream = torch.cuda.Stream()

    def call1(s):
        K.quantize_act_lora_down(s["x"], s["lam"], s["down"], out=(s["codes"], s["scales"], s["la"]), stream=stream)

    def call2(s):
        K.w4a4_gemm_lora_up(s["codes"], s["scales"], s["wc"], s["ws"], s["la"], s["up"], s["bias"], out=s["y"],
                            stream=stream)

    graphs = {}
    with torch.cuda.stream(stream):
        for s in sets:           # eager once: workspaces exist before capture
            call1(s)
            call2(s)
        torch.cuda.synchronize()
        for name, fns in (("a", (call1,)), ("b", (call2,)), ("ab", (call1, call2))):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for s in sets:
                    for fn in fns:
                        fn(s)
            graphs[name] = g
        torch.cuda.synchronize()
        res = {}
        for name, g in graphs.items():
            for _ in range(3):
                g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) * 1e-3 / (reps * nsets)
    return dict(spec=spec, M=Mv, K=Kd, N=N, r=r, nsets=nsets, t_quant=res["a"], t_gemm=res["b"], t_step=res["ab"])


def _pack_dev(K, w, lam, bias, r, dev, seed=0):
    import torch
    packed = K.pack_weights(w, lam, r, seed=seed)
    return {"smooth": torch.from_numpy(lam).to(dev),
            "lora_down": _bf(packed["lora_down"], dev) if r else None,
            "lora_up": _bf(packed["lora_up"], dev) if r else None,
            "w_codes": torch.from_numpy(packed["w_codes"]).to(dev), "w_scales": _bf(packed["w_scales"], dev),
            "bias": _bf(bias, dev)}


def measure_pair(pair_name, steps, warmup):
    """The chained MLP pair: up-projection with the GELU epilogue, H [M, N_up] bf16
    left in HBM, down-projection on H; four launches on one stream per step."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    import synthetic as S

    su, sd = (S.SPECS[n] for n in S.PAIRS[pair_name])
    du = S.make_linear(su)
    wd, bd = S.make_w(sd), S.make_bias(sd)
    dev = torch.device("cuda:0")
    K.check_device(0)
    absmax = np.abs(S.bf16_bits_to_f32(du["x"])).max(axis=0).astype(np.float32)
    up = _pack_dev(K, du["w"], K.smooth_from_absmax(absmax, du["w"]), du["bias"], su.r, dev)
    # the down-projection's smoothing is calibrated on the float model's GELU
    # output (offline set-up, outside the timed region)
    x = _bf(du["x"], dev)
    with torch.no_grad():
        hf = torch.nn.functional.gelu(x.float() @ _bf(du["w"], dev).float().T + _bf(du["bias"], dev).float(),
                                      approximate="tanh")
        habs = hf.abs().amax(dim=0).cpu().numpy().astype(np.float32)
    del hf
    down = _pack_dev(K, wd, K.smooth_from_absmax(habs, wd), bd, sd.r, dev)
    M, N_up, N_dn = su.M, su.N, sd.N
    per_set = 2 * M * su.K + 2 * M * N_up + 2 * M * N_dn
    nsets = int(min(16, max(2, -(-ROTATE_BYTES // per_set))))
    sets = [dict(x=x.clone(), h=torch.empty((M, N_up), dtype=torch.bfloat16, device=dev),
                 y=torch.empty((M, N_dn), dtype=torch.bfloat16, device=dev)) for _ in range(nsets)]
    stream = torch.cuda.current_stream()
    bufs = dict(cu=torch.empty((M, su.K // 2), dtype=torch.uint8, device=dev),
                su=torch.empty((M, su.K // 64), dtype=torch.bfloat16, device=dev),
                lu=torch.empty((M, su.r), dtype=torch.bfloat16, device=dev),
                cd=torch.empty((M, sd.K // 2), dtype=torch.uint8, device=dev),
                sd=torch.empty((M, sd.K // 64), dtype=torch.bfloat16, device=dev),
                ld=torch.empty((M, sd.r), dtype=torch.bfloat16, device=dev))

    def step(s, evs=None):
        rec = (lambda i: evs[i].record(stream)) if evs is not None else (lambda i: None)
        rec(0)
        K.quantize_act_lora_down(s["x"], up["smooth"], up["lora_down"], out=(bufs["cu"], bufs["su"], bufs["lu"]),
                                 stream=stream)
        rec(1)
        K.w4a4_gemm_lora_up(bufs["cu"], bufs["su"], up["w_codes"], up["w_scales"], bufs["lu"], up["lora_up"],
                            up["bias"], out=s["h"], stream=stream, epilogue="gelu_tanh")
        rec(2)
        K.quantize_act_lora_down(s["h"], down["smooth"], down["lora_down"], out=(bufs["cd"], bufs["sd"], bufs["ld"]),
                                 stream=stream)
        rec(3)
        K.w4a4_gemm_lora_up(bufs["cd"], bufs["sd"], down["w_codes"], down["w_scales"], bufs["ld"],
                            down["lora_up"], down["bias"], out=s["y"], stream=stream)
        rec(4)

    for i in range(warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        step(sets[i % nsets], evs[i])
    torch.cuda.synchronize()
    t = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e-3 for j in range(4)]
    ops = 2.0 * M * su.K * N_up + 2.0 * M * sd.K * N_dn
    return {"workload": f"{pair_name}: up M={M} K={su.K} N={N_up} + GELU-tanh epilogue, H bf16 in HBM, "
                        f"down K={sd.K} N={N_dn}, rank {su.r}, group 64",
            "buffer_sets": nsets, "us_per_pair": wall * 1e6, "eff_TOPS": ops / wall / 1e12,
            "pct_int8_peak": 100.0 * ops / wall / 1e12 / INT8_PEAK_TOPS,
            "us_quant_up": t[0] * 1e6, "us_gemm_up_gelu": t[1] * 1e6,
            "us_quant_down": t[2] * 1e6, "us_gemm_down": t[3] * 1e6,
            "quant_down_GB/s": quant_min_bytes(M, sd.K, sd.r) / t[2] / 1e9,
            "gemm_up_TOP/s": 2.0 * M * su.K * N_up / t[1] / 1e12,
            "gemm_down_TOP/s": 2.0 * M * sd.K * N_dn / t[3] / 1e12}


def measure_qkv(steps, warmup):
    """The fused QKV projection (M=4608, K=3072, N=9216, 24 heads of 128 per
    third): call 1 + call 2 with the fused Q/K RMSNorm + rotary epilogue, and
    the same with the plain epilogue, back to back on one stream."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    import synthetic as S

    spec = S.SPECS["qkv"]
    d = S.make_linear(spec)
    dev = torch.device("cuda:0")
    K.check_device(0)
    absmax = np.abs(S.bf16_bits_to_f32(d["x"])).max(axis=0).astype(np.float32)
    L = _pack_dev(K, d["w"], K.smooth_from_absmax(absmax, d["w"]), d["bias"], spec.r, dev)
    cos, sin = S.make_rope_tables(spec.M, 128)
    cos, sin = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
    qn, kn = _bf(S.make_norm_weight(spec, 0), dev), _bf(S.make_norm_weight(spec, 1), dev)
    M, Kd, N, r = spec.M, spec.K, spec.N, spec.r
    per_set = 2 * M * Kd + 2 * M * N
    nsets = int(min(16, max(NSETS, -(-ROTATE_BYTES // per_set))))
    sets = [dict(x=_bf(d["x"], dev), y=torch.empty((M, N), dtype=torch.bfloat16, device=dev))
            for _ in range(nsets)]
    q = (torch.empty((M, Kd // 2), dtype=torch.uint8, device=dev),
         torch.empty((M, Kd // 64), dtype=torch.bfloat16, device=dev),
         torch.empty((M, r), dtype=torch.bfloat16, device=dev))
    stream = torch.cuda.current_stream()

    def step(s, fused, evs=None):
        if evs is not None:
            evs[0].record(stream)
        K.quantize_act_lora_down(s["x"], L["smooth"], L["lora_down"], out=q, stream=stream)
        if evs is not None:
            evs[1].record(stream)
        if fused:
            K.w4a4_gemm_qkv_norm_rope(q[0], q[1], L["w_codes"], L["w_scales"], q[2], L["lora_up"], L["bias"],
                                      qn, kn, cos, sin, out=s["y"], stream=stream)
        else:
            K.w4a4_gemm_lora_up(q[0], q[1], L["w_codes"], L["w_scales"], q[2], L["lora_up"], L["bias"],
                                out=s["y"], stream=stream)
        if evs is not None:
            evs[2].record(stream)

    res = {"workload": f"qkv: fused QKV projection M={M} K={Kd} N={N} (3 x 24 heads of 128), rank {r}, "
                       f"group 64, per-head RMSNorm + rotary epilogue on Q and K", "buffer_sets": nsets}
    for fused in (False, True):
        for i in range(warmup):
            step(sets[i % nsets], fused)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            step(sets[i % nsets], fused, evs[i])
        torch.cuda.synchronize()
        tq = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
        tg = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e-3
        key = "fused" if fused else "plain"
        res[f"us_quant_{key}"] = tq * 1e6
        res[f"us_gemm_{key}"] = tg * 1e6
        res[f"gemm_TOP/s_{key}"] = 2.0 * M * N * Kd / tg / 1e12
    res["eff_TOPS_fused"] = 2.0 * M * N * Kd / ((res["us_quant_fused"] + res["us_gemm_fused"]) * 1e-6) / 1e12
    res["epilogue_extra_us"] = res["us_gemm_fused"] - res["us_gemm_plain"]
    return res


FP4_PEAK_TFLOPS = 10100.0   # MI355X dense FP4 MFMA, 10.1 PFLOP/s


def measure_fp4(spec_name, steps=100, warmup=50):
    """The FP4 (MXFP4) variant of the same linear: call 1 (MXFP4 quantizer with
    fused lora_down) + call 2 (block-scaled FP4 MFMA GEMM + lora_up + bias),
    weights from the host packer, rotating buffer sets, HIP events per call."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    import synthetic as S

    spec = S.SPECS[spec_name]
    d = S.make_linear(spec)
    dev = torch.device("cuda:0")
    K.check_device(0)
    absmax = np.abs(S.bf16_bits_to_f32(d["x"])).max(axis=0).astype(np.float32)
    lam = K.smooth_from_absmax(absmax, d["w"])
    pk = K.pack_weights_fp4(d["w"], lam, spec.r)
    M, Kd, N, r = spec.M, spec.K, spec.N, spec.r
    per_set = 2 * M * Kd + 2 * M * N + N * Kd // 2
    nsets = int(min(16, max(NSETS, -(-ROTATE_BYTES // per_set))))
    sets = [dict(x=_bf(d["x"], dev), wc=torch.from_numpy(pk["w_codes"]).to(dev),
                 ws=torch.from_numpy(pk["w_scales"]).to(dev),
                 y=torch.empty((M, N), dtype=torch.bfloat16, device=dev)) for _ in range(nsets)]
    lam_t = torch.from_numpy(lam).to(dev)
    down, up, bias = _bf(pk["lora_down"], dev), _bf(pk["lora_up"], dev), _bf(d["bias"], dev)
    q = (torch.empty((M, Kd // 2), dtype=torch.uint8, device=dev),
         torch.empty((M, Kd // 32), dtype=torch.uint8, device=dev),
         torch.empty((M, r), dtype=torch.bfloat16, device=dev))
    stream = torch.cuda.current_stream()

    def step(s, evs=None):
        if evs is not None:
            evs[0].record(stream)
        K.quantize_act_lora_down_fp4(s["x"], lam_t, down, out=q, stream=stream)
        if evs is not None:
            evs[1].record(stream)
        K.fp4_gemm_lora_up(q[0], q[1], s["wc"], s["ws"], q[2], up, bias, out=s["y"], stream=stream)
        if evs is not None:
            evs[2].record(stream)

    for i in range(warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(sets[i % nsets], evs[i])
    torch.cuda.synchronize()
    tq = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
    tg = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e-3
    ops = 2.0 * M * N * Kd
    return {"workload": f"{spec_name} in MXFP4: M={M} K={Kd} N={N} rank {r}, E2M1 elements, E8M0 scale per 32",
            "buffer_sets": nsets, "us_per_step": wall * 1e6, "eff_TFLOPS": ops / wall / 1e12,
            "us_quant": tq * 1e6, "us_gemm": tg * 1e6, "gemm_TFLOP/s": ops / tg / 1e12,
            "gemm_fp4_frac": ops / tg / 1e12 / FP4_PEAK_TFLOPS,
            "quant_GB/s": (2 * M * Kd + M * Kd // 2 + M * Kd // 32 + 2 * M * r) / tq / 1e9}


def awq_bytes(M, N, K):
    """Algorithmic HBM bytes of one AWQ W4A16 linear (weights, scales, zero
    points and bias read once, x and s read, Y written)."""
    return N * K // 2 + 3 * N * (K // 64) + 2 * N + 2 * M * K + 4 * K + 2 * M * N


def measure_awq(batch, steps=20, warmup=5, calib_rows=16):
    """The AWQ W4A16 modulation projections of one denoising step of a FLUX-like
    12B DiT: 19 double blocks x (image, text) 3072 -> 18432, 38 single blocks
    3072 -> 9216, the final layer 3072 -> 6144; one conditioning vector per
    image (M = batch); 77 launches, each layer with its own weight buffers.
    Each shape is packed once by the host packer (AWQ search on calib_rows
    calibration rows) and copied into every layer's buffers."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    import synthetic as S

    dev = torch.device("cuda:0")
    K.check_device(0)
    packs = {}
    t0 = time.perf_counter()
    for name, spec in S.MOD_SPECS.items():
        w = S.make_w(spec)
        pk = K.awq_pack_weights(w, S.make_calibration(spec, calib_rows))
        packs[name] = dict(spec=spec.with_m(batch), x=_bf(S.make_x(spec.with_m(batch)), dev),
                           smooth=torch.from_numpy(pk["smooth"]).to(dev),
                           codes=torch.from_numpy(pk["codes"]).to(dev), scales=_bf(pk["scales"], dev),
                           zeros=torch.from_numpy(pk["zeros"]).to(dev), bias=_bf(S.make_bias(spec), dev),
                           alpha=pk["alpha"])
    pack_s = time.perf_counter() - t0
    order = ["mod_double"] * 38 + ["mod_single"] * 38 + ["mod_final"]
    layers = []
    for name in order:
        src = packs[name]
        layers.append(dict(name=name, spec=src["spec"], x=src["x"], smooth=src["smooth"], bias=src["bias"],
                           codes=src["codes"].clone(), scales=src["scales"].clone(), zeros=src["zeros"].clone()))
    ys = {n: torch.empty((batch, p["spec"].N), dtype=torch.bfloat16, device=dev) for n, p in packs.items()}
    stream = torch.cuda.Stream()

    def step():
        for L in layers:
            K.awq_w4a16_gemm(L["x"], L["smooth"], L["codes"], L["scales"], L["zeros"], L["bias"],
                             out=ys[L["name"]], stream=stream)

    def timed(fn, n):
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            t = time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
        return (time.perf_counter() - t) / n

    byts = sum(awq_bytes(L["spec"].M, L["spec"].N, L["spec"].K) for L in layers)
    t_eager = timed(step, steps)
    # per-launch kernel time of the largest shape, HIP events on the launch stream
    L0 = layers[0]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    with torch.cuda.stream(stream):
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        evs[0].record(stream)
        for L in layers[:38]:
            K.awq_w4a16_gemm(L["x"], L["smooth"], L["codes"], L["scales"], L["zeros"], L["bias"],
                             out=ys[L["name"]], stream=stream)
        evs[1].record(stream)
    torch.cuda.synchronize()
    t_double = evs[0].elapsed_time(evs[1]) * 1e-3 / 38
    b_double = awq_bytes(batch, 18432, 3072)
    out = {"workload": f"AWQ W4A16 modulation projections of one denoising step, batch {batch}: 38 x 3072->18432, "
                       f"38 x 3072->9216, 1 x 3072->6144, group 64, M = {batch}",
           "launches": len(layers), "bytes_per_step": byts, "offline_pack_s": pack_s,
           "alpha": {n: p["alpha"] for n, p in packs.items()},
           "ms_eager": t_eager * 1e3, "GB/s_eager": byts / t_eager / 1e9,
           "us_per_launch_3072x18432": t_double * 1e6,
           "GB/s_3072x18432": b_double / t_double / 1e9,
           "hbm_frac_3072x18432": b_double / t_double / 1e9 / HBM_PEAK_GBS}
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step()
        t_graph = timed(g.replay, steps)
        out.update({"ms_graph": t_graph * 1e3, "GB/s_graph": byts / t_graph / 1e9,
                    "hbm_frac_graph": byts / t_graph / 1e9 / HBM_PEAK_GBS})
    except Exception as e:
        out["graph_error"] = f"{type(e).__name__}: {e}"
    # the same 77 projections as 3 stacked launches (every projection of one
    # shape reads the same conditioning vector): one weight buffer per shape
    # holding all of its layers, as a loader would lay them out
    stacks = []
    for name in ("mod_double", "mod_single", "mod_final"):
        Ls = [L for L in layers if L["name"] == name]
        src = packs[name]
        stacks.append(dict(x=src["x"], smooth=torch.stack([L["smooth"] for L in Ls]),
                           codes=torch.stack([L["codes"] for L in Ls]), scales=torch.stack([L["scales"] for L in Ls]),
                           zeros=torch.stack([L["zeros"] for L in Ls]), bias=torch.stack([L["bias"] for L in Ls]),
                           y=torch.empty((len(Ls), batch, src["spec"].N), dtype=torch.bfloat16, device=dev)))

    def step_stacked():
        for st in stacks:
            K.awq_w4a16_gemm_stacked(st["x"], st["smooth"], st["codes"], st["scales"], st["zeros"], st["bias"],
                                     out=st["y"], stream=stream)

    t_st = timed(step_stacked, steps)
    # the stacked 38 x 3072 -> 18432 launch alone, HIP events on the launch stream
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for _ in range(10):
            st = stacks[0]
            K.awq_w4a16_gemm_stacked(st["x"], st["smooth"], st["codes"], st["scales"], st["zeros"], st["bias"],
                                     out=st["y"], stream=stream)
        evs[1].record(stream)
    torch.cuda.synchronize()
    t_st0 = evs[0].elapsed_time(evs[1]) * 1e-3 / 10
    b_st0 = 38 * b_double
    out.update({"launches_stacked": len(stacks), "ms_stacked": t_st * 1e3, "GB/s_stacked": byts / t_st / 1e9,
                "hbm_frac_stacked": byts / t_st / 1e9 / HBM_PEAK_GBS,
                "us_stacked_38x3072x18432": t_st0 * 1e6, "GB/s_stacked_38x3072x18432": b_st0 / t_st0 / 1e9})
    return out


def measure_stack(batch, steps, warmup):
    """One denoising step's linear stack of a FLUX-like 12B DiT: 228 SVDQuant
    linears (456 launches), each layer with its own device buffers of packed
    weights, run back to back on one stream, eagerly and as one captured HIP
    graph.  Packing all 228 layers on the host would take minutes and the
    timing does not depend on the values, so each of the 6 distinct weight
    shapes is packed once and copied into every layer's own buffers; the MLP
    up-projections of the double-stream blocks carry the GELU epilogue."""
    import torch
    import bit_diffusion_transformer_svdq_amd as K
    import synthetic as S

    specs = S.stack_specs(batch)
    dev = torch.device("cuda:0")
    K.check_device(0)
    first_kn, first_mk = {}, {}
    for sp in specs:
        first_kn.setdefault((sp.K, sp.N), sp)
        first_mk.setdefault((sp.M, sp.K), sp)
    # activations: drawn once per shape at batch 1; a batch of B images
    # repeats them B times (the timing does not depend on the values)
    xs = {}
    for (m, k), sp in first_mk.items():
        x1 = _bf(S.make_x(sp.with_m(m // batch)), dev)
        xs[(m, k)] = x1.repeat(batch, 1).contiguous()
        del x1
    shape_pack = {}
    for kn, sp in first_kn.items():
        w = S.make_w(sp)
        # smoothing from the activations of the first layer with this K
        xm = next(v for (m, k), v in xs.items() if k == kn[0])
        absmax = xm.float().abs().amax(dim=0).cpu().numpy().astype(np.float32)
        shape_pack[kn] = _pack_dev(K, w, K.smooth_from_absmax(absmax, w), S.make_bias(sp), sp.r, dev)
    layers = []
    for sp in specs:
        src = shape_pack[(sp.K, sp.N)]
        layers.append(dict(spec=sp, w={k: (None if v is None else v.clone()) for k, v in src.items()},
                           gelu=sp.name.startswith("double") and sp.N == 12288))
    quant = {mk: (torch.empty((mk[0], mk[1] // 2), dtype=torch.uint8, device=dev),
                  torch.empty((mk[0], mk[1] // 64), dtype=torch.bfloat16, device=dev),
                  torch.empty((mk[0], 32), dtype=torch.bfloat16, device=dev)) for mk in first_mk}
    ys = {}
    for sp in specs:
        ys.setdefault((sp.M, sp.N), torch.empty((sp.M, sp.N), dtype=torch.bfloat16, device=dev))
    stream = torch.cuda.Stream()

    def step():
        for L in layers:
            sp, w = L["spec"], L["w"]
            q = quant[(sp.M, sp.K)]
            K.quantize_act_lora_down(xs[(sp.M, sp.K)], w["smooth"], w["lora_down"], out=q, stream=stream)
            K.w4a4_gemm_lora_up(q[0], q[1], w["w_codes"], w["w_scales"], q[2], w["lora_up"], w["bias"],
                                out=ys[(sp.M, sp.N)], stream=stream,
                                epilogue="gelu_tanh" if L["gelu"] else "none")

    def timed(fn):
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    ops = sum(2.0 * sp.M * sp.N * sp.K for sp in specs)
    t_eager = timed(step)
    # per-shape breakdown from HIP events around every launch of one more eager step
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in layers]
    with torch.cuda.stream(stream):
        for L, e in zip(layers, evs):
            sp, w = L["spec"], L["w"]
            q = quant[(sp.M, sp.K)]
            e[0].record(stream)
            K.quantize_act_lora_down(xs[(sp.M, sp.K)], w["smooth"], w["lora_down"], out=q, stream=stream)
            e[1].record(stream)
            K.w4a4_gemm_lora_up(q[0], q[1], w["w_codes"], w["w_scales"], q[2], w["lora_up"], w["bias"],
                                out=ys[(sp.M, sp.N)], stream=stream,
                                epilogue="gelu_tanh" if L["gelu"] else "none")
            e[2].record(stream)
    torch.cuda.synchronize()
    by = {}
    for L, e in zip(layers, evs):
        sp = L["spec"]
        b = by.setdefault((sp.M, sp.K, sp.N), [0, 0.0, 0.0])
        b[0] += 1
        b[1] += e[0].elapsed_time(e[1]) * 1e3
        b[2] += e[1].elapsed_time(e[2]) * 1e3
    by_shape = [{"M": m, "K": k, "N": n, "count": c, "us_quant": tq / c, "us_gemm": tg / c,
                 "gemm_TOP/s": 2.0 * m * n * k / (tg / c) / 1e6, "share_of_step": (tq + tg) / (t_eager * 1e6)}
                for (m, k, n), (c, tq, tg) in sorted(by.items())]
    out = {"workload": f"denoising-step linear stack, batch {batch}: 19 double-stream blocks (image "
                       f"{4096 * batch} and text {512 * batch} tokens; QKV, out, MLP up with GELU, MLP down) "
                       f"+ 38 single-stream blocks ({4608 * batch} tokens; 3072->21504, 15360->3072), r=32",
           "layers": len(specs), "launches": 2 * len(specs), "ops_per_step": ops,
           "weight_bytes": int(sum(v.numel() * v.element_size() for L in layers for v in L["w"].values()
                                   if v is not None)),
           "ms_eager": t_eager * 1e3, "eff_TOPS_eager": ops / t_eager / 1e12, "by_shape": by_shape}
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step()
        t_graph = timed(g.replay)
        out.update({"ms_graph": t_graph * 1e3, "eff_TOPS_graph": ops / t_graph / 1e12,
                    "pct_int8_peak_graph": 100.0 * ops / t_graph / 1e12 / INT8_PEAK_TOPS})
    except Exception as e:  # capture problems are reported, not fatal to the bench
        out["graph_error"] = f"{type(e).__name__}: {e}"
    return out


_CPU_CASE = {}


def _cpu_chunk(bounds):
    """One worker's rows of the CPU baseline: the oracle's calls 1 and 2."""
    import oracle as O
    d, lam, packed = _CPU_CASE["case"]
    lo, hi = bounds
    a = O.quantize_act_lora_down(d["x"][lo:hi], lam, packed["lora_down"])
    y, _ = O.linear_output(a["act_codes"], a["act_scales"], packed["w_codes"], packed["w_scales"],
                           a["lora_act"], packed["lora_up"], d["bias"])
    return float(y[0, 0])


def cpu_baseline(spec_name, rows=64):
    """The oracle as written, on the host's cores: the row sample is cut into one
    chunk per core and the chunks run in forked worker processes (the oracle's
    integer group products are single-threaded numpy, so the cores are used
    through processes; BLAS is held to one thread per process)."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    import oracle as O
    import synthetic as S
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    spec = S.SPECS[spec_name].with_m(max(rows, 256))
    d = S.make_linear(spec)
    lam = O.smooth_factors(O.activation_absmax(d["x"]), d["w"])
    packed = O.pack_weights(d["w"], lam, spec.r)
    _CPU_CASE["case"] = (d, lam, packed)
    bounds = [(rows * i // cores, rows * (i + 1) // cores) for i in range(cores)]
    with threadpool_limits(1):
        with mp.get_context("fork").Pool(cores) as pool:
            pool.map(_cpu_chunk, [(0, 1)] * cores)   # workers up and warm
            t0 = time.perf_counter()
            pool.map(_cpu_chunk, bounds, chunksize=1)
            t = time.perf_counter() - t0
    _CPU_CASE.clear()
    ops = 2.0 * rows * spec.N * spec.K
    return {"value": ops / t / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {S.SPECS[spec_name].M} token rows of the same linear "
                      f"(K={spec.K}, N={spec.N}, r={spec.r}), calls 1+2, numpy float64, "
                      f"one row chunk per core in {cores} forked processes; {t:.1f} s"}


def traffic_for(kernel_src_sha):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it matches this source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    info = json.load(open(TRAFFIC_FILE))
    if info.get("kernel_source_sha") != kernel_src_sha:
        return None
    return info.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="mlp_up")
    ap.add_argument("--m", type=int, default=0, help="override the token count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--extra", default="", help="write per-kernel details of extra shapes here (JSON)")
    ap.add_argument("--extra-configs", default="attn_out,qkv,mlp_down")
    ap.add_argument("--extra-m", default="64,256,1024")
    ap.add_argument("--small-m", default="64,256",
                    help="token counts of the same linear reported in the JSON line (HBM-bound regime)")
    ap.add_argument("--pair", default="mlp_pair",
                    help="chained pair reported in the JSON line ('' to skip)")
    ap.add_argument("--qkv", type=int, default=1, help="report the fused QKV projection (0 to skip)")
    ap.add_argument("--fp4", type=int, default=1, help="report the FP4 (MXFP4) variant of the headline (0 to skip)")
    ap.add_argument("--awq", default="1,4",
                    help="batches of the AWQ W4A16 modulation stack reported in the JSON line ('' or 0 to skip)")
    ap.add_argument("--stack", default="1,4",
                    help="batches of the denoising-step stack reported in the JSON line ('' or 0 to skip)")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the layer would shard along tokens with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calib:
        import torch
        n = args.copy_calib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    res = measure_gpu(args.config, args.m, args.steps, args.warmup)
    M, Kd, N, r = res["M"], res["K"], res["N"], res["r"]
    ops = 2.0 * M * N * Kd
    ms = res["wall_s"] / res["steps"] * 1e3
    tq, tg = float(np.mean(res["t_quant"])), float(np.mean(res["t_gemm"]))
    gemm_tops = ops / tg / 1e12
    quant_gbs = quant_min_bytes(M, Kd, r) / tq / 1e9
    gemm_gbs = gemm_min_bytes(M, N, Kd, r) / tg / 1e9
    out = {
        "metric": METRIC,
        "value": ops / (ms * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded; shapes and value distributions of a 12B-class DiT linear)",
        "config": {"workload": f"{res['spec'].name}: SVDQuant W4A4 linear M={M} K={Kd} N={N} rank={r} "
                               f"group=64 (one 1024x1024 image: 4096 image + 512 text tokens)",
                   "M": M, "K": Kd, "N": N, "rank": r, "group_size": 64, "buffer_sets": res["nsets"]},
        "pct_int8_peak": 100.0 * ops / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS,
        "roofline": {"bound": "mfma", "achieved": gemm_tops, "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": gemm_tops / INT8_PEAK_TOPS,
                     "traffic": traffic_for(_sha(GEMM_SRC)),
                     "kernel": "svdq_w4a4_gemm_lora_up (w4a4_gemm_kernel)",
                     "algorithmic_ops_per_launch": ops},
        "kernels": {
            "quantize_act_lora_down": {"us": tq * 1e6, "min_bytes": quant_min_bytes(M, Kd, r),
                                       "GB/s": quant_gbs, "hbm_frac": quant_gbs / HBM_PEAK_GBS},
            "w4a4_gemm_lora_up": {"us": tg * 1e6, "TOP/s": gemm_tops, "int8_frac": gemm_tops / INT8_PEAK_TOPS,
                                  "min_bytes": gemm_min_bytes(M, N, Kd, r), "GB/s": gemm_gbs},
        },
        "offline_pack_s": res["pack_s"],
        "settle_s": SETTLE_S,
    }
    if args.small_m:
        # the same linear with few tokens: K-B streams the 18.9 MB of packed
        # weights, so its figure of merit is HBM bandwidth, not MFMA rate;
        # timed from graph replays (a few-token call is shorter than the host's
        # launch path)
        small = []
        for m in [int(v) for v in args.small_m.split(",") if v]:
            e = measure_gpu_graph(args.config, m, 20)
            tq_, tg_, ts_ = e["t_quant"], e["t_gemm"], e["t_step"]
            gb = gemm_min_bytes(e["M"], e["N"], e["K"], e["r"])
            qb = quant_min_bytes(e["M"], e["K"], e["r"])
            small.append({"M": e["M"], "buffer_sets": e["nsets"], "timing": "HIP graph replays",
                          "us_quant": tq_ * 1e6, "us_gemm": tg_ * 1e6, "us_step": ts_ * 1e6,
                          "gemm_min_bytes": gb, "gemm_GB/s": gb / tg_ / 1e9,
                          "gemm_hbm_frac": gb / tg_ / 1e9 / HBM_PEAK_GBS,
                          "quant_GB/s": qb / tq_ / 1e9,
                          "linear_GB/s": (gb + qb) / ts_ / 1e9,
                          "gemm_TOP/s": 2.0 * e["M"] * e["N"] * e["K"] / tg_ / 1e12})
        out["small_m"] = small
    if args.pair:
        out["mlp_pair"] = measure_pair(args.pair, 50, 20)
    if args.qkv:
        out["qkv_fused"] = measure_qkv(50, 20)
    if args.fp4:
        out["fp4_mxfp4"] = measure_fp4(args.config)
    awq_batches = [int(b) for b in str(args.awq).split(",") if b and int(b) > 0]
    if awq_batches:
        out["awq_w4a16"] = [measure_awq(b) for b in awq_batches]
    batches = [int(b) for b in str(args.stack).split(",") if b and int(b) > 0]
    if batches:
        out["step_stack"] = [measure_stack(b, 5, 2) for b in batches]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.config, args.cpu_rows)

    if args.extra:
        extra = []
        shapes = [(c, 0) for c in args.extra_configs.split(",") if c] + \
                 [(args.config, int(m)) for m in args.extra_m.split(",") if m]
        for name, m in shapes:
            e = measure_gpu(name, m, 50, 5)
            tq_, tg_ = float(np.mean(e["t_quant"])), float(np.mean(e["t_gemm"]))
            ops_ = 2.0 * e["M"] * e["N"] * e["K"]
            extra.append({"config": name, "M": e["M"], "K": e["K"], "N": e["N"], "r": e["r"],
                          "us_quant": tq_ * 1e6, "us_gemm": tg_ * 1e6,
                          "eff_TOPS": ops_ / (e["wall_s"] / e["steps"]) / 1e12,
                          "gemm_TOPS": ops_ / tg_ / 1e12,
                          "quant_GBs": quant_min_bytes(e["M"], e["K"], e["r"]) / tq_ / 1e9,
                          "gemm_GBs": gemm_min_bytes(e["M"], e["N"], e["K"], e["r"]) / tg_ / 1e9})
        with open(args.extra, "w") as f:
            json.dump(extra, f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
