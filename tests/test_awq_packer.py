"""The library's host AWQ packer (svdq_awq_pack_weights) against the oracle's
awq_pack: same alpha, same smoothing vector, same codes, scales and zero points.

Both evaluate the grid's output errors in float64 with different summation
orders, so the two could only pick different alphas where two grid points'
errors agree to ~1e-15 relative; the test then requires exactly that near-tie
and compares the quantization at the library's alpha."""
import numpy as np
import pytest

import oracle.awq_oracle as A
import synthetic as S
from bit_diffusion_transformer_svdq_amd import awq_pack_weights


@pytest.mark.parametrize("Mc,K,N,seed", [(16, 128, 32, 0), (24, 256, 96, 1), (8, 64, 64, 2), (32, 512, 48, 3)])
def test_awq_packer_matches_oracle(Mc, K, N, seed):
    spec = S.LinearSpec(f"awqpk{seed}", 8, Mc, K, N, 0, outlier_frac=0.03, outlier_scale=10.0,
                        heavy_tail=True, silu_input=True, layer_id=seed)
    xc = S.make_calibration(spec, Mc)
    w = S.make_w(spec)
    ref = A.awq_pack(xc, w)
    got = awq_pack_weights(w, xc)
    if got["alpha"] != ref["alpha"]:
        i, j = round(got["alpha"] * 20), round(ref["alpha"] * 20)
        assert abs(ref["losses"][i] - ref["losses"][j]) <= 1e-12 * ref["losses"][j]
        ref = {**ref, **dict(zip(("q", "scales", "zeros"), A.quantize_asym_groups(
            A.bf16_to_f64(w) * got["smooth"].astype(np.float64)[None, :])))}
        ref["codes"] = A.pack_uint4(ref["q"])
        ref["smooth"] = got["smooth"]
    assert np.array_equal(got["smooth"], ref["smooth"])
    assert np.array_equal(got["codes"], ref["codes"])
    assert np.array_equal(got["scales"], ref["scales"])
    assert np.array_equal(got["zeros"], ref["zeros"])


def test_awq_packer_thread_count_does_not_matter(monkeypatch):
    spec = S.LinearSpec("awqthr", 8, 16, 256, 64, 0, outlier_frac=0.03, outlier_scale=10.0, silu_input=True)
    xc, w = S.make_calibration(spec, 16), S.make_w(spec)
    monkeypatch.setenv("SVDQ_PACK_THREADS", "1")
    one = awq_pack_weights(w, xc)
    monkeypatch.setenv("SVDQ_PACK_THREADS", "5")
    five = awq_pack_weights(w, xc)
    for k in ("smooth", "codes", "scales", "zeros"):
        assert np.array_equal(one[k], five[k])
    assert one["alpha"] == five["alpha"]
