"""The seeded input generator: reproducible bytes, exact dtype casts, outliers."""
import numpy as np
import torch

from post_weight_quantization_accum_amd import synth
from post_weight_quantization_accum_amd.configs import WORKLOADS


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000)).astype(np.float32)
    a[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]  # ties to even
    mine = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(mine),
                                  torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_layers_reproduce_and_chunks_regenerate():
    a = synth.make_layer(16, 40, 20000, dtype="bf16", sigma_w=0.02, dist="t4",
                         outlier_frac=0.05, outlier_scale=50, config=9, layer=1, threads=4)
    b = synth.make_layer(16, 40, 20000, dtype="bf16", sigma_w=0.02, dist="t4",
                         outlier_frac=0.05, outlier_scale=50, config=9, layer=1, threads=1)
    np.testing.assert_array_equal(a.W, b.W)
    np.testing.assert_array_equal(a.X, b.X)
    assert len(a.outliers) == 2
    # a shorter draw reproduces the leading chunk exactly
    c = synth.make_layer(16, 40, synth.CHUNK, dtype="bf16", sigma_w=0.02, dist="t4",
                         outlier_frac=0.05, outlier_scale=50, config=9, layer=1)
    np.testing.assert_array_equal(c.X, a.X[:synth.CHUNK])


def test_outlier_channels_are_scaled():
    L = synth.make_layer(4, 64, 30000, dtype="f32", sigma_w=0.02, dist="t4",
                         outlier_count=3, outlier_scale=100.0, config=9, layer=2)
    x = L.X_f64()
    rms = np.sqrt((x ** 2).mean(0))
    big = np.argsort(-rms)[:3]
    assert sorted(big.tolist()) == sorted(L.outliers.tolist())
    assert rms[L.outliers].min() > 30 * np.median(rms)


def test_t4_moments():
    L = synth.make_layer(1, 8, 200000, dtype="f32", sigma_w=0.02, dist="t4", config=9, layer=3)
    x = L.X_f64().ravel()
    assert abs(x.mean()) < 0.02
    assert abs(x.var() - 2.0) < 0.15  # Student-t(4) variance nu/(nu-2) = 2
    # heavy tail: P(|x| > 4) = 0.0161 for t(4) vs 6e-5 for a unit Gaussian
    assert 0.012 < np.mean(np.abs(x) > 4) < 0.021


def test_gauss_mix_and_fp16():
    L = synth.make_layer(8, 32, 4096, dtype="f16", sigma_w=0.02, dist="gauss_mix", config=9, layer=4)
    assert L.X.dtype == np.float16 and L.W.dtype == np.float16
    c = np.corrcoef(L.X_f64().T)
    assert np.abs(c - np.eye(32)).max() > 0.3  # correlated channels
    assert L.clamps == 0


def test_workload_registry():
    wl = WORKLOADS[3]
    assert ("down", 4096, 11008, 6) in wl.layers
    assert wl.quants[0].act_order and wl.quants[0].group_size == 128 and wl.quants[0].bits == 4
    assert WORKLOADS[1].quants[0].group_size <= 0
    assert {q.bits for q in WORKLOADS[4].quants} == {2, 3}
