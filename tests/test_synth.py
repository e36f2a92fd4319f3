"""The workload generator (synth/): the C encoders agree byte for byte with the
independent numpy ones, tensors are reproducible and independent of thread
count, and the distributions match the workload recipes."""
import numpy as np

import synth


def test_c_encoders_match_numpy_encoders():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((96, 512)) * np.exp(rng.uniform(-8, 8, (96, 1)))).astype(np.float32)
    x[3] = 0.0                               # an all-zero row / groups / blocks
    a = synth.quant_nvfp4(x)
    b = synth.np_quant_nvfp4(x)
    assert all(np.array_equal(u, v) for u, v in zip(a[:2], b[:2])) and a[2] == b[2]
    a = synth.quant_fp8_token(x)
    b = synth.np_quant_fp8_token(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    a = synth.quant_mxfp8(x)
    b = synth.np_quant_mxfp8(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(synth.to_bf16_bits(x), synth.np_to_bf16_bits(x))


def test_normal_reproducible_and_distribution():
    a = synth.normal((1000, 333), 0.02, 0, synth.ROLE_W)
    b = synth.normal((1000, 333), 0.02, 0, synth.ROLE_W)
    assert np.array_equal(a, b)
    c = synth.normal((1000, 333), 0.02, 1, synth.ROLE_W)
    assert not np.array_equal(a, c)
    assert abs(a.mean()) < 1e-3 and abs(a.std() / 0.02 - 1) < 0.01
    # a prefix of a longer draw is the same draw (counter-based)
    d = synth.normal((2000, 333), 0.02, 0, synth.ROLE_W)
    assert np.array_equal(d.ravel()[:a.size], a.ravel())


def test_outlier_recipe():
    cols = synth.outlier_columns(14336, 0)
    assert cols.size == 143 and np.unique(cols).size == 143
    d = synth.bf16(64, 32, 14336, seed=0)
    assert d["a"].shape == (64, 14336) and d["w"].shape == (32, 14336)


def test_routing_topk():
    ids, w = synth.topk_routing(256, 64, 8, 0)
    assert ids.shape == (256, 8) and ids.min() >= 0 and ids.max() < 64
    assert all(np.unique(r).size == 8 for r in ids)
    assert np.all(np.diff(w, axis=1) <= 0) and np.all(w.sum(axis=1) < 1)
