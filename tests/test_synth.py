"""Seeded input generator: determinism, shapes and the stated distributions."""
import numpy as np
import torch

from w8_quantized_linear_amd import synth


def test_weights_are_deterministic_and_shaped():
    a = synth.make_weights(64, 512, seed=0, layer=3, linear=2)
    b = synth.make_weights(64, 512, seed=0, layer=3, linear=2)
    c = synth.make_weights(64, 512, seed=0, layer=4, linear=2)
    assert a.hi.shape == (64, 256) and a.hi.dtype == torch.uint8
    assert a.lo.shape == (64, 256) and a.scale.shape == (64, 4) and a.scale.dtype == torch.int16
    assert torch.equal(a.hi, b.hi) and torch.equal(a.lo, b.lo) and torch.equal(a.scale, b.scale)
    assert not torch.equal(a.hi, c.hi)


def test_nibble_and_scale_distributions():
    w = synth.make_weights(512, 4096, seed=0)
    hi, lo, sc = w.numpy()
    nib_hi = np.concatenate([(hi & 15).ravel(), (hi >> 4).ravel()]).astype(np.float64)
    nib_lo = np.concatenate([(lo & 15).ravel(), (lo >> 4).ravel()]).astype(np.float64)
    # clamp(round(N(0, 2.5)) + 8, 0, 15): mean ~7.9 (the clamp is asymmetric), sd ~2.5
    assert abs(nib_hi.mean() - 8.0) < 0.1 and 2.3 < nib_hi.std() < 2.7
    assert nib_hi.min() == 0 and nib_hi.max() == 15
    counts = np.bincount(nib_lo.astype(int), minlength=16) / nib_lo.size
    assert np.all(np.abs(counts - 1 / 16) < 0.002)
    s = sc.view(np.float16).astype(np.float64)
    assert abs(np.median(np.log(s)) - np.log(0.01)) < 0.02
    assert abs(np.log(s).std() - 0.3) < 0.02


def test_activations_outliers():
    x = synth.make_activations(4, 4096, seed=0, layer=1, linear=1)
    assert x.dtype == torch.float32 and x.shape == (4, 4096)
    big = (x.abs() > 8).any(dim=0)
    n = synth.n_outliers(4096)
    assert n == 20 and synth.n_outliers(14336) == 72
    # outlier channels are shared by every token of the call
    assert 10 <= int(big.sum()) <= n
    x0 = synth.make_activations(1, 512, outliers=False)
    assert float(x0.abs().max()) < 6
