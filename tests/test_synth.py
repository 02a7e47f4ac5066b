"""The shared seeded input generator (SplitMix64 in counter form)."""
import numpy as np

import synth
from synth.gen import GAMMA, mix64


def test_splitmix64_reference_sequence():
    # SplitMix64 (Steele, Lea, Flood 2014) seeded with 0 produces, in order,
    # these four outputs (the published reference implementation's sequence).
    expected = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    ctr = (np.arange(1, 5, dtype=np.uint64) * np.uint64(GAMMA))
    got = [int(v) for v in mix64(ctr)]
    assert got == expected


def test_counter_form_matches_indices():
    a = synth.normal_f16(3, 17, (1000,), 0.5)
    idx = np.array([0, 5, 999, 123], dtype=np.uint64)
    b = synth.normal_f16(3, 17, sigma=0.5, index=idx)
    assert np.array_equal(a[idx.astype(np.int64)].view(np.uint16), b.view(np.uint16))


def test_normal_moments_and_support():
    x = synth.normal_f16(0, 1, (1 << 20,), 0.02).astype(np.float64)
    assert abs(x.mean()) < 1e-4
    assert abs(x.std() - 0.02) < 2e-4
    assert np.abs(x).max() <= 0.02 * 3.47


def test_streams_differ_and_ids_in_range():
    a = synth.normal_f16(0, 1, (4096,), 1.0)
    b = synth.normal_f16(0, 2, (4096,), 1.0)
    assert not np.array_equal(a, b)
    ids = synth.token_ids(0, synth.STREAM["prompt"], (64, 512), 50272)
    assert ids.min() >= 0 and ids.max() < 50272
    assert len(np.unique(ids)) > 20000


def test_heavy_tailed_kinds():
    """Scale and tails of the heavy-tailed test inputs: t(3) has variance 3
    sigma^2 and a far tail (P(|t| > 10) ~ 2e-3); the Laplace draw has std sigma
    and kurtosis 6; the outlier mixture has about 1/64 of its entries at 40x."""
    n = 1 << 18
    t = synth.heavy_tailed_f16(0, 5, (n,), 1.0, "student_t3").astype(np.float64)
    assert abs(np.median(t)) < 0.02
    assert 0.37 < np.mean(np.abs(t) > 1.0) < 0.41  # P(|t3| > 1) = 0.391
    assert np.mean(np.abs(t) > 10.0) > 5e-4
    lap = synth.heavy_tailed_f16(0, 6, (n,), 0.02, "laplace").astype(np.float64)
    assert abs(lap.std() - 0.02) < 5e-4
    kurt = np.mean(lap ** 4) / np.mean(lap ** 2) ** 2
    assert 5.0 < kurt < 7.0
    o = synth.heavy_tailed_f16(0, 7, (n,), 0.02, "outliers").astype(np.float64)
    frac = np.mean(np.abs(o) > 0.02 * 6)
    assert 0.8 / 64 < frac < 1.2 / 64
    # counter form: the same element from a longer tensor
    a = synth.heavy_tailed_f16(1, 9, (100,), 1.0, "laplace")
    b = synth.heavy_tailed_f16(1, 9, (10, 20), 1.0, "laplace").ravel()[:100]
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
