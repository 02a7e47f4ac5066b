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
