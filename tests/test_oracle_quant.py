"""Pins of the oracle's 4-bit group quantiser against facts outside itself:
hand-worked examples (tests/golden/quant_worked_examples.json), brute force over
the 16 levels, the round-trip bound, and the ~70 % memory saving the FlexGen
README states for --compress-weight ("Handle Out-of-memory" section)."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import quantize, dequant_f16, dequant_f64, pack_nibbles, unpack_nibbles

GOLD = os.path.join(os.path.dirname(__file__), "golden", "quant_worked_examples.json")


def _group_from(spec):
    if spec.get("x") == "ramp16":
        x = np.arange(64) % 16
    else:
        x = np.full(64, spec["fill"], dtype=np.float64)
        head = spec["x_head"]
        x[:len(head)] = head
    return x.astype(np.float16)


def _codes_from(spec):
    if spec.get("codes") == "ramp16":
        return (np.arange(64) % 16).astype(np.uint8)
    c = np.full(64, spec["fill_code"], dtype=np.uint8)
    c[:len(spec["codes_head"])] = spec["codes_head"]
    return c


@pytest.mark.parametrize("spec", json.load(open(GOLD))["groups"], ids=lambda s: s["name"])
def test_worked_examples(spec):
    x = _group_from(spec)
    codes, meta = quantize(x[None])
    assert np.array_equal(unpack_nibbles(codes)[0], _codes_from(spec))
    mbits = meta.view(np.uint16)[0, 0]
    assert int(mbits[0]) == int(spec["min_bits"], 16)
    assert int(mbits[1]) == int(spec["scale_bits"], 16)
    rec = dequant_f64(codes, meta)[0]
    if spec.get("recon_exact"):
        assert np.array_equal(rec, x.astype(np.float64))
    if "recon_head" in spec:
        assert np.array_equal(rec[:len(spec["recon_head"])], np.array(spec["recon_head"]))
    if "max_abs_err" in spec:
        assert np.abs(rec - x.astype(np.float64)).max() == spec["max_abs_err"]


def test_nibble_order_low_is_even():
    assert pack_nibbles(np.array([1, 2, 3, 4], np.uint8)).tolist() == [0x21, 0x43]
    assert unpack_nibbles(np.array([0x21, 0x43], np.uint8)).tolist() == [1, 2, 3, 4]


def _random_groups(n_groups, seed=0):
    rows = []
    base = synth.normal_f16(seed, synth.STREAM["aux"], (n_groups, 64), 1.0)
    rows.append(base)
    # wide dynamic range and tiny ranges
    rows.append((base.astype(np.float32) * 1000).astype(np.float16))
    rows.append((1.0 + base.astype(np.float32) * 1e-3).astype(np.float16))
    rows.append((base.astype(np.float32) * 1e-4).astype(np.float16))
    return np.concatenate(rows, 0)


def test_invariants_and_roundtrip_bound():
    x = _random_groups(2048)
    codes, meta = quantize(x)
    c = unpack_nibbles(codes)
    assert c.max() <= 15
    v = x.astype(np.float64)
    mn, s = meta[..., 0, 0].astype(np.float64), meta[..., 0, 1].astype(np.float64)
    # min reconstructs exactly and maps to code 0; the maximum element maps to code 15
    assert np.array_equal(mn, v.min(1))
    nondeg = s > 0
    imin, imax = v.argmin(1), v.argmax(1)
    r = np.arange(len(v))
    assert np.all(c[r, imin] == 0)
    assert np.all(c[r[nondeg], imax[nondeg]] == 15)
    rec = dequant_f64(codes, meta)
    err = np.abs(rec - v)
    assert np.all(err[nondeg] <= (s[nondeg] / 2 * (1 + 2.0 ** -22))[:, None])
    assert np.all(err[~nondeg] == 0)


def test_brute_force_nearest_level():
    """Each code is the nearest of the 16 levels mn + c*s (ties to the even code),
    except within 2^-20 of a half-way point, where fp32 division may land on either side."""
    x = _random_groups(512, seed=1)
    codes, meta = quantize(x)
    c = unpack_nibbles(codes).astype(np.int64)
    v = x.astype(np.float64)
    mn, s = meta[..., 0, 0].astype(np.float64), meta[..., 0, 1].astype(np.float64)
    ok = s > 0
    v, c, mn, s = v[ok], c[ok], mn[ok], s[ok]
    levels = mn[:, None, None] + np.arange(16)[None, None, :] * s[:, None, None]
    d = np.abs(v[..., None] - levels)
    best = d.min(-1, keepdims=True)
    cand = d <= best * (1 + 1e-12)
    n_cand = cand.sum(-1)
    even_pick = np.where(n_cand > 1, np.argmax(cand & (np.arange(16) % 2 == 0), -1), np.argmax(cand, -1))
    frac = (v - mn[:, None]) / s[:, None]
    near_tie = np.abs(frac - np.floor(frac) - 0.5) < 2.0 ** -20
    clamp_hi = frac > 15
    expect = np.where(clamp_hi, 15, even_pick)
    bad = (c != expect) & ~near_tie
    assert not bad.any()


def test_dequant_f16_single_rounding():
    x = _random_groups(256)
    codes, meta = quantize(x)
    a = dequant_f16(codes, meta)
    exact = dequant_f64(codes, meta)
    # fp16 RNE of the exact value: within half an fp16 ulp, and a grid-exact value is unchanged
    ulp = np.spacing(np.abs(a).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(a.astype(np.float64) - exact) <= ulp / 2 + 1e-30)


def test_memory_saving_matches_readme():
    # README, "Handle Out-of-memory": --compress-weight cuts weight memory by around 70 %.
    rows, cols = 128, 4096
    x = np.zeros((rows, cols), np.float16)
    codes, meta = quantize(x)
    ratio = (codes.nbytes + meta.nbytes) / x.nbytes
    assert ratio == 0.28125
    assert 0.65 <= 1 - ratio <= 0.75
