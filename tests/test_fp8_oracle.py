"""Pins of the FP8 (e4m3) oracle: the format definition's values, hand-worked rounding
cases, brute force over all codes, and agreement with torch's float8_e4m3fn cast."""

import json
import math
import os

import numpy as np
import torch

from oracle import fp8

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fp8_e4m3.json")


def test_codes_match_the_format_definition():
    g = json.load(open(GOLDEN))
    for code, val in g["codes"]:
        got = float(fp8.decode(np.array([int(code, 16)], np.uint8))[0])
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_every_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8.decode(codes)
    finite = ~np.isnan(vals)
    back = fp8.round_to_code(vals[finite])
    assert np.array_equal(back, codes[finite])
    assert np.isnan(vals).sum() == 2


def test_hand_worked_rounding_cases():
    g = json.load(open(GOLDEN))
    for x, code, why in g["round"]:
        assert int(fp8.quantize(np.array([x], np.float32), 1.0)[0]) == int(code, 16), why


def test_quantize_is_the_nearest_code_by_brute_force():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(4000) * rng.choice([1e-3, 0.1, 1, 30, 300], 4000)).astype(np.float32)
    inv = np.float32(1 / 0.37)
    got = fp8.quantize(x, inv)
    y = np.clip((x * inv).astype(np.float64), -448, 448)
    allv = fp8.decode(np.arange(256, dtype=np.uint8))
    for i in range(len(x)):
        d = np.abs(allv - y[i])
        d[np.isnan(d)] = np.inf
        best = np.flatnonzero(d == d.min())
        best = [b for b in best if (b >= 128) == (y[i] < 0 or (y[i] == 0 and np.signbit(y[i])))] or list(best)
        if len(best) > 1:
            best = [b for b in best if (b & 1) == 0]
        assert int(got[i]) == int(best[0]), (x[i], y[i], got[i], best)


def test_agrees_with_torch_float8_e4m3fn_inside_the_range():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * 50).astype(np.float32)
    x = x[np.abs(x) <= 440]
    ours = fp8.quantize(x, 1.0)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_dequantize_scales_by_the_float32_scale():
    assert fp8.dequantize(np.array([0x38], np.uint8), 0.5)[0] == 0.5
    s = np.float32(0.1)
    assert fp8.dequantize(np.array([0x40], np.uint8), s)[0] == 2.0 * float(s)
