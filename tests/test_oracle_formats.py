"""Pins of the oracle's number formats against sources other than itself.

E4M3: torch's float8_e4m3fn conversions (a library routine, RNE and exact
decode) and the OCP table values in golden/formats.json.  E2M1: the OCP MX
table in golden/formats.json and the midpoint ladder derived by hand from it.
"""
import json
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def torch_e4m3_decode(code):
    return torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()


def torch_e4m3_encode(x):
    """torch's RNE cast; it does not saturate (beyond 464 it gives NaN), so
    callers only use it for |x| < 464."""
    return torch.tensor([x], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item()


def test_e4m3_decode_all_codes_match_torch(oracle_mod):
    for c in range(256):
        got = oracle_mod.e4m3_decode(c)
        ref = torch_e4m3_decode(c)
        if np.isnan(ref):
            assert np.isnan(got), c
        else:
            assert got == ref, (c, got, ref)


def test_e4m3_table_points(oracle_mod):
    g = _gold("formats.json")["e4m3"]
    for key in ("max_normal", "min_normal", "max_subnormal", "min_subnormal"):
        assert oracle_mod.e4m3_decode(int(g[key + "_code"], 16)) == g[key]
    assert oracle_mod.e4m3_decode(int(g["one_code"], 16)) == 1.0
    for c in g["nan_codes"]:
        assert np.isnan(oracle_mod.e4m3_decode(int(c, 16)))
    assert oracle_mod.e4m3_encode(1.0) == int(g["one_code"], 16)


def _e4m3_test_values():
    vals = []
    finite = [torch_e4m3_decode(c) for c in range(0x7F)]  # 0 .. 448, ascending
    for i in range(len(finite) - 1):
        lo, hi = finite[i], finite[i + 1]
        mid = np.float32((lo + hi) / 2)  # exact in fp32 (5 significant bits)
        vals += [lo, hi, mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    g = np.random.Generator(np.random.PCG64(7))
    vals += list(np.exp2(g.uniform(-22, 9, 4000)).astype(np.float32))
    vals += [1e-40, 1e-45, 0.0, 447.9, 448.0, 455.9, 463.99]
    vals = np.asarray(vals, dtype=np.float32)
    return np.concatenate([vals, -vals])


def test_e4m3_encode_matches_torch_rne_in_range(oracle_mod):
    for x in _e4m3_test_values():
        if abs(x) >= 464.0:
            continue
        assert oracle_mod.e4m3_encode(float(x)) == torch_e4m3_encode(float(x)), float(x)


def test_e4m3_encode_saturates(oracle_mod):
    for x in (464.0, 480.0, 1e4, 3.4e38, float("inf")):
        assert oracle_mod.e4m3_encode(x) == 0x7E
        assert oracle_mod.e4m3_encode(-x) == 0xFE


def test_e4m3_encode_signed_zero(oracle_mod):
    assert oracle_mod.e4m3_encode(0.0) == 0x00
    assert oracle_mod.e4m3_encode(-0.0) == 0x80
    assert oracle_mod.e4m3_encode(-1e-9) == 0x80  # rounds to -0


def test_e2m1_decode_matches_ocp_table(oracle_mod):
    mags = _gold("formats.json")["e2m1_magnitudes_by_code"]
    for c in range(8):
        assert oracle_mod.e2m1_decode(c) == mags[c]
        assert oracle_mod.e2m1_decode(c | 8) == -mags[c]


# Midpoints between adjacent E2M1 magnitudes and the code a tie goes to (the
# even one): 0.25 -> 0, 0.75 -> 2, 1.25 -> 2, 1.75 -> 4, 2.5 -> 4, 3.5 -> 6, 5 -> 6.
LADDER = [(0.25, 0, 1), (0.75, 2, 1), (1.25, 2, 3), (1.75, 4, 3), (2.5, 4, 5), (3.5, 6, 5),
          (5.0, 6, 7)]


@pytest.mark.parametrize("mid,tie_code,other", LADDER)
def test_e2m1_encode_ladder(oracle_mod, mid, tie_code, other):
    below = float(np.nextafter(np.float32(mid), np.float32(0)))
    above = float(np.nextafter(np.float32(mid), np.float32(100)))
    assert oracle_mod.e2m1_encode(mid) == tie_code
    lo_code, hi_code = sorted([tie_code, other])
    assert oracle_mod.e2m1_encode(below) == lo_code
    assert oracle_mod.e2m1_encode(above) == hi_code
    assert oracle_mod.e2m1_encode(-mid) == tie_code | 8


def test_e2m1_encode_exact_values_and_saturation(oracle_mod):
    mags = _gold("formats.json")["e2m1_magnitudes_by_code"]
    for c, m in enumerate(mags):
        assert oracle_mod.e2m1_encode(m) == c
    for x in (6.0, 7.0, 1e6, float("inf")):
        assert oracle_mod.e2m1_encode(x) == 7
        assert oracle_mod.e2m1_encode(-x) == 15
    assert oracle_mod.e2m1_encode(-0.0) == 8
    assert oracle_mod.e2m1_encode(0.1) == 0
