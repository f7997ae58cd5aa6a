"""Pins for the oracle's format tables and rounding functions (CPU only).

Pinned against things other than the oracle itself: printed value lists from
the format definitions (tests/golden), torch's float8_e4m3fn decode and cast
(a library routine), and an independent binade-by-binade np.rint formulation
of round-to-nearest-even onto the E2M1 grid.
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            out[int(code, 16)] = float(val)
    return out


def test_e2m1_values_match_format_definition(oracle_mod):
    gold = _read_table("e2m1_values.txt")
    assert sorted(gold) == list(range(16))
    for code, val in gold.items():
        got = oracle_mod.e2m1_value(code)
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e2m1_qmax_is_six(oracle_mod):
    # q_max of Eq. 3 is the largest finite FP4 magnitude.
    assert np.max(np.abs(oracle_mod.e2m1_table())) == 6.0


def test_e4m3_table_matches_torch_decode(oracle_mod):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle_mod.e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_landmarks(oracle_mod):
    for code, val in _read_table("e4m3_landmarks.txt").items():
        got = oracle_mod.e4m3_value(code)
        assert got == val and np.signbit(got) == np.signbit(val), (hex(code), got, val)
    fin = oracle_mod.e4m3_table()[:127]
    assert np.all(np.diff(fin) > 0), "non-negative E4M3 codes must be ordered by value"


def _e4m3_probe_points(oracle_mod):
    vals = oracle_mod.e4m3_table()[:127]
    mids = (vals[:-1] + vals[1:]) / 2.0
    pts = np.concatenate([vals, mids]).astype(np.float32)
    bits = pts.view(np.int32)
    around = (bits[:, None] + np.arange(-64, 65, dtype=np.int32)[None, :]).ravel()
    around = around[around >= 0].view(np.float32)
    rng = np.random.default_rng(7)
    rand = rng.uniform(0, 464, size=200_000).astype(np.float32)
    logu = np.exp2(rng.uniform(-30, np.log2(464), size=200_000)).astype(np.float32)
    return np.concatenate([pts, around, rand, logu, np.float32([0.0, 2.0 ** -10, 3 * 2.0 ** -11])])


def test_e4m3_encode_matches_torch_cast(oracle_mod):
    s = _e4m3_probe_points(oracle_mod)
    s = s[(s >= 0) & (s <= 464.0)]  # torch's cast gives NaN above 464 instead of saturating
    ref = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle_mod.e4m3_encode(s)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(s[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


def test_e4m3_encode_corners(oracle_mod):
    enc = lambda v: int(oracle_mod.e4m3_encode([v])[0])
    assert enc(0.0) == 0
    assert enc(2.0 ** -10) == 0x00  # tie between 0 and 2^-9 goes to the even code 0
    assert enc(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 0x01
    assert enc(3 * 2.0 ** -11) == 0x01
    assert enc(1.0625) == 0x38  # tie between 1.0 and 1.125 -> 1.0
    assert enc(1.1875) == 0x3A  # tie between 1.125 and 1.25 -> 1.25
    assert enc(448.0) == 0x7E
    for big in (449.0, 464.0, 465.0, 1e6, 3.0e38, float("inf")):
        assert enc(big) == 0x7E  # saturates at 448


def _e2m1_rint_reference(v: np.ndarray) -> np.ndarray:
    """Independent formulation: scale by the binade's grid step, np.rint (ties to
    even), clip at 6, re-attach the sign; then map the value back to its code."""
    a = np.abs(v.astype(np.float64))
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = np.minimum(np.rint(a / step) * step, 6.0)
    mag_code = np.select([q == 0, q == 0.5, q == 1, q == 1.5, q == 2, q == 3, q == 4, q == 6],
                         [0, 1, 2, 3, 4, 5, 6, 7], default=-1)
    assert np.all(mag_code >= 0)
    return (mag_code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def test_e2m1_encode_matches_rint_formulation(oracle_mod):
    grid = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7, 8], dtype=np.float32)
    bits = grid.view(np.int32)
    around = (bits[:, None] + np.arange(-2048, 2049, dtype=np.int32)[None, :]).ravel()
    around = around[around >= 0].view(np.float32)
    stride = np.arange(0, np.float32(8.0).view(np.int32), 257, dtype=np.int32).view(np.float32)
    pos = np.concatenate([around, stride, np.float32([0.0, 6.5, 100.0, 3e38, np.inf])])
    v = np.concatenate([pos, -pos])
    got = oracle_mod.e2m1_encode(v)
    ref = _e2m1_rint_reference(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


def test_e2m1_ties_and_signed_zero(oracle_mod):
    enc = lambda x: int(oracle_mod.e2m1_encode([x])[0])
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, code in ties.items():
        assert enc(t) == code and enc(-t) == code | 8
    assert enc(-0.0) == 0x8 and enc(0.0) == 0x0
    assert enc(-1e-30) == 0x8
    assert enc(6.0) == 7 and enc(1e30) == 7 and enc(-1e30) == 0xF
