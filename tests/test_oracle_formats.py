"""Pins of the oracle's element formats against sources other than itself:
torch's own float8/e8m0 decoders and BF16 rounding, the OCP element table of FP4,
brute-force nearest-value search, and hand-worked examples under tests/golden/."""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _torch_e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def test_e2m1_decode_matches_ocp_table(orc):
    rows = _rows("e2m1_values.txt")
    assert len(rows) == 16
    for nib, val in rows:
        v = orc.e2m1_value(int(nib))
        assert v == float(val) and math.copysign(1, v) == math.copysign(1, float(val))


def test_e4m3_decode_matches_torch(orc):
    ref = _torch_e4m3_table()
    for c in range(256):
        v = orc.e4m3_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(v), c
        else:
            assert v == ref[c] and math.copysign(1, v) == math.copysign(1, ref[c]), c
    assert orc.e4m3_value(0x7E) == 448.0 and math.isnan(orc.e4m3_value(0x7F))


def test_e8m0_decode_matches_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    for c in range(256):
        v = orc.e8m0_value(c)
        if math.isnan(ref[c]):
            assert math.isnan(v)
        else:
            assert v == ref[c], c


def _brute_force_e4m3(values):
    """Nearest finite e4m3 value (by torch's decode table), ties to the even code,
    saturating: the definition of RNE-satfinite written as a search."""
    table = _torch_e4m3_table()
    codes = np.arange(127)                      # 0x00..0x7E: finite non-negative codes
    mags = table[:127]
    out = []
    for v in values:
        a = abs(float(v))
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:                       # a tie: keep the even mantissa
            best = [b for b in best if b % 2 == 0]
        c = int(codes[best[0]])
        if math.copysign(1.0, float(v)) < 0:
            c |= 0x80
        out.append(c)
    return np.array(out, np.uint8)


def test_e4m3_encode_golden(orc):
    for val, code, *_ in _rows("e4m3_encode.txt"):
        got = int(orc.e4m3_encode(np.array([float(val)], np.float32))[0])
        assert got == int(code, 16), (val, hex(got), code)


def test_e4m3_encode_matches_brute_force(orc):
    rng = np.random.default_rng(0)
    table = _torch_e4m3_table()[:127]
    mids = (table[1:] + table[:-1]) / 2           # every tie point
    vals = np.concatenate([
        table, -table, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        rng.standard_normal(4000) * 30, rng.uniform(-600, 600, 2000),
        rng.uniform(-0.02, 0.02, 2000), [448.0, 464.0, 470.0, 1e6, -1e6, 2.0 ** -12],
    ]).astype(np.float32)
    got = orc.e4m3_encode(vals)
    ref = _brute_force_e4m3(vals)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_e4m3_encode_agrees_with_torch_rne_inside_range(orc):
    """torch's cast is RNE (but NaN instead of saturation beyond 464): inside the
    finite range the two must agree code for code."""
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(20000) * 64).astype(np.float32)
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(v), ref)


def test_block_exponent_golden(orc):
    for amax, rule, scale, elem in _rows("block_exponent.txt"):
        e = int(orc.block_exponent(np.array([float(amax)], np.float32), rule == "floor")[0])
        assert e + 127 == int(scale, 16), (amax, rule, e)
        block = np.zeros(32, np.float32)
        block[3] = float(amax)
        codes, scales = orc.quantize_blocks(block, rule == "floor")
        assert int(scales[0]) == int(scale, 16)
        assert int(codes[3]) == int(elem, 16), (amax, rule, hex(codes[3]))


def test_block_exponent_properties(orc):
    """ceil: the smallest e with amax*2^-e <= 448; floor: amax*2^-e in [256, 512)."""
    rng = np.random.default_rng(2)
    amax = np.concatenate([np.exp(rng.uniform(-60, 60, 5000)),
                           [1.75, 1.7500001, 3.5, 448.0, 449.0, 2.0 ** -119]]).astype(np.float32)
    ec = orc.block_exponent(amax, False)
    ef = orc.block_exponent(amax, True)
    for a, c, f in zip(amax.astype(np.float64), ec, ef):
        assert a * 2.0 ** -int(c) <= 448.0 < a * 2.0 ** -(int(c) - 1) or c == -127
        assert 256.0 <= a * 2.0 ** -int(f) < 512.0 or f == -127


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(5000) * 100,
                        # exact ties between two BF16 values
                        (np.arange(1, 2000, dtype=np.float64) * 2 + 1) * 2.0 ** -8]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.uint16).numpy()
    got = np.array([orc.float_to_bf16(float(x)) for x in v], np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("rule", [False, True])
def test_quantize_block_codes_match_torch_cast(orc, rule):
    """Codes of a block = torch's RNE cast of clamp(v * 2^-e, +-448), with e the
    block exponent (pinned above)."""
    rng = np.random.default_rng(4 + rule)
    v = (rng.standard_normal((400, 32)) * np.exp(rng.uniform(-8, 8, (400, 1)))).astype(np.float32)
    v[5] = 0.0
    v[6, 7] = -0.0
    codes, scales = orc.quantize_blocks(v, rule)
    e = scales.astype(np.int64) - 127
    scaled = np.clip(v.astype(np.float64) * 2.0 ** (-e), -448, 448).astype(np.float32)
    ref = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    amax = np.abs(v).max(axis=1)
    assert np.array_equal(e[:, 0], orc.block_exponent(amax, rule))
