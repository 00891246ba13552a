"""Pins of the oracle's bf16 and e4m3 codecs against the format definitions,
hand-derived fixtures and library conversions (torch CPU)."""
import math
import os

import numpy as np
import pytest
import torch
import yaml

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32_bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# ----------------------------------------------------------------- bf16 ----

def test_bf16_round_matches_torch_on_fp32(oracle_lib):
    """Every fp32 value is a double, so one-step rounding from double must
    equal torch's fp32 -> bf16 conversion (round to nearest even)."""
    rng = np.random.default_rng(7)
    vals = rng.standard_normal(4000).astype(np.float32) * np.float32(3.0)
    # exact ties: bf16 value + half an ulp, both parities
    base = _f32_bits(rng.standard_normal(2000).astype(np.float32)) & 0xFFFF0000
    ties = (base | 0x8000).view(np.float32)
    tiny = (rng.standard_normal(500) * 1e-39).astype(np.float32)       # fp32 subnormals
    big = (rng.standard_normal(500) * 1e37).astype(np.float32)
    allv = np.concatenate([vals, ties, tiny, big, np.float32([0.0, -0.0, 1.0, -1.0])])
    want = torch.from_numpy(allv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle_lib.bf16_round(float(v))[0] for v in allv], np.uint16)
    assert np.array_equal(got, want)


def test_bf16_round_hand_cases(oracle_lib):
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    assert oracle_lib.bf16_round(1 + 2 ** -8)[0] == 0x3F80
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even -> 1 + 2^-6
    assert oracle_lib.bf16_round(1 + 3 * 2 ** -8)[0] == 0x3F82
    # just above the midpoint rounds up; a double-rounding path through fp32
    # would have produced the tie and then 1.0
    assert oracle_lib.bf16_round(1 + 2 ** -8 + 2 ** -30)[0] == 0x3F81
    assert oracle_lib.bf16_round(-(1 + 2 ** -8 + 2 ** -30))[0] == 0xBF81
    assert oracle_lib.bf16_round(-0.0)[0] == 0x8000
    # above the largest finite bf16 plus half an ulp: infinity
    assert oracle_lib.bf16_round(2.0 ** 128)[0] == 0x7F80


def test_bf16_near_tie_flag(oracle_lib):
    d = 2.0 ** -18
    # 2^-20 above the midpoint of [1, 1 + 2^-7]: relative distance < 2^-18
    code, near, other = oracle_lib.bf16_round(1 + 2 ** -8 + 2 ** -20, d)
    assert (code, near, other) == (0x3F81, True, 0x3F80)
    code, near, other = oracle_lib.bf16_round(1 + 2 ** -8 - 2 ** -20, d)
    assert (code, near, other) == (0x3F80, True, 0x3F81)
    # 2^-16 away is beyond the band
    code, near, _ = oracle_lib.bf16_round(1 + 2 ** -8 + 2 ** -16, d)
    assert (code, near) == (0x3F81, False)
    # exactly representable values are never near a midpoint
    assert oracle_lib.bf16_round(1.5, d)[1] is False


def test_bf16_decode_matches_torch(oracle_lib):
    codes = np.arange(0, 65536, 13, dtype=np.int64)
    t = torch.from_numpy(codes.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    ref = t.double().numpy()
    for c, r in zip(codes, ref):
        got = oracle_lib.bf16_decode(int(c))
        assert (math.isnan(got) and math.isnan(r)) or got == r, hex(c)


# ----------------------------------------------------------------- e4m3 ----

def test_e4m3_golden_decode_encode(oracle_lib):
    with open(os.path.join(GOLDEN, "e4m3_codes.yaml")) as f:
        g = yaml.safe_load(f)
    for code, val in g["decode"].items():
        got = oracle_lib.e4m3_decode(code)
        if isinstance(val, str) or (isinstance(val, float) and math.isnan(val)):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)
    for x, code in g["encode"]:
        assert oracle_lib.e4m3_encode(x) == code, (x, hex(code))


def test_e4m3_decode_matches_torch(oracle_lib):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy()
    for c in range(256):
        got = oracle_lib.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got)
        else:
            assert got == float(ref[c]), hex(c)


def test_e4m3_roundtrip_every_code(oracle_lib):
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert oracle_lib.e4m3_encode(oracle_lib.e4m3_decode(c)) == c


def test_e4m3_encode_matches_torch_when_clamped(oracle_lib):
    """torch's float -> float8_e4m3fn rounds to nearest even but turns
    overflow into NaN, so compare on values clamped to +-448 first."""
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(3000) * 100, rng.standard_normal(2000) * 0.01,
        rng.uniform(-600, 600, 2000), rng.standard_normal(500) * 1e-4,
    ]).astype(np.float32)
    # every midpoint between consecutive finite codes, and its neighbours
    vals = np.array([oracle_lib.e4m3_decode(c) for c in range(0x7F)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1000))]).astype(np.float32)
    clamped = np.clip(x, -448, 448).astype(np.float32)
    want = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle_lib.e4m3_encode(float(v)) for v in x], np.uint8)
    assert np.array_equal(got, want)


def test_fp8_store_is_fp32_division_then_e4m3(oracle_lib):
    """x / scale in IEEE fp32 (numpy float32 division), then e4m3."""
    rng = np.random.default_rng(5)
    xs = rng.standard_normal(3000).astype(np.float32) * 8
    bits = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    scales = rng.uniform(0.05, 0.5, 3000).astype(np.float32)
    xf = (bits.astype(np.uint32) << 16).view(np.float32)
    q = np.clip(xf / scales, -448, 448).astype(np.float32)
    want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle_lib.fp8_store(int(b), float(s)) for b, s in zip(bits, scales)], np.uint8)
    assert np.array_equal(got, want)
    # hand case: 1.0 / 0.05f = 20.0 exactly in fp32 -> 1.25 * 2^4 = 0x5A
    assert oracle_lib.fp8_store(0x3F80, 0.05) == 0x5A
