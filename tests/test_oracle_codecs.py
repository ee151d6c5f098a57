"""Pins of the oracle's number-format codecs (CPU only).

Decoders are checked over every bit pattern against numpy / torch conversions
(library routines); encoders against hand-derived tie and saturation cases
(tests/golden/codec_cases.txt, derived from the format definitions), against
library RNE conversions on random values, and by round trips.
"""
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden", "codec_cases.txt")


def test_f16_decode_all_patterns(orc):
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = orc.decode16(pats, "f16")
    ref = pats.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_decode_all_patterns(orc):
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = orc.decode16(pats, "bf16")
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_e4m3_decode_all_patterns(orc):
    pats = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(pats)
    ref = torch.from_numpy(pats).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2                                   # 0x7f and 0xff
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.nanmax(ours) == 448.0


def _random_f32(n, seed):
    rng = np.random.default_rng(seed)
    mant = rng.uniform(-1, 1, n)
    expo = rng.integers(-30, 20, n)
    return (mant * np.exp2(expo)).astype(np.float32)


def test_f16_encode_matches_numpy_rne(orc):
    x = _random_f32(400_000, 1)
    x = x[np.abs(x) < 65000]
    ours = orc.encode16(x, "f16")
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_encode_matches_torch_rne(orc):
    x = _random_f32(400_000, 2)
    ours = orc.encode16(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_encode_matches_torch_in_range(orc):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-448, 448, 200_000),
                        rng.uniform(-1, 1, 200_000) * np.exp2(rng.integers(-12, 0, 200_000))])
    x = x.astype(np.float32)
    ours = orc.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_round_trips(orc):
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for fmt in ("f16", "bf16"):
        dec = orc.decode16(pats, fmt)
        fin = np.isfinite(dec)
        assert np.array_equal(orc.encode16(dec[fin], fmt), pats[fin])
    p8 = np.array([b for b in range(256) if b not in (0x7f, 0xff)], np.uint8)
    assert np.array_equal(orc.e4m3_encode(orc.e4m3_decode(p8)), p8)


def _golden():
    rows = []
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line:
            continue
        fmt, val, code = line.split()[:3]
        rows.append((fmt, float.fromhex(val), int(code, 16)))
    return rows


@pytest.mark.parametrize("fmt,val,code", _golden())
def test_golden_encode_cases(orc, fmt, val, code):
    x = np.array([val], np.float32)
    assert float(x[0]) == val                      # the case is exact in FP32
    if fmt == "e4m3":
        got = int(orc.e4m3_encode(x)[0])
    else:
        got = int(orc.encode16(x, fmt)[0])
    assert got == code, f"{fmt} {val!r}: {got:#x} != {code:#x}"
