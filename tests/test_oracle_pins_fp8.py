"""Pins of two oracle steps against definitions outside the oracle (CPU only).

* The E4M3 P operand of the SageAttention2 recipe (ComfyUI blog on
  SageAttention, feature item 2: P.V in FP8).  With a single key tile the
  online softmax is the plain one, so the recipe's output is the textbook
      o = sum_j e4m3(448 p_j) dec(v^_j) * v_scale / 448 / sum_j p_j  (+ mu_v),
  p_j = e^(s_j - max s).  Here the E4M3 rounding is torch's float8_e4m3fn
  conversion and the V codes are decoded by torch as well; the scores are
  formed in FP32 as the recipe states.  An oracle that skipped the rounding,
  rounded to another format, used another P scale or summed l from the
  rounded p misses the bar.
* The reciprocal order of the INT8 quantizer (the pages fix no FP32 order;
  the reading taken is inv = fl32(127 / a) with one correctly rounded
  division, code = rne(fl32(x * inv))).  The cases below were found by a
  search over random blocks for elements where that order and the other
  natural one, fl32(1 / fl32(a / 127)), give different codes.  The expected
  codes are computed here with exact rational arithmetic (Python fractions):
  each step of the reading is rounded to binary32 exactly, and on the first
  cases the exact quotient x * 127 / a rounds to the same code.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

F32 = np.float32


def _enc(x, dtype):
    x = np.asarray(x, np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _dec(x, dtype):
    x = np.ascontiguousarray(x, np.uint16)
    if dtype == "f16":
        return x.view(np.float16).astype(np.float64)
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()


def _e4m3_torch(x):
    """FP32 values -> their E4M3 (e4m3fn) rounding by torch, as FP64."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.float8_e4m3fn).double().numpy()


def _e4m3_codes_torch(codes):
    """E4M3 bytes -> values, decoded by torch."""
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return t.view(torch.float8_e4m3fn).double().numpy()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("smooth_q", [False, True])
@pytest.mark.parametrize("smooth_v", [False, True])
def test_fp8_one_tile_is_textbook_softmax(orc, dtype, smooth_q, smooth_v):
    rng = np.random.default_rng(31 + 2 * smooth_q + smooth_v + (dtype == "bf16") * 4)
    d, nq, nkv = 64, 9, 100                     # one 128-key tile
    q = _enc(rng.normal(0, 1, (1, 1, nq, d)) + (1.0 if smooth_q else 0.0), dtype)
    k = _enc(rng.normal(0, 1, (1, 1, nkv, d)) * 1.5, dtype)
    v = _enc(rng.normal(0, 1, (1, 1, nkv, d)) + rng.normal(0, 2, (1, 1, 1, d)), dtype)
    prob = orc.Problem(dtype, "HND", 1, 1, d, [(nq, nkv)], smooth_q=smooth_q,
                       smooth_v=smooth_v)
    pre = orc.prepass(prob, q, k, v)
    out, lse = orc.forward_rows(prob, pre, bkv=128)
    # the integer scores by brute force in int64 (not the oracle's routine)
    S = pre.qc[0][0].astype(np.int64) @ pre.kc[0][0].astype(np.int64).T
    sq = np.repeat(pre.qs[0][0], 64)[:nq]
    sk = np.repeat(pre.ks[0][0], 64)[:nkv]
    vdec = _e4m3_codes_torch(pre.vc[0][0])               # [nkv, d]
    vs = pre.vs[0][0].astype(np.float64)
    moved = 0
    for i in range(nq):
        comb = (F32(sq[i]) * sk.astype(F32)).astype(F32) * F32(prob.scale)
        s = (S[i].astype(F32) * comb).astype(F32)
        if smooth_q:
            s = (s + (pre.ds[0][0] * F32(prob.scale)).astype(F32)).astype(F32)
        p = np.exp((s - s.max()).astype(F32).astype(np.float64)).astype(F32)
        p8 = _e4m3_torch((p * F32(448)).astype(F32))     # P^ = e4m3(448 p)
        L = p.astype(np.float64).sum()                   # l from the FP32 p
        want = (p8 @ vdec) * vs / 448.0 / L
        if smooth_v:
            want = want + pre.mu_v[0][0].astype(np.float64)
        # FP32 accumulation of <= 100 exact products: a few ulps of the
        # products' magnitude
        mag = (np.abs(p8) @ np.abs(vdec)) * vs / 448.0 / L
        tol = 1e-6 * np.maximum(mag, 1.0)
        assert np.all(np.abs(out[0][0][i] - want) <= tol), (i, np.abs(out[0][0][i] - want).max())
        # the rounding of P^ matters: the unrounded p lands elsewhere
        plain = (p.astype(np.float64) * 448.0 @ vdec) * vs / 448.0 / L
        moved = max(moved, float(np.abs(plain - (want - (pre.mu_v[0][0] if smooth_v else 0))).max()))
        # the log-sum-exp of the scores as the recipe forms them
        assert abs(lse[0][0][i] - (float(s.max()) + math.log(L))) < 1e-5
    assert moved > 1e-3


def test_fp8_one_tile_p_scale_is_448(orc):
    # scores spread so that p covers E4M3's whole range: a P scale that is not
    # 448 times a power of two changes which codes the p round to (a power of
    # two only moves the exponent, so it rounds alike outside the subnormals)
    d, nkv = 64, 128
    rng = np.random.default_rng(41)
    q = _enc(np.ones((1, 1, 1, d)), "f16")
    k = _enc(rng.normal(0, 3, (1, 1, nkv, d)), "f16")
    v = _enc(rng.normal(0, 1, (1, 1, nkv, d)), "f16")
    prob = orc.Problem("f16", "HND", 1, 1, d, [(1, nkv)], smooth_k=False)
    pre = orc.prepass(prob, q, k, v)
    out, _ = orc.forward_rows(prob, pre, bkv=128)
    S = pre.qc[0][0].astype(np.int64) @ pre.kc[0][0].astype(np.int64).T
    comb = (F32(pre.qs[0][0][0]) * np.repeat(pre.ks[0][0], 64).astype(F32)).astype(F32) \
        * F32(prob.scale)
    s = (S[0].astype(F32) * comb).astype(F32)
    p = np.exp((s - s.max()).astype(F32).astype(np.float64)).astype(F32)
    vdec = _e4m3_codes_torch(pre.vc[0][0])
    vs = pre.vs[0][0].astype(np.float64)
    L = p.astype(np.float64).sum()
    got = out[0][0][0]
    res = {}
    for scale in (448.0, 256.0, 240.0, 384.0):
        p8 = _e4m3_torch((p * F32(scale)).astype(F32))
        res[scale] = float(np.abs(got - (p8 @ vdec) * vs / scale / L).max())
    assert res[448.0] < 1e-6
    assert min(res[256.0], res[240.0], res[384.0]) > 1e-4


# ------------------------------------------------------------- R-4 cases ---

def _f32_exact(fr: Fraction) -> Fraction:
    """Round a rational to the nearest binary32 value (ties to even), exactly."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                              # subnormals share the last binade's step
    step = Fraction(2) ** (e - 23)
    m = a / step                                  # in [2^23, 2^24) for normals
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * step


def _rne(fr: Fraction) -> int:
    lo = fr.numerator // fr.denominator
    rem = fr - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        return lo + 1
    return lo


def _h(x: str) -> float:
    return float(np.frombuffer(bytes.fromhex(x)[::-1], np.float32)[0])


# (block absmax a, element x) as binary32 bit patterns.  For the first four
# the exact quotient x * 127 / a rounds to the same code as the reading; the
# last two show the reading is its FP32 steps, not the exact quotient.
R4_CASES = [
    ("402698a1", "bc27e873"),   # a ~ 2.60307, x ~ -0.0102483
    ("40a5a336", "beeffa92"),   # a ~ 5.17617, x ~ -0.468709
    ("40a31eec", "403288a5"),   # a ~ 5.09752, x ~ 2.78959
    ("40238b11", "4007db55"),   # a ~ 2.55536, x ~ 2.12276
    ("40646a64", "404c229b"),   # a ~ 3.56899, x ~ 3.18961
    ("40b3fd26", "4039a865"),   # a ~ 5.62465, x ~ 2.90090
]


def test_r4_cases_are_what_the_search_found():
    # the stored bit patterns are the decimal values the search printed
    vals = [(_h(a), _h(x)) for a, x in R4_CASES]
    want = [(2.6030657291412354, -0.010248291306197643), (5.176173210144043, -0.4687085747718811),
            (5.097524642944336, 2.7895901203155518), (2.5553629398345947, 2.1227619647979736),
            (3.56899356842041, 3.1896121501922607), (5.624651908874512, 2.9009029865264893)]
    assert vals == want


@pytest.mark.parametrize("case", range(len(R4_CASES)))
def test_int8_reciprocal_order(orc, case):
    a, x = (_h(h) for h in R4_CASES[case])
    A, X = Fraction(a), Fraction(x)
    inv = _f32_exact(Fraction(127) / A)           # fl32(127 / a)
    want = max(-127, min(127, _rne(_f32_exact(X * inv))))
    other = max(-127, min(127, _rne(_f32_exact(X * _f32_exact(1 / _f32_exact(A / 127))))))
    assert want != other                          # the case separates the two orders
    if case < 4:
        assert want == _rne(X * 127 / A)          # ... and the exact quotient agrees
    # a one-token block holding the absmax and the element
    blk = np.array([[a, x, -a / 3, 0.0]], np.float32)
    codes, scales = orc.quant_int8_blocks(blk, 64)
    assert int(codes[0, 1]) == want
    assert int(codes[0, 0]) == 127
    assert Fraction(float(scales[0])) == _f32_exact(A / 127)
