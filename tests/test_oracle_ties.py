"""Pins of the oracle's rounding-tie bound (CPU only).

The P operand p^ is a code picked by rounding p (times 448 for E4M3) in FP32,
so two correct FP32 evaluations of the recipe, with their products and the
exponential taken in another order or base, can pick neighbouring codes
where p sits at a rounding midpoint.  forward_rows(tie=True) bounds, per
output element, what such re-roundings can move it.  The checks:

* p evaluated independently here in another order (log2 units, the P scale
  folded into the exponent, one fused multiply-add, as a GPU kernel would)
  picks the oracle's code except at a few keys; recomputing the output with
  those codes moves it by no more than the bound, and a row with one such key
  moves by the bound itself (one code step times |v| over L);
* the same for the 16-bit P operand (fp16 and bf16 rounding of p);
* the bound is zero on rows with no near-midpoint p, and such rows are few;
* on the inputs where a GPU run differed from the oracle by one E4M3 step of
  a dominant key (p*448 = 200.000046 against the midpoint 200, between the
  codes 192 and 208), the bound covers the difference.
"""
import math

import numpy as np
import pytest

import synth

F32 = np.float32


def _inputs(orc, w, qb=64):
    prob = orc.problem_from_workload(w, "fp8", 0, qb)
    q, k, v, _ = synth.make_inputs(w, device="cpu")
    u = lambda t: t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)
    pre = orc.prepass(prob, u(q), u(k), u(v))
    return prob, pre


def _codes_oracle_order(orc, S, sq, ks_row, sm):
    """p^ codes (rows of S) in the order the recipe states: s = S*((sq*sk)*sm),
    p = e^(s - m).  S [rows, keys] int, sq [rows], ks_row [keys]."""
    comb = ((F32(1) * sq[:, None]).astype(F32) * ks_row[None, :]).astype(F32) * F32(sm)
    s = (S.astype(F32) * comb.astype(F32)).astype(F32)
    m = s.max(axis=1, keepdims=True)
    p = np.exp((s - m).astype(F32).astype(np.float64)).astype(F32)
    return orc.e4m3_encode((p * F32(448)).astype(F32)).reshape(S.shape), p


def _codes_kernel_order(orc, S, sq, ks_row, sm):
    """p^ codes with log2 units and the P scale in the exponent: c = (sq*sk)*
    (sm*log2 e), m2 = max fl(S*c), x = fma(S, c, log2 448 - m2), p^ = 2^x."""
    c = ((F32(1) * sq[:, None]).astype(F32) * ks_row[None, :]).astype(F32)
    c = (c * F32(sm * math.log2(math.e))).astype(F32)
    y = (S.astype(F32) * c).astype(F32)
    nm = (F32(math.log2(448.0)) - y.max(axis=1, keepdims=True)).astype(F32)
    x = (S.astype(np.float64) * c.astype(np.float64) + nm.astype(np.float64)).astype(F32)
    return orc.e4m3_encode(np.exp2(x.astype(np.float64)).astype(F32)).reshape(S.shape)


def test_bound_covers_other_evaluation_orders(orc):
    # one 128-key tile per row, so each row is a single softmax over its keys
    w = synth.Workload(name="ties", dtype="f16", layout="HND", B=1, Hq=8, Hkv=8, Nq=4096,
                       Nkv=128, d=128, smooth_k=True, seed=7, k_off_sigma=2.0,
                       qv_mean_sigma=1.0)
    prob, pre = _inputs(orc, w)
    out, _, tie = orc.forward_rows(prob, pre, bkv=128, tie=True)
    flips = single = 0
    rows_with_bound = 0
    for h in range(w.Hq):
        qc, qs = pre.qc[0][h], pre.qs[0][h]
        kc, ks, vc, vs = pre.kc[0][h], pre.ks[0][h], pre.vc[0][h], pre.vs[0][h]
        vdec = orc.e4m3_decode(vc).astype(np.float64).reshape(vc.shape)   # [nkv, d]
        ks_row = ks[np.arange(w.Nkv) // 64].astype(F32)
        sq = qs[np.arange(w.Nq) // 64].astype(F32)
        S = qc.astype(np.int64) @ kc.astype(np.int64).T                    # [nq, nkv]
        co, p = _codes_oracle_order(orc, S, sq, ks_row, prob.scale)
        ck = _codes_kernel_order(orc, S, sq, ks_row, prob.scale)
        rows_with_bound += int(tie[0][h].any(axis=1).sum())
        for i in np.nonzero((co != ck).any(axis=1))[0]:
            diff = np.nonzero(co[i] != ck[i])[0]
            b = tie[0][h, i]
            flips += diff.size
            L = float(p[i].astype(np.float64).sum())
            dp = (orc.e4m3_decode(ck[i, diff]).astype(np.float64)
                  - orc.e4m3_decode(co[i, diff]))
            # the output recomputed with the other codes moves by
            delta = (dp @ vdec[diff]) * vs.astype(np.float64) / 448.0 / L
            assert np.all(np.abs(delta) <= b * (1 + 1e-4) + 1e-7), (h, i, diff)
            if diff.size == 1:
                single += 1
                np.testing.assert_allclose(np.abs(delta), b, rtol=1e-4, atol=1e-7)
    assert flips > 0 and single > 0          # the check saw re-rounded codes
    assert rows_with_bound < 0.1 * w.Hq * w.Nq


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bound_covers_other_orders_16bit_p(orc, dtype):
    # the 16-bit P.V variant: p itself is rounded to the input's 16-bit type
    # (numpy's float16 / torch's bfloat16 conversion here), with no P scale
    import torch
    w = synth.Workload(name="ties16", dtype=dtype, layout="HND", B=1, Hq=4, Hkv=4, Nq=2048,
                       Nkv=128, d=64, smooth_k=True, seed=11, k_off_sigma=2.0,
                       qv_mean_sigma=1.0)
    prob = orc.problem_from_workload(w, "half", 0, 64)
    q, k, v, _ = synth.make_inputs(w, device="cpu")
    u = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    pre = orc.prepass(prob, u(q), u(k), u(v))
    _, _, tie = orc.forward_rows(prob, pre, bkv=128, tie=True)

    def r16(x):
        if dtype == "f16":
            return x.astype(np.float16).astype(np.float64)
        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()

    flips = 0
    for h in range(w.Hq):
        qc, qs, kc, ks = pre.qc[0][h], pre.qs[0][h], pre.kc[0][h], pre.ks[0][h]
        vdec = orc.decode16(pre.vc[0][h], dtype).astype(np.float64)
        ks_row = ks[np.arange(w.Nkv) // 64].astype(F32)
        sq = qs[np.arange(w.Nq) // 64].astype(F32)
        S = qc.astype(np.int64) @ kc.astype(np.int64).T
        # the recipe's order
        comb = (sq[:, None] * ks_row[None, :]).astype(F32) * F32(prob.scale)
        s = (S.astype(F32) * comb.astype(F32)).astype(F32)
        p = np.exp((s - s.max(axis=1, keepdims=True)).astype(F32).astype(np.float64)).astype(F32)
        # log2 units and one fused multiply-add
        c = ((sq[:, None] * ks_row[None, :]).astype(F32)
             * F32(prob.scale * math.log2(math.e))).astype(F32)
        y = (S.astype(F32) * c).astype(F32)
        nm = (-y.max(axis=1, keepdims=True)).astype(F32)
        x = (S.astype(np.float64) * c.astype(np.float64) + nm.astype(np.float64)).astype(F32)
        pk = np.exp2(x.astype(np.float64)).astype(F32)
        a, b = r16(p), r16(pk)
        for i in np.nonzero((a != b).any(axis=1))[0]:
            diff = np.nonzero(a[i] != b[i])[0]
            flips += diff.size
            L = float(p[i].astype(np.float64).sum())
            delta = ((b[i, diff] - a[i, diff]) @ vdec[diff]) / L
            assert np.all(np.abs(delta) <= tie[0][h, i] * (1 + 1e-4) + 1e-9), (h, i, diff)
    assert flips > 0


def test_bound_zero_without_midpoints(orc):
    # all scores equal: p = 1 for every key, p*448 = 448 is the top code
    w = synth.Workload(name="flat", dtype="f16", layout="HND", B=1, Hq=1, Hkv=1, Nq=64,
                       Nkv=100, d=64, smooth_k=False, seed=3)
    prob, pre = _inputs(orc, w)
    pre.qc[0][:] = 0
    _, _, tie = orc.forward_rows(prob, pre, bkv=128, tie=True)
    assert not tie[0].any()


def test_bound_covers_observed_gpu_difference(orc):
    # two varlen sequences (43 x 247 and 98 x 72 tokens), d = 128, fp16 NHD,
    # K smoothing, Q/K blocks of 32 tokens, 128-key splits
    w = synth.Workload(name="tie201", dtype="f16", layout="NHD", B=2, Hq=2, Hkv=2, Nq=0,
                       Nkv=0, d=128, smooth_k=True, seed=251, k_off_sigma=2.0,
                       qv_mean_sigma=1.0, seqlens_q=[43, 98], seqlens_kv=[247, 72])
    prob = orc.problem_from_workload(w, "fp8", 128, 32)
    q, k, v, _ = synth.make_inputs(w, device="cpu")
    u = lambda t: t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)
    pre = orc.prepass(prob, u(q), u(k), u(v))
    out, _, tie = orc.forward_rows(prob, pre, bkv=128, tie=True)
    # the row of sequence 1, head 0, query 39: key 19 sits at a midpoint
    S = pre.qc[1][0][39:40].astype(np.int64) @ pre.kc[1][0].astype(np.int64).T
    ks_row = pre.ks[1][0][np.arange(72) // 32].astype(F32)
    co, p = _codes_oracle_order(orc, S, pre.qs[1][0][39 // 32:39 // 32 + 1].astype(F32),
                                ks_row, prob.scale)
    co, p = co[0], p[0]
    assert orc.e4m3_decode(co[19]) == 208.0
    x = float((p[19] * F32(448)).astype(F32))
    assert abs(x - 200.0) < 1e-4
    # the other code (192) moves channel 30 by 0.0216; the GPU output there
    # was -1.7197266 against the oracle's -1.7413206
    vdec = orc.e4m3_decode(pre.vc[1][0][19]).astype(np.float64)
    L = float(p.astype(np.float64).sum())
    delta = -16.0 * vdec * pre.vs[1][0].astype(np.float64) / 448.0 / L
    assert abs(out[1][0, 39, 30] - -1.7413206) < 1e-6
    assert abs(delta[30]) > 0.02
    assert np.all(np.abs(delta) <= tie[1][0, 39] * (1 + 1e-4))
    assert abs((-1.7197266) - out[1][0, 39, 30]) <= tie[1][0, 39, 30] + 2e-2
