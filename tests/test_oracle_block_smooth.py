"""Pins of the oracle's per-block Q smoothing (sage_oracle.c: orc_block_mean,
orc_smooth_blocks, orc_mu_code, orc_delta_s_block) against closed forms,
exact rational arithmetic, FP64 products and the method's purpose.

SageAttention2 summary, "Main concepts" item 2: Q is smoothed by subtracting
its channel mean before quantization.  The per-block reading takes one mean
per quantization block; the scores then owe mu_b.k_j, split into the
sequence mean's share (exact, from K_s) and the block's deviation, formed
from its 15-bit code and the INT8 key codes."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import oracle as orc
from tests import parity_util as pu
from tests.test_oracle_pins_fp8 import _f32_exact


def _int_rows(n, d, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(-40, 41, size=(n, d)).astype(np.float32)


@pytest.mark.parametrize("n,blk", [(64, 64), (150, 64), (150, 32), (33, 32), (1, 64)])
def test_block_mean_of_integer_rows_is_the_rounded_rational(n, blk):
    # integer rows: every partial sum is exact in FP32, so the mean is the
    # exact rational sum / n_b rounded once to FP32
    d = 16
    x = _int_rows(n, d, seed=n + blk)
    mu = orc.block_mean(x, blk)
    assert mu.shape == (-(-n // blk), d)
    for b in range(mu.shape[0]):
        rows = x[b * blk:min(n, (b + 1) * blk)]
        for c in range(d):
            want = _f32_exact(Fraction(int(rows[:, c].sum()), len(rows)))
            assert Fraction(float(mu[b, c])) == want, (b, c)


def test_block_means_are_independent_and_ragged_tail_uses_its_own_rows():
    x = _int_rows(150, 8, seed=3)
    mu = orc.block_mean(x, 64)
    y = x.copy()
    y[64:128] += 1000.0                     # only block 1 changes
    mv = orc.block_mean(y, 64)
    assert np.array_equal(mu[0], mv[0]) and np.array_equal(mu[2], mv[2])
    assert np.array_equal(mv[1], mu[1] + 1000.0)
    # the 22-token tail block: its mean is over 22 rows, not 64
    assert np.allclose(mu[2], x[128:].mean(0), rtol=0, atol=1e-5)


def test_smoothed_blocks_have_zero_column_sums():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((200, 32)) * 3 + 7).astype(np.float32)
    for blk in (64, 32):
        mu = orc.block_mean(x, blk)
        xs = orc.smooth_blocks(x, mu, blk)
        u = 2.0 ** -24
        for b in range(mu.shape[0]):
            rows = xs[b * blk:(b + 1) * blk].astype(np.float64)
            raw = np.abs(x[b * blk:(b + 1) * blk].astype(np.float64))
            n = len(rows)
            # the FP32 running sum errs by at most (n-1) u sum|x| (that error
            # reaches the column sum n times over through the mean), and each
            # subtraction by half an ulp
            bound = (n + 2) * u * raw.sum(0) + n * u * raw.max(0)
            assert np.all(np.abs(rows.sum(0)) <= bound)
        assert np.array_equal(xs[0], x[0] - mu[0])


@pytest.mark.parametrize("seed", range(20))
def test_mu_code_reconstructs_within_half_a_unit(seed):
    rng = np.random.default_rng(seed)
    d = 128
    x = (rng.standard_normal(d) * 10.0 ** rng.uniform(-3, 2)).astype(np.float32)
    hi, lo, sc = orc.mu_code(x)
    a = float(np.abs(x).max())
    assert Fraction(float(sc)) == _f32_exact(Fraction(a) / 16256)
    assert np.abs(hi.astype(int)).max() <= 127 and np.abs(lo.astype(int)).max() <= 64
    rec = float(sc) * (128 * hi.astype(np.float64) + lo)
    # within half a code unit, plus the FP32 rounding of the scaled value
    assert np.all(np.abs(rec - x) <= float(sc) * (0.5 + 16256 * 2.0 ** -22))


def test_mu_code_special_cases():
    hi, lo, sc = orc.mu_code(np.zeros(8, np.float32))
    assert sc == 0 and not hi.any() and not lo.any()
    x = np.array([2.0, -2.0, 1.0, 0.5, -0.25, 0.0, 0.015625, 1.5], np.float32)
    hi, lo, sc = orc.mu_code(x)
    # a = 2: y = 8128 * x (exact for these values)
    assert sc == np.float32(2.0 / 16256)
    assert hi.tolist() == [127, -127, 64, 32, -16, 0, 1, 95]
    # 8128 / 128 = 63.5 rounds to the even 64, leaving lo = -64; 4064 / 128 =
    # 31.75 -> 32, lo = -32; 127 / 128 -> 1, lo = -1; 12192 / 128 = 95.25 -> 95
    assert lo.tolist() == [0, 0, -64, -32, 16, 0, -1, 32]
    # the two parts rebuild the scaled values exactly
    assert (128 * hi.astype(int) + lo).tolist() == [16256, -16256, 8128, 4064, -2032, 0, 127, 12192]


def _keys(nkv, d, seed):
    rng = np.random.default_rng(seed)
    ks = (rng.standard_normal((nkv, d)) * 2).astype(np.float32)
    kc, kscale = orc.quant_int8_blocks(ks, 64)
    return ks, kc, kscale


@pytest.mark.parametrize("seed", range(6))
def test_delta_s_block_matches_fp64_within_the_code_bound(seed):
    rng = np.random.default_rng(100 + seed)
    d, nkv = 64, 200
    ks, kc, kscale = _keys(nkv, d, seed)
    mu_bar = (rng.standard_normal(d) * 3).astype(np.float32)
    dev = (rng.standard_normal(d) * 0.7).astype(np.float32)
    ds_seq = orc.delta_s(mu_bar, ks)
    hi, lo, sc = orc.mu_code(dev)
    ds = orc.delta_s_block(ds_seq, hi, lo, sc, kc, kscale, 64)
    kdq = kc.astype(np.float64) * np.repeat(kscale, 64)[:nkv, None]       # k^ * sk
    exact = ds_seq.astype(np.float64) + kdq @ dev.astype(np.float64)
    bound = (float(sc) * (0.5 + 16256 * 2.0 ** -22) * np.abs(kdq).sum(1)
             + 2.0 ** -22 * (np.abs(ds_seq) + np.abs(kdq @ dev)) + 1e-30)
    assert np.all(np.abs(ds - exact) <= bound)
    # without the sequence part only the deviation's product is left
    corr = orc.delta_s_block(None, hi, lo, sc, kc, kscale, 64)
    assert np.all(np.abs(corr - kdq @ dev.astype(np.float64)) <= bound)


def _score_rms(w, mode):
    """RMS over rows of the recipe's score error against FP64 q.k_s, with
    each row's mean error removed (the softmax does not see it)."""
    q, k, v, _ = synth.make_inputs(w)
    prob = orc.problem_from_workload(synth.scaled_down(w, smooth_q=mode))
    pre = orc.prepass(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    qh = orc.split_heads(prob, pu.u16(q), "q")
    kh = orc.split_heads(prob, pu.u16(k), "k")
    n = w.Nq
    errs = []
    for h in range(w.Hq):
        qf = orc.decode16(qh[0][h], prob.dtype).astype(np.float64)
        kf = orc.decode16(kh[0][h], prob.dtype).astype(np.float64)
        exact = qf @ (kf - pre.mu_k[0][h]).T
        S = orc.qk_int32(pre.qc[0][h], pre.kc[0][h]).astype(np.float64)
        rec = (S * np.repeat(pre.qs[0][h], 64)[:n, None]
               * np.repeat(pre.ks[0][h], 64)[None, :n])
        if mode == "block":
            rec += np.repeat(pre.ds[0][h], 64, axis=0)[:n]
        elif mode:
            rec += pre.ds[0][h][None, :]
        e = rec - exact
        e -= e.mean(1, keepdims=True)
        errs.append(np.sqrt((e ** 2).mean()))
    return float(np.mean(errs))


def test_block_smoothing_lowers_the_score_error_of_a_drifting_q():
    # a Q offset that drifts along the sequence: one mean per block removes
    # what one mean per sequence leaves (the purpose of the finer smoothing);
    # a dropped or mis-signed compensation term would raise the error far
    # above both
    w = synth.scaled_down(synth.WORKLOADS["video_dit_block"], Hq=2, Hkv=2, Nq=640, Nkv=640,
                          qv_outlier_mult=1.0)
    blk, seq, none = _score_rms(w, "block"), _score_rms(w, True), _score_rms(w, False)
    assert blk < 0.9 * seq < 0.9 * none, (blk, seq, none)


def test_block_recipe_tracks_exact_attention():
    w = synth.scaled_down(synth.WORKLOADS["video_dit_block"], Hq=2, Hkv=2, Nq=300, Nkv=270)
    q, k, v, _ = synth.make_inputs(w)
    prob = orc.problem_from_workload(w)
    pre = orc.prepass(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    out, lse = orc.forward_rows(prob, pre)
    ex, exl = orc.exact_rows(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    assert pu.cos(out[0], ex[0]) >= 0.999
    # K smoothing leaves out the row constant scale * q_i.mu_k of every score,
    # so the recipe's LSE is the exact one less that constant
    qh = orc.split_heads(prob, pu.u16(q), "q")
    for h in range(w.Hq):
        qf = orc.decode16(qh[0][h], prob.dtype).astype(np.float64)
        shift = prob.scale * (qf @ pre.mu_k[0][h].astype(np.float64))
        # (the logits reach 20 here; a dropped or mis-signed compensation moves
        # the LSE by whole units)
        assert np.abs(lse[0][h] - (exl[0][h] - shift)).max() < 0.25


def test_constant_query_blocks_leave_only_the_compensation():
    # every query of a block equal: the smoothed block is zero (zero codes and
    # scale) and the scores are the compensation alone
    w = synth.scaled_down(synth.WORKLOADS["video_dit_block"], Hq=1, Hkv=1, Nq=128, Nkv=192,
                          qv_outlier_mult=1.0)
    q, k, v, _ = synth.make_inputs(w)
    q = q.clone()
    q[0, :64] = q[0, 5]
    q[0, 64:] = q[0, 70]
    prob = orc.problem_from_workload(w)
    pre = orc.prepass(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    assert not pre.qc[0].any() and not pre.qs[0].any()
    out, _ = orc.forward_rows(prob, pre)
    ex, _ = orc.exact_rows(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    assert pu.cos(out[0], ex[0]) >= 0.999
