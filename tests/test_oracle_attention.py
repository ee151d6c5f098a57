"""Pins of the oracle's attention functions (CPU only).

* exact FP64 attention == torch's scaled_dot_product_attention in FP64 with an
  explicit bottom-right causal mask (library routine), and its invariances
  under a per-channel shift of K and of V;
* int32 Q.K^T == brute force;
* the same-recipe forward on textbook special cases (one key, uniform weights,
  a dominant key, rows with no visible key), against exact FP64 attention on
  tiny inputs of every head dim, its LSE, and its independence of the tile
  width up to FP8 rounding;
* the 16-bit P.V variant (pv_mode "half"): one key gives v exactly, uniform
  weights give the plain mean of V, one tile equals the textbook softmax with
  p rounded by numpy's float16 / torch's bfloat16 conversion (library
  routines), its V operand is the input (or v - mu_v rounded by numpy), and it
  is closer to exact attention than the FP8 recipe;
* the key range cut into splits and merged (flash-decoding): equal scores
  give the plain mean of V, the LSE does not depend on the split (l is summed
  from the FP32 p), the output moves only by the P rounding, and the merge
  weights follow the splits' maxima (an unweighted merge misses exact
  attention).
"""
import math

import numpy as np
import pytest
import torch


def _cos(a, b):
    a, b = np.ravel(a).astype(np.float64), np.ravel(b).astype(np.float64)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def _sdpa64(q, k, v, scale, causal):
    nq, nkv = q.shape[0], k.shape[0]
    mask = None
    if causal:
        i = torch.arange(nq)[:, None]
        j = torch.arange(nkv)[None, :]
        mask = j <= i + nkv - nq
    t = lambda a: torch.from_numpy(a.astype(np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=mask, scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("nq,nkv,d,causal", [(17, 17, 64, False), (33, 70, 96, True),
                                             (64, 50, 128, False), (8, 40, 64, True)])
def test_exact_matches_torch_sdpa(orc, nq, nkv, d, causal):
    rng = np.random.default_rng(nq + nkv)
    q = rng.normal(0, 1, (nq, d)).astype(np.float32)
    k = rng.normal(0, 1, (nkv, d)).astype(np.float32)
    v = rng.normal(0, 1, (nkv, d)).astype(np.float32)
    sc = 1 / math.sqrt(d)
    out, lse = orc.attn_exact_rows(q, k, v, sc, causal, np.arange(nq))
    ref = _sdpa64(q, k, v, sc, causal)
    assert np.max(np.abs(out - ref)) < 1e-12
    # LSE: log sum_j exp(t_ij)
    t = (q.astype(np.float64) @ k.T.astype(np.float64)) * sc
    if causal:
        t = np.where(np.arange(nkv)[None, :] <= np.arange(nq)[:, None] + nkv - nq, t, -np.inf)
    ref_lse = np.log(np.exp(t - t.max(1, keepdims=True)).sum(1)) + t.max(1)
    assert np.max(np.abs(lse - ref_lse)) < 1e-10


def test_exact_shift_invariance(orc):
    rng = np.random.default_rng(5)
    nq, nkv, d = 20, 45, 64
    # fp16-representable inputs and a dyadic shift: K - mu and V - mu are exact
    q = rng.normal(0, 1, (nq, d)).astype(np.float16).astype(np.float32)
    k = rng.normal(0, 1, (nkv, d)).astype(np.float16).astype(np.float32)
    v = rng.normal(0, 1, (nkv, d)).astype(np.float16).astype(np.float32)
    mu = (rng.integers(-16, 16, d) / 4.0).astype(np.float32)
    rows = np.arange(nq)
    for causal in (False, True):
        base, _ = orc.attn_exact_rows(q, k, v, 0.125, causal, rows)
        ks, _ = orc.attn_exact_rows(q, k - mu, v, 0.125, causal, rows)
        vs, _ = orc.attn_exact_rows(q, k, v - mu, 0.125, causal, rows)
        assert np.max(np.abs(ks - base)) <= 1e-12 * np.abs(base).max()
        assert np.max(np.abs(vs + mu - base)) <= 1e-12 * np.abs(base).max() + 1e-13


def test_qk_int32_brute_force(orc):
    rng = np.random.default_rng(6)
    qc = rng.integers(-127, 128, (7, 96)).astype(np.int8)
    kc = rng.integers(-127, 128, (9, 96)).astype(np.int8)
    s = orc.qk_int32(qc, kc)
    for i in range(7):
        for j in range(9):
            assert s[i, j] == sum(int(qc[i, c]) * int(kc[j, c]) for c in range(96))
    # extreme codes: d * 127^2 fits in int32 and in FP32 exactly
    big = np.full((2, 128), 127, np.int8)
    assert orc.qk_int32(big, -big)[0, 0] == -128 * 127 * 127


def _prob(orc, nq, nkv, d, **kw):
    return orc.Problem("f16", "HND", kw.pop("Hq", 1), kw.pop("Hkv", 1), d, [(nq, nkv)], **kw)


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def _run(orc, prob, q, k, v, bkv=128):
    pre = orc.prepass(prob, q, k, v)
    out, lse = orc.forward_rows(prob, pre, bkv=bkv)
    return pre, out[0], lse[0]


def test_one_key_returns_v(orc):
    rng = np.random.default_rng(7)
    d = 64
    q = _f16(rng.normal(0, 1, (1, 1, 5, d)))
    k = _f16(rng.normal(0, 1, (1, 1, 1, d)))
    v = _f16(rng.normal(0, 1, (1, 1, 1, d)))
    vf = orc.decode16(v, "f16")[0, 0, 0]
    # smooth_v: V - mean = 0 exactly, so O = mu_v = v exactly
    _, out, _ = _run(orc, _prob(orc, 5, 1, d, smooth_v=True), q, k, v)
    assert np.array_equal(out[0], np.broadcast_to(vf, (5, d)))
    # without smoothing O = dec(v^) * scale_v within the FP8 error of v
    _, out, _ = _run(orc, _prob(orc, 5, 1, d), q, k, v)
    assert np.all(np.abs(out[0] - vf) <= np.abs(vf) * 2 ** -4 + np.abs(vf).max() * 2 ** -9)


def test_uniform_weights(orc):
    rng = np.random.default_rng(8)
    d, n = 96, 150
    v = _f16(rng.normal(0, 1, (1, 1, n, d)))
    # constant keys: all scores equal after smoothing -> every p^ is 448 and
    # O is the plain mean of the visible (dequantized) v rows
    krow = rng.normal(0, 1, (1, 1, 1, d))
    k = _f16(np.broadcast_to(krow, (1, 1, n, d)))
    q = _f16(rng.normal(0, 1, (1, 1, n, d)))
    vf = orc.decode16(v, "f16")[0, 0].astype(np.float64)
    for causal in (False, True):
        pre, out, _ = _run(orc, _prob(orc, n, n, d, causal=causal), q, k, v)
        vq = orc.e4m3_decode(pre.vc[0][0]).astype(np.float64) * pre.vs[0][0]
        for i in (0, 1, 63, 64, 149):
            m = (i + 1) if causal else n
            assert np.max(np.abs(out[0][i] - vq[:m].mean(0))) < 1e-5
            assert np.max(np.abs(out[0][i] - vf[:m].mean(0))) < 2 ** -4 * np.abs(vf).max()
    # q = 0 -> uniform as well
    q0 = _f16(np.zeros((1, 1, 4, d)))
    pre, out, _ = _run(orc, _prob(orc, 4, n, d, smooth_k=False), q0, k, v)
    vq = orc.e4m3_decode(pre.vc[0][0]).astype(np.float64) * pre.vs[0][0]
    assert np.max(np.abs(out[0] - vq.mean(0))) < 1e-5


def test_dominant_key(orc):
    rng = np.random.default_rng(9)
    d, n = 64, 100
    q = rng.normal(0, 1, (1, 1, 3, d))
    k = rng.normal(0, 0.1, (1, 1, n, d))
    k[0, 0, 37] = q[0, 0, 0] * 3.0                     # row 0 attends to key 37
    v = rng.normal(0, 1, (1, 1, n, d))
    qh, kh, vh = _f16(q), _f16(k), _f16(v)
    _, out, _ = _run(orc, _prob(orc, 3, n, d, sm_scale=1.0), qh, kh, vh)
    v37 = orc.decode16(vh, "f16")[0, 0, 37]
    assert _cos(out[0][0], v37) > 0.999


def test_rows_without_visible_keys(orc):
    rng = np.random.default_rng(10)
    d, nq, nkv = 64, 50, 20                            # rows 0..29 see nothing
    q, k, v = (_f16(rng.normal(0, 1, (1, 1, n, d))) for n in (nq, nkv, nkv))
    _, out, lse = _run(orc, _prob(orc, nq, nkv, d, causal=True, smooth_v=True), q, k, v)
    assert not out[0][:30].any() and np.all(np.isneginf(lse[0][:30]))
    assert np.all(np.isfinite(lse[0][30:])) and np.abs(out[0][30:]).min(1).max() > 0


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("nq,nkv,causal", [(65, 65, False), (33, 64, True), (64, 17, False),
                                          (40, 65, True)])
def test_recipe_vs_exact_tiny(orc, d, nq, nkv, causal):
    rng = np.random.default_rng(d * 1000 + nq)
    q = rng.normal(0, 1, (1, 2, nq, d))
    k = rng.normal(0, 1, (1, 1, nkv, d)) + rng.normal(0, 3, (1, 1, 1, d))
    v = rng.normal(0, 1, (1, 1, nkv, d))
    qh, kh, vh = _f16(q), _f16(k), _f16(v)
    prob = _prob(orc, nq, nkv, d, causal=causal, Hq=2, Hkv=1)
    pre, out, lse = _run(orc, prob, qh, kh, vh)
    ex, ex_lse = orc.exact_rows(prob, qh, kh, vh)
    assert _cos(out, ex[0]) >= 0.99
    assert np.max(np.abs(out - ex[0])) < 0.1
    # LSE of the recipe is that of the smoothed scores: exact LSE - q.mu_k*scale
    qf = orc.decode16(qh, "f16")[0].astype(np.float64)
    shift = (qf @ pre.mu_k[0][0].astype(np.float64)) / math.sqrt(d)
    assert np.max(np.abs(lse - (ex_lse[0] - shift))) < 0.05


def test_q_and_v_smoothing_recipe(orc):
    rng = np.random.default_rng(11)
    d, n = 64, 130
    q = rng.normal(0, 1, (1, 1, n, d)) + rng.normal(0, 1.5, (1, 1, 1, d))
    k = rng.normal(0, 1, (1, 1, n, d))
    v = rng.normal(0, 1, (1, 1, n, d)) + rng.normal(0, 1.5, (1, 1, 1, d))
    qh, kh, vh = _f16(q), _f16(k), _f16(v)
    prob = _prob(orc, n, n, d, smooth_q=True, smooth_v=True)
    pre, out, _ = _run(orc, prob, qh, kh, vh)
    ex, _ = orc.exact_rows(prob, qh, kh, vh)
    assert pre.ds[0] is not None and pre.mu_v[0] is not None
    assert _cos(out, ex[0]) >= 0.999
    # dropping the compensation must visibly break the result
    pre.ds[0] = np.zeros_like(pre.ds[0])
    bad, _ = orc.forward_rows(prob, pre)
    assert _cos(bad[0], ex[0]) < _cos(out, ex[0]) - 1e-3


def test_tile_width_only_moves_fp8_rounding(orc):
    rng = np.random.default_rng(12)
    d, n = 128, 300
    q, k, v = (_f16(rng.normal(0, 1, (1, 1, n, d))) for _ in range(3))
    prob = _prob(orc, n, n, d, causal=True)
    pre = orc.prepass(prob, q, k, v)
    a, la = orc.forward_rows(prob, pre, bkv=16)
    b, lb = orc.forward_rows(prob, pre, bkv=n)
    assert np.max(np.abs(a[0] - b[0])) < 0.05 and _cos(a[0], b[0]) > 0.9995
    assert np.max(np.abs(la[0] - lb[0])) < 1e-4


def test_dequantized_score_bound(orc):
    rng = np.random.default_rng(13)
    d, n = 128, 200
    q = rng.normal(0, 1, (n, d)).astype(np.float32)
    k = (rng.normal(0, 1, (n, d)) + 2.0).astype(np.float32)
    mu = orc.channel_mean(k)
    ks = orc.smooth(k, mu)
    qc, qsc = orc.quant_int8_blocks(q)
    kc, ksc = orc.quant_int8_blocks(ks)
    S = orc.qk_int32(qc, kc).astype(np.float64)
    sq = np.repeat(qsc, 64)[:n].astype(np.float64)
    sk = np.repeat(ksc, 64)[:n].astype(np.float64)
    s = S * sq[:, None] * sk[None, :]
    t = q.astype(np.float64) @ ks.T.astype(np.float64)
    bound = (np.abs(q) @ np.ones((d, n))) * sk[None, :] / 2 \
        + (np.ones((n, d)) @ np.abs(ks).T) * sq[:, None] / 2 + d * sq[:, None] * sk[None, :] / 4
    assert np.all(np.abs(s - t) <= bound * (1 + 1e-6))


# ------------------------------------------------- 16-bit P.V variant ---

def _bf16(x):
    t = torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _enc(x, dtype):
    return _f16(x) if dtype == "f16" else _bf16(x)


def _round_p(p, dtype):
    """p rounded to the 16-bit type by the libraries' own conversions."""
    if dtype == "f16":
        return np.asarray(p, np.float32).astype(np.float16).astype(np.float64)
    return torch.from_numpy(np.asarray(p, np.float32)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_half_one_key_returns_v(orc, dtype):
    rng = np.random.default_rng(21)
    d = 96
    q = _enc(rng.normal(0, 1, (1, 1, 7, d)), dtype)
    k = _enc(rng.normal(0, 1, (1, 1, 1, d)), dtype)
    v = _enc(rng.normal(0, 1, (1, 1, 1, d)), dtype)
    vf = orc.decode16(v, dtype)[0, 0, 0]
    for smooth_v in (False, True):
        prob = orc.Problem(dtype, "HND", 1, 1, d, [(7, 1)], smooth_v=smooth_v, pv_mode="half")
        pre = orc.prepass(prob, q, k, v)
        out, _ = orc.forward_rows(prob, pre)
        # p = 1 is exact in 16 bits and l = 1: o = v with no rounding at all
        assert np.array_equal(out[0][0], np.broadcast_to(vf, (7, d)))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_half_uniform_weights(orc, dtype):
    rng = np.random.default_rng(22)
    d, n = 64, 200
    v = _enc(rng.normal(0, 1, (1, 1, n, d)), dtype)
    k = _enc(np.broadcast_to(rng.normal(0, 1, (1, 1, 1, d)), (1, 1, n, d)), dtype)
    q = _enc(rng.normal(0, 1, (1, 1, n, d)), dtype)
    vf = orc.decode16(v, dtype)[0, 0].astype(np.float64)
    for causal in (False, True):
        prob = orc.Problem(dtype, "HND", 1, 1, d, [(n, n)], causal=causal, pv_mode="half")
        out, _ = orc.forward_rows(prob, orc.prepass(prob, q, k, v))
        for i in (0, 1, 127, 128, 199):
            m = (i + 1) if causal else n
            # every p is exactly 1: o is the plain mean of the visible rows
            assert np.max(np.abs(out[0][0][i] - vf[:m].mean(0))) < 1e-5


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("smooth_q", [False, True])
def test_half_one_tile_is_textbook_softmax(orc, dtype, smooth_q):
    """With one key tile the online softmax is the plain one: o = sum_j
    r(p_j) v_j / sum_j p_j, p_j = e^(s_j - max s) (difference in FP32, as the
    recipe forms it), where r is the 16-bit
    rounding done here by numpy / torch.  Dropping the rounding, rounding to
    the other type or normalising by sum r(p) all miss the 1e-6 bar."""
    rng = np.random.default_rng(23 + smooth_q)
    d, nq, nkv = 64, 9, 100
    q = _enc(rng.normal(0, 1, (1, 1, nq, d)) + (1.0 if smooth_q else 0.0), dtype)
    k = _enc(rng.normal(0, 1, (1, 1, nkv, d)), dtype)
    v = _enc(rng.normal(0, 1, (1, 1, nkv, d)), dtype)
    prob = orc.Problem(dtype, "HND", 1, 1, d, [(nq, nkv)], smooth_q=smooth_q, pv_mode="half")
    pre = orc.prepass(prob, q, k, v)
    out, _ = orc.forward_rows(prob, pre, bkv=128)
    S = orc.qk_int32(pre.qc[0][0], pre.kc[0][0]).astype(np.float64)
    sq = np.repeat(pre.qs[0][0], 64)[:nq]
    sk = np.repeat(pre.ks[0][0], 64)[:nkv]
    vf = orc.decode16(v, dtype)[0, 0].astype(np.float64)
    for i in range(nq):
        comb = np.float32(np.float32(sq[i]) * sk) * np.float32(prob.scale)
        s = (np.float32(S[i]) * comb).astype(np.float32)
        if smooth_q:
            s = (s + (pre.ds[0][0] * np.float32(prob.scale)).astype(np.float32)).astype(np.float32)
        p = np.exp((s - s.max()).astype(np.float64)).astype(np.float32)   # s - m in FP32
        want = (_round_p(p, dtype) @ vf) / p.astype(np.float64).sum()
        assert np.max(np.abs(out[0][0][i] - want)) < 1e-6 * max(1.0, np.abs(want).max())


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_half_v_operand(orc, dtype):
    rng = np.random.default_rng(24)
    d, n = 128, 70
    q, k = (_enc(rng.normal(0, 1, (1, 1, n, d)), dtype) for _ in range(2))
    v = _enc(rng.normal(0, 1, (1, 1, n, d)) + rng.normal(0, 2, (1, 1, 1, d)), dtype)
    prob = orc.Problem(dtype, "HND", 1, 1, d, [(n, n)], pv_mode="half")
    pre = orc.prepass(prob, q, k, v)
    assert pre.vs[0] is None and np.array_equal(pre.vc[0][0], v[0, 0])
    prob = orc.Problem(dtype, "HND", 1, 1, d, [(n, n)], smooth_v=True, pv_mode="half")
    pre = orc.prepass(prob, q, k, v)
    vf = orc.decode16(v, dtype)[0, 0]
    vs = (vf - pre.mu_v[0][0]).astype(np.float32)       # FP32 difference
    assert np.array_equal(pre.vc[0][0], _enc(vs, dtype))


@pytest.mark.parametrize("d", [64, 128])
def test_half_closer_to_exact_than_fp8(orc, d):
    rng = np.random.default_rng(25 + d)
    nq, nkv = 70, 300
    q = _f16(rng.normal(0, 1, (1, 2, nq, d)))
    k = _f16(rng.normal(0, 1, (1, 1, nkv, d)) + rng.normal(0, 3, (1, 1, 1, d)))
    v = _f16(rng.normal(0, 1, (1, 1, nkv, d)))
    errs = {}
    for mode in ("fp8", "half"):
        prob = orc.Problem("f16", "HND", 2, 1, d, [(nq, nkv)], causal=True, pv_mode=mode)
        out, _ = orc.forward_rows(prob, orc.prepass(prob, q, k, v))
        ex, _ = orc.exact_rows(prob, q, k, v)
        errs[mode] = float(np.abs(out[0] - ex[0]).max())
        assert _cos(out[0], ex[0]) >= (0.9999 if mode == "half" else 0.999)
    assert errs["half"] < 0.5 * errs["fp8"]


# ------------------------------------------- split key range (merge) ---

@pytest.mark.parametrize("mode", ["fp8", "half"])
def test_split_uniform_weights(orc, mode):
    """Equal scores: every split's p is 1, every merge weight is 1, and o is
    the plain mean of the (dequantized) V rows."""
    rng = np.random.default_rng(31)
    d, n = 64, 700
    v = _f16(rng.normal(0, 1, (1, 1, n, d)))
    k = _f16(np.broadcast_to(rng.normal(0, 1, (1, 1, 1, d)), (1, 1, n, d)))
    q = _f16(rng.normal(0, 1, (1, 1, 3, d)))
    prob = orc.Problem("f16", "HND", 1, 1, d, [(3, n)], pv_mode=mode, kv_split=256)
    pre = orc.prepass(prob, q, k, v)
    out, _ = orc.forward_rows(prob, pre)
    if mode == "fp8":
        vq = orc.e4m3_decode(pre.vc[0][0]).astype(np.float64) * pre.vs[0][0]
    else:
        vq = orc.decode16(pre.vc[0][0], "f16").astype(np.float64)
    assert np.max(np.abs(out[0][0] - vq.mean(0))) < 1e-5


@pytest.mark.parametrize("mode", ["fp8", "half"])
@pytest.mark.parametrize("causal,nq,nkv", [(False, 5, 1000), (True, 40, 777), (True, 1, 513)])
def test_split_lse_is_split_invariant(orc, mode, causal, nq, nkv):
    """l is summed from the FP32 p, so the merged LSE is the same quantity for
    any split (up to FP32 rounding), while p^ (hence o) only moves by its own
    rounding."""
    rng = np.random.default_rng(32 + nq)
    d = 128
    q = _f16(rng.normal(0, 1, (1, 2, nq, d)))
    k = _f16(rng.normal(0, 1, (1, 1, nkv, d)) + rng.normal(0, 3, (1, 1, 1, d)))
    v = _f16(rng.normal(0, 1, (1, 1, nkv, d)))
    base = orc.Problem("f16", "HND", 2, 1, d, [(nq, nkv)], causal=causal, pv_mode=mode)
    pre = orc.prepass(base, q, k, v)
    o0, l0 = orc.forward_rows(base, pre)
    for split in (128, 256, 512):
        sp = orc.Problem("f16", "HND", 2, 1, d, [(nq, nkv)], causal=causal, pv_mode=mode,
                         kv_split=split)
        o1, l1 = orc.forward_rows(sp, pre)
        fin = np.isfinite(l0[0])
        assert np.array_equal(fin, np.isfinite(l1[0]))
        assert np.max(np.abs(l1[0][fin] - l0[0][fin])) < 1e-5 * max(1.0, np.abs(l0[0][fin]).max())
        bound = 0.05 if mode == "fp8" else 2e-3
        assert np.max(np.abs(o1[0] - o0[0])) < bound and _cos(o1[0], o0[0]) > 0.9995


def test_split_merge_weights_follow_the_maxima(orc):
    """Split 0 holds keys aligned with the query (large scores), split 1 small
    ones: the merge must weight the splits by e^(m_s - M).  Equal weights would
    put half the mass on split 1 and miss exact attention by far."""
    rng = np.random.default_rng(33)
    d, n = 64, 512
    q = rng.normal(0, 1, (1, 1, 2, d))
    k = rng.normal(0, 0.2, (1, 1, n, d))
    k[0, 0, :256] += 0.5 * q[0, 0, 0]              # split 0 scores high for row 0
    v = rng.normal(0, 1, (1, 1, n, d))
    v[0, 0, 256:] += 3.0                            # split 1's values stand apart
    qh, kh, vh = _f16(q), _f16(k), _f16(v)
    for mode in ("fp8", "half"):
        prob = orc.Problem("f16", "HND", 1, 1, d, [(2, n)], smooth_k=False, sm_scale=1.0,
                           pv_mode=mode, kv_split=256)
        out, lse = orc.forward_rows(prob, orc.prepass(prob, qh, kh, vh))
        ex, ex_lse = orc.exact_rows(prob, qh, kh, vh)
        assert _cos(out[0][0], ex[0][0]) > 0.999
        assert np.max(np.abs(out[0][0][0] - ex[0][0][0])) < 0.05
        assert abs(lse[0][0][0] - ex_lse[0][0][0]) < 1e-3 * max(1.0, abs(ex_lse[0][0][0]))


# -------------------------------------------- 32-token Q/K blocks ---

@pytest.mark.parametrize("mode", ["fp8", "half"])
def test_finer_qk_blocks_track_exact_attention_closer(orc, mode):
    """32-token Q/K blocks: scores stay within the dequantization bound of their
    own (finer) scales, so with a few loud tokens the recipe lands closer to
    exact FP64 attention than with 64-token blocks."""
    rng = np.random.default_rng(41)
    d, nq, nkv = 128, 96, 320
    q = rng.normal(0, 1, (1, 1, nq, d))
    k = rng.normal(0, 1, (1, 1, nkv, d))
    q[0, 0, 5::37] *= 10.0                           # loud query tokens
    k[0, 0, 3::41] *= 10.0                           # loud keys
    v = rng.normal(0, 1, (1, 1, nkv, d))
    qh, kh, vh = _f16(q), _f16(k), _f16(v)
    errs = {}
    for bs in (64, 32):
        prob = orc.Problem("f16", "HND", 1, 1, d, [(nq, nkv)], pv_mode=mode, qk_block=bs)
        pre = orc.prepass(prob, qh, kh, vh)
        assert pre.qs[0].shape == (1, -(-nq // bs)) and pre.ks[0].shape == (1, -(-nkv // bs))
        out, _ = orc.forward_rows(prob, pre)
        ex, _ = orc.exact_rows(prob, qh, kh, vh)
        errs[bs] = float(np.sqrt(np.mean((out[0] - ex[0]) ** 2)))
        assert _cos(out[0], ex[0]) > 0.98
    assert errs[32] < 0.9 * errs[64]


def test_finer_qk_blocks_score_bound(orc):
    """The dequantized-score bound with 32-token scales (one scale per 32
    query rows and per 32 keys)."""
    rng = np.random.default_rng(42)
    d, n = 64, 100
    q = rng.normal(0, 1, (n, d)).astype(np.float32)
    k = (rng.normal(0, 1, (n, d)) * np.repeat(rng.uniform(0.2, 5, (n, 1)), d, 1)).astype(np.float32)
    qc, qsc = orc.quant_int8_blocks(q, 32)
    kc, ksc = orc.quant_int8_blocks(k, 32)
    S = orc.qk_int32(qc, kc).astype(np.float64)
    sq = np.repeat(qsc, 32)[:n].astype(np.float64)
    sk = np.repeat(ksc, 32)[:n].astype(np.float64)
    s = S * sq[:, None] * sk[None, :]
    t = q.astype(np.float64) @ k.T.astype(np.float64)
    bound = (np.abs(q) @ np.ones((d, n))) * sk[None, :] / 2 \
        + (np.ones((n, d)) @ np.abs(k).T) * sq[:, None] / 2 + d * sq[:, None] * sk[None, :] / 4
    assert np.all(np.abs(s - t) <= bound * (1 + 1e-6))
