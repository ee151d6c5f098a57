"""Pins of the oracle's pre-pass: channel means, smoothing, INT8 per-block and
FP8 per-channel quantization, and the Q-smoothing score bias (CPU only)."""
import numpy as np
import pytest


def test_mean_closed_form_dyadic(orc):
    # x[t,c] = o_c + e_t * z with sum_t e_t = 0 and dyadic values: every partial
    # sum is exact in FP32, so the mean is exactly o_c.
    rng = np.random.default_rng(0)
    for n in (1, 2, 64, 65, 200, 1000):
        d = 32
        o = rng.integers(-64, 64, d) / 8.0
        e = np.where(np.arange(n) % 2 == 0, 1.0, -1.0)
        if n % 2:
            e[-1] = 0.0
        x = (o[None, :] + e[:, None] * 0.25).astype(np.float32)
        mu = orc.channel_mean(x)
        assert np.array_equal(mu, o.astype(np.float32)), n


def test_mean_sequential_order_within_and_across_chunks(orc):
    # chunk 0: 2^24 then 63 ones -> each +1 rounds back to 2^24 (ties to even)
    x = np.ones((128, 1), np.float32)
    x[0, 0] = 2.0 ** 24
    # chunk 1 sums to 64 exactly; 2^24 + 64 is exact, so the total is 2^24+64
    mu = orc.channel_mean(x)
    assert mu[0] == np.float32((2.0 ** 24 + 64) / 128)
    # a single chunk: the sequential FP32 order loses all 63 ones
    mu1 = orc.channel_mean(x[:64])
    assert mu1[0] == np.float32(2.0 ** 24 / 64)
    # chunk sums are added in chunk order: 64 ones, then 2^24 in the next chunk
    y = np.ones((65, 1), np.float32)
    y[64, 0] = 2.0 ** 24
    # chunk 0 = 64, chunk 1 = 2^24 -> 64 + 2^24 exact
    assert orc.channel_mean(y)[0] == np.float32((64 + 2.0 ** 24) / 65)


def test_mean_close_to_fp64(orc):
    rng = np.random.default_rng(1)
    x = rng.normal(3.0, 2.0, (4096, 64)).astype(np.float32)
    mu = orc.channel_mean(x)
    ref = x.astype(np.float64).mean(0)
    assert np.max(np.abs(mu - ref)) < 1e-4


@pytest.mark.parametrize("bs", [64, 32])
def test_int8_blocks_roundtrip_bound(orc, bs):
    rng = np.random.default_rng(2)
    for n in (1, 31, 32, 33, 63, 64, 65, 300):
        x = (rng.normal(0, 1, (n, 96)) * rng.uniform(0.1, 10)).astype(np.float32)
        codes, scales = orc.quant_int8_blocks(x, bs)
        assert codes.dtype == np.int8 and scales.shape == (-(-n // bs),)
        assert codes.min() >= -127 and codes.max() <= 127
        for b in range(scales.size):
            blk = x[bs * b:bs * (b + 1)].astype(np.float64)
            cb = codes[bs * b:bs * (b + 1)].astype(np.float64)
            s = float(scales[b])
            a = np.abs(blk).max()
            assert s == np.float32(np.float32(a) / np.float32(127.0))
            err = np.abs(blk - s * cb)
            assert err.max() <= s * 0.5 * (1 + 1e-5)
            # the block's absmax element maps to +-127
            idx = np.unravel_index(np.abs(blk).argmax(), blk.shape)
            assert abs(cb[idx]) == 127 and np.sign(cb[idx]) == np.sign(blk[idx])


def test_int8_finer_blocks_are_the_halves(orc):
    """A 32-token block is quantized exactly as a 64-token block holding only
    those rows: each half gets its own absmax and scale."""
    rng = np.random.default_rng(4)
    x = rng.normal(0, 1, (128, 64)).astype(np.float32)
    x[40] *= 30.0                                   # one loud row in the second half
    c32, s32 = orc.quant_int8_blocks(x, 32)
    for b in range(4):
        cb, sb = orc.quant_int8_blocks(x[32 * b:32 * (b + 1)], 64)
        assert np.array_equal(c32[32 * b:32 * (b + 1)], cb) and s32[b] == sb[0]
    c64, s64 = orc.quant_int8_blocks(x, 64)
    # the loud row coarsens only its own 32-token block
    assert s32[0] < s64[0] and s32[1] == s64[0]


def test_int8_zero_block(orc):
    x = np.zeros((100, 64), np.float32)
    x[70:, :] = 1.5
    codes, scales = orc.quant_int8_blocks(x)
    assert scales[0] == 0.0 and not codes[:64].any()
    assert np.all(codes[70:] == 127) and not codes[64:70].any()


def test_int8_rne_ties(orc):
    # block absmax 127 -> inv = 1 exactly; x = k + 0.5 rounds to even
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5]], np.float32)
    codes, scales = orc.quant_int8_blocks(x)
    assert scales[0] == 1.0
    assert codes[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 126]


def test_fp8_channels_bounds(orc):
    rng = np.random.default_rng(3)
    v = rng.normal(0, 1, (500, 64)).astype(np.float32)
    v[:, 5] *= 10.0
    v[:, 6] = 0.0
    codes, scales = orc.quant_fp8_channels(v)
    assert scales[6] == 0.0 and not codes[:, 6].any()
    dec = orc.e4m3_decode(codes).astype(np.float64)
    for c in range(64):
        if c == 6:
            continue
        s = float(scales[c])
        a = np.abs(v[:, c]).max()
        assert s == np.float32(np.float32(a) / np.float32(448.0))
        recon = dec[:, c] * s
        x = v[:, c].astype(np.float64)
        big = np.abs(x) >= s * 2.0 ** -6          # normal range of the codes
        assert np.all(np.abs(recon[big] - x[big]) <= np.abs(x[big]) * 2.0 ** -4 * (1 + 1e-5))
        assert np.all(np.abs(recon[~big] - x[~big]) <= s * 2.0 ** -10 * (1 + 1e-5))
        # the channel absmax maps to +-448 (codes 0x7e / 0xfe)
        i = np.abs(x).argmax()
        assert codes[i, c] in (0x7e, 0xfe)


def test_delta_s_compensates_q_smoothing(orc):
    # (q - mu_q).k_s + ds = q.k_s for every pair: checks the bias's sign,
    # index and the mean it uses.
    rng = np.random.default_rng(4)
    q = rng.normal(0.5, 1.0, (80, 64)).astype(np.float32)
    k = rng.normal(0, 1, (90, 64)).astype(np.float32)
    mu = orc.channel_mean(q)
    qs = orc.smooth(q, mu)
    ds = orc.delta_s(mu, k)
    lhs = qs.astype(np.float64) @ k.T.astype(np.float64) + ds[None, :].astype(np.float64)
    rhs = q.astype(np.float64) @ k.T.astype(np.float64)
    assert np.max(np.abs(lhs - rhs)) < 1e-4 * np.abs(rhs).max()


def test_smooth_is_exact_subtraction(orc):
    x = np.array([[1.0, 2.0], [3.0, 5.0]], np.float32)
    mu = np.array([0.5, 3.0], np.float32)
    assert np.array_equal(orc.smooth(x, mu), np.array([[0.5, -1.0], [2.5, 2.0]], np.float32))
    assert np.array_equal(orc.smooth(x, None), x)


@pytest.mark.parametrize("k", [0, 40, 100, 110, 122, 126, 130])
def test_quantizers_are_scale_invariant_down_to_tiny_blocks(orc, k):
    # codes depend on x / a only, so scaling a block by 2^-k (exact for these
    # small integers, subnormal results included) leaves every INT8 and
    # deviation code as it is; below an absmax of about 10^-36 the plain
    # quotient 127/a (16256/a) would overflow FP32 and give sign-only codes
    # (NaN for zeros), which this catches.  Zeros stay zero codes.
    rng = np.random.default_rng(k)
    f = np.float32(2.0 ** -k)
    x = rng.integers(-1000, 1001, size=(150, 16)).astype(np.float32)
    x[3, :5] = 0.0
    c0, s0 = orc.quant_int8_blocks(x, 64)
    c1, s1 = orc.quant_int8_blocks(x * f, 64)
    assert np.array_equal(c0, c1)
    assert np.all(c1[3, :5] == 0)
    # the scale is a/127 of the scaled block (subnormal where that is)
    a1 = np.abs(x * f).reshape(-1)[:64 * 16].max()
    assert s1[0] == np.float32(a1) / np.float32(127)
    # V channels keep their codes down to an absmax of 2^-100 and count as
    # zero below it (scale 0, codes 0)
    v0, t0 = orc.quant_fp8_channels(x)
    v1, t1 = orc.quant_fp8_channels(x * f)
    amax = np.abs(x * f).max(axis=0)
    keep = amax >= np.float32(2.0 ** -100)
    assert np.array_equal(v0[:, keep], v1[:, keep])
    assert not v1[:, ~keep].any() and not t1[~keep].any()
    if k >= 110:
        assert not keep.any()
    h0, l0, _ = orc.mu_code(x[0])
    h1, l1, _ = orc.mu_code(x[0] * f)
    assert np.array_equal(h0, h1) and np.array_equal(l0, l1)
