"""GPU parity at the edges of the input values, through the C ABI.

The seeded inputs of a small causal GQA problem (and of a bf16 one) are
rescaled or partly zeroed on the GPU, and both sides see the same bits:

* large: Q and K scaled up (fp16 by 30 and 500, bf16 by 300; the fp16 x500
  case also with the 16-bit P.V variant), so that the
  logits reach 10^3 .. 2*10^6 and each row's softmax is nearly one-hot; row
  maxima up to 2^21.4 in log2 units, where the FP32 roundings of the
  exponent could lift the top P code past the E4M3 convert's headroom (to
  the NaN code) unless the kernel raises the maximum first;
* tiny: Q, K and V scaled down to 10^-3 and 10^-5 of their size (fp16
  subnormals included; bf16 with the 16-bit P.V variant too), and bf16 Q
  and K to 10^-38 (FP32 subnormals; absmaxes below 2^-100, where the INT8
  quantizer rescales by 2^64 before forming 127/a, or the codes would be
  sign-only), so that the scores are nearly zero and the softmax nearly
  uniform; and V to 10^-38, whose channels (absmax below 2^-100) count as
  zero in the E4M3 quantizer: the output is 0 on both sides;
* zero blocks: one 64-token Q block, one 64-token K block (no K smoothing)
  and one V channel all zero: their scales and codes are 0;
* constant keys: every key row equal, which K smoothing turns into all-zero
  codes and scales (every score 0, a uniform softmax over the visible keys).

Beyond row maxima of 2^22 (log2 units; logits of about 3*10^6) one unit in
the last place of the maximum exceeds half a unit of the exponent, so no
FP32 evaluation of the exponent can place P on the E4M3 scale and the
recipe's output there is not defined; the case "beyond_range" (bf16 scaled
by 10^4, maxima near 2^31, both P.V variants) checks only that no NaN comes
out.

Each case in range checks the pre-pass bit for bit, every output element finite,
the output within max-abs 2e-2 (beyond the oracle's rounding-tie bound) and
cosine 0.999 of the same-recipe oracle, the LSE, and, where the logits stay
small enough for INT8 Q.K^T to keep each row's ranking (all but "large"),
cosine 0.99 against exact FP64 attention.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as orc
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
R = synth.scaled_down
BASE = R(W["causal_gqa"], Hq=4, Hkv=2, Nq=200, Nkv=300, seed=41)
BASE_BF16 = R(W["llm_prefill"], B=1, Hq=4, Hkv=4, Nq=150, Nkv=260, causal=True, seed=42)


def _scaled(fq, fk, fv):
    def f(q, k, v):
        return ((q.float() * fq).to(q.dtype), (k.float() * fk).to(k.dtype),
                (v.float() * fv).to(v.dtype))
    return f


def _zero_blocks(q, k, v):
    # HND: [B, H, N, d]
    q, k, v = q.clone(), k.clone(), v.clone()
    q[:, :, 64:128] = 0
    k[:, :, 128:192] = 0
    v[..., 5] = 0
    return q, k, v


def _constant_keys(q, k, v):
    k = k.clone()
    k[:] = k[:, :, 7:8]
    return q, k, v


CASES = {
    # (workload, transform, compare with exact FP64[, P.V mode])
    "large_x30_f16": (BASE, _scaled(30.0, 30.0, 1.0), False),
    "large_x500_f16": (BASE, _scaled(500.0, 500.0, 1.0), False),
    "large_x300_bf16": (BASE_BF16, _scaled(300.0, 300.0, 1.0), False),
    "large_x500_f16_pv_half": (BASE, _scaled(500.0, 500.0, 1.0), False, "half"),
    "tiny_1e-5_bf16_pv_half": (BASE_BF16, _scaled(1e-5, 1e-5, 1e-5), True, "half"),
    "tiny_qk_1e-38_bf16": (BASE_BF16, _scaled(1e-38, 1e-38, 1.0), True),
    "tiny_qk_1e-38_bf16_pv_half": (BASE_BF16, _scaled(1e-38, 1e-38, 1.0), True, "half"),
    "tiny_1e-3_f16": (BASE, _scaled(1e-3, 1e-3, 1e-3), True),
    "tiny_1e-5_f16_subnormal": (BASE, _scaled(1e-5, 1e-5, 1e-5), True),
    "zero_blocks": (R(BASE, smooth_k=False), _zero_blocks, True),
    "constant_keys": (BASE, _constant_keys, True),
}


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    name = request.param
    w, fn, exact, pv = (CASES[name] + ("fp8",))[:4]
    pu.say(f"[edge values {name}] {w} pv={pv}")
    q, k, v, meta = pu.gpu_inputs(w)
    q, k, v = fn(q, k, v)
    torch.cuda.synchronize()
    prob = orc.problem_from_workload(w, pv)
    ref = orc.prepass(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    return name, w, exact, pv, q, k, v, meta, prob, ref


def test_prepass_bit_exact(case):
    name, w, exact, pv, q, k, v, meta, prob, ref = case
    pu.say(f"[edge prepass {name}]")
    bufs = pu.run_quant(w, q, k, v, meta, pv=pv)
    torch.cuda.synchronize()
    gpu, pads_ok = pu.unpack_quant(w, bufs, pv=pv)
    assert pads_ok
    pu.assert_prepass_equal(gpu, ref, w)


def test_tiny_v_channels_count_as_zero():
    w = BASE_BF16
    pu.say("[edge tiny V: bf16 V x 1e-38]")
    q, k, v, meta = pu.gpu_inputs(w)
    q, k, v = _scaled(1.0, 1.0, 1e-38)(q, k, v)
    prob = orc.problem_from_workload(w)
    ref = orc.prepass(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    assert not any(x.any() for x in ref.vs) and not any(x.any() for x in ref.vc)
    bufs = pu.run_quant(w, q, k, v, meta)
    torch.cuda.synchronize()
    gpu, pads_ok = pu.unpack_quant(w, bufs)
    assert pads_ok
    pu.assert_prepass_equal(gpu, ref, w)
    o, lse = pu.run_fwd(w, q, k, v, meta)
    torch.cuda.synchronize()
    assert not o.float().abs().max().item()
    _, rec_lse = orc.forward_rows(prob, ref, bkv=pu.KVT)
    gl = lse.cpu().numpy()[0]
    assert np.abs(gl - rec_lse[0]).max() < 2e-3 * max(1.0, np.abs(rec_lse[0]).max())


@pytest.mark.parametrize("pv", ["fp8", "half"])
def test_beyond_range_gives_no_nan(pv):
    w = BASE_BF16
    pu.say(f"[edge beyond range: bf16 x 1e4, pv={pv}]")
    q, k, v, meta = pu.gpu_inputs(w)
    q, k, v = _scaled(1e4, 1e4, 1.0)(q, k, v)
    o, lse = pu.run_fwd(w, q, k, v, meta, pv=pv)
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    assert not torch.isnan(lse).any()


def test_forward_matches_oracle(case):
    name, w, exact, pv, q, k, v, meta, prob, ref = case
    pu.say(f"[edge forward {name}]")
    o, lse = pu.run_fwd(w, q, k, v, meta, pv=pv)
    torch.cuda.synchronize()
    got = pu.gpu_out_per_seq(w, o, meta)
    rec, rec_lse, tie = orc.forward_rows(prob, ref, bkv=pu.KVT, tie=True)
    ex, _ = orc.exact_rows(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    lse_h = lse.cpu().numpy()
    for si, (nq, nkv) in enumerate(w.seq_lens()):
        g, r, e = got[si], rec[si], ex[si]
        assert np.all(np.isfinite(g)), (si, int(np.sum(~np.isfinite(g))))
        err = pu.max_excess(g, r, w.dtype, tie[si])
        assert err <= 2e-2, (si, err)
        assert pu.cos(g, r) >= 0.999, (si, pu.cos(g, r))
        if exact:
            assert pu.cos(g, e) >= 0.99, (si, pu.cos(g, e))
        gl = lse_h[si]
        fin = np.isfinite(r_l := rec_lse[si])
        assert np.array_equal(np.isfinite(gl), fin)
        if fin.any():
            assert np.abs(gl[fin] - r_l[fin]).max() < 2e-3 * max(1.0, np.abs(r_l[fin]).max())
