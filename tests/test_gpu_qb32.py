"""GPU parity of 32-token Q/K quantization blocks (qk_block = 32: one scale
per wave's 32 query rows and per 32-key MFMA block) through the C ABI,
against the oracle with the same block size.

* pre-pass bit for bit (every code and the doubled scale arrays);
* forward within the usual bars, on d 64/96/128, GQA, causal, all smoothing,
  varlen with empty sequences, the 16-bit P.V variant and a split key range;
* at full llm_prefill size (Q outlier channels) on sampled rows, closer to
  exact attention than 64-token blocks.
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

# (workload, pv mode, kv_split)
CASES = {
    "tiny": (W["tiny"], "fp8", 0),
    "llm_prefill_small": (R(W["llm_prefill"], B=2, Hq=4, Hkv=4, Nq=300, Nkv=300), "fp8", 0),
    "causal_gqa_small": (R(W["causal_gqa"], Hq=8, Hkv=2, Nq=520, Nkv=520), "fp8", 0),
    "video_dit_small": (R(W["video_dit"], Hq=2, Hkv=2, Nq=333, Nkv=333), "fp8", 0),
    "d96_ragged": (R(W["tiny"], d=96, B=2, Hq=2, Hkv=2, Nq=63, Nkv=95, seed=7), "fp8", 0),
    "varlen_empty": (R(W["varlen_d128"], Hq=4, Hkv=2, seqlens_q=[5, 0, 70, 33],
                       seqlens_kv=[0, 40, 129, 1]), "fp8", 0),
    "half_bf16_smooth_all": (R(W["video_dit"], Hq=4, Hkv=2, Nq=190, Nkv=260, d=128, seed=13,
                               layout="HND"), "half", 0),
    "decode_split": (R(W["decode_gqa"], B=2, Hq=8, Hkv=2, Nq=3, Nkv=1200), "fp8", 256),
}


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    name = request.param
    w, pv, split = CASES[name]
    pu.say(f"[qb32 case {name}] pv={pv} split={split} {w}")
    q, k, v, meta = pu.gpu_inputs(w)
    prob = orc.problem_from_workload(w, pv, split, 32)
    ref = orc.prepass(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    return name, w, pv, split, q, k, v, meta, prob, ref


def _fwd(w, q, k, v, meta, pv, split, qb=32):
    kw = dict(tensor_layout=w.layout, is_causal=w.causal, smooth_q=w.smooth_q,
              smooth_k=w.smooth_k, smooth_v=w.smooth_v, sm_scale=w.sm_scale, return_lse=True,
              pv_mode=pv, kv_split=split, qk_block=qb)
    if w.varlen:
        return pu.qa.sage_attn_fwd_varlen(q, k, v, meta["cu_seqlens_q"], meta["cu_seqlens_kv"],
                                          **kw)
    return pu.qa.sage_attn_fwd(q, k, v, **kw)


def test_qb32_prepass_bit_exact(case):
    name, w, pv, split, q, k, v, meta, prob, ref = case
    pu.say(f"[qb32 prepass {name}]")
    bufs = pu.run_quant(w, q, k, v, meta, pv=pv, qb=32)
    torch.cuda.synchronize()
    gpu, pads_ok = pu.unpack_quant(w, bufs, pv=pv, qb=32)
    assert pads_ok
    pu.assert_prepass_equal(gpu, ref, w)


def test_qb32_forward_matches_oracle(case):
    name, w, pv, split, q, k, v, meta, prob, ref = case
    pu.say(f"[qb32 forward {name}]")
    o, lse = _fwd(w, q, k, v, meta, pv, split)
    torch.cuda.synchronize()
    got = pu.gpu_out_per_seq(w, o, meta)
    rec, rec_lse, tie = orc.forward_rows(prob, ref, bkv=pu.KVT, tie=True)
    ex, _ = orc.exact_rows(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    lse_h = lse.cpu().numpy()
    for si, (nq, nkv) in enumerate(w.seq_lens()):
        g, r, e = got[si], rec[si], ex[si]
        if g.size == 0:
            continue
        assert np.all(np.isfinite(g))
        assert pu.max_excess(g, r, w.dtype, tie[si]) <= 2e-2
        assert pu.cos(g, r) >= 0.999
        assert pu.cos(g, e) >= 0.99
        gl = lse_h[:, meta["cu_seqlens_q"][si]:meta["cu_seqlens_q"][si] + nq] if w.varlen \
            else lse_h[si]
        fin = np.isfinite(rec_lse[si])
        assert np.array_equal(np.isfinite(gl), fin)
        if fin.any():
            assert np.abs(gl[fin] - rec_lse[si][fin]).max() < \
                2e-3 * max(1.0, np.abs(rec_lse[si][fin]).max())


def test_qb32_full_size_llm_prefill():
    w = W["llm_prefill"]
    pu.say("[qb32 full size llm_prefill]")
    q, k, v, meta = pu.gpu_inputs(w)
    qh, kh, vh = pu.u16(q), pu.u16(k), pu.u16(v)
    prob = orc.problem_from_workload(w, "fp8", 0, 32)
    bufs = pu.run_quant(w, q, k, v, meta, qb=32)
    torch.cuda.synchronize()
    gpu_pre, pads_ok = pu.unpack_quant(w, bufs, qb=32)
    ref = orc.prepass(prob, qh, kh, vh)
    assert pads_ok
    pu.assert_prepass_equal(gpu_pre, ref, w)
    o32, _ = _fwd(w, q, k, v, meta, "fp8", 0, 32)
    o64, _ = _fwd(w, q, k, v, meta, "fp8", 0, 64)
    torch.cuda.synchronize()
    g32 = pu.gpu_out_per_seq(w, o32, meta)
    g64 = pu.gpu_out_per_seq(w, o64, meta)
    rows = [pu.sample_rows(nq, 24, 300 + s) for s, (nq, _) in enumerate(w.seq_lens())]
    rec, _, tie = orc.forward_rows(prob, ref, rows=rows, bkv=pu.KVT, tie=True)
    ex, _ = orc.exact_rows(prob, qh, kh, vh, rows=rows)
    e32 = e64 = 0.0
    for s in range(len(rows)):
        a = g32[s][:, rows[s]]
        assert pu.max_excess(a, rec[s], w.dtype, tie[s]) <= 2e-2
        assert pu.cos(a, rec[s]) >= 0.999
        e32 += float(np.sum((a - ex[s]) ** 2))
        e64 += float(np.sum((g64[s][:, rows[s]] - ex[s]) ** 2))
    pu.say(f"  squared error vs FP64: 32-token {e32:.4g}, 64-token {e64:.4g}")
    assert e32 < e64
