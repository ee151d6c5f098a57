"""GPU parity of per-block Q smoothing (smooth_q = "block") against the oracle.

The pre-pass outputs -- the sequence means, the per-block means, the codes of
the blocks' deviations and their scales, the INT8/E4M3 codes and scales --
are bit-exact; the sequence mean's score bias is within rtol 1e-5 (an FP32
dot product in a different order); the output, whose per-block compensation
the fused kernel forms from the deviation codes and the INT8 key codes, is
within max-abs 2e-2 and cosine 0.999 of the oracle's same-recipe result
(beyond the final rounding into the output dtype and the rounding-tie bound
of the P codes) and within cosine 0.99 of exact FP64 attention.  Cases span
head dims 64/96/128, 64- and 32-token blocks, one, two and four query heads
per workgroup, causal masks, ragged and empty varlen sequences and split
key ranges.
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
VB = W["video_dit_block"]

CASES = {
    # (workload, qk_block, kv_split)
    "d64_mha": (R(VB, Hq=2, Hkv=2, Nq=333, Nkv=300), 64, 0),
    "d64_mha_qb32": (R(VB, Hq=2, Hkv=2, Nq=333, Nkv=300), 32, 0),
    "d128_gqa4_causal": (R(W["causal_gqa"], smooth_q="block", q_drift_sigma=2.0, Hq=8, Hkv=2,
                           Nq=390, Nkv=520, seed=31), 64, 0),
    "d128_gqa4_causal_qb32": (R(W["causal_gqa"], smooth_q="block", q_drift_sigma=2.0, Hq=8,
                                Hkv=2, Nq=390, Nkv=520, seed=31), 32, 0),
    "d96_gqa2_nhd": (R(W["varlen_d96"], smooth_q="block", q_drift_sigma=2.0, Hq=4, Hkv=2,
                       causal=False, seqlens_q=[70, 200, 1], seqlens_kv=[300, 200, 129],
                       seed=32), 64, 0),
    "d128_varlen_empty": (R(W["varlen_d128"], smooth_q="block", q_drift_sigma=1.0, Hq=4, Hkv=2,
                            seqlens_q=[5, 0, 130, 33], seqlens_kv=[0, 40, 260, 1], seed=33),
                          32, 0),
    "d64_split": (R(VB, Hq=2, Hkv=2, Nq=200, Nkv=700, seed=34), 64, 256),
    "d128_decode_shape": (R(W["decode_gqa"], smooth_q="block", B=2, Hq=8, Hkv=2, Nq=3,
                            Nkv=900, seed=35), 64, "auto"),
}


def _kw(w, meta, qb, split):
    kw = dict(tensor_layout=w.layout, is_causal=w.causal, smooth_q=w.smooth_q,
              smooth_k=w.smooth_k, smooth_v=w.smooth_v, sm_scale=w.sm_scale, qk_block=qb,
              kv_split=split)
    if w.varlen:
        kw.update(cu_seqlens_q=meta["cu_seqlens_q"], cu_seqlens_kv=meta["cu_seqlens_kv"])
    return kw


def _fwd(w, q, k, v, meta, qb, split):
    kw = _kw(w, meta, qb, split)
    kw["return_lse"] = True
    if w.varlen:
        cq, ck = kw.pop("cu_seqlens_q"), kw.pop("cu_seqlens_kv")
        return pu.qa.sage_attn_fwd_varlen(q, k, v, cq, ck, **kw)
    return pu.qa.sage_attn_fwd(q, k, v, **kw)


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    name = request.param
    w, qb, split = CASES[name]
    pu.say(f"[block smoothing {name}] {w} qk_block={qb} kv_split={split}")
    q, k, v, meta = pu.gpu_inputs(w)
    prob = orc.problem_from_workload(w, qk_block=qb)
    ref = orc.prepass(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    return name, w, qb, split, q, k, v, meta, prob, ref


def test_prepass_bit_exact(case):
    name, w, qb, split, q, k, v, meta, prob, ref = case
    pu.say(f"[block prepass {name}]")
    kw = _kw(w, meta, qb, split)
    bufs = pu.qa.sage_quant_qkv(q, k, v, **kw)
    torch.cuda.synchronize()
    gpu, pads_ok = pu.unpack_quant(w, bufs, qb=qb)
    assert pads_ok, "padding rows/blocks must be zero"
    pu.assert_prepass_equal(gpu, ref, w)


def test_forward_matches_oracle(case):
    name, w, qb, split, q, k, v, meta, prob, ref = case
    pu.say(f"[block forward {name}]")
    o, lse = _fwd(w, q, k, v, meta, qb, split)
    torch.cuda.synchronize()
    got = pu.gpu_out_per_seq(w, o, meta)
    # the oracle takes the library's split of the key range (the P codes
    # depend on it)
    dkw = {x: y for x, y in _kw(w, meta, qb, split).items() if not x.startswith("cu_")}
    desc = pu.qa.make_desc(q, k, v, varlen=w.varlen, **dkw)
    keys = pu.qa.kv_split_size(desc, meta.get("cu_seqlens_q"), meta.get("cu_seqlens_kv"))
    prob_s = orc.problem_from_workload(w, qk_block=qb, kv_split=keys)
    rec, rec_lse, tie = orc.forward_rows(prob_s, ref, bkv=pu.KVT, tie=True)
    ex, _ = orc.exact_rows(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    lse_h = lse.cpu().numpy()
    for si, (nq, nkv) in enumerate(w.seq_lens()):
        g, r, e = got[si], rec[si], ex[si]
        assert np.all(np.isfinite(g))
        err = pu.max_excess(g, r, w.dtype, tie[si])
        assert err <= 2e-2, (si, err)
        assert pu.cos(g, r) >= 0.999, (si, pu.cos(g, r))
        assert pu.cos(g, e) >= 0.99, (si, pu.cos(g, e))
        gl = lse_h[:, meta["cu_seqlens_q"][si]:meta["cu_seqlens_q"][si] + nq] if w.varlen \
            else lse_h[si]
        fin = np.isfinite(r_l := rec_lse[si])
        assert np.array_equal(np.isfinite(gl), fin)
        if fin.any():
            assert np.abs(gl[fin] - r_l[fin]).max() < 2e-3 * max(1.0, np.abs(r_l[fin]).max())


def test_quantized_entry_and_determinism(case):
    name, w, qb, split, q, k, v, meta, prob, ref = case
    pu.say(f"[block quantized entry {name}]")
    o1, l1 = _fwd(w, q, k, v, meta, qb, split)
    o2, l2 = _fwd(w, q, k, v, meta, qb, split)
    kw = _kw(w, meta, qb, split)
    bufs = pu.qa.sage_quant_qkv(q, k, v, **kw)
    o3 = torch.zeros_like(q)
    l3 = torch.zeros_like(l1)
    ckw = {x: kw[x] for x in ("cu_seqlens_q", "cu_seqlens_kv") if x in kw}
    pu.qa.sage_attn_fwd_quantized(bufs, o3, lse=l3, **ckw)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    assert torch.equal(o3.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l3.view(torch.int32), l1.view(torch.int32))
