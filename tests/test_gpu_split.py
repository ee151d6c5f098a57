"""GPU parity of a split key range (flash-decoding: kv_split keys per split,
each split an online softmax of its own, merged by the log-sum-exp rule)
through the C ABI, against the oracle's split recipe.

* few queries against long key ranges (decode shapes, where a GQA group's
  heads and queries fill one wave's 32 rows), GQA, d 64/96/128, causal and
  not, every smoothing flag, varlen with empty sequences, both P.V modes,
  explicit and automatic splits, and shapes too large for one wave (the
  fused kernel's split);
* the LSE equals the unsplit oracle's (it does not depend on the split);
* the kernel-only entry point reproduces the full call; runs are
  deterministic;
* the decode workload at full size (8 x 32 heads, one query, 32K keys), both
  P.V modes.
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

# (workload, kv_split, pv mode)
CASES = {
    "decode_q1": (R(W["decode_gqa"], B=3, Hq=8, Hkv=2, Nkv=1500), 256, "fp8"),
    "decode_q1_auto": (R(W["decode_gqa"], B=2, Hq=8, Hkv=2, Nkv=3000), "auto", "fp8"),
    "decode_q5_noncausal": (R(W["decode_gqa"], B=2, Hq=4, Hkv=4, Nq=5, Nkv=1000, causal=False,
                              seed=21), 128, "fp8"),
    "chunk_q40_causal_d96": (R(W["decode_gqa"], B=1, Hq=4, Hkv=2, Nq=40, Nkv=777, d=96,
                               seed=22), 256, "fp8"),
    "decode_d64_bf16_nhd": (R(W["decode_gqa"], dtype="bf16", layout="NHD", B=2, Hq=6, Hkv=2,
                              Nq=3, Nkv=900, d=64, seed=23), 128, "fp8"),
    "decode_smooth_all": (R(W["video_dit"], B=1, Hq=4, Hkv=2, Nq=7, Nkv=1100, d=128, seed=24,
                            layout="HND"), 384, "fp8"),
    # the fused kernel's split partials with Q, K and V smoothed (V scales and
    # means read from the workgroup's LDS copy; 80 rows per kv head, too many
    # for the one-wave kernel)
    "chunk_q40_smooth_all": (R(W["video_dit"], B=1, Hq=4, Hkv=2, Nq=40, Nkv=900, d=128,
                               seed=32, layout="HND"), 256, "fp8"),
    "decode_half": (R(W["decode_gqa"], B=2, Hq=8, Hkv=2, Nkv=1300, seed=25), 256, "half"),
    "decode_half_bf16_smooth_v": (R(W["decode_gqa"], dtype="bf16", B=1, Hq=4, Hkv=4, Nq=2,
                                    Nkv=800, smooth_v=True, seed=26), 128, "half"),
    "varlen_split": (R(W["varlen_d128"], Hq=4, Hkv=2, seqlens_q=[1, 0, 3, 2],
                       seqlens_kv=[700, 40, 1, 0]), 256, "fp8"),
    "split_wider_than_keys": (R(W["decode_gqa"], B=1, Hq=4, Hkv=4, Nq=4, Nkv=200, seed=27),
                              1024, "fp8"),
    # the one-wave decode kernel at its limits: an odd GQA group with the
    # score bias (Q smoothing), a full wave of 32 rows with the 16-bit P.V
    # and the bias (the copies that exceed the wave's counter budget), d 96
    # with 32 rows, d 64 in the 16-bit mode, and a shape one row too large
    # for it (the fused kernel then takes the split)
    "decode_g3_smooth_q": (R(W["video_dit"], B=1, Hq=6, Hkv=2, Nq=2, Nkv=900, d=128, seed=28,
                             layout="HND"), 256, "fp8"),
    "decode_rows32_half_ds": (R(W["video_dit"], B=1, Hq=32, Hkv=1, Nq=1, Nkv=700, d=128,
                                seed=29, layout="HND"), 256, "half"),
    "decode_rows32_d96": (R(W["decode_gqa"], B=1, Hq=16, Hkv=2, Nq=4, Nkv=1000, d=96, seed=30),
                          384, "fp8"),
    "decode_d64_half": (R(W["decode_gqa"], B=2, Hq=4, Hkv=2, Nq=1, Nkv=600, d=64, seed=31),
                        128, "half"),
    "rows33_fused_split": (R(W["decode_gqa"], B=1, Hq=3, Hkv=1, Nq=11, Nkv=700, seed=32),
                           256, "fp8"),
    # more than 64 splits: the merge walks its splits 64 per pass (71 here),
    # after the one-wave kernel and after the fused kernel's split
    "many_splits_decode": (R(W["decode_gqa"], B=1, Hq=4, Hkv=2, Nq=1, Nkv=9000, seed=33),
                           128, "fp8"),
    "many_splits_fused": (R(W["decode_gqa"], B=1, Hq=4, Hkv=1, Nq=9, Nkv=9000, seed=34),
                          128, "fp8"),
}


def _kw(w, split, pv):
    kw = dict(tensor_layout=w.layout, is_causal=w.causal, smooth_q=w.smooth_q,
              smooth_k=w.smooth_k, smooth_v=w.smooth_v, sm_scale=w.sm_scale, pv_mode=pv,
              kv_split=split)
    return kw


def _run(w, q, k, v, meta, split, pv):
    kw = _kw(w, split, pv)
    if w.varlen:
        return pu.qa.sage_attn_fwd_varlen(q, k, v, meta["cu_seqlens_q"], meta["cu_seqlens_kv"],
                                          return_lse=True, **kw)
    return pu.qa.sage_attn_fwd(q, k, v, return_lse=True, **kw)


def _effective_split(w, q, k, v, meta, split, pv):
    desc = pu.qa.make_desc(q, k, v, varlen=w.varlen, **_kw(w, split, pv))
    if w.varlen:
        return pu.qa.kv_split_size(desc, meta["cu_seqlens_q"], meta["cu_seqlens_kv"])
    return pu.qa.kv_split_size(desc)


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    name = request.param
    w, split, pv = CASES[name]
    pu.say(f"[split case {name}] split={split} pv={pv} {w}")
    q, k, v, meta = pu.gpu_inputs(w)
    eff = _effective_split(w, q, k, v, meta, split, pv)
    prob = orc.problem_from_workload(w, pv, eff)
    ref = orc.prepass(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    return name, w, split, pv, eff, q, k, v, meta, prob, ref


def _lse_of(w, lse_h, meta, si, nq):
    if w.varlen:
        t0 = meta["cu_seqlens_q"][si]
        return lse_h[:, t0:t0 + nq]
    return lse_h[si]


def test_split_forward_matches_oracle(case):
    name, w, split, pv, eff, q, k, v, meta, prob, ref = case
    pu.say(f"[split forward {name}] effective split {eff}")
    if split == "auto":
        assert eff > 0, "the decode shape must be split by the automatic rule"
    o, lse = _run(w, q, k, v, meta, split, pv)
    torch.cuda.synchronize()
    got = pu.gpu_out_per_seq(w, o, meta)
    rec, rec_lse, tie = orc.forward_rows(prob, ref, bkv=pu.KVT, tie=True)
    ex, _ = orc.exact_rows(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    unsplit = orc.Problem(**{**prob.__dict__, "kv_split": 0})
    _, l0 = orc.forward_rows(unsplit, ref, bkv=pu.KVT)
    lse_h = lse.cpu().numpy()
    for si, (nq, nkv) in enumerate(w.seq_lens()):
        g, r, e = got[si], rec[si], ex[si]
        assert np.all(np.isfinite(g))
        if g.size == 0:
            continue
        err = pu.max_excess(g, r, w.dtype, tie[si])
        assert err <= 2e-2, (si, err)
        assert pu.cos(g, r) >= 0.999, (si, pu.cos(g, r))
        assert pu.cos(g, e) >= 0.99, (si, pu.cos(g, e))
        gl = _lse_of(w, lse_h, meta, si, nq)
        fin = np.isfinite(rec_lse[si])
        assert np.array_equal(np.isfinite(gl), fin)
        if fin.any():
            tol = 2e-3 * max(1.0, np.abs(rec_lse[si][fin]).max())
            assert np.abs(gl[fin] - rec_lse[si][fin]).max() < tol
            # the LSE does not depend on the split
            assert np.abs(gl[fin] - l0[si][fin]).max() < tol
        # rows without any visible key give 0
        assert not g[:, ~np.isfinite(rec_lse[si][0])].any() if g.shape[1] else True


def test_split_quantized_entry_and_determinism(case):
    name, w, split, pv, eff, q, k, v, meta, prob, ref = case
    pu.say(f"[split quantized entry {name}]")
    o1, l1 = _run(w, q, k, v, meta, split, pv)
    o2, l2 = _run(w, q, k, v, meta, split, pv)
    kw = _kw(w, split, pv)
    cu = {}
    if w.varlen:
        cu = dict(cu_seqlens_q=meta["cu_seqlens_q"], cu_seqlens_kv=meta["cu_seqlens_kv"])
    bufs = pu.qa.sage_quant_qkv(q, k, v, **kw, **cu)
    o3 = torch.zeros_like(o1)
    l3 = torch.zeros_like(l1)
    pu.qa.sage_attn_fwd_quantized(bufs, o3, lse=l3, **cu)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l3.view(torch.int32))


@pytest.mark.parametrize("pv", ["fp8", "half"])
def test_decode_full_size_split(pv):
    """The decode workload at full size in the launch configuration bench.py
    times (automatic split, one-wave decode kernel), both P.V modes."""
    w = W["decode_gqa"]
    pu.say(f"[split full size decode_gqa {pv}] generating inputs")
    q, k, v, meta = pu.gpu_inputs(w)
    eff = _effective_split(w, q, k, v, meta, "auto", pv)
    assert eff > 0
    prob = orc.problem_from_workload(w, pv, eff)
    qh, kh, vh = pu.u16(q), pu.u16(k), pu.u16(v)
    pu.say(f"[split full size decode_gqa {pv}] split {eff}")
    o, lse = _run(w, q, k, v, meta, "auto", pv)
    torch.cuda.synchronize()
    got = pu.gpu_out_per_seq(w, o, meta)
    ref = orc.prepass(prob, qh, kh, vh)
    rec, rec_lse, tie = orc.forward_rows(prob, ref, bkv=pu.KVT, tie=True)
    ex, _ = orc.exact_rows(prob, qh, kh, vh)
    lse_h = lse.cpu().numpy()
    for si in range(w.B):
        err = pu.max_excess(got[si], rec[si], w.dtype, tie[si])
        pu.say(f"  seq {si}: max_excess {err:.4g} cos {pu.cos(got[si], rec[si]):.6f}")
        assert err <= 2e-2
        assert pu.cos(got[si], rec[si]) >= 0.999
        assert pu.cos(got[si], ex[si]) >= 0.99
        assert np.abs(lse_h[si] - rec_lse[si]).max() < 2e-3 * max(1.0, np.abs(rec_lse[si]).max())
