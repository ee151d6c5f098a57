"""Pins of the oracle's whole-problem driver: layouts, GQA head mapping,
variable-length packing and the scaled-down workloads (CPU only)."""
import numpy as np
import pytest
import torch

import synth


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _cos(a, b):
    a, b = np.ravel(a).astype(np.float64), np.ravel(b).astype(np.float64)
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def test_layouts_agree(orc):
    w = synth.scaled_down(synth.WORKLOADS["llm_prefill"], B=2, Hq=4, Hkv=2, Nq=70, Nkv=90,
                          d=64, layout="HND")
    q, k, v, _ = synth.make_inputs(w)
    outs = {}
    for lay in ("HND", "NHD"):
        pq, pk, pv = (t if lay == "HND" else t.permute(0, 2, 1, 3) for t in (q, k, v))
        prob = orc.problem_from_workload(synth.scaled_down(w, layout=lay))
        pre = orc.prepass(prob, _u16(pq), _u16(pk), _u16(pv))
        o, _ = orc.forward_rows(prob, pre)
        outs[lay] = o
    for a, b in zip(outs["HND"], outs["NHD"]):
        assert np.array_equal(a, b)


def test_generator_layout_independent():
    w = synth.scaled_down(synth.WORKLOADS["tiny"], B=2, Hq=2, Hkv=2, Nq=33, Nkv=33)
    a = synth.make_inputs(w)
    b = synth.make_inputs(synth.scaled_down(w, layout="NHD"))
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y.permute(0, 2, 1, 3))


def test_gqa_mapping(orc):
    # with Hq = 4, Hkv = 2, query head h must equal an MHA run whose K/V head
    # h is a copy of kv head h // 2
    w = synth.scaled_down(synth.WORKLOADS["causal_gqa"], Hq=4, Hkv=2, Nq=80, Nkv=80, d=64)
    q, k, v, _ = synth.make_inputs(w)
    prob = orc.problem_from_workload(w)
    o, _ = orc.forward_rows(prob, orc.prepass(prob, _u16(q), _u16(k), _u16(v)))
    k2, v2 = k.repeat_interleave(2, dim=1), v.repeat_interleave(2, dim=1)
    wm = synth.scaled_down(w, Hkv=4)
    pm = orc.problem_from_workload(wm)
    om, _ = orc.forward_rows(pm, orc.prepass(pm, _u16(q), _u16(k2), _u16(v2)))
    assert np.array_equal(o[0], om[0])


def test_varlen_equals_separate_sequences(orc):
    w = synth.scaled_down(synth.WORKLOADS["varlen_d128"], Hq=2, Hkv=2, d=96,
                          seqlens_q=[30, 70], seqlens_kv=[100, 130])
    q, k, v, meta = synth.make_inputs(w)
    prob = orc.problem_from_workload(w)
    o, _ = orc.forward_rows(prob, orc.prepass(prob, _u16(q), _u16(k), _u16(v)))
    cq, ck = meta["cu_seqlens_q"], meta["cu_seqlens_kv"]
    for s in range(2):
        qs = q[cq[s]:cq[s + 1]][None]
        ks = k[ck[s]:ck[s + 1]][None]
        vs = v[ck[s]:ck[s + 1]][None]
        ps = orc.Problem("f16", "NHD", 2, 2, 96, [(qs.shape[1], ks.shape[1])], causal=True)
        os_, _ = orc.forward_rows(ps, orc.prepass(ps, _u16(qs), _u16(ks), _u16(vs)))
        assert np.array_equal(o[s], os_[0])


@pytest.mark.parametrize("name", ["tiny", "llm_prefill", "causal_gqa", "video_dit",
                                  "varlen_d128", "varlen_d96"])
def test_scaled_workloads_vs_exact(orc, name):
    w = synth.WORKLOADS[name]
    if name != "tiny":
        if w.varlen:
            w = synth.scaled_down(w, Hq=2, Hkv=2, seqlens_q=[40, 100], seqlens_kv=[200, 330])
        else:
            w = synth.scaled_down(w, B=1, Hq=2 * w.Hq // w.Hkv, Hkv=2, Nq=200, Nkv=200)
    q, k, v, _ = synth.make_inputs(w)
    prob = orc.problem_from_workload(w)
    o, _ = orc.forward_rows(prob, orc.prepass(prob, _u16(q), _u16(k), _u16(v)))
    e, _ = orc.exact_rows(prob, _u16(q), _u16(k), _u16(v))
    for a, b in zip(o, e):
        assert _cos(a, b) >= 0.99
