"""GPU parity of the 16-bit P.V variant (pv_mode "half": P and V in the
input's 16-bit type, FP32 accumulation), through the C ABI, against the
oracle's same-recipe variant (orc_attn_recipe_half_rows).

* pre-pass: every mean, INT8 code and scale and the 16-bit V operand bit for
  bit (and no V scale);
* forward: max-abs 2e-2 beyond the output rounding and cosine 0.999 against
  the same-recipe oracle, cosine 0.99 against exact FP64 attention, LSE;
* the kernel-only entry point reproduces the full call, runs are
  deterministic;
* full workload sizes on sampled rows (bf16 LLM prefill, fp16 causal GQA).
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

CASES = {
    "tiny": W["tiny"],
    "llm_prefill_small": R(W["llm_prefill"], B=2, Hq=4, Hkv=4, Nq=300, Nkv=300),
    "causal_gqa_small": R(W["causal_gqa"], Hq=8, Hkv=2, Nq=520, Nkv=520),
    "video_dit_small": R(W["video_dit"], Hq=2, Hkv=2, Nq=333, Nkv=333),
    "varlen_d128_small": R(W["varlen_d128"], Hq=4, Hkv=4,
                           seqlens_q=[100, 37, 300, 65], seqlens_kv=[700, 37, 130, 1]),
    "varlen_d96_small": R(W["varlen_d96"], Hq=4, Hkv=2,
                          seqlens_q=[64, 200, 1], seqlens_kv=[300, 200, 129]),
    "d96_hnd_ragged": R(W["tiny"], d=96, B=2, Hq=2, Hkv=2, Nq=63, Nkv=65, seed=7),
    "d64_nq_gt_nkv_causal": R(W["tiny"], Hq=2, Hkv=1, Nq=200, Nkv=70, causal=True, seed=8),
    "d128_one_key_smooth_v": R(W["tiny"], d=128, Hq=2, Hkv=2, Nq=129, Nkv=1, smooth_v=True,
                               seed=10),
    "gqa2_smooth_all_d128": R(W["video_dit"], Hq=4, Hkv=2, Nq=190, Nkv=260, d=128, seed=13,
                              layout="HND"),
    "varlen_empty_seqs": R(W["varlen_d128"], Hq=4, Hkv=2,
                           seqlens_q=[5, 0, 70, 33], seqlens_kv=[0, 40, 129, 1]),
}


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    name = request.param
    w = CASES[name]
    pu.say(f"[half case {name}] {w}")
    q, k, v, meta = pu.gpu_inputs(w)
    prob = orc.problem_from_workload(w, "half")
    ref = orc.prepass(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    return name, w, q, k, v, meta, prob, ref


def _check_forward(w, got, rec, rec_lse, ex, lse_h, meta, rows=None, tie=None):
    for si, (nq, nkv) in enumerate(w.seq_lens()):
        g = got[si] if rows is None else got[si][:, rows[si]]
        r, e = rec[si], ex[si]
        assert np.all(np.isfinite(g))
        err = pu.max_excess(g, r, w.dtype, None if tie is None else tie[si])
        assert err <= 2e-2, (si, err)
        assert pu.cos(g, r) >= 0.999, (si, pu.cos(g, r))
        assert pu.cos(g, e) >= 0.99, (si, pu.cos(g, e))
        if lse_h is None:
            continue
        if w.varlen:
            t0 = meta["cu_seqlens_q"][si]
            gl = lse_h[:, t0:t0 + nq]
        else:
            gl = lse_h[si]
        if rows is not None:
            gl = gl[:, rows[si]]
        fin = np.isfinite(r_l := rec_lse[si])
        assert np.array_equal(np.isfinite(gl), fin)
        if fin.any():
            assert np.abs(gl[fin] - r_l[fin]).max() < 2e-3 * max(1.0, np.abs(r_l[fin]).max())


def test_half_prepass_bit_exact(case):
    name, w, q, k, v, meta, prob, ref = case
    pu.say(f"[half prepass {name}]")
    bufs = pu.run_quant(w, q, k, v, meta, pv="half")
    torch.cuda.synchronize()
    gpu, pads_ok = pu.unpack_quant(w, bufs, pv="half")
    assert pads_ok, "padding rows/blocks must be zero"
    assert bufs["_sizes"]["v_scale"] == 0
    pu.assert_prepass_equal(gpu, ref, w)


def test_half_forward_matches_oracle(case):
    name, w, q, k, v, meta, prob, ref = case
    pu.say(f"[half forward {name}]")
    o, lse = pu.run_fwd(w, q, k, v, meta, pv="half")
    torch.cuda.synchronize()
    got = pu.gpu_out_per_seq(w, o, meta)
    rec, rec_lse, tie = orc.forward_rows(prob, ref, bkv=pu.KVT, tie=True)
    ex, _ = orc.exact_rows(prob, pu.u16(q), pu.u16(k), pu.u16(v))
    _check_forward(w, got, rec, rec_lse, ex, lse.cpu().numpy(), meta, tie=tie)


def test_half_quantized_entry_and_determinism(case):
    name, w, q, k, v, meta, prob, ref = case
    pu.say(f"[half quantized entry {name}]")
    o1, l1 = pu.run_fwd(w, q, k, v, meta, pv="half")
    o2, l2 = pu.run_fwd(w, q, k, v, meta, pv="half")
    bufs = pu.run_quant(w, q, k, v, meta, pv="half")
    o3 = torch.zeros_like(o1)
    l3 = torch.zeros_like(l1)
    kw = {}
    if w.varlen:
        kw = dict(cu_seqlens_q=meta["cu_seqlens_q"], cu_seqlens_kv=meta["cu_seqlens_kv"])
    pu.qa.sage_attn_fwd_quantized(bufs, o3, lse=l3, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l3.view(torch.int32))


def test_half_differs_from_fp8_path():
    """The mode switch reaches the kernel: on the same inputs the two recipes
    give different outputs, each matching its own oracle."""
    w = CASES["causal_gqa_small"]
    q, k, v, meta = pu.gpu_inputs(w)
    pu.say("[half vs fp8]")
    oh = pu.run_fwd(w, q, k, v, meta, return_lse=False, pv="half")
    of = pu.run_fwd(w, q, k, v, meta, return_lse=False, pv="fp8")
    torch.cuda.synchronize()
    assert not torch.equal(oh.view(torch.int16), of.view(torch.int16))
    ex, _ = orc.exact_rows(orc.problem_from_workload(w), pu.u16(q), pu.u16(k), pu.u16(v))
    gh = pu.gpu_out_per_seq(w, oh, meta)[0]
    gf = pu.gpu_out_per_seq(w, of, meta)[0]
    # 16-bit P and V are the more accurate operands
    assert np.abs(gh - ex[0]).max() < np.abs(gf - ex[0]).max()


@pytest.mark.parametrize("name", ["llm_prefill", "causal_gqa"])
def test_half_full_size(name):
    w = W[name]
    pu.say(f"[half full size {name}] generating inputs")
    q, k, v, meta = pu.gpu_inputs(w)
    prob = orc.problem_from_workload(w, "half")
    qh, kh, vh = pu.u16(q), pu.u16(k), pu.u16(v)
    pu.say(f"[half full size {name}] pre-pass")
    bufs = pu.run_quant(w, q, k, v, meta, pv="half")
    torch.cuda.synchronize()
    gpu_pre, pads_ok = pu.unpack_quant(w, bufs, pv="half")
    ref = orc.prepass(prob, qh, kh, vh)
    assert pads_ok
    pu.assert_prepass_equal(gpu_pre, ref, w)
    pu.say(f"[half full size {name}] forward")
    o, lse = pu.run_fwd(w, q, k, v, meta, pv="half")
    torch.cuda.synchronize()
    got = pu.gpu_out_per_seq(w, o, meta)
    rows = [pu.sample_rows(nq, 24, 200 + s) for s, (nq, _) in enumerate(w.seq_lens())]
    rec, rec_lse, tie = orc.forward_rows(prob, ref, rows=rows, bkv=pu.KVT, tie=True)
    ex, _ = orc.exact_rows(prob, qh, kh, vh, rows=rows)
    _check_forward(w, got, rec, rec_lse, ex, lse.cpu().numpy(), meta, rows=rows, tie=tie)
