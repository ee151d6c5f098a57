"""The library under HIP graph capture: a whole forward call (pre-pass and
attention kernels on the caller's stream, buffers preallocated) captured
once and replayed several times, with eager work and synchronizations
between the replays.  Every replay must reproduce the eager result bit for
bit, and a replay after the inputs change in place must match an eager call
on the new inputs.  Cases: the fused kernel, the split key range with the
one-wave decode kernel and its merge, a varlen problem with every smoothing
flag in the 16-bit P.V mode, and per-block Q smoothing (the block bias formed
in the fused kernel) with a split key range."""
import pytest
import torch

import synth
import quantized_attention_03_amd as qa
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
R = synth.scaled_down

CASES = {
    "fused_causal_gqa": (R(W["causal_gqa"], Hq=8, Hkv=2, Nq=300, Nkv=300), "fp8", 0),
    "decode_split": (R(W["decode_gqa"], B=2, Hq=8, Hkv=2, Nkv=2000), "fp8", "auto"),
    "varlen_half_smooth": (R(W["varlen_d128"], Hq=4, Hkv=2, seqlens_q=[100, 0, 37],
                             seqlens_kv=[130, 20, 300], smooth_q=True, smooth_v=True),
                           "half", 0),
    "block_smoothing_split": (R(W["video_dit_block"], Hq=4, Hkv=2, Nq=200, Nkv=600),
                              "fp8", 256),
}


def _call(w, q, k, v, meta, pv, split, o, ws):
    kw = dict(tensor_layout=w.layout, is_causal=w.causal, smooth_q=w.smooth_q,
              smooth_k=w.smooth_k, smooth_v=w.smooth_v, sm_scale=w.sm_scale, pv_mode=pv,
              kv_split=split, out=o, workspace=ws)
    if w.varlen:
        qa.sage_attn_fwd_varlen(q, k, v, meta["cu_seqlens_q"], meta["cu_seqlens_kv"], **kw)
    else:
        qa.sage_attn_fwd(q, k, v, **kw)


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    w, pv, split = CASES[name]
    pu.say(f"[graph {name}] {w}")
    q, k, v, meta = pu.gpu_inputs(w)
    desc = qa.make_desc(q, k, v, tensor_layout=w.layout, is_causal=w.causal,
                        smooth_q=w.smooth_q, smooth_k=w.smooth_k, smooth_v=w.smooth_v,
                        varlen=w.varlen, pv_mode=pv, kv_split=split)
    cu = (meta["cu_seqlens_q"], meta["cu_seqlens_kv"]) if w.varlen else ()
    ws = torch.empty(qa.workspace_size(desc, *cu), dtype=torch.uint8, device=q.device)
    o_eager = torch.empty_like(q)
    _call(w, q, k, v, meta, pv, split, o_eager, ws)      # also sets kernel attributes
    torch.cuda.synchronize()

    o = torch.zeros_like(q)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _call(w, q, k, v, meta, pv, split, o, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for rep in range(3):
        o.zero_()
        junk = torch.randn(1 << 20, device=q.device).sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(o.view(torch.int16), o_eager.view(torch.int16)), f"replay {rep}"

    # new inputs in place: the graph reads them live
    gen = torch.Generator(device=q.device).manual_seed(7)
    for t in (q, k, v):
        t.copy_(torch.randn(t.shape, generator=gen, device=t.device, dtype=torch.float32)
                .to(t.dtype))
    torch.cuda.synchronize()
    g.replay()
    o_new = torch.empty_like(q)
    _call(w, q, k, v, meta, pv, split, o_new, torch.empty_like(ws))
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_new.view(torch.int16))
    assert not torch.equal(o_new.view(torch.int16), o_eager.view(torch.int16))
