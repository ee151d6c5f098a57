"""The allocation-free entry point sage_attn_fwd_noalloc (the library's own
static workspace) against sage_attn_fwd with a caller workspace, through the
C ABI: calls in a row on one GPU, each with a smaller problem than the last, each
bit for bit equal (output and log-sum-exp) to the workspace entry point's
result on the same inputs, and a problem whose workspace exceeds the static
array refused with SAGE_ERR_WORKSPACE."""
import pytest
import torch

import synth
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


def _lse_like(w, q):
    return torch.full((w.B, w.Hq, w.Nq), float("nan"), dtype=torch.float32, device=q.device)


def test_noalloc_matches_workspace_entry_twice():
    # each call smaller than the one before; the last one smooths Q per block,
    # which places the block means and deviation codes in the static array too
    cases = [synth.WORKLOADS["causal_gqa"],
             synth.scaled_down(synth.WORKLOADS["video_dit"], Hq=4, Hkv=4, Nq=700, Nkv=900,
                               d=128, layout="HND", seed=31),
             synth.scaled_down(synth.WORKLOADS["video_dit_block"], Hq=2, Hkv=2, Nq=600, Nkv=500,
                               seed=32)]
    for w in cases:
        pu.say(f"[noalloc] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} Nq={w.Nq} Nkv={w.Nkv} d={w.d}")
        q, k, v, meta = pu.gpu_inputs(w)
        kw = dict(tensor_layout=w.layout, is_causal=w.causal, smooth_q=w.smooth_q,
                  smooth_k=w.smooth_k, smooth_v=w.smooth_v, sm_scale=w.sm_scale)
        # the allocation-free call first (in a fresh process, the first call)
        o = torch.full_like(q, 3.0)
        lse = _lse_like(w, q)
        pu.qa.sage_attn_fwd_noalloc(q, k, v, o, lse=lse, **kw)
        torch.cuda.synchronize()
        o_ref, lse_ref = pu.qa.sage_attn_fwd(q, k, v, return_lse=True, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))


def test_noalloc_refuses_a_workspace_beyond_its_array():
    # llm_prefill needs about 100 MB of workspace, more than the 64 MiB array
    w = synth.WORKLOADS["llm_prefill"]
    q = torch.empty((w.B, w.Nq, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    desc = pu.qa.make_desc(q, q, q, q, tensor_layout="NHD")
    assert pu.qa.workspace_size(desc) > pu.qa._abi.NOALLOC_WS_MAX
    with pytest.raises(pu.qa.SageError, match="SAGE_ERR_WORKSPACE"):
        pu.qa.sage_attn_fwd_noalloc(q, q, q, torch.empty_like(q), tensor_layout="NHD")
