"""The SDPA-signature drop-in: arguments the method cannot honour are refused
on the host (CPU tests); on the GPU it is the library call itself, close to
torch's own attention."""
import numpy as np
import pytest
import torch

import quantized_attention_03_amd as qa


def _t(*shape, dtype=torch.float16):
    return torch.zeros(*shape, dtype=dtype)


@pytest.mark.parametrize("kw,msg", [
    (dict(attn_mask=torch.ones(4, 4, dtype=torch.bool)), "attn_mask"),
    (dict(dropout_p=0.1), "dropout"),
])
def test_unsupported_arguments_raise(kw, msg):
    with pytest.raises(ValueError, match=msg):
        qa.sdpa(_t(1, 2, 4, 64), _t(1, 2, 4, 64), _t(1, 2, 4, 64), **kw)


def test_gqa_needs_enable_gqa_and_causal_needs_square():
    with pytest.raises(ValueError, match="enable_gqa"):
        qa.sdpa(_t(1, 4, 8, 64), _t(1, 2, 8, 64), _t(1, 2, 8, 64))
    with pytest.raises(ValueError, match="top-left"):
        qa.sdpa(_t(1, 2, 8, 64), _t(1, 2, 16, 64), _t(1, 2, 16, 64), is_causal=True)
    with pytest.raises(ValueError, match=r"\[B, H, N, d\]"):
        qa.sdpa(_t(2, 8, 64), _t(2, 8, 64), _t(2, 8, 64))


@pytest.mark.gpu
@pytest.mark.parametrize("causal,hkv,dtype", [(False, 4, torch.float16), (True, 2, torch.bfloat16)])
def test_sdpa_is_the_library_call(causal, hkv, dtype):
    g = torch.Generator(device="cuda").manual_seed(5)
    q = torch.randn(2, 4, 300, 128, device="cuda", generator=g).to(dtype)
    k = torch.randn(2, hkv, 300, 128, device="cuda", generator=g).to(dtype)
    v = torch.randn(2, hkv, 300, 128, device="cuda", generator=g).to(dtype)
    o = qa.sdpa(q, k, v, is_causal=causal, enable_gqa=hkv != 4)
    o2 = qa.sageattn(q, k, v, tensor_layout="HND", is_causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    # close to torch's attention (float32 reference on the host)
    rep = 4 // hkv
    kf = k.float().cpu().repeat_interleave(rep, dim=1)
    vf = v.float().cpu().repeat_interleave(rep, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q.float().cpu(), kf, vf,
                                                           is_causal=causal)
    a, b = o.float().cpu().flatten().double(), ref.flatten().double()
    assert float(a @ b / (a.norm() * b.norm())) > 0.99
