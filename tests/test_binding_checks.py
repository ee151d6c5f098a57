"""CPU checks of the Python binding's refusals: tensors that do not describe
one problem raise ValueError before anything reaches the library's compute
entry points (the kernels would otherwise read or write out of bounds)."""
import pytest
import torch

import quantized_attention_03_amd as qa


def _t(*shape, dtype=torch.float16):
    return torch.zeros(*shape, dtype=dtype)


def _desc(q, k, v, o=None, **kw):
    return qa.make_desc(q, k, v, o, **kw)


@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_consistent_cpu_tensors_reach_the_device_check(layout):
    q = _t(2, 4, 64, 128)
    with pytest.raises(ValueError, match="CUDA device"):
        _desc(q, q.clone(), q.clone(), q.clone(), tensor_layout=layout)


@pytest.mark.parametrize("bad,match", [
    (dict(v=_t(2, 4, 65, 128)), "v must have k's shape"),
    (dict(k=_t(2, 4, 64, 64), v=_t(2, 4, 64, 64)), "head dims differ"),
    (dict(k=_t(3, 4, 64, 128), v=_t(3, 4, 64, 128)), "batch sizes differ"),
    (dict(o=_t(2, 4, 63, 128)), "out must have q's shape"),
    (dict(o=_t(2, 4, 64, 128, dtype=torch.bfloat16)), "out must have q's shape"),
    (dict(q=_t(4, 64, 128)), "must have 4 dimensions"),
    (dict(k=_t(2, 4, 64, 128, dtype=torch.bfloat16)), "share dtype"),
])
def test_mismatches_raise(bad, match):
    args = dict(q=_t(2, 4, 64, 128), k=_t(2, 4, 64, 128), v=_t(2, 4, 64, 128), o=None)
    args.update(bad)
    with pytest.raises(ValueError, match=match):
        _desc(args["q"], args["k"], args["v"], args["o"])


def test_expanded_views_raise():
    # strides (0, 0, 0, 1): would read as the contiguous layout's all-zero
    # stride triple and run past the one row that exists
    q = torch.zeros(128, dtype=torch.float16).expand(2, 4, 64, 128)
    k = _t(2, 4, 64, 128)
    with pytest.raises(ValueError, match="stride 0"):
        _desc(q, k, k.clone())
    with pytest.raises(ValueError, match="stride 0"):
        _desc(_t(2, 4, 64, 128), k, k.clone(), q)


def test_head_dim_stride_must_be_one():
    q = _t(2, 4, 128, 64).transpose(2, 3)
    with pytest.raises(ValueError, match="stride 1"):
        _desc(q, _t(2, 4, 64, 128), _t(2, 4, 64, 128))


def test_varlen_token_counts():
    q = _t(100, 4, 64)
    k = _t(300, 2, 64)
    qa._check_tokens(q, k, "NHD", [0, 60, 100], 2, [0, 200, 300], 2)
    with pytest.raises(ValueError, match="cu_seqlens_q ends at 101"):
        qa._check_tokens(q, k, "NHD", [0, 60, 101], 2, [0, 200, 300], 2)
    with pytest.raises(ValueError, match="cu_seqlens_kv ends at 301"):
        qa._check_tokens(q, k, "NHD", [0, 60, 100], 2, [0, 200, 301], 2)
    # HND packs tokens in the second dimension
    qh, kh = _t(4, 100, 64), _t(2, 300, 64)
    qa._check_tokens(qh, kh, "HND", [0, 100], 1, [0, 300], 1)
    with pytest.raises(ValueError, match="cu_seqlens_kv"):
        qa._check_tokens(qh, kh, "HND", [0, 100], 1, [0, 301], 1)
