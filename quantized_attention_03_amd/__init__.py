"""Thin Python binding of libsage (include/sage.h): argument marshalling only.

Every step of the forward pass runs in the HIP library; PyTorch provides the
device memory and the stream.  If libsage.so has not been built, every call
raises (there is no CPU or eager fallback).

    from quantized_attention_03_amd import sageattn
    o = sageattn(q, k, v, tensor_layout="HND", is_causal=False, smooth_k=True)

mirrors the `sageattn` call of the "sageattention" package page (Quickstart).
Every entry point takes pv_mode="fp8" (E4M3 P and V, SageAttention2; the
default) or pv_mode="half" (P and V in the input's 16-bit type, the first
SageAttention's INT8-QK / 16-bit-PV kernel), and kv_split: 0 (no split of
the key range), a multiple of 128 keys, or "auto" (the library's rule; see
kv_split_size), and qk_block: 64 (default) or 32 tokens per Q/K quantization
block.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _abi
from ._abi import BF16, F16, HND, NHD, KV_TILE, QK_BLOCK, SageError, lib

__all__ = ["sageattn", "sdpa", "sage_attn_fwd", "sage_attn_fwd_varlen", "sage_quant_qkv",
           "sage_attn_fwd_noalloc",
           "sage_attn_fwd_quantized", "kv_split_size",
           "sage_debug_qk_int32", "sage_debug_e4m3_encode", "workspace_size", "quant_buf_sizes", "make_desc",
           "SageError", "lib", "abi_version"]

_DT = {torch.float16: F16, torch.bfloat16: BF16}


def abi_version() -> int:
    return lib().sage_abi_version()


def _strides(t: torch.Tensor, layout: str, varlen: bool):
    if t.stride(-1) != 1:
        raise ValueError("the head_dim dimension must have stride 1")
    for size, st in zip(t.shape, t.stride()):
        if size > 1 and st == 0:
            raise ValueError("a dimension of size > 1 has stride 0 (an expanded view): "
                             "call .contiguous() first")
    s = t.stride()
    if varlen:
        return (0, s[1], s[0]) if layout == "NHD" else (0, s[0], s[1])
    return (s[0], s[2], s[1]) if layout == "NHD" else (s[0], s[1], s[2])


def _check_shapes(q, k, v, o, layout, varlen):
    """Refuse, before any GPU call, tensors whose shapes, devices or dtypes do
    not describe one problem (the kernels would read or write out of bounds)."""
    nd = 3 if varlen else 4
    for name, t in (("q", q), ("k", k), ("v", v)) + ((("out", o),) if o is not None else ()):
        if t.dim() != nd:
            raise ValueError(f"{name} must have {nd} dimensions "
                             f"({'packed [T,H,d] / [H,T,d]' if varlen else '[B,H,N,d] / [B,N,H,d]'}),"
                             f" got {tuple(t.shape)}")
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v must have k's shape {tuple(k.shape)}, got {tuple(v.shape)}")
    if k.shape[-1] != q.shape[-1]:
        raise ValueError(f"q and k head dims differ ({q.shape[-1]} vs {k.shape[-1]})")
    if not varlen and k.shape[0] != q.shape[0]:
        raise ValueError(f"q and k batch sizes differ ({q.shape[0]} vs {k.shape[0]})")
    if o is not None and (tuple(o.shape) != tuple(q.shape) or o.dtype != q.dtype):
        raise ValueError(f"out must have q's shape {tuple(q.shape)} and dtype {q.dtype}, "
                         f"got {tuple(o.shape)} {o.dtype}")


def _check_devices(q, k, v, o):
    for name, t in (("q", q), ("k", k), ("v", v)) + ((("out", o),) if o is not None else ()):
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be on q's CUDA device ({q.device}), got {t.device}")


def _check_tokens(q, k, layout, cu_q, n_q, cu_k, n_k):
    """Varlen: the packed tensors must hold the tokens cu_seqlens names."""
    tq = q.shape[0] if layout == "NHD" else q.shape[1]
    tk = k.shape[0] if layout == "NHD" else k.shape[1]
    if n_q > 0 and cu_q[n_q] > tq:
        raise ValueError(f"cu_seqlens_q ends at {cu_q[n_q]} but q holds {tq} tokens")
    if n_k > 0 and cu_k[n_k] > tk:
        raise ValueError(f"cu_seqlens_kv ends at {cu_k[n_k]} but k and v hold {tk} tokens")


def make_desc(q, k, v, o=None, *, tensor_layout="HND", is_causal=False, smooth_q=False,
              smooth_k=True, smooth_v=False, sm_scale=None, varlen=False,
              pv_mode="fp8", kv_split=0, qk_block=64) -> _abi.Desc:
    """Descriptor for q/k/v torch tensors (dense [B,H,N,d] / [B,N,H,d], or packed
    varlen [T,H,d] / [H,T,d])."""
    if tensor_layout not in ("HND", "NHD"):
        raise ValueError(f"tensor_layout must be 'HND' or 'NHD', got {tensor_layout!r}")
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share dtype float16 or bfloat16")
    _check_shapes(q, k, v, o, tensor_layout, varlen)
    if pv_mode not in _abi.PV_MODES:
        raise ValueError(f"pv_mode must be 'fp8' or 'half', got {pv_mode!r}")
    d = _abi.Desc()
    lay = NHD if tensor_layout == "NHD" else HND
    hd = q.shape[-1]
    if varlen:
        hq = q.shape[1] if lay == NHD else q.shape[0]
        hkv = k.shape[1] if lay == NHD else k.shape[0]
        lib().sage_desc_init(ctypes.byref(d), _DT[q.dtype], lay, 0, hq, hkv, 0, 0, hd)
    else:
        B = q.shape[0]
        if lay == NHD:
            nq, hq, nkv, hkv = q.shape[1], q.shape[2], k.shape[1], k.shape[2]
        else:
            hq, nq, hkv, nkv = q.shape[1], q.shape[2], k.shape[1], k.shape[2]
        lib().sage_desc_init(ctypes.byref(d), _DT[q.dtype], lay, B, hq, hkv, nq, nkv, hd)
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o if o is not None else q)):
        arr = getattr(d, name)
        for i, x in enumerate(_strides(t, tensor_layout, varlen)):
            arr[i] = x
    d.is_causal = int(bool(is_causal))
    if smooth_q == "block":
        d.smooth_q = _abi.SMOOTH_Q_BLOCK
    elif smooth_q in (False, True, 0, 1, None):
        d.smooth_q = int(bool(smooth_q))
    else:
        raise ValueError(f"smooth_q must be False, True or 'block', got {smooth_q!r}")
    d.smooth_k = int(bool(smooth_k))
    d.smooth_v = int(bool(smooth_v))
    d.sm_scale = float(sm_scale) if sm_scale else 0.0
    d.pv_mode = _abi.PV_MODES[pv_mode]
    d.kv_split = _abi.KV_SPLIT_AUTO if kv_split == "auto" else int(kv_split)
    d.qk_block = int(qk_block)
    _check_devices(q, k, v, o)
    return d


def _cu(cu):
    if cu is None:
        return None, 0
    vals = [int(x) for x in (cu.tolist() if isinstance(cu, torch.Tensor) else cu)]
    arr = (ctypes.c_int32 * len(vals))(*vals)
    return arr, len(vals) - 1


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def kv_split_size(desc, cu_seqlens_q=None, cu_seqlens_kv=None) -> int:
    """Keys per split the library uses for this problem (0: no split)."""
    cq, n = _cu(cu_seqlens_q)
    ck, _ = _cu(cu_seqlens_kv)
    out = ctypes.c_int32(0)
    _abi.check("sage_kv_split_size",
               lib().sage_kv_split_size(ctypes.byref(desc), cq, ck, n, ctypes.byref(out)))
    return out.value


def workspace_size(desc, cu_seqlens_q=None, cu_seqlens_kv=None) -> int:
    cq, n = _cu(cu_seqlens_q)
    ck, _ = _cu(cu_seqlens_kv)
    out = ctypes.c_size_t(0)
    _abi.check("sage_workspace_size",
               lib().sage_workspace_size(ctypes.byref(desc), cq, ck, n, ctypes.byref(out)))
    return out.value


def quant_buf_sizes(desc, cu_seqlens_q=None, cu_seqlens_kv=None) -> dict:
    cq, n = _cu(cu_seqlens_q)
    ck, _ = _cu(cu_seqlens_kv)
    z = _abi.QuantSizes()
    _abi.check("sage_quant_buf_sizes",
               lib().sage_quant_buf_sizes(ctypes.byref(desc), cq, ck, n, ctypes.byref(z)))
    return {name: getattr(z, name) for name, _ in _abi.QuantSizes._fields_}


_BUF_DT = {"mu_q": torch.float32, "mu_k": torch.float32, "mu_v": torch.float32,
           "q_codes": torch.int8, "q_scale": torch.float32, "k_codes": torch.int8,
           "k_scale": torch.float32, "v_codes": torch.uint8, "v_scale": torch.float32,
           "delta_s": torch.float32, "mu_qb": torch.float32, "mu_q_code": torch.int8,
           "mu_q_cscale": torch.float32}


def sage_quant_qkv(q, k, v, *, tensor_layout="HND", is_causal=False, smooth_q=False,
                   smooth_k=True, smooth_v=False, sm_scale=None, cu_seqlens_q=None,
                   cu_seqlens_kv=None, bufs=None, pv_mode="fp8", kv_split=0, qk_block=64):
    """Run the pre-pass alone; returns a dict of flat device tensors laid out as
    documented for sage_quant_bufs in include/sage.h.  Passing the dict of an
    earlier call on the same problem as `bufs` reuses its buffers and
    workspace (nothing is allocated)."""
    varlen = cu_seqlens_q is not None
    desc = make_desc(q, k, v, tensor_layout=tensor_layout, is_causal=is_causal,
                     smooth_q=smooth_q, smooth_k=smooth_k, smooth_v=smooth_v,
                     sm_scale=sm_scale, varlen=varlen, pv_mode=pv_mode, kv_split=kv_split,
                     qk_block=qk_block)
    if bufs is None:
        sizes = quant_buf_sizes(desc, cu_seqlens_q, cu_seqlens_kv)
        bufs = {name: torch.zeros(max(1, nbytes // torch.empty((), dtype=_BUF_DT[name]).element_size()),
                                  dtype=_BUF_DT[name], device=q.device)
                for name, nbytes in sizes.items()}
        ws = torch.empty(workspace_size(desc, cu_seqlens_q, cu_seqlens_kv), dtype=torch.uint8,
                         device=q.device)
    else:
        sizes, ws = bufs["_sizes"], bufs["_workspace"]
        bufs = {name: bufs[name] for name in sizes}
    qb = _abi.QuantBufs(**{name: (t.data_ptr() if sizes[name] else None) for name, t in bufs.items()})
    cq, n = _cu(cu_seqlens_q)
    ck, nk = _cu(cu_seqlens_kv)
    if varlen:
        if nk != n:
            raise ValueError("cu_seqlens_q and cu_seqlens_kv must have the same length")
        _check_tokens(q, k, tensor_layout, cq, n, ck, nk)
    _abi.check("sage_quant_qkv",
               lib().sage_quant_qkv(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), cq, ck, n,
                                    ctypes.byref(qb), _ptr(ws), ws.numel(), _stream(q)))
    bufs["_desc"] = desc
    bufs["_workspace"] = ws
    bufs["_sizes"] = sizes
    bufs["_q_shape"] = (tuple(q.shape), q.dtype)
    return bufs


def quant_bufs_struct(bufs) -> _abi.QuantBufs:
    """ctypes sage_quant_bufs for a dict returned by sage_quant_qkv."""
    sizes = bufs["_sizes"]
    return _abi.QuantBufs(**{name: (bufs[name].data_ptr() if sizes[name] else None)
                             for name in sizes})


def sage_attn_fwd_quantized(bufs, out, *, cu_seqlens_q=None, cu_seqlens_kv=None, lse=None):
    """The fused kernel alone on buffers from sage_quant_qkv (same problem).
    `out` has q's shape and dtype; lse (optional) is FP32 as in sage_attn_fwd.
    A split key range keeps its partials in the workspace of the pre-pass
    call (sized by sage_workspace_size, which covers both)."""
    desc = bufs["_desc"]
    cq, n = _cu(cu_seqlens_q)
    ck, _ = _cu(cu_seqlens_kv)
    shape = bufs.get("_q_shape")
    if shape is not None and (tuple(out.shape) != shape[0] or out.dtype != shape[1]
                              or out.device != bufs["q_codes"].device):
        raise ValueError(f"out must have the quantized q's shape {shape[0]} and dtype "
                         f"{shape[1]} on its device")
    qb = quant_bufs_struct(bufs)
    ws = bufs["_workspace"]
    _abi.check("sage_attn_fwd_quantized",
               lib().sage_attn_fwd_quantized(ctypes.byref(desc), cq, ck, n, ctypes.byref(qb),
                                             _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
                                             _stream(out)))
    return out


def sage_debug_qk_int32(bufs, *, cu_seqlens_q=None, cu_seqlens_kv=None, device=None):
    """int32 Q.K^T of the codes produced by sage_quant_qkv (same desc)."""
    desc = bufs["_desc"]
    cq, n = _cu(cu_seqlens_q)
    ck, _ = _cu(cu_seqlens_kv)
    if cq is None:
        total = desc.batch * desc.hq * desc.nq * desc.nkv
    else:
        lq = [cq[i + 1] - cq[i] for i in range(n)]
        lk = [ck[i + 1] - ck[i] for i in range(n)]
        total = sum(desc.hq * a * b for a, b in zip(lq, lk))
    dev = device or bufs["q_codes"].device
    out = torch.empty(max(1, total), dtype=torch.int32, device=dev)
    qb = _abi.QuantBufs(q_codes=bufs["q_codes"].data_ptr(), k_codes=bufs["k_codes"].data_ptr())
    _abi.check("sage_debug_qk_int32",
               lib().sage_debug_qk_int32(ctypes.byref(desc), cq, ck, n, ctypes.byref(qb),
                                         _ptr(out), _stream(out)))
    return out[:total]


def sage_debug_e4m3_encode(first: int, count: int, out=None, device="cuda"):
    """E4M3 codes (uint8 device tensor of `count` bytes) of the FP32 values
    whose bit patterns are first .. first+count-1, converted by the library's
    own device conversion (test hook)."""
    if out is None:
        out = torch.empty(max(1, count), dtype=torch.uint8, device=device)
    elif out.dtype != torch.uint8 or not out.is_cuda or out.numel() < count:
        raise ValueError("out must be a CUDA uint8 tensor of at least count bytes")
    _abi.check("sage_debug_e4m3_encode",
               lib().sage_debug_e4m3_encode(ctypes.c_uint32(first), ctypes.c_uint32(count),
                                            _ptr(out), _stream(out)))
    return out[:count]


def sage_micro_rate(op: str, reps: int = 4096, device="cuda") -> float:
    """Measured rate of one execution unit on `device`: "i8" and "f8" matrix
    operations (2 per multiply-add) per second, "exp" results per second,
    "fma" flops per second (one timed launch after a warm-up; blocks)."""
    if op not in _abi.MICRO_OPS:
        raise ValueError(f"op must be one of {sorted(_abi.MICRO_OPS)}")
    dev = torch.device(device)
    rate = ctypes.c_double(0.0)
    with torch.cuda.device(dev):
        st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        _abi.check("sage_micro_rate",
                   lib().sage_micro_rate(_abi.MICRO_OPS[op], int(reps), ctypes.byref(rate), st))
    return rate.value


def sage_attn_fwd(q, k, v, *, tensor_layout="HND", is_causal=False, smooth_q=False,
                  smooth_k=True, smooth_v=False, sm_scale=None, return_lse=False,
                  out=None, workspace=None, pv_mode="fp8", kv_split=0, qk_block=64):
    """Dense forward pass.  Returns o (and lse [B, hq, nq] FP32 if asked)."""
    o = torch.empty_like(q) if out is None else out
    desc = make_desc(q, k, v, o, tensor_layout=tensor_layout, is_causal=is_causal,
                     smooth_q=smooth_q, smooth_k=smooth_k, smooth_v=smooth_v,
                     sm_scale=sm_scale, pv_mode=pv_mode, kv_split=kv_split,
                     qk_block=qk_block)
    lse = None
    if return_lse:
        lse = torch.empty((desc.batch, desc.hq, desc.nq), dtype=torch.float32, device=q.device)
    need = workspace_size(desc)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _abi.check("sage_attn_fwd",
               lib().sage_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(lse), _ptr(workspace), workspace.numel(), _stream(q)))
    return (o, lse) if return_lse else o


def sage_attn_fwd_noalloc(q, k, v, out, *, tensor_layout="HND", is_causal=False,
                          smooth_q=False, smooth_k=True, smooth_v=False, sm_scale=None,
                          lse=None, pv_mode="fp8", kv_split=0, qk_block=64):
    """Dense forward pass into the caller's `out` (and optional FP32 `lse`
    [B, hq, nq]) with the library's own static workspace: the call allocates
    nothing, on the device or through torch (for code that cannot).  Calls
    that overlap on one GPU race (they share its workspace)."""
    desc = make_desc(q, k, v, out, tensor_layout=tensor_layout, is_causal=is_causal,
                     smooth_q=smooth_q, smooth_k=smooth_k, smooth_v=smooth_v,
                     sm_scale=sm_scale, pv_mode=pv_mode, kv_split=kv_split,
                     qk_block=qk_block)
    _abi.check("sage_attn_fwd_noalloc",
               lib().sage_attn_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(out), _ptr(lse), _stream(q)))
    return out


def sage_attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_kv, *, tensor_layout="NHD",
                         is_causal=False, smooth_q=False, smooth_k=True, smooth_v=False,
                         sm_scale=None, return_lse=False, out=None, workspace=None,
                         pv_mode="fp8", kv_split=0, qk_block=64):
    """Packed variable-length forward pass (q [T,H,d] for NHD or [H,T,d] for
    HND; cu_seqlens are host int32 prefix offsets).  lse is [hq, T_q]."""
    o = torch.empty_like(q) if out is None else out
    desc = make_desc(q, k, v, o, tensor_layout=tensor_layout, is_causal=is_causal,
                     smooth_q=smooth_q, smooth_k=smooth_k, smooth_v=smooth_v,
                     sm_scale=sm_scale, varlen=True, pv_mode=pv_mode, kv_split=kv_split,
                     qk_block=qk_block)
    cq, n = _cu(cu_seqlens_q)
    ck, nk = _cu(cu_seqlens_kv)
    if nk != n:
        raise ValueError("cu_seqlens_q and cu_seqlens_kv must have the same length")
    _check_tokens(q, k, tensor_layout, cq, n, ck, nk)
    lse = None
    if return_lse:
        tq = cq[n] if n > 0 else 0
        lse = torch.empty((desc.hq, tq), dtype=torch.float32, device=q.device)
    need = workspace_size(desc, cu_seqlens_q, cu_seqlens_kv)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _abi.check("sage_attn_fwd_varlen",
               lib().sage_attn_fwd_varlen(ctypes.byref(desc), cq, ck, n, _ptr(q), _ptr(k),
                                          _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                                          workspace.numel(), _stream(q)))
    return (o, lse) if return_lse else o


def sageattn(q, k, v, tensor_layout="HND", is_causal=False, smooth_k=True, sm_scale=None,
             smooth_q=False, smooth_v=False, return_lse=False, pv_mode="fp8", kv_split=0,
             qk_block=64):
    """The package page's call: attention output of the quantized forward pass."""
    return sage_attn_fwd(q, k, v, tensor_layout=tensor_layout, is_causal=is_causal,
                         smooth_q=smooth_q, smooth_k=smooth_k, smooth_v=smooth_v,
                         sm_scale=sm_scale, return_lse=return_lse, pv_mode=pv_mode,
                         kv_split=kv_split, qk_block=qk_block)


def sdpa(query, key, value, attn_mask=None, dropout_p=0.0, is_causal=False, scale=None,
         enable_gqa=False):
    """Drop-in for torch.nn.functional.scaled_dot_product_attention (the
    package page, "What it is and what it does": a drop-in replacement for
    scaled_dot_product_attention).  Tensors are [B, H, N, d] (HND), fp16 or
    bf16, d in {64, 96, 128}; GQA needs enable_gqa=True, as in torch.  What
    the quantized method cannot honour raises ValueError before any GPU
    call: an attention mask, dropout, and a causal mask when Nq != Nkv (torch
    aligns it top-left; this library bottom-right)."""
    if attn_mask is not None:
        raise ValueError("sdpa: attn_mask is not supported (only is_causal)")
    if dropout_p:
        raise ValueError("sdpa: dropout is not supported (inference only)")
    if query.dim() != 4 or key.dim() != 4 or value.dim() != 4:
        raise ValueError("sdpa: expects [B, H, N, d] tensors")
    if key.shape[1] != query.shape[1] and not enable_gqa:
        raise ValueError("sdpa: query and key head counts differ; pass enable_gqa=True")
    if is_causal and query.shape[2] != key.shape[2]:
        raise ValueError("sdpa: is_causal with Nq != Nkv aligns top-left in torch; "
                         "use sageattn (bottom-right) instead")
    return sage_attn_fwd(query, key, value, tensor_layout="HND", is_causal=is_causal,
                         sm_scale=scale)
