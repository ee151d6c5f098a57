"""Helpers of the GPU parity tests: run the HIP library through its binding,
unpack its quantized buffers (layout documented in include/sage.h) into the
oracle's logical per-(sequence, head) arrays, and compare."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import quantized_attention_03_amd as qa
import synth
from oracle import oracle as orc

KVT, QB = qa.KV_TILE, qa.QK_BLOCK


def say(*a):
    """Name the case before any GPU step (flushed, so a fault still shows it)."""
    print(*a, flush=True)
    sys.stdout.flush()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def gpu_inputs(w: synth.Workload):
    """Seeded inputs generated on the GPU (fast at full size) plus their bytes on
    the host for the oracle: both sides see the same bits."""
    q, k, v, meta = synth.make_inputs(w, device="cuda")
    return q, k, v, meta


def run_quant(w, q, k, v, meta, pv="fp8", qb=64):
    kw = dict(tensor_layout=w.layout, is_causal=w.causal, smooth_q=w.smooth_q,
              smooth_k=w.smooth_k, smooth_v=w.smooth_v, sm_scale=w.sm_scale, pv_mode=pv,
              qk_block=qb)
    if w.varlen:
        kw.update(cu_seqlens_q=meta["cu_seqlens_q"], cu_seqlens_kv=meta["cu_seqlens_kv"])
    return qa.sage_quant_qkv(q, k, v, **kw)


def run_fwd(w, q, k, v, meta, return_lse=True, pv="fp8", qb=64):
    kw = dict(tensor_layout=w.layout, is_causal=w.causal, smooth_q=w.smooth_q,
              smooth_k=w.smooth_k, smooth_v=w.smooth_v, sm_scale=w.sm_scale,
              return_lse=return_lse, pv_mode=pv, qk_block=qb)
    if w.varlen:
        return qa.sage_attn_fwd_varlen(q, k, v, meta["cu_seqlens_q"], meta["cu_seqlens_kv"], **kw)
    return qa.sage_attn_fwd(q, k, v, **kw)


def _pad(x, m):
    return (x + m - 1) // m * m


def unpack_quant(w, bufs, pv="fp8", qb=64):
    """GPU buffers -> oracle.Prepass-shaped lists (numpy), plus pad checks.
    With pv = "half" the V operand is 16-bit (uint16 patterns), unscaled."""
    seqs = w.seq_lens()
    hq, hkv, d = w.Hq, w.Hkv, w.d
    host = {k: v.cpu().numpy() for k, v in bufs.items() if not k.startswith("_")}
    R = orc.Prepass()
    rq = rk = 0
    pads_ok = True
    for s, (nq, nkv) in enumerate(seqs):
        npq, npk = _pad(nq, QB), _pad(nkv, KVT)
        qc = host["q_codes"][rq * hq * d:(rq * hq + hq * npq) * d].reshape(hq, npq, d)
        qs = host["q_scale"][rq * hq // qb:(rq * hq + hq * npq) // qb].reshape(hq, npq // qb)
        kc = host["k_codes"][rk * hkv * d:(rk * hkv + hkv * npk) * d].reshape(hkv, npk, d)
        ks = host["k_scale"][rk * hkv // qb:(rk * hkv + hkv * npk) // qb].reshape(hkv, npk // qb)
        vall = host["v_codes"].view(np.uint16) if pv == "half" else host["v_codes"]
        vc = vall[rk * hkv * d:(rk * hkv + hkv * npk) * d].reshape(hkv, d, npk)
        pads_ok &= not qc[:, nq:].any() and not kc[:, nkv:].any() and not vc[:, :, nkv:].any()
        pads_ok &= not ks[:, -(-nkv // qb):].any()
        R.qc.append(qc[:, :nq])
        R.qs.append(qs[:, :-(-nq // qb)])
        R.kc.append(kc[:, :nkv])
        R.ks.append(ks[:, :-(-nkv // qb)])
        R.vc.append(vc.transpose(0, 2, 1)[:, :nkv])
        R.vs.append(None if pv == "half" else host["v_scale"].reshape(-1, hkv, d)[s])
        R.mu_q.append(host["mu_q"].reshape(-1, hq, d)[s] if w.smooth_q else None)
        R.mu_k.append(host["mu_k"].reshape(-1, hkv, d)[s] if w.smooth_k else None)
        R.mu_v.append(host["mu_v"].reshape(-1, hkv, d)[s] if w.smooth_v else None)
        blockwise = w.smooth_q == "block"
        if w.smooth_q:
            ds = host["delta_s"][rk * hq:rk * hq + hq * npk].reshape(hq, npk)
            # per-block smoothing: the buffer holds the sequence mean's share;
            # the blocks' compensations are formed inside the fused kernel
            (R.ds_seq if blockwise else R.ds).append(ds[:, :nkv])
            (R.ds if blockwise else R.ds_seq).append(None)
        else:
            R.ds.append(None)
            R.ds_seq.append(None)
        if blockwise:
            nb, nbp = -(-nq // qb), npq // qb
            b0 = rq * hq // qb
            mub = host["mu_qb"][b0 * d:(b0 + hq * nbp) * d].reshape(hq, nbp, d)
            code = host["mu_q_code"][b0 * 2 * d:(b0 + hq * nbp) * 2 * d].reshape(hq, nbp, 2, d)
            csc = host["mu_q_cscale"][b0:b0 + hq * nbp].reshape(hq, nbp)
            pads_ok &= not mub[:, nb:].any() and not code[:, nb:].any() and not csc[:, nb:].any()
            R.mu_qb.append(mub[:, :nb])
            R.mu_code.append(code[:, :nb])
            R.mu_cscale.append(csc[:, :nb])
        else:
            R.mu_qb.append(None)
            R.mu_code.append(None)
            R.mu_cscale.append(None)
        rq += npq
        rk += npk
    return R, pads_ok


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_prepass_equal(gpu: orc.Prepass, ref: orc.Prepass, w):
    for name in ("mu_q", "mu_k", "mu_v", "qc", "qs", "kc", "ks", "vc", "vs", "mu_qb", "mu_code",
                 "mu_cscale"):
        for s, (g, r) in enumerate(zip(getattr(gpu, name), getattr(ref, name))):
            if r is None:
                assert g is None, name
                continue
            assert g.shape == r.shape, (name, s, g.shape, r.shape)
            if not np.array_equal(bits(g), bits(r)):
                bad = np.argwhere(bits(g) != bits(r))
                raise AssertionError(f"{name}[seq {s}] differs at {len(bad)} places, first "
                                     f"{bad[:3].tolist()}: gpu {g[tuple(bad[0])]} ref {r[tuple(bad[0])]}")
    blockwise = w.smooth_q == "block"
    for s, (g, r) in enumerate(zip(gpu.ds_seq if blockwise else gpu.ds,
                                   ref.ds_seq if blockwise else ref.ds)):
        if r is not None:
            assert g.shape == r.shape, ("ds", s, g.shape, r.shape)
            if r.size:
                np.testing.assert_allclose(g, r, rtol=1e-5, atol=1e-5 * np.abs(r).max())


def half_ulp(x, dtype: str):
    """Half an ulp of the output dtype at |x| (the last step of both sides is a
    round-to-nearest-even into that dtype, worth up to this much)."""
    mant = 7 if dtype == "bf16" else 10
    emin = -126 if dtype == "bf16" else -14
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), np.finfo(np.float64).tiny)
    e = np.maximum(np.floor(np.log2(ax)), emin)
    return np.exp2(e - mant) / 2


def max_excess(g, r, dtype: str, tie=None) -> float:
    """max |g - r| beyond the final output rounding (g: decoded GPU output,
    r: the oracle's FP32 result before that rounding) and, with tie (the
    oracle's rounding-tie bound, forward_rows(tie=True)), beyond what the
    P-operand codes that sit at a rounding midpoint can move each element."""
    if np.size(g) == 0:
        return 0.0
    d = np.abs(np.asarray(g, np.float64) - np.asarray(r, np.float64)) - half_ulp(r, dtype)
    if tie is not None:
        d = d - np.asarray(tie, np.float64)
    return float(np.max(np.maximum(d, 0.0)))


def cos(a, b):
    a, b = np.ravel(a).astype(np.float64), np.ravel(b).astype(np.float64)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def gpu_out_per_seq(w, o: torch.Tensor, meta):
    """Output tensor -> list over sequences of [Hq, nq, d] FP32 (decoded)."""
    prob = orc.problem_from_workload(w)
    parts = orc.split_heads(prob, u16(o), "q")
    return [orc.decode16(p, w.dtype) for p in parts]


def sample_rows(nq: int, k: int, seed: int):
    if nq <= k:
        return np.arange(nq)
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, nq - 65, nq - 64, nq - 2, nq - 1]
    fixed = [x for x in fixed if 0 <= x < nq]
    rest = rng.choice(nq, size=k - len(fixed), replace=False)
    return np.unique(np.concatenate([fixed, rest]))
