"""GPU parity on seeded random problem shapes and options, through the C ABI.

Each case draws, from a fixed seed: dtype, layout, head dim, GQA group, batch
or varlen lengths (empty sequences included; a quarter of the dense cases
have 1-4 queries against up to 1,200 keys), causal, the smoothing flags,
the P.V mode, the Q/K block and the key split (none, explicit or automatic).
It then checks, against the oracle on the same seeded inputs:

* the pre-pass bit for bit (means, codes, scales; the score bias to FP32
  rounding);
* the output within max-abs 2e-2 (beyond the oracle's rounding-tie bound:
  P codes whose p sits at a rounding midpoint may round either way) and
  cosine 0.999 of the same-recipe oracle, and cosine 0.99 of exact FP64
  attention;
* the LSE against the oracle's.

A second set of 64 cases (seeds of their own) draws the same way and then
smooths Q per quantization block (FP8 P.V), with a Q offset that drifts
along the sequence.

A third set of 64 cases (seeds of their own) draws the same way and then
scales Q and K by 10^u (u uniform in [-5, 2.3] for fp16, [-38, 2.3] for
bf16: from subnormal inputs to row maxima near 2^18 in log2 units, inside
the recipe's range) and, in about a third of them, V by 10^u' (u' in
[-3, 3], or [-38, 3] for bf16, down to where V's channels count as zero).
The comparison with exact FP64 attention is kept where the logits are at
most 4 times their seeded size and V is above 10^-20: larger logits make
rows nearly one-hot, where INT8 Q.K^T need not keep the exact ranking, and
V below 2^-100 per channel is flushed by the recipe's E4M3 quantizer.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as orc
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

NCASES = 256
NBLOCK = 64
NSCALE = 64


def _draw(i: int):
    if i >= NCASES + NBLOCK:
        import dataclasses
        w, pv, qb, split = _draw_plain(7000 + i)
        return dataclasses.replace(w, name=f"fuzz{i}"), pv, qb, split
    if i >= NCASES:
        # per-block Q smoothing: a case of its own seed with that mode
        w, _, qb, split = _draw_plain(5000 + i)
        import dataclasses
        return dataclasses.replace(w, name=f"fuzz{i}", smooth_q="block",
                                   q_drift_sigma=1.5), "fp8", qb, split
    return _draw_plain(i)


def _draw_plain(i: int):
    rng = np.random.default_rng(1000 + i)
    d = int(rng.choice([64, 96, 128]))
    hkv = int(rng.choice([1, 2, 3]))
    g = int(rng.choice([1, 2, 3, 4, 8]))
    varlen = bool(rng.random() < 0.3)
    common = dict(name=f"fuzz{i}", dtype=str(rng.choice(["f16", "bf16"])),
                  layout=str(rng.choice(["HND", "NHD"])), Hq=hkv * g, Hkv=hkv, d=d,
                  causal=bool(rng.random() < 0.5), smooth_q=bool(rng.random() < 0.3),
                  smooth_k=bool(rng.random() < 0.8), smooth_v=bool(rng.random() < 0.3),
                  seed=50 + i, k_off_sigma=2.0, qv_mean_sigma=1.0)
    if varlen:
        n = int(rng.integers(1, 4))
        lq = [int(x) for x in rng.integers(0, 300, n)]
        lk = [int(x) for x in rng.integers(0, 400, n)]
        lq[0] = max(lq[0], 1)
        lk[0] = max(lk[0], 1)
        if n > 1 and i % 2 == 0:
            lq[-1] = 0                       # an empty sequence
        w = synth.Workload(B=n, Nq=0, Nkv=0, seqlens_q=lq, seqlens_kv=lk, **common)
    else:
        if rng.random() < 0.25:              # few queries, longer keys (decode)
            nq = int(rng.integers(1, 5))
            nkv = int(rng.integers(200, 1200))
        else:
            nq = int(rng.integers(1, 300))
            nkv = int(rng.integers(1, 400))
        w = synth.Workload(B=int(rng.integers(1, 3)), Nq=nq, Nkv=nkv, **common)
    pv = str(rng.choice(["fp8", "half"]))
    qb = int(rng.choice([64, 32]))
    split = rng.choice([0, 128, 256, -1])
    split = "auto" if split == -1 else int(split)
    return w, pv, qb, split


def _magnitudes(i: int, w):
    """(Q and K factor, V factor) of a case of the third set, else (1, 1)."""
    if i < NCASES + NBLOCK:
        return 1.0, 1.0
    r = np.random.default_rng(123000 + i)
    fqk = 10.0 ** float(r.uniform(-5, 2.3) if w.dtype == "f16" else r.uniform(-38, 2.3))
    fv = 1.0
    if r.random() < 0.3:
        fv = 10.0 ** float(r.uniform(-3, 3) if w.dtype == "f16" else r.uniform(-38, 3))
    return fqk, fv


def _kw(w, pv, qb, split):
    return dict(tensor_layout=w.layout, is_causal=w.causal, smooth_q=w.smooth_q,
                smooth_k=w.smooth_k, smooth_v=w.smooth_v, sm_scale=w.sm_scale, pv_mode=pv,
                qk_block=qb, kv_split=split)


@pytest.mark.parametrize("i", range(NCASES + NBLOCK + NSCALE))
def test_fuzz_case(i):
    w, pv, qb, split = _draw(i)
    fqk, fv = _magnitudes(i, w)
    pu.say(f"[fuzz {i}] pv={pv} qk_block={qb} kv_split={split} qk x{fqk:.3g} v x{fv:.3g} {w}")
    q, k, v, meta = pu.gpu_inputs(w)
    if fqk != 1.0 or fv != 1.0:
        q = (q.float() * fqk).to(q.dtype)
        k = (k.float() * fqk).to(k.dtype)
        v = (v.float() * fv).to(v.dtype)
    exact = fqk <= 2.0 and fv >= 1e-20
    kw = _kw(w, pv, qb, split)
    cu = {}
    if w.varlen:
        cu = dict(cu_seqlens_q=meta["cu_seqlens_q"], cu_seqlens_kv=meta["cu_seqlens_kv"])
    desc = pu.qa.make_desc(q, k, v, varlen=w.varlen, **{a: b for a, b in kw.items()})
    eff = pu.qa.kv_split_size(desc, cu.get("cu_seqlens_q"), cu.get("cu_seqlens_kv"))
    prob = orc.problem_from_workload(w, pv, eff, qb)
    qh, kh, vh = pu.u16(q), pu.u16(k), pu.u16(v)
    ref = orc.prepass(prob, qh, kh, vh)

    bufs = pu.qa.sage_quant_qkv(q, k, v, **kw, **cu)
    torch.cuda.synchronize()
    gpu_pre, pads_ok = pu.unpack_quant(w, bufs, pv, qb)
    assert pads_ok
    pu.assert_prepass_equal(gpu_pre, ref, w)

    if w.varlen:
        o, lse = pu.qa.sage_attn_fwd_varlen(q, k, v, cu["cu_seqlens_q"], cu["cu_seqlens_kv"],
                                            return_lse=True, **kw)
    else:
        o, lse = pu.qa.sage_attn_fwd(q, k, v, return_lse=True, **kw)
    torch.cuda.synchronize()
    got = pu.gpu_out_per_seq(w, o, meta)
    rec, rec_lse, tie = orc.forward_rows(prob, ref, bkv=pu.KVT, tie=True)
    ex, _ = orc.exact_rows(prob, qh, kh, vh)
    lse_h = lse.cpu().numpy()
    for si, (nq, nkv) in enumerate(w.seq_lens()):
        g, r, e = got[si], rec[si], ex[si]
        if g.size == 0:
            continue
        assert np.all(np.isfinite(g))
        err = pu.max_excess(g, r, w.dtype, tie[si])
        assert err <= 2e-2, (si, err)
        if np.abs(r).max() > 0:
            assert pu.cos(g, r) >= 0.999, (si, pu.cos(g, r))
            if exact:
                assert pu.cos(g, e) >= 0.99, (si, pu.cos(g, e))
        if w.varlen:
            t0 = meta["cu_seqlens_q"][si]
            gl = lse_h[:, t0:t0 + nq]
        else:
            gl = lse_h[si]
        fin = np.isfinite(rec_lse[si])
        assert np.array_equal(np.isfinite(gl), fin)
        if fin.any():
            tol = 2e-3 * max(1.0, np.abs(rec_lse[si][fin]).max())
            assert np.abs(gl[fin] - rec_lse[si][fin]).max() < tol
