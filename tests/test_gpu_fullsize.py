"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one sage_attn_fwd / sage_attn_fwd_varlen call).

* The whole pre-pass (every channel mean, INT8 code and scale, E4M3 code and
  scale) is compared bit for bit with the oracle's.
* The output is compared on sampled query rows of every head (rows the oracle
  can compute one by one): the block and tile edges, the first and last rows,
  and seeded random rows.  Bars as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import oracle as orc
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

ROWS = 24


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_full_size(name):
    w = synth.WORKLOADS[name]
    pu.say(f"[full size {name}] generating inputs")
    q, k, v, meta = pu.gpu_inputs(w)
    prob = orc.problem_from_workload(w)
    qh, kh, vh = pu.u16(q), pu.u16(k), pu.u16(v)

    pu.say(f"[full size {name}] pre-pass")
    bufs = pu.run_quant(w, q, k, v, meta)
    torch.cuda.synchronize()
    gpu_pre, pads_ok = pu.unpack_quant(w, bufs)
    del bufs
    ref = orc.prepass(prob, qh, kh, vh)
    assert pads_ok
    pu.assert_prepass_equal(gpu_pre, ref, w)
    del gpu_pre

    pu.say(f"[full size {name}] forward")
    o, lse = pu.run_fwd(w, q, k, v, meta)
    torch.cuda.synchronize()
    got = pu.gpu_out_per_seq(w, o, meta)
    rows = [pu.sample_rows(nq, ROWS, 100 + s) for s, (nq, _) in enumerate(w.seq_lens())]
    rec, _, tie = orc.forward_rows(prob, ref, rows=rows, bkv=pu.KVT, tie=True)
    ex, _ = orc.exact_rows(prob, qh, kh, vh, rows=rows)
    for s in range(len(rows)):
        g = got[s][:, rows[s]]
        err = pu.max_excess(g, rec[s], w.dtype, tie[s])
        pu.say(f"  seq {s}: rows {len(rows[s])} max_excess {err:.4g} cos_recipe "
               f"{pu.cos(g, rec[s]):.6f} cos_fp64 {pu.cos(g, ex[s]):.6f}")
        assert np.all(np.isfinite(g))
        assert err <= 2e-2
        assert pu.cos(g, rec[s]) >= 0.999
        assert pu.cos(g, ex[s]) >= 0.99
