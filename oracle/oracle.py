"""Python driver of the CPU oracle (sage_oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares nothing with the HIP library: it loads its own
shared object (built from sage_oracle.c with gcc) and works on numpy arrays.

The per-(sequence, head) functions of the C file do all the arithmetic; this
module only slices the caller's tensors into per-(sequence, head) [N, d]
arrays, calls them, and gathers the results.  Layouts: HND = [B, H, N, d],
NHD = [B, N, H, d]; variable-length inputs are packed over the sequences as
[T, H, d] (NHD) or [H, T, d] (HND) with int32 prefix offsets cu_seqlens.
GQA: query head h reads key/value head h // (Hq // Hkv).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sage_oracle.c")
_SO = os.path.join(_HERE, "libsage_oracle.so")
BLK = 64          # Q/K quantization block (tokens)
P_SCALE = 448.0   # static P scale before the e4m3 rounding

_lib = None


def build() -> str:
    """Compile the oracle with gcc (plain C, no contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", _SRC, "-lm", "-o", _SO + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build()
    L = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
    sig = {
        "orc_f16_decode": (f32, [ctypes.c_uint16]),
        "orc_f16_encode": (ctypes.c_uint16, [f32]),
        "orc_bf16_decode": (f32, [ctypes.c_uint16]),
        "orc_bf16_encode": (ctypes.c_uint16, [f32]),
        "orc_e4m3_decode": (f32, [ctypes.c_uint8]),
        "orc_e4m3_encode_sat": (ctypes.c_uint8, [f32]),
        "orc_decode16": (None, [P, P, i64, i32]),
        "orc_encode16": (None, [P, P, i64, i32]),
        "orc_decode_e4m3": (None, [P, P, i64]),
        "orc_encode_e4m3": (None, [P, P, i64]),
        "orc_channel_mean": (None, [P, i64, i32, P]),
        "orc_smooth": (None, [P, P, i64, i32, P]),
        "orc_quant_int8_blocks": (None, [P, i64, i32, i32, P, P]),
        "orc_quant_fp8_channels": (None, [P, i64, i32, P, P]),
        "orc_delta_s": (None, [P, P, i64, i32, P]),
        "orc_block_mean": (None, [P, i64, i32, i32, P]),
        "orc_smooth_blocks": (None, [P, P, i64, i32, i32, P]),
        "orc_mu_code": (None, [P, i32, P, P, P]),
        "orc_delta_s_block": (None, [P, P, P, f32, P, P, i64, i32, i32, P]),
        "orc_qk_int32": (None, [P, P, i64, i64, i32, P]),
        "orc_attn_recipe_rows": (None, [P, P, P, P, P, P, P, P, i64, i64, i32, f32,
                                        i32, i32, i32, i64, P, i64, P, P, P]),
        "orc_attn_recipe_rows_blockds": (None, [P, P, P, P, P, P, P, i64, P, i64, i64, i32, f32,
                                                i32, i32, i32, i64, P, i64, P, P, P]),
        "orc_attn_recipe_half_rows": (None, [P, P, P, P, P, i32, P, P, i64, i64, i32, f32,
                                             i32, i32, i32, i64, P, i64, P, P, P]),
        "orc_attn_exact_rows": (None, [P, P, P, i64, i64, i32, f64, i32, P, i64, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------- codecs ---

def decode16(x, dtype: str) -> np.ndarray:
    """fp16 / bf16 bit patterns (uint16) -> exact FP32."""
    x = _c(x, np.uint16)
    out = np.empty(x.shape, np.float32)
    lib().orc_decode16(_p(x), _p(out), x.size, 1 if dtype == "bf16" else 0)
    return out


def encode16(x, dtype: str) -> np.ndarray:
    """FP32 -> fp16 / bf16 bit patterns, round to nearest even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_encode16(_p(x), _p(out), x.size, 1 if dtype == "bf16" else 0)
    return out


def e4m3_decode(b) -> np.ndarray:
    b = _c(b, np.uint8)
    out = np.empty(b.shape, np.float32)
    lib().orc_decode_e4m3(_p(b), _p(out), b.size)
    return out


def e4m3_encode(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_encode_e4m3(_p(x), _p(out), x.size)
    return out


# ------------------------------------------------------- per-head steps ---

def channel_mean(x) -> np.ndarray:
    x = _c(x, np.float32)
    n, d = x.shape
    mu = np.empty(d, np.float32)
    lib().orc_channel_mean(_p(x), n, d, _p(mu))
    return mu


def smooth(x, mu) -> np.ndarray:
    x = _c(x, np.float32)
    n, d = x.shape
    out = np.empty_like(x)
    lib().orc_smooth(_p(x), _p(None if mu is None else _c(mu, np.float32)), n, d, _p(out))
    return out


def quant_int8_blocks(xs, blk: int = BLK):
    xs = _c(xs, np.float32)
    n, d = xs.shape
    codes = np.empty((n, d), np.int8)
    scales = np.empty(max(1, -(-n // blk)), np.float32)
    lib().orc_quant_int8_blocks(_p(xs), n, d, blk, _p(codes), _p(scales))
    return codes, scales[: -(-n // blk)]


def quant_fp8_channels(vs):
    vs = _c(vs, np.float32)
    n, d = vs.shape
    codes = np.empty((n, d), np.uint8)
    scales = np.empty(d, np.float32)
    lib().orc_quant_fp8_channels(_p(vs), n, d, _p(codes), _p(scales))
    return codes, scales


def delta_s(mu_q, ks) -> np.ndarray:
    ks = _c(ks, np.float32)
    n, d = ks.shape
    out = np.empty(n, np.float32)
    lib().orc_delta_s(_p(_c(mu_q, np.float32)), _p(ks), n, d, _p(out))
    return out


def block_mean(x, blk: int = BLK) -> np.ndarray:
    """Channel means of each `blk`-token block (sage_oracle.c, orc_block_mean)."""
    x = _c(x, np.float32)
    n, d = x.shape
    nb = -(-n // blk)
    mu = np.empty((max(1, nb), d), np.float32)
    lib().orc_block_mean(_p(x), n, d, blk, _p(mu))
    return mu[:nb]


def smooth_blocks(x, mu, blk: int = BLK) -> np.ndarray:
    x = _c(x, np.float32)
    n, d = x.shape
    out = np.empty_like(x)
    lib().orc_smooth_blocks(_p(x), _p(_c(mu, np.float32)), n, d, blk, _p(out))
    return out


def mu_code(x):
    """(hi, lo, scale) of one block-mean deviation vector (orc_mu_code)."""
    x = _c(x, np.float32)
    d = x.shape[0]
    hi, lo = np.empty(d, np.int8), np.empty(d, np.int8)
    sc = np.empty(1, np.float32)
    lib().orc_mu_code(_p(x), d, _p(hi), _p(lo), _p(sc))
    return hi, lo, np.float32(sc[0])


def delta_s_block(ds_seq, hi, lo, scale, kc, ks, blk: int = BLK) -> np.ndarray:
    """Score compensation of one Q block (orc_delta_s_block)."""
    kc = _c(kc, np.int8)
    n, d = kc.shape
    out = np.empty(max(1, n), np.float32)
    lib().orc_delta_s_block(_p(None if ds_seq is None else _c(ds_seq, np.float32)),
                            _p(_c(hi, np.int8)), _p(_c(lo, np.int8)), float(scale), _p(kc),
                            _p(_c(ks, np.float32)), n, d, blk, _p(out))
    return out[:n]


def qk_int32(qc, kc) -> np.ndarray:
    qc, kc = _c(qc, np.int8), _c(kc, np.int8)
    nq, d = qc.shape
    nkv = kc.shape[0]
    s = np.empty((nq, nkv), np.int32)
    lib().orc_qk_int32(_p(qc), _p(kc), nq, nkv, d, _p(s))
    return s


def attn_recipe_rows(qc, qs, kc, ks, vc, vs, ds, mu_v, sm_scale, causal, bkv, rows, split=0,
                     blk=BLK, tie=False, ds_rows=0):
    """The INT8-QK / FP8-PV recipe for selected rows.  Returns (out, lse), and
    with tie=True also the rounding-tie bound [nrows, d] (sage_oracle.c).
    ds_rows > 0: ds is [Q blocks, nkv], one compensation per ds_rows rows."""
    qc, kc, vc = _c(qc, np.int8), _c(kc, np.int8), _c(vc, np.uint8)
    nq, d = qc.shape
    nkv = kc.shape[0]
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, d), np.float32)
    lse = np.empty(rows.size, np.float32)
    tb = np.empty((rows.size, d), np.float32) if tie else None
    dsp = _p(None if ds is None else _c(ds, np.float32))
    args = (_p(qc), _p(_c(qs, np.float32)), _p(kc), _p(_c(ks, np.float32)), _p(vc),
            _p(_c(vs, np.float32)))
    tail = (_p(None if mu_v is None else _c(mu_v, np.float32)), nq, nkv, d,
            float(sm_scale), int(causal), int(bkv), int(blk), int(split), _p(rows), rows.size,
            _p(out), _p(lse), _p(tb))
    if ds_rows:
        lib().orc_attn_recipe_rows_blockds(*args, dsp, int(ds_rows), *tail)
    else:
        lib().orc_attn_recipe_rows(*args, dsp, *tail)
    return (out, lse, tb) if tie else (out, lse)


def attn_recipe_half_rows(qc, qs, kc, ks, vh, dtype, ds, mu_v, sm_scale, causal, bkv, rows,
                          split=0, blk=BLK, tie=False):
    """The 16-bit P.V variant: vh [nkv, d] fp16/bf16 bit patterns of the V
    operand; p^ is p rounded to the same type."""
    qc, kc, vh = _c(qc, np.int8), _c(kc, np.int8), _c(vh, np.uint16)
    nq, d = qc.shape
    nkv = kc.shape[0]
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, d), np.float32)
    lse = np.empty(rows.size, np.float32)
    tb = np.empty((rows.size, d), np.float32) if tie else None
    lib().orc_attn_recipe_half_rows(
        _p(qc), _p(_c(qs, np.float32)), _p(kc), _p(_c(ks, np.float32)), _p(vh),
        1 if dtype == "bf16" else 0, _p(None if ds is None else _c(ds, np.float32)),
        _p(None if mu_v is None else _c(mu_v, np.float32)), nq, nkv, d,
        float(sm_scale), int(causal), int(bkv), int(blk), int(split), _p(rows), rows.size,
        _p(out), _p(lse), _p(tb))
    return (out, lse, tb) if tie else (out, lse)


def attn_exact_rows(q, k, v, sm_scale, causal, rows):
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    nq, d = q.shape
    nkv = k.shape[0]
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, d), np.float64)
    lse = np.empty(rows.size, np.float64)
    lib().orc_attn_exact_rows(_p(q), _p(k), _p(v), nq, nkv, d, float(sm_scale), int(causal),
                              _p(rows), rows.size, _p(out), _p(lse))
    return out, lse


# ------------------------------------------------------- whole problems ---

@dataclass
class Problem:
    """What one forward call computes (mirrors the library's descriptor)."""
    dtype: str                  # "f16" | "bf16"
    layout: str                 # "HND" | "NHD"
    Hq: int
    Hkv: int
    d: int
    seqs: list                  # [(nq, nkv)] per sequence (B entries)
    varlen: bool = False
    causal: bool = False
    smooth_q: bool | str = False   # False, True (one mean per sequence) or "block"
    smooth_k: bool = True
    smooth_v: bool = False
    sm_scale: float | None = None
    pv_mode: str = "fp8"        # "fp8" (SageAttention2) | "half" (16-bit P.V)
    kv_split: int = 0           # keys per split of the key range (0: one split)
    qk_block: int = BLK         # tokens per Q/K quantization block (64, or 32)

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale else 1.0 / math.sqrt(self.d)


def problem_from_workload(w, pv_mode: str = "fp8", kv_split: int = 0,
                          qk_block: int = BLK) -> Problem:
    return Problem(w.dtype, w.layout, w.Hq, w.Hkv, w.d, w.seq_lens(), w.varlen, w.causal,
                   w.smooth_q, w.smooth_k, w.smooth_v, w.sm_scale, pv_mode, kv_split, qk_block)


def split_heads(prob: Problem, x, which: str):
    """Physical tensor (uint16 bit patterns) -> list over sequences of
    [H, N, d] uint16 arrays in logical order."""
    x = np.asarray(x)
    out = []
    if prob.varlen:
        lens = [s[0] if which == "q" else s[1] for s in prob.seqs]
        t0 = 0
        for n in lens:
            seg = x[t0:t0 + n] if prob.layout == "NHD" else x[:, t0:t0 + n]
            out.append(np.ascontiguousarray(seg.transpose(1, 0, 2) if prob.layout == "NHD" else seg))
            t0 += n
        return out
    for b in range(x.shape[0]):
        xb = x[b]
        out.append(np.ascontiguousarray(xb.transpose(1, 0, 2) if prob.layout == "NHD" else xb))
    return out


def merge_heads(prob: Problem, per_seq):
    """Inverse of split_heads for outputs: list of [H, N, d] -> physical."""
    if prob.varlen:
        if prob.layout == "NHD":
            return np.concatenate([a.transpose(1, 0, 2) for a in per_seq], axis=0)
        return np.concatenate(per_seq, axis=1)
    st = np.stack(per_seq, axis=0)
    return st.transpose(0, 2, 1, 3) if prob.layout == "NHD" else st


@dataclass
class Prepass:
    """Logical pre-pass results per sequence s (lists indexed by s)."""
    mu_q: list = field(default_factory=list)     # [Hq, d] FP32 or None
    mu_qb: list = field(default_factory=list)    # smooth_q "block": [Hq, nqb, d] FP32
    mu_k: list = field(default_factory=list)     # [Hkv, d] FP32 or None
    mu_v: list = field(default_factory=list)     # [Hkv, d] FP32 or None
    qc: list = field(default_factory=list)       # [Hq, nq, d] int8
    qs: list = field(default_factory=list)       # [Hq, ceil(nq/qk_block)] FP32
    kc: list = field(default_factory=list)       # [Hkv, nkv, d] int8
    ks: list = field(default_factory=list)       # [Hkv, ceil(nkv/qk_block)] FP32
    vc: list = field(default_factory=list)       # [Hkv, nkv, d] e4m3 bytes, or
                                                 # 16-bit patterns (pv_mode "half")
    vs: list = field(default_factory=list)       # [Hkv, d] FP32 (None for "half")
    ds: list = field(default_factory=list)       # [Hq, nkv] FP32 or None; with
                                                 # smooth_q "block": [Hq, nqb, nkv]
    ds_seq: list = field(default_factory=list)   # "block": [Hq, nkv] FP32, the sequence
                                                 # mean's share of ds
    mu_code: list = field(default_factory=list)  # "block": [Hq, nqb, 2, d] int8 (hi, lo)
    mu_cscale: list = field(default_factory=list)  # "block": [Hq, nqb] FP32


def prepass(prob: Problem, q, k, v, threads: int | None = None) -> Prepass:
    """Smoothing and quantization for every (sequence, head)."""
    qh, kh, vh = (split_heads(prob, t, w) for t, w in ((q, "q"), (k, "k"), (v, "k")))
    G = prob.Hq // prob.Hkv
    S = len(prob.seqs)

    def kv_unit(u):
        s, h = u
        kf = decode16(kh[s][h], prob.dtype)
        vf = decode16(vh[s][h], prob.dtype)
        mu_k = channel_mean(kf) if prob.smooth_k else None
        mu_v = channel_mean(vf) if prob.smooth_v else None
        k_s = smooth(kf, mu_k)
        kc, ks = quant_int8_blocks(k_s, prob.qk_block)
        if prob.pv_mode == "half":
            # the V operand stays 16-bit: v (or v - mu_v rounded to the type)
            vc, vs = encode16(smooth(vf, mu_v), prob.dtype), None
        else:
            vc, vs = quant_fp8_channels(smooth(vf, mu_v))
        return mu_k, mu_v, k_s, kc, ks, vc, vs

    blockwise = prob.smooth_q == "block"

    def q_unit(u, kvu):
        s, h = u
        qf = decode16(qh[s][h], prob.dtype)
        if blockwise:
            # one mean per quantization block: the sequence mean's compensation
            # from the unquantized K_s, plus each block's deviation from it
            # through its code and the INT8 key codes
            mu_bar = channel_mean(qf)
            ds_seq = delta_s(mu_bar, kvu[2])
            mu_b = block_mean(qf, prob.qk_block)
            qc, qs = quant_int8_blocks(smooth_blocks(qf, mu_b, prob.qk_block), prob.qk_block)
            codes = [mu_code(m - mu_bar) for m in mu_b]      # FP32 difference per channel
            nkv = kvu[3].shape[0]
            ds = np.stack([delta_s_block(ds_seq, hi, lo, sc, kvu[3], kvu[4], prob.qk_block)
                           for hi, lo, sc in codes]) if codes else np.zeros((0, nkv), np.float32)
            code = (np.stack([np.stack([hi, lo]) for hi, lo, _ in codes]) if codes
                    else np.zeros((0, 2, prob.d), np.int8))
            csc = np.array([sc for _, _, sc in codes], np.float32)
            return (mu_bar, mu_b, ds_seq), qc, qs, ds, code, csc
        mu_q = channel_mean(qf) if prob.smooth_q else None
        qc, qs = quant_int8_blocks(smooth(qf, mu_q), prob.qk_block)
        ds = delta_s(mu_q, kvu[2]) if prob.smooth_q else None
        return mu_q, qc, qs, ds, None, None

    with ThreadPoolExecutor(max_workers=threads or os.cpu_count()) as ex:
        kv = list(ex.map(kv_unit, [(s, h) for s in range(S) for h in range(prob.Hkv)]))
        qq = list(ex.map(lambda u: q_unit(u, kv[u[0] * prob.Hkv + u[1] // G]),
                         [(s, h) for s in range(S) for h in range(prob.Hq)]))
    R = Prepass()
    for s in range(S):
        ks_ = kv[s * prob.Hkv:(s + 1) * prob.Hkv]
        qs_ = qq[s * prob.Hq:(s + 1) * prob.Hq]
        R.mu_k.append(np.stack([x[0] for x in ks_]) if prob.smooth_k else None)
        R.mu_v.append(np.stack([x[1] for x in ks_]) if prob.smooth_v else None)
        R.kc.append(np.stack([x[3] for x in ks_]))
        R.ks.append(np.stack([x[4] for x in ks_]))
        R.vc.append(np.stack([x[5] for x in ks_]))
        R.vs.append(np.stack([x[6] for x in ks_]) if prob.pv_mode != "half" else None)
        if blockwise:
            R.mu_q.append(np.stack([x[0][0] for x in qs_]))
            R.mu_qb.append(np.stack([x[0][1] for x in qs_]))
            R.ds_seq.append(np.stack([x[0][2] for x in qs_]))
        else:
            R.mu_q.append(np.stack([x[0] for x in qs_]) if prob.smooth_q else None)
            R.mu_qb.append(None)
            R.ds_seq.append(None)
        R.qc.append(np.stack([x[1] for x in qs_]))
        R.qs.append(np.stack([x[2] for x in qs_]))
        R.ds.append(np.stack([x[3] for x in qs_]) if prob.smooth_q else None)
        R.mu_code.append(np.stack([x[4] for x in qs_]) if blockwise else None)
        R.mu_cscale.append(np.stack([x[5] for x in qs_]) if blockwise else None)
    return R


def forward_rows(prob: Problem, pre: Prepass, rows=None, bkv: int = 128,
                 threads: int | None = None, tie: bool = False):
    """Same-recipe forward.  rows: None (all rows) or a list over sequences of
    int arrays of query rows.  Returns (out, lse): lists over sequences of
    [Hq, nrows, d] FP32 and [Hq, nrows] FP32; with tie=True also the
    rounding-tie bound of each output element (same shape as out), the most
    that re-rounding the P operands that sit at a rounding midpoint can move
    it (sage_oracle.c, recipe_rows)."""
    G = prob.Hq // prob.Hkv
    units = [(s, h) for s in range(len(prob.seqs)) for h in range(prob.Hq)]

    def one(u):
        s, h = u
        nq = prob.seqs[s][0]
        r = np.arange(nq) if rows is None else np.asarray(rows[s])
        # per-block Q smoothing: ds is [Q blocks, nkv], row i takes block i / qk_block
        ds_rows = prob.qk_block if prob.smooth_q == "block" else 0
        return one_rows(s, h, r, None if pre.ds[s] is None else pre.ds[s][h], ds_rows)

    def one_rows(s, h, r, ds, ds_rows=0):
        hk = h // G
        mu_v = None if pre.mu_v[s] is None else pre.mu_v[s][hk]
        if prob.pv_mode == "half":
            return attn_recipe_half_rows(pre.qc[s][h], pre.qs[s][h], pre.kc[s][hk],
                                         pre.ks[s][hk], pre.vc[s][hk], prob.dtype, ds, mu_v,
                                         prob.scale, prob.causal, bkv, r, prob.kv_split,
                                         prob.qk_block, tie=tie)
        return attn_recipe_rows(pre.qc[s][h], pre.qs[s][h], pre.kc[s][hk], pre.ks[s][hk],
                                pre.vc[s][hk], pre.vs[s][hk], ds, mu_v,
                                prob.scale, prob.causal, bkv, r, prob.kv_split, prob.qk_block,
                                tie=tie, ds_rows=ds_rows)

    with ThreadPoolExecutor(max_workers=threads or os.cpu_count()) as ex:
        res = list(ex.map(one, units))
    outs, lses, ties = [], [], []
    for s in range(len(prob.seqs)):
        part = res[s * prob.Hq:(s + 1) * prob.Hq]
        outs.append(np.stack([p[0] for p in part]))
        lses.append(np.stack([p[1] for p in part]))
        if tie:
            ties.append(np.stack([p[2] for p in part]))
    return (outs, lses, ties) if tie else (outs, lses)


def exact_rows(prob: Problem, q, k, v, rows=None, threads: int | None = None):
    """Exact FP64 softmax attention on the decoded inputs (no smoothing, no
    quantization).  Returns lists over sequences of [Hq, nrows, d] FP64."""
    qh, kh, vh = (split_heads(prob, t, w) for t, w in ((q, "q"), (k, "k"), (v, "k")))
    G = prob.Hq // prob.Hkv
    units = [(s, h) for s in range(len(prob.seqs)) for h in range(prob.Hq)]

    def one(u):
        s, h = u
        nq = prob.seqs[s][0]
        r = np.arange(nq) if rows is None else np.asarray(rows[s])
        return attn_exact_rows(decode16(qh[s][h], prob.dtype), decode16(kh[s][h // G], prob.dtype),
                               decode16(vh[s][h // G], prob.dtype), prob.scale, prob.causal, r)

    with ThreadPoolExecutor(max_workers=threads or os.cpu_count()) as ex:
        res = list(ex.map(one, units))
    outs, lses = [], []
    for s in range(len(prob.seqs)):
        part = res[s * prob.Hq:(s + 1) * prob.Hq]
        outs.append(np.stack([p[0] for p in part]))
        lses.append(np.stack([p[1] for p in part]))
    return outs, lses
