"""Seeded synthetic inputs for the quantized-attention workloads.

This module only draws numbers; it holds none of the attention method's
arithmetic, so that both the HIP library's callers and the CPU oracle can take
their inputs from it.  Every value is a pure function of (seed, tensor id,
logical element index):

* a SplitMix64 stream per (seed, tensor id): the i-th 64-bit draw is
  ``mix(base + (i + 1) * GOLDEN)`` with the published SplitMix64 finaliser
  ``mix`` (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014);
* a standard normal from draws 2i and 2i+1 by the Box-Muller transform in
  FP64;
* scale and offset in FP64, then rounding to FP32 and from there to the
  tensor dtype (round to nearest even at each step).

Logical element order is [b][h][n][c] for batched tensors and [h][t][c] for
packed variable-length tensors (t = token index in the packing); the physical
layout (HND, NHD, packed) is applied afterwards, so the values do not depend on
the layout chosen.

The workloads mirror the shapes the pages benchmark (LLM prefill, causal GQA,
video-DiT attention, long-context varlen at head dims 64/96/128); models and
datasets are not used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

GOLDEN = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
M64 = (1 << 64) - 1


def _s64(x: int) -> int:
    """Two's-complement view of an unsigned 64-bit integer."""
    x &= M64
    return x - (1 << 64) if x >> 63 else x


def _mix_int(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * MIX1) & M64
    z = ((z ^ (z >> 27)) * MIX2) & M64
    return z ^ (z >> 31)


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    return (z >> k) & ((1 << (64 - k)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(MIX1)
    z = (z ^ _lsr(z, 27)) * _s64(MIX2)
    return z ^ _lsr(z, 31)


def stream_base(seed: int, tensor_id: int) -> int:
    return _mix_int(_mix_int(seed * GOLDEN + 1) + tensor_id * GOLDEN)


def uniform64(seed: int, tensor_id: int, start: int, count: int,
              device="cpu") -> torch.Tensor:
    """Raw 64-bit draws start .. start+count-1 (as int64 bit patterns)."""
    base = stream_base(seed, tensor_id)
    i = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    return _mix(i * _s64(GOLDEN) + _s64(base))


def normal(seed: int, tensor_id: int, count: int, device="cpu",
           chunk: int = 1 << 23) -> torch.Tensor:
    """`count` standard normals in FP64 (Box-Muller on draw pairs)."""
    out = torch.empty(count, dtype=torch.float64, device=device)
    two53 = float(1 << 53)
    for s in range(0, count, chunk):
        n = min(chunk, count - s)
        z = uniform64(seed, tensor_id, 2 * s, 2 * n, device).view(n, 2)
        u1 = (_lsr(z[:, 0], 11).to(torch.float64) + 1.0) / two53      # (0, 1]
        u2 = _lsr(z[:, 1], 11).to(torch.float64) / two53               # [0, 1)
        out[s:s + n] = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * math.pi * u2)
    return out


def choose_channels(seed: int, tensor_id: int, groups: int, d: int, k: int,
                    device="cpu") -> torch.Tensor:
    """k distinct channels per group, by ranking seeded draws (sampling
    without replacement).  Returns int64 [groups, k]."""
    z = uniform64(seed, tensor_id, 0, groups * d, device).view(groups, d)
    key = _lsr(z, 11)
    return torch.argsort(key, dim=1)[:, :k]


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

DT = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    name: str
    dtype: str                      # "f16" | "bf16"
    layout: str                     # "HND" | "NHD" (varlen: packed NHD [T,H,d] or HND [H,T,d])
    B: int
    Hq: int
    Hkv: int
    Nq: int                         # dense only
    Nkv: int
    d: int
    causal: bool = False
    smooth_q: bool | str = False    # False, True (one mean per sequence) or "block"
    smooth_k: bool = True
    smooth_v: bool = False
    sm_scale: float | None = None
    seed: int = 0
    k_off_sigma: float = 0.0        # per (b,h,c) K offset ~ N(0, sigma^2)
    q_outlier_frac: float = 0.0     # fraction of Q channels scaled (per b,h)
    q_outlier_mult: float = 1.0
    qv_mean_sigma: float = 0.0      # per-channel mean of Q and V ~ N(0, sigma^2)
    qv_outlier_mult: float = 1.0    # 1 outlier channel of Q and V per head
    q_drift_sigma: float = 0.0      # Q offset drifting along the tokens: per (b,h,c)
                                    # A + (2t/(N-1) - 1) * B with A, B ~ N(0, sigma^2)
    seqlens_q: list = field(default_factory=list)   # varlen only
    seqlens_kv: list = field(default_factory=list)

    @property
    def varlen(self) -> bool:
        return bool(self.seqlens_q)

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale is not None else 1.0 / math.sqrt(self.d)

    def seq_lens(self):
        if self.varlen:
            return list(zip(self.seqlens_q, self.seqlens_kv))
        return [(self.Nq, self.Nkv)] * self.B

    def pairs(self) -> int:
        """Visible (query, key) pairs per query head, summed over sequences."""
        tot = 0
        for nq, nkv in self.seq_lens():
            tot += _causal_pairs(nq, nkv) if self.causal else nq * nkv
        return tot * self.Hq

    def formula_ops(self) -> float:
        """4*B*Hq*Nq*Nkv*d, halved when causal (the headline formula)."""
        ops = sum(4.0 * self.Hq * nq * nkv * self.d for nq, nkv in self.seq_lens())
        return ops / 2 if self.causal else ops

    def exact_ops(self) -> float:
        return 4.0 * self.d * self.pairs()


def _causal_pairs(nq: int, nkv: int) -> int:
    """Row i sees keys j <= i + nkv - nq (bottom-right alignment)."""
    return sum(min(nkv, max(0, i + nkv - nq + 1)) for i in range(nq))


C5_LENS = [(1024, 16384), (1024, 32768), (4096, 16384), (4096, 32768)]

WORKLOADS = {
    "tiny": Workload("tiny", "f16", "HND", 1, 2, 2, 256, 256, 64, seed=0,
                     k_off_sigma=2.0),
    "llm_prefill": Workload("llm_prefill", "bf16", "NHD", 2, 32, 32, 4096, 4096, 128,
                            seed=1, k_off_sigma=3.0, q_outlier_frac=0.01,
                            q_outlier_mult=20.0),
    "causal_gqa": Workload("causal_gqa", "f16", "HND", 1, 32, 8, 8192, 8192, 128,
                           causal=True, seed=2, k_off_sigma=3.0),
    "video_dit": Workload("video_dit", "bf16", "NHD", 1, 48, 48, 17776, 17776, 64,
                          smooth_q=True, smooth_v=True, seed=3, qv_mean_sigma=1.5,
                          qv_outlier_mult=10.0),
    "varlen_d128": Workload("varlen_d128", "f16", "NHD", 4, 32, 32, 0, 0, 128,
                            causal=True, seed=4, k_off_sigma=3.0,
                            seqlens_q=[a for a, _ in C5_LENS],
                            seqlens_kv=[b for _, b in C5_LENS]),
    "varlen_d96": Workload("varlen_d96", "f16", "NHD", 4, 32, 32, 0, 0, 96,
                           causal=True, seed=4, k_off_sigma=3.0,
                           seqlens_q=[a for a, _ in C5_LENS],
                           seqlens_kv=[b for _, b in C5_LENS]),
    # video DiT with a Q offset that drifts along the sequence, smoothed per
    # 64-token query block
    "video_dit_block": Workload("video_dit_block", "bf16", "NHD", 1, 48, 48, 17776, 17776, 64,
                                smooth_q="block", smooth_v=True, seed=6, qv_mean_sigma=1.5,
                                qv_outlier_mult=10.0, q_drift_sigma=3.0),
    # one new query per sequence against a 32K-token context (decode)
    "decode_gqa": Workload("decode_gqa", "f16", "HND", 8, 32, 8, 1, 32768, 128,
                           causal=True, seed=5, k_off_sigma=3.0),
}

# tensor ids inside one seed
TID_Q, TID_K, TID_V, TID_KOFF, TID_QOUT, TID_QMEAN, TID_VMEAN, TID_QVOUT = range(8)
TID_QDRIFT_A, TID_QDRIFT_B = 8, 9


def _lens(w: Workload):
    if w.varlen:
        return list(w.seqlens_q), list(w.seqlens_kv)
    return [w.Nq] * w.B, [w.Nkv] * w.B


def make_inputs(w: Workload, device="cpu"):
    """Return (q, k, v, meta) as torch tensors of dtype w.dtype on `device`.

    Dense: HND -> [B, H, N, d], NHD -> [B, N, H, d].
    Varlen: NHD -> [T, H, d], HND -> [H, T, d] packed over the sequences;
    meta["cu_seqlens_q"], meta["cu_seqlens_kv"] hold the int32 prefix offsets.
    """
    lq, lkv = _lens(w)
    S, d = len(lq), w.d
    dt = DT[w.dtype]

    def logical(tid, H, lens, extra_off=None):
        # logical layout: varlen [H][T][d]; dense [B][H][N][d]
        T = sum(lens)
        x = normal(w.seed, tid, H * T * d, device).view(-1)
        if w.varlen:
            x = x.view(H, T, d)
            segs = [(s, sum(lens[:s]), lens[s]) for s in range(S)]
        else:
            x = x.view(S, H, lens[0], d)
            segs = None
        return x, segs

    def per_seq_head(tid, H):
        return normal(w.seed, tid, S * H * d, device).view(S, H, d)

    def add_per_channel(x, vals, segs):
        # vals [S, H, d] broadcast over tokens of each sequence
        if segs is None:
            return x + vals[:, :, None, :]
        for s, t0, n in segs:
            x[:, t0:t0 + n, :] += vals[s][:, None, :]
        return x

    def scale_channels(x, chans, mult, H, segs):
        # chans [S*H, k]
        m = torch.ones(S, H, d, dtype=torch.float64, device=device)
        m.view(S * H, d).scatter_(1, chans, mult)
        if segs is None:
            return x * m[:, :, None, :]
        for s, t0, n in segs:
            x[:, t0:t0 + n, :] *= m[s][:, None, :]
        return x

    q, segq = logical(TID_Q, w.Hq, lq)
    k, segk = logical(TID_K, w.Hkv, lkv)
    v, _ = logical(TID_V, w.Hkv, lkv)
    if w.k_off_sigma:
        k = add_per_channel(k, w.k_off_sigma * per_seq_head(TID_KOFF, w.Hkv), segk)
    if w.q_outlier_frac:
        nout = math.ceil(w.q_outlier_frac * d)
        ch = choose_channels(w.seed, TID_QOUT, S * w.Hq, d, nout, device)
        q = scale_channels(q, ch, w.q_outlier_mult, w.Hq, segq)
    if w.qv_mean_sigma:
        q = add_per_channel(q, w.qv_mean_sigma * per_seq_head(TID_QMEAN, w.Hq), segq)
        v = add_per_channel(v, w.qv_mean_sigma * per_seq_head(TID_VMEAN, w.Hkv), segk)
    if w.q_drift_sigma:
        a = w.q_drift_sigma * per_seq_head(TID_QDRIFT_A, w.Hq)
        b = w.q_drift_sigma * per_seq_head(TID_QDRIFT_B, w.Hq)
        if segq is None:
            n = lq[0]
            ramp = (2.0 * torch.arange(n, dtype=torch.float64, device=device) / max(1, n - 1)
                    - 1.0)
            q = q + a[:, :, None, :] + ramp[None, None, :, None] * b[:, :, None, :]
        else:
            for s_, t0, n in segq:
                ramp = (2.0 * torch.arange(n, dtype=torch.float64, device=device) /
                        max(1, n - 1) - 1.0)
                q[:, t0:t0 + n, :] += a[s_][:, None, :] + ramp[None, :, None] * b[s_][:, None, :]
    if w.qv_outlier_mult != 1.0:
        chq = choose_channels(w.seed, TID_QVOUT, S * w.Hq, d, 1, device)
        q = scale_channels(q, chq, w.qv_outlier_mult, w.Hq, segq)
        chv = choose_channels(w.seed, TID_QVOUT + 100, S * w.Hkv, d, 1, device)
        v = scale_channels(v, chv, w.qv_outlier_mult, w.Hkv, segk)

    def finish(x):
        x = x.to(torch.float32).to(dt)          # FP64 -> dtype (via FP32)
        if w.varlen:
            return x.permute(1, 0, 2).contiguous() if w.layout == "NHD" else x.contiguous()
        return x.permute(0, 2, 1, 3).contiguous() if w.layout == "NHD" else x.contiguous()

    meta = {}
    if w.varlen:
        import itertools
        meta["cu_seqlens_q"] = [0] + list(itertools.accumulate(lq))
        meta["cu_seqlens_kv"] = [0] + list(itertools.accumulate(lkv))
    return finish(q), finish(k), finish(v), meta


def scaled_down(w: Workload, **over) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    import dataclasses
    return dataclasses.replace(w, **over)
