"""Benchmark of the quantized attention forward pass on one MI355X.

One step = one sage_attn_fwd call (pre-pass: means, INT8/FP8 quantization;
then the fused INT8-QK / online-softmax / FP8-PV kernel) over the causal GQA
workload (B=1, Hq=32, Hkv=8, N=8192, d=128, fp16, seeded synthetic inputs
already resident in HBM).  The metric is attention TOPS with the headline
formula 4*B*Hq*Nq*Nkv*d, halved for causal.

Prints ONE JSON line.  Besides the standard fields it carries
  roofline     : the fused kernel (the dominant launch) against the dense
                 INT8/FP8 MFMA peak of MI355X (5.0 POPS): algorithmic ops
                 (4*d per visible (q, k) pair) per launch / its average
                 duration.  The call is split into two halves
                 (sage_quant_qkv, then sage_attn_fwd_quantized on the same
                 buffers), and each half is timed in a loop of its own with
                 HIP events on the launch stream around the loop; kernel_ms
                 is the fused kernel's half, prepass_ms the other, measured,
                 not a difference, and halves_sum_ms their sum next to
                 ms_per_step.  Inside sage_attn_fwd (without Q smoothing)
                 the fused kernel quantizes Q itself in its prologue and the
                 pre-pass skips Q, so the call is a little shorter than the
                 halves' sum;
                 kernel_ms is the same kernel reading the pre-pass's Q
                 codes (its loop and softmax are the same);
  n32k         : the same figures for the long-context varlen workload at
                 d=128 (four packed sequences, keys up to 32768 per
                 sequence), the metric's N=32K point;
  cpu_baseline : the CPU oracle (same recipe, plain C) timed on a bounded
                 sample of the same workload on the host cores.
--pv half times the 16-bit P.V variant instead (P and V in the input's type
on the 16-bit MFMA); its roofline peak is that of the op mix, half INT8 at
5.0 POPS and half fp16/bf16 at 2.5 PFLOP/s, i.e. 3.33 POPS.
The W warm-up steps are untimed and continue until --min-warmup-s of wall
time has passed (the clocks settle); the JSON line reports how many ran.
--kv-split N|auto splits the key range (flash-decoding).  A workload whose
arithmetic intensity (ops per algorithmic byte of the fused kernel) is below
the ridge of 5.0 POPS / 8 TB/s is reported against HBM instead: achieved =
algorithmic bytes (Q, K, V codes and scales, O, split partials written and
read back) per call / the fused kernel's time, peak 8 TB/s.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TOPS = 5000.0           # MI355X dense INT8 / FP8 MFMA peak (T-ops/s)
PEAK_16 = 2500.0             # ... dense fp16 / bf16 MFMA peak
PEAK_HBM = 8000.0            # MI355X HBM3E bandwidth (GB/s)
WORKLOAD = "causal_gqa"
SECOND = "varlen_d128"         # the N=32K point, reported next to the N=8K one


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--min-warmup-s", type=float, default=0.3,
                    help="keep warming up (untimed) until this much wall time has passed, "
                         "so that the GPU clocks have settled")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--pv", choices=("fp8", "half"), default="fp8",
                    help="P.V operands: E4M3 (default) or the input's 16-bit type")
    ap.add_argument("--kv-split", default="0",
                    help="keys per split of the key range (multiple of 128), 0 or auto")
    ap.add_argument("--qk-block", type=int, choices=(64, 32), default=64,
                    help="tokens per Q/K quantization block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-second", action="store_true",
                    help="skip the N=32K point (varlen_d128) that the default workload adds")
    ap.add_argument("--cpu-rows", type=int, default=8192, help="oracle rows per query head")
    ap.add_argument("--no-micro", action="store_true",
                    help="skip the measured INT8/FP8 matrix peak beside the published one")
    ap.add_argument("--micro", action="store_true",
                    help="only print the measured rates of the INT8 and FP8 matrix "
                         "instructions, v_exp_f32 and v_fma_f32, then exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (the reference "
                         "kernel for scaling the HBM byte counters), then exit")
    return ap.parse_args()


KERNEL_SRC = os.path.join(ROOT, "quantized_attention_03_amd", "csrc", "sage_attn.hip")


def kernel_digest() -> str:
    """sha256[:16] of the kernel source's code: comments removed and runs of
    whitespace collapsed, so that a change to comments alone keeps the
    committed counter summaries valid, and any change to the code does not."""
    import hashlib
    import re
    with open(KERNEL_SRC, encoding="utf-8") as f:
        src = f.read()
    # string and character literals are kept whole (a "//" inside one is not
    # a comment); block and line comments go
    tok = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|/\*.*?\*/|//[^\n]*', re.S)
    code = tok.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", src)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(workload: str, kernel: str = "k_attn"):
    """HBM bytes per launch of the kernel from the committed counter summary
    profiles/<kernel>_<workload>_traffic.txt, or None when it is missing or
    was taken on a different kernel source."""
    try:
        fields = {}
        with open(os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")) as f:
            for ln in f:
                if ":" in ln and not ln.startswith("#"):
                    k, v = ln.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("workload") != workload or fields.get("kernel_source_sha256_16") != kernel_digest():
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration(mib: int):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}),
          flush=True)


def cpu_baseline(w, q, k, v, rows_per_head: int, pv: str = "fp8", split: int = 0,
                 qb: int = 64):
    """Time the oracle's same-recipe forward on evenly spaced query rows of
    every head (the pre-pass is run first and not timed)."""
    import numpy as np
    import torch

    from oracle import oracle as orc

    def u16(t):
        return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    prob = orc.problem_from_workload(w, pv, split, qb)
    pre = orc.prepass(prob, u16(q), u16(k), u16(v))
    threads = os.cpu_count() or 1
    rows, pairs = [], 0
    for nq, nkv in w.seq_lens():
        r = np.unique(np.linspace(0, nq - 1, rows_per_head).astype(np.int64))
        rows.append(r)
        vis = np.minimum(nkv, np.maximum(0, r + nkv - nq + 1)) if w.causal else np.full(r.size, nkv)
        pairs += int(vis.sum()) * w.Hq
    t0 = time.perf_counter()
    orc.forward_rows(prob, pre, rows=rows, bkv=128, threads=threads)
    dt = time.perf_counter() - t0
    ops = 4.0 * w.d * pairs
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "cpu_model": host_cpu_model(),
            "sample": f"same-recipe forward of {sum(len(r) for r in rows)} query rows per head "
                      f"group ({rows_per_head} evenly spaced rows x {w.Hq} heads, {pairs} visible "
                      f"pairs, {dt:.1f} s wall), pre-pass excluded"}


def kernel_bytes(w, pv: str, nsplit: int) -> float:
    """Algorithmic HBM bytes of one fused-kernel call: the Q, K and V codes
    and their scales read once, the output written once, and (split key
    range) the partials written by the kernel and read back by the merge."""
    ves = 2 if pv == "half" else 1
    tot = 0.0
    for nq, nkv in w.seq_lens():
        tot += w.Hq * nq * w.d * (1 + 2) + w.Hq * math.ceil(nq / 64) * 4      # Q codes, O
        tot += w.Hkv * nkv * w.d * (1 + ves) + w.Hkv * math.ceil(nkv / 64) * 4
        tot += 0 if pv == "half" else w.Hkv * w.d * 4                         # V scales
        if nsplit > 1:
            tot += 2 * nsplit * w.Hq * nq * (w.d + 2) * 4                     # partials
    return tot


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measure(w, args, dev):
    """Time one workload: the whole call (the step) and its two halves.
    Returns the inputs and a dict of timings (ms)."""
    import torch

    import quantized_attention_03_amd as qa
    import synth

    q, k, v, meta = synth.make_inputs(w, device=dev)
    kv_split = args.kv_split if args.kv_split == "auto" else int(args.kv_split)
    kw = dict(tensor_layout=w.layout, is_causal=w.causal, smooth_q=w.smooth_q,
              smooth_k=w.smooth_k, smooth_v=w.smooth_v, sm_scale=w.sm_scale,
              pv_mode=args.pv, kv_split=kv_split, qk_block=args.qk_block)
    o = torch.empty_like(q)
    cu = {}
    if w.varlen:
        cu = dict(cu_seqlens_q=meta["cu_seqlens_q"], cu_seqlens_kv=meta["cu_seqlens_kv"])
        desc = qa.make_desc(q, k, v, o, varlen=True, **kw)
        ws = torch.empty(qa.workspace_size(desc, cu["cu_seqlens_q"], cu["cu_seqlens_kv"]),
                         dtype=torch.uint8, device=dev)

        def step():
            qa.sage_attn_fwd_varlen(q, k, v, cu["cu_seqlens_q"], cu["cu_seqlens_kv"], out=o,
                                    workspace=ws, **kw)
    else:
        desc = qa.make_desc(q, k, v, o, **kw)
        ws = torch.empty(qa.workspace_size(desc), dtype=torch.uint8, device=dev)

        def step():
            qa.sage_attn_fwd(q, k, v, out=o, workspace=ws, **kw)

    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # W untimed steps, continued until the clocks have settled (min-warmup-s
    # of wall time): with a short warm-up the timed loop still ran part of
    # the time at lower clocks (7% slower at W = 10 on causal_gqa)
    tw = time.perf_counter()
    warm = 0
    while warm < args.warmup or time.perf_counter() - tw < args.min_warmup_s:
        step()
        warm += 1
        if warm % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev0, ev1 = ev(), ev()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    # the same steps timed one by one (median and minimum of the whole call)
    evs = [(ev(), ev()) for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per_step = sorted(a.elapsed_time(b) for a, b in evs)

    # The call's two halves, each timed in a loop of its own with events only
    # around the loop: the pre-pass (sage_quant_qkv) into buffers of the same
    # layout as the call's workspace, and the fused kernel
    # (sage_attn_fwd_quantized) on them -- together the same launches as
    # sage_attn_fwd.  (An event recorded between the two halves of every
    # call slows the fused kernel by about 18% in the kernel trace, so the
    # halves are not timed inside one loop.)
    bufs = qa.sage_quant_qkv(q, k, v, **kw, **cu)

    def half_loop(fn):
        t1 = time.perf_counter()
        n = 0
        while n < 10 or time.perf_counter() - t1 < 0.1:
            fn()
            n += 1
        torch.cuda.synchronize()
        ka, kb = ev(), ev()
        ka.record(stream)
        for _ in range(args.steps):
            fn()
        kb.record(stream)
        torch.cuda.synchronize()
        return ka.elapsed_time(kb) / args.steps

    pre_ms = half_loop(lambda: qa.sage_quant_qkv(q, k, v, **kw, **cu, bufs=bufs))
    kern_ms = half_loop(lambda: qa.sage_attn_fwd_quantized(bufs, o, **cu))
    res = {"ms": ms, "ms_median": per_step[len(per_step) // 2], "ms_min": per_step[0],
           "kernel_ms": kern_ms, "prepass_ms": pre_ms, "wall": wall, "warm": warm,
           "split": qa.kv_split_size(desc, cu.get("cu_seqlens_q"), cu.get("cu_seqlens_kv"))}
    del bufs, ws, o
    return (q, k, v), res


def micro_rates(ops, reps=16384):
    """Measured rates of the matrix instructions (TOPS) and of v_exp_f32 (G
    results/s) and v_fma_f32 (TFLOP/s), one timed launch each."""
    import quantized_attention_03_amd as qa
    unit = {"i8": ("TOPS", 1e12), "f8": ("TFLOP/s", 1e12), "exp": ("Gexp/s", 1e9),
            "fma": ("TFLOP/s", 1e12)}
    out = {}
    for op in ops:
        u, sc = unit[op]
        out[op] = {"rate": round(qa.sage_micro_rate(op, reps) / sc, 1), "unit": u}
    return out


def roofline(w, args, r):
    """The fused kernel against its roofline, from the timings of measure()."""
    half = args.pv == "half"
    exact = w.exact_ops()
    # half the ops are INT8 Q.K^T, half P.V in the operand type
    peak = PEAK_TOPS if not half else 1.0 / (0.5 / PEAK_TOPS + 0.5 / PEAK_16)
    split = r["split"]
    max_nkv = max(nkv for _, nkv in w.seq_lens())
    nsplit = math.ceil(max_nkv / split) if split else 1
    kbytes = kernel_bytes(w, args.pv, nsplit)
    kern_ms = r["kernel_ms"]
    # a split key range whose GQA group x queries fit one wave's 32 rows runs
    # the one-wave decode kernel
    dec = bool(split) and (w.Hq // w.Hkv) * max(1, max(nq for nq, _ in w.seq_lens())) <= 32
    hbm_bound = exact / kbytes < peak * 1e12 / (PEAK_HBM * 1e9)
    pvt = ("f16" if w.dtype == "f16" else "bf16") if half else "fp8"
    if not hbm_bound:
        achieved = exact / (kern_ms * 1e-3) / 1e12
        rl = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
              "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    else:
        gbs = kbytes / (kern_ms * 1e-3) / 1e9
        rl = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM, "unit": "GB/s",
              "frac": round(gbs / PEAK_HBM, 4), "bytes_per_launch": kbytes}
    rl["traffic"] = (measured_traffic(w.name, "k_decode")
                     if dec and not half and args.kv_split == "auto" and args.qk_block == 64 else
                     None if half or split or args.qk_block != 64 else measured_traffic(w.name))
    rl["kernel"] = ((f"k_decode (one wave per kv head and split, INT8-QK / softmax / "
                     f"{pvt.upper()}-PV)" if dec else
                     f"k_attn (fused INT8-QK / softmax / {pvt.upper()}-PV)")
                    + (f" + k_merge ({nsplit} splits of {split} keys)" if split else ""))
    rl["kernel_ms"] = round(kern_ms, 4)
    rl["ops_per_launch"] = exact
    return rl


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the forward pass shards over batch and heads with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.micro:
        print(json.dumps(micro_rates(("i8", "f8", "exp", "fma"))), flush=True)
        return

    import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    (q, k, v), r = measure(w, args, dev)
    ms = r["ms"]
    formula = w.formula_ops()
    exact = w.exact_ops()
    value = formula / (ms * 1e-3) / 1e12
    half = args.pv == "half"
    io = "fp16 io" if w.dtype == "f16" else "bf16 io"
    pvt = ("f16" if w.dtype == "f16" else "bf16") if half else "fp8"
    line = {
        "metric": "attention TOPS at d=128, N=8K/32K; % of dense INT8/FP8 MFMA peak",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": r["warm"],
        "ms_per_step": round(ms, 4),
        "ms_median": round(r["ms_median"], 4),
        "ms_min": round(r["ms_min"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int8-qk/{pvt}-pv ({io})",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} "
                               f"Nq=Nkv={w.Nq} d={w.d} {w.dtype} {w.layout}"
                               f"{' causal' if w.causal else ''}"
                               f"{', 16-bit P.V' if half else ''}"
                               f"{', 32-token Q/K blocks' if args.qk_block == 32 else ''}",
                   "global_batch": w.B, "seq_len": w.Nq, "parallelism": "single-gpu"},
        "roofline": roofline(w, args, r),
        # the call's two halves, each timed in its own loop (their sum is
        # within a few percent of ms_per_step)
        "prepass_ms": round(r["prepass_ms"], 4),
        "kernel_ms": round(r["kernel_ms"], 4),
        "halves_sum_ms": round(r["prepass_ms"] + r["kernel_ms"], 4),
        "exact_pair_tops": round(exact / (ms * 1e-3) / 1e12, 2),
        "wall_s": round(r["wall"], 3),
    }
    if w.varlen:
        line["config"]["workload"] = (f"{w.name}: {len(w.seq_lens())} packed sequences "
                                      f"(Nq, Nkv) = {w.seq_lens()}, H={w.Hq} d={w.d} "
                                      f"{w.dtype} {w.layout}{' causal bottom-right' if w.causal else ''}")
        line["config"]["seq_len"] = max(nkv for _, nkv in w.seq_lens())
    second = None if args.no_second or args.workload != WORKLOAD else SECOND
    if second:
        w2 = synth.WORKLOADS[second]
        _, r2 = measure(w2, args, dev)
        rl2 = roofline(w2, args, r2)
        line["n32k"] = {
            "workload": f"{w2.name}: {len(w2.seq_lens())} packed sequences (Nq, Nkv) = "
                        f"{w2.seq_lens()}, H={w2.Hq} d={w2.d} {w2.dtype} {w2.layout} causal "
                        f"bottom-right",
            "value": round(w2.formula_ops() / (r2["ms"] * 1e-3) / 1e12, 2),
            "exact_pair_tops": round(w2.exact_ops() / (r2["ms"] * 1e-3) / 1e12, 2),
            "unit": "TOPS", "ms_per_step": round(r2["ms"], 4),
            "prepass_ms": round(r2["prepass_ms"], 4), "kernel_ms": round(r2["kernel_ms"], 4),
            "frac": rl2["frac"], "achieved": rl2["achieved"]}
    rl = line["roofline"]
    if not args.no_micro and rl["bound"] == "mfma" and not half:
        # half the ops run on each instruction, so their times add
        m = micro_rates(("i8", "f8"))
        mix = 1.0 / (0.5 / m["i8"]["rate"] + 0.5 / m["f8"]["rate"])
        rl["peak_measured"] = {"i8": m["i8"]["rate"], "f8": m["f8"]["rate"],
                               "mix": round(mix, 1), "unit": "TOPS"}
        rl["frac_of_measured"] = round(rl["achieved"] / mix, 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_rows, args.pv, r["split"],
                                            args.qk_block)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
