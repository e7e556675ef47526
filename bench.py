"""Benchmark of the KDA forward on one MI355X.

A step is one chunked-prefill forward of the long-context workload (B=1,
T=65536, 16 query/key heads for 64 value heads, K=V=128, chunk 64 requested,
bf16 q/k/v, fp32 gate inputs and state, safe gate): gate, cumulative decay,
intra-chunk solve and inter-chunk propagation, all in one launch of the fused
chunk kernel, which solves each chunk's triangular system in 16-token diagonal
blocks (the block size is reported next to the requested chunk size).  The
other chunked-prefill workloads (prefill: B=4, T=4096, H=HV=16; GVA: B=2,
T=16384, 8 q/k heads for 32 value heads, standard gate, random initial state)
run at full size through the same kernel ("configs" object).  The recurrent
decode row is timed in the same run on the decode workload (B=256, HV=32, 256
single-token steps over a 512 MiB fp32 state) and reported in the "decode"
object; the fused multi-token recurrent forward runs the same 256 tokens as
16-token calls and as one 256-token call ("recurrent" object), the chunked
forward runs the prefill shape with one gate per (token, value head)
("head_gate" object), and the one-sequence long shard (T=65536, 8 value heads)
runs through both the fused chunk kernel and the three-stage split schedule
("split" object).  The backward pass (kda_bwd) runs on the prefill shape
("backward" object): its roofline covers the whole call (the forward pass
that writes the segment checkpoints, the prep, segment and gate kernels),
its algorithmic FLOPs against the fp32 MFMA peak, on which all of its
products run.

Prints ONE JSON line (rank 0).  Inputs are synthetic, seeded, resident in
HBM before timing starts.  `roofline` covers the chunk kernel: algorithmic
bytes per launch / mean launch time (HIP events on the launch stream) against
the 8 TB/s HBM peak; `mfma` adds algorithmic FLOPs (counted at the 16-token
block the kernel solves) against the 2.5166 PFLOP/s dense bf16 MFMA peak and,
from the committed counter passes, the fraction of cycles the matrix pipes
were busy and the MFMA flops executed.  `cpu_baseline` times the fp64 CPU
oracle on all host cores over a sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6
FP32_VECTOR_PEAK_TFLOPS = 157.3
FP32_MFMA_PEAK_TFLOPS = 157.3


def chunk_bytes(w):
    """Algorithmic HBM bytes of one chunked forward: every input read once
    (q, k once per query/key head), o written once, final (and initial) state."""
    qk = 2 * w.B * w.T * w.H * w.K * (2 if w.dtype == "bf16" else 4)
    v = w.B * w.T * w.HV * w.V * (2 if w.dtype == "bf16" else 4)
    g = w.B * w.T * w.HV * (1 if w.per_head_gate else w.K) * 4
    beta = w.B * w.T * w.HV * 4
    o = w.B * w.T * w.HV * w.V * 4
    state = w.B * w.HV * w.K * w.V * 4 * (2 if w.s0_std > 0 else 1)
    return qk + v + g + beta + o + state


# The fused chunk kernel solves every chunk's triangular system in diagonal
# blocks of this many tokens, whatever chunk size is requested (the result
# does not depend on it).
BLOCK = 16


def chunk_flops(w, C=BLOCK):
    """Dense FLOPs of the chunkwise algorithm with blocks of C tokens:
    2 (3 C K + 2 C V + 3 K V) per token and value head (A_qk, R, w, u, U,
    Q S, A U, state update)."""
    return 2 * (3 * C * w.K + 2 * C * w.V + 3 * w.K * w.V) * w.B * w.T * w.HV


def bwd_flops(w):
    """Arithmetic of the backward's reverse pass per token and value head,
    an FMA counted as two: the state rebuilt from its segment checkpoint
    (Sd = alpha S, Sd^T k, S = Sd + beta k r^T: 5 K V) and the reverse step
    (dS += s q do^T, S_t do, dS^T k, beta dS r - Sd dr, dS - k dr^T,
    rowsum(dSd Sd), alpha dSd: 15 K V)."""
    return 20 * w.K * w.V * w.B * w.T * w.HV


def bwd_call_flops(w):
    """A whole backward call: the forward pass that writes the checkpoints,
    at its 16-token block, plus the reverse pass."""
    return chunk_flops(w, 16) + bwd_flops(w)


def bwd_bytes(w):
    """Algorithmic HBM bytes of one backward pass: the forward's inputs and
    dL/do read once, every gradient written once (dq, dk per query/key head)."""
    e = 2 if w.dtype == "bf16" else 4
    tok = w.B * w.T
    reads = (2 * tok * w.H * w.K * e + tok * w.HV * w.V * e + tok * w.HV * w.K * 4
             + tok * w.HV * 4 + tok * w.HV * w.V * 4)
    writes = 2 * tok * w.H * w.K * 4 + tok * w.HV * w.V * 4 + tok * w.HV * 4 + tok * w.HV * w.K * 4
    state = w.B * w.HV * w.K * w.V * 4 * (2 if w.s0_std > 0 else 0)
    return reads + writes + state


def decode_bytes(w):
    """Per step: the fp32 state read and written once, plus q, k, v, g_raw,
    beta and o for one token."""
    e = 2 if w.dtype == "bf16" else 4
    return (2 * w.B * w.HV * w.K * w.V * 4 + 2 * w.B * w.H * w.K * e + w.B * w.HV * w.V * e
            + w.B * w.HV * w.K * 4 + w.B * w.HV * 4 + w.B * w.HV * w.V * 4)


def recurrent_bytes(w, tokens):
    """One multi-token call: the fp32 state read and written once, plus q, k,
    v, g_raw, beta and o of every token of the call."""
    e = 2 if w.dtype == "bf16" else 4
    per_token = (2 * w.B * w.H * w.K * e + w.B * w.HV * w.V * e + w.B * w.HV * w.K * 4
                 + w.B * w.HV * 4 + w.B * w.HV * w.V * 4)
    return 2 * w.B * w.HV * w.K * w.V * 4 + tokens * per_token


def profile_record(key):
    """The counter-pass record of a kernel in profiles/traffic.json, or None
    when the kernel sources changed since it was taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[key]
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        return rec if h.hexdigest()[:16] == rec["source_sha256_16"] else None
    except (OSError, KeyError, ValueError):
        return None


def measured_traffic(key):
    """HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE passes."""
    rec = profile_record(key)
    return rec["traffic_bytes_per_launch"] if rec else None


def measured_mfma(key):
    """MFMA counters of the same kernel: the fraction of SIMD cycles its
    matrix pipe was busy (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x
    SIMDs) and the MFMA flops it executed (SQ_INSTS_VALU_MFMA_MOPS_* x 512)."""
    rec = profile_record(key)
    return rec.get("mfma") if rec else None


def chunk_line(kda, synth, w, dev, stream, steps, warmup):
    """Times kda.chunk_fwd on workload w (inputs resident in HBM, HIP events
    on the launch stream around the timed launches); returns the line's
    fields and the device inputs."""
    import torch

    d = synth.make_inputs(w)
    g = {n: (t.to(dev) if t is not None else None) for n, t in d.items()}
    o = torch.empty((w.B, w.T, w.HV, w.V), dtype=torch.float32, device=dev)
    S = torch.empty((w.B, w.HV, w.K, w.V), dtype=torch.float32, device=dev)

    def step():
        kda.chunk_fwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dt_bias"],
                      gate=w.gate, lower_bound=w.lower_bound, chunk_size=w.chunk,
                      initial_state=g["S0"], o=o, final_state=S)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t_wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    ms = ev[0].elapsed_time(ev[-1]) / steps
    launch_ms = sum(per) / len(per)
    nbytes, flops = chunk_bytes(w), chunk_flops(w)
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    key = "chunk_" + w.name
    line = {
        "ms_per_step": ms, "value": w.B * w.T / (ms * 1e-3), "unit": "tokens/s",
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(key),
                     "kernel": "chunk_fwd_kernel<128, bf16, %s gate>" % w.gate,
                     "bytes_per_launch": nbytes, "launch_ms": launch_ms},
        "mfma": {"algorithmic_flops": flops, "block": BLOCK,
                 "algorithmic_flops_chunk_%d" % w.chunk: chunk_flops(w, w.chunk),
                 "achieved_tflops": flops / (launch_ms * 1e-3) / 1e12,
                 "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "frac": flops / (launch_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                 "rocprof": measured_mfma(key)},
        "wall_s_timed": t_wall,
    }
    return line, d, g


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long", choices=["long", "prefill", "gva", "tiny"])
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-split", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward line")
    ap.add_argument("--no-gate", action="store_true", help="skip the standalone gate line")
    ap.add_argument("--no-head-gate", action="store_true", help="skip the per-head gate line")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other full-size chunked-prefill workloads")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import kimi_delta_attention_02_amd as kda
    from kimi_delta_attention_02_amd import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    w = synth.WORKLOADS[args.workload]
    line, d, g = chunk_line(kda, synth, w, dev, stream, args.steps, args.warmup)
    result = {
        "metric": "KDA fwd tokens/s (chunked prefill, decode) + % of MFMA / HBM roofline",
        "value": line["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": line["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v,g_raw N(0,1), beta=sigmoid(N(0,1)))",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "HV": w.HV, "K": w.K,
                   "V": w.V, "chunk": w.chunk, "block": BLOCK, "gate": w.gate,
                   "initial_state": w.s0_std > 0, "global_batch": w.B,
                   "seq_len": w.T, "parallelism": "none (1 GPU)"},
        "roofline": line["roofline"],
        "mfma": line["mfma"],
        "wall_s_timed": line["wall_s_timed"],
    }
    # The standalone gate entry point on the headline workload's g_raw: the
    # activation and the chunk-local cumulative log-decay (chunk 64), one
    # read and one write of every element.
    if not args.no_gate:
        gout = torch.empty_like(g["g_raw"])

        def gstep():
            kda.gate(g["g_raw"], g["A_log"], g["dt_bias"], gate=w.gate, lower_bound=w.lower_bound,
                     chunk_size=w.chunk, out=gout)

        for _ in range(args.warmup):
            gstep()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(args.steps):
            gstep()
        a1.record(stream)
        torch.cuda.synchronize()
        gms = a0.elapsed_time(a1) / args.steps
        gbytes = 2 * g["g_raw"].numel() * 4
        ggbs = gbytes / (gms * 1e-3) / 1e9
        result["gate"] = {
            "workload": w.name, "elements": g["g_raw"].numel(), "chunk": w.chunk, "gate": w.gate,
            "ms_per_call": gms,
            "roofline": {"bound": "hbm", "achieved": ggbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ggbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_launch": gbytes,
                         "kernel": "gate_cumsum_kernel"}}
        del gout
    del g

    # The other chunked-prefill workloads at full size, through the same
    # kernel: prefill (B=4, T=4096, H=HV=16), GVA (B=2, T=16384, 8 q/k heads
    # for 32 value heads, standard gate, random initial state) and long
    # context (B=1, T=65536, 16 q/k heads for 64 value heads), less the
    # headline workload.
    if not args.no_configs:
        result["configs"] = {}
        for name in ("prefill", "gva", "long"):
            if name == w.name:
                continue
            wc = synth.WORKLOADS[name]
            n_c = max(1, min(args.steps, 10))
            cl, _, gc = chunk_line(kda, synth, wc, dev, stream, n_c, 1)
            del gc
            result["configs"][name] = dict(
                {"B": wc.B, "T": wc.T, "H": wc.H, "HV": wc.HV, "K": wc.K, "V": wc.V,
                 "chunk": wc.chunk, "block": BLOCK, "gate": wc.gate,
                 "initial_state": wc.s0_std > 0, "calls": n_c}, **cl)

    if not args.no_head_gate:
        # The same chunked forward with one gate per (token, value head) (the
        # Gated DeltaNet form) on the prefill shape.
        wh = synth.WORKLOADS["prefill_head_gate"]
        dh = synth.make_inputs(wh)
        gh = {n: (t.to(dev) if t is not None else None) for n, t in dh.items()}
        oh = torch.empty((wh.B, wh.T, wh.HV, wh.V), dtype=torch.float32, device=dev)
        Sh = torch.empty((wh.B, wh.HV, wh.K, wh.V), dtype=torch.float32, device=dev)

        def hstep():
            kda.chunk_fwd(gh["q"], gh["k"], gh["v"], gh["g_raw"], gh["beta"], gh["A_log"],
                          gh["dt_bias"], gate=wh.gate, lower_bound=wh.lower_bound,
                          chunk_size=wh.chunk, initial_state=gh["S0"], o=oh, final_state=Sh)

        for _ in range(args.warmup):
            hstep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            hstep()
        e1.record(stream)
        torch.cuda.synchronize()
        hms = e0.elapsed_time(e1) / args.steps
        hbytes = chunk_bytes(wh)
        hgbs = hbytes / (hms * 1e-3) / 1e9
        result["head_gate"] = {
            "workload": wh.name, "B": wh.B, "T": wh.T, "H": wh.H, "HV": wh.HV, "K": wh.K,
            "gate": wh.gate + ", one per (token, value head)", "value": wh.B * wh.T / (hms * 1e-3),
            "unit": "tokens/s", "ms_per_step": hms,
            "roofline": {"bound": "hbm", "achieved": hgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": hgbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_launch": hbytes,
                         "kernel": "chunk_fwd_kernel<128, bf16, per-head gate>"}}
        del gh, oh, Sh

    # One GPU's share of the long-context workload (one sequence, 8 value
    # heads): the fused chunk kernel against the three-stage split schedule.
    if not args.no_split:
        ws_ = synth.WORKLOADS["long_shard"]
        dsh = synth.make_inputs(ws_)
        gsh = {n: (t.to(dev) if t is not None else None) for n, t in dsh.items()}
        osh = torch.empty((ws_.B, ws_.T, ws_.HV, ws_.V), dtype=torch.float32, device=dev)
        Ssh = torch.empty((ws_.B, ws_.HV, ws_.K, ws_.V), dtype=torch.float32, device=dev)
        wsp = torch.empty(kda.chunk_fwd_split_workspace_bytes(ws_.B, ws_.T, ws_.H, ws_.HV, ws_.K,
                                                              ws_.V, ws_.chunk),
                          dtype=torch.uint8, device=dev)
        args_sh = (gsh["q"], gsh["k"], gsh["v"], gsh["g_raw"], gsh["beta"], gsh["A_log"],
                   gsh["dt_bias"])
        kw_sh = dict(gate=ws_.gate, lower_bound=ws_.lower_bound, chunk_size=ws_.chunk,
                     initial_state=gsh["S0"], o=osh, final_state=Ssh)

        def time_calls(fn, n):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n):
                fn()
            z.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(z) / n

        n_sh = max(1, min(args.steps, 5))
        fused_ms = time_calls(lambda: kda.chunk_fwd(*args_sh, **kw_sh), n_sh)
        split_ms = time_calls(lambda: kda.chunk_fwd_split(*args_sh, workspace=wsp, **kw_sh), n_sh)
        sbytes = chunk_bytes(ws_)
        tok = ws_.B * ws_.T

        def line(ms, kernel, traffic):
            gbs = sbytes / (ms * 1e-3) / 1e9
            return {"ms_per_call": ms, "value": tok / (ms * 1e-3), "unit": "tokens/s",
                    "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                                 "bytes_per_launch": sbytes, "kernel": kernel}}

        result["split"] = {
            "workload": ws_.name, "B": ws_.B, "T": ws_.T, "H": ws_.H, "HV": ws_.HV, "K": ws_.K,
            "chunk": ws_.chunk, "gate": ws_.gate,
            "fused": line(fused_ms, "chunk_fwd_kernel<128, bf16>", None),
            "split": dict(line(split_ms, "split_intra + split_state + split_output <128, 64>",
                               measured_traffic("split")), mfma_rocprof=measured_mfma("split")),
            "speedup": fused_ms / split_ms}
        del gsh, osh, Ssh, wsp

    if not args.no_decode:
        wd = synth.WORKLOADS["decode"]
        dd = synth.make_inputs(wd)
        st = dd["S0"].to(dev)
        qs, ks, vs = (dd[n].transpose(0, 1).contiguous().to(dev) for n in ("q", "k", "v"))
        gs = dd["g_raw"].transpose(0, 1).contiguous().to(dev)
        bs = dd["beta"].transpose(0, 1).contiguous().to(dev)
        A_log, dtb = dd["A_log"].to(dev), dd["dt_bias"].to(dev)
        od = torch.empty((wd.steps, wd.B, wd.HV, wd.V), dtype=torch.float32, device=dev)

        def dstep(t):
            kda.recurrent_step(qs[t], ks[t], vs[t], gs[t], bs[t], A_log, dtb, st, gate=wd.gate,
                               lower_bound=wd.lower_bound, o=od[t])

        for t in range(min(8, wd.steps)):
            dstep(t)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(wd.steps):
            dstep(t)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1)
        per_step_ms = dms / wd.steps
        dgbs = decode_bytes(wd) / (per_step_ms * 1e-3) / 1e9
        result["decode"] = {
            "workload": wd.name, "B": wd.B, "HV": wd.HV, "K": wd.K, "V": wd.V, "steps": wd.steps,
            "value": wd.B * wd.steps / (dms * 1e-3), "unit": "tokens/s",
            "ms_per_token_step": per_step_ms,
            "roofline": {"bound": "hbm+llc", "achieved": dgbs, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode"),
                         "kernel": "decode_step_kernel<128, 128, bf16>",
                         "bytes_per_launch": decode_bytes(wd),
                         "note": "cache-assisted: the 512 MiB state is read with ordinary "
                                 "loads, so the 256 MB last-level cache serves part of each "
                                 "step's reads and achieved exceeds what HBM alone streams; "
                                 "hbm_roofline is the same step on a 1 GiB state"},
        }

        # The same steps with two and four times the sequences (1 and 2 GiB
        # states, read with non-temporal loads): the step as HBM alone streams it.
        import dataclasses

        nl = 32
        for rep, key in ((2, "large_state"), (4, "xl_state")):
            wl = dataclasses.replace(wd, B=rep * wd.B)
            st2 = torch.cat([st] * rep)
            q2, k2, v2, g2, b2 = (torch.cat([x] * rep, 1) for x in (qs, ks, vs, gs, bs))
            o2 = torch.empty((wl.B, wl.HV, wl.V), dtype=torch.float32, device=dev)

            def lstep(t):
                kda.recurrent_step(q2[t], k2[t], v2[t], g2[t], b2[t], A_log, dtb, st2, gate=wl.gate,
                                   lower_bound=wl.lower_bound, o=o2)

            for t in range(4):
                lstep(t)
            torch.cuda.synchronize()
            e0.record(stream)
            for t in range(nl):
                lstep(t)
            e1.record(stream)
            torch.cuda.synchronize()
            lms = e0.elapsed_time(e1) / nl
            lgbs = decode_bytes(wl) / (lms * 1e-3) / 1e9
            mib = wl.B * wl.HV * wl.K * wl.V * 4 >> 20
            if key == "large_state":
                result["decode"]["hbm_roofline"] = {
                    "bound": "hbm", "achieved": lgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": lgbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_launch": decode_bytes(wl),
                    "kernel": "decode_step_kernel<128, 128, bf16, non-temporal loads>",
                    "note": "the decode step with twice the sequences (1 GiB state, beyond the "
                            "last-level cache): HBM alone; xl_state has it at 2 GiB"}
            result["decode"][key] = {
                "B": wl.B, "state_mib": mib, "steps": nl,
                "ms_per_token_step": lms, "value": wl.B / (lms * 1e-3), "unit": "tokens/s",
                "roofline": {"bound": "hbm", "achieved": lgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": lgbs / HBM_PEAK_GBS, "traffic": None,
                             "bytes_per_launch": decode_bytes(wl)}}
            del q2, k2, v2, g2, b2, o2, st2
        del qs, ks, vs, gs, bs, od, st

        # The fused multi-token recurrent forward on the same workload: the 256
        # tokens as 16 calls of 16 tokens (state handed from call to call, so
        # read and written once per call) and as one call of 256 tokens.
        gd = {n: dd[n].to(dev) for n in ("q", "k", "v", "g_raw", "beta")}
        st = dd["S0"].to(dev)
        rec = {"workload": wd.name, "B": wd.B, "HV": wd.HV, "K": wd.K, "V": wd.V,
               "tokens": wd.steps, "kernel": "recurrent_fwd_kernel<128, 128, bf16>"}
        for per_call in (16, wd.steps):
            calls = wd.steps // per_call
            chunks = [{n: gd[n][:, c * per_call:(c + 1) * per_call].contiguous() for n in gd}
                      for c in range(calls)]
            outs = [torch.empty((wd.B, per_call, wd.HV, wd.V), dtype=torch.float32, device=dev)
                    for _ in range(calls)]

            def rcall(c):
                x = chunks[c]
                kda.recurrent_fwd(x["q"], x["k"], x["v"], x["g_raw"], x["beta"], A_log, dtb,
                                  gate=wd.gate, lower_bound=wd.lower_bound, initial_state=st,
                                  final_state=st, o=outs[c])

            rcall(0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for c in range(calls):
                rcall(c)
            e1.record(stream)
            torch.cuda.synchronize()
            rms_ = e0.elapsed_time(e1)
            nbytes = recurrent_bytes(wd, per_call)
            gbs = nbytes * calls / (rms_ * 1e-3) / 1e9
            rec["calls_of_%d" % per_call] = {
                "calls": calls, "value": wd.B * wd.steps / (rms_ * 1e-3), "unit": "tokens/s",
                "ms_per_call": rms_ / calls,
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": gbs / HBM_PEAK_GBS,
                             "traffic": measured_traffic("recurrent") if per_call == 16 else None,
                             "bytes_per_launch": nbytes}}
            del chunks, outs
        result["recurrent"] = rec
        del gd, st

    # Backward pass on the prefill shape: kda_bwd (the forward in checkpoint
    # mode, then the prep, segment and gate kernels), timed as whole calls.
    if not args.no_bwd:
        wb = synth.WORKLOADS["prefill"]
        db = synth.make_inputs(wb)
        gb = {n: (t.to(dev) if t is not None else None) for n, t in db.items()}
        gen = torch.Generator(device="cpu").manual_seed(77)
        dout = torch.randn((wb.B, wb.T, wb.HV, wb.V), generator=gen).to(dev)
        wsb = torch.empty(kda.bwd_workspace_bytes(wb.B, wb.T, wb.H, wb.HV, wb.K, wb.V),
                          dtype=torch.uint8, device=dev)
        argsb = (gb["q"], gb["k"], gb["v"], gb["g_raw"], gb["beta"], gb["A_log"], gb["dt_bias"])

        def timed(fn, n):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n):
                fn()
            z.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(z) / n

        n_b = max(1, min(args.steps, 5))
        bwd_ms = timed(lambda: kda.bwd(*argsb, gate=wb.gate, lower_bound=wb.lower_bound,
                                       initial_state=gb["S0"], dout=dout, workspace=wsb), n_b)
        fl = bwd_call_flops(wb)
        result["backward"] = {
            "workload": wb.name, "B": wb.B, "T": wb.T, "H": wb.H, "HV": wb.HV, "K": wb.K,
            "gate": wb.gate, "dtype": wb.dtype, "calls": n_b, "ms_per_call": bwd_ms,
            "value": wb.B * wb.T / (bwd_ms * 1e-3), "unit": "tokens/s",
            "algorithmic_bytes": bwd_bytes(wb),
            "hbm_frac_whole_call": bwd_bytes(wb) / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "roofline": {"bound": "mfma", "achieved": fl / (bwd_ms * 1e-3) / 1e12,
                         "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": fl / (bwd_ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS,
                         "traffic": measured_traffic("bwd_prefill"), "flops_per_launch": fl,
                         "launch_ms": bwd_ms,
                         "kernel": "kda_bwd, whole call (checkpoint-mode chunk forward, "
                                   "bwd_segment_kernel<128, bf16, safe gate>, "
                                   "gate kernel; the outputs zeroed by the first)"}}
        del gb, dout, wsb

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 1024 * 1024 // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 4 * n

    if not args.no_cpu:
        import oracle

        cores = os.cpu_count() or 1
        npf = lambda x: None if x is None else x.float().numpy()
        # Bounded sample: whole (sequence, value head) pairs of the same workload,
        # at most ~64 x 4096 token-heads per pass, passes repeated until about ten
        # seconds of CPU work have been timed (at most 30 passes).
        pairs = [(b, hv) for b in range(w.B) for hv in range(w.HV)]
        heads = pairs[:max(1, cores, (64 * 4096) // max(1, w.T))]
        args_np = [npf(d[n]) for n in ("q", "k", "v", "g_raw", "beta", "A_log", "dt_bias")]
        s0 = npf(d["S0"])
        passes, t0 = 0, time.perf_counter()
        while True:
            oracle.default().kda_fwd_heads(*args_np, w.gate, w.lower_bound, s0, heads, threads=cores)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or passes >= 30:
                break
        token_heads = passes * len(heads) * w.T
        result["cpu_baseline"] = {
            "value": token_heads / dt / w.HV, "unit": "tokens/s", "cores": min(cores, len(heads)),
            "kind": "oracle",
            "sample": "%d pass(es) over %d (sequence, value head) pairs x %d tokens of the %s "
                      "workload (%s), fp64 recurrence, one pair per thread; tokens/s = "
                      "token-heads/s / HV" % (passes, len(heads), w.T, w.name,
                                              "all of it" if len(heads) == len(pairs) else
                                              "a subset of its pairs"),
            "seconds": dt}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
