"""Helpers shared by the GPU parity tests: device copies of synthetic inputs,
calls through the binding, oracle references, and the error metric.

The metric is max |gpu - oracle| / RMS(oracle), taken separately over the
outputs and over the final states that are compared.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import kimi_delta_attention_02_amd as kda
from kimi_delta_attention_02_amd import synth

DEV = torch.device("cuda:0")

# tolerances stated for the two arithmetic paths
TOL_F32 = 1e-4
TOL_BF16 = 1e-2


def to_dev(d):
    return {n: (t.to(DEV) if t is not None else None) for n, t in d.items()}


def rel_err(got, ref):
    got = got.detach().cpu().double().numpy() if hasattr(got, "detach") else np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = math.sqrt(float((ref * ref).mean()))
    err = np.abs(got - ref)
    if np.isnan(err).any():
        return float("nan")
    return float(err.max() / rms) if rms > 0 else float(err.max())


def run_chunk(d, w_gate, lower_bound, chunk, initial_state=True):
    g = to_dev(d)
    o, S = kda.chunk_fwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dt_bias"],
                         gate=w_gate, lower_bound=lower_bound, chunk_size=chunk,
                         initial_state=g["S0"] if initial_state else None)
    torch.cuda.synchronize()
    return o, S


def run_decode(d, w_gate, lower_bound, state0):
    """T single-token steps through kda_recurrent_step; returns (o [B,T,HV,V], state)."""
    g = to_dev(d)
    B, T, H, K = d["q"].shape
    HV, V = d["v"].shape[2], d["v"].shape[3]
    state = (state0.to(DEV).clone() if state0 is not None
             else torch.zeros((B, HV, K, V), dtype=torch.float32, device=DEV))
    qs, ks, vs = (g[n].transpose(0, 1).contiguous() for n in ("q", "k", "v"))
    gs, bs = g["g_raw"].transpose(0, 1).contiguous(), g["beta"].transpose(0, 1).contiguous()
    o = torch.empty((T, B, HV, V), dtype=torch.float32, device=DEV)
    for t in range(T):
        kda.recurrent_step(qs[t], ks[t], vs[t], gs[t], bs[t], g["A_log"], g["dt_bias"], state,
                           gate=w_gate, lower_bound=lower_bound, o=o[t])
    torch.cuda.synchronize()
    return o.transpose(0, 1), state


def per_channel_gate(d):
    """A per-head gate (g_raw without the K axis, dt_bias [HV]) written out as
    the per-channel gate it is, every key channel carrying the head's value:
    the form the oracle takes."""
    K = d["q"].shape[-1]
    if d["g_raw"].dim() == d["q"].dim():
        return d
    e = dict(d)
    e["g_raw"] = d["g_raw"].unsqueeze(-1).expand(*d["g_raw"].shape, K).contiguous()
    if d["dt_bias"] is not None:
        e["dt_bias"] = d["dt_bias"].unsqueeze(-1).expand(d["dt_bias"].shape[0], K).contiguous()
    return e


def oracle_full(d, w_gate, lower_bound, initial_state=True):
    d = per_channel_gate(d)
    return oracle.default().kda_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"],
                                    d["dt_bias"], w_gate, lower_bound,
                                    d["S0"] if initial_state else None)


def oracle_heads(d, w_gate, lower_bound, heads):
    d = per_channel_gate(d)
    npf = lambda x: None if x is None else x.float().numpy()
    return oracle.default().kda_fwd_heads(npf(d["q"]), npf(d["k"]), npf(d["v"]), npf(d["g_raw"]),
                                          npf(d["beta"]), npf(d["A_log"]), npf(d["dt_bias"]),
                                          w_gate, lower_bound, npf(d["S0"]), heads)


def sample_heads(B, HV, n, seed=0):
    """n distinct (b, hv) pairs, always including the first and the last."""
    rng = np.random.default_rng(seed)
    allp = [(b, hv) for b in range(B) for hv in range(HV)]
    pick = {allp[0], allp[-1]}
    for i in rng.permutation(len(allp)):
        if len(pick) >= min(n, len(allp)):
            break
        pick.add(allp[i])
    return sorted(pick)


def compare_heads(o, S, ref, tol, what):
    """Errors over the sampled heads, pooled (one RMS per tensor kind)."""
    go, ro, gS, rS = [], [], [], []
    for (b, hv), (o_ref, s_ref) in ref.items():
        go.append(o[b, :, hv].detach().cpu().double().numpy())
        ro.append(o_ref)
        gS.append(S[b, hv].detach().cpu().double().numpy())
        rS.append(s_ref)
    eo = rel_err(np.stack(go), np.stack(ro))
    eS = rel_err(np.stack(gS), np.stack(rS))
    print("%s: max|err|/rms  o %.3e  S %.3e  (tol %.0e, %d heads)" % (what, eo, eS, tol, len(ref)))
    assert eo <= tol, "%s: o error %.3e > %.0e" % (what, eo, tol)
    assert eS <= tol, "%s: state error %.3e > %.0e" % (what, eS, tol)
    return eo, eS


def compare_all_heads(d, w_gate, lower_bound, o, S, tol, what, group=16):
    """Every (b, hv) pair against the oracle, element by element: the oracle
    runs `group` pairs at a time (one per thread) so that host memory stays
    bounded; the error is max |gpu - oracle| over all pairs divided by the RMS
    of the oracle over all pairs, separately for o and the final state."""
    d = per_channel_gate(d)
    npf = lambda x: None if x is None else x.float().numpy()
    args = [npf(d[n]) for n in ("q", "k", "v", "g_raw", "beta", "A_log", "dt_bias")]
    s0 = npf(d["S0"])
    B, HV = d["v"].shape[0], d["v"].shape[2]
    o_cpu, S_cpu = o.detach().cpu(), S.detach().cpu()
    pairs = [(b, hv) for b in range(B) for hv in range(HV)]
    stats = {"o": [0.0, 0.0, 0], "S": [0.0, 0.0, 0]}  # max |err|, sum of squares, count

    def acc(key, got, ref):
        got = got.double().numpy()
        if np.isnan(got).any():
            raise AssertionError("%s: NaN in %s" % (what, key))
        st = stats[key]
        st[0] = max(st[0], float(np.abs(got - ref).max()) if ref.size else 0.0)
        st[1] += float((ref * ref).sum())
        st[2] += ref.size

    orc = oracle.default()
    for i in range(0, len(pairs), group):
        ref = orc.kda_fwd_heads(*args, w_gate, lower_bound, s0, pairs[i:i + group])
        for (b, hv), (o_ref, s_ref) in ref.items():
            acc("o", o_cpu[b, :, hv], o_ref)
            acc("S", S_cpu[b, hv], s_ref)
    err = {k: (v[0] / math.sqrt(v[1] / v[2]) if v[1] > 0 else v[0]) for k, v in stats.items()}
    print("%s: max|err|/rms  o %.3e  S %.3e  (tol %.0e, all %d pairs)" % (what, err["o"], err["S"],
                                                                         tol, len(pairs)))
    assert err["o"] <= tol, "%s: o error %.3e > %.0e" % (what, err["o"], tol)
    assert err["S"] <= tol, "%s: state error %.3e > %.0e" % (what, err["S"], tol)
    return err["o"], err["S"]


def run_split(d, w_gate, lower_bound, chunk, initial_state=True):
    """kda_chunk_fwd_split with the chunk-entry states; returns (o, S, h)."""
    g = to_dev(d)
    o, S, h = kda.chunk_fwd_split(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"],
                                  g["dt_bias"], gate=w_gate, lower_bound=lower_bound,
                                  chunk_size=chunk,
                                  initial_state=g["S0"] if initial_state else None,
                                  output_states=True)
    torch.cuda.synchronize()
    return o, S, h


def oracle_by_chunks(d, w_gate, lower_bound, chunk, initial_state=True, nchunks=None):
    """The oracle's recurrence run chunk after chunk, each chunk starting from
    the state the previous one ended with: (o, final state, h) where
    h[:, :, c] is the state entering chunk c.  With nchunks, only the first
    nchunks chunks are run (o and the state then cover those tokens only)."""
    d = per_channel_gate(d)
    orc = oracle.default()
    B, T, H, K = d["q"].shape
    HV, V = d["v"].shape[2], d["v"].shape[3]
    S = (d["S0"].double().numpy() if (initial_state and d["S0"] is not None)
         else np.zeros((B, HV, K, V)))
    nc = (T + chunk - 1) // chunk
    if nchunks is not None:
        nc = min(nc, nchunks)
    hs, os_ = [], []
    for c in range(nc):
        sl = slice(c * chunk, min(T, (c + 1) * chunk))
        hs.append(S)
        o_c, S = orc.kda_fwd(d["q"][:, sl], d["k"][:, sl], d["v"][:, sl], d["g_raw"][:, sl],
                             d["beta"][:, sl], d["A_log"], d["dt_bias"], w_gate, lower_bound, S)
        os_.append(o_c)
    o = np.concatenate(os_, axis=1) if os_ else np.zeros((B, 0, HV, V))
    h = np.stack(hs, axis=2) if hs else np.zeros((B, HV, 0, K, V))
    return o, S, h
