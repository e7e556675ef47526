"""GPU parity of the backward pass (kda_bwd through the C ABI) against the
fp64 gradient oracle, every gradient tensor element by element.

Bar: max |gpu - oracle| <= 1e-4 * RMS(oracle) per gradient tensor.  The GPU
path computes in fp32 throughout (bf16 inputs are widened exactly, the
forward that writes the segment states runs its fp32 products), so the fp32
bar holds for bf16 inputs too; dA_log, a sum over every token and channel of
a sequence, is held to the same bar relative to its own RMS.
"""
import math

import numpy as np
import pytest
import torch

import kda_testlib as L
import kimi_delta_attention_02_amd as kda
import oracle
from kimi_delta_attention_02_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-4
NAMES = ("dq", "dk", "dv", "dbeta", "dg_raw", "dA_log", "ddt_bias", "dS0")


def _case(B, T, H, HV, K, *, gate, dtype="f32", seed=0, s0=True, dst=True, bias=True):
    d = synth.random_inputs(B, T, H, HV, K, K, seed=seed, dtype=dtype, s0_std=0.3 if s0 else 0.0)
    if gate == "none":  # the caller's own log-decay: keep it negative and moderate
        d["g_raw"] = -0.2 * d["g_raw"].abs()
    if not bias:
        d["dt_bias"] = None
    gen = torch.Generator().manual_seed(1000 + seed)
    dout = torch.randn((B, T, HV, K), generator=gen)
    dST = torch.randn((B, HV, K, K), generator=gen) if dst else None
    return d, dout, dST


def _run(d, dout, dST, gate):
    g = L.to_dev(d)
    print("bwd: shape q %s v %s gate %s dtype %s S0 %s dST %s" % (
        tuple(d["q"].shape), tuple(d["v"].shape), gate, d["q"].dtype, d["S0"] is not None,
        dST is not None), flush=True)
    got = kda.bwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dt_bias"],
                  gate=gate, lower_bound=-5.0, initial_state=g["S0"], dout=dout.to(L.DEV),
                  dfinal_state=None if dST is None else dST.to(L.DEV), want_dinitial_state=True,
                  want_ddt_bias=d["dt_bias"] is not None)
    torch.cuda.synchronize()
    ref = oracle.default().kda_bwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"],
                                   d["dt_bias"], gate, -5.0, d["S0"], dout, dST)
    return got, ref


def _compare(got, ref, what, tol=TOL):
    errs = {}
    for n in NAMES:
        if ref.get(n) is None or got.get(n) is None:
            continue
        g = got[n].detach().cpu().double().numpy()
        r = np.asarray(ref[n])
        assert g.shape == r.shape, (n, g.shape, r.shape)
        assert not np.isnan(g).any(), "%s: NaN in %s" % (what, n)
        if r.size == 0:
            continue
        rms = math.sqrt(float((r * r).mean()))
        err = float(np.abs(g - r).max())
        errs[n] = err / rms if rms > 0 else err
    print("%s: max|err|/rms %s" % (what, "  ".join("%s %.2e" % kv for kv in errs.items())))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, "%s: over %.0e: %s" % (what, tol, bad)
    return errs


@pytest.mark.parametrize("gate", ["safe", "standard", "none"])
@pytest.mark.parametrize("K", [32, 64, 128])
def test_bwd_gates_and_head_sizes(gate, K):
    """Two sequences, GVA (H = 2, HV = 4), 37 tokens (two full 16-token
    segments and a ragged one), initial state and dL/dS_T."""
    d, dout, dST = _case(2, 37, 2, 4, K, gate=gate, seed=K + len(gate))
    got, ref = _run(d, dout, dST, gate)
    _compare(got, ref, "%s K=%d" % (gate, K))


@pytest.mark.parametrize("gate", ["safe", "standard"])
def test_bwd_bf16_inputs(gate):
    d, dout, dST = _case(1, 70, 1, 4, 128, gate=gate, dtype="bf16", seed=5)
    got, ref = _run(d, dout, dST, gate)
    _compare(got, ref, "bf16 %s" % gate)


def test_bwd_no_initial_state_no_final_grad_no_bias():
    d, dout, dST = _case(2, 40, 1, 2, 64, gate="safe", seed=9, s0=False, dst=False, bias=False)
    got, ref = _run(d, dout, dST, "safe")
    _compare(got, ref, "plain")


@pytest.mark.parametrize("T", [1, 15, 16, 17, 48])
def test_bwd_segment_boundaries(T):
    d, dout, dST = _case(1, T, 2, 2, 32, gate="standard", seed=20 + T)
    got, ref = _run(d, dout, dST, "standard")
    _compare(got, ref, "T=%d" % T)


def test_bwd_longer_sequence():
    """600 tokens (38 segments), K = 128, a GVA group of four value heads."""
    d, dout, dST = _case(1, 600, 1, 4, 128, gate="safe", dtype="bf16", seed=31)
    got, ref = _run(d, dout, dST, "safe")
    _compare(got, ref, "T=600")


def test_bwd_empty_sequence_passes_final_grad_through():
    """T = 0: dL/dS_0 = dL/dS_T, the per-head sums are zero."""
    B, H, HV, K = 2, 1, 2, 32
    d = synth.random_inputs(B, 0, H, HV, K, K, seed=3, s0_std=0.3)
    g = L.to_dev(d)
    dST = torch.randn((B, HV, K, K), device=L.DEV)
    got = kda.bwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dt_bias"],
                  gate="safe", lower_bound=-5.0, initial_state=g["S0"],
                  dout=torch.zeros((B, 0, HV, K), device=L.DEV), dfinal_state=dST)
    torch.cuda.synchronize()
    assert torch.equal(got["dS0"], dST)
    assert torch.count_nonzero(got["dA_log"]) == 0 and torch.count_nonzero(got["ddt_bias"]) == 0


def test_bwd_zero_cotangent_gives_zero_gradients():
    """dL/do = 0 and dL/dS_T = 0: every gradient is exactly zero."""
    d, dout, _ = _case(1, 33, 1, 2, 64, gate="safe", seed=4)
    g = L.to_dev(d)
    got = kda.bwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dt_bias"],
                  gate="safe", lower_bound=-5.0, initial_state=g["S0"],
                  dout=torch.zeros_like(dout, device=L.DEV))
    torch.cuda.synchronize()
    for n, t in got.items():
        if t is not None:
            assert torch.count_nonzero(t) == 0, n


def test_bwd_unsupported_and_invalid():
    d = L.to_dev(synth.random_inputs(1, 8, 1, 1, 16, 16, seed=1))
    dout = torch.zeros((1, 8, 1, 16), device=L.DEV)
    with pytest.raises(kda.KDAError, match="UNSUPPORTED"):
        kda.bwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"], d["dt_bias"],
                dout=dout)


def test_bwd_strong_decay_takes_the_per_token_path():
    """Safe gate with L = -20 and a wide g_raw: many 16-token segments decay
    below 2^-100 in some channel and run the per-token key sums; the others
    run the matrix form.  Both must match the oracle."""
    d, dout, dST = _case(1, 120, 2, 4, 64, gate="safe", seed=41)
    d["g_raw"] = d["g_raw"] * 4.0 + 4.0
    g = L.to_dev(d)
    got = kda.bwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dt_bias"],
                  gate="safe", lower_bound=-20.0, initial_state=g["S0"], dout=dout.to(L.DEV),
                  dfinal_state=dST.to(L.DEV))
    torch.cuda.synchronize()
    ref = oracle.default().kda_bwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"],
                                   d["dt_bias"], "safe", -20.0, d["S0"], dout, dST)
    _compare(got, ref, "strong decay")


def test_bwd_growth_gate_none():
    """Gate none with positive log-decays inside segments (the cumulative
    factor grows above 1, within the matrix form's range)."""
    d, dout, dST = _case(1, 64, 1, 2, 32, gate="none", seed=43)
    gen = torch.Generator().manual_seed(44)
    d["g_raw"] = 0.15 * torch.randn(d["g_raw"].shape, generator=gen)
    got, ref = _run(d, dout, dST, "none")
    _compare(got, ref, "growth")


@pytest.mark.timeout(600)
def test_bwd_workload_prefill_all_heads():
    """The backward at the size the benchmark times it (the prefill workload:
    B = 4, T = 4096, H = HV = 16, K = V = 128, bf16, safe gate), one call on
    the whole input.  The oracle recomputes every value head, one at a time
    (all four sequences over their whole length, which bounds host memory),
    so every gradient, including the sums over the sequences (A_log,
    dt_bias), is compared element by element; the bar applies per head and
    tensor."""
    w = synth.WORKLOADS["prefill"]
    d = synth.make_inputs(w)
    gen = torch.Generator().manual_seed(77)
    dout = torch.randn((w.B, w.T, w.HV, w.V), generator=gen)
    g = L.to_dev(d)
    print("bwd prefill: B=%d T=%d HV=%d K=%d" % (w.B, w.T, w.HV, w.K), flush=True)
    got = kda.bwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dt_bias"],
                  gate=w.gate, lower_bound=w.lower_bound, dout=dout.to(L.DEV))
    torch.cuda.synchronize()
    got = {n: (t.cpu() if t is not None else None) for n, t in got.items()}
    assert w.H == w.HV
    ref_alog, ref_bias = np.zeros(w.HV), np.zeros((w.HV, w.K))
    for hv in range(w.HV):
        sl = slice(hv, hv + 1)
        sub = lambda x, ax: x.narrow(ax, hv, 1) if x is not None else None
        ref = oracle.default().kda_bwd(sub(d["q"], 2), sub(d["k"], 2), sub(d["v"], 2),
                                       sub(d["g_raw"], 2), sub(d["beta"], 2), d["A_log"][sl],
                                       d["dt_bias"][sl], w.gate, w.lower_bound, None,
                                       dout[:, :, sl], None)
        mine = {"dq": got["dq"][:, :, sl], "dk": got["dk"][:, :, sl], "dv": got["dv"][:, :, sl],
                "dbeta": got["dbeta"][:, :, sl], "dg_raw": got["dg_raw"][:, :, sl]}
        ref_alog[hv], ref_bias[hv] = ref["dA_log"][0], ref["ddt_bias"][0]
        ref["dA_log"] = ref["ddt_bias"] = ref["dS0"] = None
        _compare(mine, ref, "prefill head %d" % hv)
    # the per-head sums over all tokens, as whole tensors (one scalar per head
    # for A_log: its RMS over the heads, like every other gradient here)
    _compare({"dA_log": got["dA_log"], "ddt_bias": got["ddt_bias"]},
             {"dA_log": ref_alog, "ddt_bias": ref_bias}, "prefill per-head sums")


@pytest.mark.parametrize("gate", ["safe", "standard", "none"])
def test_bwd_per_head_gate(gate):
    """One gate value per (token, value head), broadcast over the key channels
    (Gated DeltaNet's scalar gate): against the oracle run on the gate written
    out per channel, whose g_raw and dt_bias gradients sum over the channels."""
    d = synth.random_inputs(2, 37, 2, 4, 64, 64, seed=50, s0_std=0.3, per_head_gate=True)
    if gate == "none":
        d["g_raw"] = -0.2 * d["g_raw"].abs()
    gen = torch.Generator().manual_seed(51)
    dout = torch.randn((2, 37, 4, 64), generator=gen)
    dST = torch.randn((2, 4, 64, 64), generator=gen)
    g = L.to_dev(d)
    got = kda.bwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dt_bias"],
                  gate=gate, lower_bound=-5.0, initial_state=g["S0"], dout=dout.to(L.DEV),
                  dfinal_state=dST.to(L.DEV))
    torch.cuda.synchronize()
    assert got["dg_raw"].shape == (2, 37, 4) and got["ddt_bias"].shape == (4,)
    e = L.per_channel_gate(d)
    ref = oracle.default().kda_bwd(e["q"], e["k"], e["v"], e["g_raw"], e["beta"], e["A_log"],
                                   e["dt_bias"], gate, -5.0, e["S0"], dout, dST)
    ref["dg_raw"] = ref["dg_raw"].sum(axis=-1)
    ref["ddt_bias"] = ref["ddt_bias"].sum(axis=-1)
    _compare(got, ref, "per-head %s" % gate)
