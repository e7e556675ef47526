"""Pins for the gradient oracle (oracle/kda_oracle_bwd.c).

The pages give no derivation of the backward pass, so the gradients are fixed
by what mathematics fixes about any correct one:

* central finite differences of the forward oracle (itself pinned by
  ``oracle_pins.py`` against the pages) for every element of every input;
* closed forms where the recurrence reduces to a plain read (g = 0, beta = 0:
  o_t = s q_t S0);
* GVA: the gradient of a shared query/key head is the sum over the value
  heads that read it, as with explicit repeat_interleave'd inputs.

Each ``pin_*(orc)`` raises AssertionError when the oracle ``orc`` disagrees;
``test_oracle_bwd_pins.py`` also runs them on copies with planted mistakes.
"""
from __future__ import annotations

import math

import numpy as np

NAMES = ("q", "k", "v", "g_raw", "beta", "A_log", "dt_bias", "S0")


def _inputs(seed, B=2, T=5, H=1, HV=2, K=4, V=3, gate="safe"):
    r = np.random.default_rng(seed)
    d = {"q": r.standard_normal((B, T, H, K)) * 0.5, "k": r.standard_normal((B, T, H, K)) * 0.5,
         "v": r.standard_normal((B, T, HV, V)),
         "g_raw": r.standard_normal((B, T, HV, K)) * (0.3 if gate == "none" else 1.0),
         "beta": 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, HV)))),
         "A_log": r.standard_normal(HV) * 0.5, "dt_bias": r.standard_normal((HV, K)) - 1.0,
         "S0": r.standard_normal((B, HV, K, V)) * 0.3}
    if gate == "none":
        d["g_raw"] = -np.abs(d["g_raw"])
    return d, r.standard_normal((B, T, HV, V)), r.standard_normal((B, HV, K, V))


def _loss(orc, d, gate, do, dST):
    o, S = orc.kda_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"], d["dt_bias"],
                       gate, -5.0, d["S0"])
    return float((o * do).sum() + (S * dST).sum())


def _grads(orc, d, gate, do, dST):
    return orc.kda_bwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"], d["dt_bias"],
                       gate, -5.0, d["S0"], do, dST)


def pin_bwd_finite_differences(orc):
    """Every gradient element against (L(x + h) - L(x - h)) / 2h, for the three
    gates, under GVA (H = 1, HV = 2), two sequences, an initial state."""
    for seed, gate in ((1, "safe"), (2, "standard"), (3, "none")):
        d, do, dST = _inputs(seed, gate=gate)
        g = _grads(orc, d, gate, do, dST)
        gname = {"q": "dq", "k": "dk", "v": "dv", "g_raw": "dg_raw", "beta": "dbeta",
                 "A_log": "dA_log", "dt_bias": "ddt_bias", "S0": "dS0"}
        for name in NAMES:
            x = d[name]
            flat = x.reshape(-1)
            got = g[gname[name]].reshape(-1)
            for i in range(flat.size):
                h = 1e-6 * max(1.0, abs(flat[i]))
                keep = flat[i]
                flat[i] = keep + h
                lp = _loss(orc, d, gate, do, dST)
                flat[i] = keep - h
                lm = _loss(orc, d, gate, do, dST)
                flat[i] = keep
                fd = (lp - lm) / (2 * h)
                assert abs(fd - got[i]) <= 2e-6 * (1.0 + abs(fd)), \
                    "%s gate, d%s[%d]: %.9g vs finite difference %.9g" % (gate, name, i, got[i], fd)


def pin_bwd_plain_read(orc):
    """g = 0 (gate none) and beta = 0: the state stays S0, o_t = s q_t S0, so
    dq_t = s S0 do_t, dS0 = s sum_t q_t do_t^T + dS_T, dk = dv = 0, and
    dg_t = rowsum(dS_t (.) S0) with dS_t the gradient reaching S_t."""
    d, do, dST = _inputs(7, B=1, T=6, H=1, HV=1, K=5, V=4, gate="none")
    d["g_raw"][:] = 0.0
    d["beta"][:] = 0.0
    g = _grads(orc, d, "none", do, dST)
    s = 1.0 / math.sqrt(5)
    S0 = d["S0"][0, 0]
    for t in range(6):
        assert np.allclose(g["dq"][0, t, 0], s * S0 @ do[0, t, 0], atol=1e-12)
    want = dST[0, 0] + s * sum(np.outer(d["q"][0, t, 0], do[0, t, 0]) for t in range(6))
    assert np.allclose(g["dS0"][0, 0], want, atol=1e-12)
    assert np.abs(g["dk"]).max() == 0.0 and np.abs(g["dv"]).max() == 0.0
    dS = dST[0, 0].copy()
    for t in range(5, -1, -1):
        dS = dS + s * np.outer(d["q"][0, t, 0], do[0, t, 0])
        assert np.allclose(g["dg_raw"][0, t, 0], (dS * S0).sum(axis=1), atol=1e-12)


def pin_bwd_gva_sum(orc):
    """A query/key head shared by two value heads gets the sum of what
    explicit copies of it would get."""
    d, do, dST = _inputs(11, B=2, T=4, H=1, HV=2, K=3, V=4, gate="standard")
    g = _grads(orc, d, "standard", do, dST)
    e = dict(d)
    e["q"] = np.repeat(d["q"], 2, axis=2)
    e["k"] = np.repeat(d["k"], 2, axis=2)
    ge = _grads(orc, e, "standard", do, dST)
    assert np.allclose(g["dq"][:, :, 0], ge["dq"].sum(axis=2), atol=1e-12)
    assert np.allclose(g["dk"][:, :, 0], ge["dk"].sum(axis=2), atol=1e-12)
    for n in ("dv", "dbeta", "dg_raw", "dA_log", "ddt_bias", "dS0"):
        assert np.allclose(g[n], ge[n], atol=1e-12), n


ALL_PINS = [pin_bwd_finite_differences, pin_bwd_plain_read, pin_bwd_gva_sum]
