"""The CPU oracle against its pins, and the pins against planted mistakes."""
import os

import numpy as np
import pytest

import oracle
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_oracle_rejects_bad_arguments(orc):
    z = np.zeros((1, 2, 2, 4))
    with pytest.raises(ValueError):  # HV (3) not a multiple of H (2)
        orc.kda_fwd(z, z, np.zeros((1, 2, 3, 4)), np.zeros((1, 2, 3, 4)), np.zeros((1, 2, 3)),
                    np.zeros(3), None, "none")
    with pytest.raises(KeyError):
        orc.gate(z, np.zeros(2), None, "bogus")


def test_oracle_empty_sequence(orc):
    """T = 0: no tokens, the final state is the initial state."""
    S0 = np.random.default_rng(0).standard_normal((1, 2, 3, 4))
    o, S = orc.kda_fwd(np.zeros((1, 0, 1, 3)), np.zeros((1, 0, 1, 3)), np.zeros((1, 0, 2, 4)),
                       np.zeros((1, 0, 2, 3)), np.zeros((1, 0, 2)), np.zeros(2), None, "safe",
                       -5.0, S0)
    assert o.shape == (1, 0, 2, 4)
    assert np.array_equal(S, S0)


def test_heads_slicing_matches_full_run(orc):
    """kda_fwd_heads (one (b, hv) pair at a time) equals the full run."""
    d = P._inputs(40, B=2, T=7, H=2, HV=4, K=5, V=3)
    o, S = orc.kda_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"], d["dt_bias"],
                       "standard", -5.0, d["S0"])
    heads = [(0, 0), (1, 3), (1, 2)]
    got = orc.kda_fwd_heads(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"],
                            d["dt_bias"], "standard", -5.0, d["S0"], heads)
    for (b, hv) in heads:
        assert np.array_equal(got[(b, hv)][0], o[b, :, hv])
        assert np.array_equal(got[(b, hv)][1], S[b, hv])


# Planted mistakes: name -> list of (text in kda_oracle.c, replacement).
# Each is a plausible slip (dropped term, wrong sign, wrong index, transposed
# operand, wrong order); the pins must catch every one.
_READ = ("    for (long j = 0; j < V; ++j) { double acc = 0.0;"
         " for (long c = 0; c < K; ++c) acc += qt[c] * S[c * V + j]; ot[j] = scale * acc; }\n")
MUTANTS = {
    "drop read scale": [("ot[j] = scale * acc;", "ot[j] = acc;")],
    "residual sign": [("p[j] = vt[j] - p[j];", "p[j] = vt[j] + p[j];")],
    "predict before decay": [("p[j] += kt[c] * S[c * V + j];",
                              "p[j] += kt[c] * S[c * V + j] / alpha[c];")],
    "write with query": [("double a = bt * kt[c];", "double a = bt * qt[c];")],
    "drop beta": [("double a = bt * kt[c];", "double a = kt[c];")],
    "read with key": [("acc += qt[c] * S[c * V + j];", "acc += kt[c] * S[c * V + j];")],
    "decay on value index": [("S[c * V + j] *= alpha[c];", "S[c * V + j] *= alpha[j % K];")],
    "GVA tiled instead of interleaved": [("const long h = hv / (HV / H);",
                                          "const long h = hv % H;")],
    "rate outside sigmoid": [("return L * sigmoid(rate * input);",
                              "return rate * L * sigmoid(input);")],
    "softplus of negated input": [("return -rate * softplus(input);",
                                   "return -rate * softplus(-input);")],
    "dt_bias ignored": [("double input = graw + bias;", "double input = graw;")],
    "decay without exp": [("alpha[c] = exp(gate_one(", "alpha[c] = (gate_one(")],
    "initial state ignored": [(
        "memcpy(S, J->S0 + (b * HV + hv) * K * V, sizeof(double) * K * V);",
        "memset(S, 0, sizeof(double) * K * V);")],
    # the read moves above the write (o_t would miss token t's own write)
    "read before write": [("    /* 3. rank-1 write", _READ + "    /* 3. rank-1 write"),
                          ("      ot[j] = scale * acc;\n", "      (void)acc;\n")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    text = open(oracle.SOURCE).read()
    for old, new in MUTANTS[name]:
        assert text.count(old) == 1, "mutation anchor not unique: %r" % old
        text = text.replace(old, new)
    mutant = oracle.build_variant(text, str(tmp_path))
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "no pin caught the planted mistake %r" % name
