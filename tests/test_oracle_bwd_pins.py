"""The gradient oracle against its pins, and the pins against planted mistakes."""
import numpy as np
import pytest

import oracle
import oracle_bwd_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(orc, pin):
    pin(orc)


def test_bwd_threads_do_not_change_the_result(orc):
    d, do, dST = P._inputs(5, B=3, T=9, H=2, HV=4, K=4, V=5)
    a = orc.kda_bwd(*[d[n] for n in P.NAMES[:7]], "safe", -5.0, d["S0"], do, dST, threads=1)
    b = orc.kda_bwd(*[d[n] for n in P.NAMES[:7]], "safe", -5.0, d["S0"], do, dST, threads=5)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


# Planted mistakes in kda_oracle_bwd.c: (text, replacement); the pins must
# catch each one.
MUTANTS = {
    "dk without the prediction term": [("dkt[c] += be * a - pr;", "dkt[c] += be * a;")],
    "dr without beta": [("dr[j] = be * a;", "dr[j] = a;")],
    "state gradient not decayed": [("dS[c * V + j] = al * dSd[c * V + j];",
                                    "dS[c * V + j] = dSd[c * V + j];")],
    "read gradient without scale": [("dS[c * V + j] += s * qt[c] * dot[j];",
                                     "dS[c * V + j] += qt[c] * dot[j];")],
    "safe-gate derivative without rate": [("*dg_dx = L * sg * (1.0 - sg) * rate;",
                                           "*dg_dx = L * sg * (1.0 - sg);")],
    "dq from the state before the write": [("acc += St[c * V + j] * dot[j];",
                                            "acc += Sp[c * V + j] * dot[j];")],
    "dSd sign": [("dSd[c * V + j] = dS[c * V + j] - kt[c] * dr[j];",
                  "dSd[c * V + j] = dS[c * V + j] + kt[c] * dr[j];")],
    "dt_bias gradient under the none gate": [
        ("if (J->kind != BWD_GATE_NONE) dbias[c] += dg * dgx[t * K + c];",
         "dbias[c] += dg * dgx[t * K + c];")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_pins_catch_planted_mistake(tmp_path, name):
    text = open(oracle.BWD_SOURCE).read()
    for old, new in MUTANTS[name]:
        assert text.count(old) == 1, "mutation anchor not unique: %r" % old
        text = text.replace(old, new)
    mutant = oracle.build_bwd_variant(text, str(tmp_path))
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "no pin caught the planted mistake %r" % name
