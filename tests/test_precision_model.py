"""Why every MFMA operand of the chunk kernel is a pair of bf16 words.

The CPU model in ``precision_model.py`` replays the kernel's 16-token block
algebra ("DeltaNet family" page, "Chunkwise KDA") with each product's
operands rounded as the kernel rounds them, and is compared with the fp64
oracle on the prefill workload's recipe (safe gate, A_log ~ N(0, 0.5),
dt_bias = -4, bf16 q/k/v; one sequence of 1,024 tokens, all 16 value heads).
The bar for the bf16 path is max|err| <= 1e-2 RMS(oracle), for the outputs
and the final state alike; the GPU tests also hold the chunk kernel to a
guard at a tenth of it.

Measured with this model (o / final state):
  float32 operands                 ~1e-6
  hi + lo words everywhere         1.2e-4 / 9.7e-5   (the kernel; GPU: 5-8e-5)
  one word everywhere              6.3e-2 / 4.2e-2   (six times the bar)
  one operand of one product with a single word: 2.8e-3 .. 2.5e-2, i.e. above
  the guard for every product and above the bar for all but the coupling R.
"""
import numpy as np
import pytest

import oracle
import precision_model as pm
from kimi_delta_attention_02_amd import synth

BAR, GUARD = 1e-2, 1e-3


@pytest.fixture(scope="module")
def case():
    w = synth.WORKLOADS["prefill"]
    d = synth.make_inputs(w, B=1, T=1024)
    HV, G = w.HV, w.HV // w.H
    npf = lambda x: None if x is None else x.float().numpy()
    q, k, v, g_raw, beta = (npf(d[n])[0] for n in ("q", "k", "v", "g_raw", "beta"))
    A_log, dt_bias = npf(d["A_log"]), npf(d["dt_bias"])
    heads = [(0, hv) for hv in range(HV)]
    ref = oracle.default().kda_fwd_heads(npf(d["q"]), npf(d["k"]), npf(d["v"]), npf(d["g_raw"]),
                                         npf(d["beta"]), A_log, dt_bias, w.gate, w.lower_bound,
                                         None, heads)
    args = dict(
        q=np.stack([q[:, hv // G] for hv in range(HV)]),
        k=np.stack([k[:, hv // G] for hv in range(HV)]),
        v=np.stack([v[:, hv] for hv in range(HV)]),
        alpha=np.stack([pm.retain_factors(g_raw[:, hv], A_log[hv], dt_bias[hv], w.gate,
                                          w.lower_bound) for hv in range(HV)]),
        beta=np.stack([beta[:, hv] for hv in range(HV)]),
        S0=np.zeros((HV, w.K, w.V), dtype=np.float32))
    ro = np.stack([ref[h][0] for h in heads])
    rS = np.stack([ref[h][1] for h in heads])

    def errors(precision):
        o, S = pm.chunk_forward(precision=precision, **args)
        return pm.max_rel_err(o, ro), pm.max_rel_err(S, rS)

    return errors


def test_bf16_rounding_matches_torch():
    import torch

    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 10.0 ** \
        np.random.default_rng(1).integers(-20, 20, 10000)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(pm.bf16(x), want)


def test_model_algebra_in_fp32(case):
    """Without bf16 rounding the block algebra reproduces the recurrence to
    float32 rounding: the model itself is right."""
    eo, eS = case(pm.FP32)
    assert eo < 2e-5 and eS < 2e-5, (eo, eS)


def test_hi_lo_words_meet_the_guard(case):
    eo, eS = case(pm.KERNEL)
    assert eo < 3e-4 and eS < 3e-4, (eo, eS)


def test_single_words_break_the_bar(case):
    eo, eS = case(pm.SINGLE)
    assert eo > 3 * BAR and eS > 2 * BAR, (eo, eS)


@pytest.mark.parametrize("name", sorted(pm.PRODUCTS))
@pytest.mark.parametrize("side", [0, 1])
def test_each_lo_word_is_needed(case, name, side):
    """Dropping the lo word of either operand of any one product costs more
    than the guard; for every product but R it costs about the whole bar."""
    prec = dict(pm.KERNEL)
    modes = ["hl", "hl"]
    modes[side] = "h"
    prec[name] = tuple(modes)
    eo, eS = case(prec)
    worst = max(eo, eS)
    assert worst > 2 * GUARD, (name, side, eo, eS)
    if name != "R":
        assert worst > 0.4 * BAR, (name, side, eo, eS)
