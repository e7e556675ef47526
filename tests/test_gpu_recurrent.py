"""GPU parity of the fused multi-token recurrent forward (kda_recurrent_fwd)
against the oracle, through the C ABI: shapes with K != V, GVA, both gates
and the gate-free kind, ragged T, T = 0 and T = 1, an aliased state buffer,
agreement with the one-token step and with the chunked path, and the decode
workload at full size as multi-token calls."""
import pytest
import torch

import kda_testlib as L
import kimi_delta_attention_02_amd as kda
from kimi_delta_attention_02_amd import synth

pytestmark = pytest.mark.gpu


def _run(d, gate, lower_bound, initial_state=True, final_state=None):
    g = L.to_dev(d)
    o, S = kda.recurrent_fwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"],
                             g["dt_bias"], gate=gate, lower_bound=lower_bound,
                             initial_state=g["S0"] if initial_state else None,
                             final_state=final_state)
    torch.cuda.synchronize()
    return o, S


REC_CASES = [
    # B, T, H, HV, K, V, dtype, gate, s0
    (2, 37, 2, 4, 128, 128, "bf16", "safe", True),
    (3, 20, 2, 2, 64, 32, "f32", "standard", False),
    (1, 9, 1, 1, 16, 128, "bf16", "safe", True),
    (4, 1, 4, 4, 32, 64, "f32", "safe", True),
    (2, 50, 1, 2, 128, 16, "bf16", "standard", True),
    (3, 24, 3, 3, 16, 16, "f32", "safe", False),
]


@pytest.mark.parametrize("B,T,H,HV,K,V,dtype,gate,s0", REC_CASES)
def test_recurrent_fwd_matches_oracle(B, T, H, HV, K, V, dtype, gate, s0):
    d = synth.random_inputs(B, T, H, HV, K, V, seed=3000 + 7 * K + V + T, dtype=dtype,
                            s0_std=0.2 if s0 else 0.0)
    o, S = _run(d, gate, -5.0, initial_state=s0)
    ro, rS = L.oracle_full(d, gate, -5.0, initial_state=s0)
    eo, eS = L.rel_err(o, ro), L.rel_err(S, rS)
    print("recurrent_fwd %s: o %.2e S %.2e" % ((B, T, H, HV, K, V, dtype, gate, s0), eo, eS))
    assert eo <= L.TOL_F32 and eS <= L.TOL_F32


def test_recurrent_fwd_gate_none_beta_zero_reads_state():
    """beta = 0 and g = 0 (gate none): o_t = s q_t S0 and the state is unchanged."""
    d = synth.random_inputs(2, 6, 1, 2, 64, 32, seed=3101, s0_std=0.3)
    d["beta"] = torch.zeros_like(d["beta"])
    d["g_raw"] = torch.zeros_like(d["g_raw"])
    o, S = _run(d, "none", -5.0)
    ro, rS = L.oracle_full(d, "none", -5.0)
    assert L.rel_err(o, ro) <= L.TOL_F32
    assert torch.equal(S.cpu(), d["S0"])


def test_recurrent_fwd_empty_sequence_copies_state():
    d = synth.random_inputs(2, 0, 2, 2, 32, 64, seed=3102, s0_std=0.5)
    o, S = _run(d, "safe", -5.0)
    assert o.numel() == 0
    assert torch.equal(S.cpu(), d["S0"])
    _, Z = _run(d, "safe", -5.0, initial_state=False)
    assert torch.count_nonzero(Z) == 0


def test_recurrent_fwd_state_in_place():
    """final_state may be the initial_state tensor itself."""
    d = synth.random_inputs(2, 11, 2, 4, 128, 64, seed=3103, dtype="bf16", s0_std=0.2)
    g = L.to_dev(d)
    st = g["S0"].clone()
    o, S = kda.recurrent_fwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"],
                             g["dt_bias"], initial_state=st, final_state=st)
    torch.cuda.synchronize()
    ro, rS = L.oracle_full(d, "safe", -5.0)
    assert S.data_ptr() == st.data_ptr()
    assert L.rel_err(o, ro) <= L.TOL_F32 and L.rel_err(st, rS) <= L.TOL_F32


def test_recurrent_fwd_equals_token_steps_and_chunked():
    """The same 24 tokens as one call, as 24 one-token steps, and chunked."""
    d = synth.random_inputs(3, 24, 2, 4, 128, 128, seed=3104, dtype="bf16", s0_std=0.2)
    o1, S1 = _run(d, "safe", -5.0)
    o2, S2 = L.run_decode(d, "safe", -5.0, d["S0"])
    o3, S3 = L.run_chunk(d, "safe", -5.0, 64)
    ref = lambda x: x.detach().cpu().double().numpy()
    assert L.rel_err(o1, ref(o2)) <= 1e-5 and L.rel_err(S1, ref(S2)) <= 1e-5
    assert L.rel_err(o1, ref(o3)) <= L.TOL_BF16 and L.rel_err(S1, ref(S3)) <= L.TOL_BF16


def test_recurrent_fwd_split_calls_continue():
    """Two calls of 10 and 7 tokens, the state handed over, equal one call of 17
    (up to rounding: a call boundary folds the running decay into the state)."""
    d = synth.random_inputs(2, 17, 1, 2, 64, 64, seed=3105, s0_std=0.2)
    g = L.to_dev(d)
    cut = 10
    part = lambda x, a, b: x[:, a:b].contiguous()
    args = lambda a, b: [part(g[n], a, b) for n in ("q", "k", "v", "g_raw", "beta")]
    oa, Sa = kda.recurrent_fwd(*args(0, cut), g["A_log"], g["dt_bias"], initial_state=g["S0"])
    ob, Sb = kda.recurrent_fwd(*args(cut, 17), g["A_log"], g["dt_bias"], initial_state=Sa)
    o, S = kda.recurrent_fwd(*args(0, 17), g["A_log"], g["dt_bias"], initial_state=g["S0"])
    torch.cuda.synchronize()
    ref = lambda x: x.detach().cpu().double().numpy()
    assert L.rel_err(torch.cat([oa, ob], 1), ref(o)) <= 1e-5 and L.rel_err(Sb, ref(S)) <= 1e-5


@pytest.mark.parametrize("gate", ["safe", "standard", "none"])
def test_recurrent_fwd_strong_and_growing_decay(gate):
    """Decays that drive the running per-row product far past 2^-64 (and, for
    the gate-free kind, past 2^64) within a call: the state is refolded."""
    d = synth.random_inputs(2, 60, 1, 2, 64, 32, seed=3106, s0_std=0.3, g_std=4.0)
    if gate == "none":
        # log-decay drifting upwards (the running product passes 2^64 within the
        # call), with small beta so that the state itself stays within fp32
        d["g_raw"] = d["g_raw"] * 0.125 + 0.9
        d["beta"] = d["beta"] * 0.02
    o, S = _run(d, gate, -20.0)
    ro, rS = L.oracle_full(d, gate, -20.0)
    eo, eS = L.rel_err(o, ro), L.rel_err(S, rS)
    print("recurrent_fwd strong decay %s: o %.2e S %.2e" % (gate, eo, eS))
    assert eo <= L.TOL_F32 and eS <= L.TOL_F32


@pytest.mark.timeout(600)
def test_recurrent_fwd_decode_workload_multi_token():
    """The decode workload (B=256, HV=32, K=V=128, 256 tokens) as 16 calls of
    16 tokens, the state handed from call to call; sampled heads vs the oracle."""
    w = synth.WORKLOADS["decode"]
    d = synth.make_inputs(w)
    g = L.to_dev(d)
    print("decode workload as 16-token calls: B=%d T=%d HV=%d" % (w.B, w.steps, w.HV), flush=True)
    st = g["S0"].clone()
    outs = []
    for c in range(0, w.steps, 16):
        sl = lambda n: g[n][:, c:c + 16].contiguous()
        oc, _ = kda.recurrent_fwd(sl("q"), sl("k"), sl("v"), sl("g_raw"), sl("beta"), g["A_log"],
                                  g["dt_bias"], gate=w.gate, lower_bound=w.lower_bound,
                                  initial_state=st, final_state=st)
        outs.append(oc)
    o = torch.cat(outs, 1)
    torch.cuda.synchronize()
    heads = L.sample_heads(w.B, w.HV, 16, seed=w.seed)
    ref = L.oracle_heads(d, w.gate, w.lower_bound, heads)
    L.compare_heads(o, st, ref, L.TOL_F32, "decode workload, 16-token calls")


@pytest.mark.timeout(600)
def test_large_state_takes_the_streaming_loads():
    """A state above the cached-state size (800 MiB here) is read with
    non-temporal loads by both the one-token step and the multi-token
    forward: the same results as the oracle on sampled heads."""
    w = synth.WORKLOADS["decode"]
    B, T = 400, 3
    d = synth.make_inputs(w, B=B, T=T, seed=77)
    assert B * w.HV * w.K * w.V * 4 > 768 << 20
    print("large state: B=%d HV=%d (%d MiB)" % (B, w.HV, B * w.HV * w.K * w.V * 4 >> 20), flush=True)
    heads = L.sample_heads(B, w.HV, 6, seed=3)
    ref = L.oracle_heads(d, w.gate, w.lower_bound, heads)
    o, S = L.run_decode(d, w.gate, w.lower_bound, d["S0"])
    L.compare_heads(o, S, ref, L.TOL_F32, "large state, one-token steps")
    del o, S
    torch.cuda.empty_cache()
    o, S = _run(d, w.gate, w.lower_bound)
    L.compare_heads(o, S, ref, L.TOL_F32, "large state, one multi-token call")
