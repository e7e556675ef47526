"""GPU parity of the per-head (Gated DeltaNet) gate layout through every
entry point: one gate per (token, value head), g_raw without the K axis and
dt_bias [HV].  The oracle takes the same gate written out over the K channels
(tests/kda_testlib.per_channel_gate)."""
import pytest
import torch

import kda_testlib as L
import kimi_delta_attention_02_amd as kda
from kimi_delta_attention_02_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gate", ["safe", "standard", "none"])
@pytest.mark.parametrize("chunk", [0, 16])
def test_head_gate_activation_and_cumsum(gate, chunk):
    d = synth.random_inputs(2, 37, 1, 3, 8, 8, seed=4000 + chunk, per_head_gate=True)
    g = L.to_dev(d)
    out = kda.gate(g["g_raw"], g["A_log"], g["dt_bias"], gate=gate, lower_bound=-5.0,
                   chunk_size=chunk)
    torch.cuda.synchronize()
    e = L.per_channel_gate(d)
    import oracle
    ref = oracle.default().gate(e["g_raw"].numpy(), e["A_log"].numpy(), e["dt_bias"].numpy(),
                                gate, -5.0)[..., 0]
    if chunk:
        T = ref.shape[1]
        ref = ref.copy()
        for c0 in range(0, T, chunk):
            ref[:, c0:c0 + chunk] = ref[:, c0:c0 + chunk].cumsum(axis=1)
    assert out.shape == d["g_raw"].shape
    assert L.rel_err(out, ref) <= 1e-5


HEAD_CASES = [
    # B, T, H, HV, K, dtype, gate, s0, chunk
    (2, 100, 2, 4, 128, "bf16", "safe", True, 64),
    (3, 45, 1, 2, 64, "f32", "standard", False, 32),
    (1, 33, 2, 2, 16, "f32", "safe", True, 16),
    (2, 70, 2, 2, 32, "bf16", "none", True, 64),
]


@pytest.mark.parametrize("B,T,H,HV,K,dtype,gate,s0,chunk", HEAD_CASES)
def test_head_gate_chunk_matches_oracle(B, T, H, HV, K, dtype, gate, s0, chunk):
    d = synth.random_inputs(B, T, H, HV, K, K, seed=4100 + K + T, dtype=dtype,
                            s0_std=0.2 if s0 else 0.0, per_head_gate=True)
    o, S = L.run_chunk(d, gate, -5.0, chunk, initial_state=s0)
    ro, rS = L.oracle_full(d, gate, -5.0, initial_state=s0)
    tol = L.TOL_F32 if dtype == "f32" else L.TOL_BF16
    eo, eS = L.rel_err(o, ro), L.rel_err(S, rS)
    print("head gate chunk %s: o %.2e S %.2e" % ((B, T, H, HV, K, dtype, gate, s0), eo, eS))
    assert eo <= tol and eS <= tol


def test_head_gate_chunk_equals_expanded_per_channel_gate():
    """The per-head kernel against the per-channel kernel fed the same gate on
    every channel: the arithmetic is the same, so the results agree bit for bit."""
    d = synth.random_inputs(2, 77, 2, 4, 128, 128, seed=4200, dtype="bf16", s0_std=0.2,
                            per_head_gate=True)
    a = L.run_chunk(d, "safe", -5.0, 64)
    b = L.run_chunk(L.per_channel_gate(d), "safe", -5.0, 64)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_head_gate_chunk_fast_decay_takes_exact_path():
    """A per-head decay strong enough to leave the 16-token bound runs token by token."""
    d = synth.random_inputs(1, 48, 1, 2, 64, 64, seed=4201, s0_std=0.2, per_head_gate=True,
                            dt_bias_mean=6.0, a_log_std=0.0)
    d["A_log"] = torch.full_like(d["A_log"], 2.0)
    o, S = L.run_chunk(d, "standard", -5.0, 64)
    ro, rS = L.oracle_full(d, "standard", -5.0)
    assert L.rel_err(o, ro) <= L.TOL_F32 and L.rel_err(S, rS) <= L.TOL_F32


@pytest.mark.parametrize("K,V,dtype,gate", [(128, 64, "bf16", "safe"), (32, 128, "f32", "standard"),
                                            (16, 16, "f32", "none")])
def test_head_gate_recurrent_fwd_and_step(K, V, dtype, gate):
    d = synth.random_inputs(3, 21, 1, 3, K, V, seed=4300 + K + V, dtype=dtype, s0_std=0.2,
                            per_head_gate=True)
    g = L.to_dev(d)
    o1, S1 = kda.recurrent_fwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"],
                               g["dt_bias"], gate=gate, lower_bound=-5.0, initial_state=g["S0"])
    o2, S2 = L.run_decode(d, gate, -5.0, d["S0"])
    torch.cuda.synchronize()
    ro, rS = L.oracle_full(d, gate, -5.0)
    for o, S, what in ((o1, S1, "recurrent_fwd"), (o2, S2, "recurrent_step")):
        eo, eS = L.rel_err(o, ro), L.rel_err(S, rS)
        print("head gate %s %s: o %.2e S %.2e" % (what, (K, V, dtype, gate), eo, eS))
        assert eo <= L.TOL_F32 and eS <= L.TOL_F32


def test_deltanet_is_gate_none_with_zero_log_decay():
    """DeltaNet: no decay at all (gate none, g = 0 per head)."""
    d = synth.random_inputs(2, 40, 2, 2, 64, 64, seed=4400, dtype="bf16", s0_std=0.2,
                            per_head_gate=True)
    d["g_raw"] = torch.zeros_like(d["g_raw"])
    o, S = L.run_chunk(d, "none", -5.0, 64)
    ro, rS = L.oracle_full(d, "none", -5.0)
    assert L.rel_err(o, ro) <= L.TOL_BF16 and L.rel_err(S, rS) <= L.TOL_BF16
