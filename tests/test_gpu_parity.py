"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars: fp32 paths max|err| <= 1e-4 * RMS(oracle); bf16-MFMA chunked path
<= 1e-2 * RMS, for outputs and final states alike.
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


# ------------------------------------------------------------------- gate

@pytest.mark.parametrize("gate", ["safe", "standard", "none"])
@pytest.mark.parametrize("chunk", [0, 16, 64])
def test_gate_matches_oracle(gate, chunk):
    d = synth.random_inputs(2, 150, 2, 6, 32, 32, seed=10, g_std=3.0)
    g = L.to_dev(d)
    bias = g["dt_bias"] if gate != "none" else None
    got = kda.gate(g["g_raw"], g["A_log"], bias, gate=gate, lower_bound=-5.0, chunk_size=chunk)
    ref = oracle.default().gate(d["g_raw"], d["A_log"], d["dt_bias"] if gate != "none" else None,
                                gate, -5.0)
    if chunk:
        T = ref.shape[1]
        ref = np.concatenate([np.cumsum(ref[:, s:s + chunk], axis=1) for s in range(0, T, chunk)], 1)
    err = np.abs(got.cpu().double().numpy() - ref).max()
    bound = 2e-6 * max(1.0, np.abs(ref).max())
    assert err <= bound, (err, bound)


@pytest.mark.parametrize("K", [5, 32])
@pytest.mark.parametrize("chunk", [0, 16])
def test_gate_in_place_both_layouts(K, chunk):
    """g_out aliasing g_raw, for a K that takes the per-channel layout (5) and
    one that takes the four-channel one (32); T = 150 leaves ragged chunks."""
    d = synth.random_inputs(2, 150, 2, 6, K, K, seed=11, g_std=3.0)
    g = L.to_dev(d)
    ref = oracle.default().gate(d["g_raw"], d["A_log"], d["dt_bias"], "safe", -5.0)
    if chunk:
        T = ref.shape[1]
        ref = np.concatenate([np.cumsum(ref[:, s:s + chunk], axis=1) for s in range(0, T, chunk)], 1)
    buf = g["g_raw"].clone()
    got = kda.gate(buf, g["A_log"], g["dt_bias"], gate="safe", lower_bound=-5.0, chunk_size=chunk, out=buf)
    assert got.data_ptr() == buf.data_ptr()
    err = np.abs(buf.cpu().double().numpy() - ref).max()
    assert err <= 2e-6 * max(1.0, np.abs(ref).max()), err


def test_gate_printed_default_value():
    """Defaults table of the gate section: g ~ -0.09, exp(g) ~ 0.91."""
    g_raw = torch.zeros((1, 1, 1, 1), device=L.DEV)
    g = kda.gate(g_raw, torch.zeros(1, device=L.DEV), torch.full((1, 1), -4.0, device=L.DEV),
                 gate="safe", lower_bound=-5.0).item()
    assert abs(g - (-5.0 / (1.0 + math.exp(4.0)))) < 1e-6
    assert abs(g + 0.09) < 0.005 and abs(math.exp(g) - 0.91) < 0.005


def test_gate_nan_propagates():
    g_raw = torch.full((1, 2, 1, 4), float("nan"), device=L.DEV)
    for gate in ("safe", "standard"):
        g = kda.gate(g_raw, torch.zeros(1, device=L.DEV), None, gate=gate, lower_bound=-5.0)
        assert torch.isnan(g).all()


# ------------------------------------------------------------- tiny (fp32)

def test_tiny_chunked_fp32():
    w = synth.WORKLOADS["tiny"]
    d = synth.make_inputs(w)
    o, S = L.run_chunk(d, w.gate, w.lower_bound, w.chunk)
    ro, rS = L.oracle_full(d, w.gate, w.lower_bound)
    eo, eS = L.rel_err(o, ro), L.rel_err(S, rS)
    print("tiny chunked: o %.2e S %.2e" % (eo, eS))
    assert eo <= L.TOL_F32 and eS <= L.TOL_F32


def test_tiny_recurrent_fp32():
    w = synth.WORKLOADS["tiny"]
    d = synth.make_inputs(w)
    o, S = L.run_decode(d, w.gate, w.lower_bound, None)
    ro, rS = L.oracle_full(d, w.gate, w.lower_bound)
    eo, eS = L.rel_err(o, ro), L.rel_err(S, rS)
    print("tiny recurrent: o %.2e S %.2e" % (eo, eS))
    assert eo <= L.TOL_F32 and eS <= L.TOL_F32


# ------------------------------------------------- chunked: shapes and edges

CHUNK_CASES = [
    # B, T, H, HV, K, dtype, gate, S0, chunk
    (1, 16, 1, 1, 16, "f32", "safe", False, 16),
    (2, 70, 2, 2, 16, "f32", "standard", True, 16),      # ragged tail
    (1, 45, 1, 2, 32, "f32", "safe", True, 32),
    (2, 33, 2, 4, 64, "f32", "standard", True, 64),
    (1, 100, 2, 2, 128, "f32", "safe", True, 64),
    (1, 48, 1, 1, 16, "bf16", "safe", True, 16),
    (2, 77, 1, 3, 32, "bf16", "standard", True, 16),
    (1, 130, 2, 4, 64, "bf16", "safe", False, 32),
    (2, 257, 2, 4, 128, "bf16", "safe", True, 64),
    (1, 1000, 1, 2, 128, "bf16", "standard", True, 64),
    (3, 1, 1, 1, 128, "bf16", "safe", True, 64),          # one token
]


# A tenth of the bf16 bar: the hi/lo pairs hold the measured errors near 1e-4
# (a single bf16 rounding of any derived operand would cost 2-6e-2), so a
# change that drops a lo word shows here long before the bar itself is hit.
BF16_GUARD = 1e-3


@pytest.mark.parametrize("B,T,H,HV,K,dtype,gate,s0,chunk", CHUNK_CASES)
def test_chunk_matches_oracle(B, T, H, HV, K, dtype, gate, s0, chunk):
    d = synth.random_inputs(B, T, H, HV, K, K, seed=1000 + T + K, dtype=dtype,
                            s0_std=0.3 if s0 else 0.0)
    o, S = L.run_chunk(d, gate, -5.0, chunk)
    ro, rS = L.oracle_full(d, gate, -5.0)
    tol = L.TOL_F32 if dtype == "f32" else L.TOL_BF16
    eo, eS = L.rel_err(o, ro), L.rel_err(S, rS)
    print("chunk %s: o %.2e S %.2e" % ((B, T, H, HV, K, dtype, gate, s0, chunk), eo, eS))
    assert eo <= tol and eS <= tol
    if dtype == "bf16":  # the hi/lo operand pairs keep this near 1e-4: guard a tenth of the bar
        assert eo <= BF16_GUARD and eS <= BF16_GUARD, (eo, eS)


def test_chunk_empty_sequence_copies_state():
    d = synth.random_inputs(2, 0, 1, 2, 32, 32, seed=5, s0_std=1.0)
    o, S = L.run_chunk(d, "safe", -5.0, 64)
    assert o.shape == (2, 0, 2, 32)
    assert torch.equal(S.cpu(), d["S0"])
    d["S0"] = None
    o, S = L.run_chunk(d, "safe", -5.0, 64)
    assert torch.count_nonzero(S) == 0


def test_chunk_beta_zero_and_gate_none():
    """beta = 0 with g = 0 (gate 'none'): the state is untouched and every
    output is the plain read (1/sqrt(K)) q S0."""
    d = synth.random_inputs(1, 40, 2, 4, 64, 64, seed=7, dtype="f32", s0_std=0.5)
    d["beta"].zero_()
    d["g_raw"].zero_()
    o, S = L.run_chunk(d, "none", -5.0, 16)
    q = d["q"].double()
    want = torch.einsum("bthk,bhkv->bthv", q.repeat_interleave(2, dim=2), d["S0"].double()) / 8.0
    assert L.rel_err(o, want.numpy()) <= L.TOL_F32
    assert torch.equal(S.cpu(), d["S0"])


def test_chunk_fast_decay_takes_exact_path():
    """Standard gate with huge inputs: 16-token decay spans far beyond what the
    factored intra-block products can hold; those blocks run token by token."""
    d = synth.random_inputs(1, 64, 1, 2, 32, 32, seed=8, dtype="f32", s0_std=0.5)
    d["g_raw"][:, 20:40] += 25.0  # softplus ~ 21 per token -> ~340 nats per block
    o, S = L.run_chunk(d, "standard", -5.0, 16)
    ro, rS = L.oracle_full(d, "standard", -5.0)
    assert L.rel_err(o, ro) <= L.TOL_F32 and L.rel_err(S, rS) <= L.TOL_F32
    d["q"], d["k"], d["v"] = (d[n].to(torch.bfloat16) for n in ("q", "k", "v"))
    o, S = L.run_chunk(d, "standard", -5.0, 16)
    ro, rS = L.oracle_full(d, "standard", -5.0)
    assert L.rel_err(o, ro) <= L.TOL_BF16 and L.rel_err(S, rS) <= L.TOL_BF16


def test_chunk_nan_propagates():
    d = synth.random_inputs(1, 32, 1, 1, 32, 32, seed=9, dtype="bf16")
    d["g_raw"][0, 5, 0, 3] = float("nan")
    o, S = L.run_chunk(d, "safe", -5.0, 16)
    assert torch.isnan(o[0, 5:]).any() and torch.isnan(S).any()
    assert not torch.isnan(o[0, :5]).any()


def test_chunk_gva_equals_repeated_heads():
    d = synth.random_inputs(2, 80, 2, 6, 64, 64, seed=11, dtype="bf16", s0_std=0.1)
    o1, S1 = L.run_chunk(d, "safe", -5.0, 64)
    d2 = dict(d)
    d2["q"] = d["q"].repeat_interleave(3, dim=2).contiguous()
    d2["k"] = d["k"].repeat_interleave(3, dim=2).contiguous()
    o2, S2 = L.run_chunk(d2, "safe", -5.0, 64)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_chunk_split_continuation_and_decode_handoff():
    """Prefill T1 tokens, continue with T2 more from the returned state, then
    decode T3 single steps: equals the oracle over T1 + T2 + T3 tokens."""
    d = synth.random_inputs(2, 200, 2, 4, 128, 128, seed=12, dtype="bf16", s0_std=0.05)
    part = lambda a, b: {n: (t[:, a:b].contiguous() if n not in ("A_log", "dt_bias", "S0") else t)
                         for n, t in d.items()}
    o1, S1 = L.run_chunk(part(0, 100), "safe", -5.0, 64)
    p2 = part(100, 180)
    p2["S0"] = S1.cpu()
    o2, S2 = L.run_chunk(p2, "safe", -5.0, 64)
    o3, S3 = L.run_decode(part(180, 200), "safe", -5.0, S2)
    ro, rS = L.oracle_full(d, "safe", -5.0)
    o = torch.cat([o1, o2, o3], dim=1)
    assert L.rel_err(o, ro) <= L.TOL_BF16 and L.rel_err(S3, rS) <= L.TOL_BF16


@pytest.mark.parametrize("K,dtype", [(128, "bf16"), (64, "f32")])
def test_chunk_state_in_place(K, dtype):
    """final_state may be the initial_state tensor itself: each workgroup reads
    its columns of the state before any of them is written back."""
    d = synth.random_inputs(2, 150, 2, 4, K, K, seed=14 + K, dtype=dtype, s0_std=0.3)
    g = L.to_dev(d)
    st = g["S0"].clone()
    o, S = kda.chunk_fwd(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dt_bias"],
                         gate="standard", lower_bound=-5.0, chunk_size=64, initial_state=st,
                         final_state=st)
    torch.cuda.synchronize()
    ro, rS = L.oracle_full(d, "standard", -5.0)
    tol = L.TOL_F32 if dtype == "f32" else L.TOL_BF16
    assert S.data_ptr() == st.data_ptr()
    assert L.rel_err(o, ro) <= tol and L.rel_err(st, rS) <= tol


def test_chunk_deterministic():
    d = synth.random_inputs(1, 300, 2, 4, 128, 128, seed=13, dtype="bf16", s0_std=0.05)
    a = L.run_chunk(d, "safe", -5.0, 64)
    b = L.run_chunk(d, "safe", -5.0, 64)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------ recurrent: shapes

DECODE_CASES = [
    (3, 20, 1, 2, 16, 16, "f32"),
    (2, 12, 2, 2, 32, 64, "f32"),
    (2, 12, 1, 3, 128, 32, "f32"),
    (4, 16, 2, 4, 64, 128, "bf16"),
    (2, 30, 2, 2, 128, 128, "bf16"),
]


@pytest.mark.parametrize("B,T,H,HV,K,V,dtype", DECODE_CASES)
def test_decode_matches_oracle(B, T, H, HV, K, V, dtype):
    d = synth.random_inputs(B, T, H, HV, K, V, seed=2000 + K + V, dtype=dtype, s0_std=0.2)
    o, S = L.run_decode(d, "safe", -5.0, d["S0"])
    ro, rS = L.oracle_full(d, "safe", -5.0)
    eo, eS = L.rel_err(o, ro), L.rel_err(S, rS)
    print("decode %s: o %.2e S %.2e" % ((B, T, H, HV, K, V, dtype), eo, eS))
    assert eo <= L.TOL_F32 and eS <= L.TOL_F32


@pytest.mark.parametrize("K,dtype", [(16, "f32"), (128, "bf16")])
def test_mixed_sign_decay_inside_a_block(K, dtype):
    """Gate none with a log-decay of +15 then -15 per token inside a block,
    entered with a zero state and beta = 0 up to the end of the growth: the
    block's total decay is 1, but the partial products reach e^120, beyond
    what the factorised form can hold, so the block must run token by token.
    The recurrence stays finite."""
    d = synth.random_inputs(1, 64, 2, 4, K, K, seed=31, dtype=dtype, s0_std=0.0)
    g = torch.zeros_like(d["g_raw"])
    g[:, 16:24] = 15.0
    g[:, 24:32] = -15.0
    d["g_raw"] = g
    beta = d["beta"].clone()
    beta[:, :24] = 0.0
    d["beta"] = beta
    print("mixed-sign decay: K=%d %s" % (K, dtype), flush=True)
    o, S = L.run_chunk(d, "none", -5.0, 64)
    ro, rS = L.oracle_full(d, "none", -5.0)
    tol = L.TOL_F32 if dtype == "f32" else L.TOL_BF16
    eo, eS = L.rel_err(o, ro), L.rel_err(S, rS)
    print("  max|err|/rms o %.2e S %.2e" % (eo, eS))
    assert eo <= tol and eS <= tol
