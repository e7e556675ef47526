"""The allocation-free split forward (kda_chunk_fwd_split_noalloc) against the
workspace-taking one (kda_chunk_fwd_split) it is a variant of: the same
kernels on the same inputs, so o, the final state and every chunk-entry
state agree bit for bit.  Two calls in a row, the second smaller, show that
the fixed scratch is reused correctly."""
import pytest
import torch

import kda_testlib as L
import kimi_delta_attention_02_amd as kda
from kimi_delta_attention_02_amd import synth

pytestmark = pytest.mark.gpu


def _pair(B, T, H, HV, K, dtype, gate, chunk, s0):
    print("noalloc split: B=%d T=%d H=%d HV=%d K=%d %s %s chunk %d" % (B, T, H, HV, K, dtype, gate,
                                                                       chunk), flush=True)
    d = synth.random_inputs(B, T, H, HV, K, K, seed=300 + T + K, dtype=dtype, s0_std=s0)
    g = L.to_dev(d)
    args = (g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"], g["dt_bias"])
    NC = (T + chunk - 1) // chunk
    kw = dict(gate=gate, lower_bound=-5.0, chunk_size=chunk, initial_state=g["S0"])
    o1, S1, h1 = kda.chunk_fwd_split(*args, output_states=True, **kw)
    o2 = torch.empty_like(o1)
    S2 = torch.empty_like(S1)
    h2 = torch.empty((B, HV, NC, K, K), dtype=torch.float32, device=L.DEV)
    kda.chunk_fwd_split_noalloc(*args, o=o2, final_state=S2, h=h2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(h1, h2)
    return d, o2, S2


def test_noalloc_two_calls_second_smaller():
    d, o, S = _pair(1, 3136, 2, 8, 128, "bf16", "safe", 64, 0.02)  # the largest that fits
    ro, rS = L.oracle_full(d, "safe", -5.0)
    assert L.rel_err(o, ro) <= L.TOL_BF16 and L.rel_err(S, rS) <= L.TOL_BF16
    _pair(2, 200, 2, 4, 64, "f32", "standard", 32, 0.02)


def test_noalloc_rejects_beyond_scratch():
    d = synth.random_inputs(1, 3200, 2, 8, 128, 128, seed=1, dtype="bf16")
    g = L.to_dev(d)
    with pytest.raises(kda.KDAError) as e:
        kda.chunk_fwd_split_noalloc(g["q"], g["k"], g["v"], g["g_raw"], g["beta"], g["A_log"],
                                    g["dt_bias"], gate="safe")
    assert e.value.status == 5
