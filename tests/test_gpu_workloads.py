"""GPU parity at the full sizes of the five synthetic workloads, in the launch
configuration the benchmark times.  The oracle recomputes every (sequence,
value head) pair over its whole length, a group of pairs at a time; every
output and every final state is compared element by element."""
import pytest
import torch

import kda_testlib as L
from kimi_delta_attention_02_amd import synth

pytestmark = pytest.mark.gpu


def _chunked(name):
    w = synth.WORKLOADS[name]
    d = synth.make_inputs(w)
    print("%s: B=%d T=%d H=%d HV=%d K=%d" % (name, w.B, w.T, w.H, w.HV, w.K), flush=True)
    o, S = L.run_chunk(d, w.gate, w.lower_bound, w.chunk)
    tol = L.TOL_F32 if w.dtype == "f32" else L.TOL_BF16
    L.compare_all_heads(d, w.gate, w.lower_bound, o, S, tol, name)


def test_workload_tiny_chunked_all_heads():
    _chunked("tiny")


@pytest.mark.timeout(300)
def test_workload_prefill():
    _chunked("prefill")


@pytest.mark.timeout(300)
def test_workload_gva():
    _chunked("gva")


@pytest.mark.timeout(300)
def test_workload_prefill_head_gate():
    _chunked("prefill_head_gate")


@pytest.mark.timeout(600)
def test_workload_long():
    _chunked("long")


@pytest.mark.timeout(600)
def test_workload_decode():
    """256 single-token steps over B=256, HV=32 with a 512 MiB fp32 state;
    all 8,192 (sequence, value head) pairs."""
    w = synth.WORKLOADS["decode"]
    d = synth.make_inputs(w)
    print("decode: B=%d steps=%d HV=%d K=%d" % (w.B, w.steps, w.HV, w.K), flush=True)
    o, S = L.run_decode(d, w.gate, w.lower_bound, d["S0"])
    L.compare_all_heads(d, w.gate, w.lower_bound, o, S, L.TOL_F32, "decode", group=256)
