"""CPU checks of bench.py's accounting: the algorithmic bytes and FLOPs its
roofline objects divide by, the staleness rule of the counter records, and
the one-GPU contract.  The byte counts are pinned to the tensors the
synthetic inputs actually are (tiny workload) and to the figures stated for
the full-size workloads; the FLOP counts to their per-token definitions."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from kimi_delta_attention_02_amd import synth  # noqa: E402

W = synth.WORKLOADS


def test_chunk_bytes_is_the_size_of_the_tensors_read_and_written():
    """tiny workload: every input tensor once, o and the final state (and the
    initial state when one is given), summed from the tensors themselves."""
    w = W["tiny"]
    d = synth.make_inputs(w)
    nbytes = lambda t: t.numel() * t.element_size()
    ins = sum(nbytes(d[n]) for n in ("q", "k", "v", "g_raw", "beta"))
    o = w.B * w.T * w.HV * w.V * 4
    state = w.B * w.HV * w.K * w.V * 4
    s0 = nbytes(d["S0"]) if d["S0"] is not None else 0
    assert bench.chunk_bytes(w) == ins + o + state + s0


@pytest.mark.parametrize("name,mb", [("prefill", 475.0), ("gva", 1489.0), ("long", 5926.6)])
def test_chunk_bytes_of_the_full_size_workloads(name, mb):
    assert round(bench.chunk_bytes(W[name]) / 1e6, 1) == mb


@pytest.mark.parametrize("name,gflop", [("prefill", 31.1), ("long", 498.2)])
def test_chunk_flops_at_the_16_token_block(name, gflop):
    w = W[name]
    per = 2 * (3 * 16 * w.K + 2 * 16 * w.V + 3 * w.K * w.V)  # per token and value head
    assert bench.chunk_flops(w) == per * w.B * w.T * w.HV
    assert round(bench.chunk_flops(w) / 1e9, 1) == gflop
    # a requested chunk of 64 would count 1.52x more at K = V = 128
    assert abs(bench.chunk_flops(w, 64) / bench.chunk_flops(w) - 1.52) < 0.01


def test_backward_call_flops():
    w = W["prefill"]
    assert bench.bwd_flops(w) == 20 * w.K * w.V * w.B * w.T * w.HV
    assert bench.bwd_call_flops(w) == bench.chunk_flops(w, 16) + bench.bwd_flops(w)
    assert round(bench.bwd_call_flops(w) / 1e9, 1) == 117.0


def test_decode_bytes_per_step():
    w = W["decode"]
    state = w.B * w.HV * w.K * w.V * 4
    assert bench.decode_bytes(w) == 1088454656
    assert bench.decode_bytes(w) > 2 * state  # the state read and written, plus one token's rows
    assert bench.recurrent_bytes(w, 1) == bench.decode_bytes(w)


def test_profile_record_is_dropped_once_its_sources_change(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    (tmp_path / "profiles").mkdir()
    h = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    rec = {"traffic_bytes_per_launch": 123.0, "sources": ["k.hip"], "source_sha256_16": h}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"x": rec}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("x") == 123.0
    assert bench.measured_traffic("missing") is None
    src.write_text("kernel v2\n")
    assert bench.profile_record("x") is None
    assert bench.measured_traffic("x") is None


def test_committed_records_name_existing_sources():
    d = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for key, rec in d.items():
        for f in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, f)), (key, f)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
