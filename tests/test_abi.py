"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point that include/kda.h declares, and rejects bad arguments
before it enqueues anything."""
import ctypes
import os
import re

import pytest

from kimi_delta_attention_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def _gpu_visible():
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libkda.so is not built; run __graft_entry__.build()")
    return _lib.load()


def test_header_declares_the_boundary():
    assert _declared() == sorted(["kda_status_string", "kda_version", "kda_gate",
                                  "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd",
                                  "kda_recurrent_step", "kda_recurrent_fwd",
                                  "kda_chunk_fwd_split_workspace_bytes", "kda_chunk_fwd_split",
                                  "kda_chunk_fwd_split_noalloc", "kda_bwd_workspace_bytes",
                                  "kda_bwd"])


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name


def test_status_strings(lib):
    for s in range(6):
        assert lib.kda_status_string(s).decode().startswith("KDA_")
    assert lib.kda_status_string(99) == b"unknown kda_status"
    assert lib.kda_version() >= 10000


def test_workspace_is_zero(lib):
    assert lib.kda_chunk_fwd_workspace_bytes(4, 4096, 16, 16, 128, 128, 64, 1) == 0


# Argument checks with fake (never dereferenced) pointers.  They only run where
# no GPU is visible, so a validation bug can never reach a kernel launch.
needs_no_gpu = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer checks run on CPU hosts only")

P = 4096  # a 16-byte-aligned fake device address


def _chunk(lib, **kw):
    a = dict(q=P, k=P, v=P, dt=_lib.KDA_BF16, g=P, beta=P, A=P, bias=P, gate=1, L=-5.0, S0=None,
             o=P, S=P, B=1, T=64, H=2, HV=4, K=128, V=128, C=64, ws=None, wsb=0)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["dt"], a["g"], a["beta"], a["A"], a["bias"],
                             a["gate"], a["L"], a["S0"], a["o"], a["S"], a["B"], a["T"], a["H"],
                             a["HV"], a["K"], a["V"], a["C"], a["ws"], a["wsb"], None)


def _step(lib, **kw):
    a = dict(q=P, k=P, v=P, dt=_lib.KDA_BF16, g=P, beta=P, A=P, bias=None, gate=1, L=-5.0,
             state=P, o=P, B=2, H=2, HV=4, K=128, V=128)
    a.update(kw)
    return lib.kda_recurrent_step(a["q"], a["k"], a["v"], a["dt"], a["g"], a["beta"], a["A"],
                                  a["bias"], a["gate"], a["L"], a["state"], a["o"], a["B"], a["H"],
                                  a["HV"], a["K"], a["V"], None)


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(HV=3), _lib.KDA_ERR_INVALID_ARG),          # HV % H != 0
    (dict(q=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(o=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(beta=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(A=None), _lib.KDA_ERR_INVALID_ARG),         # gate needs A_log
    (dict(q=P + 2), _lib.KDA_ERR_INVALID_ARG),        # misaligned
    (dict(T=-1), _lib.KDA_ERR_INVALID_ARG),
    (dict(H=0), _lib.KDA_ERR_INVALID_ARG),
    (dict(L=1.0), _lib.KDA_ERR_INVALID_ARG),          # safe gate needs L < 0
    (dict(L=float("nan")), _lib.KDA_ERR_INVALID_ARG),
    (dict(gate=7), _lib.KDA_ERR_INVALID_ARG),
    (dict(dt=5), _lib.KDA_ERR_INVALID_ARG),
    (dict(K=96, V=96), _lib.KDA_ERR_UNSUPPORTED),
    (dict(K=128, V=64), _lib.KDA_ERR_UNSUPPORTED),
    (dict(C=48), _lib.KDA_ERR_UNSUPPORTED),
    (dict(H=1, HV=(1 << 17) + 1), _lib.KDA_ERR_UNSUPPORTED),  # HV * K > 2^24 (32-bit row offsets)
    (dict(B=0), _lib.KDA_OK),                         # empty batch: nothing to do
])
def test_chunk_fwd_validation(lib, kw, status):
    assert _chunk(lib, **kw) == status


@needs_no_gpu
def test_gate_none_needs_no_A_log(lib):
    assert _chunk(lib, A=None, gate=2, B=0) == _lib.KDA_OK


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(HV=3), _lib.KDA_ERR_INVALID_ARG),
    (dict(state=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(state=P + 4), _lib.KDA_ERR_INVALID_ARG),
    (dict(K=48), _lib.KDA_ERR_UNSUPPORTED),
    (dict(V=8), _lib.KDA_ERR_UNSUPPORTED),
    (dict(L=0.0), _lib.KDA_ERR_INVALID_ARG),
    (dict(B=0), _lib.KDA_OK),
])
def test_recurrent_step_validation(lib, kw, status):
    assert _step(lib, **kw) == status


def _rec(lib, **kw):
    a = dict(q=P, k=P, v=P, dt=_lib.KDA_BF16, g=P, beta=P, A=P, bias=None, gate=1, L=-5.0,
             S0=None, o=P, S=P, B=2, T=16, H=2, HV=4, K=128, V=64)
    a.update(kw)
    return lib.kda_recurrent_fwd(a["q"], a["k"], a["v"], a["dt"], a["g"], a["beta"], a["A"],
                                 a["bias"], a["gate"], a["L"], a["S0"], a["o"], a["S"], a["B"],
                                 a["T"], a["H"], a["HV"], a["K"], a["V"], None)


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(HV=3), _lib.KDA_ERR_INVALID_ARG),
    (dict(v=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(o=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(S0=P + 8), _lib.KDA_ERR_INVALID_ARG),       # misaligned initial state
    (dict(T=-2), _lib.KDA_ERR_INVALID_ARG),
    (dict(A=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(K=24), _lib.KDA_ERR_UNSUPPORTED),
    (dict(V=256), _lib.KDA_ERR_UNSUPPORTED),
    (dict(gate=2, A=None, B=0), _lib.KDA_OK),
    (dict(B=0), _lib.KDA_OK),
])
def test_recurrent_fwd_validation(lib, kw, status):
    assert _rec(lib, **kw) == status


def test_split_workspace_bytes(lib):
    # per (b, hv, chunk): an image of W and Kt^T (two C x K fp32 arrays, or
    # their hi/lo bf16 pairs, with padded rows) and gamma, plus u and h
    nc = (4100 + 63) // 64
    n = lib.kda_chunk_fwd_split_workspace_bytes(2, 4100, 4, 8, 128, 128, 64)
    per = n // (2 * 8 * nc)
    assert n == per * 2 * 8 * nc and per % 1024 == 0
    assert per >= (2 * 64 * 128 + 128 + 64 * 128 + 128 * 128) * 4
    assert per <= (2 * 64 * 128 + 128 + 64 * 128 + 128 * 128) * 4 * 1.1
    assert lib.kda_chunk_fwd_split_workspace_bytes(2, 0, 4, 8, 128, 128, 64) == 0
    assert lib.kda_chunk_fwd_split_workspace_bytes(0, 64, 4, 8, 128, 128, 64) == 0


def _split(lib, **kw):
    a = dict(q=P, k=P, v=P, dt=_lib.KDA_BF16, g=P, beta=P, A=P, bias=P, gate=1, L=-5.0, S0=None,
             o=P, S=P, h=None, B=1, T=64, H=2, HV=4, K=128, V=128, C=64, ws=P, wsb=1 << 40)
    a.update(kw)
    return lib.kda_chunk_fwd_split(a["q"], a["k"], a["v"], a["dt"], a["g"], a["beta"], a["A"],
                                   a["bias"], a["gate"], a["L"], a["S0"], a["o"], a["S"], a["h"],
                                   a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"], a["C"],
                                   a["ws"], a["wsb"], None)


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(HV=3), _lib.KDA_ERR_INVALID_ARG),
    (dict(k=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(o=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(h=P + 4), _lib.KDA_ERR_INVALID_ARG),        # misaligned h
    (dict(ws=P + 8), _lib.KDA_ERR_INVALID_ARG),       # misaligned workspace
    (dict(ws=None), _lib.KDA_ERR_WORKSPACE),
    (dict(wsb=1000), _lib.KDA_ERR_WORKSPACE),
    (dict(T=-1), _lib.KDA_ERR_INVALID_ARG),
    (dict(A=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(L=0.5), _lib.KDA_ERR_INVALID_ARG),
    (dict(K=96, V=96), _lib.KDA_ERR_UNSUPPORTED),
    (dict(K=64, V=128), _lib.KDA_ERR_UNSUPPORTED),
    (dict(C=8), _lib.KDA_ERR_UNSUPPORTED),
    (dict(B=0), _lib.KDA_OK),
    (dict(gate=_lib.KDA_GATE_PER_HEAD | 2, A=None, B=0), _lib.KDA_OK),
])
def test_chunk_fwd_split_validation(lib, kw, status):
    assert _split(lib, **kw) == status


@needs_no_gpu
def test_per_head_gate_flag_validation(lib):
    ph = _lib.KDA_GATE_PER_HEAD
    assert _chunk(lib, gate=ph | 1, B=0) == _lib.KDA_OK
    assert _chunk(lib, gate=ph | 1, L=0.0) == _lib.KDA_ERR_INVALID_ARG   # safe still needs L < 0
    assert _chunk(lib, gate=ph | 3) == _lib.KDA_ERR_INVALID_ARG          # no such kind
    assert _chunk(lib, gate=32 | 1) == _lib.KDA_ERR_INVALID_ARG          # unknown flag bit
    assert _chunk(lib, gate=ph | 0, A=None) == _lib.KDA_ERR_INVALID_ARG  # standard needs A_log
    assert _chunk(lib, gate=ph | 2, A=None, B=0) == _lib.KDA_OK
    assert _rec(lib, gate=ph | 1, B=0) == _lib.KDA_OK
    assert _step(lib, gate=ph | 7) == _lib.KDA_ERR_INVALID_ARG


@needs_no_gpu
def test_gate_validation(lib):
    f = lambda **kw: lib.kda_gate(kw.get("g", P), kw.get("A", P), None, kw.get("gate", 1),
                                  kw.get("L", -5.0), kw.get("B", 1), kw.get("T", 4), 2, 8,
                                  kw.get("C", 0), kw.get("out", P), None)
    assert f(g=None) == _lib.KDA_ERR_INVALID_ARG
    assert f(out=None) == _lib.KDA_ERR_INVALID_ARG
    assert f(C=-1) == _lib.KDA_ERR_INVALID_ARG
    assert f(A=None) == _lib.KDA_ERR_INVALID_ARG
    assert f(T=0) == _lib.KDA_OK


def test_binding_refuses_without_library(tmp_path):
    """A missing library is an error, never a silent fallback."""
    saved = _lib._lib
    _lib._lib = None
    try:
        with pytest.raises(RuntimeError):
            _lib.load(str(tmp_path / "missing.so"))
    finally:
        _lib._lib = saved


def _split_noalloc(lib, **kw):
    a = dict(q=P, k=P, v=P, dt=_lib.KDA_BF16, g=P, beta=P, A=P, bias=P, gate=1, L=-5.0, S0=None,
             o=P, S=P, h=None, B=1, T=64, H=2, HV=4, K=128, V=128, C=64)
    a.update(kw)
    return lib.kda_chunk_fwd_split_noalloc(a["q"], a["k"], a["v"], a["dt"], a["g"], a["beta"],
                                           a["A"], a["bias"], a["gate"], a["L"], a["S0"], a["o"],
                                           a["S"], a["h"], a["B"], a["T"], a["H"], a["HV"], a["K"],
                                           a["V"], a["C"], None)


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    # 8 value heads x 3,200 tokens at chunk 64 need 8 * 50 * 164 KiB > 64 MiB
    (dict(HV=8, T=3200), _lib.KDA_ERR_SCRATCH),
    (dict(B=2, HV=64, T=4096), _lib.KDA_ERR_SCRATCH),
    (dict(HV=3), _lib.KDA_ERR_INVALID_ARG),
    (dict(k=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(h=P + 4), _lib.KDA_ERR_INVALID_ARG),
    (dict(K=96, V=96), _lib.KDA_ERR_UNSUPPORTED),
    (dict(C=8), _lib.KDA_ERR_UNSUPPORTED),
    (dict(B=0), _lib.KDA_OK),
])
def test_chunk_fwd_split_noalloc_validation(lib, kw, status):
    """Rejected on the host before anything touches a device, including a
    problem whose workspace exceeds the fixed scratch."""
    assert _split_noalloc(lib, **kw) == status


def test_noalloc_scratch_limit(lib):
    """8 value heads x 3,136 tokens (49 chunks of 164 KiB each) fit in 64 MiB,
    3,200 tokens (50 chunks) do not."""
    assert lib.kda_chunk_fwd_split_workspace_bytes(1, 3136, 2, 8, 128, 128, 64) <= 64 << 20
    assert lib.kda_chunk_fwd_split_workspace_bytes(1, 3200, 2, 8, 128, 128, 64) > 64 << 20


def _bwd(lib, **kw):
    a = dict(q=P, k=P, v=P, dt=_lib.KDA_F32, g=P, beta=P, A=P, bias=P, gate=1, L=-5.0, S0=None,
             do=P, dST=None, dq=P, dk=P, dv=P, dbeta=P, dg=P, dA=P, dbias=P, dS0=None,
             B=2, T=37, H=2, HV=4, K=64, V=64, ws=P, wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = lib.kda_bwd_workspace_bytes(a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"])
    return lib.kda_bwd(a["q"], a["k"], a["v"], a["dt"], a["g"], a["beta"], a["A"], a["bias"],
                       a["gate"], a["L"], a["S0"], a["do"], a["dST"], a["dq"], a["dk"], a["dv"],
                       a["dbeta"], a["dg"], a["dA"], a["dbias"], a["dS0"], a["B"], a["T"], a["H"],
                       a["HV"], a["K"], a["V"], a["ws"], a["wsb"], None)


@needs_no_gpu
@pytest.mark.parametrize("kw,status", [
    (dict(gate=_lib.KDA_GATE_PER_HEAD | 3), _lib.KDA_ERR_INVALID_ARG),
    (dict(gate=_lib.KDA_GATE_PER_HEAD | 1, g=P + 4, bias=P + 4, B=0, ws=None, wsb=0, dA=None,
          dbias=None), _lib.KDA_OK),
    (dict(K=16, V=16), _lib.KDA_ERR_UNSUPPORTED),
    (dict(K=64, V=32), _lib.KDA_ERR_UNSUPPORTED),
    (dict(dq=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(do=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(dv=P + 4), _lib.KDA_ERR_INVALID_ARG),
    (dict(dq=P + 2), _lib.KDA_ERR_INVALID_ARG),
    (dict(HV=3), _lib.KDA_ERR_INVALID_ARG),
    (dict(A=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(L=0.0), _lib.KDA_ERR_INVALID_ARG),
    (dict(ws=None), _lib.KDA_ERR_WORKSPACE),
    (dict(wsb=1024), _lib.KDA_ERR_WORKSPACE),
    (dict(B=0, ws=None, wsb=0, dA=None, dbias=None), _lib.KDA_OK),
])
def test_bwd_validation(lib, kw, status):
    assert _bwd(lib, **kw) == status


def test_bwd_workspace_bytes(lib):
    """Per 16 tokens: the entering K x V fp32 state, U (16 x V fp32), three
    16 x 16 fp32 operand blocks, the 16 x K retain factors and a flag."""
    n = lib.kda_bwd_workspace_bytes(1, 4096, 16, 16, 128, 128)
    segs = 16 * 256
    need = segs * (128 * 128 * 4 + 16 * 128 * 4 + 3 * 256 * 4 + 16 * 128 * 4 + 4)
    assert need <= n <= need + 5 * 256
    assert lib.kda_bwd_workspace_bytes(1, 4096, 16, 16, 16, 16) == 0
    assert lib.kda_bwd_workspace_bytes(0, 4096, 16, 16, 128, 128) == 0

