"""Kimi Delta Attention forward on MI355X (gfx950): thin Python binding.

Every function marshals torch tensors (device memory, the current HIP stream)
into the C ABI of ``include/kda.h`` and nothing else: each step of the
computation runs in the HIP kernels of ``libkda.so``.

Gates are per key channel (g_raw with a trailing K axis, dt_bias [HV, K]) or,
when g_raw has no K axis, one scalar per (token, value head) as in Gated
DeltaNet (dt_bias [HV]); the binding passes KDA_GATE_PER_HEAD for the latter.

* :func:`gate`           -- gate activation (+ optional chunk-local cumulative sum)
* :func:`chunk_fwd`      -- chunkwise forward over whole sequences
* :func:`chunk_fwd_split` -- the chunkwise forward as three stages with the
                            chunk-entry states materialised (few heads, long sequences)
* :func:`recurrent_fwd`  -- T tokens per call with the state kept on chip
* :func:`recurrent_step` -- one decode token, state updated in place
"""
from __future__ import annotations

import torch

from . import _lib

__all__ = ["gate", "chunk_fwd", "chunk_fwd_split", "chunk_fwd_split_noalloc", "recurrent_fwd",
           "recurrent_step", "bwd",
           "chunk_fwd_workspace_bytes", "chunk_fwd_split_workspace_bytes", "bwd_workspace_bytes",
           "KDAError"]

KDAError = _lib.KDAError


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _gate_code(gate, per_head):
    return _lib.GATES[gate] | (_lib.KDA_GATE_PER_HEAD if per_head else 0)


def _check_gate_inputs(g_raw, dt_bias, A_log, lead, HV, K, dev):
    """g_raw is lead + (HV, K) (per channel) or lead + (HV,) (per head)."""
    per_head = g_raw.dim() == len(lead) + 1
    _need(g_raw, "g_raw", torch.float32, tuple(lead) + ((HV,) if per_head else (HV, K)), dev)
    if A_log is not None:
        _need(A_log, "A_log", torch.float32, (HV,), dev)
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", torch.float32, (HV,) if per_head else (HV, K), dev)
    return per_head


def _qkv_dtype(q):
    if q.dtype == torch.float32:
        return _lib.KDA_F32
    if q.dtype == torch.bfloat16:
        return _lib.KDA_BF16
    raise TypeError("q, k, v must be float32 or bfloat16, got %s" % q.dtype)


def gate(g_raw, A_log, dt_bias=None, *, gate="safe", lower_bound=-5.0, chunk_size=0, out=None):
    """Gate activation of g_raw [B, T, HV, K] or, per head, [B, T, HV]
    (float32); with chunk_size > 0 the chunk-local inclusive cumulative sum of
    the log-decay.  Returns float32 of g_raw's shape."""
    lib = _lib.load()
    dev = g_raw.device
    if g_raw.dim() == 3:
        (B, T, HV), K = g_raw.shape, 1
    else:
        B, T, HV, K = g_raw.shape
    per_head = _check_gate_inputs(g_raw, dt_bias, A_log, (B, T), HV, K, dev)
    if out is None:
        out = torch.empty_like(g_raw)
    _need(out, "out", torch.float32, tuple(g_raw.shape), dev)
    st = lib.kda_gate(_ptr(g_raw), _ptr(A_log), _ptr(dt_bias), _gate_code(gate, per_head),
                      float(lower_bound), B, T, HV, K, int(chunk_size), _ptr(out), _stream(dev))
    _lib.check("kda_gate", st)
    return out


def chunk_fwd_workspace_bytes(B, T, H, HV, K, V, chunk_size=64, dtype=torch.bfloat16):
    d = _lib.KDA_BF16 if dtype == torch.bfloat16 else _lib.KDA_F32
    return int(_lib.load().kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, chunk_size, d))


def chunk_fwd(q, k, v, g_raw, beta, A_log, dt_bias=None, *, gate="safe", lower_bound=-5.0,
              chunk_size=64, initial_state=None, output_final_state=True, o=None,
              final_state=None, workspace=None):
    """Chunkwise KDA forward.

    q, k [B, T, H, K] and v [B, T, HV, V] (float32 or bfloat16, one dtype);
    g_raw [B, T, HV, K] (or [B, T, HV] for a per-head gate), beta [B, T, HV],
    A_log [HV], dt_bias [HV, K] (or [HV]) or None, initial_state [B, HV, K, V]
    or None (float32).  Returns (o, final_state) with o [B, T, HV, V] float32
    and final_state [B, HV, K, V] float32 (None when output_final_state is
    False).
    """
    lib = _lib.load()
    qkv = _qkv_dtype(q)
    dev, B, T, H, HV, K, V, per_head = _check_sequence_args(q, k, v, g_raw, beta, A_log, dt_bias,
                                                            initial_state)
    if o is None:
        o = torch.empty((B, T, HV, V), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (B, T, HV, V), dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((B, HV, K, V), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (B, HV, K, V), dev)
    need = int(lib.kda_chunk_fwd_workspace_bytes(B, T, H, HV, K, V, chunk_size, qkv))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), qkv, _ptr(g_raw), _ptr(beta), _ptr(A_log),
                           _ptr(dt_bias), _gate_code(gate, per_head), float(lower_bound),
                           _ptr(initial_state),
                           _ptr(o), _ptr(final_state), B, T, H, HV, K, V, int(chunk_size),
                           _ptr(workspace), ws_bytes, _stream(dev))
    _lib.check("kda_chunk_fwd", st)
    return o, final_state


def chunk_fwd_split_workspace_bytes(B, T, H, HV, K, V, chunk_size=64):
    return int(_lib.load().kda_chunk_fwd_split_workspace_bytes(B, T, H, HV, K, V, chunk_size))


def chunk_fwd_split(q, k, v, g_raw, beta, A_log, dt_bias=None, *, gate="safe", lower_bound=-5.0,
                    chunk_size=64, initial_state=None, output_final_state=True,
                    output_states=False, o=None, final_state=None, h=None, workspace=None,
                    output_o=True):
    """Chunkwise forward in three stages (intra-chunk, state pass, output),
    with the entry state of every chunk materialised.  Arguments as
    :func:`chunk_fwd`.  Returns (o, final_state, h): h [B, HV, NC, K, V]
    float32 with NC = ceil(T / chunk_size) when output_states is True (or an
    ``h`` tensor is given), else None.  With output_o=False (h required) the
    output stage is skipped and o is None."""
    lib = _lib.load()
    qkv = _qkv_dtype(q)
    dev, B, T, H, HV, K, V, per_head = _check_sequence_args(q, k, v, g_raw, beta, A_log, dt_bias,
                                                            initial_state)
    if not output_o:
        if not (output_states or h is not None):
            raise ValueError("output_o=False needs the states (output_states or h)")
        o = None
    elif o is None:
        o = torch.empty((B, T, HV, V), dtype=torch.float32, device=dev)
    if o is not None:
        _need(o, "o", torch.float32, (B, T, HV, V), dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((B, HV, K, V), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (B, HV, K, V), dev)
    NC = (T + chunk_size - 1) // chunk_size if chunk_size > 0 else 0
    if output_states and h is None:
        h = torch.empty((B, HV, NC, K, V), dtype=torch.float32, device=dev)
    if h is not None:
        _need(h, "h", torch.float32, (B, HV, NC, K, V), dev)
    need = int(lib.kda_chunk_fwd_split_workspace_bytes(B, T, H, HV, K, V, chunk_size))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_fwd_split(_ptr(q), _ptr(k), _ptr(v), qkv, _ptr(g_raw), _ptr(beta),
                                 _ptr(A_log), _ptr(dt_bias), _gate_code(gate, per_head),
                                 float(lower_bound), _ptr(initial_state), _ptr(o),
                                 _ptr(final_state), _ptr(h), B, T, H, HV, K, V, int(chunk_size),
                                 _ptr(workspace), ws_bytes, _stream(dev))
    _lib.check("kda_chunk_fwd_split", st)
    return o, final_state, h


def chunk_fwd_split_noalloc(q, k, v, g_raw, beta, A_log, dt_bias=None, *, gate="safe",
                            lower_bound=-5.0, chunk_size=64, initial_state=None, o=None,
                            final_state=None, h=None):
    """:func:`chunk_fwd_split` without a workspace: the library's fixed 64 MiB
    scratch holds it (kda_chunk_fwd_split_noalloc), so the call allocates no
    device memory when o, final_state (and h, if wanted) are given.  Calls on
    one device share that scratch and must not overlap.  Returns (o,
    final_state, h)."""
    lib = _lib.load()
    qkv = _qkv_dtype(q)
    dev, B, T, H, HV, K, V, per_head = _check_sequence_args(q, k, v, g_raw, beta, A_log, dt_bias,
                                                            initial_state)
    if o is None:
        o = torch.empty((B, T, HV, V), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (B, T, HV, V), dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (B, HV, K, V), dev)
    if h is not None:
        NC = (T + chunk_size - 1) // chunk_size if chunk_size > 0 else 0
        _need(h, "h", torch.float32, (B, HV, NC, K, V), dev)
    st = lib.kda_chunk_fwd_split_noalloc(_ptr(q), _ptr(k), _ptr(v), qkv, _ptr(g_raw), _ptr(beta),
                                         _ptr(A_log), _ptr(dt_bias), _gate_code(gate, per_head),
                                         float(lower_bound), _ptr(initial_state), _ptr(o),
                                         _ptr(final_state), _ptr(h), B, T, H, HV, K, V,
                                         int(chunk_size), _stream(dev))
    _lib.check("kda_chunk_fwd_split_noalloc", st)
    return o, final_state, h


def bwd_workspace_bytes(B, T, H, HV, K, V):
    """Device workspace bytes kda_bwd needs for these sizes."""
    return int(_lib.load().kda_bwd_workspace_bytes(B, T, H, HV, K, V))


def bwd(q, k, v, g_raw, beta, A_log, dt_bias=None, *, gate="safe", lower_bound=-5.0,
        initial_state=None, dout, dfinal_state=None, want_dA_log=True, want_ddt_bias=None,
        want_dinitial_state=None, workspace=None):
    """Gradients of the forward (kda_bwd) for dL/do = dout [B, T, HV, V] and
    dL/dS_T = dfinal_state (or zero).  Returns a dict of float32 tensors: dq,
    dk [B, T, H, K], dv [B, T, HV, V], dbeta [B, T, HV], dg_raw [B, T, HV, K]
    ([B, T, HV] for a per-head gate), dA_log [HV] (None unless want_dA_log),
    ddt_bias [HV, K] or [HV] (by default when dt_bias is given), dS0
    [B, HV, K, V] (by default when initial_state is given)."""
    lib = _lib.load()
    qkv = _qkv_dtype(q)
    dev, B, T, H, HV, K, V, per_head = _check_sequence_args(q, k, v, g_raw, beta, A_log, dt_bias,
                                                            initial_state)
    _need(dout, "dout", torch.float32, (B, T, HV, V), dev)
    if dfinal_state is not None:
        _need(dfinal_state, "dfinal_state", torch.float32, (B, HV, K, V), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    gk = () if per_head else (K,)  # a per-head gate has no key axis
    out = {"dq": torch.empty((B, T, H, K), **f32), "dk": torch.empty((B, T, H, K), **f32),
           "dv": torch.empty((B, T, HV, V), **f32), "dbeta": torch.empty((B, T, HV), **f32),
           "dg_raw": torch.empty((B, T, HV) + gk, **f32)}
    out["dA_log"] = torch.empty((HV,), **f32) if want_dA_log else None
    if want_ddt_bias is None:
        want_ddt_bias = dt_bias is not None
    out["ddt_bias"] = torch.empty((HV,) + gk, **f32) if want_ddt_bias else None
    if want_dinitial_state is None:
        want_dinitial_state = initial_state is not None
    out["dS0"] = torch.empty((B, HV, K, V), **f32) if want_dinitial_state else None
    need = int(lib.kda_bwd_workspace_bytes(B, T, H, HV, K, V))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.kda_bwd(_ptr(q), _ptr(k), _ptr(v), qkv, _ptr(g_raw), _ptr(beta), _ptr(A_log),
                     _ptr(dt_bias), _gate_code(gate, per_head), float(lower_bound),
                     _ptr(initial_state), _ptr(dout), _ptr(dfinal_state), _ptr(out["dq"]),
                     _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]), _ptr(out["dg_raw"]),
                     _ptr(out["dA_log"]), _ptr(out["ddt_bias"]), _ptr(out["dS0"]),
                     B, T, H, HV, K, V, _ptr(workspace), ws_bytes, _stream(dev))
    _lib.check("kda_bwd", st)
    return out


def _check_sequence_args(q, k, v, g_raw, beta, A_log, dt_bias, initial_state):
    dev = q.device
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    dt = q.dtype
    _need(q, "q", dt, (B, T, H, K), dev)
    _need(k, "k", dt, (B, T, H, K), dev)
    _need(v, "v", dt, (B, T, HV, V), dev)
    per_head = _check_gate_inputs(g_raw, dt_bias, A_log, (B, T), HV, K, dev)
    _need(beta, "beta", torch.float32, (B, T, HV), dev)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (B, HV, K, V), dev)
    return dev, B, T, H, HV, K, V, per_head


def recurrent_fwd(q, k, v, g_raw, beta, A_log, dt_bias=None, *, gate="safe", lower_bound=-5.0,
                  initial_state=None, output_final_state=True, o=None, final_state=None):
    """Fused recurrent forward over the T tokens of a call, the state kept on
    chip.  Arguments and returns as :func:`chunk_fwd` (no chunk size); K and V
    may differ.  ``final_state`` may be the ``initial_state`` tensor itself."""
    lib = _lib.load()
    qkv = _qkv_dtype(q)
    dev, B, T, H, HV, K, V, per_head = _check_sequence_args(q, k, v, g_raw, beta, A_log, dt_bias,
                                                            initial_state)
    if o is None:
        o = torch.empty((B, T, HV, V), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (B, T, HV, V), dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((B, HV, K, V), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (B, HV, K, V), dev)
    st = lib.kda_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), qkv, _ptr(g_raw), _ptr(beta),
                               _ptr(A_log), _ptr(dt_bias), _gate_code(gate, per_head),
                               float(lower_bound),
                               _ptr(initial_state), _ptr(o), _ptr(final_state), B, T, H, HV, K, V,
                               _stream(dev))
    _lib.check("kda_recurrent_fwd", st)
    return o, final_state


def recurrent_step(q, k, v, g_raw, beta, A_log, dt_bias, state, *, gate="safe", lower_bound=-5.0,
                   o=None):
    """One decode token: q, k [B, H, K], v [B, HV, V], g_raw [B, HV, K] (or
    [B, HV] for a per-head gate), beta [B, HV]; state [B, HV, K, V] float32 is
    updated in place.  Returns o [B, HV, V] float32."""
    lib = _lib.load()
    dev = q.device
    B, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    dt = q.dtype
    qkv = _qkv_dtype(q)
    _need(q, "q", dt, (B, H, K), dev)
    _need(k, "k", dt, (B, H, K), dev)
    _need(v, "v", dt, (B, HV, V), dev)
    per_head = _check_gate_inputs(g_raw, dt_bias, A_log, (B,), HV, K, dev)
    _need(beta, "beta", torch.float32, (B, HV), dev)
    _need(state, "state", torch.float32, (B, HV, K, V), dev)
    if o is None:
        o = torch.empty((B, HV, V), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (B, HV, V), dev)
    st = lib.kda_recurrent_step(_ptr(q), _ptr(k), _ptr(v), qkv, _ptr(g_raw), _ptr(beta),
                                _ptr(A_log), _ptr(dt_bias), _gate_code(gate, per_head),
                                float(lower_bound),
                                _ptr(state), _ptr(o), B, H, HV, K, V, _stream(dev))
    _lib.check("kda_recurrent_step", st)
    return o
