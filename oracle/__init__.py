"""CPU oracle for the Kimi Delta Attention forward pass (fp64).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library's compute path.  It shares
no code with the HIP library.

The arithmetic lives in ``kda_oracle.c`` (plain C, binary64); this module only
compiles it with gcc, marshals numpy arrays into float64 buffers, and slices
out single heads so that long sequences can be checked one (b, hv) pair at a
time.  Definitions followed, all from the "K3 notes" pages:

* gate: section "Gate 激活" (two-gate table, kda_gate_reference panel);
* recurrence: section "KDA 递归核心", four-step update with the 1/sqrt(K) read
  scale of step 4;
* GVA: the input table of the same section (q, k repeat_interleave'd to HV).

``kda_oracle_bwd.c`` differentiates the same recurrence and gate in reverse
mode (the gradients the backward pass must produce); it is pinned by finite
differences of the forward oracle, not by anything of its own.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kda_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

GATE_KINDS = {"standard": 0, "safe": 1, "none": 2}

_dp = ctypes.POINTER(ctypes.c_double)


BWD_SOURCE = os.path.join(_HERE, "kda_oracle_bwd.c")


def build(source: str = SOURCE, out: str = LIBRARY, extra=(BWD_SOURCE,)) -> str:
    """Compile the oracle with gcc into a shared library (the forward source,
    plus the gradient source unless `extra` is empty); returns its path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-D_POSIX_C_SOURCE=200809L",
           "-o", tmp, source] + list(extra) + ["-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _arr(x, shape=None):
    if x is None:
        return None, None
    if hasattr(x, "detach"):  # torch tensor -> numpy, exact widening to float64
        import torch

        x = x.detach().to("cpu", torch.float64).numpy()
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    return a, a.ctypes.data_as(_dp)


class Oracle:
    """Handle on one compiled oracle library (the real one, or a test mutant)."""

    def __init__(self, path: str = LIBRARY):
        if path == LIBRARY and not os.path.exists(path):
            build()
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_gate.restype = ctypes.c_int
        lib.oracle_gate.argtypes = [_dp, _dp, _dp, ctypes.c_int, ctypes.c_double,
                                    ctypes.c_long, ctypes.c_long, ctypes.c_long, ctypes.c_long, _dp]
        lib.oracle_kda_fwd.restype = ctypes.c_int
        lib.oracle_kda_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int,
                                       ctypes.c_double, _dp] + [ctypes.c_long] * 6 + [_dp, _dp,
                                                                                       ctypes.c_int]
        if hasattr(lib, "oracle_kda_bwd"):
            lib.oracle_kda_bwd.restype = ctypes.c_int
            lib.oracle_kda_bwd.argtypes = ([_dp] * 7 + [ctypes.c_int, ctypes.c_double] + [_dp] * 3
                                           + [ctypes.c_long] * 6 + [_dp] * 8 + [ctypes.c_int])
        self.lib = lib

    def gate(self, g_raw, A_log, dt_bias=None, gate="safe", lower_bound=-5.0):
        """g = gate(g_raw) for g_raw of shape [B, T, HV, K] (float64 result)."""
        g, gp = _arr(g_raw)
        if g.ndim != 4:
            raise ValueError("g_raw must be [B, T, HV, K]")
        B, T, HV, K = g.shape
        _, ap = _arr(A_log, (HV,))
        _, dp = _arr(dt_bias, (HV, K))
        out = np.empty_like(g)
        rc = self.lib.oracle_gate(gp, ap, dp, GATE_KINDS[gate], float(lower_bound), B, T, HV, K,
                                  out.ctypes.data_as(_dp))
        if rc != 0:
            raise ValueError("oracle_gate rejected its arguments")
        return out

    def kda_fwd(self, q, k, v, g_raw, beta, A_log, dt_bias=None, gate="safe", lower_bound=-5.0,
                initial_state=None, threads=None):
        """Naive four-step recurrence.  Returns (o [B,T,HV,V], S_T [B,HV,K,V]) in float64."""
        qa, qp = _arr(q)
        B, T, H, K = qa.shape
        va, vp = _arr(v)
        HV, V = va.shape[2], va.shape[3]
        _, kp = _arr(k, (B, T, H, K))
        _, gp = _arr(g_raw, (B, T, HV, K))
        _, bp = _arr(beta, (B, T, HV))
        _, ap = _arr(A_log, (HV,))
        _, dp = _arr(dt_bias, (HV, K))
        _, sp = _arr(initial_state, (B, HV, K, V))
        o = np.empty((B, T, HV, V))
        s_out = np.empty((B, HV, K, V))
        n = threads or os.cpu_count() or 1
        rc = self.lib.oracle_kda_fwd(qp, kp, vp, gp, bp, ap, dp, GATE_KINDS[gate],
                                     float(lower_bound), sp, B, T, H, HV, K, V,
                                     o.ctypes.data_as(_dp), s_out.ctypes.data_as(_dp), int(n))
        if rc != 0:
            raise ValueError("oracle_kda_fwd rejected its arguments")
        return o, s_out

    def kda_bwd(self, q, k, v, g_raw, beta, A_log, dt_bias=None, gate="safe", lower_bound=-5.0,
                initial_state=None, dout=None, dfinal_state=None, threads=None):
        """Gradients of sum(o * dout) + sum(S_T * dfinal_state) with respect to
        the inputs (reverse mode through the naive recurrence and the gate, in
        float64).  Returns a dict with dq, dk [B,T,H,K], dv [B,T,HV,V], dbeta
        [B,T,HV], dg_raw [B,T,HV,K], dA_log [HV], ddt_bias [HV,K] (None without
        dt_bias) and dS0 [B,HV,K,V]."""
        qa, qp = _arr(q)
        B, T, H, K = qa.shape
        va, vp = _arr(v)
        HV, V = va.shape[2], va.shape[3]
        _, kp = _arr(k, (B, T, H, K))
        _, gp = _arr(g_raw, (B, T, HV, K))
        _, bp = _arr(beta, (B, T, HV))
        _, ap = _arr(A_log, (HV,))
        _, dp = _arr(dt_bias, (HV, K))
        _, sp = _arr(initial_state, (B, HV, K, V))
        _, op = _arr(dout, (B, T, HV, V))
        _, fp = _arr(dfinal_state, (B, HV, K, V))
        out = {"dq": np.empty((B, T, H, K)), "dk": np.empty((B, T, H, K)),
               "dv": np.empty((B, T, HV, V)), "dbeta": np.empty((B, T, HV)),
               "dg_raw": np.empty((B, T, HV, K)), "dA_log": np.empty((HV,)),
               "ddt_bias": np.empty((HV, K)) if dt_bias is not None else None,
               "dS0": np.empty((B, HV, K, V))}
        ptr = lambda a: None if a is None else a.ctypes.data_as(_dp)
        n = threads or os.cpu_count() or 1
        rc = self.lib.oracle_kda_bwd(qp, kp, vp, gp, bp, ap, dp, GATE_KINDS[gate],
                                     float(lower_bound), sp, op, fp, B, T, H, HV, K, V,
                                     ptr(out["dq"]), ptr(out["dk"]), ptr(out["dv"]),
                                     ptr(out["dbeta"]), ptr(out["dg_raw"]), ptr(out["dA_log"]),
                                     ptr(out["ddt_bias"]), ptr(out["dS0"]), int(n))
        if rc != 0:
            raise ValueError("oracle_kda_bwd rejected its arguments")
        return out

    def kda_fwd_heads(self, q, k, v, g_raw, beta, A_log, dt_bias, gate, lower_bound,
                      initial_state, heads, threads=None):
        """Run the recurrence for selected (b, hv) pairs only.

        Each pair is independent, so a pair is sliced out (q/k of its GVA head
        h = hv / (HV/H), its own v, g_raw, beta, A_log, dt_bias, S0) and run as
        a B=H=HV=1 problem.  Returns {(b, hv): (o [T, V], S_T [K, V])}.
        """
        from concurrent.futures import ThreadPoolExecutor

        H, HV = q.shape[2], v.shape[2]

        def one(pair):
            b, hv = pair
            h = hv // (HV // H)
            o, s = self.kda_fwd(
                q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, hv:hv + 1],
                g_raw[b:b + 1, :, hv:hv + 1], beta[b:b + 1, :, hv:hv + 1], A_log[hv:hv + 1],
                None if dt_bias is None else dt_bias[hv:hv + 1], gate, lower_bound,
                None if initial_state is None else initial_state[b:b + 1, hv:hv + 1],
                threads=1)
            return o[0, :, 0], s[0, 0]

        heads = [tuple(p) for p in heads]
        n = threads or os.cpu_count() or 1
        with ThreadPoolExecutor(max_workers=max(1, min(n, len(heads)))) as ex:
            res = list(ex.map(one, heads))
        out = dict(zip(heads, res))
        return out


_default = None


def default() -> Oracle:
    """The oracle built from ``kda_oracle.c`` (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def build_variant(source_text: str, directory: str | None = None) -> Oracle:
    """Compile a modified copy of the oracle source (used by the mutation
    tests, which plant a mistake and check that some pin catches it)."""
    d = directory or tempfile.mkdtemp(prefix="oracle_variant_")
    src = os.path.join(d, "variant.c")
    with open(src, "w") as f:
        f.write(source_text)
    return Oracle(build(src, os.path.join(d, "libvariant.so"), extra=()))


def build_bwd_variant(source_text: str, directory: str | None = None) -> Oracle:
    """Compile the oracle with a modified copy of the gradient source (the
    gradient pins plant a mistake there and check that they catch it)."""
    d = directory or tempfile.mkdtemp(prefix="oracle_bwd_variant_")
    src = os.path.join(d, "variant_bwd.c")
    with open(src, "w") as f:
        f.write(source_text)
    return Oracle(build(SOURCE, os.path.join(d, "libvariant.so"), extra=(src,)))
