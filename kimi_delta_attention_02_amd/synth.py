"""Seeded synthetic inputs for the KDA forward pass.

This module only draws random inputs; it contains none of the method's
arithmetic, and both the HIP path and the CPU oracle consume what it returns.

Every tensor is drawn in float32 on the CPU from ``torch.Generator`` seeded with
the workload's seed, in a fixed order:

    S0 (if random), q, k, v, g_raw, beta_logit, A_log (if random), dt_bias (if random)

then q and k are L2-normalised over the key dimension in float32,
beta = sigmoid(beta_logit), and q/k/v are rounded to bfloat16 (round to
nearest even) when the workload says so.  ``N(mu, s)`` means mean mu and
standard deviation s.

The named workloads follow the KDA notes' defaults (A_log = 0, dt_bias = -4,
lower bound -5, from the "Gate 激活" defaults table) and the five synthetic
shapes this library is measured on.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    HV: int
    K: int
    V: int
    chunk: int
    dtype: str            # "f32" or "bf16": storage type of q, k, v
    gate: str             # "safe" | "standard" | "none"
    lower_bound: float
    a_log_std: float      # 0 -> A_log = 0 exactly
    dt_bias_mean: float
    dt_bias_std: float    # 0 -> dt_bias constant
    s0_std: float         # 0 -> zero initial state
    seed: int
    steps: int = 0        # decode workloads: number of single-token steps
    per_head_gate: bool = False  # g_raw [B,T,HV] and dt_bias [HV] (Gated DeltaNet's scalar gate)

    @property
    def tokens(self) -> int:
        return self.B * (self.steps if self.steps else self.T)


WORKLOADS = {
    # tiny fp32 correctness case: chunked and recurrent both checked
    "tiny": Workload("tiny", 1, 64, 2, 2, 16, 16, 16, "f32", "safe", -5.0,
                     0.0, -4.0, 0.0, 0.0, seed=1),
    # chunked prefill, B4 T4096 H=HV16 K=V128, chunk 64
    "prefill": Workload("prefill", 4, 4096, 16, 16, 128, 128, 64, "bf16", "safe", -5.0,
                        0.5, -4.0, 0.0, 0.0, seed=2),
    # GVA chunked prefill with the standard gate and a random initial state
    "gva": Workload("gva", 2, 16384, 8, 32, 128, 128, 64, "bf16", "standard", -5.0,
                    0.5, -4.0, 0.5, 0.02, seed=3),
    # recurrent decode: 256 single-token steps over B256 HV32 K=V128
    "decode": Workload("decode", 256, 1, 32, 32, 128, 128, 64, "bf16", "safe", -5.0,
                       0.0, -4.0, 0.0, 0.02, seed=4, steps=256),
    # long-context GVA chunked prefill
    "long": Workload("long", 1, 65536, 16, 64, 128, 128, 64, "bf16", "safe", -5.0,
                     0.5, -4.0, 0.0, 0.0, seed=5),
    # the prefill shape with one gate per (token, value head), as in Gated DeltaNet
    "prefill_head_gate": Workload("prefill_head_gate", 4, 4096, 16, 16, 128, 128, 64, "bf16",
                                  "safe", -5.0, 0.5, -4.0, 0.0, 0.0, seed=6, per_head_gate=True),
    # one GPU's share of the long-context workload split over eight GPUs by GVA
    # head groups: one 65,536-token sequence, 2 q/k heads, 8 value heads
    "long_shard": Workload("long_shard", 1, 65536, 2, 8, 128, 128, 64, "bf16", "safe", -5.0,
                           0.5, -4.0, 0.0, 0.0, seed=7),
}


def _normal(shape, gen, mean=0.0, std=1.0):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    if mean != 0.0:
        x = x + mean
    return x


def _l2(x):
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def make_inputs(w: Workload, *, T: int | None = None, B: int | None = None, seed: int | None = None):
    """Draw one batch of inputs for workload ``w`` (CPU tensors).

    Returns a dict with q, k [B,T,H,K], v [B,T,HV,V] (float32 or bfloat16),
    g_raw [B,T,HV,K], beta [B,T,HV], A_log [HV], dt_bias [HV,K], S0 [B,HV,K,V]
    or None (all float32); with a per-head gate g_raw is [B,T,HV] and dt_bias
    [HV].  For decode workloads T is the number of steps and
    step t reads q[:, t] etc.  ``T``, ``B`` and ``seed`` override the workload.
    """
    B = w.B if B is None else B
    T = (w.steps if w.steps else w.T) if T is None else T
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    S0 = _normal((B, w.HV, w.K, w.V), gen, std=w.s0_std) if w.s0_std > 0 else None
    q = _l2(_normal((B, T, w.H, w.K), gen))
    k = _l2(_normal((B, T, w.H, w.K), gen))
    v = _normal((B, T, w.HV, w.V), gen)
    gk = () if w.per_head_gate else (w.K,)
    g_raw = _normal((B, T, w.HV) + gk, gen)
    beta = torch.sigmoid(_normal((B, T, w.HV), gen))
    A_log = (_normal((w.HV,), gen, std=w.a_log_std) if w.a_log_std > 0
             else torch.zeros(w.HV, dtype=torch.float32))
    dt_bias = (_normal((w.HV,) + gk, gen, mean=w.dt_bias_mean, std=w.dt_bias_std)
               if w.dt_bias_std > 0 else torch.full((w.HV,) + gk, w.dt_bias_mean, dtype=torch.float32))
    if w.dtype == "bf16":
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    return dict(q=q, k=k, v=v, g_raw=g_raw, beta=beta, A_log=A_log, dt_bias=dt_bias, S0=S0)


def random_inputs(B, T, H, HV, K, V, *, seed, dtype="f32", a_log_std=0.5, dt_bias_mean=-4.0,
                  dt_bias_std=0.5, s0_std=0.0, g_std=1.0, per_head_gate=False):
    """Inputs of arbitrary shape with the same recipe (used by edge-case tests)."""
    w = Workload("custom", B, T, H, HV, K, V, 16, dtype, "safe", -5.0, a_log_std,
                 dt_bias_mean, dt_bias_std, s0_std, seed, per_head_gate=per_head_gate)
    d = make_inputs(w)
    if g_std != 1.0:
        d["g_raw"] = d["g_raw"] * g_std
    return d


def rms(x) -> float:
    """Root mean square of a tensor/array (for tolerance scaling)."""
    x = torch.as_tensor(x, dtype=torch.float64)
    return math.sqrt(float((x * x).mean())) if x.numel() else 0.0
