"""CPU model of the bf16-MFMA arithmetic of the fused chunk kernel.

This is test infrastructure: a numpy replay of the kernel's 16-token block
algebra with every MFMA operand rounded to bfloat16 the way the kernel rounds
it, so the error that each rounding choice costs can be measured against the
fp64 oracle on the CPU.  It is not the oracle (the oracle is the plain
recurrence) and shares nothing with the HIP code.

The algebra is the "DeltaNet family" page, section "Chunkwise KDA", in blocks
of n = 16 tokens and in the K x V state layout of the "K3 notes".  For a block
entering with state S, with E_i the product of the retain factors exp(g) of
the block's tokens up to and including i (per key channel), gamma = E_{n-1}
and Suf_j = gamma / E_j:

    Ebar = beta (v - (k E) S)                       temporary errors
    R_ij = beta_i sum_c (k_ic E_ic)(k_jc / E_jc)    j < i
    U    = (I + R)^{-1} Ebar                        causal solve
    O    = s (q E) S + A U,  A_ij = s sum_c (q_ic E_ic)(k_jc / E_jc)   j <= i
    S'   = diag(gamma) S + (k Suf)^T U

Each product is a named term; an operand of it is carried either as one bf16
word ("h") or as hi + lo bf16 words ("hl", hi = bf16(x), lo = bf16(x - hi)),
and a product of two operands takes the cross terms hi*hi + hi*lo + lo*hi
that the kernel issues as MFMAs (fp32 accumulation); "f" keeps an operand in
float32, which checks the algebra itself.  The solve, the gate,
the decays and the state itself stay in fp32, as in the kernel.
"""
from __future__ import annotations

import numpy as np

# product name -> its two operands
PRODUCTS = {
    "KS": ("k_E", "S"),        # (k E) S                     prediction
    "R": ("k_E", "k_iE"),      # (k E)(k / E)^T              coupling
    "A": ("k_iE", "q_E"),      # (k / E)(q E)^T              intra-block read
    "U": ("inv", "Ebar"),      # (I + R)^{-1} Ebar           solve
    "QS": ("q_E", "S"),        # (q E) S                     inter-block read
    "AU": ("A", "U"),          # A U                         intra-block output
    "SU": ("k_Suf", "U"),      # (k Suf)^T U                 state update
}

# what the kernel carries: every operand as hi + lo words
KERNEL = {name: ("hl", "hl") for name in PRODUCTS}
# one bf16 word per operand everywhere
SINGLE = {name: ("h", "h") for name in PRODUCTS}
# float32 operands everywhere: the algebra without bf16 rounding
FP32 = {name: ("f", "f") for name in PRODUCTS}


def bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _words(x, mode):
    if mode == "f":  # no rounding: float32 operands (checks the algebra itself)
        return np.asarray(x, dtype=np.float32), None
    hi = bf16(x)
    if mode == "h":
        return hi, None
    return hi, bf16(x.astype(np.float32) - hi)


def product(a, b, modes, transpose_a=False):
    """a @ b (or a^T @ b) with each operand rounded per `modes`, summing the
    cross terms hi*hi + hi*lo + lo*hi in float64 and rounding the sum to
    float32 (the accumulation order of the MFMAs is below this precision)."""
    ah, al = _words(a, modes[0])
    bh, bl = _words(b, modes[1])
    mm = (lambda x, y: np.swapaxes(x, -1, -2).astype(np.float64) @ y.astype(np.float64)) \
        if transpose_a else (lambda x, y: x.astype(np.float64) @ y.astype(np.float64))
    acc = mm(ah, bh)
    if bl is not None:
        acc = acc + mm(ah, bl)
    if al is not None:
        acc = acc + mm(al, bh)
    return acc.astype(np.float32)


def retain_factors(g_raw, A_log, dt_bias, gate, lower_bound):
    """exp(g) in float32 from the gate formulas ("K3 notes", "Gate 激活"),
    evaluated in float64.  g_raw [T, K] of one head; A_log scalar; dt_bias
    [K] or None."""
    x = g_raw.astype(np.float64) + (0.0 if dt_bias is None else dt_bias.astype(np.float64))
    rate = np.exp(np.float64(A_log))
    if gate == "safe":
        g = lower_bound / (1.0 + np.exp(-rate * x))
    elif gate == "standard":
        g = -rate * (np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))
    else:
        g = x
    return np.exp(g).astype(np.float32)


def chunk_forward(q, k, v, alpha, beta, S0, precision=KERNEL, block=16):
    """The block algebra above for a batch of heads.

    q, k [N, T, K], v [N, T, V], alpha [N, T, K] retain factors, beta [N, T],
    S0 [N, K, V] (float32 values; q, k, v as the kernel reads them).  T must
    be a multiple of `block`.  Returns (o [N, T, V], S [N, K, V]) in float32.
    """
    N, T, K = q.shape
    assert T % block == 0
    s = np.float32(1.0 / np.sqrt(K))
    S = S0.astype(np.float32).copy()
    o = np.empty(v.shape, dtype=np.float32)
    lower = np.tril(np.ones((block, block), dtype=bool))
    strict = np.tril(np.ones((block, block), dtype=bool), -1)
    eye = np.eye(block)
    P = precision
    for t0 in range(0, T, block):
        sl = slice(t0, t0 + block)
        a = alpha[:, sl].astype(np.float32)
        E = np.cumprod(a, axis=1, dtype=np.float32)
        gam = E[:, -1]                                      # [N, K]
        suf = np.flip(np.cumprod(np.flip(a, 1), axis=1, dtype=np.float32), 1)
        suf = np.concatenate([suf[:, 1:], np.ones_like(suf[:, :1])], axis=1)
        qb, kb, vb, bb = q[:, sl], k[:, sl], v[:, sl], beta[:, sl]
        q_E, k_E = qb * E, kb * E
        k_Suf = kb * suf
        k_iE = k_Suf * (np.float32(1.0) / gam)[:, None, :]
        KS = product(k_E, S, P["KS"])
        Ebar = bb[:, :, None] * (vb - KS)
        R = product(k_E, np.swapaxes(k_iE, 1, 2), P["R"]) * bb[:, :, None]
        R = np.where(strict, R, 0.0)
        inv = np.linalg.inv(eye + R.astype(np.float64)).astype(np.float32)
        U = product(inv, Ebar, P["U"])
        A = s * product(q_E, np.swapaxes(k_iE, 1, 2), P["A"])
        A = np.where(lower, A, 0.0).astype(np.float32)
        o[:, sl] = s * product(q_E, S, P["QS"]) + product(A, U, P["AU"])
        S = gam[:, :, None] * S + product(k_Suf, U, P["SU"], transpose_a=True)
    return o, S


def max_rel_err(got, ref):
    """max |got - ref| / RMS(ref)."""
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(np.asarray(got, dtype=np.float64) - ref).max()
                 / np.sqrt((ref * ref).mean()))
