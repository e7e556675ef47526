"""Pins for the CPU oracle: checks against facts that the pages and plain
mathematics fix, each computed by arithmetic independent of the oracle's own.

Every pin is a function ``pin_*(orc)`` that raises AssertionError when the
oracle ``orc`` (an ``oracle.Oracle``) disagrees.  ``test_oracle_pins.py`` runs
them on the real oracle; the mutation tests run them on copies of the oracle
with a planted mistake and require that some pin fails.

Sources (page titles and sections):
* "K3 notes" section "KDA 递归核心": the four-step update (decay, predict,
  write, read with 1/sqrt(K)), input table (q, k repeat_interleave'd to HV).
* "K3 notes" section "Gate 激活": gate table, code panel, defaults table.
* "DeltaNet family" page (hi.news.hada.io summary of the doubleword blog):
  DeltaNet reconstruction identity and locality, eigenvalues of I - b k k^T,
  the online-gradient-descent view, Gated DeltaNet's scalar gate, KDA's
  diagonal-plus-low-rank transition A_t = D_t (I - b_t k_t k_t^T), and the
  chunkwise form (temporary errors, triangular solve, chunk-end state,
  chunk outputs) which must reproduce the recurrence exactly.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(seed, B=1, T=8, H=1, HV=1, K=6, V=5, unit_keys=True):
    r = _rng(seed)
    q = r.standard_normal((B, T, H, K))
    k = r.standard_normal((B, T, H, K))
    if unit_keys:
        q, k = _unit(q), _unit(k)
    v = r.standard_normal((B, T, HV, V))
    g_raw = r.standard_normal((B, T, HV, K))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, HV))))
    A_log = 0.5 * r.standard_normal(HV)
    dt_bias = -4.0 + 0.5 * r.standard_normal((HV, K))
    S0 = 0.3 * r.standard_normal((B, HV, K, V))
    return dict(q=q, k=k, v=v, g_raw=g_raw, beta=beta, A_log=A_log, dt_bias=dt_bias, S0=S0)


def _run(orc, d, gate="none", L=-5.0, S0=True):
    return orc.kda_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"],
                       d["dt_bias"] if gate != "none" else None, gate, L,
                       d["S0"] if S0 else None, threads=2)


def _close(a, b, tol, what):
    """max |a - b| <= tol * max(1, max |b|)  (relative once values exceed 1)."""
    a, b = np.asarray(a), np.asarray(b)
    if not np.size(a):
        return
    err = float(np.max(np.abs(a - b)))
    bound = tol * max(1.0, float(np.max(np.abs(b))))
    assert err <= bound, "%s: max |diff| %.3e > %.1e" % (what, err, bound)


# ---------------------------------------------------------------- gate pins

def pin_gate_printed_defaults(orc):
    """Worked value printed in the defaults table: g ~ -0.09, exp(g) ~ 0.91,
    and exp(-5) ~ 0.0067 for the floor ("Gate 激活", defaults table and
    summary box)."""
    with open(os.path.join(GOLDEN, "gate_defaults.json")) as f:
        gold = json.load(f)["cases"]
    c = gold[0]
    i = c["inputs"]
    g = orc.gate(np.full((1, 1, 1, 1), i["g_raw"]), np.array([i["A_log"]]),
                 np.full((1, 1), i["dt_bias"]), i["gate"], i["lower_bound"])[0, 0, 0, 0]
    half_ulp = 0.5 * 10.0 ** (-c["printed_digits"])
    assert abs(g - c["printed"]["g"]) <= half_ulp, g
    assert abs(math.exp(g) - c["printed"]["exp_g"]) <= half_ulp, math.exp(g)
    # floor: a large positive input saturates the sigmoid, so g reaches L
    floor = orc.gate(np.full((1, 1, 1, 1), 1e4), np.zeros(1), np.zeros((1, 1)), "safe", -5.0)
    c2 = gold[1]
    assert abs(math.exp(floor[0, 0, 0, 0]) - c2["printed"]["exp_lower_bound"]) <= 0.5e-4


def pin_gate_ranges(orc):
    """Safe gate lies in [L, 0], standard gate in (-inf, 0] ("Gate 激活",
    two-gate table), for inputs from -1e4 to 1e4; NaN in gives NaN out."""
    r = _rng(11)
    x = np.concatenate([r.standard_normal(20000) * 10, [-1e4, -50, -1e-9, 0, 1e-9, 50, 1e4]])
    g_raw = x.reshape(1, -1, 1, 1)
    A_log = np.array([0.7])
    for L in (-5.0, -0.5):
        g = orc.gate(g_raw, A_log, np.zeros((1, 1)), "safe", L)
        assert np.all(g <= 0) and np.all(g >= L)
        assert np.all(np.exp(g) >= math.exp(L) * (1 - 1e-15))
    g = orc.gate(g_raw, A_log, np.zeros((1, 1)), "standard")
    assert np.all(g <= 0) and np.all(np.isfinite(g))
    nan = orc.gate(np.full((1, 1, 1, 1), np.nan), A_log, np.zeros((1, 1)), "safe", -5.0)
    assert np.isnan(nan).all()
    nan = orc.gate(np.full((1, 1, 1, 1), np.nan), A_log, np.zeros((1, 1)), "standard")
    assert np.isnan(nan).all()


def pin_gate_closed_forms(orc):
    """Identities of the two gates, evaluated without the oracle's formulas:
    standard: exp(g) = sigmoid(-x)^rate   (softplus(x) = -log sigmoid(-x));
    safe:     g(x) + g(-x) = L            (sigmoid(z) + sigmoid(-z) = 1);
    rate = exp(A_log) multiplies the input inside the sigmoid (A_log = log 2
    doubles it) and the softplus outside; dt_bias shifts the input."""
    r = _rng(12)
    x = r.standard_normal((1, 400, 1, 3)) * 3
    for a in (0.0, math.log(2.0), -0.8):
        rate = math.exp(a)
        g = orc.gate(x, np.array([a]), np.zeros((1, 3)), "standard")
        sig_neg = np.array([[[[1.0 / (1.0 + math.exp(float(xx))) for xx in row]
                              for row in x[0, t]] for t in range(x.shape[1])]])
        _close(np.exp(g), sig_neg ** rate, 1e-13, "standard gate closed form")
        gp = orc.gate(x, np.array([a]), np.zeros((1, 3)), "safe", -5.0)
        gm = orc.gate(-x, np.array([a]), np.zeros((1, 3)), "safe", -5.0)
        _close(gp + gm, np.full_like(gp, -5.0), 1e-13, "safe gate symmetry")
    # A_log = log 2 inside the sigmoid equals doubling the input at A_log = 0
    g2 = orc.gate(x, np.array([math.log(2.0)]), np.zeros((1, 3)), "safe", -5.0)
    g1 = orc.gate(2 * x, np.array([0.0]), np.zeros((1, 3)), "safe", -5.0)
    _close(g2, g1, 1e-13, "rate inside the sigmoid")
    # dt_bias per (hv, kappa) shifts the input
    bias = np.array([[0.3, -1.0, 2.0]])
    gb = orc.gate(x, np.array([0.0]), bias, "safe", -5.0)
    gs = orc.gate(x + bias.reshape(1, 1, 1, 3), np.array([0.0]), np.zeros((1, 3)), "safe", -5.0)
    _close(gb, gs, 1e-13, "dt_bias shift")
    # rate printed for A_log = 0 in the defaults table is 1: standard gate = -softplus
    g0 = orc.gate(np.zeros((1, 1, 1, 1)), np.zeros(1), np.zeros((1, 1)), "standard")
    _close(g0, -math.log(2.0), 1e-15, "standard gate at 0 with rate 1")
    # gate "none" passes g_raw through untouched
    _close(orc.gate(x, np.array([0.4]), None, "none"), x, 0.0, "gate none")


# ---------------------------------------------------------- recurrence pins

def pin_reconstruction(orc):
    """DeltaNet immediate reconstruction: with g = 0, beta = 1 and unit keys,
    reading the state back with the key just written returns v_t exactly;
    reading with q = k makes o_t = v_t / sqrt(K) (step 4's scale).  For
    general beta the read returns (1 - beta) k.S_dec + beta v."""
    d = _inputs(21, T=12, K=7, V=4)
    d["g_raw"][:] = 0.0
    d["beta"][:] = 1.0
    d["q"] = d["k"].copy()
    o, _ = _run(orc, d, "none", S0=True)
    _close(o * math.sqrt(7), d["v"], 1e-12, "k_t . S_t = v_t")
    # general beta, one step from a random state with per-channel decay
    d = _inputs(22, T=1, K=7, V=4)
    d["q"] = d["k"].copy()
    o, _ = _run(orc, d, "none", S0=True)
    alpha = np.exp(d["g_raw"][0, 0, 0])
    S_dec = alpha[:, None] * d["S0"][0, 0]
    k = d["k"][0, 0, 0]
    b = d["beta"][0, 0, 0]
    want = ((1 - b) * (k @ S_dec) + b * d["v"][0, 0, 0]) / math.sqrt(7)
    _close(o[0, 0, 0], want, 1e-12, "partial reconstruction")


def pin_locality(orc):
    """The write only touches the key direction: a query orthogonal to k_t
    reads S_t exactly as it reads S_dec (I - b k k^T has eigenvalue 1 off k)."""
    d = _inputs(23, T=1, K=6, V=3)
    k = d["k"][0, 0, 0]
    q = d["q"][0, 0, 0]
    q = q - (q @ k) * k
    d["q"][0, 0, 0] = q / np.linalg.norm(q)
    o, _ = _run(orc, d, "none", S0=True)
    S_dec = np.exp(d["g_raw"][0, 0, 0])[:, None] * d["S0"][0, 0]
    _close(o[0, 0, 0], d["q"][0, 0, 0] @ S_dec / math.sqrt(6), 1e-12, "locality")


def pin_beta_zero(orc):
    """beta = 0: nothing is written.  From a zero state o = 0 and S = 0; from
    S0 the state only decays, S_T = diag(exp(sum_t g_t)) S0, and
    o_t = (1/sqrt(K)) (q_t * exp(sum_{m<=t} g_m)) . S0."""
    d = _inputs(24, T=9, K=5, V=4)
    d["beta"][:] = 0.0
    o, S = _run(orc, d, "none", S0=False)
    assert np.all(o == 0) and np.all(S == 0)
    o, S = _run(orc, d, "none", S0=True)
    G = np.cumsum(d["g_raw"][0, :, 0], axis=0)  # [T, K]
    _close(S[0, 0], np.exp(G[-1])[:, None] * d["S0"][0, 0], 1e-12, "pure decay state")
    want = (d["q"][0, :, 0] * np.exp(G)) @ d["S0"][0, 0] / math.sqrt(5)
    _close(o[0, :, 0], want, 1e-12, "pure decay outputs")


def pin_read_gemm(orc):
    """g = 0 and beta = 0: every output is the plain product (1/sqrt(K)) q S0,
    per GVA head (value head hv reads key head hv // (HV/H))."""
    d = _inputs(25, B=2, T=5, H=2, HV=4, K=6, V=3)
    d["beta"][:] = 0.0
    d["g_raw"][:] = 0.0
    o, S = _run(orc, d, "none", S0=True)
    for b in range(2):
        for hv in range(4):
            want = d["q"][b, :, hv // 2] @ d["S0"][b, hv] / math.sqrt(6)
            _close(o[b, :, hv], want, 1e-13, "read GEMM")
    _close(S, d["S0"], 0.0, "state untouched")


def pin_one_hot_keys(orc):
    """Distinct one-hot keys turn the state into K independent rows: every row
    decays by its own channel's factor, and the keyed row becomes the convex
    mix (1 - beta) row + beta v (an exponential moving average)."""
    T, K, V = 8, 8, 3
    d = _inputs(26, T=T, K=K, V=V)
    perm = _rng(5).permutation(K)
    d["k"][:] = 0.0
    for t in range(T):
        d["k"][0, t, 0, perm[t]] = 1.0
    o, S = _run(orc, d, "none", S0=True)
    rows = d["S0"][0, 0].copy()
    for t in range(T):
        rows = rows * np.exp(d["g_raw"][0, t, 0])[:, None]
        b = d["beta"][0, t, 0]
        rows[perm[t]] = (1 - b) * rows[perm[t]] + b * d["v"][0, t, 0]
        _close(o[0, t, 0], d["q"][0, t, 0] @ rows / math.sqrt(K), 1e-12, "one-hot output")
    _close(S[0, 0], rows, 1e-12, "one-hot state")


def pin_dplr_unrolled(orc):
    """Brute force of the diagonal-plus-low-rank form, in the DeltaNet page's
    own layout (state M is d_v x d_k, key channels are columns):
    M_t = M_{t-1} A_t + b_t v_t k_t^T with A_t = D_t (I - b_t k_t k_t^T),
    unrolled as M_T = M_0 A_1...A_T + sum_j b_j v_j k_j^T A_{j+1}...A_T,
    and o_t = M_t q_t / sqrt(d_k).  Explicit d_k x d_k products, T <= 8."""
    for T in (1, 3, 8):
        d = _inputs(27 + T, T=T, K=5, V=4, unit_keys=False)
        o, S = _run(orc, d, "none", S0=True)
        K = 5
        A = []
        for t in range(T):
            k = d["k"][0, t, 0][:, None]
            D = np.diag(np.exp(d["g_raw"][0, t, 0]))
            A.append(D @ (np.eye(K) - d["beta"][0, t, 0] * (k @ k.T)))

        def chain(i, j):  # A_i ... A_j (empty -> identity), 0-based inclusive
            P = np.eye(K)
            for m in range(i, j + 1):
                P = P @ A[m]
            return P

        M0 = d["S0"][0, 0].T  # page layout
        for t in range(T):
            M = M0 @ chain(0, t)
            for j in range(t + 1):
                vk = d["beta"][0, j, 0] * np.outer(d["v"][0, j, 0], d["k"][0, j, 0])
                M = M + vk @ chain(j + 1, t)
            _close(o[0, t, 0], M @ d["q"][0, t, 0] / math.sqrt(K), 1e-12, "DPLR output")
        _close(S[0, 0], M.T, 1e-12, "DPLR state")


def pin_gated_deltanet(orc):
    """Gated DeltaNet is KDA with the same decay on every key channel: written
    in the DeltaNet page's steps (forget by a scalar, predict S k, correct
    e = b (v - v_hat), write e k^T, read S q / sqrt(d_k)) with the d_v x d_k
    layout.  With g = 0 it is DeltaNet, whose update is one gradient step of
    0.5 ||S k - v||^2 with step size b."""
    T, K, V = 10, 6, 4
    d = _inputs(31, T=T, K=K, V=V)
    a = d["g_raw"][0, :, 0, :1]  # one log-decay per token
    d["g_raw"][:] = np.repeat(a, K, axis=1)[None, :, None, :]
    o, S = _run(orc, d, "none", S0=True)
    M = d["S0"][0, 0].T.copy()
    for t in range(T):
        M = math.exp(a[t, 0]) * M
        k, v, q = d["k"][0, t, 0], d["v"][0, t, 0], d["q"][0, t, 0]
        e = d["beta"][0, t, 0] * (v - M @ k)
        M = M + np.outer(e, k)
        _close(o[0, t, 0], M @ q / math.sqrt(K), 1e-12, "gated DeltaNet output")
    _close(S[0, 0], M.T, 1e-12, "gated DeltaNet state")
    # DeltaNet as online gradient descent (g = 0)
    d["g_raw"][:] = 0.0
    o, S = _run(orc, d, "none", S0=True)
    M = d["S0"][0, 0].T.copy()
    for t in range(T):
        k, v = d["k"][0, t, 0], d["v"][0, t, 0]
        grad = np.outer(M @ k - v, k)
        M = M - d["beta"][0, t, 0] * grad
    _close(S[0, 0], M.T, 1e-12, "DeltaNet gradient step")


def pin_gva_repeat(orc):
    """GVA: H key heads serving HV value heads equals running with q and k
    repeat_interleave'd to HV heads (consecutive value heads share a key
    head), bit for bit."""
    d = _inputs(32, B=2, T=6, H=2, HV=6, K=4, V=3)
    o1, S1 = orc.kda_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"],
                         d["dt_bias"], "safe", -5.0, d["S0"], threads=2)
    q = np.repeat(d["q"], 3, axis=2)
    k = np.repeat(d["k"], 3, axis=2)
    o2, S2 = orc.kda_fwd(q, k, d["v"], d["g_raw"], d["beta"], d["A_log"], d["dt_bias"],
                         "safe", -5.0, d["S0"], threads=2)
    _close(o1, o2, 0.0, "GVA outputs")
    _close(S1, S2, 0.0, "GVA states")


def pin_split_continuation(orc):
    """The state is the whole carry: running T1 tokens, then T2 tokens from
    the returned state, equals running T1 + T2 tokens at once."""
    d = _inputs(33, B=1, T=11, H=1, HV=2, K=4, V=5)
    d["v"] = _rng(34).standard_normal((1, 11, 2, 5))
    d["g_raw"] = _rng(35).standard_normal((1, 11, 2, 4))
    d["beta"] = _rng(36).uniform(0, 1, (1, 11, 2))
    args = lambda sl: (d["q"][:, sl], d["k"][:, sl], d["v"][:, sl], d["g_raw"][:, sl],
                       d["beta"][:, sl], d["A_log"], d["dt_bias"], "safe", -5.0)
    o, S = orc.kda_fwd(*args(slice(0, 11)), d["S0"])
    oa, Sa = orc.kda_fwd(*args(slice(0, 4)), d["S0"])
    ob, Sb = orc.kda_fwd(*args(slice(4, 11)), Sa)
    _close(np.concatenate([oa, ob], axis=1), o, 0.0, "split outputs")
    _close(Sb, S, 0.0, "split state")


def pin_chunkwise_equals_recurrent(orc):
    """The chunkwise schedule from the DeltaNet page must reproduce the
    recurrence exactly (also stated as claim C3 of the notes' ledger).  Written
    in that page's layout (state d_v x d_k): per chunk of C tokens,
      cumulative decay D_{0:i}, D_{j+1:i} from a difference of prefix sums,
      temporary errors  e_bar_i = b_i (v_i - S_c D_{0:i} k_i),
      rho_ij = b_i k_j^T D_{j+1:i} k_i (j < i), E = E_bar (I + R)^{-T},
      S_{c+1} = S_c D_{0:C-1} + E K_end,
      chi_ij = s k_j^T D_{j+1:i} q_i (j <= i), O = s S_c Q_bd + E A_qk^T.
    A ragged last chunk is just a shorter chunk."""
    d = _inputs(37, B=1, T=27, H=1, HV=1, K=6, V=4)
    g = orc.gate(d["g_raw"], d["A_log"], d["dt_bias"], "safe", -5.0)
    o_ref, S_ref = orc.kda_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta"], d["A_log"],
                               d["dt_bias"], "safe", -5.0, d["S0"])
    K = 6
    s = 1.0 / math.sqrt(K)
    for C in (1, 2, 5, 8, 27):
        M = d["S0"][0, 0].T.copy()  # d_v x d_k
        outs = []
        for c0 in range(0, 27, C):
            sl = slice(c0, min(c0 + C, 27))
            q, k, v = d["q"][0, sl, 0], d["k"][0, sl, 0], d["v"][0, sl, 0]
            b = d["beta"][0, sl, 0]
            G = np.cumsum(g[0, sl, 0], axis=0)  # log D_{0:i}, [n, K]
            n = q.shape[0]
            e_bar = b[:, None] * (v - (M @ (np.exp(G) * k).T).T)
            R = np.zeros((n, n))
            A_qk = np.zeros((n, n))
            for i in range(n):
                for j in range(i + 1):
                    Dji = np.exp(G[i] - G[j])
                    if j < i:
                        R[i, j] = b[i] * (k[j] * Dji) @ k[i]
                    A_qk[i, j] = s * (k[j] * Dji) @ q[i]
            E = np.linalg.solve(np.eye(n) + R, e_bar)  # rows: e_i = e_bar_i - sum rho_ij e_j
            K_end = k * np.exp(G[-1] - G)
            Q_bd = q * np.exp(G)
            O = s * (M @ Q_bd.T).T + A_qk @ E
            M = M * np.exp(G[-1])[None, :] + E.T @ K_end
            outs.append(O)
        _close(np.concatenate(outs, axis=0), o_ref[0, :, 0], 1e-12, "chunk outputs C=%d" % C)
        _close(M.T, S_ref[0, 0], 1e-12, "chunk state C=%d" % C)


ALL_PINS = [
    pin_gate_printed_defaults,
    pin_gate_ranges,
    pin_gate_closed_forms,
    pin_reconstruction,
    pin_locality,
    pin_beta_zero,
    pin_read_gemm,
    pin_one_hot_keys,
    pin_dplr_unrolled,
    pin_gated_deltanet,
    pin_gva_repeat,
    pin_split_continuation,
    pin_chunkwise_equals_recurrent,
]
