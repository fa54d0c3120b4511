"""Pins for the KDA oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own code.

Every check takes an implementation ``impl(q, k, v, g, beta, s0) -> (o, S)``
on unit-major fp64 arrays (q, k, g [n, T, Dk]; v [n, T, Dv]; beta [n, T];
s0 [n, Dk, Dv] or None; g is the log-decay, alpha = e^g) and raises
AssertionError when the implementation disagrees.  The oracle is one such
implementation; the mutants at the bottom are deliberately wrong ones, used to
show that the pins catch plausible mistakes.

Sources (page "Kimi K3：从三条信息流到完整系统", wineandchord.com):
  eq. (1) and its expanded form, section "KDA 是带逐通道遗忘的 delta rule";
  the reference step and its 2x2 example in the same section;
  eq. (5) and the bounded_decay check, section "下界 log-decay 是一个 kernel 设计";
  the affine segment transition, its composition and eq. (17), section "FlashKDA 与 KCP".
"""
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rel(x, ref):
    return float(np.linalg.norm(np.ravel(x - ref)) / max(np.linalg.norm(np.ravel(ref)), 1e-300))


def _unit_rows(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ----------------------------------------------------------------------------- P1


def pin_worked_example(impl):
    """The page's 2x2 example of one step: S = [[5,6],[.75,1]], o = [5,6]."""
    G = _golden("kda_step_worked_example.json")
    q = np.array(G["q"])[None, None]
    k = np.array(G["k"])[None, None]
    v = np.array(G["v"])[None, None]
    g = np.log(np.array(G["alpha"]))[None, None]
    beta = np.array([[G["beta"]]])
    s0 = np.array(G["S0"])[None]
    o, S = impl(q, k, v, g, beta, s0)
    assert np.max(np.abs(S[0] - np.array(G["expected_S"]))) <= 1e-15, S
    assert np.max(np.abs(o[0, 0] - np.array(G["expected_o"]))) <= 1e-15, o


# ----------------------------------------------------------------------------- P2


def pin_scalar_hand_solved(impl):
    """d_k = d_v = 1, solved by hand (values in tests/golden)."""
    G = _golden("scalar_hand_solved.json")
    T = len(G["v"])
    for case in G["cases"]:
        q = np.full((1, T, 1), G["q"])
        k = np.full((1, T, 1), case["k"])
        v = np.array(G["v"]).reshape(1, T, 1)
        g = np.full((1, T, 1), math.log(G["alpha"]))
        beta = np.full((1, T), G["beta"])
        s0 = np.full((1, 1, 1), case["s0"])
        o, _ = impl(q, k, v, g, beta, s0)
        assert np.max(np.abs(o[0, :, 0] - np.array(case["expected_o"]))) <= 1e-15, (case, o[0, :, 0])


# ----------------------------------------------------------------------------- P3


def pin_erase_identity(impl, seed=3):
    """With ||k|| = 1 and beta = 1 one step leaves k^T S_t = v_t^T (the write
    overwrites the value stored along k instead of adding to it) and does not
    touch the part of the decayed state orthogonal to k:
    (I - k k^T) S_t = (I - k k^T) Diag(alpha) S_{t-1}."""
    rng = np.random.default_rng(seed)
    dk, dv = 16, 12
    for _ in range(4):
        k = _unit_rows(rng, (1, 1, dk))
        q = rng.standard_normal((1, 1, dk))
        v = rng.standard_normal((1, 1, dv))
        g = -5.0 * rng.random((1, 1, dk))
        s0 = rng.standard_normal((1, dk, dv))
        _, S = impl(q, k, v, g, np.ones((1, 1)), s0)
        kk = k[0, 0]
        assert np.max(np.abs(kk @ S[0] - v[0, 0])) <= 1e-13
        proj = np.eye(dk) - np.outer(kk, kk)
        expect = proj @ (np.exp(g[0, 0])[:, None] * s0[0])
        assert np.max(np.abs(proj @ S[0] - expect)) <= 1e-13


# ----------------------------------------------------------------------------- P4


def pin_beta_zero_exact(impl, seed=4):
    """beta = 0: nothing is written, so S_t = Diag(Gamma_t) S0 with
    Gamma_t = exp(sum_{r<=t} g_r) and o_t = S0^T (Gamma_t * q_t)."""
    rng = np.random.default_rng(seed)
    n, T, dk, dv = 2, 23, 8, 6
    q = rng.standard_normal((n, T, dk))
    k = _unit_rows(rng, (n, T, dk))
    v = rng.standard_normal((n, T, dv))
    g = -0.3 * rng.random((n, T, dk))
    s0 = rng.standard_normal((n, dk, dv))
    o, S = impl(q, k, v, g, np.zeros((n, T)), s0)
    gam = np.exp(np.cumsum(g, axis=1))
    for u in range(n):
        assert _rel(S[u], gam[u, -1][:, None] * s0[u]) <= 1e-14
        for t in range(T):
            assert _rel(o[u, t], s0[u].T @ (gam[u, t] * q[u, t])) <= 1e-13


def pin_beta_small_limits(impl, seed=5):
    """S0 = 0 and beta -> 0 (first order in beta, error O(beta T)):
    S_T / beta -> sum_s Diag(prod_{r=s+1..T} alpha_r) k_s v_s^T (a decayed sum), and
    with alpha = 1: o_t / beta -> sum_{s<=t} (q_t . k_s) v_s (causal linear attention),
    both written as direct sums over token pairs."""
    rng = np.random.default_rng(seed)
    n, T, dk, dv = 1, 40, 8, 5
    eps = 1e-8
    q = rng.standard_normal((n, T, dk))
    k = _unit_rows(rng, (n, T, dk))
    v = rng.standard_normal((n, T, dv))
    g = -0.2 * rng.random((n, T, dk))
    beta = np.full((n, T), eps)
    _, S = impl(q, k, v, g, beta, None)
    ref = np.zeros((dk, dv))
    for s in range(T):
        decay = np.exp(g[0, s + 1:].sum(axis=0))
        ref += (decay * k[0, s])[:, None] * v[0, s][None, :]
    assert _rel(S[0] / eps, ref) <= 1e-6
    o, _ = impl(q, k, v, np.zeros_like(g), beta, None)
    for t in range(T):
        lin = sum((q[0, t] @ k[0, s]) * v[0, s] for s in range(t + 1))
        assert _rel(o[0, t] / eps, lin) <= 1e-6


# ----------------------------------------------------------------------------- P5


def pin_basis_key_overwrite(impl, seed=6):
    """k_t = e_{p_t} and beta = 1: each write replaces row p_t of the decayed
    state by v_t, so row i of S_T is v_{last(i)} times the decay of the later
    tokens, or the decayed initial row if row i was never written."""
    rng = np.random.default_rng(seed)
    dk, dv, T = 6, 4, 15
    p = rng.integers(0, dk - 1, size=T)  # row dk-1 is never written
    k = np.zeros((1, T, dk))
    k[0, np.arange(T), p] = 1.0
    q = rng.standard_normal((1, T, dk))
    v = rng.standard_normal((1, T, dv))
    g = -2.0 * rng.random((1, T, dk))
    s0 = rng.standard_normal((1, dk, dv))
    _, S = impl(q, k, v, g, np.ones((1, T)), s0)
    for i in range(dk):
        written = [t for t in range(T) if p[t] == i]
        if written:
            last = written[-1]
            expect = np.exp(g[0, last + 1:, i].sum()) * v[0, last]
        else:
            expect = np.exp(g[0, :, i].sum()) * s0[0, i]
        assert np.max(np.abs(S[0, i] - expect)) <= 1e-14 * max(1.0, np.max(np.abs(expect)))


# ----------------------------------------------------------------------------- P6


def _dense_transition(k, g, beta):
    """P_t = (I - beta_t k_t k_t^T) Diag(alpha_t), as a dense matrix."""
    return (np.eye(k.shape[0]) - beta * np.outer(k, k)) @ np.diag(np.exp(g))


def pin_dense_products(impl, seed=7):
    """T <= 8: S_t = P_t ... P_1 S0 + sum_{s<=t} P_t ... P_{s+1} beta_s k_s v_s^T with
    dense P_t, and o_t = S_t^T q_t, for every prefix t."""
    rng = np.random.default_rng(seed)
    for T in (1, 2, 5, 8):
        dk, dv = 5, 3
        q = rng.standard_normal((1, T, dk))
        k = _unit_rows(rng, (1, T, dk)) * rng.uniform(0.5, 1.0, (1, T, 1))
        v = rng.standard_normal((1, T, dv))
        g = -5.0 * rng.random((1, T, dk))
        beta = rng.random((1, T))
        s0 = rng.standard_normal((1, dk, dv))
        o, S = impl(q, k, v, g, beta, s0)
        Pm = [_dense_transition(k[0, t], g[0, t], beta[0, t]) for t in range(T)]
        for t in range(T):
            St = s0[0].copy()
            for s in range(t + 1):
                St = Pm[s] @ St
            for s in range(t + 1):
                prod = np.eye(dk)
                for r in range(s + 1, t + 1):
                    prod = Pm[r] @ prod
                St += prod @ (beta[0, s] * np.outer(k[0, s], v[0, s]))
            assert _rel(o[0, t], St.T @ q[0, t]) <= 1e-13
            if t == T - 1:
                assert _rel(S[0], St) <= 1e-13


def compose(right, left):
    """(M2, E2) o (M1, E1) = (M2 M1, M2 E1 + E2): the affine segment transition
    F(S) = M S + E applied left first (section "FlashKDA 与 KCP")."""
    m2, e2 = right
    m1, e1 = left
    return m2 @ m1, m2 @ e1 + e2


def pin_segment_composition(impl, seed=8):
    """Split a sequence into segments.  Each segment's transition M is the
    recurrence run on S0 = I with v = 0 (d_v = d_k), and its fragment E the
    recurrence run from S0 = 0.  Composing the fragments in order (eq. (17))
    must give the state of the whole sequence, and compose is associative."""
    rng = np.random.default_rng(seed)
    dk, dv, T = 6, 4, 21
    cuts = [0, 5, 6, 14, 21]
    q = rng.standard_normal((1, T, dk))
    k = _unit_rows(rng, (1, T, dk))
    v = rng.standard_normal((1, T, dv))
    g = -3.0 * rng.random((1, T, dk))
    beta = rng.random((1, T))
    s0 = rng.standard_normal((1, dk, dv))
    _, S_full = impl(q, k, v, g, beta, s0)
    frags = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        sl = slice(a, b)
        _, M = impl(q[:, sl], k[:, sl], np.zeros((1, b - a, dk)), g[:, sl], beta[:, sl], np.eye(dk)[None])
        _, E = impl(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], None)
        frags.append((M[0], E[0]))
    total = (np.eye(dk), s0[0])
    for fr in frags:
        total = compose(fr, total)
    assert _rel(total[1], S_full[0]) <= 1e-13
    # eq. (17): S_in of the last segment from the earlier fragments, started at S0
    s_in = s0[0]
    for fr in frags[:-1]:
        s_in = fr[0] @ s_in + fr[1]
    assert _rel(frags[-1][1] + frags[-1][0] @ s_in, S_full[0]) <= 1e-13
    a, b, c = frags[0], frags[1], frags[2]
    l, r = compose(compose(c, b), a), compose(c, compose(b, a))
    assert _rel(l[0], r[0]) <= 1e-14 and _rel(l[1], r[1]) <= 1e-14


# ----------------------------------------------------------------------------- P7


def pin_gate_bound(gate_fn):
    """Eq. (5): g = -5 sigmoid(a) in [-5, 0], alpha in [e^-5, 1]; the page's
    values at a = -100, 0, 100; a 16-token tile sum stays in [-80, 0] and e^80
    is below the bf16 maximum."""
    G = _golden("gate_bound.json")
    a = np.array(G["a"])
    g = gate_fn(a)
    assert np.all((g >= G["g_min"]) & (g <= 0.0))
    alpha = np.exp(g)
    assert np.all((alpha >= math.exp(G["g_min"])) & (alpha <= 1.0))
    assert np.max(np.abs(g - np.array(G["expected_g"]))) <= 1e-15
    tile = gate_fn(np.full(G["tile_tokens"], 1e6)).sum()
    assert -80.0 <= tile <= 0.0
    assert math.exp(-G["g_min"] * G["tile_tokens"]) < G["bf16_max"]


# ----------------------------------------------------------------------------- P8


def pin_split_invariance(impl, seed=9):
    """Running T1 tokens and then T2 more from the returned state gives the same
    result as one run of T1 + T2 tokens (the resume contract), bit for bit."""
    rng = np.random.default_rng(seed)
    n, T1, T2, dk, dv = 3, 17, 30, 8, 8
    T = T1 + T2
    q = rng.standard_normal((n, T, dk))
    k = _unit_rows(rng, (n, T, dk))
    v = rng.standard_normal((n, T, dv))
    g = -5.0 * rng.random((n, T, dk))
    beta = rng.random((n, T))
    s0 = rng.standard_normal((n, dk, dv))
    o, S = impl(q, k, v, g, beta, s0)
    o1, S1 = impl(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], s0)
    o2, S2 = impl(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], S1)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
    assert np.array_equal(S2, S)


ALL_PINS = [
    pin_worked_example,
    pin_scalar_hand_solved,
    pin_erase_identity,
    pin_beta_zero_exact,
    pin_beta_small_limits,
    pin_basis_key_overwrite,
    pin_dense_products,
    pin_segment_composition,
    pin_split_invariance,
]


# ----------------------------------------------------------------------------- mutants


def _recurrence(q, k, v, g, beta, s0, mutant):
    """A numpy recurrence with one deliberate mistake, selected by `mutant`."""
    n, T, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((n, T, dv))
    S_out = np.zeros((n, dk, dv))
    for u in range(n):
        S = np.zeros((dk, dv)) if s0 is None else s0[u].copy()
        for t in range(T):
            a = np.exp(g[u, t])
            kt, qt, vt, bt = k[u, t], q[u, t], v[u, t], beta[u, t]
            if mutant == "delta_before_decay":
                S = S + bt * np.outer(kt, vt - kt @ S)
                S = a[:, None] * S
                o[u, t] = S.T @ qt
                continue
            if mutant == "read_before_write":
                o[u, t] = (a[:, None] * S).T @ qt
            old = S
            S = a[:, None] * S
            if mutant == "decay_columns":
                S = old * a[None, :dv]
            e = vt - kt @ (old if mutant == "residual_undecayed" else S)
            if mutant == "sign_flip":
                S = S - bt * np.outer(kt, e)
            elif mutant == "beta_squared":
                S = S + bt * bt * np.outer(kt, e)
            else:
                S = S + bt * np.outer(kt, e)
            if mutant == "read_before_write":
                continue
            if mutant == "transposed_read":
                o[u, t] = (S @ qt[:dv])[:dv]
            elif mutant == "stale_query" and t > 0:
                o[u, t] = S.T @ q[u, t - 1]
            else:
                o[u, t] = S.T @ qt
        S_out[u] = S
    return o, S_out


MUTANTS = ["delta_before_decay", "read_before_write", "decay_columns", "residual_undecayed", "sign_flip",
           "beta_squared", "transposed_read", "stale_query"]


def mutant_impl(name):
    def impl(q, k, v, g, beta, s0):
        return _recurrence(q, k, v, g, beta, s0, name)

    return impl


GATE_MUTANTS = {
    "missing_floor": lambda a: -1.0 / (1.0 + np.exp(-a)),
    "sign_of_logit": lambda a: -5.0 / (1.0 + np.exp(a)),
    "softplus_gate": lambda a: -np.log1p(np.exp(a)),
}
