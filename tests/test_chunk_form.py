"""Chunkwise form (eq. (3)-(4)) aligned with the token-by-token recurrence
(eq. (1)), in fp64 on the CPU -- the operator-level check the page
"Kimi K3：从三条信息流到完整系统" names in "怎样继续验证 K3".

The chunk form written here is the one the GPU kernels implement: inside a
chunk of C tokens with entering state S, b_r = sum_{s<=r} g_s, Gamma = e^b,
  L  = StrictTril((K*Gamma)(K/Gamma)^T),  A = Tril((Q*Gamma)(K/Gamma)^T)
  Vt = (I + Diag(beta) L)^{-1} Diag(beta) (V - (K*Gamma) S)     (pseudo-value U - W S)
  O  = (Q*Gamma) S + A Vt                                          (eq. (4))
  S' = Diag(Gamma_C) S + (K * Gamma_C / Gamma)^T Vt                (state carry)
The pages define eq. (3)-(4) and the pseudo-value; U, W and the carry are
derived from eq. (1) (substitute S_r = Diag(Gamma_r) R_r).  Optionally every
exponent is taken relative to a pivot token p inside the chunk, which leaves
the products unchanged and keeps the factors within e^{+-5 C/2}."""
import numpy as np
import pytest

import oracle


def chunk_forward(q, k, v, g, beta, s0, C=16, pivot=None):
    n, T, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((n, T, dv))
    S_out = np.zeros((n, dk, dv))
    for u in range(n):
        S = np.zeros((dk, dv)) if s0 is None else s0[u].copy()
        for c0 in range(0, T, C):
            sl = slice(c0, min(T, c0 + C))
            Q, K, V, G, bt = q[u, sl], k[u, sl], v[u, sl], g[u, sl], beta[u, sl]
            m = Q.shape[0]
            b = np.cumsum(G, axis=0)
            p = b[min(pivot, m - 1)] if pivot is not None else np.zeros(dk)
            Qh, Kh, Kt = Q * np.exp(b - p), K * np.exp(b - p), K * np.exp(p - b)
            L = np.tril(Kh @ Kt.T, -1)
            Am = np.tril(Qh @ Kt.T)
            Mt = np.linalg.solve(np.eye(m) + bt[:, None] * L, np.diag(bt))
            Sp = np.exp(p)[:, None] * S          # state decayed to the pivot
            Vt = Mt @ (V - Kh @ Sp)
            o[u, sl] = Qh @ Sp + Am @ Vt
            S = np.exp(b[-1])[:, None] * S + (K * np.exp(b[-1] - b)).T @ Vt
        S_out[u] = S
    return o, S_out


@pytest.mark.parametrize("T", [1, 15, 16, 17, 100])
@pytest.mark.parametrize("pivot", [None, 7])
def test_chunk_form_matches_recurrence(T, pivot):
    rng = np.random.default_rng(T)
    n, dk, dv = 2, 16, 12
    q = rng.standard_normal((n, T, dk))
    k = rng.standard_normal((n, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((n, T, dv))
    a = rng.standard_normal((n, T, dk))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((n, T))))
    s0 = 0.1 * rng.standard_normal((n, dk, dv))
    g = oracle.gate(a)
    o_ref, S_ref = oracle.forward_units(q, k, v, g, beta, s0, gate_is_logit=False)
    o, S = chunk_forward(q, k, v, g, beta, s0, pivot=pivot)
    assert np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref) < 1e-12
    assert np.linalg.norm(S - S_ref) / np.linalg.norm(S_ref) < 1e-12


def test_chunk_form_at_the_decay_floor():
    """Every gate at the floor g = -5: a 16-token tile spans e^{-80}; with the
    pivot the factors stay within e^{+-40} and the form still matches."""
    rng = np.random.default_rng(1)
    n, T, d = 1, 48, 8
    q, k, v = (rng.standard_normal((n, T, d)) for _ in range(3))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g = np.full((n, T, d), -5.0)
    g[..., : d // 2] = -1e-3
    beta = rng.random((n, T))
    o_ref, S_ref = oracle.forward_units(q, k, v, g, beta, None, gate_is_logit=False)
    o, S = chunk_forward(q, k, v, g, beta, None, pivot=7)
    assert np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref) < 1e-12
    assert np.linalg.norm(S - S_ref) / np.linalg.norm(S_ref) < 1e-12
