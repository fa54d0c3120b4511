"""The oracle pinned to what the pages and the mathematics fix (CPU only).

Each pin in tests/pins.py is run against the oracle; a planted-mistake check
runs the same pins against deliberately wrong recurrences and gates, so a
plausible mistake in the oracle (wrong order, sign, index, operand, scale)
could not pass unnoticed."""
import math

import numpy as np
import pytest

import oracle
from tests import pins


def oracle_impl(q, k, v, g, beta, s0):
    return oracle.forward_units(q, k, v, g, beta, s0, gate_is_logit=False, threads=2)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle_impl)


def test_oracle_gate_bound():
    pins.pin_gate_bound(oracle.gate)


def test_gate_logit_path_matches_log_decay_path():
    """The logit entry (g = -5 sigmoid(a) inside the oracle) equals the
    log-decay entry fed with the oracle's own gate values, bit for bit."""
    rng = np.random.default_rng(11)
    n, T, d = 2, 9, 8
    q, k, v, a = (rng.standard_normal((n, T, d)) for _ in range(4))
    beta = rng.random((n, T))
    o1, S1 = oracle.forward_units(q, k, v, a, beta, gate_is_logit=True)
    o2, S2 = oracle.forward_units(q, k, v, oracle.gate(a), beta, gate_is_logit=False)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_boundary_layout_wrapper():
    """forward() on [B, T, H, D] equals forward_units() per (b, h)."""
    rng = np.random.default_rng(12)
    B, T, H, d = 2, 7, 3, 4
    q, k, v, a = (rng.standard_normal((B, T, H, d)) for _ in range(4))
    beta = rng.random((B, T, H))
    s0 = rng.standard_normal((B, H, d, d))
    o, S = oracle.forward(q, k, v, beta, a=a, s0=s0)
    for b in range(B):
        for h in range(H):
            ou, Su = oracle.forward_units(q[b, :, h][None], k[b, :, h][None], v[b, :, h][None], a[b, :, h][None],
                                          beta[b, :, h][None], s0[b, h][None])
            assert np.array_equal(o[b, :, h], ou[0]) and np.array_equal(S[b, h], Su[0])


def test_decode_step_is_one_token_of_forward():
    rng = np.random.default_rng(13)
    B, H, d, steps = 2, 3, 8, 5
    q, k, v, a = (rng.standard_normal((B, steps, H, d)) for _ in range(4))
    beta = rng.random((B, steps, H))
    s0 = rng.standard_normal((B, H, d, d))
    o_ref, S_ref = oracle.forward(q, k, v, beta, a=a, s0=s0)
    S = s0
    for t in range(steps):
        o_t, S = oracle.decode_step(q[:, t], k[:, t], v[:, t], beta[:, t], S, a=a[:, t])
        assert np.array_equal(o_t, o_ref[:, t])
    assert np.array_equal(S, S_ref)


def test_decode_multi_hand_solved_two_tokens():
    """Two tokens with orthonormal keys, beta = 1 and no decay (g = 0), solved
    by hand from eq. (1): token 1 writes v1 under e1 (S1 = e1 v1^T), token 2
    writes v2 under e2 (S2 = e1 v1^T + e2 v2^T); o_t = S_t^T q_t.  Committing
    one token keeps S1, none keeps S0 = 0, both keep S2."""
    d = 4
    e1, e2 = np.eye(d)[0], np.eye(d)[1]
    v1, v2 = np.array([1.0, -2.0, 0.5, 3.0]), np.array([0.25, 4.0, -1.0, 2.0])
    q1, q2 = np.array([2.0, 7.0, 0.0, -1.0]), np.array([-3.0, 0.5, 9.0, 1.0])
    q = np.stack([q1, q2])[None, :, None]  # [B=1, K=2, H=1, d]
    k = np.stack([e1, e2])[None, :, None]
    v = np.stack([v1, v2])[None, :, None]
    g = np.zeros_like(q)
    beta = np.ones((1, 2, 1))
    s0 = np.zeros((1, 1, d, d))
    S1, S2 = np.outer(e1, v1), np.outer(e1, v1) + np.outer(e2, v2)
    for m, want in ((0, np.zeros((d, d))), (1, S1), (2, S2)):
        o, S = oracle.decode_multi(q, k, v, beta, s0, g=g, n_commit=[m])
        assert np.allclose(o[0, 0, 0], q1[0] * v1, rtol=0, atol=1e-15)
        assert np.allclose(o[0, 1, 0], q2[0] * v1 + q2[1] * v2, rtol=0, atol=1e-15)
        assert np.allclose(S[0, 0], want, rtol=0, atol=1e-15)
    # counts outside [0, K] are clamped
    assert np.array_equal(oracle.decode_multi(q, k, v, beta, s0, g=g, n_commit=[-3])[1], s0)
    assert np.allclose(oracle.decode_multi(q, k, v, beta, s0, g=g, n_commit=[9])[1][0, 0], S2, rtol=0, atol=1e-15)


def test_decode_multi_beta_zero_closed_form():
    """beta = 0 and g = 0 make every step the identity on S (eq. (1)), so
    o_t = S0^T q_t for every token and the committed state is S0 at every
    commit count."""
    rng = np.random.default_rng(21)
    B, K, H, d = 3, 5, 2, 6
    q, k, v = (rng.standard_normal((B, K, H, d)) for _ in range(3))
    s0 = rng.standard_normal((B, H, d, d))
    o, S = oracle.decode_multi(q, k, v, np.zeros((B, K, H)), s0, g=np.zeros((B, K, H, d)), n_commit=[0, 2, 5])
    assert np.allclose(o, np.einsum("bhij,bkhi->bkhj", s0, q), rtol=1e-13, atol=1e-13)
    assert np.allclose(S, s0, rtol=1e-13, atol=1e-13)


def test_decode_multi_uncommitted_tokens_change_nothing_committed():
    """The committed state after m tokens, and the outputs of tokens before t,
    do not depend on the inputs of later tokens; n_commit = 0 returns the
    state bit for bit."""
    rng = np.random.default_rng(22)
    B, K, H, d = 2, 6, 2, 8
    q, k, v, a = (rng.standard_normal((B, K, H, d)) for _ in range(4))
    beta = rng.random((B, K, H))
    s0 = rng.standard_normal((B, H, d, d))
    counts = [3, 0]
    o, S = oracle.decode_multi(q, k, v, beta, s0, a=a, n_commit=counts)
    assert np.array_equal(S[1], s0[1])
    q2, k2, v2, a2 = (x.copy() for x in (q, k, v, a))
    beta2 = beta.copy()
    for x in (q2, k2, v2, a2):
        x[:, 3:] = rng.standard_normal(x[:, 3:].shape)
    beta2[:, 3:] = rng.random(beta2[:, 3:].shape)
    o2, S2 = oracle.decode_multi(q2, k2, v2, beta2, s0, a=a2, n_commit=counts)
    assert np.array_equal(S2, S)
    assert np.array_equal(o2[:, :3], o[:, :3])
    assert not np.allclose(o2[:, 3:], o[:, 3:])


def test_checkpoints_beta_zero_closed_form():
    """beta = 0 leaves only the decay in eq. (1): the state after t tokens is
    Diag(exp(sum of g over tokens 1..t)) S0, computed here directly, at every
    checkpoint."""
    rng = np.random.default_rng(31)
    B, T, H, d, every = 2, 37, 2, 5, 6
    q, k, v = (rng.standard_normal((B, T, H, d)) for _ in range(3))
    g = -5.0 * rng.random((B, T, H, d))
    s0 = rng.standard_normal((B, H, d, d))
    _, S, ck = oracle.forward(q, k, v, np.zeros((B, T, H)), g=g, s0=s0, state_every=every)
    assert ck.shape == (B, H, T // every, d, d)
    for i in range(T // every):
        t = every * (i + 1)
        decay = np.exp(g[:, :t].sum(axis=1))  # [B, H, d]
        assert np.allclose(ck[:, :, i], decay[..., None] * s0, rtol=1e-12, atol=1e-14)
    assert np.allclose(S, np.exp(g.sum(axis=1))[..., None] * s0, rtol=1e-12, atol=1e-14)


def test_checkpoints_are_the_states_of_each_prefix():
    """Checkpoint i is the state a run over the first E (i + 1) tokens ends
    with, bit for bit, and a run resumed from checkpoint i over the remaining
    tokens reproduces the full run's outputs and final state."""
    rng = np.random.default_rng(32)
    B, T, H, d, every = 2, 50, 3, 6, 16
    q, k, v, a = (rng.standard_normal((B, T, H, d)) for _ in range(4))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    beta = rng.random((B, T, H))
    s0 = rng.standard_normal((B, H, d, d))
    o, S, ck = oracle.forward(q, k, v, beta, a=a, s0=s0, state_every=every)
    o2, S2 = oracle.forward(q, k, v, beta, a=a, s0=s0)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)
    assert ck.shape == (B, H, 3, d, d)
    for i in range(3):
        t = every * (i + 1)
        _, St = oracle.forward(q[:, :t], k[:, :t], v[:, :t], beta[:, :t], a=a[:, :t], s0=s0)
        assert np.array_equal(ck[:, :, i], St)
        o_rest, S_rest = oracle.forward(q[:, t:], k[:, t:], v[:, t:], beta[:, t:], a=a[:, t:], s0=ck[:, :, i])
        assert np.array_equal(o_rest, o[:, t:]) and np.array_equal(S_rest, S)
    # fewer tokens than the interval: no checkpoints
    assert oracle.forward(q[:, :10], k[:, :10], v[:, :10], beta[:, :10], a=a[:, :10], s0=s0,
                          state_every=every)[2].shape == (B, H, 0, d, d)


def test_varlen_equal_lengths_match_the_batched_layout():
    """N sequences of one length T packed along the token axis are the
    batched [N, T, H, D] problem: same outputs and states, bit for bit."""
    rng = np.random.default_rng(41)
    N, T, H, d = 3, 11, 2, 5
    q, k, v, a = (rng.standard_normal((N, T, H, d)) for _ in range(4))
    beta = rng.random((N, T, H))
    s0 = rng.standard_normal((N, H, d, d))
    o_b, S_b = oracle.forward(q, k, v, beta, a=a, s0=s0)
    cu = np.arange(N + 1) * T
    o_p, S_p = oracle.forward_varlen(q.reshape(N * T, H, d), k.reshape(N * T, H, d), v.reshape(N * T, H, d),
                                     beta.reshape(N * T, H), cu, a=a.reshape(N * T, H, d), s0=s0)
    assert np.array_equal(o_p, o_b.reshape(N * T, H, d)) and np.array_equal(S_p, S_b)


def test_varlen_empty_sequences_and_clamped_offsets():
    """A sequence of length 0 keeps its initial state (zeros without one);
    offsets outside [0, T] are clamped and a decreasing pair is empty, so the
    sequences below cover tokens [0, 4), [4, 9), [9, 12) and nothing."""
    rng = np.random.default_rng(42)
    T, H, d = 12, 2, 4
    q, k, v, a = (rng.standard_normal((T, H, d)) for _ in range(4))
    beta = rng.random((T, H))
    s0 = rng.standard_normal((4, H, d, d))
    cu = [-5, 4, 9, 40, 7]
    o, S = oracle.forward_varlen(q, k, v, beta, cu, a=a, s0=s0)
    assert np.array_equal(S[3], s0[3])
    for n, (t0, t1) in enumerate([(0, 4), (4, 9), (9, 12), (12, 12)]):
        on, Sn = oracle.forward(q[None, t0:t1], k[None, t0:t1], v[None, t0:t1], beta[None, t0:t1],
                                a=a[None, t0:t1], s0=s0[n:n + 1])
        assert np.array_equal(S[n], Sn[0]) and np.array_equal(o[t0:t1], on[0])
    _, Sz = oracle.forward_varlen(q, k, v, beta, [0, 0, 12], a=a)
    assert np.array_equal(Sz[0], np.zeros((H, d, d)))


def test_output_gate_norm_closed_forms():
    """Eq. (6) without W_o and W_g: rows of constant magnitude c normalise to
    their signs (eps = 0); the result does not change when a row is scaled
    (eps = 0); z = 0 halves RMSNorm(o) and z -> +inf leaves it."""
    rng = np.random.default_rng(51)
    signs = rng.choice([-1.0, 1.0], size=(5, 3, 128))
    z = rng.standard_normal((5, 3, 128))
    y = oracle.output_gate_norm(3.5 * signs, z, 0.0)
    assert np.allclose(y, signs / (1.0 + np.exp(-z)), rtol=1e-14, atol=0)
    o = rng.standard_normal((4, 2, 128))
    assert np.allclose(oracle.output_gate_norm(o, z[:4, :2], 0.0), oracle.output_gate_norm(7.25 * o, z[:4, :2], 0.0),
                       rtol=1e-13, atol=1e-15)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + 1e-6)
    assert np.allclose(oracle.output_gate_norm(o, np.zeros_like(o), 1e-6), 0.5 * o / rms, rtol=1e-14, atol=0)
    assert np.allclose(oracle.output_gate_norm(o, np.full_like(o, 800.0), 1e-6), o / rms, rtol=1e-14, atol=0)
    # a zero row stays zero for eps > 0
    assert not np.any(oracle.output_gate_norm(np.zeros((1, 128)), np.ones((1, 128)), 1e-6))


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(14)
    s0 = rng.standard_normal((2, 4, 4))
    e = np.zeros((2, 0, 4))
    o, S = oracle.forward_units(e, e, e, e, np.zeros((2, 0)), s0)
    assert o.shape == (2, 0, 4) and np.array_equal(S, s0)
    o, S = oracle.forward_units(e, e, e, e, np.zeros((2, 0)), None)
    assert np.array_equal(S, np.zeros((2, 4, 4)))


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(15)
    n, T, d = 7, 20, 8
    q, k, v, a = (rng.standard_normal((n, T, d)) for _ in range(4))
    beta = rng.random((n, T))
    r1 = oracle.forward_units(q, k, v, a, beta, threads=1)
    r5 = oracle.forward_units(q, k, v, a, beta, threads=5)
    assert np.array_equal(r1[0], r5[0]) and np.array_equal(r1[1], r5[1])


@pytest.mark.parametrize("name", pins.MUTANTS)
def test_pins_catch_planted_recurrence_mistake(name):
    impl = pins.mutant_impl(name)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"


@pytest.mark.parametrize("name", sorted(pins.GATE_MUTANTS))
def test_pins_catch_planted_gate_mistake(name):
    with pytest.raises(AssertionError):
        with np.errstate(over="ignore"):
            pins.pin_gate_bound(pins.GATE_MUTANTS[name])


def test_mutant_harness_is_faithful_without_a_mistake():
    """The numpy recurrence used for the mutants, run with no mistake,
    passes every pin (so the mutants fail because of their mistake)."""
    impl = pins.mutant_impl("none")
    for pin in pins.ALL_PINS:
        pin(impl)
