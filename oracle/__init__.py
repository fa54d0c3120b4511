"""fp64 CPU oracle for the KDA forward pass.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports or
links anything here, and nothing here imports the HIP library.

The computation lives in ``kda_oracle.c`` (plain C, fp64, one thread per
(batch, head) sequence).  It follows eq. (1) of the page
"Kimi K3：从三条信息流到完整系统", section "KDA 是带逐通道遗忘的 delta rule",
token by token (decay, then delta correction, then read after write), with
the bounded gate of eq. (5), section "下界 log-decay 是一个 kernel 设计".

Arrays here use the boundary's layouts: rows ``[B, T, H, D]``, beta
``[B, T, H]``, states ``[B, H, Dk, Dv]``, all float64.

Parity pins: every function here is pinned by the tests in
``tests/test_oracle_pins.py`` (worked example, hand-solved scalar case, erase
identity, beta = 0 and beta -> 0 closed forms, basis-key overwrite, dense
unrolled products with segment composition, gate bound, split invariance;
for ``decode_multi`` a hand-solved two-token commit, the beta = 0 closed form
at every commit count, and that tokens past the committed prefix change
neither the committed state nor earlier outputs; for the state checkpoints
of ``forward(..., state_every=E)`` the beta = 0 closed form, agreement with
runs over each prefix, and split runs resumed from a checkpoint; for
``forward_varlen`` equal-length packing against the batched layout, empty
sequences keeping their state, and the clamping of offsets; for
``output_gate_norm`` rows of constant magnitude, scale invariance and the
gate's limits).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB)
        p, i = ctypes.c_void_p, ctypes.c_int
        lib.kda_oracle_forward.argtypes = [i, i, i, i, p, p, p, p, i, p, p, p, p, i]
        lib.kda_oracle_forward.restype = i
        lib.kda_oracle_forward_states.argtypes = [i, i, i, i, p, p, p, p, i, p, p, p, p, p, i, i]
        lib.kda_oracle_forward_states.restype = i
        lib.kda_oracle_gate.argtypes = [p, p, ctypes.c_int64]
        lib.kda_oracle_gate.restype = None
        _lib = lib
    return _lib


def default_threads():
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def gate(a):
    """Eq. (5): g = -5 * sigmoid(a), elementwise, fp64."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    g = np.empty_like(a)
    _load().kda_oracle_gate(_ptr(a), _ptr(g), a.size)
    return g


def forward_units(q, k, v, gate_values, beta, s0=None, gate_is_logit=True, threads=None, state_every=None):
    """Unit-major entry: q, k, gate [n, T, Dk]; v [n, T, Dv]; beta [n, T];
    s0 [n, Dk, Dv] or None.  Returns (o [n, T, Dv], S [n, Dk, Dv]), and with
    state_every = E also the checkpoints [n, T // E, Dk, Dv]: the state after
    tokens E, 2E, ..."""
    q, k, v, gv, beta = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, gate_values, beta))
    n, T, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (n, T, dk) and gv.shape == (n, T, dk) and v.shape == (n, T, dv) and beta.shape == (n, T)
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        assert s0.shape == (n, dk, dv)
    o = np.empty((n, T, dv), dtype=np.float64)
    S = np.empty((n, dk, dv), dtype=np.float64)
    nthreads = default_threads() if threads is None else int(threads)
    if state_every is None:
        rc = _load().kda_oracle_forward(n, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(gv), int(bool(gate_is_logit)),
                                        _ptr(beta), _ptr(s0), _ptr(o), _ptr(S), nthreads)
        if rc != 0:
            raise RuntimeError(f"kda_oracle_forward failed with code {rc}")
        return o, S
    every = int(state_every)
    if every <= 0:
        raise ValueError("state_every must be positive")
    states = np.empty((n, T // every, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_forward_states(n, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(gv),
                                           int(bool(gate_is_logit)), _ptr(beta), _ptr(s0), _ptr(o), _ptr(S),
                                           _ptr(states), every, nthreads)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward_states failed with code {rc}")
    return o, S, states


def _units(x):
    """[B, T, H, D] -> [B*H, T, D] (or [B, T, H] -> [B*H, T])."""
    if x.ndim == 4:
        B, T, H, D = x.shape
        return np.ascontiguousarray(x.transpose(0, 2, 1, 3)).reshape(B * H, T, D)
    B, T, H = x.shape
    return np.ascontiguousarray(x.transpose(0, 2, 1)).reshape(B * H, T)


def forward(q, k, v, beta, a=None, g=None, s0=None, threads=None, state_every=None):
    """Boundary-layout entry.  q, k, v and a (gate logits) or g (log-decays)
    are [B, T, H, D]; beta [B, T, H]; s0 [B, H, Dk, Dv] or None.
    Returns (o [B, T, H, Dv], S_final [B, H, Dk, Dv]) in fp64, and with
    state_every = E also the state checkpoints [B, H, T // E, Dk, Dv] (the
    state after tokens E, 2E, ..., the sparse KDA checkpoints of the K3
    page's section "hybrid prefix cache")."""
    if (a is None) == (g is None):
        raise ValueError("pass exactly one of a (gate logits) or g (log-decay)")
    B, T, H, dk = q.shape
    dv = v.shape[3]
    gv = a if a is not None else g
    s0u = None if s0 is None else np.asarray(s0, dtype=np.float64).reshape(B * H, dk, dv)
    res = forward_units(_units(np.asarray(q, np.float64)), _units(np.asarray(k, np.float64)),
                        _units(np.asarray(v, np.float64)), _units(np.asarray(gv, np.float64)),
                        _units(np.asarray(beta, np.float64)), s0u, gate_is_logit=a is not None, threads=threads,
                        state_every=state_every)
    o = np.ascontiguousarray(res[0].reshape(B, H, T, dv).transpose(0, 2, 1, 3))
    if state_every is None:
        return o, res[1].reshape(B, H, dk, dv)
    return o, res[1].reshape(B, H, dk, dv), res[2].reshape(B, H, T // int(state_every), dk, dv)


def decode_step(q, k, v, beta, state, a=None, g=None, threads=None):
    """One recurrent step for every (b, h): q, k, v, a|g [B, H, D]; beta [B, H];
    state [B, H, Dk, Dv].  Returns (o [B, H, Dv], new state)."""
    o, S = forward(q[:, None], k[:, None], v[:, None], np.asarray(beta)[:, None],
                   a=None if a is None else a[:, None], g=None if g is None else g[:, None], s0=state,
                   threads=threads)
    return o[:, 0], S


def decode_multi(q, k, v, beta, state, a=None, g=None, n_commit=None, threads=None):
    """K tokens per (b, h) from a committed state, the replay of an accepted
    draft prefix (page "Kimi K3：从三条信息流到完整系统", section "recurrent
    speculative decoding 不能复制整个状态": the drafted tokens' inputs are
    cached and only the accepted prefix is replayed into the state; the rest
    is never committed).

    q, k, v, a|g [B, K, H, D]; beta [B, K, H]; state [B, H, Dk, Dv];
    n_commit [B] token counts (None = K), clamped to [0, K].  Returns
    (o [B, K, H, Dv] for every token, read from the running state after that
    token; the state after the first n_commit[b] tokens of batch row b)."""
    o, _ = forward(q, k, v, beta, a=a, g=g, s0=state, threads=threads)
    B, K = q.shape[0], q.shape[1]
    counts = np.full(B, K) if n_commit is None else np.clip(np.asarray(n_commit).reshape(B), 0, K)
    committed = np.array(state, dtype=np.float64, copy=True)
    gv = a if a is not None else g
    for b in range(B):
        m = int(counts[b])
        if m == 0:
            continue
        sl = slice(b, b + 1)
        kw = {"a": gv[sl, :m]} if a is not None else {"g": gv[sl, :m]}
        _, Sb = forward(q[sl, :m], k[sl, :m], v[sl, :m], np.asarray(beta)[sl, :m], s0=np.asarray(state)[sl],
                        threads=threads, **kw)
        committed[b] = Sb[0]
    return o, committed


def forward_varlen(q, k, v, beta, cu_seqlens, a=None, g=None, s0=None, threads=None):
    """N sequences packed along the token axis: q, k, v, a|g [T, H, D];
    beta [T, H]; sequence n is tokens cu_seqlens[n] .. cu_seqlens[n+1] - 1,
    offsets clamped to [0, T] (a decreasing pair is an empty sequence);
    s0 [N, H, Dk, Dv] or None.  Each sequence is the recurrence of
    ``forward`` on its own rows.  Returns (o [T, H, Dv], S [N, H, Dk, Dv]);
    rows outside every sequence are left zero."""
    if (a is None) == (g is None):
        raise ValueError("pass exactly one of a (gate logits) or g (log-decay)")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    T, H, dk = q.shape
    dv = v.shape[2]
    gv = a if a is not None else g
    o = np.zeros((T, H, dv), dtype=np.float64)
    S = np.empty((N, H, dk, dv), dtype=np.float64)
    for n in range(N):
        c0 = int(min(max(cu[n], 0), T))
        c1 = int(min(max(cu[n + 1], c0), T))
        sl = slice(c0, c1)
        kw = {"a": np.asarray(gv)[None, sl]} if a is not None else {"g": np.asarray(gv)[None, sl]}
        on, Sn = forward(np.asarray(q)[None, sl], np.asarray(k)[None, sl], np.asarray(v)[None, sl],
                         np.asarray(beta)[None, sl], s0=None if s0 is None else np.asarray(s0)[n:n + 1],
                         threads=threads, **kw)
        o[sl] = on[0]
        S[n] = Sn[0]
    return o, S


def output_gate_norm(o, z, eps):
    """The weight-free part of the K3 page's eq. (6) (section "KDA 是带逐通道遗忘
    的 delta rule" onward, the output gate): y = sigmoid(z) * RMSNorm(o), the
    RMSNorm taken head-wise, over the last axis (the value channels of one
    token and head), with no learned scale: o / sqrt(mean(o^2) + eps).  fp64."""
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + float(eps))
    return (1.0 / (1.0 + np.exp(-z))) * (o / rms)
