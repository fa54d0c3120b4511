"""Python binding of libkda (include/kda.h): the KDA forward pass on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI; torch provides device memory and the stream.  There
is no fallback: if libkda.so is missing or was not built, every call raises.

    kda_chunk_fwd(q, k, v, a, beta, initial_state=None, o=None, final_state=None)
        -> (o, final_state)
    kda_chunk_fwd_states(q, k, v, a, beta, state_every, ...) -> (o, final_state, states)
        (also the state after every state_every tokens)
    kda_chunk_fwd_varlen(q, k, v, a, beta, cu_seqlens, ...) -> (o, final_state)
        (sequences packed along the token axis, [T, H, 128])
    kda_decode_step(q, k, v, a, beta, state, o=None) -> o      (state updated in place)
    kda_output_gate_norm(o, z, eps=1e-6, y=None) -> y   (sigmoid(z) * RMSNorm(o), eq. (6) without W_o, W_g)
    kda_decode_multi(q, k, v, a, beta, state, n_commit=None, o=None) -> o
        (K tokens per sequence; the state keeps the first n_commit[b] of them)
    kda_chunk_fwd_gated / kda_decode_step_gated / kda_decode_multi_gated(..., gate=...)
        (gate "channel" = KDA, "scalar" = one fp32 logit per token and head,
        "none" = alpha = 1, the delta rule)
    kda_chunk_fwd_norm(q, k, v, a, beta, z, eps=1e-6, ...) -> (y, final_state)
        (the prefill with sigmoid(z) * RMSNorm(o) fused into its output store)
    kda_chunk_fwd_split(q, k, v, a, beta, segments, ...) -> (o, final_state)
        (each sequence cut into segments that run side by side)

Layouts (contiguous CUDA tensors): q, k, v, a, o ``[B, T, H, 128]`` (prefill),
``[B, H, 128]`` (decode) or ``[B, K, H, 128]`` (several tokens) in bfloat16 or
float32; beta ``[B, T, H]`` / ``[B, H]`` / ``[B, K, H]`` float32; states
``[B, H, 128, 128]`` float32.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP = 0, 1, 2, 3
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_CHANNEL, KDA_GATE_SCALAR, KDA_GATE_NONE = 0, 1, 2
GATES = {"channel": KDA_GATE_CHANNEL, "scalar": KDA_GATE_SCALAR, "none": KDA_GATE_NONE}
D = 128

_lib = None


class KdaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib():
    """The loaded libkda (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build(); there is no fallback")
        L = ctypes.CDLL(LIB_PATH)
        p, i = ctypes.c_void_p, ctypes.c_int
        L.kda_chunk_fwd.argtypes = [p, p, p, p, p, p, p, p, i, i, i, i, i, i, p]
        L.kda_chunk_fwd.restype = i
        L.kda_decode_step.argtypes = [p, p, p, p, p, p, p, i, i, i, i, i, p]
        L.kda_decode_step.restype = i
        L.kda_chunk_fwd_varlen.argtypes = [p, p, p, p, p, p, p, p, p, i, i, i, i, i, i, p]
        L.kda_chunk_fwd_varlen.restype = i
        L.kda_chunk_fwd_states.argtypes = [p, p, p, p, p, p, p, p, p, i, i, i, i, i, i, i, p]
        L.kda_chunk_fwd_states.restype = i
        L.kda_decode_multi.argtypes = [p, p, p, p, p, p, p, p, i, i, i, i, i, i, p]
        L.kda_decode_multi.restype = i
        L.kda_output_gate_norm.argtypes = [p, p, p, ctypes.c_int64, i, ctypes.c_float, i, p]
        L.kda_output_gate_norm.restype = i
        L.kda_compose_segments.argtypes = [p, p, p, p, i, i, i, i, i, p]
        L.kda_compose_segments.restype = i
        L.kda_chunk_fwd_gated.argtypes = [p, p, p, p, p, p, p, p, i, i, i, i, i, i, i, p]
        L.kda_chunk_fwd_gated.restype = i
        L.kda_decode_step_gated.argtypes = [p, p, p, p, p, p, p, i, i, i, i, i, i, p]
        L.kda_decode_step_gated.restype = i
        L.kda_decode_multi_gated.argtypes = [p, p, p, p, p, p, p, p, i, i, i, i, i, i, i, p]
        L.kda_decode_multi_gated.restype = i
        L.kda_chunk_fwd_norm.argtypes = [p, p, p, p, p, p, p, ctypes.c_float, p, p, i, i, i, i, i, i, p]
        L.kda_chunk_fwd_norm.restype = i
        L.kda_chunk_fwd_split_workspace.argtypes = [i, i, i, i]
        L.kda_chunk_fwd_split_workspace.restype = ctypes.c_size_t
        L.kda_chunk_fwd_split.argtypes = [p, p, p, p, p, p, p, p, i, p, ctypes.c_size_t, i, i, i, i, i, i, p]
        L.kda_chunk_fwd_split.restype = i
        L.kda_chunk_fwd_split_noalloc.argtypes = [p, p, p, p, p, p, p, p, i, i, i, i, i, i, i, p]
        L.kda_chunk_fwd_split_noalloc.restype = i
        L.kda_status_string.argtypes = [i]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_last_error.argtypes = []
        L.kda_last_error.restype = ctypes.c_char_p
        L.kda_version.argtypes = []
        L.kda_version.restype = i
        _lib = L
    return _lib


def _check(status):
    if status != KDA_OK:
        L = lib()
        raise KdaError(status, f"{L.kda_status_string(status).decode()}: {L.kda_last_error().decode()}")


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v/a must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (the device of q), got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device, stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def kda_chunk_fwd(q, k, v, a, beta, initial_state=None, o=None, final_state=None, stream=None):
    """Chunkwise prefill (kda_chunk_fwd of include/kda.h).  Allocates o and
    final_state with torch when they are not given.  Returns (o, final_state)."""
    import torch

    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, 128]")
    B, T, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _require(q, "q", (B, T, H, Dk), dt, dev)
    _require(k, "k", (B, T, H, Dk), dt, dev)
    _require(a, "a", (B, T, H, Dk), dt, dev)
    if v.dim() != 4:
        raise ValueError("v must be [B, T, H, Dv]")
    Dv = v.shape[3]
    _require(v, "v", (B, T, H, Dv), dt, dev)
    _require(beta, "beta", (B, T, H), torch.float32, dev)
    if initial_state is not None:
        _require(initial_state, "initial_state", (B, H, Dk, Dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=dt, device=dev)
    _require(o, "o", (B, T, H, Dv), dt, dev)
    if final_state is None:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    _require(final_state, "final_state", (B, H, Dk, Dv), torch.float32, dev)
    _check(lib().kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(initial_state), _ptr(o),
                               _ptr(final_state), B, T, H, Dk, Dv, code, _stream(dev, stream)))
    return o, final_state


def _gate_code(gate):
    if isinstance(gate, str):
        if gate not in GATES:
            raise ValueError(f"gate must be one of {sorted(GATES)}, got {gate!r}")
        return GATES[gate]
    if gate not in GATES.values():
        raise ValueError(f"unknown gate {gate}")
    return int(gate)


def _require_gate(a, gate, rows_shape, dt, dev):
    """a per key channel ([..., 128] in the I/O dtype), one fp32 logit per
    token and head (rows_shape), or nothing."""
    import torch

    if gate == KDA_GATE_CHANNEL:
        _require(a, "a", tuple(rows_shape) + (D,), dt, dev)
    elif gate == KDA_GATE_SCALAR:
        _require(a, "a", tuple(rows_shape), torch.float32, dev)
    elif a is not None:
        raise ValueError("gate 'none' reads no logits: pass a=None")


def kda_chunk_fwd_gated(q, k, v, a, beta, gate="channel", initial_state=None, o=None, final_state=None, stream=None):
    """kda_chunk_fwd with a choice of gate (kda_chunk_fwd_gated of
    include/kda.h): "channel" (a [B, T, H, 128] like q), "scalar" (a
    [B, T, H] float32, one logit per token and head) or "none" (a = None,
    alpha = 1).  Returns (o, final_state)."""
    import torch

    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, 128]")
    B, T, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    g = _gate_code(gate)
    _require(q, "q", (B, T, H, Dk), dt, dev)
    _require(k, "k", (B, T, H, Dk), dt, dev)
    _require(v, "v", (B, T, H, D), dt, dev)
    _require_gate(a, g, (B, T, H), dt, dev)
    _require(beta, "beta", (B, T, H), torch.float32, dev)
    if initial_state is not None:
        _require(initial_state, "initial_state", (B, H, Dk, D), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, D), dtype=dt, device=dev)
    _require(o, "o", (B, T, H, D), dt, dev)
    if final_state is None:
        final_state = torch.empty((B, H, Dk, D), dtype=torch.float32, device=dev)
    _require(final_state, "final_state", (B, H, Dk, D), torch.float32, dev)
    _check(lib().kda_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(initial_state), _ptr(o),
                                     _ptr(final_state), B, T, H, Dk, D, code, g, _stream(dev, stream)))
    return o, final_state


def kda_chunk_fwd_norm(q, k, v, a, beta, z, eps=1e-6, initial_state=None, y=None, final_state=None, stream=None):
    """The prefill with the output gate and head-wise RMSNorm of eq. (6)
    fused into its output (kda_chunk_fwd_norm of include/kda.h):
    y = sigmoid(z) * o / sqrt(mean(o^2) + eps), z like o.  Returns
    (y, final_state); o is never written."""
    import torch

    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, 128]")
    B, T, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for t, name in ((q, "q"), (k, "k"), (a, "a")):
        _require(t, name, (B, T, H, Dk), dt, dev)
    _require(v, "v", (B, T, H, D), dt, dev)
    _require(z, "z", (B, T, H, D), dt, dev)
    _require(beta, "beta", (B, T, H), torch.float32, dev)
    if initial_state is not None:
        _require(initial_state, "initial_state", (B, H, Dk, D), torch.float32, dev)
    if y is None:
        y = torch.empty((B, T, H, D), dtype=dt, device=dev)
    _require(y, "y", (B, T, H, D), dt, dev)
    if final_state is None:
        final_state = torch.empty((B, H, Dk, D), dtype=torch.float32, device=dev)
    _require(final_state, "final_state", (B, H, Dk, D), torch.float32, dev)
    _check(lib().kda_chunk_fwd_norm(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(initial_state), _ptr(z),
                                    float(eps), _ptr(y), _ptr(final_state), B, T, H, Dk, D, code,
                                    _stream(dev, stream)))
    return y, final_state


def kda_chunk_fwd_states(q, k, v, a, beta, state_every, initial_state=None, o=None, final_state=None, states=None,
                         stream=None):
    """kda_chunk_fwd that also returns the state after every `state_every`
    tokens (kda_chunk_fwd_states of include/kda.h): states [B, H, T //
    state_every, 128, 128] float32.  Returns (o, final_state, states)."""
    import torch

    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, 128]")
    B, T, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _require(q, "q", (B, T, H, Dk), dt, dev)
    _require(k, "k", (B, T, H, Dk), dt, dev)
    _require(a, "a", (B, T, H, Dk), dt, dev)
    if v.dim() != 4:
        raise ValueError("v must be [B, T, H, Dv]")
    Dv = v.shape[3]
    _require(v, "v", (B, T, H, Dv), dt, dev)
    _require(beta, "beta", (B, T, H), torch.float32, dev)
    if initial_state is not None:
        _require(initial_state, "initial_state", (B, H, Dk, Dv), torch.float32, dev)
    every = int(state_every)
    if every <= 0 or every % 16:
        raise ValueError(f"state_every must be a positive multiple of 16, got {state_every}")
    n = T // every
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=dt, device=dev)
    _require(o, "o", (B, T, H, Dv), dt, dev)
    if final_state is None:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    _require(final_state, "final_state", (B, H, Dk, Dv), torch.float32, dev)
    if states is None:
        states = torch.empty((B, H, n, Dk, Dv), dtype=torch.float32, device=dev)
    _require(states, "states", (B, H, n, Dk, Dv), torch.float32, dev)
    _check(lib().kda_chunk_fwd_states(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(initial_state), _ptr(o),
                                      _ptr(final_state), _ptr(states) if n > 0 else None, every, B, T, H, Dk, Dv, code,
                                      _stream(dev, stream)))
    return o, final_state, states


def kda_chunk_fwd_varlen(q, k, v, a, beta, cu_seqlens, initial_state=None, o=None, final_state=None, stream=None):
    """Prefill over N sequences packed along the token axis
    (kda_chunk_fwd_varlen of include/kda.h): q, k, v, a [T, H, 128]; beta
    [T, H]; cu_seqlens an int32 GPU tensor [N + 1]; states [N, H, 128, 128].
    Returns (o [T, H, 128], final_state)."""
    import torch

    if q.dim() != 3:
        raise ValueError("q must be [T, H, 128]")
    T, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _require(q, "q", (T, H, Dk), dt, dev)
    _require(k, "k", (T, H, Dk), dt, dev)
    _require(a, "a", (T, H, Dk), dt, dev)
    if v.dim() != 3:
        raise ValueError("v must be [T, H, Dv]")
    Dv = v.shape[2]
    _require(v, "v", (T, H, Dv), dt, dev)
    _require(beta, "beta", (T, H), torch.float32, dev)
    if cu_seqlens is None or cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of N + 1 offsets")
    N = cu_seqlens.shape[0] - 1
    _require(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if initial_state is not None:
        _require(initial_state, "initial_state", (N, H, Dk, Dv), torch.float32, dev)
    if o is None:
        o = torch.empty((T, H, Dv), dtype=dt, device=dev)
    _require(o, "o", (T, H, Dv), dt, dev)
    if final_state is None:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    _require(final_state, "final_state", (N, H, Dk, Dv), torch.float32, dev)
    _check(lib().kda_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(cu_seqlens),
                                      _ptr(initial_state), _ptr(o), _ptr(final_state), N, T, H, Dk, Dv, code,
                                      _stream(dev, stream)))
    return o, final_state


def kda_decode_step(q, k, v, a, beta, state, o=None, stream=None):
    """One recurrent step (kda_decode_step of include/kda.h); state is
    updated in place.  Returns o."""
    import torch

    if q.dim() != 3:
        raise ValueError("q must be [B, H, 128]")
    B, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _require(q, "q", (B, H, Dk), dt, dev)
    _require(k, "k", (B, H, Dk), dt, dev)
    _require(a, "a", (B, H, Dk), dt, dev)
    if v.dim() != 3:
        raise ValueError("v must be [B, H, Dv]")
    Dv = v.shape[2]
    _require(v, "v", (B, H, Dv), dt, dev)
    _require(beta, "beta", (B, H), torch.float32, dev)
    _require(state, "state", (B, H, Dk, Dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, Dv), dtype=dt, device=dev)
    _require(o, "o", (B, H, Dv), dt, dev)
    _check(lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(state), _ptr(o), B, H, Dk, Dv,
                                 code, _stream(dev, stream)))
    return o


def kda_decode_step_gated(q, k, v, a, beta, state, gate="channel", o=None, stream=None):
    """kda_decode_step with a choice of gate (kda_decode_step_gated of
    include/kda.h): a [B, H, 128] like q ("channel"), [B, H] float32
    ("scalar") or None ("none").  Returns o; state is updated in place."""
    import torch

    if q.dim() != 3:
        raise ValueError("q must be [B, H, 128]")
    B, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    g = _gate_code(gate)
    _require(q, "q", (B, H, Dk), dt, dev)
    _require(k, "k", (B, H, Dk), dt, dev)
    _require(v, "v", (B, H, D), dt, dev)
    _require_gate(a, g, (B, H), dt, dev)
    _require(beta, "beta", (B, H), torch.float32, dev)
    _require(state, "state", (B, H, Dk, D), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, D), dtype=dt, device=dev)
    _require(o, "o", (B, H, D), dt, dev)
    _check(lib().kda_decode_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(state), _ptr(o), B, H,
                                       Dk, D, code, g, _stream(dev, stream)))
    return o


def kda_decode_multi_gated(q, k, v, a, beta, state, gate="channel", n_commit=None, o=None, stream=None):
    """kda_decode_multi with a choice of gate: a [B, K, H, 128] like q
    ("channel"), [B, K, H] float32 ("scalar") or None ("none")."""
    import torch

    if q.dim() != 4:
        raise ValueError("q must be [B, K, H, 128]")
    B, K, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    g = _gate_code(gate)
    _require(q, "q", (B, K, H, Dk), dt, dev)
    _require(k, "k", (B, K, H, Dk), dt, dev)
    _require(v, "v", (B, K, H, D), dt, dev)
    _require_gate(a, g, (B, K, H), dt, dev)
    _require(beta, "beta", (B, K, H), torch.float32, dev)
    _require(state, "state", (B, H, Dk, D), torch.float32, dev)
    if n_commit is not None:
        _require(n_commit, "n_commit", (B,), torch.int32, dev)
    if o is None:
        o = torch.empty((B, K, H, D), dtype=dt, device=dev)
    _require(o, "o", (B, K, H, D), dt, dev)
    _check(lib().kda_decode_multi_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(state), _ptr(o),
                                        _ptr(n_commit), B, K, H, Dk, D, code, g, _stream(dev, stream)))
    return o


def kda_decode_multi(q, k, v, a, beta, state, n_commit=None, o=None, stream=None):
    """K tokens per sequence in one pass (kda_decode_multi of include/kda.h):
    q, k, v, a [B, K, H, 128]; beta [B, K, H]; n_commit None (all K) or an
    int32 GPU tensor [B] of tokens committed to the state, which is updated
    in place.  Returns o [B, K, H, 128]."""
    import torch

    if q.dim() != 4:
        raise ValueError("q must be [B, K, H, 128]")
    B, K, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _require(q, "q", (B, K, H, Dk), dt, dev)
    _require(k, "k", (B, K, H, Dk), dt, dev)
    _require(a, "a", (B, K, H, Dk), dt, dev)
    if v.dim() != 4:
        raise ValueError("v must be [B, K, H, Dv]")
    Dv = v.shape[3]
    _require(v, "v", (B, K, H, Dv), dt, dev)
    _require(beta, "beta", (B, K, H), torch.float32, dev)
    _require(state, "state", (B, H, Dk, Dv), torch.float32, dev)
    if n_commit is not None:
        _require(n_commit, "n_commit", (B,), torch.int32, dev)
    if o is None:
        o = torch.empty((B, K, H, Dv), dtype=dt, device=dev)
    _require(o, "o", (B, K, H, Dv), dt, dev)
    _check(lib().kda_decode_multi(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(state), _ptr(o),
                                  _ptr(n_commit), B, K, H, Dk, Dv, code, _stream(dev, stream)))
    return o


def kda_output_gate_norm(o, z, eps=1e-6, y=None, stream=None):
    """y = sigmoid(z) * o / sqrt(mean(o^2) + eps) over the last axis of 128
    value channels (kda_output_gate_norm of include/kda.h); o and z of one
    shape and dtype, y may be o.  Returns y."""
    if o.shape[-1] != D:
        raise ValueError(f"the last axis of o must have {D} channels")
    dev, dt = o.device, o.dtype
    code = _dtype_code(o)
    _require(o, "o", tuple(o.shape), dt, dev)
    _require(z, "z", tuple(o.shape), dt, dev)
    if y is None:
        import torch

        y = torch.empty_like(o)
    _require(y, "y", tuple(o.shape), dt, dev)
    rows = o.numel() // D
    _check(lib().kda_output_gate_norm(_ptr(o), _ptr(z), _ptr(y), rows, D, float(eps), code, _stream(dev, stream)))
    return y


def kda_chunk_fwd_split_workspace(B, T, H, segments):
    """Bytes of workspace kda_chunk_fwd_split needs for this shape."""
    return int(lib().kda_chunk_fwd_split_workspace(int(B), int(T), int(H), int(segments)))


def kda_chunk_fwd_split(q, k, v, a, beta, segments, initial_state=None, o=None, final_state=None, workspace=None,
                        stream=None):
    """kda_chunk_fwd with each sequence cut into `segments` pieces that run
    side by side (kda_chunk_fwd_split of include/kda.h: the page's KCP
    decomposition on one device).  Same arguments and results as
    kda_chunk_fwd (up to rounding).  workspace: a CUDA uint8 tensor of at
    least kda_chunk_fwd_split_workspace(B, T, H, segments) bytes, or None
    to take one from torch.  With a stream given, the workspace and the
    outputs are allocated on that stream, so torch does not hand their
    memory to other work before the stream is done with it."""
    import contextlib

    import torch

    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, 128]")
    B, T, H, Dk = q.shape
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    P = int(segments)
    if P < 1:
        raise ValueError("segments must be at least 1")
    for t, name in ((q, "q"), (k, "k"), (a, "a")):
        _require(t, name, (B, T, H, Dk), dt, dev)
    _require(v, "v", (B, T, H, D), dt, dev)
    _require(beta, "beta", (B, T, H), torch.float32, dev)
    if initial_state is not None:
        _require(initial_state, "initial_state", (B, H, Dk, D), torch.float32, dev)
    if o is not None:
        _require(o, "o", (B, T, H, D), dt, dev)
    if final_state is not None:
        _require(final_state, "final_state", (B, H, Dk, D), torch.float32, dev)
    need = kda_chunk_fwd_split_workspace(B, T, H, P)
    if workspace is not None:
        _require(workspace, "workspace", tuple(workspace.shape), torch.uint8, dev)
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
    with ctx:
        if o is None:
            o = torch.empty((B, T, H, D), dtype=dt, device=dev)
        if final_state is None:
            final_state = torch.empty((B, H, Dk, D), dtype=torch.float32, device=dev)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _check(lib().kda_chunk_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(initial_state),
                                         _ptr(o), _ptr(final_state), P, _ptr(workspace),
                                         0 if workspace is None else workspace.numel(), B, T, H, Dk, D, code,
                                         _stream(dev, stream)))
    return o, final_state


def raw_chunk_fwd(q, k, v, a, beta, initial_state, o, final_state, B, T, H, Dk, Dv, dtype, stream=0):
    """Direct call of the C entry point with raw integer pointers; returns
    the status code without raising (used by the error-path tests)."""
    return lib().kda_chunk_fwd(q, k, v, a, beta, initial_state, o, final_state, B, T, H, Dk, Dv, dtype, stream)


def raw_chunk_fwd_states(q, k, v, a, beta, initial_state, o, final_state, states, state_every, B, T, H, Dk, Dv, dtype,
                         stream=0):
    return lib().kda_chunk_fwd_states(q, k, v, a, beta, initial_state, o, final_state, states, state_every, B, T, H,
                                      Dk, Dv, dtype, stream)


def raw_chunk_fwd_varlen(q, k, v, a, beta, cu_seqlens, initial_state, o, final_state, N, T, H, Dk, Dv, dtype,
                         stream=0):
    return lib().kda_chunk_fwd_varlen(q, k, v, a, beta, cu_seqlens, initial_state, o, final_state, N, T, H, Dk, Dv,
                                      dtype, stream)


def raw_decode_step(q, k, v, a, beta, state, o, B, H, Dk, Dv, dtype, stream=0):
    return lib().kda_decode_step(q, k, v, a, beta, state, o, B, H, Dk, Dv, dtype, stream)


def raw_decode_multi(q, k, v, a, beta, state, o, n_commit, B, K, H, Dk, Dv, dtype, stream=0):
    return lib().kda_decode_multi(q, k, v, a, beta, state, o, n_commit, B, K, H, Dk, Dv, dtype, stream)


def raw_output_gate_norm(o, z, y, rows, Dv, eps, dtype, stream=0):
    return lib().kda_output_gate_norm(o, z, y, rows, Dv, eps, dtype, stream)


def raw_chunk_fwd_gated(q, k, v, a, beta, initial_state, o, final_state, B, T, H, Dk, Dv, dtype, gate, stream=0):
    return lib().kda_chunk_fwd_gated(q, k, v, a, beta, initial_state, o, final_state, B, T, H, Dk, Dv, dtype, gate,
                                     stream)


def raw_chunk_fwd_norm(q, k, v, a, beta, initial_state, z, eps, y, final_state, B, T, H, Dk, Dv, dtype, stream=0):
    return lib().kda_chunk_fwd_norm(q, k, v, a, beta, initial_state, z, eps, y, final_state, B, T, H, Dk, Dv, dtype,
                                    stream)


def raw_chunk_fwd_split(q, k, v, a, beta, initial_state, o, final_state, segments, workspace, workspace_bytes, B, T,
                        H, Dk, Dv, dtype, stream=0):
    return lib().kda_chunk_fwd_split(q, k, v, a, beta, initial_state, o, final_state, segments, workspace,
                                     workspace_bytes, B, T, H, Dk, Dv, dtype, stream)


def raw_chunk_fwd_split_noalloc(q, k, v, a, beta, initial_state, o, final_state, segments, B, T, H, Dk, Dv, dtype,
                                stream=0):
    return lib().kda_chunk_fwd_split_noalloc(q, k, v, a, beta, initial_state, o, final_state, segments, B, T, H, Dk,
                                             Dv, dtype, stream)


def raw_decode_step_gated(q, k, v, a, beta, state, o, B, H, Dk, Dv, dtype, gate, stream=0):
    return lib().kda_decode_step_gated(q, k, v, a, beta, state, o, B, H, Dk, Dv, dtype, gate, stream)


def raw_decode_multi_gated(q, k, v, a, beta, state, o, n_commit, B, K, H, Dk, Dv, dtype, gate, stream=0):
    return lib().kda_decode_multi_gated(q, k, v, a, beta, state, o, n_commit, B, K, H, Dk, Dv, dtype, gate, stream)


def last_error():
    return lib().kda_last_error().decode()
