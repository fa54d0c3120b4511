"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_23_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        pytest.fail("libkda.so is not built (run __graft_entry__.build())")
    return kda.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("kda_chunk_fwd", "kda_chunk_fwd_states", "kda_chunk_fwd_varlen", "kda_decode_step", "kda_decode_multi",
              "kda_output_gate_norm", "kda_compose_segments", "kda_status_string", "kda_last_error", "kda_version",
              "kda_chunk_fwd_gated", "kda_chunk_fwd_norm", "kda_chunk_fwd_split", "kda_chunk_fwd_split_workspace",
              "kda_decode_step_gated", "kda_decode_multi_gated"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(1) == b"KDA_ERR_INVALID_ARGUMENT"
    assert lib.kda_status_string(2) == b"KDA_ERR_UNSUPPORTED"
    assert lib.kda_status_string(3) == b"KDA_ERR_HIP"
    assert lib.kda_version() >= 100


# Fake, never-dereferenced device addresses: every case below fails validation
# before anything is launched, so no GPU is touched.
P = 0x10000
MIS = 0x10008


def chunk(**kw):
    args = dict(q=P, k=P, v=P, a=P, beta=P, initial_state=None, o=P, final_state=P, B=1, T=16, H=1, Dk=128, Dv=128,
                dtype=kda.KDA_BF16)
    args.update(kw)
    return kda.raw_chunk_fwd(*args.values())


def decode(**kw):
    args = dict(q=P, k=P, v=P, a=P, beta=P, state=P, o=P, B=1, H=1, Dk=128, Dv=128, dtype=kda.KDA_BF16)
    args.update(kw)
    return kda.raw_decode_step(*args.values())


def chunk_states(**kw):
    args = dict(q=P, k=P, v=P, a=P, beta=P, initial_state=None, o=P, final_state=P, states=P, state_every=32, B=1,
                T=64, H=1, Dk=128, Dv=128, dtype=kda.KDA_BF16)
    args.update(kw)
    return kda.raw_chunk_fwd_states(*args.values())


@pytest.mark.parametrize("every", [0, -16, 8, 24, 100])
def test_checkpoint_interval_must_be_a_positive_multiple_of_16(lib, every):
    assert chunk_states(state_every=every) == kda.KDA_ERR_INVALID_ARGUMENT
    assert "state_every" in kda.last_error()


def test_checkpoint_buffer_checks(lib):
    assert chunk_states(states=None) == kda.KDA_ERR_INVALID_ARGUMENT  # T / every = 2 checkpoints to write
    assert "states" in kda.last_error()
    assert chunk_states(states=MIS) == kda.KDA_ERR_INVALID_ARGUMENT
    assert "aligned" in kda.last_error()
    # the checks shared with kda_chunk_fwd run first
    assert chunk_states(q=None) == kda.KDA_ERR_INVALID_ARGUMENT and "q is NULL" in kda.last_error()
    assert chunk_states(Dk=64) == kda.KDA_ERR_UNSUPPORTED
    assert kda.raw_chunk_fwd_states(None, None, None, None, None, None, None, None, None, 16, 0, 16, 4, 128, 128,
                                    0) == kda.KDA_OK


def varlen(**kw):
    args = dict(q=P, k=P, v=P, a=P, beta=P, cu_seqlens=P, initial_state=None, o=P, final_state=P, N=2, T=64, H=1,
                Dk=128, Dv=128, dtype=kda.KDA_BF16)
    args.update(kw)
    return kda.raw_chunk_fwd_varlen(*args.values())


def test_varlen_argument_checks(lib):
    assert varlen(cu_seqlens=None) == kda.KDA_ERR_INVALID_ARGUMENT and "cu_seqlens" in kda.last_error()
    assert varlen(cu_seqlens=P + 2) == kda.KDA_ERR_INVALID_ARGUMENT and "aligned" in kda.last_error()
    assert varlen(q=None) == kda.KDA_ERR_INVALID_ARGUMENT and "q is NULL" in kda.last_error()
    assert varlen(N=-1) == kda.KDA_ERR_INVALID_ARGUMENT
    assert varlen(T=-1) == kda.KDA_ERR_INVALID_ARGUMENT
    assert varlen(Dk=64) == kda.KDA_ERR_UNSUPPORTED
    assert varlen(H=65537) == kda.KDA_ERR_UNSUPPORTED
    assert varlen(N=1 << 21, H=1 << 10) == kda.KDA_ERR_INVALID_ARGUMENT  # N*H above the sequence limit
    assert kda.raw_chunk_fwd_varlen(None, None, None, None, None, P, None, None, None, 0, 0, 4, 128, 128,
                                    0) == kda.KDA_OK


def test_output_gate_norm_argument_checks(lib):
    def call(**kw):
        args = dict(o=P, z=P, y=P, rows=8, Dv=128, eps=1e-6, dtype=kda.KDA_BF16)
        args.update(kw)
        return kda.raw_output_gate_norm(*args.values())

    for field in ("o", "z", "y"):
        assert call(**{field: None}) == kda.KDA_ERR_INVALID_ARGUMENT and field in kda.last_error()
        assert call(**{field: MIS}) == kda.KDA_ERR_INVALID_ARGUMENT and "aligned" in kda.last_error()
    assert call(rows=-1) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(Dv=64) == kda.KDA_ERR_UNSUPPORTED
    assert call(eps=-1.0) == kda.KDA_ERR_INVALID_ARGUMENT and "eps" in kda.last_error()
    assert call(eps=float("nan")) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(dtype=5) == kda.KDA_ERR_INVALID_ARGUMENT
    assert kda.raw_output_gate_norm(None, None, None, 0, 128, 1e-6, 0) == kda.KDA_OK


def test_compose_argument_checks(lib):
    def call(**kw):
        args = dict(M=P, E=P, S0=None, S_in=P, B=1, Pn=3, H=2, Dk=128, Dv=128)
        args.update(kw)
        return lib.kda_compose_segments(*args.values(), None)

    lib.kda_compose_segments.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    for field in ("M", "E", "S_in"):
        assert call(**{field: None}) == kda.KDA_ERR_INVALID_ARGUMENT and field in kda.last_error()
    assert call(S0=MIS) == kda.KDA_ERR_INVALID_ARGUMENT and "aligned" in kda.last_error()
    assert call(Pn=-1) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(Dk=64) == kda.KDA_ERR_UNSUPPORTED
    assert call(B=1 << 16, H=1 << 10, Pn=1 << 10) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(M=None, E=None, S_in=None, B=0) == kda.KDA_OK


def multi(**kw):
    args = dict(q=P, k=P, v=P, a=P, beta=P, state=P, o=P, n_commit=None, B=1, K=4, H=1, Dk=128, Dv=128,
                dtype=kda.KDA_BF16)
    args.update(kw)
    return kda.raw_decode_multi(*args.values())


@pytest.mark.parametrize("field", ["q", "k", "v", "a", "beta", "o", "final_state"])
def test_chunk_rejects_null_pointers(lib, field):
    assert chunk(**{field: None}) == kda.KDA_ERR_INVALID_ARGUMENT
    assert field.split("_")[0] in kda.last_error()


@pytest.mark.parametrize("field", ["q", "k", "v", "a", "beta", "o", "final_state", "initial_state"])
def test_chunk_rejects_misaligned_pointers(lib, field):
    assert chunk(**{field: MIS}) == kda.KDA_ERR_INVALID_ARGUMENT
    assert "aligned" in kda.last_error()


@pytest.mark.parametrize("field", ["q", "k", "v", "a", "beta", "state", "o"])
def test_decode_rejects_null_and_misaligned(lib, field):
    assert decode(**{field: None}) == kda.KDA_ERR_INVALID_ARGUMENT
    assert decode(**{field: MIS}) == kda.KDA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("field", ["q", "k", "v", "a", "beta", "state", "o"])
def test_multi_rejects_null_and_misaligned(lib, field):
    assert multi(**{field: None}) == kda.KDA_ERR_INVALID_ARGUMENT
    assert field in kda.last_error()
    assert multi(**{field: MIS}) == kda.KDA_ERR_INVALID_ARGUMENT
    assert "aligned" in kda.last_error()


def test_multi_commit_counts_need_only_int_alignment(lib):
    # n_commit is an int32 array: 4-byte alignment is enough, less is rejected
    assert multi(n_commit=P + 2, K=1) == kda.KDA_ERR_INVALID_ARGUMENT
    assert "n_commit" in kda.last_error()


@pytest.mark.parametrize("kw", [dict(B=-1), dict(K=-1), dict(H=-2), dict(Dk=0), dict(dtype=7)])
def test_multi_rejects_bad_sizes_and_enums(lib, kw):
    assert multi(**kw) == kda.KDA_ERR_INVALID_ARGUMENT


def test_multi_limits_and_no_ops(lib):
    assert multi(Dv=64) == kda.KDA_ERR_UNSUPPORTED
    assert multi(B=(1 << 31) - (1 << 20) + 1, H=1) == kda.KDA_ERR_INVALID_ARGUMENT
    assert multi(K=1 << 12, H=1 << 10) == kda.KDA_ERR_UNSUPPORTED  # a sequence's K rows span 2^31 bytes
    assert "K*H" in kda.last_error()
    assert multi(B=1 << 20, K=1 << 30, H=1 << 10) == kda.KDA_ERR_INVALID_ARGUMENT  # B*K*H*128 > 2^62
    assert "overflow" in kda.last_error()
    # nothing to do: no tokens, or no sequences; NULL pointers allowed
    assert kda.raw_decode_multi(None, None, None, None, None, None, None, None, 2, 0, 4, 128, 128, 1) == kda.KDA_OK
    assert kda.raw_decode_multi(None, None, None, None, None, None, None, None, 0, 4, 4, 128, 128, 0) == kda.KDA_OK


@pytest.mark.parametrize("kw", [dict(B=-1), dict(T=-1), dict(H=-2), dict(Dk=0), dict(Dv=-128), dict(dtype=7)])
def test_chunk_rejects_bad_sizes_and_enums(lib, kw):
    assert chunk(**kw) == kda.KDA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(Dk=64), dict(Dv=256), dict(Dk=96, Dv=96)])
def test_unsupported_head_sizes(lib, kw):
    assert chunk(**kw) == kda.KDA_ERR_UNSUPPORTED
    assert decode(**kw) == kda.KDA_ERR_UNSUPPORTED
    assert "128" in kda.last_error()


def test_prefill_head_limit(lib):
    # a chunk of one tensor must stay under 2^31 bytes for 32-bit buffer offsets
    assert chunk(H=65537) == kda.KDA_ERR_UNSUPPORTED
    assert "65536" in kda.last_error()


def test_size_overflow_is_rejected(lib):
    assert chunk(B=1 << 20, T=1 << 30, H=1 << 10) == kda.KDA_ERR_INVALID_ARGUMENT
    assert decode(B=1 << 20, H=1 << 20) == kda.KDA_ERR_INVALID_ARGUMENT
    # B * H keeps 2^20 of headroom below 2^31 (unit index plus one grid stride)
    assert decode(B=(1 << 31) - (1 << 20) + 1, H=1) == kda.KDA_ERR_INVALID_ARGUMENT
    assert "limit" in kda.last_error()


def test_empty_batch_is_a_no_op(lib):
    # B * H == 0: nothing to do, nothing launched, NULL pointers allowed
    assert kda.raw_chunk_fwd(None, None, None, None, None, None, None, None, 0, 16, 4, 128, 128, 0) == kda.KDA_OK
    assert kda.raw_decode_step(None, None, None, None, None, None, None, 3, 0, 128, 128, 1) == kda.KDA_OK


def test_last_error_is_per_thread(lib):
    import threading

    assert chunk(Dk=64) == kda.KDA_ERR_UNSUPPORTED
    seen = {}

    def other():
        seen["msg"] = kda.last_error()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "128" in kda.last_error()


# --------------------------------------------------------------------------- Python binding checks (no launch)


def _decode_args(torch, dtype):
    B, H, D = 2, 3, 128
    return dict(q=torch.zeros(B, H, D, dtype=dtype), k=torch.zeros(B, H, D, dtype=dtype),
                v=torch.zeros(B, H, D, dtype=dtype), a=torch.zeros(B, H, D, dtype=dtype),
                beta=torch.zeros(B, H), state=torch.zeros(B, H, D, D))


def _chunk_args(torch, dtype):
    B, T, H, D = 1, 5, 2, 128
    return dict(q=torch.zeros(B, T, H, D, dtype=dtype), k=torch.zeros(B, T, H, D, dtype=dtype),
                v=torch.zeros(B, T, H, D, dtype=dtype), a=torch.zeros(B, T, H, D, dtype=dtype),
                beta=torch.zeros(B, T, H))


def _multi_args(torch, dtype):
    B, K, H, D = 2, 3, 2, 128
    return dict(q=torch.zeros(B, K, H, D, dtype=dtype), k=torch.zeros(B, K, H, D, dtype=dtype),
                v=torch.zeros(B, K, H, D, dtype=dtype), a=torch.zeros(B, K, H, D, dtype=dtype),
                beta=torch.zeros(B, K, H), state=torch.zeros(B, H, D, D))


@pytest.mark.parametrize("entry", ["decode", "chunk", "multi", "states", "varlen"])
def test_binding_rejects_host_tensors_before_any_call(lib, entry):
    """Host (CPU) tensors never reach the C ABI: their addresses are not
    device pointers.  Every tensor argument is checked, q included."""
    torch = pytest.importorskip("torch")
    args = {"decode": _decode_args, "chunk": _chunk_args, "multi": _multi_args, "states": _chunk_args,
            "varlen": _chunk_args}[entry](torch, torch.float32)
    if entry == "states":
        args["state_every"] = 16
    if entry == "varlen":
        args = {n: t[0] for n, t in args.items()}
        args["cu_seqlens"] = torch.tensor([0, 5], dtype=torch.int32)
    fn = {"decode": kda.kda_decode_step, "chunk": kda.kda_chunk_fwd, "multi": kda.kda_decode_multi,
          "states": kda.kda_chunk_fwd_states, "varlen": kda.kda_chunk_fwd_varlen}[entry]
    with pytest.raises(ValueError, match="q must be a GPU tensor"):
        fn(**args)


def test_binding_rejects_wrong_shapes_and_dtypes(lib):
    torch = pytest.importorskip("torch")
    args = _decode_args(torch, torch.float32)
    args["q"] = torch.zeros(2, 3, 64)
    with pytest.raises(ValueError):
        kda.kda_decode_step(**args)
    args = _decode_args(torch, torch.float16)
    with pytest.raises(TypeError, match="bfloat16 or float32"):
        kda.kda_decode_step(**args)


def test_binding_raises_without_the_library(monkeypatch):
    """No CPU fallback: with the shared library absent every call fails loudly."""
    monkeypatch.setattr(kda, "_lib", None)
    monkeypatch.setattr(kda, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libkda.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        kda.lib()
    with pytest.raises(RuntimeError, match="no fallback"):
        kda.last_error()


# --------------------------------------------------------------------------- gate modes, fused norm, split


def gated(**kw):
    args = dict(q=P, k=P, v=P, a=P, beta=P, initial_state=None, o=P, final_state=P, B=1, T=16, H=1, Dk=128, Dv=128,
                dtype=kda.KDA_BF16, gate=kda.KDA_GATE_CHANNEL)
    args.update(kw)
    return kda.raw_chunk_fwd_gated(*args.values())


def test_gate_argument_checks(lib):
    assert gated(gate=3) == kda.KDA_ERR_INVALID_ARGUMENT and "gate" in kda.last_error()
    assert gated(gate=-1) == kda.KDA_ERR_INVALID_ARGUMENT
    # channel logits are rows like q: 16-byte aligned; the scalar logits are fp32 like beta: 4-byte aligned
    assert gated(a=MIS) == kda.KDA_ERR_INVALID_ARGUMENT and "aligned" in kda.last_error()
    assert gated(a=None) == kda.KDA_ERR_INVALID_ARGUMENT and "a is NULL" in kda.last_error()
    assert gated(a=None, gate=kda.KDA_GATE_SCALAR) == kda.KDA_ERR_INVALID_ARGUMENT
    assert gated(a=P + 2, gate=kda.KDA_GATE_SCALAR) == kda.KDA_ERR_INVALID_ARGUMENT
    assert gated(q=None, gate=kda.KDA_GATE_NONE) == kda.KDA_ERR_INVALID_ARGUMENT  # the other checks still run
    assert gated(Dk=64, gate=kda.KDA_GATE_NONE) == kda.KDA_ERR_UNSUPPORTED
    for entry, args in ((kda.raw_decode_step_gated, (P, P, P, P, P, P, P, 1, 1, 128, 128, kda.KDA_BF16, 7)),
                        (kda.raw_decode_multi_gated, (P, P, P, P, P, P, P, None, 1, 2, 1, 128, 128, kda.KDA_BF16, 7))):
        assert entry(*args) == kda.KDA_ERR_INVALID_ARGUMENT and "gate" in kda.last_error()
    assert kda.raw_decode_step_gated(P, P, P, None, P, P, P, 1, 1, 128, 128, kda.KDA_BF16,
                                     kda.KDA_GATE_SCALAR) == kda.KDA_ERR_INVALID_ARGUMENT
    assert kda.raw_decode_multi_gated(P, P, P, P + 4, P, P, P, None, 1, 2, 1, 128, 128, kda.KDA_BF16,
                                      kda.KDA_GATE_CHANNEL) == kda.KDA_ERR_INVALID_ARGUMENT


def test_fused_norm_argument_checks(lib):
    def call(**kw):
        args = dict(q=P, k=P, v=P, a=P, beta=P, initial_state=None, z=P, eps=1e-6, y=P, final_state=P, B=1, T=16,
                    H=1, Dk=128, Dv=128, dtype=kda.KDA_BF16)
        args.update(kw)
        return kda.raw_chunk_fwd_norm(*args.values())

    assert call(z=None) == kda.KDA_ERR_INVALID_ARGUMENT and "z" in kda.last_error()
    assert call(z=MIS) == kda.KDA_ERR_INVALID_ARGUMENT and "aligned" in kda.last_error()
    assert call(y=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(eps=-1.0) == kda.KDA_ERR_INVALID_ARGUMENT and "eps" in kda.last_error()
    assert call(eps=float("inf")) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(Dv=64) == kda.KDA_ERR_UNSUPPORTED


def split(**kw):
    args = dict(q=P, k=P, v=P, a=P, beta=P, initial_state=None, o=P, final_state=P, segments=4, workspace=P,
                workspace_bytes=1 << 40, B=1, T=4096, H=2, Dk=128, Dv=128, dtype=kda.KDA_BF16)
    args.update(kw)
    return kda.raw_chunk_fwd_split(*args.values())


def test_split_workspace_size(lib):
    state = 128 * 128 * 4
    # 4096 tokens in 4 segments of 1024: 3 transitions, 3 fragments and 4 entering states per (b, h)
    assert kda.kda_chunk_fwd_split_workspace(1, 4096, 2, 4) == 2 * state * (3 + 3 + 4)
    # 4100 tokens in 16 segments: segments of 272 tokens (whole chunks), 16 of them (the last one 20 tokens)
    assert kda.kda_chunk_fwd_split_workspace(2, 4100, 9, 16) == 2 * 9 * state * (15 + 15 + 16)
    # segments of whole chunks: 100 tokens in 8 segments are 7 segments of 16
    assert kda.kda_chunk_fwd_split_workspace(1, 100, 1, 8) == state * (6 + 6 + 7)
    for args in ((1, 4096, 2, 1), (1, 16, 2, 8), (0, 4096, 2, 4), (1, 0, 2, 4), (1, 4096, 0, 4)):
        assert kda.kda_chunk_fwd_split_workspace(*args) == 0, args


def test_split_argument_checks(lib):
    need = kda.kda_chunk_fwd_split_workspace(1, 4096, 2, 4)
    assert split(workspace_bytes=need - 1) == kda.KDA_ERR_INVALID_ARGUMENT and "workspace" in kda.last_error()
    assert split(workspace=None) == kda.KDA_ERR_INVALID_ARGUMENT and "workspace" in kda.last_error()
    assert split(workspace=MIS) == kda.KDA_ERR_INVALID_ARGUMENT and "aligned" in kda.last_error()
    assert split(segments=0) == kda.KDA_ERR_INVALID_ARGUMENT and "segments" in kda.last_error()
    for field in ("q", "k", "v", "a", "beta", "o", "final_state"):
        assert split(**{field: None}) == kda.KDA_ERR_INVALID_ARGUMENT, field
        assert split(**{field: MIS}) == kda.KDA_ERR_INVALID_ARGUMENT, field
    assert split(initial_state=MIS) == kda.KDA_ERR_INVALID_ARGUMENT
    assert split(Dk=64) == kda.KDA_ERR_UNSUPPORTED
    assert split(H=65537) == kda.KDA_ERR_UNSUPPORTED
    assert split(T=-1) == kda.KDA_ERR_INVALID_ARGUMENT
    assert split(B=1 << 20, H=1 << 8, segments=16) == kda.KDA_ERR_INVALID_ARGUMENT  # B*H*segments over the limit
    assert split(dtype=9) == kda.KDA_ERR_INVALID_ARGUMENT
    # one segment (or a short sequence) is the plain prefill and needs no workspace: checks only, B = 0 is a no-op
    assert split(segments=1, workspace=None, workspace_bytes=0, q=None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert split(B=0, workspace=None, workspace_bytes=0) == kda.KDA_OK


def _relaxed_require(t, name, shape, dtype, device):
    """The binding's argument check without the device test, so that the
    order of its checks can be seen with host tensors."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def test_split_binding_checks_outputs_before_any_call(lib, monkeypatch):
    """A non-contiguous o or a final_state of the wrong dtype is rejected by
    the split binding itself (a reshape would have written into a copy)."""
    torch = pytest.importorskip("torch")
    monkeypatch.setattr(kda, "_require", _relaxed_require)
    calls = []
    monkeypatch.setattr(kda, "_check", lambda status: calls.append(status))
    B, T, H, D = 1, 64, 2, 128
    x = {n: torch.zeros(B, T, H, D, dtype=torch.bfloat16) for n in ("q", "k", "v", "a")}
    beta = torch.zeros(B, T, H)
    o_t = torch.zeros(B, H, T, D, dtype=torch.bfloat16).transpose(1, 2)  # [B, T, H, D] view, not contiguous
    with pytest.raises(ValueError, match="o must be contiguous"):
        kda.kda_chunk_fwd_split(x["q"], x["k"], x["v"], x["a"], beta, 2, o=o_t)
    with pytest.raises(TypeError, match="final_state"):
        kda.kda_chunk_fwd_split(x["q"], x["k"], x["v"], x["a"], beta, 2,
                                final_state=torch.zeros(B, H, D, D, dtype=torch.float64))
    with pytest.raises(ValueError, match="initial_state"):
        kda.kda_chunk_fwd_split(x["q"], x["k"], x["v"], x["a"], beta, 2, initial_state=torch.zeros(B, H, D, 64))
    with pytest.raises(ValueError, match="workspace holds"):
        kda.kda_chunk_fwd_split(x["q"], x["k"], x["v"], x["a"], beta, 2, workspace=torch.zeros(16, dtype=torch.uint8))
    assert calls == []  # nothing reached the library


def test_noalloc_split_checks(lib):
    """The no-allocation split checks its arguments and its scratch limit
    (64 MiB) before it touches the device."""
    def call(**kw):
        args = dict(q=P, k=P, v=P, a=P, beta=P, initial_state=None, o=P, final_state=P, segments=16, B=1, T=8192,
                    H=8, Dk=128, Dv=128, dtype=kda.KDA_BF16)
        args.update(kw)
        return kda.raw_chunk_fwd_split_noalloc(*args.values())

    assert call(H=96) == kda.KDA_ERR_INVALID_ARGUMENT and "scratch" in kda.last_error()  # 276 MiB needed
    assert call(segments=0) == kda.KDA_ERR_INVALID_ARGUMENT and "segments" in kda.last_error()
    assert call(Dk=64) == kda.KDA_ERR_UNSUPPORTED
    assert call(T=-1) == kda.KDA_ERR_INVALID_ARGUMENT
    assert call(B=0) == kda.KDA_OK
