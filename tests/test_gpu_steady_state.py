"""GPU parity of every prefill and decode path at lengths where it runs its
steady-state loop, against the fp64 oracle.

The bf16 prefill pipelines a chunk through five iterations (gate, Gram,
solve, prep, chain) and runs iterations 5 .. nchunks - 4 without range tests,
in a separate copy of the loop per wave role when a sequence has two
workgroups: that loop starts only from 11 chunks (T >= 161).  Each case here
runs many iterations of it, in both launch layouts where the path has two
(a (sequence, head) count of at most 128 runs as workgroup pairs on a 256-CU
device; 291 = 3 x 97 runs 256 single workgroups and then 35 pairs), and
checks every sequence (or checkpoint) on its own.

The multi-token decode keeps the state scaled by the inverse of the running
decay product inside a group of eight tokens; with gates saturated at
a = +30 (g = -5) that product reaches e^-40, the edge of the range the
scaling relies on.  The decode cases drive it there."""
import numpy as np
import pytest

import oracle
import synth
from tests.conftest import gpu_available
from tests.gpu_common import TOL, WORKLOADS, device_inputs, host_inputs, print_case, rel_l2, to_np, variant

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_23_amd as kda_mod

    kda_mod.lib()
    return kda_mod


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    import gc

    import torch

    gc.collect()
    torch.cuda.empty_cache()


def per_block_worst(x, ref, axes):
    """Largest relative L2 over the blocks that remain after reducing `axes`
    (blocks whose reference is zero must be zero)."""
    num = np.sqrt(((x - ref) ** 2).sum(axis=axes))
    den = np.sqrt((ref ** 2).sum(axis=axes))
    zero = den == 0
    assert not np.any(num[zero]), "a block with a zero reference is not zero"
    return float((num[~zero] / den[~zero]).max()) if np.any(~zero) else 0.0


# --------------------------------------------------------------------------- state checkpoints


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout,every", [("pairs", 64), ("pairs", 512), ("mixed", 64), ("mixed", 512)])
def test_checkpoints_in_the_steady_loop(kda, dtype, layout, every):
    """Checkpoints every 64 or 512 tokens over 1,050 (pairs: 2 x 2
    sequences, 66 chunks, the last ragged) or 1,024 tokens (3 x 97 = 291
    sequences: single workgroups, then pairs in bf16, single workgroups in
    fp32).  Each checkpoint, each
    sequence's output and final state against the oracle; o and the final
    state equal kda_chunk_fwd's bit for bit."""
    import torch

    B, H, T = (2, 2, 1050) if layout == "pairs" else (3, 97, 1024)
    w = variant(WORKLOADS[2], index=200 + every + (layout == "mixed"), dtype=dtype)
    print_case(f"case checkpoints steady {dtype} {layout} B={B} T={T} H={H} every={every}")
    x = device_inputs(w, B=B, T=T, H=H)
    o, S, ck = kda.kda_chunk_fwd_states(x["q"], x["k"], x["v"], x["a"], x["beta"], every, initial_state=x["s0"])
    o1, S1 = kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["a"], x["beta"], initial_state=x["s0"])
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(S, S1)
    h = host_inputs(w, nb=B, nt=T, nh=H)
    o_ref, S_ref, ck_ref = oracle.forward(synth.to_f64(h["q"]), synth.to_f64(h["k"]), synth.to_f64(h["v"]),
                                          h["beta"].astype(np.float64), a=synth.to_f64(h["a"]),
                                          s0=h["s0"].astype(np.float64), state_every=every)
    worst_ck = per_block_worst(to_np(ck), ck_ref, (3, 4))
    worst_o = per_block_worst(to_np(o), o_ref, (1, 3))
    worst_s = per_block_worst(to_np(S), S_ref, (2, 3))
    print_case(f"  worst rel_l2: checkpoint {worst_ck:.3e}, o per sequence {worst_o:.3e}, S {worst_s:.3e}")
    assert max(worst_ck, worst_o, worst_s) <= TOL[dtype]


# --------------------------------------------------------------------------- packed sequences


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_varlen_long_sequences_single_workgroups(kda, dtype):
    """97 packed sequences of 300 .. 700 tokens x 3 heads = 291 (sequence,
    head) pairs: the single-workgroup layout (and pairs for the last 35)
    through its steady loop; every sequence against the oracle."""
    import torch

    w = variant(WORKLOADS[2], index=230, dtype=dtype)
    rng = np.random.default_rng(230)
    lengths = rng.integers(300, 701, size=97).tolist()
    H = 3
    T = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = len(lengths)
    print_case(f"case varlen long {dtype} N={N} T={T} H={H}")
    x = device_inputs(w, B=1, T=T, H=H)
    s0 = np.random.default_rng(231).standard_normal((N, H, 128, 128)).astype(np.float32) * 0.05
    o, S = kda.kda_chunk_fwd_varlen(x["q"][0], x["k"][0], x["v"][0], x["a"][0], x["beta"][0],
                                    torch.tensor(cu, device="cuda"), initial_state=torch.from_numpy(s0).cuda())
    torch.cuda.synchronize()
    h = host_inputs(w, nb=1, nt=T, nh=H)
    o_ref, S_ref = oracle.forward_varlen(synth.to_f64(h["q"][0]), synth.to_f64(h["k"][0]), synth.to_f64(h["v"][0]),
                                         h["beta"][0].astype(np.float64), cu, a=synth.to_f64(h["a"][0]),
                                         s0=s0.astype(np.float64))
    on, Sn = to_np(o), to_np(S)
    worst_o = max(per_block_worst(on[cu[n]:cu[n + 1]], o_ref[cu[n]:cu[n + 1]], (0, 2)) for n in range(N))
    worst_s = per_block_worst(Sn, S_ref, (2, 3))
    print_case(f"  worst per (sequence, head) rel_l2 o={worst_o:.3e} S={worst_s:.3e}")
    assert worst_o <= TOL[dtype] and worst_s <= TOL[dtype]


# --------------------------------------------------------------------------- decode at the range edge


def _saturated_inputs(seed, B, K, H):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, K, H, 128))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, K, H, 128))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, K, H, 128))
    a = np.where(rng.random((B, K, H, 128)) < 0.5, 30.0, -30.0)
    a[..., :32] = 30.0  # a quarter of the channels at g = -5 on every token
    beta = rng.random((B, K, H))
    s0 = rng.standard_normal((B, H, 128, 128)) * 0.5
    return dict(q=q, k=k, v=v, a=a, beta=beta, s0=s0)


def _upload(dtype, arrays):
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for name, val in arrays.items():
        t = torch.from_numpy(np.ascontiguousarray(val))
        out[name] = t.to("cuda", dtype=torch.float32 if name in ("beta", "s0") else tdt).contiguous()
    return out


def _as_device_sees(x):
    """Host copies of the uploaded values (after rounding to the I/O type)."""
    return {name: to_np(t) for name, t in x.items()}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_saturated_gates(kda, dtype):
    """Eight single-token steps and one eight-token kda_decode_multi call with
    gates at a = +-30 (a quarter of the channels at g = -5 throughout, so the
    multi-token kernel's decay product over its token group reaches e^-40),
    with commit counts 8, 0 and 5 for the multi-token call.  Against the
    oracle."""
    import torch

    B, K, H = 3, 8, 5
    x = _upload(dtype, _saturated_inputs(250, B, K, H))
    hx = _as_device_sees(x)
    print_case(f"case decode saturated gates {dtype} B={B} K={K} H={H}")
    state = x["s0"].clone()
    outs = [kda.kda_decode_step(*(x[n][:, t].contiguous() for n in ("q", "k", "v", "a", "beta")), state)
            for t in range(K)]
    counts = [K, 0, 5]
    state_m = x["s0"].clone()
    om = kda.kda_decode_multi(x["q"], x["k"], x["v"], x["a"], x["beta"], state_m,
                              n_commit=torch.tensor(counts, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(hx["q"], hx["k"], hx["v"], hx["beta"], a=hx["a"], s0=hx["s0"])
    om_ref, Sm_ref = oracle.decode_multi(hx["q"], hx["k"], hx["v"], hx["beta"], hx["s0"], a=hx["a"],
                                         n_commit=counts)
    e = [rel_l2(to_np(torch.stack(outs, dim=1)), o_ref), rel_l2(to_np(state), S_ref),
         rel_l2(to_np(om), om_ref), rel_l2(to_np(state_m), Sm_ref)]
    print_case("  rel_l2 decode o/S, multi o/S: " + " ".join(f"{v:.2e}" for v in e))
    assert max(e) <= TOL[dtype]
    assert torch.equal(state_m[1], x["s0"][1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_multi_saturated_two_groups(kda, dtype):
    """Sixteen tokens in one call (two full eight-token groups) with every
    channel at g = -5, so each group's decay product is exactly e^-40 on
    every channel; all committed, once with the counts given (the multi-token
    kernel) and once without (then the call runs as the chunkwise prefill)."""
    import torch

    B, K, H = 2, 16, 3
    arrays = _saturated_inputs(251, B, K, H)
    arrays["a"][:] = 30.0
    x = _upload(dtype, arrays)
    hx = _as_device_sees(x)
    o_ref, S_ref = oracle.forward(hx["q"], hx["k"], hx["v"], hx["beta"], a=hx["a"], s0=hx["s0"])
    for route, nc in (("multi-token kernel", torch.full((B,), K, dtype=torch.int32, device="cuda")),
                      ("prefill", None)):
        state = x["s0"].clone()
        o = kda.kda_decode_multi(x["q"], x["k"], x["v"], x["a"], x["beta"], state, n_commit=nc)
        torch.cuda.synchronize()
        eo, es = rel_l2(to_np(o), o_ref), rel_l2(to_np(state), S_ref)
        print_case(f"  decode multi all-saturated {dtype}, {route}: rel_l2 o={eo:.2e} S={es:.2e}")
        assert eo <= TOL[dtype] and es <= TOL[dtype], route
