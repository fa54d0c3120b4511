"""Every prefill mode in every launch layout, against the oracle.

A call runs each (sequence, head) unit as one, two or four workgroups,
chosen from how many units there are (both dtypes: four while 8 ceil(U / 8)
x 4 workgroups fit on the compute units, two while x 2 fit, else one per
unit; beyond one round, the rest of the last round as two or four).  Most
parity tests use few units, so they run the four-workgroup layout; the shapes
here put the same modes through each layout: 40 units (four workgroups),
13 (four, in a group of 8 units only partly filled), 100 (two), 356 (one
round of single workgroups, then two each for the other 100) and 286 (then
four each for the other 30).  T = 200 is 13 chunks, the last one ragged,
long enough for the loops without range tests.  Results are also compared
across the layouts: each unit's outputs do not depend on how many workgroups
serve it.

Reference: the page "Kimi K3：从三条信息流到完整系统", eq. (1) (the recurrence),
section "hybrid prefix cache" (checkpoints) and section "FlashKDA 与 KCP",
eq. (17) (the sequence split).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.conftest import gpu_available
from tests.gpu_common import TOL, WORKLOADS, device_inputs, host_inputs, print_case, to_np, variant

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

T = 200
# (B, H): 40 units, 13 (a group of 8 only partly filled), 100, 356, 286 (a rest of 30)
SHAPES = {"four": (2, 20), "four-ragged": (1, 13), "two": (4, 25), "one+two": (4, 89), "one+four": (2, 143)}


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


def worst(x, ref, axes):
    """Largest relative L2 over the blocks left after reducing `axes`."""
    num = np.sqrt(((x - ref) ** 2).sum(axis=axes))
    den = np.sqrt((ref ** 2).sum(axis=axes))
    return float((num / np.maximum(den, 1e-300)).max())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", list(SHAPES))
def test_modes_in_each_layout(kda, dtype, layout):
    """Plain prefill with S0, state checkpoints every 64 tokens, and the
    sequence split in two segments (its transition and fragment runs share a
    launch): every sequence's o, final state and checkpoints against the
    oracle, per sequence."""
    import torch

    B, H = SHAPES[layout]
    w = variant(WORKLOADS[2], index=400 + B * H, dtype=dtype, s0_scale=0.5)
    print_case(f"case layouts {dtype} {layout} B={B} H={H} T={T}")
    x = device_inputs(w, B=B, T=T, H=H)
    o, S = kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["a"], x["beta"], initial_state=x["s0"])
    oc, Sc, ck = kda.kda_chunk_fwd_states(x["q"], x["k"], x["v"], x["a"], x["beta"], 64, initial_state=x["s0"])
    osp, Ssp = kda.kda_chunk_fwd_split(x["q"], x["k"], x["v"], x["a"], x["beta"], 2, initial_state=x["s0"])
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(S, Sc), "checkpoints change o or the final state"
    h = host_inputs(w, nb=B, nt=T, nh=H)
    o_ref, S_ref, ck_ref = oracle.forward(synth.to_f64(h["q"]), synth.to_f64(h["k"]), synth.to_f64(h["v"]),
                                          h["beta"].astype(np.float64), a=synth.to_f64(h["a"]),
                                          s0=h["s0"].astype(np.float64), state_every=64)
    errs = {"o": worst(to_np(o), o_ref, (1, 3)), "S": worst(to_np(S), S_ref, (2, 3)),
            "checkpoints": worst(to_np(ck), ck_ref, (3, 4)),
            "split o": worst(to_np(osp), o_ref, (1, 3)), "split S": worst(to_np(Ssp), S_ref, (2, 3))}
    print_case("  worst per sequence: " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL[dtype], k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["scalar", "none"])
@pytest.mark.parametrize("layout", list(SHAPES))
def test_gate_modes_in_each_layout(kda, dtype, mode, layout):
    """The scalar gate (one fp32 logit per token and head) and no gate, in
    each layout, against the oracle's log-decay path with g given."""
    import torch

    B, H = SHAPES[layout]
    w = variant(WORKLOADS[2], index=450 + B * H, dtype=dtype)
    print_case(f"case layouts gate {mode} {dtype} {layout} B={B} H={H} T={T}")
    x = device_inputs(w, B=B, T=T, H=H)
    h = host_inputs(w, nb=B, nt=T, nh=H)
    if mode == "scalar":
        a_dev = x["a"][..., 0].float().contiguous()
        g = np.repeat(oracle.gate(synth.to_f64(h["a"])[..., :1]), 128, axis=3)
    else:
        a_dev = None
        g = np.zeros((B, T, H, 128))
    o, S = kda.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], a_dev, x["beta"], gate=mode, initial_state=x["s0"])
    torch.cuda.synchronize()
    s0 = h["s0"].astype(np.float64) if h["s0"] is not None else None
    o_ref, S_ref = oracle.forward(synth.to_f64(h["q"]), synth.to_f64(h["k"]), synth.to_f64(h["v"]),
                                  h["beta"].astype(np.float64), g=g, s0=s0)
    wo, ws = worst(to_np(o), o_ref, (1, 3)), worst(to_np(S), S_ref, (2, 3))
    print_case(f"  worst per sequence: o {wo:.3e}, S {ws:.3e}")
    assert wo <= TOL[dtype] and ws <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_layouts_agree_bit_for_bit(kda, dtype):
    """The first 40 units of the 356-unit call (single workgroups) equal the
    same 40 sequence-heads run alone (four workgroups each) and as part of a
    100-unit call (two each), bit for bit: the layouts only split the state's
    columns, whose updates are independent."""
    import torch

    B, H = 4, 89
    w = variant(WORKLOADS[2], index=480, dtype=dtype)
    x = device_inputs(w, B=B, T=T, H=H)
    print_case(f"case layouts bit-exact {dtype}")
    full_o, full_S = kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["a"], x["beta"])
    runs = {}
    for name, hh in (("four", 10), ("two", 25)):
        # B x hh units: the first hh heads of every sequence, contiguous copies
        sub = {k: x[k][:, :, :hh].contiguous() for k in ("q", "k", "v", "a", "beta")}
        runs[name] = kda.kda_chunk_fwd(sub["q"], sub["k"], sub["v"], sub["a"], sub["beta"])
    torch.cuda.synchronize()
    for name, (o, S) in runs.items():
        hh = o.shape[2]
        assert torch.equal(o, full_o[:, :, :hh]), name
        assert torch.equal(S, full_S[:, :hh]), name


# Lengths around the two-workgroup loop's boundaries: one partial chunk, one
# whole chunk, 3, 4 and 6 chunks (only the iterations with range tests, in
# which the chain waves also read each chunk's Gamma_C one iteration ahead),
# 11 chunks (the shortest with iterations without range tests), 12, and 14
# with a ragged last chunk.
PAIR_T = [1, 16, 33, 64, 96, 176, 192, 217]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_two_workgroup_layout_short_lengths(kda, dtype):
    """100 units (two workgroups each) at each length of PAIR_T, with S0, against the oracle per sequence."""
    import torch

    B, H = SHAPES["two"]
    for T_ in PAIR_T:
        w = variant(WORKLOADS[2], index=520 + T_, dtype=dtype, s0_scale=0.5)
        print_case(f"case two-workgroup layout {dtype} B={B} H={H} T={T_}")
        x = device_inputs(w, B=B, T=T_, H=H)
        o, S = kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["a"], x["beta"], initial_state=x["s0"])
        torch.cuda.synchronize()
        h = host_inputs(w, nb=B, nt=T_, nh=H)
        o_ref, S_ref = oracle.forward(synth.to_f64(h["q"]), synth.to_f64(h["k"]), synth.to_f64(h["v"]),
                                      h["beta"].astype(np.float64), a=synth.to_f64(h["a"]),
                                      s0=h["s0"].astype(np.float64))
        wo, ws = worst(to_np(o), o_ref, (1, 3)), worst(to_np(S), S_ref, (2, 3))
        print_case(f"  worst per sequence: o {wo:.3e}, S {ws:.3e}")
        assert wo <= TOL[dtype] and ws <= TOL[dtype], T_
