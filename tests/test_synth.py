"""The seeded input generator (CPU side): known answers, accuracy of its own
series, distributions, determinism."""
import math

import numpy as np

import synth
from synth import workloads


def test_philox_known_answers():
    # Known-answer vectors of Philox4x32-10 (Salmon et al., SC'11 reference implementation)
    assert synth.philox((0, 0, 0, 0), (0, 0)) == (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)
    assert synth.philox((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2) == (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)
    assert synth.philox((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0)) == (
        0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)


def test_series_accuracy():
    import ctypes

    lib = synth._host_lib()
    for x in np.geomspace(2.0 ** -33, 1.0, 2000):
        assert abs(lib.synth_ln_host(x) - math.log(x)) <= 4e-16 * max(1.0, abs(math.log(x)))
    s, c = ctypes.c_double(), ctypes.c_double()
    for u in np.linspace(0.0, 1.0, 4001)[:-1]:
        lib.synth_sincos_2pi_host(u, ctypes.byref(s), ctypes.byref(c))
        assert abs(s.value - math.sin(2 * math.pi * u)) < 2e-15
        assert abs(c.value - math.cos(2 * math.pi * u)) < 2e-15
    for x in np.linspace(-30.0, 30.0, 601):
        assert abs(lib.synth_exp_host(x) / math.exp(x) - 1.0) < 4e-15


def test_distributions():
    w = workloads.WORKLOADS[1]
    x = workloads.host_inputs(w, nt=256, nh=8, dtype="f64")
    for name in ("q", "k"):
        n = np.linalg.norm(x[name], axis=-1)
        assert np.allclose(n, 1.0, atol=1e-14)
    v = x["v"].ravel()
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01
    a = x["a"].ravel()
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1.0) < 0.01
    b = x["beta"].ravel()
    assert 0.0 < b.min() and b.max() < 1.0 and abs(b.mean() - 0.5) < 0.01
    w3 = workloads.WORKLOADS[3]
    a3 = workloads.host_inputs(w3, nt=64, nh=4, dtype="f64")["a"]
    assert abs(a3[..., :64].mean() - 3.0) < 0.02 and abs(a3[..., 64:].mean() + 3.0) < 0.02
    s0 = workloads.host_inputs(workloads.WORKLOADS[2], nb=1, nt=1, nh=2, dtype="f64")["s0"]
    assert abs(s0.std() - 0.02) < 0.001


def test_rounding_and_thread_independence():
    w = workloads.WORKLOADS[1]
    x64 = workloads.host_inputs(w, nt=33, nh=5, t0=100, h0=7, dtype="f64", threads=1)
    xbf = workloads.host_inputs(w, nt=33, nh=5, t0=100, h0=7, threads=7)
    x32 = workloads.host_inputs(w, nt=33, nh=5, t0=100, h0=7, dtype="f32", threads=3)
    for name in ("q", "k", "v", "a"):
        f32 = x64[name].astype(np.float32)
        assert np.array_equal(x32[name], f32)
        bits = f32.view(np.uint32)
        rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
        assert np.array_equal(xbf[name], rne)
        assert np.allclose(synth.to_f64(xbf[name]), x64[name], rtol=2 ** -8, atol=0)


def test_blocks_are_consistent_with_the_whole():
    w = workloads.WORKLOADS[2]
    whole = workloads.host_inputs(w, nb=2, nt=40, nh=3)
    part = workloads.host_inputs(w, b0=1, nb=1, t0=10, nt=20, h0=1, nh=2)
    for name in ("q", "k", "v", "a"):
        assert np.array_equal(part[name], whole[name][1:2, 10:30, 1:3])
    assert np.array_equal(part["beta"], whole["beta"][1:2, 10:30, 1:3])
    assert np.array_equal(part["s0"], whole["s0"][1:2, 1:3])
    # different sequences of a batch draw different values
    assert not np.array_equal(whole["v"][0], whole["v"][1])
