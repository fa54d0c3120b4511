"""The measured-peak micro-benchmarks that bench.py reports fractions against
(peaks/): the library loads and rejects bad arguments without a GPU; on a GPU
each loop runs and returns rates of the right order."""
import os

import pytest

import peaks

HIP_ERROR_INVALID_VALUE = 1


@pytest.fixture(scope="module")
def plib():
    if not os.path.exists(peaks.LIB):
        pytest.fail("libpeaks.so is not built (run __graft_entry__.build())")
    return peaks._load()


def test_exports(plib):
    for name in ("peaks_copy", "peaks_read", "peaks_mfma", "peaks_valu"):
        assert hasattr(plib, name), name


def test_bad_arguments_are_rejected_before_any_launch(plib):
    # fake, never-dereferenced addresses: every call fails its checks first
    assert plib.peaks_copy(0x10000, 0x10000, 17, 4, None) == HIP_ERROR_INVALID_VALUE  # not a multiple of 16 bytes
    assert plib.peaks_copy(0x10008, 0x10000, 16, 4, None) == HIP_ERROR_INVALID_VALUE  # misaligned source
    assert plib.peaks_read(0x10000, 0x10000, 16, 0, None) == HIP_ERROR_INVALID_VALUE  # no workgroups
    assert plib.peaks_mfma(0x10000, 4, 0, 1, None) == HIP_ERROR_INVALID_VALUE  # no iterations
    assert plib.peaks_valu(0x10000, 4, 16, 3, None) == HIP_ERROR_INVALID_VALUE  # no such instruction
    assert plib.peaks_valu(0x10000, 0, 16, 0, None) == HIP_ERROR_INVALID_VALUE


@pytest.mark.gpu
def test_rates_on_the_device():
    v = peaks.valu_ns_per_instruction(iters=1024, reps=2)
    assert all(x > 0 for x in v.values())
    # a transcendental holds the VALU longer than a multiply
    assert v["v_exp_f32"] > 1.5 * v["v_mul_f32"] and v["v_rcp_f32"] > 1.5 * v["v_mul_f32"]
    bf16_32 = peaks.mfma(bf16=True, shape32=True, iters=1024, reps=2)
    bf16_16 = peaks.mfma(bf16=True, iters=1024, reps=2)
    assert 5e14 < bf16_16 < bf16_32 < 3e15  # flop/s, against the 2.5 PFLOP/s spec
    read = peaks.hbm_read(nbytes=1 << 28, reps=2)
    assert 1e12 < read < 9e12  # bytes/s, against the 8 TB/s spec
