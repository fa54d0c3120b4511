"""Seeded synthetic inputs for KDA workloads.

This module is shared test and benchmark infrastructure: the fp64 oracle and
the HIP library both consume what it draws, and it holds none of the KDA
method's arithmetic.  Values come from Philox4x32-10 + Box-Muller (see
``csrc/synth_core.h``); the host library and the device library produce
identical bits, so the oracle can regenerate on the host exactly the inputs a
device buffer holds.

Row tensors (q, k, v, gate logits a) are laid out ``[B, T, H, 128]``; beta is
``[B, T, H]`` fp32; initial states are ``[B, H, 128, 128]`` fp32.
"""
import ctypes
import os

import numpy as np

from .workloads import WORKLOADS, Workload, seed_for  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEVICE_LIB = os.path.join(_HERE, "libsynth_device.so")

Q, K, V, A, BETA, STATE = 0, 1, 2, 3, 4, 5
F32, BF16, F64 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "f64": F64}
_NP = {F32: np.float32, BF16: np.uint16, F64: np.float64}
D = 128


class RowRecipe(ctypes.Structure):
    _fields_ = [
        ("seed", ctypes.c_uint32),
        ("tensor", ctypes.c_int32),
        ("l2norm", ctypes.c_int32),
        ("split", ctypes.c_int32),
        ("mean_lo", ctypes.c_double),
        ("mean_hi", ctypes.c_double),
        ("scale", ctypes.c_double),
    ]


def row_recipe(seed, tensor, l2norm=False, mean=(0.0, 0.0), split=D, scale=1.0):
    return RowRecipe(seed & 0xFFFFFFFF, tensor, int(bool(l2norm)), split, float(mean[0]), float(mean[1]), float(scale))


_host = None
_device = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        i, u32, d, p = ctypes.c_int, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p
        lib.synth_rows_host.argtypes = [ctypes.POINTER(RowRecipe), i, i, i, i, i, i, i, p, i]
        lib.synth_beta_host.argtypes = [u32, i, i, i, i, i, i, i, p, i]
        lib.synth_state_host.argtypes = [u32, d, i, i, i, i, i, p, i]
        lib.synth_philox_host.argtypes = [ctypes.POINTER(ctypes.c_uint32 * 4), ctypes.POINTER(ctypes.c_uint32 * 2),
                                          ctypes.POINTER(ctypes.c_uint32 * 4)]
        lib.synth_ln_host.argtypes = [d]
        lib.synth_ln_host.restype = d
        lib.synth_exp_host.argtypes = [d]
        lib.synth_exp_host.restype = d
        lib.synth_sincos_2pi_host.argtypes = [d, ctypes.POINTER(d), ctypes.POINTER(d)]
        for f in (lib.synth_rows_host, lib.synth_beta_host, lib.synth_state_host):
            f.restype = i
        _host = lib
    return _host


def _device_lib():
    global _device
    if _device is None:
        if not os.path.exists(DEVICE_LIB):
            raise RuntimeError(f"{DEVICE_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEVICE_LIB)
        i, u32, d, p = ctypes.c_int, ctypes.c_uint32, ctypes.c_double, ctypes.c_void_p
        lib.synth_rows_device.argtypes = [ctypes.POINTER(RowRecipe), i, i, i, i, i, i, i, p, p]
        lib.synth_beta_device.argtypes = [u32, i, i, i, i, i, i, i, p, p]
        lib.synth_state_device.argtypes = [u32, d, i, i, i, i, i, p, p]
        for f in (lib.synth_rows_device, lib.synth_beta_device, lib.synth_state_device):
            f.restype = i
        _device = lib
    return _device


def _threads(n):
    if n is not None:
        return int(n)
    return max(1, min(16, os.cpu_count() or 1))


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


# ----------------------------------------------------------------------------- host


def philox(ctr, key):
    lib = _host_lib()
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    out = (ctypes.c_uint32 * 4)()
    lib.synth_philox_host(ctypes.byref(c), ctypes.byref(k), ctypes.byref(out))
    return tuple(out)


def host_rows(recipe, dtype, b0, nb, t0, nt, h0, nh, threads=None):
    """Rows [b0,b0+nb) x [t0,t0+nt) x [h0,h0+nh) -> array [nb, nt, nh, 128]
    (uint16 bf16 bits, float32 or float64)."""
    dt = _DT[dtype] if isinstance(dtype, str) else dtype
    out = np.empty((nb, nt, nh, D), dtype=_NP[dt])
    _check(_host_lib().synth_rows_host(ctypes.byref(recipe), dt, b0, nb, t0, nt, h0, nh,
                                       out.ctypes.data_as(ctypes.c_void_p), _threads(threads)), "synth_rows_host")
    return out


def host_beta(seed, dtype, b0, nb, t0, nt, h0, nh, threads=None):
    dt = _DT[dtype] if isinstance(dtype, str) else dtype
    out = np.empty((nb, nt, nh), dtype=_NP[dt])
    _check(_host_lib().synth_beta_host(seed & 0xFFFFFFFF, dt, b0, nb, t0, nt, h0, nh,
                                       out.ctypes.data_as(ctypes.c_void_p), _threads(threads)), "synth_beta_host")
    return out


def host_state(seed, scale, dtype, b0, nb, h0, nh, threads=None):
    dt = _DT[dtype] if isinstance(dtype, str) else dtype
    out = np.empty((nb, nh, D, D), dtype=_NP[dt])
    _check(_host_lib().synth_state_host(seed & 0xFFFFFFFF, float(scale), dt, b0, nb, h0, nh,
                                        out.ctypes.data_as(ctypes.c_void_p), _threads(threads)), "synth_state_host")
    return out


def bf16_bits_to_f64(x):
    """Exact upcast of bf16 bit patterns (uint16) to float64."""
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(x):
    return bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


# ----------------------------------------------------------------------------- device


def _stream_ptr(stream):
    return ctypes.c_void_p(stream.cuda_stream if stream is not None else 0)


def device_rows(out, recipe, b0=0, t0=0, h0=0, stream=None):
    """Fill a contiguous CUDA tensor of shape [nb, nt, nh, 128] (bfloat16 or
    float32) with rows starting at (b0, t0, h0)."""
    import torch

    dt = {torch.bfloat16: BF16, torch.float32: F32, torch.float64: F64}[out.dtype]
    assert out.is_cuda and out.is_contiguous() and out.dim() == 4 and out.shape[3] == D
    nb, nt, nh, _ = out.shape
    if stream is None:
        stream = torch.cuda.current_stream(out.device)
    _check(_device_lib().synth_rows_device(ctypes.byref(recipe), dt, b0, nb, t0, nt, h0, nh,
                                           ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)), "synth_rows_device")
    return out


def device_beta(out, seed, b0=0, t0=0, h0=0, stream=None):
    import torch

    dt = {torch.float32: F32, torch.float64: F64}[out.dtype]
    assert out.is_cuda and out.is_contiguous() and out.dim() == 3
    nb, nt, nh = out.shape
    if stream is None:
        stream = torch.cuda.current_stream(out.device)
    _check(_device_lib().synth_beta_device(seed & 0xFFFFFFFF, dt, b0, nb, t0, nt, h0, nh,
                                           ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)), "synth_beta_device")
    return out


def device_state(out, seed, scale, b0=0, h0=0, stream=None):
    import torch

    dt = {torch.float32: F32, torch.float64: F64}[out.dtype]
    assert out.is_cuda and out.is_contiguous() and out.dim() == 4 and out.shape[2:] == (D, D)
    nb, nh = out.shape[:2]
    if stream is None:
        stream = torch.cuda.current_stream(out.device)
    _check(_device_lib().synth_state_device(seed & 0xFFFFFFFF, float(scale), dt, b0, nb, h0, nh,
                                            ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)), "synth_state_device")
    return out
