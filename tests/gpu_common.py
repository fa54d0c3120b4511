"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
on inputs drawn in device memory, regenerate the same inputs on the host and
run the fp64 oracle on them."""
import dataclasses

import numpy as np

import oracle
import synth
from synth.workloads import WORKLOADS, Workload, device_inputs, host_inputs

# Relative L2 gates: fp32 I/O and bf16 I/O (o and final state, separately).
TOL = {"f32": 1e-5, "bf16": 2e-2}


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def to_np(t):
    import torch

    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy().astype(np.float64)


def variant(w, **kw):
    """A copy of workload w with fields overridden (new index = new seed)."""
    return dataclasses.replace(w, **kw)


def oracle_block(w, b0=0, nb=None, t0=0, nt=None, h0=0, nh=None, s0=None, dtype=None, threads=None):
    """Regenerate a block of w on the host and run the oracle on it.  s0:
    None -> the workload's own initial state for the block if it has one
    (and t0 == 0), else zeros; an array -> that state."""
    h = host_inputs(w, b0=b0, nb=nb, t0=t0, nt=nt, h0=h0, nh=nh, dtype=dtype)
    if s0 is None and h["s0"] is not None and t0 == 0:
        s0 = h["s0"].astype(np.float64)
    return oracle.forward(synth.to_f64(h["q"]), synth.to_f64(h["k"]), synth.to_f64(h["v"]),
                          h["beta"].astype(np.float64), a=synth.to_f64(h["a"]), s0=s0, threads=threads)


def print_case(msg):
    print(msg, flush=True)


__all__ = ["TOL", "WORKLOADS", "Workload", "device_inputs", "host_inputs", "oracle_block", "rel_l2", "to_np",
           "variant", "print_case"]
