"""The five KDA workloads (shapes and input distributions) and helpers that
draw them on the host or directly in device memory.

Distributions (all seeded, synthetic):
  q, k   ~ N(0, 1) per channel, then L2-normalised per (b, t, h) row in fp64
  v      ~ N(0, 1)
  a      ~ N(mean, 1) gate logits; mean 0, or (kda_long_1m) +3 on key channels
           0..63 and -3 on 64..127
  beta   = sigmoid(N(0, 1)) per (b, t, h), fp32
  S0     ~ N(0, 0.02^2) fp32 per state entry, where the workload has one
Each value is rounded once to the I/O dtype (bf16 via fp32, round to nearest
even); beta and states stay fp32.  The Philox key is (seed, b), so every
sequence of a batch has its own stream.
"""
from dataclasses import dataclass
from typing import Optional, Tuple

D = 128
BASE_SEED = 20260727


def seed_for(index):
    return BASE_SEED + 97 * index


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    kind: str                 # "prefill" or "decode"
    B: int
    H: int
    T: int                    # tokens per sequence (decode: number of steps)
    dtype: str                # "f32" or "bf16" for q, k, v, a, o
    a_mean: Tuple[float, float] = (0.0, 0.0)
    a_split: int = D          # channels < a_split use a_mean[0], the rest a_mean[1]
    s0_scale: Optional[float] = None

    @property
    def seed(self):
        return seed_for(self.index)

    def tokens(self):
        return self.B * self.T


WORKLOADS = {
    0: Workload(0, "kda_prefill_f32_b1_h2_t512", "prefill", 1, 2, 512, "f32"),
    1: Workload(1, "kda_prefill_bf16_b1_h96_t8192", "prefill", 1, 96, 8192, "bf16"),
    2: Workload(2, "kda_prefill_bf16_b4_h96_t32768_s0", "prefill", 4, 96, 32768, "bf16", s0_scale=0.02),
    3: Workload(3, "kda_prefill_bf16_b1_h96_t1048576_mixed_decay", "prefill", 1, 96, 1048576, "bf16",
                a_mean=(3.0, -3.0), a_split=64),
    4: Workload(4, "kda_decode_bf16_b256_h96_64steps_s0", "decode", 256, 96, 64, "bf16", s0_scale=0.02),
}


def recipes(w, seed=None):
    """Row recipes for q, k, v, a of workload w."""
    from . import A, K, Q, V, row_recipe

    s = w.seed if seed is None else seed
    return {
        "q": row_recipe(s, Q, l2norm=True),
        "k": row_recipe(s, K, l2norm=True),
        "v": row_recipe(s, V),
        "a": row_recipe(s, A, mean=w.a_mean, split=w.a_split),
    }


def host_inputs(w, b0=0, nb=None, t0=0, nt=None, h0=0, nh=None, dtype=None, threads=None, seed=None):
    """Draw a block of workload w on the host.  Returns numpy arrays
    q, k, v, a [nb, nt, nh, 128] (uint16 bf16 bits or float32/64),
    beta [nb, nt, nh] float32 (float64 when dtype='f64'), s0 [nb, nh, 128, 128]
    float32 or None."""
    from . import host_beta, host_rows, host_state

    nb = w.B - b0 if nb is None else nb
    nt = w.T - t0 if nt is None else nt
    nh = w.H - h0 if nh is None else nh
    dt = w.dtype if dtype is None else dtype
    s = w.seed if seed is None else seed
    out = {name: host_rows(r, dt, b0, nb, t0, nt, h0, nh, threads) for name, r in recipes(w, s).items()}
    out["beta"] = host_beta(s, "f64" if dt == "f64" else "f32", b0, nb, t0, nt, h0, nh, threads)
    out["s0"] = None
    if w.s0_scale is not None:
        out["s0"] = host_state(s, w.s0_scale, "f64" if dt == "f64" else "f32", b0, nb, h0, nh, threads)
    return out


def device_inputs(w, device="cuda", stream=None, T=None, B=None, H=None, seed=None, dtype=None):
    """Draw workload w directly in device memory (torch tensors).  B, T, H
    override the shape (the first B sequences, T tokens, H heads of the same
    streams); dtype overrides the I/O type ("bf16" or "f32")."""
    import torch

    from . import device_beta, device_rows, device_state

    s = w.seed if seed is None else seed
    T = w.T if T is None else T
    B = w.B if B is None else B
    H = w.H if H is None else H
    dt = w.dtype if dtype is None else dtype
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = {}
    for name, r in recipes(w, s).items():
        out[name] = device_rows(torch.empty((B, T, H, D), dtype=tdt, device=device), r, stream=stream)
    out["beta"] = device_beta(torch.empty((B, T, H), dtype=torch.float32, device=device), s, stream=stream)
    out["s0"] = None
    if w.s0_scale is not None:
        out["s0"] = device_state(torch.empty((B, H, D, D), dtype=torch.float32, device=device), s, w.s0_scale,
                                 stream=stream)
    return out
