"""Benchmark of the KDA forward path on one MI355X.

One step = one kda_chunk_fwd call over the prefill workload
kda_prefill_bf16_b1_h96_t8192 (B=1, T=8192, H=96, d=128, bf16 q/k/v/a, fp32
beta and state), inputs already resident in HBM.  Printed as one JSON line:
value = tokens/s; `roofline` is the prefill kernel against HBM (its binding
roof), with `mfma` its algorithmic flops against the bf16 MFMA peak;
`configs` times the other prefill workloads (the fp32 T=512 case, the
4 x 32K batch with an initial state and, unless --no-long, the 1M-token
sequence) with the same fields; `peaks` holds the HBM bandwidth and MFMA
rates measured on the same box (a device copy and MFMA loops), and every
fraction is also given against those; `decode` adds kda_decode_step on the
decode workload (256 sequences x 96 heads, fp32 state updated in place, 64
steps with fresh inputs); `decode_multi` takes the same 64 tokens per state
four at a time through kda_decode_multi; `gate_modes` the prefill with a
scalar gate and with none, `fused_norm` the prefill with the output gate and
norm fused against two passes, `split` the sequence split against the plain
prefill from 8 to 96 heads; `cpu_baseline` is the fp64 oracle timed on the
host on the default workload, with stated samples of the others.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-configs] [--no-long]
                    [--no-split] [--decode-tokens K] [--workload 0|1|2|3]   (the prefill workload of the main line)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H=96,d=128) + decode seq-steps/s; % MFMA/HBM peak"
HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
BF16_MFMA_PEAK = 2.5e15    # MI355X dense bf16 MFMA, flop/s
D = 128
CHUNK = 16
# Algorithmic work per token and head (bf16 I/O): read q, k, a, v (2 B each per
# channel) and beta (4 B), write o (2 B per channel); flops of the chunkwise
# form at C = 16: 6 d^2 (the three state contractions) + 2 C (3 d + 2 d).
BYTES_PER_TOKEN_HEAD_BF16 = 2 * (3 * D + D) + 4 + 2 * D   # 1284
BYTES_PER_TOKEN_HEAD_F32 = 4 * (3 * D + D) + 4 + 4 * D    # 2564
FLOPS_PER_TOKEN_HEAD = 6 * D * D + 2 * CHUNK * (3 * D + 2 * D)  # 118784
STATE_BYTES = D * D * 4
# Decode, per (sequence, head) step: state read + written once, q/k/v/a in, o out.
DECODE_BYTES_PER_UNIT = 2 * STATE_BYTES + BYTES_PER_TOKEN_HEAD_BF16  # 132356
# fp32 VALU work of one token on one state: x = S^T(alpha k) and y = S^T(alpha q)
# (d^2 multiply-adds, 2 d^2 flops, each) and S' = Diag(alpha) S + k (beta e)^T
# (a multiply and a multiply-add, 3 flops, per entry): 7 d^2 flops in all.
DECODE_FLOPS_PER_UNIT = 7 * D * D  # 114688
FP32_VALU_PEAK = 157.3e12  # MI355X fp32 vector, flop/s
FP32_MFMA_PEAK = 157.3e12  # MI355X fp32 matrix, flop/s

PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
PREFILL_KERNEL = "chunk_fwd_bf16_kernel"  # the kernel the bf16 prefill workload runs
COPY_CALIBRATION_BYTES = 1 << 30  # one device-to-device copy of this many bytes (--calibrate-copy)
# the sources each measured kernel is built from: its counters stay valid while these do not change
KERNEL_SOURCES = {
    "chunk_fwd_bf16_kernel": ("kda_prefill_bf16.hip", "kda_bf16_tiles.h", "kda_common.h"),
    "decode_kernel": ("kda_decode.hip", "kda_common.h"),
    "decode_multi_kernel": ("kda_decode.hip", "kda_common.h"),
}


def strip_comments(text):
    """C/C++ source with comments removed and every run of whitespace made one
    space: what the compiler sees, up to formatting.  String and character
    literals are kept as they are."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_sha(kernel):
    """Hash of the sources of `kernel` without their comments and formatting,
    so that edits of comments keep the committed counter summary valid."""
    h = hashlib.sha256()
    for n in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "gated_delta_rule_23_amd", "csrc", n), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
            h.update(b"\0")
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (lines "kernel=<name> kernel_source_sha=<sha> hbm_bytes_per_launch=<n>"),
    or None when there is none or the kernel sources changed since."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            lines = f.readlines()
    except OSError:
        return None
    for line in lines:
        fields = dict(tok.split("=", 1) for tok in line.split() if "=" in tok)
        if fields.get("kernel") == kernel and fields.get("kernel_source_sha") == kernel_source_sha(kernel):
            return float(fields["hbm_bytes_per_launch"])
    return None


def calibrate_copy():
    """One plain device copy of COPY_CALIBRATION_BYTES (read once, written
    once), outside any timed region: under rocprofv3 --pmc its FETCH_SIZE and
    WRITE_SIZE scale the counters of the KDA kernels to bytes."""
    import torch

    n = COPY_CALIBRATION_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def timed_launches(fn, n, stream):
    """Run fn n times back to back; HIP events bracket every launch on the
    stream the kernel runs on.  Returns per-launch milliseconds."""
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def timed_block(fn, n, stream):
    """Run fn n times back to back between two HIP events on the stream the
    kernel runs on (no event between launches, so the stream holds nothing
    but the work).  Returns the average milliseconds per launch."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def draw_prefill(workload):
    """The inputs and output buffers of a prefill workload, on the device."""
    import torch

    from synth.workloads import WORKLOADS, device_inputs

    w = WORKLOADS[workload]
    t_gen = time.perf_counter()
    x = device_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    o = torch.empty((w.B, w.T, w.H, D), dtype=dt, device="cuda")
    S = torch.empty((w.B, w.H, D, D), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    return w, x, o, S, time.perf_counter() - t_gen


def bench_prefill(steps, warmup, workload=1, drawn=None, release=True):
    """kda_chunk_fwd over a whole prefill workload: warmup untimed launches,
    then steps timed ones between two HIP events on the launch stream.
    drawn: the workload's inputs from draw_prefill, drawn earlier (else now);
    release: hand the freed memory back to the device at once (else it stays
    in torch's cache, which takes no time)."""
    import torch

    import gated_delta_rule_23_amd as kda

    w, x, o, S, t_gen = drawn if drawn is not None else draw_prefill(workload)
    drawn = None
    stream = torch.cuda.current_stream()

    def step():
        kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["a"], x["beta"], initial_state=x["s0"], o=o, final_state=S,
                          stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    avg_ms = timed_block(step, steps, stream)
    wall = time.perf_counter() - t0
    tokens = w.B * w.T
    per_token_head = BYTES_PER_TOKEN_HEAD_BF16 if w.dtype == "bf16" else BYTES_PER_TOKEN_HEAD_F32
    # inputs and o per token-head, the final state written, and the initial state read when there is one
    launch_bytes = (w.B * w.T * w.H * per_token_head
                    + w.B * w.H * STATE_BYTES * (2 if x["s0"] is not None else 1))
    launch_flops = w.B * w.T * w.H * FLOPS_PER_TOKEN_HEAD
    del x, o, S
    if release:
        torch.cuda.empty_cache()
    return dict(workload=w, tokens=tokens, wall=wall, launches=steps, avg_ms=avg_ms,
                launch_bytes=launch_bytes, launch_flops=launch_flops, gen_s=t_gen)


def prefill_fields(pre, peaks_measured):
    """The roofline and MFMA fields of one prefill measurement."""
    w = pre["workload"]
    avg_s = pre["avg_ms"] / 1e3
    achieved = pre["launch_bytes"] / avg_s
    fl = pre["launch_flops"] / avg_s
    mfma_peak = BF16_MFMA_PEAK if w.dtype == "bf16" else FP32_MFMA_PEAK
    mfma_meas = (peaks_measured or {}).get("mfma_bf16_tflops" if w.dtype == "bf16" else "mfma_f32_tflops")
    hbm_meas = (peaks_measured or {}).get("hbm_gbs")
    roof = {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
            "frac": achieved / HBM_PEAK, "frac_of_measured_peak": achieved / 1e9 / hbm_meas if hbm_meas else None,
            "kernel": PREFILL_KERNEL if w.dtype == "bf16" else "chunk_fwd_kernel", "launch_ms": pre["avg_ms"],
            "algorithmic_bytes_per_launch": pre["launch_bytes"]}
    mfma = {"algorithmic_flops_per_launch": pre["launch_flops"], "achieved_tflops": fl / 1e12,
            "dtype": w.dtype, "peak_tflops": mfma_peak / 1e12, "frac": fl / mfma_peak,
            "frac_of_measured_peak": fl / 1e12 / mfma_meas if mfma_meas else None}
    return roof, mfma


def measure_peaks():
    """HBM and MFMA rates on this machine (peaks/): the best of a device copy and
    a read pass (2 GiB, 16-byte non-temporal accesses, two workgroups of 256
    threads per compute unit, the best of a sweep of 2 to 32), and the best of
    loops of independent MFMAs of each bf16 shape (on gfx950 the 32x32x16
    instruction reaches about twice the flop rate of the 16x16 ones)."""
    import peaks

    copy = peaks.hbm_copy(blocks_per_cu=2) / 1e9
    read = peaks.hbm_read(blocks_per_cu=2) / 1e9
    bf16 = {"16x16x32": peaks.mfma(bf16=True) / 1e12, "16x16x16": peaks.mfma(bf16=True, k16=True) / 1e12,
            "32x32x16": peaks.mfma(bf16=True, shape32=True) / 1e12}
    return {"hbm_copy_gbs": copy, "hbm_read_gbs": read, "hbm_gbs": max(copy, read),
            "mfma_bf16_tflops": max(bf16.values()), "mfma_bf16_tflops_by_shape": bf16,
            "mfma_f32_tflops": peaks.mfma(bf16=False) / 1e12,
            "valu_ns_per_wave_instruction": peaks.valu_ns_per_instruction(),
            "spec": {"hbm_gbs": HBM_PEAK / 1e9, "mfma_bf16_tflops": BF16_MFMA_PEAK / 1e12,
                     "mfma_f32_tflops": FP32_MFMA_PEAK / 1e12},
            "how": "best of 5 launches: 2 GiB copy (read + written bytes) and read; MFMA loops of 8 or 16 "
                   "independent accumulators per wave, 4 waves per SIMD; VALU loops of 8 independent chains a lane "
                   "(the time per wave64 instruction per SIMD)"}


def bench_gate_norm(w, reps=50):
    """kda_output_gate_norm over a prefill output's B*T*H rows of 128 bf16
    channels (o and the gate read, y written)."""
    import torch

    import gated_delta_rule_23_amd as kda

    g = torch.Generator(device="cuda").manual_seed(w.seed)
    o = torch.randn((w.B, w.T, w.H, D), device="cuda", generator=g).to(torch.bfloat16)
    z = torch.randn((w.B, w.T, w.H, D), device="cuda", generator=g).to(torch.bfloat16)
    y = torch.empty_like(o)
    stream = torch.cuda.current_stream()

    def one():
        kda.kda_output_gate_norm(o, z, 1e-6, y=y, stream=stream)

    for _ in range(5):
        one()
    torch.cuda.synchronize()
    avg_ms = timed_block(one, reps, stream)
    rows = w.B * w.T * w.H
    return dict(rows=rows, avg_ms=avg_ms, bytes=3 * rows * D * 2)


# (H, T, segments) of single bf16 sequences: few heads (the split's use) up to the default workload's 96
SPLIT_CASES = ((8, 65536, 16), (16, 65536, 8), (32, 32768, 8), (48, 32768, 4), (64, 32768, 4), (96, 8192, 2))


def median_launch_ms(fn, stream, warm=10, reps=20):
    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ms = sorted(timed_launches(fn, reps, stream))
    return ms[len(ms) // 2]


def bench_gate_modes(w):
    """kda_chunk_fwd_gated on the default workload's shape with one fp32
    logit per token and head ("scalar") and with no gate ("none"), against
    the per-channel gate: median launch time and HBM rate (the gate's bytes
    are 4 per token-head for the scalar gate, none without)."""
    import torch

    import gated_delta_rule_23_amd as kda
    from synth.workloads import device_inputs

    x = device_inputs(w)
    o = torch.empty((w.B, w.T, w.H, D), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((w.B, w.H, D, D), dtype=torch.float32, device="cuda")
    a_scalar = x["a"][..., 0].float().contiguous()
    stream = torch.cuda.current_stream()
    out = {}
    modes = (("channel", x["a"], 2 * D), ("scalar", a_scalar, 4), ("none", None, 0))
    # alternated rounds, so that no mode runs on a colder clock than the others; the best round counts
    best = {}
    for _ in range(3):
        for mode, a, _gb in modes:
            ms = median_launch_ms(lambda: kda.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], a, x["beta"], gate=mode,
                                                                 o=o, final_state=S, stream=stream),
                                  stream, warm=3, reps=10)
            best[mode] = min(best.get(mode, ms), ms)
    for mode, a, gate_bytes in modes:
        ms = best[mode]
        nbytes = w.B * w.T * w.H * (BYTES_PER_TOKEN_HEAD_BF16 - 2 * D + gate_bytes) + w.B * w.H * STATE_BYTES
        out[mode] = {"ms_per_launch": ms, "tokens_per_s": w.B * w.T / (ms / 1e3),
                     "gate_bytes_per_token_head": gate_bytes, "algorithmic_bytes_per_launch": nbytes,
                     "hbm_frac": nbytes / (ms / 1e3) / HBM_PEAK}
    del x, o, S, a_scalar
    torch.cuda.empty_cache()
    return out


def bench_fused_norm(w):
    """The prefill with sigmoid(z) * RMSNorm(o) fused into its output store
    (kda_chunk_fwd_norm) against the prefill followed by the separate
    kda_output_gate_norm pass, on the default workload's shape."""
    import torch

    import gated_delta_rule_23_amd as kda
    from synth.workloads import device_inputs

    x = device_inputs(w)
    z = x["v"].clone()
    o = torch.empty((w.B, w.T, w.H, D), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(o)
    S = torch.empty((w.B, w.H, D, D), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def two():
        kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["a"], x["beta"], initial_state=x["s0"], o=o, final_state=S,
                          stream=stream)
        kda.kda_output_gate_norm(o, z, 1e-6, y=y, stream=stream)

    def fused():
        kda.kda_chunk_fwd_norm(x["q"], x["k"], x["v"], x["a"], x["beta"], z, eps=1e-6, initial_state=x["s0"], y=y,
                               final_state=S, stream=stream)

    # alternated rounds, so that neither side runs on a colder clock than the other
    reps = 10 if w.T * w.B <= 8192 else 3
    rounds = {"fused": [], "two": []}
    for _ in range(3):
        rounds["fused"].append(median_launch_ms(fused, stream, warm=2, reps=reps))
        rounds["two"].append(median_launch_ms(two, stream, warm=2, reps=reps))
    ms_fused, ms_two = min(rounds["fused"]), min(rounds["two"])
    # z read as well; the initial state when there is one
    nbytes = (w.B * w.T * w.H * (BYTES_PER_TOKEN_HEAD_BF16 + 2 * D)
              + w.B * w.H * STATE_BYTES * (2 if x["s0"] is not None else 1))
    del x, z, o, y, S
    torch.cuda.empty_cache()
    return {"workload": w.name, "ms_fused": ms_fused, "ms_prefill_then_norm": ms_two, "speedup": ms_two / ms_fused,
            "algorithmic_bytes_fused": nbytes, "hbm_frac_fused": nbytes / (ms_fused / 1e3) / HBM_PEAK,
            "layout": ("the prefill into y, then the gate and norm in place (sequences that fit as workgroup pairs)"
                       if w.B * w.H <= 8 * (torch.cuda.get_device_properties(0).multi_processor_count // 16) else
                       "fused into the O store (one workgroup per sequence: a row's 128 value channels in one "
                       "workgroup)")}


def bench_split(cases=SPLIT_CASES, reps=10):
    """kda_chunk_fwd against kda_chunk_fwd_split on single sequences with
    few heads (B = 1; H, T, segments per case), bf16, median launch times."""
    import dataclasses

    import torch

    import gated_delta_rule_23_amd as kda
    from synth.workloads import WORKLOADS, device_inputs

    out = []
    for H, T, P in cases:
        w = dataclasses.replace(WORKLOADS[1], B=1, H=H, T=T)
        x = device_inputs(w)
        o = torch.empty((1, T, H, D), dtype=torch.bfloat16, device="cuda")
        S = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
        stream = torch.cuda.current_stream()
        times = {}
        for name, segs in (("unsplit", 1), ("split", P)):
            def one(segs=segs):
                kda.kda_chunk_fwd_split(x["q"], x["k"], x["v"], x["a"], x["beta"], segs, o=o, final_state=S,
                                        stream=stream)

            for _ in range(3):
                one()
            torch.cuda.synchronize()
            ms = sorted(timed_launches(one, reps, stream))
            times[name] = ms[len(ms) // 2]
        out.append({"B": 1, "H": H, "T": T, "segments": P, "ms_unsplit": times["unsplit"], "ms_split": times["split"],
                    "speedup": times["unsplit"] / times["split"]})
        del x, o, S
        torch.cuda.empty_cache()
    return out


def bench_decode(reps=3):
    import torch

    import gated_delta_rule_23_amd as kda
    from synth.workloads import WORKLOADS, device_inputs

    w = WORKLOADS[4]
    x = device_inputs(w)
    steps = [{k: x[k][:, t].contiguous() for k in ("q", "k", "v", "a", "beta")} for t in range(w.T)]
    for k in ("q", "k", "v", "a", "beta"):
        del x[k]
    s0 = x["s0"]
    state = torch.empty_like(s0)
    outs = [torch.empty((w.B, w.H, D), dtype=torch.bfloat16, device="cuda") for _ in range(w.T)]
    stream = torch.cuda.current_stream()
    totals = []
    per_step = []
    for rep in range(reps + 1):
        state.copy_(s0)  # restore the initial state outside the timed region
        torch.cuda.synchronize()
        it = iter(range(w.T))

        def one():
            t = next(it)
            s = steps[t]
            kda.kda_decode_step(s["q"], s["k"], s["v"], s["a"], s["beta"], state, o=outs[t], stream=stream)

        ms = timed_block(one, w.T, stream)  # the 64 steps back to back, as a decode loop issues them
        if rep > 0:  # the first repetition is the warm-up
            totals.append(ms * w.T)
            per_step.append(ms)
    best = min(totals)
    unit_bytes = w.B * w.H * DECODE_BYTES_PER_UNIT
    avg_step_ms = sum(per_step) / len(per_step)
    return dict(workload=w, seq_steps_per_s=w.B * w.T / (best / 1e3), avg_step_ms=avg_step_ms,
                step_bytes=unit_bytes, steps=w.T, reps=reps)


def bench_decode_multi(k_tokens, reps=3):
    """The decode workload's 64 tokens per state taken k_tokens at a time by
    kda_decode_multi (every token committed): one state read and one write
    per call instead of per token."""
    import torch

    import gated_delta_rule_23_amd as kda
    from synth.workloads import WORKLOADS, device_inputs

    w = WORKLOADS[4]
    if k_tokens < 1 or w.T % k_tokens:
        raise SystemExit(f"--decode-tokens must divide the workload's {w.T} tokens")
    x = device_inputs(w)
    calls = [{n: x[n][:, t:t + k_tokens].contiguous() for n in ("q", "k", "v", "a", "beta")}
             for t in range(0, w.T, k_tokens)]
    for n in ("q", "k", "v", "a", "beta"):
        del x[n]
    s0 = x["s0"]
    state = torch.empty_like(s0)
    outs = [torch.empty((w.B, c["q"].shape[1], w.H, D), dtype=torch.bfloat16, device="cuda") for c in calls]
    stream = torch.cuda.current_stream()
    totals, per_call = [], []
    for rep in range(reps + 1):
        state.copy_(s0)  # restore the initial state outside the timed region
        torch.cuda.synchronize()
        it = iter(range(len(calls)))

        def one():
            i = next(it)
            c = calls[i]
            kda.kda_decode_multi(c["q"], c["k"], c["v"], c["a"], c["beta"], state, o=outs[i], stream=stream)

        ms = timed_block(one, len(calls), stream)
        if rep > 0:
            totals.append(ms * len(calls))
            per_call.append(ms)
    best = min(totals)
    avg_call_ms = sum(per_call) / len(per_call)
    call_bytes = w.B * w.H * (2 * STATE_BYTES + k_tokens * BYTES_PER_TOKEN_HEAD_BF16)
    call_flops = w.B * w.H * k_tokens * DECODE_FLOPS_PER_UNIT
    return dict(workload=w, seq_steps_per_s=w.B * w.T / (best / 1e3), avg_call_ms=avg_call_ms,
                call_bytes=call_bytes, call_flops=call_flops, calls=len(calls), k=k_tokens, reps=reps)


def host_description():
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": cpu_model, "nproc": os.cpu_count(), "cpus_available": affinity, "rocm": rocm}


def cpu_threads():
    """The host threads the oracle uses: every CPU this process may run on,
    at most 16 (the host CPUs that go with one GPU of an eight-GPU, 128-core
    node)."""
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, avail))


def _oracle_timed(w, threads, b0=0, nb=None, t0=0, nt=None, h0=0, nh=None):
    """Regenerate a block of workload w on the host (not timed) and time the
    oracle over it.  Returns (seconds, token-heads)."""
    import numpy as np

    import oracle
    import synth
    from synth.workloads import host_inputs

    h = host_inputs(w, b0=b0, nb=nb, t0=t0, nt=nt, h0=h0, nh=nh, threads=threads)
    args = (synth.to_f64(h["q"]), synth.to_f64(h["k"]), synth.to_f64(h["v"]), h["beta"].astype(np.float64))
    a = synth.to_f64(h["a"])
    s0 = None if h["s0"] is None or t0 != 0 else h["s0"].astype(np.float64)
    del h
    t = time.perf_counter()
    oracle.forward(*args, a=a, s0=s0, threads=threads)
    return time.perf_counter() - t, args[0].shape[0] * args[0].shape[1] * args[0].shape[2]


def cpu_baseline(threads, others=True):
    """The oracle as it stands, on the default prefill workload (all 96
    heads, all 8192 tokens), and, with others, on stated samples of the
    other workloads.  Input generation on the host is not timed."""
    from synth.workloads import WORKLOADS

    w = WORKLOADS[1]
    dt, th = _oracle_timed(w, threads)
    out = {"value": w.B * w.T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"the whole {w.name} workload ({th} token-heads) in {dt:.2f} s, "
                     f"fp64, one thread per (batch, head) sequence", "host": host_description()}
    if others:
        per = {}
        w0 = WORKLOADS[0]
        dt0, th0 = _oracle_timed(w0, threads)
        per[w0.name] = {"tokens_per_s": w0.B * w0.T / dt0, "s": dt0, "sample": f"whole ({th0} token-heads)"}
        w2 = WORKLOADS[2]
        dt2, th2 = _oracle_timed(w2, threads, h0=0, nh=8)
        # tokens/s of the whole workload at the sample's rate: 8 of 96 heads were run
        per[w2.name] = {"tokens_per_s": w2.B * w2.T * 8 / w2.H / dt2, "s": dt2,
                        "sample": f"heads 0-7 of all 4 sequences, all 32768 tokens ({th2} token-heads); "
                                  "tokens/s scaled to all 96 heads"}
        w3 = WORKLOADS[3]
        nt3 = 131072
        dt3, th3 = _oracle_timed(w3, threads, nt=nt3, h0=0, nh=3)
        per[w3.name] = {"tokens_per_s": nt3 * 3 / dt3 / w3.H, "s": dt3,
                        "sample": f"heads 0-2, the first {nt3} tokens ({th3} token-heads); "
                                  "tokens/s scaled to all 96 heads"}
        w4 = WORKLOADS[4]
        dt4, th4 = _oracle_timed(w4, threads, nb=64)
        per[w4.name] = {"seq_steps_per_s": 64 * w4.H * w4.T / dt4 / w4.H, "s": dt4,
                        "sample": f"64 of the 256 sequences, all 96 heads, all 64 steps ({th4} token-heads); "
                                  "seq-steps/s counts (sequence, step) pairs over all heads"}
        out["other_workloads"] = per
    return out


def log(msg):
    """Progress on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# The other prefill workloads timed beside the main line: (index, untimed warm-up, timed launches).
OTHER_CONFIGS = ((2, 2, 10), (0, 3, 20), (3, 1, 3))


def config_entry(pre, peaks_measured):
    w = pre["workload"]
    roof, mfma = prefill_fields(pre, peaks_measured)
    return {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "dtype": w.dtype, "initial_state": w.s0_scale is not None,
            "tokens_per_s": pre["tokens"] / (pre["avg_ms"] / 1e3), "ms_per_launch": pre["avg_ms"],
            "launches": pre["launches"], "roofline": roof, "mfma": mfma,
            "input_generation_s": pre["gen_s"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The prefill settles at its steady launch time after some 20 launches
    # (clock ramp): the default warm-up covers that, and the timed launches
    # dominate the average a kernel trace of the same command reports.  The
    # other workloads run first, so the main line's clock is warm whatever
    # --warmup says.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-configs", action="store_true", help="skip the other prefill workloads and the peaks")
    ap.add_argument("--no-long", action="store_true", help="skip the 1M-token workload among the other workloads")
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 2, 3],
                    help="prefill workload of the main line: 1 = B1 H96 T8192 (default), 0 = fp32 B1 H2 T512, "
                         "2 = B4 H96 T32768 with S0, 3 = B1 H96 T1048576 mixed decay")
    ap.add_argument("--no-split", action="store_true",
                    help="skip timing kda_chunk_fwd_split against kda_chunk_fwd on single sequences")
    ap.add_argument("--decode-tokens", type=int, default=4,
                    help="tokens per kda_decode_multi call on the decode workload (1 skips that measurement)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (every (batch, head) "
              "sequence is independent; the multi-GPU split is described in DESIGN.md, not run)", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import __graft_entry__

    __graft_entry__._ensure_built()
    if args.calibrate_copy:
        calibrate_copy()

    measured = None
    others = []
    # The main line's inputs are drawn before the other workloads run, so that
    # its launches follow the last of them directly: the GPU's clock settles
    # to each kernel's load over ~30 launches (8K x 96 prefill right after a
    # fresh draw: 437 us falling to 400 us; right after the 1M-token workload,
    # which runs the same kernel: 400 us from the second launch).  The last
    # workload's memory goes back to the device only after the main line,
    # since releasing 125 GB leaves the GPU idle long enough to cool it.
    main_drawn = draw_prefill(args.workload)
    if not args.no_configs:
        measured = measure_peaks()
        log(f"peaks: HBM {measured['hbm_gbs']:.0f} GB/s, bf16 MFMA {measured['mfma_bf16_tflops']:.0f} "
            f"TFLOP/s, fp32 MFMA {measured['mfma_f32_tflops']:.1f} TFLOP/s; VALU ns per wave instruction "
            + ", ".join(f"{k} {v:.2f}" for k, v in measured["valu_ns_per_wave_instruction"].items()))
        for idx, warm, n in OTHER_CONFIGS:
            if idx == args.workload or (idx == 3 and args.no_long):
                continue
            pre_i = bench_prefill(n, warm, idx, release=False)
            others.append(config_entry(pre_i, measured))
            log(f"workload {idx}: {pre_i['avg_ms']:.3f} ms per launch (inputs drawn in {pre_i['gen_s']:.1f} s)")

    pre = bench_prefill(args.steps, args.warmup, args.workload, drawn=main_drawn)
    del main_drawn
    torch.cuda.empty_cache()
    log(f"main line: {pre['avg_ms']:.4f} ms per launch")
    w = pre["workload"]
    wall_per_step = pre["wall"] / args.steps
    roof, mfma = prefill_fields(pre, measured)
    # counters were taken on the default workload
    roof["traffic"] = measured_traffic(PREFILL_KERNEL) if args.workload == 1 else None
    result = {
        "metric": METRIC,
        "value": pre["tokens"] / wall_per_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "d_k": D, "d_v": D, "chunk": CHUNK,
                   "io": f"{w.dtype} q/k/v/a/o, fp32 beta and state", "seed": w.seed},
        "roofline": roof,
        "mfma": mfma,
    }
    if measured is not None:
        result["peaks"] = measured
        result["configs"] = others
    if args.workload == 1:
        # the eq. (6) epilogue over the prefill's output rows (o and the gate read, y written once)
        gn = bench_gate_norm(pre["workload"])
        result["output_gate_norm"] = {
            "rows": gn["rows"], "ms_per_launch": gn["avg_ms"], "kernel": "gate_norm_kernel",
            "hbm": {"achieved": gn["bytes"] / (gn["avg_ms"] / 1e3) / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                    "frac": gn["bytes"] / (gn["avg_ms"] / 1e3) / HBM_PEAK, "algorithmic_bytes_per_launch": gn["bytes"]},
        }
    if not args.no_decode:
        torch.cuda.empty_cache()
        dec = bench_decode()
        log(f"decode: {dec['avg_step_ms']:.4f} ms per step")
        dach = dec["step_bytes"] / (dec["avg_step_ms"] / 1e3)
        hbm_meas = measured["hbm_gbs"] if measured else None
        result["decode"] = {
            "workload": dec["workload"].name, "value": dec["seq_steps_per_s"], "unit": "seq-steps/s",
            "steps": dec["steps"], "reps": dec["reps"], "ms_per_step": dec["avg_step_ms"],
            "roofline": {"bound": "hbm", "achieved": dach / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                         "frac": dach / HBM_PEAK, "frac_of_measured_peak": dach / 1e9 / hbm_meas if hbm_meas else None,
                         "traffic": measured_traffic("decode_kernel"),
                         "kernel": "decode_kernel", "algorithmic_bytes_per_launch": dec["step_bytes"]},
        }
        if args.decode_tokens > 1:
            torch.cuda.empty_cache()
            mul = bench_decode_multi(args.decode_tokens)
            log(f"multi-token decode: {mul['avg_call_ms']:.4f} ms per call")
            mb = mul["call_bytes"] / (mul["avg_call_ms"] / 1e3)
            mf = mul["call_flops"] / (mul["avg_call_ms"] / 1e3)
            result["decode_multi"] = {
                "workload": mul["workload"].name, "tokens_per_call": mul["k"], "value": mul["seq_steps_per_s"],
                "unit": "seq-steps/s", "calls": mul["calls"], "reps": mul["reps"], "ms_per_call": mul["avg_call_ms"],
                "vs_single_step": mul["seq_steps_per_s"] / dec["seq_steps_per_s"],
                "hbm": {"achieved": mb / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": mb / HBM_PEAK,
                        "frac_of_measured_peak": mb / 1e9 / hbm_meas if hbm_meas else None,
                        "algorithmic_bytes_per_launch": mul["call_bytes"]},
                # past eight tokens a fully committed call runs as the chunkwise prefill, whose
                # counters are taken on the prefill workload, not on this one
                "traffic": measured_traffic("decode_multi_kernel") if mul["k"] <= 8 else None,
                "alu": {"achieved": mf / 1e12, "peak": FP32_VALU_PEAK / 1e12, "unit": "TFLOP/s",
                        "frac": mf / FP32_VALU_PEAK, "algorithmic_flops_per_launch": mul["call_flops"]},
                "kernel": "decode_multi_kernel" if mul["k"] <= 8 else "chunk_fwd_bf16_kernel",
            }
    if args.workload == 1 and not args.no_configs:
        result["gate_modes"] = bench_gate_modes(pre["workload"])
        log("gate modes: " + ", ".join(f"{k} {v['ms_per_launch']:.3f} ms" for k, v in result["gate_modes"].items()))
        from synth.workloads import WORKLOADS

        result["fused_norm"] = [bench_fused_norm(pre["workload"]), bench_fused_norm(WORKLOADS[2])]
        log("fused norm: " + ", ".join(f"{f['workload']} {f['ms_fused']:.3f} ms against {f['ms_prefill_then_norm']:.3f}"
                                       f" ms in two passes" for f in result["fused_norm"]))
    if not args.no_split:
        result["split"] = bench_split()
        log("split: " + ", ".join(f"H{c['H']} {c['speedup']:.2f}x" for c in result["split"]))
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(cpu_threads(), others=not args.no_configs)
        log("oracle timed")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
