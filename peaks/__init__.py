"""Measured peaks of the MI355X the benchmark runs on: a streaming device copy
(HBM bytes/s, read + written) and back-to-back bf16 and fp32 MFMA loops
(flop/s).  Measurement infrastructure for bench.py; the KDA library does not
use it.  Each figure is the best of a few timed launches, timed with HIP
events on the launch stream."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libpeaks.so")
_lib = None

MFMA_FLOPS = {True: 16 * 16 * 32 * 2, False: 16 * 16 * 4 * 2}  # per instruction: bf16 16x16x32, fp32 16x16x4


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        L.peaks_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
        L.peaks_copy.restype = ctypes.c_int
        L.peaks_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.peaks_mfma.restype = ctypes.c_int
        L.peaks_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
        L.peaks_read.restype = ctypes.c_int
        L.peaks_valu.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.peaks_valu.restype = ctypes.c_int
        _lib = L
    return _lib


def _best_ms(fn, reps):
    import torch

    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    return best


def hbm_read(nbytes=2 << 30, reps=5, blocks_per_cu=8):
    """Bytes/s of one read pass over nbytes."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    out = torch.empty(blocks_per_cu * cus * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def one():
        rc = _load().peaks_read(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(out.data_ptr()), nbytes,
                                blocks_per_cu * cus, stream)
        if rc != 0:
            raise RuntimeError(f"peaks_read failed with hipError {rc}")

    ms = _best_ms(one, reps)
    del src, out
    torch.cuda.empty_cache()
    return nbytes / (ms / 1e3)


def hbm_copy(nbytes=2 << 30, reps=5, blocks_per_cu=8):
    """Bytes/s of a device copy of nbytes (read once, written once)."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def one():
        rc = _load().peaks_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                                blocks_per_cu * cus, stream)
        if rc != 0:
            raise RuntimeError(f"peaks_copy failed with hipError {rc}")

    ms = _best_ms(one, reps)
    ok = bool(torch.equal(src[:1024], dst[:1024])) and bool(torch.equal(src[-1024:], dst[-1024:]))
    del src, dst
    torch.cuda.empty_cache()
    if not ok:
        raise RuntimeError("peaks_copy produced a wrong copy")
    return 2 * nbytes / (ms / 1e3)


def mfma(bf16=True, iters=4096, reps=3, shape32=False, k16=False):
    """flop/s of a loop of independent MFMAs on every SIMD (4 waves per
    compute unit and SIMD); shape32: the 32x32x16 bf16 instruction; k16: the
    16x16x16 bf16 one."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 4 * cus
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def one():
        mode = 2 if shape32 else 3 if k16 else int(bool(bf16))
        rc = _load().peaks_mfma(ctypes.c_void_p(out.data_ptr()), blocks, iters, mode, stream)
        if rc != 0:
            raise RuntimeError(f"peaks_mfma failed with hipError {rc}")

    ms = _best_ms(one, reps)
    flops = blocks * 4 * iters * 8 * MFMA_FLOPS[bool(bf16)]
    return flops / (ms / 1e3)


def valu_ns_per_instruction(iters=4096, reps=3):
    """Nanoseconds a SIMD takes per wave64 instruction in loops of independent
    v_exp_f32, v_rcp_f32 and v_mul_f32 (4 waves per SIMD), keyed by name."""
    import torch

    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    blocks = 4 * cus
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for op, name in enumerate(("v_exp_f32", "v_rcp_f32", "v_mul_f32")):
        def one():
            rc = _load().peaks_valu(ctypes.c_void_p(out.data_ptr()), blocks, iters, op, stream)
            if rc != 0:
                raise RuntimeError(f"peaks_valu failed with hipError {rc}")

        ms = _best_ms(one, reps)
        per_simd = (blocks * 4) / (cus * 4) * iters * 8  # instructions each SIMD issues
        res[name] = ms * 1e6 / per_simd
    return res
