"""Measured peaks of the GPU the benchmark runs on: matrix-core rates from
kernels that do nothing but MFMAs (libslapeak.so, built from csrc/peak.hip)
and the HBM rate of a plain device copy.  They are the practical ceilings a
roofline fraction is also quoted against, beside the published peaks."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libslapeak.so")

# kind -> (instruction, operand type); the 16x16 and 32x32 forms of each type
KINDS = {
    0: ("v_mfma_i32_16x16x64_i8", "int8"),
    1: ("v_mfma_i32_32x32x32_i8", "int8"),
    2: ("v_mfma_f32_16x16x32_bf16", "bf16"),
    3: ("v_mfma_f32_32x32x16_bf16", "bf16"),
}
PUBLISHED = {"int8": 5.0e15, "bf16": 2.5e15}
WAVES_PER_SIMD = 8  # workgroups of 4 waves, 8 per compute unit

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run python -m sparse_bit_attention_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.slapeak_mfma.restype = ctypes.c_int
        L.slapeak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
        L.slapeak_mfma_ops.restype = ctypes.c_longlong
        L.slapeak_mfma_ops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.slapeak_stream.restype = ctypes.c_int
        L.slapeak_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
        L.slapeak_issue.restype = ctypes.c_int
        L.slapeak_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def ops_per_launch(kind: int, iters: int, grid: int) -> int:
    n = lib().slapeak_mfma_ops(kind, iters, grid)
    if n < 0:
        raise ValueError(f"bad peak kernel arguments kind={kind} iters={iters} grid={grid}")
    return n


def mfma_rate(kind: int, target_ms: float = 25.0, reps: int = 3) -> float:
    """Best of `reps` timed launches of one MFMA kind, in ops (flops) per
    second; each launch is sized to last about target_ms at the published
    peak, with 8 waves on every SIMD."""
    import torch
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    grid = cus * WAVES_PER_SIMD
    per_iter = ops_per_launch(kind, 1, grid)
    iters = max(1, int(target_ms * 1e-3 * PUBLISHED[KINDS[kind][1]] / per_iter))
    out = torch.empty(grid * 4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    L = lib()

    def launch():
        rc = L.slapeak_mfma(kind, iters, grid, ctypes.c_void_p(out.data_ptr()),
                            ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"slapeak_mfma(kind={kind}) failed with {rc}")

    launch()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    return ops_per_launch(kind, iters, grid) / best


def copy_rate(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """HBM bytes per second (read + write) of a plain device-to-device copy."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3)


# issue-probe kinds: (name, instructions per slot); a round is 8 slots
ISSUE_KINDS = {
    0: ("v_fma_f32", 1),
    1: ("v_exp_f32", 1),
    2: ("v_mfma_f32_16x16x32_bf16", 1),
    3: ("v_mfma_f32_16x16x32_bf16 + 2 v_fma_f32", 3),
}


def issue_cycles(kind: int, wps: int, iters: int = 4000) -> dict:
    """One launch (after an untimed one) of the issue probe on every compute
    unit, wps waves per SIMD running the same mix.  Returns the shader-clock
    cycles per slot (one instruction, or for kind 3 one MFMA and the two FMAs
    after it) that one SIMD takes: per workgroup, the span from the first
    wave's start to the last wave's end over the slots its waves ran per
    SIMD, averaged over the workgroups; and the shader clock in GHz (s_memtime
    ticks over 100 MHz real-time ticks)."""
    import torch
    dev = torch.device("cuda:0")
    grid = torch.cuda.get_device_properties(dev).multi_processor_count
    cyc = torch.zeros(grid * 8 * 4, dtype=torch.int64, device=dev)
    dig = torch.zeros(grid * 8, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    L = lib()
    for _ in range(2):
        rc = L.slapeak_issue(kind, wps, iters, grid, ctypes.c_void_p(cyc.data_ptr()),
                             ctypes.c_void_p(dig.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"slapeak_issue(kind={kind}, wps={wps}) failed with {rc}")
    torch.cuda.synchronize()
    c = cyc.view(grid, 8, 4)[:, :4 * wps].double().cpu()
    span = c[:, :, 1].max(dim=1).values - c[:, :, 0].min(dim=1).values
    rspan = c[:, :, 3].max(dim=1).values - c[:, :, 2].min(dim=1).values
    slots_per_simd = 8.0 * iters * wps
    return {"cycles_per_slot_per_simd": float((span / slots_per_simd).mean()),
            "clock_GHz": float((span / rspan).mean()) * 0.1}


def issue_table() -> dict:
    """The issue probe's cycles per slot and clock for each kind at one and
    two waves per SIMD."""
    return {ISSUE_KINDS[k][0]: {f"{w}_wave_per_simd": issue_cycles(k, w) for w in (1, 2)}
            for k in ISSUE_KINDS}


def stream_rate(kind: int, waves: int, iters: int = 2000) -> float:
    """Bytes per shader cycle one compute unit delivers into registers when
    `waves` waves read 16-byte pieces back to back: kind 0 from its L1 (a
    16 KiB block of global memory per workgroup), kind 1 from LDS.  Per
    workgroup the bytes over the span from the first wave's start to the last
    wave's end, averaged over one launch on every compute unit (after one
    untimed launch)."""
    import torch
    dev = torch.device("cuda:0")
    grid = torch.cuda.get_device_properties(dev).multi_processor_count
    buf = torch.zeros(grid * 16384, dtype=torch.uint8, device=dev)
    cyc = torch.zeros(grid * 8 * 2, dtype=torch.int64, device=dev)
    dig = torch.zeros(grid * 8, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    L = lib()
    for _ in range(2):
        rc = L.slapeak_stream(kind, waves, iters, grid, ctypes.c_void_p(buf.data_ptr()),
                              ctypes.c_void_p(cyc.data_ptr()), ctypes.c_void_p(dig.data_ptr()),
                              ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"slapeak_stream(kind={kind}, waves={waves}) failed with {rc}")
    torch.cuda.synchronize()
    c = cyc.view(grid, 8, 2)[:, :waves].double().cpu()
    span = c[:, :, 1].max(dim=1).values - c[:, :, 0].min(dim=1).values
    return float((waves * 8192.0 * iters / span).mean())


def stream_table() -> dict:
    """L1 and LDS delivery rates (bytes per cycle per CU) at 4 and 8 waves."""
    return {name: {f"{w}_waves_per_cu": stream_rate(k, w) for w in (4, 8)}
            for k, name in ((0, "l1_global_load_dwordx4"), (1, "lds_ds_read_b128"))}


def measure() -> dict:
    """Measured peaks: the rate of each MFMA kind, the best of each operand
    type (ops or flops per second) and the copy rate (bytes per second)."""
    rates = {k: mfma_rate(k) for k in KINDS}
    res = {"mfma": {KINDS[k][0]: r for k, r in rates.items()}}
    for typ in ("int8", "bf16"):
        res[typ] = max(r for k, r in rates.items() if KINDS[k][1] == typ)
    res["hbm_copy"] = copy_rate()
    return res
