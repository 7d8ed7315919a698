"""SageSLA forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan14b-720p]
                    [--qk int8|int8-fine|bf16]
    python bench.py --op w8a8 [--linear wan14b-720p-qkv]   (the W8A8 linear layer)
    python bench.py --op bwd [--workload wan14b-720p]      (plain-SLA backward)

One step = the whole forward (sla_quantize, then sla_prepare_kv and
sla_attend) over one batch of seeded synthetic inputs already resident in
HBM.  Prints one JSON line: dense-equivalent TFLOP/s (4*B*H*N^2*d per call /
time), ms per call (mean, and p10 / median / p90 of the per-call times), the
per-stage times, the roofline of the dominant kernel (the block-sparse
attention kernel, timed with HIP events on the stream it runs on) against the
published peaks and against peaks measured on the same GPU after the timed
region (MFMA-only kernels, a device copy), the SHA-256 of each input as
uploaded, and the CPU oracle timed on the host's cores: a bounded sample of
the same workload on one pinned core and on all cores (host CPU model and
core count recorded), plus the small workloads run in full.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_bit_attention_amd import synth  # noqa: E402

# MI355X published peaks
P_I8 = 5.0e15        # dense INT8 MFMA, ops/s
P_BF16 = 2.5e15      # dense bf16 MFMA, flop/s
P_HBM = 8.0e12       # bytes/s
METRIC = "SageSLA fwd ms/call + dense-equiv TFLOPS (%MFMA peak), Wan-14B-720P shape"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_attn_wan14b-720p_traffic.json")
ATTN_SRC = os.path.join(ROOT, "sparse_bit_attention_amd", "csrc", "k_attn.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_work(wl, kb, T, qk_int8=True):
    """Algorithmic MFMA work of one launch of the attention kernel.

    Per kept (query block, key block) pair: 2*64*64*d INT8 ops (QK^T; bf16
    flops in the plain SLA mode) and 2*64*64*d bf16 flops (PV).  Per query
    block with the linear branch on: 2*64*d*d (H^T phi(Q)^T) + 2*64*d*d
    (projection) bf16 flops."""
    BH = wl.B * wl.H
    pairs = BH * T * kb
    qk = pairs * 2 * 64 * 64 * wl.d
    bf = pairs * 2 * 64 * 64 * wl.d
    if wl.use_linear and kb < T:
        bf += BH * T * 4 * 64 * wl.d * wl.d
    if qk_int8:
        return qk, bf, pairs
    return 0, bf + qk, pairs


def src_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_entry():
    """HBM bytes per launch of the attention kernel from committed rocprofv3
    counter runs, if they were taken on the current kernel source."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_sha256_16") != src_hash(ATTN_SRC):
        return None
    return t.get("bytes_per_launch")


def measured_peaks(skip=False):
    """The GPU's own ceilings, measured after the timed region: MFMA-only
    kernels per operand type (best of the 16x16 and 32x32 forms) and a plain
    device copy.  Returned in the units the JSON line uses; None if skipped."""
    if skip:
        return None
    from sparse_bit_attention_amd import peak
    r = peak.measure()
    return {
        "int8_TOPs": r["int8"] / 1e12,
        "bf16_TFLOPs": r["bf16"] / 1e12,
        "hbm_copy_GBs": r["hbm_copy"] / 1e9,
        "per_instruction_T": {k: v / 1e12 for k, v in r["mfma"].items()},
        "how": "MFMA-only kernels, 8 waves per SIMD, independent accumulator chains, best of 3 "
               "launches of ~25 ms; copy = torch device copy of 1 GiB (read + write bytes)",
        "issue_cycles_per_slot": peak.issue_table(),
        "operand_bytes_per_cycle_per_cu": peak.stream_table(),
        "issue_how": "shader-clock cycles (s_memtime) one SIMD takes per instruction slot: per "
                     "workgroup the span from the first wave's start to the last wave's end over "
                     "the slots run per SIMD (8 per round, 4000 rounds), 1 or 2 waves per SIMD "
                     "running the same mix, every compute unit; operand rates: 16-byte reads of "
                     "L1-resident global memory or of LDS by 4 or 8 waves per CU, bytes per "
                     "s_memtime cycle",
    }


def spread(ms):
    """p10, median and p90 of per-call times (ms)."""
    return [float(np.percentile(ms, 10)), float(np.median(ms)), float(np.percentile(ms, 90))]


def host_cpu():
    """CPU model (from /proc/cpuinfo) and the cores this process may use."""
    model = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def oracle_threads(nproc):
    # worker threads of the all-core runs: the host's cores, at most 16 (a
    # GPU's share of a shared host)
    return max(1, min(16, nproc))


def _oracle_head(wl, b, h, blocks, qk_int8, fine, barrier=None):
    """The oracle on head (b, h): selection, quantisation and linear states for
    the whole head, then the query blocks ``blocks`` (all when None).  Inputs
    are generated before the clock starts.  Returns (prep seconds, block
    seconds, thread CPU seconds)."""
    import oracle
    q, k, v = synth.head_inputs(wl, b, h)
    w = synth.proj_weight(wl)
    if barrier is not None:
        barrier.wait()
    c0, t0 = time.thread_time(), time.perf_counter()
    prep = oracle.head_prep(q, k, float(np.float32(wl.topk)), fine=fine)
    states = oracle.linear_states(k, v) if wl.use_linear else None
    t1 = time.perf_counter()
    if barrier is not None:
        barrier.wait()
        t1 = time.perf_counter()
    oracle.head_forward(q, k, v, w, float(np.float32(wl.topk)), use_linear=bool(wl.use_linear),
                        blocks=blocks, prep=prep, states=states, qk_int8=qk_int8, fine=fine)
    t2 = time.perf_counter()
    return t1 - t0, t2 - t1, time.thread_time() - c0


def _parallel(fn, jobs, threads):
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, jobs))


def oracle_full(wl, threads, qk_int8=True, fine=False, log_fn=log):
    """The oracle over the whole workload (every head, every query block) with
    the (b, h) loop split over ``threads`` threads: wall seconds and the sum
    of the threads' CPU seconds (the single-core time of the same work)."""
    t0 = time.perf_counter()
    heads = wl.heads()
    r = _parallel(lambda bh: _oracle_head(wl, bh[0], bh[1], None, qk_int8, fine), heads,
                  min(threads, len(heads)))
    wall = time.perf_counter() - t0
    cpu = sum(x[2] for x in r)
    log_fn(f"[cpu] {wl.name} in full: {wall:.1f}s wall on {min(threads, len(heads))} threads "
           f"(input generation included), {cpu:.1f} CPU-s")
    return {"heads": len(heads), "threads": min(threads, len(heads)),
            "wall_s_incl_input_generation": wall, "cpu_s": cpu,
            "ms_per_call_single_core": cpu * 1e3}


def cpu_baseline(wl, n_blocks, log_fn=log, qk_int8=True, fine=False, full=("tiny",)):
    """The oracle on the host's cores, on a bounded sample of the workload.

    Single core: head (0,0) with the process pinned to one core: its whole
    selection/quantisation and linear states plus n_blocks query blocks, the
    block time extrapolated to all T blocks.  All cores: the same sample on
    one head per thread (heads (0,0), (0,1), ...), the selection phase and the
    block phase each timed by wall clock between barriers; one round of
    ``threads`` heads is then extrapolated to all B*H heads.  Both reported as
    dense-equivalent TFLOP/s; the headline value is the all-core one.
    ``full``: workloads also run in full (all heads and blocks)."""
    import threading
    import oracle
    model, nproc = host_cpu()
    T = oracle.nblocks(wl.N)
    rng = np.random.default_rng(0)
    blocks = sorted(rng.choice(T, size=min(n_blocks, T), replace=False).tolist())
    dense = 4.0 * wl.B * wl.H * wl.N * wl.N * wl.d
    BH = wl.B * wl.H

    # single core, pinned
    prev = os.sched_getaffinity(0)
    core = min(prev)
    os.sched_setaffinity(0, {core})
    try:
        tp, tb, _ = _oracle_head(wl, 0, 0, blocks, qk_int8, fine)
    finally:
        os.sched_setaffinity(0, prev)
    head_s = tp + tb * T / len(blocks)
    log_fn(f"[cpu] one core: prep+states {tp:.2f}s, {len(blocks)} blocks {tb:.2f}s, "
           f"head extrapolated {head_s:.1f}s")

    # all cores
    threads = min(oracle_threads(nproc), BH)
    bar = threading.Barrier(threads, timeout=900)  # a failing worker breaks it instead of hanging the rest
    heads = wl.heads()[:threads]
    t0 = time.perf_counter()
    r = _parallel(lambda bh: _oracle_head(wl, bh[0], bh[1], blocks, qk_int8, fine, bar), heads,
                  threads)
    wall_prep = max(x[0] for x in r)
    wall_blocks = max(x[1] for x in r)
    round_s = wall_prep + wall_blocks * T / len(blocks)
    job_s = round_s * -(-BH // threads)
    log_fn(f"[cpu] {threads} threads: prep+states {wall_prep:.2f}s, {len(blocks)} blocks "
           f"{wall_blocks:.2f}s wall (total {time.perf_counter() - t0:.1f}s), "
           f"call extrapolated {job_s:.0f}s")

    res = {
        "value": dense / job_s / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{wl.name}: per head, selection, quantisation and linear states for the "
                   f"whole head plus {len(blocks)} of {T} query blocks (the same blocks on "
                   f"every head), block time extrapolated to the head; all cores: heads "
                   f"(0,0)..(0,{threads - 1}) on {threads} threads, one round extrapolated to "
                   f"{BH} heads ({-(-BH // threads)} rounds); one core: head (0,0) pinned to "
                   f"core {core}"),
        "host_cpu": model,
        "nproc": nproc,
        "ms_per_call_extrapolated": job_s * 1e3,
        "all_core": {"threads": threads, "prep_wall_s": wall_prep,
                     "blocks_wall_s": wall_blocks, "ms_per_call_extrapolated": job_s * 1e3},
        "single_core": {"value": dense / (head_s * BH) / 1e12, "core": core, "prep_s": tp,
                        "blocks_s": tb, "head_s_extrapolated": head_s,
                        "ms_per_call_extrapolated": head_s * BH * 1e3},
    }
    if full:
        res["full_runs"] = {name: oracle_full(synth.WORKLOADS[name], oracle_threads(nproc),
                                              qk_int8, fine, log_fn)
                            for name in full}
    return res


def input_sha256(**arrays):
    """SHA-256 of each input's bytes as generated on the host (bf16 bits,
    row-major), the form they are uploaded in."""
    return {k: hashlib.sha256(np.ascontiguousarray(a).data).hexdigest() for k, a in arrays.items()}


def bench_w8a8(args, dev):
    """One step = quantise the activations (block-128 INT8) + the block-scaled
    INT8 GEMM, weights quantised once beforehand (as a deployed layer keeps
    them).  Roofline: dense INT8 MFMA peak for the GEMM's 2*M*N*K ops."""
    import torch
    from sparse_bit_attention_amd import sla
    lw = synth.LINEAR_WORKLOADS[args.linear]
    log(f"[bench] generating {lw.name} inputs")
    x, w = synth.linear_inputs(lw)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    X, W = up(x), up(w)
    wq, sw = sla.quant_b128(W)
    xq = torch.empty((lw.M, lw.K), dtype=torch.int8, device=dev)
    sx = torch.empty(((lw.M + 127) // 128, lw.K // 128), dtype=torch.float32, device=dev)
    y = torch.empty((lw.M, lw.N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    import ctypes
    L = sla.lib()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        sla._check(L.sla_quant_b128(ctypes.c_void_p(X.data_ptr()), lw.M, lw.K,
                                    ctypes.c_void_p(xq.data_ptr()), ctypes.c_void_p(sx.data_ptr()),
                                    ctypes.c_void_p(stream.cuda_stream)), "sla_quant_b128")
        if ev is not None:
            ev[1].record(stream)
        sla.w8a8_gemm(xq, sx, wq, sw, out=y, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(events[s_])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    q_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    g_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    ops = 2.0 * lw.M * lw.N * lw.K
    log(f"[bench] ms/step {ms_step:.3f} (quantize X {q_ms:.3f}, gemm {g_ms:.3f})")
    mp = measured_peaks(args.no_peaks)
    res = {
        "metric": "W8A8 block-128 linear layer TOPS (INT8 MFMA), Wan-14B-720P projection shape",
        "value": ops / (ms_step * 1e-3) / 1e12,
        "unit": "TOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": lw.name, "M": lw.M, "N": lw.N, "K": lw.K, "block": 128},
        "stage_ms": {"sla_quant_b128(X)": q_ms, "sla_w8a8_gemm": g_ms},
        "ms_per_call_p10_median_p90": spread([e[0].elapsed_time(e[2]) for e in events]),
        "roofline": {"kernel": "k_w8a8_gemm", "bound": "mfma", "achieved": ops / (g_ms * 1e-3) / 1e12,
                     "peak": P_I8 / 1e12, "unit": "TOP/s",
                     "frac": ops / (g_ms * 1e-3) / P_I8, "traffic": None,
                     "peak_measured": mp and mp["int8_TOPs"],
                     "frac_of_measured": mp and ops / (g_ms * 1e-3) / 1e12 / mp["int8_TOPs"]},
        "measured_peaks": mp,
    }
    if args.cpu_blocks > 0:
        # the oracle on a sample: rows of one 128-row block against all N columns
        import oracle
        t1 = time.perf_counter()
        rxq, rsx = oracle.quant_b128(x[:128])
        rwq, rsw = oracle.quant_b128(w)
        t2 = time.perf_counter()
        nrow = min(args.cpu_blocks // 60 + 1, 4)
        oracle.w8a8_gemm(rxq[:nrow], rsx, rwq, rsw)
        t3 = time.perf_counter()
        sample_ops = 2.0 * nrow * lw.N * lw.K
        res["cpu_baseline"] = {
            "value": sample_ops / (t3 - t2) / 1e12, "unit": "TOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{nrow} rows x all {lw.N} columns of the GEMM ({t3 - t2:.1f}s; quantisation "
                      f"of 128 X rows and all of W {t2 - t1:.1f}s not counted), single thread"}
    print(json.dumps(res), flush=True)


def bwd_work(wl, T, kb):
    """MFMA flops the backward kernels execute per call (bf16): per kept pair
    seven 64x64xd products (S, dP and dQ in the query-block kernel; S, dP,
    dV and dK in the key-block kernel); with the linear branch, per query
    block four 64xdxd products (phi(Q) H, dO W, dnum H^T, phi(Q)^T dnum) plus
    one for dW, per key block two (dHb^T phi(K), dHb V), and per head the
    transposed marginal GEMM 2 T^2 F."""
    BH = wl.B * wl.H
    pairs = BH * T * kb
    flops = pairs * 7 * 2 * 64 * 64 * wl.d
    if wl.use_linear and kb < T:
        F = (wl.d * wl.d + wl.d + 127) // 128 * 128
        flops += BH * T * (5 + 2) * 2 * 64 * wl.d * wl.d + BH * 2.0 * T * T * F
    return flops


def bench_bwd(args, dev):
    """One step = the plain-SLA training pair on one batch: the forward of a
    backward plan (sla_quantize, sla_attention_fwd; bf16 QK^T) then
    sla_attention_bwd with a seeded output gradient.  value = backward
    dense-equivalent TFLOP/s (the FlashAttention convention: 2.5 x the
    forward's 4 B H N^2 d); the roofline is the whole backward call's
    executed MFMA flops against the dense bf16 peak."""
    import torch
    from sparse_bit_attention_amd import sla
    wl = synth.WORKLOADS[args.workload]
    log(f"[bench] generating {wl.name} inputs and the output gradient")
    q, k, v, w = synth.all_inputs(wl)
    do = synth.grad_output(wl)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    Q, K, V, W, dO = up(q), up(k), up(v), up(w), up(do)
    del q, k, v, do
    m = sla.SageSLA(wl.B, wl.H, wl.N, wl.d, wl.topk, use_linear=bool(wl.use_linear), device=dev,
                    qk_int8=False, backward=True)
    T, kb = m.plan.info.T, m.plan.info.kb
    Wp = W if wl.use_linear else None
    out = torch.empty_like(Q)
    dq, dk, dv = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    dw = torch.empty((wl.d, wl.d), dtype=torch.float32, device=dev) if wl.use_linear else None
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        m.quantize(Q, K, stream)
        m.attention(Q, K, V, Wp, out, stream)
        if ev is not None:
            ev[1].record(stream)
        m.backward(Q, K, V, Wp, dO, dq, dk, dv, dw, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(events[s_])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    log(f"[bench] ms/step {ms_step:.3f} (forward {f_ms:.3f}, backward {b_ms:.3f})")
    dense = 10.0 * wl.B * wl.H * wl.N * wl.N * wl.d
    flops = bwd_work(wl, T, kb)
    mp = measured_peaks(args.no_peaks)
    res = {
        "metric": "SLA backward (bf16 QK^T, block mask fixed), dense-equivalent TFLOP/s",
        "value": dense / (b_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s (dense-equivalent, 10 B H N^2 d per backward)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d, "block": 64,
                   "topk": wl.topk, "kb": kb, "use_linear": wl.use_linear},
        "stage_ms": {"forward (sla_quantize + sla_attention_fwd)": f_ms, "sla_attention_bwd": b_ms},
        "bwd_ms_p10_median_p90": spread([e[1].elapsed_time(e[2]) for e in events]),
        "roofline": {"kernel": "sla_attention_bwd (all backward kernels)", "bound": "mfma",
                     "achieved": flops / (b_ms * 1e-3) / 1e12, "peak": P_BF16 / 1e12,
                     "unit": "TFLOP/s", "frac": flops / (b_ms * 1e-3) / P_BF16, "traffic": None,
                     "peak_measured": mp and mp["bf16_TFLOPs"],
                     "frac_of_measured": mp and flops / (b_ms * 1e-3) / 1e12 / mp["bf16_TFLOPs"]},
        "measured_peaks": mp,
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan14b-720p", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--cpu-blocks", type=int, default=240,
                    help="query blocks per head the CPU oracle baseline computes (0 = skip)")
    ap.add_argument("--cpu-full", default="tiny,wan1.3b-480p",
                    help="workloads the CPU oracle also runs in full on all cores "
                         "(comma-separated; empty = none)")
    ap.add_argument("--qk", choices=("int8", "int8-fine", "bf16"), default="int8",
                    help="QK^T operands: int8 (SageSLA with one scale per 64-row block, the "
                         "default), int8-fine (one Q scale per 16 rows, one K scale per 4 "
                         "keys) or bf16 (plain SLA)")
    ap.add_argument("--op", choices=("sagesla", "w8a8", "bwd"), default="sagesla",
                    help="sagesla: the attention forward (default); w8a8: the W8A8 linear layer; "
                         "bwd: plain-SLA forward + backward (training pair)")
    ap.add_argument("--linear", default="wan14b-720p-qkv", choices=sorted(synth.LINEAR_WORKLOADS))
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured peaks (profiled runs: keeps their kernels out of the trace)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads shard across GPUs with no communication; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_bit_attention_amd import sla

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 5}))
        return

    if args.op == "w8a8":
        bench_w8a8(args, dev)
        return
    if args.op == "bwd":
        bench_bwd(args, dev)
        return

    wl = synth.WORKLOADS[args.workload]
    log(f"[bench] generating {wl.name} inputs")
    t0 = time.perf_counter()
    q, k, v, w = synth.all_inputs(wl)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    Q, K, V, W = up(q), up(k), up(v), up(w)
    sha = input_sha256(q=q, k=k, v=v, w=w)
    del q, k, v
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s")
    qk_int8 = args.qk != "bf16"
    fine = args.qk == "int8-fine"
    m = sla.SageSLA(wl.B, wl.H, wl.N, wl.d, wl.topk, use_linear=bool(wl.use_linear), device=dev,
                    qk_int8=qk_int8, qk_fine=fine)
    T, kb = m.plan.info.T, m.plan.info.kb
    out = torch.empty_like(Q)
    Wp = W if wl.use_linear else None
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        m.quantize(Q, K, stream)
        if ev is not None:
            ev[1].record(stream)
        m.prepare_kv(K, V, Wp, stream)
        if ev is not None:
            ev[2].record(stream)
        m.attend(Q, out, stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    st = np.array([[e[a].elapsed_time(e[a + 1]) for a in range(3)] for e in events])  # ms
    ms_step = wall * 1e3 / args.steps
    q_ms, kv_ms, at_ms = (float(np.mean(st[:, a])) for a in range(3))
    log(f"[bench] ms/step {ms_step:.3f} (quantize {q_ms:.3f}, prepare_kv {kv_ms:.3f}, "
        f"attend {at_ms:.3f})")

    dense = 4.0 * wl.B * wl.H * wl.N * wl.N * wl.d
    i8, bf, pairs = attn_work(wl, kb, T, qk_int8)
    # the MFMA roofline time of the kept-block work: int8 and bf16 share the units
    t_roof_kept = (pairs * 2 * 64 * 64 * wl.d) / (P_I8 if qk_int8 else P_BF16) + \
        (pairs * 2 * 64 * 64 * wl.d) / P_BF16
    t_roof_attn = i8 / P_I8 + bf / P_BF16
    blended_peak = (i8 + bf) / t_roof_attn
    achieved = (i8 + bf) / (at_ms * 1e-3)
    traffic = traffic_entry() if args.qk == "int8" else None
    mp = measured_peaks(args.no_peaks)
    blended_measured = t_roof_kept_m = None
    if mp:
        p_i8_m, p_bf_m = mp["int8_TOPs"] * 1e12, mp["bf16_TFLOPs"] * 1e12
        blended_measured = (i8 + bf) / (i8 / p_i8_m + bf / p_bf_m)
        t_roof_kept_m = (pairs * 2 * 64 * 64 * wl.d) / (p_i8_m if qk_int8 else p_bf_m) + \
            (pairs * 2 * 64 * 64 * wl.d) / p_bf_m

    res = {
        "metric": METRIC,
        "value": dense / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+bf16" if qk_int8 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d, "block": 64,
                   "topk": wl.topk, "kb": kb, "use_linear": wl.use_linear,
                   "qk": args.qk},
        "ms_per_call": ms_step,
        "stage_ms": {"sla_quantize": q_ms, "sla_prepare_kv": kv_ms, "sla_attend": at_ms},
        "ms_per_call_p10_median_p90": spread(st.sum(axis=1)),
        "attend_ms_p10_median_p90": spread(st[:, 2]),
        "pct_mfma_roofline_kept_blocks": 100.0 * t_roof_kept / (ms_step * 1e-3),
        "pct_mfma_roofline_kept_blocks_measured_peaks":
            mp and 100.0 * t_roof_kept_m / (ms_step * 1e-3),
        "roofline": {
            "kernel": "k_attn (sla_attend)",
            "bound": "mfma",
            "achieved": achieved / 1e12,
            "peak": blended_peak / 1e12,
            "unit": "TFLOP/s",
            "frac": achieved / blended_peak,
            "traffic": traffic,
            "peak_measured": mp and blended_measured / 1e12,
            "frac_of_measured": mp and achieved / blended_measured,
        },
        "measured_peaks": mp,
        "inputs_sha256": sha,
    }
    if args.cpu_blocks > 0:
        log("[bench] CPU oracle baseline")
        full = tuple(x for x in args.cpu_full.split(",") if x)
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_blocks, qk_int8=qk_int8, fine=fine,
                                           full=full)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
