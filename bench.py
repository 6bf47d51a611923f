#!/usr/bin/env python3
"""Benchmark of the packed binary low-rank linear forward on one MI355X.

Default workload: Llama-2-70B-shaped decode, 80 blocks x {q, k, v, o, gate, up,
down} linears at 0.8 bits/weight (ranks from the storage rule r(m+n) bits +
16-bit scales), batch 1, bf16 activations and outputs, fp16 scales.  Every layer
has its own seeded random signs and scales (no attention, norm or embedding
between the linears).  One step = the 80 blocks in order, each as its four
shared-input groups q+k+v, o, gate+up, down (nq_linear_fwd_group: two launches
per group), each finished before the next starts, captured once as a HIP graph
and replayed; the same layers run one linear at a time (560 linears) are timed
too, for comparison (`unfused_chain`; --unfused makes that the headline).

Prints one JSON line.  `value` is algorithmic GB/s over the whole step: per
linear r(m+n)/8 sign bytes + 2(m+n+r) scale bytes + 2Bm y bytes, plus 2Bn x
bytes per group.  `roofline` is for the dominant kernel (largest share of the
step), timed with HIP events around each of its launches on the stream it runs
on.  After the timed region one layer of every distinct shape of block 0 is
checked against the fp64 oracle on the host (`parity`).  Further sections of
the same line: `read_probe` (achievable read rates), `prefill` (2048-token
GEMMs, MFMA utilisation), `initializer` (one ADMM step on a 7B shape),
`variants` (transposed product and rank-l envelope on a 70B shape) and
`cpu_baseline` (the fp64 oracle on the host cores).

  python bench.py [--steps K --warmup W]           70B decode chain (the metric)
  python bench.py --batch B                        the same chain at batch B (B > 4 in passes of four rows)
  python bench.py --suite 7b --out FILE            7B shapes, B in {1,2,4,8,16}, 0.55/0.8/1.0 bpw:
                                                   per-shape GB/s over >= 1 GiB of rotating layer copies
  python bench.py --initializer-only | --variants-only
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode70b_traffic.json")
DEC_SOURCE = os.path.join(ROOT, "binary_rank_gemv_packed_amd", "csrc", "nq_dec.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--bpw", type=float, default=0.8)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "gemv", "valu"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true", help="time the 560 linears one by one (no layer groups)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 2048-token prefill section")
    ap.add_argument("--no-initializer", action="store_true", help="skip the ADMM initialiser section")
    ap.add_argument("--no-variants", action="store_true", help="skip the transposed / envelope section")
    ap.add_argument("--variants-only", action="store_true", help="run only the transposed / envelope section")
    ap.add_argument("--initializer-only", action="store_true", help="run only the ADMM initialiser section")
    ap.add_argument("--prefill-only", action="store_true", help="run only the 2048-token prefill section")
    ap.add_argument("--suite", default=None, choices=["7b"])
    ap.add_argument("--out", default=None)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the known-size elementwise kernel used to scale HBM counters")
    ap.add_argument("--rocprof-summary", metavar="DIR", default=None,
                    help="print per-kernel tables from rocprofv3 csv output under DIR (no GPU)")
    ap.add_argument("--make-traffic-file", nargs=5, metavar=("BENCH_JSON", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    default=None, help="write the dominant kernel's counter traffic from --pmc csv dirs (no GPU)")
    return ap.parse_args()


# ------------------------------------------------------------------ helpers
def hip_runtime():
    """The HIP runtime library already loaded in this process (the one torch and
    libnq share), for raw event handles."""
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                lib = ctypes.CDLL(line.split()[-1])
                lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
                lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
                lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
                lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
                lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
                lib.hipEventQuery.argtypes = [ctypes.c_void_p]
                return lib
    raise RuntimeError("libamdhip64 is not loaded")


class Events:
    # hipEventDisableSystemFence: an event only for timing, recorded without the
    # system-scope cache write-back and invalidate that would slow the next kernel
    TIMING_ONLY = 0x20000000

    def __init__(self, hip, n, flags=0):
        self.hip = hip
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert hip.hipEventCreateWithFlags(ctypes.byref(h), flags) == 0
            self.ev.append(h.value)

    def ms(self, i, j):
        f = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(f), self.ev[i], self.ev[j]) == 0
        return f.value

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)


def alg_bytes(m, n, r, B, xb=2, yb=2, sb=2):
    return r * (m + n) / 8 + sb * (m + n + r) + B * n * xb + B * m * yb


def cpu_info():
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def chain_spec(shapes, nblocks, bpw):
    import binary_rank_gemv_packed_amd as nq
    import synth
    out = []
    for b in range(nblocks):
        for li, name in enumerate(synth.LAYER_ORDER):
            m, n = shapes[name]
            out.append((b, li, name, m, n, nq.rank_for_bits(m, n, bpw, 16)))
    return out


def make_layer_gpu(m, n, r, B, seed, dev, keep=False):
    """Seeded random layer generated on the GPU (torch generator), packed by the
    library.  With keep, also returns host copies of its inputs."""
    import torch
    import binary_rank_gemv_packed_amd as nq
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    U = (torch.randint(0, 2, (m, r), generator=g, device=dev, dtype=torch.int8) * 2 - 1).to(torch.int8)
    V = (torch.randint(0, 2, (n, r), generator=g, device=dev, dtype=torch.int8) * 2 - 1).to(torch.int8)
    s1 = (torch.randn(m, generator=g, device=dev).abs() + 0.1).half()
    gg = (torch.randn(r, generator=g, device=dev).abs() + 0.1).half()
    s2 = (torch.randn(n, generator=g, device=dev).abs() + 0.1).half()
    x = torch.randn(B, n, generator=g, device=dev).to(torch.bfloat16)
    layer = nq.pack(U, V, s1, gg, s2)
    host = None
    if keep:
        host = dict(U=U.cpu().numpy(), V=V.cpu().numpy(), s1=s1.cpu().numpy(), g=gg.cpu().numpy(),
                    s2=s2.cpu().numpy(), x=x.float().cpu().numpy())
    del U, V
    return layer, x, host


def oracle_check(host, y):
    """Relative L2 of a bf16 output against the fp64 factored oracle, and the
    error that rounding the exact result to bf16 alone costs."""
    import numpy as np
    import synth
    from oracle import nq_oracle as O
    f64 = lambda a: np.asarray(a, np.float64)
    ref = O.linear_factored(f64(host["x"]), host["U"], host["V"], f64(host["s1"]), f64(host["g"]), f64(host["s2"]))
    yy = np.asarray(y, np.float64)
    rr = synth.round_to_bf16(ref.astype(np.float32)).astype(np.float64)
    nrm = np.linalg.norm(ref)
    return float(np.linalg.norm(yy - ref) / nrm), float(np.linalg.norm(rr - ref) / nrm)


def cpu_baseline(spec, B):
    """The fp64 oracle (factored mode, as it stands) on block 0's seven linears,
    median of 3 runs, on every host core this process may use; scaled to the 80
    blocks of the chain."""
    import numpy as np
    import synth
    from oracle import nq_oracle as O
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:
        limiter = None
    block0 = [s for s in spec if s[0] == 0]
    nblocks = len({s[0] for s in spec})
    layers = [synth.make_layer(m, n, r, B, cfg=4, block=blk, layer=li) for (blk, li, name, m, n, r) in block0]
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        for L in layers:
            O.linear_factored(L.x.astype(np.float64), L.U, L.V, L.s1.astype(np.float64), L.g.astype(np.float64),
                              L.s2.astype(np.float64))
        runs.append(time.perf_counter() - t0)
    t_block = statistics.median(runs)
    block_bytes = sum(alg_bytes(m, n, r, B) for (_, _, _, m, n, r) in block0)
    if limiter is not None:
        limiter.unregister()
    return {"value": round(block_bytes / t_block / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": (f"factored fp64 oracle on block 0's 7 linears (B={B}), median of 3 runs "
                       f"({', '.join(f'{t:.2f}' for t in runs)} s), scaled x{nblocks} blocks; {cpu_info()}"),
            "tokens_per_s": round(B / (t_block * nblocks), 4)}


def traffic_entry():
    """Counter-backed HBM traffic of the dominant kernel from the committed
    profile summary, if it was taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    with open(DEC_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    if t.get("source_sha") != sha:
        log(f"[bench] {TRAFFIC_FILE} was taken on another kernel source; traffic = null")
        return None
    return t


KERNEL_NAMES = {2: ["stage1", "stage2"], 3: ["stage1", "mid", "stage2"]}
# the linears of a block that read the same input, in block order
GROUPS = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")), ("down", ("down",)))


def make_units(spec, fused):
    """The chain as a list of (name, [linear indices]) in step order: every
    linear alone, or the shared-input groups of each block."""
    if not fused:
        return [(s[2], [i]) for i, s in enumerate(spec)]
    units = []
    by_block = {}
    for i, s in enumerate(spec):
        by_block.setdefault(s[0], {})[s[2]] = i
    for blk in sorted(by_block):
        for gname, members in GROUPS:
            units.append((gname, [by_block[blk][nm] for nm in members]))
    return units


def unit_call(nq, units, layers, xs, ys, ws, path):
    """Launches of one pass over the units (x of a group = x of its first linear)."""
    def step():
        for _, idx in units:
            if len(idx) == 1:
                nq.linear_into(xs[idx[0]], layers[idx[0]], ys[idx[0]], ws, path)
            else:
                nq.linear_group_into(xs[idx[0]], [layers[i] for i in idx], [ys[i] for i in idx], ws)
    return step


def unit_alg_bytes(kind, spec, idx, B):
    """Algorithmic bytes of one kernel of a unit (x read once per unit): stage 1
    reads x, s2 and packed V^T; stage 2 packed U, s1 and g and writes y."""
    n = spec[idx[0]][4]
    if kind == "stage1":
        return 2 * B * n + sum(spec[i][5] * n / 8 + 2 * n for i in idx)
    if kind == "mid":
        return 0.0
    return sum(spec[i][5] * spec[i][3] / 8 + 2 * (spec[i][3] + spec[i][5]) + 2 * B * spec[i][3] for i in idx)


def kernel_durations(nq, stream, units, layers, xs, ys, ws, path, hold_cycles=100_000_000):
    """Duration of every kernel of one eager pass over the whole chain: HIP
    events recorded on `stream` before each launch and after the last one.

    The stream is first held by a GPU spin of hold_cycles clock ticks (40 ms at
    2.4 GHz) so that the host can queue the whole pass before it runs; then the
    kernels run back to back as in the graph and no host launch latency leaks
    into the gaps between events.  Returns {"unit.kernel": [ms per launch]},
    {"unit.kernel": (workgroups, threads)} and whether the spin was still
    running when the last unit had been queued."""
    import torch
    hip = hip_runtime()
    EV = 4
    ev = Events(hip, EV * len(units) + 1, Events.TIMING_ONLY)
    lib = nq.lib()
    st = stream.cuda_stream
    pth = nq.PATHS[path]
    calls = []
    for u, (name, idx) in enumerate(units):
        arr = (ctypes.c_void_p * EV)(*ev.ev[EV * u:EV * u + EV])
        dims = (ctypes.c_int32 * (2 * EV))()
        nl = ctypes.c_int32(0)
        x = xs[idx[0]]
        if len(idx) == 1:
            L, y = layers[idx[0]], ys[idx[0]]
            args = (L.ref, x.data_ptr(), nq._DT[x.dtype], y.data_ptr(), nq._DT[y.dtype], x.shape[0],
                    ws.data_ptr(), ws.numel(), st, pth, ctypes.cast(arr, ctypes.c_void_p), EV, ctypes.byref(nl),
                    ctypes.cast(dims, ctypes.c_void_p))
            calls.append((lib.nq_linear_fwd_profiled, args, (arr, dims, nl)))
        else:
            refs, yp = nq._group_arrays([layers[i] for i in idx], [ys[i] for i in idx])
            args = (ctypes.cast(refs, ctypes.c_void_p), len(idx), x.data_ptr(), nq._DT[x.dtype],
                    ctypes.cast(yp, ctypes.c_void_p), nq._DT[ys[idx[0]].dtype], x.shape[0], ws.data_ptr(),
                    ws.numel(), st, ctypes.cast(arr, ctypes.c_void_p), EV, ctypes.byref(nl),
                    ctypes.cast(dims, ctypes.c_void_p))
            calls.append((lib.nq_linear_fwd_group_profiled, args, (arr, dims, nl, refs, yp)))
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(hold_cycles)
        hip.hipEventRecord(ctypes.c_void_p(ev.ev[-1]), ctypes.c_void_p(st))
        for fn, args, _ in calls:
            status = fn(*args)
            if status != 0:
                raise nq.NQError(status, lib.nq_last_error().decode())
        held = hip.hipEventQuery(ctypes.c_void_p(ev.ev[-1])) != 0  # not yet reached: still spinning
    torch.cuda.synchronize()
    per_key, dims_of = {}, {}
    for u, (fn, args, keep) in enumerate(calls):
        dims, nl = keep[1], keep[2].value
        for j, kn in enumerate(KERNEL_NAMES[nl]):
            key = f"{units[u][0]}.{kn}"
            per_key.setdefault(key, []).append(ev.ms(EV * u + j, EV * u + j + 1))
            dims_of[key] = (dims[2 * j], dims[2 * j + 1])
    ev.close()
    return per_key, dims_of, held


# ------------------------------------------------------------------ 70B decode chain
def time_graph(torch, stream, step, warmup, steps):
    """Captures one step as a HIP graph and times `steps` replays on `stream`
    with events on that stream; returns (ms per step, wall ms per step)."""
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(steps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    return e0.elapsed_time(e1) / steps, wall * 1e3 / steps


def read_probe(dev, one_shot_bytes, gib=4, reps=5, launches=48, hold_cycles=50_000_000):
    """Achievable HBM read rates from the library's read probe (sixteen 1 KiB
    loads in flight per wave, as in the decode kernels' weight stream):
    `stream` reads `gib` GiB in one launch (best of `reps`); `one_shot` reads
    `one_shot_bytes` (rounded up to 16 KiB) per launch, `launches` launches back
    to back on a held stream, each from another region of a buffer far larger
    than the caches, timed like the decode kernels (event interval per
    launch, dispatch gap included)."""
    import torch
    import binary_rank_gemv_packed_amd as nq
    stream = torch.cuda.Stream(device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    buf = torch.ones(gib << 28, dtype=torch.int32, device=dev)
    best = None
    with torch.cuda.stream(stream):
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            nq.read_probe(buf, sink, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3
            best = t if best is None or t < best else best
    out = {"stream": {"bytes": gib << 30, "gbs": round((gib << 30) / best / 1e9, 1)}}
    words = -(-one_shot_bytes // 16384) * 4096  # int32 words per region
    regions = buf.numel() // words
    with torch.cuda.stream(stream):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(hold_cycles)
        e0.record(stream)
        for k in range(launches):
            r = k % regions
            grid = nq.read_probe(buf[r * words:(r + 1) * words], sink, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    out["one_shot"] = {"bytes": words * 4, "us": round(us, 3), "gbs": round(words * 4 / us / 1e3, 1),
                       "launch": {"workgroups": grid[0], "threads": grid[1]}, "regions": int(regions)}
    out["how"] = "nq_read_probe: 16 x 1 KiB loads in flight per wave, XOR of the words"
    del buf
    torch.cuda.empty_cache()
    return out


MFMA_PEAK_FP16_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA


def run_prefill70b(dev, tokens=2048, bpw=0.8, reps=5):
    """One 70B block's distinct linear shapes at `tokens` rows (the prefill
    path: fp16 MFMA GEMMs with exact +-1 operands), each timed per kernel with
    HIP events on its stream; MFMA utilisation = 2 B r (m + n) / (t x peak).
    Eight sampled output rows per shape are checked against the fp64 oracle."""
    import numpy as np
    import torch
    import binary_rank_gemv_packed_amd as nq
    import synth
    from oracle import nq_oracle as O
    hip = hip_runtime()
    stream = torch.cuda.Stream()
    out, block_s, block_flops = {}, 0.0, 0.0
    for name in ("q", "k", "gate", "down"):
        m, n = synth.LLAMA70B[name]
        r = nq.rank_for_bits(m, n, bpw, 16)
        layer, x, host = make_layer_gpu(m, n, r, tokens, 777 + m + 3 * n, dev, keep=True)
        y = torch.empty(tokens, m, device=dev, dtype=torch.bfloat16)
        ws = torch.empty(nq.workspace_bytes(layer, tokens, "gemm"), dtype=torch.uint8, device=dev)
        ev = Events(hip, 8 * reps)
        with torch.cuda.stream(stream):
            nq.linear_into(x, layer, y, ws, "gemm")
            launches = []
            for k in range(reps):
                launches = nq.linear_into_profiled(x, layer, y, ws, ev.ev[8 * k:8 * k + 8], "gemm")
        torch.cuda.synchronize()
        nk = len(launches)
        per = [statistics.mean(ev.ms(8 * k + j, 8 * k + j + 1) for k in range(reps)) for j in range(nk)]
        total = statistics.mean(ev.ms(8 * k, 8 * k + nk) for k in range(reps))
        ev.close()
        flops = 2.0 * tokens * r * (m + n)
        f1, f2 = 2.0 * tokens * r * n, 2.0 * tokens * r * m
        rows = np.linspace(0, tokens - 1, 8).astype(int)
        yy = y[rows].float().cpu().numpy()
        f64 = lambda a: np.asarray(a, np.float64)
        ref = O.linear_factored(f64(host["x"][rows]), host["U"], host["V"], f64(host["s1"]), f64(host["g"]),
                                f64(host["s2"]))
        rr = synth.round_to_bf16(ref.astype(np.float32)).astype(np.float64)
        e = float(np.linalg.norm(yy - ref) / np.linalg.norm(ref))
        er = float(np.linalg.norm(rr - ref) / np.linalg.norm(ref))
        out[name] = {"m": m, "n": n, "r": r, "ms": round(total, 4), "tflops": round(flops / (total * 1e-3) / 1e12, 1),
                     "mfma_util": round(flops / (total * 1e-3) / 1e12 / MFMA_PEAK_FP16_TFLOPS, 4),
                     "gemm_xv_ms": round(per[1], 4), "gemm_xv_util": round(f1 / (per[1] * 1e-3) / 1e12 /
                                                                           MFMA_PEAK_FP16_TFLOPS, 4),
                     "gemm_tu_ms": round(per[3], 4), "gemm_tu_util": round(f2 / (per[3] * 1e-3) / 1e12 /
                                                                           MFMA_PEAK_FP16_TFLOPS, 4),
                     "prep_ms": round(per[0], 4), "mid_ms": round(per[2], 4),
                     "sampled_rows_rel_l2": float(f"{e:.3e}"), "bf16_rounding_rel_l2": float(f"{er:.3e}"),
                     "ok": bool(e <= 2e-3 + er)}
        c = {"q": 2, "k": 2, "gate": 2, "down": 1}[name]  # q~o, k~v, gate~up
        block_s += c * total * 1e-3
        block_flops += c * flops
        log(f"[bench] prefill {name}: {total:.3f} ms, {out[name]['tflops']} TFLOP/s, "
            f"MFMA util {out[name]['mfma_util']:.3f}, sampled rows rel L2 {e:.2e}")
        del layer, x, y, ws, host
        torch.cuda.empty_cache()
    return {"workload": f"llama2-70b block linears at {tokens} tokens, {bpw} bpw, bf16 x and y, fp16 scales",
            "per_shape": out, "block_ms": round(block_s * 1e3, 3),
            "block_tflops": round(block_flops / block_s / 1e12, 1),
            "mfma_util": round(block_flops / block_s / 1e12 / MFMA_PEAK_FP16_TFLOPS, 4),
            "peak_tflops": MFMA_PEAK_FP16_TFLOPS, "tokens_per_s": round(tokens / (block_s * 80), 1)}


def run_decode70b(args):
    import torch
    import binary_rank_gemv_packed_amd as nq
    import synth

    dev = "cuda:0"
    B = args.batch
    spec = chain_spec(synth.LLAMA70B, 80, args.bpw)
    fused = not args.unfused and args.path == "auto"
    check_ids = {0: "q", 1: "k", 4: "gate", 6: "down"}  # one linear per distinct shape of block 0
    layers, xs, ys, hosts = [], [], [], {}
    t0 = time.time()
    for i, (blk, li, name, m, n, r) in enumerate(spec):
        keep = blk == 0 and li in check_ids
        layer, x, host = make_layer_gpu(m, n, r, B, 20260206 * 1000003 + 4 * 100003 + blk * 101 + li, dev, keep)
        layers.append(layer)
        xs.append(x)
        ys.append(torch.empty(B, m, device=dev, dtype=torch.bfloat16))
        if keep:
            hosts[i] = host
    log(f"[bench] generated and packed {len(spec)} layers in {time.time() - t0:.1f}s")
    units = make_units(spec, fused)
    ws_bytes = max(nq.workspace_bytes(L, B, args.path) for L in layers)
    for _, idx in units:
        if len(idx) > 1:
            ws_bytes = max(ws_bytes, nq.workspace_bytes_group([layers[i] for i in idx], B))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()

    ms, wall = time_graph(torch, stream, unit_call(nq, units, layers, xs, ys, ws, args.path), args.warmup,
                          args.steps)
    log(f"[bench] {'fused' if fused else 'unfused'} chain, {len(units)} units, {args.steps} steps: "
        f"{ms:.4f} ms/step (events), wall {wall:.4f} ms/step")
    step_bytes = sum(unit_alg_bytes("stage1", spec, idx, B) + unit_alg_bytes("stage2", spec, idx, B)
                     for _, idx in units)
    gbs = step_bytes / (ms * 1e-3) / 1e9

    # parity of the timed chain's own outputs (last replay), one linear per
    # distinct shape; a group member's input is its group's (first linear's) x
    leader = {i: idx[0] for _, idx in units for i in idx}
    parity = {}
    for i, host in hosts.items():
        if leader[i] != i:
            host = dict(host, x=xs[leader[i]].float().cpu().numpy())
        e, er = oracle_check(host, ys[i].float().cpu().numpy())
        name = spec[i][2]
        parity[name] = {"rel_l2": float(f"{e:.3e}"), "bf16_rounding_rel_l2": float(f"{er:.3e}"),
                        "ok": bool(e <= 2e-3 + er)}
        log(f"[bench] parity {name}: rel L2 {e:.3e} (bf16 rounding alone {er:.3e})")

    unfused_ms = None
    if fused:  # the per-linear chain on the same layers, for comparison
        unfused_ms, _ = time_graph(torch, stream, unit_call(nq, make_units(spec, False), layers, xs, ys, ws,
                                                            args.path), args.warmup, args.steps)
        log(f"[bench] unfused chain (560 linears one by one): {unfused_ms:.4f} ms/step")

    # per-kernel durations: HIP events around every launch of one more pass over
    # the whole chain, on the stream the graph ran on (see kernel_durations)
    kernels = {}
    roof = None
    per_key = None
    if args.path in ("auto", "decode") and B <= 4:
        try:
            per_key, dims_of, held = kernel_durations(nq, stream, units, layers, xs, ys, ws, args.path)
            log(f"[bench] per-kernel pass: GPU held until all {len(units)} units were queued: {held}")
        except nq.NQError as e:  # a group without a fused plan at this batch runs its layers one by one
            torch.cuda.synchronize()
            log(f"[bench] no per-kernel timing at B={B}: {e}")
    if per_key is not None:
        unit_idx = {name: idx for name, idx in units}
        best = None
        for key, durs in per_key.items():
            uname, kn = key.split(".")
            d = statistics.mean(durs)
            byts = unit_alg_bytes(kn, spec, unit_idx[uname], B)
            kernels[key] = {"us": round(d * 1e3, 3), "alg_bytes": int(byts), "gbs": round(byts / (d * 1e-3) / 1e9, 1),
                            "per_step": len(durs), "workgroups": dims_of[key][0], "threads": dims_of[key][1]}
            share = d * len(durs)
            if best is None or share > best[0]:
                best = (share, key, byts, d)
        _, key, byts, d = best
        achieved = byts / (d * 1e-3) / 1e9
        tr = traffic_entry()
        traffic = None
        if tr is not None and tr.get("kernel") == key:
            traffic = int(tr["traffic_bytes"])
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": key,
                "us_per_launch": round(d * 1e3, 3), "alg_bytes_per_launch": int(byts),
                "launch": {"workgroups": dims_of[key][0], "threads": dims_of[key][1]}}
        log(f"[bench] dominant kernel {key}: {d * 1e3:.2f} us/launch, {achieved:.1f} GB/s "
            f"({dims_of[key][0]} workgroups x {dims_of[key][1]} threads)")

    out = {
        "metric": "binary low-rank GEMV GB/s (% HBM peak) + tokens/s, 70B-shaped layers, B=1",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4xfp8-f32acc",
        "data": "synthetic",
        "tokens_per_s": round(B / (ms * 1e-3), 2),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "config": {
            "workload": "llama2-70b-shaped decode linears: 80 blocks x q,k,v,o,gate,up,down at 0.8 bpw, B=1",
            "blocks": 80, "linears_per_block": 7, "batch": B, "bits_per_weight": args.bpw,
            "ranks": {s[2]: s[5] for s in spec[:7]}, "x_dtype": "bf16", "y_dtype": "bf16", "scale_dtype": "fp16",
            "path": args.path, "graph": True, "bytes_per_step": int(step_bytes),
            "chain": ("fused groups per block: q+k+v, o, gate+up, down (2 launches each)" if fused else
                      "560 linears one by one"),
        },
        "parity": parity,
        "kernels": kernels,
    }
    if unfused_ms is not None:
        out["unfused_chain"] = {"ms_per_step": round(unfused_ms, 5), "tokens_per_s": round(B / (unfused_ms * 1e-3), 2),
                                "speedup_of_fused": round(unfused_ms / ms, 3)}
    if roof is not None:
        out["roofline"] = roof
    if not args.no_prefill:
        del layers, xs, ys, ws
        torch.cuda.empty_cache()
        one = roof["alg_bytes_per_launch"] if roof is not None else 36 << 20
        rp = out["read_probe"] = read_probe(dev, one)
        log(f"[bench] read probe: {rp['stream']['gbs']} GB/s over {rp['stream']['bytes'] >> 30} GiB; "
            f"{rp['one_shot']['bytes'] / 1e6:.2f} MB per launch: {rp['one_shot']['us']} us, "
            f"{rp['one_shot']['gbs']} GB/s ({rp['one_shot']['launch']['workgroups']} workgroups)")
        out["prefill"] = run_prefill70b(dev)
    if not args.no_initializer:
        out["initializer"] = run_initializer(dev)
    if not args.no_variants:
        out["variants"] = run_variants(dev)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline(spec, B)
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ initialiser (ADMM)
FP32_MFMA_PEAK_TFLOPS = 157.3


def run_initializer(dev, m=4096, n=4096, bpw=0.8, power_iters=8, rho=10.0):
    """ADMM initialiser (nq_admm_factorize) on a Llama-2-7B q-projection shape
    at 0.8 bits/weight: time per ADMM step = (time of 2 steps - time of 0
    steps) / 2, HIP events on the launch stream, median of 3.  Flops per step:
    the four products W B, W^T A, T Ginv (twice) and the two Gram matrices,
    4 m n r + 4 (m + n) r^2, plus 2 r^3 per Gauss-Jordan inverse (two per
    step); utilisation against the fp32 matrix peak.  Inputs: W ~ N(0, 1/n)
    and latent starts ~ N(0, 1), seeded (torch generator)."""
    import torch
    import binary_rank_gemv_packed_amd as nq
    hip = hip_runtime()
    r = nq.rank_for_bits(m, n, bpw, 16)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260206)
    W = torch.randn(m, n, generator=gen, device=dev) / (n ** 0.5)
    A0 = torch.randn(m, r, generator=gen, device=dev)
    B0 = torch.randn(n, r, generator=gen, device=dev)
    stream = torch.cuda.Stream()
    ev = Events(hip, 2)

    def timed(iters):
        with torch.cuda.stream(stream):
            hip.hipEventRecord(ctypes.c_void_p(ev.ev[0]), ctypes.c_void_p(stream.cuda_stream))
            res = nq.admm_factorize(W, A0, B0, rho, iters, power_iters, with_err=False, stream=stream)
            hip.hipEventRecord(ctypes.c_void_p(ev.ev[1]), ctypes.c_void_p(stream.cuda_stream))
        torch.cuda.synchronize()
        return ev.ms(0, 1), res

    timed(1)
    t0 = statistics.median(timed(0)[0] for _ in range(3))
    t2 = statistics.median(timed(2)[0] for _ in range(3))
    ev.close()
    per = (t2 - t0) / 2
    gemm_flops = 4.0 * m * n * r + 4.0 * (m + n) * r * r
    inv_flops = 2 * 2.0 * r ** 3
    tf = (gemm_flops + inv_flops) / (per * 1e-3) / 1e12
    log(f"[bench] initializer {m}x{n} r={r}: {per:.2f} ms per ADMM step, {tf:.1f} TFLOP/s")
    return {"workload": f"ADMM initialiser, llama2-7b q-projection shape {m}x{n}, r={r} (0.8 bpw), fp32",
            "m": m, "n": n, "r": r, "rho": rho, "power_iters": power_iters,
            "ms_per_step": round(per, 3), "ms_setup_and_projection": round(t0, 3),
            "flops_per_step": gemm_flops + inv_flops, "tflops": round(tf, 2),
            "mfma_util_fp32": round(tf / FP32_MFMA_PEAK_TFLOPS, 4), "peak_tflops": FP32_MFMA_PEAK_TFLOPS}


# ------------------------------------------------------------------ transposed product and envelope
def run_variants(dev, copies=6, calls=48, bpw=0.8):
    """One 70B gate-projection shape (28672 x 8192 at 0.8 bpw), B = 1, single
    linears captured as a HIP graph of `calls` calls rotating over `copies`
    layers (141 MB, beyond the caches): the forward y = x W_hat^T, the
    transposed product dx = dy W_hat on the bit-transposed layer, and the rank-l
    envelope forward for l = 2 and 4.  GB/s = algorithmic bytes per call
    (sign bits, scales incl. the l envelope pairs, x, y) / time per call."""
    import torch
    import binary_rank_gemv_packed_amd as nq
    m, n = 28672, 8192
    r = nq.rank_for_bits(m, n, bpw, 16)
    layers = [make_layer_gpu(m, n, r, 1, 900 + c, dev)[0] for c in range(copies)]
    tlayers = [nq.transpose(L) for L in layers]
    g = torch.Generator(device=dev)
    g.manual_seed(20260206)
    x = torch.randn(1, n, generator=g, device=dev).to(torch.bfloat16)
    dy = torch.randn(1, m, generator=g, device=dev).to(torch.bfloat16)
    s1e = (torch.randn(4, m, generator=g, device=dev).abs() + 0.1).half()
    s2e = (torch.randn(4, n, generator=g, device=dev).abs() + 0.1).half()
    stream = torch.cuda.Stream()
    out = {"workload": f"llama2-70b gate shape {m}x{n}, r={r} (0.8 bpw), B=1, bf16, {copies} rotating copies"}

    def measure(name, fn, bytes_per_call):
        def step():
            for k in range(calls):
                fn(k % copies)
        ms, _ = time_graph(torch, stream, step, 3, 10)
        us = ms * 1e3 / calls
        out[name] = {"us_per_call": round(us, 3), "gbs": round(bytes_per_call / us / 1e3, 1)}
        log(f"[bench] {name}: {us:.2f} us per call, {out[name]['gbs']} GB/s")

    base = r * (m + n) / 8 + 2 * r
    measure("forward", lambda c: nq.linear(x, layers[c]), base + 2 * (m + n) + 2 * n + 2 * m)
    measure("transposed", lambda c: nq.linear(dy, tlayers[c]), base + 2 * (m + n) + 2 * m + 2 * n)
    for env in (2, 3, 4):
        try:
            measure(f"envelope_l{env}", lambda c, e=env: nq.linear_envelope(x, layers[c], s1e[:e], s2e[:e]),
                    base + 2 * env * (m + n) + 2 * n + 2 * m)
        except nq.NQError as e:  # the envelope's t' image for env terms must fit the workgroup's LDS
            torch.cuda.synchronize()
            out[f"envelope_l{env}"] = {"unsupported": str(e)}
            log(f"[bench] envelope_l{env}: {e}")
    del layers, tlayers
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ 7B per-shape suite
def run_suite7b(args):
    import torch
    import binary_rank_gemv_packed_amd as nq
    import synth

    dev = "cuda:0"
    rows = []
    shapes = [("q", 4096, 4096), ("gate", 11008, 4096), ("down", 4096, 11008)]
    for bpw in (1.0, 0.8, 0.55):
        for (name, m, n) in shapes:
            r = nq.rank_for_bits(m, n, bpw, 16)
            base, _, _ = make_layer_gpu(m, n, r, 16, 777 + m + n + r, dev)
            lb = base.blob.numel()
            copies = max(8, (1 << 30) // lb + 1)  # >= 1 GiB of distinct layer memory
            blobs = [base.blob.clone() for _ in range(copies)]
            layers = [nq.Layer(m, n, r, torch.float16, bl) for bl in blobs]
            for B in (1, 2, 4, 8, 16):
                if bpw != 0.8 and B != 1 and not (bpw == 0.55):
                    continue
                x = torch.randn(copies, B, n, device=dev).to(torch.bfloat16)
                y = torch.empty(copies, B, m, device=dev, dtype=torch.bfloat16)
                ws = torch.empty(max(nq.workspace_bytes(layers[0], B), 256), dtype=torch.uint8, device=dev)
                stream = torch.cuda.Stream()

                def step():
                    for i in range(copies):
                        nq.linear_into(x[i], layers[i], y[i], ws)

                with torch.cuda.stream(stream):
                    step()
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=stream):
                    step()
                with torch.cuda.stream(stream):
                    graph.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with torch.cuda.stream(stream):
                    e0.record(stream)
                    for _ in range(3):
                        graph.replay()
                    e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (3 * copies)
                byts = alg_bytes(m, n, r, B)
                row = {"config": 2 if bpw == 1.0 else 3, "shape": name, "m": m, "n": n, "r": r, "bpw": bpw, "B": B,
                       "us_per_call": round(us, 3), "alg_bytes": int(byts),
                       "gbs": round(byts / (us * 1e-6) / 1e9, 1),
                       "pct_hbm_peak": round(100 * byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                       "tokens_per_s_per_layer": round(B / (us * 1e-6), 1), "rotating_copies": copies}
                rows.append(row)
                log(json.dumps(row))
                del graph, x, y
            del blobs, layers, base
            torch.cuda.empty_cache()
    if args.out:
        with open(args.out, "w") as f:
            for row in rows:
                f.write(json.dumps(row) + "\n")


# ------------------------------------------------------------------ profiler summaries
_DEMANGLED = {}


def _demangle(name):
    if name not in _DEMANGLED:
        import subprocess
        try:
            _DEMANGLED[name] = subprocess.run(["c++filt", name], capture_output=True, text=True,
                                              check=True).stdout.strip()
        except (OSError, subprocess.CalledProcessError):
            _DEMANGLED[name] = name
        if _DEMANGLED[name].startswith("_Z"):
            # a name the profiler cut short: keep its last <length><identifier> piece
            import re
            best, i = name, 0
            while True:
                mt = re.compile(r"(\d+)").search(name, i)
                if not mt:
                    break
                k, j = int(mt.group(1)), mt.end()
                ident = name[j:j + k]
                if k and len(ident) == k and (ident[0].isalpha() or ident[0] == "_"):
                    if "kernel" in ident:
                        best = ident + "<" + name[j + k:j + k + 12] + "...>"
                    i = j + k
                else:
                    i = mt.start() + 1
            _DEMANGLED[name] = best
    return _DEMANGLED[name]


def _short_kernel(name):
    name = name.strip('"')
    if name.startswith("_Z"):
        name = _demangle(name)
    name = name.replace("(anonymous namespace)", "anon")
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    name = name[:cut]
    return name.replace("nq::anon::", "").replace("nq::", "").replace("at::native::anon::", "").replace(
        "at::native::", "")


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def trace_table(d):
    """Per (kernel, workgroups, threads): dispatches and duration statistics
    from a rocprofv3 --kernel-trace csv directory."""
    groups = {}
    for r in _csv_rows(d, "kernel_trace.csv"):
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        key = (_short_kernel(r["Kernel_Name"]), grid // max(wg, 1), wg)
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    return groups


def counter_table(d):
    """Per (kernel, workgroups, threads) and counter: the values of every
    dispatch, from a rocprofv3 --pmc csv directory."""
    groups = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        wg = int(float(r["Workgroup_Size"]))
        key = (_short_kernel(r["Kernel_Name"]), int(float(r["Grid_Size"])) // max(wg, 1), wg)
        groups.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return groups


def print_summary(d, top=40):
    if _csv_rows(d, "kernel_trace.csv"):
        groups = trace_table(d)
        total = sum(sum(v) for v in groups.values())
        print(f"{'kernel':58s} {'wgs':>6s} {'thr':>5s} {'calls':>7s} {'avg us':>9s} {'min us':>9s} "
              f"{'max us':>9s} {'total %':>8s}")
        for key, v in sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:top]:
            print(f"{key[0][:58]:58s} {key[1]:6d} {key[2]:5d} {len(v):7d} {statistics.mean(v):9.3f} "
                  f"{min(v):9.3f} {max(v):9.3f} {100 * sum(v) / total:8.2f}")
    if _csv_rows(d, "counter_collection.csv"):
        groups = counter_table(d)
        names = sorted({c for g in groups.values() for c in g})
        print(f"{'kernel':58s} {'wgs':>6s} {'thr':>5s} {'calls':>7s} " + " ".join(f"{c:>16s}" for c in names))
        for key, g in sorted(groups.items(), key=lambda kv: -max(statistics.mean(v) for v in kv[1].values()))[:top]:
            n = max(len(v) for v in g.values())
            print(f"{key[0][:58]:58s} {key[1]:6d} {key[2]:5d} {n:7d} " +
                  " ".join(f"{statistics.mean(g[c]):16.1f}" if c in g else f"{'-':>16s}" for c in names))


def copy_calibration():
    """A plain elementwise kernel of known traffic for scaling the HBM counters:
    y = -x over 1 GiB of fp32 (reads 1 GiB, writes 1 GiB), three launches."""
    import torch
    x = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    log("[bench] copy calibration: 3 x neg over 1 GiB fp32 done")


KERNEL_PREFIX = {"stage1": "dec_s1", "mid": "dec_mid_kernel", "stage2": "dec_s2"}


def make_traffic_file(bench_json, fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    """profiles/decode70b_traffic.json from two --pmc runs of the bench (FETCH_SIZE,
    WRITE_SIZE) and two of the copy calibration, for the dominant kernel named in
    the bench's JSON line."""
    with open(bench_json) as f:
        line = [ln for ln in f if ln.startswith("{")][-1]
    roof = json.loads(line)["roofline"]
    key = roof["kernel"]
    wgs, thr = roof["launch"]["workgroups"], roof["launch"]["threads"]
    prefix = KERNEL_PREFIX[key.split(".")[1]]

    def per_dispatch(d, counter, match):
        vals = []
        for k, g in counter_table(d).items():
            if match(k) and counter in g:
                vals.extend(g[counter])
        if not vals:
            raise SystemExit(f"no {counter} rows in {d}")
        return statistics.median(vals), len(vals)

    big = lambda k: "neg" in k[0] or "elementwise" in k[0] or "vectorized" in k[0]
    cf, _ = per_dispatch(cfetch_dir, "FETCH_SIZE", big)
    cw, _ = per_dispatch(cwrite_dir, "WRITE_SIZE", big)
    ffac, wfac = (1 << 30) / (cf * 1024), (1 << 30) / (cw * 1024)
    mine = lambda k: k[0].startswith(prefix) and k[1] == wgs and k[2] == thr
    kf, nf = per_dispatch(fetch_dir, "FETCH_SIZE", mine)
    kw, nw = per_dispatch(write_dir, "WRITE_SIZE", mine)
    with open(DEC_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    out = {"kernel": key, "launch": {"workgroups": wgs, "threads": thr}, "source_sha": sha,
           "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw, "dispatches": [nf, nw],
           "copy_fetch_kib": cf, "copy_write_kib": cw, "fetch_factor": round(ffac, 4), "write_factor": round(wfac, 4),
           "traffic_bytes": int(kf * 1024 * ffac + kw * 1024 * wfac),
           "alg_bytes_per_launch": roof["alg_bytes_per_launch"]}
    out["traffic_over_alg"] = round(out["traffic_bytes"] / out["alg_bytes_per_launch"], 4)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def main():
    args = parse()
    if args.rocprof_summary:
        print_summary(args.rocprof_summary)
        return
    if args.make_traffic_file:
        make_traffic_file(*args.make_traffic_file)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus above 1 is not supported "
                                   "(the multi-GPU split is a design note, not built)"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
    elif args.suite == "7b":
        run_suite7b(args)
    elif args.initializer_only:
        print(json.dumps({"initializer": run_initializer("cuda:0")}), flush=True)
    elif args.variants_only:
        print(json.dumps({"variants": run_variants("cuda:0")}), flush=True)
    elif args.prefill_only:
        print(json.dumps({"prefill": run_prefill70b("cuda:0")}), flush=True)
    else:
        run_decode70b(args)


if __name__ == "__main__":
    main()
