#!/usr/bin/env python3
"""Benchmark of the packed binary low-rank linear forward on one MI355X.

Default workload: Llama-2-70B-shaped decode, 80 blocks x {q, k, v, o, gate, up,
down} linears at 0.8 bits/weight (ranks from the storage rule r(m+n) bits +
16-bit scales), batch 1, bf16 activations and outputs, fp16 scales.  Every layer
has its own seeded random signs and scales and every linear its own seeded
input (no attention, norm or embedding between them).  One step = the 560
linears in block order on one stream, each finished before the next starts,
captured once as a HIP graph and replayed.

Prints one JSON line.  `value` is algorithmic GB/s over the whole step: per
linear r(m+n)/8 sign bytes + 2(m+n+r) scale bytes + 2Bn x bytes + 2Bm y bytes.
`roofline` is for the dominant kernel (largest share of the step), timed with
HIP events around each of its launches on the stream it runs on.  After the
timed region one layer of every distinct shape of block 0 is checked against
the fp64 oracle on the host (`parity`).

  python bench.py [--steps K --warmup W]           70B decode chain (the metric)
  python bench.py --suite 7b --out FILE            7B shapes, B in {1,2,4,8,16}, 0.55/0.8/1.0 bpw:
                                                   per-shape GB/s over >= 1 GiB of rotating layer copies
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
    ap.add_argument("--suite", default=None, choices=["7b"])
    ap.add_argument("--out", default=None)
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
                lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
                lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
                return lib
    raise RuntimeError("libamdhip64 is not loaded")


class Events:
    def __init__(self, hip, n):
        self.hip = hip
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(h)) == 0
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


def kernel_alg_bytes(kind, m, n, r, B, xb=2, yb=2, sb=2):
    """Algorithmic bytes each kernel of the decode path owns: stage 1 reads x,
    s2 and the packed V^T bits; stage 2 the packed U bits, s1 and g and writes
    y (intermediates such as the partial sums of t are not counted)."""
    if kind == "stage1":
        return r * n / 8 + B * n * xb + sb * n
    if kind == "mid":
        return 0.0
    return r * m / 8 + sb * (m + r) + B * m * yb


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
    from oracle import nq_oracle  # noqa: F401  (rank rule lives in the library; imported below)
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


# ------------------------------------------------------------------ 70B decode chain
def run_decode70b(args):
    import numpy as np
    import torch
    import binary_rank_gemv_packed_amd as nq
    import synth

    dev = "cuda:0"
    B = args.batch
    spec = chain_spec(synth.LLAMA70B, 80, args.bpw)
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
    ws_bytes = max(nq.workspace_bytes(L, B, args.path) for L in layers)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()

    def step():
        for L, x, y in zip(layers, xs, ys):
            nq.linear_into(x, L, y, ws, args.path)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    torch.cuda.synchronize()
    # replays run on `stream`, and the events are recorded on that same stream
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/step (events), wall {wall * 1e3 / args.steps:.4f} ms/step")
    step_bytes = sum(alg_bytes(m, n, r, B) for (_, _, _, m, n, r) in spec)
    gbs = step_bytes / (ms * 1e-3) / 1e9

    # parity of the timed chain's own outputs (last replay), one linear per distinct shape
    parity = {}
    for i, host in hosts.items():
        e, er = oracle_check(host, ys[i].float().cpu().numpy())
        name = spec[i][2]
        parity[name] = {"rel_l2": float(f"{e:.3e}"), "bf16_rounding_rel_l2": float(f"{er:.3e}"),
                        "ok": bool(e <= 2e-3 + er)}
        log(f"[bench] parity {name}: rel L2 {e:.3e} (bf16 rounding alone {er:.3e})")

    # per-kernel durations with HIP events around each launch, block 0's seven linears
    kernels = {}
    roof = None
    if args.path in ("auto", "decode") and B <= 4:
        hip = hip_runtime()
        reps = 20
        ev = Events(hip, 8 * reps)
        per_kind = {}
        with torch.cuda.stream(stream):
            for li in range(7):
                _, _, name, m, n, r = spec[li]
                durs = None
                launches = 0
                for k in range(reps):
                    launches = nq.linear_into_profiled(xs[li], layers[li], ys[li], ws, ev.ev[8 * k:8 * k + 8],
                                                       args.path)
                torch.cuda.synchronize()
                names = ["stage1", "mid", "stage2"] if launches == 3 else ["stage1", "stage2"]
                durs = {nm: statistics.mean(ev.ms(8 * k + j, 8 * k + j + 1) for k in range(reps))
                        for j, nm in enumerate(names)}
                per_kind[name] = (m, n, r, durs)
        ev.close()
        counts = {nm: sum(1 for s in spec if s[2] == nm) for nm in per_kind}
        best = None
        for name, (m, n, r, durs) in per_kind.items():
            for kn, d in durs.items():
                byts = kernel_alg_bytes(kn, m, n, r, B)
                key = f"{name}.{kn}"
                kernels[key] = {"us": round(d * 1e3, 3), "alg_bytes": int(byts),
                                "gbs": round(byts / (d * 1e-3) / 1e9, 1), "per_step": counts[name]}
                share = d * counts[name]
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
                "us_per_launch": round(d * 1e3, 3), "alg_bytes_per_launch": int(byts)}
        log(f"[bench] dominant kernel {key}: {d * 1e3:.2f} us/launch, {achieved:.1f} GB/s")

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
        },
        "parity": parity,
        "kernels": kernels,
    }
    if roof is not None:
        out["roofline"] = roof
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle baseline ...")
        out["cpu_baseline"] = cpu_baseline(spec, B)
    print(json.dumps(out), flush=True)


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


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus above 1 is not supported "
                                   "(the multi-GPU split is a design note, not built)"}))
        sys.exit(2)
    if args.suite == "7b":
        run_suite7b(args)
    else:
        run_decode70b(args)


if __name__ == "__main__":
    main()
