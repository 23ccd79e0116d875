#!/usr/bin/env python3
"""Throughput of the GDN chunkwise forward pass on one MI355X.

One step = one gdn_fwd call (chunk map when packed, gate prologue, WY, state
pass, output) over one batch of seeded synthetic inputs that are already
resident in HBM.  Default workload: B=2, T=2048, H=HV=8, K=V=128, bf16 q/k/v,
fp32 gate/beta, chunk 64 (the pages' shape).

Prints ONE JSON line with the headline tokens/s, the roofline of the dominant
kernel (per-kernel durations measured live with HIP events on the launch
stream), and the fp64 CPU oracle timed on this host as a baseline.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunk-fwd tokens/s (B=2,T=2048,H=8,K=V=128 bf16); % MFMA/HBM peak"
HBM_PEAK = 8.0e12            # bytes/s, MI355X HBM3E
MFMA_PEAK = {"bf16": 2.5e15, "fp32": 157.3e12}  # dense flop/s
CHUNK = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="pages_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def source_hash():
    """Hash of the kernel sources (traffic counters are only valid for this code)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_deltanet_chunkwise_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def algorithmic(shape, esz, has_h0, used_slots):
    """Algorithmic bytes and flops per launch of each kernel and of the whole pass.

    Each tensor a kernel consumes or produces counts once at its stored width;
    flops count the triangular products by their nonzero half.
    """
    B, T, H, HV, K, V, N = (shape[k] for k in ("B", "T", "H", "HV", "K", "V", "N"))
    ntok = T if shape.get("packed") else B * T
    U = ntok * HV                       # token-heads
    Ck = used_slots * HV                # chunk-heads
    state = N * HV * K * V * 4          # one fp32 state tensor
    C = CHUNK
    k_in = ntok * H * K * esz
    kern = {
        "chunk_map": dict(bytes=(N + 1) * 8 + used_slots * 16 + (N + 1) * 4, flops=0),
        # WY includes the gate prologue: reads g_raw, beta (8 B) and writes the
        # stride-1 cumulative gate and beta rows (8 B) per token-head.
        "wy": dict(bytes=k_in + ntok * HV * V * esz + U * 16 + U * (2 * K + V) * esz,
                   flops=U * C * (2 * K + V)),
        "chain": dict(bytes=U * (2 * K + V) * esz + Ck * 4 + Ck * K * V * esz + U * V * esz
                      + (state if has_h0 else 0) + state,
                      flops=U * 4 * K * V),
        "output": dict(bytes=2 * k_in + Ck * K * V * esz + U * V * esz + U * 4 + U * V * esz,
                       flops=U * (C * K + C * V + 2 * K * V)),
    }
    path = dict(bytes=2 * k_in + ntok * HV * V * esz + U * 8 + U * V * esz
                + (state if has_h0 else 0) + state,
                flops=U * (C * (3 * K + 2 * V) + 6 * K * V))
    return kern, path, ntok


def hip_runtime():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    return hip


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)


def cpu_baseline(inp, target_s):
    """fp64 oracle on the same (rounded) inputs, all host cores."""
    import numpy as np
    import oracle
    f = lambda t: None if t is None else t.float().numpy().astype(np.float64)  # noqa: E731
    args = [f(inp.q), f(inp.k), f(inp.v), f(inp.g_raw), f(inp.beta), f(inp.A_log),
            f(inp.dt_bias)]
    cu = None if inp.cu_seqlens is None else inp.cu_seqlens.numpy()
    h0 = f(inp.h0)
    threads = oracle.default_threads()
    s = inp.shape
    units = s["N"] * s["HV"]
    ntok = s["T"] if inp.cu_seqlens is not None else s["B"] * s["T"]
    oracle.load()
    # repeat the whole workload until the sample holds about target_s of work
    reps, total = 0, 0.0
    while total < target_s:
        t0 = time.perf_counter()
        oracle.fwd(*args, cu_seqlens=cu, h0=h0, scale=inp.scale, nthreads=threads)
        total += time.perf_counter() - t0
        reps += 1
    return {"value": reps * ntok / total, "unit": "tokens/s", "cores": min(threads, units),
            "kind": "oracle",
            "sample": "whole workload (%d tokens x %d value heads, %d units), %d run(s), "
                      "%.1f s; threads=%d" % (ntok, s["HV"], units, reps, total, threads)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return
    import gated_deltanet_chunkwise_amd as gdn
    from gated_deltanet_chunkwise_amd.inputs import WORKLOADS, workload_inputs

    wl = args.workload
    cfg = WORKLOADS[wl]
    inp_cpu = workload_inputs(wl)
    inp = inp_cpu.to("cuda")
    s = inp.shape
    packed = inp.cu_seqlens is not None
    plan = gdn.GdnForward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], inp.q.dtype, "cuda",
                          num_seqs=s["N"] if packed else None, scale=inp.scale)
    call = lambda ev=None: plan(inp.q, inp.k, inp.v, inp.g_raw, inp.beta, inp.A_log,  # noqa
                                inp.dt_bias, inp.cu_seqlens, inp.h0, events=ev)
    stream = torch.cuda.current_stream()

    step = plan.bind(inp.q, inp.k, inp.v, inp.g_raw, inp.beta, inp.A_log, inp.dt_bias,
                     inp.cu_seqlens, inp.h0, stream=stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # headline: K eager steps, events on the launch stream, synchronized on both sides
    ms = timed(step, args.steps)

    # the same step captured once in a HIP graph and replayed (launch overhead view)
    graph_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            gstep = plan.bind(inp.q, inp.k, inp.v, inp.g_raw, inp.beta, inp.A_log, inp.dt_bias,
                              inp.cu_seqlens, inp.h0, stream=cap)
            with torch.cuda.graph(g, stream=cap):
                gstep()
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = timed(g.replay, args.steps)
    except Exception as exc:  # graph capture is an extra view, not the headline
        print("graph timing skipped: %s" % exc, file=sys.stderr, flush=True)

    # per-kernel durations: the same K steps with events between the stages
    hip = hip_runtime()
    nev = gdn.NUM_STAGES + 1
    handles = []
    for _ in range(nev * args.steps):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        handles.append(e.value)
    per_step = [(ctypes.c_void_p * nev)(*handles[i * nev:(i + 1) * nev])
                for i in range(args.steps)]
    torch.cuda.synchronize()
    for arr in per_step:
        call(arr)
    torch.cuda.synchronize()
    stage_ms = [0.0] * gdn.NUM_STAGES
    f = ctypes.c_float()
    for arr in per_step:
        for i in range(gdn.NUM_STAGES):
            if hip.hipEventElapsedTime(ctypes.byref(f), arr[i], arr[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            stage_ms[i] += f.value / args.steps
    for h in handles:
        hip.hipEventDestroy(h)

    dtype = cfg["dtype"]
    esz = 2 if dtype == "bf16" else 4
    sh = dict(s, packed=packed)
    used = plan.layout.num_slots
    if packed:
        lens = (inp_cpu.cu_seqlens[1:] - inp_cpu.cu_seqlens[:-1]).tolist()
        used = sum((L + CHUNK - 1) // CHUNK for L in lens)
    kern, path, ntok = algorithmic(sh, esz, inp.h0 is not None, used)
    kernels = {}
    for name, t in zip(gdn.STAGES, stage_ms):
        if name == "chunk_map" and not packed:
            continue
        a = kern[name]
        sec = t / 1e3
        kernels[name] = dict(us=round(t * 1e3, 3), bytes=a["bytes"], flops=a["flops"],
                             hbm_gbs=round(a["bytes"] / sec / 1e9, 1) if sec > 0 else None,
                             hbm_frac=round(a["bytes"] / sec / HBM_PEAK, 4) if sec > 0 else None,
                             mfma_tflops=round(a["flops"] / sec / 1e12, 2) if sec > 0 else None,
                             mfma_frac=round(a["flops"] / sec / MFMA_PEAK[dtype], 4)
                             if sec > 0 else None)
    dom = max(kernels, key=lambda n: kernels[n]["us"])
    d = kernels[dom]
    ai = d["flops"] / d["bytes"]
    ridge = MFMA_PEAK[dtype] / HBM_PEAK
    if ai >= ridge:
        roof = dict(bound="mfma", achieved=d["mfma_tflops"], peak=MFMA_PEAK[dtype] / 1e12,
                    unit="TFLOP/s", frac=d["mfma_frac"])
    else:
        roof = dict(bound="hbm", achieved=d["hbm_gbs"], peak=HBM_PEAK / 1e9, unit="GB/s",
                    frac=d["hbm_frac"])
    roof["kernel"] = dom
    roof["traffic"] = None
    src = source_hash()
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        ent = tr.get(wl, {}).get(dom)
        if ent and ent.get("source_hash") == src:
            roof["traffic"] = ent["bytes_per_launch"]
    sec = ms / 1e3
    out = {
        "metric": METRIC,
        "value": round(ntok / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl, "B": s["B"], "T": s["T"], "H": s["H"], "HV": s["HV"],
                   "K": s["K"], "V": s["V"], "chunk": CHUNK, "packed_seqs": s["N"] if packed
                   else None, "initial_state": inp.h0 is not None},
        "roofline": roof,
        "path_roofline": {"bytes": path["bytes"], "flops": path["flops"],
                          "hbm_frac": round(path["bytes"] / sec / HBM_PEAK, 4),
                          "mfma_frac": round(path["flops"] / sec / MFMA_PEAK[dtype], 4)},
        "kernels": kernels,
        "kernel_source_hash": src,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp_cpu, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
