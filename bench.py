#!/usr/bin/env python3
"""Throughput of the GDN chunkwise forward pass on one MI355X (--op selects
the backward pass, the KDA gate or the decode step instead).

One step = one gdn_fwd call (chunk map when packed, gate prologue, WY, state
pass, output) over one batch of seeded synthetic inputs that are already
resident in HBM.  Default workload: B=2, T=2048, H=HV=8, K=V=128, bf16 q/k/v,
fp32 gate/beta, chunk 64 (the pages' shape).

Prints ONE JSON line with the headline tokens/s, the roofline of the dominant
kernel (per-kernel durations measured live with HIP events on the launch
stream), and the fp64 CPU oracle timed on this host as a baseline.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunk-fwd tokens/s (B=2,T=2048,H=8,K=V=128 bf16); % MFMA/HBM peak"
HBM_PEAK = 8.0e12            # bytes/s, MI355X HBM3E
MFMA_PEAK = {"bf16": 2.5e15, "fp32": 157.3e12}  # dense flop/s
CHUNK = 64
GRAPH_PER = 10               # steps per HIP graph in the many-steps graph view
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def metric_label(op, cfg):
    """The metric string of a forward or backward line, named after the workload
    it measures: B, T, heads (HV only when it differs from H), head sizes and
    dtype, or the packed total and sequence count.  For the forward pass at
    B=2, T=2048, H=HV=8, K=V=128 bf16 this is METRIC exactly."""
    kind = {"gdn_fwd": "chunk-fwd", "gdn_bwd": "chunk-bwd"}[op]
    heads = "H=%d" % cfg["H"] + ("" if cfg["HV"] == cfg["H"] else ",HV=%d" % cfg["HV"])
    dims = ("K=V=%d" % cfg["K"]) if cfg["K"] == cfg["V"] else "K=%d,V=%d" % (cfg["K"], cfg["V"])
    if cfg.get("num_seqs"):
        seqs = "packed T=%d in %d seqs" % (cfg["T"], cfg["num_seqs"])
    else:
        seqs = "B=%d,T=%d" % (cfg["B"], cfg["T"])
    extra = ",h0" if cfg.get("h0") else ""
    return "GDN %s tokens/s (%s,%s,%s%s %s); %% MFMA/HBM peak" % (kind, seqs, heads, dims, extra,
                                                                cfg["dtype"])


def kernel_figures(a, t_ms, dtype):
    """Rates of one kernel (algorithmic bytes and flops `a`, average duration
    t_ms) against the HBM peak and the MFMA peak of the dtype its products
    take: the call's dtype, for every forward and backward kernel (a bf16 call
    runs all of its products on the bf16 MFMA, an fp32 call on the fp32 MFMA)."""
    sec = t_ms / 1e3
    if sec <= 0:
        return dict(us=round(t_ms * 1e3, 3), bytes=a["bytes"], flops=a["flops"], hbm_gbs=None,
                    hbm_frac=None, mfma_tflops=None, mfma_frac=None, mfma_dtype=dtype)
    return dict(us=round(t_ms * 1e3, 3), bytes=a["bytes"], flops=a["flops"],
                hbm_gbs=round(a["bytes"] / sec / 1e9, 1),
                hbm_frac=round(a["bytes"] / sec / HBM_PEAK, 4),
                mfma_tflops=round(a["flops"] / sec / 1e12, 2),
                mfma_frac=round(a["flops"] / sec / MFMA_PEAK[dtype], 4), mfma_dtype=dtype)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="pages_bf16")
    ap.add_argument("--op", default="gdn_fwd", choices=["gdn_fwd", "gdn_bwd", "kda_gate", "decode"],
                    help="gdn_fwd: the forward pass (headline); gdn_bwd: the backward pass "
                         "(forward recompute included) on --workload; kda_gate: the KDA "
                         "per-channel gate on the guide's timing shape; decode: one recurrent "
                         "step for a batch of sequences")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="forward: also time this many steps each after touching 1 GiB on the "
                         "stream (inputs and intermediates out of the 256 MB last-level cache)")
    ap.add_argument("--seg-chunks", type=int, default=0,
                    help="segment-parallel state pass with segments of this many chunks (0: off, "
                         "-1: the library's automatic choice)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="no GPU: turn the rocprofv3 FETCH_SIZE / WRITE_SIZE passes under DIR "
                         "(fetch/, write/, copy_fetch/, copy_write/) into profiles/traffic.json "
                         "for --workload (with --op gdn_bwd: the backward's kernels, under "
                         "'<workload>:bwd')")
    return ap.parse_args()


# The sources each op's kernels and launches are built from: traffic counters
# taken for an op stay valid while these files are unchanged.
OP_SOURCES = {
    "gdn_fwd": ("gdn_api.hip", "gdn_common.h", "gdn_kernels.h"),
    "gdn_bwd": ("gdn_api.hip", "gdn_bwd.h", "gdn_common.h", "gdn_kernels.h"),
    "kda_gate": ("gdn_common.h", "gdn_kda.h"),
    "decode": ("gdn_common.h", "gdn_decode.h"),
}


_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def code_text(text):
    """C++ source with its comments removed and whitespace collapsed (string and
    character literals kept as written): what the compiler sees."""
    kept = _TOKENS.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), text)
    return " ".join(kept.split())


def source_hash(op="gdn_fwd"):
    """Hash of the code of one op (traffic counters are only valid for this code;
    comments and layout do not enter it)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_deltanet_chunkwise_amd", "csrc")
    for f in OP_SOURCES[op]:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def algorithmic(shape, esz, has_h0, used_slots, fused=False):
    """Algorithmic bytes and flops per launch of each kernel and of the whole pass.

    Each tensor a kernel consumes or produces counts once at its stored width;
    flops count the triangular products by their nonzero half.  fused: the
    output stage runs inside the state pass ("chain_out"), and WY also reads Q
    and writes the masked, decayed Q K^T (six 1 KB bf16 fragments per chunk and
    head at bf16).
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
    if fused:
        p_bytes = Ck * 6 * 64 * 8 * esz        # the P^T fragments WY writes and chain_out reads
        kern["wy"] = dict(bytes=kern["wy"]["bytes"] + k_in + p_bytes,
                          flops=kern["wy"]["flops"] + U * C * K)
        kern["chain_out"] = dict(
            bytes=U * (2 * K + V) * esz + U * 4 + k_in + p_bytes + U * V * esz
            + (state if has_h0 else 0) + state,
            flops=U * (4 * K * V + C * V + 2 * K * V))
        del kern["chain"], kern["output"]
    path = dict(bytes=2 * k_in + ntok * HV * V * esz + U * 8 + U * V * esz
                + (state if has_h0 else 0) + state,
                flops=U * (C * (3 * K + 2 * V) + 6 * K * V))
    return kern, path, ntok


def algorithmic_bwd(shape, esz, has_h0, has_dht, used_slots):
    """Algorithmic bytes and flops per launch of each backward stage (the
    forward-recompute stage is two kernels, WY and the state pass), and of the
    whole pass.  Each intermediate counts at its stored width: T, H_c, v_new,
    dH, dv_new, dw and the dO term bq in the call's dtype (esz), dv_local, the
    dq / dk partials and the per-chunk sums in fp32; triangular products by
    their nonzero half."""
    B, T, H, HV, K, V, N = (shape[k] for k in ("B", "T", "H", "HV", "K", "V", "N"))
    ntok = T if shape.get("packed") else B * T
    U = ntok * HV
    Ck = used_slots * HV
    state = N * HV * K * V * 4
    C = CHUNK
    k_in = ntok * H * K * esz
    kv = Ck * K * V * esz          # one K x V per chunk and value head (H_c, dH, bq)
    tv = U * V * esz               # one V per token and value head (v_new, dv_new)
    fwd, _, _ = algorithmic(shape, esz, has_h0, used_slots)
    dq_out = U * K * (esz if HV == H else 4)  # dq (or dk): dtype, else fp32 partials
    kern = {
        # WY storing T, then the state pass storing H_c and v_new
        "recompute": dict(
            bytes=fwd["wy"]["bytes"] + Ck * C * C * esz + U * (2 * K + V) * esz + Ck * 4
            + (state if has_h0 else 0) + kv + tv,
            flops=fwd["wy"]["flops"] + U * 4 * K * V),
        # q, k, do, gates, w in; kd, w^T fragments, bq and dv_local (fp32) out
        "prep": dict(bytes=2 * k_in + U * V * esz + U * 4 + U * K * esz + 2 * U * K * esz
                     + kv + U * V * 4,
                     flops=U * C * (K + V) + U * 2 * K * V),
        # kd, w^T, bq, dv_local, gates in; dH, dv_new and dh0 out
        "bwd_chain": dict(bytes=2 * U * K * esz + kv + U * V * 4 + Ck * 4
                          + (state if has_dht else 0) + kv + tv + state,
                          flops=U * 4 * K * V),
        # q, k, do, v_new, dv_new, H_c, dH, gates in; dq, dk partial (fp32),
        # dw, dG out
        "dqk": dict(bytes=2 * k_in + U * V * esz + 2 * tv + 2 * kv + U * 4
                    + dq_out + U * K * 4 + U * K * esz + U * 4,
                    flops=U * (6 * K * V + C * V + 3 * C * K)),
        # k, v, dw, dk partial, dv_new, T, gates in; dk, dv, dbeta, dg_raw and
        # the per-chunk sums out
        "bwd_wy": dict(bytes=k_in + U * V * esz + U * K * esz + U * K * 4 + tv + Ck * C * C * esz
                       + 4 * U * 4 + dq_out + U * V * esz + 2 * U * 4
                       + 2 * Ck * 4,
                       flops=U * (2 * C * (K + V) + 2 * C * C // 3 + 3 * C * K)),
        # per-head parameter sums, plus the key-head dq/dk sums when value heads
        # share a key head (else dq, dk are written by the dq/dk and WY kernels)
        "sums": dict(bytes=2 * Ck * 4 + 2 * HV * 4 + (2 * U * K * 4 + 2 * k_in if HV > H else 0),
                     flops=0),
    }
    path = dict(bytes=4 * k_in + 3 * U * V * esz + 4 * U * 4 + (state if has_h0 else 0)
                + (state if has_dht else 0) + state,
                flops=sum(v["flops"] for v in kern.values()))
    return kern, path, ntok


KERNEL_STAGE = (("gdn_chunk_map_kernel", "chunk_map"), ("gdn_wy_kernel", "wy"),
                ("gdn_chain_out_kernel", "chain_out"),
                ("gdn_chain_ring_kernel", "chain"), ("gdn_chain_kernel", "chain"),
                ("gdn_chain2_kernel", "chain"), ("gdn_chain_ks_kernel", "chain"),
                ("gdn_output_kernel", "output"), ("gdn_kda_gate_vec_kernel", "kda_gate"),
                ("gdn_kda_gate_scalar_kernel", "kda_gate"), ("gdn_decode_kernel", "decode"),
                ("gdn_bwd_prep_kernel", "prep"), ("gdn_bwd_prep_bf16_kernel", "prep"),
                ("gdn_bwd_chain_kernel", "bwd_chain"), ("gdn_bwd_chain_ks_kernel", "bwd_chain"),
                ("gdn_bwd_dqk_kernel", "dqk"), ("gdn_bwd_dqk_bf16_kernel", "dqk"),
                ("gdn_bwd_wy_kernel", "bwd_wy"), ("gdn_bwd_wy_bf16_kernel", "bwd_wy"),
                ("gdn_bwd_qk_sum_kernel", "sums"))


def counter_means(path):
    """Mean counter value (KiB) per dispatch of each stage's kernel, and of the
    largest plain copy, from one rocprofv3 counter_collection.csv."""
    import csv
    vals, copies = {}, []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            for key, stage in KERNEL_STAGE:
                if key in name:
                    vals.setdefault(stage, []).append(v)
                    break
            else:
                if "copyBuffer" in name:
                    copies.append(v)
    return {k: sum(v) / len(v) for k, v in vals.items()}, (max(copies) if copies else None)


def counters_by_name(path):
    """Mean value per dispatch of every counter in one rocprofv3
    counter_collection.csv, per stage: {stage: {counter: mean}}."""
    import csv
    vals = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            for key, stage in KERNEL_STAGE:
                if key in r["Kernel_Name"]:
                    vals.setdefault(stage, {}).setdefault(r["Counter_Name"], []).append(
                        float(r["Counter_Value"]))
                    break
    return {st: {c: sum(v) / len(v) for c, v in cs.items()} for st, cs in vals.items()}


# Optional counter passes read by --write-traffic besides the byte counters:
# MFMA-busy cycles over active SIMD cycles, and matrix flops counted by the
# SQ (512 per MFMA "mop").
MFMA_PASSES = (("mfma_util", "MfmaUtil"), ("mfma_flops", "MfmaFlopsBF16 MfmaFlopsF32"))


def kernel_counters(ent):
    """The MFMA figures of one traffic.json kernel entry, if its passes ran."""
    c = ent.get("counters", {})
    out = {}
    if "MfmaUtil" in c:
        out["mfma_util"] = round(c["MfmaUtil"] / 100.0, 4)
    fl = [c[k] for k in ("MfmaFlopsBF16", "MfmaFlopsF32") if k in c]
    if fl:
        out["mfma_flops"] = int(round(sum(fl)))
    return out


def write_traffic(d, workload, copy_bytes, op="gdn_fwd"):
    """HBM bytes per launch of each kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by copy_bytes / (the same counter for a plain copy of
    copy_bytes bytes read and copy_bytes written)."""
    import glob

    def one(sub):
        f = glob.glob(os.path.join(d, sub, "*_counter_collection.csv"))
        if len(f) != 1:
            raise SystemExit("expected one counter_collection.csv under %s/%s" % (d, sub))
        return counter_means(f[0])
    fetch, _ = one("fetch")
    write, _ = one("write")
    _, copy_fetch = one("copy_fetch")
    _, copy_write = one("copy_write")
    kf = copy_bytes / (copy_fetch * 1024.0)
    kw = copy_bytes / (copy_write * 1024.0)
    src = source_hash(op)
    tr = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
    ent = {}
    for stage in fetch:
        fb, wb = fetch[stage] * 1024.0 * kf, write.get(stage, 0.0) * 1024.0 * kw
        ent[stage] = {"bytes_per_launch": int(round(fb + wb)), "fetch_bytes": int(round(fb)),
                      "write_bytes": int(round(wb)), "fetch_kib_raw": round(fetch[stage], 2),
                      "write_kib_raw": round(write.get(stage, 0.0), 2),
                      "fetch_scale": round(kf, 4), "write_scale": round(kw, 4),
                      "source_hash": src}
    for sub, _ in MFMA_PASSES:
        f = glob.glob(os.path.join(d, sub, "*_counter_collection.csv"))
        if len(f) == 1:
            for stage, cs in counters_by_name(f[0]).items():
                if stage in ent:
                    ent[stage].setdefault("counters", {}).update(
                        {k: round(v, 2) for k, v in cs.items()})
    tr[workload] = ent
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(tr, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(tr[workload]), flush=True)


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


# The KDA gate guide's timing configuration ("performance tests"): T=2048,
# H=16, D=128, bf16, with a bias; its inputs as in its tests (N(0,1)).
KDA_SHAPE = dict(T=2048, H=16, D=128)


def bench_kda(args):
    """One JSON line for the KDA per-channel gate: elements/s, its HBM roofline and
    the fp64 oracle on the host."""
    import numpy as np
    import torch
    import gated_deltanet_chunkwise_amd as gdn
    T, H, D = KDA_SHAPE["T"], KDA_SHAPE["H"], KDA_SHAPE["D"]
    gen = torch.Generator().manual_seed(20270)
    g = torch.randn((T, H, D), generator=gen).to(torch.bfloat16)
    A = torch.randn(H, generator=gen)
    b = torch.randn(H * D, generator=gen)
    gd, Ad, bd = g.cuda(), A.cuda(), b.cuda()
    out = torch.empty_like(gd)
    # one launch takes a few microseconds, less than the host needs to issue one,
    # so the timed region replays a HIP graph of back-to-back launches
    out.fill_(float("nan"))
    ms, steps = graph_time(
        lambda st: gdn.kda_gate_launcher(gd, Ad, bd, out=out, stream=st)[0], args.steps,
        args.warmup)
    # the graph's result equals one eager call's (the gate is deterministic)
    ref_launch, ref = gdn.kda_gate_launcher(gd, Ad, bd)
    ref_launch()
    torch.cuda.synchronize()
    if not torch.equal(ref, out):
        raise RuntimeError("graph replay of the KDA gate differs from an eager call")
    n = T * H * D
    nbytes = n * (2 + 2) + H * 4 + H * D * 4     # g in, yg out (bf16), A_log, dt_bias
    sec = ms / 1e3
    line = {
        "metric": "KDA gate elements/s (T=2048,H=16,D=128 bf16, bias)",
        "value": round(n / sec, 1), "unit": "elements/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kda_gate", "T": T, "H": H, "D": D, "bias": True,
                   "out_dtype": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / sec / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(nbytes / sec / HBM_PEAK, 4), "kernel": "kda_gate",
                     "traffic": None},
        "kernel_source_hash": source_hash("kda_gate"),
    }
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            ent = json.load(fh).get("kda_gate", {}).get("kda_gate")
        if ent and ent.get("source_hash") == line["kernel_source_hash"]:
            line["roofline"]["traffic"] = ent["bytes_per_launch"]
    if not args.no_cpu_baseline:
        import oracle
        g64 = g.float().numpy().astype(np.float64)
        A64, b64 = A.numpy().astype(np.float64), b.numpy().astype(np.float64)
        oracle.load()
        reps, total = 0, 0.0
        while total < args.cpu_seconds:
            t0 = time.perf_counter()
            oracle.kda_gate(g64, A64, b64)
            total += time.perf_counter() - t0
            reps += 1
        line["cpu_baseline"] = {"value": reps * n / total, "unit": "elements/s", "cores": 1,
                                "kind": "oracle",
                                "sample": "the whole shape (%d elements), %d run(s), %.1f s, "
                                          "one thread" % (n, reps, total)}
    print(json.dumps(line), flush=True)


def graph_time(make_launch, steps, warmup, per=20):
    """Milliseconds per launch, from a HIP graph of `per` back-to-back launches
    replayed between two events (for kernels shorter than one host launch).
    make_launch(stream) returns a zero-argument callable that enqueues one
    launch on `stream` (the capture stream)."""
    import torch
    cap = torch.cuda.Stream()
    launch = make_launch(cap)
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for _ in range(3):
            launch()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for _ in range(per):
            launch()
    stream = torch.cuda.current_stream()
    reps = max(1, steps // per)
    for _ in range(max(1, warmup // per)):
        graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * per), reps * per


# A batch-decode shape: 64 sequences, one new token each, with the pages' heads
# (H = HV = 8, K = V = 128, bf16); the pages give no decode configuration.
DECODE_SHAPE = dict(B=64, T=1, H=8, HV=8, K=128, V=128)


def bench_decode(args):
    """One JSON line for the recurrent step: tokens/s, HBM roofline (the state is
    read and written once per call), and the fp64 oracle on the host."""
    import numpy as np
    import torch
    import gated_deltanet_chunkwise_amd as gdn
    from gated_deltanet_chunkwise_amd.inputs import make_inputs
    c = DECODE_SHAPE
    inp = make_inputs(dtype="bf16", seed=20280, h0=True, **c)
    d = inp.to("cuda")
    state = d.h0.clone()
    out = torch.empty((c["B"], c["T"], c["HV"], c["V"]), dtype=d.q.dtype, device="cuda")
    out.fill_(float("nan"))
    ms, steps = graph_time(
        lambda st: gdn.decode_launcher(d.q, d.k, d.v, d.g_raw, d.beta, d.A_log, state,
                                       dt_bias=d.dt_bias, out=out, stream=st)[0],
        args.steps, args.warmup)
    torch.cuda.synchronize()
    if not torch.isfinite(out).all() or torch.equal(state, d.h0):
        raise RuntimeError("the timed decode launches did not run")
    B, T, H, HV, K, V = (c[x] for x in ("B", "T", "H", "HV", "K", "V"))
    nbytes = (2 * B * HV * K * V * 4 + 2 * B * T * H * K * 2 + 2 * B * T * HV * V * 2
              + B * T * HV * 8 + HV * 8)
    sec = ms / 1e3
    line = {
        "metric": "GDN decode tokens/s (B=64 sequences x 1 token, H=HV=8, K=V=128 bf16)",
        "value": round(B * T / sec, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": dict(c, workload="decode"),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / sec / 1e9, 1),
                     "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(nbytes / sec / HBM_PEAK, 4), "kernel": "decode",
                     "traffic": None},
        "kernel_source_hash": source_hash("decode"),
    }
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            ent = json.load(fh).get("decode", {}).get("decode")
        if ent and ent.get("source_hash") == line["kernel_source_hash"]:
            line["roofline"]["traffic"] = ent["bytes_per_launch"]
    if not args.no_cpu_baseline:
        import oracle
        f = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
        a = [f(inp.q), f(inp.k), f(inp.v), f(inp.g_raw), f(inp.beta), f(inp.A_log),
             f(inp.dt_bias)]
        h0 = f(inp.h0)
        threads = oracle.default_threads()
        oracle.load()
        reps, total = 0, 0.0
        while total < args.cpu_seconds:
            t0 = time.perf_counter()
            oracle.fwd(*a, h0=h0, nthreads=threads)
            total += time.perf_counter() - t0
            reps += 1
        line["cpu_baseline"] = {"value": reps * B * T / total, "unit": "tokens/s",
                                "cores": min(threads, B * HV), "kind": "oracle",
                                "sample": "the whole shape (%d sequences x %d value heads), %d "
                                          "run(s), %.1f s; threads=%d"
                                          % (B, HV, reps, total, threads)}
    print(json.dumps(line), flush=True)


def bench_bwd(args):
    """One JSON line for the backward pass on --workload: tokens/s, per-stage
    durations (HIP events recorded by gdn_bwd_timed on the launch stream), the
    roofline of the dominant stage, and the fp64 oracle's backward on the host."""
    import ctypes
    import numpy as np
    import torch
    import gated_deltanet_chunkwise_amd as gdn
    from gated_deltanet_chunkwise_amd.inputs import WORKLOADS, make_grads, workload_inputs
    wl = args.workload
    cfg = WORKLOADS[wl]
    inp_cpu = workload_inputs(wl)
    d_o_cpu, dht_cpu = make_grads(inp_cpu, SEEDS_BWD)
    inp = inp_cpu.to("cuda")
    d_o, dht = d_o_cpu.cuda(), dht_cpu.cuda()
    s = inp.shape
    packed = inp.cu_seqlens is not None
    plan = gdn.GdnBackward(s["B"], s["T"], s["H"], s["HV"], s["K"], s["V"], inp.q.dtype,
                           "cuda", num_seqs=s["N"] if packed else None, scale=inp.scale)
    stream = torch.cuda.current_stream()
    step = plan.bind(inp.q, inp.k, inp.v, inp.g_raw, inp.beta, inp.A_log, inp.dt_bias, d_o, dht,
                     inp.cu_seqlens, inp.h0, stream=stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # per-stage durations: gdn_bwd_timed records an event after each stage
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(gdn.BWD_NUM_STAGES + 1)]
    for e in evs:
        e.record(stream)  # creates the underlying hipEvent_t
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * len(evs))(*[e.cuda_event for e in evs])
    acc = [0.0] * gdn.BWD_NUM_STAGES
    reps = max(1, args.steps // 4)
    for _ in range(reps):
        plan(inp.q, inp.k, inp.v, inp.g_raw, inp.beta, inp.A_log, inp.dt_bias, d_o, dht,
             inp.cu_seqlens, inp.h0, stream=stream, events=handles)
        torch.cuda.synchronize()
        for i in range(gdn.BWD_NUM_STAGES):
            acc[i] += evs[i].elapsed_time(evs[i + 1])
    stage_ms = [a / reps for a in acc]
    dtype = cfg["dtype"]
    esz = 2 if dtype == "bf16" else 4
    sh = dict(s, packed=packed)
    if packed:
        lens = (inp_cpu.cu_seqlens[1:] - inp_cpu.cu_seqlens[:-1]).tolist()
        used = sum((L + CHUNK - 1) // CHUNK for L in lens)
    else:
        used = s["B"] * ((s["T"] + CHUNK - 1) // CHUNK)
    kern, path, ntok = algorithmic_bwd(sh, esz, inp.h0 is not None, True, used)
    kernels = {}
    for name, t in zip(gdn.BWD_STAGES, stage_ms):
        kernels[name] = kernel_figures(kern[name], t, dtype)
    single = [n for n in kernels if n != "recompute"]  # stages of one kernel
    dom = max(single, key=lambda n: kernels[n]["us"])
    d = kernels[dom]
    mpk = MFMA_PEAK[d["mfma_dtype"]]
    if d["flops"] / d["bytes"] >= mpk / HBM_PEAK:
        roof = dict(bound="mfma", achieved=d["mfma_tflops"], peak=mpk / 1e12,
                    unit="TFLOP/s", frac=d["mfma_frac"], dtype=d["mfma_dtype"])
    else:
        roof = dict(bound="hbm", achieved=d["hbm_gbs"], peak=HBM_PEAK / 1e9, unit="GB/s",
                    frac=d["hbm_frac"])
    roof["kernel"] = dom
    roof["traffic"] = None
    src = source_hash("gdn_bwd")
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh).get(wl + ":bwd", {})
        ent = tr.get(dom)
        if ent and ent.get("source_hash") == src:
            roof["traffic"] = ent["bytes_per_launch"]
            roof.update(kernel_counters(ent))
        for name, k in kernels.items():
            e = tr.get(name)
            if e and e.get("source_hash") == src:
                k.update({"counters_" + a: b for a, b in kernel_counters(e).items()})
    sec = ms / 1e3
    out = {
        "metric": metric_label("gdn_bwd", cfg), "value": round(ntok / sec, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": wl, "B": s["B"], "T": s["T"], "H": s["H"], "HV": s["HV"],
                   "K": s["K"], "V": s["V"], "chunk": CHUNK,
                   "packed_seqs": s["N"] if packed else None,
                   "initial_state": inp.h0 is not None, "final_state_grad": True},
        "roofline": roof,
        "path_roofline": {"bytes": path["bytes"], "flops": path["flops"],
                          "hbm_frac": round(path["bytes"] / sec / HBM_PEAK, 4),
                          "mfma_frac": round(path["flops"] / sec / MFMA_PEAK[dtype], 4)},
        "kernels": kernels,
        "kernel_source_hash": src,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        f = lambda t: None if t is None else t.float().numpy().astype(np.float64)  # noqa: E731
        a = [f(inp_cpu.q), f(inp_cpu.k), f(inp_cpu.v), f(inp_cpu.g_raw), f(inp_cpu.beta),
             f(inp_cpu.A_log), f(inp_cpu.dt_bias), f(d_o_cpu), f(dht_cpu)]
        cu = None if inp_cpu.cu_seqlens is None else inp_cpu.cu_seqlens.numpy()
        threads = oracle.default_threads()
        oracle.load()
        reps, total = 0, 0.0
        while total < args.cpu_seconds:
            t0 = time.perf_counter()
            oracle.bwd(*a, cu_seqlens=cu, h0=f(inp_cpu.h0), scale=inp_cpu.scale,
                       nthreads=threads)
            total += time.perf_counter() - t0
            reps += 1
        out["cpu_baseline"] = {
            "value": reps * ntok / total, "unit": "tokens/s",
            "cores": min(threads, s["N"] * s["HV"]), "kind": "oracle",
            "sample": "whole workload (%d tokens x %d value heads), %d run(s), %.1f s; "
                      "threads=%d" % (ntok, s["HV"], reps, total, threads)}
    print(json.dumps(out), flush=True)


SEEDS_BWD = 20290  # output-gradient seed of the backward benchmark


def traffic_key(workload, op="gdn_fwd", seg_chunks=0):
    """traffic.json key of one measured configuration: the workload, then
    ':bwd' for the backward, or ':seg=L' (':seg=auto') for a forward with the
    segment-parallel state pass, whose kernels differ from the plain pass's."""
    if op == "gdn_bwd":
        return workload + ":bwd"
    if seg_chunks:
        return workload + (":seg=auto" if seg_chunks < 0 else ":seg=%d" % seg_chunks)
    return workload


def main():
    args = parse()
    if args.write_traffic:
        op = {"kda_gate": "kda_gate", "decode": "decode"}.get(
            args.workload, "gdn_bwd" if args.op == "gdn_bwd" else "gdn_fwd")
        key = traffic_key(args.workload, op, args.seg_chunks if op == "gdn_fwd" else 0)
        write_traffic(args.write_traffic, key, args.copy_mib << 20, op)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return
    if args.op == "kda_gate":
        bench_kda(args)
        return
    if args.op == "decode":
        bench_decode(args)
        return
    if args.op == "gdn_bwd":
        bench_bwd(args)
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
                          num_seqs=s["N"] if packed else None, scale=inp.scale,
                          seg_chunks=args.seg_chunks)
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

    # cold: each step timed alone after an untimed pass over 1 GiB on the same
    # stream, so that its inputs and intermediates come from HBM rather than the
    # last-level cache (the pages' working set fits in it)
    cold_ms = None
    if args.cold_steps > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        total = 0.0
        for _ in range(args.cold_steps):
            flush.add_(1.0)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1)
        cold_ms = total / args.cold_steps
        del flush

    # the same step captured in HIP graphs and replayed (launch overhead view):
    # one step per graph, and GRAPH_PER steps per graph (per step: the
    # difference between the two is the cost of one graph launch); each
    # replay's o must equal the eager step's bit for bit (the same work)
    graph_ms = graph_many_ms = None
    try:
        o_eager = plan.o.clone()
        graphs = {}
        for per in (1, GRAPH_PER):
            g = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(stream)
            with torch.cuda.stream(cap):
                gstep = plan.bind(inp.q, inp.k, inp.v, inp.g_raw, inp.beta, inp.A_log,
                                  inp.dt_bias, inp.cu_seqlens, inp.h0, stream=cap)
                with torch.cuda.graph(g, stream=cap):
                    for _ in range(per):
                        gstep()
            stream.wait_stream(cap)
            torch.cuda.synchronize()
            graphs[per] = g
        for per, g in graphs.items():
            plan.o.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(plan.o, o_eager):
                raise RuntimeError("graph replay (%d steps) differs from the eager step" % per)
        graph_ms = timed(graphs[1].replay, args.steps)
        reps = max(1, args.steps // GRAPH_PER)
        graph_many_ms = timed(graphs[GRAPH_PER].replay, reps) / GRAPH_PER
    except Exception as exc:  # graph capture is an extra view, not the headline
        print("graph timing skipped: %s" % exc, file=sys.stderr, flush=True)

    # per-kernel durations: each kernel alone, K back-to-back launches between two
    # events on the launch stream (gdn_fwd_stages re-runs one stage on the
    # workspace the full steps above left; results are unchanged by it)
    # (with the output fused into the state pass, the two run as one kernel,
    # "chain_out", timed with both stage bits)
    fused = gdn.fuses_output(plan.params, packed)
    B = gdn.STAGE_BITS
    stage_list = [(n, B[n]) for n in gdn.STAGES]
    if fused:
        stage_list = [("chunk_map", B["chunk_map"]), ("wy", B["wy"]),
                      ("chain_out", B["chain"] | B["output"])]
    stage_ms = []
    for name, bits in stage_list:
        if name == "chunk_map" and not packed:
            stage_ms.append(0.0)
            continue
        one = plan.bind(inp.q, inp.k, inp.v, inp.g_raw, inp.beta, inp.A_log, inp.dt_bias,
                        inp.cu_seqlens, inp.h0, stream=stream, stage_mask=bits)
        for _ in range(max(1, args.warmup)):
            one()
        stage_ms.append(timed(one, args.steps))

    dtype = cfg["dtype"]
    esz = 2 if dtype == "bf16" else 4
    sh = dict(s, packed=packed)
    used = plan.layout.num_slots
    if packed:
        lens = (inp_cpu.cu_seqlens[1:] - inp_cpu.cu_seqlens[:-1]).tolist()
        used = sum((L + CHUNK - 1) // CHUNK for L in lens)
    kern, path, ntok = algorithmic(sh, esz, inp.h0 is not None, used, fused)
    kernels = {}
    for (name, _), t in zip(stage_list, stage_ms):
        if name == "chunk_map" and not packed:
            continue
        kernels[name] = kernel_figures(kern[name], t, dtype)
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
        tk = traffic_key(wl, "gdn_fwd", args.seg_chunks)
        ent = tr.get(tk, {}).get(dom)
        if ent and ent.get("source_hash") == src:
            roof["traffic"] = ent["bytes_per_launch"]
            roof.update(kernel_counters(ent))
        # counter-measured MFMA utilisation and matrix flops of every kernel
        for name, k in kernels.items():
            e = tr.get(tk, {}).get(name)
            if e and e.get("source_hash") == src:
                k.update({"counters_" + a: b for a, b in kernel_counters(e).items()})
    sec = ms / 1e3
    out = {
        "metric": metric_label("gdn_fwd", cfg),
        "value": round(ntok / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "graph%d_ms_per_step" % GRAPH_PER: None if graph_many_ms is None
        else round(graph_many_ms, 5),
        "cold_ms_per_step": None if cold_ms is None else round(cold_ms, 5),
        "cold_tokens_per_s": None if cold_ms is None else round(ntok / (cold_ms / 1e3), 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl, "B": s["B"], "T": s["T"], "H": s["H"], "HV": s["HV"],
                   "K": s["K"], "V": s["V"], "chunk": CHUNK, "packed_seqs": s["N"] if packed
                   else None, "initial_state": inp.h0 is not None,
                   "seg_chunks": args.seg_chunks,
                   "seg_chunks_used": gdn.seg_chunks(plan.params, packed)},
        "output_fused": fused,
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
