"""bench.py host logic on the CPU: the one-GPU rule, the algorithmic byte and
flop counts the roofline uses, and the parsing of rocprofv3 counter CSVs into
traffic and MFMA figures (synthetic CSV files, no GPU)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_counts_at_the_pages_shape():
    # B=2, T=2048, H=HV=8, K=V=128, bf16, no initial state: 64 slots of 64 tokens
    shape = dict(B=2, T=2048, H=8, HV=8, K=128, V=128, N=2)
    kern, path, ntok = bench.algorithmic(shape, 2, False, 64)
    assert ntok == 4096
    U = 4096 * 8
    # the whole pass: q, k (per key head), v, o at 2 bytes, gates and beta, final state
    assert path["bytes"] == 2 * 4096 * 8 * 128 * 2 + U * 128 * 2 + U * 8 + U * 128 * 2 + 2 * 8 * 128 * 128 * 4
    # C(3K + 2V) + 6KV flops per token-head: 139,264 at C = 64, K = V = 128
    assert path["flops"] == U * 139264
    assert kern["chain"]["flops"] == U * 4 * 128 * 128
    # fused: the output's bytes move into the state pass, P^T and q into WY
    fk, fpath, _ = bench.algorithmic(shape, 2, False, 64, fused=True)
    assert set(fk) == {"chunk_map", "wy", "chain_out"}
    assert fpath == path
    p_bytes = 64 * 8 * 6 * 64 * 8 * 2
    assert fk["wy"]["bytes"] == kern["wy"]["bytes"] + 4096 * 8 * 128 * 2 + p_bytes


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow([i, kernel, counter, value])


def test_write_traffic_scales_counters_and_reads_mfma_passes(tmp_path, monkeypatch):
    d = str(tmp_path)
    wy = "_ZN3gdn13gdn_wy_kernelIDF16bLi128ELi128ELb0ELb0ELb0EEEv"
    chain = "_ZN3gdn21gdn_chain_ring_kernelIDF16bLi128ELi128ELb0ELi1ELi0EEEv"
    copy = "__amd_rocclr_copyBuffer"
    mib = 256 << 20
    # the copy reads FETCH_SIZE = half its bytes and WRITE_SIZE = all of them (KiB)
    _counter_csv(os.path.join(d, "copy_fetch", "c_counter_collection.csv"),
                 [(copy, "FETCH_SIZE", mib / 2048.0)])
    _counter_csv(os.path.join(d, "copy_write", "c_counter_collection.csv"),
                 [(copy, "WRITE_SIZE", mib / 1024.0)])
    _counter_csv(os.path.join(d, "fetch", "f_counter_collection.csv"),
                 [(wy, "FETCH_SIZE", 100.0), (wy, "FETCH_SIZE", 300.0), (chain, "FETCH_SIZE", 50.0)])
    _counter_csv(os.path.join(d, "write", "w_counter_collection.csv"),
                 [(wy, "WRITE_SIZE", 400.0), (chain, "WRITE_SIZE", 10.0)])
    _counter_csv(os.path.join(d, "mfma_util", "u_counter_collection.csv"),
                 [(wy, "MfmaUtil", 4.0), (wy, "MfmaUtil", 6.0), (chain, "MfmaUtil", 2.5)])
    _counter_csv(os.path.join(d, "mfma_flops", "m_counter_collection.csv"),
                 [(wy, "MfmaFlopsBF16", 1000.0), (wy, "MfmaFlopsF32", 24.0),
                  (chain, "MfmaFlopsBF16", 512.0)])
    out = os.path.join(d, "traffic.json")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", out)
    bench.write_traffic(d, "wl", mib)
    ent = json.load(open(out))["wl"]
    # mean per dispatch (KiB) x 1024 x calibration (2 for FETCH_SIZE, 1 for WRITE_SIZE)
    assert ent["wy"]["fetch_bytes"] == 200.0 * 1024 * 2
    assert ent["wy"]["write_bytes"] == 400.0 * 1024
    assert ent["wy"]["bytes_per_launch"] == 200 * 1024 * 2 + 400 * 1024
    assert ent["chain"]["bytes_per_launch"] == 50 * 1024 * 2 + 10 * 1024
    assert ent["wy"]["source_hash"] == bench.source_hash("gdn_fwd")
    assert bench.kernel_counters(ent["wy"]) == {"mfma_util": 0.05, "mfma_flops": 1024}
    assert bench.kernel_counters(ent["chain"]) == {"mfma_util": 0.025, "mfma_flops": 512}


def test_code_text_drops_comments_and_layout_only():
    src = 'int a; // note\nasm("s_waitcnt // kept");  /* block\n comment */ char c = \'/\';\n'
    assert bench.code_text(src) == 'int a; asm("s_waitcnt // kept"); char c = \'/\';'
    assert bench.code_text("x  =\n  y; // z") == bench.code_text("x = y;")
    assert bench.code_text("x = y;") != bench.code_text("x = z;")


def test_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    import shutil
    csrc = os.path.join(str(tmp_path), "gated_deltanet_chunkwise_amd", "csrc")
    shutil.copytree(os.path.join(ROOT, "gated_deltanet_chunkwise_amd", "csrc"), csrc)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.source_hash("decode")
    path = os.path.join(csrc, "gdn_decode.h")
    text = open(path).read()
    open(path, "w").write("// an added comment\n" + text.replace(";", "; /* c */", 1))
    assert bench.source_hash("decode") == base
    open(path, "w").write(text + "\nstatic int extra_symbol;\n")
    assert bench.source_hash("decode") != base


def test_source_hash_covers_each_op_only_with_its_sources():
    ops = ("gdn_fwd", "gdn_bwd", "kda_gate", "decode")
    hashes = {op: bench.source_hash(op) for op in ops}
    assert len(set(hashes.values())) == len(ops)
    for op in ops:
        for f in bench.OP_SOURCES[op]:
            assert os.path.exists(os.path.join(ROOT, "gated_deltanet_chunkwise_amd", "csrc", f))


def test_every_state_pass_variant_maps_to_its_stage(tmp_path):
    # each launchable state-pass kernel's counters must land on its stage, or
    # the bench line's traffic for that stage would be null
    names = {
        "_ZN3gdn21gdn_chain_ring_kernelIDF16bLi128ELi128ELb0ELi1ELi0EEEv": "chain",
        "_ZN3gdn16gdn_chain_kernelIDF16bLi128ELi128ELb0ELi0EEEv": "chain",
        "_ZN3gdn17gdn_chain2_kernelIDF16bLi128ELi128ELb0EEEv": "chain",
        "_ZN3gdn19gdn_chain_ks_kernelIfLi64ELi64ELb0ELi2EEEv": "chain",
        "_ZN3gdn20gdn_chain_out_kernelIDF16bLi128ELi128ELb0ELi2EEEv": "chain_out",
        "_ZN3gdn20gdn_bwd_chain_kernelIDF16bLi128ELi128ELb0EEEv": "bwd_chain",
        "_ZN3gdn23gdn_bwd_chain_ks_kernelIDF16bLi128ELi128ELb0ELi2EEEv": "bwd_chain",
    }
    for i, (kernel, stage) in enumerate(names.items()):
        path = os.path.join(str(tmp_path), "k%d.csv" % i)
        _counter_csv(path, [(kernel, "FETCH_SIZE", 8.0)])
        means, _ = bench.counter_means(path)
        assert means == {stage: 8.0}, kernel


def test_metric_names_the_measured_workload():
    from gated_deltanet_chunkwise_amd.inputs import WORKLOADS
    # the forward pass at the pages' shape carries the headline metric string
    assert bench.metric_label("gdn_fwd", WORKLOADS["pages_bf16"]) == bench.METRIC
    labels = {(op, wl): bench.metric_label(op, WORKLOADS[wl])
              for op in ("gdn_fwd", "gdn_bwd") for wl in WORKLOADS}
    assert len(set(labels.values())) == len(labels)
    assert labels[("gdn_bwd", "pages_bf16")].startswith("GDN chunk-bwd tokens/s (B=2,T=2048,H=8,")
    assert "B=4,T=8192,H=16,K=V=128,h0 bf16" in labels[("gdn_fwd", "wide_bf16_h0")]
    assert "packed T=32768 in 12 seqs,H=16" in labels[("gdn_fwd", "packed_bf16")]
    assert "B=1,T=65536,H=16,HV=32,K=V=128 bf16" in labels[("gdn_fwd", "long_gqa_bf16")]
    assert "K=V=64 fp32" in labels[("gdn_fwd", "tiny_fp32")]


@pytest.mark.parametrize("dtype,peak", [("bf16", 2.5e15), ("fp32", 157.3e12)])
def test_every_kernel_is_rated_against_its_own_dtype_peak(dtype, peak):
    """bf16 calls run every forward and backward product on the bf16 MFMA, so
    each stage's MFMA fraction is taken against the bf16 peak (and fp32 calls
    against the fp32 one)."""
    shape = dict(B=2, T=2048, H=8, HV=8, K=128, V=128, N=2)
    esz = 2 if dtype == "bf16" else 4
    kern, _, _ = bench.algorithmic_bwd(shape, esz, False, True, 64)
    for name in ("recompute", "prep", "bwd_chain", "dqk", "bwd_wy"):
        f = bench.kernel_figures(kern[name], 0.02, dtype)
        assert f["mfma_dtype"] == dtype
        assert f["mfma_frac"] == round(kern[name]["flops"] / 2e-5 / peak, 4), name
        assert f["hbm_frac"] == round(kern[name]["bytes"] / 2e-5 / 8.0e12, 4), name
    fwd, _, _ = bench.algorithmic(shape, esz, False, 64)
    for name in ("wy", "chain", "output"):
        assert bench.kernel_figures(fwd[name], 0.01, dtype)["mfma_frac"] == round(
            fwd[name]["flops"] / 1e-5 / peak, 4)


def test_traffic_keys_separate_configurations():
    """Counters of a run with segments, or of the backward, never stand in for
    the plain forward of the same workload (their kernels differ)."""
    assert bench.traffic_key("pages_bf16") == "pages_bf16"
    assert bench.traffic_key("pages_bf16", "gdn_bwd") == "pages_bf16:bwd"
    assert bench.traffic_key("pages_bf16", "gdn_bwd", -1) == "pages_bf16:bwd"
    assert bench.traffic_key("long_h2_bf16", "gdn_fwd", -1) == "long_h2_bf16:seg=auto"
    assert bench.traffic_key("long_h2_bf16", "gdn_fwd", 32) == "long_h2_bf16:seg=32"
    assert bench.traffic_key("decode", "decode") == "decode"
