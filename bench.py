"""Benchmark: one C4A decode step at 64K context on one MI355X.

A step is the whole hot path over one batch: index scores -> top-k select ->
sparse MLA decode (+ split merge), for B=32 queries, H=64 heads, 16384
compressed slots per sequence (context 65536, ratio 4), top-k 512, SWA 128,
indexer 64 heads x 128 dims, 64-row paged blocks with permuted tables.
Inputs are resident in HBM before timing; the step cycles through several
independent input replicas so the 256 MB last-level cache cannot hold them.

Prints one JSON line (see the repository's measurement notes for fields).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode queries/s + achieved HBM GB/s (C4A, 64K ctx, 1 GPU)"
HBM_PEAK_GBPS = 8000.0

B, H, CTX, SLOTS, K, W, HI = 32, 64, 65536, 16384, 512, 128, 64

# algorithmic bytes (each byte the step must move once)
IDX_BYTES_PER_SLOT = 128 + 4 + 4            # key codes + key scale + score written
IDX_BYTES_PER_QUERY = HI * 128 + HI * 8     # index query codes + scale + weight
TOPK_BYTES_PER_QUERY = SLOTS * 4 + K * 4 + 4
ATTN_BYTES_PER_QUERY = (H * 576 * 2 + W * 1152 + K * 672 + K * 4 + H * 512 * 2 + H * 4)
STEP_BYTES = B * (SLOTS * 132 + IDX_BYTES_PER_QUERY + K * 4 + ATTN_BYTES_PER_QUERY)
INDEX_KERNEL_BYTES = B * (SLOTS * IDX_BYTES_PER_SLOT + IDX_BYTES_PER_QUERY)
# ratio-4 compress of 4096 tokens: each token's kv (bf16) and score (fp32)
# rows of 576 read once, each of the 1024 slots written once (672 B)
COMPRESS_4K_BYTES = 4096 * (576 * 2 + 576 * 4) + 1024 * 672


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=6)
    ap.add_argument("--graph", type=int, default=1, help="replay the steps as a HIP graph")
    ap.add_argument("--graph-cycles", type=int, default=4,
                    help="passes over the replicas captured in the one graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=32, help="queries the oracle times")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain elementwise copy (y = -x, fp32) of this size, "
                         "the known-size kernel the HBM byte counters are scaled by")
    ap.add_argument("--workload", default="c4a_decode_64k",
                    choices=["c4a_decode_64k", "c4a_prefill_2k", "c128a_decode_128k",
                             "swaonly_decode_b64", "c4a_single_layer_4k",
                             "c4a_decode_64k_stages", "c4a_decode_64k_fp8swa",
                             "c4a_decode_64k_fp4keys", "c4a_decode_64k_fp8swa_fp4keys",
                             "c4a_compress_stream_b32"],
                    help="c4a_decode_64k is the headline; the others print supplementary "
                         "per-stage timings of the same kernels on the other workloads")
    ap.add_argument("--report-stats", nargs=2, metavar=("TRACE_DIR", "OUT_MD"),
                    help="summarise a rocprofv3 --stats csv directory into OUT_MD and exit")
    ap.add_argument("--report-counters", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_STEM"),
                    help="turn FETCH_SIZE / WRITE_SIZE csv runs into OUT_STEM.json/.md and exit")
    ap.add_argument("--report-mfma", nargs=2, metavar=("PMC_DIR", "OUT_STEM"),
                    help="turn an MFMA counter run (MfmaUtil, SQ_INSTS_VALU_MFMA_MOPS_BF16, "
                         "SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE) into OUT_STEM.json/.md and exit")
    ap.add_argument("--cmd", action="append", default=[],
                    help="a command recorded verbatim in a report (repeatable)")
    return ap.parse_args()


PROBE_SRC = os.path.join(ROOT, "bench_probe.hip")
PROBE_LIB = os.path.join(ROOT, "bench_probe.so")


def build_probe() -> str:
    """Compile the measurement-only streaming-read probe (bench_probe.hip) for
    gfx950 into bench_probe.so beside this file; the library never holds it."""
    import subprocess
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on bench_probe.hip:\n" + r.stdout + r.stderr)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


_probe = None


def stream_read(buf, sink) -> None:
    """Read every byte of the device tensor buf once on torch's current stream
    (bench_probe.so; sink: int32 [workgroups] on the same device)."""
    global _probe
    import ctypes as C
    import torch
    if _probe is None:
        if not os.path.exists(PROBE_LIB):
            raise ImportError(f"{PROBE_LIB} is missing: run __graft_entry__.build()")
        _probe = C.CDLL(PROBE_LIB)
        _probe.bench_stream_read.restype = C.c_int
        _probe.bench_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int,
                                             C.c_void_p]
    rc = _probe.bench_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                  sink.data_ptr(), sink.numel(),
                                  torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"bench_stream_read failed ({rc})")


def kernel_source_hash(name: str = "index.hip") -> str:
    p = os.path.join(ROOT, "sparse_long_context_compressor_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


# the source file each library kernel is built from (for tying counter
# summaries to the code they were taken on)
KERNEL_SOURCES = {"index_score_kernel": "index.hip", "index_score_mq_kernel": "index.hip",
                  "topk_kernel": "topk.hip",
                  "topk_warm_kernel": "topk.hip", "topk_small_kernel": "topk.hip",
                  "topk_long_kernel": "topk.hip", "mla_decode_kernel": "decode.hip",
                  "mla_combine_kernel": "attention.hip", "mla_prefill_kernel": "attention.hip",
                  "compress_r4_kernel": "compress.hip", "compress_r128_kernel": "compress.hip"}


def _kernel_key(name: str) -> str:
    """slc::mla_decode_kernel<2, false>(slc::AttnArgs) -> mla_decode_kernel"""
    base = name.split("(")[0].replace("void ", "").strip()
    return base.split("::")[-1].split("<")[0]


def traffic_from_profile():
    """HBM bytes per index-score launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "index_score_c4a_decode_64k_counters.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("index_hip_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _short(name: str) -> str:
    name = name.split("(")[0] if not name.startswith("void at::") else name[:60]
    return name.replace("void ", "").strip()


def report_stats(trace_dir: str, out_md: str, cmds, workload: str = "c4a_decode_64k"):
    """Kernel-time summary of one rocprofv3 --kernel-trace --stats run."""
    rows = _csv_rows(trace_dir, "kernel_stats.csv")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# Kernel time, {workload} benchmark (rocprofv3 kernel trace)", "",
             "Made by:", ""] + [f"    {c}" for c in cmds] + [
        "", "| kernel | calls | avg us | min us | max us | share of GPU time |",
        "|---|---:|---:|---:|---:|---:|"]
    ours = [r for r in rows if "slc::" in r["Name"]]
    for r in ours:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    rest = sum(float(r["Percentage"]) for r in rows if r not in ours)
    lines += ["", f"The remaining {rest:.1f}% of GPU time is torch kernels that generate the "
                  "synthetic inputs before timing starts."]
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def report_counters(fetch_dir: str, write_dir: str, stem: str, calib_mib: int, cmds,
                    workload: str = "c4a_decode_64k"):
    """HBM bytes per launch of every library kernel in a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch), each scaled by the same counter's
    reading for a plain fp32 elementwise copy that reads and writes calib_mib
    MiB.  Writes OUT_STEM.json / .md; for the headline workload the index
    kernel's record (the bench line's `traffic`) keeps its own file."""
    if calib_mib <= 0:
        raise SystemExit("--calib-copy-mib must give the calibration copy's size")

    def per_kernel(d, counter):
        vals = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] == counter:
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        out = {}
        for (name, _), v in vals.items():
            out.setdefault(name, []).append(v)
        return {n: (sum(v) / len(v), len(v), min(v), max(v)) for n, v in out.items()}

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    cp = [n for n in fetch if "neg_kernel" in n]
    cpw = [n for n in write if "neg_kernel" in n]
    if not cp or not cpw:
        raise SystemExit("no calibration copy (neg_kernel) in the counter runs")
    known = calib_mib * 1024.0                      # KiB read = KiB written by the copy
    f_cp, w_cp = fetch[cp[0]][0], write[cpw[0]][0]
    kf, kw = known / f_cp, known / w_cp
    # algorithmic bytes per launch where this file states them
    algo = {}
    if workload == "c4a_decode_64k":
        algo = {"slc::index_score_kernel<4, 2, false>": INDEX_KERNEL_BYTES,
                # the step's select + decode call: the attention's bytes plus
                # the score rows it selects from
                "slc::mla_decode_kernel<2, false, true> + slc::mla_combine_kernel<4>":
                    B * (ATTN_BYTES_PER_QUERY + SLOTS * 4 + 4),
                "slc::mla_decode_kernel<2, false, false> + slc::mla_combine_kernel<4>":
                    B * ATTN_BYTES_PER_QUERY}
    elif workload == "c4a_single_layer_4k":
        algo = {"slc::compress_r4_kernel": COMPRESS_4K_BYTES}
    kernels = {}
    for name in sorted(fetch):
        if "slc::" not in name or name not in write:
            continue
        key = _short(name)
        base = _kernel_key(name)
        f, w = fetch[name], write[name]
        kernels[key] = {"name": _short(name), "fetch_kib": f[0], "write_kib": w[0],
                        "dispatches": [f[1], w[1]], "fetch_range_kib": [f[2], f[3]],
                        "hbm_read_bytes": f[0] * kf * 1024.0,
                        "hbm_write_bytes": w[0] * kw * 1024.0,
                        "source": KERNEL_SOURCES.get(base),
                        "source_sha256_16": kernel_source_hash(KERNEL_SOURCES[base])
                        if base in KERNEL_SOURCES else None}
        kernels[key]["hbm_bytes"] = kernels[key]["hbm_read_bytes"] + kernels[key]["hbm_write_bytes"]
    groups = {}
    for label, ab in algo.items():
        parts = [k.strip() for k in label.split("+")]
        if all(p_ in kernels for p_ in parts):
            t = sum(kernels[p_]["hbm_bytes"] for p_ in parts)
            groups[label] = {"hbm_bytes": t, "algorithmic_bytes": ab, "ratio": t / ab}
    calib = {"copy_mib": calib_mib, "fetch_kib": f_cp, "write_kib": w_cp,
             "fetch_factor": kf, "write_factor": kw}
    json.dump({"workload": workload, "kernels": kernels, "vs_algorithmic": groups,
               "calibration": calib, "commands": cmds}, open(stem + ".json", "w"), indent=1)
    md = [f"# HBM traffic per launch, {workload} (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
          "Made by:", ""] + [f"    {c}" for c in cmds] + [
        "", f"Calibration: a plain fp32 copy of {calib_mib} MiB reads FETCH_SIZE {f_cp:.0f} KiB "
            f"and WRITE_SIZE {w_cp:.0f} KiB, so the counters are scaled by {kf:.4f} (read) and "
            f"{kw:.4f} (write).", "",
        "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB | source sha256[:16] |",
        "|---|---:|---:|---:|---:|---:|---|"]
    for key, k in kernels.items():
        md.append(f"| `{k['name']}` | {k['dispatches'][0]} | {k['fetch_kib']:.0f} | {k['write_kib']:.0f} | "
                  f"{k['hbm_read_bytes'] / 1e6:.2f} | {k['hbm_write_bytes'] / 1e6:.2f} | "
                  f"{k['source']} {k['source_sha256_16']} |")
    if groups:
        md += ["", "| against the algorithmic bytes | HBM MB | algorithmic MB | ratio |",
               "|---|---:|---:|---:|"]
        for label, gr in groups.items():
            md.append(f"| {label} | {gr['hbm_bytes'] / 1e6:.2f} | {gr['algorithmic_bytes'] / 1e6:.2f} | "
                      f"{gr['ratio']:.3f} |")
    open(stem + ".md", "w").write("\n".join(md) + "\n")
    print("\n".join(md))
    if workload == "c4a_decode_64k" and "slc::index_score_kernel<4, 2, false>" in kernels:
        k = kernels["slc::index_score_kernel<4, 2, false>"]
        rec = {"kernel": "index_score_kernel", "workload": workload,
               "fetch_kib_per_dispatch": k["fetch_kib"], "write_kib_per_dispatch": k["write_kib"],
               "dispatches": k["dispatches"], "calibration": calib,
               "hbm_bytes_per_launch": k["hbm_bytes"], "algorithmic_bytes_per_launch": INDEX_KERNEL_BYTES,
               "traffic_over_algorithmic": k["hbm_bytes"] / INDEX_KERNEL_BYTES,
               "index_hip_sha256_16": kernel_source_hash(), "commands": cmds}
        d = os.path.dirname(stem) or "."
        json.dump(rec, open(os.path.join(d, "index_score_c4a_decode_64k_counters.json"), "w"), indent=1)


def report_mfma(pmc_dir: str, stem: str, cmds, workload: str):
    """MFMA use per library kernel from one counter run: MfmaUtil (rocprofv3's
    derived percentage: MFMA-busy SIMD cycles over active cycles times SIMDs),
    the bf16 MFMA work (SQ_INSTS_VALU_MFMA_MOPS_BF16, in units of 512 FLOP),
    means per dispatch.  Writes OUT_STEM.json / .md."""
    vals = {}
    for r in _csv_rows(pmc_dir, "counter_collection.csv"):
        key = (r["Kernel_Name"], r["Dispatch_Id"], r["Counter_Name"])
        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    per = {}
    for (name, disp, ctr), v in vals.items():
        if "slc::" in name:
            per.setdefault(name, {}).setdefault(ctr, []).append(v)
    kernels = {}
    for name, ctrs in per.items():
        key = _kernel_key(name)
        mean = {c: sum(v) / len(v) for c, v in ctrs.items()}
        kernels[key] = {"name": _short(name), "dispatches": max(len(v) for v in ctrs.values()),
                        "mfma_util_pct": mean.get("MfmaUtil"),
                        "bf16_mfma_flop": mean.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512.0,
                        "mfma_busy_cycles_sum": mean.get("SQ_VALU_MFMA_BUSY_CYCLES"),
                        "grbm_gui_active": mean.get("GRBM_GUI_ACTIVE"),
                        "source": KERNEL_SOURCES.get(key),
                        "source_sha256_16": kernel_source_hash(KERNEL_SOURCES[key])
                        if key in KERNEL_SOURCES else None}
    json.dump({"workload": workload, "kernels": kernels, "commands": cmds},
              open(stem + ".json", "w"), indent=1)
    md = [f"# MFMA use per launch, {workload} (rocprofv3 counters)", "", "Made by:", ""] + \
         [f"    {c}" for c in cmds] + [
        "", "MfmaUtil is rocprofv3's derived counter: the SIMDs' summed MFMA-busy cycles "
            "(SQ_VALU_MFMA_BUSY_CYCLES) over the kernel's active cycles (GRBM_GUI_ACTIVE, "
            "largest over the XCDs) times the 1024 SIMDs, in per cent. The bf16 MFMA work is "
            "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOP.", "",
        "| kernel | dispatches | MfmaUtil % | bf16 MFMA GFLOP per launch | source sha256[:16] |",
        "|---|---:|---:|---:|---|"]
    for key, k in kernels.items():
        u = k["mfma_util_pct"]
        md.append(f"| `{k['name']}` | {k['dispatches']} | {u:.1f} | {k['bf16_mfma_flop'] / 1e9:.1f} | "
                  f"{k['source']} {k['source_sha256_16']} |" if u is not None else
                  f"| `{k['name']}` | {k['dispatches']} | - | {k['bf16_mfma_flop'] / 1e9:.1f} | "
                  f"{k['source']} {k['source_sha256_16']} |")
    open(stem + ".md", "w").write("\n".join(md) + "\n")
    print("\n".join(md))


def mfma_from_profile(workload: str):
    """MfmaUtil per kernel from the committed counter summary of a workload,
    for kernels whose source is unchanged since it was taken; else None."""
    p = os.path.join(ROOT, "profiles", f"mfma_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    out = {}
    for key, k in d.get("kernels", {}).items():
        src = k.get("source")
        if src and k.get("source_sha256_16") == kernel_source_hash(src) and k.get("mfma_util_pct") is not None:
            out[key] = k["mfma_util_pct"] / 100.0
    return out or None


def cpu_baseline(n_q: int):
    """The oracle (as it stands) on a bounded sample: n_q sequences of the same
    workload shape, index top-k then attention, on the host's cores."""
    import numpy as np  # noqa: F401
    import oracle as O
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import oracle_attention, oracle_index_topk
    from sparse_long_context_compressor_amd import inputs as I
    lay = I.c4a_decode_64k(seed=2, device="cpu", batch=n_q)
    passes, t0 = 0, time.perf_counter()
    while passes == 0 or time.perf_counter() - t0 < 10.0:     # about 10 s of CPU work
        idx, _ = oracle_index_topk(O, lay, want_scores=False)
        oracle_attention(O, lay, idx)
        passes += 1
    dt = time.perf_counter() - t0
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": passes * n_q / dt, "unit": "queries/s", "cores": int(O.num_threads()),
            "kind": "oracle", "cpu_model": model,
            "sample": f"{passes} passes over {n_q} of the 32 sequences (one query each, same "
                      f"shapes: 16384 slots, H_I=64, k=512, H=64, SWA 128), index top-k + "
                      f"attention, {dt:.2f} s wall"}


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


BF16_PEAK_TFLOPS = 2500.0


def other_workload(args):
    """Per-stage timings of one pass over a non-headline workload (synthetic,
    inputs resident, replicas cycled): one JSON line."""
    import torch
    from sparse_long_context_compressor_amd import inputs as I
    from sparse_long_context_compressor_amd import slc
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    slc.lib()
    name = args.workload
    n_rep = 2 if name == "c4a_prefill_2k" else args.replicas
    fp8, fp4 = "fp8swa" in name, "fp4keys" in name
    if name.startswith("c4a_decode_64k_"):
        # the headline workload with per-stage timings (stages), with its SWA
        # pool in fp8 rows (fp8swa), with MXFP4 index keys (fp4keys)
        reps = [I.c4a_decode_64k(seed=200 + r, device=dev, swa_fp8=fp8, key_fp4=fp4)
                for r in range(n_rep)]
    else:
        reps = [I.CONFIGS[name](seed=200 + r, device=dev) for r in range(n_rep)]
    fl = slc.SWA_FP8 if fp8 else 0
    kf = slc.KEY_MXFP4 if fp4 else 0
    torch.cuda.synchronize()
    log(f"{n_rep} input replicas of {name} resident")
    lay0 = reps[0]
    Q, Hh, Ww, Kk, HIi, r = lay0.n_q, lay0.H, lay0.W, lay0.k, lay0.H_I, lay0.ratio
    ms_ = lay0.max_slots
    decode = name != "c4a_prefill_2k"
    stages = {}
    if name == "c4a_single_layer_4k":
        def compress(lay):
            slc.compress(4, lay.cu_seqlens, 4096, lay.kv, lay.score, lay.gamma, lay.eps,
                         lay.cos_sin, lay.cmp_pool, lay.cmp_table)
        stages["compress"] = compress
    if r == 4 and HIi > 0:
        sc = torch.empty((Q, ms_), dtype=torch.float32, device=dev)
        idx = torch.empty((Q, Kk), dtype=torch.int32, device=dev)
        ln = torch.empty(Q, dtype=torch.int32, device=dev)

        def index_scores(lay):
            slc.index_scores(lay.qi, lay.qi_scale, lay.qi_w, lay.q_seq, lay.q_pos, 4 | kf,
                             lay.key_pool, lay.key_table, lay.n_slots, ms_, sc)

        def topk(lay):
            if decode:      # with the decode's L2 warm-up, as the headline step runs it
                slc.topk_select_warm(Kk, sc, ms_, lay.q_seq, lay.q_pos, 4 | fl, lay.n_slots, idx,
                                     ln, lay.q, Ww, lay.swa_pool, lay.swa_table)
            else:
                slc.topk_select(Kk, sc, ms_, lay.q_seq, lay.q_pos, 4, lay.n_slots, idx, ln)
        stages["index_scores"] = index_scores
        stages["topk_select"] = topk
        get_idx = lambda lay: idx  # noqa: E731
    else:
        get_idx = lambda lay: lay.given_idx  # noqa: E731
    out = torch.empty((Q, Hh, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Q, Hh), dtype=torch.float32, device=dev)
    ws = torch.empty(max(slc.sparse_mla_workspace_size(decode, Q, Hh, Ww, Kk), 256),
                     dtype=torch.uint8, device=dev)
    f = slc.sparse_mla_decode if decode else slc.sparse_mla_prefill

    def attention(lay):
        if r == 1:
            f(1 | fl, lay.q, lay.q_seq, lay.q_pos, Ww, lay.swa_pool, lay.swa_table,
              sm_scale=lay.sm_scale, out=out, lse=lse, workspace=ws)
        else:
            f(r | fl, lay.q, lay.q_seq, lay.q_pos, Ww, lay.swa_pool, lay.swa_table, lay.cmp_pool,
              lay.cmp_table, get_idx(lay), lay.n_slots, lay.sm_scale, out, lse, ws)
    stages["sparse_mla_decode" if decode else "sparse_mla_prefill"] = attention
    fused = decode and r == 4 and HIi > 0

    def topk_decode(lay):
        # the select and the decode over its list in one call
        slc.sparse_mla_decode_topk(4 | fl, lay.q, lay.q_seq, lay.q_pos, Ww, lay.swa_pool,
                                   lay.swa_table, lay.cmp_pool, lay.cmp_table, Kk, sc, ms_,
                                   lay.n_slots, idx, ln, lay.sm_scale, out, lse, ws)
    if fused:
        stages["sparse_mla_decode_topk"] = topk_decode

    def step_calls(lay):
        for k_, fn in stages.items():
            if k_ != "sparse_mla_decode_topk":
                fn(lay)

    def step(lay):
        if fused:
            # the step as the library's fastest form: (compress,) index, then
            # the select and decode in one call
            for k_, fn in stages.items():
                if k_ not in ("topk_select", "sparse_mla_decode"):
                    fn(lay)
        else:
            step_calls(lay)

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            fn(reps[i % len(reps)])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def graph_timed(fn, n):
        """ms per call of fn as replays of a graph of back-to-back calls over the
        replicas (an eager loop of one short op is bound by the host)."""
        per_graph = len(reps) * 4
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for rr in reps:
                fn(rr)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(per_graph):
                fn(reps[i % len(reps)])
        g.replay()
        torch.cuda.synchronize()
        n_rep = max(1, n // per_graph)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_rep):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (n_rep * per_graph)

    steps = max(10, args.steps // (10 if name == "c4a_prefill_2k" else 1))
    for i in range(args.warmup):
        step(reps[i % len(reps)])
    torch.cuda.synchronize()
    ms_step = timed(step, steps)
    long_ops = name == "c4a_prefill_2k"     # milliseconds per op: eager launches suffice
    per = {k: (timed if long_ops else graph_timed)(fn, steps) * 1e3 for k, fn in stages.items()}
    rec = {"workload": name, "queries": Q, "heads": Hh, "window": Ww, "topk": Kk,
           "ms_per_pass": ms_step, "queries_per_s": Q / (ms_step * 1e-3), "stages_us": per,
           "stages_timing": "eager_launches" if long_ops else "graph_replay",
           "steps": steps, "data": "synthetic"}
    if fused:
        rec["ms_per_pass_three_calls"] = timed(step_calls, steps)
        rec["graph_ms_per_pass"] = graph_timed(step, steps)
    # algorithmic bytes / flops of the attention stage
    n_cmp = Kk if r > 1 else 0
    att_us = per["sparse_mla_decode" if decode else "sparse_mla_prefill"]
    if "index_scores" in per and decode:
        # algorithmic bytes of the index stage: every visible key (132 B fp8,
        # 68 B MXFP4) plus the query's heads, weights and scales
        key_b = 68 if fp4 else 132
        nv_tot = float(sum(min(int(lay0.n_slots[int(s)]), (int(p) + 1) // 4)
                           for s, p in zip(lay0.q_seq.tolist(), lay0.q_pos.tolist())))
        ib = nv_tot * key_b + Q * HIi * (128 + 8)
        rec["index_GBps"] = ib / (per["index_scores"] * 1e-6) / 1e9
        rec["index_hbm_frac"] = rec["index_GBps"] / HBM_PEAK_GBPS
        # IndexCache freq 2: every other ratio-4 layer reuses the previous
        # layer's list and runs the attention alone
        rec["indexcache_freq2_us_per_layer"] = (ms_step * 1e3 + att_us) / 2
    if decode:
        cmp_row = 672
        swa_row = 672 if fp8 else 1152
        b = Q * (Hh * 576 * 2 + Ww * swa_row + n_cmp * (cmp_row + 4) + Hh * 512 * 2 + Hh * 4)
        rec["attention_GBps"] = b / (att_us * 1e-6) / 1e9
        rec["attention_hbm_frac"] = rec["attention_GBps"] / HBM_PEAK_GBPS
    else:
        flops = 2.0 * Q * Hh * (Ww + n_cmp) * (576 + 512)
        rec["attention_TFLOPs"] = flops / (att_us * 1e-6) / 1e12
        rec["attention_mfma_frac_bf16"] = rec["attention_TFLOPs"] / BF16_PEAK_TFLOPS
        if "index_scores" in per:
            import numpy as np
            nv = np.minimum(lay0.n_slots.cpu().numpy()[lay0.q_seq.cpu().numpy()],
                            (lay0.q_pos.cpu().numpy() + 1) // 4)
            iflops = 2.0 * float(nv.sum()) * HIi * 128
            rec["index_TFLOPs"] = iflops / (per["index_scores"] * 1e-6) / 1e12
            rec["index_mfma_frac_bf16"] = rec["index_TFLOPs"] / BF16_PEAK_TFLOPS
        # MFMA busy share per kernel from the committed counter run (null once
        # a kernel's source has changed since)
        rec["mfma_util"] = mfma_from_profile(name)
    if args.calib_copy_mib:
        # the known-size copy the HBM byte counters are scaled by
        a_ = torch.ones((args.calib_copy_mib << 20) // 4, dtype=torch.float32, device=dev)
        b_ = torch.empty_like(a_)
        torch.neg(a_, out=b_)
        torch.cuda.synchronize()
    print(json.dumps(rec), flush=True)


def compress_stream_workload(args):
    """The streaming compressor in a C4A decode: 32 sequences at 64K context,
    one new token each per step (positions 65532..65535 cycle, so one step in
    four emits a slot); per step the latent compressor and the indexer's key
    compressor, both with 4-row state blocks, one launch each (one token per
    sequence per call).  One JSON line."""
    import torch
    from sparse_long_context_compressor_amd import inputs as I
    from sparse_long_context_compressor_amd import pools as P
    from sparse_long_context_compressor_amd import slc
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    slc.lib()
    n, ctx = 32, 65536
    g = torch.Generator().manual_seed(7)
    kv = torch.randn((4, n, 1152), generator=g).to(torch.bfloat16).to(dev)
    sc = torch.randn((4, n, 1152), generator=g).to(dev)
    kv_i = torch.randn((4, n, 256), generator=g).to(torch.bfloat16).to(dev)
    sc_i = torch.randn((4, n, 256), generator=g).to(dev)
    ape = torch.randn((4, 1152), generator=g).to(dev)
    ape_i = torch.randn((4, 256), generator=g).to(dev)
    gamma, gamma_i = torch.ones(576, device=dev), torch.ones(128, device=dev)
    cs = I.rope_table(ctx, device=dev)
    blocks = ctx // 4
    st_table, n_st = I.block_table([list(range(blocks - 2, blocks))] * n, blocks, 8, "st", dev)
    state = torch.zeros((n_st, 4, 2304), device=dev)
    state_i = torch.zeros((n_st, 4, 512), device=dev)
    c_table, n_cb = I.block_table([list(range(256))] * n, 256, 9, "ct", dev)
    cmp_pool = P.cmp_pool_empty(n_cb, dev)
    key_pool = P.key_pool_empty(n_cb, dev)
    seq = torch.arange(n, dtype=torch.int32, device=dev)
    pos = [torch.full((n,), ctx - 4 + i, dtype=torch.int32, device=dev) for i in range(4)]

    def step(i):
        j = i % 4
        slc.compress_stream(4, seq, pos[j], kv[j], sc[j], ape, state, st_table, 4, gamma, 1e-6,
                            cs, cmp_pool, c_table, one_per_seq=True)
        slc.compress_index_keys_stream(seq, pos[j], kv_i[j], sc_i[j], ape_i, state_i, st_table, 4,
                                       gamma_i, 1e-6, cs, key_pool, c_table, one_per_seq=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    steps = 4 * max(1, args.steps // 4)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    # the same four steps captured once and replayed (no host work per call)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(4):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(4):
            step(i)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps // 4):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us_graph = e0.elapsed_time(e1) * 1e3 / steps

    # all of a step's writers in one launch: the new tokens' rows into an fp8
    # SWA pool plus both compressors (slc_decode_step_writers)
    swa_kv = torch.randn((4, n, 576), generator=g).to(torch.bfloat16).to(dev)
    swa_table, n_sb = I.block_table([[ctx // 64 - 1]] * n, ctx // 64, 10, "swa", dev)
    swa_pool = P.cmp_pool_empty(n_sb, dev)

    def writers(i):
        j = i % 4
        slc.decode_step_writers(
            seq, pos[j], cs, swa=dict(kv=swa_kv[j], pool=swa_pool, table=swa_table),
            latent=dict(ratio=4, kv=kv[j], score=sc[j], ape=ape, gamma=gamma, eps=1e-6,
                        state=state, state_table=st_table, state_block=4, pool=cmp_pool,
                        table=c_table),
            keys=dict(kv=kv_i[j], score=sc_i[j], ape=ape_i, gamma=gamma_i, eps=1e-6,
                      state=state_i, state_table=st_table, state_block=4, pool=key_pool,
                      table=c_table))
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(4):
            writers(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph2):
        for i in range(4):
            writers(i)
    for _ in range(3):
        graph2.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps // 4):
        graph2.replay()
    e1.record()
    torch.cuda.synchronize()
    us_writers = e0.elapsed_time(e1) * 1e3 / steps
    print(json.dumps({"workload": "c4a_compress_stream_b32", "sequences": n, "context": ctx,
                      "us_per_step": us, "graph_us_per_step": us_graph, "steps": steps,
                      "emitting_steps": "1 in 4", "calls_per_step": 2, "kernels_per_step": 2,
                      "writers_one_launch_graph_us_per_step": us_writers,
                      "writers_note": "SWA insert (fp8 pool) + both compressors, one launch",
                      "data": "synthetic"}), flush=True)


def main():
    args = parse()
    if args.report_stats:
        return report_stats(*args.report_stats, args.cmd, args.workload)
    if args.report_counters:
        return report_counters(*args.report_counters, args.calib_copy_mib, args.cmd, args.workload)
    if args.report_mfma:
        return report_mfma(*args.report_mfma, args.cmd, args.workload)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path shards by sequence with no exchange "
              "between GPUs, so one GPU's share at the real shape is the measurement. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.workload == "c4a_compress_stream_b32":
        return compress_stream_workload(args)
    if args.workload != "c4a_decode_64k":
        return other_workload(args)

    import torch
    from sparse_long_context_compressor_amd import inputs as I
    from sparse_long_context_compressor_amd import slc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    slc.lib()
    reps = [I.c4a_decode_64k(seed=100 + r, device=dev) for r in range(args.replicas)]
    torch.cuda.synchronize()
    log(f"{args.replicas} input replicas resident")

    scores = torch.empty((B, SLOTS), dtype=torch.float32, device=dev)
    idx = torch.empty((B, K), dtype=torch.int32, device=dev)
    ln = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws_bytes = slc.sparse_mla_workspace_size(True, B, H, W, K)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def index_scores(lay):
        slc.index_scores(lay.qi, lay.qi_scale, lay.qi_w, lay.q_seq, lay.q_pos, 4, lay.key_pool,
                         lay.key_table, lay.n_slots, SLOTS, scores)

    def topk(lay):
        # the select plus the decode's L2 warm-up (its queries and window rows
        # are read beside the select, into the L2 the decode then reads)
        slc.topk_select_warm(K, scores, SLOTS, lay.q_seq, lay.q_pos, 4, lay.n_slots, idx, ln,
                             lay.q, W, lay.swa_pool, lay.swa_table)

    def decode(lay):
        slc.sparse_mla_decode(4, lay.q, lay.q_seq, lay.q_pos, W, lay.swa_pool, lay.swa_table,
                              lay.cmp_pool, lay.cmp_table, idx, lay.n_slots, lay.sm_scale, out,
                              lse, ws)

    def topk_decode(lay):
        # the select and the decode over its list in one call (one launch
        # plus the merge of the splits)
        slc.sparse_mla_decode_topk(4, lay.q, lay.q_seq, lay.q_pos, W, lay.swa_pool, lay.swa_table,
                                   lay.cmp_pool, lay.cmp_table, K, scores, SLOTS, lay.n_slots, idx,
                                   ln, lay.sm_scale, out, lse, ws)

    def step(lay):
        index_scores(lay)
        topk_decode(lay)

    def step_separate(lay):
        # the same step as three calls: index, select (with the decode's L2
        # warm-up), decode
        index_scores(lay)
        topk(lay)
        decode(lay)

    def timed(fn, n):
        """Average ms of n back-to-back calls of fn(replica) bracketed by one event pair."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            fn(reps[i % len(reps)])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for i in range(args.warmup):
        step(reps[i % len(reps)])
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        # the K timed steps captured once, as one graph cycling the replicas
        # (a serving loop replays its decode step the same way); its first
        # replay is part of the warm-up
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for r in reps:
                step(r)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(reps[i % len(reps)])
        graph.replay()
        torch.cuda.synchronize()

    log("warm-up done")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # ---- K whole steps launched back to back, no event in between ----
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(reps[i % len(reps)])
    t_end.record()
    torch.cuda.synchronize()
    ms_step_eager = t_start.elapsed_time(t_end) / args.steps
    # ---- headline: the same K steps as one replay of the captured graph ----
    ms_step = ms_step_eager
    if graph is not None:
        torch.cuda.synchronize()
        t_start.record()
        graph.replay()
        t_end.record()
        torch.cuda.synchronize()
        ms_step = t_start.elapsed_time(t_end) / args.steps
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step_separate(reps[i % len(reps)])
    t_end.record()
    torch.cuda.synchronize()
    ms_step_separate = t_start.elapsed_time(t_end) / args.steps


    # ---- per-kernel: back-to-back launches of one op over the replicas, as
    # replays of a graph of that op alone (an eager loop of one short op is
    # bound by the host's launch rate, not by the GPU) ----
    per_graph = len(reps) * args.graph_cycles

    def graph_timed(fn, n):
        if not args.graph:
            return timed(fn, n)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for r in reps:
                fn(r)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(per_graph):
                fn(reps[i % len(reps)])
        g.replay()
        torch.cuda.synchronize()
        reps_n = max(1, n // per_graph)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps_n):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps_n * per_graph)

    idx_ms = graph_timed(index_scores, args.steps)
    topk_decode_ms = graph_timed(topk_decode, args.steps)
    topk_ms = graph_timed(topk, args.steps)
    attn_ms = graph_timed(decode, args.steps)

    if args.calib_copy_mib:
        a = torch.ones((args.calib_copy_mib << 20) // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()

    # practical HBM peaks of this GPU, outside the timed step: a streaming read
    # of 2 GiB (a sum) and a device-to-device copy of 1 GiB (read + write)
    def _rate(fn, nbytes, n=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(n):
            fn()
        c1.record()
        torch.cuda.synchronize()
        return nbytes * n / (c0.elapsed_time(c1) * 1e-3) / 1e9
    big = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)     # 16 workgroups per CU
    read_GBps = _rate(lambda: stream_read(big, sink), big.numel() * 4)
    half = big[: 1 << 28]
    dst_ = torch.empty_like(half)
    copy_GBps = _rate(lambda: dst_.copy_(half), 2 * half.numel() * 4)
    del big, half, dst_, sink

    log(f"timed: {ms_step * 1e3:.1f} us/step")
    achieved = INDEX_KERNEL_BYTES / (idx_ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": B / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c4a_decode_64k", "batch": B, "heads": H, "context": CTX,
                   "slots_per_seq": SLOTS, "topk": K, "window": W, "index_heads": HI,
                   "block_rows": 64, "replicas": args.replicas},
        "achieved_step_GBps": STEP_BYTES / (ms_step * 1e-3) / 1e9,
        "step_hbm_frac": STEP_BYTES / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "timing": "graph_replay" if graph is not None else "eager_launches",
        "eager_ms_per_step": ms_step_eager,
        "ms_per_step_three_calls": ms_step_separate,
        "kernels_us": {"index_scores": idx_ms * 1e3,
                       "sparse_mla_decode_topk": topk_decode_ms * 1e3,
                       "topk_select_separate": topk_ms * 1e3,
                       "sparse_mla_decode_separate": attn_ms * 1e3},
        "kernels_timing": "graph_replay" if args.graph else "eager_launches",
        "roofline": {"kernel": "index_score_kernel", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic_from_profile(), "algorithmic_bytes": INDEX_KERNEL_BYTES},
        "practical_peak": {"read_GBps": read_GBps, "copy_GBps": copy_GBps,
                           "what": "2 GiB streaming read (bench_probe.hip: one contiguous 512 KB region per workgroup, 8 non-temporal loads in flight per thread); 1 GiB torch device copy, read + write",
                           "index_frac_of_read": achieved / read_GBps,
                           "step_frac_of_read": STEP_BYTES / (ms_step * 1e-3) / 1e9 / read_GBps},
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on a sample")
        rec["cpu_baseline"] = cpu_baseline(args.cpu_sample)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
