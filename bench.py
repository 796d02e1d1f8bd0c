"""Throughput of the DSA hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: the
lightning-indexer scores, the causal top-k and the sparse MLA attention of one DSA layer
at T=65536, k=2048 (dsa_layer_stack with pattern "F": query chunks of scores -> top-k
into the index buffer -> attention over the selected keys).  The JSON line also carries
the batched-decode step (64 sequences x 65536 cached tokens, fp8 latent cache, FSS over
three layers), a roofline entry for the dominant kernel timed with HIP events on the
stream it runs on, per-kernel event timings, and the CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

METRIC = "query tokens/sec through indexer+top-k+sparse attn, T=65536 k=2048; decode tok/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_VALU_PEAK_TFLOPS = 157.3  # published fp32 vector peak (packed FMA)
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")


PROBE_LIB = os.path.join(ROOT, "libdsa_probe.so")
_probe_lib = None


def probe():
    """libdsa_probe.so (bench_probe.hip): the read and gather ceiling kernels."""
    global _probe_lib
    if _probe_lib is None:
        import ctypes

        if not os.path.exists(PROBE_LIB):
            raise ImportError(f"{PROBE_LIB} is missing: run `python -m deepseek_sparse_attention_amd.build`")
        L = ctypes.CDLL(PROBE_LIB)
        P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.probe_read.argtypes = [P, SZ, P, I, P]
        L.probe_gather.argtypes = [P, I, I64, P, I64, I, I, P, P]
        _probe_lib = L
    return _probe_lib


TRAFFIC_FILE = os.path.join(PROFILES, "hbm_traffic_t65536_and_decode.txt")


def _short(name):
    return name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def summarize_traffic(fetch_csv, write_csv, out_path=TRAFFIC_FILE):
    """Turn two rocprofv3 --pmc runs of `bench.py --copy-calibration` (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch) into the bytes per launch that each kernel moved between
    L2 and memory (the last-level cache or HBM), each counter scaled by what it reads for
    the plain 1 GiB device copy."""
    import collections
    import csv

    def per_kernel(path, counter):
        vals = collections.defaultdict(list)
        copy = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            n = r["Kernel_Name"]
            if "copyBuffer" in n or "copy_kernel" in n:
                copy.append(float(r["Counter_Value"]))
            elif "at::" not in n and ("dsa::" in n or "::gather_kernel<" in n or "::read_kernel(" in n):
                # one line per kernel and launch shape (grid size in threads)
                vals[f"{_short(n)} grid={r['Grid_Size']}"].append(float(r["Counter_Value"]))
        return vals, copy

    fv, fc = per_kernel(fetch_csv, "FETCH_SIZE")
    wv, wc = per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = 1 << 30
    f_scale = copy_bytes / (max(fc) * 1024.0)  # the copy reads 1 GiB
    w_scale = copy_bytes / (max(wc) * 1024.0)  # and writes 1 GiB
    lines = [
        "# Bytes each kernel moved between L2 and memory per launch (FETCH_SIZE + WRITE_SIZE, KiB per",
        "# dispatch, scaled by the counts of a plain 1 GiB device copy in the same run): the T=65536,",
        "# k=2048 prefill layer, the 64 x 65536 decode step and the bench's ceiling kernels",
        "# made by (from the repository root):",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d prof_out/fetch_D -o fetch -- "
        "python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-kl --copy-calibration",
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d prof_out/write_D -o write -- "
        "python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-kl --copy-calibration",
        "#   python3 bench.py --summarize-traffic <fetch csv> <write csv>",
        f"copy_fetch_kib: {max(fc):.1f}",
        f"copy_write_kib: {max(wc):.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"source_hash: {source_hash(*LIB_SOURCES)}",
        "# kernel grid=<threads> | dispatches | fetch bytes/launch | write bytes/launch | total bytes/launch",
    ]
    for name in sorted(set(fv) | set(wv), key=lambda n: -(sum(fv.get(n, [0])) / max(1, len(fv.get(n, [1]))))):
        f = fv.get(name, [0.0])
        w = wv.get(name, [0.0])
        fb = sum(f) / len(f) * 1024.0 * f_scale
        wb = sum(w) / len(w) * 1024.0 * w_scale
        lines.append(f"{name} | {len(f)} | {int(fb)} | {int(wb)} | {int(fb + wb)}")
    with open(out_path, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_FILE = os.path.join(PROFILES, "indexer_t65536_mfma_counters.txt")
MFMA_COUNTERS = "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU GRBM_GUI_ACTIVE"


def summarize_mfma(pmc_csv, trace_csv, out_path=MFMA_FILE):
    """MFMA counters of the indexer kernels (the fused route's filter and the score kernel)
    from a `rocprofv3 --pmc ... --kernel-trace` run of the prefill bench: bf16 MFMA work in
    FLOP (MOPS_BF16 counts units of 512), per-dispatch duration from the kernel trace, and
    the resulting rate against the 2.5 PFLOP/s peak; VALU instructions per MFMA."""
    import collections
    import csv

    dur = {}
    for r in csv.DictReader(open(trace_csv)):
        dur[r["Dispatch_Id"]] = (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-9
    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    seen = collections.defaultdict(set)
    for r in csv.DictReader(open(pmc_csv)):
        name = r["Kernel_Name"]
        key = ("fz_filter_kernel<16, 64>" if "fz_filter_kernel<16, 64>" in name else
               "index_scores_kernel<16, 64, false, 4, 0>" if "index_scores_kernel<16, 64, false, 4, 0>" in name else None)
        if key is None:
            continue
        agg[key][r["Counter_Name"]] += float(r["Counter_Value"])
        seen[key].add(r["Dispatch_Id"])
    lines = [
        "# bf16 MFMA counters of the indexer kernels at T=65536 (16 heads x 64, workload mla_t65536_k2048_sink)",
        "# command (from the repository root):",
        f"#   rocprofv3 --pmc {MFMA_COUNTERS} --kernel-trace --output-format csv "
        "-d prof_out/mfma_D -o mfma -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-decode --no-kl",
        "#   python3 bench.py --summarize-mfma <counter_collection csv> <kernel_trace csv>",
        "# flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; rate = flop / the dispatches' summed duration;",
        "# algorithmic indexer work of one layer: 2 x 16 x 64 x T(T+1)/2 = 4.398e12 flop",
    ]
    for key in ("fz_filter_kernel<16, 64>", "index_scores_kernel<16, 64, false, 4, 0>"):
        if key not in agg:
            continue
        c, ids = agg[key], seen[key]
        t = sum(dur.get(i, 0.0) for i in ids)
        flop = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        lines += [f"kernel: {key}", f"  dispatches: {len(ids)}", f"  seconds: {t:.6f}",
                  f"  mfma_flop: {flop:.4e}",
                  f"  tflops: {flop / t / 1e12 if t else 0:.1f}",
                  f"  frac_of_2.5_pflops: {flop / t / 2.5e15 if t else 0:.4f}",
                  f"  valu_insts_per_mfma: {c.get('SQ_INSTS_VALU', 0) / max(1.0, c.get('SQ_INSTS_MFMA', 0)):.2f}"]
        for n in sorted(c):
            lines.append(f"  {n}: {c[n]:.6g}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


STATS_FILE = os.path.join(PROFILES, "prefill_t65536_k2048_kernel_stats.txt")


def summarize_stats(stats_csv, out_path=STATS_FILE):
    """Turn a `rocprofv3 --kernel-trace --stats` run of the bench (its kernel_stats.csv, and the
    kernel_trace.csv beside it) into the per-kernel summary kept with the repository: one
    line per library kernel and launch shape (grid size in threads); torch's own
    input-generation kernels only enter the total."""
    import collections
    import csv

    total_ns = sum(float(r["TotalDurationNs"]) for r in csv.DictReader(open(stats_csv)))
    trace_csv = stats_csv.replace("kernel_stats.csv", "kernel_trace.csv")
    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        if "dsa::" not in r["Kernel_Name"]:
            continue
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        groups[(_short(r["Kernel_Name"]), grid)].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    lines = [
        "# rocprofv3 kernel-trace summary: one T=65536, k=2048 DSA layer (workload mla_t65536_k2048_sink),",
        "# the 64 x 65536 decode step (FSS over 3 layers; fp8, paged fp8 and MXFP4 latent caches) and",
        "# the indexer KL objective on the ablation shape (T=3072, top-512 and dense), on one MI355X",
        "# command (from the repository root):",
        "#   rocprofv3 --kernel-trace --stats --output-format csv -d prof_out/trace_D -o trace -- "
        "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline",
        "#   python3 bench.py --summarize-stats prof_out/trace_D/trace_kernel_stats.csv",
        "# calls: 1 warmup + 3 timed layer_stack steps (fused index/top-k: fz_sample, fz_threshold,",
        "# fz_filter, fz_select, fz_exact once each, then attention), 3 event-timed launches of each",
        "# kernel group (the unfused indexer and top-k once per query chunk, the fused group, the",
        "# unfused step), then the decode steps and the bench's timings of their parts, the per-layer",
        "# attention launches, then the KL objective (sparse and dense, with gradients).",
        "# mla_attn_wk_kernel<f, waves>: latent rows f = 0 bf16, 1 fp8, 2 MXFP4, four waves per row;",
        "# topk_seg_kernel + topk_merge_kernel: the decode rows' split top-k (segment lists, merge;",
        "# inside the decode step the held indexer builds the lists and the merge runs alone);",
        "# index_scores_kernel<H_I, d_I, paged, query tiles per wave, held score tiles per wave (0:",
        "# staged and written during the key stream)>.  grid = threads of the launch (the 64-row",
        "# decode: grouped 3-layer attention 49152, one layer in 4 key splits 65536; decode indexer",
        "# 131072)",
        "# columns: calls, average us, min us, max us, total ms, % of all GPU time, kernel, grid",
        "",
    ]
    for (name, grid), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(d):6d} {sum(d) / len(d) / 1e3:12.1f} {min(d) / 1e3:10.1f} {max(d) / 1e3:10.1f} "
                     f"{sum(d) / 1e6:10.2f} {100 * sum(d) / total_ns:6.2f}%  {name}  grid={grid}")
    lines += ["", f"# all kernels (incl. torch's input generation): {total_ns / 1e6:.1f} ms"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def run_configs(steps, warmup):
    """One timed step of each workload (A-E) through dsa_layer_stack, one JSON line each:
    the per-config measurements (the default run's single line is the headline)."""
    import torch

    import synth
    import deepseek_sparse_attention_amd as dsa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def selected(T, k):
        return k * T - k * (k - 1) // 2 if T >= k else T * (T + 1) // 2

    for key in "ABCDE":
        w = synth.workload(key)
        if w.decode:
            kc = synth.decode_indexer_cache(w, device=dev)
            layers = []
            for l in range(len(w.pattern)):
                d = synth.decode_layer_inputs(w, l, device=dev)
                if "q_idx" in d:
                    d["k_idx"] = kc
                layers.append(d)
            klen = torch.full((w.B,), w.T, dtype=torch.int32, device=dev)
            cache = torch.empty((w.B, 1, w.k), dtype=torch.int32, device=dev)
            ms = timed(lambda: dsa.layer_stack(w.pattern, layers, w.k, w.scale(), Dv=w.Dv, kv_len=klen,
                                               index_cache=cache))
            nF = w.pattern.count("F")
            nbytes = nF * w.B * w.T * (w.d_I * 2 + 4) + len(w.pattern) * w.B * w.k * (w.Dqk + 4)
            line = {"config": key, "workload": w.name, "ms_per_step": round(ms, 4), "value": round(w.B / (ms * 1e-3), 1),
                    "unit": "tokens/s", "algorithmic_bytes": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        else:
            layers = [synth.layer_inputs(w, l, device=dev) for l in range(len(w.pattern))]
            cache = torch.empty((w.B, w.T, w.k), dtype=torch.int32, device=dev)
            ms = timed(lambda: dsa.layer_stack(w.pattern, layers, w.k, w.scale(), Dv=w.Dv, index_cache=cache))
            nF, nL = w.pattern.count("F"), len(w.pattern)
            row = w.Hkv * (w.Dqk + (w.Dv if not w.mla else 0)) * 2  # gathered bytes per selected key
            gather = nL * selected(w.T, w.k) * row
            flops = nF * 2 * w.H_I * w.d_I * w.T * (w.T + 1) // 2
            line = {"config": key, "workload": w.name, "layers": nL, "pattern": w.pattern,
                    "ms_per_step": round(ms, 3), "value": round(w.T / (ms * 1e-3), 1), "unit": "query tokens/s",
                    "gather_bytes": gather, "gather_gbs": round(gather / (ms * 1e-3) / 1e9, 1),
                    "indexer_flops": flops}
        print(json.dumps(line), flush=True)
        del layers, cache
        torch.cuda.empty_cache()


def read_traffic():
    """Counter bytes per launch by kernel from the committed summary ({} once any library
    source changed since the counters were taken)."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    out, ok = {}, False
    for line in open(TRAFFIC_FILE):
        if line.startswith("source_hash:"):
            ok = line.split(":", 1)[1].strip() == source_hash(*LIB_SOURCES)
        elif not line.startswith("#") and line.count("|") == 4:
            name, _, _, _, tot = (x.strip() for x in line.split("|"))
            out[name] = int(tot)
    return out if ok else {}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--T", type=int, default=65536, help="prefill length (default: the named workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-kl", action="store_true", help="skip the indexer KL objective timings")
    ap.add_argument("--cpu-rows", type=int, default=1024, help="rows in the oracle's timed sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference dispatch for HBM counters)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM traffic summary from two rocprofv3 --pmc counter CSVs and exit")
    ap.add_argument("--configs", action="store_true",
                    help="time one step of each workload A-E (one JSON line each) instead of the headline")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_CSV", "TRACE_CSV"),
                    help="write the indexer MFMA counter summary under profiles/ and exit")
    ap.add_argument("--summarize-stats", metavar="STATS_CSV",
                    help="write the per-kernel summary from a rocprofv3 kernel_stats.csv and exit")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


LIB_SOURCES = ("api.hip", "indexer.hip", "topk.hip", "index_topk.hip", "attention.hip", "indexer_kl.hip", "common.hpp",
               "indexer_core.hpp", "internal.hpp", "selection.hpp", "seglist.hpp")


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "deepseek_sparse_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)
    if args.configs:
        run_configs(args.steps, args.warmup)
        return

    import torch

    import synth
    import deepseek_sparse_attention_amd as dsa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.workload("D", T=args.T)
    T, k = w.T, w.k
    log(f"generating workload {w.name} T={T} on the GPU")
    layer = synth.layer_inputs(w, 0, device=dev)
    kv_len = None
    idx_cache = torch.empty((1, T, k), dtype=torch.int32, device=dev)
    out = torch.empty((1, T, w.H, w.Dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, T, w.H), dtype=torch.float32, device=dev)
    layer["out"], layer["lse"] = out, lse
    shp = dsa._shape(1, T, T, w.H, w.Hkv, w.Dqk, w.Dv, k, w.scale(), dsa.KV_BF16, w.H_I, w.d_I)
    ws = torch.empty(max(1, dsa.workspace_size(shp, dsa.OP_STACK)), dtype=torch.uint8, device=dev)

    def step():
        dsa.layer_stack("F", [layer], k, w.scale(), Dv=w.Dv, index_cache=idx_cache, ws=ws)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt / args.steps * 1e3
    value = T / (dt / args.steps)
    log(f"prefill: {ms_step:.2f} ms/step, {value:.0f} q-tok/s")

    # ---- per-kernel event timings on the library's stream (torch's current stream)
    stream = torch.cuda.current_stream()
    reps = max(1, args.steps)

    def timed(fn):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / reps

    # the attention launch as the step runs it: the stack's attention over the index cache
    # the step wrote (top-k rows, each row's extent from its position)
    attn_ms = timed(lambda: dsa.layer_stack("S", [layer], k, w.scale(), Dv=w.Dv, index_cache=idx_cache, ws=ws,
                                            prefilled=True, topk_rows=True))
    Tc = dsa.stack_chunk_rows(shp)
    ld = (T + 63) // 64 * 64
    chunk = torch.empty((1, Tc, ld), dtype=torch.float32, device=dev)
    chunk_idx = torch.empty((1, Tc, k), dtype=torch.int32, device=dev)
    starts = list(range(0, T, Tc))
    kvl = [torch.tensor([r0 + min(Tc, T - r0)], dtype=torch.int32, device=dev) for r0 in starts]

    def indexer_all():
        for r0, kl in zip(starts, kvl):
            n = min(Tc, T - r0)
            dsa.index_scores(layer["q_idx"][:, r0:r0 + n], layer["k_idx"], layer["w_idx"][:, r0:r0 + n], kv_len=kl,
                             scores=chunk[:, :n], ld=ld)

    def topk_all():
        for r0, kl in zip(starts, kvl):
            n = min(Tc, T - r0)
            dsa.topk(chunk[:, :n], k, Tk=r0 + n, kv_len=kl, idx=chunk_idx[:, :n])

    indexer_ms = timed(indexer_all)
    topk_ms = timed(topk_all)  # (on the last chunk's scores: same row lengths per chunk)
    # the fused route the step takes (dsa_index_topk over all rows: sample, threshold, filter,
    # select, exact recompute of failed rows), and the step over score chunks for comparison
    fz_ws = torch.empty(max(1, dsa.workspace_size(shp, dsa.OP_INDEX_TOPK)), dtype=torch.uint8, device=dev)
    fused_ms = timed(lambda: dsa.index_topk(layer["q_idx"], layer["k_idx"], layer["w_idx"], k, idx=idx_cache,
                                            ws=fz_ws))
    del fz_ws
    unfused_step_ms = timed(lambda: dsa.layer_stack("F", [layer], k, w.scale(), Dv=w.Dv, index_cache=idx_cache,
                                                    ws=ws, unfused=True))

    # ---- roofline of the dominant kernel (sparse MLA attention).  Its contraction is MFMA
    # work (34,816 flop per selected key: 16 heads x 2 x (576 + 512)); its gathered rows
    # (1152 B per selected key) come mostly from L2 and the last-level cache (75.5 MB of
    # latent rows, each gathered ~2000 times), so the logical gather rate exceeds the HBM
    # peak and is held instead against the same gather without the arithmetic
    # (bench_probe.hip) on the kernel's own index rows.
    sel = k * T - k * (k - 1) // 2 if T >= k else T * (T + 1) // 2
    attn_bytes = sel * w.Dqk * 2 + T * w.H * w.Dqk * 2 + T * k * 4 + T * w.H * w.Dv * 2 + T * w.H * 4
    attn_flops = sel * w.H * 2 * (w.Dqk + w.Dv)
    logical = attn_bytes / (attn_ms * 1e-3) / 1e9
    traffic_all = read_traffic()
    # one resident workgroup per CU when the launch has more (row, head group) pairs
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    traffic = traffic_all.get(f"dsa::mla_attn_wk_kernel<0, 4> grid={min(T * w.H // 16, n_cu) * 256}")
    pl = probe()
    psum = torch.empty(T * 4, dtype=torch.int32, device=dev)

    def gather_probe():
        rc = pl.probe_gather(layer["kv"].data_ptr(), w.Dqk * 2, T, idx_cache.data_ptr(), T, k, 1, psum.data_ptr(),
                             stream.cuda_stream)
        assert rc == 0, rc

    probe_ms = timed(gather_probe)
    probe_logical = attn_bytes / (probe_ms * 1e-3) / 1e9
    rbuf = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    rsum = torch.empty(1024 * 256, dtype=torch.int32, device=dev)

    def read_probe():
        rc = pl.probe_read(rbuf.data_ptr(), rbuf.numel() // 4, rsum.data_ptr(), 1024, stream.cuda_stream)
        assert rc == 0, rc

    read_gbs = rbuf.numel() * 4 / (timed(read_probe) * 1e-3) / 1e9
    del rbuf, rsum, psum
    tflops = attn_flops / (attn_ms * 1e-3) / 1e12
    roofline = {"kernel": "mla_attn_wk_kernel (bf16 rows)", "bound": "mfma", "achieved": round(tflops, 1),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic, "flops": attn_flops, "ms_per_launch": round(attn_ms, 3),
                "gather": {"algorithmic_bytes": attn_bytes, "logical_gbs": round(logical, 1),
                           "probe_ms": round(probe_ms, 3), "probe_logical_gbs": round(probe_logical, 1),
                           "frac_of_probe": round(logical / probe_logical, 4),
                           "l2_to_memory_gbs": None if traffic is None else round(traffic / (attn_ms * 1e-3) / 1e9, 1)},
                "hbm_read_probe_gbs": round(read_gbs, 1)}
    pairs = T * (T + 1) // 2
    idx_flops = 2 * w.H_I * w.d_I * pairs
    kernels = {
        "indexer": {"ms": round(indexer_ms, 3), "tflops": round(idx_flops / (indexer_ms * 1e-3) / 1e12, 1),
                    "frac_mfma_bf16": round(idx_flops / (indexer_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "index_topk_fused": {"ms": round(fused_ms, 3),
                             "tflops": round(idx_flops / (fused_ms * 1e-3) / 1e12, 1)},
        "step_unfused": {"ms": round(unfused_step_ms, 3)},
        "topk": {"ms": round(topk_ms, 3),
                 "gbs": round((pairs * 4 + T * k * 4) / (topk_ms * 1e-3) / 1e9, 1)},
        "sparse_attn": {"ms": round(attn_ms, 3), "gbs_logical": round(logical, 1)},
    }
    # the platform's own bf16 GEMM (torch -> hipBLASLt) on random data, as context for the
    # indexer's MFMA fraction: a large square product and the indexer's contraction shape
    # ((query, head) rows x keys, K = d_I)
    def gemm_tflops(M, N, K):
        ga = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
        gb = torch.randn(K, N, device=dev, dtype=torch.bfloat16)
        ga @ gb
        ms = timed(lambda: ga @ gb)
        return round(2 * M * N * K / (ms * 1e-3) / 1e12, 1)

    ref_sq = gemm_tflops(8192, 8192, 8192)
    ref_idx = gemm_tflops(T * w.H_I // 4, 2048, w.d_I)
    kernels["reference_gemm_bf16"] = {"8192x8192x8192_tflops": ref_sq,
                                      f"{T * w.H_I // 4}x2048x{w.d_I}_tflops": ref_idx,
                                      "frac_mfma_bf16_square": round(ref_sq / MFMA_BF16_PEAK_TFLOPS, 4)}
    kernels["index_topk_fused"]["frac_of_square_gemm"] = round(kernels["index_topk_fused"]["tflops"] / ref_sq, 4)
    log(f"kernels: {kernels}")

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": 1, "T": T, "k": k, "pattern": "F", "indexer": f"{w.H_I}x{w.d_I}",
                   "heads": w.H, "dqk": w.Dqk, "dv": w.Dv, "chunk_rows": Tc},
        "roofline": roofline, "kernels": kernels,
    }

    if args.copy_calibration:  # a plain 1 GiB device copy: reference dispatch for HBM counters
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = a.numel() * 4
        del a, b

    # ---- batched decode: 64 x 65536 fp8 cache, FSS over 3 layers
    if not args.no_decode:
        del chunk, chunk_idx
        e = synth.workload("E")
        log(f"generating decode workload {e.name}")
        kc = synth.decode_indexer_cache(e, device=dev)
        dl = []
        for l in range(3):
            d = synth.decode_layer_inputs(e, l, device=dev)
            if "q_idx" in d:
                d["k_idx"] = kc
            dl.append(d)
        klen = torch.full((e.B,), e.T, dtype=torch.int32, device=dev)
        dcache = torch.empty((e.B, 1, e.k), dtype=torch.int32, device=dev)
        dshp = dsa._shape(e.B, 1, e.T, e.H, 1, e.Dqk, e.Dv, e.k, e.scale(), dsa.KV_FP8_E4M3, e.H_I, e.d_I, klen)
        dws = torch.empty(max(1, dsa.workspace_size(dshp, dsa.OP_STACK)), dtype=torch.uint8, device=dev)
        for L in dl:
            L["out"] = torch.empty((e.B, 1, e.H, e.Dv), dtype=torch.bfloat16, device=dev)
            L["lse"] = torch.empty((e.B, 1, e.H), dtype=torch.float32, device=dev)

        def dstep():
            dsa.layer_stack(e.pattern, dl, e.k, e.scale(), Dv=e.Dv, kv_len=klen, index_cache=dcache, ws=dws)

        for _ in range(args.warmup):
            dstep()
        torch.cuda.synchronize()
        # back-to-back steps, as a serving loop runs them (10 steps left ~17 us per step of
        # start-up and final synchronization in the figure)
        dsteps = max(args.steps, 100)
        t0 = time.perf_counter()
        for _ in range(dsteps):
            dstep()
        torch.cuda.synchronize()
        ddt = (time.perf_counter() - t0) / dsteps
        dbytes = e.B * e.T * e.d_I * 2 + e.B * e.T * 4 + 3 * e.B * e.k * (e.Dqk + 4)
        result["decode"] = {"workload": e.name, "value": round(e.B / ddt, 1), "unit": "tokens/s",
                            "ms_per_step": round(ddt * 1e3, 4), "steps": dsteps, "pattern": e.pattern,
                            "algorithmic_bytes": dbytes, "gbs": round(dbytes / ddt / 1e9, 1)}
        log(f"decode: {ddt * 1e3:.3f} ms/step, {e.B / ddt:.0f} tok/s")

        # the step's parts, event-timed: selection (indexer + top-k through dsa_index_topk,
        # scores in its workspace), top-k alone on those scores, and the three attention
        # layers alone (an "SSS" stack over the cached indices: one grouped launch and its
        # merge); each against the ceiling kernels of bench_probe.hip
        nrep = 10
        sshp = dsa._shape(e.B, 1, e.T, 1, 1, 1, 1, e.k, 1.0, dsa.KV_BF16, e.H_I, e.d_I, klen)
        sws = torch.empty(max(1, dsa.workspace_size(sshp, dsa.OP_INDEX_TOPK)), dtype=torch.uint8, device=dev)
        sidx = torch.empty_like(dcache)
        L0 = dl[0]

        def sel_batch():
            for _ in range(nrep):
                dsa.index_topk(L0["q_idx"], kc, L0["w_idx"], e.k, kv_len=klen, idx=sidx, ws=sws)

        sel_us = 1e3 * timed(sel_batch) / nrep
        dscores = dsa.index_scores(L0["q_idx"], kc, L0["w_idx"], kv_len=klen)
        tshp = dsa._shape(e.B, 1, e.T, 1, 1, 1, 1, e.k, 1.0, dsa.KV_BF16)
        tws = torch.empty(max(1, dsa.workspace_size(tshp, dsa.OP_TOPK)), dtype=torch.uint8, device=dev)

        def topk_batch():
            for _ in range(nrep):
                dsa.topk(dscores, e.k, kv_len=klen, idx=sidx, ws=tws)

        topk_us = 1e3 * timed(topk_batch) / nrep
        same_sel = bool(torch.equal(sidx, dcache))
        del dscores, sws, tws

        def attn3_batch():
            for _ in range(nrep):
                dsa.layer_stack("SSS", dl, e.k, e.scale(), Dv=e.Dv, kv_len=klen, index_cache=dcache, ws=dws,
                                prefilled=True, topk_rows=True)

        attn3_us = 1e3 * timed(attn3_batch) / nrep
        goff = (torch.arange(e.B, device=dev, dtype=torch.int32) * e.T).view(e.B, 1, 1)
        gidx = torch.where(dcache >= 0, dcache + goff, -1).to(torch.int32).contiguous()
        gsplit = 8  # workgroups per decode row, as the attention splits its keys
        gsum = torch.empty(e.B * gsplit * 4, dtype=torch.int32, device=dev)

        def gather3_batch():
            for _ in range(nrep):
                for L in dl:
                    rc = pl.probe_gather(L["kv"].data_ptr(), e.Dqk, e.B * e.T, gidx.data_ptr(), e.B, e.k, gsplit,
                                         gsum.data_ptr(), stream.cuda_stream)
                    assert rc == 0, rc

        gather3_us = 1e3 * timed(gather3_batch) / nrep
        del gidx, gsum
        key_bytes = e.B * e.T * e.d_I * 2
        score_bytes = e.B * e.T * 4 + e.B * e.k * 4
        attn3_bytes = 3 * (e.B * e.k * (e.Dqk + 4) + e.B * e.H * (e.Dqk * 2 + e.Dv * 2 + 4))
        idx_us = sel_us - topk_us

        def rate(nb, us, probe_gbs=None):
            g = nb / (us * 1e-6) / 1e9
            d = {"us": round(us, 2), "bytes": nb, "gbs": round(g, 1), "frac_of_hbm_peak": round(g / HBM_PEAK_GBS, 4),
                 "frac_of_read_probe": round(g / read_gbs, 4)}
            if probe_gbs:
                d["frac_of_gather_probe"] = round(g / probe_gbs, 4)
            return d

        gather3_gbs = attn3_bytes / (gather3_us * 1e-6) / 1e9
        decode_kernels = {"indexer": rate(key_bytes, idx_us), "topk": rate(score_bytes, topk_us),
                          "attention_3_layers": rate(attn3_bytes, attn3_us, gather3_gbs),
                          "gather_probe_3_layers_us": round(gather3_us, 2), "selection_matches_step": same_sel}
        result["decode"]["kernels"] = decode_kernels
        log(f"decode kernels: {decode_kernels}")

        # the same step over paged caches: the same rows in shuffled 64-token pages of shared
        # pools (one block table for every layer); must give the dense step's results
        page = 64
        nblk = e.T // page
        g = torch.Generator().manual_seed(4242)
        table = torch.randperm(e.B * nblk, generator=g).to(torch.int32).view(e.B, nblk).to(dev)

        def paged(dense):  # dense [B, T, ...] -> pool [B*T, ...] laid out by the table
            pool = torch.empty((e.B * nblk, page) + tuple(dense.shape[2:]), dtype=dense.dtype, device=dev)
            pool[table.flatten().long()] = dense.reshape((e.B * nblk, page) + tuple(dense.shape[2:]))
            return pool.reshape((e.B * nblk * page,) + tuple(dense.shape[2:]))

        pg = dsa.paged_kv(table, page, e.B * nblk)
        pl = []
        for L in dl:
            P = {"q": L["q"], "kv": paged(L["kv"][:, :, 0]), "kv_scale": paged(L["kv_scale"]),
                 "out": torch.empty_like(L["out"]), "lse": torch.empty_like(L["lse"])}
            if "q_idx" in L:
                P.update(q_idx=L["q_idx"], w_idx=L["w_idx"], k_idx=paged(kc))
            pl.append(P)
        pcache = torch.empty_like(dcache)
        pws = torch.empty(max(1, dsa.workspace_size(dshp, dsa.OP_STACK_PAGED)), dtype=torch.uint8, device=dev)

        def pstep():
            dsa.layer_stack(e.pattern, pl, e.k, e.scale(), Dv=e.Dv, kv_len=klen, index_cache=pcache, ws=pws,
                            pages=pg, Tk=e.T, H_I=e.H_I, d_I=e.d_I)

        for _ in range(max(1, args.warmup)):
            pstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(dsteps):
            pstep()
        torch.cuda.synchronize()
        pdt = (time.perf_counter() - t0) / dsteps
        same = bool(torch.equal(pcache, dcache) and all(torch.equal(a["out"], b["out"]) for a, b in zip(pl, dl)))
        result["decode"]["paged"] = {"page_size": page, "ms_per_step": round(pdt * 1e3, 4),
                                     "value": round(e.B / pdt, 1), "matches_dense": same}
        log(f"decode, paged caches: {pdt * 1e3:.3f} ms/step, {e.B / pdt:.0f} tok/s, matches dense: {same}")
        del pl, pws

        # the same step with MXFP4 latent caches drawn from the same values (320 bytes per key
        # instead of 576 + a 4-byte scale), and one layer's attention alone in both formats
        ml = []
        for l, L in enumerate(dl):
            mx = synth.decode_layer_inputs(e, l, device=dev, kv_format="mxfp4")
            M = {"q": L["q"], "kv": mx["kv"], "out": torch.empty_like(L["out"]), "lse": torch.empty_like(L["lse"])}
            if "q_idx" in L:
                M.update(q_idx=L["q_idx"], w_idx=L["w_idx"], k_idx=kc)
            ml.append(M)
            del mx
        mcache = torch.empty_like(dcache)
        mshp = dsa._shape(e.B, 1, e.T, e.H, 1, e.Dqk, e.Dv, e.k, e.scale(), dsa.KV_MXFP4, e.H_I, e.d_I, klen)
        mws = torch.empty(max(1, dsa.workspace_size(mshp, dsa.OP_STACK)), dtype=torch.uint8, device=dev)

        def mstep():
            dsa.layer_stack(e.pattern, ml, e.k, e.scale(), Dv=e.Dv, kv_len=klen, index_cache=mcache, ws=mws)

        for _ in range(max(1, args.warmup)):
            mstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(dsteps):
            mstep()
        torch.cuda.synchronize()
        mdt = (time.perf_counter() - t0) / dsteps
        result["decode"]["mxfp4"] = {"ms_per_step": round(mdt * 1e3, 4), "value": round(e.B / mdt, 1),
                                     "bytes_per_key": dsa.mxfp4_row_bytes(e.Dqk),
                                     "same_indices": bool(torch.equal(mcache, dcache))}
        log(f"decode, MXFP4 latent caches: {mdt * 1e3:.3f} ms/step, {e.B / mdt:.0f} tok/s")

        def attn_layer(L, kv_scale, row_bytes):
            def batch():  # back-to-back launches, so host work overlaps the kernels
                for _ in range(20):
                    dsa.sparse_attn(L["q"], L["kv"], dcache, e.scale(), kv_scale=kv_scale, Dv=e.Dv, out=L["out"],
                                    lse=L["lse"], ws=dws)
            us = 1e3 * timed(batch) / 20
            nb = (e.B * e.k * (row_bytes + 4) + e.B * e.H * (e.Dqk * 2 + e.Dv * 2 + 4))
            return {"us": round(us, 2), "algorithmic_bytes": nb, "gbs": round(nb / (us * 1e-6) / 1e9, 1)}

        result["decode"]["attn_layer"] = {"fp8": attn_layer(dl[1], dl[1]["kv_scale"], e.Dqk + 4),
                                          "mxfp4": attn_layer(ml[1], None, dsa.mxfp4_row_bytes(e.Dqk))}
        log(f"decode attention, one layer: {result['decode']['attn_layer']}")
        del kc, dl, ml, mws

    # ---- indexer KL objective on the ablation card's shape (indexer 2x16, four 32-wide
    # heads, T=3072): top-512 sparse rows and the dense warm-up over every causal key
    if not args.no_kl:
        a = synth.workload("A")
        la = synth.layer_inputs(a, indexer=True, device=dev)
        sa = dsa.index_scores(la["q_idx"], la["k_idx"], la["w_idx"])
        ia = dsa.topk(sa, a.k)
        del sa
        kin = [la[x] for x in ("q_idx", "k_idx", "w_idx", "q", "kv")]
        kout = dsa.indexer_kl(*kin, a.scale(), idx=ia)  # outputs reused by the timed calls
        kws = torch.empty(max(dsa.indexer_kl_workspace_size(a.B, a.T, a.T, a.H_I, a.d_I, kk=a.k),
                              dsa.indexer_kl_workspace_size(a.B, a.T, a.T, a.H_I, a.d_I)), dtype=torch.uint8,
                          device=dev)
        nrep = 20

        def kl_batch(ix):  # back-to-back launches, so host work overlaps the kernels
            for _ in range(nrep):
                dsa.indexer_kl(*kin, a.scale(), idx=ix, out=kout, ws=kws)

        sparse_ms = timed(lambda: kl_batch(ia)) / nrep
        dense_ms = timed(lambda: kl_batch(None)) / nrep
        pairs_sparse = sum(min(t + 1, a.k) for t in range(a.T))
        pairs_dense = a.T * (a.T + 1) // 2
        # fp32 flops per (row, key) pair: main logits twice (2 * H * 32 * 2), indexer dots
        # twice (2 * H_I * d_I * 2), then the dq and dk products (2 * H_I * d_I * 2)
        per_pair = 2 * a.H * a.Dqk * 2 + 4 * a.H_I * a.d_I * 2
        def kl_entry(ms, pairs):
            tf = per_pair * pairs / (ms * 1e-3) / 1e12
            return {"ms": round(ms, 4), "pairs": pairs, "gpairs_per_s": round(pairs / (ms * 1e-3) / 1e9, 2),
                    "tflops_fp32": round(tf, 2), "frac_fp32_valu": round(tf / FP32_VALU_PEAK_TFLOPS, 4)}
        result["indexer_kl"] = {"workload": a.name, "flops_per_pair": per_pair,
                                "sparse_top512": kl_entry(sparse_ms, pairs_sparse),
                                "dense_warmup": kl_entry(dense_ms, pairs_dense)}
        log(f"indexer KL: {result['indexer_kl']}")
        del la, ia, kin

    # ---- CPU oracle on a bounded, evenly spread sample of the same prefill rows
    if not args.no_cpu_baseline:
        import numpy as np

        import oracle

        stride = max(1, T // args.cpu_rows)
        rows = np.arange(stride // 2, T, stride, dtype=np.int32)[: args.cpu_rows]
        host = {x: layer[x].cpu() for x in ("q_idx", "k_idx", "w_idx", "q", "kv")}
        nproc = len(os.sched_getaffinity(0))  # the cores this process may run on (nproc)
        nthreads = nproc
        log(f"oracle on {len(rows)} rows with {nthreads} threads (nproc {nproc})")
        t0 = time.perf_counter()
        ridx, rout = oracle.dsa_rows(host["q_idx"][0], host["k_idx"][0], host["w_idx"][0], host["q"][0],
                                     host["kv"][0], rows, k, w.scale(), Dv=w.Dv, nthreads=nthreads)
        cdt = time.perf_counter() - t0
        # the sample spreads evenly over positions, so rows/s estimates the whole layer's rate
        got_out = out[0, torch.from_numpy(rows).long().to(dev)].double().cpu().numpy()
        got_idx = idx_cache[0, torch.from_numpy(rows).long().to(dev)].cpu().numpy()
        same_sets = float(np.mean([len(np.intersect1d(a[a >= 0], b[b >= 0])) / max(1, (b >= 0).sum())
                                   for a, b in zip(got_idx, ridx)]))
        result["cpu_baseline"] = {
            "value": round(len(rows) / cdt, 3), "unit": "query tokens/s", "cores": nthreads, "nproc": nproc,
            "kind": "oracle",
            "sample": f"{len(rows)} query rows of the T={T} layer (every {stride}th position), "
                      f"scores+top-k+attention in fp64, {cdt:.1f} s wall",
            "sample_check": {"max_abs_out_diff": float(np.max(np.abs(got_out - rout))),
                             "index_set_agreement": round(same_sets, 6)},
        }
        log(f"oracle: {len(rows) / cdt:.2f} rows/s")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
