"""Benchmark of the DSA stage (indexer scoring -> Top-K -> sparse MLA attention) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|prefill|skewed|fp8|tiny]

A step is one dsa_forward over one batch of synthetic inputs already resident
in HBM; for decode, eight independent input sets rotate (about 1.2 GB touched
per cycle of sets) so that each step's cache rows come from HBM rather than
the 256 MB Infinity Cache.  Prints one JSON line: whole-step throughput (query
tokens/s), the roofline of the dominant kernel (timed with HIP events on the
launch stream), and the CPU oracle timed on the host's cores over a bounded
sample of the same workload.  The metric is quoted on decode B32 x 8k and
prefill 32k: with the default decode workload, the line also carries a
"prefill" record of the same form, whose roofline is the indexer and
attention contractions against the bf16 MFMA peak (its traffic: one indexer
launch plus one attention launch).
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

METRIC = "DSA tokens/s (LI+TopK+SFA), decode B32@8k & prefill 32k; % HBM/MFMA peak"
WORKLOADS = {"tiny": 1, "decode": 2, "prefill": 3, "skewed": 4, "fp8": 5, "fp8pages": 6}
WORKLOAD_NAMES = {v: k for k, v in WORKLOADS.items()}
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def algorithmic(wl):
    """Bytes and flops the method must move/compute per step, per stage.

    The scores intermediate is not counted; gathers count one latent row per
    selected (row, position); the attention counts QK^T over d_qk and PV over d_v.
    """
    import numpy as np
    L = wl.row_lens().astype(np.int64)
    k = np.minimum(L, wl.top_k)
    rows = wl.rows
    esz = {"f32": 4, "bf16": 2, "e4m3": 1, "mxfp8": 1, "e4m3_128": 1}
    # scale bytes per index vector (d_I) and per latent row (d_qk)
    idx_sc = {"e4m3": 4, "mxfp8": wl.d_I // 32}.get(wl.idx_dtype, 0)
    kv_sc = {"mxfp8": wl.d_qk // 32, "e4m3_128": 4 * ((wl.d_qk + 127) // 128)}.get(wl.kv_dtype, 0)
    # indexer: each sequence's K_I rows once (shared by its n_q queries), q_I, w, scales
    seq_hist = wl.seq_lens.astype(np.int64)
    k_row = wl.d_I * esz[wl.idx_dtype] + idx_sc
    q_row = wl.H_I * wl.d_I * esz[wl.idx_dtype] + wl.H_I * (4 + idx_sc)  # codes, scales, head weights
    idx_bytes = int(seq_hist.sum() * k_row + rows * q_row)
    idx_flops = int(2 * L.sum() * wl.H_I * wl.d_I)
    # Top-K: the k_r indices written (scores are the unfused intermediate)
    topk_bytes = int(rows * wl.top_k * 4)
    # attention: gathered latent rows, q, out, indices
    kv_row = wl.d_qk * esz[wl.kv_dtype] + kv_sc
    qb = wl.H * wl.d_qk * esz[wl.q_dtype]
    ob = wl.H * wl.d_v * (4 if wl.out_dtype == "f32" else 2)
    attn_bytes = int(k.sum() * kv_row + rows * (qb + ob + wl.top_k * 4))
    attn_flops = int(2 * k.sum() * wl.H * (wl.d_qk + wl.d_v))
    return {"indexer": (idx_bytes, idx_flops), "topk": (topk_bytes, 0), "attention": (attn_bytes, attn_flops)}


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


# kernels of each stage, by name, as rocprofv3 reports them; the attention
# kernel's fused form (it selects the Top-K too, template argument TK != 0,
# run by dsa_forward) is not the attention stage's
STAGE_KERNELS = {"indexer": ("indexer_f32_kernel", "indexer_decode_kernel", "indexer_prefill_kernel"),
                 "topk": ("topk_",), "attention": ("sfa_",), "prolog": ("indexer_prolog_kernel",)}
STAGE_EXCLUDE = {"attention": (", 16>",)}


def stage_kernel(stage: str, name: str) -> bool:
    return any(t in name for t in STAGE_KERNELS[stage]) and not any(x in name for x in STAGE_EXCLUDE.get(stage, ()))
COPY_KERNEL = "neg_kernel"  # the plain copy used to calibrate the byte counters

KERNEL_SOURCES = {
    "indexer": ["sparse_attention_lightningindexer_amd/csrc/indexer.hip",
                "sparse_attention_lightningindexer_amd/csrc/common.hpp"],
    "topk": ["sparse_attention_lightningindexer_amd/csrc/topk.hip",
             "sparse_attention_lightningindexer_amd/csrc/select.hpp",
             "sparse_attention_lightningindexer_amd/csrc/common.hpp"],
    "attention": ["sparse_attention_lightningindexer_amd/csrc/sfa.hip",
                  "sparse_attention_lightningindexer_amd/csrc/select.hpp",
                  "sparse_attention_lightningindexer_amd/csrc/common.hpp"],
    "prolog": ["sparse_attention_lightningindexer_amd/csrc/prolog.hip",
               "sparse_attention_lightningindexer_amd/csrc/common.hpp"],
}


def measured_traffic(stage: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json.txt")
    if not os.path.exists(path):
        return None
    try:
        rec = json.loads(open(path).read())
    except ValueError:
        return None
    if rec.get("source_hash") != source_hash(KERNEL_SOURCES[stage]):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_means(csv_dir: str, counter: str):
    """Per-kernel mean of one counter over its dispatches in a rocprofv3 --pmc csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {csv_dir}")
    per = {}
    for f in files:
        with open(f, newline="") as fh:
            for rec in csv.DictReader(fh):
                if rec["Counter_Name"] != counter:
                    continue
                d = per.setdefault(rec["Kernel_Name"], {})
                d[rec["Dispatch_Id"]] = d.get(rec["Dispatch_Id"], 0.0) + float(rec["Counter_Value"])
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in per.items()}


def traffic_summary(stage: str, workload: str, fetch_dir: str, write_dir: str, copy_mib: int, cmd: str):
    """HBM bytes per launch of a stage from FETCH_SIZE / WRITE_SIZE passes (KiB per
    dispatch), each scaled by what the same counter reads for a plain copy of
    copy_mib MiB (read copy_mib, write copy_mib) in the same run."""
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    copy_bytes = copy_mib * 2 ** 20

    def one(table, what):
        cal = [v for k, v in table.items() if COPY_KERNEL in k]
        if not cal:
            raise SystemExit(f"the calibration copy ({COPY_KERNEL}) is missing from the {what} run")
        factor = copy_bytes / (cal[0][0] * 1024.0)
        ks = {k: v for k, v in table.items() if stage_kernel(stage, k)}
        if not ks:
            raise SystemExit(f"no {stage} kernels in the {what} run")
        raw = sum(v[0] for v in ks.values()) * 1024.0
        return factor, raw, {k[:120]: {"kib_per_dispatch": v[0], "dispatches": v[1]} for k, v in ks.items()}

    ff, fraw, fk = one(fetch, "FETCH_SIZE")
    wf, wraw, wk = one(write, "WRITE_SIZE")
    rec = {"stage": stage, "workload": workload, "source_hash": source_hash(KERNEL_SOURCES[stage]),
           "hbm_bytes_per_launch": fraw * ff + wraw * wf,
           "read_bytes_per_launch": fraw * ff, "write_bytes_per_launch": wraw * wf,
           "fetch_factor": ff, "write_factor": wf, "copy_mib": copy_mib,
           "fetch_kernels": fk, "write_kernels": wk, "command": cmd}
    return rec


def prolog_bytes(rows, d_x, H_I, d_I, mx):
    """Algorithmic HBM bytes of one indexer prolog: both weight matrices, the hidden
    states and keys read once, and every output written once."""
    reads = 2 * (H_I * d_I + H_I) * d_x + 2 * rows * d_x + 2 * rows * d_I + 4 * d_I
    writes = rows * H_I * d_I * (1 if mx else 2) + (rows * H_I * d_I // 32 if mx else 0) + 4 * rows * H_I \
        + 2 * rows * d_I
    return reads + writes


def time_prolog(wl0, args, stream):
    """The indexer prolog for this workload's query rows from a hidden state of width
    7168: 3 weight sets rotating (356 MB, more than the Infinity Cache), K launches
    between two events after a spin, like the stages."""
    import torch
    from sparse_attention_lightningindexer_amd import binding as B
    from sparse_attention_lightningindexer_amd.inputs import PROLOG, make_prolog
    fmt = "mxfp8" if wl0.idx_dtype == "mxfp8" else "bf16"
    pds, outs = [], []
    for s in range(3):
        p = make_prolog(wl0.rows, PROLOG["d_x"], wl0.H_I, wl0.d_I, seed=PROLOG["seed"], rotation=s,
                        eps=PROLOG["eps"])
        pds.append(B.PrologDevice(p))
        outs.append(B.dsa_indexer_prolog(pds[-1], fmt, stream=stream))
    torch.cuda.synchronize()
    torch.cuda._sleep(600_000 * args.steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        B.dsa_indexer_prolog(pds[i % 3], fmt, outs=outs[i % 3], stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    nb = prolog_bytes(wl0.rows, PROLOG["d_x"], wl0.H_I, wl0.d_I, fmt == "mxfp8")
    ach = nb / (us * 1e-6) / 1e9
    return {"us": us, "rows": wl0.rows, "d_x": PROLOG["d_x"], "q_format": fmt, "algorithmic_bytes": nb,
            "achieved_GBs": ach, "frac_hbm": ach / HBM_PEAK_GBS,
            "traffic": measured_traffic("prolog", args.workload)}


def cpu_baseline_prolog(wl0, budget_s: float):
    """The oracle's prolog (fp64 projections and normalization) on the host's cores,
    on the same inputs as the GPU prolog, repeated for about budget_s seconds."""
    from oracle import oracle as O
    from sparse_attention_lightningindexer_amd.inputs import PROLOG, make_prolog
    p = make_prolog(wl0.rows, PROLOG["d_x"], wl0.H_I, wl0.d_I, seed=PROLOG["seed"], eps=PROLOG["eps"])
    reps, t0 = 0, time.perf_counter()
    while True:
        O.indexer_prolog(p)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": p.rows * reps / dt, "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"all {p.rows} rows of one prolog x {reps}; {dt:.1f} s"}


def cpu_baseline(wl, budget_s: float):
    """The oracle as it stands, on the host's cores, over a bounded sample of rows,
    repeated for about budget_s seconds."""
    import numpy as np
    from oracle import oracle as O
    if wl.rows > 64:  # prefill: rows spread evenly over the causal range
        sample = np.linspace(0, wl.rows - 1, 64).astype(np.int32)
        what = f"64 of {wl.rows} query rows, evenly spaced over positions (whole stage per row)"
    else:
        sample = np.arange(wl.rows, dtype=np.int32)
        what = f"all {wl.rows} query rows of one step (whole stage)"
    done, reps, t0 = 0, 0, time.perf_counter()
    while True:
        O.forward(wl, rows=sample)
        done += len(sample)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": what + f" x {reps}; {dt:.1f} s"}


def spin_then_time(call, n, stream):
    """n calls back to back between two HIP events on `stream`, after a GPU spin of
    ~0.6 ms per call so that the host has queued them all before the first runs;
    returns microseconds per call."""
    import torch
    torch.cuda.synchronize()
    torch.cuda._sleep(600_000 * n)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3


def measure(cfg, args, steps, warmup, nsets, extras):
    """One workload: the timed dsa_forward steps, their spread, the per-stage
    durations and the roofline of the dominant kernel (both stages of the indexer
    + attention contraction for prefill); with `extras`, also the quantized
    indexer's recall, the cache append and the indexer prolog."""
    import numpy as np
    import torch
    from sparse_attention_lightningindexer_amd import binding as B
    from sparse_attention_lightningindexer_amd.inputs import make_workload

    print(f"[bench] generating {nsets} input set(s) of workload {cfg}", file=sys.stderr, flush=True)
    sets = []
    for s in range(nsets):
        wl = make_workload(cfg, rotation=s)
        dev = B.DeviceInputs(wl)
        ws = torch.empty(max(1, B.dsa_forward_workspace_bytes(dev)), dtype=torch.uint8, device="cuda")
        idx = torch.empty((wl.rows, wl.top_k), dtype=torch.int32, device="cuda")
        sets.append((wl, dev, ws, idx))
        if s == 0:
            wl0 = wl
    del wl
    stream = torch.cuda.current_stream()

    def step(i):
        _, dev, ws, idx = sets[i % nsets]
        B.dsa_forward(dev, indices_out=idx, ws=ws, stream=stream)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps of the whole stage
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = gpu_ms / steps
    value = wl0.rows * steps / (gpu_ms / 1e3)
    print(f"[bench] {wl0.cfg['name']}: {steps} steps, {ms_per_step * 1e3:.1f} us/step "
          f"(wall {wall / steps * 1e6:.1f} us)", file=sys.stderr, flush=True)

    # the spread of single steps: a separate loop (not the timed region) with an
    # event between consecutive steps, after a spin that lets the host queue
    # the loop ahead of the GPU
    n_one = min(steps, 100)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_one + 1)]
    torch.cuda.synchronize()
    torch.cuda._sleep(600_000 * n_one)
    evs[0].record(stream)
    for i in range(n_one):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    one = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n_one)])
    step_us = {"p10": float(np.percentile(one, 10)), "p50": float(np.percentile(one, 50)),
               "p90": float(np.percentile(one, 90)), "steps": n_one}

    # per-stage durations: the same kernels through the three unfused calls,
    # each stage `steps` times back to back with the input sets rotating
    scores = [torch.empty((s[0].rows, max(1, s[0].max_seq_len)), dtype=torch.float32, device="cuda")
              for s in sets]
    attn_ws = [torch.empty(max(1, B.dsa_sparse_attn_workspace_bytes(s[1])), dtype=torch.uint8, device="cuda")
               for s in sets]
    for i in range(nsets):  # every set's scores and indices, for the loops below
        _, dev, _, idx = sets[i]
        B.dsa_indexer_scores(dev, scores[i], stream=stream)
        B.dsa_topk(dev, scores[i], indices=idx, stream=stream)
    calls = {
        "indexer": lambda i: B.dsa_indexer_scores(sets[i % nsets][1], scores[i % nsets], stream=stream),
        "topk": lambda i: B.dsa_topk(sets[i % nsets][1], scores[i % nsets], indices=sets[i % nsets][3],
                                     stream=stream),
        "attention": lambda i: B.dsa_sparse_attn(sets[i % nsets][1], sets[i % nsets][3], ws=attn_ws[i % nsets],
                                                 stream=stream),
    }
    stage_us = {name: spin_then_time(call, steps, stream) for name, call in calls.items()}
    del scores, attn_ws
    algo = algorithmic(wl0)
    if cfg == 3:
        # prefill: the indexer and attention contractions together against the
        # bf16 MFMA peak (their flops over their kernel time)
        nflops = algo["indexer"][1] + algo["attention"][1]
        dur_us = stage_us["indexer"] + stage_us["attention"]
        ach = nflops / (dur_us * 1e-6) / 1e12
        # HBM bytes of one indexer launch plus one attention launch (counters)
        parts = [measured_traffic(k, WORKLOAD_NAMES[cfg]) for k in ("indexer", "attention")]
        roof = {"bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / BF16_PEAK_TFLOPS, "traffic": None if None in parts else sum(parts),
                "kernel": "indexer scoring + sparse attention (indexer_prefill_kernel, sfa_mla_kernel)",
                "algorithmic_flops": nflops, "avg_us": dur_us,
                "stage_frac": {k: algo[k][1] / (stage_us[k] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS
                               for k in ("indexer", "attention")}}
    else:
        dom = max(stage_us, key=stage_us.get)
        nbytes, nflops = algo[dom]
        ach = nbytes / (stage_us[dom] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                "traffic": measured_traffic(dom, WORKLOAD_NAMES[cfg]),
                "kernel": {"indexer": "indexer scoring (indexer_*_kernel)",
                           "topk": "top-k (topk_reg_kernel or topk_kernel)",
                           "attention": "sparse attention (sfa_mla_kernel, plus sfa_combine_kernel when split)"}[dom],
                "algorithmic_bytes": nbytes, "algorithmic_flops": nflops, "avg_us": stage_us[dom],
                "mfma_frac": nflops / (stage_us[dom] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS}

    res = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "e4m3": "fp8e4m3+bf16", "mxfp8": "fp8e4m3+bf16"}[wl0.idx_dtype],
        "data": "synthetic",
        "config": {"workload": wl0.cfg["name"], "batch": wl0.batch, "n_q": wl0.n_q,
                   "context": int(wl0.max_seq_len), "top_k": wl0.top_k, "index_heads": wl0.H_I,
                   "index_dim": wl0.d_I, "heads": wl0.H, "d_qk": wl0.d_qk, "d_v": wl0.d_v,
                   "paging": wl0.cfg["paging"], "input_sets": nsets},
        "roofline": roof,
        "step_us": step_us,
        "stages_us": stage_us,
    }
    if extras and wl0.idx_dtype in ("e4m3", "mxfp8"):
        # reported, not a parity bound: how much of the quantized indexer's
        # Top-K the bf16 indexer (same drawn values, rounded to bf16) also
        # selects, over every row of the first input set
        wl_b = make_workload(cfg, rotation=0, idx_dtype="bf16")
        dev_b = B.DeviceInputs(wl_b)
        idx_b = B.dsa_topk(dev_b, B.dsa_indexer_scores(dev_b)).cpu().numpy()
        idx_q = sets[0][3].cpu().numpy()
        rec = [len(set(a[a >= 0].tolist()) & set(c[c >= 0].tolist())) / max(1, int((c >= 0).sum()))
               for a, c in zip(idx_q, idx_b)]
        res["topk_recall_vs_bf16"] = {"mean": float(np.mean(rec)), "min": float(np.min(rec)), "rows": len(rec)}
        del dev_b
    if extras:
        # cache append (the step before the indexer): this step's index keys and
        # latent rows written into the first input set's pools, quantized when
        # the pool is; after every other measurement (it overwrites pool rows)
        _, dev0, _, _ = sets[0]
        dt = torch.bfloat16 if wl0.idx_dtype != "f32" else torch.float32
        k_new = torch.randn(wl0.rows, wl0.d_I, device="cuda").to(dt)
        kv_new = torch.randn(wl0.rows, wl0.d_qk, device="cuda").to(dt)
        B.dsa_cache_append(dev0, k_new, kv_new, stream=stream)
        res["append_us"] = spin_then_time(lambda i: B.dsa_cache_append(dev0, k_new, kv_new, stream=stream),
                                          steps, stream)
        if wl0.rows <= 256:
            res["prolog"] = time_prolog(wl0, args, stream)
            if not args.no_cpu:
                res["prolog"]["cpu_baseline"] = cpu_baseline_prolog(wl0, min(args.cpu_budget, 5.0))
    del sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl0, args.cpu_budget)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode", choices=list(WORKLOADS))
    ap.add_argument("--sets", type=int, default=8, help="rotating input sets (decode workloads)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="with the decode workload, skip the nested prefill 32k record")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="after the run, copy MIB MiB three times (byte-counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: summarize two rocprofv3 --pmc csv runs (FETCH_SIZE, WRITE_SIZE) "
                         "of this script into profiles/traffic_<stage>_<workload>.json.txt")
    ap.add_argument("--stage", default="attention", choices=list(STAGE_KERNELS))
    ap.add_argument("--command", default="", help="with --traffic-from: the command the runs came from")
    args = ap.parse_args()
    if args.traffic_from:
        rec = traffic_summary(args.stage, args.workload, *args.traffic_from, args.copy_calib, args.command)
        path = os.path.join(ROOT, "profiles", f"traffic_{args.stage}_{args.workload}.json.txt")
        with open(path, "w") as fh:
            fh.write(json.dumps(rec, indent=1) + "\n")
        print(json.dumps({k: rec[k] for k in ("hbm_bytes_per_launch", "fetch_factor", "write_factor")}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(decode shards by sequence, with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_lightningindexer_amd import binding as B

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()  # fail loudly when the HIP library is missing
    cfg = WORKLOADS[args.workload]
    nsets = 1 if cfg == 3 else args.sets  # prefill: one set already exceeds the caches many times over
    res = measure(cfg, args, args.steps, args.warmup, nsets, extras=True)
    if cfg == 2 and not args.no_prefill:
        # the metric is quoted on decode B32 x 8k and prefill 32k: the prefill
        # record rides in the same line, with its own roofline and CPU baseline
        res["prefill"] = measure(3, args, args.prefill_steps, min(args.warmup, 3), 1, extras=False)
    if args.copy_calib:
        src = torch.randn(args.copy_calib * 2 ** 18, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(res))


if __name__ == "__main__":
    main()
