#!/usr/bin/env python3
"""Benchmark of the static embedding / tied lm_head service on one MI355X.

A step is one decode step of the service on the 31B-shaped tied table
(bf16, V = 262,144, hidden = 5,376, 2.82 GB): embed_gather of one token id
(ADR-0008 "POST /v1/embed") and logits_topk of one residual with k = 10
(ADR-0008 "POST /v1/logits"), which streams the whole table once.  Inputs are
seeded synthetic arrays (synth/), resident in HBM before the timed region.

value = algorithmic bytes of the step / time per step, in GB/s.  The roofline
object times the table-streaming kernel alone with HIP events recorded on the
stream it runs on.  The other workloads of the page set are measured after the
timed steps and reported under "also": batches of 8 to 64 (and the exact wide
kernel at 64), the response with probabilities, the raw logits mode, the same
lm_head stored as Q8_0, the 1,024-row contraction (rank path and split
contraction), and the EmbeddingGemma-shaped Q8_0 gather with f32, f16 and i8
output rows, and the Qwen2.5-0.5B-shaped prompt gather and one-row logits.  The
CPU oracle is timed on a bounded sample of the same workload under
"cpu_baseline".

    python bench.py [--gpus 1] [--steps K] [--warmup W]
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

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# sources of the roofline kernel: the traffic record is void once either changes
KERNEL_SOURCES = [os.path.join(ROOT, "embedding_table_gather_amd", "csrc", f)
                  for f in ("stream.hip", "etg_device.hpp")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the kernel source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("source_sha256_16") != _source_hash():
        return None
    return ent.get("bytes_per_launch")


def _counter_means(csv_path: str, counter: str):
    """Per-dispatch values of one rocprofv3 counter, grouped by kernel name."""
    import csv
    out = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def write_traffic(fetch_csv: str, write_csv: str, kernel: str = "stream_logits_kernel<1, 0>") -> dict:
    """Turn a FETCH_SIZE run and a WRITE_SIZE run of `bench.py --no-extras --calib-copy`
    (rocprofv3 --pmc ..., csv output) into profiles/traffic.json.

    Both counters are in KiB per dispatch.  Each is scaled by what it reads for the
    plain 1 GiB device copy of the same run (the largest copy dispatches), so that
    bytes_per_launch is in the copy's units: a copy of N bytes counts as N read
    and N written.
    """
    import synth
    fetch, write = _counter_means(fetch_csv, "FETCH_SIZE"), _counter_means(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)

    def copy_factor(d):
        vals = [v for name, vs in d.items() if "copyBuffer" in name for v in vs]
        big = [v for v in vals if v > 0.25 * gib_kib]
        if not big:
            raise SystemExit("no 1 GiB copy dispatch in the counter file (run bench.py with --calib-copy)")
        return gib_kib / (sum(big) / len(big))

    def kernel_values(d):
        vs = [v for name, vals in d.items() if kernel in name for v in vals]
        if not vs:
            raise SystemExit(f"{kernel} not found in the counter file")
        return vs

    ff, fw = copy_factor(fetch), copy_factor(write)
    # the same kernel also streams the smaller Qwen-shaped table in the same run:
    # keep the dispatches that fetch at least half of the 31B-shaped table, and the
    # WRITE_SIZE dispatches at the same positions (both runs issue the same sequence)
    fv, wv = kernel_values(fetch), kernel_values(write)
    table_kib = synth.CONFIGS["lm31b"].table_bytes / 1024.0
    keep = [i for i, v in enumerate(fv) if v * ff >= 0.5 * table_kib]
    if not keep:
        raise SystemExit(f"no {kernel} dispatch over the 31B-shaped table in the counter file")
    fk = sum(fv[i] for i in keep) / len(keep)
    wsel = [wv[i] for i in keep] if len(wv) == len(fv) else wv
    wk = sum(wsel) / len(wsel)
    rec = {kernel: {
        "source_sha256_16": _source_hash(),
        "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
        "copy_fetch_factor": round(ff, 5), "copy_write_factor": round(fw, 5),
        "bytes_per_launch": round((fk * ff + wk * fw) * 1024),
    }}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


class _HipEvents:
    """Timing events created with hipEventDisableSystemFence, passed to the library
    as raw hipEvent_t handles.  Events with the default system-scope fence (torch's)
    cost about 13 us per step around the table kernel; these cost nothing
    measurable, so the step time stays the step's own."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.made = []

    def pair(self):
        evs = []
        for _ in range(2):
            h = self.ct.c_void_p()
            if self.hip.hipEventCreateWithFlags(self.ct.byref(h), self.ct.c_uint(self.DISABLE_SYSTEM_FENCE)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.made.append(h.value)
            evs.append(h.value)
        return tuple(evs)

    def record(self, ev, torch) -> None:
        if self.hip.hipEventRecord(self.ct.c_void_p(ev), self.ct.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b) -> float:
        out = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(out), self.ct.c_void_p(a), self.ct.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for h in self.made:
            self.hip.hipEventDestroy(self.ct.c_void_p(h))
        self.made = []


def _timed(torch, fn, iters: int, events: _HipEvents = None):
    """Average ms per call of fn(); with events given, fn takes (ev_before, ev_after)
    (raw hipEvent_t handles the library records around its table kernel) and the
    mean kernel ms between them is returned too."""
    evs = [events.pair() for _ in range(iters)] if events else None
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for i in range(iters):
        fn(evs[i]) if events else fn()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / iters
    kms = sum(events.ms(a, b) for a, b in evs) / iters if events else None
    if events:
        events.close()
    return ms, kms


def _settle(torch, fn, seconds: float = 0.1):
    """Run fn back to back for about `seconds` before it is timed.  The GPU's clocks
    drop while the host generates a table and take tens of milliseconds of load to
    come back (measured after a 1.5 s idle: the Q8_0 one-row call ran 284, 273, 269
    and 266 us in its first four windows of 30 calls and 263-265 us from then on; the
    Qwen-shaped one-row call 58.2, then 55.4, then 54.5-54.8 us per call in windows
    of 120 calls), so every distribution below is taken in that settled state."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def _dist(torch, fn, iters: int, events: _HipEvents, kernel: bool = False) -> dict:
    """Per-call time of fn over `iters` repeats: median, p10 and p90 in us.  A
    repeat is a batch of back-to-back calls between two events (batches of about
    200 us, so that the events' own cost, a few us, stays out of the per-call
    time of short calls), its time divided by the calls in it.  With kernel=True
    fn takes (ev_before, ev_after), recorded by the library around its table
    kernel on one call of each batch, and the kernel's median is added."""
    import numpy as np
    _settle(torch, fn)
    t1 = time.perf_counter()
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    est_us = (time.perf_counter() - t1) / 3 * 1e6
    per_batch = int(min(64, max(1, 200.0 // max(est_us, 1.0))))
    bounds = [events.pair() for _ in range(iters)]
    kev = [events.pair() for _ in range(iters)] if kernel else None
    torch.cuda.synchronize()
    for i in range(iters):
        events.record(bounds[i][0], torch)
        for j in range(per_batch):
            fn(kev[i]) if kernel and j == per_batch - 1 else fn()
        events.record(bounds[i][1], torch)
    torch.cuda.synchronize()
    per = np.array([events.ms(a, b) for a, b in bounds]) * 1e3 / per_batch
    out = {"median_us": round(float(np.median(per)), 2), "p10_us": round(float(np.percentile(per, 10)), 2),
           "p90_us": round(float(np.percentile(per, 90)), 2), "repeats": iters, "calls_per_repeat": per_batch}
    if kernel:
        kk = np.array([events.ms(a, b) for a, b in kev]) * 1e3
        out["kernel_median_us"] = round(float(np.median(kk)), 2)
    events.close()
    return out


def _single(torch, fn, iters: int = 30) -> float:
    """Median wall time (us) of one call between two synchronisations."""
    import numpy as np
    lat = []
    for _ in range(iters):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - t1) * 1e6)
    return round(float(np.median(lat)), 1)


def _graph(torch, fn):
    """fn captured in a HIP graph (after one run on a side stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extras", action="store_true", help="only the timed decode steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter files and exit")
    args = ap.parse_args()
    if args.traffic_from:
        print(json.dumps(write_traffic(*args.traffic_from)))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the vocab-sharded multi-GPU design is not built", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import embedding_table_gather_amd as etg
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.CONFIGS["lm31b"]
    B, k = 1, 10
    log(f"generating the {cfg.name} table ({cfg.table_bytes / 1e9:.2f} GB)")
    t0 = time.time()
    host = cfg.table()
    log(f"generated in {time.time() - t0:.1f} s; uploading")
    rows = torch.from_numpy(host.view(np.int16)).to(dev)
    table = etg.Table(rows, cfg.dtype, cfg.V, cfg.d)
    ids = torch.from_numpy(synth.zipf_ids(B, cfg.V, cfg.ids_seed)).to(dev)
    R = torch.from_numpy(cfg.residuals(B)).to(dev)
    x = torch.empty((B, cfg.d), dtype=torch.float32, device=dev)
    ws = table.workspace(B, k)
    oid = torch.empty((B, k), dtype=torch.int32, device=dev)
    osc = torch.empty((B, k), dtype=torch.float32, device=dev)

    def step(evs=None):
        table.embed_gather(ids, out=x, check=False)
        table.logits_topk(R, k, workspace=ws, out_ids=oid, out_scores=osc, events=evs)

    hev = _HipEvents()
    rd = None
    if not args.no_extras:
        # the plain read stream over the same table (the library's probe), as a measured
        # reference beside the 8 TB/s nominal; taken first, it also brings the GPU's
        # clocks out of the idle state the host-side table generation leaves
        sink = torch.empty(1, dtype=torch.int32, device=dev)
        rd = _dist(torch, lambda: etg.hbm_read_probe(rows, sink), 20, hev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    # eager steps, with the table kernel timed alone by events around it
    ms, kms = _timed(torch, step, args.steps, events=hev)
    ms_graph = None
    if not args.no_extras:
        # the same step captured once in a HIP graph and replayed (one launch per
        # step instead of three); reported beside the eager steps
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        ms_graph, _ = _timed(torch, graph.replay, args.steps)
        del graph
        log(f"eager {ms * 1e3:.1f} us/step, graph replay {ms_graph * 1e3:.1f} us/step")

    gather_bytes = B * cfg.row_bytes + B * cfg.d * 4 + B * 4
    logits_bytes = cfg.table_bytes + B * cfg.d * 4 + B * k * 8
    step_bytes = gather_bytes + logits_bytes
    value = step_bytes / (ms * 1e-3) / 1e9
    kernel_name = "stream_logits_kernel<1, 0>"
    achieved = cfg.table_bytes / (kms * 1e-3) / 1e9
    traffic = _traffic(kernel_name)
    out = {
        "metric": "lm_head logits+top-k GB/s (% HBM peak) at V=262144; gather rows/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 table, N(0,1) residual)",
        "config": {
            "workload": "31B-shaped tied lm_head decode step: embed_gather(1 id) + logits_topk(1 residual, k=10)",
            "table_dtype": "bf16", "vocab": cfg.V, "hidden": cfg.d, "batch": B, "k": k,
            "table_bytes": cfg.table_bytes,
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 1),
        "roofline": {
            "kernel": kernel_name,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel_us": round(kms * 1e3, 2),
            "bytes_per_launch": cfg.table_bytes,
        },
    }
    log(f"step {ms * 1e3:.1f} us, table kernel {kms * 1e3:.1f} us -> {achieved:.0f} GB/s")

    also = {}
    if not args.no_extras:
        also["decode_step"] = _dist(torch, step, 50, hev)
        also["decode_step"]["single_call_us"] = _single(torch, step)
        if ms_graph is not None:
            also["decode_step"]["hipgraph_replay_us"] = round(ms_graph * 1e3, 1)
        # plain read (taken before the steps) and write streams on the same box
        rs_gbps = cfg.table_bytes / (rd["median_us"] * 1e-6) / 1e9
        also["read_stream_reference"] = {
            "what": "etg_hbm_read_probe over the 2.82 GB table", "us_per_call": rd["median_us"],
            "GBps": round(rs_gbps, 1), "pct_hbm_peak": round(100 * rs_gbps / HBM_PEAK_GBPS, 1),
            "roofline_kernel_pct_of_it": round(100 * achieved / rs_gbps, 1)}
        log(f"read stream reference: {rs_gbps:.0f} GB/s")
        wref = {}
        for name, nbytes in (("50MB", 50331648), ("1GB", 1 << 30)):
            wb = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
            wd = _dist(torch, lambda: etg.hbm_write_probe(wb, 0), 50, hev)
            wref[name] = {"bytes": nbytes, "us_per_call": wd["median_us"],
                          "GBps": round(nbytes / (wd["median_us"] * 1e-6) / 1e9, 1)}
            del wb
        also["write_stream_reference"] = {"what": "etg_hbm_write_probe (non-temporal 16-byte stores)", **wref}
        log(f"write stream reference: {wref}")

        def logits_entry(tbl, Rb, kk, path, nbytes, iters=50):
            wsb = tbl.workspace(Rb.shape[0], kk, path)
            f = lambda evs=None: tbl.logits_topk(Rb, kk, path=path, workspace=wsb, events=evs)
            for _ in range(3):
                f()
            d = _dist(torch, f, iters, hev, kernel=True)
            d["GBps"] = round(nbytes / (d["median_us"] * 1e-6) / 1e9, 1)
            d["pct_hbm_peak"] = round(100 * d["GBps"] / HBM_PEAK_GBPS, 1)
            return d

        # the automatic choice (stream up to 8 rows, wide up to 16, then the rank
        # path), the exact wide kernel at 64 rows, and past 64 rows the rank path
        # beside the split contraction
        for b, path, key in ((8, etg.PATH_AUTO, "lm31b_logits_top10_B8"), (16, etg.PATH_AUTO, "lm31b_logits_top10_B16"),
                             (32, etg.PATH_AUTO, "lm31b_logits_top10_B32"), (64, etg.PATH_AUTO, "lm31b_logits_top10_B64"),
                             (64, etg.PATH_WIDE, "lm31b_logits_top10_B64_exact_wide"),
                             (96, etg.PATH_AUTO, "lm31b_logits_top10_B96"), (128, etg.PATH_AUTO, "lm31b_logits_top10_B128"),
                             (128, etg.PATH_GEMM, "lm31b_logits_top10_B128_split_gemm"),
                             (192, etg.PATH_AUTO, "lm31b_logits_top10_B192"), (256, etg.PATH_AUTO, "lm31b_logits_top10_B256"),
                             (256, etg.PATH_GEMM, "lm31b_logits_top10_B256_split_gemm")):
            Rb = torch.from_numpy(cfg.residuals(b)).to(dev)
            also[key] = logits_entry(table, Rb, k, path, cfg.table_bytes, iters=50 if b <= 64 else 20)
            log(f"B={b} path={path}: {also[key]['median_us']:.1f} us")
            del Rb
        # the logits response with probabilities at T = 1, and the raw logits mode
        R1 = torch.from_numpy(cfg.residuals(1)).to(dev)
        ws1 = table.workspace(1, k)
        d = _dist(torch, lambda: table.logits_topk_probs(R1, k, temperature=1.0, workspace=ws1), 50, hev)
        d["GBps"] = round(cfg.table_bytes / (d["median_us"] * 1e-6) / 1e9, 1)
        d["pct_hbm_peak"] = round(100 * d["GBps"] / HBM_PEAK_GBPS, 1)
        also["lm31b_logits_top10_probs_B1"] = d
        raw = torch.empty((1, cfg.V), dtype=torch.float32, device=dev)
        wsr = torch.empty(max(table.workspace_bytes(1, 1), 256), dtype=torch.uint8, device=dev)
        d = _dist(torch, lambda: table.logits_raw(R1, out=raw, workspace=wsr), 50, hev)
        rbytes = cfg.table_bytes + cfg.V * 4
        d["GBps"] = round(rbytes / (d["median_us"] * 1e-6) / 1e9, 1)
        d["pct_hbm_peak"] = round(100 * d["GBps"] / HBM_PEAK_GBPS, 1)
        also["lm31b_logits_raw_B1"] = d
        log(f"probs B=1: {also['lm31b_logits_top10_probs_B1']['median_us']} us, raw B=1: {d['median_us']} us")
    del table, rows
    torch.cuda.empty_cache()

    if not args.no_extras:
        # tiny f32 table (4,096 x 256): gather of 64 ids, logits + top-5 for 4 rows,
        # and the two as one step; eager calls beside the same calls replayed from a
        # captured HIP graph
        c1 = synth.CONFIGS["tiny"]
        t1 = etg.Table(torch.from_numpy(c1.table()).to(dev), c1.dtype, c1.V, c1.d)
        ids1 = torch.from_numpy(c1.ids()).to(dev)
        x1 = torch.empty((ids1.numel(), c1.d), dtype=torch.float32, device=dev)
        R4 = torch.from_numpy(c1.residuals(4)).to(dev)
        ws4 = t1.workspace(4, c1.k)
        oi4 = torch.empty((4, c1.k), dtype=torch.int32, device=dev)
        os4 = torch.empty((4, c1.k), dtype=torch.float32, device=dev)
        g1 = lambda: t1.embed_gather(ids1, out=x1, check=False)
        l1 = lambda evs=None: t1.logits_topk(R4, c1.k, workspace=ws4, out_ids=oi4, out_scores=os4, events=evs)
        s1 = lambda: (g1(), l1())
        for key, fn, kern in (("tiny_gather_64", g1, False), ("tiny_logits_top5_B4", l1, True),
                              ("tiny_gather_then_logits", s1, False)):
            for _ in range(5):
                fn()
            d = _dist(torch, fn, 50, hev, kernel=kern)
            d["single_call_us"] = _single(torch, fn)
            gr = _graph(torch, fn if not kern else (lambda: l1()))
            d["hipgraph_replay"] = _dist(torch, gr.replay, 50, hev)
            d["hipgraph_replay"]["single_call_us"] = _single(torch, gr.replay)
            del gr
            also[key] = d
        also["tiny_gather_64"]["rows_per_s"] = round(ids1.numel() / (also["tiny_gather_64"]["median_us"] * 1e-6))
        log(f"tiny: {also['tiny_gather_then_logits']}")
        # the service step from host ids to a host answer: host ids -> device, gather,
        # logits + top-5 of 4 rows -> page-locked host memory behind an event; eager
        # calls of the plain entry points beside the graph-cached step calls (one
        # graph per configuration, captured on the second hit)
        ss = torch.cuda.Stream()
        with torch.cuda.stream(ss):
            ids1_h = torch.from_numpy(c1.ids()).pin_memory()
            ids1_d = torch.empty_like(ids1_h, device=dev)
            ho = (torch.empty((4, c1.k), dtype=torch.int32, pin_memory=True),
                  torch.empty((4, c1.k), dtype=torch.float32, pin_memory=True))

            def eager_step():
                ids1_d.copy_(ids1_h, non_blocking=True)
                t1.embed_gather(ids1_d, out=x1, check=False)
                return t1.logits_topk_to_host(R4, c1.k, workspace=ws4, host_out=ho)

            ids1_np = ids1_h.numpy()
            d = {"plain_calls_with_copies": _dist(torch, eager_step, 50, hev)}
            d["plain_calls_with_copies"]["single_call_us"] = _single(torch, lambda: eager_step()[2].synchronize())
            # the step cache: kernels read the ids from and write the answer to mapped
            # page-locked memory; run eagerly, then with graphs
            for name, use_graphs in (("step_eager", False), ("step_graph_cached", True)):
                sc1 = etg.StepCache(t1, max_ids=ids1_h.numel(), max_batch=4, k=c1.k, use_graphs=use_graphs)
                sc1.residual.copy_(R4)

                def graph_step():
                    sc1.gather(ids1_np)
                    return sc1.logits(4)
                d[name] = _dist(torch, graph_step, 50, hev)
                d[name]["single_call_us"] = _single(torch, lambda: graph_step().synchronize())
                d[name]["graphs_captured"], d[name]["graph_launches"] = sc1.stats()
                del sc1
            also["tiny_step_host_ids_to_host_top5"] = d
            log(f"tiny step: {d}")
        del t1
        # Qwen2.5-0.5B-shaped tied table (bf16 151,936 x 896, 272 MB): the prompt's
        # gather of 628 Zipf ids over 109 distinct rows, and logits + top-10 for 1 row
        qc = synth.CONFIGS["qwen05b"]
        qw = qc.table()
        # four copies (1.09 GB), cycled call by call, so that the 272 MB table is read
        # from HBM and not from the 256 MB MALL
        qwts = [etg.Table(torch.from_numpy(qw.view(np.int16)).to(dev), qc.dtype, qc.V, qc.d) for _ in range(4)]
        qwt = qwts[0]
        del qw
        qids_host = qc.ids()
        qids = torch.from_numpy(qids_host).to(dev)
        qx = torch.empty((qids.numel(), qc.d), dtype=torch.float32, device=dev)
        f = lambda: qwt.embed_gather(qids, out=qx, check=False)
        for _ in range(5):
            f()
        d = _dist(torch, f, 50, hev)
        d["single_call_us"] = _single(torch, f)
        gr = _graph(torch, f)
        d["hipgraph_replay"] = _dist(torch, gr.replay, 50, hev)
        del gr
        d.update({"rows": int(qids.numel()), "distinct_rows": int(np.unique(qids_host).size),
                  "rows_per_s": round(qids.numel() / (d["median_us"] * 1e-6))})
        also["qwen05b_gather_628_zipf_ids"] = d
        Rq1 = torch.from_numpy(qc.residuals(1)).to(dev)
        wsq1 = qwt.workspace(1, qc.k)
        turn = [0]

        def fq(evs=None):
            turn[0] += 1
            return qwts[turn[0] % 4].logits_topk(Rq1, qc.k, workspace=wsq1, events=evs)
        for _ in range(4):
            fq()
        d = _dist(torch, fq, 52, hev, kernel=True)
        d["GBps"] = round(qc.table_bytes / (d["median_us"] * 1e-6) / 1e9, 1)
        d["pct_hbm_peak"] = round(100 * d["GBps"] / HBM_PEAK_GBPS, 1)
        d["kernel_pct_hbm_peak"] = round(100 * qc.table_bytes / (d["kernel_median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1)
        d["single_call_us"] = _single(torch, fq)
        d["tables"] = "4 copies, cycled"
        # a plain read stream over the same copies, cycled alike: what a pass over
        # 272 MB costs on its own (launch, ramp and tail included)
        sink = torch.empty(1, dtype=torch.int32, device=dev)
        pturn = [0]

        def fprobe():
            pturn[0] += 1
            etg.hbm_read_probe(qwts[pturn[0] % 4].rows, sink)
        for _ in range(4):
            fprobe()
        dp = _dist(torch, fprobe, 52, hev)
        dp["GBps"] = round(qc.table_bytes / (dp["median_us"] * 1e-6) / 1e9, 1)
        dp["pct_hbm_peak"] = round(100 * dp["GBps"] / HBM_PEAK_GBPS, 1)
        d["read_stream_reference_272MB"] = dp
        d["pct_of_read_stream_272MB"] = round(100 * dp["median_us"] / d["median_us"], 1)
        also["qwen05b_logits_top10_B1"] = d
        log(f"qwen05b gather {also['qwen05b_gather_628_zipf_ids']['median_us']} us, logits B=1 {d['median_us']} us")
        # the same calls from host ids / to a host answer, eager beside graph-cached
        ss = torch.cuda.Stream()
        with torch.cuda.stream(ss):
            qids_h = torch.from_numpy(qids_host).pin_memory()
            qids_d = torch.empty_like(qids_h, device=dev)

            def eager_gather():
                qids_d.copy_(qids_h, non_blocking=True)
                return qwt.embed_gather(qids_d, out=qx, check=False)
            qids_np = qids_h.numpy()
            hoq = (torch.empty((1, qc.k), dtype=torch.int32, pin_memory=True),
                   torch.empty((1, qc.k), dtype=torch.float32, pin_memory=True))

            def eager_logits():
                turn[0] += 1
                return qwts[turn[0] % 4].logits_topk_to_host(Rq1, qc.k, workspace=wsq1, host_out=hoq)
            dq = {"plain_calls_with_copies": _dist(torch, eager_gather, 50, hev)}
            dl = {"plain_calls_with_copies": _dist(torch, eager_logits, 52, hev)}
            dl["plain_calls_with_copies"]["single_call_us"] = _single(torch, lambda: eager_logits()[2].synchronize())
            for name, use_graphs in (("step_eager", False), ("step_graph_cached", True)):
                scq = [etg.StepCache(tq, max_ids=qids_h.numel(), max_batch=1, k=qc.k, use_graphs=use_graphs)
                       for tq in qwts]
                for sq in scq:
                    sq.residual.copy_(Rq1)
                dq[name] = _dist(torch, lambda: scq[0].gather(qids_np), 50, hev)

                def step_logits():
                    turn[0] += 1
                    return scq[turn[0] % 4].logits(1)
                dl[name] = _dist(torch, step_logits, 52, hev)
                dl[name]["single_call_us"] = _single(torch, lambda: step_logits().synchronize())
                del scq
            dq["graph_bucket_rows"] = 640
            dl["tables"] = "4 copies, cycled"
            also["qwen05b_step_gather_628_host_ids"] = dq
            also["qwen05b_step_logits_top10_B1_to_host"] = dl
            log(f"qwen05b step gather {dq}, logits {dl}")
        del qwt, qwts
        torch.cuda.empty_cache()

        g = synth.CONFIGS["gemma_embed"]
        gh = g.table()
        gt = etg.Table(torch.from_numpy(gh).to(dev), g.dtype, g.V, g.d)
        gids_host = g.ids()
        gids = torch.from_numpy(gids_host).to(dev)
        gx = torch.empty((gids.numel(), g.d), dtype=torch.float32, device=dev)
        f = lambda: gt.embed_gather(gids, scale="sqrt_d", out=gx, check=False)
        for _ in range(5):
            f()
        d = _dist(torch, f, 100, hev)
        U = int(np.unique(gids_host).size)
        alg = U * g.row_bytes + gids.numel() * g.d * 4 + gids.numel() * 4
        wref50 = also.get("write_stream_reference", {}).get("50MB", {}).get("us_per_call")
        d.update({"rows": int(gids.numel()), "distinct_rows": U, "us_per_call": d["median_us"],
                  "rows_per_s": round(gids.numel() / (d["median_us"] * 1e-6)),
                  "alg_GBps": round(alg / (d["median_us"] * 1e-6) / 1e9, 1),
                  "pct_of_write_stream_50MB": round(100 * wref50 / d["median_us"], 1) if wref50 else None})
        also["gemma_embed_gather_q8_0_x_sqrt_d"] = d
        out["gather_rows_per_s"] = d["rows_per_s"]
        log(f"gather: {d['median_us']} us")
        # the same gather with its output in the f16 and i8 residual wire formats
        for wname, wire in (("f16", etg.WIRE_F16), ("i8", etg.WIRE_I8)):
            wb = torch.empty((gids.numel(), etg.wire_row_bytes(wire, g.d)), dtype=torch.uint8, device=dev)
            f = lambda: gt.embed_gather_wire(gids, wire, scale="sqrt_d", out=wb)
            f()
            d = _dist(torch, f, 100, hev)
            algw = U * g.row_bytes + gids.numel() * wb.shape[1] + gids.numel() * 4
            d.update({"rows_per_s": round(gids.numel() / (d["median_us"] * 1e-6)), "bytes_per_row_out": int(wb.shape[1]),
                      "alg_GBps": round(algw / (d["median_us"] * 1e-6) / 1e9, 1)})
            also[f"gemma_embed_gather_q8_0_x_sqrt_d_{wname}_wire"] = d
            del wb
        del gt
        torch.cuda.empty_cache()

        # the Q8_0 lm_head (31B-shaped, 1.50 GB)
        q = synth.CONFIGS["lm31b_q8"]
        qh = q.table()
        qt = etg.Table(torch.from_numpy(qh).to(dev), q.dtype, q.V, q.d)
        del qh
        for b in q.batches:
            Rq = torch.from_numpy(q.residuals(b)).to(dev)
            d = logits_entry(qt, Rq, q.k, etg.PATH_AUTO, q.table_bytes)
            d["kernel_pct_hbm_peak"] = round(100 * q.table_bytes / (d["kernel_median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1)
            also[f"lm31b_q8_0_logits_top10_B{b}"] = d
            log(f"q8_0 B={b}: {d['median_us']} us")
        del qt
        torch.cuda.empty_cache()

        p = synth.CONFIGS["prefill"]
        ph = p.table()
        pt = etg.Table(torch.from_numpy(ph.view(np.int16)).to(dev), p.dtype, p.V, p.d)
        del ph
        Bp = p.batches[0]
        Rp = torch.from_numpy(p.residuals(Bp)).to(dev)
        flops = 2.0 * Bp * p.V * p.d
        # the automatic choice (rank path: bf16-residual tiles + exact rescoring),
        # then the hi + lo split contraction that probabilities and raw logits use
        for key, path in (("prefill_logits_top40_B1024", etg.PATH_AUTO),
                          ("prefill_logits_top40_B1024_split_gemm", etg.PATH_GEMM)):
            wsp = pt.workspace(Bp, p.k, path)
            f = lambda evs=None: pt.logits_topk(Rp, p.k, path=path, workspace=wsp, events=evs)
            for _ in range(5):  # the clocks settle over the first calls of this contraction
                f()
            d = _dist(torch, f, 20, hev, kernel=True)
            d.update({"ms_per_call": round(d["median_us"] * 1e-3, 3), "kernel_ms": round(d["kernel_median_us"] * 1e-3, 3),
                      "TFLOPs": round(flops / (d["median_us"] * 1e-6) / 1e12, 1),
                      "pct_bf16_mfma_peak": round(100 * flops / (d["median_us"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 1)})
            also[key] = d
            log(f"prefill B=1024 path={path}: {d['ms_per_call']} ms")
        del pt
        torch.cuda.empty_cache()
    if also:
        out["also"] = also

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = 1 << 30

    if not args.no_cpu_baseline:
        import oracle
        log("timing the CPU oracle on the same decode workload")
        Rh = cfg.residuals(B)
        reps, t_cpu = 0, 0.0
        while t_cpu < 10.0 and reps < 100:  # about 10 s of CPU work
            t1 = time.perf_counter()
            L, _ = oracle.logits(host, cfg.dtype, cfg.V, cfg.d, Rh)
            oracle.topk(L, k)
            t_cpu += time.perf_counter() - t1
            reps += 1
        out["cpu_baseline"] = {
            "value": round(cfg.table_bytes * reps / t_cpu / 1e9, 3),
            "unit": "GB/s",
            "cores": oracle.max_threads(),
            "cpu_model": _cpu_model(),
            "kind": "oracle",
            "sample": f"{reps} full pass(es) of logits+top-10 for 1 residual over the "
                      f"262,144 x 5,376 bf16 table (f64 accumulation), {t_cpu:.1f} s",
        }
        log(f"oracle: {reps} passes in {t_cpu:.1f} s")
        if not args.no_extras:
            # the oracle on one thread: C1-C3 and one pass of the decode step
            nthr = oracle.max_threads()
            oracle.set_threads(1)
            one = {}
            t1 = time.perf_counter()
            L, _ = oracle.logits(host, cfg.dtype, cfg.V, cfg.d, Rh)
            oracle.topk(L, k)
            one["lm31b_logits_top10_B1_s"] = round(time.perf_counter() - t1, 3)
            c1 = synth.CONFIGS["tiny"]
            h1 = c1.table()
            t1 = time.perf_counter()
            oracle.embed_gather(h1, c1.dtype, c1.V, c1.d, c1.ids())
            one["tiny_gather_64_us"] = round((time.perf_counter() - t1) * 1e6, 1)
            t1 = time.perf_counter()
            L, _ = oracle.logits(h1, c1.dtype, c1.V, c1.d, c1.residuals(4))
            oracle.topk(L, c1.k)
            one["tiny_logits_top5_B4_ms"] = round((time.perf_counter() - t1) * 1e3, 2)
            c2 = synth.CONFIGS["qwen05b"]
            h2 = c2.table()
            t1 = time.perf_counter()
            oracle.embed_gather(h2, c2.dtype, c2.V, c2.d, c2.ids())
            one["qwen05b_gather_628_us"] = round((time.perf_counter() - t1) * 1e6, 1)
            t1 = time.perf_counter()
            L, _ = oracle.logits(h2, c2.dtype, c2.V, c2.d, c2.residuals(1))
            oracle.topk(L, c2.k)
            one["qwen05b_logits_top10_B1_ms"] = round((time.perf_counter() - t1) * 1e3, 1)
            c3 = synth.CONFIGS["gemma_embed"]
            h3 = c3.table()
            t1 = time.perf_counter()
            oracle.embed_gather(h3, c3.dtype, c3.V, c3.d, c3.ids(), scale=oracle.sqrt_d(c3.d))
            one["gemma_embed_gather_16384_ms"] = round((time.perf_counter() - t1) * 1e3, 1)
            oracle.set_threads(nthr)
            out["cpu_baseline"]["single_thread"] = one
            log(f"oracle on one thread: {one}")

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
