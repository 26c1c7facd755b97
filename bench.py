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


def write_traffic(fetch_csv: str, write_csv: str, kernel: str = "stream_logits_kernel<1>") -> dict:
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    hev = _HipEvents()
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
    kernel_name = "stream_logits_kernel<1>"
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
        # single-call latency of the decode step: each step alone between two
        # synchronisations (median, p10, p90 of 20), beside the back-to-back average
        lat = []
        for _ in range(20):
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            s0.record()
            step()
            s1.record()
            torch.cuda.synchronize()
            lat.append(s0.elapsed_time(s1) * 1e3)
        also["decode_step_single_call_us"] = {
            "median": round(float(np.median(lat)), 1), "p10": round(float(np.percentile(lat, 10)), 1),
            "p90": round(float(np.percentile(lat, 90)), 1)}
        # a plain read stream of the same 2.82 GB on the same box (the library's
        # etg_hbm_read_probe), as a measured reference beside the 8 TB/s nominal
        sink = torch.empty(1, dtype=torch.int32, device=dev)
        f = lambda: etg.hbm_read_probe(rows, sink)
        for _ in range(3):
            f()
        mrs, _ = _timed(torch, f, 20)
        rs_gbps = cfg.table_bytes / (mrs * 1e-3) / 1e9
        also["read_stream_reference"] = {
            "what": "etg_hbm_read_probe over the 2.82 GB table", "us_per_call": round(mrs * 1e3, 1),
            "GBps": round(rs_gbps, 1), "pct_hbm_peak": round(100 * rs_gbps / HBM_PEAK_GBPS, 1),
            "roofline_kernel_pct_of_it": round(100 * achieved / rs_gbps, 1)}
        log(f"read stream reference: {rs_gbps:.0f} GB/s")
    if ms_graph is not None:
        also["decode_step_hipgraph_replay"] = {
            "ms_per_step": round(ms_graph, 4),
            "GBps": round(step_bytes / (ms_graph * 1e-3) / 1e9, 1)}
    if not args.no_extras:
        # the automatic choice (stream up to 8 rows, wide up to 16, then the rank
        # path), and the exact wide kernel at 64 rows for comparison
        for b, path, key in ((8, etg.PATH_AUTO, "lm31b_logits_top10_B8"), (16, etg.PATH_AUTO, "lm31b_logits_top10_B16"),
                             (32, etg.PATH_AUTO, "lm31b_logits_top10_B32"), (64, etg.PATH_AUTO, "lm31b_logits_top10_B64"),
                             (64, etg.PATH_WIDE, "lm31b_logits_top10_B64_exact_wide")):
            Rb = torch.from_numpy(cfg.residuals(b)).to(dev)
            wsb = table.workspace(b, k, path)
            f = lambda evs=None: table.logits_topk(Rb, k, path=path, workspace=wsb, events=evs)
            for _ in range(3):
                f()
            mb, kb = _timed(torch, f, 20, events=hev)
            also[key] = {
                "us_per_call": round(mb * 1e3, 1), "kernel_us": round(kb * 1e3, 1),
                "GBps": round(cfg.table_bytes / (mb * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * cfg.table_bytes / (mb * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1)}
            log(f"B={b} path={path}: {mb * 1e3:.1f} us")
        # the logits response with probabilities at T = 1, and the raw logits mode
        R1 = torch.from_numpy(cfg.residuals(1)).to(dev)
        ws1 = table.workspace(1, k)
        f = lambda: table.logits_topk_probs(R1, k, temperature=1.0, workspace=ws1)
        f()
        mq, _ = _timed(torch, f, 20)
        also["lm31b_logits_top10_probs_B1"] = {
            "us_per_call": round(mq * 1e3, 1), "GBps": round(cfg.table_bytes / (mq * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * cfg.table_bytes / (mq * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1)}
        raw = torch.empty((1, cfg.V), dtype=torch.float32, device=dev)
        wsr = torch.empty(max(table.workspace_bytes(1, 1), 256), dtype=torch.uint8, device=dev)
        f = lambda: table.logits_raw(R1, out=raw, workspace=wsr)
        f()
        mr, _ = _timed(torch, f, 20)
        rbytes = cfg.table_bytes + cfg.V * 4
        also["lm31b_logits_raw_B1"] = {
            "us_per_call": round(mr * 1e3, 1), "GBps": round(rbytes / (mr * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * rbytes / (mr * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1)}
        log(f"probs B=1: {mq * 1e3:.1f} us, raw B=1: {mr * 1e3:.1f} us")
    del table, rows
    torch.cuda.empty_cache()

    if not args.no_extras:
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
        f()
        mqg, _ = _timed(torch, f, 100)
        also["qwen05b_gather_628_zipf_ids"] = {
            "rows": int(qids.numel()), "distinct_rows": int(np.unique(qids_host).size),
            "us_per_call": round(mqg * 1e3, 2), "rows_per_s": round(qids.numel() / (mqg * 1e-3))}
        Rq1 = torch.from_numpy(qc.residuals(1)).to(dev)
        wsq1 = qwt.workspace(1, qc.k)
        turn = [0]

        def fq(evs=None):
            turn[0] += 1
            return qwts[turn[0] % 4].logits_topk(Rq1, qc.k, workspace=wsq1, events=evs)
        for _ in range(4):
            fq()
        mql, kql = _timed(torch, fq, 52, events=hev)
        also["qwen05b_logits_top10_B1"] = {
            "us_per_call": round(mql * 1e3, 1), "kernel_us": round(kql * 1e3, 1),
            "GBps": round(qc.table_bytes / (mql * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * qc.table_bytes / (mql * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
            "tables": "4 copies, cycled"}
        log(f"qwen05b gather {mqg * 1e3:.1f} us, logits B=1 {mql * 1e3:.1f} us")
        del qwt, qwts
        torch.cuda.empty_cache()

        g = synth.CONFIGS["gemma_embed"]
        gh = g.table()
        gt = etg.Table(torch.from_numpy(gh).to(dev), g.dtype, g.V, g.d)
        gids_host = g.ids()
        gids = torch.from_numpy(gids_host).to(dev)
        gx = torch.empty((gids.numel(), g.d), dtype=torch.float32, device=dev)
        f = lambda: gt.embed_gather(gids, scale="sqrt_d", out=gx, check=False)
        f()
        mg, _ = _timed(torch, f, 100)
        U = int(np.unique(gids_host).size)
        alg = U * g.row_bytes + gids.numel() * g.d * 4 + gids.numel() * 4
        also["gemma_embed_gather_q8_0_x_sqrt_d"] = {
            "rows": int(gids.numel()), "distinct_rows": U, "us_per_call": round(mg * 1e3, 2),
            "rows_per_s": round(gids.numel() / (mg * 1e-3)), "alg_GBps": round(alg / (mg * 1e-3) / 1e9, 1)}
        out["gather_rows_per_s"] = also["gemma_embed_gather_q8_0_x_sqrt_d"]["rows_per_s"]
        log(f"gather: {mg * 1e3:.1f} us")
        # the same gather with its output in the f16 and i8 residual wire formats
        for wname, wire in (("f16", etg.WIRE_F16), ("i8", etg.WIRE_I8)):
            wb = torch.empty((gids.numel(), etg.wire_row_bytes(wire, g.d)), dtype=torch.uint8, device=dev)
            f = lambda: gt.embed_gather_wire(gids, wire, scale="sqrt_d", out=wb)
            f()
            mw, _ = _timed(torch, f, 100)
            algw = U * g.row_bytes + gids.numel() * wb.shape[1] + gids.numel() * 4
            also[f"gemma_embed_gather_q8_0_x_sqrt_d_{wname}_wire"] = {
                "us_per_call": round(mw * 1e3, 2), "rows_per_s": round(gids.numel() / (mw * 1e-3)),
                "bytes_per_row_out": int(wb.shape[1]), "alg_GBps": round(algw / (mw * 1e-3) / 1e9, 1)}
            del wb
        del gt
        torch.cuda.empty_cache()

        # the Q8_0 lm_head (31B-shaped, 1.50 GB): the q8 stream path
        q = synth.CONFIGS["lm31b_q8"]
        qh = q.table()
        qt = etg.Table(torch.from_numpy(qh).to(dev), q.dtype, q.V, q.d)
        del qh
        for b in q.batches:
            Rq = torch.from_numpy(q.residuals(b)).to(dev)
            wsq = qt.workspace(b, q.k)
            f = lambda evs=None: qt.logits_topk(Rq, q.k, workspace=wsq, events=evs)
            f()
            mq8, kq8 = _timed(torch, f, 20, events=hev)
            also[f"lm31b_q8_0_logits_top10_B{b}"] = {
                "us_per_call": round(mq8 * 1e3, 1), "kernel_us": round(kq8 * 1e3, 1),
                "GBps": round(q.table_bytes / (mq8 * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * q.table_bytes / (mq8 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1)}
            log(f"q8_0 B={b}: {mq8 * 1e3:.1f} us")
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
            mp, kp = _timed(torch, f, 10, events=hev)
            also[key] = {
                "ms_per_call": round(mp, 3), "kernel_ms": round(kp, 3),
                "TFLOPs": round(flops / (mp * 1e-3) / 1e12, 1),
                "pct_bf16_mfma_peak": round(100 * flops / (mp * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 1)}
            log(f"prefill B=1024 path={path}: {mp:.2f} ms")
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
