#!/usr/bin/env python3
"""Benchmark of the C2KV hot path on one MI355X.

One step = one pass of the whole hot path over the Llama3.1-8B-shaped
single-layer workload (bf16, 32 query / 8 KV heads, head_dim 128, RoPE theta
5e5): structured-flow extraction attention of 8 documents x 4096 tokens at
k = 4 (1024 slots each, sink = first 4 tokens), composition of their slot
caches in a seeded order into an 8192-slot cache covering 32768 original
positions, a 64-token question prefill, and 256 decode steps with random
query vectors (batch 1).  Inputs are synthetic N(0, 1) tensors resident in
HBM before timing starts.

The metric is the decode attention's KV read rate (GB/s, algorithmic bytes)
together with the extraction's masked-attention TFLOP/s (visible cells only).
The 256 decode launches of a step are replayed from one HIP graph.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

Prints one JSON line.  Besides the step, it summarises the host-pool load
(--host-pool) and the extractor layer (--layer) unless --no-extras, reports the decode rate with the
256 steps spread over 16 replicas of the cache (a working set of about
0.6 GB, above the 256 MB last-level cache) and the compose rate with
its inputs and caches spread over 16 replicas (about 3 GB), and, when a counter summary
for the current decode sources is committed under profiles/, the HBM
traffic the hardware counters measured for one decode call.  It also
measures, live, the rates this GPU sustains (dense bf16 MFMA from the probe
library, HBM from a 1 GiB device copy) and reports each kernel against them
as well as against the published peaks, and times compose from a graph of
20 back-to-back calls.

Decode sweep over the other decode workloads (one JSON line each, not the
step): the Qwen2.5-7B pool (32 requests composed from 64 ragged documents
at k = 16) and the long-context sweep (64 requests at 16k..128k original
tokens at k = 4, with the uncompressed cache of the same original length as
the comparator), each a graph of decode calls over caches well above the
last-level cache:
    python bench.py --decode-sweep
Extraction at the Qwen3-14B shapes (k = 4, 8, 16; 40 layers over two buffer
sets) and compose of the Qwen2.5-7B pool, one JSON line each:
    python bench.py --extract-sweep
    python bench.py --compose-sweep
Loading stored caches from pinned host memory (32 layers of the Llama
shapes): compose reading the slot caches in place across the host link,
against copying the full caches, one JSON line:
    python bench.py --host-pool
One extractor layer (norms, frozen / C2 projections, attention, FFN) at the
Llama3.1-8B shapes over the 8 x 4096-token batch, one JSON line:
    python bench.py --layer

One phase alone, for counter runs under rocprofv3:
    python bench.py --profile-phase extract --calls 2

Profiling helpers (no GPU work):
    python bench.py --summarize DIR [DIR2] --out FILE --cmd "COMMAND"
summarises rocprofv3 output directories into a short text file: a
kernel-trace table, or (for --pmc runs, FETCH_SIZE and WRITE_SIZE passes)
per-kernel counter averages scaled by a device copy of known size that
`--calibration-copy-mib N` adds to a run.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s

# sources that define the decode call's kernels and launch shapes; a counter
# summary applies to the build whose sources hash to the recorded value
DECODE_SOURCES = ("compressed_composable_kv_amd/csrc/c2kv_decode.hip",
                  "compressed_composable_kv_amd/csrc/c2kv_device.hpp",
                  "compressed_composable_kv_amd/csrc/c2kv_launch.hpp",
                  "compressed_composable_kv_amd/csrc/c2kv_abi.cpp")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_decode_llama31_8b_1layer.txt")
CALIB_KERNEL = "neg_kernel"    # torch.neg over int32: reads and writes N MiB


def sources_sha(paths=DECODE_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for pth in paths:
        with open(os.path.join(ROOT, pth), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _db(d):
    import glob
    import sqlite3
    dbs = glob.glob(os.path.join(d, "**", "*.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return sqlite3.connect(dbs[0])


def summarize(dirs, out, cmd, calib_mib):
    """Short text summary of rocprofv3 output (see the module docstring)."""
    lines = []
    con = _db(dirs[0])
    has_pmc = con.execute("select count(*) from sqlite_master where name='counters_collection'").fetchone()[0] and \
        con.execute("select count(*) from counters_collection").fetchone()[0] > 0
    if not has_pmc:
        rows = con.execute("select name, count(*), avg(end-start), sum(end-start), min(end-start), max(end-start) "
                           "from kernels group by name order by sum(end-start) desc").fetchall()
        tot = sum(r[3] for r in rows)
        lines.append("# rocprofv3 kernel-trace summary (durations from the kernel dispatch records)")
        lines.append(f"# command: {cmd}")
        lines.append("# calls    avg_us      min_us      max_us    total_ms   share  kernel")
        for r in rows:
            lines.append(f"{r[1]:7d} {r[2] / 1e3:9.2f} {r[4] / 1e3:11.2f} {r[5] / 1e3:11.2f} {r[3] / 1e6:11.3f} "
                         f"{100 * r[3] / tot:6.1f}%  {r[0][:110]}")
    else:
        avg = {}
        for d in dirs:
            c = _db(d)
            q = ("select kernel_name, counter_name, avg(v), count(*) from (select dispatch_id, kernel_name, "
                 "counter_name, sum(value) as v from counters_collection group by dispatch_id, counter_name) "
                 "group by kernel_name, counter_name")
            for kname, cname, v, n in c.execute(q).fetchall():
                avg.setdefault(kname, {})[cname] = (v, n)
        names = sorted({c for cs in avg.values() for c in cs})
        if "FETCH_SIZE" not in names or "WRITE_SIZE" not in names:
            lines.append("# rocprofv3 --pmc summary: counter values per dispatch, averaged over dispatches")
            lines.append(f"# command: {cmd}")
            for kname, cs in sorted(avg.items()):
                if "c2kv" not in kname:
                    continue
                lines.append(f"{kname.split('(')[0][:80]}  (dispatches {max(v[1] for v in cs.values())})")
                for cname in sorted(cs):
                    lines.append(f"    {cname:32s} {cs[cname][0]:20.1f}")
            with open(out, "w") as f:
                f.write("\n".join(lines) + "\n")
            print("\n".join(lines))
            return
        calib = [k for k in avg if CALIB_KERNEL in k]
        if not calib:
            raise SystemExit("no calibration copy in the counter runs (use --calibration-copy-mib)")
        cal = avg[calib[0]]
        known_kib = calib_mib * 1024.0
        fs = known_kib / cal["FETCH_SIZE"][0]
        ws = known_kib / cal["WRITE_SIZE"][0]
        lines.append("# rocprofv3 --pmc summary: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged),")
        lines.append("# each pass a run of its own; scale factors from a device copy of known size")
        lines.append(f"# command: {cmd}")
        lines.append(f"# calibration: {calib_mib} MiB read + {calib_mib} MiB written by {CALIB_KERNEL}: "
                     f"FETCH_SIZE {cal['FETCH_SIZE'][0]:.0f} KiB, WRITE_SIZE {cal['WRITE_SIZE'][0]:.0f} KiB "
                     f"-> scale {fs:.4f} / {ws:.4f}")
        lines.append("# dispatches  FETCH_KiB  WRITE_KiB  traffic_MB(scaled)  kernel")
        traffic = {}
        for kname, cs in sorted(avg.items()):
            if "c2kv" not in kname or "FETCH_SIZE" not in cs or "WRITE_SIZE" not in cs:
                continue
            t = (cs["FETCH_SIZE"][0] * fs + cs["WRITE_SIZE"][0] * ws) * 1024.0
            short = kname.split("(")[0][:80]
            traffic[short] = t
            lines.append(f"{cs['FETCH_SIZE'][1]:11d} {cs['FETCH_SIZE'][0]:10.1f} {cs['WRITE_SIZE'][0]:10.1f} "
                         f"{t / 1e6:18.3f}  {short}")
        lines.append("# json: " + json.dumps({"sources_sha": sources_sha(), "fetch_scale": fs, "write_scale": ws,
                                              "traffic_bytes": traffic}))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def committed_traffic(kernel_keys):
    """HBM bytes per decode call from the committed counter summary, or
    None when there is none or the decode sources changed since."""
    try:
        with open(PMC_SUMMARY) as f:
            js = [l for l in f if l.startswith("# json: ")]
        info = json.loads(js[-1][len("# json: "):])
    except (OSError, IndexError, ValueError):
        return None
    if info.get("sources_sha") != sources_sha():
        return None
    tot = 0.0
    for key in kernel_keys:
        hits = [v for k, v in info["traffic_bytes"].items() if key in k]
        if len(hits) != 1:
            return None
        tot += hits[0]
    return tot


def visible_cells(n: int, k: int) -> int:
    """Visible cells of one document's structured mask with sink = k:
    n(n+1)/2 doc->doc, (m-1)k + n slot->doc (n >= k), m(m+1)/2 slot->slot."""
    m = (n + k - 1) // k
    sd = (m - 1) * k + n if n >= k else n
    return n * (n + 1) // 2 + sd + m * (m + 1) // 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the host-pool load and extractor-layer summaries")
    ap.add_argument("--cpu-decode-steps", type=int, default=24)
    ap.add_argument("--cold-replicas", type=int, default=16)
    ap.add_argument("--calibration-copy-mib", type=int, default=0)
    ap.add_argument("--summarize", nargs="+", metavar="DIR")
    ap.add_argument("--decode-sweep", action="store_true")
    ap.add_argument("--extract-sweep", action="store_true")
    ap.add_argument("--compose-sweep", action="store_true")
    ap.add_argument("--host-pool", action="store_true")
    ap.add_argument("--layer", action="store_true")
    ap.add_argument("--profile-phase", choices=("extract", "compose", "prefill", "decode"),
                    help="run only this phase of the step --calls times (for counter runs), print nothing else")
    ap.add_argument("--calls", type=int, default=2)
    ap.add_argument("--out")
    ap.add_argument("--cmd", default="")
    return ap.parse_args()


def cpu_baseline(w, M, P, tq, nsteps):
    """The oracle, as it stands, on a bounded sample of the same workload:
    `nsteps` decode steps over the full composed cache (M slots + question),
    and the extraction of one document (all 32 heads)."""
    import numpy as np
    import oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    d, hq, hkv = w.head_dim, w.hq, w.hkv
    L0 = M + tq
    ck = W.normal((L0, hkv, d), w.dtype, 90, W.P_K).float().numpy()
    cv = W.normal((L0, hkv, d), w.dtype, 90, W.P_V).float().numpy()
    t0 = time.perf_counter()
    nbytes = 0
    for s in range(nsteps):
        q = W.normal((hq, d), w.dtype, 90, W.P_DEC_Q, salt=s).float().numpy()
        kn = W.normal((hkv, d), w.dtype, 90, W.P_NEW_KV, salt=s).float().numpy()
        vn = W.normal((hkv, d), w.dtype, 90, W.P_NEW_KV, salt=1000 + s).float().numpy()
        _, _, ck, cv = O.decode_step(q, kn, vn, ck, cv, P + tq + s, w.rope_theta, "bf16")
        nbytes += ck.shape[0] * hkv * d * 2 * 2
    dec_s = time.perf_counter() - t0
    n, k = w.doc_lens[0], w.ratio_k
    rows = n + O.num_slots(n, k)
    q = W.normal((rows, hq, d), w.dtype, 91, W.P_Q).float().numpy()
    kk = W.normal((rows, hkv, d), w.dtype, 91, W.P_K).float().numpy()
    v = W.normal((rows, hkv, d), w.dtype, 91, W.P_V).float().numpy()
    t0 = time.perf_counter()
    O.extract_attn(q, kk, v, [n], k, w.sink_len, w.rope_theta)
    ext_s = time.perf_counter() - t0
    ext_flops = hq * 4 * d * visible_cells(n, k)
    return {
        "value": nbytes / dec_s / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"{nsteps} decode steps over the full {L0}-row composed cache (32/8 heads, d=128), "
                  f"plus extraction of 1 of the 8 documents (all 32 heads)",
        "decode_seconds": dec_s, "extraction_tflops": ext_flops / ext_s / 1e12, "extraction_seconds": ext_s,
        "host_cores": len(os.sched_getaffinity(0)),
    }


def decode_sweep():
    """Decode rate (algorithmic KV bytes per second) of the other decode
    workloads; caches are device-generated N(0, 1) rows (decode time does
    not depend on their values)."""
    import torch
    import compressed_composable_kv_amd as c2kv
    import workloads as W
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def run(name, lens, w, steps, extra):
        d, hq, hkv, dt = w.head_dim, w.hq, w.hkv, w.dtype
        R = len(lens)
        cap = max(lens) + steps
        ck = W.device_normal((R, hkv, cap, d), dt, w.wid, W.P_K, dev, salt=7)
        cv = W.device_normal((R, hkv, cap, d), dt, w.wid, W.P_V, dev, salt=7)
        qd = W.device_normal((steps, R, hq, d), dt, w.wid, W.P_DEC_Q, dev, salt=7)
        kd = W.device_normal((steps, R, hkv, d), dt, w.wid, W.P_NEW_KV, dev, salt=7)
        vd = W.device_normal((steps, R, hkv, d), dt, w.wid, W.P_NEW_KV, dev, salt=8)
        ws = torch.empty(max(c2kv.workspace_size_decode([x + s for x in lens], hq, hkv, d, dt)
                             for s in range(steps)), dtype=torch.uint8, device=dev)

        def loop():
            for s in range(steps):
                c2kv.attn_decode(qd[s], kd[s], vd[s], ck, cv, [x + s for x in lens], [4 * x + s for x in lens],
                                 w.rope_theta, workspace=ws)
        loop()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            loop()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (3 * steps)
        nbytes = sum((x + steps / 2 + 1) * hkv * d * 2 * 2 + (2 * hq + 2 * hkv) * d * 2 for x in lens)
        gbs = nbytes / (us * 1e-6) / 1e9
        print(json.dumps({"workload": name, "requests": R, "rows_min": min(lens), "rows_max": max(lens),
                          "us_per_step": us, "kv_bytes_per_step": nbytes, "gbs": gbs,
                          "hbm_frac": gbs / HBM_PEAK_GBS, **extra}), flush=True)
        del ck, cv, g
        torch.cuda.empty_cache()

    w3 = W.QWEN25
    pool = W.qwen25_pool(w3)
    lens3 = [sum(c2kv.num_slots(pool[t], w3.ratio_k) for t in r) for r in W.qwen25_requests(w3)]
    run("qwen25_7b_pool_decode", lens3, w3, 32, {"cache": "composed, k=16"})
    w4 = W.LONGCTX
    for nd in W.longctx_doc_counts():
        L = 4096 * nd
        run(f"llama31_8b_longctx_{L // 1024}k_c2kv", [nd * c2kv.num_slots(4096, w4.ratio_k)] * w4.num_reqs, w4, 8,
            {"cache": "composed, k=4", "original_tokens": L})
        run(f"llama31_8b_longctx_{L // 1024}k_full", [L] * w4.num_reqs, w4, 4,
            {"cache": "uncompressed comparator", "original_tokens": L})


def extract_sweep():
    """Extraction throughput at the Qwen3-14B shapes (40 query / 8 KV heads,
    d = 128, theta 1e6, bf16): 64 documents of 8192 tokens at k = 4, 8, 16
    (sink = k), 40 attention-only layers whose calls alternate over two
    input/output buffer sets.  One JSON line per k."""
    import torch
    import compressed_composable_kv_amd as c2kv
    import workloads as W
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = W.QWEN3_14B
    d, hq, hkv, dt = w.head_dim, w.hq, w.hkv, w.dtype
    lens = list(w.doc_lens)
    ach = achievable_peaks(torch, dev)
    for k in (4, 8, 16):
        rows = c2kv.packed_rows(lens, k)
        sets = []
        for b in range(2):
            q = W.device_normal((rows, hq, d), dt, w.wid, W.P_Q, dev, salt=10 * k + b)
            kk = W.device_normal((rows, hkv, d), dt, w.wid, W.P_K, dev, salt=10 * k + b)
            v = W.device_normal((rows, hkv, d), dt, w.wid, W.P_V, dev, salt=10 * k + b)
            sets.append((q, kk, v, torch.empty_like(q)))
        ws = torch.empty(c2kv.workspace_size_extract(lens, k, hkv, d, dt), dtype=torch.uint8, device=dev)

        def layer(i):
            q, kk, v, o = sets[i % 2]
            c2kv.extract_attn(q, kk, v, lens, k, k, w.rope_theta, out=o, workspace=ws)
        layer(0)
        layer(1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(w.layers):
            layer(i)
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3
        flops = w.layers * hq * 4 * d * sum(visible_cells(n, k) for n in lens)
        tf = flops / sec / 1e12
        print(json.dumps({"workload": f"qwen3_14b_extract_k{k}", "docs": len(lens), "doc_tokens": lens[0],
                          "ratio_k": k, "layers": w.layers, "seconds_40_layers": sec, "pflop": flops / 1e15,
                          "tflops": tf, "frac_of_peak": tf / BF16_PEAK_TFLOPS,
                          "frac_of_achievable": tf / ach["mfma_bf16_tflops"] if ach["mfma_bf16_tflops"] else None,
                          "target_seconds_at_half_peak": flops / (0.5 * BF16_PEAK_TFLOPS * 1e12)}), flush=True)
        del sets, ws
        torch.cuda.empty_cache()


def compose_sweep():
    """Compose throughput of the Qwen2.5-7B pool workload: 64 pre-extracted
    documents (k = 16, lengths uniform on 1024..8192, slot K/V N(0, 1)), 32
    requests each composing a seeded subset of 8..32 documents in seeded
    order.  Reports algorithmic bytes (read and write every composed row)
    and minimum traffic (the pool read once plus the writes), per call from
    a graph of 10 calls."""
    import torch
    import compressed_composable_kv_amd as c2kv
    import workloads as W
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = W.QWEN25
    d, hkv, dt, k = w.head_dim, w.hkv, w.dtype, w.ratio_k
    pool = W.qwen25_pool(w)
    reqs = W.qwen25_requests(w)
    slots = [c2kv.num_slots(n, k) for n in pool]
    kv = [(W.device_normal((m, hkv, d), dt, w.wid, W.P_K, dev, salt=100 + i),
           W.device_normal((m, hkv, d), dt, w.wid, W.P_V, dev, salt=100 + i)) for i, m in enumerate(slots)]
    requests = [[(kv[t][0], kv[t][1], pool[t]) for t in r] for r in reqs]
    M = [sum(slots[t] for t in r) for r in reqs]
    cap = max(M) + 128
    ck = torch.empty((len(reqs), hkv, cap, d), dtype=dt, device=dev)
    cv = torch.empty_like(ck)
    c2kv.compose(requests, k, w.rope_theta, ck, cv)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(10):
            c2kv.compose(requests, k, w.rope_theta, ck, cv)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 30
    es = 2
    alg = 4 * sum(M) * hkv * d * es
    used = sorted({t for r in reqs for t in r})
    minimum = 2 * sum(slots[t] for t in used) * hkv * d * es + 2 * sum(M) * hkv * d * es
    ach = achievable_peaks(torch, dev)
    print(json.dumps({"workload": "qwen25_7b_pool_compose", "requests": len(reqs), "composed_rows": sum(M),
                      "us_per_call": us, "algorithmic_bytes": alg, "min_traffic_bytes": minimum,
                      "gbs_algorithmic": alg / (us * 1e-6) / 1e9, "gbs_min_traffic": minimum / (us * 1e-6) / 1e9,
                      "frac_of_peak_min_traffic": minimum / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                      "frac_of_achievable_min_traffic": minimum / (us * 1e-6) / 1e9 / ach["hbm_copy_gbs"]}),
          flush=True)


def layer_bench(ach=None, emit=True):
    """One extractor layer at the Llama3.1-8B shapes (dm 4096, 32/8 heads of
    128, FFN 14336, bf16, theta 5e5) over 8 documents of 4096 tokens at
    k = 4 (40 960 packed rows): norms, frozen / C2 projections, structured
    attention, output projection and SwiGLU FFN.  Random N(0, 1)/sqrt(fan_in)
    weights.  FLOPs count the matrix products (dense) plus the attention's
    visible cells.  Best of five calls, HIP events."""
    import torch
    import compressed_composable_kv_amd as c2kv
    import workloads as W
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = W.LLAMA
    d, hq, hkv, k, theta = w.head_dim, w.hq, w.hkv, w.ratio_k, w.rope_theta
    dm, ffn = 4096, 14336
    lens = list(w.doc_lens)
    rows = c2kv.packed_rows(lens, k)

    def lin(o, i, salt):
        return (W.device_normal((o, i), torch.float32, w.wid, W.P_K, dev, salt=400 + salt) / math.sqrt(i)).to(
            torch.bfloat16)
    nq = (hq + 2 * hkv) * d
    wts = {"attn_norm": torch.ones(dm, dtype=torch.bfloat16, device=dev), "wqkv": lin(nq, dm, 1),
           "wqkv_c2": lin(nq, dm, 2), "wo": lin(dm, hq * d, 3),
           "ffn_norm": torch.ones(dm, dtype=torch.bfloat16, device=dev), "w_gate_up": lin(2 * ffn, dm, 4),
           "w_down": lin(dm, ffn, 5)}
    x0 = W.device_normal((rows, dm), torch.bfloat16, w.wid, W.P_Q, dev, salt=400)
    x = x0.clone()
    ko = torch.empty((rows, hkv, d), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    emb = W.device_normal((dm,), torch.bfloat16, w.wid, W.P_V, dev, salt=400)
    ws = torch.empty(c2kv.workspace_size_extract_layer(lens, k, dm, hq, hkv, d, ffn), dtype=torch.uint8, device=dev)

    def call():
        x.copy_(x0)
        c2kv.extract_layer(x, wts, ko, vo, lens, k, k, hq, theta, 1e-5, slot_embed=emb, workspace=ws)
    call()
    torch.cuda.synchronize()
    copy_ms = None
    best = None
    for _ in range(5):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record()
        x.copy_(x0)
        e1.record()
        c2kv.extract_layer(x, wts, ko, vo, lens, k, k, hq, theta, 1e-5, slot_embed=emb, workspace=ws)
        e2.record()
        torch.cuda.synchronize()
        t = e1.elapsed_time(e2)
        best = t if best is None else min(best, t)
        copy_ms = e0.elapsed_time(e1)
    gemm = 2 * rows * dm * (nq + hq * d + 2 * ffn + ffn)
    attn = hq * 4 * d * sum(visible_cells(n, k) for n in lens)
    tf = (gemm + attn) / (best * 1e-3) / 1e12
    if ach is None:
        ach = achievable_peaks(torch, dev)
    res = {"workload": "llama31_8b_extractor_layer", "docs": len(lens), "doc_tokens": lens[0],
           "ratio_k": k, "rows": rows, "dm": dm, "ffn": ffn, "ms": best, "gemm_tflop": gemm / 1e12,
           "attn_tflop": attn / 1e12, "tflops": tf, "frac_of_peak": tf / BF16_PEAK_TFLOPS,
           "frac_of_achievable": tf / ach["mfma_bf16_tflops"] if ach["mfma_bf16_tflops"] else None,
           "input_restore_copy_ms": copy_ms}
    del wts, x0, x, ko, vo, ws
    torch.cuda.empty_cache()
    if emit:
        print(json.dumps(res), flush=True)
    return res


PCIE_PEAK_GBS = 64.0           # MI355X host link, PCIe 5.0 x16, one direction, GB/s


def host_pool(emit=True):
    """Loading stored caches from host memory for one request of the
    Llama3.1-8B shapes: 8 documents of 4096 tokens, all 32 layers (8 KV
    heads, d = 128, bf16, theta 5e5), composed in the seeded order.  The
    stored caches sit in pinned host memory.  Four ways to get them into a
    realigned device cache, each over the 32 layers:
      c2kv_zero_copy   compose at k = 4 reading the slot caches in place
                       across the host link (1024 slot rows per document)
      c2kv_staged      c2kv_compose_staged: the library copies the slot
                       caches into a device workspace, then composes
      full_zero_copy   compose at k = 1 from the full caches (every token
                       kept, positions realigned: full-cache reuse)
      full_dma         copy the full caches to the device (no realignment;
                       the plain load of an uncompressed cache)
    The compose loops (staged ones with their copies) are replayed from HIP
    graphs; the full-cache copies run eagerly.
    Best of three passes.  Rates count the bytes read from host memory."""
    import torch
    import compressed_composable_kv_amd as c2kv
    import workloads as W
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = W.LLAMA
    d, hkv, dt, theta = w.head_dim, w.hkv, w.dtype, w.rope_theta
    L, ndoc, n = 32, len(w.doc_lens), w.doc_lens[0]
    k = w.ratio_k
    m = c2kv.num_slots(n, k)
    order = W.llama_doc_order(w)
    row_b = hkv * d * 2

    def pool(rows):
        hk = torch.empty((L, ndoc, rows, hkv, d), dtype=dt, pin_memory=True)
        hv = torch.empty((L, ndoc, rows, hkv, d), dtype=dt, pin_memory=True)
        for l in range(L):
            hk[l].copy_(W.device_normal((ndoc, rows, hkv, d), dt, w.wid, W.P_K, dev, salt=300 + l))
            hv[l].copy_(W.device_normal((ndoc, rows, hkv, d), dt, w.wid, W.P_V, dev, salt=300 + l))
        return hk, hv

    t0 = time.time()
    hk_c, hv_c = pool(m)
    hk_f, hv_f = pool(n)
    print(f"host pools ready ({time.time() - t0:.1f} s)", file=sys.stderr, flush=True)
    ck_c = torch.empty((L, 1, hkv, ndoc * m, d), dtype=dt, device=dev)
    cv_c = torch.empty_like(ck_c)
    ck_f = torch.empty((L, 1, hkv, ndoc * n, d), dtype=dt, device=dev)
    cv_f = torch.empty_like(ck_f)
    ws_st = torch.empty(L * 2 * ndoc * m * row_b, dtype=torch.uint8, device=dev).view(L, -1)

    def compose_layers(hk, hv, ck, cv, ratio):
        for l in range(L):
            c2kv.compose([[(hk[l, t], hv[l, t], n) for t in order]], ratio, theta, ck[l], cv[l])

    def graph_of(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        # host segments are mapped (a pointer-attribute query) while capturing
        with torch.cuda.graph(g, capture_error_mode="relaxed"):
            fn()
        torch.cuda.synchronize()
        return g

    def best_ms(fn, reps=3):
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1)
            best = t if best is None else min(best, t)
        return best

    g_c = graph_of(lambda: compose_layers(hk_c, hv_c, ck_c, cv_c, k))
    g_f = graph_of(lambda: compose_layers(hk_f, hv_f, ck_f, cv_f, 1))

    def staged_layers():
        for l in range(L):
            c2kv.compose_staged([[(hk_c[l, t], hv_c[l, t], n) for t in order]], k, theta, ck_c[l], cv_c[l],
                                workspace=ws_st[l])
    g_s = graph_of(staged_layers)
    c2kv_zc = best_ms(g_c.replay)
    full_zc = best_ms(g_f.replay)
    print(f"zero-copy compose: c2kv {c2kv_zc:.2f} ms, full {full_zc:.2f} ms", file=sys.stderr, flush=True)

    def full_dma():
        ck_f.view(L, ndoc, n, hkv, d).copy_(hk_f, non_blocking=True)
        cv_f.view(L, ndoc, n, hkv, d).copy_(hv_f, non_blocking=True)

    full_dma()
    torch.cuda.synchronize()
    full_d = best_ms(full_dma)
    c2kv_d = best_ms(g_s.replay)
    print(f"dma: full {full_d:.2f} ms, c2kv staged {c2kv_d:.2f} ms", file=sys.stderr, flush=True)
    c_bytes = 2 * L * ndoc * m * row_b
    f_bytes = 2 * L * ndoc * n * row_b
    h2d = f_bytes / (full_d * 1e-3) / 1e9
    zc = c_bytes / (c2kv_zc * 1e-3) / 1e9
    res = {
        "workload": "llama31_8b_32layer_host_pool_load", "docs": ndoc, "doc_tokens": n, "layers": L,
        "ratio_k": k, "slot_rows_per_layer": ndoc * m, "host_bytes_c2kv": c_bytes, "host_bytes_full": f_bytes,
        "c2kv_zero_copy_ms": c2kv_zc, "c2kv_staged_ms": c2kv_d, "full_zero_copy_k1_ms": full_zc,
        "full_dma_copy_ms": full_d, "c2kv_staged_gbs": c_bytes / (c2kv_d * 1e-3) / 1e9,
        "c2kv_staged_frac_of_pcie_peak": c_bytes / (c2kv_d * 1e-3) / 1e9 / PCIE_PEAK_GBS,
        "c2kv_zero_copy_gbs": zc, "full_zero_copy_gbs": f_bytes / (full_zc * 1e-3) / 1e9,
        "h2d_copy_gbs": h2d, "pcie_peak_gbs": PCIE_PEAK_GBS,
        "c2kv_zero_copy_frac_of_pcie_peak": zc / PCIE_PEAK_GBS, "c2kv_zero_copy_frac_of_h2d_copy": zc / h2d,
        "speedup_c2kv_zero_copy_vs_full_dma": full_d / c2kv_zc,
        "speedup_c2kv_best_vs_full_best": min(full_d, full_zc) / min(c2kv_zc, c2kv_d)}
    del g_c, g_f, g_s, ck_c, cv_c, ck_f, cv_f, ws_st, hk_c, hv_c, hk_f, hv_f
    torch.cuda.empty_cache()
    if emit:
        print(json.dumps(res), flush=True)
    return res


def achievable_peaks(torch, dev):
    """Rates this GPU sustains, measured live: dense bf16 MFMA from the probe
    library (independent MFMA chains on register operands, 4 waves per SIMD),
    and HBM from a 1 GiB device-to-device copy (read + write bytes).  They
    sit below the published peaks because the chip holds a lower clock under
    sustained load than its nominal 2.4 GHz."""
    import ctypes
    from compressed_composable_kv_amd import build_lib
    mfma = None
    if os.path.exists(build_lib.PROBE_LIB):
        lib = ctypes.CDLL(build_lib.PROBE_LIB)
        lib.c2kv_probe_mfma_bf16.restype = ctypes.c_double
        lib.c2kv_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
        ms = ctypes.c_float()
        rates = [lib.c2kv_probe_mfma_bf16(512, 512, 4000, ctypes.byref(ms)) for _ in range(3)]
        mfma = max(rates) if max(rates) > 0 else None
    n = 1 << 29                                   # 1 GiB of bf16
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        best = t if best is None else min(best, t)
    del src, dst
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": mfma, "hbm_copy_gbs": 2 * 2 * n / (best * 1e-3) / 1e9,
            "how": "MFMA: probe/mfma_peak.hip, 512 workgroups x 8 waves, 16 independent chains per wave; "
                   "HBM: torch copy of 1 GiB, read + write bytes over the best of 3"}


def main():
    a = parse()
    if a.summarize:
        summarize(a.summarize, a.out, a.cmd, a.calibration_copy_mib)
        return
    if a.decode_sweep:
        decode_sweep()
        return
    if a.extract_sweep:
        extract_sweep()
        return
    if a.compose_sweep:
        compose_sweep()
        return
    if a.host_pool:
        host_pool()
        return
    if a.layer:
        layer_bench()
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (this path does not shard "
              f"across GPUs).", file=sys.stderr)
        sys.exit(2)
    import torch
    import compressed_composable_kv_amd as c2kv
    import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = W.LLAMA
    d, hq, hkv, k, theta, dt = w.head_dim, w.hq, w.hkv, w.ratio_k, w.rope_theta, w.dtype
    lens = list(w.doc_lens)
    rows = c2kv.packed_rows(lens, k)
    q = W.device_normal((rows, hq, d), dt, w.wid, W.P_Q, dev)
    kk = W.device_normal((rows, hkv, d), dt, w.wid, W.P_K, dev)
    v = W.device_normal((rows, hkv, d), dt, w.wid, W.P_V, dev)
    o_ext = torch.empty_like(q)
    order = W.llama_doc_order(w)
    views = c2kv.slot_views(kk, v, lens, k)
    requests = [[views[t] for t in order]]
    M = sum(c2kv.num_slots(n, k) for n in lens)
    P = sum(lens)
    tq, S = w.tq, w.decode_steps
    cap = M + tq + S
    ck = torch.zeros((1, hkv, cap, d), dtype=dt, device=dev)
    cv = torch.zeros_like(ck)
    qp = W.device_normal((1, tq, hq, d), dt, w.wid, W.P_PREFILL, dev)
    kp = W.device_normal((1, tq, hkv, d), dt, w.wid, W.P_NEW_KV, dev)
    vp = W.device_normal((1, tq, hkv, d), dt, w.wid, W.P_NEW_KV, dev, salt=1)
    qd = W.device_normal((S, 1, hq, d), dt, w.wid, W.P_DEC_Q, dev)
    kd = W.device_normal((S, 1, hkv, d), dt, w.wid, W.P_NEW_KV, dev, salt=2)
    vd = W.device_normal((S, 1, hkv, d), dt, w.wid, W.P_NEW_KV, dev, salt=3)
    ws_ext = torch.empty(c2kv.workspace_size_extract(lens, k, hkv, d, dt), dtype=torch.uint8, device=dev)
    ws_pre = torch.empty(c2kv.workspace_size_prefill([M], tq, hq, hkv, d, dt), dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(max(c2kv.workspace_size_decode([M + tq + s], hq, hkv, d, dt) for s in range(S)),
                         dtype=torch.uint8, device=dev)

    def extract():
        c2kv.extract_attn(q, kk, v, lens, k, w.sink_len, theta, out=o_ext, workspace=ws_ext)

    def compose():
        c2kv.compose(requests, k, theta, ck, cv)

    def prefill():
        c2kv.attn_prefill(qp, kp, vp, ck, cv, [M], [P], theta, workspace=ws_pre)

    def decode_loop():
        for s in range(S):
            c2kv.attn_decode(qd[s], kd[s], vd[s], ck, cv, [M + tq + s], [P + tq + s], theta, workspace=ws_dec)

    if a.profile_phase:
        fn = {"extract": extract, "compose": compose, "prefill": prefill,
              "decode": lambda: c2kv.attn_decode(qd[0], kd[0], vd[0], ck, cv, [M + tq], [P + tq], theta,
                                                 workspace=ws_dec)}[a.profile_phase]
        if a.profile_phase in ("prefill", "decode"):
            compose()
        for _ in range(a.calls):
            fn()
        torch.cuda.synchronize()
        print(f"{a.profile_phase}: {a.calls} calls done", flush=True)
        return

    # eager pass (also the reference for the graph), then capture the decode loop
    extract(); compose(); prefill(); decode_loop()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode_loop()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_loop()
    torch.cuda.synchronize()

    def step(ev=None):
        if ev: ev[0].record()
        extract()
        if ev: ev[1].record()
        compose()
        if ev: ev[2].record()
        prefill()
        if ev: ev[3].record()
        graph.replay()
        if ev: ev[4].record()

    if a.calibration_copy_mib:
        src = torch.ones(a.calibration_copy_mib * 262144, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(a.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(a.steps):
        step(evs[i])
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)

    # decode with the steps spread over replicas of the cache (working set
    # above the last-level cache); not part of the step
    cold_gbs = None
    if a.cold_replicas > 1:
        reps = [(ck.clone(), cv.clone()) for _ in range(a.cold_replicas)]
        torch.cuda.synchronize()
        gcold = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gcold):
            for s in range(S):
                rk_, rv_ = reps[s % a.cold_replicas]
                c2kv.attn_decode(qd[s], kd[s], vd[s], rk_, rv_, [M + tq + s], [P + tq + s], theta, workspace=ws_dec)
        gcold.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            gcold.replay()
        e1.record()
        torch.cuda.synchronize()
        cold_ms = e0.elapsed_time(e1) / 3
        del gcold, reps
        torch.cuda.empty_cache()
    # compose with its inputs and caches spread over replicas (each call
    # reads and writes a different copy: a working set of about 3 GB, far
    # above the last-level cache); not part of the step
    comp_cold_gbs = None
    if a.cold_replicas > 1:
        creps = []
        for _ in range(a.cold_replicas):
            kk_r, v_r = kk.clone(), v.clone()
            vw = c2kv.slot_views(kk_r, v_r, lens, k)
            creps.append(([[vw[t] for t in order]], torch.empty_like(ck), torch.empty_like(cv), kk_r, v_r))
        torch.cuda.synchronize()
        gcc = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gcc):
            for req_r, ck_r, cv_r, _, _ in creps:
                c2kv.compose(req_r, k, theta, ck_r, cv_r)
        gcc.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            gcc.replay()
        e1.record()
        torch.cuda.synchronize()
        comp_cold_ms = e0.elapsed_time(e1) / (3 * a.cold_replicas)
        comp_cold_gbs = 4 * M * hkv * d * 2 / (comp_cold_ms * 1e-3) / 1e9
        del gcc, creps
        torch.cuda.empty_cache()
    # compose on its own: 20 back-to-back calls from a graph, per-call time
    # without the launch gap of a single eager call; not part of the step
    gcomp = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gcomp):
        for _ in range(20):
            compose()
    gcomp.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        gcomp.replay()
    e1.record()
    torch.cuda.synchronize()
    comp_graph_ms = e0.elapsed_time(e1) / 100
    del gcomp
    ach = achievable_peaks(torch, dev)

    ph = [0.0] * 4
    for e in evs:
        for j in range(4):
            ph[j] += e[j].elapsed_time(e[j + 1])
    ph = [x / a.steps for x in ph]   # ms per step
    ms_step = total_ms / a.steps

    es = 2
    ext_flops = hq * 4 * d * sum(visible_cells(n, k) for n in lens)
    comp_bytes = 4 * M * hkv * d * es
    pre_flops = 4 * d * hq * tq * (M + (tq + 1) / 2)
    dec_bytes = sum((M + tq + s + 1) * hkv * d * es * 2 + (2 * hq + 2 * hkv) * d * es for s in range(S))
    ext_tflops = ext_flops / (ph[0] * 1e-3) / 1e12
    dec_gbs = dec_bytes / (ph[3] * 1e-3) / 1e9
    if a.cold_replicas > 1:
        cold_gbs = dec_bytes / (cold_ms * 1e-3) / 1e9
    comp_gbs = comp_bytes / (ph[1] * 1e-3) / 1e9

    # dominant kernel of the step: the phase with the largest share of the step
    if ph[0] >= ph[3]:
        roof = {"bound": "mfma", "kernel": "extract_attn_kernel<bf16,128>", "achieved": ext_tflops,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ext_tflops / BF16_PEAK_TFLOPS,
                "traffic": None, "per_launch_ms": ph[0], "algorithmic_per_launch": ext_flops}
    else:
        # one launch = one c2kv_attn_decode call: decode_attn_kernel plus
        # merge_kernel, timed per call from the graph replay
        per_launch_ms = ph[3] / S
        # the decode call's merge is the 32-dim-slice instantiation (the prefill one takes whole rows)
        traffic = committed_traffic(("decode_attn_kernel", "merge_kernelIDF16bLi128ELi32E"))
        roof = {"bound": "hbm", "kernel": "c2kv_attn_decode (decode_attn_kernel<bf16,128> + merge_kernel<bf16,128,32>)",
                "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                "traffic": traffic, "per_launch_ms": per_launch_ms, "algorithmic_per_launch": dec_bytes / S}

    line = {
        "metric": "C2KV decode-attn KV GB/s (% HBM peak) + extraction masked-attn TFLOP/s",
        "value": dec_gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) Q/K/V of the workload's shapes, resident in HBM",
        "config": {"workload": "llama31_8b_1layer: extract 8 docs x 4096 tok (k=4, sink 4), compose 8192 slots "
                               "(32768 positions), prefill 64, 256 decode steps, batch 1",
                   "hq": hq, "hkv": hkv, "head_dim": d, "rope_theta": theta, "decode_graph": True},
        "hbm_frac": dec_gbs / HBM_PEAK_GBS,
        "extraction_tflops": ext_tflops,
        "extraction_frac": ext_tflops / BF16_PEAK_TFLOPS,
        "phase_ms": {"extract": ph[0], "compose": ph[1], "prefill": ph[2], "decode_256": ph[3]},
        "compose_gbs": comp_gbs,
        "compose_gbs_graph": comp_bytes / (comp_graph_ms * 1e-3) / 1e9,
        "compose_gbs_cache_replicas": comp_cold_gbs,
        "achievable": ach,
        "extraction_frac_of_achievable": ext_tflops / ach["mfma_bf16_tflops"] if ach["mfma_bf16_tflops"] else None,
        "decode_frac_of_achievable": dec_gbs / ach["hbm_copy_gbs"],
        "compose_graph_frac_of_achievable": comp_bytes / (comp_graph_ms * 1e-3) / 1e9 / ach["hbm_copy_gbs"],
        "decode_gbs_cache_replicas": cold_gbs,
        "cache_replicas": a.cold_replicas,
        "prefill_tflops": pre_flops / (ph[2] * 1e-3) / 1e12,
        "wall_s": t_wall,
        "roofline": roof,
    }
    if not a.no_extras:
        # the paths around the step, one summary each (their own modes print the full lines)
        hp = host_pool(emit=False)
        line["host_pool_load"] = {k_: hp[k_] for k_ in (
            "c2kv_zero_copy_ms", "c2kv_staged_ms", "full_dma_copy_ms", "full_zero_copy_k1_ms", "c2kv_zero_copy_gbs",
            "h2d_copy_gbs", "c2kv_zero_copy_frac_of_pcie_peak", "speedup_c2kv_best_vs_full_best")}
        line["host_pool_load"]["workload"] = "32 layers of the Llama shapes, 8 x 4096-token documents, k=4, from pinned host memory"
        ly = layer_bench(ach=ach, emit=False)
        line["extractor_layer"] = {k_: ly[k_] for k_ in ("ms", "tflops", "frac_of_peak", "frac_of_achievable")}
        line["extractor_layer"]["workload"] = "one Llama3.1-8B-shaped extractor layer over 8 x 4096 tokens (synthetic weights)"
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, M, P, tq, a.cpu_decode_steps)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
