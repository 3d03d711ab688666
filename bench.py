#!/usr/bin/env python3
"""Benchmark of the C2KV hot path on one MI355X.

Metric: C2KV decode-attention KV read rate (GB/s of algorithmic bytes, and
its fraction of the 8 TB/s HBM peak) together with the extraction's
masked-attention rate (TFLOP/s of visible cells, and its fraction of the
2.5 PFLOP/s dense bf16 MFMA peak).  Each part is measured on the largest
workload of its kind that fits one GPU:

  headline (value, roofline)  long-context decode, Llama3.1-8B shapes (32/8
      heads, d 128, bf16, theta 5e5), all 32 layers attention-only, 64
      requests, composed context of 32 documents of 4096 tokens at k = 4:
      32 768 composed slots covering 131 072 original tokens.  One step is
      one decode call per layer (32 calls, each appending a row and reading
      every cache row of the 64 requests).  The 32 layer caches cycle over a
      pool of distinct layer buffers, each far above the 256 MB last-level
      cache; the K timed steps are replayed from one HIP graph.
  extraction_roofline  Qwen3-14B-shaped extraction (40/8 heads, d 128,
      theta 1e6): 64 documents of 8192 tokens at k = 4, 40 attention-only
      layers over two buffer sets.

Reported alongside, in the same JSON line:
  longctx_sweep   decode at 16k/32k/64k/128k original tokens (4096..32768
                  slots), C2KV and the uncompressed full-cache comparator
  extraction      Qwen3-14B extraction at k = 4, 8 and 16
  qwen25          the Qwen2.5-7B pool (64 documents, k = 16, lengths
                  uniform on 1024..8192): decode of 32 requests composed
                  from 8..32 documents each, and their composition (minimum
                  traffic basis), both over replicas well above the
                  last-level cache
  llama_layer     the Llama3.1-8B single layer pass: extraction of 8 x 4096
                  tokens, composition into 8192 slots, 64-token prefill and
                  256 decode steps (batch 1), decode over cache replicas
  host_pool_load, extractor_layer  (unless --no-extras)
  achievable      rates this GPU sustains, measured live: dense bf16 MFMA
                  (probe), a streaming HBM read (probe), a device copy
  cpu_baseline    the oracle on a bounded sample, timed on the host cores

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]

Inputs are synthetic N(0, 1) tensors resident in HBM before timing starts.

Sections on their own (one JSON line each), e.g. for profiler runs:
    python bench.py --only headline|longctx|extract|qwen25|llama
One phase of a workload alone, for counter runs under rocprofv3:
    python bench.py --profile-phase decode128k|compose_qwen25|extract_qwen3|extract|compose|prefill|decode
Older single-purpose modes: --decode-sweep, --extract-sweep, --compose-sweep, --host-pool, --layer.

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
PCIE_PEAK_GBS = 64.0           # MI355X host link, PCIe 5.0 x16, one direction, GB/s

# sources that define the decode call's kernels and launch shapes; a counter
# summary applies to the build whose sources hash to the recorded value
DECODE_SOURCES = ("compressed_composable_kv_amd/csrc/c2kv_decode.hip",
                  "compressed_composable_kv_amd/csrc/c2kv_device.hpp",
                  "compressed_composable_kv_amd/csrc/c2kv_cache.cpp")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_decode_llama31_8b_longctx_128k.txt")
# the same for the compose kernel and its launch table
COMPOSE_SOURCES = ("compressed_composable_kv_amd/csrc/c2kv_aux.hip",
                   "compressed_composable_kv_amd/csrc/c2kv_launch.hpp",
                   "compressed_composable_kv_amd/csrc/c2kv_device.hpp",
                   "compressed_composable_kv_amd/csrc/c2kv_abi.cpp")
COMPOSE_PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_compose_qwen25_7b_pool.txt")
CALIB_KERNEL = "neg_kernel"    # torch.neg over int32: reads and writes N MiB
POOL_BYTES = 96 << 30          # device memory given to a pool of layer buffers


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def sources_sha(paths=DECODE_SOURCES) -> str:
    """Hash of the sources' code: comments and blank space are dropped
    first, so an edit to the wording of a comment does not retire a counter
    summary taken from the same code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for pth in paths:
        with open(os.path.join(ROOT, pth), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
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
        durs = {}
        for name, dt in con.execute("select name, end-start from kernels"):
            durs.setdefault(name, []).append(dt)
        tot = sum(r[3] for r in rows)
        lines.append("# rocprofv3 kernel-trace summary (durations from the kernel dispatch records)")
        lines.append(f"# command: {cmd}")
        lines.append("# calls    avg_us   median_us      min_us      max_us    total_ms   share  kernel")
        for r in rows:
            d = sorted(durs[r[0]])
            med = d[len(d) // 2] if len(d) % 2 else 0.5 * (d[len(d) // 2 - 1] + d[len(d) // 2])
            lines.append(f"{r[1]:7d} {r[2] / 1e3:9.2f} {med / 1e3:11.2f} {r[4] / 1e3:11.2f} {r[5] / 1e3:11.2f} "
                         f"{r[3] / 1e6:11.3f} {100 * r[3] / tot:6.1f}%  {r[0][:110]}")
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
        lines.append("# json: " + json.dumps({"sources_sha": sources_sha(), "compose_sources_sha": sources_sha(COMPOSE_SOURCES),
                                              "fetch_scale": fs, "write_scale": ws, "traffic_bytes": traffic}))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def committed_traffic(kernel_keys, path=PMC_SUMMARY, sources=DECODE_SOURCES, sha_key="sources_sha"):
    """HBM bytes per call from a committed counter summary, or None when
    there is none or the sources changed since it was taken."""
    try:
        with open(path) as f:
            js = [l for l in f if l.startswith("# json: ")]
        info = json.loads(js[-1][len("# json: "):])
    except (OSError, IndexError, ValueError):
        return None
    if info.get(sha_key) != sources_sha(sources):
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


def decode_call_bytes(lens, hq, hkv, d, es=2):
    """Algorithmic bytes of one decode call: every cache row (the new one
    included) of K and V read once, plus q, o, k_new and v_new."""
    return sum((L + 1) * hkv * d * es * 2 for L in lens) + len(lens) * (2 * hq + 2 * hkv) * d * es


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the host-pool load and extractor-layer summaries")
    ap.add_argument("--only", choices=("headline", "longctx", "extract", "qwen25", "llama"))
    ap.add_argument("--cold-replicas", type=int, default=16)
    ap.add_argument("--calibration-copy-mib", type=int, default=0)
    ap.add_argument("--summarize", nargs="+", metavar="DIR")
    ap.add_argument("--decode-sweep", action="store_true")
    ap.add_argument("--extract-sweep", action="store_true")
    ap.add_argument("--compose-sweep", action="store_true")
    ap.add_argument("--host-pool", action="store_true")
    ap.add_argument("--layer", action="store_true")
    ap.add_argument("--profile-phase", choices=("decode128k", "compose_qwen25", "extract_qwen3",
                                                "extract", "compose", "prefill", "decode"),
                    help="run only this phase (for rocprofv3 counter runs)")
    ap.add_argument("--calls", type=int, default=2)
    ap.add_argument("--out")
    ap.add_argument("--cmd", default="")
    return ap.parse_args()


# ------------------------------------------------------------ timing helpers

def _torch():
    import torch
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    return torch, dev


def fill_normal(torch, shape, dtype, seed, dev):
    """Bulk N(0, 1) device tensor drawn directly in its dtype (timing
    inputs: values do not change the work)."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return torch.empty(tuple(int(s) for s in shape), dtype=dtype, device=dev).normal_(generator=g)


def capture(torch, fn):
    """fn run once eagerly on a side stream, then captured in a HIP graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_replays(torch, g, reps=1):
    """Milliseconds per replay of g (HIP events around `reps` back-to-back
    replays on the stream they run on), after one untimed replay."""
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def free(torch):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def achievable_peaks(torch, dev):
    """Rates this GPU sustains, measured live: dense bf16 MFMA from the probe
    library (independent MFMA chains on register operands), a non-temporal
    streaming read of 16 GiB (probe library: read bytes per second, the
    ceiling for read-dominated kernels such as decode), and a 1 GiB device copy (read +
    write bytes per second).  They sit below the published peaks because the
    chip holds a lower clock under sustained load than its nominal 2.4 GHz,
    and HBM never delivers its full pin rate."""
    import ctypes
    from compressed_composable_kv_amd import build_lib
    mfma = mfma_data = read = None
    read_blocks = None
    if os.path.exists(build_lib.PROBE_LIB):
        lib = ctypes.CDLL(build_lib.PROBE_LIB)
        lib.c2kv_probe_mfma_bf16.restype = ctypes.c_double
        lib.c2kv_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
        lib.c2kv_probe_mfma_bf16_data.restype = ctypes.c_double
        lib.c2kv_probe_mfma_bf16_data.argtypes = lib.c2kv_probe_mfma_bf16.argtypes
        ms = ctypes.c_float()
        # 40 000 iterations: about 20 ms per kernel, long enough for the
        # clock to settle where the board's power allows
        rates = [lib.c2kv_probe_mfma_bf16(512, 512, 40000, ctypes.byref(ms)) for _ in range(3)]
        mfma = max(rates) if max(rates) > 0 else None
        rates = [lib.c2kv_probe_mfma_bf16_data(512, 512, 40000, ctypes.byref(ms)) for _ in range(3)]
        mfma_data = max(rates) if max(rates) > 0 else None
        lib.c2kv_probe_hbm_read.restype = ctypes.c_double
        lib.c2kv_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64,
                                            ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
        buf = torch.ones(16 << 30, dtype=torch.uint8, device=dev)
        out = torch.empty(4 * 256 * 16384, dtype=torch.uint8, device=dev)
        for blocks in (256, 512, 1024, 2048):
            r = lib.c2kv_probe_hbm_read(buf.data_ptr(), buf.numel(), out.data_ptr(), out.numel(), blocks, 5,
                                        ctypes.byref(ms))
            if r > 0 and (read is None or r > read):
                read, read_blocks = r, blocks
        del buf, out
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
    free(torch)
    return {"mfma_bf16_tflops": mfma, "mfma_bf16_data_tflops": mfma_data, "hbm_read_gbs": read,
            "hbm_copy_gbs": 2 * 2 * n / (best * 1e-3) / 1e9,
            "how": "MFMA: probe/mfma_peak.hip, 512 workgroups x 8 waves, 16 independent chains per wave, "
                   "40 000 iterations, best of 3; constant operands (the same two registers for every MFMA) and "
                   "data operands (4 x 4 random operand registers, different for consecutive MFMAs: the rate "
                   "left for MFMA work on real data at the board's power limit); "
                   f"HBM read: probe/hbm_read.hip, non-temporal streaming read of 16 GiB, a contiguous share per "
                   f"workgroup ({read_blocks} workgroups; best of 256-2048), best of 5; "
                   "copy: torch copy of 1 GiB, read + write bytes, best of 3"}


def _frac(x, peak):
    return x / peak if (x is not None and peak) else None


# ------------------------------------------- long-context decode (32 layers)

def longctx_decode(torch, dev, ndocs, full, steps, warmup, pool_bytes=POOL_BYTES, emit=False):
    """Decode over the long-context workload: 64 requests of the Llama
    shapes, all 32 layers, composed context of `ndocs` documents of 4096
    tokens at k = 4 (C2KV: ndocs * 1024 slots per request) or the
    uncompressed cache of the same original length (full = True).  The 32
    layer calls of a step go to a pool of P distinct layer buffers (layer l
    uses buffer l mod P; P from the memory budget, at most 32), each layer
    buffer far above the last-level cache.  `warmup` eager steps, then
    `steps` steps captured in one HIP graph, replayed once untimed and once
    timed (HIP events around the replay).  Layers that share a buffer append
    to the same row of it, which changes no amount of work."""
    import compressed_composable_kv_amd as c2kv
    import workloads as W
    w = W.LONGCTX
    d, hq, hkv, theta, dt = w.head_dim, w.hq, w.hkv, w.rope_theta, w.dtype
    R, layers = w.num_reqs, w.layers
    L_orig = 4096 * ndocs
    M = L_orig if full else ndocs * c2kv.num_slots(4096, w.ratio_k)
    cap = M + warmup + steps + 8
    layer_bytes = 2 * R * hkv * cap * d * 2
    P = int(max(2, min(layers, pool_bytes // layer_bytes)))
    t0 = time.time()
    bufs = [(fill_normal(torch, (R, hkv, cap, d), dt, 4_000_000 + 10 * i, dev),
             fill_normal(torch, (R, hkv, cap, d), dt, 4_000_001 + 10 * i, dev)) for i in range(P)]
    qd = fill_normal(torch, (layers, R, hq, d), dt, 4_100_000 + ndocs, dev)
    kd = fill_normal(torch, (layers, R, hkv, d), dt, 4_100_001 + ndocs, dev)
    vd = fill_normal(torch, (layers, R, hkv, d), dt, 4_100_002 + ndocs, dev)
    ws = torch.empty(max(c2kv.workspace_size_decode([M + s] * R, hq, hkv, d, dt) for s in range(warmup + steps + 1)),
                     dtype=torch.uint8, device=dev)
    free(torch)
    log(f"longctx {L_orig // 1024}k {'full' if full else 'c2kv'}: {P} layer buffers of {layer_bytes / 1e9:.2f} GB "
        f"ready ({time.time() - t0:.1f} s)")

    def step(s):
        for layer in range(layers):
            ck, cv = bufs[layer % P]
            c2kv.attn_decode(qd[layer], kd[layer], vd[layer], ck, cv, [M + s] * R, [L_orig + s] * R, theta,
                             workspace=ws)
    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    g = capture(torch, lambda: [step(warmup + s) for s in range(steps)])
    ms = time_replays(torch, g, 1)
    nbytes = sum(decode_call_bytes([M + warmup + s] * R, hq, hkv, d) for s in range(steps)) * layers
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"workload": f"llama31_8b_longctx_{L_orig // 1024}k_{'full' if full else 'c2kv'}",
           "cache": "uncompressed comparator" if full else "composed, k=4",
           "original_tokens": L_orig, "rows_per_request": M, "requests": R, "layers": layers,
           "layer_buffers": P, "layer_buffer_gb": layer_bytes / 1e9, "steps": steps, "warmup": warmup,
           "ms_per_step": ms / steps, "ms_per_call": ms / (steps * layers),
           "bytes_per_step": nbytes / steps, "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    del g, bufs, qd, kd, vd, ws
    free(torch)
    if emit:
        print(json.dumps(res), flush=True)
    return res


def longctx_sweep(torch, dev, headline=None, emit=False):
    """C2KV and full-cache decode at 16k..128k original tokens (32 layers,
    64 requests); the 128k C2KV entry is the headline's own run when given."""
    import workloads as W
    out = []
    for nd in W.longctx_doc_counts():
        c = headline if (headline is not None and nd == 32) else longctx_decode(torch, dev, nd, False, 4, 1)
        f = longctx_decode(torch, dev, nd, True, 2 if nd >= 16 else 4, 1)
        row = {"original_tokens": 4096 * nd, "c2kv_ms_per_step": c["ms_per_step"], "c2kv_gbs": c["gbs"],
               "c2kv_hbm_frac": c["hbm_frac"], "c2kv_layer_buffers": c["layer_buffers"],
               "full_ms_per_step": f["ms_per_step"], "full_gbs": f["gbs"], "full_hbm_frac": f["hbm_frac"],
               "full_layer_buffers": f["layer_buffers"], "speedup_c2kv_vs_full": f["ms_per_step"] / c["ms_per_step"]}
        log(f"longctx {nd * 4}k: c2kv {c['ms_per_step']:.2f} ms/step {c['gbs']:.0f} GB/s, "
            f"full {f['ms_per_step']:.2f} ms/step {f['gbs']:.0f} GB/s")
        out.append(row)
        if emit:
            print(json.dumps(row), flush=True)
    return out


# --------------------------------------------- Qwen3-14B extraction (40 layers)

def qwen3_extract(torch, dev, k, emit=False):
    """Extraction at the Qwen3-14B shapes (40 query / 8 KV heads, d = 128,
    theta 1e6, bf16): 64 documents of 8192 tokens at ratio k (sink = k), 40
    attention-only layer calls alternating over two input/output buffer
    sets (eager, HIP events around the 40 calls, after two untimed calls)."""
    import compressed_composable_kv_amd as c2kv
    import workloads as W
    w = W.QWEN3_14B
    d, hq, hkv, dt = w.head_dim, w.hq, w.hkv, w.dtype
    lens = list(w.doc_lens)
    rows = c2kv.packed_rows(lens, k)
    sets = []
    for b in range(2):
        q = fill_normal(torch, (rows, hq, d), dt, 5_000_000 + 10 * k + b, dev)
        kk = fill_normal(torch, (rows, hkv, d), dt, 5_100_000 + 10 * k + b, dev)
        v = fill_normal(torch, (rows, hkv, d), dt, 5_200_000 + 10 * k + b, dev)
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
    flops_call = hq * 4 * d * sum(visible_cells(n, k) for n in lens)
    tf = w.layers * flops_call / sec / 1e12
    res = {"workload": f"qwen3_14b_extract_k{k}", "docs": len(lens), "doc_tokens": lens[0], "ratio_k": k,
           "layers": w.layers, "seconds_40_layers": sec, "ms_per_call": sec * 1e3 / w.layers,
           "flop_per_call": flops_call, "pflop_40_layers": w.layers * flops_call / 1e15, "tflops": tf,
           "frac_of_peak": tf / BF16_PEAK_TFLOPS,
           "target_seconds_at_half_peak": w.layers * flops_call / (0.5 * BF16_PEAK_TFLOPS * 1e12)}
    del sets, ws
    free(torch)
    if emit:
        print(json.dumps(res), flush=True)
    return res


# -------------------------------------------------- Qwen2.5-7B pool (decode, compose)

def qwen25(torch, dev, replicas=8, steps=16, emit=False):
    """The Qwen2.5-7B pool (28/4 heads, d = 128, theta 1e6, k = 16; 64
    documents with lengths uniform on 1024..8192): 32 requests composing
    seeded subsets of 8..32 documents in seeded order.
      decode   `steps` steps of all 32 requests from one graph, step s over
               replica s mod `replicas` of the composed caches (each replica
               holds every request's cache; the set spans several GB)
      compose  one call per replica of (pool, caches) from one graph;
               rates on the algorithmic basis (every composed row read and
               written) and the minimum-traffic basis (each pool document
               read once, every composed row written)."""
    import compressed_composable_kv_amd as c2kv
    import workloads as W
    w = W.QWEN25
    d, hq, hkv, dt, k, theta = w.head_dim, w.hq, w.hkv, w.dtype, w.ratio_k, w.rope_theta
    pool = W.qwen25_pool(w)
    reqs = W.qwen25_requests(w)
    slots = [c2kv.num_slots(n, k) for n in pool]
    Ms = [sum(slots[t] for t in r) for r in reqs]
    R = len(reqs)
    cap = max(Ms) + steps + 2
    # decode over cache replicas
    reps = [(fill_normal(torch, (R, hkv, cap, d), dt, 3_000_000 + 2 * i, dev),
             fill_normal(torch, (R, hkv, cap, d), dt, 3_000_001 + 2 * i, dev)) for i in range(replicas)]
    qd = fill_normal(torch, (steps, R, hq, d), dt, 3_100_000, dev)
    kd = fill_normal(torch, (steps, R, hkv, d), dt, 3_100_001, dev)
    vd = fill_normal(torch, (steps, R, hkv, d), dt, 3_100_002, dev)
    nxt = [sum(pool[t] for t in r) for r in reqs]
    ws = torch.empty(max(c2kv.workspace_size_decode([x + s for x in Ms], hq, hkv, d, dt) for s in range(steps)),
                     dtype=torch.uint8, device=dev)

    def dec():
        for s in range(steps):
            ck, cv = reps[s % replicas]
            c2kv.attn_decode(qd[s], kd[s], vd[s], ck, cv, [x + s for x in Ms], [x + s for x in nxt], theta,
                             workspace=ws)
    g = capture(torch, dec)
    dms = time_replays(torch, g, 3)
    dbytes = sum(decode_call_bytes([x + s for x in Ms], hq, hkv, d) for s in range(steps))
    del g, reps, qd, kd, vd, ws
    free(torch)
    # compose over replicas of the pool and the caches
    creps = []
    for i in range(replicas):
        kv = [(fill_normal(torch, (m, hkv, d), dt, 3_200_000 + 1000 * i + 2 * t, dev),
               fill_normal(torch, (m, hkv, d), dt, 3_200_001 + 1000 * i + 2 * t, dev)) for t, m in enumerate(slots)]
        requests = [[(kv[t][0], kv[t][1], pool[t]) for t in r] for r in reqs]
        ck = torch.empty((R, hkv, max(Ms), d), dtype=dt, device=dev)
        creps.append((requests, ck, torch.empty_like(ck)))
    g = capture(torch, lambda: [c2kv.compose(rq, k, theta, ck, cv) for rq, ck, cv in creps])
    cms = time_replays(torch, g, 3) / replicas
    alg = 4 * sum(Ms) * hkv * d * 2
    used = sorted({t for r in reqs for t in r})
    minimum = 2 * sum(slots[t] for t in used) * hkv * d * 2 + 2 * sum(Ms) * hkv * d * 2
    del g, creps
    free(torch)
    res = {"workload": "qwen25_7b_pool", "requests": R, "composed_rows": sum(Ms), "rows_min": min(Ms),
           "rows_max": max(Ms), "replicas": replicas,
           "decode_us_per_step": dms * 1e3 / steps, "decode_bytes_per_step": dbytes / steps,
           "decode_gbs": dbytes / (dms * 1e-3) / 1e9, "decode_hbm_frac": dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "compose_us_per_call": cms * 1e3, "compose_algorithmic_bytes": alg, "compose_min_traffic_bytes": minimum,
           "compose_gbs_algorithmic": alg / (cms * 1e-3) / 1e9,
           "compose_gbs_min_traffic": minimum / (cms * 1e-3) / 1e9,
           "compose_hbm_frac_min_traffic": minimum / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "compose_traffic_bytes": committed_traffic(("compose_kernel",), COMPOSE_PMC_SUMMARY, COMPOSE_SOURCES,
                                                      "compose_sources_sha")}
    if emit:
        print(json.dumps(res), flush=True)
    return res


# ------------------------------------------ Llama3.1-8B single layer (the old step)

def llama_layer_step(torch, dev, steps, warmup, replicas=16, emit=False, profile_phase=None, calls=2,
                     calibration_copy_mib=0):
    """The Llama3.1-8B single-layer pass (bf16, 32/8 heads, d = 128, theta
    5e5): extraction of 8 documents x 4096 tokens at k = 4 (sink 4),
    composition of their slot caches in a seeded order into 8192 slots
    covering 32768 positions, a 64-token question prefill and 256 decode
    steps (batch 1, one graph).  Reports each phase per pass, and decode and
    compose again over `replicas` copies of their inputs and caches so the
    working set is far above the last-level cache (these are the figures of
    record for the two small HBM-bound steps)."""
    import compressed_composable_kv_amd as c2kv
    import workloads as W
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

    if profile_phase:
        fn = {"extract": extract, "compose": compose, "prefill": prefill,
              "decode": lambda: c2kv.attn_decode(qd[0], kd[0], vd[0], ck, cv, [M + tq], [P + tq], theta,
                                                 workspace=ws_dec)}[profile_phase]
        if profile_phase in ("prefill", "decode"):
            compose()
        if calibration_copy_mib:
            _calibration_copy(torch, dev, calibration_copy_mib)
        for _ in range(calls):
            fn()
        torch.cuda.synchronize()
        print(f"{profile_phase}: {calls} calls done", flush=True)
        return None

    extract(); compose(); prefill(); decode_loop()
    torch.cuda.synchronize()
    graph = capture(torch, decode_loop)

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
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    ph = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j in range(4)]
    del graph
    # decode over cache replicas (working set ~0.55 GB)
    reps = [(ck.clone(), cv.clone()) for _ in range(replicas)]
    gcold = capture(torch, lambda: [c2kv.attn_decode(qd[s], kd[s], vd[s], reps[s % replicas][0],
                                                     reps[s % replicas][1], [M + tq + s], [P + tq + s], theta,
                                                     workspace=ws_dec) for s in range(S)])
    cold_ms = time_replays(torch, gcold, 3)
    del gcold, reps
    free(torch)
    # compose over replicas of its inputs and caches (~3 GB)
    creps = []
    for _ in range(replicas):
        kk_r, v_r = kk.clone(), v.clone()
        vw = c2kv.slot_views(kk_r, v_r, lens, k)
        creps.append(([[vw[t] for t in order]], torch.empty_like(ck), torch.empty_like(cv), kk_r, v_r))
    gcc = capture(torch, lambda: [c2kv.compose(rq, k, theta, a, b) for rq, a, b, _, _ in creps])
    comp_cold_ms = time_replays(torch, gcc, 3) / replicas
    del gcc, creps
    free(torch)
    es = 2
    ext_flops = hq * 4 * d * sum(visible_cells(n, k) for n in lens)
    comp_bytes = 4 * M * hkv * d * es
    pre_flops = 4 * d * hq * tq * (M + (tq + 1) / 2)
    pre_bytes = (M + tq) * hkv * d * es * 2 + tq * (2 * hq + 2 * hkv) * d * es
    dec_bytes = sum(decode_call_bytes([M + tq + s], hq, hkv, d) for s in range(S))
    res = {"workload": "llama31_8b_1layer: extract 8 docs x 4096 tok (k=4, sink 4), compose 8192 slots "
                       "(32768 positions), prefill 64, 256 decode steps, batch 1",
           "steps": steps, "phase_ms": {"extract": ph[0], "compose": ph[1], "prefill": ph[2], "decode_256": ph[3]},
           "extraction_tflops": ext_flops / (ph[0] * 1e-3) / 1e12,
           "extraction_frac": ext_flops / (ph[0] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
           "compose_us_eager": ph[1] * 1e3, "compose_us_cold": comp_cold_ms * 1e3,
           "compose_gbs_cold": comp_bytes / (comp_cold_ms * 1e-3) / 1e9,
           "compose_hbm_frac_cold": comp_bytes / (comp_cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "prefill_us": ph[2] * 1e3, "prefill_tflops": pre_flops / (ph[2] * 1e-3) / 1e12,
           "prefill_gbs": pre_bytes / (ph[2] * 1e-3) / 1e9,
           "prefill_roofline_floor_us": max(pre_bytes / (HBM_PEAK_GBS * 1e9), pre_flops / (BF16_PEAK_TFLOPS * 1e12)) * 1e6,
           "decode_us_per_step_warm": ph[3] * 1e3 / S, "decode_us_per_step_cold": cold_ms * 1e3 / S,
           "decode_gbs_cold": dec_bytes / (cold_ms * 1e-3) / 1e9,
           "decode_hbm_frac_cold": dec_bytes / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "decode_gbs_warm_mall": dec_bytes / (ph[3] * 1e-3) / 1e9, "cache_replicas": replicas}
    del q, kk, v, o_ext, ck, cv, ws_ext, ws_pre, ws_dec
    free(torch)
    if emit:
        print(json.dumps(res), flush=True)
    return res


def _calibration_copy(torch, dev, mib):
    src = torch.ones(mib * 262144, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def profile_phase(a):
    """One phase alone for counter runs (FETCH_SIZE / WRITE_SIZE, SQ)."""
    torch, dev = _torch()
    import compressed_composable_kv_amd as c2kv
    import workloads as W
    if a.profile_phase in ("extract", "compose", "prefill", "decode"):
        llama_layer_step(torch, dev, 1, 0, profile_phase=a.profile_phase, calls=a.calls,
                         calibration_copy_mib=a.calibration_copy_mib)
        return
    if a.profile_phase == "decode128k":
        w = W.LONGCTX
        d, hq, hkv, theta, dt = w.head_dim, w.hq, w.hkv, w.rope_theta, w.dtype
        R, M, L = w.num_reqs, 32 * 1024, 32 * 4096
        ck = fill_normal(torch, (R, hkv, M + 8, d), dt, 7, dev)
        cv = fill_normal(torch, (R, hkv, M + 8, d), dt, 8, dev)
        q = fill_normal(torch, (R, hq, d), dt, 9, dev)
        kn = fill_normal(torch, (R, hkv, d), dt, 10, dev)
        ws = torch.empty(c2kv.workspace_size_decode([M] * R, hq, hkv, d, dt), dtype=torch.uint8, device=dev)
        fn = lambda: c2kv.attn_decode(q, kn, kn, ck, cv, [M] * R, [L] * R, theta, workspace=ws)  # noqa: E731
    elif a.profile_phase == "compose_qwen25":
        w = W.QWEN25
        d, hkv, dt, k = w.head_dim, w.hkv, w.dtype, w.ratio_k
        pool, reqs = W.qwen25_pool(w), W.qwen25_requests(w)
        slots = [c2kv.num_slots(n, k) for n in pool]
        kv = [(fill_normal(torch, (m, hkv, d), dt, 11 + 2 * t, dev), fill_normal(torch, (m, hkv, d), dt, 12 + 2 * t, dev))
              for t, m in enumerate(slots)]
        requests = [[(kv[t][0], kv[t][1], pool[t]) for t in r] for r in reqs]
        Mx = max(sum(slots[t] for t in r) for r in reqs)
        ck = torch.empty((len(reqs), hkv, Mx, d), dtype=dt, device=dev)
        cv = torch.empty_like(ck)
        fn = lambda: c2kv.compose(requests, k, w.rope_theta, ck, cv)  # noqa: E731
    else:   # extract_qwen3
        w = W.QWEN3_14B
        d, hq, hkv, dt, k = w.head_dim, w.hq, w.hkv, w.dtype, 4
        lens = list(w.doc_lens)
        rows = c2kv.packed_rows(lens, k)
        q = fill_normal(torch, (rows, hq, d), dt, 13, dev)
        kk = fill_normal(torch, (rows, hkv, d), dt, 14, dev)
        v = fill_normal(torch, (rows, hkv, d), dt, 15, dev)
        o = torch.empty_like(q)
        ws = torch.empty(c2kv.workspace_size_extract(lens, k, hkv, d, dt), dtype=torch.uint8, device=dev)
        fn = lambda: c2kv.extract_attn(q, kk, v, lens, k, k, w.rope_theta, out=o, workspace=ws)  # noqa: E731
    if a.calibration_copy_mib:
        _calibration_copy(torch, dev, a.calibration_copy_mib)
    for _ in range(a.calls):
        fn()
    torch.cuda.synchronize()
    print(f"{a.profile_phase}: {a.calls} calls done", flush=True)


# --------------------------------------------------------------- CPU baseline

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(nsteps=16):
    """The oracle, as it stands, on a bounded sample of the benchmark's
    workloads, on the host cores: `nsteps` decode steps of one request and
    one layer of the 128k long-context workload (32 768 composed slots,
    32/8 heads, d = 128), and the extraction of one 8192-token Qwen3-14B
    document at k = 4 for one KV-head group (5 query heads) of one layer."""
    import numpy as np
    import oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = None
    w = W.LONGCTX
    d, hq, hkv = w.head_dim, w.hq, w.hkv
    M = 32 * 1024
    ck = W.normal((M, hkv, d), w.dtype, 90, W.P_K).float().numpy()
    cv = W.normal((M, hkv, d), w.dtype, 90, W.P_V).float().numpy()
    t0 = time.perf_counter()
    nbytes = 0
    for s in range(nsteps):
        q = W.normal((hq, d), w.dtype, 90, W.P_DEC_Q, salt=s).float().numpy()
        kn = W.normal((hkv, d), w.dtype, 90, W.P_NEW_KV, salt=s).float().numpy()
        vn = W.normal((hkv, d), w.dtype, 90, W.P_NEW_KV, salt=1000 + s).float().numpy()
        _, _, ck, cv = O.decode_step(q, kn, vn, ck, cv, 131072 + s, w.rope_theta, "bf16")
        nbytes += decode_call_bytes([ck.shape[0] - 1], hq, hkv, d)
    dec_s = time.perf_counter() - t0
    w5 = W.QWEN3_14B
    n, k, G = 8192, 4, w5.hq // w5.hkv
    rows = n + O.num_slots(n, k)
    q = W.normal((rows, G, d), w5.dtype, 91, W.P_Q).float().numpy()
    kk = W.normal((rows, 1, d), w5.dtype, 91, W.P_K).float().numpy()
    v = W.normal((rows, 1, d), w5.dtype, 91, W.P_V).float().numpy()
    t0 = time.perf_counter()
    O.extract_attn(q, kk, v, [n], k, k, w5.rope_theta)
    ext_s = time.perf_counter() - t0
    ext_flops = G * 4 * d * visible_cells(n, k)
    return {
        "value": nbytes / dec_s / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"{nsteps} decode steps of 1 request x 1 layer over the 128k long-context cache ({M} composed "
                  f"slots, 32/8 heads, d=128), plus extraction of one 8192-token Qwen3-14B document at k=4 for "
                  f"one KV-head group (5 query heads)",
        "decode_seconds": dec_s, "extraction_tflops": ext_flops / ext_s / 1e12, "extraction_seconds": ext_s,
        "host_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
        "threads_note": "cores = BLAS threads numpy used (threadpoolctl)"}


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


def main():
    a = parse()
    if a.summarize:
        summarize(a.summarize, a.out, a.cmd, a.calibration_copy_mib)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (this path does not shard "
              f"across GPUs).", file=sys.stderr)
        sys.exit(2)
    if a.profile_phase:
        profile_phase(a)
        return
    if a.host_pool:
        host_pool()
        return
    if a.layer:
        layer_bench()
        return
    torch, dev = _torch()
    if a.decode_sweep:
        longctx_sweep(torch, dev, emit=True)
        qwen25(torch, dev, emit=True)
        return
    if a.extract_sweep:
        for k in (4, 8, 16):
            qwen3_extract(torch, dev, k, emit=True)
        return
    if a.compose_sweep:
        qwen25(torch, dev, emit=True)
        return
    if a.only:
        if a.only == "headline":
            longctx_decode(torch, dev, 32, False, a.steps, a.warmup, emit=True)
        elif a.only == "longctx":
            longctx_sweep(torch, dev, emit=True)
        elif a.only == "extract":
            qwen3_extract(torch, dev, 4, emit=True)
        elif a.only == "qwen25":
            qwen25(torch, dev, emit=True)
        else:
            llama_layer_step(torch, dev, a.steps, a.warmup, emit=True)
        return

    t_all = time.time()
    ach = achievable_peaks(torch, dev)
    log(f"achievable: {json.dumps(ach)}")
    # headline: 32-layer decode at 128k original tokens, 64 requests (timed K steps)
    head = longctx_decode(torch, dev, 32, False, a.steps, a.warmup)
    log(f"headline: {head['ms_per_step']:.3f} ms/step, {head['gbs']:.0f} GB/s")
    sweep = longctx_sweep(torch, dev, headline=head)
    ext = {}
    for k in (4, 8, 16):
        ext[k] = qwen3_extract(torch, dev, k)
        log(f"qwen3-14b extraction k={k}: {ext[k]['seconds_40_layers']:.3f} s / 40 layers, {ext[k]['tflops']:.0f} TFLOP/s")
    q25 = qwen25(torch, dev)
    log(f"qwen2.5 pool: decode {q25['decode_us_per_step']:.1f} us/step {q25['decode_gbs']:.0f} GB/s, compose "
        f"{q25['compose_us_per_call']:.1f} us")
    lla = llama_layer_step(torch, dev, steps=5, warmup=2)
    log(f"llama layer: {json.dumps(lla['phase_ms'])}")

    # at this size every (request, KV head) is one key piece: a decode call is
    # one decode_attn_kernel launch, with no merge launch
    dec_traffic = committed_traffic(("decode_attn_kernel",))
    roof = {"bound": "hbm", "kernel": "c2kv_attn_decode: decode_attn_kernel<bf16,128> (one key piece per request and "
                                      "KV head at this size, so no merge launch)",
            "achieved": head["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": head["gbs"] / HBM_PEAK_GBS,
            "traffic": dec_traffic, "per_launch_ms": head["ms_per_call"],
            "algorithmic_per_launch": head["bytes_per_step"] / head["layers"],
            "frac_of_achievable_read": _frac(head["gbs"], ach["hbm_read_gbs"]),
            "workload": "one decode call: 64 requests x 32768 composed slots (128k original tokens), 8 KV heads"}
    e4 = ext[4]
    ext_roof = {"bound": "mfma", "kernel": "extract_attn_kernel<bf16,128,XAttn32<128>> (+ rotate_k_kernel, rope_table_kernel)",
                "achieved": e4["tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": e4["frac_of_peak"],
                "traffic": None, "per_launch_ms": e4["ms_per_call"], "algorithmic_per_launch": e4["flop_per_call"],
                "frac_of_achievable_mfma": _frac(e4["tflops"], ach["mfma_bf16_tflops"]),
                "frac_of_achievable_mfma_data": _frac(e4["tflops"], ach["mfma_bf16_data_tflops"]),
                "workload": "one layer call: 64 documents x 8192 tokens at k=4, 40/8 heads"}
    line = {
        "metric": "C2KV decode-attn KV GB/s (% HBM peak) + extraction masked-attn TFLOP/s",
        "value": head["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) Q/K/V of the workloads' shapes, resident in HBM",
        "config": {"workload": "llama31_8b_longctx_128k_decode: Llama3.1-8B shapes (32/8 heads, d=128, theta 5e5), "
                               "32 attention-only layers, 64 requests, composed context of 32 documents x 4096 "
                               "tokens at k=4 (32768 slots, 131072 original tokens); one step = one decode call per "
                               "layer; extraction measured on qwen3_14b_extract (64 docs x 8192 tokens, k=4/8/16, "
                               "40 layers)",
                   "hq": 32, "hkv": 8, "head_dim": 128, "rope_theta": 500000.0, "requests": 64, "layers": 32,
                   "layer_buffers": head["layer_buffers"], "decode_graph": True},
        "hbm_frac": head["gbs"] / HBM_PEAK_GBS,
        "extraction_tflops": e4["tflops"],
        "extraction_frac": e4["frac_of_peak"],
        "roofline": roof,
        "extraction_roofline": ext_roof,
        "longctx_sweep": sweep,
        "extraction": [ext[k] for k in (4, 8, 16)],
        "qwen25": q25,
        "llama_layer": lla,
        "achievable": ach,
    }
    if not a.no_extras:
        hp = host_pool(emit=False)
        line["host_pool_load"] = {k_: hp[k_] for k_ in (
            "c2kv_zero_copy_ms", "c2kv_staged_ms", "full_dma_copy_ms", "full_zero_copy_k1_ms", "c2kv_zero_copy_gbs",
            "h2d_copy_gbs", "c2kv_zero_copy_frac_of_pcie_peak", "speedup_c2kv_best_vs_full_best")}
        line["host_pool_load"]["workload"] = "32 layers of the Llama shapes, 8 x 4096-token documents, k=4, from pinned host memory"
        ly = layer_bench(ach=ach, emit=False)
        line["extractor_layer"] = {k_: ly[k_] for k_ in ("ms", "tflops", "frac_of_peak", "frac_of_achievable")}
        line["extractor_layer"]["workload"] = "one Llama3.1-8B-shaped extractor layer over 8 x 4096 tokens (synthetic weights)"
    line["gpu_sections_wall_s"] = time.time() - t_all
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(8)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
