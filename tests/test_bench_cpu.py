"""CPU checks of the benchmark's own arithmetic and bookkeeping: the
algorithmic FLOP and byte counts that its roofline figures divide by (pinned
to the oracle's mask and byte definitions), and the summaries of rocprofv3
databases that the committed profiles are made from."""
import json
import sqlite3

import pytest

import bench
import oracle as O


# ------------------------------------------------------- algorithmic work

@pytest.mark.parametrize("n,k", [(12, 4), (10, 4), (37, 8), (3, 4), (1, 4), (4, 4), (64, 4), (40, 4),
                                 (513, 8), (1000, 16), (4096, 4)])
def test_visible_cells_equal_the_oracle_mask(n, k):
    """The extraction FLOP count uses visible cells with sink = k (as the
    benchmark's workloads run); it must equal the dense mask's count."""
    assert bench.visible_cells(n, k) == int(O.structured_mask(n, k, k).sum())
    assert bench.visible_cells(n, k) == sum(O.mask_cell_counts(n, k, k))


def test_extraction_flops_of_the_qwen3_workload():
    """4 d FLOPs per visible (query head, key) cell, summed over documents:
    the 1.870 PFLOP per 40 layers at k = 4 quoted for the Qwen3-14B shapes
    (40 query heads, d = 128, 64 documents of 8192 tokens)."""
    import workloads as W
    w = W.QWEN3_14B
    per_doc = sum(O.mask_cell_counts(8192, 4, 4))
    flops_call = w.hq * 4 * w.head_dim * sum(bench.visible_cells(n, 4) for n in w.doc_lens)
    assert flops_call == w.hq * 4 * w.head_dim * per_doc * len(w.doc_lens)
    assert abs(w.layers * flops_call / 1e15 - 1.870) < 0.001


def test_decode_call_bytes():
    """Every cache row (the appended one included) of K and V read once per
    request, plus q and o (Hq rows) and the new k and v (Hkv rows)."""
    lens, hq, hkv, d, es = [0, 1, 4095, 32768], 32, 8, 128, 2
    kv = sum(O.decode_kv_bytes(L + 1, hkv, d, es) for L in lens)
    io = len(lens) * (2 * hq + 2 * hkv) * d * es
    assert bench.decode_call_bytes(lens, hq, hkv, d, es) == kv + io


# ------------------------------------------------ profile summaries

def _trace_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, start integer, end integer)")
    con.executemany("insert into kernels values (?, ?, ?)", rows)
    con.commit()
    con.close()


def test_trace_summary_reports_avg_median_min_max(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    durs = [10_000, 20_000, 30_000, 1_000_000]          # ns
    rows = [("kernel_a", 0, t) for t in durs] + [("kernel_b", 0, 5_000)]
    _trace_db(str(d / "t_results.db"), rows)
    out = tmp_path / "s.txt"
    bench.summarize([str(d)], str(out), "the command", 0)
    lines = out.read_text().splitlines()
    assert lines[1] == "# command: the command"
    assert "median_us" in lines[2]
    a = next(l for l in lines if l.endswith("kernel_a")).split()
    # calls, avg, median, min, max (microseconds), total (ms)
    assert a[:6] == ["4", "265.00", "25.00", "10.00", "1000.00", "1.060"]


def _pmc_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, counter_name text, "
                "value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_counter_summary_scales_by_the_calibration_copy(tmp_path):
    """FETCH_SIZE and WRITE_SIZE are per-instance values summed per dispatch
    and averaged over dispatches; each is scaled by what it reads for a copy
    of known size (here FETCH_SIZE counts half the bytes, as on MI355X)."""
    mib = 8
    f, w = tmp_path / "f", tmp_path / "w"
    f.mkdir()
    w.mkdir()
    calib = bench.CALIB_KERNEL + "(int*)"
    _pmc_db(str(f / "f_results.db"), [
        (1, calib, "FETCH_SIZE", mib * 1024 / 4), (1, calib, "FETCH_SIZE", mib * 1024 / 4),   # two instances
        (2, "c2kv::k", "FETCH_SIZE", 600.0), (2, "c2kv::k", "FETCH_SIZE", 400.0),
        (3, "c2kv::k", "FETCH_SIZE", 1000.0)])
    _pmc_db(str(w / "w_results.db"), [
        (1, calib, "WRITE_SIZE", mib * 1024),
        (2, "c2kv::k", "WRITE_SIZE", 10.0), (3, "c2kv::k", "WRITE_SIZE", 30.0)])
    out = tmp_path / "p.txt"
    bench.summarize([str(f), str(w)], str(out), "cmd", mib)
    js = json.loads(next(l for l in out.read_text().splitlines() if l.startswith("# json: "))[len("# json: "):])
    assert js["fetch_scale"] == pytest.approx(2.0) and js["write_scale"] == pytest.approx(1.0)
    # per dispatch: fetch 1000 KiB, write 20 KiB on average
    assert js["traffic_bytes"]["c2kv::k"] == pytest.approx((1000 * 2.0 + 20 * 1.0) * 1024)
    assert js["sources_sha"] == bench.sources_sha(bench.DECODE_SOURCES)


def test_committed_traffic_needs_matching_sources(tmp_path):
    info = {"sources_sha": bench.sources_sha(bench.DECODE_SOURCES), "traffic_bytes": {"_Zdecode_attn_kernel_x": 5.0}}
    p = tmp_path / "ok.txt"
    p.write_text("# header\n# json: " + json.dumps(info) + "\n")
    assert bench.committed_traffic(("decode_attn_kernel",), str(p)) == 5.0
    info["sources_sha"] = "0" * 16
    p.write_text("# json: " + json.dumps(info) + "\n")
    assert bench.committed_traffic(("decode_attn_kernel",), str(p)) is None
    assert bench.committed_traffic(("decode_attn_kernel",), str(tmp_path / "missing.txt")) is None


def test_committed_profiles_match_the_current_sources():
    """The counter summaries in profiles/ were taken on the sources as they
    stand: the bench line's traffic figures are then not null."""
    assert bench.committed_traffic(("decode_attn_kernel",)) is not None
    assert bench.committed_traffic(("compose_kernel",), bench.COMPOSE_PMC_SUMMARY, bench.COMPOSE_SOURCES,
                                   "compose_sources_sha") is not None


def test_source_hash_ignores_comments_and_layout(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    b.write_text("/* note */ int f(int x) {   return x + 1;\n\n}  // other\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.sources_sha((str(a),)) == bench.sources_sha((str(b),))
    assert bench.sources_sha((str(a),)) != bench.sources_sha((str(c),))
