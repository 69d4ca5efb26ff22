"""The benchmark's accounting, on the CPU: the bytes each kernel must move
(against an independent walk over the tree's geometry), the decode floor,
the scaling of HBM byte counters, the source digest that guards them, and
the kernel-trace summary's grouping of launches by the cache state before
them."""
from __future__ import annotations

import json

import numpy as np
import sqlite3

import pytest

import bench
import workloads

LARGE = ["alhr_1k", "gqa_32k", "gqa_256k", "long_1m", "deep_planted"]


def _walk_counts(w):
    """Candidates a query scores, by simulating the walk's sets: the levels
    that keep every node are skipped, the first level that cuts scores all of
    its nodes, each later one the children of the beam it kept."""
    b, W = w.branching, w.beam
    kept, scored = 1, 0  # the implicit root
    for l in range(1, w.levels + 1):
        cand = kept * b
        if cand > W:
            scored += cand
        kept = min(cand, W)
    return scored


@pytest.mark.parametrize("name", LARGE)
def test_algorithmic_bytes_match_the_geometry(name):
    w = workloads.get(name)
    by = bench.algorithmic_bytes(w)
    heads = w.batch * w.kv_heads
    nodes = 0
    n = 1
    for _ in range(w.levels):
        n *= w.branching
        nodes += n
    s, d = w.elem_bytes, w.head_dim
    assert w.branching ** w.levels * w.leaf_block == w.n_keys  # the leaves are the last level
    assert by["build"] == heads * (w.n_keys * d * s + nodes * 4 * d)
    # a level that keeps everything is not scored by the kernels, but it is
    # counted: the pages' cost is the descent, every level a candidate read
    cand = by["candidates_per_query"]
    assert cand >= _walk_counts(w)
    first = bench.first_cut(w)
    unscored = sum(w.branching ** l for l in range(1, first))
    assert cand == _walk_counts(w) + unscored
    assert by["route"] == w.queries * (cand * 4 * d + d * s + 4 * w.beam)
    assert by["attend"] == w.queries * (w.beam * w.leaf_block * d * s * 2 + d * s
                                        + 4 * w.beam + 4 * d)


def test_headline_bytes_as_quoted():
    by = bench.algorithmic_bytes(workloads.get("gqa_32k"))
    assert by["build"] == 278_003_712
    assert by["route"] == 8_949_760 and by["attend"] == 33_656_832
    assert by["candidates_per_query"] == 136


def test_summary_row_widths():
    w = workloads.get("gqa_32k")
    f32, bf16, fp8 = (bench.algorithmic_bytes(w, sd) for sd in ("f32", "bf16", "fp8"))
    heads, nodes = w.batch * w.kv_heads, 8 + 64 + 512
    assert f32["build"] - bf16["build"] == heads * nodes * 2 * w.head_dim
    assert f32["build"] - fp8["build"] == heads * nodes * (3 * w.head_dim - 4)


def test_first_cut_and_floor():
    for name, l0 in (("alhr_1k", 2), ("gqa_32k", 2), ("long_1m", 2), ("deep_planted", 2)):
        assert bench.first_cut(workloads.get(name)) == l0
    w = workloads.get("long_1m")
    # 4 scored levels (2..5), then the leaf blocks: 5 dependent round trips
    f = bench.decode_floor(w, 5000.0, 0.5, 10_000_000)
    assert f == pytest.approx(5 * 0.5 + 10_000_000 / (5000.0 * 1e3))


def _counter_csv(path, counter, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name",
            "Counter_Value"]
    with open(path, "w") as f:
        f.write(",".join(cols) + "\n")
        for i, (name, value) in enumerate(rows):
            f.write(f'{i},"{name}",1024,256,"{counter}",{value}\n')


def test_traffic_from_counters_scales_by_the_reference_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic_{}.json"))
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # the copy reads and writes 256 MiB; this counter reads half of the reads
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 131072.0),
                                       ("void tis::k_build<bf16_bits, float, 128, false>(x)", 100.0),
                                       ("void tis::k_build<bf16_bits, float, 128, false>(x)", 300.0),
                                       ("void tis::k_decode<...>(x)", 9999.0)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 262144.0),
                                       ("void tis::k_build<bf16_bits, float, 128, false>(x)", 50.0),
                                       ("void tis::k_build<bf16_bits, float, 128, false>(x)", 50.0)])
    out = bench.traffic_from_counters("w", str(fetch), str(write))
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    assert out["build_bytes_per_launch"] == pytest.approx((200.0 * 2 + 50.0) * 1024)
    saved = json.load(open(tmp_path / "traffic_w.json"))
    assert saved["build_source_sha256_16"] == bench._source_digest()
    # the stored figure is used only while the build's code is unchanged
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic_{}.json"))
    assert bench.load_traffic("w") == pytest.approx(out["build_bytes_per_launch"])
    saved["build_source_sha256_16"] = "0" * 16
    json.dump(saved, open(tmp_path / "traffic_w.json", "w"))
    assert bench.load_traffic("w") is None
    assert bench.load_traffic("absent") is None


def test_source_digest_ignores_comments_and_spacing(tmp_path, monkeypatch):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // add one\n}\n")
    b.write_text("// header\nint f(int x) { return x + 1; }\n\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    digests = []
    for p in (a, b, c):
        monkeypatch.setattr(bench, "BUILD_SOURCE", str(p))
        digests.append(bench._source_digest())
    assert digests[0] == digests[1] != digests[2]


def _trace_db(path):
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, start integer, end integer, grid_x integer, "
                "workgroup_x integer, queue_id integer)")
    t = [0]

    def k(name, us, wgs, threads=256, q=1):
        con.execute("insert into kernels values (?,?,?,?,?,?)",
                    (name, t[0], t[0] + int(us * 1000), wgs * threads, threads, q))
        t[0] += int(us * 1000) + 500
    flush = "void tis::(anonymous namespace)::k_probe_read<false>(uint4 const*, unsigned long, unsigned int*)"
    build = "void tis::(anonymous namespace)::k_build<bf16_bits, float, 128, false>(tis::BuildArgs)"
    dec = "void tis::(anonymous namespace)::k_decode<bf16_bits, float, 128, false>(tis::RouteArgs, tis::AttendArgs)"
    k(flush, 4.0, 64)          # marker of workload 0
    for _ in range(3):
        k(flush, 190.0, 16384)  # 1 GiB flush
        k(build, 50.0, 256, 512)
    k(flush, 190.0, 16384)
    k(dec, 15.0, 128, 1024)
    k(dec, 11.0, 128, 1024)     # back to back
    k(flush, 4.0, 128)         # marker of workload 1
    k(flush, 190.0, 16384)
    k(flush, 5.0, 584)         # the summaries read (steady)
    k(dec, 18.0, 128, 1024)
    con.commit()
    con.close()


def test_trace_summary_groups_by_cache_state(tmp_path):
    db = tmp_path / "t.db"
    _trace_db(db)
    out = tmp_path / "k_{workload}.md"
    bench.trace_summary(str(db), str(out), "T", "cmd", "first,second")
    first = (tmp_path / "k_first.md").read_text()
    second = (tmp_path / "k_second.md").read_text()
    rows = [ln for ln in first.splitlines() if ln.startswith("| first")]
    build = [ln for ln in rows if "`k_build" in ln]
    assert len(build) == 1 and "| probe read of 1 GiB (cold) | 3 | 50.00 |" in build[0]
    dec = [ln for ln in rows if "`k_decode" in ln]
    assert any("probe read of 1 GiB (cold) | 1 | 15.00" in ln for ln in dec)
    assert any("same kernel | 1 | 11.00" in ln for ln in dec)
    rows2 = [ln for ln in second.splitlines() if ln.startswith("| second")]
    assert any("`k_decode" in ln and "probe read of the summaries | 1 | 18.00" in ln for ln in rows2)
    assert not any("`k_build" in ln for ln in rows2)
    assert "cmd" in first and first.startswith("# T: first")


def test_counters_summary_means_per_kernel(tmp_path):
    csv_path = tmp_path / "c.csv"
    grp = "void tis::(anonymous namespace)::k_attend_group<bf16_bits, 128, 1>(tis::AttendArgs)"
    att = "void tis::(anonymous namespace)::k_attend<bf16_bits, 128>(tis::AttendArgs)"
    rows = ["Dispatch_Id,Kernel_Name,Grid_Size,Workgroup_Size,Counter_Name,Counter_Value"]
    for i, (name, util) in enumerate([(grp, 1.5), (grp, 2.5), (att, 0.0)]):
        rows.append(f'{i},"{name}",65536,512,MfmaUtil,{util}')
        rows.append(f'{i},"{name}",65536,512,SQ_INSTS_VALU,{1000 * (i + 1)}')
    rows.append('9,"at::native::fill",1,1,MfmaUtil,7')
    csv_path.write_text("\n".join(rows) + "\n")
    out = tmp_path / "c.md"
    bench.counters_summary(str(csv_path), str(out), "T", "cmd", "k_attend")
    text = out.read_text()
    lines = [ln for ln in text.splitlines() if ln.startswith("| `")]
    assert len(lines) == 2 and not any("fill" in ln for ln in lines)
    g = [ln for ln in lines if "k_attend_group" in ln][0]
    assert "| 65536 x 512 | 2 | 2 | 1500 |" in g      # means over the two dispatches
    assert "| MfmaUtil | SQ_INSTS_VALU |" in text and text.startswith("# T")


def test_timeline_phases_from_stamps():
    """The decode timeline summary: times from the launch's first entry, the
    level phases over the 8 walking waves only, unpassed phases left out."""
    st = np.zeros((2, 16, 24), dtype=np.int64)
    st[:, :, 0] = 1000
    st[0, 0, 0] = 900                      # the launch's first entry
    st[:, :8, 8] = 1100                    # level 1 scored by the walking waves
    st[:, 8:, 8] = 5000                    # the other waves' stamps are not counted
    st[:, :8, 9] = 1200
    st[:, :, 1] = 1300
    st[:, :, 7] = 2000
    st[1, 3, 7] = 2500
    ph = bench.timeline_phases(st, 100_000, 1)  # 100 MHz: 100 ticks a microsecond
    assert ph["entry"]["median_us"] == pytest.approx(1.0)
    assert ph["level 1 scored"] == {"median_us": pytest.approx(2.0), "max_us": pytest.approx(2.0)}
    assert ph["level 1 ranked"]["max_us"] == pytest.approx(3.0)
    assert ph["descent done"]["median_us"] == pytest.approx(4.0)
    assert ph["end"]["max_us"] == pytest.approx(16.0)
    assert "K arrived" not in ph and "level 2 scored" not in ph
