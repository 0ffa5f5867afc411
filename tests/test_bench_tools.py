"""Host logic of bench.py on the CPU: the algorithmic byte count, the
rocprofv3 trace and counter summaries (on small synthetic CSV files in the
profiler's column layout), the dispatch selection, the report generator,
and that the committed profile records belong to the current kernel
sources."""
import csv
import json
import pathlib
import re
import types

import pytest

import bench

ROOT = pathlib.Path(__file__).resolve().parents[1]


def tiny_workload(ranks=(32, 64), name="tiny"):
    return types.SimpleNamespace(name=name, layers=len(ranks), ranks=list(ranks), batch=2,
                                 num_q_heads=8, num_kv_heads=2, head_dim=128, num_beacons=64,
                                 raw_window=32, elem_bytes=2)


def test_layer_bytes_match_the_rank64_layer():
    # bytes are linear in the rank and the c3 step's ranks average 64, so the
    # mean over its layers is the bytes of one rank-64 layer: 128 units x
    # (8192 x 2 x 64 + 2 x 2048 x 128) x 2 bytes of cache, plus the bases
    # (8 x 128 x 2 x 64 x 2), q (16 x 32 x 128 x 2) and out + lse (16 x 32 x
    # 129 x 4) -- 403.3 MB per launch
    import synth
    wl = synth.get_workload("c3")
    assert sum(wl.ranks) == 64 * wl.layers
    mean = sum(bench.layer_call_bytes(wl, i, 2)[1] for i in range(wl.layers)) / wl.layers
    cache = 128 * (8192 * 2 * 64 + 2 * 2048 * 128) * 2
    assert mean == cache + 8 * 128 * 2 * 64 * 2 + 16 * 32 * 128 * 2 + 16 * 32 * 129 * 4
    assert mean == 403_310_592
    # and the cache part alone
    c0, t0 = bench.layer_call_bytes(wl, 0, 2)
    assert c0 < t0


def test_kernel_name():
    assert (bench.kernel_name("void slimkv::attention_kernel<4, 2, true, false>(slimkv::AttnArgs)")
            == "slimkv::attention_kernel<4, 2, true, false>")
    anon = "void at::native::(anonymous namespace)::fill_kernel<float>(int, float)"
    assert bench.kernel_name(anon) == "at::native::(anonymous namespace)::fill_kernel<float>"
    assert bench.kernel_name("slimkv_bench_stream_read_kernel(int)") == "slimkv_bench_stream_read_kernel"


def test_pct():
    med, p10, p90 = bench.pct([float(x) for x in range(1, 12)])
    assert (med, p10, p90) == (6.0, 2.0, 10.0)


def test_headline_dispatches_picks_the_timed_steps():
    wl = tiny_workload()
    steps, warm, other_warm = 3, 7, 5
    seq = []
    for phase, count in (("warm", warm), ("timed", steps), ("owarm", other_warm), ("otimed", steps)):
        for s in range(count):
            seq += [(phase, s, layer) for layer in range(wl.layers)]
    got = bench.headline_dispatches(seq, wl, steps, other_warm)
    assert got == [("timed", s, layer) for s in range(steps) for layer in range(wl.layers)]
    with pytest.raises(SystemExit):
        bench.headline_dispatches(seq[-10:], wl, steps, other_warm)


TRACE_FIELDS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
                "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp"]


def write_trace(path, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=TRACE_FIELDS, quoting=csv.QUOTE_NONNUMERIC)
        w.writeheader()
        for i, (name, start, end) in enumerate(rows):
            w.writerow({"Kind": "KERNEL_DISPATCH", "Agent_Id": "Agent 1", "Queue_Id": 1, "Stream_Id": 0,
                        "Thread_Id": 1, "Dispatch_Id": i + 1, "Kernel_Id": 1, "Kernel_Name": name,
                        "Correlation_Id": i + 1, "Start_Timestamp": start, "End_Timestamp": end})


def test_profile_summary_on_a_synthetic_trace(tmp_path):
    wl = tiny_workload()
    names = ["void slimkv::attention_kernel<4, 1, true, false>(slimkv::AttnArgs)",
             "void slimkv::attention_kernel<4, 2, true, false>(slimkv::AttnArgs)"]
    steps, other_warm = 2, 3
    rows, t = [("void fill_kernel(int)", 0, 1000)], 10_000
    timed = []
    # warm-up (4 steps), timed (2 steps), the other form's warm-up and timed
    for phase, count in (("warm", 4), ("timed", steps), ("owarm", other_warm), ("otimed", steps)):
        for s in range(count):
            for layer in range(wl.layers):
                dur = 50_000 + 10_000 * layer + (1000 * s if phase == "timed" else 7_000)  # ns
                rows.append((names[layer], t, t + dur))
                if phase == "timed":
                    timed.append((layer, dur / 1e3))
                t += dur + 500
    write_trace(tmp_path / "run" / "x_kernel_trace.csv", rows)
    summ = bench.profile_summary(str(tmp_path), wl, steps, other_warm)
    assert summ["dispatches"] == steps * wl.layers
    assert summ["launch_us"] == pytest.approx(sum(d for _, d in timed) / len(timed))
    by_layer = {layer: [d for lay, d in timed if lay == layer] for layer in range(wl.layers)}
    assert summ["per_rank"]["32"]["avg_us"] == pytest.approx(sum(by_layer[0]) / steps, abs=0.01)
    assert summ["per_rank"]["64"]["kernel"] == "slimkv::attention_kernel<4, 2, true, false>"
    assert summ["kernel_sum_per_step_us"] == pytest.approx(sum(d for _, d in timed) / steps, abs=0.1)
    assert summ["other_kernels"] == {"fill_kernel": {"calls": 1, "sum_us": 1.0}}
    mean_bytes = (bench.layer_call_bytes(wl, 0, 2)[1] + bench.layer_call_bytes(wl, 1, 2)[1]) / 2
    assert summ["gbps"] == pytest.approx(mean_bytes / (summ["launch_us"] * 1e-6) / 1e9, abs=0.051)  # 0.1 GB/s steps


COUNTER_FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
                  "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
                  "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
                  "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_counters(path, counter, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=COUNTER_FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i + 1, "Dispatch_Id": i + 1, "Agent_Id": "Agent 1",
                        "Queue_Id": 1, "Process_Id": 1, "Thread_Id": 1, "Grid_Size": 256, "Kernel_Id": 1,
                        "Kernel_Name": name, "Workgroup_Size": 256, "LDS_Block_Size": 0, "Scratch_Size": 0,
                        "VGPR_Count": 8, "Accum_VGPR_Count": 0, "SGPR_Count": 16, "Counter_Name": counter,
                        "Counter_Value": value, "Start_Timestamp": 0, "End_Timestamp": 1})


def test_traffic_summary_on_synthetic_counters(tmp_path):
    wl = tiny_workload()
    steps = 1
    gib_kib = (1 << 30) / 1024
    # calibration: the read kernel's FETCH_SIZE is half its bytes, the write
    # kernel's WRITE_SIZE all of them (scales 2 and 1)
    write_counters(tmp_path / "cf" / "c_counter_collection.csv", "FETCH_SIZE",
                   [("void slimkv::stream_read_kernel(int)", ((1 << 30) - 16) / 1024 / 2)] * 3
                   + [("void copy_kernel(int)", gib_kib)])
    write_counters(tmp_path / "cw" / "c_counter_collection.csv", "WRITE_SIZE",
                   [("void slimkv::flush_kernel(int)", gib_kib)] * 3)
    att = "void slimkv::attention_kernel<4, 1, true, false>(slimkv::AttnArgs)"
    # one headline step, the other form's 2 warm-up steps and 1 timed step
    fetch = [(att, 100.0 + i) for i in range(wl.layers * 4)]
    write = [(att, 10.0) for _ in range(wl.layers * 4)]
    write_counters(tmp_path / "f" / "x_counter_collection.csv", "FETCH_SIZE", fetch)
    write_counters(tmp_path / "w" / "x_counter_collection.csv", "WRITE_SIZE", write)
    rs, ws_, copy = bench.calibration_scales(str(tmp_path / "cf"), str(tmp_path / "cw"))
    assert rs == pytest.approx(2.0) and ws_ == pytest.approx(1.0) and copy == pytest.approx(gib_kib)
    summ = bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                                 str(tmp_path / "cw"), wl, steps, (2, 2))
    # the headline step's dispatches are the first two (fetch 100, 101 KiB)
    read = (100.0 + 101.0) / 2 * 1024 * 2.0
    assert summ["read_bytes_per_launch"] == int(read)
    assert summ["write_bytes_per_launch"] == int(10.0 * 1024)
    assert summ["traffic_bytes_per_launch"] == int(read + 10.0 * 1024)


def test_report_regenerates_from_its_source_line(tmp_path):
    text = (ROOT / "REPORT.md").read_text()
    m = re.search(r"```json\n(\{.*\})\n```", text)
    assert m, "REPORT.md holds its bench line"
    line = json.loads(m.group(1))
    src = tmp_path / "line.json"
    src.write_text(json.dumps(line) + "\n")
    body = bench.report([str(src)])
    rows = [ln for ln in body.splitlines() if ln.startswith("| ") and "Source" not in ln]
    assert len(rows) > 20
    for ln in rows:
        assert ln in text, ln
    assert line["parity"]["pass"] is True
    assert line["roofline"]["frac"] == pytest.approx(line["roofline"]["achieved"] / line["roofline"]["peak"],
                                                     abs=1e-4)


def test_committed_profiles_match_the_kernel_sources():
    sha = bench.source_sha256()
    recs = sorted((ROOT / "profiles").glob("*.json"))
    assert recs
    for p in recs:
        rec = json.loads(p.read_text())
        assert rec["source_sha256"] == sha, f"{p.name} was taken on other kernel sources"
        md = p.with_suffix(".md")
        assert md.exists() and sha in md.read_text()


def test_even_lengths_keep_the_drawn_means():
    """The even-lengths serving line: every sequence gets the drawn lengths'
    rounded means, so the live rows (and bytes) match the drawn step's to
    within rounding and the pieces of the schedule all carry the same tiles."""
    import synth

    wl = synth.get_workload("c3")
    stand_in = types.SimpleNamespace(num_beacons=wl.num_beacons, raw_window=wl.raw_window, layer=0)
    first = synth.make_step(wl, stand_in, beacons=(0.5, 1.0), raw=(0.5, 1.0))
    even = bench.even_lengths(synth, wl, stand_in, "cpu", first)
    nb, rw = first.num_beacons.numpy(), first.raw_len.numpy()
    assert len(set(even.num_beacons.tolist())) == 1 and len(set(even.raw_len.tolist())) == 1
    assert abs(int(even.num_beacons.sum()) - int(nb.sum())) <= wl.batch // 2
    assert abs(int(even.raw_len.sum()) - int(rw.sum())) <= wl.batch // 2
    assert nb.min() < nb.max()  # the drawn lengths are ragged
