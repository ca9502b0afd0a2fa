"""bench.py's algorithmic byte accounting against the oracle's traffic model."""
import numpy as np
import pytest

import bench
from oracle import bytemodel as bm


@pytest.mark.parametrize("name", sorted(bench.WORKLOADS))
@pytest.mark.parametrize("L", [1, 4, 8, 16, 32])
@pytest.mark.parametrize("state", ["f32", "f16"])
def test_window_bytes_match_model(name, L, state):
    c = dict(bench.WORKLOADS[name])
    c["L"], c["state"] = L, state
    args = (c["form"], c["H"], c["dv"], c["dk"], c["B"], c["state"], c["rec"], c["io"])
    io = (2 * c["dk"] + c["dv"]) * 2 + 4 + (4 if c["form"] == 1 else 0) + 4 * c["dv"]
    ms = bm.state_bytes(c["dv"], c["dk"], 4 if state == "f32" else 2)
    rec = bm.record_bytes(c["dv"], c["dk"])   # fp16 x and k, fp32 decay
    per_row_meta = 9 * c["B"] * L
    got = bench.window_bytes(*args, L) - c["B"] * c["H"] * L * io - per_row_meta
    assert got == c["B"] * c["H"] * bm.replay_window_bytes(L, ms, rec)
    got_c = bench.window_bytes(*args, L, "conventional") - c["B"] * c["H"] * L * io - 4 * c["B"] * L
    assert got_c == c["B"] * c["H"] * bm.conventional_window_bytes(L, ms)


@pytest.mark.parametrize("L", [1, 2, 8, 16, 32])
@pytest.mark.parametrize("read", ["f16", "bf16", "e4m3"])
def test_two_copy_window_bytes_match_model(L, read):
    c = dict(bench.WORKLOADS["nemotron"])
    args = (c["form"], c["H"], c["dv"], c["dk"], c["B"], "f32", c["rec"], c["io"])
    io = (2 * c["dk"] + c["dv"]) * 2 + 4 + 4 * c["dv"]
    m_hi = bm.state_bytes(c["dv"], c["dk"], 4)
    # E4M3: one byte per element plus an fp32 scale per state row
    m_lo = bm.state_bytes(c["dv"], c["dk"], 1) + 4 * c["dv"] if read == "e4m3" else bm.state_bytes(c["dv"], c["dk"], 2)
    rec = bm.record_bytes(c["dv"], c["dk"])
    got = bench.window_bytes(*args, L, read=read) - c["B"] * c["H"] * L * io - 9 * c["B"] * L
    assert got == c["B"] * c["H"] * bm.two_copy_window_bytes(L, m_hi, m_lo, rec)
    # a read copy as wide as the recurrence copy costs one more write per window
    assert bm.two_copy_window_bytes(L, m_hi, m_hi, rec) == bm.replay_window_bytes(L, m_hi, rec) + m_hi


def test_headline_ratio():
    """The headline workload's algorithmic traffic ratio, inputs included: the
    state + record part is the blog's 0.581; q/k/v/out add a little."""
    c = bench.WORKLOADS["nemotron"]
    args = (c["form"], c["H"], c["dv"], c["dk"], c["B"], c["state"], c["rec"], c["io"], c["L"])
    r = bench.window_bytes(*args) / bench.window_bytes(*args, "conventional")
    assert 0.581 < r < 0.60


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("L", [1, 4, 16, 32])
def test_grouped_window_bytes_match_model(L):
    """Grouped keys (8 groups of 16 heads): the per-head share of a layer
    record is the blog's 18,944-byte released record over 128 heads; q and k
    inputs are read once per group."""
    c = dict(bench.WORKLOADS["nemotron-grouped"])
    H, G = c["H"], c["groups"]
    args = (c["form"], H, c["dv"], c["dk"], c["B"], c["state"], c["rec"], c["io"])
    io = (2 * c["dk"] / (H // G) + c["dv"]) * 2 + 4 + 4 * c["dv"]
    ms = bm.state_bytes(c["dv"], c["dk"], 4)
    rec = bm.grouped_record_bytes(H, c["dv"], c["dk"], G) / H
    got = bench.window_bytes(*args, L, groups=G) - c["B"] * H * L * io - 9 * c["B"] * L
    assert got == pytest.approx(c["B"] * H * bm.replay_window_bytes(L, ms, rec), rel=1e-12)
    conv = bench.window_bytes(*args, L, "conventional", groups=G) - c["B"] * H * L * io - 4 * c["B"] * L
    assert conv == pytest.approx(c["B"] * H * bm.conventional_window_bytes(L, ms), rel=1e-12)
    if L == 16:  # the blog's "about 0.55 of conventional traffic"
        assert abs(got / conv - 0.5503) < 5e-4


def _simulate(L, pools, warmup, steps, per_cursor):
    """Drive the host cursor rule (rs_meta_step / rs_meta_advance, what
    DecodeLayer calls) over the benchmark's schedule: pool preparation, W
    warm-up and K timed launches.  Returns the timed launches' cursors."""
    import numpy as np
    import linear_attention_decode_replay_amd as rs
    phi, starts = bench.cursor_schedule(L, pools, warmup, steps, per_cursor)
    anchors = [np.zeros(3, np.int32) for _ in range(pools)]   # three rows per pool, all in phase
    for p, n in enumerate(starts):
        for _ in range(n):
            _, fl = rs.rs_meta_step(L, anchors[p])
            rs.rs_meta_advance(L, anchors[p], fl)
    timed = []
    for s in range(warmup + steps):
        a = anchors[s % pools]
        wp, fl = rs.rs_meta_step(L, a)
        assert len(set(wp.tolist())) == 1 and int(wp[0]) == (s + phi) % L
        assert bool(fl[0]) == (int(wp[0]) == L - 1)
        rs.rs_meta_advance(L, a, fl)
        if s >= warmup:
            timed.append(int(wp[0]))
    return timed


@pytest.mark.parametrize("L,pools,warmup,steps", [
    (16, 17, 5, 20), (16, 17, 64, 64), (16, 17, 0, 64), (16, 33, 3, 50), (16, 17, 16, 1),
    (16, 17, 7, 15), (16, 17, 9, 8), (8, 9, 5, 20), (32, 33, 5, 20), (4, 5, 1, 9), (1, 1, 2, 3)])
def test_timed_cursor_mix(L, pools, warmup, steps):
    """The K timed launches are floor(K/L) whole windows plus one run of
    K mod L consecutive cursors, for any warm-up; whole windows exactly when
    L divides K; the run is the one whose mean algorithmic bytes are closest
    to the window average."""
    c = dict(bench.WORKLOADS["nemotron"], L=L)
    per = bench.cursor_bytes(c)
    timed = _simulate(L, pools, warmup, steps, per)
    counts = [timed.count(w) for w in range(L)]
    full, extra = divmod(steps, L)
    assert sorted(counts) == [full] * (L - extra) + [full + 1] * extra
    c0 = timed[0]
    assert c0 == bench.timed_phase(per, steps)
    assert all(timed[i] == (c0 + i) % L for i in range(steps))
    win = sum(per) / L
    got = sum(per[w] for w in timed) / steps
    for alt in range(L):   # no other start is closer to the window average
        m = sum(per[(alt + i) % L] for i in range(steps)) / steps
        assert abs(got - win) <= abs(m - win) * (1 + 1e-12)
    if extra == 0:
        assert c0 == 0 and got == pytest.approx(win, rel=1e-15)


def test_driver_schedule_is_near_the_window_average():
    """--steps 20 --warmup 5 at the headline shape: one flush among the 20
    timed launches, and their algorithmic bytes within 0.1 % of the window
    average (the flush-free 6/16 of a window that a plain rotation of
    in-phase pools would time is 9 % below it)."""
    c = dict(bench.WORKLOADS["nemotron"])
    per = bench.cursor_bytes(c)
    timed = _simulate(16, 17, 5, 20, per)
    assert timed.count(15) == 1
    win = sum(per) / 16
    assert abs(sum(per[w] for w in timed) / 20 / win - 1) < 1e-3
    assert sum(per[w] for w in range(1, 7)) / 6 / win < 0.92


def test_pool_count_must_be_one_mod_L():
    c = dict(bench.WORKLOADS["nemotron"])
    with pytest.raises(ValueError):
        bench.cursor_schedule(16, 4, 5, 20, bench.cursor_bytes(c))
    assert bench.main(["--pools", "4", "--steps", "20"]) == 2


def test_counter_lineup():
    """Counter dispatches are matched to logged launches per kernel, in order;
    the counters' KiB are scaled by the calibration copy."""
    rows = [(0, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)] * 3
    rows += [(1, "void rs::(anonymous namespace)::k_replay_step<0, 64>(rs::StepParams)", "FETCH_SIZE", 10.0),
             (2, "void rs::(anonymous namespace)::k_conventional_step<0>(rs::StepParams)", "FETCH_SIZE", 7.0),
             (3, "void rs::(anonymous namespace)::k_replay_step<0, 64, true>(rs::StepParams)", "FETCH_SIZE", 12.0)]
    scale = bench.counter_scale(rows, 1, "fetch")
    assert scale == 2.0
    got = bench.line_up(rows, [("k_replay_step", "w0", 20480.0), ("k_conventional_step", "conventional", 1.0),
                               ("k_replay_step", "flush", 24576.0)], scale)
    assert got[("k_replay_step", "w0")] == [(20480.0, 20480.0)]
    assert got[("k_replay_step", "flush")] == [(24576.0, 24576.0)]
    assert got[("k_conventional_step", "conventional")] == [(14336.0, 1.0)]
    with pytest.raises(SystemExit):
        bench.line_up(rows, [("k_replay_step", "w0", 1.0)], scale)


def test_suite_counters_are_stored(tmp_path, monkeypatch, capsys):
    """A suite run's counters (speculative verify, layer stack) are stored in
    counters.json under the suite's key, one entry per (kernel, case)."""
    import csv
    import json
    monkeypatch.setattr(bench, "COUNTERS_PATH", str(tmp_path / "counters.json"))
    key = bench.suite_key(bench.build_parser().parse_args(["--suite", "x", "--suite-only", "spec", "--spec-T", "8"]))
    assert key == "suite-spec-T8-nemotron-gdn"
    log = {"launches": [("k_spec_verify", "T=8 accept all", 3000.0), ("k_spec_commit", "commit", 10.0)],
           "suite_key": key}
    (tmp_path / "log.json").write_text(json.dumps(log))
    for counter, vals in (("FETCH_SIZE", (2.0, 0.01)), ("WRITE_SIZE", (1.0, 0.0))):
        with open(tmp_path / f"{counter}.csv", "w", newline="") as f:
            w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for i in range(3):
                w.writerow({"Dispatch_Id": i, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                            "Counter_Value": 1024.0})
            w.writerow({"Dispatch_Id": 5, "Kernel_Name": "void rs::k_spec_verify<64>(rs::StepParams)",
                        "Counter_Name": counter, "Counter_Value": vals[0]})
            w.writerow({"Dispatch_Id": 6, "Kernel_Name": "void rs::k_spec_commit(rs::StepParams)",
                        "Counter_Name": counter, "Counter_Value": vals[1]})
    assert bench.main(["--summarize-counters", str(tmp_path / "FETCH_SIZE.csv"), str(tmp_path / "WRITE_SIZE.csv"),
                       "--calibrate-copy", "1", "--launch-log", str(tmp_path / "log.json")]) == 0
    entry = json.load(open(tmp_path / "counters.json"))[key]
    assert entry["kernel_source"] == bench.kernel_source_hash()
    v = entry["by_label"]["k_spec_verify T=8 accept all"]
    assert (v["fetch"], v["write"], v["total"], v["algorithmic"], v["ratio"]) == (2048, 1024, 3072, 3000, 1.024)


def test_trace_summary_per_cursor(tmp_path, capsys):
    """--summarize-trace lines the kernel trace up with the launch log and
    averages each cursor position first, then the window."""
    import csv
    import json
    L = 2
    log = {"L": L, "launches": [("k_replay_step", "w0", 100.0), ("k_conventional_step", "conventional", 50.0),
                                ("k_replay_step", "flush", 300.0), ("k_replay_step", "w0", 100.0)]}
    durations = {1: ("k_replay_step<0>", 10_000), 2: ("k_conventional_step<0>", 7_000),
                 3: ("k_replay_step<1>", 30_000), 4: ("k_replay_step<0>", 20_000)}
    path = tmp_path / "kt.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for did, (name, ns) in durations.items():
            w.writerow({"Dispatch_Id": did, "Kernel_Name": f"void rs::{name}(rs::StepParams)",
                        "Start_Timestamp": 1000 * did, "End_Timestamp": 1000 * did + ns})
    lp = tmp_path / "log.json"
    lp.write_text(json.dumps(log))
    assert bench.main(["--summarize-trace", str(path), "--launch-log", str(lp)]) == 0
    lines = [json.loads(x) for x in capsys.readouterr().out.splitlines()]
    by = {(d["kernel"], d["label"]): d for d in lines}
    assert by[("k_replay_step", "w0")]["us_mean"] == 15.0
    assert by[("k_replay_step", "flush")]["us_mean"] == 30.0
    assert by[("k_conventional_step", "conventional")]["us_mean"] == 7.0
    win = by[("k_replay_step", "window average over cursors")]
    assert win["us"] == 22.5 and win["bytes"] == 200


def test_grouped_spec_step_bytes():
    """Grouped keys: a group's key records and draft q, k are counted once,
    and the commit moves each flushed row's accepted keys (read + write per
    group); per-head keys move nothing."""
    H, G, dv, dk, B, T = 128, 8, 64, 128, 2, 4
    h = np.array([3, 14])
    fl = np.array([False, True])
    a = np.array([2, 3])
    per = bench.spec_step_bytes(H, dv, dk, B, T, "f32", "f16", "bf16", h, fl, 0)
    grp = bench.spec_step_bytes(H, dv, dk, B, T, "f32", "f16", "bf16", h, fl, 0, G, a)
    shared = (H - G) * (int(h.sum()) * dk * 2 + B * T * (dk * 2 + 2 * dk * 2))
    moved = 2 * G * dk * 2 * 3          # row 1 flushed with 3 accepted drafts
    assert grp == per - shared + moved
    assert bench.spec_commit_key_bytes(dk, "f16", fl, a, G) == moved
    with pytest.raises(ValueError):
        bench.spec_step_bytes(H, dv, dk, B, T, "f32", "f16", "bf16", h, fl, 0, G)


def test_spec_step_bytes_with_read_copy():
    """A two-precision speculative layer: rows that do not flush read the
    read copy instead of the checkpoint; flushing rows read the recurrence
    copy and write both copies."""
    H, dv, dk, B, T = 128, 64, 128, 2, 4
    h = np.array([3, 14])
    fl = np.array([False, True])
    one = bench.spec_step_bytes(H, dv, dk, B, T, "f32", "f16", "bf16", h, fl, 0)
    two = bench.spec_step_bytes(H, dv, dk, B, T, "f32", "f16", "bf16", h, fl, 0, read="e4m3")
    ms, ml = dv * dk * 4, dv * dk + 4 * dv
    assert two - one == H * ((ml - ms) + ml)   # row 0 reads the read copy; row 1 also writes it


def test_trace_summary_of_timed_launches(tmp_path, capsys):
    """The one-line benchmark logs each launch's phase; --summarize-trace
    reports the mean of the timed launches, which is what bench.py's
    launch_us measures (plus the gaps between launches)."""
    import csv
    import json
    log = {"L": 2, "launches": [("k_replay_step", "w0", 100.0, "prepare"), ("k_replay_step", "flush", 300.0, "timed"),
                                ("k_replay_step", "w0", 100.0, "timed"), ("k_replay_step", "flush", 300.0, "events")]}
    path = tmp_path / "kt.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for did, ns in enumerate((50_000, 30_000, 10_000, 90_000)):
            w.writerow({"Dispatch_Id": did, "Kernel_Name": "void rs::k_replay_step<0>(rs::StepParams)",
                        "Start_Timestamp": 1000 * did, "End_Timestamp": 1000 * did + ns})
    lp = tmp_path / "log.json"
    lp.write_text(json.dumps(log))
    assert bench.main(["--summarize-trace", str(path), "--launch-log", str(lp)]) == 0
    lines = [json.loads(x) for x in capsys.readouterr().out.splitlines()]
    timed = [d for d in lines if d.get("label") == "timed launches"]
    assert len(timed) == 1 and timed[0]["launches"] == 2 and timed[0]["us_mean"] == 20.0



def test_kernel_hash_ignores_comments_only():
    """The stored counters follow the code, not its comments: removing
    comments and collapsing whitespace keeps string and character literals
    (which may hold //) and every token of code."""
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "a//b /*c*/"; char c = \'/\'; x = a / 2;'
    assert bench.code_text(src) == 'int a = 1; const char* s = "a//b /*c*/"; char c = \'/\'; x = a / 2;'
    assert bench.code_text(src.replace("// note", "// other words")) == bench.code_text(src)
    assert bench.code_text(src.replace("a / 2", "a / 3")) != bench.code_text(src)
