"""bench.py's algorithmic byte accounting against the oracle's traffic model."""
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
