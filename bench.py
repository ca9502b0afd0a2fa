"""Benchmark: checkpoint + buffer decode step vs conventional decode step.

    python bench.py [--steps K] [--warmup W] [--workload nemotron|gdn] [--batch B]
                    [--L L] [--state f32|f16] [--pools P] [--no-cpu-baseline]

Default workload: one Mamba-2 layer at the Nemotron-3-Super shape (128 heads,
d_v=64, d_k=128, fp32 state, 4 MiB per sequence), batch 256, L=16, bf16
v/k/q, fp16 records, fp32 log-decay, every row of a pool at the same cursor.
A step is one pass of the whole hot path over the batch: host cursor/flush
metadata, its async upload when it changed, and one kernel launch that
serves flush and non-flush rows.

Cursor schedule.  The method's cost is per window of L tokens (L - 1
appends and one checkpoint write), so a step's cost depends on its cursor.
P state pools (default L + 1, like P layers of a model; P = 1 mod L) are
used in rotation, launch s on pool s mod P, and pool p starts at cursor
(p + phi) mod L, so launch s runs at cursor (s + phi) mod L: any L
consecutive launches visit every cursor once, the flush included.  phi is
chosen from W and K so that the K timed launches are floor(K / L) whole
windows plus a run of K mod L consecutive cursors whose algorithmic bytes
are as close as possible to the window average (exactly whole windows when
L divides K).  Bringing a pool to its starting cursor takes untimed decode
steps before the warm-up.  No launch reuses the previous P - 1 launches'
state, so none finds it in the 256 MB Infinity Cache.

Inputs are seeded synthetic tensors (16 distinct token batches, cycled),
resident in HBM before the timed region.

Prints ONE JSON line.  `value` is the decode steps/s of the checkpoint +
buffer path (wall clock over K steps); the conventional kernel is timed the
same way under "conventional".  "roofline" describes the dominant kernel
(the checkpoint + buffer step): algorithmic bytes of the timed launches /
their time, the time between one pair of HIP events recorded on the launch
stream around the K timed launches; against 8 TB/s.  The per-cursor times
("us_by_cursor") come from 2 L more launches after the timed region, with
events around each launch.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode steps/s + achieved HBM TB/s (% peak), replay vs conventional at bs=256"

WORKLOADS = {
    "nemotron": dict(form=0, H=128, dv=64, dk=128, B=256, L=16, state="f32", rec="f16", io="bf16", read=None),
    # the same layer with the released grouped-key layout: 8 key groups of 16 heads
    "nemotron-grouped": dict(form=0, H=128, dv=64, dk=128, B=256, L=16, state="f32", rec="f16", io="bf16",
                             read=None, groups=8),
    "gdn": dict(form=1, H=32, dv=128, dk=128, B=256, L=16, state="f32", rec="f16", io="bf16", read=None),
}

_ES = {"f32": 4, "f16": 2, "bf16": 2}

# measured HBM bytes per launch (--summarize-counters writes, the roofline's
# `traffic` reads)
COUNTERS_PATH = os.path.join(ROOT, "profiles", "counters.json")

# Launch log: when enabled (a list), every timed-suite launch of one of the
# library's kernels is appended in launch order as (kernel, label, algorithmic
# bytes), so that rocprofv3's per-dispatch counters of the same run can be
# lined up with the launches (summarize_counters).
_LAUNCH_LOG = None


def log_launch(kernel, label, nbytes, phase=""):
    """phase (the one-line benchmark): "prepare", "warm-up", "timed" or
    "events" (the per-cursor breakdown with events around each launch)."""
    if _LAUNCH_LOG is not None:
        _LAUNCH_LOG.append((kernel, label, float(nbytes), phase))


# ----------------------------------------------------------- byte accounting --
def step_bytes(form, H, dv, dk, B, state, rec, io, w, flush, kind="replay", read=None, groups=0):
    """Algorithmic HBM bytes of one launch over B rows at cursor w.

    Checkpoint + buffer step, per (row, head): read the checkpoint (d_v d_k
    state elements) and the w buffered records (x: d_v, k: d_k record
    elements, one fp32 log-decay each); a non-flush row writes one record, a
    flush row writes the checkpoint back.  Conventional step: read and write
    the state.  Both: read q, k (d_k), v (d_v) in the io dtype, the fp32
    log-decay (and beta for Gated DeltaNet), write the fp32 output (d_v); per
    row, read the block id (4 bytes) plus, for the checkpoint + buffer
    step, the cursor and flag (5 bytes).  With a two-precision checkpoint
    (`read` = the read copy's dtype) a non-flush row reads the read copy, a
    flush row reads the recurrence copy and writes both.  With `groups` key
    groups (0: a key per head) the key record and the q, k inputs of a group
    are counted once, spread over its heads."""
    hg = H // groups if groups else 1
    ms = dv * dk * _ES[state]
    r = dv * _ES[rec] + dk * _ES[rec] / hg + 4
    io_b = (2 * dk / hg + dv) * _ES[io] + 4 + (4 if form == 1 else 0) + 4 * dv
    if kind == "conventional":
        return B * (H * (2 * ms + io_b) + 4)
    if read:
        ml = read_copy_bytes(dv, dk, read)
        per_head = (ms + ms + ml if flush else ml + r) + w * r + io_b
    else:
        per_head = ms + w * r + (ms if flush else r) + io_b
    return B * (H * per_head + 9)


def read_copy_bytes(dv, dk, read):
    """One head's read copy: d_v d_k elements, plus an fp32 scale per state
    row for E4M3."""
    if read == "e4m3":
        return dv * dk + 4 * dv
    return dv * dk * _ES[read]


def window_bytes(form, H, dv, dk, B, state, rec, io, L, kind="replay", read=None, groups=0):
    return sum(step_bytes(form, H, dv, dk, B, state, rec, io, w, w == L - 1, kind, read, groups) for w in range(L))


def cursor_bytes(cfg, L=None):
    """Algorithmic bytes of one replay launch at each cursor 0..L-1 (the
    last one flushes)."""
    L = L or cfg["L"]
    return [step_bytes(cfg["form"], cfg["H"], cfg["dv"], cfg["dk"], cfg["B"], cfg["state"], cfg["rec"], cfg["io"],
                       w, w == L - 1, "replay", cfg.get("read"), cfg.get("groups", 0)) for w in range(L)]


def timed_phase(per_cursor, steps):
    """The cursor c0 of the first timed launch: the K timed launches run at
    cursors c0, c0 + 1, ... (mod L); c0 minimises the distance between their
    mean algorithmic bytes and the window average (smallest c0 on ties).
    With L dividing K every c0 gives whole windows and c0 = 0."""
    L = len(per_cursor)
    if steps < 1:
        return 0
    win = sum(per_cursor) / L
    best, best_d = 0, None
    for c0 in range(L):
        m = sum(per_cursor[(c0 + i) % L] for i in range(steps)) / steps
        d = abs(m - win)
        if best_d is None or d < best_d * (1 - 1e-12):
            best, best_d = c0, d
    return best


def cursor_schedule(L, n_pools, warmup, steps, per_cursor):
    """The launch schedule of the replay benchmark.  Returns (phi, starts):
    launch s (counted from the first warm-up launch) runs on pool s mod P at
    cursor (s + phi) mod L, and pool p starts at cursor starts[p] = (p + phi)
    mod L.  Needs P = 1 (mod L): pool p is visited at launches p, p + P, ...
    and its cursor moves by one per visit, which stays (s + phi) mod L only
    when P = 1 (mod L)."""
    if n_pools < 1 or n_pools % L != 1 % L:
        raise ValueError(f"the number of state pools must be 1 mod L (L={L}, got {n_pools})")
    c0 = timed_phase(per_cursor, steps)
    phi = (c0 - warmup) % L
    return phi, [(p + phi) % L for p in range(n_pools)]


def window_us(by_cursor, L):
    """Mean launch time over the L cursor positions (events around each
    launch), or None if a position is missing."""
    keys = [f"w{w}" for w in range(L - 1)] + ["flush"]
    if any(k not in by_cursor for k in keys):
        return None
    return round(float(np.mean([by_cursor[k] for k in keys])), 2)


# C/C++ comments and string or character literals (kept: they can hold //)
_CPP_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def code_text(src: str) -> str:
    """The source with comments removed and whitespace runs collapsed, so
    that editing a comment does not change what counts as the same code."""
    out = _CPP_TOKENS.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), src)
    return " ".join(out.split())


def kernel_source_hash() -> str:
    """Hash of the library's code (comments and layout excluded): stored
    counters are reported only for the code they were measured on."""
    h = hashlib.sha256()
    for f in ("rs_kernels.hip", "rs_api.cpp", "rs_internal.h"):
        with open(os.path.join(ROOT, "linear_attention_decode_replay_amd", "csrc", f)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def workload_key(name, cfg) -> str:
    key = f"{name}-B{cfg['B']}-L{cfg['L']}-{cfg['state']}"
    if cfg.get("groups"):
        key += f"-g{cfg['groups']}"
    if cfg.get("sr"):
        key += "-sr"
    return key + (f"-read{cfg['read']}" if cfg.get("read") else "")


def load_traffic(workload_key: str):
    """HBM traffic per launch measured with rocprofv3 counters, if a summary
    for the current kernel source exists under profiles/."""
    path = COUNTERS_PATH
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    entry = data.get(workload_key)
    if not entry or entry.get("kernel_source") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


# --------------------------------------------------------------- CPU baseline --
def cpu_baseline(cfg, n_steps=None, rows=None, min_seconds=10.0, max_windows=32):
    """The fp64 oracle (both routes) on the host cores over a bounded sample:
    `rows` rows (default all), whole windows of L steps repeated until the
    checkpoint + buffer route has run `min_seconds` (at most `max_windows`
    windows), after one untimed window; reported as steps/s of the full
    batch."""
    import oracle
    import workloads
    o = oracle.get()
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    o.set_num_threads(threads)
    B = rows or cfg["B"]
    n_steps = n_steps or cfg["L"]
    toks = [workloads.tokens(cfg["form"], 7, s, B, cfg["H"], cfg["dv"], cfg["dk"], cfg["io"])
            for s in range(n_steps)]
    f64 = [(t.q.double().numpy(), t.k.double().numpy(), t.v.double().numpy(), t.lam.double().numpy(),
            None if t.beta is None else t.beta.double().numpy()) for t in toks]
    w, fl = o.cursor_run(cfg["L"], 0, n_steps)
    if cfg.get("read"):
        rep = oracle.TwoCopyReplayModel(B, cfg["H"], cfg["dv"], cfg["dk"], cfg["L"], cfg["read"])
    else:
        rep = oracle.ReplayModel(cfg["form"], B, cfg["H"], cfg["dv"], cfg["dk"], cfg["L"])
    def window(model, replay):
        for s in range(n_steps):
            q, k, v, lam, beta = f64[s]
            if replay:
                model.step(q, k, v, lam, np.full(B, fl[s]), beta)
            else:
                model.step(q, k, v, lam, beta)

    window(rep, True)  # untimed: first touch of the model's memory
    n_win = 0
    t0 = time.perf_counter()
    while n_win < max_windows and (n_win == 0 or time.perf_counter() - t0 < min_seconds):
        window(rep, True)
        n_win += 1
    t_rep = time.perf_counter() - t0
    del rep
    conv = oracle.ConventionalModel(cfg["form"], B, cfg["H"], cfg["dv"], cfg["dk"])
    window(conv, False)
    t0 = time.perf_counter()
    for _ in range(n_win):
        window(conv, False)
    t_conv = time.perf_counter() - t0
    # the same route on one thread, over a sixteenth of the rows (one window)
    b1 = max(1, B // 16)
    one = (oracle.TwoCopyReplayModel(b1, cfg["H"], cfg["dv"], cfg["dk"], cfg["L"], cfg["read"]) if cfg.get("read")
           else oracle.ReplayModel(cfg["form"], b1, cfg["H"], cfg["dv"], cfg["dk"], cfg["L"]))
    f64_all = f64
    f64 = [tuple(None if a is None else a[:b1] for a in t) for t in f64_all]
    o.set_num_threads(1)
    Bsave, B = B, b1
    t0 = time.perf_counter()
    window(one, True)
    t_one = time.perf_counter() - t0
    B = Bsave
    o.set_num_threads(threads)
    del one
    one_thread = n_steps * (b1 / cfg["B"]) / t_one
    scale = B / cfg["B"]
    total = n_win * n_steps
    route = "two-copy checkpoint+buffer" if cfg.get("read") else "checkpoint+buffer"
    return {
        "value": round(total * scale / t_rep, 4),
        "unit": "steps/s",
        "cores": o.num_threads(),
        "kind": "oracle",
        "sample": (f"fp64 oracle, {route} route, {total} steps ({n_win} windows of {n_steps}) over "
                   f"{B} of {cfg['B']} rows x {cfg['H']} heads; conventional route "
                   f"{round(total * scale / t_conv, 4)} steps/s; the checkpoint+buffer route on 1 thread "
                   f"({b1} rows, one window, scaled to the batch) {round(one_thread, 4)} steps/s; "
                   f"{t_rep + t_conv + t_one:.1f} s of CPU time"),
    }


# ------------------------------------------------------------------------ GPU --
def run_gpu(cfg, steps, warmup, n_pools, kind):
    """Time K steps of one kernel kind on the cursor schedule above.  Returns
    the timings plus `launches`: (cursor, flush, algorithmic bytes) of every
    launch in launch order (pool preparation, warm-up, timed, breakdown),
    which lines the launches up with rocprofv3's per-dispatch counters."""
    import torch
    import linear_attention_decode_replay_amd as rs
    import workloads
    from linear_attention_decode_replay_amd.state import DecodeLayer

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    L = cfg["L"]
    # the conventional step has one state copy whatever the replay layout
    read = cfg["read"] if kind == "replay" else None
    groups = cfg.get("groups", 0)
    lay = rs.layer(cfg["form"], cfg["H"], cfg["dv"], cfg["dk"], L, cfg["state"], cfg["rec"], cfg["io"], read,
                   0, groups, stochastic=bool(cfg.get("sr")))
    B = cfg["B"]
    per_cursor = cursor_bytes(cfg)
    phi, starts = cursor_schedule(L, n_pools, warmup, steps, per_cursor)
    layers = []
    for p in range(n_pools):
        d = DecodeLayer(lay, B, B, dev, sr_key=(0x5EED0000 + p, 0x243F6A8885A308D3))
        for b in range(B):
            d.assign(b, b)
        d.reset_rows(range(B))
        layers.append(d)
    n_inputs = 16
    ios, keep = [], []
    for s in range(n_inputs):
        t = workloads.tokens(cfg["form"], 11, s, B, cfg["H"], cfg["dv"], cfg["dk"], cfg["io"])
        if groups:  # the group's key and query: those drawn for its first head
            hg = cfg["H"] // groups
            t = workloads.Tokens(t.q[:, ::hg].contiguous(), t.k[:, ::hg].contiguous(), t.v, t.lam, t.beta)
        q, k, v, lam = (x.to(dev) for x in (t.q, t.k, t.v, t.lam))
        beta = t.beta.to(dev) if t.beta is not None else None
        out = torch.empty((B, cfg["H"], cfg["dv"]), dtype=torch.float32, device=dev)
        keep.append((q, k, v, lam, beta, out))
        ios.append(rs.make_io(q, k, v, lam, out, beta))
    torch.cuda.synchronize()
    launches = []

    phase = ["prepare"]

    def launch(d, io, events=None):
        if kind == "replay":
            wp, fl = d.step(io, events=events)
            w, f = int(wp[0]), bool(fl[0])
        else:
            d.conventional_step(io, events=events)
            w, f = 0, False
        nb = step_bytes(cfg["form"], cfg["H"], cfg["dv"], cfg["dk"], B, cfg["state"], cfg["rec"], cfg["io"], w, f,
                        kind, cfg["read"], groups)
        launches.append((w, f, nb))
        if kind == "replay":
            log_launch("k_replay_step", "flush" if f else f"w{w}", nb, phase[0])
        else:
            log_launch("k_conventional_step", "conventional", nb, phase[0])
        return w, f

    # pool preparation (untimed): pool p decodes starts[p] tokens
    if kind == "replay":
        for p, n in enumerate(starts):
            for i in range(n):
                launch(layers[p], ios[i % n_inputs])
    torch.cuda.synchronize()

    def one(s, events=None):
        w, f = launch(layers[s % n_pools], ios[s % n_inputs], events)
        if kind == "replay" and w != (s + phi) % L:
            raise RuntimeError(f"launch {s} ran at cursor {w}, the schedule says {(s + phi) % L}")
        return w, f

    phase[0] = "warm-up"
    for s in range(warmup):
        one(s)
    torch.cuda.synchronize()
    phase[0] = "timed"
    # Timed region: K back-to-back steps, bracketed by one pair of HIP events
    # on the launch stream (no event between launches, so none of their
    # overhead lands inside a launch).
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    first = len(launches)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        one(warmup + i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = start.elapsed_time(end)
    timed = launches[first:]
    errs = sum(int(d.err.item()) for d in layers)
    if errs:
        raise RuntimeError(f"{errs} tiles skipped by the kernel's bounds checks")
    nbytes = [b for (_, _, b) in timed]
    # Breakdown by cursor position (after the timed region, not part of it):
    # 2 L more launches (every cursor twice) with events around each.
    by_pos = {}
    phase[0] = "events"
    if kind == "replay":
        n_brk = 2 * L
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_brk)]
        brk = [one(warmup + steps + i, ev[i]) for i in range(n_brk)]
        torch.cuda.synchronize()
        for (w, f), (a, b) in zip(brk, ev):
            by_pos.setdefault("flush" if f else f"w{w}", []).append(a.elapsed_time(b))
    mix = {}
    for (w, f, _) in timed:
        key = "flush" if f else f"w{w}"
        mix[key] = mix.get(key, 0) + 1
    return {
        "wall_s": wall,
        "steps_per_s": steps / wall,
        "ms_per_step": 1e3 * wall / steps,
        "kernel_ms_mean": region_ms / steps,
        "bytes_per_launch_mean": float(np.mean(nbytes)),
        "window_bytes_per_launch": float(np.mean(per_cursor)),
        "achieved_gbs": float(np.sum(nbytes) / (region_ms * 1e-3) / 1e9),
        "by_position_us": {k: round(1e3 * float(np.mean(v)), 1) for k, v in sorted(by_pos.items())},
        "timed_cursor_counts": dict(sorted(mix.items())),
        "first_timed_cursor": (warmup + phi) % L,
        "launches": launches,
    }


# ------------------------------------------------------------------- suite --
def _inputs(cfg, B, n, dev, seed=11):
    import linear_attention_decode_replay_amd as rs
    import torch
    import workloads
    ios, keep = [], []
    hg = cfg["H"] // cfg["groups"] if cfg.get("groups") else 1
    for s in range(n):
        t = workloads.tokens(cfg["form"], seed, s, B, cfg["H"], cfg["dv"], cfg["dk"], cfg["io"])
        if hg > 1:  # the group's key and query: those drawn for its first head
            t = workloads.Tokens(t.q[:, ::hg].contiguous(), t.k[:, ::hg].contiguous(), t.v, t.lam, t.beta)
        q, k, v, lam = (x.to(dev) for x in (t.q, t.k, t.v, t.lam))
        beta = t.beta.to(dev) if t.beta is not None else None
        out = torch.empty((B, cfg["H"], cfg["dv"]), dtype=torch.float32, device=dev)
        keep.append((q, k, v, lam, beta, out))
        ios.append(rs.make_io(q, k, v, lam, out, beta))
    return ios, keep


def _layer_stack(cfg, B, n_layers, dev, reconstruct=False):
    import linear_attention_decode_replay_amd as rs
    from linear_attention_decode_replay_amd.state import DecodeLayer
    lay = rs.layer(cfg["form"], cfg["H"], cfg["dv"], cfg["dk"], cfg["L"], cfg["state"], cfg["rec"], cfg["io"],
                   cfg["read"], 0, cfg.get("groups", 0), reconstruct=reconstruct)
    layers = []
    for _ in range(n_layers):
        d = DecodeLayer(lay, B, B, dev)
        for b in range(B):
            d.assign(b, b)
        d.reset_rows(range(B))
        layers.append(d)
    return layers


def suite_gdn_sweep(out, steps=32):
    """Gated DeltaNet, 32 heads, 128x128, L=16: replay (output-only route),
    replay (state-reconstruction route) and conventional kernel time per
    launch over batch sizes, fp32 and fp16 state.  Reading a 1 GiB
    buffer between launches (outside the timed events) evicts the state from
    the 256 MB Infinity Cache and the L2s without leaving dirty lines behind,
    so every launch is cold."""
    import torch
    dev = torch.device("cuda", 0)
    scrub = torch.ones(2**28, dtype=torch.int32, device=dev)
    for state in ("f32", "f16"):
        for B in (1, 8, 32, 128, 256, 512):
            cfg = dict(WORKLOADS["gdn"], B=B, state=state)
            ios, keep = _inputs(cfg, B, 16, dev)
            res = {}
            for kind in ("replay", "reconstruct", "conventional"):
                d = _layer_stack(cfg, B, 1, dev, reconstruct=kind == "reconstruct")[0]
                times, nbytes = [], []
                for s in range(16 + steps):
                    scrub.sum()
                    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    if kind != "conventional":
                        wp, fl = d.step(ios[s % 16], events=ev)
                        w, f = int(wp[0]), bool(fl[0])
                    else:
                        d.conventional_step(ios[s % 16], events=ev)
                        w, f = 0, False
                    nb = step_bytes(cfg["form"], cfg["H"], cfg["dv"], cfg["dk"], B, state, cfg["rec"], cfg["io"], w,
                                    f, "conventional" if kind == "conventional" else "replay")
                    log_launch("k_conventional_step" if kind == "conventional" else "k_replay_step",
                               f"gdn B={B} {state} {kind}" + ("" if s >= 16 else " warm-up"), nb)
                    if s >= 16:
                        times.append(ev)
                        nbytes.append(nb)
                torch.cuda.synchronize()
                us = float(np.mean([a.elapsed_time(b) for a, b in times])) * 1e3
                res[kind] = {"us": round(us, 2), "tbs": round(float(np.mean(nbytes)) / (us * 1e-6) / 1e12, 3)}
                del d
            line = {"suite": "gdn_batch_sweep", "state": state, "batch": B, "L": 16,
                    "replay_us": res["replay"]["us"], "replay_tbs": res["replay"]["tbs"],
                    "reconstruct_us": res["reconstruct"]["us"], "reconstruct_tbs": res["reconstruct"]["tbs"],
                    "conventional_us": res["conventional"]["us"], "conventional_tbs": res["conventional"]["tbs"],
                    "speedup": round(res["conventional"]["us"] / res["replay"]["us"], 3),
                    "speedup_reconstruct": round(res["conventional"]["us"] / res["reconstruct"]["us"], 3)}
            print(json.dumps(line), file=out, flush=True)
            del ios, keep
            torch.cuda.empty_cache()


def suite_stack(out, n_layers=40, quick=False):
    """40 Mamba-2 layers at the Nemotron-3-Super shape, batch 256: time and
    algorithmic bytes of one decode step over all layers (one launch per
    layer), replay for L in {8, 16, 32} with fp32 and fp16 checkpoints, replay
    at L=16 with an fp32 recurrence copy and an fp16, bf16 or E4M3 read copy, and
    the conventional step with fp32 and fp16 state.  Two windows timed after
    one window of warm-up."""
    import torch
    dev = torch.device("cuda", 0)
    base = dict(WORKLOADS["nemotron"])
    ios, keep = _inputs(base, base["B"], 16, dev)
    results = {}
    runs = [("conventional", 16, "f32", None), ("conventional", 16, "f16", None)]
    runs += [("replay", L, st, None) for st in ("f32", "f16") for L in (8, 16, 32)]
    runs += [("replay", 16, "f32", rd) for rd in ("f16", "bf16", "e4m3")]
    if quick:  # the fp32 conventional step and the L = 16 fp32 replay step only
        runs = [("conventional", 16, "f32", None), ("replay", 16, "f32", None)]
    for kind, L, state, read in runs:
        cfg = dict(base, L=L, state=state, read=read)
        layers = _layer_stack(cfg, base["B"], n_layers, dev)
        n_warm, n_time = L, 2 * L
        nbytes = 0
        for s in range(n_warm + n_time):
            if s == n_warm:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                e0 = torch.cuda.Event(enable_timing=True)
                e0.record()
            for li, d in enumerate(layers):
                io = ios[(s + li) % 16]
                if kind == "replay":
                    wp, fl = d.step(io)
                    w, f = int(wp[0]), bool(fl[0])
                else:
                    d.conventional_step(io)
                    w, f = 0, False
                nb = step_bytes(cfg["form"], cfg["H"], cfg["dv"], cfg["dk"], cfg["B"], state, cfg["rec"], cfg["io"],
                                w, f, kind, read)
                log_launch("k_replay_step" if kind == "replay" else "k_conventional_step",
                           f"stack40 {kind} L={L} {state}" + (f" read {read}" if read else ""), nb)
                if s >= n_warm:
                    nbytes += nb
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = e0.elapsed_time(e1) / n_time
        gb = nbytes / n_time / 1e9
        results[(kind, L, state, read)] = ms
        line = {"suite": "stack40", "kind": kind, "L": L if kind == "replay" else None, "state": state,
                "read_copy": read,
                "ms_per_step": round(ms, 3), "wall_ms_per_step": round(1e3 * wall / n_time, 3),
                "gb_per_step": round(gb, 3), "tbs": round(gb / ms, 3)}
        print(json.dumps(line), file=out, flush=True)
        del layers
        torch.cuda.empty_cache()
    for (kind, L, state, read), ms in results.items():
        if kind == "replay":
            c16 = results.get(("conventional", 16, "f16", None))
            line = {"suite": "stack40_ratio", "L": L, "state": state, "read_copy": read,
                    "speedup_vs_conventional_f32": round(results[("conventional", 16, "f32", None)] / ms, 3),
                    "speedup_vs_conventional_f16": round(c16 / ms, 3) if c16 else None}
            print(json.dumps(line), file=out, flush=True)


def spec_step_bytes(H, dv, dk, B, T, state, rec, io, h, flush, form=0, groups=0, accepted=None, read=None):
    """Algorithmic HBM bytes of one speculative verify launch (rows with h
    committed records, flushing or not) plus its commit launch.  Per (row,
    head): read the checkpoint and the h committed records, read T draft
    tokens (q, k, v, log-decay), write T records and T fp32 outputs; a
    flushing row also writes the checkpoint.  Per row: block id, count and
    flag read by the verify; the commit reads block id, count, flag and the
    accepted count and writes the next count and flag.  With `groups` key
    groups the key records and q, k inputs of a group are counted once,
    spread over its heads, and the commit moves each flushed row's accepted
    keys (`accepted`) out of the staging slots: read and write once per
    group (see spec_commit_key_bytes).  With a two-precision checkpoint
    (`read` = the read copy's dtype) a row that does not flush reads the read
    copy; a flushing row reads the recurrence copy and writes both."""
    h = np.asarray(h)
    flush = np.asarray(flush, bool)
    hg = H // groups if groups else 1
    ms = dv * dk * _ES[state]
    r = (dv + dk / hg) * _ES[rec] + 4
    tok = (2 * dk / hg + dv) * _ES[io] + 4 + (4 if form == 1 else 0)  # q, k, v, log-decay (and beta)
    if read:
        ml = read_copy_bytes(dv, dk, read)
        ck = np.where(flush, ms + ms + ml, ml)
    else:
        ck = np.where(flush, ms + ms, ms)
    per_head = ck + h * r + T * (tok + r + 4 * dv)
    moved = spec_commit_key_bytes(dk, rec, flush, accepted, groups) if hg > 1 else 0.0
    return float(np.sum(H * per_head + 9) + B * 18 + moved)


def spec_commit_key_bytes(dk, rec, flush, accepted, groups):
    """Bytes the commit moves for grouped keys: each flushed row's accepted
    draft keys, read from the staging slots and written to slot 0, per
    group (block id, count and flag re-read per (row, group) are counted
    with the commit's per-row bytes)."""
    if accepted is None:
        raise ValueError("grouped keys: the accepted counts decide the commit's key moves")
    a = np.where(np.asarray(flush, bool), np.asarray(accepted), 0)
    return float(2 * groups * dk * _ES[rec] * np.sum(a))


def suite_spec(out, steps=48, n_pools=4, workload="nemotron", Ts=(4, 8), read=None):
    """Speculative verify at the Nemotron-3-Super layer shape (workload
    "nemotron-grouped": with its 8 key groups; "gdn": the Gated DeltaNet
    layer, 32 heads, 128 x 128), batch 256,
    L = 16, fp32 checkpoint, fp16 records, bf16 inputs, T in {4, 8}, with
    every draft accepted, one token per step, and uniform 0..T acceptance.
    One step = one verify launch + one commit launch (the committed counts
    stay on the device); time per step from one pair of HIP events around
    the timed steps; 4 state pools in rotation (cold caches).  Reported per
    committed token next to the standard replay step and the conventional
    step measured the same way."""
    import torch
    import linear_attention_decode_replay_amd as rs
    import workloads
    from linear_attention_decode_replay_amd.state import SpecDecodeLayer
    dev = torch.device("cuda", 0)
    base = dict(WORKLOADS[workload])
    B, H, dv, dk, L = base["B"], base["H"], base["dv"], base["dk"], base["L"]
    form = base["form"]
    groups = base.get("groups", 0)
    hg = H // groups if groups else 1
    # standard steps for reference (one token per row per step)
    ios, keep = _inputs(base, B, 16, dev)
    ref_us = {}
    for kind in ("replay", "conventional"):
        # the reference replay step keeps the same read copy; the conventional one has one state copy
        kread = read if kind == "replay" else None
        layers = _layer_stack(dict(base, read=kread), B, n_pools, dev)
        n_warm, n_time = L * n_pools, 2 * L * n_pools
        for s in range(n_warm + n_time):
            if s == n_warm:
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e0.record()
            d = layers[s % n_pools]
            if kind == "replay":
                wp, fl = d.step(ios[s % 16])
                w, f = int(wp[0]), bool(fl[0])
            else:
                d.conventional_step(ios[s % 16])
                w, f = 0, False
            log_launch("k_replay_step" if kind == "replay" else "k_conventional_step", f"{workload} reference {kind}",
                       step_bytes(form, H, dv, dk, B, "f32", base["rec"], base["io"], w, f, kind, kread, groups))
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record()
        torch.cuda.synchronize()
        ref_us[kind] = 1e3 * e0.elapsed_time(e1) / n_time
        del layers
        torch.cuda.empty_cache()
    del ios, keep
    for T in Ts:
        lay = rs.layer(form, H, dv, dk, L, "f32", "f16", "bf16", read, T, groups)
        drafts = []
        for s in range(8):
            t = workloads.spec_tokens(11, s, B, H, T, dv, dk, "bf16", form=form)
            if hg > 1:  # the group's key and query: those drawn for its first head
                t.q, t.k = t.q[:, :, ::hg].contiguous(), t.k[:, :, ::hg].contiguous()
            q, k, v, lam = (x.to(dev) for x in (t.q, t.k, t.v, t.lam))
            beta = t.beta.to(dev) if t.beta is not None else None
            o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
            drafts.append(((q, k, v, lam, o, beta), rs.make_spec_io(q, k, v, lam, o, beta)))
        for policy in ("all", "one", "random"):
            pools = []
            for _ in range(n_pools):
                d = SpecDecodeLayer(lay, B, B, dev)
                for b in range(B):
                    d.assign(b, b)
                d.upload(rows=range(B))
                pools.append(d)
            acc = [torch.from_numpy(workloads.spec_accepted(3, s, B, T, policy)).to(dev) for s in range(steps)]
            acc_host = [a.cpu().numpy() for a in acc]
            hmirror = [np.zeros(B, np.int32) for _ in range(n_pools)]
            n_warm = steps // 2
            nbytes, tokens, n_flush = 0.0, 0, 0
            for s in range(n_warm + steps):
                if s == n_warm:
                    torch.cuda.synchronize()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                pi = s % n_pools
                d, hm = pools[pi], hmirror[pi]
                a = acc_host[s % steps]
                fl = rs.rs_spec_meta_step(L, T, hm)
                nb = spec_step_bytes(H, dv, dk, B, T, "f32", "f16", "bf16", hm, fl, form, groups, a, read)
                moved = spec_commit_key_bytes(dk, "f16", fl, a, groups) if hg > 1 else 0.0
                if s >= n_warm:
                    nbytes += nb
                    tokens += int(a.sum())
                    n_flush += int(fl.sum())
                d.verify(drafts[s % 8][1])
                d.commit(acc[s % steps])
                label = f"{workload}{' read ' + read if read else ''} T={T} accept {policy}"
                log_launch("k_spec_verify" if form == 0 else "k_spec_verify_gdn", label, nb - B * 18 - moved)
                if hg > 1:
                    log_launch("k_spec_commit_keys", label, moved)
                log_launch("k_spec_commit", label, B * 18)
                rs.rs_spec_meta_advance(L, T, hm, fl, a)
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record()
            torch.cuda.synchronize()
            us = 1e3 * e0.elapsed_time(e1) / steps
            errs = sum(int(d.err.item()) for d in pools)
            if errs:
                raise RuntimeError(f"{errs} tiles or rows flagged by the speculative kernels' checks")
            gb = nbytes / steps / 1e9
            tok_per_row = tokens / steps / B
            line = {"suite": "spec_verify", "workload": workload, "read_copy": read, "T": T, "accept": policy,
                    "batch": B, "L": L,
                    "us_per_step": round(us, 2), "gb_per_step": round(gb, 4), "tbs": round(gb / (us * 1e-6) / 1e3, 3),
                    "committed_tokens_per_row_step": round(tok_per_row, 3),
                    "flush_fraction": round(n_flush / (steps * B), 4),
                    "us_per_committed_token": round(us / tok_per_row, 2) if tokens else None,
                    "replay_step_us": round(ref_us["replay"], 2), "conventional_step_us": round(ref_us["conventional"], 2),
                    "speedup_per_token_vs_replay": round(ref_us["replay"] / (us / tok_per_row), 3) if tokens else None,
                    "speedup_per_token_vs_conventional":
                        round(ref_us["conventional"] / (us / tok_per_row), 3) if tokens else None}
            print(json.dumps(line), file=out, flush=True)
            del pools
            torch.cuda.empty_cache()
        del drafts
        torch.cuda.empty_cache()


def suite_continuous(out, steps=200, n_layers=4):
    """Continuous batching at the Nemotron-3-Super layer shape: 256 request
    slots over a shuffled pool of 384 blocks, rows starting mid-window (cursor
    U{0..15}), each live row retiring with p = 1/32 per step and each empty
    slot taking a new request with p = 1/2.  n_layers layers of one model
    share the slots (one block table, one set of cursors and flags: one
    metadata upload per step when rows retire or join) and each has its own
    pool, so that no launch finds its state in the caches.  A joining row of
    the checkpoint + buffer layers starts with a zero checkpoint that is not
    read until its first flush (RS_CURSOR_ZERO_CKPT: no launch); the
    conventional layers zero a joining row's state with replay_state_reset
    (its launches are in the timed region).  Each kind runs the schedule
    twice on fresh pools: once timed as a whole (one event pair around the
    run), once with events around every launch (the per-launch
    distribution)."""
    import torch
    import linear_attention_decode_replay_amd as rs
    import workloads
    from linear_attention_decode_replay_amd.state import DecodeLayer
    dev = torch.device("cuda", 0)
    cfg = dict(WORKLOADS["nemotron"])
    B, H, dv, dk, L, NB = cfg["B"], cfg["H"], cfg["dv"], cfg["dk"], cfg["L"], 384
    lay = rs.layer(0, H, dv, dk, L, cfg["state"], cfg["rec"], cfg["io"])
    ios, keep = _inputs(cfg, B, 16, dev)
    blocks0, w0s, events = workloads.continuous_schedule(17, B, steps, NB)
    ms_state = dv * dk * _ES[cfg["state"]]
    rec = (dv + dk) * _ES[cfg["rec"]] + 4
    io_b = (2 * dk + dv) * _ES[cfg["io"]] + 4 + 4 * dv
    for kind in ("replay", "conventional"):
        res = {}
        for per_launch_events in (False, True):
            d = DecodeLayer(lay, B, NB, dev, n_layers=n_layers)
            for slot in range(B):
                d.assign(slot, int(blocks0[slot]))
            d.reset_rows(range(B))
            for slot in range(B):  # mid-window starts (the records' values do not matter for timing)
                d.assign(slot, int(blocks0[slot]), int(w0s[slot]))
            torch.cuda.synchronize()
            flush_frac, live_rows, nbytes, ev, uploads0 = [], [], 0.0, [], d.uploads
            e0 = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record()
            for s in range(steps):
                e = events[s]
                for slot in e.retire:
                    d.retire(slot)
                for slot, b in e.join:
                    d.assign(slot, int(b))
                joined = [slot for slot, _ in e.join]
                if joined:
                    if kind == "replay":
                        d.join_rows(joined)
                    else:
                        d.reset_rows(joined)
                pairs = None
                if per_launch_events:
                    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                             for _ in range(n_layers)]
                    ev.extend(pairs)
                step_ios = [ios[(s + li) % 16] for li in range(n_layers)]
                live = d.live()
                if kind == "replay":
                    zc = d.zero_ckpt & live
                    wp, fl = d.step(step_ios, events=pairs)
                    flush_frac.append(float(np.mean(fl[live])) if live.any() else 0.0)
                    live_rows.append(int(live.sum()))
                    f = fl[live].astype(bool)
                    w = wp[live]
                    # a zero checkpoint counts no read (one cache line per tile at most; its flush still writes it)
                    ck_read = np.where(zc[live], 0, ms_state)
                    nb = float(np.sum(H * (ck_read + w * rec + np.where(f, ms_state, rec) + io_b) + 9))
                    nb += 4.0 * int((~live).sum())
                else:
                    d.conventional_step(step_ios, events=pairs)
                    nb = float(live.sum()) * (H * (2 * ms_state + io_b) + 4) + 4.0 * int((~live).sum())
                nbytes += n_layers * nb
                for _ in range(n_layers):
                    log_launch("k_replay_step" if kind == "replay" else "k_conventional_step",
                               f"continuous {kind}" + (" (events per launch)" if per_launch_events else ""), nb)
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            total_us = e0.elapsed_time(e1) * 1e3
            errs = int(d.err.item())
            if errs:
                raise RuntimeError(f"{errs} tiles skipped by the kernel's bounds checks")
            n = steps * n_layers
            if per_launch_events:
                per_launch = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
                res.update({"us_per_launch_mean": round(float(per_launch.mean()), 2),
                            "us_per_launch_p50": round(float(np.percentile(per_launch, 50)), 2),
                            "us_per_launch_p90": round(float(np.percentile(per_launch, 90)), 2),
                            "us_per_launch_max": round(float(per_launch.max()), 2)})
            else:
                res.update({"us_per_launch_region": round(total_us / n, 2),
                            "wall_us_per_launch": round(1e6 * wall / n, 2),
                            "gb_per_launch": round(nbytes / n / 1e9, 4),
                            "tbs_region": round(nbytes / (total_us * 1e-6) / 1e12, 3),
                            "metadata_uploads": d.uploads - uploads0})
                if kind == "replay":
                    res["flushing_rows_mean"] = round(float(np.mean(flush_frac)), 4)
                    res["live_rows_mean"] = round(float(np.mean(live_rows)), 1)
            del d
            torch.cuda.empty_cache()
        line = {"suite": "continuous_batching", "kind": kind, "slots": B, "pool_blocks": NB, "steps": steps,
                "layers": n_layers, **res}
        print(json.dumps(line), file=out, flush=True)


def calibrate_copy(mib: int) -> None:
    """A plain device-to-device copy of `mib` MiB, three times: its
    FETCH_SIZE / WRITE_SIZE readings give the scale of those counters."""
    import torch
    n = mib * 2**20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def _read_counter_csv(path):
    """Per-dispatch counter values from a rocprofv3 counter_collection.csv:
    returns [(dispatch id, kernel_name, counter_name, value)] in dispatch
    order."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for i, r in enumerate(csv.DictReader(f)):
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or r.get("kernel_name") or ""
            cname = r.get("Counter_Name") or r.get("Counter-Name") or ""
            val = r.get("Counter_Value") or r.get("Counter-Value") or "0"
            did = r.get("Dispatch_Id") or r.get("Dispatch-Id") or r.get("dispatch_id") or i
            rows.append((int(did), name, cname, float(val)))
    rows.sort(key=lambda t: t[0])
    return rows


def kernel_family(name: str) -> str:
    """The function name of a (demangled) kernel: 'k_replay_step' for
    'void rs::(anonymous namespace)::k_replay_step<0, 64, ...>(rs::StepParams)'."""
    import re
    m = re.search(r"(k_[A-Za-z0-9_]+)\s*[<(]", name)
    return m.group(1) if m else name


def config_from_args(args):
    """The workload's configuration with the command line's overrides."""
    cfg = dict(WORKLOADS[args.workload])
    if args.batch:
        cfg["B"] = args.batch
    if args.L:
        cfg["L"] = args.L
    if args.state:
        cfg["state"] = args.state
    cfg["read"] = args.read
    cfg["sr"] = args.rounding == "stochastic"
    return cfg


def counter_scale(rows, mib, what):
    """Bytes per counter unit: the counters are KiB per dispatch; the
    calibration copy of `mib` MiB (three dispatches, the largest copies of the
    run) gives the scale."""
    copy = sorted((v for (_, n, _, v) in rows if "copy" in n.lower() and not n.lstrip().startswith("void rs::")),
                  reverse=True)[:3]
    if not copy or copy[-1] * 1024 < 0.25 * mib * 2**20:
        raise SystemExit(f"no calibration copy of ~{mib} MiB found in the {what} counters")
    return mib * 2**20 / (float(np.median(copy)) * 1024)


def line_up(rows, log, scale):
    """Measured bytes per logged launch: the dispatches of each kernel
    family, in dispatch order, against that family's logged launches, in
    launch order.  Returns {(family, label): [(measured, algorithmic), ...]}."""
    disp = {}
    for (_, name, _, v) in rows:
        disp.setdefault(kernel_family(name), []).append(v * 1024 * scale)
    logged = {}
    for fam, label, nb, *_ in log:
        logged.setdefault(fam, []).append((label, nb))
    out = {}
    for fam, launches in logged.items():
        got = disp.get(fam, [])
        if len(got) != len(launches):
            raise SystemExit(f"{fam}: {len(got)} dispatches in the counters, {len(launches)} launches logged")
        for (label, nb), m in zip(launches, got):
            out.setdefault((fam, label), []).append((m, nb))
    return out


def suite_key(args) -> str:
    """The counters.json key of a suite run: which suite and its options."""
    parts = ["suite", args.suite_only or "all"]
    if args.suite_only == "spec":
        parts += [f"T{t}" for t in (args.spec_T or (4, 8))] + list(args.spec_workload or ["nemotron", "gdn"])
        if args.read:
            parts.append(f"read{args.read}")
    if args.suite_only == "stack" and args.stack_quick:
        parts.append("quick")
    return "-".join(str(x) for x in parts)


def summarize_counters(args, fetch_csv, write_csv):
    """FETCH_SIZE and WRITE_SIZE are in KiB per dispatch.  Each is scaled by
    (known bytes of the calibration copy) / (its reading).  The dispatches
    are lined up with the launch log that the profiled run wrote
    (--launch-log), which gives each launch's label (cursor, suite case) and
    algorithmic bytes.  Prints one JSON line per (kernel, label) with the
    mean measured fetch, write and total per launch and the ratio to the
    algorithmic bytes.  For the one-line benchmark (labels = cursors), the
    window average over cursors is stored in profiles/counters.json under
    the workload's key."""
    mib = args.calibrate_copy
    if not mib:
        raise SystemExit("--summarize-counters needs --calibrate-copy MIB (the size used in the profiled run)")
    if not args.launch_log:
        raise SystemExit("--summarize-counters needs --launch-log PATH (written by the profiled run)")
    log = json.load(open(args.launch_log))
    per = {}
    scales = {}
    for label, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = _read_counter_csv(path)
        scales[label] = counter_scale(rows, mib, label)
        per[label] = line_up(rows, log["launches"], scales[label])
    table = {}
    for key in per["fetch"]:
        f = np.array([m for m, _ in per["fetch"][key]])
        w = np.array([m for m, _ in per["write"][key]])
        alg = np.array([nb for _, nb in per["fetch"][key]])
        table[key] = {"kernel": key[0], "label": key[1], "launches": len(f), "fetch": float(f.mean()),
                      "write": float(w.mean()), "total": float((f + w).mean()), "algorithmic": float(alg.mean()),
                      "ratio": float((f + w).sum() / alg.sum())}
        print(json.dumps({k: (round(v) if isinstance(v, float) and k != "ratio" else
                              (round(v, 4) if k == "ratio" else v)) for k, v in table[key].items()}))
    path = COUNTERS_PATH
    if log.get("suite_key"):  # a suite: every (kernel, case) as measured
        data = json.load(open(path)) if os.path.exists(path) else {}
        data[log["suite_key"]] = {
            "kernel_source": kernel_source_hash(),
            "basis": "mean per launch of each (kernel, case) label",
            "by_label": {f"{t['kernel']} {t['label']}": {"launches": t["launches"], "fetch": round(t["fetch"]),
                                                         "write": round(t["write"]), "total": round(t["total"]),
                                                         "algorithmic": round(t["algorithmic"]),
                                                         "ratio": round(t["ratio"], 4)}
                         for t in table.values()},
            "scale": {"fetch": round(scales["fetch"], 4), "write": round(scales["write"], 4)},
            "calibration_copy_mib": mib}
        with open(path, "w") as fo:
            json.dump(data, fo, indent=1, sort_keys=True)
            fo.write("\n")
    # the one-line benchmark's launches: window averages over the cursors
    L = log.get("L")
    if L and log.get("workload_key"):
        def window(fam):
            labels = [f"w{w}" for w in range(L - 1)] + ["flush"]
            if fam == "k_conventional_step":
                labels = ["conventional"]
            rows = [table.get((fam, lb)) for lb in labels]
            if any(r is None for r in rows):
                raise SystemExit(f"{fam}: not every cursor position was profiled")
            return {k: float(np.mean([r[k] for r in rows])) for k in ("fetch", "write", "total", "algorithmic")}
        rep, conv = window("k_replay_step"), window("k_conventional_step")
        entry = {"kernel_source": kernel_source_hash(),
                 "bytes_per_launch": round(rep["total"]),
                 "basis": "window average: mean over the L cursor positions of the mean per launch",
                 "replay": {"fetch": round(rep["fetch"]), "write": round(rep["write"]),
                            "algorithmic": round(rep["algorithmic"]),
                            "by_cursor": {lb: round(table[("k_replay_step", lb)]["total"])
                                          for lb in [f"w{w}" for w in range(L - 1)] + ["flush"]}},
                 "conventional": {"fetch": round(conv["fetch"]), "write": round(conv["write"]),
                                  "bytes_per_launch": round(conv["total"]), "algorithmic": round(conv["algorithmic"])},
                 "scale": {"fetch": round(scales["fetch"], 4), "write": round(scales["write"], 4)},
                 "calibration_copy_mib": mib}
        data = json.load(open(path)) if os.path.exists(path) else {}
        data[log["workload_key"]] = entry
        with open(path, "w") as fo:
            json.dump(data, fo, indent=1, sort_keys=True)
            fo.write("\n")
        print(json.dumps({log["workload_key"]: entry}))
    return 0


def summarize_trace(trace_csv, launch_log):
    """Kernel durations from a rocprofv3 --kernel-trace csv, lined up with the
    launch log of the same run (dispatches of each kernel in dispatch order
    against its logged launches in launch order).  Prints one JSON line per
    (kernel, label): launches, mean / min / max duration in us, and the
    algorithmic bytes over the summed duration; for the one-line benchmark
    (labels = cursors) also the window average over cursors."""
    import csv
    rows = []
    with open(trace_csv, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Dispatch_Id"]), kernel_family(r["Kernel_Name"]),
                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    log = json.load(open(launch_log))
    disp = {}
    for _, fam, us in rows:
        disp.setdefault(fam, []).append(us)
    logged = {}
    for fam, label, nb, *rest in log["launches"]:
        logged.setdefault(fam, []).append((label, nb, rest[0] if rest else ""))
    table, phases = {}, {}
    for fam, launches in logged.items():
        got = disp.get(fam, [])
        if len(got) != len(launches):
            raise SystemExit(f"{fam}: {len(got)} dispatches in the trace, {len(launches)} launches logged")
        for (label, nb, ph), us in zip(launches, got):
            table.setdefault((fam, label), []).append((us, nb))
            if ph:
                phases.setdefault((fam, ph), []).append((us, nb))
    for (fam, label), v in table.items():
        us = np.array([a for a, _ in v])
        nb = np.array([b for _, b in v])
        print(json.dumps({"kernel": fam, "label": label, "launches": len(v), "us_mean": round(float(us.mean()), 2),
                          "us_min": round(float(us.min()), 2), "us_max": round(float(us.max()), 2),
                          "tbs": round(float(nb.sum() / us.sum() / 1e6), 3)}))
    # the one-line benchmark's timed launches alone (the phase its log records):
    # bench.py's launch_us is their mean plus the gaps between them
    for (fam, ph), v in phases.items():
        if ph == "timed":
            us = np.array([a for a, _ in v])
            nb = np.array([b for _, b in v])
            print(json.dumps({"kernel": fam, "label": "timed launches", "launches": len(v),
                              "us_mean": round(float(us.mean()), 2), "tbs": round(float(nb.sum() / us.sum() / 1e6), 3),
                              "frac_of_8tbs": round(float(nb.sum() / us.sum() / 1e6) / 8.0, 4)}))
    L = log.get("L")
    if L:
        labels = [f"w{w}" for w in range(L - 1)] + ["flush"]
        if all(("k_replay_step", lb) in table for lb in labels):
            means = [float(np.mean([a for a, _ in table[("k_replay_step", lb)]])) for lb in labels]
            nbs = [float(np.mean([b for _, b in table[("k_replay_step", lb)]])) for lb in labels]
            win = float(np.mean(means))
            print(json.dumps({"kernel": "k_replay_step", "label": "window average over cursors",
                              "us": round(win, 2), "non_flush_us": round(float(np.mean(means[:-1])), 2),
                              "flush_us": round(means[-1], 2), "bytes": round(float(np.mean(nbs))),
                              "tbs": round(float(np.mean(nbs)) / win / 1e6, 3),
                              "frac_of_8tbs": round(float(np.mean(nbs)) / win / 1e6 / 8.0, 4)}))
    return 0


def build_parser():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="nemotron", choices=sorted(WORKLOADS))
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--L", type=int, default=None)
    ap.add_argument("--state", default=None, choices=["f32", "f16"])
    ap.add_argument("--read", default=None, choices=["f16", "bf16", "e4m3"],
                    help="two-precision checkpoint (Mamba-2, fp32 state): dtype of the read copy (also for the "
                         "Mamba-2 layers of --suite-only spec)")
    ap.add_argument("--rounding", default="nearest", choices=["nearest", "stochastic"],
                    help="state stores: nearest even, or stochastic rounding (fp16 state)")
    ap.add_argument("--pools", type=int, default=None,
                    help="state pools in rotation (default L + 1; must be 1 mod L)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=None, help="rows in the CPU-baseline sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (scale for rocprofv3 byte counters)")
    ap.add_argument("--suite", metavar="PATH",
                    help="instead of the one-line benchmark, run the Gated DeltaNet batch sweep and the "
                         "40-layer stack and write JSON lines to PATH")
    ap.add_argument("--suite-only", choices=["gdn", "stack", "spec", "continuous"], default=None,
                    help="with --suite: run one part of it")
    ap.add_argument("--spec-T", type=int, action="append", default=None,
                    help="with --suite-only spec: the draft counts to run (default 4 and 8)")
    ap.add_argument("--spec-workload", choices=["nemotron", "nemotron-grouped", "gdn"], action="append", default=None,
                    help="with --suite-only spec: the layers to run (default both)")
    ap.add_argument("--stack-quick", action="store_true",
                    help="with --suite-only stack: only the fp32 conventional and the L = 16 fp32 replay stacks")
    ap.add_argument("--summarize-trace", metavar="TRACE_CSV",
                    help="kernel durations from a rocprofv3 --kernel-trace csv, per launch-log label (needs "
                         "--launch-log of the same run); runs nothing on the GPU")
    ap.add_argument("--launch-log", metavar="PATH",
                    help="write every launch of the library's kernels (kernel, label, algorithmic bytes) in launch "
                         "order to PATH (for --summarize-counters); with --summarize-counters: read it")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) "
                         "into per-launch HBM bytes in profiles/counters.json and print them; runs nothing on the GPU")
    return ap


def main(argv=None):
    args = build_parser().parse_args(argv)
    if args.summarize_counters:
        return summarize_counters(args, *args.summarize_counters)
    if args.summarize_trace:
        if not args.launch_log:
            raise SystemExit("--summarize-trace needs --launch-log PATH")
        return summarize_trace(args.summarize_trace, args.launch_log)
    global _LAUNCH_LOG
    if args.launch_log:
        _LAUNCH_LOG = []
    if args.suite:
        if args.gpus != 1:
            print("the suite runs on one GPU", file=sys.stderr)
            return 2
        if args.calibrate_copy:
            calibrate_copy(args.calibrate_copy)
        with open(args.suite, "w") as out:
            if args.suite_only in (None, "gdn"):
                suite_gdn_sweep(out)
            if args.suite_only in (None, "stack"):
                suite_stack(out, quick=args.stack_quick)
            if args.suite_only in (None, "spec"):
                for wl in args.spec_workload or ["nemotron", "gdn"]:
                    suite_spec(out, workload=wl, Ts=tuple(args.spec_T or (4, 8)),
                               read=args.read if wl != "gdn" else None)
            if args.suite_only in (None, "continuous"):
                suite_continuous(out)
        print(open(args.suite).read(), end="")
        if args.launch_log:
            with open(args.launch_log, "w") as f:
                json.dump({"launches": _LAUNCH_LOG, "suite_key": suite_key(args)}, f)
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the decode step exchanges no data between GPUs, so each "
              f"GPU runs its own rows or heads independently (--gpus {args.gpus} is not supported).",
              file=sys.stderr)
        return 2
    cfg = config_from_args(args)
    pools = args.pools or cfg["L"] + 1
    try:
        cursor_schedule(cfg["L"], pools, args.warmup, args.steps, cursor_bytes(cfg))
    except ValueError as e:
        print(f"bench.py: {e}", file=sys.stderr)
        return 2

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
    rep = run_gpu(cfg, args.steps, args.warmup, pools, "replay")
    conv = run_gpu(cfg, args.steps, args.warmup, pools, "conventional")

    groups = cfg.get("groups", 0)
    wb_r = window_bytes(cfg["form"], cfg["H"], cfg["dv"], cfg["dk"], cfg["B"], cfg["state"], cfg["rec"], cfg["io"], cfg["L"],
                        read=cfg["read"], groups=groups)
    wb_c = window_bytes(cfg["form"], cfg["H"], cfg["dv"], cfg["dk"], cfg["B"], cfg["state"], cfg["rec"], cfg["io"], cfg["L"],
                        "conventional", groups=groups)
    form_name = "mamba2" if cfg["form"] == 0 else "gdn"
    state_desc = f"{cfg['state']} state" + (f" + {cfg['read']} read copy" if cfg["read"] else "")
    state_desc += " (stochastic rounding)" if cfg["sr"] else ""
    keys = f", keys shared by {groups} groups" if groups else ""
    workload = (f"{form_name} layer, {cfg['H']} heads{keys}, d_v={cfg['dv']}, d_k={cfg['dk']}, {state_desc}, "
                f"{cfg['rec']} records, {cfg['io']} q/k/v, batch {cfg['B']}, L={cfg['L']}")
    key = workload_key(args.workload, cfg)
    traffic = load_traffic(key)
    achieved = rep["achieved_gbs"]
    line = {
        "metric": METRIC,
        "value": round(rep["steps_per_s"], 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(rep["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": cfg["B"], "seq_len": None, "heads": cfg["H"],
                   "d_v": cfg["dv"], "d_k": cfg["dk"], "L": cfg["L"], "state_dtype": cfg["state"],
                   "read_copy_dtype": cfg["read"], "state_rounding": args.rounding,
                   "record_dtype": cfg["rec"], "io_dtype": cfg["io"], "state_pools": pools,
                   "key_groups": groups or cfg["H"],
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "k_replay_step", "bytes_per_launch": round(rep["bytes_per_launch_mean"]),
                     "window_bytes_per_launch": round(rep["window_bytes_per_launch"]),
                     "basis": "timed launches: floor(K/L) whole windows plus K mod L consecutive cursors; "
                              "traffic: window average over the L cursors (rocprofv3 counters)",
                     "launch_us": round(1e3 * rep["kernel_ms_mean"], 2)},
        "replay": {"steps_per_s": round(rep["steps_per_s"], 2), "kernel_us": round(1e3 * rep["kernel_ms_mean"], 2),
                   "kernel_steps_per_s": round(1e3 / rep["kernel_ms_mean"], 2),
                   "achieved_tbs": round(achieved / 1e3, 3), "pct_peak": round(100 * achieved / HBM_PEAK_GBS, 1),
                   "timed_cursor_counts": rep["timed_cursor_counts"],
                   "first_timed_cursor": rep["first_timed_cursor"],
                   "us_by_cursor": rep["by_position_us"],
                   "window_us_from_cursors": window_us(rep["by_position_us"], cfg["L"])},
        "conventional": {"steps_per_s": round(conv["steps_per_s"], 2), "kernel_us": round(1e3 * conv["kernel_ms_mean"], 2),
                         "kernel_steps_per_s": round(1e3 / conv["kernel_ms_mean"], 2),
                         "achieved_tbs": round(conv["achieved_gbs"] / 1e3, 3),
                         "pct_peak": round(100 * conv["achieved_gbs"] / HBM_PEAK_GBS, 1)},
        "speedup_replay_vs_conventional": round(conv["kernel_ms_mean"] / rep["kernel_ms_mean"], 3),
        "speedup_wall": round(rep["steps_per_s"] / conv["steps_per_s"], 3),
        "algorithmic_bytes_ratio": round(wb_r / wb_c, 4),
        "kernel_source": kernel_source_hash(),
    }
    if args.launch_log:
        with open(args.launch_log, "w") as f:
            json.dump({"launches": _LAUNCH_LOG, "L": cfg["L"], "workload_key": key}, f)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, rows=args.cpu_rows)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
