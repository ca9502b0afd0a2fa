"""Drive the HIP path and the fp64 oracle side by side on the same inputs.

Used by the GPU parity tests and the smoke check.  Everything the GPU
computes goes through the C ABI (via the package's DecodeLayer); the oracle
runs on the CPU in float64 on the sampled rows.

Error metric (per (step, row, head) tile): max_i |got_i - ref_i| / max_i |ref_i|,
the gate being the maximum over all compared tiles.  Flushed checkpoints and
conventional states are compared the same way per (row, head).
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field

import numpy as np
import torch

import linear_attention_decode_replay_amd as rs
import oracle
from oracle import formats as oracle_formats
import workloads
from linear_attention_decode_replay_amd.state import DecodeLayer

TOL_F32 = 1e-4   # fp32 state and fp32 records
TOL_LOW = 2e-2   # fp16/bf16 records or checkpoint


def tolerance(state_dt, rec_dt, io_dt=None):
    """The gate for a layer's state and record dtypes: 1e-4 with an fp32
    state and fp32 records, 2e-2 with fp16/bf16 records or checkpoint.  The
    io dtype does not enter: the oracle is given the same (bf16/fp16-valued)
    inputs as the kernels."""
    return TOL_F32 if (state_dt, rec_dt) == ("f32", "f32") else TOL_LOW


def rel_err(got: np.ndarray, ref: np.ndarray, tile_dims: int = 1) -> float:
    """Worst per-tile relative error; a tile is the trailing `tile_dims` axes."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    n = int(np.prod(ref.shape[-tile_dims:]))
    g = got.reshape(-1, n)
    r = ref.reshape(-1, n)
    den = np.abs(r).max(-1)
    num = np.abs(g - r).max(-1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max()) if num.size else 0.0


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Case:
    form: int = rs.MAMBA2
    B: int = 2
    H: int = 4
    dv: int = 16
    dk: int = 32
    L: int = 4
    steps: int = 64
    state_dt: str = "f32"
    rec_dt: str = "f32"
    io_dt: str = "f32"
    seed: int = 0
    a_lo: float = 1.0
    a_hi: float = 8.0
    sample: list | None = None       # rows checked against the oracle (None: all)
    pad_rows: list = field(default_factory=list)
    n_blocks: int | None = None      # pool size (default B + 3: spare blocks)
    strided: bool = False            # q/k/v as strided views of wider buffers
    check_conventional: bool = True
    force_every: int = 0             # > 0: force a flush on row 0 every n steps
    read_dt: str | None = None       # two-precision checkpoint: read copy dtype
    groups: int = 0                  # key groups (0: a key and query per head)
    reconstruct: bool = False        # Gated DeltaNet: the state-reconstruction route
    flush_hints: bool = True         # pass the host's flush hint (False: RS_FLUSH_UNKNOWN)
    forget_every: int = 0            # > 0: every n-th (step, row, head) has lam = -inf (alpha = 0)
    join: bool = False               # replay rows join with a zero checkpoint (join_rows) instead of a reset

    def name(self):
        f = "gdn" if self.form == rs.GDN else "mamba2"
        return (f"{f} B={self.B} H={self.H} {self.dv}x{self.dk} L={self.L} steps={self.steps} "
                f"state={self.state_dt} rec={self.rec_dt} io={self.io_dt} read={self.read_dt} "
                f"strided={self.strided} pad={self.pad_rows} groups={self.groups} "
                f"route={'reconstruct' if self.reconstruct else 'output-only'} hints={self.flush_hints} "
                f"forget_every={self.forget_every} join={self.join} seed={self.seed}")


def full_forgetting(lam: torch.Tensor, every: int, step: int) -> None:
    """Set every `every`-th log-decay of this step to -inf (alpha = 0, a
    legal decay: the blog's weights are products of the alphas), counting
    over (step, row, ...) in row-major order, in place."""
    if every > 0:
        n = lam.numel()
        idx = torch.arange(n).reshape(lam.shape) + step * n
        lam[(idx % every) == 0] = float("-inf")


def grouped(tok, hg: int):
    """Tokens of a layer whose keys and queries are shared by groups of hg
    heads: the group takes the key and query drawn for its first head, and
    every head of the group sees them (what the oracle, which works per head,
    is given).  Returns (per-head tokens, group q [B, G, dk], group k)."""
    if hg == 1:
        return tok, tok.q, tok.k
    qg, kg = tok.q[:, ::hg].contiguous(), tok.k[:, ::hg].contiguous()
    full = workloads.Tokens(qg.repeat_interleave(hg, dim=1), kg.repeat_interleave(hg, dim=1), tok.v, tok.lam,
                            tok.beta)
    return full, qg, kg


def _device_tokens(tok, strided: bool, dev, qk=None):
    q_in, k_in = qk if qk is not None else (tok.q, tok.k)
    if not strided:
        return q_in.to(dev), k_in.to(dev), tok.v.to(dev)
    out = []
    for t in (q_in, k_in, tok.v):
        B, H, d = t.shape
        wide = torch.full((B, H + 1, d + 8), float("nan"), dtype=t.dtype, device=dev)
        view = wide[:, 1:, 8:]
        view.copy_(t.to(dev))
        out.append(view)
    return tuple(out)


def run_case(c: Case, dev="cuda") -> dict:
    """Run c.steps decode steps through both GPU kernels and the oracle.

    Returns the worst errors seen; raises AssertionError on any bit-exact
    mismatch (cursor, flush flag, copied record fields, untouched pad rows)."""
    say(f"[case] {c.name()}")
    lay = rs.layer(c.form, c.H, c.dv, c.dk, c.L, c.state_dt, c.rec_dt, c.io_dt, c.read_dt, 0, c.groups,
                   reconstruct=c.reconstruct)
    hg = c.H // c.groups if c.groups else 1
    n_blocks = c.n_blocks or (c.B + 3)
    rep = DecodeLayer(lay, c.B, n_blocks, dev)
    rep.flush_hints = c.flush_hints
    conv = DecodeLayer(lay, c.B, n_blocks, dev) if c.check_conventional else None
    for d in (rep, conv):
        if d is not None:
            d.pool.raw.fill_(0xFF)   # NaN in every dtype: reading an unwritten slot shows up
    blocks = workloads.shuffled_blocks(c.seed, c.B, n_blocks)
    live_rows = [b for b in range(c.B) if b not in c.pad_rows]
    for d in (rep, conv):
        if d is None:
            continue
        for b in live_rows:
            d.assign(b, int(blocks[b]))
        if c.join and d is rep:
            d.join_rows(live_rows)   # the checkpoints stay NaN-filled: never used until written
        else:
            d.reset_rows(live_rows)
    sample = [b for b in (c.sample if c.sample is not None else range(c.B)) if b in live_rows]
    ns = len(sample)
    ref = oracle.ConventionalModel(c.form, ns, c.H, c.dv, c.dk)
    # a two-precision checkpoint is compared with the oracle's two-copy model
    ref_two = oracle.TwoCopyReplayModel(ns, c.H, c.dv, c.dk, c.L, c.read_dt) if c.read_dt else None
    orc = oracle.get()
    forced = np.zeros(c.steps, np.uint8)
    if c.force_every:
        forced[c.force_every - 1::c.force_every] = 1
    want_w, want_f = orc.cursor_run(c.L, 0, c.steps, forced)
    rdt = workloads.torch_dtype(c.rec_dt)
    err = {"out_replay": 0.0, "out_conv": 0.0, "ckpt_flush": 0.0, "state_conv": 0.0, "ring_x": 0.0,
           "out_replay_step": 0.0, "out_replay_vs_exact": 0.0, "flushes": 0}
    for s in range(c.steps):
        tok = workloads.tokens(c.form, c.seed, s, c.B, c.H, c.dv, c.dk, c.io_dt, c.a_lo, c.a_hi)
        full_forgetting(tok.lam, c.forget_every, s)
        tok, qg, kg = grouped(tok, hg)
        q, k, v = _device_tokens(tok, c.strided, dev, (qg, kg))
        lam = tok.lam.to(dev)
        beta = tok.beta.to(dev) if tok.beta is not None else None
        out_r = torch.full((c.B, c.H, c.dv), float("nan"), device=dev)
        force = np.zeros(c.B, np.uint8)
        force[0] = forced[s]
        wp, fl = rep.step(rs.make_io(q, k, v, lam, out_r, beta), force)
        if conv is not None:
            out_c = torch.full((c.B, c.H, c.dv), float("nan"), device=dev)
            conv.conventional_step(rs.make_io(q, k, v, lam, out_c, beta))
        # host metadata is bit-exact against the oracle's cursor, and the
        # cursors the kernel wrote for the next step equal the host's
        assert wp[0] == want_w[s] and bool(fl[0]) == bool(want_f[s]), (s, wp[0], fl[0])
        nxt = rep.device_cursor()
        lv = rep.live()
        assert np.array_equal(nxt[lv], rep.anchor[lv] % c.L), f"device cursor, step {s}"
        # the zero-checkpoint flag the device carries equals the host's
        zbit = (rep.device_cursor(words=True) & rs.RS_CURSOR_ZERO_CKPT) != 0
        assert np.array_equal(zbit[lv], rep.zero_ckpt[lv]), f"zero-checkpoint flags, step {s}"
        for b in live_rows[1:]:
            assert wp[b] == s % c.L and bool(fl[b]) == (s % c.L == c.L - 1), (s, b)
        for b in c.pad_rows:
            assert wp[b] == 0 and fl[b] == 0
        o_ref, x_ref = ref.step(tok.q[sample].double().numpy(), tok.k[sample].double().numpy(),
                                tok.v[sample].double().numpy(), tok.lam[sample].double().numpy(),
                                None if tok.beta is None else tok.beta[sample].double().numpy(),
                                want_x=True)
        torch.cuda.synchronize()
        got_r = out_r[sample].double().cpu().numpy()
        if ref_two is not None:
            q64, lam64 = tok.q[sample].double().numpy(), tok.lam[sample].double().numpy()
            # blog, "The precision argument, derived": a non-flush output is off
            # by gamma_h eps q, eps one rounding of the last checkpoint, so
            # |o - o_exact| <= gamma_h sum_c u_c |q_c| (u: half an ulp in the
            # read format).  Twice that: the kernel rounds the fp32 recurrence
            # copy, whose values (and hence an E4M3 row's scale) may sit one
            # rounding boundary away from the exact ones; plus the fp32
            # tolerance (TOL_F32 of the tile's largest output) for the rest of
            # the step's arithmetic.
            bound = ref_two.read_error_bound(q64, lam64)
            o_two = ref_two.step(q64, tok.k[sample].double().numpy(), tok.v[sample].double().numpy(), lam64,
                                 np.asarray(fl)[sample].astype(bool))
            tile_max = np.abs(o_ref).max(axis=-1, keepdims=True)
            excess = np.abs(got_r - o_ref) - (2 * bound + TOL_F32 * tile_max)
            err["read_bound_excess"] = max(err.get("read_bound_excess", -np.inf), float(excess.max()))
            err["out_replay_vs_exact"] = max(err["out_replay_vs_exact"], rel_err(got_r, o_ref))
            o_ref_replay = o_two
        else:
            o_ref_replay = o_ref
        err["out_replay"] = max(err["out_replay"], rel_err(got_r, o_ref_replay))
        # the same, normalised by the whole step's output instead of each tile's
        err["out_replay_step"] = max(err["out_replay_step"],
                                     float(np.abs(got_r - o_ref_replay).max() / max(np.abs(o_ref_replay).max(), 1e-300)))
        if conv is not None:
            got_c = out_c[sample].double().cpu().numpy()
            err["out_conv"] = max(err["out_conv"], rel_err(got_c, o_ref))
        for b in c.pad_rows:  # padding rows are neither read nor written
            assert torch.isnan(out_r[b]).all()
        # records appended by non-flush rows: copied fields are bit-exact
        blk = torch.as_tensor(blocks[sample], device=dev, dtype=torch.long)
        nonflush = [i for i, b in enumerate(sample) if not fl[b]]
        if nonflush:
            rows = [sample[i] for i in nonflush]
            bsel = blk[nonflush]
            slots = torch.as_tensor(wp[rows].astype(np.int64), device=dev)
            got_k = rep.pool.rec_k()[bsel, :, slots].cpu()   # one key record per group
            assert torch.equal(got_k, kg[rows].to(rdt)), f"k record, step {s}"
            got_l = rep.pool.rec_lam()[bsel, :, slots].cpu()
            assert torch.equal(got_l, tok.lam[rows]), f"lam record, step {s}"
            got_x = rep.pool.rec_x()[bsel, :, slots].cpu()
            if c.form == rs.MAMBA2:
                assert torch.equal(got_x, tok.v[rows].to(rdt)), f"v record, step {s}"
            else:
                err["ring_x"] = max(err["ring_x"], rel_err(got_x.double().numpy(), x_ref[nonflush]))
        flushed = [i for i, b in enumerate(sample) if fl[b]]
        if flushed:
            err["flushes"] += 1
            ckt = rep.pool.ckpt()[blk[flushed]]
            ck = ckt.double().cpu().numpy()
            err["ckpt_flush"] = max(err["ckpt_flush"], rel_err(ck, ref.state()[flushed], 2))
            if c.read_dt == "e4m3":
                # codes and row scales: the oracle's E4M3 encoding of the
                # kernel's own fp32 recurrence copy, bit for bit
                lo = rep.pool.ckpt_lo()[blk[flushed]].cpu().numpy()
                sc = rep.pool.ckpt_scale()[blk[flushed]].cpu().numpy()
                codes, e = oracle_formats.e4m3_quantize_rows(ckt.cpu().double().numpy())
                codes = codes[..., rep.pool.ckpt_lo_columns()]  # stored in lane order
                assert np.array_equal(lo, codes), f"E4M3 codes, step {s}: {np.sum(lo != codes)} differ"
                assert np.array_equal(sc, np.ldexp(1.0, e).astype(np.float32)), f"E4M3 scales, step {s}"
            elif c.read_dt:  # the read copy is the RNE cast of the same values, bit for bit
                lo = rep.pool.ckpt_lo()[blk[flushed]].cpu()
                cols = torch.as_tensor(rep.pool.ckpt_lo_columns())  # stored in lane order
                want = ckt.cpu()[..., cols].to(workloads.torch_dtype(c.read_dt))
                assert torch.equal(lo, want), f"read copy, step {s}"
        if conv is not None and (s % 8 == 7 or s == c.steps - 1):
            st = conv.pool.ckpt()[blk].double().cpu().numpy()
            err["state_conv"] = max(err["state_conv"], rel_err(st, ref.state(), 2))
    assert int(rep.err.item()) == 0 and (conv is None or int(conv.err.item()) == 0)
    say(f"[errors] {c.name()}: " + ", ".join(f"{k}={v:.3g}" for k, v in err.items()))
    return err


def assert_within(err: dict, tol: float) -> None:
    for k in ("out_replay", "out_conv", "ckpt_flush", "state_conv", "ring_x"):
        assert err[k] <= tol, f"{k} = {err[k]:.3g} > {tol}"
