"""Drive the speculative verify path (HIP, through the C ABI) and the fp64
oracle side by side on the same inputs.

Every step checks, on the sampled rows: the committed counts and flags the
device holds for the step against the host mirror (bit-exact); the T outputs
against the oracle's verify route and against running the drafts token by
token (tolerance); checkpoints written by flushing rows against the
committed state (tolerance); the drafts stored as records (bit-exact copies
of the inputs, cast to nearest even); padding rows untouched.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import linear_attention_decode_replay_amd as rs
import oracle
import workloads
from gpu_harness import full_forgetting, rel_err, say
from oracle import formats as oracle_formats
from linear_attention_decode_replay_amd.state import SpecDecodeLayer


@dataclass
class SpecCase:
    form: int = rs.MAMBA2
    B: int = 2
    H: int = 4
    dv: int = 16
    dk: int = 32
    L: int = 8
    T: int = 4
    steps: int = 40
    state_dt: str = "f32"
    rec_dt: str = "f32"
    io_dt: str = "f32"
    seed: int = 0
    a_lo: float = 0.05
    a_hi: float = 1.0
    accept: str = "random"           # accepted counts: random / all / one / none
    sample: list | None = None       # rows checked against the oracle (None: all)
    pad_rows: list = field(default_factory=list)
    strided: bool = False            # q/k/v as strided views of wider buffers
    force_row0_every: int = 0        # > 0: force a flush on row 0 every n steps
    forget_every: int = 0            # > 0: every n-th (step, row, draft, head) has lam = -inf
    groups: int = 0                  # key groups (0: a key and query per head)
    read_dt: str | None = None       # two-precision checkpoint: read copy dtype (fp32 recurrence copy)

    def name(self):
        f = "gdn" if self.form == rs.GDN else "mamba2"
        return (f"spec {f} B={self.B} H={self.H} {self.dv}x{self.dk} L={self.L} T={self.T} steps={self.steps} "
                f"state={self.state_dt} rec={self.rec_dt} io={self.io_dt} accept={self.accept} "
                f"strided={self.strided} pad={self.pad_rows} forget_every={self.forget_every} groups={self.groups} "
                f"read={self.read_dt} seed={self.seed}")


def _device(t: torch.Tensor, strided: bool, dev):
    if not strided:
        return t.to(dev)
    B, T, H, d = t.shape
    wide = torch.full((B, T + 1, H + 2, d + 8), float("nan"), dtype=t.dtype, device=dev)
    view = wide[:, 1:, 2:, 8:]
    view.copy_(t.to(dev))
    return view


def run_spec_case(c: SpecCase, dev="cuda") -> dict:
    say(f"[case] {c.name()}")
    lay = rs.layer(c.form, c.H, c.dv, c.dk, c.L, c.state_dt, c.rec_dt, c.io_dt, c.read_dt, c.T, c.groups)
    hg = c.H // c.groups if c.groups else 1  # heads per key group
    n_blocks = c.B + 3
    d = SpecDecodeLayer(lay, c.B, n_blocks, dev)
    d.pool.raw.fill_(0xFF)  # NaN in every dtype: a slot read before it is written shows up
    blocks = workloads.shuffled_blocks(c.seed, c.B, n_blocks)
    live = [b for b in range(c.B) if b not in c.pad_rows]
    for b in live:
        d.assign(b, int(blocks[b]))
    d.upload(rows=live)
    sample = [b for b in (c.sample if c.sample is not None else range(c.B)) if b in live]
    ns = len(sample)
    if c.read_dt:
        spec = oracle.SpecTwoCopyModel(ns, c.H, c.dv, c.dk, c.L, c.T, c.read_dt)
        cols = d.pool.ckpt_lo_columns()  # the read copy keeps each row in lane order
    else:
        spec = oracle.SpecReplayModel(ns, c.H, c.dv, c.dk, c.L, c.T, form=c.form)
    ref = oracle.SpecTokenByToken(ns, c.H, c.dv, c.dk, c.T, form=c.form)
    h = np.full(c.B, -1, np.int32)
    h[live] = 0
    rdt = workloads.torch_dtype(c.rec_dt)
    err = {"out_spec": 0.0, "out_vs_tokens": 0.0, "ckpt_flush": 0.0, "rec_u": 0.0, "flushes": 0, "accepted": 0}
    for s in range(c.steps):
        tok = workloads.spec_tokens(c.seed, s, c.B, c.H, c.T, c.dv, c.dk, c.io_dt, c.a_lo, c.a_hi, c.form)
        full_forgetting(tok.lam, c.forget_every, s)
        # grouped keys: the device takes one q and k per group (its first
        # head's draw), the oracle every head's copy of its group's
        qg, kg = tok.q[:, :, ::hg].contiguous(), tok.k[:, :, ::hg].contiguous()
        tok.q, tok.k = qg.repeat_interleave(hg, dim=2), kg.repeat_interleave(hg, dim=2)
        force = np.zeros(c.B, np.uint8)
        if c.force_row0_every and (s + 1) % c.force_row0_every == 0 and 0 in live:
            force[0] = 1
        fl = rs.rs_spec_meta_step(c.L, c.T, h, force)
        if force.any():  # a forced flag is the caller's to set on the device
            d.flag[d._cur][:c.B].copy_(torch.from_numpy(fl.copy()).to(dev))
        # the device holds exactly the host mirror's counts and flags
        dh, dflag = d.device_committed()
        assert np.array_equal(dh[live], h[live]), f"device committed counts, step {s}"
        assert np.array_equal(dflag[live].astype(bool), fl[live].astype(bool)), f"device flags, step {s}"
        q, k, v = (_device(t, c.strided, dev) for t in (qg, kg, tok.v))
        lam = tok.lam.to(dev)
        beta = tok.beta.to(dev) if tok.beta is not None else None
        out = torch.full((c.B, c.T, c.H, c.dv), float("nan"), device=dev)
        d.verify(rs.make_spec_io(q, k, v, lam, out, beta))
        # oracle routes on the sampled rows, tile-major [rows, H, T, d]
        tm = lambda t: t[sample].double().numpy().transpose(0, 2, 1, 3)
        q64, k64, v64 = tm(tok.q), tm(tok.k), tm(tok.v)
        lam64 = tok.lam[sample].double().numpy().transpose(0, 2, 1)
        beta64 = None if tok.beta is None else tok.beta[sample].double().numpy().transpose(0, 2, 1)
        flr = fl[sample].astype(bool)
        o_spec = spec.verify(q64, k64, v64, lam64, flr, beta=beta64)
        o_tok = ref.verify(q64, k64, v64, lam64, beta64)
        torch.cuda.synchronize()
        got = out[sample].double().cpu().numpy().transpose(0, 2, 1, 3)
        err["out_spec"] = max(err["out_spec"], rel_err(got, o_spec))
        err["out_vs_tokens"] = max(err["out_vs_tokens"], rel_err(got, o_tok))
        for b in c.pad_rows:
            assert torch.isnan(out[b]).all(), f"padding row {b} written, step {s}"
        blk = torch.as_tensor(blocks[sample], device=dev, dtype=torch.long)
        # drafts stored as records from slot (flushed ? 0 : h); with grouped
        # keys, a flushing row's keys from the staging slot L until the commit
        base = np.where(fl[sample] != 0, 0, h[sample])
        kbase = np.where(fl[sample] != 0, c.L, h[sample]) if hg > 1 else base
        for i_row, b in enumerate(sample):
            sl = torch.arange(int(base[i_row]), int(base[i_row]) + c.T, device=dev)
            ksl = torch.arange(int(kbase[i_row]), int(kbase[i_row]) + c.T, device=dev)
            got_k = d.pool.rec_k()[blk[i_row], :, ksl].cpu()         # [G, T, dk]
            assert torch.equal(got_k, kg[b].transpose(0, 1).to(rdt)), f"k records, row {b}, step {s}"
            got_v = d.pool.rec_x()[blk[i_row], :, sl].cpu()
            if c.form == rs.MAMBA2:
                assert torch.equal(got_v, tok.v[b].transpose(0, 1).to(rdt)), f"v records, row {b}, step {s}"
            else:  # the drafts' corrected values, against running them token by token
                err["rec_u"] = max(err["rec_u"], rel_err(got_v.double().numpy(), ref.drafts_x[i_row]))
            got_l = d.pool.rec_lam()[blk[i_row], :, sl].cpu()
            assert torch.equal(got_l, tok.lam[b].transpose(0, 1)), f"lam records, row {b}, step {s}"
        flushed = [i for i, b in enumerate(sample) if fl[b]]
        if flushed:
            err["flushes"] += len(flushed)
            ckt = d.pool.ckpt()[blk[flushed]]
            ck = ckt.double().cpu().numpy()
            err["ckpt_flush"] = max(err["ckpt_flush"], rel_err(ck, ref.state()[flushed], 2))
            if c.read_dt:
                # the read copy is the cast of the kernel's own fp32 fold, bit
                # for bit; the oracle then reads the device's read copy (its
                # own, cast from the fp64 fold, may sit one rounding away)
                lo = d.pool.ckpt_lo()[blk[flushed]].cpu()
                if c.read_dt == "e4m3":
                    sc = d.pool.ckpt_scale()[blk[flushed]].cpu().numpy()
                    codes, e = oracle_formats.e4m3_quantize_rows(ck)
                    assert np.array_equal(lo.numpy(), codes[..., cols]), f"E4M3 codes, step {s}"
                    assert np.array_equal(sc, np.ldexp(1.0, e).astype(np.float32)), f"E4M3 scales, step {s}"
                    got = oracle_formats.e4m3_dequantize_rows(lo.numpy(), np.log2(sc).astype(np.int64))
                else:
                    want = ckt.cpu()[..., torch.as_tensor(cols)].to(workloads.torch_dtype(c.read_dt))
                    assert torch.equal(lo, want), f"read copy, step {s}"
                    got = lo.double().numpy()
                nat = np.empty_like(got)
                nat[..., cols] = got
                C_lo = spec.C_lo.reshape(ns, c.H, c.dv, c.dk)
                C_lo[flushed] = nat
                err["read_resync"] = max(err.get("read_resync", 0.0),
                                         rel_err(nat, oracle.round_to(ref.state()[flushed], c.read_dt), 2))
        a = workloads.spec_accepted(c.seed, s, c.B, c.T, c.accept)
        a[c.pad_rows] = 0
        d.commit(torch.from_numpy(a).to(dev))
        if hg > 1:  # the commit moved a flushed row's accepted keys to slots 0 .. a - 1
            for i_row, b in enumerate(sample):
                if fl[b] and a[b]:
                    got_k = d.pool.rec_k()[blk[i_row], :, :int(a[b])].cpu()
                    assert torch.equal(got_k, kg[b, :int(a[b])].transpose(0, 1).to(rdt)), \
                        f"committed keys of flushed row {b}, step {s}"
        spec.commit(a[sample])
        ref.commit(a[sample])
        rs.rs_spec_meta_advance(c.L, c.T, h, fl, a)
        err["accepted"] += int(a[live].sum())
    dh, dflag = d.device_committed()
    assert np.array_equal(dh[live], h[live]), "device committed counts after the last commit"
    assert int(d.err.item()) == 0, f"{int(d.err.item())} tiles or rows flagged by the kernels' checks"
    say(f"[errors] {c.name()}: " + ", ".join(f"{k}={v:.3g}" for k, v in err.items()))
    return err
