"""Stochastic rounding of an fp16 checkpoint / state on the GPU (through the
C ABI) against the oracle.

Exact-arithmetic cases (dyadic inputs, alpha = 1): the kernel's fp32 sums
equal the oracle's fp64 ones, so every stored fp16 value must equal the
oracle's stochastic rounding with the same Philox words, bit for bit.

Generic cases (random inputs, real decays): before each store the oracle is
given the GPU's last stored state, so each comparison covers one store.  The
stored value must be one of the two fp16 neighbours of the oracle's fp64
value (widened by the fp32 arithmetic's error), the same neighbour the
oracle's own rounding picks for all but a small fraction (values whose fp32
and fp64 sums fall on different sides of the random threshold), and unbiased
over the millions of values stored.
"""
import numpy as np
import pytest
import torch

import linear_attention_decode_replay_amd as rs
import oracle
import workloads
from oracle import formats
from gpu_harness import TOL_F32, TOL_LOW, rel_err, say
from linear_attention_decode_replay_amd.state import DecodeLayer, SpecDecodeLayer

pytestmark = pytest.mark.gpu

KEY = (0x243F6A8885A308D3, 0x13198A2E03707344)


def _f16_ulp(x):
    """Spacing of fp16 values at |x| (subnormal spacing below 2^-14)."""
    e = np.frexp(np.abs(x))[1] - 1
    return np.ldexp(1.0, np.maximum(e, -14) - 10)


class StoreStats:
    """Compares stored fp16 values with the oracle's fp64 values before
    rounding and with the oracle's stochastic rounding of them."""

    def __init__(self):
        self.n = 0
        self.differ = 0
        self.bias_sum = 0.0
        self.not_rne = 0

    def add(self, got, exact, rounded):
        """Arrays [tiles, d_v, d_k]."""
        got, exact, rounded = (np.asarray(a, np.float64) for a in (got, exact, rounded))
        # one of the two neighbours: within one fp16 spacing, plus the fp32
        # sums' error (which can move a value across an fp16 grid point; it
        # scales with the terms summed, bounded here by the tile's largest
        # value)
        slack = _f16_ulp(exact) + 1e-5 * np.abs(exact).max(axis=(1, 2), keepdims=True) + 1e-30
        got, exact, rounded, slack = (a.reshape(-1) for a in (got, exact, rounded, slack * np.ones_like(exact)))
        ulp = _f16_ulp(exact)
        assert np.all(np.abs(got - exact) <= slack), f"{np.sum(np.abs(got - exact) > slack)} values off by > 1 ulp"
        self.n += got.size
        self.differ += int(np.sum(got != rounded))
        self.bias_sum += float(np.sum((got - exact) / ulp))
        self.not_rne += int(np.sum(got != exact.astype(np.float16).astype(np.float64)))

    def check(self, label):
        frac, bias, nr = self.differ / self.n, self.bias_sum / self.n, self.not_rne / self.n
        say(f"[sr] {label}: {self.n} values, {frac:.2e} differ from the oracle's rounding, "
            f"mean error {bias:+.2e} ulp, {nr:.3f} differ from nearest-even")
        assert frac < 1e-2, frac   # unrelated random words would disagree on about 1/3
        assert abs(bias) < 3.0 / np.sqrt(self.n) + 1e-3, bias
        assert nr > 0.1, nr   # rounding is stochastic: not nearest-even


def _run(B, H, dv, dk, L, steps, seed, exact, io_dt="bf16", rec_dt="f16", sample=None, token_less_at=None):
    tag = (f"B={B} H={H} {dv}x{dk} L={L} steps={steps} io={io_dt} rec={rec_dt} exact={exact} "
           f"sample={sample} seed={seed}")
    say(f"[case] stochastic rounding {tag}")
    lay = rs.layer(rs.MAMBA2, H, dv, dk, L, "f16", rec_dt, io_dt, None, stochastic=True)
    n_blocks = B + 3
    rep = DecodeLayer(lay, B, n_blocks, "cuda", sr_key=KEY)
    conv = DecodeLayer(lay, B, n_blocks, "cuda", sr_key=KEY)
    blocks = workloads.shuffled_blocks(seed, B, n_blocks)
    for d in (rep, conv):
        d.pool.raw.fill_(0xFF)
        for b in range(B):
            d.assign(b, int(blocks[b]))
        d.reset_rows(range(B))
    sample = list(range(B)) if sample is None else sample
    ns = len(sample)
    tiles = np.array([b * H + h for b in sample for h in range(H)])
    sr_rep = oracle.SRReplayModel(rs.MAMBA2, ns, H, dv, dk, L, KEY, tiles)
    sr_conv = oracle.SRConventionalModel(rs.MAMBA2, ns, H, dv, dk, KEY, tiles)
    blk = torch.as_tensor(blocks[sample], device="cuda", dtype=torch.long)
    st_rep, st_conv = StoreStats(), StoreStats()
    err = {"out_replay": 0.0, "out_conv": 0.0, "flushes": 0}
    for s in range(steps):
        if exact:
            tok = workloads.dyadic_tokens(seed, s, B, H, dv, dk, io_dt)
        else:
            tok = workloads.mamba2_tokens(seed, s, B, H, dv, dk, io_dt)
        q, k, v, lam = (t.to("cuda") for t in (tok.q, tok.k, tok.v, tok.lam))
        out_r = torch.empty(B, H, dv, device="cuda")
        out_c = torch.empty(B, H, dv, device="cuda")
        step_r, step_c = rep.sr_step, conv.sr_step
        _, fl = rep.step(rs.make_io(q, k, v, lam, out_r))
        conv.conventional_step(rs.make_io(q, k, v, lam, out_c))
        a64 = [t[sample].double().numpy() for t in (tok.q, tok.k, tok.v, tok.lam)]
        flr = np.asarray(fl)[sample].astype(bool)
        if not exact:  # the oracle state before this store, unrounded
            pre = oracle.ReplayModel(rs.MAMBA2, ns, H, dv, dk, L)
            pre.C, pre.rec_lam, pre.rec_x, pre.rec_k, pre.w = (sr_rep.C.copy(), sr_rep.rec_lam.copy(),
                                                             sr_rep.rec_x.copy(), sr_rep.rec_k.copy(),
                                                             sr_rep.w.copy())
            pre.step(*a64, flr)
            pre_c = oracle.ConventionalModel(rs.MAMBA2, ns, H, dv, dk, sr_conv.S.reshape(ns, H, dv, dk).copy())
            pre_c.step(*a64)
        o_r = sr_rep.step(*a64, flr, sr_step=step_r)
        o_c, _ = sr_conv.step(*a64, want_x=True, sr_step=step_c)
        torch.cuda.synchronize()
        tol = TOL_F32 if exact else TOL_LOW
        err["out_replay"] = max(err["out_replay"], rel_err(out_r[sample].double().cpu().numpy(), o_r))
        err["out_conv"] = max(err["out_conv"], rel_err(out_c[sample].double().cpu().numpy(), o_c))
        assert err["out_replay"] <= tol and err["out_conv"] <= tol, (s, err)
        got_c = conv.pool.ckpt()[blk].double().cpu().numpy().reshape(ns * H, dv, dk)
        if exact:
            assert np.array_equal(got_c, sr_conv.S), f"conventional state, step {s}: " \
                f"{np.sum(got_c != sr_conv.S)} values differ"
        else:
            st_conv.add(got_c, pre_c.S, sr_conv.S)
            sr_conv.S[:] = got_c   # continue from the GPU's state
        fl_t = np.repeat(flr, H)
        if fl_t.any():
            err["flushes"] += 1
            got_r = rep.pool.ckpt()[blk].double().cpu().numpy().reshape(ns * H, dv, dk)[fl_t]
            if exact:
                assert np.array_equal(got_r, sr_rep.C[fl_t]), f"flushed checkpoint, step {s}: " \
                    f"{np.sum(got_r != sr_rep.C[fl_t])} values differ"
            else:
                st_rep.add(got_r, pre.C[fl_t], sr_rep.C[fl_t])
                sr_rep.C[fl_t] = got_r
        if token_less_at is not None and s == token_less_at:
            step_f = rep.sr_step
            rep.flush_rows(range(B))
            sr_rep.fold(np.isin(np.arange(ns), range(ns)), sr_step=step_f)
            torch.cuda.synchronize()
            got_f = rep.pool.ckpt()[blk].double().cpu().numpy().reshape(ns * H, dv, dk)
            assert np.array_equal(got_f, sr_rep.C), f"token-less flush: {np.sum(got_f != sr_rep.C)} values differ"
    assert int(rep.err.item()) == 0 and int(conv.err.item()) == 0
    if not exact:
        st_rep.check(f"replay flushes, {tag}")
        st_conv.check(f"conventional steps, {tag}")
    say(f"[errors] stochastic rounding {tag}: " + ", ".join(f"{k}={v:.3g}" for k, v in err.items()))
    return err


@pytest.mark.parametrize("L", [1, 4, 8])
def test_sr_exact_bit_for_bit(L):
    """Dyadic inputs: flushed checkpoints and conventional states equal the
    oracle's stochastic rounding bit for bit (L = 1: every step flushes)."""
    err = _run(B=3, H=4, dv=16, dk=32, L=L, steps=3 * L + 2, seed=L, exact=True)
    assert err["flushes"] >= 2


def test_sr_exact_token_less_flush_and_fp32_records():
    """The token-less flush rounds the same way; fp32 records and io."""
    _run(B=2, H=2, dv=16, dk=32, L=6, steps=9, seed=5, exact=True, io_dt="f32", rec_dt="f32",
         token_less_at=3)


def test_sr_exact_nemotron_shape():
    """Nemotron-3-Super layer shape (128 heads, 64 x 128), 2 of 16 rows
    checked; the counter's tile word is row * 128 + head."""
    _run(B=16, H=128, dv=64, dk=128, L=4, steps=9, seed=9, exact=True, sample=[3, 14])


def test_sr_generic_inputs():
    """Random inputs and decays: the stored neighbour agrees with the
    oracle's rounding of its fp64 value except where fp32 and fp64 fall on
    different sides of the threshold, and the rounding is unbiased."""
    _run(B=8, H=32, dv=64, dk=128, L=4, steps=10, seed=13, exact=False, sample=[0, 5])


def test_sr_changes_with_key_and_counter():
    """Two launches with different counter words (and a different key)
    round the same values differently; the same words, identically."""
    lay = rs.layer(rs.MAMBA2, 4, 16, 32, 1, "f16", "f16", "bf16", None, stochastic=True)
    states = []
    for key, step0 in ((KEY, 0), (KEY, 0), (KEY, 7), ((1, 2), 0)):
        d = DecodeLayer(lay, 2, 2, "cuda", sr_key=key)
        for b in range(2):
            d.assign(b, b)
        d.reset_rows([0, 1])
        d.sr_step = step0
        tok = workloads.mamba2_tokens(3, 0, 2, 4, 16, 32, "bf16")
        io = rs.make_io(tok.q.cuda(), tok.k.cuda(), tok.v.cuda(), tok.lam.cuda(), torch.empty(2, 4, 16, device="cuda"))
        d.step(io)   # L = 1: every step flushes
        torch.cuda.synchronize()
        states.append(d.pool.ckpt()[:2].clone())
    assert torch.equal(states[0], states[1])
    for other in states[2:]:
        n = int((other != states[0]).sum())
        assert n > states[0].numel() // 20, n
        # only the choice of neighbour changes: at most one fp16 spacing apart
        a, b = states[0].double().cpu().numpy(), other.double().cpu().numpy()
        assert np.all(np.abs(a - b) <= _f16_ulp(np.maximum(np.abs(a), np.abs(b)))), "not neighbours"
    say("[sr] key and counter select the rounding")


def test_sr_spec_flush_exact():
    """The speculative verify's flush stores the checkpoint with the same
    rounding: dyadic drafts, every draft accepted, T = 2, L = 4."""
    B, H, dv, dk, L, T = 2, 4, 16, 32, 4, 2
    lay = rs.layer(rs.MAMBA2, H, dv, dk, L, "f16", "f16", "bf16", None, T, stochastic=True)
    d = SpecDecodeLayer(lay, B, B, "cuda", sr_key=KEY)
    for b in range(B):
        d.assign(b, b)
    d.upload(rows=range(B))
    spec = oracle.SpecReplayModel(B, H, dv, dk, L, T)
    h = np.zeros(B, np.int32)
    flushes = 0
    for s in range(8):
        toks = [workloads.dyadic_tokens(21, s * T + i, B, H, dv, dk) for i in range(T)]
        st = lambda name: torch.stack([getattr(t, name) for t in toks], dim=1)   # [B, T, H, d]
        q, k, v, lam = st("q"), st("k"), st("v"), st("lam")
        fl = rs.rs_spec_meta_step(L, T, h, np.zeros(B, np.uint8))
        step = d.sr_step
        out = torch.empty(B, T, H, dv, device="cuda")
        d.verify(rs.make_spec_io(q.cuda(), k.cuda(), v.cuda(), lam.cuda(), out))
        tm = lambda t: t.double().numpy().transpose(0, 2, 1, 3)
        o = spec.verify(tm(q), tm(k), tm(v), lam.double().numpy().transpose(0, 2, 1), fl.astype(bool))
        flt = np.repeat(fl.astype(bool), H)
        if flt.any():
            flushes += 1
            oracle.sr_round_tiles(spec.C, KEY, step, np.nonzero(flt)[0])
        torch.cuda.synchronize()
        assert rel_err(out.double().cpu().numpy().transpose(0, 2, 1, 3), o) <= TOL_F32
        if flt.any():
            got = d.pool.ckpt()[:B].double().cpu().numpy().reshape(B * H, dv, dk)
            assert np.array_equal(got[flt], spec.C[flt]), f"step {s}: {np.sum(got[flt] != spec.C[flt])} differ"
        a = np.full(B, T, np.int32)
        d.commit(torch.from_numpy(a).cuda())
        spec.commit(a)
        rs.rs_spec_meta_advance(L, T, h, fl, a)
    assert flushes >= 3 and int(d.err.item()) == 0
    say("[sr] speculative flush rounds bit for bit")


def _run_two_copy(B, H, L, steps, seed, exact, stochastic=True, sample=None):
    """A two-precision checkpoint with an fp16 recurrence copy (stochastic
    or nearest rounding) under an E4M3 read copy, Nemotron head shape,
    against oracle.TwoCopyReplayModel.  Both copies of a flushed tile come
    from the same unrounded fold: exact inputs make both bit-exact; random
    inputs check the recurrence copy as above and the read copy's codes and
    row scales against the oracle's encoding of its fp64 fold, then
    resynchronise the model to the GPU's copies."""
    dv, dk = 64, 128
    tag = f"two-copy f16/e4m3 B={B} H={H} L={L} steps={steps} exact={exact} sr={stochastic} seed={seed}"
    say(f"[case] {tag}")
    lay = rs.layer(rs.MAMBA2, H, dv, dk, L, "f16", "f16", "bf16", "e4m3", stochastic=stochastic)
    n_blocks = B + 3
    rep = DecodeLayer(lay, B, n_blocks, "cuda", sr_key=KEY)
    rep.pool.raw.fill_(0xFF)
    blocks = workloads.shuffled_blocks(seed, B, n_blocks)
    for b in range(B):
        rep.assign(b, int(blocks[b]))
    rep.reset_rows(range(B))
    sample = list(range(B)) if sample is None else sample
    ns = len(sample)
    tiles = np.array([b * H + h for b in sample for h in range(H)])
    model = oracle.TwoCopyReplayModel(ns, H, dv, dk, L, "e4m3", rec_dtype="f16", key=KEY if stochastic else None,
                                      tile_ids=tiles)
    blk = torch.as_tensor(blocks[sample], device="cuda", dtype=torch.long)
    inv = np.argsort(rep.pool.ckpt_lo_columns())   # stored position of each column
    stats = StoreStats()
    n_rne = n_rne_diff = 0
    code_diff = code_n = scale_diff = scale_n = 0
    tie_off = 0.0
    err, flushes = 0.0, 0
    for s in range(steps):
        tok = (workloads.dyadic_tokens(seed, s, B, H, dv, dk) if exact
               else workloads.mamba2_tokens(seed, s, B, H, dv, dk, "bf16"))
        q, k, v, lam = (t.to("cuda") for t in (tok.q, tok.k, tok.v, tok.lam))
        out = torch.empty(B, H, dv, device="cuda")
        step_r = rep.sr_step
        _, fl = rep.step(rs.make_io(q, k, v, lam, out))
        a64 = [t[sample].double().numpy() for t in (tok.q, tok.k, tok.v, tok.lam)]
        flr = np.asarray(fl)[sample].astype(bool)
        pre = oracle.ReplayModel(rs.MAMBA2, ns, H, dv, dk, L)   # the unrounded fold of flushing tiles
        pre.C, pre.rec_lam, pre.rec_x, pre.rec_k, pre.w = (model.C.copy(), model.rec_lam.copy(),
                                                         model.rec_x.copy(), model.rec_k.copy(), model.w.copy())
        pre.step(*a64, flr)
        o = model.step(*a64, flr, sr_step=step_r)
        torch.cuda.synchronize()
        err = max(err, rel_err(out[sample].double().cpu().numpy(), o))
        assert err <= (TOL_F32 if exact else TOL_LOW), (s, err)
        fl_t = np.repeat(flr, H)
        if not fl_t.any():
            continue
        flushes += 1
        got_hi = rep.pool.ckpt()[blk].double().cpu().numpy().reshape(ns * H, dv, dk)[fl_t]
        codes = rep.pool.ckpt_lo()[blk].cpu().numpy().reshape(ns * H, dv, dk)[fl_t][..., inv]
        scales = rep.pool.ckpt_scale()[blk].cpu().numpy().reshape(ns * H, dv)[fl_t].astype(np.float64)
        want_codes, want_e = formats.e4m3_quantize_rows(pre.C[fl_t])
        if exact:
            assert np.array_equal(got_hi, model.C[fl_t]), f"recurrence copy, step {s}"
            assert np.array_equal(codes, want_codes), f"read-copy codes, step {s}"
            assert np.array_equal(scales, np.ldexp(1.0, want_e)), f"read-copy scales, step {s}"
            continue
        if stochastic:
            stats.add(got_hi, pre.C[fl_t], model.C[fl_t])
        else:
            x, ref = pre.C[fl_t], model.C[fl_t]
            assert np.all(np.abs(got_hi - x) <= _f16_ulp(x) + 1e-5 * np.abs(x).max())
            bad = got_hi != ref
            n_rne += got_hi.size
            n_rne_diff += int(bad.sum())
            if bad.any():
                # the other neighbour only where the fp64 value lies within
                # the fp32 sums' error (bounded by 1e-5 of the tile's largest
                # value, as above) of the midpoint between the two
                scale = np.broadcast_to(np.abs(x).max(axis=(1, 2), keepdims=True), x.shape)[bad]
                off = np.abs(x[bad] - 0.5 * (got_hi[bad] + ref[bad])) / scale
                tie_off = max(tie_off, float(off.max()))
        same_row = scales == np.ldexp(1.0, want_e)
        scale_diff += int(np.sum(~same_row))
        scale_n += same_row.size
        cd = codes != want_codes
        code_diff += int(np.sum(cd[same_row]))
        code_n += int(np.sum(same_row)) * dk
        # continue from the GPU's copies
        model.C[fl_t] = got_hi
        model.C_lo[fl_t] = formats.e4m3_dequantize_rows(codes, np.log2(scales).astype(np.int64))
    assert int(rep.err.item()) == 0
    assert flushes >= 2
    if not exact:
        say(f"[two-copy] {tag}: read-copy rows with another scale {scale_diff}/{scale_n}, "
            f"codes differing {code_diff}/{code_n}, nearest-even recurrence values differing {n_rne_diff}/{n_rne} "
            f"(at most {tie_off:.2e} of the tile's largest value from a tie)")
        assert scale_diff <= max(1, scale_n // 1000) and code_diff <= max(2, code_n // 10000)
        if stochastic:
            stats.check(tag)
        else:
            assert n_rne_diff <= max(2, n_rne // 500) and tie_off < 1e-5, (n_rne_diff, tie_off)
    say(f"[errors] {tag}: out={err:.3g}, flushes={flushes}")


@pytest.mark.parametrize("stochastic", [True, False])
def test_two_copy_f16_recurrence_exact(stochastic):
    """fp16 recurrence copy + E4M3 read copy, dyadic inputs: both copies
    bit-exact against the oracle, outputs from the read copy."""
    _run_two_copy(B=4, H=8, L=4, steps=10, seed=31, exact=True, stochastic=stochastic)


@pytest.mark.parametrize("stochastic", [True, False])
def test_two_copy_f16_recurrence_generic(stochastic):
    _run_two_copy(B=8, H=32, L=4, steps=10, seed=33, exact=False, stochastic=stochastic, sample=[1, 6])
