"""Serving-path behaviour on the GPU against the fp64 oracle (needs an MI355X).

Token-less flush and state reset, the kernels' own checks of per-row
metadata, padding-only and very large batches, continuous batching with
rows retiring and joining, and a 40-layer stack."""
import numpy as np
import pytest
import torch

import linear_attention_decode_replay_amd as rs
import oracle
import workloads
from gpu_harness import TOL_F32, TOL_LOW, Case, assert_within, rel_err, run_case, say
from linear_attention_decode_replay_amd.state import DecodeLayer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev_io(tok, B, H, dv):
    q, k, v, lam = (x.to(DEV) for x in (tok.q, tok.k, tok.v, tok.lam))
    beta = tok.beta.to(DEV) if tok.beta is not None else None
    out = torch.full((B, H, dv), float("nan"), device=DEV)
    return rs.make_io(q, k, v, lam, out, beta), out, (q, k, v, lam, beta)


def _f64(tok, rows):
    g = lambda x: None if x is None else x[rows].double().numpy()
    return g(tok.q), g(tok.k), g(tok.v), g(tok.lam), g(tok.beta)


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
@pytest.mark.parametrize("shape,dts", [((16, 32), ("f32", "f32", "f32")), ((64, 128), ("f32", "f16", "bf16"))])
def test_token_less_flush_and_reset(form, shape, dts):
    """Mid-window token-less flush of some rows (their checkpoint must equal
    the conventional state at that step), reset of another (a new request
    from zero), and decoding that continues correctly afterwards."""
    dv, dk = shape
    sdt, rdt, io = dts
    B, H, L = 4, 3, 8
    tol = TOL_F32 if dts == ("f32", "f32", "f32") else TOL_LOW
    lay = rs.layer(form, H, dv, dk, L, sdt, rdt, io)
    d = DecodeLayer(lay, B, B + 2, DEV)
    d.pool.raw.fill_(0xFF)
    for b in range(B):
        d.assign(b, b + 1)
    d.reset_rows(range(B))
    ref = oracle.ConventionalModel(form, B, H, dv, dk)
    worst = 0.0
    for s in range(20):
        tok = workloads.tokens(form, 77, s, B, H, dv, dk, io)
        iod, out, keep = _dev_io(tok, B, H, dv)
        d.step(iod)
        o_ref = ref.step(*_f64(tok, slice(None)))
        torch.cuda.synchronize()
        worst = max(worst, rel_err(out.double().cpu().numpy(), o_ref))
        if s == 5:  # rows 0 and 2 hold 6 records: materialise them
            d.flush_rows([0, 2])
            torch.cuda.synchronize()
            ck = d.pool.ckpt()[torch.tensor([1, 3], device=DEV)].double().cpu().numpy()
            e = rel_err(ck, ref.state()[[0, 2]], 2)
            say(f"[flush] form={form} shape={shape} ckpt err {e:.3g}")
            assert e <= tol
            assert list(d.anchor) == [0, 6, 0, 6]
        if s == 11:  # row 3 retires; a new request joins in its slot on another block
            d.retire(3)
            d.assign(3, 0)
            d.reset_rows([3])
            ref.S.reshape(B, H, dv, dk)[3] = 0.0
    say(f"[errors] flush/reset form={form} shape={shape}: out={worst:.3g}")
    assert worst <= tol
    assert int(d.err.item()) == 0


def test_kernel_rejects_out_of_range_metadata():
    """A block id beyond the pool or a cursor beyond L-1 is skipped by the
    kernel's own bounds checks and counted; other rows are unaffected."""
    B, H, dv, dk, L = 5, 2, 16, 32, 4
    lay = rs.layer(rs.MAMBA2, H, dv, dk, L, "f32", "f32", "f32")
    pool = rs.Pool(lay, 6, DEV)
    pool.raw.zero_()
    bt = torch.tensor([0, 1, 7, 3, -1], dtype=torch.int32, device=DEV)   # row 2: block 7 >= 6
    wp = torch.tensor([0, 4, 0, 1, 0], dtype=torch.int32, device=DEV)    # row 1: cursor 4 > L-1
    fl = torch.zeros(8, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    nxt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    batch = rs.make_batch(pool.raw, 6, bt, wp, fl, err, next_write_pos=nxt)
    tok = workloads.tokens(0, 5, 0, B, H, dv, dk, "f32")
    iod, out, keep = _dev_io(tok, B, H, dv)
    rs.replay_decode_step(lay, batch, iod)
    torch.cuda.synchronize()
    assert int(err.item()) == 2 * H
    o = out.cpu()
    for b in (1, 2, 4):  # skipped rows and the padding row are untouched
        assert torch.isnan(o[b]).all()
    assert nxt.cpu().tolist() == [1, -7, -7, 2, -7]
    # rows 0 and 3 start from a zero checkpoint and no records that count:
    # row 3 holds one zero record, so both outputs are v (k . q)
    want = (tok.v * (tok.k * tok.q).sum(-1, keepdim=True)).double().numpy()
    assert rel_err(o[[0, 3]].double().numpy(), want[[0, 3]]) < 1e-5


def test_all_padding_batch():
    B, H, dv, dk, L = 3, 2, 16, 32, 4
    lay = rs.layer(rs.GDN, H, dv, dk, L, "f32", "f32", "f32")
    d = DecodeLayer(lay, B, 4, DEV)
    tok = workloads.tokens(1, 5, 0, B, H, dv, dk, "f32")
    iod, out, keep = _dev_io(tok, B, H, dv)
    d.step(iod)
    d.conventional_step(iod)
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and int(d.err.item()) == 0


def test_maximum_rows():
    """The largest batch one launch takes (65535 rows), tiny heads."""
    err = run_case(Case(B=65535, H=1, L=4, steps=6, sample=[0, 1, 32767, 65534], n_blocks=65535,
                        seed=9))
    assert_within(err, TOL_F32)


def _load_row_start(d: DecodeLayer, block: int, C0, rec_lam, rec_x, rec_k, w0):
    """Write one row's checkpoint and first w0 records into its pool block."""
    b = torch.tensor([block], device=DEV)
    ck = d.pool.ckpt()
    ck[b] = torch.from_numpy(C0).to(ck.dtype).to(DEV)[None]
    if w0:
        rx, rk, rl = d.pool.rec_x(), d.pool.rec_k(), d.pool.rec_lam()
        rx[block, :, :w0] = torch.from_numpy(rec_x[:, :w0]).to(rx.dtype).to(DEV)
        rk[block, :, :w0] = torch.from_numpy(rec_k[:, :w0]).to(rk.dtype).to(DEV)
        rl[block, :, :w0] = torch.from_numpy(rec_lam[:, :w0]).float().to(DEV)


@pytest.mark.parametrize("join", [False, True])
def test_continuous_batching(join):
    """Nemotron-3-Super layer shapes, 256 request slots over a shuffled pool
    of 384 blocks, each starting mid-window (cursor ~ U{0..15}, random
    checkpoint and records); 200 steps in which each live row retires with
    p = 1/32 and each empty slot takes a new request with p = 1/2 (its state
    zeroed by a reset launch, or, join=True, joined with a zero checkpoint
    that is not read until the row's first flush).  Every step checks 32
    sampled slots against the oracle (through their retires and joins), the
    host and device cursors, and that empty slots are not written."""
    H, dv, dk, L, B, NB, steps = 128, 64, 128, 16, 256, 384, 200
    seed = 4
    lay = rs.layer(rs.MAMBA2, H, dv, dk, L, "f32", "f16", "bf16")
    rep = DecodeLayer(lay, B, NB, DEV)
    conv = DecodeLayer(lay, B, NB, DEV)
    rep.pool.raw.fill_(0xFF)
    blocks0, w0s, events = workloads.continuous_schedule(seed, B, steps, NB)
    sample = list(range(0, B, 8))
    ns = len(sample)
    ref = oracle.ConventionalModel(rs.MAMBA2, ns, H, dv, dk)
    orc_rep = oracle.ReplayModel(rs.MAMBA2, 1, H, dv, dk, L)
    for slot in range(B):
        C0, rl, rx, rk = workloads.random_row_start(seed, slot, H, dv, dk, int(w0s[slot]), L - 1)
        _load_row_start(rep, int(blocks0[slot]), C0, rl, rx, rk, int(w0s[slot]))
        rep.assign(slot, int(blocks0[slot]), int(w0s[slot]))
        conv.assign(slot, int(blocks0[slot]), int(w0s[slot]))
        if slot in sample:  # the oracle's start state: fold the records into C0 in fp64
            orc_rep.set_row(0, C0, rl, rx, rk, int(w0s[slot]))
            orc_rep.fold(np.array([True]))
            i = sample.index(slot)
            ref.S[i * H:(i + 1) * H] = orc_rep.C
    # the conventional pool starts from the same (checkpoint + records) states
    conv.pool.raw.copy_(rep.pool.raw)
    conv.flush_rows(range(B))  # token-less fold of every row's records (anchors -> 0)
    assert np.all(conv.anchor == 0)
    live = np.ones(B, bool)
    worst_r = worst_c = 0.0
    for s in range(steps):
        ev = events[s]
        for slot in ev.retire:
            rep.retire(slot)
            conv.retire(slot)
            live[slot] = False
        for slot, blk in ev.join:
            rep.assign(slot, blk)
            conv.assign(slot, blk)
            live[slot] = True
            if slot in sample:
                i = sample.index(slot)
                ref.S[i * H:(i + 1) * H] = 0.0
        joined = [slot for slot, _ in ev.join]
        if joined:
            if join:
                rep.join_rows(joined)
            else:
                rep.reset_rows(joined)
            conv.reset_rows(joined)
        tok = workloads.tokens(rs.MAMBA2, seed, s, B, H, dv, dk, "bf16")
        iod, out_r, keep = _dev_io(tok, B, H, dv)
        out_c = torch.full_like(out_r, float("nan"))
        ioc = rs.make_io(keep[0], keep[1], keep[2], keep[3], out_c)
        wp, fl = rep.step(iod)
        conv.conventional_step(ioc)
        act = np.array([live[b] for b in sample])
        o_ref = ref.step(*_f64(tok, sample)[:4], active_rows=act)
        nxt = rep.device_cursor()
        assert np.array_equal(nxt[live], rep.anchor[live] % L), f"device cursor, step {s}"
        gr = out_r[sample].double().cpu().numpy()
        gc = out_c[sample].double().cpu().numpy()
        if act.any():
            worst_r = max(worst_r, rel_err(gr[act], o_ref[act]))
            worst_c = max(worst_c, rel_err(gc[act], o_ref[act]))
        dead = ~live
        if dead.any():
            assert torch.isnan(out_r[torch.as_tensor(dead, device=DEV)]).all()
    say(f"[errors] continuous batching: out_replay={worst_r:.3g} out_conv={worst_c:.3g} "
        f"uploads={rep.uploads}")
    assert worst_r <= TOL_LOW and worst_c <= TOL_LOW
    assert int(rep.err.item()) == 0 and int(conv.err.item()) == 0


@pytest.mark.parametrize("L,state_dt", [(8, "f32"), (16, "f32"), (32, "f32"), (8, "f16"), (16, "f16"), (32, "f16")])
def test_stack_of_40_layers(L, state_dt):
    """40 Mamba-2 layers at the Nemotron-3-Super shape, batch 256, one pool
    per layer; one window plus three steps.  All layers run on the GPU with
    distinct inputs; 2 layers x 16 rows are checked against the oracle."""
    H, dv, dk, B, n_layers = 128, 64, 128, 256, 40
    steps = L + 3
    lay = rs.layer(rs.MAMBA2, H, dv, dk, L, state_dt, "f16", "bf16")
    layers = []
    for _ in range(n_layers):
        d = DecodeLayer(lay, B, B, DEV)
        for b in range(B):
            d.assign(b, b)
        d.reset_rows(range(B))
        layers.append(d)
    checked = {5: None, 33: None}
    rows = list(range(0, B, 16))
    for li in checked:
        checked[li] = oracle.ConventionalModel(rs.MAMBA2, len(rows), H, dv, dk)
    g = torch.Generator(device=DEV)
    worst = 0.0
    for s in range(steps):
        outs = {}
        for li, d in enumerate(layers):
            if li in checked:
                tok = workloads.tokens(rs.MAMBA2, 100 + li, s, B, H, dv, dk, "bf16")
                iod, out, keep = _dev_io(tok, B, H, dv)
                outs[li] = (out, tok, keep)
            else:
                g.manual_seed(1000 * li + s)
                q = torch.randn((B, H, dk), generator=g, device=DEV).bfloat16()
                k = torch.randn((B, H, dk), generator=g, device=DEV).bfloat16()
                v = torch.randn((B, H, dv), generator=g, device=DEV).bfloat16()
                lam = -torch.rand((B, H), generator=g, device=DEV) * 4
                out = torch.empty((B, H, dv), device=DEV)
                iod = rs.make_io(q, k, v, lam, out)
                outs[li] = (out, None, (q, k, v, lam))
            d.step(iod)
        torch.cuda.synchronize()
        for li, m in checked.items():
            out, tok, _ = outs[li]
            o_ref = m.step(*_f64(tok, rows)[:4])
            worst = max(worst, rel_err(out[rows].double().cpu().numpy(), o_ref))
    say(f"[errors] 40-layer stack L={L} state={state_dt}: out_replay={worst:.3g}")
    assert worst <= TOL_LOW
    assert all(int(d.err.item()) == 0 for d in layers)
    del layers
    torch.cuda.empty_cache()


@pytest.mark.parametrize("form,shape,groups", [(rs.MAMBA2, (16, 32), 0), (rs.MAMBA2, (64, 128), 0),
                                               (rs.GDN, (128, 128), 0), (rs.MAMBA2, (16, 32), 2),
                                               (rs.GDN, (64, 128), 2)])
def test_token_less_flush_of_speculative_layer(form, shape, groups):
    """replay_flush on a speculative layer (a ring of L committed records):
    after verify + commit steps with random acceptance, every row's h
    committed records are folded into its checkpoint, which must equal the
    committed state (the oracle, token by token).  At 64 x 128 with fp16
    records and L = 16 the flush's LDS holds L (not L - 1) record slots.
    With grouped keys (4 heads in 2 groups) the flush reads each group's
    keys, which the commits of flushed rows moved out of the staging slots."""
    from linear_attention_decode_replay_amd.state import SpecDecodeLayer
    dv, dk = shape
    B, H, L, T = 3, 4 if groups else 2, 16, 4
    hg = H // groups if groups else 1
    lowp = shape != (16, 32)
    rdt, io = ("f16", "bf16") if lowp else ("f32", "f32")
    lay = rs.layer(form, H, dv, dk, L, "f32", rdt, io, None, T, groups)
    d = SpecDecodeLayer(lay, B, B + 1, DEV)
    d.pool.raw.fill_(0xFF)
    for b in range(B):
        d.assign(b, b + 1)
    d.upload(rows=range(B))
    ref = oracle.SpecTokenByToken(B, H, dv, dk, T, form=form)
    h = np.zeros(B, np.int32)
    for s in range(7):
        tok = workloads.spec_tokens(91, s, B, H, T, dv, dk, io, 0.05, 1.0, form)
        qg, kg = tok.q[:, :, ::hg].contiguous(), tok.k[:, :, ::hg].contiguous()
        tok.q, tok.k = qg.repeat_interleave(hg, dim=2), kg.repeat_interleave(hg, dim=2)
        fl = rs.rs_spec_meta_step(L, T, h)
        q, k, v, lam = (x.to(DEV) for x in (qg, kg, tok.v, tok.lam))
        beta = tok.beta.to(DEV) if tok.beta is not None else None
        out = torch.empty((B, T, H, dv), device=DEV)
        d.verify(rs.make_spec_io(q, k, v, lam, out, beta))
        tm = lambda t: t.double().numpy().transpose(0, 2, 1, 3)
        ref.verify(tm(tok.q), tm(tok.k), tm(tok.v), tok.lam.double().numpy().transpose(0, 2, 1),
                   None if tok.beta is None else tok.beta.double().numpy().transpose(0, 2, 1))
        a = workloads.spec_accepted(91, s, B, T, "random")
        d.commit(torch.from_numpy(a).to(DEV))
        ref.commit(a)
        rs.rs_spec_meta_advance(L, T, h, fl, a)
    assert (h > 0).any()
    # materialise: flag every row, cursor = committed count (the device's)
    dh, _ = d.device_committed()
    assert np.array_equal(dh, h)
    n4 = d.flag[0].numel()
    flags = torch.ones(n4, dtype=torch.uint8, device=DEV)
    batch = rs.make_batch(d.pool.raw, d.pool.n_blocks, d.block_table, d.committed[d._cur], flags, d.err)
    rs.replay_flush(lay, batch)
    torch.cuda.synchronize()
    blk = torch.arange(1, B + 1, device=DEV)
    ck = d.pool.ckpt()[blk].double().cpu().numpy()
    e = rel_err(ck, ref.state(), 2)
    tol = TOL_LOW if lowp else TOL_F32
    say(f"[errors] token-less flush of a speculative layer form={form} shape={shape}: ckpt={e:.3g} h={list(h)}")
    assert e <= tol
    assert int(d.err.item()) == 0


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
def test_token_less_flush_of_joining_rows(form):
    """Rows joined with a zero checkpoint (never written, NaN-filled pool):
    a token-less flush of one at w = 6 writes the fold of its records into
    zero, of one that has just joined (w = 0) writes zeros; both equal the
    conventional state, the other joined row keeps its flag until its own
    first flush, and decoding continues from all of them."""
    B, H, dv, dk, L = 3, 2, 16, 32, 8
    lay = rs.layer(form, H, dv, dk, L, "f32", "f32", "f32")
    d = DecodeLayer(lay, B, B, DEV)
    d.pool.raw.fill_(0xFF)
    for b in (0, 1):
        d.assign(b, b)
    d.join_rows([0, 1])
    ref = oracle.ConventionalModel(form, B, H, dv, dk)
    worst = 0.0
    for s in range(12):
        if s == 6:  # row 2 joins, then rows 0 (6 records) and 2 (none) are materialised
            d.assign(2, 2)
            d.join_rows([2])
            d.flush_rows([0, 2])
            torch.cuda.synchronize()
            ck = d.pool.ckpt()[torch.tensor([0, 2], device=DEV)].double().cpu().numpy()
            e = rel_err(ck, ref.state()[[0, 2]], 2)
            say(f"[flush] joined rows form={form}: ckpt err {e:.3g}")
            assert e <= TOL_F32 and np.all(np.isfinite(ck)) and not ck[1].any()
            assert list(d.zero_ckpt) == [False, True, False]
            assert list(d.anchor) == [0, 6, 0]
        tok = workloads.tokens(form, 91, s, B, H, dv, dk, "f32")
        if s < 6:  # row 2 is empty: the oracle's row 2 stays at zero state
            tok.v[2] = 0.0
        iod, out, keep = _dev_io(tok, B, H, dv)
        d.step(iod)
        o_ref = ref.step(*_f64(tok, slice(None)))
        torch.cuda.synchronize()
        rows = [0, 1, 2] if s >= 6 else [0, 1]
        worst = max(worst, rel_err(out[rows].double().cpu().numpy(), o_ref[rows]))
        if s == 7:  # row 1's first flush (w = L - 1) wrote its checkpoint
            assert not d.zero_ckpt.any()
    say(f"[errors] joined rows + token-less flush form={form}: out={worst:.3g}")
    assert worst <= TOL_F32
    assert int(d.err.item()) == 0


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
def test_layers_sharing_metadata(form):
    """Three layers over the same slots share one block table and one set of
    cursors (DecodeLayer with n_layers = 3: one upload per step, each launch
    writing the same next cursors): every layer matches its own oracle
    through a retire, a join with a zero checkpoint and a forced flush."""
    B, H, dv, dk, L, NL = 4, 2, 16, 32, 4, 3
    lay = rs.layer(form, H, dv, dk, L, "f32", "f32", "f32")
    d = DecodeLayer(lay, B, B + 1, DEV, n_layers=NL)
    for pl in d.pools:
        pl.raw.fill_(0xFF)
    for b in range(B):
        d.assign(b, b)
    d.join_rows(range(B))
    refs = [oracle.ConventionalModel(form, B, H, dv, dk) for _ in range(NL)]
    worst = 0.0
    uploads = []
    for s in range(14):
        if s == 5:  # row 1 retires; a new request takes its slot on the spare block
            d.retire(1)
            d.assign(1, B)
            d.join_rows([1])
            for r in refs:
                r.S.reshape(B, H, dv, dk)[1] = 0.0
        force = np.zeros(B, np.uint8)
        if s == 8:
            force[2] = 1
        toks = [workloads.tokens(form, 200 + li, s, B, H, dv, dk, "f32") for li in range(NL)]
        devs = [_dev_io(t, B, H, dv) for t in toks]
        u0 = d.uploads
        d.step([x[0] for x in devs], force)
        uploads.append(d.uploads - u0)
        torch.cuda.synchronize()
        for li in range(NL):
            o_ref = refs[li].step(*_f64(toks[li], slice(None)))
            worst = max(worst, rel_err(devs[li][1].double().cpu().numpy(), o_ref))
        assert np.array_equal(d.device_cursor()[d.live()], d.anchor[d.live()] % L)
    say(f"[errors] {NL} layers sharing metadata form={form}: out={worst:.3g} uploads={uploads}")
    assert worst <= TOL_F32
    assert max(uploads) == 1 and sum(uploads) <= 4   # first step, the join, the forced flush and the step after
    assert int(d.err.item()) == 0
