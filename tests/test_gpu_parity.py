"""HIP path vs the fp64 oracle, element by element (needs an MI355X).

Every case runs the checkpoint + buffer kernel and the conventional kernel
through the C ABI on the same seeded inputs as the oracle and checks, on
every step: host cursor and flush flags (bit-exact), outputs and flushed
checkpoints (within tolerance), appended record fields (bit-exact copies),
padding rows (untouched)."""
import pytest

import linear_attention_decode_replay_amd as rs
from gpu_harness import TOL_F32, TOL_LOW, Case, assert_within, run_case, tolerance

pytestmark = pytest.mark.gpu


def _go(c: Case):
    err = run_case(c)
    assert_within(err, tolerance(c.state_dt, c.rec_dt, c.io_dt))
    return err


def test_tiny_mamba2():
    """Tiny Mamba-2 decode: batch 2, 4 heads, 16x32, L=4, 64 steps from zero, fp32."""
    err = _go(Case())
    assert err["flushes"] == 16


def test_tiny_mamba2_long_memory():
    """Added case (not a named workload): slowly decaying heads, a ~ U[0.001, 0.01],
    so the checkpoint term dominates the output."""
    _go(Case(seed=3, a_lo=0.001, a_hi=0.01))


def test_tiny_gdn():
    err = _go(Case(form=rs.GDN, seed=1))
    assert err["flushes"] == 16


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
@pytest.mark.parametrize("L", [1, 2, 16, 64])
def test_tiny_buffer_lengths(form, L):
    _go(Case(form=form, L=L, steps=max(3 * L + 5, 12), seed=10 + L))


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
def test_largest_buffer_128x128_fp32_records(form):
    """L = 64 with fp32 records at 128 x 128, the largest record area (63
    slots of 1 KiB per head, staged in LDS): 70 steps, one flush, fp32
    throughout."""
    err = _go(Case(form=form, B=2, H=2, dv=128, dk=128, L=64, steps=70, seed=64))
    assert err["flushes"] == 1


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
@pytest.mark.parametrize("shape,dts", [((16, 32), ("f32", "f32", "f32")), ((64, 128), ("f32", "f16", "bf16")),
                                       ((128, 128), ("f16", "f16", "bf16"))])
def test_full_forgetting(form, shape, dts):
    """alpha = 0 (lam = -inf) on every 5th (step, row, head): the checkpoint
    and the records before it drop out of the output (oracle pin
    pin_full_forgetting), in flush and non-flush steps, appended records
    carry lam = -inf bit for bit, and nothing turns into NaN."""
    dv, dk = shape
    sdt, rdt, io = dts
    err = _go(Case(form=form, B=3, H=3, dv=dv, dk=dk, L=4, steps=24, state_dt=sdt, rec_dt=rdt, io_dt=io,
                   forget_every=5, force_every=7, seed=70))
    assert err["flushes"] >= 6


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
@pytest.mark.parametrize("sdt,rdt,io", [("f32", "f16", "bf16"), ("f16", "f16", "bf16"),
                                        ("f16", "f32", "f16"), ("f32", "f32", "bf16")])
def test_tiny_dtypes(form, sdt, rdt, io):
    _go(Case(form=form, state_dt=sdt, rec_dt=rdt, io_dt=io, seed=20))


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
def test_tiny_strided_pad_forced(form):
    """Strided q/k/v views, padding rows, shuffled blocks in a larger pool,
    and forced flushes on row 0 every 5 steps."""
    _go(Case(form=form, B=6, pad_rows=[2, 5], n_blocks=11, strided=True, force_every=5, seed=30))


@pytest.mark.parametrize("form,shape", [(rs.MAMBA2, (64, 128)), (rs.GDN, (128, 128))])
def test_production_shapes_small_batch(form, shape):
    dv, dk = shape
    _go(Case(form=form, B=3, H=5, dv=dv, dk=dk, L=16, steps=40, state_dt="f32", rec_dt="f16",
             io_dt="bf16", seed=40, strided=True, pad_rows=[1]))


def test_nemotron_layer_full_size():
    """One Mamba-2 layer at the Nemotron-3-Super shape: 128 heads, 64x128, fp32
    state, batch 256, L=16, 64 steps, bf16 inputs, fp16 records; 6 rows sampled
    (all heads) against the oracle, all rows run on the GPU."""
    err = _go(Case(B=256, H=128, dv=64, dk=128, L=16, steps=64, state_dt="f32", rec_dt="f16",
                   io_dt="bf16", sample=[0, 1, 77, 128, 200, 255], n_blocks=300, seed=2))
    assert err["flushes"] == 4


@pytest.mark.parametrize("state_dt", ["f32", "f16"])
@pytest.mark.parametrize("B", [1, 8, 32, 128, 256, 512])
def test_gdn_batch_sweep(B, state_dt):
    """Gated DeltaNet: 32 heads, 128x128, unit-norm k and q, L=16; 20 steps
    (one flush) with up to 4 rows sampled."""
    sample = sorted({0, B // 3, B // 2, B - 1})
    _go(Case(form=rs.GDN, B=B, H=32, dv=128, dk=128, L=16, steps=20, state_dt=state_dt,
             rec_dt="f16", io_dt="bf16", sample=sample, seed=50 + B))


TWO_COPY_TOL = 1e-3


@pytest.mark.parametrize("read_dt", ["f16", "bf16"])
@pytest.mark.parametrize("rec_dt,io", [("f32", "f32"), ("f16", "bf16")])
@pytest.mark.parametrize("hints", [True, False])
def test_two_precision_checkpoint_tiny(read_dt, rec_dt, io, hints):
    """fp32 recurrence copy + fp16/bf16 read copy (Mamba-2), tiny heads with
    strided inputs, padding and forced flushes; compared with the oracle's
    two-copy model (outputs) and its exact recurrence (flushed checkpoints).
    With the host's flush hints, non-flush steps run the kernel without the
    fold and forced-flush steps a pair of launches; without, one kernel."""
    err = run_case(Case(B=5, pad_rows=[3], strided=True, force_every=5, rec_dt=rec_dt, io_dt=io,
                        read_dt=read_dt, seed=60, flush_hints=hints))
    _check_two_precision(err, read_dt)


def _check_two_precision(err, read_dt="f16"):
    # every output within the error bound of one rounding of the last
    # checkpoint (checked element by element in the harness)
    assert err["read_bound_excess"] <= 0, err
    assert err["ckpt_flush"] <= TOL_F32  # the recurrence copy is fp32
    if read_dt == "e4m3":
        return  # an 8-bit read error exceeds the 16-bit tolerance by design; the bound is the check
    # same arithmetic as the oracle's two-copy model: they differ by fp32
    # rounding and, rarely, by one 16-bit ulp where the read copy rounds an
    # fp32 value that lies on the other side of a rounding boundary than the
    # exact one
    assert err["out_replay"] <= TWO_COPY_TOL, err
    # against exact decoding: one rounding of the last checkpoint, within the
    # 16-bit tolerance
    assert err["out_replay_vs_exact"] <= TOL_LOW, err
    assert_within(err, TOL_LOW)


@pytest.mark.parametrize("rec_dt,io", [("f32", "f32"), ("f16", "bf16")])
def test_e4m3_read_copy_small(rec_dt, io):
    """An E4M3 read copy with per-row power-of-two scales over an fp32
    recurrence copy (Mamba-2, 64 x 128 heads: the smallest head an E4M3 tile
    covers), strided inputs, padding and forced flushes.  Outputs within the
    one-rounding bound of exact decoding; codes and scales bit-exact against
    the oracle's E4M3 encoding of the recurrence copy at every flush."""
    err = run_case(Case(B=4, H=3, dv=64, dk=128, L=4, steps=24, pad_rows=[2], strided=True, force_every=5,
                        rec_dt=rec_dt, io_dt=io, read_dt="e4m3", a_lo=0.001, a_hi=0.01, seed=62))
    _check_two_precision(err, "e4m3")
    assert err["flushes"] >= 6


def test_e4m3_read_copy_rejects_small_heads():
    lay = rs.layer(rs.MAMBA2, 4, 16, 32, 4, "f32", "f32", "f32", "e4m3")
    assert rs.layer_supported(lay) == rs.RS_EUNSUPPORTED and "E4M3" in rs.last_error()


@pytest.mark.parametrize("read_dt", ["f16", "bf16", "e4m3"])
def test_two_precision_checkpoint_nemotron(read_dt):
    """The Nemotron-3-Super layer at batch 256 with a two-precision checkpoint
    (E4M3: long-memory heads, where the checkpoint term dominates every step
    of the window)."""
    a = (0.001, 0.01) if read_dt == "e4m3" else (1.0, 8.0)
    err = run_case(Case(B=256, H=128, dv=64, dk=128, L=16, steps=40, state_dt="f32", rec_dt="f16",
                        io_dt="bf16", read_dt=read_dt, sample=[0, 100, 255], n_blocks=260, a_lo=a[0],
                        a_hi=a[1], seed=61))
    _check_two_precision(err, read_dt)
    assert err["flushes"] == 2


# ------------------------------------------------------------ grouped keys --
@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
def test_grouped_keys_tiny(form):
    """Keys and queries shared by pairs of heads (the released grouped-key
    layout): one key record per group, values and decays per head; fp32."""
    err = _go(Case(form=form, H=4, groups=2, seed=70))
    assert err["flushes"] == 16


def test_grouped_keys_strided_pad_forced_lowprec():
    _go(Case(B=5, H=6, groups=3, pad_rows=[1], n_blocks=9, strided=True, force_every=5, state_dt="f32",
             rec_dt="f16", io_dt="bf16", seed=71))


def test_grouped_keys_two_precision():
    err = run_case(Case(H=4, groups=2, read_dt="f16", seed=72))
    assert err["out_replay"] <= TOL_LOW and err["ckpt_flush"] <= TOL_F32


def test_grouped_keys_nemotron_layer():
    """The Nemotron-3-Super Mamba-2 layer as released: 128 heads in 8 key
    groups, 64x128, fp32 state, batch 256, L = 16, bf16 inputs, fp16 records;
    40 steps, 4 rows sampled."""
    err = _go(Case(B=256, H=128, groups=8, dv=64, dk=128, L=16, steps=40, state_dt="f32", rec_dt="f16",
                   io_dt="bf16", sample=[0, 99, 160, 255], n_blocks=260, seed=73))
    assert err["flushes"] == 2


def test_grouped_keys_gdn_production():
    """Gated DeltaNet 128x128 with 2 value heads per key head."""
    _go(Case(form=rs.GDN, B=16, H=32, groups=16, dv=128, dk=128, L=16, steps=20, rec_dt="f16", io_dt="bf16",
             sample=[0, 15], seed=74))


@pytest.mark.parametrize("name,case", [
    ("mamba2-groups-of-4", dict(B=7, H=8, groups=2)),                       # 56 tiles: 32 mapped, 24 in the tail
    ("gdn-128-fp32-parts", dict(form=rs.GDN, B=5, H=3, dv=128, dk=128)),     # 30 half tiles: 16 mapped
    ("gdn-128-fp32-groups", dict(form=rs.GDN, B=4, H=4, groups=2, dv=128, dk=128)),  # units of 4: all mapped
])
def test_xcd_unit_map_covers_every_tile(name, case):
    """Workgroups that share bytes (a tile's parts, a key group's heads)
    are mapped to one XCD in blocks of 8 units, with the identity on a last
    partial block: every row of the batch is checked, so a tile computed
    twice or never shows up."""
    _go(Case(L=4, steps=13, seed=75, **case))


# ------------------------------------------ GDN state-reconstruction route --
@pytest.mark.parametrize("L", [1, 4, 16])
def test_gdn_reconstruct_tiny(L):
    """The PR's route: every step rebuilds S_{t-1} from the checkpoint and
    the buffered (d, k, g) records; outputs, records and checkpoints against
    the conventional recurrence, like the output-only route."""
    err = _go(Case(form=rs.GDN, L=L, steps=max(3 * L + 5, 24), reconstruct=True, seed=70 + L))
    assert err["flushes"] >= 2


@pytest.mark.parametrize("sdt,rdt,io", [("f16", "f16", "bf16"), ("f32", "f16", "f16")])
def test_gdn_reconstruct_dtypes_strided(sdt, rdt, io):
    _go(Case(form=rs.GDN, B=6, pad_rows=[2], n_blocks=9, strided=True, force_every=5, state_dt=sdt,
             rec_dt=rdt, io_dt=io, reconstruct=True, seed=75))


@pytest.mark.parametrize("state_dt", ["f32", "f16"])
def test_gdn_reconstruct_production_shape(state_dt):
    """32 heads, 128 x 128 (split over two workgroups per tile), batch 64,
    L = 16, 20 steps with one flush; 3 rows sampled."""
    _go(Case(form=rs.GDN, B=64, H=32, dv=128, dk=128, L=16, steps=20, state_dt=state_dt, rec_dt="f16",
             io_dt="bf16", sample=[0, 31, 63], reconstruct=True, seed=77))


# ------------------------------------------------------------- flush hints --
@pytest.mark.parametrize("read", ["f16", None])
@pytest.mark.parametrize("hint", ["none", "all"])
def test_flush_hint_broken_promise(hint, read):
    """A row that breaks the caller's flush hint is skipped (its outputs and
    checkpoint untouched) and counted once per tile; the other rows are
    computed as without a hint.  Two-copy checkpoints use every hint; a
    single fp32 Mamba-2 checkpoint uses RS_FLUSH_NONE only (its persistent
    kernel) and computes every row under RS_FLUSH_ALL."""
    import numpy as np
    import torch
    import workloads
    from gpu_harness import say
    from linear_attention_decode_replay_amd.state import DecodeLayer

    H, L = 4, 4
    lay = rs.layer(rs.MAMBA2, H, 16, 32, L, "f32", "f32", "f32", read)
    tok = workloads.tokens(rs.MAMBA2, 5, 0, 3, H, 16, 32, "f32")
    outs, ckpts, errs = [], [], []
    for use in (rs.RS_FLUSH_UNKNOWN, rs.RS_FLUSH_NONE if hint == "none" else rs.RS_FLUSH_ALL):
        d = DecodeLayer(lay, 3, 3, "cuda")
        d.pool.raw.zero_()              # zero records in the slots the rows read
        for b in range(3):
            d.assign(b, b)
        d.reset_rows(range(3))
        d.anchor[:] = [L - 1, 1, 1]     # row 0 flushes this step, rows 1 and 2 do not
        d._dirty = True
        d._hint = lambda fl, use=use: use
        out = torch.full((3, H, 16), float("nan"), device="cuda")
        _, fl = d.step(rs.make_io(tok.q.cuda(), tok.k.cuda(), tok.v.cuda(), tok.lam.cuda(), out))
        assert list(fl) == [1, 0, 0]
        torch.cuda.synchronize()
        outs.append(out.cpu())
        ckpts.append(d.pool.ckpt()[:3].cpu())
        errs.append(int(d.err.item()))
    ref, got = outs
    assert errs[0] == 0
    if read is None and hint == "all":   # not used: every row computed
        assert errs[1] == 0 and torch.allclose(got, ref, rtol=1e-6, atol=1e-6)
        assert torch.allclose(ckpts[1], ckpts[0], rtol=1e-6, atol=1e-7)
        return
    broken = [0] if hint == "none" else [1, 2]
    kept = [b for b in range(3) if b not in broken]
    assert errs[1] == H * len(broken)
    assert torch.isnan(got[broken]).all()
    assert torch.allclose(got[kept], ref[kept], rtol=1e-6, atol=1e-6)
    if hint == "none":  # the skipped flush left the zero checkpoint alone
        assert torch.count_nonzero(ckpts[1][0]) == 0 and torch.count_nonzero(ckpts[0][0]) > 0
    else:
        assert torch.allclose(ckpts[1][0], ckpts[0][0], rtol=1e-6, atol=1e-7)
    say(f"[hint] broken '{hint}' promise (read copy {read}): {errs[1]} tiles skipped and counted")


# ------------------------------------------- persistent non-flush kernel --
@pytest.mark.parametrize("B,H,shape,L,pad,force,sample", [
    (1, 1, (64, 128), 16, [], 0, None),           # one tile: a grid of one workgroup
    (3, 5, (16, 32), 4, [1], 0, None),
    (17, 128, (64, 128), 16, [], 0, [0, 8, 16]),  # 2,176 tiles: 4 or 5 per workgroup
    (300, 40, (16, 32), 8, [7, 299], 5, None),    # 12,000 tiles: 23 or 24 per workgroup
    (513, 64, (16, 32), 2, [], 0, None),          # L = 2: every other step flushes
])
def test_persistent_step_shapes(B, H, shape, L, pad, force, sample):
    """The persistent non-flush step (Mamba-2, one fp32 checkpoint) over odd
    shapes: grids from one workgroup up, uneven item counts, padding rows and
    forced flushes, the shortest ring."""
    dv, dk = shape
    _go(Case(form=rs.MAMBA2, B=B, H=H, dv=dv, dk=dk, L=L, steps=3 * L + 1, state_dt="f32", rec_dt="f16",
             io_dt="bf16", pad_rows=pad, force_every=force, sample=sample, check_conventional=False,
             seed=90 + B))


@pytest.mark.parametrize("B,H,pad,force", [(40, 40, [3, 17], 3), (1024, 40, [5, 600], 0)])
def test_persistent_step_item_counts(B, H, pad, force):
    """Steps with no flushing row of a Mamba-2 layer with one fp32 checkpoint
    run as a persistent grid of two workgroups per compute unit.  More
    (row, head) tiles than the grid: every workgroup takes several, in odd
    and even numbers (1600 tiles: 3 or 4 each, fewer where padding rows
    drop out), with forced flushes every third step in between (those steps
    run the one-launch kernel); 40960 tiles: 80 per workgroup, more than the
    64 whose writes it holds back at once."""
    _go(Case(form=rs.MAMBA2, B=B, H=H, dv=16, dk=32, L=4, steps=12, state_dt="f32", rec_dt="f16", io_dt="bf16",
             pad_rows=pad, force_every=force, check_conventional=False, seed=81 + B))


@pytest.mark.parametrize("rec_dt,L", [("f16", 32), ("f32", 16)])
def test_persistent_step_long_ring(rec_dt, L):
    """Rings whose records take 3 chunks per thread to stage (31 fp16
    records, or 15 fp32 records, of a 64 x 128 head) run the persistent
    non-flush form's long-ring instantiation: 17 rows x 128 heads (4 or 5
    tiles per workgroup), two windows and a flush."""
    _go(Case(B=17, H=128, dv=64, dk=128, L=L, steps=2 * L + 3, state_dt="f32", rec_dt=rec_dt, io_dt="bf16",
             sample=[0, 9, 16], check_conventional=False, seed=95 + L))


@pytest.mark.parametrize("form,dv,L,groups", [(rs.MAMBA2, 64, 4, 0), (rs.MAMBA2, 64, 64, 0), (rs.GDN, 128, 4, 0),
                                             (rs.GDN, 128, 64, 0), (rs.MAMBA2, 64, 16, 2), (rs.GDN, 128, 16, 2)])
def test_fp16_state_fold_on_matrix_cores(form, dv, L, groups):
    """An fp16 state with fp16 records at d_k = 128 folds its records on the
    matrix cores at every flush (16 records per pass, the weights as fp16
    hi + lo pairs): rings of 3 records (one partial pass), 15 with keys
    shared by pairs of heads, and 63 (four passes); forced flushes on row 0
    at other cursors, a padding row."""
    _go(Case(form=form, B=3, H=4 if groups else 2, dv=dv, dk=128, L=L, steps=L + 8, state_dt="f16", rec_dt="f16",
             io_dt="bf16", pad_rows=[1], force_every=5, groups=groups, seed=120 + L + dv + groups))


@pytest.mark.parametrize("name,case", [
    ("mamba2-tiny", dict()),
    ("gdn-tiny", dict(form=rs.GDN)),
    ("mamba2-nemotron-heads", dict(B=5, H=3, dv=64, dk=128, L=8, steps=20, rec_dt="f16", io_dt="bf16",
                                   pad_rows=[2], force_every=3)),
    ("mamba2-no-hints", dict(B=3, H=3, dv=64, dk=128, L=4, steps=12, rec_dt="f16", io_dt="bf16",
                             flush_hints=False)),
    ("e4m3-read-copy", dict(B=3, H=3, dv=64, dk=128, L=4, steps=12, rec_dt="f16", io_dt="bf16", read_dt="e4m3")),
    ("f16-read-copy", dict(B=3, H=3, dv=64, dk=128, L=4, steps=12, rec_dt="f16", io_dt="bf16", read_dt="f16")),
    ("gdn-128-f16-state", dict(form=rs.GDN, B=3, H=2, dv=128, dk=128, L=8, steps=20, state_dt="f16",
                               rec_dt="f16", io_dt="bf16", force_every=5)),
    ("gdn-reconstruct", dict(form=rs.GDN, B=3, H=3, L=4, steps=12, reconstruct=True)),
    # rings with no slot (L = 1: every step flushes) or one; the one-workgroup
    # kernel's loads for an empty ring and a zero checkpoint read fallback
    # addresses whose values are discarded
    ("mamba2-L1", dict(L=1, steps=8)),
    ("gdn-L1", dict(form=rs.GDN, L=1, steps=8)),
    ("mamba2-L2-f16-state", dict(L=2, steps=9, state_dt="f16", rec_dt="f16", io_dt="bf16")),
])
def test_join_with_zero_checkpoint(name, case):
    """Rows join with RS_CURSOR_ZERO_CKPT instead of a state reset: their
    checkpoints stay NaN-filled in the pool and their values must never be
    used before the row's first flush writes them (any use would turn the
    outputs into NaN); the flag the device carries in its cursors is
    bit-exact against the host's, and is cleared by each row's first flush."""
    c = Case(join=True, seed=80, **case)
    if c.read_dt:
        err = run_case(c)
        assert err["out_replay"] <= TWO_COPY_TOL and err["ckpt_flush"] <= tolerance(c.state_dt, c.rec_dt)
        assert err["read_bound_excess"] <= 0
    else:
        _go(c)
