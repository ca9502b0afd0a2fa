"""Speculative verify on the GPU (through the C ABI) against the fp64 oracle.

Gates (the decode path's): 1e-4 of each tile's largest output when inputs,
records and state are fp32; 2e-2 with fp16/bf16 anywhere.  Committed counts,
flags and the stored draft records are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import linear_attention_decode_replay_amd as rs
from gpu_harness import TOL_F32, TOL_LOW, say
from gpu_spec_harness import SpecCase, run_spec_case
from linear_attention_decode_replay_amd.state import SpecDecodeLayer

pytestmark = pytest.mark.gpu


def _check(err, tol):
    assert err["out_spec"] <= tol, err
    assert err["out_vs_tokens"] <= tol, err
    assert err["ckpt_flush"] <= tol, err


def _check_gdn(err, tol):
    _check(err, tol)
    assert err["rec_u"] <= tol, err   # the drafts' corrected values, stored as records


@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_spec_tiny_fp32(T):
    """Tiny shapes, everything fp32, random accepted counts 0..T, L = 8."""
    err = run_spec_case(SpecCase(T=T, steps=40, seed=T))
    assert err["flushes"] >= 4
    _check(err, TOL_F32)


@pytest.mark.parametrize("accept", ["all", "one", "none"])
def test_spec_accept_policies(accept):
    """Every draft accepted (a flush every L / T steps), one token per step,
    and nothing accepted (the ring never grows, no flush)."""
    err = run_spec_case(SpecCase(T=4, L=16, steps=36, accept=accept, seed=11))
    if accept == "none":
        assert err["flushes"] == 0 and err["accepted"] == 0
    else:
        assert err["flushes"] >= 2
    _check(err, TOL_F32)


def test_spec_long_memory():
    """Slowly decaying heads: the checkpoint term dominates every output."""
    err = run_spec_case(SpecCase(T=4, L=8, steps=30, a_lo=0.001, a_hi=0.01, seed=3))
    _check(err, TOL_F32)


def test_spec_strided_padding_forced_lowprec():
    """bf16 inputs as strided views, fp16 records, a padding row, a forced
    flush on row 0 every 5 steps."""
    err = run_spec_case(SpecCase(B=4, T=4, L=8, steps=30, rec_dt="f16", io_dt="bf16", strided=True,
                                 pad_rows=[2], force_row0_every=5, seed=4))
    _check(err, TOL_LOW)


@pytest.mark.parametrize("state_dt", ["f32", "f16"])
def test_spec_nemotron_shape(state_dt):
    """Nemotron-3-Super layer shape: 128 heads, 64 x 128, batch 256, L = 16,
    T = 4, bf16 inputs, fp16 records; 4 rows sampled through the oracle (all
    heads), every row on the GPU."""
    err = run_spec_case(SpecCase(B=256, H=128, dv=64, dk=128, L=16, T=4, steps=16, state_dt=state_dt,
                                 rec_dt="f16", io_dt="bf16", a_lo=1.0, a_hi=8.0, sample=[0, 77, 128, 255],
                                 seed=21))
    assert err["flushes"] >= 1
    _check(err, TOL_LOW)


@pytest.mark.parametrize("state_dt", ["f32", "f16"])
def test_spec_T8_nemotron_shape(state_dt):
    """T = 8 at 64 x 128: lane groups of 32 (fp32 state) and 16 (fp16 state)
    lanes, so the reductions over the draft index use both sets of
    select-free levels."""
    err = run_spec_case(SpecCase(B=64, H=128, dv=64, dk=128, L=16, T=8, steps=12, state_dt=state_dt, rec_dt="f16",
                                 io_dt="bf16", a_lo=1.0, a_hi=8.0, sample=[0, 63], seed=22))
    _check(err, TOL_LOW)


def test_spec_commit_rejects_out_of_range_accept():
    """An accepted count outside 0..T commits nothing for that row and is
    counted; the other rows commit normally."""
    lay = rs.layer(rs.MAMBA2, 2, 16, 32, 8, "f32", "f32", "f32", None, 4)
    d = SpecDecodeLayer(lay, 3, 3, "cuda")
    for b in range(3):
        d.assign(b, b)
    d.upload(rows=range(3))
    q = torch.randn(3, 4, 2, 32, device="cuda")
    out = torch.empty(3, 4, 2, 16, device="cuda")
    lam = -torch.rand(3, 4, 2, device="cuda")
    d.verify(rs.make_spec_io(q, q, q[..., :16].contiguous(), lam, out))
    d.commit(torch.tensor([2, 5, -1], dtype=torch.int32, device="cuda"))
    h, fl = d.device_committed()
    assert list(h) == [2, 0, 0] and list(fl) == [0, 0, 0]
    assert int(d.err.item()) == 2
    say("[spec] out-of-range accepted counts rejected")


def test_spec_layer_rejects_standard_step():
    lay = rs.layer(rs.MAMBA2, 2, 16, 32, 8, "f32", "f32", "f32", None, 4)
    d = SpecDecodeLayer(lay, 2, 2, "cuda")
    io = rs.make_io(torch.zeros(2, 2, 32, device="cuda"), torch.zeros(2, 2, 32, device="cuda"),
                    torch.zeros(2, 2, 16, device="cuda"), torch.zeros(2, 2, device="cuda"),
                    torch.zeros(2, 2, 16, device="cuda"))
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.replay_decode_step(lay, d.batch[0], io)
    assert e.value.code == rs.RS_EINVAL


@pytest.mark.parametrize("state_dt,T", [("f32", 4), ("f16", 4), ("f32", 8)])
def test_spec_mamba2_128x128(state_dt, T):
    """Mamba-2 with 128 x 128 heads in one workgroup per tile: batch 32,
    16 heads, L = 16, bf16 inputs, fp16 records; 3 rows sampled."""
    err = run_spec_case(SpecCase(B=32, H=16, dv=128, dk=128, L=16, T=T, steps=16, state_dt=state_dt, rec_dt="f16",
                                 io_dt="bf16", sample=[0, 17, 31], seed=41 + T))
    assert err["flushes"] >= 1
    _check(err, TOL_LOW)


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
@pytest.mark.parametrize("T", [2, 4])
def test_spec_grouped_keys_tiny(form, T):
    """Keys and queries shared by pairs of heads (4 heads, 2 groups), fp32,
    random acceptance with forced flushes: the group's first head stores the
    draft keys, a flushing row's in the staging slots until the commit moves
    the accepted ones to slot 0; every head reads its group's keys."""
    err = run_spec_case(SpecCase(form=form, B=3, H=4, L=8, T=T, steps=40, groups=2, force_row0_every=5,
                                 seed=60 + T))
    assert err["flushes"] >= 3
    (_check_gdn if form == rs.GDN else _check)(err, TOL_F32)


@pytest.mark.parametrize("form,H,groups,shape,T,state_dt", [
    (rs.MAMBA2, 16, 2, (64, 128), 8, "f32"),     # 8 heads per group, as the released Nemotron-H layout
    (rs.MAMBA2, 16, 2, (64, 128), 4, "f16"),
    (rs.GDN, 8, 4, (128, 128), 4, "f32"),
])
def test_spec_grouped_keys(form, H, groups, shape, T, state_dt):
    """Grouped keys at full head sizes: batch 32, L = 16, bf16 inputs,
    fp16 records, strided inputs and a padding row; 3 rows sampled."""
    dv, dk = shape
    err = run_spec_case(SpecCase(form=form, B=32, H=H, dv=dv, dk=dk, L=16, T=T, steps=16, groups=groups,
                                 state_dt=state_dt, rec_dt="f16", io_dt="bf16", strided=True, pad_rows=[5],
                                 sample=[0, 17, 31], seed=70 + T))
    assert err["flushes"] >= 1
    (_check_gdn if form == rs.GDN else _check)(err, TOL_LOW)


def _check_read_copy(err, tol):
    """A read copy moves non-flush outputs away from the exact recurrence by
    its rounding: they are compared with the oracle's two-copy model (which
    reads the device's read copy), the flushed recurrence copy with the
    exact committed state."""
    assert err["out_spec"] <= tol, err
    assert err["ckpt_flush"] <= tol, err


@pytest.mark.parametrize("read_dt", ["f16", "bf16"])
@pytest.mark.parametrize("T", [2, 4])
def test_spec_two_copy_tiny(read_dt, T):
    """Speculative verify over an fp32 recurrence copy and a 16-bit read copy
    (tiny heads, fp32 records and inputs, forced flushes): non-flush outputs
    from the read copy, flushes fold the recurrence copy and store both; the
    read copy is the nearest-even cast of the fp32 fold, bit for bit."""
    err = run_spec_case(SpecCase(B=3, H=4, L=8, T=T, steps=40, read_dt=read_dt, force_row0_every=5, seed=80 + T))
    assert err["flushes"] >= 3
    _check_read_copy(err, TOL_F32)


@pytest.mark.parametrize("read_dt,T,groups,state", [("e4m3", 8, 0, "f32"), ("f16", 4, 0, "f32"),
                                                    ("e4m3", 4, 2, "f32")])
def test_spec_two_copy_nemotron_heads(read_dt, T, groups, state):
    """Nemotron heads (64 x 128), batch 32 x 16 heads, L = 16, bf16 inputs,
    fp16 records, strided inputs and a padding row: E4M3 codes and row
    scales of the read copy are the oracle's encoding of the kernel's fp32
    fold, bit for bit; one case with keys in 2 groups."""
    err = run_spec_case(SpecCase(B=32, H=16, dv=64, dk=128, L=16, T=T, steps=16, groups=groups, state_dt=state,
                                 rec_dt="f16", io_dt="bf16", read_dt=read_dt, strided=True, pad_rows=[5],
                                 sample=[0, 17, 31], seed=85 + T))
    assert err["flushes"] >= 1
    _check_read_copy(err, TOL_LOW)


# ------------------------------------------------------- Gated DeltaNet form --


@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_spec_gdn_tiny_fp32(T):
    """Gated DeltaNet drafts through the triangular solve: tiny heads, fp32,
    random accepted counts, L = 8."""
    err = run_spec_case(SpecCase(form=rs.GDN, T=T, steps=40, seed=30 + T))
    assert err["flushes"] >= 3
    _check_gdn(err, TOL_F32)


@pytest.mark.parametrize("accept", ["all", "none"])
def test_spec_gdn_accept_policies(accept):
    err = run_spec_case(SpecCase(form=rs.GDN, T=4, L=16, steps=30, accept=accept, seed=37))
    _check_gdn(err, TOL_F32)


def test_spec_gdn_strided_padding_forced_lowprec():
    err = run_spec_case(SpecCase(form=rs.GDN, B=4, T=4, L=8, steps=30, rec_dt="f16", io_dt="bf16", strided=True,
                                 pad_rows=[1], force_row0_every=4, seed=38))
    _check_gdn(err, TOL_LOW)


@pytest.mark.parametrize("state_dt", ["f32", "f16"])
def test_spec_gdn_128x128(state_dt):
    """The Gated DeltaNet head (32 heads, 128 x 128, one workgroup per tile),
    batch 64, L = 16, T = 4, bf16 inputs, fp16 records; 3 rows sampled."""
    err = run_spec_case(SpecCase(form=rs.GDN, B=64, H=32, dv=128, dk=128, L=16, T=4, steps=16, state_dt=state_dt,
                                 rec_dt="f16", io_dt="bf16", sample=[0, 31, 63], seed=39))
    assert err["flushes"] >= 1
    _check_gdn(err, TOL_LOW)


def test_spec_gdn_T8_64x128():
    err = run_spec_case(SpecCase(form=rs.GDN, B=16, H=16, dv=64, dk=128, L=16, T=8, steps=12, rec_dt="f16",
                                 io_dt="bf16", sample=[0, 15], seed=40))
    _check_gdn(err, TOL_LOW)


_GDN_MF = {
    "T8-strided-pad-forced": dict(T=8, L=16, rec_dt="f16", io_dt="bf16", strided=True, pad_rows=[5],
                                  force_row0_every=3),
    "T8-fp32-all": dict(T=8, L=16, rec_dt="f32", io_dt="f32", accept="all"),
    "T8-fp32-none": dict(T=8, L=16, rec_dt="f32", io_dt="f32", accept="none"),
    "T1-fp32": dict(T=1, L=8, rec_dt="f32", io_dt="f32"),
    "T2": dict(T=2, L=8, rec_dt="f16", io_dt="bf16"),
    "T4-L4": dict(T=4, L=4, rec_dt="f16", io_dt="bf16"),
    "T8-full-forgetting": dict(T=8, L=16, rec_dt="f16", io_dt="bf16", forget_every=7),
    "T4-L64-fp32-records": dict(T=4, L=64, rec_dt="f32", io_dt="f32", steps=48),
    "64x128-T8-fp32": dict(dv=64, T=8, L=16, rec_dt="f32", io_dt="f32"),
}


@pytest.mark.parametrize("name", list(_GDN_MF))
def test_spec_gdn_fp32_state_on_matrix_cores(name):
    """fp32 state at 128 x 128 (and 64 x 128): at T = 4 and 8 the verify's
    state products S_h [q_1 .. q_T, k_1 .. k_T], the committed records' share
    of them and the flush fold run as 16 x 16 x 4 fp32 matrix products (T = 1
    and 2 take the VALU form), flushes every step (L = 4) or
    with 63 slots of fp32 records (L = 64, more than four 16-record blocks),
    nothing / everything accepted, lam = -inf drafts, strided inputs, padding
    and forced flushes; batch 16, 8 heads, 2 rows sampled."""
    c = dict(dv=128, steps=20, accept="random")
    c.update(_GDN_MF[name])
    err = run_spec_case(SpecCase(form=rs.GDN, B=16, H=8, dk=128, state_dt="f32", sample=[0, 15],
                                 seed=90 + len(name), **c))
    if c["accept"] != "none":
        assert err["flushes"] >= 1
    _check_gdn(err, TOL_F32 if c["rec_dt"] == "f32" and c["io_dt"] == "f32" else TOL_LOW)


_M2_MF = {
    "strided-pad-forced": dict(rec_dt="f16", io_dt="bf16", strided=True, pad_rows=[5], force_row0_every=3),
    "fp32-all": dict(rec_dt="f32", io_dt="f32", accept="all"),
    "fp32-none": dict(rec_dt="f32", io_dt="f32", accept="none"),
    "full-forgetting": dict(rec_dt="f16", io_dt="bf16", forget_every=7, steps=24),
    "L8-every-step": dict(rec_dt="f32", io_dt="f32", L=8),
    "L64-fp32-records": dict(rec_dt="f32", io_dt="f32", L=64, steps=24, accept="all"),
    "128x128": dict(dv=128, rec_dt="f16", io_dt="bf16"),
    "grouped-2": dict(rec_dt="f16", io_dt="bf16", groups=2, H=8, strided=True, pad_rows=[3]),
}


@pytest.mark.parametrize("name", list(_M2_MF))
def test_spec_mamba2_fp32_state_on_matrix_cores(name):
    """Mamba-2 verify at T = 8 over an fp32 state: C [g_1 q_1 .. g_8 q_8], the
    committed and draft values' share (X Wq) and the flush fold run as
    16 x 16 x 4 fp32 matrix products, the outputs stored from the product
    registers.  Strided / padded / forced-flush rows, everything or nothing
    accepted, lam = -inf drafts, a flush every step (L = 8), 63 slots of fp32
    records, 128 x 128 heads, keys shared by pairs of heads; batch 16, 2 rows
    sampled."""
    c = dict(dv=64, H=8, L=16, steps=20, accept="random")
    c.update(_M2_MF[name])
    err = run_spec_case(SpecCase(form=rs.MAMBA2, B=16, dk=128, T=8, state_dt="f32", sample=[0, 15],
                                 seed=120 + len(name), **c))
    if c["accept"] != "none":
        assert err["flushes"] >= 1
    _check(err, TOL_F32 if c["rec_dt"] == "f32" and c["io_dt"] == "f32" else TOL_LOW)


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
@pytest.mark.parametrize("T", [4, 8])
def test_spec_full_forgetting(form, T):
    """lam = -inf (alpha = 0) on every 7th (step, row, draft, head), committed
    records included: the masked draft weights and the committed decay sums
    stay sums of log-decays, so a -inf draft zeroes what comes before it and
    nothing becomes NaN; outputs and flushes against the oracle."""
    err = run_spec_case(SpecCase(form=form, T=T, L=16, steps=24, accept="random", forget_every=7, seed=17 + T))
    assert err["flushes"] >= 1
    _check(err, TOL_F32)
