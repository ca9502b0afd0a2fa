"""C ABI on the CPU: symbols, block layout, validation, host metadata.

No GPU work here: device entry points are only called with arguments that
fail host-side validation or with n_rows == 0 (which launches nothing)."""
import ctypes
import os
import re

import numpy as np
import pytest

import linear_attention_decode_replay_amd as rs
import oracle

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "replayssm.h")


def _declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert {"replay_decode_step", "replay_flush", "conventional_decode_step", "replay_state_reset",
            "rs_block_layout_get", "rs_meta_step", "rs_meta_advance", "rs_last_error"} <= set(names)
    lib = ctypes.CDLL(rs.LIBRARY_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in replayssm.h but not exported"


def _c2(**kw):
    args = dict(form=rs.MAMBA2, n_heads=128, d_v=64, d_k=128, L=16, state_dtype="f32",
                record_dtype="f16", io_dtype="bf16")
    args.update(kw)
    return rs.layer(**args)


def test_block_layout_nemotron_layer():
    lay = rs.block_layout(_c2())
    assert lay.ckpt_off == 0
    assert lay.rec_x_off == 4 * 2**20            # the 4 MiB checkpoint
    assert lay.slots == 15
    assert lay.rec_k_off == lay.rec_x_off + 128 * 15 * 64 * 2
    assert lay.rec_lam_off == lay.rec_k_off + 128 * 15 * 128 * 2
    assert lay.block_bytes == lay.rec_lam_off + 128 * 15 * 4   # already 256-aligned
    for off in (lay.rec_x_off, lay.rec_k_off, lay.rec_lam_off, lay.block_bytes):
        assert off % 256 == 0


@pytest.mark.parametrize("L", [1, 2, 16, 64])
@pytest.mark.parametrize("shape", [(16, 32), (64, 128), (128, 128)])
@pytest.mark.parametrize("sdt,rdt", [("f32", "f32"), ("f16", "f16"), ("f32", "f16")])
def test_block_layout_regions_disjoint(L, shape, sdt, rdt):
    dv, dk = shape
    layer = _c2(n_heads=3, d_v=dv, d_k=dk, L=L, state_dtype=sdt, record_dtype=rdt)
    if rs.layer_supported(layer) != rs.RS_OK:
        pytest.skip(rs.last_error())
    lay = rs.block_layout(layer)
    sb, rb = (4 if sdt == "f32" else 2), (4 if rdt == "f32" else 2)
    ends = [(lay.ckpt_off, 3 * dv * dk * sb), (lay.rec_x_off, 3 * (L - 1) * dv * rb),
            (lay.rec_k_off, 3 * (L - 1) * dk * rb), (lay.rec_lam_off, 3 * (L - 1) * 4)]
    for (a, na), (b, _) in zip(ends, ends[1:]):
        assert a + na <= b
    assert ends[-1][0] + ends[-1][1] <= lay.block_bytes and lay.block_bytes % 256 == 0


@pytest.mark.parametrize("bad,code", [
    (dict(L=0), rs.RS_EINVAL), (dict(L=65), rs.RS_EINVAL), (dict(form=7), rs.RS_EINVAL),
    (dict(n_heads=0), rs.RS_EINVAL), (dict(d_v=32, d_k=32), rs.RS_EUNSUPPORTED),
    (dict(state_dtype="bf16"), rs.RS_EUNSUPPORTED), (dict(io_dtype=9), rs.RS_EINVAL),
])
def test_layer_validation(bad, code):
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.block_layout(_c2(**bad))
    assert e.value.code == code
    assert rs.last_error()


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
@pytest.mark.parametrize("spec_T", [0, 8])
def test_largest_buffers_fit_the_workgroup_lds(form, spec_T):
    """L = 64 with fp32 records at 128 x 128 (the largest record area) is
    supported: its records fit one gfx950 workgroup's LDS."""
    if spec_T and form == rs.MAMBA2:
        shape = dict(d_v=64, d_k=128)   # the Mamba-2 verify's largest head
    else:
        shape = dict(d_v=128, d_k=128)
    layer = _c2(form=form, L=64, record_dtype="f32", state_dtype="f32", io_dtype="f32", spec_T=spec_T, **shape)
    assert rs.layer_supported(layer) == rs.RS_OK, rs.last_error()
    assert rs.block_layout(layer).slots == (64 if spec_T else 63)


def test_empty_batch_launches_nothing():
    layer = _c2()
    empty = rs.RsBatch(0, 0, 1, None, None, None, None, None)
    io = rs.RsStepIO()
    rs.replay_decode_step(layer, empty, io, stream=0)
    rs.conventional_decode_step(layer, empty, io, stream=0)
    rs.replay_flush(layer, empty, stream=0)
    rs.replay_state_reset(layer, empty, None, stream=0)


def test_device_calls_reject_bad_arguments_on_host():
    layer = _c2()
    buf = (ctypes.c_uint8 * 512)()
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    batch = rs.RsBatch(4, 0, 4, None, base, base, None, None)      # NULL pool
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.replay_decode_step(layer, batch, rs.RsStepIO(), stream=0)
    assert e.value.code == rs.RS_EINVAL and "pool" in rs.last_error()
    batch = rs.RsBatch(4, 0, 4, base + 8, base, base, None, None)  # misaligned pool
    with pytest.raises(rs.ReplaySSMError):
        rs.replay_decode_step(layer, batch, rs.RsStepIO(), stream=0)
    batch = rs.RsBatch(4, 0, 4, base, base, base, None, None)
    io = rs.RsStepIO(base, base, base, 128 * 128, 128, 128 * 128, 128, 128 * 64, 64, base, None, base)
    io.q = base + 8                                                # misaligned q
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.replay_decode_step(layer, batch, io, stream=0)
    assert "q" in rs.last_error()
    io.q = base
    io.k_head_stride = 100                                         # head stride < d_k
    with pytest.raises(rs.ReplaySSMError):
        rs.replay_decode_step(layer, batch, io, stream=0)
    io.k_head_stride = 128
    with pytest.raises(rs.ReplaySSMError) as e:                    # GDN needs beta
        rs.replay_decode_step(_c2(form=rs.GDN), batch, io, stream=0)
    assert "beta" in rs.last_error()
    with pytest.raises(rs.ReplaySSMError):                         # token-less flush needs flags
        rs.replay_flush(layer, batch, stream=0)
    with pytest.raises(rs.ReplaySSMError):                         # reset needs a mask
        rs.replay_state_reset(layer, batch, None, stream=0)


# ------------------------------------------------------------ host metadata --
def _run_meta(L, n_steps, w0, forced=None):
    """Drive rs_meta_step / rs_meta_advance for one row over n_steps."""
    anchor = np.array([w0], np.int32)
    ws, fs = [], []
    for s in range(n_steps):
        f = None if forced is None else np.array([forced[s]], np.uint8)
        wp, fl = rs.rs_meta_step(L, anchor, f)
        ws.append(int(wp[0]))
        fs.append(bool(fl[0]))
        rs.rs_meta_advance(L, anchor, fl)
    return np.array(ws, np.int32), np.array(fs)


@pytest.mark.parametrize("L", [1, 2, 4, 16, 64])
def test_meta_matches_oracle_cursor(L):
    orc = oracle.get()
    rng = np.random.default_rng(L)
    for w0 in sorted({0, L // 2, L - 1}):
        for forced in (None, (rng.random(3 * L + 7) < 0.15).astype(np.uint8)):
            w, f = _run_meta(L, 3 * L + 7, w0, forced)
            ow, of = orc.cursor_run(L, w0, 3 * L + 7, forced)
            assert np.array_equal(w, ow) and np.array_equal(f, of), (L, w0)


def test_meta_cases():
    """Fresh decode, flush boundary, buffer wrap, resume re-anchor, pad rows
    and per-row independence in one batch."""
    L = 16
    anchor = np.array([0, 14, 15, 40, -1, 3], np.int32)   # row 3: anchor counted past L (wraps)
    force = np.array([0, 0, 0, 0, 1, 1], np.uint8)        # pad row ignores its force flag
    wp, fl = rs.rs_meta_step(L, anchor, force)
    assert list(wp) == [0, 14, 15, 8, 0, 3]
    assert list(fl) == [0, 0, 1, 0, 0, 1]
    rs.rs_meta_advance(L, anchor, fl)
    assert list(anchor) == [1, 15, 0, 41, -1, 0]
    # resume after preemption: the caller re-anchors the row at 0
    anchor[3] = 0
    wp, fl = rs.rs_meta_step(L, anchor)
    assert wp[3] == 0 and fl[3] == 0 and wp[1] == 15 and fl[1] == 1


def test_meta_rejects_bad_arguments():
    with pytest.raises(rs.ReplaySSMError):
        rs.rs_meta_step(0, np.zeros(3, np.int32))
    with pytest.raises(rs.ReplaySSMError):
        rs.rs_meta_step(65, np.zeros(3, np.int32))


# ----------------------------------------------------- speculative layers --
def test_spec_block_layout_ring_of_L():
    """A speculative layer's ring holds L committed records (the standard
    buffer L - 1)."""
    lay = rs.block_layout(_c2(spec_T=4))
    assert lay.slots == 16
    assert lay.rec_k_off == lay.rec_x_off + 128 * 16 * 64 * 2
    assert lay.block_bytes == lay.rec_lam_off + 128 * 16 * 4


@pytest.mark.parametrize("bad,code", [
    (dict(spec_T=3), rs.RS_EUNSUPPORTED), (dict(spec_T=8, L=4), rs.RS_EINVAL),
    (dict(spec_T=-1), rs.RS_EINVAL),
    (dict(spec_T=4, form=rs.GDN, d_v=32, d_k=64), rs.RS_EUNSUPPORTED),
    (dict(spec_T=4, form=rs.GDN, read_dtype="f16"), rs.RS_EUNSUPPORTED),
    (dict(spec_T=4, state_dtype="f16", read_dtype="e4m3"), rs.RS_EUNSUPPORTED),
])
def test_spec_layer_validation(bad, code):
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.block_layout(_c2(**bad))
    assert e.value.code == code and rs.last_error()


@pytest.mark.parametrize("read", ["f16", "bf16", "e4m3"])
def test_spec_layer_with_read_copy(read):
    """A speculative Mamba-2 layer over an fp32 recurrence copy may keep a
    read copy: the block holds both copies (and E4M3 row scales)."""
    lay = rs.block_layout(_c2(spec_T=4, read_dtype=read))
    assert lay.ckpt_lo_off >= lay.rec_lam_off + 128 * 16 * 4
    assert (lay.ckpt_scale_off > 0) == (read == "e4m3")


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
@pytest.mark.parametrize("state", ["f32", "f16"])
def test_spec_layer_128x128_is_supported(form, state):
    lay = rs.block_layout(_c2(spec_T=8, form=form, d_v=128, d_k=128, state_dtype=state))
    assert lay.slots == 16


def test_spec_device_calls_reject_bad_arguments_on_host():
    spec, std = _c2(spec_T=4), _c2()
    buf = (ctypes.c_uint8 * 1024)()
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    batch = rs.RsBatch(4, 0, 4, base, base, base, None, None, base + 256)
    io = rs.RsSpecIO(base, base, base, 4 * 128 * 128, 128 * 128, 128, 4 * 128 * 128, 128 * 128, 128,
                     4 * 128 * 64, 128 * 64, 64, base, base)
    with pytest.raises(rs.ReplaySSMError) as e:                    # standard step on a speculative layer
        rs.replay_decode_step(spec, batch, rs.RsStepIO(), stream=0)
    assert e.value.code == rs.RS_EINVAL
    with pytest.raises(rs.ReplaySSMError) as e:                    # verify on a standard layer
        rs.replay_spec_verify(std, batch, io, stream=0)
    assert e.value.code == rs.RS_EINVAL
    io.q_token_stride = 100                                        # tokens overlap
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.replay_spec_verify(spec, batch, io, stream=0)
    assert "token stride" in rs.last_error()
    io.q_token_stride = 128 * 128
    io.k_row_stride = 2 * 128 * 128                                # rows overlap T tokens
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.replay_spec_verify(spec, batch, io, stream=0)
    assert "row stride" in rs.last_error()
    acc = (ctypes.c_int32 * 4)()
    nf = (ctypes.c_uint8 * 4)()
    with pytest.raises(rs.ReplaySSMError):                         # accepted NULL
        rs._check(rs._lib.replay_spec_commit(ctypes.byref(spec), ctypes.byref(batch), None,
                                              ctypes.addressof(nf), None))
    nb = rs.RsBatch(4, 0, 4, base, base, base, None, None, None)
    with pytest.raises(rs.ReplaySSMError) as e:                    # next_write_pos NULL
        rs._check(rs._lib.replay_spec_commit(ctypes.byref(spec), ctypes.byref(nb), ctypes.addressof(acc),
                                              ctypes.addressof(nf), None))
    assert "next_write_pos" in rs.last_error()
    empty = rs.RsBatch(0, 0, 1, None, None, None, None, None)
    rs.replay_spec_verify(spec, empty, rs.RsSpecIO(), stream=0)    # nothing to launch


@pytest.mark.parametrize("L,T", [(8, 1), (8, 4), (16, 4), (16, 8), (64, 8)])
def test_spec_meta_matches_oracle_cursor(L, T):
    """Host flush rule and commit, bit-exact against the oracle's own
    derivation of the speculative cursor, with random accepted counts and
    forced flushes."""
    orc = oracle.get()
    rng = np.random.default_rng(L * 10 + T)
    n = 6 * L
    acc = rng.integers(0, T + 1, n).astype(np.int32)
    forced = (rng.random(n) < 0.1).astype(np.uint8)
    for h0 in sorted({0, L // 2, L - T + 1 if L - T + 1 >= 0 else 0}):
        h = np.array([h0], np.int32)
        hs, fs = [], []
        for s in range(n):
            fl = rs.rs_spec_meta_step(L, T, h, forced[s:s + 1])
            hs.append(int(h[0]))
            fs.append(bool(fl[0]))
            rs.rs_spec_meta_advance(L, T, h, fl, acc[s:s + 1])
        oh, of = orc.spec_cursor_run(L, T, h0, acc, forced)
        assert np.array_equal(np.array(hs), oh) and np.array_equal(np.array(fs), of), (L, T, h0)


def test_spec_meta_pad_rows_and_bad_arguments():
    h = np.array([-1, 12, 13], np.int32)
    fl = rs.rs_spec_meta_step(16, 4, h, np.array([1, 0, 0], np.uint8))
    assert list(fl) == [0, 0, 1]
    rs.rs_spec_meta_advance(16, 4, h, fl, np.array([3, 4, 2], np.int32))
    assert list(h) == [-1, 16, 2]
    with pytest.raises(rs.ReplaySSMError):
        rs.rs_spec_meta_step(16, 17, h)
    with pytest.raises(rs.ReplaySSMError):
        rs.rs_spec_meta_step(16, 0, h)
    # an accepted count outside 0..T is an error and moves no row (a padding
    # row's count is not looked at)
    for bad in ([0, 5, 1], [0, 1, -1]):
        h2 = np.array([-1, 3, 7], np.int32)
        with pytest.raises(rs.ReplaySSMError) as e:
            rs.rs_spec_meta_advance(16, 4, h2, np.zeros(3, np.uint8), np.array(bad, np.int32))
        assert e.value.code == rs.RS_EINVAL and "accepted" in rs.last_error()
        assert list(h2) == [-1, 3, 7]
    h3 = np.array([-1, 3], np.int32)
    rs.rs_spec_meta_advance(16, 4, h3, np.zeros(2, np.uint8), np.array([99, 4], np.int32))
    assert list(h3) == [-1, 7]


# ------------------------------------------------------------ grouped keys --
def test_grouped_block_layout():
    """128 heads in 8 key groups: the key ring holds 8 x 15 records."""
    lay = rs.block_layout(_c2(n_groups=8))
    assert lay.rec_k_off == lay.rec_x_off + 128 * 15 * 64 * 2
    assert lay.rec_lam_off == lay.rec_k_off + 8 * 15 * 128 * 2
    per = rs.block_layout(_c2())
    assert per.rec_lam_off - per.rec_k_off == 16 * (lay.rec_lam_off - lay.rec_k_off)


def test_grouped_speculative_block_layout():
    """A speculative layer with 8 key groups: each group's key ring holds L
    committed records plus T staging slots (the drafts of a row that flushed
    in its verify, until the commit moves them); per-head keys need none."""
    lay = rs.block_layout(_c2(n_groups=8, spec_T=4))
    assert lay.slots == 16 and lay.key_slots == 20
    assert lay.rec_lam_off == lay.rec_k_off + 8 * 20 * 128 * 2
    per = rs.block_layout(_c2(spec_T=4))
    assert per.key_slots == per.slots == 16
    std = rs.block_layout(_c2(n_groups=8))
    assert std.key_slots == std.slots == 15


@pytest.mark.parametrize("bad,code", [
    (dict(n_groups=3), rs.RS_EINVAL), (dict(n_groups=-1), rs.RS_EINVAL),
    (dict(n_groups=3, spec_T=4), rs.RS_EINVAL),
])
def test_grouped_layer_validation(bad, code):
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.block_layout(_c2(**bad))
    assert e.value.code == code


def test_grouped_io_strides():
    """q / k rows of a grouped layer hold n_groups vectors."""
    layer = _c2(n_groups=8)
    buf = (ctypes.c_uint8 * 512)()
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    batch = rs.RsBatch(4, 0, 4, base, base, base, None, None)
    io = rs.RsStepIO(base, base, base, 8 * 128, 128, 7 * 128, 128, 128 * 64, 64, base, None, base)
    with pytest.raises(rs.ReplaySSMError) as e:                    # k rows shorter than 8 groups
        rs.replay_decode_step(layer, batch, io, stream=0)
    assert "row strides" in rs.last_error()


def test_grouped_speculative_io_strides():
    """Draft q / k tokens of a grouped speculative layer hold n_groups
    vectors (v tokens n_heads): a token stride of 7 groups is rejected."""
    layer = _c2(n_groups=8, spec_T=4)
    buf = (ctypes.c_uint8 * 1024)()
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    batch = rs.RsBatch(4, 0, 4, base, base, base, None, None, base + 256)
    io = rs.RsSpecIO(base, base, base, 4 * 8 * 128, 8 * 128, 128, 4 * 7 * 128, 7 * 128, 128,
                     4 * 128 * 64, 128 * 64, 64, base, base)
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.replay_spec_verify(layer, batch, io, stream=0)
    assert e.value.code == rs.RS_EINVAL and "k token stride" in rs.last_error()


# ------------------------------------------------------ stochastic rounding --
def _rounded(mode, **kw):
    lay = _c2(**kw)
    lay.state_rounding = mode
    return lay


@pytest.mark.parametrize("mode,kw,code", [
    (2, dict(), rs.RS_EINVAL), (-1, dict(), rs.RS_EINVAL),
    (rs.RS_ROUND_STOCHASTIC, dict(), rs.RS_EUNSUPPORTED),                      # fp32 state
    (rs.RS_ROUND_STOCHASTIC, dict(state_dtype="f16", read_dtype="bf16"), rs.RS_EUNSUPPORTED),
])
def test_rounding_validation(mode, kw, code):
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.block_layout(_rounded(mode, **kw))
    assert e.value.code == code


@pytest.mark.parametrize("state,read,code", [
    ("f32", "f16", rs.RS_OK), ("f32", "bf16", rs.RS_OK), ("f32", "e4m3", rs.RS_OK), ("f16", "e4m3", rs.RS_OK),
    ("f16", "bf16", rs.RS_EUNSUPPORTED), ("f16", "f32", rs.RS_EUNSUPPORTED),
])
def test_two_precision_pairings(state, read, code):
    """Recurrence copy / read copy pairs: fp32 under any read copy, fp16
    under E4M3 only."""
    lay = _c2(state_dtype=state, read_dtype=read)
    assert rs.layer_supported(lay) == code
    if code == rs.RS_OK:
        b = rs.block_layout(lay)
        elem = 128 * 64 * 128
        assert b.ckpt_lo_off >= b.ckpt_off + elem * (4 if state == "f32" else 2)
        if read == "e4m3":
            assert b.ckpt_scale_off >= b.ckpt_lo_off + elem


def test_stochastic_rounding_layers_accepted():
    """An fp16 state with stochastic rounding: standard, grouped and
    speculative layers and an fp16 recurrence copy under an E4M3 read copy;
    the block layout is the nearest-even one's."""
    for extra in (dict(), dict(n_groups=8), dict(spec_T=4), dict(read_dtype="e4m3")):
        lay = rs.block_layout(_c2(state_dtype="f16", stochastic=True, **extra))
        ref = rs.block_layout(_c2(state_dtype="f16", **extra))
        assert (lay.block_bytes, lay.ckpt_off, lay.rec_k_off) == (ref.block_bytes, ref.ckpt_off, ref.rec_k_off)
        assert rs.layer_supported(_c2(state_dtype="f16", stochastic=True, **extra)) == rs.RS_OK


def test_batch_struct_carries_key_and_counter():
    b = rs.RsBatch(4, 0, 4, None, None, None, None, None, None, 2**64 - 1, 5, 2**63 + 7)
    assert (b.sr_key0, b.sr_key1, b.sr_step) == (2**64 - 1, 5, 2**63 + 7)
    # 2 int32 + int64 + 6 pointers + 3 uint64; 13 int32
    assert ctypes.sizeof(rs.RsBatch) == 88
    assert ctypes.sizeof(rs.RsLayer) == 52


@pytest.mark.parametrize("state,read", [("f32", "f16"), ("f32", "bf16"), ("f32", "e4m3"), ("f16", "e4m3")])
def test_read_copy_columns_permutation(state, read):
    """The read copy's lane order is a permutation of the columns, with each
    16-byte read chunk holding whole recurrence-copy chunks (contiguous runs
    of 16 / element size columns)."""
    lay = _c2(state_dtype=state, read_dtype=read)
    cols = rs.read_copy_columns(lay)
    assert sorted(cols) == list(range(128))
    m = 4 if state == "f32" else 2
    run = 16 // m
    assert all(cols[i + 1] == cols[i] + 1 for i in range(128) if (i + 1) % run and i + 1 < 128)


@pytest.mark.parametrize("route,form,code", [
    (rs.RS_GDN_RECONSTRUCT, rs.GDN, rs.RS_OK), (rs.RS_GDN_OUTPUT_ONLY, rs.GDN, rs.RS_OK),
    (rs.RS_GDN_RECONSTRUCT, rs.MAMBA2, rs.RS_EINVAL), (2, rs.GDN, rs.RS_EINVAL), (-1, rs.GDN, rs.RS_EINVAL),
])
def test_gdn_route_validation(route, form, code):
    lay = rs.layer(form, 32, 128, 128, 16, "f32", "f16", "bf16")
    lay.gdn_route = route
    assert rs.layer_supported(lay) == code
    if code == rs.RS_OK:   # the route changes no layout
        assert rs.block_layout(lay).block_bytes == rs.block_layout(rs.layer(form, 32, 128, 128, 16, "f32", "f16",
                                                                            "bf16")).block_bytes


def test_flush_hint_validation():
    layer = _c2()
    buf = (ctypes.c_uint8 * 512)()
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    io = rs.RsStepIO(base, base, base, 128 * 128, 128, 128 * 128, 128, 128 * 64, 64, base, None, base)
    for bad in (-1, 4):
        batch = rs.RsBatch(4, bad, 4, base, base, base, None, None)
        with pytest.raises(rs.ReplaySSMError) as e:
            rs.replay_decode_step(layer, batch, io, stream=0)
        assert e.value.code == rs.RS_EINVAL and "flush_hint" in rs.last_error()


def test_gdn_spec_layers_accepted():
    """Gated DeltaNet speculative layers at 16 x 32, 64 x 128 and 128 x 128;
    the verify needs beta."""
    for dv, dk in ((16, 32), (64, 128), (128, 128)):
        lay = rs.layer(rs.GDN, 4, dv, dk, 16, "f32", "f16", "bf16", None, 4)
        assert rs.layer_supported(lay) == rs.RS_OK
        assert rs.block_layout(lay).slots == 16
    layer = rs.layer(rs.GDN, 2, 16, 32, 8, "f32", "f32", "f32", None, 2)
    buf = (ctypes.c_uint8 * 4096)()
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    batch = rs.RsBatch(1, 0, 1, base, base, base, None, None)
    io = rs.RsSpecIO(base, base, base, 2 * 2 * 32, 2 * 32, 32, 2 * 2 * 32, 2 * 32, 32, 2 * 2 * 16, 2 * 16, 16,
                     base, base, None)
    with pytest.raises(rs.ReplaySSMError) as e:
        rs.replay_spec_verify(layer, batch, io, stream=0)
    assert e.value.code == rs.RS_EINVAL and "beta" in rs.last_error()
