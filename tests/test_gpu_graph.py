"""Decode steps captured in a HIP graph (through torch.cuda.CUDAGraph) give
the eager launches' results bit for bit, on every replay, with eager work
and synchronisations between the replays.

The cursor, the flush decision and (speculative layers) the commit all live
on the device, so a steady batch needs no host work inside the graph; the
host mirror is advanced after each replay.
"""
import numpy as np
import pytest
import torch

import linear_attention_decode_replay_amd as rs
import workloads
from gpu_harness import say
from linear_attention_decode_replay_amd.state import DecodeLayer, SpecDecodeLayer

pytestmark = pytest.mark.gpu


def _layer_pair(lay, B, seed):
    out = []
    blocks = workloads.shuffled_blocks(seed, B, B + 2)
    for _ in range(2):
        d = DecodeLayer(lay, B, B + 2, "cuda")
        d.pool.raw.zero_()
        for b in range(B):
            d.assign(b, int(blocks[b]))
        d.reset_rows(range(B))
        out.append(d)
    return out, torch.as_tensor(blocks, device="cuda", dtype=torch.long)


@pytest.mark.parametrize("form,shape,L", [(rs.MAMBA2, (16, 32), 4), (rs.GDN, (16, 32), 4),
                                          (rs.MAMBA2, (64, 128), 16)])
def test_decode_steps_in_a_graph(form, shape, L):
    dv, dk = shape
    B, H, n_rep = 3, 4, 2 * L + 1          # replays of 2 steps: several windows, flushes included
    lay = rs.layer(form, H, dv, dk, L, "f32", "f16", "bf16")
    (eager, graphed), blk = _layer_pair(lay, B, 5)
    beta_on = form == rs.GDN

    def tokens(s):
        t = workloads.tokens(form, 7, s, B, H, dv, dk, "bf16")
        return [x.cuda() for x in (t.q, t.k, t.v, t.lam)] + [t.beta.cuda() if beta_on else None]

    # static input and output buffers of the two captured steps
    static = [tokens(0) for _ in range(2)]
    outs = [torch.zeros(B, H, dv, device="cuda") for _ in range(2)]
    ios = [rs.make_io(*static[i][:4], outs[i], static[i][4]) for i in range(2)]
    # one eager step on both layers first (it uploads the metadata)
    t0 = tokens(0)
    o0 = torch.zeros(B, H, dv, device="cuda")
    for d in (eager, graphed):
        d.step(rs.make_io(*t0[:4], o0, t0[4]))
    g = graphed.capture_steps(ios)
    flushes = 0
    for r in range(n_rep):
        for i in range(2):
            for dst, src in zip(static[i], tokens(1 + 2 * r + i)):
                if dst is not None:
                    dst.copy_(src)
        g.replay()
        graphed.advance_host(2)
        for i in range(2):   # the same two steps, eagerly
            t = tokens(1 + 2 * r + i)
            o = torch.zeros(B, H, dv, device="cuda")
            _, fl = eager.step(rs.make_io(*t[:4], o, t[4]))
            flushes += int(fl.any())
            torch.cuda.synchronize()
            assert torch.equal(outs[i], o), f"replay {r}, step {i}"
        assert np.array_equal(graphed.device_cursor(), eager.device_cursor()), f"cursors, replay {r}"
        assert np.array_equal(graphed.anchor, eager.anchor)
    assert flushes >= 2
    assert torch.equal(graphed.pool.ckpt()[blk], eager.pool.ckpt()[blk])
    assert int(graphed.err.item()) == 0 and int(eager.err.item()) == 0
    say(f"[graph] form={form} {dv}x{dk} L={L}: {n_rep} replays of 2 steps bit-exact, {flushes} flush steps")


def test_graph_capture_refuses_pending_work():
    lay = rs.layer(rs.MAMBA2, 2, 16, 32, 4, "f32", "f16", "f32")
    d = DecodeLayer(lay, 2, 2, "cuda")
    d.assign(0, 0)
    with pytest.raises(ValueError):
        d.capture_steps([None, None])     # upload pending
    sr = rs.layer(rs.MAMBA2, 2, 16, 32, 4, "f16", "f16", "f32", stochastic=True)
    with pytest.raises(ValueError):
        DecodeLayer(sr, 2, 2, "cuda").capture_steps([None, None])


@pytest.mark.parametrize("form", [rs.MAMBA2, rs.GDN])
def test_speculative_steps_in_a_graph(form):
    """verify + commit, twice per replay, with the accepted counts written
    into static device tensors before each replay (as a sampler on the
    device would); against the same steps run eagerly."""
    B, H, dv, dk, L, T = 3, 4, 16, 32, 8, 4
    lay = rs.layer(form, H, dv, dk, L, "f32", "f16", "bf16", None, T)
    layers = []
    for _ in range(2):
        d = SpecDecodeLayer(lay, B, B, "cuda")
        d.pool.raw.zero_()
        for b in range(B):
            d.assign(b, b)
        d.upload(rows=range(B))
        layers.append(d)
    eager, graphed = layers

    def drafts(s):
        t = workloads.spec_tokens(9, s, B, H, T, dv, dk, "bf16", form=form)
        return [x.cuda() for x in (t.q, t.k, t.v, t.lam)] + [t.beta.cuda() if t.beta is not None else None]

    static = [drafts(0) for _ in range(2)]
    outs = [torch.zeros(B, T, H, dv, device="cuda") for _ in range(2)]
    ios = [rs.make_spec_io(*static[i][:4], outs[i], static[i][4]) for i in range(2)]
    acc = [torch.zeros(B, dtype=torch.int32, device="cuda") for _ in range(2)]
    # one eager verify + commit on both layers first (kernels loaded, same state)
    d0 = drafts(100)
    for d in layers:
        d.verify(rs.make_spec_io(*d0[:4], torch.zeros(B, T, H, dv, device="cuda"), d0[4]))
        d.commit(torch.full((B,), 2, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    g = graphed.capture_steps(ios, acc)
    flushes = 0
    for r in range(10):
        a = [workloads.spec_accepted(4, 2 * r + i, B, T) for i in range(2)]
        for i in range(2):
            for dst, src in zip(static[i], drafts(2 * r + i)):
                if dst is not None:
                    dst.copy_(src)
            acc[i].copy_(torch.from_numpy(a[i]))
        g.replay()
        for i in range(2):
            d = drafts(2 * r + i)
            o = torch.zeros(B, T, H, dv, device="cuda")
            flushes += int(eager.device_committed()[1].any())
            eager.verify(rs.make_spec_io(*d[:4], o, d[4]))
            eager.commit(torch.from_numpy(a[i]).cuda())
            torch.cuda.synchronize()
            assert torch.equal(outs[i], o), f"replay {r}, step {i}"
        h_g, f_g = graphed.device_committed()
        h_e, f_e = eager.device_committed()
        assert np.array_equal(h_g, h_e) and np.array_equal(f_g, f_e), f"committed counts, replay {r}"
    assert flushes >= 2
    assert torch.equal(graphed.pool.ckpt()[:B], eager.pool.ckpt()[:B])
    assert int(graphed.err.item()) == 0 and int(eager.err.item()) == 0
    say(f"[graph] speculative form={form}: 10 replays of 2 verify + commit steps bit-exact")
