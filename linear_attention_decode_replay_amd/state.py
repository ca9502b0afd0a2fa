"""Host-side state of one SSM layer for a batch of request slots.

Owns the paged block pool (device memory from torch), the per-slot block
assignment and each slot's anchor (decode steps since its checkpoint was
last anchored), and drives the C ABI once per step:

  1. ``rs_meta_step`` (C, host) turns anchors into the step's write
     positions and flush flags (vLLM pull request "[Kernel] ReplaySSM: cache
     SSM inputs for faster Gated DeltaNet standard decode", section "CUDA
     graphs and continuous batching": position = steps since anchor mod L,
     flush at position L-1 or when forced);
  2. one kernel launch serves flush and non-flush rows alike;
  3. ``rs_meta_advance`` re-anchors the rows that flushed.

The device keeps its own copy of the cursors: each replay step writes every
row's next cursor (0 after a flush, else w + 1, the rule of step 3) into the
second of two cursor arrays, and the next step reads it.  Host and device
therefore stay equal by construction, and the host copies metadata to the
device (one asynchronous copy from pinned memory, no device -> host sync)
only when it changes: a slot joins or retires, a flush is forced (and on the
step after, to clear the flag), or rows are re-anchored.  In steady decoding
a step is a single kernel launch.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (RS_CURSOR_ZERO_CKPT, RS_FLUSH_ALL, RS_FLUSH_MIXED, RS_FLUSH_NONE, RS_FLUSH_UNKNOWN, Pool, RsLayer,
               conventional_decode_step, make_batch, replay_decode_step, replay_flush, replay_spec_commit,
               replay_spec_verify, replay_state_reset, rs_meta_advance, rs_meta_step)


def _layout(n: int):
    """Byte offsets of the per-row arrays in one metadata buffer, each 4-byte
    aligned: block_table int32, flush uint8, mask uint8, cursor0 int32,
    cursor1 int32."""
    n4 = (n + 3) // 4 * 4
    off = {"bt": 0, "fl": 4 * n, "mk": 4 * n + n4, "c0": 4 * n + 2 * n4, "c1": 8 * n + 2 * n4}
    return off, 12 * n + 2 * n4


def _views(buf: torch.Tensor, n: int):
    off, _ = _layout(n)
    return (buf[off["bt"]:off["bt"] + 4 * n].view(torch.int32), buf[off["fl"]:off["fl"] + n],
            buf[off["mk"]:off["mk"] + n], buf[off["c0"]:off["c0"] + 4 * n].view(torch.int32),
            buf[off["c1"]:off["c1"] + 4 * n].view(torch.int32))


class _Stage:
    """Pinned host image of the metadata buffer (one upload in flight)."""

    def __init__(self, n: int):
        _, size = _layout(n)
        self.buf = torch.zeros(size, dtype=torch.uint8, pin_memory=True)
        self.bt, self.fl, self.mk, c0, c1 = (t.numpy() for t in _views(self.buf, n))
        self.c = (c0, c1)
        self.event = None


class DecodeLayer:
    """n_layers > 1: that many layers of the same shape (one pool each) over
    the same request slots, as the layers of a model are: they share the
    block table, the cursors and the flags (one metadata buffer, one upload
    per step), and step() takes one rs_step_io per layer and launches them in
    order; each launch writes the same next cursors."""

    def __init__(self, lay: RsLayer, n_slots: int, n_blocks: int | None = None, device="cuda",
                 staging: int = 4, sr_key=(0, 0), n_layers: int = 1):
        self.layer = lay
        self.L = int(lay.L)
        self.n_slots = n = int(n_slots)
        self.pools = [Pool(lay, n_blocks or n_slots, device) for _ in range(int(n_layers))]
        self.pool = self.pools[0]
        self.device = self.pool.raw.device
        self.anchor = np.full(n, -1, np.int32)   # -1: empty slot (padding row)
        self.blocks = np.full(n, -1, np.int32)
        # rows whose checkpoint counts as zero until their first flush
        # (joined with join_rows; RS_CURSOR_ZERO_CKPT in the cursor word)
        self.zero_ckpt = np.zeros(n, bool)
        _, size = _layout(n)
        self.meta = torch.zeros(size, dtype=torch.uint8, device=self.device)
        self.block_table, self.flush, self.mask, c0, c1 = _views(self.meta, n)
        self.cursor = (c0, c1)
        self.err = torch.zeros(1, dtype=torch.int32, device=self.device)
        # batches[layer][i] reads cursor i and writes the next cursors into
        # cursor 1-i (each layer its own stochastic-rounding key)
        self.batches = [[make_batch(pl.raw, pl.n_blocks, self.block_table, self.cursor[i], self.flush, self.err,
                                    next_write_pos=self.cursor[1 - i], sr_key=(sr_key[0] + li, sr_key[1]))
                         for i in (0, 1)] for li, pl in enumerate(self.pools)]
        self.batch = self.batches[0]
        # stochastic rounding: the counter's first word, one value per launch
        self.sr_step = 0
        # tell the library which rows flush (it then runs the kernel built
        # without the fold wherever it can); False: RS_FLUSH_UNKNOWN always
        self.flush_hints = True
        self._cur = 0
        self._stages = [_Stage(n) for _ in range(staging)]
        self._next = 0
        self._dirty = True          # device metadata differs from the host's
        self._forced_last = False   # the device flag array holds forced flags
        self.uploads = 0

    # ---------------------------------------------------------- bookkeeping --
    def assign(self, slot: int, block: int, steps_since_anchor: int = 0) -> None:
        """Place a request in `slot` on pool block `block`."""
        if not 0 <= block < self.pool.n_blocks:
            raise ValueError(f"block {block} outside the pool of {self.pool.n_blocks}")
        self.blocks[slot] = block
        self.anchor[slot] = steps_since_anchor
        self.zero_ckpt[slot] = False
        self._dirty = True

    def retire(self, slot: int) -> None:
        self.blocks[slot] = -1
        self.anchor[slot] = -1
        self.zero_ckpt[slot] = False
        self._dirty = True

    def live(self) -> np.ndarray:
        return self.blocks >= 0

    def device_cursor(self, words: bool = False) -> np.ndarray:
        """The device's cursors for the next step (synchronises; for tests):
        the record counts, or with words=True the cursor words
        (RS_CURSOR_ZERO_CKPT included)."""
        torch.cuda.synchronize(self.device)
        c = self.cursor[self._cur].cpu().numpy()
        return c if words else np.where(c >= 0, c & ~RS_CURSOR_ZERO_CKPT, c)

    def _words(self, wp) -> np.ndarray:
        """Cursor words of the rows: the record count, with
        RS_CURSOR_ZERO_CKPT on live rows whose checkpoint is still zero."""
        return np.where(self.zero_ckpt & self.live(), np.asarray(wp, np.int32) | RS_CURSOR_ZERO_CKPT,
                        np.asarray(wp, np.int32)).astype(np.int32)

    # ------------------------------------------------------------- transfers --
    def _upload(self, stream, wp, flags=None, mask=None) -> None:
        """One async host -> device copy of block table, flags, mask and the
        current cursor array."""
        st = self._stages[self._next]
        self._next = (self._next + 1) % len(self._stages)
        if st.event is not None:
            st.event.synchronize()  # the previous copy out of this buffer is done
        st.bt[:] = self.blocks
        st.fl[:] = 0 if flags is None else flags
        st.mk[:] = 0 if mask is None else mask
        st.c[self._cur][:] = self._words(wp)
        off, _ = _layout(self.n_slots)
        with torch.cuda.stream(stream):
            if self._cur == 0:
                end = off["c1"]
                self.meta[:end].copy_(st.buf[:end], non_blocking=True)
            else:
                self.meta[:off["c0"]].copy_(st.buf[:off["c0"]], non_blocking=True)
                end = off["c1"] + 4 * self.n_slots
                self.meta[off["c1"]:end].copy_(st.buf[off["c1"]:end], non_blocking=True)
            st.event = torch.cuda.Event()
            st.event.record(stream)
        self.uploads += 1

    def _batch(self, hint=RS_FLUSH_UNKNOWN, layer: int = 0):
        """The batch struct for the next launch, stamped with a fresh
        stochastic-rounding counter word and the flush hint."""
        b = self.batches[layer][self._cur]
        b.sr_step = self.sr_step
        b.flush_hint = hint
        self.sr_step += 1
        return b

    def _hint(self, fl) -> int:
        live = self.live()
        if not self.flush_hints or not live.any():
            return RS_FLUSH_UNKNOWN
        n = int(np.count_nonzero(np.asarray(fl)[live]))
        if n == 0:
            return RS_FLUSH_NONE
        return RS_FLUSH_ALL if n == int(live.sum()) else RS_FLUSH_MIXED

    # ----------------------------------------------------------------- steps --
    def _per_layer(self, io, events):
        if len(self.pools) == 1:
            return [io], [events]
        if len(io) != len(self.pools):
            raise ValueError(f"{len(self.pools)} layers: one rs_step_io per layer")
        return list(io), list(events) if events else [None] * len(io)

    def step(self, io, force: np.ndarray | None = None, stream=None, events=None):
        """One checkpoint + buffer decode step.  Returns the host (write_pos,
        flush) arrays that were used.  `events` = (start, end) torch events
        recorded on the stream right around the kernel launch (with several
        layers: io and events are lists, one entry per layer)."""
        stream = stream or torch.cuda.current_stream(self.device)
        ios, evs = self._per_layer(io, events)
        wp, fl = rs_meta_step(self.L, self.anchor, force)
        forced = None
        if force is not None:
            forced = (np.asarray(force, bool) & self.live()).astype(np.uint8)
            if not forced.any():
                forced = None
        if self._dirty or forced is not None or self._forced_last:
            self._upload(stream, wp, forced)
            self._forced_last = forced is not None
            self._dirty = False
        hint = self._hint(fl)
        for li, (io_l, ev) in enumerate(zip(ios, evs)):
            if ev:
                ev[0].record(stream)
            replay_decode_step(self.layer, self._batch(hint, li), io_l, stream)
            if ev:
                ev[1].record(stream)
        self._cur ^= 1
        rs_meta_advance(self.L, self.anchor, fl)
        self.zero_ckpt &= ~(np.asarray(fl, bool) & self.live())  # a flush wrote the checkpoint
        return wp, fl

    def capture_steps(self, ios, stream=None):
        """Capture consecutive checkpoint + buffer steps into a HIP graph
        (PR "CUDA graphs and continuous batching": the cursor and the flush
        decision live on the device, so a steady decode loop can be
        captured).  ios: one rs_step_io per step, an even number of them (the
        graph returns the cursor arrays to the parity it started from); the
        caller refreshes the buffers behind them before each replay and calls
        advance_host(len(ios)) after it.  The batch must be steady: no upload
        pending, no forced flush, no stochastic rounding (its counter would be
        fixed in the graph).  Every step runs one kernel over all rows."""
        if len(ios) % 2:
            raise ValueError("capture an even number of steps")
        if self.layer.state_rounding:
            raise ValueError("stochastic rounding draws a fresh counter per launch: no graph capture")
        if len(self.pools) != 1:
            raise ValueError("graph capture of one layer at a time")
        if self._dirty or self._forced_last:
            raise ValueError("metadata upload pending: run an eager step first")
        stream = stream or torch.cuda.Stream(self.device)
        stream.wait_stream(torch.cuda.current_stream(self.device))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            cur = self._cur
            for io in ios:
                b = self.batch[cur]
                b.flush_hint = RS_FLUSH_UNKNOWN
                replay_decode_step(self.layer, b, io, stream)
                cur ^= 1
        torch.cuda.current_stream(self.device).wait_stream(stream)
        return g

    def advance_host(self, n_steps: int) -> None:
        """The host cursor after n_steps steps run outside step() (graph
        replays): no row forced, every live row one token per step."""
        for _ in range(n_steps):
            _, fl = rs_meta_step(self.L, self.anchor)
            rs_meta_advance(self.L, self.anchor, fl)

    def conventional_step(self, io, stream=None, events=None) -> None:
        stream = stream or torch.cuda.current_stream(self.device)
        ios, evs = self._per_layer(io, events)
        if self._dirty:
            wp, _ = rs_meta_step(self.L, self.anchor)
            self._upload(stream, wp)
            self._dirty = False
        for li, (io_l, ev) in enumerate(zip(ios, evs)):
            if ev:
                ev[0].record(stream)
            conventional_decode_step(self.layer, self._batch(layer=li), io_l, stream)
            if ev:
                ev[1].record(stream)

    def flush_rows(self, rows, stream=None) -> None:
        """Token-less flush of the given slots (materialise their state, e.g.
        before retiring or preempting them); they are re-anchored."""
        stream = stream or torch.cuda.current_stream(self.device)
        sel = np.zeros(self.n_slots, bool)
        sel[np.asarray(rows, dtype=np.int64)] = True
        sel &= self.live()
        wp, _ = rs_meta_step(self.L, self.anchor)
        self._upload(stream, wp, sel.astype(np.uint8))
        for li in range(len(self.pools)):
            replay_flush(self.layer, self._batch(layer=li), stream)
        self.anchor[sel] = 0
        self.zero_ckpt[sel] = False
        self._dirty = True

    def join_rows(self, rows) -> None:
        """New requests in the given slots, without a launch: their
        checkpoints count as zero (RS_CURSOR_ZERO_CKPT) and their stored values
        are not used until each row's first flush writes them; anchored at 0.  The metadata goes
        up with the next step's upload.  (The conventional step reads no
        cursor: its rows need reset_rows.)"""
        sel = np.zeros(self.n_slots, bool)
        sel[np.asarray(rows, dtype=np.int64)] = True
        sel &= self.live()
        self.anchor[sel] = 0
        self.zero_ckpt[sel] = True
        self._dirty = True

    def reset_rows(self, rows, stream=None) -> None:
        """Zero the checkpoint of the given slots (new requests) and anchor
        them at 0."""
        stream = stream or torch.cuda.current_stream(self.device)
        sel = np.zeros(self.n_slots, bool)
        sel[np.asarray(rows, dtype=np.int64)] = True
        sel &= self.live()
        wp, _ = rs_meta_step(self.L, self.anchor)
        self._upload(stream, wp, mask=sel.astype(np.uint8))
        for li in range(len(self.pools)):
            replay_state_reset(self.layer, self.batches[li][self._cur], self.mask, stream)
        self.anchor[sel] = 0
        self.zero_ckpt[sel] = False
        self._dirty = True


class SpecDecodeLayer:
    """Host-side state of one speculative layer (rs_layer.spec_T = T) for a
    batch of request slots: the pool, the block table and, on the device, two
    (committed count, flush flag) array pairs.  verify() reads one pair;
    commit(accepted) writes the other from the device-side accepted counts
    (blog "Speculative decoding: rollback becomes a pointer": the commit runs
    on the device and sets the next step's flag), so a decode loop never
    copies the cursor back to the host.  Joining or leaving rows is an upload
    of the block table with the new rows' counts set to 0."""

    def __init__(self, lay: RsLayer, n_slots: int, n_blocks: int | None = None, device="cuda",
                 sr_key=(0, 0)):
        if lay.spec_T < 1:
            raise ValueError("SpecDecodeLayer needs a speculative layer (spec_T > 0)")
        self.layer = lay
        self.L, self.T = int(lay.L), int(lay.spec_T)
        self.n_slots = n = int(n_slots)
        self.pool = Pool(lay, n_blocks or n_slots, device)
        self.device = self.pool.raw.device
        self.blocks = np.full(n, -1, np.int32)
        self.block_table = torch.full((n,), -1, dtype=torch.int32, device=self.device)
        # (committed, flag) pairs; the byte arrays are padded to a multiple of 4
        n4 = (n + 3) // 4 * 4
        self.committed = [torch.zeros(n, dtype=torch.int32, device=self.device) for _ in range(2)]
        self.flag = [torch.zeros(n4, dtype=torch.uint8, device=self.device) for _ in range(2)]
        self.err = torch.zeros(1, dtype=torch.int32, device=self.device)
        self._cur = 0
        self.batch = [make_batch(self.pool.raw, self.pool.n_blocks, self.block_table, self.committed[i],
                                 self.flag[i], self.err, next_write_pos=self.committed[1 - i], sr_key=sr_key)
                      for i in (0, 1)]
        self.sr_step = 0  # stochastic rounding: one counter word per verify launch

    def assign(self, slot: int, block: int) -> None:
        if not 0 <= block < self.pool.n_blocks:
            raise ValueError(f"block {block} outside the pool of {self.pool.n_blocks}")
        self.blocks[slot] = block

    def retire(self, slot: int) -> None:
        self.blocks[slot] = -1

    def upload(self, rows=None, stream=None) -> None:
        """Copy the block table to the device; `rows` (joining slots) start
        with 0 committed records, a zero checkpoint and no flag."""
        stream = stream or torch.cuda.current_stream(self.device)
        with torch.cuda.stream(stream):
            self.block_table.copy_(torch.from_numpy(self.blocks))
            if rows is not None:
                sel = torch.zeros(self.n_slots, dtype=torch.bool)
                sel[torch.as_tensor(list(rows), dtype=torch.long)] = True
                sel = sel.to(self.device)
                self.committed[self._cur].masked_fill_(sel, 0)
                self.flag[self._cur][:self.n_slots].masked_fill_(sel, 0)
                mask = torch.zeros(self.flag[0].numel(), dtype=torch.uint8, device=self.device)
                mask[:self.n_slots] = sel.to(torch.uint8)
                replay_state_reset(self.layer, self.batch[self._cur], mask, stream)

    def verify(self, io, stream=None, events=None) -> None:
        stream = stream or torch.cuda.current_stream(self.device)
        if events:
            events[0].record(stream)
        b = self.batch[self._cur]
        b.sr_step = self.sr_step
        self.sr_step += 1
        replay_spec_verify(self.layer, b, io, stream)
        if events:
            events[1].record(stream)

    def commit(self, accepted, stream=None) -> None:
        """accepted: int32 device tensor [n_slots] (0..T)."""
        stream = stream or torch.cuda.current_stream(self.device)
        replay_spec_commit(self.layer, self.batch[self._cur], accepted, self.flag[1 - self._cur], stream)
        self._cur ^= 1

    def capture_steps(self, ios, accepted, stream=None):
        """Capture verify + commit steps into a HIP graph (the blog,
        "Speculative decoding": the flush rule depends only on h and T, so
        the decision lives inside a captured graph).  ios: one rs_spec_io per
        step, an even number of them; accepted: one device int32 [n_slots]
        tensor per step, which the caller fills (from sampling on the
        device) before each replay.  No stochastic rounding (its counter
        would be fixed in the graph)."""
        if len(ios) % 2 or len(ios) != len(accepted):
            raise ValueError("an even number of steps, one accepted-count tensor per step")
        if self.layer.state_rounding:
            raise ValueError("stochastic rounding draws a fresh counter per launch: no graph capture")
        stream = stream or torch.cuda.Stream(self.device)
        stream.wait_stream(torch.cuda.current_stream(self.device))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            cur = self._cur
            for io, acc in zip(ios, accepted):
                replay_spec_verify(self.layer, self.batch[cur], io, stream)
                replay_spec_commit(self.layer, self.batch[cur], acc, self.flag[1 - cur], stream)
                cur ^= 1
        torch.cuda.current_stream(self.device).wait_stream(stream)
        return g

    def device_committed(self):
        """(committed counts, flags) the next verify will read (synchronises)."""
        torch.cuda.synchronize(self.device)
        return (self.committed[self._cur].cpu().numpy(), self.flag[self._cur][:self.n_slots].cpu().numpy())
