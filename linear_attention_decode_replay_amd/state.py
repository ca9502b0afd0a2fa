"""Host-side state of one SSM layer for a batch of request slots.

Owns the paged block pool (device memory from torch), the per-slot block
assignment and each slot's anchor (decode steps since its checkpoint was
last anchored), and drives the C ABI once per step:

  1. ``rs_meta_step`` (C, host) turns anchors into the step's write
     positions and flush flags (vLLM pull request "[Kernel] ReplaySSM: cache
     SSM inputs for faster Gated DeltaNet standard decode", section "CUDA
     graphs and continuous batching": position = steps since anchor mod L,
     flush at position L-1 or when forced);
  2. the block table, positions and flags are copied host -> device
     asynchronously from pinned staging buffers (no device -> host sync);
  3. one kernel launch serves flush and non-flush rows alike;
  4. ``rs_meta_advance`` re-anchors the rows that flushed.

A ring of staging buffers lets the host run several steps ahead of the
device; a buffer is reused only after the event recorded behind its copy
has completed.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (Pool, RsLayer, conventional_decode_step, make_batch, replay_decode_step,
               replay_flush, replay_state_reset, rs_meta_advance, rs_meta_step)


class _Stage:
    def __init__(self, n: int):
        self.wp = torch.zeros(n, dtype=torch.int32, pin_memory=True)
        self.fl = torch.zeros(n, dtype=torch.uint8, pin_memory=True)
        self.bt = torch.zeros(n, dtype=torch.int32, pin_memory=True)
        self.mask = torch.zeros(n, dtype=torch.uint8, pin_memory=True)
        self.event = None


class DecodeLayer:
    def __init__(self, lay: RsLayer, n_slots: int, n_blocks: int | None = None, device="cuda",
                 staging: int = 4):
        self.layer = lay
        self.L = int(lay.L)
        self.n_slots = int(n_slots)
        self.pool = Pool(lay, n_blocks or n_slots, device)
        self.device = self.pool.raw.device
        self.anchor = np.full(self.n_slots, -1, np.int32)   # -1: empty slot (padding row)
        self.blocks = np.full(self.n_slots, -1, np.int32)
        dev = self.device
        self.block_table = torch.full((self.n_slots,), -1, dtype=torch.int32, device=dev)
        self.write_pos = torch.zeros(self.n_slots, dtype=torch.int32, device=dev)
        self.flush = torch.zeros(self.n_slots, dtype=torch.uint8, device=dev)
        self.mask = torch.zeros(self.n_slots, dtype=torch.uint8, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self._stages = [_Stage(self.n_slots) for _ in range(staging)]
        self._next = 0
        self.batch = make_batch(self.pool.raw, self.pool.n_blocks, self.block_table, self.write_pos,
                                self.flush, self.err)

    # ---------------------------------------------------------- bookkeeping --
    def assign(self, slot: int, block: int, steps_since_anchor: int = 0) -> None:
        """Place a request in `slot` on pool block `block`."""
        if not 0 <= block < self.pool.n_blocks:
            raise ValueError(f"block {block} outside the pool of {self.pool.n_blocks}")
        self.blocks[slot] = block
        self.anchor[slot] = steps_since_anchor

    def retire(self, slot: int) -> None:
        self.blocks[slot] = -1
        self.anchor[slot] = -1

    def live(self) -> np.ndarray:
        return self.blocks >= 0

    # ------------------------------------------------------------- transfers --
    def _upload(self, stream, wp=None, fl=None, mask=None) -> None:
        st = self._stages[self._next]
        self._next = (self._next + 1) % len(self._stages)
        if st.event is not None:
            st.event.synchronize()
        st.bt.numpy()[:] = self.blocks
        with torch.cuda.stream(stream):
            self.block_table.copy_(st.bt, non_blocking=True)
            if wp is not None:
                st.wp.numpy()[:] = wp
                st.fl.numpy()[:] = fl
                self.write_pos.copy_(st.wp, non_blocking=True)
                self.flush.copy_(st.fl, non_blocking=True)
            if mask is not None:
                st.mask.numpy()[:] = mask
                self.mask.copy_(st.mask, non_blocking=True)
            st.event = torch.cuda.Event()
            st.event.record(stream)

    # ----------------------------------------------------------------- steps --
    def step(self, io, force: np.ndarray | None = None, stream=None, events=None):
        """One checkpoint + buffer decode step.  Returns the host (write_pos,
        flush) arrays that were used.  `events` = (start, end) torch events
        recorded on the stream right around the kernel launch."""
        stream = stream or torch.cuda.current_stream(self.device)
        wp, fl = rs_meta_step(self.L, self.anchor, force)
        self._upload(stream, wp, fl)
        if events:
            events[0].record(stream)
        replay_decode_step(self.layer, self.batch, io, stream)
        if events:
            events[1].record(stream)
        rs_meta_advance(self.L, self.anchor, fl)
        return wp, fl

    def conventional_step(self, io, stream=None, events=None) -> None:
        stream = stream or torch.cuda.current_stream(self.device)
        self._upload(stream)
        if events:
            events[0].record(stream)
        conventional_decode_step(self.layer, self.batch, io, stream)
        if events:
            events[1].record(stream)

    def flush_rows(self, rows, stream=None) -> None:
        """Token-less flush of the given slots (materialise their state, e.g.
        before retiring or preempting them); they are re-anchored."""
        stream = stream or torch.cuda.current_stream(self.device)
        sel = np.zeros(self.n_slots, bool)
        sel[np.asarray(rows, dtype=np.int64)] = True
        sel &= self.live()
        wp, _ = rs_meta_step(self.L, self.anchor)
        self._upload(stream, wp, sel.astype(np.uint8))
        replay_flush(self.layer, self.batch, stream)
        self.anchor[sel] = 0

    def reset_rows(self, rows, stream=None) -> None:
        """Zero the checkpoint of the given slots (new requests) and anchor
        them at 0."""
        stream = stream or torch.cuda.current_stream(self.device)
        sel = np.zeros(self.n_slots, bool)
        sel[np.asarray(rows, dtype=np.int64)] = True
        sel &= self.live()
        self._upload(stream, mask=sel.astype(np.uint8))
        replay_state_reset(self.layer, self.batch, self.mask, stream)
        self.anchor[sel] = 0
