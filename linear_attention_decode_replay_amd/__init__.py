"""Batched SSM decode step served from a checkpoint plus a record buffer, on
MI355X (gfx950).

This package is a thin ctypes binding over ``libreplayssm.so`` (C ABI in
``include/replayssm.h``).  It only marshals arguments: every step of the
decode path runs in the HIP kernels.  PyTorch supplies device memory and the
stream.  If the library is missing, importing this package raises
ImportError; there is no fallback.

Entry points (same names and meaning as the C ABI):
    replay_decode_step, replay_flush, conventional_decode_step,
    replay_state_reset, rs_meta_step, rs_meta_advance, replay_spec_verify,
    replay_spec_commit, rs_spec_meta_step, rs_spec_meta_advance,
    block_layout, layer_supported.
Struct builders: layer(), make_batch(), make_io(), make_spec_io(); device memory helper:
Pool (allocates the paged block pool with torch and exposes typed views).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libreplayssm.so")

MAMBA2, GDN = 0, 1
F32, F16, BF16, E4M3 = 0, 1, 2, 3
RS_OK, RS_EINVAL, RS_EUNSUPPORTED, RS_EHIP = 0, -1, -2, -3
RS_ROUND_NEAREST, RS_ROUND_STOCHASTIC = 0, 1
RS_GDN_OUTPUT_ONLY, RS_GDN_RECONSTRUCT = 0, 1
RS_FLUSH_UNKNOWN, RS_FLUSH_NONE, RS_FLUSH_ALL, RS_FLUSH_MIXED = 0, 1, 2, 3
# write_pos flag: the row's checkpoint is zero and is not read (replayssm.h)
RS_CURSOR_ZERO_CKPT = 1 << 30

_c = ctypes
_vp = _c.c_void_p


class RsLayer(_c.Structure):
    _fields_ = [("form", _c.c_int32), ("n_heads", _c.c_int32), ("d_v", _c.c_int32),
                ("d_k", _c.c_int32), ("L", _c.c_int32), ("state_dtype", _c.c_int32),
                ("record_dtype", _c.c_int32), ("io_dtype", _c.c_int32), ("read_dtype", _c.c_int32),
                ("spec_T", _c.c_int32), ("n_groups", _c.c_int32), ("state_rounding", _c.c_int32),
                ("gdn_route", _c.c_int32)]


class RsBlockLayout(_c.Structure):
    _fields_ = [("ckpt_off", _c.c_int64), ("rec_x_off", _c.c_int64), ("rec_k_off", _c.c_int64),
                ("rec_lam_off", _c.c_int64), ("block_bytes", _c.c_int64), ("slots", _c.c_int32),
                ("key_slots", _c.c_int32), ("ckpt_lo_off", _c.c_int64), ("ckpt_scale_off", _c.c_int64)]


class RsBatch(_c.Structure):
    _fields_ = [("n_rows", _c.c_int32), ("flush_hint", _c.c_int32), ("n_blocks", _c.c_int64),
                ("pool", _vp), ("block_table", _vp), ("write_pos", _vp), ("flush", _vp),
                ("err_count", _vp), ("next_write_pos", _vp), ("sr_key0", _c.c_uint64),
                ("sr_key1", _c.c_uint64), ("sr_step", _c.c_uint64)]


class RsStepIO(_c.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp),
                ("q_row_stride", _c.c_int64), ("q_head_stride", _c.c_int64),
                ("k_row_stride", _c.c_int64), ("k_head_stride", _c.c_int64),
                ("v_row_stride", _c.c_int64), ("v_head_stride", _c.c_int64),
                ("log_decay", _vp), ("beta", _vp), ("out", _vp)]


class RsSpecIO(_c.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp),
                ("q_row_stride", _c.c_int64), ("q_token_stride", _c.c_int64), ("q_head_stride", _c.c_int64),
                ("k_row_stride", _c.c_int64), ("k_token_stride", _c.c_int64), ("k_head_stride", _c.c_int64),
                ("v_row_stride", _c.c_int64), ("v_token_stride", _c.c_int64), ("v_head_stride", _c.c_int64),
                ("log_decay", _vp), ("out", _vp), ("beta", _vp)]


class ReplaySSMError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"replayssm error {code}: {msg}")
        self.code = code


def _load():
    # torch ships its own HIP runtime (same SONAME as ROCm's).  Loading torch
    # first makes the dynamic linker bind this library to that same runtime
    # instance, so torch's device memory and stream handles are valid here.
    # Loaded the other way round, the process would hold two HIP runtimes.
    import torch  # noqa: F401
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m linear_attention_decode_replay_amd.build` "
                          "(or __graft_entry__.build()) first")
    lib = _c.CDLL(_LIB_PATH)
    P = _c.POINTER
    lib.rs_block_layout_get.argtypes = [P(RsLayer), P(RsBlockLayout)]
    lib.rs_layer_supported.argtypes = [P(RsLayer)]
    for name in ("replay_decode_step", "conventional_decode_step"):
        getattr(lib, name).argtypes = [P(RsLayer), P(RsBatch), P(RsStepIO), _vp]
    lib.replay_flush.argtypes = [P(RsLayer), P(RsBatch), _vp]
    lib.replay_state_reset.argtypes = [P(RsLayer), P(RsBatch), _vp, _vp]
    lib.rs_meta_step.argtypes = [_c.c_int32, _c.c_int32, _vp, _vp, _vp, _vp]
    lib.rs_meta_advance.argtypes = [_c.c_int32, _c.c_int32, _vp, _vp]
    lib.replay_spec_verify.argtypes = [P(RsLayer), P(RsBatch), P(RsSpecIO), _vp]
    lib.replay_spec_commit.argtypes = [P(RsLayer), P(RsBatch), _vp, _vp, _vp]
    lib.rs_spec_meta_step.argtypes = [_c.c_int32, _c.c_int32, _c.c_int32, _vp, _vp, _vp]
    lib.rs_spec_meta_advance.argtypes = [_c.c_int32, _c.c_int32, _c.c_int32, _vp, _vp, _vp]
    lib.rs_last_error.restype = _c.c_char_p
    for name in ("rs_block_layout_get", "rs_layer_supported", "replay_decode_step",
                 "conventional_decode_step", "replay_flush", "replay_state_reset", "rs_meta_step",
                 "rs_meta_advance", "replay_spec_verify", "replay_spec_commit", "rs_spec_meta_step",
                 "rs_spec_meta_advance"):
        getattr(lib, name).restype = _c.c_int
    return lib


_lib = _load()
LIBRARY_PATH = _LIB_PATH


def _check(rc: int) -> None:
    if rc != RS_OK:
        raise ReplaySSMError(rc, _lib.rs_last_error().decode())


def last_error() -> str:
    return _lib.rs_last_error().decode()


# ------------------------------------------------------------------ structs --
_DT_CODE = {"f32": F32, "f16": F16, "bf16": BF16, "e4m3": E4M3}


def layer(form: int, n_heads: int, d_v: int, d_k: int, L: int, state_dtype="f32",
          record_dtype="f16", io_dtype="bf16", read_dtype=None, spec_T: int = 0, n_groups: int = 0,
          stochastic: bool = False, reconstruct: bool = False) -> RsLayer:
    """read_dtype: None for a single checkpoint, "f16" / "bf16" / "e4m3" for
    a two-precision checkpoint (fp32 recurrence copy + read copy; E4M3 with a
    power-of-two scale per state row).  spec_T: 0 for standard decoding, T
    for a speculative layer verifying T drafts per step.  n_groups: 0 for a
    key and query per head, else the number of key groups (q, k inputs then
    [rows, n_groups, d_k], one key record per group).  stochastic: store an
    fp16 state with stochastic rounding (the key and counter travel in the
    batch: sr_key0/sr_key1, sr_step).  reconstruct: Gated DeltaNet only, the
    state-reconstruction route instead of the output-only one."""
    code = lambda d: _DT_CODE[d] if isinstance(d, str) else int(d)
    return RsLayer(int(form), int(n_heads), int(d_v), int(d_k), int(L), code(state_dtype),
                   code(record_dtype), code(io_dtype), -1 if read_dtype is None else code(read_dtype),
                   int(spec_T), int(n_groups), RS_ROUND_STOCHASTIC if stochastic else RS_ROUND_NEAREST,
                   RS_GDN_RECONSTRUCT if reconstruct else RS_GDN_OUTPUT_ONLY)


def block_layout(lay: RsLayer) -> RsBlockLayout:
    out = RsBlockLayout()
    _check(_lib.rs_block_layout_get(_c.byref(lay), _c.byref(out)))
    return out


def layer_supported(lay: RsLayer) -> int:
    return int(_lib.rs_layer_supported(_c.byref(lay)))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def make_batch(pool, n_blocks: int, block_table, write_pos=None, flush=None, err_count=None,
               next_write_pos=None, sr_key=(0, 0), sr_step=0) -> RsBatch:
    """pool: uint8 device tensor; block_table/write_pos/next_write_pos: int32
    [n_rows]; flush: uint8 [n_rows]; err_count: int32 [1]; sr_key: two
    uint64, sr_step: uint64 (stochastic rounding only).  The tensors must
    outlive the launches that use the returned struct."""
    return RsBatch(int(block_table.numel()), 0, int(n_blocks), _ptr(pool), _ptr(block_table),
                   _ptr(write_pos), _ptr(flush), _ptr(err_count), _ptr(next_write_pos),
                   int(sr_key[0]), int(sr_key[1]), int(sr_step))


def make_io(q, k, v, log_decay, out, beta=None) -> RsStepIO:
    """q, k: [n_rows, n_heads, d_k]; v: [n_rows, n_heads, d_v] (any row/head
    strides, unit last stride); log_decay, beta: fp32 [n_rows, n_heads]
    contiguous; out: fp32 [n_rows, n_heads, d_v] contiguous."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{name} must be [rows, heads, d] with unit last stride")
    for name, t in (("log_decay", log_decay), ("beta", beta), ("out", out)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return RsStepIO(_ptr(q), _ptr(k), _ptr(v), q.stride(0), q.stride(1), k.stride(0), k.stride(1),
                    v.stride(0), v.stride(1), _ptr(log_decay), _ptr(beta), _ptr(out))


def make_spec_io(q, k, v, log_decay, out, beta=None) -> RsSpecIO:
    """q, k: [n_rows, T, n_heads, d_k] ([n_rows, T, n_groups, d_k] with
    grouped keys); v: [n_rows, T, n_heads, d_v] (any row/token/head strides,
    unit last stride); log_decay, beta (Gated
    DeltaNet only): fp32 [n_rows, T, n_heads] contiguous; out: fp32
    [n_rows, T, n_heads, d_v] contiguous."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{name} must be [rows, T, heads, d] with unit last stride")
    for name, t in (("log_decay", log_decay), ("out", out), ("beta", beta)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return RsSpecIO(_ptr(q), _ptr(k), _ptr(v), q.stride(0), q.stride(1), q.stride(2), k.stride(0), k.stride(1),
                    k.stride(2), v.stride(0), v.stride(1), v.stride(2), _ptr(log_decay), _ptr(out), _ptr(beta))


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ------------------------------------------------------------- entry points --
def replay_decode_step(lay: RsLayer, batch: RsBatch, io: RsStepIO, stream=None) -> None:
    _check(_lib.replay_decode_step(_c.byref(lay), _c.byref(batch), _c.byref(io), _stream(stream)))


def replay_flush(lay: RsLayer, batch: RsBatch, stream=None) -> None:
    _check(_lib.replay_flush(_c.byref(lay), _c.byref(batch), _stream(stream)))


def conventional_decode_step(lay: RsLayer, batch: RsBatch, io: RsStepIO, stream=None) -> None:
    _check(_lib.conventional_decode_step(_c.byref(lay), _c.byref(batch), _c.byref(io), _stream(stream)))


def replay_state_reset(lay: RsLayer, batch: RsBatch, mask, stream=None) -> None:
    _check(_lib.replay_state_reset(_c.byref(lay), _c.byref(batch), _ptr(mask), _stream(stream)))


def replay_spec_verify(lay: RsLayer, batch: RsBatch, io: RsSpecIO, stream=None) -> None:
    _check(_lib.replay_spec_verify(_c.byref(lay), _c.byref(batch), _c.byref(io), _stream(stream)))


def replay_spec_commit(lay: RsLayer, batch: RsBatch, accepted, next_flush, stream=None) -> None:
    """accepted: int32 device [n_rows]; next_flush: uint8 device [n_rows]."""
    _check(_lib.replay_spec_commit(_c.byref(lay), _c.byref(batch), _ptr(accepted), _ptr(next_flush),
                                   _stream(stream)))


def rs_spec_meta_step(L: int, T: int, committed: np.ndarray, force: np.ndarray | None = None) -> np.ndarray:
    """Host mirror: this step's flush flags (uint8) for the committed counts."""
    h = np.ascontiguousarray(committed, dtype=np.int32)
    f = None if force is None else np.ascontiguousarray(force, dtype=np.uint8)
    out = np.zeros(h.shape[0], np.uint8)
    _check(_lib.rs_spec_meta_step(int(L), int(T), h.shape[0], h.ctypes.data, None if f is None else f.ctypes.data,
                                  out.ctypes.data))
    return out


def rs_spec_meta_advance(L: int, T: int, committed: np.ndarray, flush: np.ndarray, accepted: np.ndarray) -> None:
    """Host mirror of the commit, in place on an int32 contiguous array."""
    assert committed.dtype == np.int32 and committed.flags.c_contiguous
    f = np.ascontiguousarray(flush, dtype=np.uint8)
    a = np.ascontiguousarray(accepted, dtype=np.int32)
    _check(_lib.rs_spec_meta_advance(int(L), int(T), committed.shape[0], committed.ctypes.data, f.ctypes.data,
                                     a.ctypes.data))


def rs_meta_step(L: int, steps_since_anchor: np.ndarray, force_flush: np.ndarray | None = None):
    """Host metadata for one step.  Returns (write_pos int32, flush uint8)."""
    s = np.ascontiguousarray(steps_since_anchor, dtype=np.int32)
    n = s.shape[0]
    f = None if force_flush is None else np.ascontiguousarray(force_flush, dtype=np.uint8)
    wp = np.zeros(n, np.int32)
    fl = np.zeros(n, np.uint8)
    _check(_lib.rs_meta_step(int(L), n, s.ctypes.data, None if f is None else f.ctypes.data,
                             wp.ctypes.data, fl.ctypes.data))
    return wp, fl


def rs_meta_advance(L: int, steps_since_anchor: np.ndarray, flush: np.ndarray) -> None:
    """In place on an int32 contiguous array."""
    assert steps_since_anchor.dtype == np.int32 and steps_since_anchor.flags.c_contiguous
    f = np.ascontiguousarray(flush, dtype=np.uint8)
    _check(_lib.rs_meta_advance(int(L), steps_since_anchor.shape[0], steps_since_anchor.ctypes.data,
                                f.ctypes.data))


def read_copy_columns(lay: RsLayer) -> np.ndarray:
    """For a two-precision layer: the column held by each stored position of
    a read-copy row.  With n read elements and m recurrence-copy elements per
    16 bytes (m = 4 for fp32, 8 for fp16), position p (chunk c = p // n,
    e = p % n) holds column m (c + (d_k // n) (e // m)) + e % m."""
    n = {F16: 8, BF16: 8, E4M3: 16}[lay.read_dtype]
    m = {F32: 4, F16: 8}[lay.state_dtype]
    p = np.arange(lay.d_k)
    c, e = p // n, p % n
    return m * (c + (lay.d_k // n) * (e // m)) + e % m


# ------------------------------------------------------------ device memory --
class Pool:
    """The paged block pool of one layer, allocated with torch on a device,
    with typed views of each region (memory plumbing for callers and tests)."""

    def __init__(self, lay: RsLayer, n_blocks: int, device="cuda"):
        import torch
        self.layer = lay
        self.layout = block_layout(lay)
        self.n_blocks = int(n_blocks)
        self.block_bytes = int(self.layout.block_bytes)
        self.raw = torch.empty((self.n_blocks, self.block_bytes), dtype=torch.uint8, device=device)
        self._tdt = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}

    def _region(self, off, nbytes, dtype, shape):
        return self.raw[:, off:off + nbytes].view(dtype).view(self.n_blocks, *shape)

    def ckpt(self):
        """[n_blocks, H, d_v, d_k] in the state dtype."""
        L = self.layer
        dt = self._tdt[L.state_dtype]
        es = 4 if L.state_dtype == F32 else 2
        n = L.n_heads * L.d_v * L.d_k
        return self._region(self.layout.ckpt_off, n * es, dt, (L.n_heads, L.d_v, L.d_k))

    def rec_x(self):
        """[n_blocks, H, slots, d_v] in the record dtype."""
        L, s = self.layer, self.layout.slots
        es = 4 if L.record_dtype == F32 else 2
        return self._region(self.layout.rec_x_off, L.n_heads * s * L.d_v * es,
                            self._tdt[L.record_dtype], (L.n_heads, s, L.d_v))

    def rec_k(self):
        """[n_blocks, G, key_slots, d_k] in the record dtype (G = key groups,
        n_heads unless the layer groups its keys; key_slots = slots, plus T
        staging slots on a speculative layer with grouped keys)."""
        L, s = self.layer, self.layout.key_slots
        es = 4 if L.record_dtype == F32 else 2
        G = L.n_groups if L.n_groups > 0 else L.n_heads
        return self._region(self.layout.rec_k_off, G * s * L.d_k * es,
                            self._tdt[L.record_dtype], (G, s, L.d_k))

    def ckpt_lo(self):
        """[n_blocks, H, d_v, d_k] read copy of a two-precision checkpoint
        (E4M3: the raw codes as uint8)."""
        import torch
        L = self.layer
        if L.read_dtype < 0 or L.read_dtype == L.state_dtype:
            raise ValueError("this layer has a single checkpoint")
        es, dt = {F16: (2, torch.float16), BF16: (2, torch.bfloat16), E4M3: (1, torch.uint8)}[L.read_dtype]
        return self._region(self.layout.ckpt_lo_off, L.n_heads * L.d_v * L.d_k * es, dt,
                            (L.n_heads, L.d_v, L.d_k))

    def ckpt_lo_columns(self):
        """Column of each stored position of a read-copy row (the read copy
        keeps each row in lane order; ckpt_lo()[..., i] is column cols[i])."""
        return read_copy_columns(self.layer)

    def ckpt_scale(self):
        """[n_blocks, H, d_v] fp32 row scales of an E4M3 read copy."""
        import torch
        L = self.layer
        if L.read_dtype != E4M3:
            raise ValueError("this layer has no scaled read copy")
        return self._region(self.layout.ckpt_scale_off, L.n_heads * L.d_v * 4, torch.float32, (L.n_heads, L.d_v))

    def rec_lam(self):
        """[n_blocks, H, slots] fp32."""
        import torch
        L, s = self.layer, self.layout.slots
        return self._region(self.layout.rec_lam_off, L.n_heads * s * 4, torch.float32, (L.n_heads, s))


__all__ = [
    "MAMBA2", "GDN", "F32", "F16", "BF16", "E4M3", "RsLayer", "RsBlockLayout", "RsBatch", "RsStepIO",
    "ReplaySSMError", "layer", "block_layout", "layer_supported", "make_batch", "make_io",
    "replay_decode_step", "replay_flush", "conventional_decode_step", "replay_state_reset",
    "rs_meta_step", "rs_meta_advance", "last_error", "Pool", "LIBRARY_PATH", "read_copy_columns",
    "RsSpecIO", "make_spec_io", "replay_spec_verify", "replay_spec_commit", "rs_spec_meta_step",
    "rs_spec_meta_advance",
]
