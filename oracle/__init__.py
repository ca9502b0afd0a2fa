"""fp64 CPU oracle for the batched SSM decode step (checkpoint + record buffer).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It shares no code with the GPU path and never imports it.

The arithmetic lives in ``replay_oracle.c`` (plain loops, double precision,
OpenMP over independent (row, head) tiles); this module only marshals numpy
arrays into it.  ``bytemodel.py`` holds the traffic model.  Each C function
cites the passage of the pages it follows.

Array conventions (one tile = one (row, head) pair, tiles flattened):
    S, C       float64 [n, d_v, d_k]   state / checkpoint, row-major
    q, k       float64 [n, d_k]
    v, out     float64 [n, d_v]
    lam, beta  float64 [n]             log-decay (alpha = exp(lam)), GDN beta
    rec_lam    float64 [n, cap]        buffered log-decays
    rec_x      float64 [n, cap, d_v]   buffered values (v, or GDN's corrected d)
    rec_k      float64 [n, cap, d_k]   buffered keys
    w          int32   [n]             records held per tile
    flush      uint8   [n]             this step's flush decision
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .formats import half_ulp, round_to, sr_f16, sr_words  # noqa: F401  (storage roundings)

MAMBA2 = 0
GDN = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "replay_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_F64P = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_I32P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_U8P = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")


def _opt(ptr_type):
    """ndpointer that also accepts None (NULL)."""

    class _Opt(ptr_type):
        @classmethod
        def from_param(cls, obj):
            if obj is None:
                return None
            return ptr_type.from_param(obj)

    return _Opt


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str = _LIB):
        if not os.path.exists(path):
            if path != _LIB:
                raise FileNotFoundError(path)
            build()
        self.path = path
        lib = ctypes.CDLL(path)
        i64, i32, c_int = ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        lib.oc_conventional_step.argtypes = [c_int, i64, c_int, c_int, _F64P, _F64P, _F64P, _F64P,
                                             _F64P, _opt(_F64P), _opt(_U8P), _F64P, _opt(_F64P)]
        lib.oc_conventional_step.restype = None
        lib.oc_replay_step.argtypes = [c_int, i64, c_int, c_int, c_int, _F64P, _F64P, _F64P, _F64P,
                                       _I32P, _U8P, _F64P, _F64P, _F64P, _F64P, _opt(_F64P),
                                       _opt(_U8P), _F64P]
        lib.oc_replay_step.restype = i64
        lib.oc_replay_fold.argtypes = [i64, c_int, c_int, c_int, _F64P, _F64P, _F64P, _F64P, _I32P,
                                       _opt(_U8P)]
        lib.oc_replay_fold.restype = None
        lib.oc_cursor_run.argtypes = [c_int, i32, i64, _opt(_U8P), _I32P, _U8P]
        lib.oc_cursor_run.restype = None
        lib.oc_spec_verify.argtypes = [i64, c_int, c_int, c_int, c_int, _F64P, _F64P, _F64P, _F64P, _I32P,
                                       _U8P, _F64P, _F64P, _F64P, _F64P, _opt(_U8P), _F64P]
        lib.oc_spec_verify.restype = i64
        lib.oc_spec_verify_gdn.argtypes = [i64, c_int, c_int, c_int, c_int, _F64P, _F64P, _F64P, _F64P, _I32P,
                                           _U8P, _F64P, _F64P, _F64P, _F64P, _F64P, _opt(_U8P), _F64P]
        lib.oc_spec_verify_gdn.restype = i64
        lib.oc_spec_commit.argtypes = [i64, _I32P, _I32P, _opt(_U8P)]
        lib.oc_spec_commit.restype = None
        lib.oc_spec_cursor_run.argtypes = [c_int, c_int, i32, i64, _I32P, _opt(_U8P), _I32P, _U8P]
        lib.oc_spec_cursor_run.restype = None
        lib.oc_num_threads.restype = c_int
        lib.oc_set_num_threads.argtypes = [c_int]
        self.lib = lib

    # -- threads ---------------------------------------------------------
    def num_threads(self) -> int:
        return int(self.lib.oc_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.oc_set_num_threads(int(n))

    # -- steps -----------------------------------------------------------
    def conventional_step(self, form, S, q, k, v, lam, beta=None, active=None, want_x=False):
        """Returns out, or (out, x) with x the value written into the state."""
        n, dv, dk = S.shape
        out = np.zeros((n, dv), np.float64)
        x = np.zeros((n, dv), np.float64) if want_x else None
        _check(S, q, k, v, lam, beta, n, dv, dk)
        self.lib.oc_conventional_step(int(form), n, dv, dk, S, q, k, v, lam, beta,
                                      _u8(active), out, x)
        return (out, x) if want_x else out

    def replay_step(self, form, C, rec_lam, rec_x, rec_k, w, flush, q, k, v, lam, beta=None,
                    active=None):
        n, dv, dk = C.shape
        cap = rec_lam.shape[1]
        assert rec_x.shape == (n, cap, dv) and rec_k.shape == (n, cap, dk)
        assert w.dtype == np.int32 and w.shape == (n,)
        _check(C, q, k, v, lam, beta, n, dv, dk)
        out = np.zeros((n, dv), np.float64)
        ovf = self.lib.oc_replay_step(int(form), n, dv, dk, cap, C, rec_lam, rec_x, rec_k, w,
                                      _u8(flush), q, k, v, lam, beta, _u8(active), out)
        if ovf:
            raise ValueError(f"{ovf} tiles would overflow the record buffer (cap={cap})")
        return out

    def replay_fold(self, C, rec_lam, rec_x, rec_k, w, mask=None):
        n, dv, dk = C.shape
        cap = rec_lam.shape[1]
        self.lib.oc_replay_fold(n, dv, dk, cap, C, rec_lam, rec_x, rec_k, w, _u8(mask))

    def cursor_run(self, L, w0, n_steps, forced=None):
        w = np.zeros(n_steps, np.int32)
        f = np.zeros(n_steps, np.uint8)
        self.lib.oc_cursor_run(int(L), int(w0), int(n_steps), _u8(forced), w, f)
        return w, f.astype(bool)

    # -- speculative verify (Mamba-2 form) ---------------------------------
    def spec_verify(self, C, rec_lam, rec_x, rec_k, h, flush, q, k, v, lam, active=None, beta=None):
        """q, k: [n, T, dk]; v: [n, T, dv]; lam: [n, T]; beta: [n, T] for the
        Gated DeltaNet form (None: Mamba-2).  Returns out [n, T, dv]."""
        n, dv, dk = C.shape
        cap = rec_lam.shape[1]
        T = q.shape[1]
        assert rec_x.shape == (n, cap, dv) and rec_k.shape == (n, cap, dk)
        assert h.dtype == np.int32 and h.shape == (n,)
        for a in (C, q, k, v, lam) + (() if beta is None else (beta,)):
            assert a.dtype == np.float64 and a.flags.c_contiguous
        assert q.shape == (n, T, dk) and k.shape == (n, T, dk) and v.shape == (n, T, dv) and lam.shape == (n, T)
        out = np.zeros((n, T, dv), np.float64)
        if beta is None:
            ovf = self.lib.oc_spec_verify(n, dv, dk, cap, T, C, rec_lam, rec_x, rec_k, h, _u8(flush), q, k, v,
                                          lam, _u8(active), out)
        else:
            assert beta.shape == (n, T)
            ovf = self.lib.oc_spec_verify_gdn(n, dv, dk, cap, T, C, rec_lam, rec_x, rec_k, h, _u8(flush), q, k,
                                              v, lam, beta, _u8(active), out)
        if ovf:
            raise ValueError(f"{ovf} tiles would overflow the record ring (cap={cap}, T={T})")
        return out

    def spec_commit(self, h, accepted, active=None):
        self.lib.oc_spec_commit(h.shape[0], h, np.ascontiguousarray(accepted, np.int32), _u8(active))

    def spec_cursor_run(self, L, T, h0, accepted, forced=None):
        accepted = np.ascontiguousarray(accepted, np.int32)
        n_steps = accepted.shape[0]
        h = np.zeros(n_steps, np.int32)
        f = np.zeros(n_steps, np.uint8)
        self.lib.oc_spec_cursor_run(int(L), int(T), int(h0), int(n_steps), accepted, _u8(forced), h, f)
        return h, f.astype(bool)


def _u8(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a).astype(np.uint8))


def _check(S, q, k, v, lam, beta, n, dv, dk):
    for a in (S, q, k, v, lam) + ((beta,) if beta is not None else ()):
        assert a.dtype == np.float64 and a.flags.c_contiguous
    assert q.shape == (n, dk) and k.shape == (n, dk) and v.shape == (n, dv)
    assert lam.shape == (n,)
    assert beta is None or beta.shape == (n,)


_default = None


def get() -> Oracle:
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


class ConventionalModel:
    """Conventional decode for B rows x H heads, fp64 state in memory."""

    def __init__(self, form, B, H, dv, dk, S0=None, oracle=None):
        self.o = oracle or get()
        self.form, self.B, self.H, self.dv, self.dk = form, B, H, dv, dk
        n = B * H
        self.S = np.zeros((n, dv, dk)) if S0 is None else np.ascontiguousarray(S0, np.float64).reshape(n, dv, dk).copy()

    def step(self, q, k, v, lam, beta=None, active_rows=None, want_x=False):
        """q, k: [B, H, dk]; v: [B, H, dv]; lam, beta: [B, H].  Returns o [B, H, dv]
        (and, with want_x, the value x [B, H, dv] written into the state)."""
        B, H = self.B, self.H
        act = None if active_rows is None else np.repeat(np.asarray(active_rows, bool), H)
        n = B * H
        res = self.o.conventional_step(self.form, self.S, _vec(q, n), _vec(k, n), _vec(v, n),
                                       _scal(lam, n), None if beta is None else _scal(beta, n),
                                       act, want_x)
        if want_x:
            return res[0].reshape(B, H, self.dv), res[1].reshape(B, H, self.dv)
        return res.reshape(B, H, self.dv)

    def state(self):
        return self.S.reshape(self.B, self.H, self.dv, self.dk)


class ReplayModel:
    """Checkpoint + record buffer for B rows x H heads, fp64, buffer of L - 1 slots."""

    def __init__(self, form, B, H, dv, dk, L, oracle=None):
        self.o = oracle or get()
        self.form, self.B, self.H, self.dv, self.dk, self.L = form, B, H, dv, dk, L
        n = B * H
        cap = max(L - 1, 0)
        self.cap = cap
        self.C = np.zeros((n, dv, dk))
        self.rec_lam = np.zeros((n, cap))
        self.rec_x = np.zeros((n, cap, dv))
        self.rec_k = np.zeros((n, cap, dk))
        self.w = np.zeros(n, np.int32)

    def set_row(self, b, C, rec_lam, rec_x, rec_k, w):
        """Load one row's checkpoint [H, dv, dk] and its first w records."""
        H = self.H
        sl = slice(b * H, (b + 1) * H)
        self.C[sl] = C
        self.rec_lam[sl] = 0.0
        self.rec_x[sl] = 0.0
        self.rec_k[sl] = 0.0
        if w:
            self.rec_lam[sl, :w] = rec_lam[:, :w]
            self.rec_x[sl, :w] = rec_x[:, :w]
            self.rec_k[sl, :w] = rec_k[:, :w]
        self.w[sl] = w

    def step(self, q, k, v, lam, flush_rows, beta=None, active_rows=None):
        """flush_rows: [B] bools.  Returns o [B, H, dv]."""
        B, H = self.B, self.H
        fl = np.repeat(np.asarray(flush_rows, bool), H)
        act = None if active_rows is None else np.repeat(np.asarray(active_rows, bool), H)
        n = B * H
        out = self.o.replay_step(self.form, self.C, self.rec_lam, self.rec_x, self.rec_k, self.w,
                                 fl, _vec(q, n), _vec(k, n), _vec(v, n), _scal(lam, n),
                                 None if beta is None else _scal(beta, n), act)
        return out.reshape(B, H, self.dv)

    def fold(self, rows_mask):
        mask = np.repeat(np.asarray(rows_mask, bool), self.H)
        self.o.replay_fold(self.C, self.rec_lam, self.rec_x, self.rec_k, self.w, mask)

    def checkpoint(self):
        return self.C.reshape(self.B, self.H, self.dv, self.dk)

    def records_held(self):
        return self.w.reshape(self.B, self.H)


class TwoCopyReplayModel(ReplayModel):
    """Checkpoint + buffer with two checkpoint copies (blog, section "The
    precision argument, derived"): the recurrence copy C is read only by
    flushes; the read copy C_lo is what non-flush steps read.  A flush folds
    from C and casts the same unrounded fold into both copies: C_lo rounded
    to `read_dtype` (formats.round_to: f16, bf16 or e4m3 with a power-of-two
    scale per state row), C kept exact (rec_dtype None) or stored in fp16
    (rec_dtype "f16"), to nearest even or, given a Philox key, with
    stochastic rounding (the paper's preferred recurrence copy, in the
    blog's account); `tile_ids` as in SRReplayModel.  Mamba-2 form."""

    def __init__(self, B, H, dv, dk, L, read_dtype="f16", oracle=None, rec_dtype=None, key=None, tile_ids=None):
        super().__init__(MAMBA2, B, H, dv, dk, L, oracle)
        self.read_dtype = read_dtype
        self.C_lo = np.zeros_like(self.C)
        if rec_dtype not in (None, "f16"):
            raise ValueError(f"recurrence copy dtype {rec_dtype!r}: None (exact) or 'f16'")
        self.rec_dtype = rec_dtype
        self.key = None if key is None else np.asarray(key, np.uint64)
        self.tile_ids = np.arange(B * H) if tile_ids is None else np.asarray(tile_ids)

    def _store(self, mask, sr_step):
        """Both copies of the masked tiles from the unrounded fold in C."""
        self.C_lo[mask] = round_to(self.C[mask], self.read_dtype)
        if self.rec_dtype is None:
            return
        for t in np.nonzero(mask)[0]:
            if self.key is None:
                self.C[t] = round_to(self.C[t], "f16")
            else:
                self.C[t] = sr_f16(self.C[t].reshape(-1), sr_words(self.key, sr_step, self.tile_ids[t],
                                                                   self.dv * self.dk)).reshape(self.dv, self.dk)

    def step(self, q, k, v, lam, flush_rows, beta=None, active_rows=None, sr_step=0):
        B, H = self.B, self.H
        n = B * H
        fl = np.repeat(np.asarray(flush_rows, bool), H)
        act = np.ones(n, bool) if active_rows is None else np.repeat(np.asarray(active_rows, bool), H)
        args = (_vec(q, n), _vec(k, n), _vec(v, n), _scal(lam, n), None)
        # non-flush rows: output from the read copy, record appended
        out = self.o.replay_step(MAMBA2, self.C_lo, self.rec_lam, self.rec_x, self.rec_k, self.w, fl, *args,
                                 act & ~fl)
        # flush rows: fold from the recurrence copy, then re-round the read copy
        out += self.o.replay_step(MAMBA2, self.C, self.rec_lam, self.rec_x, self.rec_k, self.w, fl, *args,
                                  act & fl)
        self._store(act & fl, sr_step)
        return out.reshape(B, H, self.dv)

    def fold(self, rows_mask, sr_step=0):
        super().fold(rows_mask)
        self._store(np.repeat(np.asarray(rows_mask, bool), self.H), sr_step)

    def read_error_bound(self, q, lam):
        """Before step(q, ..., lam, ...): per output component, the most the
        read copy can move a non-flush output, gamma_h sum_c u_ic |q_c| with
        u = half an ulp of the recurrence copy in the read format and
        gamma_h = exp(buffered log-decays + lam) [B, H, dv]."""
        B, H = self.B, self.H
        n = B * H
        q = _vec(q, n)
        held = np.arange(self.cap)[None, :] < self.w[:, None]
        g = np.exp((self.rec_lam * held).sum(axis=1) + _scal(lam, n))
        u = half_ulp(self.C, self.read_dtype)
        return (g[:, None] * np.einsum("nic,nc->ni", u, np.abs(q))).reshape(B, H, self.dv)


def sr_round_tiles(X, key, step, tiles):
    """Stochastic rounding to fp16 of the given tiles of X [n, d_v, d_k] in
    place, tile t (its index = row * n_heads + head) with the random words of
    (step, t)."""
    n, dv, dk = X.shape
    for t in tiles:
        X[t] = sr_f16(X[t].reshape(-1), sr_words(key, step, t, dv * dk)).reshape(dv, dk)


class SRReplayModel(ReplayModel):
    """Checkpoint + buffer whose checkpoint is stored in fp16 with stochastic
    rounding at every flush (blog "The precision argument, derived": the
    recurrence copy kept in FP16 with stochastic rounding, so rounding enters
    the recurrence once per window).  Records are kept exactly; `tile_ids`
    maps this model's tiles to the (row * n_heads + head) indices the random
    words are drawn for."""

    def __init__(self, form, B, H, dv, dk, L, key, tile_ids=None, oracle=None):
        super().__init__(form, B, H, dv, dk, L, oracle)
        self.key = np.asarray(key, np.uint64)
        self.tile_ids = np.arange(B * H) if tile_ids is None else np.asarray(tile_ids)

    def step(self, q, k, v, lam, flush_rows, beta=None, active_rows=None, sr_step=0):
        out = super().step(q, k, v, lam, flush_rows, beta, active_rows)
        fl = np.repeat(np.asarray(flush_rows, bool), self.H)
        if active_rows is not None:
            fl &= np.repeat(np.asarray(active_rows, bool), self.H)
        for t in np.nonzero(fl)[0]:
            self.C[t] = sr_f16(self.C[t].reshape(-1), sr_words(self.key, sr_step, self.tile_ids[t],
                                                               self.dv * self.dk)).reshape(self.dv, self.dk)
        return out


    def fold(self, rows_mask, sr_step=0):
        """Token-less flush; the folded checkpoints are stored with
        stochastic rounding like a flush's."""
        super().fold(rows_mask)
        for t in np.nonzero(np.repeat(np.asarray(rows_mask, bool), self.H))[0]:
            self.C[t] = sr_f16(self.C[t].reshape(-1), sr_words(self.key, sr_step, self.tile_ids[t],
                                                               self.dv * self.dk)).reshape(self.dv, self.dk)


class SRConventionalModel(ConventionalModel):
    """Conventional decode with the state stored in fp16 with stochastic
    rounding after every step (the per-step rounding the blog's argument
    starts from)."""

    def __init__(self, form, B, H, dv, dk, key, tile_ids=None, S0=None, oracle=None):
        super().__init__(form, B, H, dv, dk, S0, oracle)
        self.key = np.asarray(key, np.uint64)
        self.tile_ids = np.arange(B * H) if tile_ids is None else np.asarray(tile_ids)

    def step(self, q, k, v, lam, beta=None, active_rows=None, want_x=False, sr_step=0):
        res = super().step(q, k, v, lam, beta, active_rows, want_x)
        act = np.ones(self.B * self.H, bool) if active_rows is None else np.repeat(np.asarray(active_rows, bool), self.H)
        for t in np.nonzero(act)[0]:
            self.S[t] = sr_f16(self.S[t].reshape(-1), sr_words(self.key, sr_step, self.tile_ids[t],
                                                               self.dv * self.dk)).reshape(self.dv, self.dk)
        return res


class SpecReplayModel:
    """Speculative verify from a checkpoint plus a ring of L committed records
    (blog, "Speculative decoding: rollback becomes a pointer"), B rows x H
    heads, fp64, Mamba-2 form or (form=GDN, blog "The delta-rule wrinkle")
    Gated DeltaNet, whose records hold corrected values.  verify() computes
    the T draft outputs and stores the drafts as records behind the committed
    ones (after folding the committed records on flush rows); commit()
    advances the committed pointer."""

    def __init__(self, B, H, dv, dk, L, T, oracle=None, form=MAMBA2):
        self.o = oracle or get()
        self.form = form
        self.B, self.H, self.dv, self.dk, self.L, self.T = B, H, dv, dk, L, T
        n = B * H
        self.cap = L
        self.C = np.zeros((n, dv, dk))
        self.rec_lam = np.zeros((n, L))
        self.rec_x = np.zeros((n, L, dv))
        self.rec_k = np.zeros((n, L, dk))
        self.h = np.zeros(n, np.int32)

    def verify(self, q, k, v, lam, flush_rows, active_rows=None, beta=None):
        """q, k: [B, H, T, dk]; v: [B, H, T, dv]; lam, beta: [B, H, T];
        flush_rows [B].  Returns o [B, H, T, dv]."""
        B, H, T = self.B, self.H, self.T
        n = B * H
        fl = np.repeat(np.asarray(flush_rows, bool), H)
        act = None if active_rows is None else np.repeat(np.asarray(active_rows, bool), H)
        f = lambda a, d: np.ascontiguousarray(np.asarray(a, np.float64).reshape(n, T, d))
        sc = lambda a: np.ascontiguousarray(np.asarray(a, np.float64).reshape(n, T))
        if (self.form == GDN) != (beta is not None):
            raise ValueError("beta is given for the Gated DeltaNet form and only for it")
        out = self.o.spec_verify(self.C, self.rec_lam, self.rec_x, self.rec_k, self.h, fl, f(q, self.dk),
                                 f(k, self.dk), f(v, self.dv), sc(lam), act,
                                 None if beta is None else sc(beta))
        return out.reshape(B, H, T, self.dv)

    def commit(self, accepted_rows, active_rows=None):
        acc = np.repeat(np.asarray(accepted_rows, np.int32), self.H)
        act = None if active_rows is None else np.repeat(np.asarray(active_rows, bool), self.H)
        self.o.spec_commit(self.h, acc, act)

    def fold(self, rows_mask):
        """Token-less flush of the committed records (the standard step's fold)."""
        mask = np.repeat(np.asarray(rows_mask, bool), self.H)
        self.o.replay_fold(self.C, self.rec_lam, self.rec_x, self.rec_k, self.h, mask)

    def committed(self):
        return self.h.reshape(self.B, self.H)

    def checkpoint(self):
        return self.C.reshape(self.B, self.H, self.dv, self.dk)


class SpecTwoCopyModel(SpecReplayModel):
    """Speculative verify over a two-precision checkpoint (blog, "The
    precision argument, derived", and "Speculative decoding: rollback becomes
    a pointer"), Mamba-2 form: a row that does not flush reads the read copy
    C_lo for its outputs; a flushing row folds its committed records into the
    recurrence copy C (exact, fp64) and computes its outputs from it, and the
    read copy is then the same fold rounded to `read_dtype`
    (formats.round_to: f16, bf16, or e4m3 with a power-of-two scale per
    state row)."""

    def __init__(self, B, H, dv, dk, L, T, read_dtype, oracle=None):
        super().__init__(B, H, dv, dk, L, T, oracle, MAMBA2)
        self.read_dtype = read_dtype
        self.C_lo = np.zeros_like(self.C)

    def verify(self, q, k, v, lam, flush_rows, active_rows=None, beta=None):
        if beta is not None:
            raise ValueError("two-precision checkpoints are Mamba-2 only")
        B, H, T = self.B, self.H, self.T
        n = B * H
        fl = np.repeat(np.asarray(flush_rows, bool), H)
        act = np.ones(n, bool) if active_rows is None else np.repeat(np.asarray(active_rows, bool), H)
        f = lambda a, d: np.ascontiguousarray(np.asarray(a, np.float64).reshape(n, T, d))
        sc = lambda a: np.ascontiguousarray(np.asarray(a, np.float64).reshape(n, T))
        args = (f(q, self.dk), f(k, self.dk), f(v, self.dv), sc(lam))
        # rows that do not flush: outputs from the read copy, drafts appended
        out = self.o.spec_verify(self.C_lo, self.rec_lam, self.rec_x, self.rec_k, self.h, fl, *args, act & ~fl)
        # flushing rows: fold into the recurrence copy, outputs from it
        out += self.o.spec_verify(self.C, self.rec_lam, self.rec_x, self.rec_k, self.h, fl, *args, act & fl)
        self.C_lo[act & fl] = round_to(self.C[act & fl], self.read_dtype)
        return out.reshape(B, H, T, self.dv)

    def fold(self, rows_mask):
        super().fold(rows_mask)
        mask = np.repeat(np.asarray(rows_mask, bool), self.H)
        self.C_lo[mask] = round_to(self.C[mask], self.read_dtype)


class SpecTokenByToken:
    """The definition a speculative verify must reproduce: the conventional
    recurrence run token by token.  The committed state S advances only by
    accepted drafts; verify() runs the T drafts on a copy of S and returns
    every draft's output (Mamba-2 form)."""

    def __init__(self, B, H, dv, dk, T, S0=None, oracle=None, form=MAMBA2):
        self.conv = ConventionalModel(form, B, H, dv, dk, S0, oracle)
        self.B, self.H, self.dv, self.dk, self.T = B, H, dv, dk, T
        self.form = form
        self._drafts = None
        self.drafts_x = None  # [B, H, T, dv]: the value each draft writes (v, or GDN's corrected value)

    def verify(self, q, k, v, lam, beta=None):
        """q, k: [B, H, T, dk]; v: [B, H, T, dv]; lam, beta: [B, H, T] (beta:
        Gated DeltaNet only)."""
        q, k, v, lam = (np.asarray(a, np.float64) for a in (q, k, v, lam))
        beta = None if beta is None else np.asarray(beta, np.float64)
        S = self.conv.S.copy()
        outs, xs = [], []
        for i in range(self.T):
            o, x = self.conv.step(q[:, :, i], k[:, :, i], v[:, :, i], lam[:, :, i],
                                  None if beta is None else beta[:, :, i], want_x=True)
            outs.append(o)
            xs.append(x)
        self.conv.S = S  # the committed state is unchanged until commit()
        self._drafts = (q, k, v, lam, beta)
        self.drafts_x = np.stack(xs, axis=2)
        return np.stack(outs, axis=2)

    def commit(self, accepted_rows):
        """Advance each row's committed state by its first `accepted` drafts."""
        q, k, v, lam, beta = self._drafts
        acc = np.asarray(accepted_rows)
        for i in range(self.T):
            rows = acc > i
            if rows.any():
                self.conv.step(q[:, :, i], k[:, :, i], v[:, :, i], lam[:, :, i],
                               None if beta is None else beta[:, :, i], active_rows=rows)

    def state(self):
        return self.conv.state()


def _vec(a, n):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).reshape(n, -1))


def _scal(a, n):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).reshape(n))
