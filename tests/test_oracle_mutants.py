"""Every plausible mistake planted in the oracle must fail at least one pin.

Each case copies oracle/replay_oracle.c, applies one textual change (a dropped
term, a wrong sign, an off-by-one index, a swapped operand), compiles the copy
on the CPU with gcc into a temporary directory and runs all pins against it.
The real oracle source is never modified.
"""
import os

import pytest

import oracle
from pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "replay_oracle.c")

MUTANTS = [
    ("conv_drop_decay",
     "St[(int64_t)i * dk + c] = alpha * St[(int64_t)i * dk + c] + d[i] * kt[c];",
     "St[(int64_t)i * dk + c] = St[(int64_t)i * dk + c] + d[i] * kt[c];"),
    ("conv_gdn_sign",
     "d[i] = beta[t] * (vt[i] - alpha * a[i]);",
     "d[i] = beta[t] * (vt[i] + alpha * a[i]);"),
    ("conv_gdn_drop_alpha_in_correction",
     "d[i] = beta[t] * (vt[i] - alpha * a[i]);",
     "d[i] = beta[t] * (vt[i] - a[i]);"),
    ("conv_gdn_drop_beta",
     "d[i] = beta[t] * (vt[i] - alpha * a[i]);",
     "d[i] = (vt[i] - alpha * a[i]);"),
    ("matvec_wrong_stride",
     "for (int i = 0; i < dv; ++i) y[i] = dot(S + (int64_t)i * dk, x, dk);",
     "for (int i = 0; i < dv; ++i) y[i] = dot(S + (int64_t)i, x, dk);"),
    ("replay_gamma_off_by_one",
     "o += gamma_range(alpha1, j + 1, h) * xt[(int64_t)(j - 1) * dv + i] * dotq[j];",
     "o += gamma_range(alpha1, j, h) * xt[(int64_t)(j - 1) * dv + i] * dotq[j];"),
    ("replay_checkpoint_gamma_short",
     "const double gh = gamma_range(alpha1, 1, h);",
     "const double gh = gamma_range(alpha1, 1, h - 1);"),
    ("replay_drop_current_token",
     "o += vt[i] * kq; /* j = h: gamma_{h+1:h} = 1 */",
     "/* dropped */"),
    ("replay_ckpt_gemv_with_k",
     "matvec(Ct, qt, dv, dk, cq);",
     "matvec(Ct, kt, dv, dk, cq);"),
    ("replay_flush_drop_current",
     "s += vt[i] * kt[c];",
     "/* dropped */"),
    ("replay_flush_gamma_off_by_one",
     "s += gamma_range(alpha1, j + 1, h) * xt[(int64_t)(j - 1) * dv + i] *",
     "s += gamma_range(alpha1, j + 2, h) * xt[(int64_t)(j - 1) * dv + i] *"),
    ("replay_gdn_key_dots_swapped",
     "sk += r * dotk[j] * dj;",
     "sk += r * dotq[j] * dj;"),
    ("replay_gdn_drop_alpha_out",
     "ot[i] = alpha * sq + d[i] * kq;",
     "ot[i] = sq + d[i] * kq;"),
    ("replay_gdn_flush_drop_alpha",
     "Ct[(int64_t)i * dk + c] = alpha * s + d[i] * kt[c];",
     "Ct[(int64_t)i * dk + c] = s + d[i] * kt[c];"),
    ("replay_gdn_T_includes_current",
     "const double T = gamma_range(alpha1, 1, wt);",
     "const double T = gamma_range(alpha1, 1, wt) * alpha;"),
    ("replay_append_wrong_slot",
     "lamt[wt] = lam[t];\n                    memcpy(xt + (int64_t)wt * dv, vt,",
     "lamt[wt] = lam[t];\n                    memcpy(xt + (int64_t)(wt > 0 ? wt - 1 : 0) * dv, vt,"),
    ("fold_gamma_short",
     "const double gw = gamma_range(alpha1, 1, wt);",
     "const double gw = gamma_range(alpha1, 2, wt);"),
    ("cursor_flush_late",
     "const int f = (w == L - 1) || (forced && forced[s]);",
     "const int f = (w == L) || (forced && forced[s]);"),
    ("cursor_force_ignored",
     "const int f = (w == L - 1) || (forced && forced[s]);",
     "const int f = (w == L - 1);"),
    ("spec_no_causal_mask",
     "for (int m = 1; m <= i; ++m) {\n                    const double wgt = gamma_range(ad, m + 1, i) * dot(kt + "
     "(int64_t)(m - 1) * dk, qi, dk);\n                    for (int r = 0; r < dv; ++r) ot[(int64_t)(i - 1) * dv + r] "
     "+= wgt * vt[",
     "for (int m = 1; m <= T; ++m) {\n                    const double wgt = gamma_range(ad, m + 1, i) * dot(kt + "
     "(int64_t)(m - 1) * dk, qi, dk);\n                    for (int r = 0; r < dv; ++r) ot[(int64_t)(i - 1) * dv + r] "
     "+= wgt * vt["),
    ("spec_draft_decay_short",
     "const double Di = gamma_range(ad, 1, i);\n                matvec(Ct, qi, dv, dk, cq);",
     "const double Di = gamma_range(ad, 1, i - 1);\n                matvec(Ct, qi, dv, dk, cq);"),
    ("spec_gdn_draft_decay_short",
     "const double Di = gamma_range(ad, 1, i);\n                double* ui",
     "const double Di = gamma_range(ad, 1, i - 1);\n                double* ui"),
    ("spec_W_off_by_one",
     "const double wgt = gamma_range(ad, m + 1, i) * dot(kt + (int64_t)(m - 1) * dk, qi, dk);\n"
     "                    for (int r = 0; r < dv; ++r) ot[(int64_t)(i - 1) * dv + r] += wgt * vt[",
     "const double wgt = gamma_range(ad, m, i) * dot(kt + (int64_t)(m - 1) * dk, qi, dk);\n"
     "                    for (int r = 0; r < dv; ++r) ot[(int64_t)(i - 1) * dv + r] += wgt * vt["),
    ("spec_gdn_W_off_by_one",
     "const double wgt = gamma_range(ad, m + 1, i) * dot(kt + (int64_t)(m - 1) * dk, qi, dk);\n"
     "                    for (int r = 0; r < dv; ++r) ot[(int64_t)(i - 1) * dv + r] += wgt * u[",
     "const double wgt = gamma_range(ad, m, i) * dot(kt + (int64_t)(m - 1) * dk, qi, dk);\n"
     "                    for (int r = 0; r < dv; ++r) ot[(int64_t)(i - 1) * dv + r] += wgt * u["),
    ("spec_committed_drop_draft_decay",
     "const double wgt = gamma_range(ac, j + 1, ht) * Di * dot(krt + (int64_t)(j - 1) * dk, qi, dk);",
     "const double wgt = gamma_range(ac, j + 1, ht) * dot(krt + (int64_t)(j - 1) * dk, qi, dk);"),
    ("spec_drafts_after_flushed_records",
     "const int base = flush[t] ? 0 : ht; /* first slot",
     "const int base = ht; /* first slot"),
    ("spec_gdn_drafts_after_flushed_records",
     "const int base = flush[t] ? 0 : ht;\n",
     "const int base = ht;\n"),
    ("spec_flush_rule_inclusive",
     "const int f = (room < T) || (forced && forced[s]);",
     "const int f = (room <= T) || (forced && forced[s]);"),
    ("spec_gdn_solve_sign",
     "for (int r = 0; r < dv; ++r) ui[r] -= a * u[(int64_t)(m - 1) * dv + r];",
     "for (int r = 0; r < dv; ++r) ui[r] += a * u[(int64_t)(m - 1) * dv + r];"),
    ("spec_gdn_no_triangular_solve",
     "for (int m = 1; m < i; ++m) {\n                    const double a = bt[i - 1]",
     "for (int m = 1; m < 1; ++m) {\n                    const double a = bt[i - 1]"),
    ("spec_gdn_solve_decay_off_by_one",
     "const double a = bt[i - 1] * gamma_range(ad, m + 1, i) * dot(",
     "const double a = bt[i - 1] * gamma_range(ad, m, i) * dot("),
    ("spec_gdn_drop_beta",
     "ui[r] = bt[i - 1] * (vt[(int64_t)(i - 1) * dv + r] - Di * shk[r]);",
     "ui[r] = (vt[(int64_t)(i - 1) * dv + r] - Di * shk[r]);"),
    ("spec_gdn_state_read_at_q",
     "matvec(Ct, ki, dv, dk, y);",
     "matvec(Ct, qi, dv, dk, y);"),
    ("spec_gdn_drafts_store_v",
     "memcpy(xt + (int64_t)(base + i) * dv, u + (int64_t)i * dv, sizeof(double) * (size_t)dv);",
     "memcpy(xt + (int64_t)(base + i) * dv, vt + (int64_t)i * dv, sizeof(double) * (size_t)dv);"),
    ("spec_commit_one_short",
     "if (!active || active[t]) h[t] += accepted[t];",
     "if (!active || active[t]) h[t] += accepted[t] > 0 ? accepted[t] - 1 : 0;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut_src = tmp_path / "mutant.c"
    mut_src.write_text(src.replace(old, new))
    lib = oracle.build(str(mut_src), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


# ------------------------------------------------ two-copy model mutants --
def _broken_two_copy(kind):
    """A TwoCopyReplayModel with one planted mistake (Python level)."""
    import numpy as np
    from oracle import MAMBA2, TwoCopyReplayModel, _scal, _vec, round_to

    class Broken(TwoCopyReplayModel):
        def step(self, q, k, v, lam, flush_rows, beta=None, active_rows=None):
            B, H = self.B, self.H
            n = B * H
            fl = np.repeat(np.asarray(flush_rows, bool), H)
            act = np.ones(n, bool)
            args = (_vec(q, n), _vec(k, n), _vec(v, n), _scal(lam, n), None)
            read = self.C if kind == "nonflush_reads_recurrence_copy" else self.C_lo
            fold = self.C_lo if kind == "flush_folds_read_copy" else self.C
            out = self.o.replay_step(MAMBA2, read, self.rec_lam, self.rec_x, self.rec_k, self.w, fl, *args,
                                     act & ~fl)
            out += self.o.replay_step(MAMBA2, fold, self.rec_lam, self.rec_x, self.rec_k, self.w, fl, *args,
                                      act & fl)
            if kind == "flush_folds_read_copy":
                self.C[fl] = fold[fl]
            if kind != "read_copy_not_refreshed":
                self.C_lo[fl] = round_to(self.C[fl], self.read_dtype)
            return out.reshape(B, H, self.dv)

    return Broken


@pytest.mark.parametrize("kind", ["nonflush_reads_recurrence_copy", "flush_folds_read_copy",
                                  "read_copy_not_refreshed"])
def test_two_copy_mutant_is_caught(monkeypatch, kind):
    import pins
    monkeypatch.setattr(oracle, "TwoCopyReplayModel", _broken_two_copy(kind))
    caught = []
    for pin in (pins.pin_two_copy_read_error_is_one_rounding, pins.pin_two_copy_error_does_not_accumulate):
        try:
            pin(oracle.get())
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"two-copy mutant {kind} passed both pins"


def _broken_spec_two_copy(kind):
    """A SpecTwoCopyModel with one planted mistake (Python level)."""
    import numpy as np
    from oracle import MAMBA2, SpecTwoCopyModel, round_to

    class Broken(SpecTwoCopyModel):
        def verify(self, q, k, v, lam, flush_rows, active_rows=None, beta=None):
            B, H, T = self.B, self.H, self.T
            n = B * H
            fl = np.repeat(np.asarray(flush_rows, bool), H)
            act = np.ones(n, bool)
            f = lambda a, d: np.ascontiguousarray(np.asarray(a, np.float64).reshape(n, T, d))
            sc = lambda a: np.ascontiguousarray(np.asarray(a, np.float64).reshape(n, T))
            args = (f(q, self.dk), f(k, self.dk), f(v, self.dv), sc(lam))
            if kind == "read_copy_refreshed_before_the_fold":
                self.C_lo[fl] = round_to(self.C[fl], self.read_dtype)
            read = self.C if kind == "nonflush_reads_recurrence_copy" else self.C_lo
            fold = self.C_lo if kind == "flush_reads_read_copy" else self.C
            out = self.o.spec_verify(read, self.rec_lam, self.rec_x, self.rec_k, self.h, fl, *args, act & ~fl)
            out += self.o.spec_verify(fold, self.rec_lam, self.rec_x, self.rec_k, self.h, fl, *args, act & fl)
            if kind == "flush_reads_read_copy":
                self.C[fl] = fold[fl]
            if kind not in ("read_copy_not_refreshed", "read_copy_refreshed_before_the_fold"):
                self.C_lo[fl] = round_to(self.C[fl], self.read_dtype)
            return out.reshape(B, H, T, self.dv)

    return Broken


@pytest.mark.parametrize("kind", ["nonflush_reads_recurrence_copy", "flush_reads_read_copy",
                                  "read_copy_not_refreshed", "read_copy_refreshed_before_the_fold"])
def test_spec_two_copy_mutant_is_caught(monkeypatch, kind):
    """Mistakes in which copy a speculative verify reads, or in when the read
    copy is refreshed, must fail pin_spec_two_copy."""
    import pins
    monkeypatch.setattr(oracle, "SpecTwoCopyModel", _broken_spec_two_copy(kind))
    with pytest.raises(AssertionError):
        pins.pin_spec_two_copy(oracle.get())


@pytest.mark.parametrize("kind", ["read_copy_from_rounded_recurrence", "recurrence_nearest_even",
                                  "recurrence_words_of_step_zero"])
def test_two_copy_store_mutant_is_caught(monkeypatch, kind):
    """Mistakes in how a flush stores the two copies of an fp16 recurrence
    copy must fail the two-copy pins."""
    import numpy as np
    import pins
    from oracle import formats

    def broken_store(self, mask, sr_step):
        for t in np.nonzero(mask)[0]:
            step = 0 if kind == "recurrence_words_of_step_zero" else sr_step
            if kind == "read_copy_from_rounded_recurrence":
                self.C[t] = formats.sr_f16(self.C[t].reshape(-1), formats.sr_words(
                    self.key, step, self.tile_ids[t], self.dv * self.dk)).reshape(self.dv, self.dk)
                self.C_lo[t] = formats.round_to(self.C[t], self.read_dtype)
                continue
            self.C_lo[t] = formats.round_to(self.C[t], self.read_dtype)
            if kind == "recurrence_nearest_even":
                self.C[t] = formats.round_to(self.C[t], "f16")
            else:
                self.C[t] = formats.sr_f16(self.C[t].reshape(-1), formats.sr_words(
                    self.key, step, self.tile_ids[t], self.dv * self.dk)).reshape(self.dv, self.dk)

    monkeypatch.setattr(oracle.TwoCopyReplayModel, "_store", broken_store)
    with pytest.raises(AssertionError):
        pins.pin_two_copy_f16_recurrence(oracle.get())


# ---------------------------------------------- read-format mutants --
def _format_mutants():
    import numpy as np
    from oracle import formats as F
    enc, rexp, hu = F.e4m3_encode, F.e4m3_row_exponent, F.half_ulp

    def truncating_encode(y):
        # rounds toward zero instead of to nearest even
        y = np.asarray(y, np.float64)
        a = np.abs(y)
        fr, ex = np.frexp(np.maximum(a, 2.0**-6))
        E = ex - 1
        q = np.where(a < 2.0**-6, 2.0**-9, np.ldexp(1.0, (E - 3).astype(np.int32)))
        code = np.where(a < 2.0**-6, np.floor(a / q), (E + 7) * 8 + np.floor(a / q) - 8).astype(np.int64)
        return (np.minimum(code, 0x7E) | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)

    def fnuz_encode(y):
        # the other common E4M3 variant: exponent bias 8
        return enc(np.asarray(y, np.float64) * 2.0)

    return {
        "e4m3_truncates": ("e4m3_encode", truncating_encode),
        "e4m3_bias_8": ("e4m3_encode", fnuz_encode),
        "row_exponent_one_low": ("e4m3_row_exponent", lambda x: rexp(x) - 1),
        "row_exponent_not_minimal": ("e4m3_row_exponent", lambda x: rexp(x) + 1),
        "half_ulp_too_big": ("half_ulp", lambda x, dt: 2 * hu(x, dt)),
        "half_ulp_too_small": ("half_ulp", lambda x, dt: 0.5 * hu(x, dt)),
    }


@pytest.mark.parametrize("kind", sorted(_format_mutants()))
def test_format_mutant_is_caught(monkeypatch, kind):
    import pins
    from oracle import formats
    name, fn = _format_mutants()[kind]
    monkeypatch.setattr(formats, name, fn)
    if name == "half_ulp":
        monkeypatch.setattr(oracle, "half_ulp", fn)
    caught = []
    for pin in (pins.pin_e4m3_matches_library_cast, pins.pin_e4m3_spec_values,
                pins.pin_read_rounding_within_half_ulp, pins.pin_two_copy_read_error_is_one_rounding):
        try:
            pin(oracle.get())
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"format mutant {kind} passed every pin"


def test_two_copy_bound_without_decay_is_caught(monkeypatch):
    """read_error_bound that forgets gamma_h (too loose on decayed steps)."""
    import numpy as np
    import pins
    from oracle import TwoCopyReplayModel, _vec, half_ulp

    class Broken(TwoCopyReplayModel):
        def read_error_bound(self, q, lam):
            n = self.B * self.H
            u = half_ulp(self.C, self.read_dtype)
            return np.einsum("nic,nc->ni", u, np.abs(_vec(q, n))).reshape(self.B, self.H, self.dv) * 50.0

    monkeypatch.setattr(oracle, "TwoCopyReplayModel", Broken)
    with pytest.raises(AssertionError):
        pins.pin_two_copy_read_error_is_one_rounding(oracle.get())


# ------------------------------------------ stochastic-rounding mutants --
def _sr_mutants():
    import numpy as np
    from oracle import formats as F
    sr, ph = F.sr_f16, F.philox4x64

    def nearest(x, r):                      # no stochastic choice at all
        return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)

    def flipped(x, r):                      # rounds up with probability 1 - p
        return sr(x, 2.0**16 - 1 - np.asarray(r, np.float64))

    def truncate(x, r):                     # always the neighbour towards zero
        return sr(x, np.full(np.shape(x), 2.0**16))

    def no_key_bump(counter, key):          # key not advanced between rounds
        import numpy as np
        c = np.array(np.broadcast_to(np.asarray(counter, np.uint64), np.shape(counter)), np.uint64)
        k = np.asarray(key, np.uint64)
        c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
        with np.errstate(over="ignore"):
            for _ in range(10):
                hi0, lo0 = F._mulhilo64(F._PH_M0, c0)
                hi1, lo1 = F._mulhilo64(F._PH_M1, c2)
                c0, c1, c2, c3 = hi1 ^ c1 ^ k[..., 0], lo1, hi0 ^ c3 ^ k[..., 1], lo0
        return np.stack([c0, c1, c2, c3], axis=-1)

    def nine_rounds(counter, key):
        import numpy as np
        out = ph(counter, key)
        return out ^ np.uint64(1)           # any corruption of the output words

    def _words(key, step, tile, n, per_block, order):
        n_blk = (n + per_block - 1) // per_block
        ctr = np.zeros((n_blk, 4), np.uint64)
        ctr[:, 0], ctr[:, 1] = np.uint64(step), np.uint64(tile)
        ctr[:, 2] = np.arange(n_blk, dtype=np.uint64)
        out = ph(ctr, np.asarray(key, np.uint64))
        sh = np.arange(4, dtype=np.uint64)[::order] * np.uint64(16)
        w = ((out[..., None] >> sh) & np.uint64(0xFFFF)).reshape(n_blk, 16)[:, :per_block]
        return w.reshape(-1)[:n]

    def words_high_first(key, step, tile, n):     # most significant half-word first
        return _words(key, step, tile, n, 16, -1)

    def words_eight_per_block(key, step, tile, n):  # a block per 8 elements
        return _words(key, step, tile, n, 8, 1)

    def words_step_tile_swapped(key, step, tile, n):
        return _words(key, tile, step, n, 16, 1)

    return {"sr_nearest": ("sr_f16", nearest), "sr_flipped": ("sr_f16", flipped),
            "sr_truncate": ("sr_f16", truncate), "philox_no_key_bump": ("philox4x64", no_key_bump),
            "philox_corrupt": ("philox4x64", nine_rounds), "words_high_first": ("sr_words", words_high_first),
            "words_eight_per_block": ("sr_words", words_eight_per_block),
            "words_step_tile_swapped": ("sr_words", words_step_tile_swapped)}


@pytest.mark.parametrize("kind", sorted(_sr_mutants()))
def test_sr_mutant_is_caught(monkeypatch, kind):
    import pins
    from oracle import formats
    name, fn = _sr_mutants()[kind]
    monkeypatch.setattr(formats, name, fn)
    caught = []
    for pin in (pins.pin_philox_matches_library, pins.pin_sr_rule, pins.pin_sr_words_layout,
                pins.pin_sr_once_per_window):
        try:
            pin(oracle.get())
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"stochastic-rounding mutant {kind} passed every pin"
