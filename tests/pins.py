"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with the fact it checks.  ``test_oracle.py`` runs
them on the real oracle; ``test_oracle_mutants.py`` runs them on copies of the
oracle with planted mistakes and requires every mistake to be caught.

Sources of the facts (pages):
  [blog] "ReplaySSM: an SSM decoder that writes its state once every 16
         tokens": recurrence ("Why a fixed-size state is not cheap to
         decode"), the unrolled identity ("The identity"), the output-only
         bracketing ("Output without a state"), the delta-rule expansion
         ("The delta-rule wrinkle"), two checkpoint copies ("The precision
         argument, derived").
  [pr]   vLLM pull request "[Kernel] ReplaySSM: cache SSM inputs for faster
         Gated DeltaNet standard decode": cursor and flush rule ("CUDA graphs
         and continuous batching").
  [ofp8] Open Compute Project "OCP 8-bit Floating Point Specification
         (OFP8)": the E4M3 encoding (bias 7, no infinities, max 448,
         subnormals m/8 * 2^-6); the format is not on the pages.
  [philox] Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
         1, 2, 3" (SC 2011): the Philox4x64-10 generator (not on the pages;
         it supplies the random bits of stochastic rounding).
  [nv]   NVIDIA technical blog "ReplaySSM: Rethinking state storage for
         faster hybrid model decoding", section "Benefit 2: Simplify rollback
         and speed up verification" (speculative verify); with [blog]
         "Speculative decoding: rollback becomes a pointer".
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads

M2, GDN = oracle.MAMBA2, oracle.GDN


def _tok(form, seed, step, B, H, dv, dk, a_lo=1.0, a_hi=8.0):
    t = workloads.tokens(form, seed, step, B, H, dv, dk, "f32", a_lo, a_hi)
    f = lambda x: x.double().numpy()
    return f(t.q), f(t.k), f(t.v), f(t.lam), (None if t.beta is None else f(t.beta))


def _rel(a, b):
    """max |a - b| / max |b| over the last axis, worst case over the rest."""
    a, b = np.asarray(a), np.asarray(b)
    num = np.abs(a - b).reshape(-1, a.shape[-1]).max(-1)
    den = np.maximum(np.abs(b).reshape(-1, b.shape[-1]).max(-1), 1e-300)
    return float((num / den).max())


def run_both(orc, form, B, H, dv, dk, L, n_steps, seed=0, a_lo=1.0, a_hi=8.0, forced=None,
             check_flush_state=True):
    """Run the conventional and the checkpoint + buffer routes side by side.

    Returns (max output relative deviation, max flushed-state deviation,
    number of flush steps).  Both routes start from a zero state; the flush
    schedule comes from the oracle's cursor."""
    conv = oracle.ConventionalModel(form, B, H, dv, dk, oracle=orc)
    rep = oracle.ReplayModel(form, B, H, dv, dk, L, oracle=orc)
    ws, fls = orc.cursor_run(L, 0, n_steps, forced)
    worst_o, worst_s, n_flush = 0.0, 0.0, 0
    for s in range(n_steps):
        q, k, v, lam, beta = _tok(form, seed, s, B, H, dv, dk, a_lo, a_hi)
        assert np.all(rep.w == ws[s]), "replay route holds a different number of records than the cursor"
        o_c = conv.step(q, k, v, lam, beta)
        o_r = rep.step(q, k, v, lam, np.full(B, fls[s]), beta)
        worst_o = max(worst_o, _rel(o_r, o_c))
        if fls[s]:
            n_flush += 1
            if check_flush_state:
                worst_s = max(worst_s, _rel(rep.checkpoint(), conv.state()))
    return worst_o, worst_s, n_flush


# ---------------------------------------------------------------- identity --
def pin_identity_mamba2_tiny(orc):
    """[blog] "The identity": both sides are the same matrix; outputs agree up
    to floating-point order.  Tiny Mamba-2 workload: batch 2, 4 heads, 16x32,
    L=4, 64 steps from zero (16 flushes)."""
    o, s, nf = run_both(orc, M2, 2, 4, 16, 32, 4, 64)
    assert nf == 16
    assert o < 1e-12 and s < 1e-12, (o, s)


def pin_identity_mamba2_long_memory(orc):
    """Same identity with slowly decaying heads (a ~ U[0.001, 0.01]), where the
    checkpoint term stays dominant and an error in it cannot hide."""
    o, s, _ = run_both(orc, M2, 2, 4, 16, 32, 4, 64, seed=3, a_lo=0.001, a_hi=0.01)
    assert o < 1e-12 and s < 1e-12, (o, s)


def pin_identity_gdn_tiny(orc):
    """[pr] reviewer comment: S_{t-1} q and S_{t-1} k rebuilt from checkpoint
    plus buffer equal the conventional delta-rule state's."""
    o, s, nf = run_both(orc, GDN, 2, 4, 16, 32, 4, 64, seed=1)
    assert nf == 16
    assert o < 1e-12 and s < 1e-12, (o, s)


def pin_identity_long_window(orc):
    """L=16 (the pages' default) and forced flushes at irregular steps."""
    forced = np.zeros(80, np.uint8)
    forced[[5, 6, 30, 51]] = 1
    for form in (M2, GDN):
        o, s, nf = run_both(orc, form, 1, 2, 16, 32, 16, 80, seed=7, forced=forced)
        assert nf >= 4
        assert o < 1e-12 and s < 1e-12, (form, o, s)


# ---------------------------------------------------------- special cases --
def pin_single_step_from_zero(orc):
    """One update from a zero state: o = (v k^T) q = v (k^T q) ([blog]
    "Output without a state").  For Gated DeltaNet the zero state makes the
    corrected value beta v, so o = beta v (k . q)."""
    B, H, dv, dk = 2, 3, 16, 32
    for form in (M2, GDN):
        q, k, v, lam, beta = _tok(form, 11, 0, B, H, dv, dk)
        want = v * np.einsum("bhc,bhc->bh", k, q)[..., None]
        if form == GDN:
            want = want * beta[..., None]
        conv = oracle.ConventionalModel(form, B, H, dv, dk, oracle=orc)
        got_c = conv.step(q, k, v, lam, beta)
        for fl in (False, True):
            rep = oracle.ReplayModel(form, B, H, dv, dk, 4, oracle=orc)
            got_r = rep.step(q, k, v, lam, np.full(B, fl), beta)
            assert _rel(got_r, want) < 1e-13, (form, fl)
        assert _rel(got_c, want) < 1e-13, form


def pin_no_decay_is_plain_sum(orc):
    """alpha = 1 (lam = 0): the state is the plain sum of outer products."""
    B, H, dv, dk, n = 1, 2, 16, 32, 9
    conv = oracle.ConventionalModel(M2, B, H, dv, dk, oracle=orc)
    rep = oracle.ReplayModel(M2, B, H, dv, dk, 4, oracle=orc)
    ws, fls = orc.cursor_run(4, 0, n)
    acc = np.zeros((B, H, dv, dk))
    for s in range(n):
        q, k, v, lam, _ = _tok(M2, 5, s, B, H, dv, dk)
        lam = np.zeros_like(lam)
        acc += np.einsum("bhi,bhc->bhic", v, k)
        want = np.einsum("bhic,bhc->bhi", acc, q)
        assert _rel(conv.step(q, k, v, lam), want) < 1e-12
        assert _rel(rep.step(q, k, v, lam, np.full(B, fls[s])), want) < 1e-12
        assert _rel(conv.state(), acc) < 1e-12


def pin_constant_decay_geometric(orc):
    """Constant alpha: S_t = sum_{j<=t} alpha^{t-j} v_j k_j^T (the unrolled
    recurrence with gamma_{j+1:t} = alpha^{t-j})."""
    B, H, dv, dk, n, L = 1, 2, 16, 32, 11, 4
    alpha = 0.8
    conv = oracle.ConventionalModel(M2, B, H, dv, dk, oracle=orc)
    rep = oracle.ReplayModel(M2, B, H, dv, dk, L, oracle=orc)
    ws, fls = orc.cursor_run(L, 0, n)
    vs, ks = [], []
    for s in range(n):
        q, k, v, lam, _ = _tok(M2, 6, s, B, H, dv, dk)
        lam = np.full_like(lam, np.log(alpha))
        vs.append(v)
        ks.append(k)
        S = sum(alpha ** (s - j) * np.einsum("bhi,bhc->bhic", vs[j], ks[j]) for j in range(s + 1))
        want = np.einsum("bhic,bhc->bhi", S, q)
        assert _rel(conv.step(q, k, v, lam), want) < 1e-12, s
        assert _rel(rep.step(q, k, v, lam, np.full(B, fls[s])), want) < 1e-12, s


def pin_full_forgetting(orc):
    """alpha = 0 (lam = -inf): S_t = v_t k_t^T and the checkpoint and buffer
    contribute nothing."""
    B, H, dv, dk = 1, 2, 16, 32
    conv = oracle.ConventionalModel(M2, B, H, dv, dk, oracle=orc)
    rep = oracle.ReplayModel(M2, B, H, dv, dk, 4, oracle=orc)
    ws, fls = orc.cursor_run(4, 0, 7)
    for s in range(7):
        q, k, v, lam, _ = _tok(M2, 8, s, B, H, dv, dk)
        if s in (2, 5):
            lam = np.full_like(lam, -np.inf)
            want = v * np.einsum("bhc,bhc->bh", k, q)[..., None]
        o_c = conv.step(q, k, v, lam)
        o_r = rep.step(q, k, v, lam, np.full(B, fls[s]))
        assert _rel(o_r, o_c) < 1e-12
        if s in (2, 5):
            assert _rel(o_c, want) < 1e-13 and _rel(o_r, want) < 1e-13


def pin_gdn_product_form(orc):
    """[blog] "The delta-rule wrinkle": the conventional Gated DeltaNet update
    equals the product form S_t = alpha S_{t-1} (I - beta k k^T) + beta v k^T,
    evaluated here with plain matrix products."""
    B, H, dv, dk = 2, 2, 16, 32
    conv = oracle.ConventionalModel(GDN, B, H, dv, dk, oracle=orc)
    S = np.zeros((B, H, dv, dk))
    I = np.eye(dk)
    for s in range(6):
        q, k, v, lam, beta = _tok(GDN, 9, s, B, H, dv, dk)
        k = k * 1.3  # off the unit sphere so that the k k^T term is not special
        o = conv.step(q, k, v, lam, beta)
        for b in range(B):
            for h in range(H):
                a, bt = np.exp(lam[b, h]), beta[b, h]
                P = I - bt * np.outer(k[b, h], k[b, h])
                S[b, h] = a * S[b, h] @ P + bt * np.outer(v[b, h], k[b, h])
        assert _rel(conv.state(), S) < 1e-12, s
        assert _rel(o, np.einsum("bhic,bhc->bhi", S, q)) < 1e-12, s


def pin_gdn_unit_key_stores_value(orc):
    """Gated DeltaNet with beta = 1 and |k| = 1: the update overwrites the
    state's response to k with v, S_t k_t = v_t, for any alpha and prior state
    (expand alpha S (I - k k^T) k + v k^T k)."""
    B, H, dv, dk, L = 2, 2, 16, 32, 4
    conv = oracle.ConventionalModel(GDN, B, H, dv, dk, oracle=orc)
    rep = oracle.ReplayModel(GDN, B, H, dv, dk, L, oracle=orc)
    ws, fls = orc.cursor_run(L, 0, 9)
    for s in range(9):
        q, k, v, lam, beta = _tok(GDN, 10, s, B, H, dv, dk)
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)  # exactly unit in fp64
        beta = np.ones_like(beta)
        conv.step(q, k, v, lam, beta)
        rep.step(q, k, v, lam, np.full(B, fls[s]), beta)
        Sk = np.einsum("bhic,bhc->bhi", conv.state(), k)
        assert _rel(Sk, v) < 1e-12, s
        if fls[s]:
            assert _rel(np.einsum("bhic,bhc->bhi", rep.checkpoint(), k), v) < 1e-12, s


def pin_gdn_zero_beta_only_decays(orc):
    """Gated DeltaNet with beta = 0 writes nothing: S_t = alpha S_{t-1}, and the
    buffered corrected values are zero."""
    B, H, dv, dk, L = 1, 2, 16, 32, 4
    conv = oracle.ConventionalModel(GDN, B, H, dv, dk, oracle=orc)
    rep = oracle.ReplayModel(GDN, B, H, dv, dk, L, oracle=orc)
    ws, fls = orc.cursor_run(L, 0, 12)
    for s in range(12):
        q, k, v, lam, beta = _tok(GDN, 12, s, B, H, dv, dk)
        if s >= 5:
            beta = np.zeros_like(beta)
        before = conv.state().copy()
        o_c = conv.step(q, k, v, lam, beta)
        o_r = rep.step(q, k, v, lam, np.full(B, fls[s]), beta)
        if s >= 5:
            want = np.exp(lam)[..., None, None] * before
            assert _rel(conv.state(), want) < 1e-13, s
            assert _rel(o_c, np.einsum("bhic,bhc->bhi", want, q)) < 1e-12
        assert _rel(o_r, o_c) < 1e-12, s
        if s == 10:  # steps 8, 9, 10 are buffered, all with beta = 0
            assert np.all(rep.w == 3)
            assert np.all(rep.rec_x[:, :3] == 0.0)


# ------------------------------------------------------------------- fold --
def pin_fold_materialises_state(orc):
    """A token-less fold of w records gives the conventional state after
    those w tokens ([blog] "The identity" with h = w); folding nothing leaves
    the checkpoint unchanged; decoding continues identically afterwards."""
    B, H, dv, dk, L = 2, 2, 16, 32, 8
    for form in (M2, GDN):
        conv = oracle.ConventionalModel(form, B, H, dv, dk, oracle=orc)
        rep = oracle.ReplayModel(form, B, H, dv, dk, L, oracle=orc)
        for s in range(13):
            q, k, v, lam, beta = _tok(form, 13, s, B, H, dv, dk)
            conv.step(q, k, v, lam, beta)
            rep.step(q, k, v, lam, rep.records_held()[:, 0] == L - 1, beta)
            if s in (4, 9):
                rep.fold(np.array([True, s == 9]))
                sel = [0] if s == 4 else [0, 1]
                assert _rel(rep.checkpoint()[sel], conv.state()[sel]) < 1e-12, (form, s)
                assert np.all(rep.records_held()[sel] == 0)
        rep.fold(np.array([True, True]))
        assert _rel(rep.checkpoint(), conv.state()) < 1e-12
        after = rep.checkpoint().copy()
        rep.fold(np.array([True, True]))  # no records left: unchanged
        assert np.array_equal(rep.checkpoint(), after)
        for s in range(13, 20):  # decoding continues from the folded state
            q, k, v, lam, beta = _tok(form, 13, s, B, H, dv, dk)
            o_c = conv.step(q, k, v, lam, beta)
            o_r = rep.step(q, k, v, lam, rep.records_held()[:, 0] == L - 1, beta)
            assert _rel(o_r, o_c) < 1e-12, (form, s)


# ----------------------------------------------------------------- cursor --
def pin_cursor_closed_form(orc):
    """[pr] "CUDA graphs and continuous batching": without forcing, the write
    position after n steps from w0 is (w0 + n) mod L, a row flushes when it
    reaches L - 1, and n steps hold floor((w0 + n) / L) flushes."""
    for L in (1, 2, 4, 16, 33, 64):
        for w0 in sorted({0, min(1, L - 1), L // 2, L - 1}):
            n = 5 * L + 3
            w, f = orc.cursor_run(L, w0, n)
            assert np.array_equal(w, (w0 + np.arange(n)) % L), (L, w0)
            assert np.array_equal(f, w == L - 1)
            assert int(f.sum()) == (w0 + n) // L
    w, f = orc.cursor_run(4, 0, 64)
    assert list(np.nonzero(f)[0]) == list(range(3, 64, 4))


def pin_cursor_forced_flush(orc):
    """A forced flush (prefix-cache align mode, [pr] "What this PR adds")
    empties the buffer at once: the next step writes position 0."""
    forced = np.zeros(20, np.uint8)
    forced[[2, 3, 11]] = 1
    w, f = orc.cursor_run(16, 0, 20, forced)
    assert list(w[:6]) == [0, 1, 2, 0, 0, 1]
    assert list(np.nonzero(f)[0]) == [2, 3, 11]
    assert w[12] == 0 and w[19] == 7


# ------------------------------------------------- two-precision checkpoint --
def pin_two_copy_read_error_is_one_rounding(orc):
    """[blog] "The precision argument, derived": with an exact recurrence copy
    and a read copy rounded once per flush, a non-flush step h positions into
    the window outputs o_t + gamma_h eps_m q_t, eps_m = C_lo - C; a flush step
    reads the recurrence copy and is exact.  Checked against the exact
    checkpoint + buffer route on the same inputs for each read format, with
    eps_m one rounding of the last checkpoint (within half an ulp of it), and
    the model's error bound gamma_h sum |u| |q| holding and not loose."""
    B, H, dv, dk, L = 2, 3, 16, 32, 4
    for dt in ("f16", "bf16", "e4m3"):
        exact = oracle.ReplayModel(M2, B, H, dv, dk, L, oracle=orc)
        two = oracle.TwoCopyReplayModel(B, H, dv, dk, L, dt, oracle=orc)
        ws, fls = orc.cursor_run(L, 0, 40)
        since = np.zeros((B, H))  # log of gamma_h: decays since the checkpoint, current token included
        tight = 0.0
        for s in range(40):
            q, k, v, lam, _ = _tok(M2, 21, s, B, H, dv, dk, 0.001, 0.01)
            since = since + lam
            eps = (two.C_lo - two.C).reshape(B, H, dv, dk)
            bound = two.read_error_bound(q, lam)
            o_e = exact.step(q, k, v, lam, np.full(B, fls[s]))
            o_t = two.step(q, k, v, lam, np.full(B, fls[s]))
            if fls[s]:
                assert _rel(o_t, o_e) < 1e-12, (dt, s)
                since = np.zeros((B, H))
            else:
                want = np.exp(since)[..., None] * np.einsum("bhic,bhc->bhi", eps, q)
                d = o_t - o_e
                scale = np.abs(o_e).max()
                assert np.abs(d - want).max() <= 1e-12 * scale, (dt, s)
                assert np.all(np.abs(d) <= bound * (1 + 1e-9) + 1e-12 * scale), (dt, s)
                if s > 4:
                    tight = max(tight, float((np.abs(d) / np.maximum(bound, 1e-300)).max()))
            # the read copy is one rounding of the recurrence copy
            C = two.C
            assert np.all(np.abs(two.C_lo - C) <= oracle.half_ulp(C, dt)), (dt, s)
            assert _rel(two.C.reshape(B, H, dv, dk), exact.checkpoint()) < 1e-12
        assert tight > 0.05, (dt, tight)


def pin_two_copy_error_does_not_accumulate(orc):
    """The read error stays at one rounding over many windows, while a single
    checkpoint rounded at every flush (and fed back) drifts further: long-memory
    heads, 50 windows."""
    B, H, dv, dk, L, steps = 1, 4, 16, 32, 8, 400
    exact = oracle.ReplayModel(M2, B, H, dv, dk, L, oracle=orc)
    two = oracle.TwoCopyReplayModel(B, H, dv, dk, L, "f16", oracle=orc)
    single = oracle.ReplayModel(M2, B, H, dv, dk, L, oracle=orc)  # its checkpoint re-rounded at each flush
    ws, fls = orc.cursor_run(L, 0, steps)
    err_two, err_single = [], []
    for s in range(steps):
        q, k, v, lam, _ = _tok(M2, 22, s, B, H, dv, dk, 0.0005, 0.001)
        o_e = exact.step(q, k, v, lam, np.full(B, fls[s]))
        o_t = two.step(q, k, v, lam, np.full(B, fls[s]))
        o_s = single.step(q, k, v, lam, np.full(B, fls[s]))
        if fls[s]:
            single.C[:] = oracle.round_to(single.C, "f16")
        scale = max(np.abs(o_e).max(), 1e-300)
        err_two.append(np.abs(o_t - o_e).max() / scale)
        err_single.append(np.abs(o_s - o_e).max() / scale)
    late_two, late_single = max(err_two[-50:]), max(err_single[-50:])
    assert late_two < 2.0**-10, late_two          # about one fp16 rounding
    assert max(err_two[-50:]) < 3 * max(err_two[50:100])  # not growing
    assert late_single > 2 * late_two, (late_single, late_two)


def pin_two_copy_f16_recurrence(orc):
    """[blog] "The precision argument, derived": a flush casts the same
    unrounded fold into both copies.  With an fp16 recurrence copy under
    stochastic rounding and an E4M3 read copy, three windows: after each
    flush the read copy is the E4M3 rounding of the fold computed (by a
    separate exact model started from the stored recurrence copy) before any
    rounding, the recurrence copy is that fold under the Philox words of
    (flush step, tile), and the non-flush outputs are those of the exact
    model from the read copy."""
    from oracle import formats
    B, H, dv, dk, L = 2, 3, 16, 32, 4
    key = np.array([3, 5], np.uint64)
    tiles = np.arange(B * H) + 40
    two = oracle.TwoCopyReplayModel(B, H, dv, dk, L, "e4m3", oracle=orc, rec_dtype="f16", key=key, tile_ids=tiles)
    ws, fls = orc.cursor_run(L, 0, 3 * L)
    for s in range(3 * L):
        q, k, v, lam, _ = _tok(M2, 31, s, B, H, dv, dk)
        ref = oracle.ReplayModel(M2, B, H, dv, dk, L, oracle=orc)
        ref.C, ref.rec_lam, ref.rec_x, ref.rec_k, ref.w = (two.C.copy(), two.rec_lam.copy(), two.rec_x.copy(),
                                                       two.rec_k.copy(), two.w.copy())
        if not fls[s]:
            ref.C = two.C_lo.copy()      # a non-flush step reads the read copy
        o_ref = ref.step(q, k, v, lam, np.full(B, fls[s]))
        o = two.step(q, k, v, lam, np.full(B, fls[s]), sr_step=100 + s)
        assert np.allclose(o, o_ref, rtol=1e-12, atol=1e-12 * np.abs(o_ref).max()), s
        if fls[s]:
            assert np.array_equal(two.C_lo, formats.round_to(ref.C, "e4m3")), s
            for t in range(B * H):
                want = formats.sr_f16(ref.C[t].reshape(-1), formats.sr_words(key, 100 + s, tiles[t], dv * dk))
                assert np.array_equal(two.C[t].reshape(-1), want), (s, t)
            assert not np.array_equal(two.C, oracle.round_to(ref.C, "f16"))   # not nearest even
    assert int(fls.sum()) == 3


def pin_e4m3_matches_library_cast(orc):
    """[ofp8] E4M3 codes with round to nearest even: equal to torch's
    float8_e4m3fn cast (a library routine) on fp32 values spread over the
    whole finite range, ties and subnormals included; decoding equals the
    library's for all 256 codes."""
    import torch
    from oracle import formats
    rng = np.random.default_rng(5)
    x = rng.standard_normal(20000) * np.exp2(rng.uniform(-14, 9, 20000))
    ties = np.array([1 + 1 / 16, 1 + 3 / 16, 2.0**-9 * 1.5, 2.0**-9 * 2.5, 2.0**-10, 416.0, 240.0 + 8])
    x = np.concatenate([x, ties, -ties, [0.0, -0.0, 448.0, -448.0]])
    x = x[np.abs(x) <= 448].astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(formats.e4m3_encode(x), want)
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ours = formats.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(lib)) and np.array_equal(ours[~np.isnan(lib)], lib[~np.isnan(lib)])


def pin_e4m3_spec_values(orc):
    """[ofp8] Values the specification fixes: max normal 448 = S.1111.110,
    min normal 2^-6 = S.0001.000, max subnormal 7/8 2^-6, min subnormal 2^-9,
    1.0 = S.0111.000; halfway cases go to the even mantissa."""
    from oracle import formats
    enc = lambda v: int(formats.e4m3_encode(np.array([v]))[0])
    assert enc(448.0) == 0x7E and enc(-448.0) == 0xFE
    assert enc(2.0**-6) == 0x08 and enc(0.875 * 2.0**-6) == 0x07 and enc(2.0**-9) == 0x01
    assert enc(1.0) == 0x38 and enc(-2.0) == 0xC0 and enc(0.0) == 0x00
    assert enc(1 + 1 / 16) == 0x38 and enc(1 + 3 / 16) == 0x3A      # ties to even
    assert enc(2.0**-10) == 0x00 and enc(3 * 2.0**-10) == 0x02       # subnormal ties
    assert enc(0.9375 * 2.0**-6) == 0x08                             # rounds up into the normals
    assert np.isnan(formats.e4m3_decode(np.array([0x7F]))[0])


def pin_read_rounding_within_half_ulp(orc):
    """Every read format: round_to moves a value by at most half an ulp of
    its representation, the bound is reached (not loose), and an E4M3 row's
    power-of-two scale is the smallest that keeps the row within 448."""
    from oracle import formats
    rng = np.random.default_rng(6)
    x = rng.standard_normal((400, 64)) * np.exp2(rng.uniform(-12, 12, (400, 1)))
    for dt in ("f16", "bf16", "e4m3"):
        u = formats.half_ulp(x, dt)
        d = np.abs(formats.round_to(x, dt) - x)
        assert np.all(d <= u), dt
        assert (d / u).max() > 0.9, dt
    e = formats.e4m3_row_exponent(x)
    amax = np.abs(x).max(axis=1)
    assert np.all(np.ldexp(amax, -e) <= 448.0) and np.all(np.ldexp(amax, -(e - 1)) > 448.0)
    assert formats.e4m3_row_exponent(np.zeros((1, 8)))[0] == formats.E4M3_MIN_EXP


# ------------------------------------------------------ speculative verify --
def _spec_tok(seed, step, B, H, T, dv, dk, a_lo=0.05, a_hi=1.0):
    """T draft tokens per row: q, k [B, H, T, dk], v [B, H, T, dv], lam [B, H, T]."""
    toks = [_tok(M2, seed, 1000 * step + i, B, H, dv, dk, a_lo, a_hi) for i in range(T)]
    st = lambda idx: np.stack([t[idx] for t in toks], axis=2)
    return st(0), st(1), st(2), st(3)


def _spec_tok_gdn(seed, step, B, H, T, dv, dk):
    """Gated DeltaNet drafts: q, k [B, H, T, dk] unit-norm, v [B, H, T, dv],
    lam, beta [B, H, T]."""
    toks = [_tok(GDN, seed, 1000 * step + i, B, H, dv, dk) for i in range(T)]
    st = lambda idx: np.stack([t[idx] for t in toks], axis=2)
    return st(0), st(1), st(2), st(3), st(4)


def run_spec(orc, B, H, dv, dk, L, T, n_steps, accept, seed=0, a_lo=0.05, a_hi=1.0, form=M2):
    """Speculative verify against the token-by-token recurrence.  accept(s)
    gives the accepted counts [B] of step s.  Returns (max output deviation,
    max deviation of a flushed checkpoint from the committed state, number of
    flushing row-steps); for the Gated DeltaNet form also checks that the
    drafts' stored records hold the token-by-token corrected values."""
    spec = oracle.SpecReplayModel(B, H, dv, dk, L, T, oracle=orc, form=form)
    ref = oracle.SpecTokenByToken(B, H, dv, dk, T, oracle=orc, form=form)
    h = np.zeros(B, np.int32)
    worst_o = worst_s = 0.0
    n_flush = 0
    for s in range(n_steps):
        beta = None
        if form == M2:
            q, k, v, lam = _spec_tok(seed, s, B, H, T, dv, dk, a_lo, a_hi)
        else:
            q, k, v, lam, beta = _spec_tok_gdn(seed, s, B, H, T, dv, dk)
        fl = np.array([orc.spec_cursor_run(L, T, int(h[b]), np.zeros(1, np.int32))[1][0] for b in range(B)])
        assert np.array_equal(spec.committed()[:, 0], h), "the ring holds a different committed count"
        o_s = spec.verify(q, k, v, lam, fl, beta=beta)
        o_r = ref.verify(q, k, v, lam, beta)
        worst_o = max(worst_o, _rel(o_s, o_r))
        if form != M2:
            base = np.where(fl, 0, h)
            for b in range(B):
                x = spec.rec_x.reshape(B, H, L, dv)[b, :, base[b]:base[b] + T]
                worst_o = max(worst_o, _rel(x, ref.drafts_x[b]))
        if fl.any():
            n_flush += int(fl.sum())
            worst_s = max(worst_s, _rel(spec.checkpoint()[fl], ref.state()[fl]))
        a = np.asarray(accept(s), np.int32)
        spec.commit(a)
        ref.commit(a)
        h = np.where(fl, 0, h) + a
    return worst_o, worst_s, n_flush


def pin_spec_identity(orc):
    """[nv] "Benefit 2" / [blog] "Speculative decoding": the T outputs of one
    verify, from one checkpoint read, K^T Q and the causal decay matrix, are
    the outputs of running the drafts token by token; committing a drafts
    advances the pointer; a flush folds only committed records, and the
    folded checkpoint equals the committed state.  T = 1, 2, 4 with random
    accepted counts 0..T (several flushes per row)."""
    rng = np.random.default_rng(5)
    for T in (1, 2, 4):
        o, st, nf = run_spec(orc, 3, 2, 8, 12, 8, T, 30, lambda s: rng.integers(0, T + 1, 3), seed=T)
        assert nf >= 3, (T, nf)
        assert o < 1e-12 and st < 1e-12, (T, o, st)


def pin_spec_two_copy(orc):
    """[blog] "The precision argument, derived" with "Speculative
    decoding": over a two-precision checkpoint, a flushing row's outputs come
    from the exact recurrence copy (they equal the drafts run token by token
    from the committed state), and afterwards the read copy is that fold
    rounded to the read format; a row that does not flush reads the read
    copy: right after a flush that committed nothing, its outputs equal the
    drafts run token by token from the read copy.  f16 and E4M3, T = 2,
    every third step forced to flush with nothing accepted."""
    B, H, dv, dk, L, T = 2, 2, 8, 12, 8, 2
    rng = np.random.default_rng(61)
    for rd in ("f16", "e4m3"):
        two = oracle.SpecTwoCopyModel(B, H, dv, dk, L, T, rd, oracle=orc)
        ref = oracle.SpecTokenByToken(B, H, dv, dk, T, oracle=orc)
        h = np.zeros(B, np.int32)
        checked_lo = checked_fl = 0
        shows = False
        for s in range(24):
            q, k, v, lam = _spec_tok(61, s, B, H, T, dv, dk)
            forced = s % 3 == 1
            fl = np.array([forced or orc.spec_cursor_run(L, T, int(h[b]), np.zeros(1, np.int32))[1][0]
                           for b in range(B)], bool)
            from_lo = None
            if s % 3 == 2:  # after a forced flush that committed nothing: h = 0 on every row
                assert not h.any() and not fl.any()
                from_lo = oracle.SpecTokenByToken(B, H, dv, dk, T, S0=two.C_lo.copy(), oracle=orc).verify(q, k, v, lam)
            o = two.verify(q, k, v, lam, fl)
            o_exact = ref.verify(q, k, v, lam)
            if fl.any():
                assert _rel(o[fl], o_exact[fl]) < 1e-12, (rd, s)
                C = two.checkpoint()[fl]
                assert _rel(C, ref.state()[fl]) < 1e-12, (rd, s)
                assert np.array_equal(two.C_lo.reshape(B, H, dv, dk)[fl], oracle.round_to(C, rd)), (rd, s)
                checked_fl += 1
            if from_lo is not None:
                assert _rel(o, from_lo) < 1e-12, (rd, s)
                shows = shows or _rel(o, o_exact) > 1e-6  # the read copy's rounding shows
                checked_lo += 1
            a = np.zeros(B, np.int32) if forced else rng.integers(0, T + 1, B).astype(np.int32)
            two.commit(a)
            ref.commit(a)
            h = np.where(fl, 0, h) + a
        assert checked_lo >= 6 and checked_fl >= 8 and shows, (rd, checked_lo, checked_fl, shows)


def pin_spec_gdn_identity(orc):
    """[blog] "The delta-rule wrinkle" and "Speculative decoding": Gated
    DeltaNet drafts through the T x T triangular solve, from checkpoint plus
    committed records, equal running the drafts token by token through the
    recurrence (outputs, the corrected values stored as records, flushed
    checkpoints); T = 1, 2, 4, random accepted counts, several flushes."""
    rng = np.random.default_rng(12)
    for T in (1, 2, 4):
        o, st, nf = run_spec(orc, 3, 2, 8, 12, 8, T, 30, lambda s: rng.integers(0, T + 1, 3), seed=40 + T, form=GDN)
        assert o < 1e-12 and st < 1e-12, (T, o, st)
        assert nf >= 3, (T, nf)


def pin_spec_gdn_T1_is_standard_decode(orc):
    """A one-draft Gated DeltaNet verify with every draft accepted is the
    standard step's output-only route (ReplayModel, an independent code
    path), flushes included (ring of L, flush when h + 1 > L)."""
    B, H, dv, dk, L = 2, 3, 8, 12, 4
    spec = oracle.SpecReplayModel(B, H, dv, dk, L, 1, oracle=orc, form=GDN)
    std = oracle.ReplayModel(GDN, B, H, dv, dk, L + 1, oracle=orc)   # L records + the current token
    h = 0
    for s in range(3 * L + 2):
        q, k, v, lam, beta = _spec_tok_gdn(51, s, B, H, 1, dv, dk)
        fl = h + 1 > L
        o_s = spec.verify(q, k, v, lam, np.full(B, fl), beta=beta)[:, :, 0]
        # the standard step flushes the records with the current token; the
        # speculative one folds the committed records and keeps the draft
        if fl:
            std.fold(np.ones(B, bool))
        o_r = std.step(q[:, :, 0], k[:, :, 0], v[:, :, 0], lam[:, :, 0], np.zeros(B, bool), beta[:, :, 0])
        assert _rel(o_s, o_r) < 1e-12, s
        spec.commit(np.ones(B, np.int32))
        h = (0 if fl else h) + 1


def pin_spec_gdn_zero_beta(orc):
    """beta = 0 writes nothing: every corrected value is 0 and draft i's
    output is the decayed committed state read at q_i, D_{1:i} S_h q_i."""
    B, H, dv, dk, L, T = 2, 2, 8, 12, 8, 4
    spec = oracle.SpecReplayModel(B, H, dv, dk, L, T, oracle=orc, form=GDN)
    ref = oracle.SpecTokenByToken(B, H, dv, dk, T, oracle=orc, form=GDN)
    for s in range(2):   # some committed history first (h = 4, room for T = 4)
        q, k, v, lam, beta = _spec_tok_gdn(61, s, B, H, T, dv, dk)
        spec.verify(q, k, v, lam, np.zeros(B, bool), beta=beta)
        ref.verify(q, k, v, lam, beta)
        spec.commit(np.full(B, 2))
        ref.commit(np.full(B, 2))
    q, k, v, lam, beta = _spec_tok_gdn(62, 9, B, H, T, dv, dk)
    o = spec.verify(q, k, v, lam, np.zeros(B, bool), beta=np.zeros_like(beta))
    Sh = ref.state()
    D = np.exp(np.cumsum(lam, axis=2))
    want = D[..., None] * np.einsum("bhvk,bhtk->bhtv", Sh, q)
    assert _rel(o, want) < 1e-12
    held = spec.committed()[0, 0]
    assert np.all(spec.rec_x.reshape(B, H, L, dv)[:, :, held:held + T] == 0)


def pin_spec_long_memory(orc):
    """Same identity with slowly decaying heads (the checkpoint term dominant)."""
    o, st, nf = run_spec(orc, 2, 2, 8, 12, 16, 4, 24, lambda s: np.full(2, 4), seed=9, a_lo=0.001, a_hi=0.01)
    assert nf >= 4 and o < 1e-12 and st < 1e-12, (o, st, nf)


def pin_spec_causal(orc):
    """Draft i's output depends on drafts 1..i only (W is causally masked):
    changing drafts after i leaves o_1..o_i bit-identical."""
    B, H, dv, dk, L, T = 2, 2, 8, 12, 16, 4
    outs = []
    for variant in range(2):
        spec = oracle.SpecReplayModel(B, H, dv, dk, L, T, oracle=orc)
        for s in range(3):
            q, k, v, lam = _spec_tok(21, s, B, H, T, dv, dk)
            if s == 2 and variant:
                k[:, :, 2:] *= -3.0
                v[:, :, 2:] += 1.0
                lam[:, :, 2:] *= 0.5
            o = spec.verify(q, k, v, lam, np.zeros(B, bool))
            spec.commit(np.full(B, 2))
        outs.append(o)
    assert np.array_equal(outs[0][:, :, :2], outs[1][:, :, :2])
    assert not np.allclose(outs[0][:, :, 2:], outs[1][:, :, 2:])


def pin_spec_rejected_drafts_never_read(orc):
    """[blog]: records past the committed pointer are ignored and overwritten.
    Poisoning the rejected drafts' records with NaN after each commit changes
    no later output, checkpoint or committed record."""
    B, H, dv, dk, L, T = 2, 2, 8, 12, 8, 4
    rng = np.random.default_rng(3)
    acc = [rng.integers(0, T + 1, B) for _ in range(14)]
    runs = []
    for poison in (False, True):
        spec = oracle.SpecReplayModel(B, H, dv, dk, L, T, oracle=orc)
        h = np.zeros(B, np.int32)
        outs = []
        for s in range(14):
            q, k, v, lam = _spec_tok(33, s, B, H, T, dv, dk)
            fl = h + T > L
            outs.append(spec.verify(q, k, v, lam, fl))
            spec.commit(acc[s])
            h = np.where(fl, 0, h) + acc[s]
            if poison:
                for b in range(B):
                    sl = slice(b * H, (b + 1) * H)
                    spec.rec_x[sl, h[b]:] = np.nan
                    spec.rec_k[sl, h[b]:] = np.nan
                    spec.rec_lam[sl, h[b]:] = np.nan
        runs.append((np.stack(outs), spec.checkpoint().copy()))
    assert np.array_equal(runs[0][0], runs[1][0]) and np.array_equal(runs[0][1], runs[1][1])


def pin_spec_T1_is_standard_decode(orc):
    """With one draft per step, all accepted, a verify is a plain decode step:
    its outputs equal the standard checkpoint + buffer step's (a textbook
    reduction of the draft sum to the current-token term)."""
    B, H, dv, dk, L = 2, 3, 8, 12, 6
    spec = oracle.SpecReplayModel(B, H, dv, dk, L, 1, oracle=orc)
    rep = oracle.ReplayModel(M2, B, H, dv, dk, L, oracle=orc)
    h = np.zeros(B, np.int32)
    for s in range(20):
        q, k, v, lam = _spec_tok(41, s, B, H, 1, dv, dk)
        o_s = spec.verify(q, k, v, lam, h + 1 > L)[:, :, 0]
        o_r = rep.step(q[:, :, 0], k[:, :, 0], v[:, :, 0], lam[:, :, 0], rep.records_held()[:, 0] == L - 1)
        assert _rel(o_s, o_r) < 1e-12, s
        h = np.where(h + 1 > L, 0, h) + 1
        spec.commit(np.ones(B, np.int32))


def pin_spec_cursor(orc):
    """[blog] "Speculative decoding": flush when h + T > L (h committed
    records before the step), h <- (flush ? 0 : h) + a.  The vLLM fork's
    form, next_is_flush = (new_wp + 2 T > L + T) for a ring of L + T, is the
    same rule.  All accepted (a = T = 4, L = 16): h = 0, 4, 8, 12, 16, then
    every fourth step flushes; every draft rejected (a = 1): a flush every 13
    steps (at h = 13)."""
    L, T = 16, 4
    for hp in range(L + 1):
        for t in range(1, L + 1):
            _, f = orc.spec_cursor_run(L, t, hp, np.zeros(1, np.int32))
            assert bool(f[0]) == (hp + 2 * t > L + t), (hp, t)
    h, f = orc.spec_cursor_run(L, T, 0, np.full(21, T))
    assert list(h[:9]) == [0, 4, 8, 12, 16, 4, 8, 12, 16]
    assert list(np.nonzero(f)[0]) == [4, 8, 12, 16, 20]
    h, f = orc.spec_cursor_run(L, T, 0, np.ones(40, np.int32))
    assert list(np.nonzero(f)[0]) == [13, 26, 39] and h[13] == 13 and h[14] == 1
    forced = np.zeros(6, np.uint8)
    forced[2] = 1
    h, f = orc.spec_cursor_run(L, T, 0, np.full(6, 2), forced)
    assert list(h) == [0, 2, 4, 2, 4, 6] and list(np.nonzero(f)[0]) == [2]


# ------------------------------------------------------ stochastic rounding --
def pin_philox_matches_library(orc):
    """[philox] The oracle's Philox4x64-10 equals numpy's Philox bit
    generator (an independent implementation of the same definition; numpy
    increments its counter before each block)."""
    from oracle import formats
    rng = np.random.default_rng(17)
    for _ in range(20):
        ctr = rng.integers(0, 2**62, 4, dtype=np.uint64)
        key = rng.integers(0, 2**63, 2, dtype=np.uint64)
        ref = np.random.Philox(counter=ctr, key=key).random_raw(4)
        nxt = ctr.copy()
        nxt[0] += np.uint64(1)
        assert np.array_equal(formats.philox4x64(nxt, key), ref)


def pin_sr_rule(orc):
    """Stochastic rounding to fp16 with 16-bit words: the result is one of the
    two fp16 neighbours, up with probability exactly p = (|x| - lo) / ulp (all
    2^16 random words round up exactly p 2^16 times), fp16 values are
    unchanged, the sign is kept, E[SR(x)] = x, and the fp16 subnormal range
    (spacing 2^-24) and the top of the range behave the same way."""
    from oracle import formats
    grid = np.arange(65536, dtype=np.float64)
    for lo, ulp in ((1.0, 2.0**-10), (503 * 2.0**-24, 2.0**-24), (-1000.0, 0.5), (2.0**-20, 2.0**-24),
                    (65472.0, 32.0), (2.0**-14, 2.0**-24)):
        for k8 in range(8):
            p = k8 / 8.0
            x = np.sign(lo) * (abs(lo) + p * ulp)
            got = formats.sr_f16(np.full(65536, x), grid)
            a, b = np.sign(x) * abs(lo), np.sign(x) * (abs(lo) + ulp)
            assert np.all((got == a) | (got == b)), (lo, k8)
            assert int(np.sum(got == b)) == int(p * 65536), (lo, k8, int(np.sum(got == b)))
    # p = m / 2^13 for fp32 values (13 bits below the fp16 mantissa): every
    # m rounds up exactly m 2^3 times out of 2^16
    m = np.arange(0, 8192, 37)
    x = 1.0 + m * 2.0**-23
    ups = [int(np.sum(formats.sr_f16(np.full(65536, xi), grid) > 1.0)) for xi in x]
    assert ups == list(8 * m)
    # the convention both sides implement: round up exactly when r < p 2^16
    half = 1.0 + 2.0**-11
    assert formats.sr_f16(np.array([half, half, half]), np.array([0.0, 2.0**15 - 1, 2.0**15])).tolist() == \
        [1.0 + 2.0**-10, 1.0 + 2.0**-10, 1.0]
    vals = np.float16(np.linspace(-3, 3, 97)).astype(np.float64)
    assert np.array_equal(formats.sr_f16(vals, np.full(97, 2.0**16 - 1)), vals)
    assert np.array_equal(formats.sr_f16(np.array([0.0, -0.0]), np.zeros(2)), np.array([0.0, -0.0]))
    assert np.signbit(formats.sr_f16(np.array([-0.0]), np.zeros(1))[0])
    # at and above 65504, and for non-finite values: nearest even
    top = np.array([65504.0, 65519.0, 65520.0, -70000.0, np.inf, -np.inf])
    assert np.array_equal(formats.sr_f16(top, np.zeros(6)), np.array([65504.0, 65504.0, np.inf, -np.inf, np.inf, -np.inf]))
    assert np.isnan(formats.sr_f16(np.array([np.nan]), np.zeros(1))[0])
    rng = np.random.default_rng(2)
    x = rng.standard_normal(200000).astype(np.float32).astype(np.float64)
    r = rng.integers(0, 2**16, 200000).astype(np.float64)
    err = formats.sr_f16(x, r) - x
    e = np.frexp(np.abs(x))[1] - 1                  # |x| in [2^e, 2^(e+1))
    ulp = np.ldexp(1.0, np.maximum(e, -14) - 10)      # fp16 spacing there
    assert abs(np.mean(err / ulp)) < 0.01           # unbiased
    assert np.all(np.abs(err) <= ulp * 1.0000001)


def pin_sr_words_layout(orc):
    """The word layout: element e of a tile takes 16-bit word e % 16 of the
    Philox4x64-10 block for counter (step, tile, e // 16, 0), least
    significant half-word of output 0 first; checked against numpy's Philox
    (whose counter is incremented before each block) for a few elements."""
    from oracle import formats
    key = np.array([0x243F6A8885A308D3, 0x13198A2E03707344], np.uint64)
    w = formats.sr_words(key, 5, 9, 8192)
    assert w.dtype == np.uint64 and w.max() < 2**16 and len(w) == 8192
    for e in (0, 1, 3, 4, 7, 15, 16, 33, 8191):
        ctr = np.array([4, 9, e // 16, 0], np.uint64)   # numpy adds 1 to word 0 first
        out = np.random.Philox(counter=ctr, key=key).random_raw(4)
        want = (int(out[(e % 16) // 4]) >> (16 * (e % 4))) & 0xFFFF
        assert int(w[e]) == want, e
    # distinct (step, tile) pairs draw distinct words
    assert not np.array_equal(w[:64], formats.sr_words(key, 6, 9, 64))
    assert not np.array_equal(w[:64], formats.sr_words(key, 5, 10, 64))


def pin_sr_once_per_window(orc):
    """[blog] "The precision argument, derived": with independent rounding
    errors of variance s^2 and constant decay alpha, the deviation of a state
    rounded every step settles at variance s^2 / (1 - alpha^2); rounded once
    per window of L steps (a checkpoint), at s^2 / (1 - alpha^(2L)).  Scalar
    toy: 4096 independent chains around 1.5 (one fp16 binade), alpha = 0.9,
    L = 16, stochastic rounding with Philox words; the measured variance ratio
    matches the closed form within 10 %, and both deviations have mean ~ 0."""
    from oracle import formats
    alpha, L, n_chain, n_step = 0.9, 16, 4096, 160
    rng = np.random.default_rng(8)
    key = np.array([7, 11], np.uint64)
    exact = np.full(n_chain, 1.5)
    per_step = exact.copy()
    per_window = exact.copy()
    devs_s, devs_w = [], []
    for t in range(n_step):
        u = 0.15 + 0.01 * rng.standard_normal(n_chain)
        exact = alpha * exact + u
        w = formats.sr_words(key, t, 0, 2 * n_chain).astype(np.float64)
        per_step = formats.sr_f16(alpha * per_step + u, w[:n_chain])
        per_window = alpha * per_window + u
        if t % L == L - 1:
            per_window = formats.sr_f16(per_window, w[n_chain:])
            if t >= 4 * L:
                devs_w.append(per_window - exact)
        if t >= 4 * L:
            devs_s.append(per_step - exact)
    var_s, var_w = np.var(np.concatenate(devs_s)), np.var(np.concatenate(devs_w))
    want = (1 - alpha ** (2 * L)) / (1 - alpha ** 2)
    assert abs(var_s / var_w / want - 1) < 0.10, (var_s / var_w, want)
    ulp = 2.0 ** -10
    assert abs(np.mean(np.concatenate(devs_s))) < 0.02 * ulp * np.sqrt(1 / (1 - alpha**2)) * 10


ALL_PINS = [
    pin_identity_mamba2_tiny,
    pin_identity_mamba2_long_memory,
    pin_identity_gdn_tiny,
    pin_identity_long_window,
    pin_single_step_from_zero,
    pin_no_decay_is_plain_sum,
    pin_constant_decay_geometric,
    pin_full_forgetting,
    pin_gdn_product_form,
    pin_gdn_unit_key_stores_value,
    pin_gdn_zero_beta_only_decays,
    pin_fold_materialises_state,
    pin_cursor_closed_form,
    pin_cursor_forced_flush,
    pin_two_copy_read_error_is_one_rounding,
    pin_two_copy_error_does_not_accumulate,
    pin_two_copy_f16_recurrence,
    pin_e4m3_matches_library_cast,
    pin_e4m3_spec_values,
    pin_read_rounding_within_half_ulp,
    pin_spec_identity,
    pin_spec_two_copy,
    pin_spec_gdn_identity,
    pin_spec_gdn_T1_is_standard_decode,
    pin_spec_gdn_zero_beta,
    pin_spec_long_memory,
    pin_spec_causal,
    pin_spec_rejected_drafts_never_read,
    pin_spec_T1_is_standard_decode,
    pin_spec_cursor,
    pin_philox_matches_library,
    pin_sr_rule,
    pin_sr_words_layout,
    pin_sr_once_per_window,
]
