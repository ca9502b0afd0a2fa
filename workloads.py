"""Seeded synthetic inputs for the decode-step workloads.

Shared by the tests, the smoke check and the benchmark, and by both the GPU
path and the CPU oracle.  This module draws random numbers and casts them to
the input dtypes; it contains none of the decode arithmetic.

Every generator is a pure function of (seed, step, shape): each draw uses a
torch CPU generator seeded from numpy's SeedSequence([seed, stream, step]),
so a step's inputs do not depend on how many earlier steps were generated
(a test can regenerate step s alone) nor on the thread count.

Input recipes (the workloads the pages measure on):
  * Mamba-2 form: v, k, q ~ N(0, 1); log-decay lam = -softplus(x) * a with
    x ~ N(0, 1) per (step, row, head) and a ~ U[a_lo, a_hi] drawn once per
    head.  alpha = exp(lam) lies in (0, 1).
  * Gated DeltaNet form: k, q = unit-norm(N(0, 1)) (normalised in float64
    before the cast), v ~ N(0, 1), beta = sigmoid(N(0, 1)),
    g = lam = -softplus(N(0, 1)).
Token tensors are returned as CPU torch tensors in the requested io dtype;
lam and beta are float32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

_TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# independent random streams
_S_TOKENS, _S_HEADS, _S_INIT, _S_SCHED, _S_POOL, _S_DYADIC = 1, 2, 3, 4, 5, 6


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DT[name]


def _softplus(x):
    if isinstance(x, torch.Tensor):
        return torch.logaddexp(torch.zeros_like(x), x)
    return np.logaddexp(0.0, x)


def _gen(*key: int) -> torch.Generator:
    seed = int(np.random.SeedSequence(list(key)).generate_state(1, dtype=np.uint64)[0] >> 1)
    return torch.Generator().manual_seed(seed)


def head_decay_scale(seed: int, H: int, a_lo: float = 1.0, a_hi: float = 8.0) -> np.ndarray:
    """Per-head decay scale a ~ U[a_lo, a_hi] (fixed for the whole run)."""
    rng = np.random.default_rng([seed, _S_HEADS])
    return rng.uniform(a_lo, a_hi, size=H)


@dataclass
class Tokens:
    q: torch.Tensor      # [B, H, dk] io dtype
    k: torch.Tensor      # [B, H, dk] io dtype
    v: torch.Tensor      # [B, H, dv] io dtype
    lam: torch.Tensor    # [B, H] float32 log-decay
    beta: torch.Tensor | None  # [B, H] float32 (GDN) or None


def mamba2_tokens(seed: int, step: int, B: int, H: int, dv: int, dk: int, io: str = "f32",
                  a_lo: float = 1.0, a_hi: float = 8.0) -> Tokens:
    g = _gen(seed, _S_TOKENS, step)
    dt = _TORCH_DT[io]
    q = torch.randn((B, H, dk), generator=g).to(dt)
    k = torch.randn((B, H, dk), generator=g).to(dt)
    v = torch.randn((B, H, dv), generator=g).to(dt)
    x = torch.randn((B, H), generator=g, dtype=torch.float64)
    a = torch.from_numpy(head_decay_scale(seed, H, a_lo, a_hi))
    lam = (-_softplus(x) * a[None, :]).float()
    return Tokens(q, k, v, lam, None)


def gdn_tokens(seed: int, step: int, B: int, H: int, dv: int, dk: int, io: str = "bf16") -> Tokens:
    g = _gen(seed, _S_TOKENS, step)
    dt = _TORCH_DT[io]
    q = torch.randn((B, H, dk), generator=g, dtype=torch.float64)
    k = torch.randn((B, H, dk), generator=g, dtype=torch.float64)
    q = (q / q.norm(dim=-1, keepdim=True)).to(dt)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dt)
    v = torch.randn((B, H, dv), generator=g).to(dt)
    beta = torch.sigmoid(torch.randn((B, H), generator=g, dtype=torch.float64)).float()
    lam = (-_softplus(torch.randn((B, H), generator=g, dtype=torch.float64))).float()
    return Tokens(q, k, v, lam, beta)


def dyadic_tokens(seed: int, step: int, B: int, H: int, dv: int, dk: int, io: str = "bf16",
                  bits: int = 6) -> Tokens:
    """Mamba-2 tokens on which fp32 and fp64 arithmetic agree exactly: q, k,
    v uniform on the integer multiples of 2^-bits in [-1, 1] (exact in bf16
    and fp16 for bits <= 7), log-decay 0 (alpha = 1), so every product is a
    multiple of 2^-2bits and short sums of them are exact in fp32."""
    g = _gen(seed, _S_DYADIC, step)
    dt = _TORCH_DT[io]
    m = 1 << bits
    draw = lambda d: (torch.randint(-m, m + 1, (B, H, d), generator=g).double() / m).to(dt)
    q, k, v = draw(dk), draw(dk), draw(dv)
    return Tokens(q, k, v, torch.zeros((B, H)), None)


def tokens(form: int, seed: int, step: int, B: int, H: int, dv: int, dk: int, io: str,
           a_lo: float = 1.0, a_hi: float = 8.0) -> Tokens:
    """form 0 = Mamba-2, 1 = Gated DeltaNet."""
    if form == 0:
        return mamba2_tokens(seed, step, B, H, dv, dk, io, a_lo, a_hi)
    return gdn_tokens(seed, step, B, H, dv, dk, io)


def random_row_start(seed: int, row: int, H: int, dv: int, dk: int, w0: int, cap: int,
                     form: int = 0, state_dt: str = "f32", rec_dt: str = "f16"):
    """A row that joins mid-window: checkpoint C0 ~ N(0, 1/dk) and w0 records.

    Returns float64 numpy arrays whose values are exactly representable in the
    state / record dtypes: C0 [H, dv, dk], rec_lam [H, cap] (float32 values),
    rec_x [H, cap, dv], rec_k [H, cap, dk].  Slots >= w0 are zero.
    """
    rng = np.random.default_rng([seed, _S_INIT, row])
    sdt, rdt = _TORCH_DT[state_dt], _TORCH_DT[rec_dt]
    C0 = torch.from_numpy(rng.standard_normal((H, dv, dk)) / np.sqrt(dk)).to(sdt).double().numpy()
    rec_lam = np.zeros((H, cap))
    rec_x = np.zeros((H, cap, dv))
    rec_k = np.zeros((H, cap, dk))
    if w0:
        if form == 0:
            a = head_decay_scale(seed, H)
            lam = -_softplus(rng.standard_normal((H, w0))) * a[:, None]
        else:
            lam = -_softplus(rng.standard_normal((H, w0)))
        rec_lam[:, :w0] = lam.astype(np.float32)
        rec_x[:, :w0] = torch.from_numpy(rng.standard_normal((H, w0, dv))).to(rdt).double().numpy()
        kk = rng.standard_normal((H, w0, dk))
        if form == 1:
            kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
        rec_k[:, :w0] = torch.from_numpy(kk).to(rdt).double().numpy()
    return C0, rec_lam, rec_x, rec_k


@dataclass
class Event:
    step: int
    retire: list      # slots that retire before this step
    join: list        # (slot, block) pairs that join before this step


def continuous_schedule(seed: int, n_slots: int, n_steps: int, n_blocks: int,
                        p_retire: float = 1.0 / 32, p_join: float = 0.5):
    """Retire/join events for a continuous-batching run.

    Initial state: every slot live on a distinct block drawn from a shuffled
    pool of n_blocks.  Before each step, each live slot retires with
    probability p_retire (its block returns to the free list) and each empty
    slot receives a new row with probability p_join, on a block drawn at
    random from the free list.  Empty slots are padding for that step.
    Returns (initial_blocks [n_slots] int32, initial w0 draws [n_slots] in
    U{0..15}, events list).
    """
    rng = np.random.default_rng([seed, _S_SCHED])
    perm = rng.permutation(n_blocks)
    blocks = perm[:n_slots].astype(np.int32).copy()
    free = list(perm[n_slots:])
    w0 = rng.integers(0, 16, size=n_slots).astype(np.int32)
    live = np.ones(n_slots, bool)
    events = []
    for s in range(n_steps):
        retire, join = [], []
        for slot in range(n_slots):
            if live[slot]:
                if rng.random() < p_retire:
                    live[slot] = False
                    free.append(int(blocks[slot]))
                    blocks[slot] = -1
                    retire.append(slot)
            else:
                if free and rng.random() < p_join:
                    i = int(rng.integers(0, len(free)))
                    b = free.pop(i)
                    blocks[slot] = b
                    live[slot] = True
                    join.append((slot, b))
        events.append(Event(s, retire, join))
    return perm[:n_slots].astype(np.int32), w0, events


def shuffled_blocks(seed: int, n_rows: int, n_blocks: int) -> np.ndarray:
    """A block table mapping each row to a distinct block, in shuffled order."""
    rng = np.random.default_rng([seed, _S_POOL])
    return rng.permutation(n_blocks)[:n_rows].astype(np.int32)


@dataclass
class SpecTokens:
    q: torch.Tensor      # [B, T, H, dk] io dtype
    k: torch.Tensor      # [B, T, H, dk] io dtype
    v: torch.Tensor      # [B, T, H, dv] io dtype
    lam: torch.Tensor    # [B, T, H] float32
    beta: torch.Tensor | None = None  # [B, T, H] float32 (Gated DeltaNet) or None


def spec_tokens(seed: int, step: int, B: int, H: int, T: int, dv: int, dk: int, io: str = "bf16",
                a_lo: float = 1.0, a_hi: float = 8.0, form: int = 0) -> SpecTokens:
    """T draft tokens per row for speculative step `step`; draft i of step s
    is the token of step T s + i of the form's recipe (Mamba-2: the same
    per-head decay scales apply; Gated DeltaNet: unit-norm q, k and beta)."""
    if form == 0:
        toks = [mamba2_tokens(seed, T * step + i, B, H, dv, dk, io, a_lo, a_hi) for i in range(T)]
    else:
        toks = [gdn_tokens(seed, T * step + i, B, H, dv, dk, io) for i in range(T)]
    st = lambda name: torch.stack([getattr(t, name) for t in toks], dim=1).contiguous()
    return SpecTokens(st("q"), st("k"), st("v"), st("lam"), st("beta") if form else None)


def spec_accepted(seed: int, step: int, B: int, T: int, policy: str = "random") -> np.ndarray:
    """Accepted draft counts per row for one verify step: "random" (uniform
    0..T), "all" (T), "one" (1) or "none" (0)."""
    if policy == "all":
        return np.full(B, T, np.int32)
    if policy == "one":
        return np.ones(B, np.int32)
    if policy == "none":
        return np.zeros(B, np.int32)
    rng = np.random.default_rng([seed, _S_SCHED, 7919, step])
    return rng.integers(0, T + 1, size=B).astype(np.int32)
