"""Traffic model of conventional vs checkpoint + buffer decoding.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring).

All formulas follow the blog "ReplaySSM: an SSM decoder that writes its state
once every 16 tokens", section "The identity" (state and record terms of one
window), "Output without a state" (shrink of the state-building term) and
"Why 16" (the window-length optimum); the two-copy window follows section
"The precision argument, derived" (non-flush steps read only the read copy;
a flush reads the recurrence copy and writes both).  Units are bytes per head unless a
function says otherwise.
"""
from __future__ import annotations

import math


def state_bytes(d_v: int, d_k: int, elem_bytes: int) -> int:
    """Bytes of one head's d_v x d_k state."""
    return d_v * d_k * elem_bytes


def layer_state_bytes(n_heads: int, d_v: int, d_k: int, elem_bytes: int) -> int:
    """Bytes of one layer's state for one sequence (all heads)."""
    return n_heads * state_bytes(d_v, d_k, elem_bytes)


def record_bytes(d_v: int, d_k: int) -> int:
    """One buffered record per head as the pages price it: a 16-bit value
    vector, a 16-bit key and a 4-byte decay, 2 d_v + 2 d_k + 4 bytes."""
    return 2 * d_v + 2 * d_k + 4


def conventional_window_bytes(L: int, m_state: int) -> int:
    """Conventional decoding reads and writes the state on each of L steps."""
    return 2 * L * m_state


def replay_window_bytes(L: int, m_state: int, rec: int) -> int:
    """Checkpoint + buffer over one window of L steps: the state is read on
    every step and written once (L + 1 state transfers); step i reads the
    i - 1 records before it (L (L - 1) / 2 in total) and L - 1 records are
    written."""
    return (L + 1) * m_state + rec * (L * (L - 1) // 2 + (L - 1))


def two_copy_window_bytes(L: int, m_hi: int, m_lo: int, rec: int) -> int:
    """Checkpoint + buffer with a recurrence copy (m_hi bytes) and a read copy
    (m_lo bytes): the L - 1 non-flush steps read the read copy, the flush
    reads the recurrence copy and writes both; records as in
    replay_window_bytes."""
    return (L - 1) * m_lo + m_hi + (m_hi + m_lo) + rec * (L * (L - 1) // 2 + (L - 1))


def state_term_ratio(L: int) -> float:
    """Replay over conventional for the state term alone: (L + 1) / 2L."""
    return (L + 1) / (2 * L)


def traffic_ratio(L: int, d_v: int, d_k: int, state_elem_bytes: int, rec: int | None = None) -> float:
    m = state_bytes(d_v, d_k, state_elem_bytes)
    r = record_bytes(d_v, d_k) if rec is None else rec
    return replay_window_bytes(L, m, r) / conventional_window_bytes(L, m)


def optimal_window(m_state_over_rec: float, tokens_per_step: float = 1.0, mean_accepted: float = 1.0) -> float:
    """L* = sqrt(2 a (M_S / r - T)) ("Why 16")."""
    return math.sqrt(2.0 * mean_accepted * (m_state_over_rec - tokens_per_step))


def output_only_shrink(d_v: int, d_k: int) -> float:
    """Factor by which the output-only bracketing shrinks the state-building
    term: building v k^T costs d_v d_k per record, v (k . q) costs d_v + d_k."""
    return d_v * d_k / (d_v + d_k)


def grouped_record_bytes(n_heads: int, d_v: int, d_k: int, n_groups: int) -> int:
    """One layer-record in the released grouped-key layout: per value head a
    d_v-wide 16-bit value row plus a 4-byte step size, per key group one
    d_k-wide 16-bit key ("The identity", paragraph on the released kernel)."""
    return n_heads * (2 * d_v + 4) + n_groups * 2 * d_k


# ------------------------------------------------------ speculative verify --
def snapshot_verify_step_bytes(T: int, m_state: int) -> int:
    """The snapshot scheme the blog compares against ("Speculative decoding:
    rollback becomes a pointer"): one state read and one state snapshot
    written per draft, T + 1 state transfers per verify step."""
    return (T + 1) * m_state


def plain_decode_token_bytes(m_state: int) -> int:
    """Plain (conventional) decoding: the state read and written per token."""
    return 2 * m_state


def spec_replay_state_bytes_per_token(L: int, T: int, accepted: int, m_state: int,
                                      n_steps: int = 100000) -> float:
    """State bytes per committed token of checkpoint + ring verification with
    T drafts per step, every step accepting `accepted` of them, in steady
    state: every step reads the checkpoint once; a step whose h committed
    records leave no room for T more (h + T > L) also writes it.  Counted
    step by step over n_steps after a warm-up of 4 L steps."""
    h, reads, writes, tokens = 0, 0, 0, 0
    for s in range(4 * L + n_steps):
        flush = h + T > L
        if s >= 4 * L:
            reads += 1
            writes += int(flush)
            tokens += accepted
        h = (0 if flush else h) + accepted
    return (reads + writes) * m_state / tokens


def spec_replay_bytes_per_token(L: int, T: int, accepted: int, m_state: int, rec_layer: int,
                                n_steps: int = 100000) -> float:
    """spec_replay_state_bytes_per_token plus the record writes: every verify
    step stores its T draft records (rec_layer bytes each for the whole
    layer), accepted or not ("appends all T draft records behind the h
    committed ones")."""
    per_token = spec_replay_state_bytes_per_token(L, T, accepted, m_state, n_steps)
    return per_token + T * rec_layer / accepted
