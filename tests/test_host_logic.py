"""Host-side logic of the decode loop that needs no GPU."""
import numpy as np

import linear_attention_decode_replay_amd as rs
from linear_attention_decode_replay_amd.state import DecodeLayer


class _Rows:
    """The two attributes DecodeLayer._hint reads."""

    def __init__(self, blocks, hints=True):
        self.blocks = np.asarray(blocks)
        self.flush_hints = hints

    def live(self):
        return self.blocks >= 0


def test_flush_hint_from_host_flags():
    hint = DecodeLayer._hint
    rows = _Rows([3, -1, 5, 7])            # slot 1 is padding
    assert hint(rows, np.array([0, 0, 0, 0], np.uint8)) == rs.RS_FLUSH_NONE
    assert hint(rows, np.array([1, 0, 1, 1], np.uint8)) == rs.RS_FLUSH_ALL
    assert hint(rows, np.array([1, 1, 1, 1], np.uint8)) == rs.RS_FLUSH_ALL  # padding is ignored
    assert hint(rows, np.array([0, 1, 1, 0], np.uint8)) == rs.RS_FLUSH_MIXED
    assert hint(_Rows([-1, -1]), np.array([1, 1], np.uint8)) == rs.RS_FLUSH_UNKNOWN   # nothing live
    assert hint(_Rows([3, 4], hints=False), np.array([0, 0], np.uint8)) == rs.RS_FLUSH_UNKNOWN


def test_flush_hint_matches_the_cursor_rule():
    """Over a run of steps the hint agrees with rs_meta_step's flags: with
    rows in different phases most steps are mixed, in phase none or all."""
    L = 4
    for anchors, expect in (([0, 0, 0], {rs.RS_FLUSH_NONE, rs.RS_FLUSH_ALL}),
                            ([0, 1, 2], {rs.RS_FLUSH_MIXED, rs.RS_FLUSH_NONE})):
        a = np.array(anchors, np.int32)
        seen = set()
        for _ in range(3 * L):
            wp, fl = rs.rs_meta_step(L, a)
            h = DecodeLayer._hint(_Rows([0, 1, 2]), fl)
            n = int(fl.sum())
            assert h == (rs.RS_FLUSH_NONE if n == 0 else rs.RS_FLUSH_ALL if n == 3 else rs.RS_FLUSH_MIXED)
            seen.add(h)
            rs.rs_meta_advance(L, a, fl)
        assert seen == expect
