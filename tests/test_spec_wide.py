"""CPU checks of the wide configuration's specification helpers (tests/spec.py):
the expert-major tile order is a bijection onto (row-block, column tile) that
keeps each tile inside its expert's run, and the tail-split rule gives pieces
only after a full round and for a tail of at most half the grid."""
import numpy as np

from tests import spec


def test_expert_major_order_is_a_bijection():
    rng = np.random.default_rng(3)
    for _ in range(20):
        counts = rng.integers(0, 5, 6)
        be = [e for e, c in enumerate(counts) for _ in range(c)]
        if not be:
            continue
        ncol = int(rng.integers(1, 7))
        seen = set()
        for t in range(len(be) * ncol):
            rb, nt = spec.expert_major_tile(t, be, ncol)
            assert 0 <= nt < ncol and be[rb] == be[t // ncol]
            seen.add((rb, nt))
        assert len(seen) == len(be) * ncol


def test_wide_pieces_rule():
    assert spec.wide_pieces(200, 256, 448) == 0      # no full round
    assert spec.wide_pieces(256, 256, 448) == 0      # no tail
    assert spec.wide_pieces(256 + 129, 256, 448) == 0  # tail above half the grid
    assert spec.wide_pieces(256 + 128, 256, 448) == 2
    assert spec.wide_pieces(256 + 64, 256, 448) == 4
    assert spec.wide_pieces(256 + 1, 256, 448) == 56   # capped at nst / 8
    assert spec.wide_pieces(256 + 8, 256, 24) == 3
    assert spec.wide_pieces(256 + 8, 256, 12) == 0     # 12 stages: at most one piece of two groups
