"""Host-side alternative choosers: each policy's rule on hand-built loads whose right
answer is fixed by the rule itself."""
import math

import numpy as np
import pytest

from routing_aware_grouped_amd import choosers as C


def _ld(tokens, counts, times, alpha=1.0, rep=0):
    return dict(tokens=tokens, counts=list(counts), times_us=list(times), alpha=alpha, rep=rep)


def test_exemplar_sorts_and_normalises():
    e = C.exemplar([0, 3, 4])
    assert np.allclose(e, [0.8, 0.6, 0.0])
    assert np.allclose(C.exemplar([0, 0, 0]), [0, 0, 0])


def test_padding_and_load_over_mean():
    # rows round up to 16: 5 -> 16, 16 -> 16, 0 -> 0, 17 -> 32; 38 of 64 rows are real
    assert C.padding([5, 16, 0, 17], 16) == pytest.approx(1 - 38 / 64)
    assert C.padding([0, 0], 128) == 0.0
    assert C.load_over_mean([1, 1, 1, 5]) == pytest.approx(2.5)
    assert C.load_over_mean([0, 0]) == 0.0


def test_bucket_is_nearest_on_log_scale():
    b = [8, 64, 512]
    assert C._bucket(1, b) == 8
    assert C._bucket(22, b) == 8      # log2 22 = 4.46: 1.46 from 8, 1.54 from 64
    assert C._bucket(23, b) == 64
    assert C._bucket(4096, b) == 512


def test_token_table_takes_geometric_mean_best():
    # configuration 0 wins one load by 2x and loses the other by 1.5x: geomean favours 0
    loads = [_ld(16, [1, 1], [1.0, 2.0]), _ld(16, [2, 0], [3.0, 2.0])]
    t = C.TokenTable().fit(loads)
    assert t.choose(16, [5, 5]) == 0
    # the arithmetic mean would pick 1 here; the geometric mean picks 0
    loads = [_ld(16, [1, 1], [1.0, 4.0]), _ld(16, [2, 0], [10.0, 5.0])]
    assert C.TokenTable().fit(loads).choose(16, [1, 1]) == 0


def test_noda_uses_the_most_uniform_input_only():
    loads = [_ld(32, [8, 8], [1.0, 2.0], alpha=30.0, rep=100),
             _ld(32, [16, 0], [5.0, 1.0], alpha=0.03, rep=100),
             _ld(32, [16, 0], [5.0, 1.0], alpha=0.5, rep=100)]
    p = C.NoDA().fit(loads)
    assert p.choose(32, [16, 0]) == 0
    assert p.choose(40, [0, 20]) == 0


def test_exemplar_matcher_ignores_expert_identity_and_scale():
    loads = [_ld(64, [60, 2, 1, 1], [3.0, 1.0, 2.0]),    # skewed -> config 1
             _ld(64, [16, 16, 16, 16], [1.0, 3.0, 2.0])]  # uniform -> config 0
    p = C.ExemplarMatcher().fit(loads)
    assert p.choose(64, [1, 2, 60, 1]) == 1              # same skew, other hot expert
    assert p.choose(80, [20, 20, 20, 20]) == 0           # nearest bucket, other scale
    assert p.choose(64, [40, 20, 3, 1]) == 1


def test_padding_table_splits_a_token_bucket_by_padding():
    bm = 16
    loads = []
    for i in range(4):  # low padding: 16-row multiples; config 0 fastest
        loads.append(_ld(64, [16, 16, 16, 16], [1.0, 2.0 + i]))
    for i in range(4):  # high padding: one row per expert; config 1 fastest
        loads.append(_ld(64, [61, 1, 1, 1], [2.0 + i, 1.0]))
    p = C.PaddingTable(bm, nbins=2).fit(loads)
    assert p.choose(64, [16, 32, 16, 0]) == 0
    assert p.choose(64, [1, 1, 1, 61]) == 1


def test_nearest_neighbours_with_one_neighbour_returns_its_best():
    loads = [_ld(8, [8, 0, 0, 0], [1.0, 2.0]), _ld(4096, [2048] * 4, [2.0, 1.0])]
    p = C.NearestNeighbors(128, k=1).fit(loads)
    assert p.choose(8, [7, 1, 0, 0]) == 0
    assert p.choose(2048, [1024] * 4) == 1


@pytest.mark.parametrize("counts,want", [
    ([0, 0, 0, 0], 16),         # m = 0
    ([4, 4, 4, 4], 16),         # 4 + 2 = 6
    ([12, 12, 12, 12], 16),     # 12 + 3.46 = 15.5
    ([16, 16, 16, 16], 32),     # 16 + 4 = 20
    ([49, 49, 49, 49], 64),     # 49 + 7 = 56
    ([100, 100, 100, 100], 128),
    ([500, 0, 0, 0], 128),      # m = 125: 136 exceeds every candidate, take the largest
])
def test_block_m_heuristic(counts, want):
    menu = [16, 32, 64, 128]
    p = C.BlockSizeHeuristic(menu).fit([])
    assert menu[p.choose(sum(counts), counts)] == want


def test_score_reports_gap_to_the_best_configuration():
    class Fixed:
        def choose(self, tokens, counts):
            return 0
    pts = [dict(tokens=1, counts=[1], us_per_variant=[2.0, 1.0]),
           dict(tokens=1, counts=[1], us_per_variant=[1.0, 3.0])]
    s = C.score(Fixed(), pts)
    assert s["worst_gap"] == pytest.approx(1.0)
    assert s["geomean_gap"] == pytest.approx(math.sqrt(2.0) - 1.0, abs=1e-4)
    assert s["within_5pct"] == 0.5


def test_every_policy_fits_and_scores_on_stored_fit_loads():
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    path = os.path.join(root, "routing_aware_grouped_amd", "theta", "mixtral.json")
    loads = json.load(open(path))["loads"]
    pts = [dict(tokens=ld["tokens"], counts=ld["counts"], us_per_variant=ld["times_us"])
           for ld in loads]
    res = C.compare(loads, pts, [16, 32, 64, 128])
    assert len(res) == 6
    for g in res.values():
        assert 0.0 <= g["geomean_gap"] <= g["worst_gap"]
        assert 0.0 <= g["within_5pct"] <= 1.0
