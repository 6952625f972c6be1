"""The offline chooser fit (RaMP section 3.1): features equal the oracle's cost-model
inputs, the NNLS fit equals a brute-force solve over active sets on small
problems, and the greedy menu picks what exhaustive enumeration picks."""
import itertools

import numpy as np
import pytest

import oracle
from routing_aware_grouped_amd import tune
from tests import spec


def test_features_match_oracle_select():
    rng = np.random.default_rng(3)
    for trial in range(30):
        El = int(rng.choice([8, 32, 128]))
        H, I = (2048, 768) if trial % 2 else (4096, 14336)
        cc = spec.cost_constants(H, I, 256)
        cnt = (rng.integers(0, 300, El) * (rng.random(El) < 0.6)).astype(np.int32)
        F = tune.features(cnt, cc)
        th = np.zeros((len(spec.MENU), 4), np.float32)
        _, _, feat = oracle.select(cnt, cc["b"], cc["q1"], cc["q2"], cc["S1"], cc["S2"], th)
        np.testing.assert_array_equal(F[:, 1:].astype(np.int64), feat.astype(np.int64))
        assert np.all(F[:, 0] == 1.0)


def _nnls_brute(Fs, y):
    """Minimise ||Fs th - y|| over th >= 0 by solving every active set."""
    n = Fs.shape[1]
    best, best_th = np.inf, np.zeros(n)
    for r in range(n + 1):
        for S in itertools.combinations(range(n), r):
            th = np.zeros(n)
            if S:
                sol, *_ = np.linalg.lstsq(Fs[:, S], y, rcond=None)
                if np.any(sol < -1e-12):
                    continue
                th[list(S)] = np.maximum(sol, 0)
            res = float(np.sum((Fs @ th - y) ** 2))
            if res < best - 1e-12:
                best, best_th = res, th
    return best_th, best


@pytest.mark.parametrize("seed", range(6))
def test_fit_is_relative_error_nnls(seed):
    rng = np.random.default_rng(seed)
    n = 14
    F = np.column_stack([np.ones(n), rng.integers(1, 9, n), rng.integers(10, 500, n),
                         rng.integers(1, 64, n)]).astype(np.float64)
    true = np.array([5.0, 2.0, 0.05, 0.3]) * (rng.random(4) > 0.3)
    t = (F @ true + 1.0) * np.exp(rng.normal(0, 0.1, n))
    th = tune.fit_nnls(F, t)
    assert np.all(th >= 0)
    bt, best = _nnls_brute(F / t[:, None], np.ones(n))
    got = float(np.sum((F @ th / t - 1.0) ** 2))
    assert got <= best * (1 + 1e-6) + 1e-12


def test_greedy_menu_matches_enumeration_for_one_and_two():
    rng = np.random.default_rng(9)
    t = rng.random((25, 5)) + 0.1
    first = tune.greedy_menu(t, 1)[0]
    assert first == int(np.argmin(t.sum(axis=0)))
    two = tune.greedy_menu(t, 2)
    assert two[0] == first and len(set(two)) == 2
    second = min((np.minimum(t[:, first], t[:, v]).sum(), v) for v in range(5) if v != first)[1]
    assert two[1] == second


def test_served_greedy_matches_enumeration_for_one_and_two():
    """greedy_menu_served: the first pick is the configuration with the lowest
    geomean time when it alone is served; the second is the best pair holding the
    first, scored by what the argmin of pred serves inside the pair."""
    rng = np.random.default_rng(12)
    t = rng.random((40, 6)) + 0.1
    pred = t * (1 + 0.3 * rng.standard_normal(t.shape))
    first = tune.greedy_menu_served(pred, t, 1)[0]
    assert first == int(np.argmin(np.log(t).mean(axis=0)))
    two = tune.greedy_menu_served(pred, t, 2)
    assert two[0] == first

    def served(m):
        m = sorted(m)
        pick = np.asarray(m)[np.argmin(pred[:, m], axis=1)]
        return np.log(t[np.arange(len(t)), pick]).mean()
    assert two[1] == min((served([first, v]), v) for v in range(6) if v != first)[1]


def test_served_greedy_skips_a_configuration_the_model_cannot_serve():
    """A configuration predicted exactly like one already in the menu (same cost
    constants and fit) loses every tie to the lower index, so adding it serves
    nothing: the served greedy takes the next useful one, while the best-entry
    greedy would take it for its (unreachable) fast loads."""
    n = 30
    half = np.arange(n) < n // 2
    t = np.empty((n, 4))
    t[:, 0] = 0.5                          # best alone
    t[:, 3] = np.where(half, 0.2, 2.0)     # fast on half the loads ...
    t[:, 1] = np.where(half, 0.4, 1.5)
    t[:, 2] = 1.5
    pred = np.empty((n, 4))
    pred[:, 0] = 0.5
    pred[:, 3] = pred[:, 0]                # ... but indistinguishable from 0
    pred[:, 1] = np.where(half, 0.3, 1.5)
    pred[:, 2] = 1.5
    assert tune.greedy_menu(t, 2, relative=True) == [0, 3]
    assert tune.greedy_menu_served(pred, t, 2) == [0, 1]


def test_served_menu_excludes_the_rest():
    """fit() with a menu: the menu is greedy_menu_served's choice, the other
    configurations get the off-menu prediction, and the oracle's argmin over the
    resulting theta never picks one of them."""
    import oracle
    rng = np.random.default_rng(4)
    V, El = len(spec.MENU), 16
    cc = spec.cost_constants(2048, 768, 256)
    loads = []
    for i in range(30):
        cnt = (rng.integers(0, 300, El) * (rng.random(El) < 0.7)).astype(int)
        loads.append(dict(counts=cnt.tolist(), times_us=(rng.random(V) * 100 + 50).tolist()))
    res = tune.fit(dict(variants=V, cost_constants=cc, loads=loads), menu_size=4)
    assert len(res["menu"]) == 4 and res["menu"] == sorted(set(res["menu"]))
    th = np.asarray(res["theta"], np.float32)
    off = [v for v in range(V) if v not in res["menu"]]
    assert np.all(th[off, 0] == np.float32(tune.OFF_MENU_THETA0)) and np.all(th[off, 1:] == 0)
    assert res["menu_geomean_loss"] >= 0
    for ld in loads:
        v, _, _ = oracle.select(np.asarray(ld["counts"], np.int32), cc["b"], cc["q1"], cc["q2"],
                                cc["S1"], cc["S2"], th)
        assert v in res["menu"]
