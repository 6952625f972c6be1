"""Pins of the oracle's shared-expert lanes (GC-MoE section 4: shared experts see
every token, need no dispatch, and their output is one more lane of the combine,
added with weight 1 after the k routed lanes).  The pins use a dense numpy FFN,
not the oracle's own expert loop."""
import dataclasses

import numpy as np

import synth


def _dense_ffn(x, w1, w3, w2):
    g = x @ w1.T
    u = x @ w3.T
    return ((g / (1.0 + np.exp(-g))) * u) @ w2.T


def _layer(T, E, k, H, I, n_shared, seed):
    rng = np.random.default_rng(seed)
    shape = synth.Shape("t", H, I, E, E, k, synth.F32, synth.F32, synth.F32, "normal", 0, n_shared)
    x = (rng.standard_normal((T, H)) * 0.5).astype(np.float32)
    w = {n: (rng.standard_normal((E + n_shared,) + s) * 0.3).astype(np.float32)
         for n, s in (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I)))}
    lg = rng.standard_normal((T, E)).astype(np.float32)
    return synth.Layer(shape, T, None, 0, lg, x, w["w1"], w["w3"], w["w2"])


def test_shared_lanes_add_dense_ffns(oracle_lib):
    """Y = routed layer (the same layer without shared experts) + the dense FFN of
    every shared expert."""
    L = _layer(7, 6, 2, 16, 24, 2, 1)
    out = oracle_lib.full_layer(L, b=4)
    routed = dataclasses.replace(L, shape=dataclasses.replace(L.shape, shared=0))
    base = oracle_lib.full_layer(routed, b=4)["Y"]
    x = L.x.astype(np.float64)
    dense = sum(_dense_ffn(x, L.w1[6 + i].astype(np.float64), L.w3[6 + i].astype(np.float64),
                           L.w2[6 + i].astype(np.float64)) for i in range(2))
    np.testing.assert_allclose(out["Y"], base + dense, rtol=1e-12, atol=1e-13)
    assert np.abs(dense).max() > 0.1 * np.abs(base).max()


def test_shared_only_when_routed_outputs_vanish(oracle_lib):
    """Routed experts with zero down projections leave exactly the shared lanes."""
    L = _layer(5, 4, 2, 8, 16, 1, 2)
    L.w2[:4] = 0.0
    out = oracle_lib.full_layer(L, b=2)
    x = L.x.astype(np.float64)
    ref = _dense_ffn(x, L.w1[4].astype(np.float64), L.w3[4].astype(np.float64),
                     L.w2[4].astype(np.float64))
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-14)


def test_zero_shared_expert_changes_nothing(oracle_lib):
    L = _layer(6, 5, 3, 8, 8, 1, 3)
    L.w2[5] = 0.0
    out = oracle_lib.full_layer(L, b=2)
    routed = dataclasses.replace(L, shape=dataclasses.replace(L.shape, shared=0))
    np.testing.assert_array_equal(out["Y"], oracle_lib.full_layer(routed, b=2)["Y"])
