"""Pins of the CPU oracle against facts fixed by the pages and by mathematics
(brute force, library routines, closed forms, the pages' worked example).
None of these tests uses the GPU library."""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.optimize
import scipy.special
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ O1 route ---
def _brute_topk(l, k):
    """Ordered top-k by exhaustive search: the unique k-subset whose every member
    precedes every non-member under (logit descending, index ascending), listed
    in that order.  Comparisons use Python floats, so -0.0 == 0.0."""
    E = len(l)
    before = lambda a, b: (l[a] > l[b]) or (l[a] == l[b] and a < b)  # noqa: E731
    found = []
    for sub in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in sub]
        if all(before(a, b) for a in sub for b in rest):
            found.append(sub)
    assert len(found) == 1
    sub = list(found[0])
    for i in range(len(sub)):
        for j in range(i + 1, len(sub)):
            if before(sub[j], sub[i]):
                sub[i], sub[j] = sub[j], sub[i]
    return sub


def test_route_brute_force_with_ties(oracle_lib):
    rng = np.random.default_rng(11)
    for trial in range(300):
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, min(E, 3) + 1))
        T = int(rng.integers(1, 7))
        # small integer-valued logits force many exact ties; sprinkle signed zeros
        lg = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
        zmask = rng.random((T, E)) < 0.3
        lg[zmask] = np.where(rng.random(zmask.sum()) < 0.5, -0.0, 0.0)
        ids, w = oracle_lib.route_topk(lg, k)
        for t in range(T):
            assert list(ids[t]) == _brute_topk([float(v) for v in lg[t]], k), (trial, lg[t])


def test_route_matches_stable_argsort(oracle_lib):
    rng = np.random.default_rng(5)
    for E, k in ((8, 2), (128, 8), (384, 8)):
        lg = rng.standard_normal((200, E)).astype(np.float32)
        lg[::7, 3] = lg[::7, 5]  # planted ties
        ids, _ = oracle_lib.route_topk(lg, k)
        ref = np.argsort(-lg, axis=1, kind="stable")[:, :k]
        np.testing.assert_array_equal(ids, ref)


def test_route_weights_softmax(oracle_lib):
    rng = np.random.default_rng(6)
    lg = (rng.standard_normal((64, 16)) * 3).astype(np.float32)
    ids, w = oracle_lib.route_topk(lg, 4, renormalize=True)
    sel = np.take_along_axis(lg.astype(np.float64), ids, axis=1)
    np.testing.assert_allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-13, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    ids2, w2 = oracle_lib.route_topk(lg, 4, renormalize=False)
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_array_equal(ids2, ids)
    np.testing.assert_allclose(w2, np.take_along_axis(full, ids, axis=1), rtol=1e-13, atol=0)
    assert np.all(np.diff(w, axis=1) <= 0)  # descending logits -> descending weights


# ----------------------------------------------------------------- O2 counts ---
def test_counts_bincount_and_sum(oracle_lib):
    rng = np.random.default_rng(7)
    B, E, k = 333, 64, 6
    lg = rng.standard_normal((B, E)).astype(np.float32)
    ids, _ = oracle_lib.route_topk(lg, k)
    full = oracle_lib.counts(ids, 0, E)
    np.testing.assert_array_equal(full, np.bincount(ids.ravel(), minlength=E))
    assert full.sum() == B * k  # RaMP 2.3: the n_e sum to Bk
    part = oracle_lib.counts(ids, 16, 8)
    np.testing.assert_array_equal(part, full[16:24])


# ----------------------------------------------------------------- O3 select ---
def test_ramp_worked_tile_example(oracle_lib):
    """RaMP 2.3 / 3.1: 16 -> 24 row-tiles at 8 rows and 16 -> 12 at 32 rows."""
    with open(os.path.join(GOLDEN, "ramp_tile_example.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        cnt = np.array(case["counts"], np.int32)
        assert cnt.sum() == g["tokens"] and len(cnt) == g["experts"]
        for b, tiles in case["row_tiles"].items():
            # one phase (q2 = 0) reduces the two-phase features to Equation 1
            _, _, feat = oracle_lib.select(cnt, [int(b)], [1], [0], [1_000_000], [1],
                                           np.zeros((1, 4), np.float32))
            W, T, A = feat[0]
            assert T == tiles, (case["name"], b)
            assert A == case["active_experts"]
            assert W == 1
        # and the waves: with 5 tiles resident per wave, W = ceil(T / 5)
        _, _, feat = oracle_lib.select(cnt, [8, 32], [1, 1], [0, 0], [5, 5], [1, 1],
                                       np.zeros((2, 4), np.float32))
        assert list(feat[:, 0]) == [-(-case["row_tiles"]["8"] // 5), -(-case["row_tiles"]["32"] // 5)]


def _round_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) float32 of an exact rational."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        if best is None or d < best[0] or (d == best[0] and (cand.view(np.uint32) & 1) == 0):
            best = (d, cand)
    return best[1]


def _fma_f32(a, b, c):
    return _round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def test_select_fp32_chain_exact_and_argmin(oracle_lib):
    rng = np.random.default_rng(8)
    V = 6
    b = [2, 4, 8, 16, 32, 64]
    q1 = [12, 12, 6, 6, 3, 3]
    q2 = [16, 8, 8, 4, 4, 2]
    S1 = [512] * V
    S2 = [768] * V
    for trial in range(200):
        El = int(rng.integers(1, 64))
        cnt = rng.integers(0, 300, El).astype(np.int32) * (rng.random(El) < 0.7)
        theta = (rng.random((V, 4)) * np.array([10, 5, 0.5, 1.0])).astype(np.float32)
        if trial % 3 == 0:
            theta[3] = theta[1]  # duplicate rows make exact ties of t_hat
        v, t_hat, feat = oracle_lib.select(cnt, b, q1, q2, S1, S2, theta)
        A = int((cnt > 0).sum())
        for c in range(V):
            rt = int(sum(-(-int(n) // b[c]) for n in cnt))
            T1, T2 = q1[c] * rt, q2[c] * rt
            W = -(-T1 // S1[c]) + -(-T2 // S2[c])
            assert list(feat[c]) == [W, T1 + T2, A]
            th = theta[c]
            ref = _fma_f32(th[3], np.float32(A), _fma_f32(th[2], np.float32(T1 + T2),
                                                           _fma_f32(th[1], np.float32(W), th[0])))
            assert t_hat[c].view(np.uint32) == ref.view(np.uint32)
        # argmin, first index on ties (RaMP Eq. 2)
        assert v == int(np.flatnonzero(t_hat == t_hat.min())[0])


# ------------------------------------------------------------------ O4 align ---
@pytest.mark.parametrize("b", [1, 2, 16, 32, 64, 128])
def test_align_bijection_order_padding(oracle_lib, b):
    rng = np.random.default_rng(100 + b)
    B, E, k, e0, El = 257, 64, 8, 16, 24
    lg = synth.routing_logits(synth.SHAPES["qwen3"], B, 0.3, rng)[0][:, :E]
    ids, _ = oracle_lib.route_topk(lg, k)
    ss, be, nb, sp = oracle_lib.align(ids, e0, El, b)
    loc = (ids.ravel() >= e0) & (ids.ravel() < e0 + El)
    local_slots = np.flatnonzero(loc)
    real = ss[ss >= 0]
    # bijection over the routed local slots
    np.testing.assert_array_equal(np.sort(real), local_slots)
    assert len(np.unique(real)) == len(real)
    # library cross-check: stable argsort of the slots' expert index
    order = np.argsort(ids.ravel()[local_slots], kind="stable")
    np.testing.assert_array_equal(real, local_slots[order])
    # padding count and block table
    cnt = np.bincount(ids.ravel()[local_slots] - e0, minlength=El)
    assert (ss < 0).sum() == int(sum(-(-n // b) * b - n for n in cnt))
    assert len(ss) == nb * b and len(be) == nb
    for blk in range(nb):
        rows = ss[blk * b:(blk + 1) * b]
        rows = rows[rows >= 0]
        assert len(rows) > 0
        assert np.all(ids.ravel()[rows] - e0 == be[blk])
    # inverse map
    for s in range(B * k):
        if loc[s]:
            assert ss[sp[s]] == s
        else:
            assert sp[s] == -1


def test_align_empty_rank(oracle_lib):
    ids = np.zeros((5, 2), np.int32)
    ids[:, 1] = 1
    ss, be, nb, sp = oracle_lib.align(ids, 8, 8, 16)
    assert nb == 0 and len(ss) == 0 and np.all(sp == -1)


# ------------------------------------------------------------- O5/O6 ffn -------
def _dense_ffn(x, w1, w3, w2):
    g = x @ w1.T
    u = x @ w3.T
    return ((g / (1.0 + np.exp(-g))) * u) @ w2.T


def _tiny_layer(T, E, k, H, I, seed, wdtype=synth.F32, x_std=0.5):
    rng = np.random.default_rng(seed)
    shape = synth.Shape("t", H, I, E, E, k, synth.F32, wdtype, synth.F32, "normal")
    x = (rng.standard_normal((T, H)) * x_std).astype(np.float32)
    w = {n: (rng.standard_normal((E,) + s) * 0.3).astype(np.float32)
         for n, s in (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I)))}
    lg = rng.standard_normal((T, E)).astype(np.float32)
    return synth.Layer(shape, T, None, 0, lg, x, w["w1"], w["w3"], w["w2"])


def test_one_hot_router_is_dense_ffn(oracle_lib):
    """"Decoding the Skew" III-C3: all tokens on one expert behave as a dense FFN."""
    L = _tiny_layer(9, 4, 1, 24, 40, 1)
    L.logits[:] = -5.0
    L.logits[:, 2] = 3.0
    out = oracle_lib.full_layer(L, b=4)
    ref = _dense_ffn(L.x.astype(np.float64), L.w1[2].astype(np.float64),
                     L.w3[2].astype(np.float64), L.w2[2].astype(np.float64))
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-13)


def test_identical_experts_any_routing_is_dense(oracle_lib):
    """With every expert equal, the softmax weights sum to 1, so any routing gives
    the dense FFN of that expert."""
    L = _tiny_layer(11, 6, 3, 16, 32, 2)
    for a in (L.w1, L.w3, L.w2):
        a[:] = a[0]
    out = oracle_lib.full_layer(L, b=2)
    ref = _dense_ffn(L.x.astype(np.float64), L.w1[0].astype(np.float64),
                     L.w3[0].astype(np.float64), L.w2[0].astype(np.float64))
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-12, atol=1e-13)


def test_tiny_brute_force_layer(oracle_lib):
    """T=4, E=4, k=2: each token's output from the matrix form of every expert,
    weighted by the softmax of its two largest logits."""
    L = _tiny_layer(4, 4, 2, 8, 12, 3)
    out = oracle_lib.full_layer(L, b=1)
    x = L.x.astype(np.float64)
    per_e = np.stack([_dense_ffn(x, L.w1[e].astype(np.float64), L.w3[e].astype(np.float64),
                                 L.w2[e].astype(np.float64)) for e in range(4)])
    for t in range(4):
        order = sorted(range(4), key=lambda e: (-float(L.logits[t, e]), e))[:2]
        z = np.array([float(L.logits[t, e]) for e in order])
        p = np.exp(z - z.max())
        p /= p.sum()
        ref = p[0] * per_e[order[0], t] + p[1] * per_e[order[1], t]
        np.testing.assert_allclose(out["Y"][t], ref, rtol=1e-12, atol=1e-14)


def test_ffn_slots_match_layer(oracle_lib):
    L = _tiny_layer(7, 5, 2, 16, 24, 4)
    out = oracle_lib.full_layer(L, b=2)
    toks = np.repeat(np.arange(7), 2).astype(np.int32)
    y = oracle_lib.ffn_slots(L, toks, out["ids"].ravel())
    Y = (y.reshape(7, 2, 16) * out["w"][:, :, None]).sum(axis=1)
    np.testing.assert_allclose(Y, out["Y"], rtol=1e-12, atol=1e-14)


def test_partial_expert_block_zero_rows(oracle_lib):
    L = _tiny_layer(16, 8, 2, 8, 16, 5)
    L.expert_begin = 4
    L.shape = synth.Shape("t", 8, 16, 8, 4, 2, synth.F32, synth.F32, synth.F32, "normal")
    L.w1, L.w3, L.w2 = L.w1[:4], L.w3[:4], L.w2[:4]
    out = oracle_lib.full_layer(L, b=2)
    none_local = ~np.any((out["ids"] >= 4) & (out["ids"] < 8), axis=1)
    assert np.all(out["Y"][none_local] == 0.0)


# ------------------------------------------------------------------ decoders ---
def test_fp8_decoder_all_codes(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_lib.decode_fp8(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_bf16_decoder(oracle_lib):
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 65536, 4096).astype(np.uint16)
    ours = oracle_lib.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])


def test_fp8_weights_decode_as_q_times_s(oracle_lib):
    """The FFN over fp8 weights equals the FFN over the dequantised fp64 weights."""
    rng = np.random.default_rng(10)
    H, I, E = 256, 128, 2
    w = {n: (rng.standard_normal((E,) + s) * 0.02).astype(np.float32)
         for n, s in (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I)))}
    q, s, deq = {}, {}, {}
    for n, a in w.items():
        qs = [synth.quantize_fp8_blocks(a[e]) for e in range(E)]
        q[n] = np.stack([t[0] for t in qs])
        s[n] = np.stack([t[1] for t in qs])
        deq[n] = np.stack([oracle_lib.decode_fp8(q[n][e]) *
                           np.kron(s[n][e].astype(np.float64), np.ones((128, 128)))
                           for e in range(E)])
    shape = synth.Shape("t", H, I, E, E, 1, synth.F32, synth.FP8, synth.F32, "normal")
    x = (rng.standard_normal((3, H)) * 0.5).astype(np.float32)
    L = synth.Layer(shape, 3, None, 0, np.zeros((3, E), np.float32), x, q["w1"], q["w3"], q["w2"],
                    s["w1"], s["w3"], s["w2"])
    y = oracle_lib.ffn_slots(L, np.arange(3, dtype=np.int32), np.array([1, 0, 1], np.int32))
    for i, e in enumerate([1, 0, 1]):
        ref = _dense_ffn(x[i:i + 1].astype(np.float64), deq["w1"][e], deq["w3"][e], deq["w2"][e])
        np.testing.assert_allclose(y[i], ref[0], rtol=1e-12, atol=1e-15)
    # and the quantisation itself stays within one E4M3 step of the fp32 weight
    rel = np.abs(deq["w1"] - w["w1"]) / np.kron(s["w1"], np.ones((1, 128, 128)))
    assert rel.max() <= 16.0  # half a step at the top binade (448 = 1.75 * 2^8, step 32)


# ------------------------------------------------------------------ NNLS pin ---
def test_nnls_relative_error_reading():
    """Scaling rows by 1/t turns the relative-error objective of RaMP 3.1 into a
    plain NNLS with target 1; the two minimisers agree."""
    rng = np.random.default_rng(12)
    X = np.c_[np.ones(40), rng.integers(1, 20, 40), rng.integers(1, 200, 40), rng.integers(1, 64, 40)]
    t = X @ np.array([3.0, 2.0, 0.05, 0.1]) * (1 + 0.05 * rng.standard_normal(40))
    th, _ = scipy.optimize.nnls(X / t[:, None], np.ones(40))
    obj = lambda p: float((((X @ p) / t - 1.0) ** 2).sum())  # noqa: E731
    for _ in range(200):
        p = np.maximum(th + 0.01 * rng.standard_normal(4) * np.abs(th + 1e-3), 0)
        assert obj(th) <= obj(p) + 1e-12
