"""Alternative configuration choosers, scored on the same exhaustive labels as the
on-device cost model.

The pages compare the routing-aware cost model (RaMP, arXiv 2604.26039) with
simpler policies; each is restated here on this library's configuration menu:

- RaMP, appendix A.2 and Table 4: tables that see the cost model's per-GPU
  inputs.  A per-GPU table keyed on the token count (also the vLLM-style
  batch-size table of Tables 9 and 10), a 2-D table keyed on the token count and
  the padding, and the 8 nearest neighbours on token count, active experts,
  padding and the largest load over the mean.
- "Decoding the Skew" (arXiv 2607.23099), section IV: DA-MoE keeps, per
  token-count bucket, one exemplar per tuned routing distribution (its per-expert
  token counts sorted in descending order and scaled to unit L2 norm) with the
  kernel that ran it fastest, and at run time takes the kernel of the exemplar
  with the highest cosine similarity to the live sorted histogram.  The
  frameworks it compares with tune on random router logits and keep one kernel
  per token-count bucket (its NoDA baseline).
- GC-MoE (arXiv 2611.04222), section 4, block-size heuristic: BLOCK_M is the
  smallest candidate that covers the expected tokens per expert plus its
  standard deviation.

Every policy is fit on the loads the cost model is fit on (the fit loads of
tune.py: token count, local expert counts and the forced time of every
configuration) and scored on the benchmark's sweep points, whose exhaustive
per-configuration times are the labels.  They run on the host from a load's token
count and local expert counts; they are yardsticks for the on-device chooser and
take no part in the layer.

Readings where the pages leave a step open:
- token-count buckets are the fit token counts; a load uses the nearest one on a
  log2 scale (DA-MoE buckets by token count; RaMP's tables by token count);
- the padding of a load is the share of padded rows when every local expert's
  rows are rounded up to the menu's largest BLOCK_M;
- with 8 fit loads per token count, the padding axis has 4 quantile buckets (fit
  over all loads) rather than RaMP's 8;
- a table cell, and the 8 neighbours, take the configuration with the lowest
  geometric-mean time over the fit loads they hold; an empty cell falls back to
  the token-count table;
- nearest neighbours use the four features, each scaled by its standard
  deviation over the fit loads, with log2 of the token count;
- NoDA's one tuning input per bucket is the fit load nearest to uniform routing
  (largest Dirichlet alpha, first rep): what random router logits produce;
- GC-MoE's expected tokens per expert is the mean of the local counts (B k / E
  when one GPU holds every expert), its standard deviation the Poisson one,
  sqrt(m); the page's formula is garbled around that root.
"""
from __future__ import annotations

import math

import numpy as np


def _log2(x: float) -> float:
    return math.log2(max(float(x), 1.0))


def _bucket(tokens: int, buckets: list[int]) -> int:
    """The fit token count nearest to `tokens` on a log2 scale (ties: the smaller)."""
    return min(buckets, key=lambda b: (abs(_log2(b) - _log2(tokens)), b))


def _geomean_best(times) -> int:
    """The configuration with the lowest geometric-mean time over the rows of `times`."""
    t = np.asarray(times, dtype=np.float64).reshape(-1, np.shape(times)[-1])
    return int(np.argmin(np.mean(np.log(t), axis=0)))


def padding(counts, block_m: int) -> float:
    """Share of padded rows when each expert's rows are rounded up to `block_m`."""
    c = np.asarray(counts, dtype=np.int64)
    rows = int((-(-c // block_m) * block_m).sum())
    return 0.0 if rows == 0 else 1.0 - float(c.sum()) / rows


def load_over_mean(counts) -> float:
    """The largest local expert count over the mean local count."""
    c = np.asarray(counts, dtype=np.float64)
    m = c.mean() if c.size else 0.0
    return 0.0 if m <= 0 else float(c.max() / m)


def exemplar(counts) -> np.ndarray:
    """The per-expert counts sorted in descending order, scaled to unit L2 norm."""
    v = np.sort(np.asarray(counts, dtype=np.float64))[::-1]
    n = np.linalg.norm(v)
    return v / n if n > 0 else v


class TokenTable:
    """One configuration per token-count bucket, the geometric-mean best over the
    bucket's fit loads (RaMP Table 4, per-GPU table; Tables 9-10, batch-size table)."""
    name = "token-count table"

    def fit(self, loads):
        by = {}
        for ld in loads:
            by.setdefault(ld["tokens"], []).append(ld["times_us"])
        self.buckets = sorted(by)
        self.table = {b: _geomean_best(ts) for b, ts in by.items()}
        return self

    def choose(self, tokens, counts):
        return self.table[_bucket(tokens, self.buckets)]


class PaddingTable:
    """Token count x padding (RaMP Table 4, 2-D table), padding in quantile buckets."""
    name = "token-count x padding table"

    def __init__(self, block_m_max: int, nbins: int = 4):
        self.bm = block_m_max
        self.nbins = nbins

    def _bin(self, counts) -> int:
        return int(np.searchsorted(self.edges, padding(counts, self.bm), side="right"))

    def fit(self, loads):
        self.fallback = TokenTable().fit(loads)
        self.buckets = self.fallback.buckets
        pads = np.array([padding(ld["counts"], self.bm) for ld in loads])
        self.edges = np.quantile(pads, np.arange(1, self.nbins) / self.nbins)
        cells = {}
        for ld in loads:
            cells.setdefault((ld["tokens"], self._bin(ld["counts"])), []).append(ld["times_us"])
        self.table = {k: _geomean_best(ts) for k, ts in cells.items()}
        return self

    def choose(self, tokens, counts):
        key = (_bucket(tokens, self.buckets), self._bin(counts))
        if key in self.table:
            return self.table[key]
        return self.fallback.choose(tokens, counts)


class NearestNeighbors:
    """The k fit loads nearest in (log2 tokens, active experts, padding, largest load
    over mean), each feature scaled by its spread (RaMP Table 4, 8 nearest neighbours)."""

    def __init__(self, block_m_max: int, k: int = 8):
        self.bm = block_m_max
        self.k = k
        self.name = f"{k} nearest neighbours"

    def _feat(self, tokens, counts):
        return np.array([_log2(tokens), float(np.count_nonzero(counts)),
                         padding(counts, self.bm), load_over_mean(counts)])

    def fit(self, loads):
        F = np.stack([self._feat(ld["tokens"], ld["counts"]) for ld in loads])
        sd = F.std(axis=0)
        self.scale = np.where(sd > 0, sd, 1.0)
        self.F = F / self.scale
        self.times = np.array([ld["times_us"] for ld in loads], dtype=np.float64)
        return self

    def choose(self, tokens, counts):
        q = self._feat(tokens, counts) / self.scale
        d = np.linalg.norm(self.F - q, axis=1)
        near = np.argsort(d, kind="stable")[: self.k]
        return _geomean_best(self.times[near])


class NoDA:
    """One configuration per token-count bucket from one tuning input, the fit load
    nearest to uniform routing ("Decoding the Skew", section IV, NoDA)."""
    name = "NoDA"

    def fit(self, loads):
        pick = {}
        for ld in loads:
            key = (ld["alpha"], -ld.get("rep", 0))
            if ld["tokens"] not in pick or key > pick[ld["tokens"]][0]:
                pick[ld["tokens"]] = (key, ld["times_us"])
        self.buckets = sorted(pick)
        self.table = {b: int(np.argmin(t)) for b, (_, t) in pick.items()}
        return self

    def choose(self, tokens, counts):
        return self.table[_bucket(tokens, self.buckets)]


class ExemplarMatcher:
    """DA-MoE ("Decoding the Skew", sections IV-A and IV-B): per token-count bucket,
    the exemplar of every fit load with its fastest configuration; a load takes the
    configuration of the exemplar with the highest cosine similarity."""
    name = "exemplar matcher"

    def fit(self, loads):
        by = {}
        for ld in loads:
            by.setdefault(ld["tokens"], []).append((exemplar(ld["counts"]),
                                                    int(np.argmin(ld["times_us"]))))
        self.buckets = sorted(by)
        self.table = {b: (np.stack([e for e, _ in rows]), [v for _, v in rows])
                      for b, rows in by.items()}
        return self

    def choose(self, tokens, counts):
        ex, kids = self.table[_bucket(tokens, self.buckets)]
        return kids[int(np.argmax(ex @ exemplar(counts)))]


class BlockSizeHeuristic:
    """GC-MoE's host heuristic on this menu: the smallest BLOCK_M covering
    m + sqrt(m), m the mean local expert count, else the largest.  Uses no timings."""
    name = "BLOCK_M heuristic"

    def __init__(self, block_m):
        self.block_m = list(block_m)

    def fit(self, loads):
        return self

    def choose(self, tokens, counts):
        c = np.asarray(counts, dtype=np.float64)
        m = float(c.mean()) if c.size else 0.0
        need = m + math.sqrt(m)
        order = sorted(range(len(self.block_m)), key=lambda v: (self.block_m[v], v))
        for v in order:
            if self.block_m[v] >= need:
                return v
        return order[-1]


def policies(block_m):
    """Every alternative policy on a menu whose configurations have these BLOCK_M."""
    bmax = max(block_m)
    return [TokenTable(), PaddingTable(bmax), NearestNeighbors(bmax), NoDA(), ExemplarMatcher(),
            BlockSizeHeuristic(block_m)]


def score(policy, points) -> dict:
    """Gap of a policy's choices to exhaustive search over `points` (dicts with
    tokens, counts and us_per_variant): the geometric mean over points of
    t(chosen) / t(best), less one, the worst gap and the share within 5%."""
    gaps = []
    for p in points:
        t = p["us_per_variant"]
        v = policy.choose(p["tokens"], p["counts"])
        gaps.append(t[v] / min(t) - 1.0)
    g = np.array(gaps)
    return dict(geomean_gap=round(float(np.exp(np.mean(np.log1p(g))) - 1.0), 4),
                worst_gap=round(float(g.max()), 4),
                within_5pct=round(float(np.mean(g <= 0.05)), 3))


def compare(fit_loads, points, block_m) -> dict:
    """Every alternative policy, fit on `fit_loads` and scored on `points`."""
    return {p.name: score(p.fit(fit_loads), points) for p in policies(block_m)}
