"""Offline tuning of the on-GPU configuration chooser.

RaMP (arXiv 2604.26039), section 3.1: the predicted time of configuration c on
load n is t_c = th_c0 + th_c1 W_c(n) + th_c2 T_c(n) + th_c3 A(n), with the
row-tiles T_c and waves W_c of section 2.2, Eq. 1 and the active experts A.  One
coefficient vector per configuration is fit offline by non-negative least
squares (Lawson-Hanson) on the relative error sum_i (t_hat / t - 1)^2.  Section
3.1 also picks the served menu greedily offline to minimise the recorded
workload's time.

This module:
- times every compiled configuration (forced) on fit loads;
- computes the chooser's features with the same integer formulas moe_select_config
  evaluates on the device;
- fits theta per configuration with scipy.optimize.nnls on rows scaled by 1/t
  (exactly the relative-error objective);
- reports the rank correlation of the fit and a greedy menu ranking;
- writes theta/<workload>.json, which the benchmark loads.

The fit loads are disjoint from the scored loads the benchmark reports:
different alphas and reps, as RaMP section 4 keeps fit and scored traffic apart.

    python -m routing_aware_grouped_amd.tune --shapes mixtral,qwen3 --out theta/
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
THETA_DIR = os.path.join(HERE, "theta")
KERNEL_SOURCES = ["csrc/grouped_ffn.hip", "csrc/moe_common.h"]

# fit grid: token counts per workload, alphas and reps disjoint from the scored sweep
FIT_TOKENS = {
    "mixtral": [1, 4, 16, 64, 128, 256, 512, 1024, 2048],
    "qwen3": [1, 4, 16, 64, 128, 256, 512, 1024, 2048, 4096],
    "dsv3_share": [8, 32, 128, 512, 1024, 2048],      # B = 8 x tokens per GPU
    "kimi_share": [8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096],
    "dsv3_share_fp8a": [8, 32, 128, 512, 1024, 2048],
    "kimi_share_fp8a": [8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096],
    "dsv3_share_fp8ah": [8, 32, 128, 512, 1024, 2048],
    "kimi_share_fp8ah": [8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096],
    "dsv3_share_sh": [8, 32, 128, 512, 1024, 2048],
}
FIT_ALPHAS = [0.03, 0.5, 3.0, 30.0]
FIT_REP0 = 100


def _code_only(text: str) -> str:
    """Source text without comments, trailing blanks and empty lines, so that an
    edit of a comment leaves the hash (and the timings filed under it) valid."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def kernel_source_hash() -> str:
    """First 16 hex digits of the sha256 of the grouped FFN's code (comments
    stripped); timings, fitted theta and counter summaries are filed under it."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------- features ----
def features(counts, cc) -> np.ndarray:
    """[V][4] rows (1, W, T, A) of RaMP Eq. 3 for one load.

    The formulas are those of moe_select_config:
    - rt = sum_e ceil(n_e / b);
    - T = (q1 + q2) rt;
    - W = ceil(q1 rt / S1) + ceil(q2 rt / S2);
    - A = #{e : n_e > 0}.

    cc holds the per-configuration constants of moe_cost_constants."""
    n = np.asarray(counts, dtype=np.int64)
    A = int((n > 0).sum())
    V = len(cc["b"])
    out = np.zeros((V, 4), dtype=np.float64)
    for v in range(V):
        b, q1, q2, S1, S2 = (int(cc[k][v]) for k in ("b", "q1", "q2", "S1", "S2"))
        rt = int(((n + b - 1) // b).sum())
        T = (q1 + q2) * rt
        W = -(-q1 * rt // S1) + -(-q2 * rt // S2)
        out[v] = (1.0, W, T, A)
    return out


# ---------------------------------------------------------------------- fit ----
def fit_nnls(F: np.ndarray, t: np.ndarray) -> np.ndarray:
    """theta >= 0 minimising sum_i (F_i theta / t_i - 1)^2 (Lawson-Hanson NNLS on
    rows scaled by 1 / t_i)."""
    from scipy.optimize import nnls
    F = np.asarray(F, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    Fs = F / t[:, None]
    # column scaling keeps the active-set iteration well conditioned; undone after
    cs = np.maximum(np.abs(Fs).max(axis=0), 1e-30)
    th, _ = nnls(Fs / cs, np.ones(len(t)), maxiter=50 * F.shape[1])
    return th / cs


def spearman(a, b) -> float:
    ra = np.argsort(np.argsort(a)).astype(np.float64)
    rb = np.argsort(np.argsort(b)).astype(np.float64)
    if ra.std() == 0 or rb.std() == 0:
        return 1.0
    return float(np.corrcoef(ra, rb)[0, 1])


def greedy_menu(times: np.ndarray, size: int, relative: bool = False) -> list[int]:
    """Greedy order of configurations: each step adds the one that most lowers the
    summed time of the loads when each load runs the best configuration chosen so
    far (RaMP section 3.1's offline menu choice).  relative=True sums log times
    instead, so that every fit load weighs by its relative loss (the chooser is
    judged per load, by the geometric mean of its gaps) rather than a few long
    loads deciding the menu."""
    times = np.asarray(times, dtype=np.float64)
    cost = np.log(times) if relative else times
    chosen: list[int] = []
    best = np.full(times.shape[0], np.inf)
    for _ in range(min(size, times.shape[1])):
        tot, v = min((np.minimum(best, cost[:, v]).sum(), v) for v in range(times.shape[1])
                     if v not in chosen)
        chosen.append(v)
        best = np.minimum(best, cost[:, v])
    return chosen


def greedy_menu_served(pred: np.ndarray, times: np.ndarray, size: int) -> list[int]:
    """Greedy served menu judged by the chooser itself: each step adds the
    configuration that most lowers the geometric mean, over the fit loads, of the
    time of the configuration the cost model would pick within the menu (argmin of
    pred over the menu's entries, ties to the lower index).  RaMP section 3.1 picks
    the menu that minimises the recorded workload's time; scoring what the fitted
    model would serve, rather than the best entry of the menu, keeps out entries
    the model cannot tell from one already in (equal cost-model constants)."""
    pred = np.asarray(pred, dtype=np.float64)
    logt = np.log(np.asarray(times, dtype=np.float64))
    n, V = logt.shape
    menu: list[int] = []
    for _ in range(min(size, V)):
        best = None
        for v in range(V):
            if v in menu:
                continue
            m = sorted(menu + [v])
            pick = np.asarray(m)[np.argmin(pred[:, m], axis=1)]
            obj = logt[np.arange(n), pick].mean()
            if best is None or obj < best[0] - 1e-12:
                best = (obj, v)
        menu.append(best[1])
    return menu


# ------------------------------------------------------------------ timing -----
class _Timer:
    def __init__(self, torch):
        self.torch = torch
        self.scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        self.n = 0

    def flush(self):
        self.n += 1
        self.scratch.fill_(self.n & 0xFF)

    def graph(self, fn):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def median_us(self, g, reps, warmup=2):
        torch = self.torch
        for _ in range(warmup):
            self.flush()
            g.replay()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            self.flush()
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)


def collect(shape_name: str, reps: int = 9, n_rep_loads: int = 1, log=print) -> dict:
    """Forced-configuration layer times (us, cold cache, graph replay) on the fit
    loads of one workload, with each load's local expert counts."""
    import torch

    import synth
    from . import moe_cost_constants, moe_num_variants
    from . import layer as L
    V = moe_num_variants()
    T = _Timer(torch)
    wdev = synth.make_weights_device(shape_name)
    wts = (wdev["w1"], wdev["w3"], wdev["w2"], wdev["s1"], wdev["s3"], wdev["s2"])
    nowts = {k: None for k in ("w1", "w3", "w2", "s1", "s3", "s2")}
    loads = []
    cc = None
    for tok in FIT_TOKENS[shape_name]:
        for a in FIT_ALPHAS:
            for r in range(n_rep_loads):
                layer = synth.make_layer(shape_name, tok, a, FIT_REP0 + r, weights=nowts)
                b = L.from_layer(layer, weights=wts)
                L.route(b)
                torch.cuda.synchronize()
                # a shared expert counts as a local expert that every token reaches
                # (the device cost model adds its row-tiles and one active expert)
                counts = np.concatenate([b.counts.cpu().numpy().astype(np.int64),
                                         np.full(layer.shape.shared, tok, np.int64)])
                if cc is None or cc["_key"] != (b.p.hidden, b.p.inter):
                    cc = moe_cost_constants(b.p)
                    cc["_key"] = (b.p.hidden, b.p.inter)
                g = T.graph(lambda: L.forward(b, forced_variant=True))
                times = []
                for v in range(V):
                    b.variant.fill_(v)
                    torch.cuda.synchronize()
                    times.append(T.median_us(g, reps))
                del g
                loads.append(dict(tokens=tok, alpha=a, rep=FIT_REP0 + r, counts=counts.tolist(),
                                  times_us=[round(x, 3) for x in times]))
                log(f"[tune] {shape_name} B={tok} alpha={a}: " + " ".join(f"{x:.1f}" for x in times))
    ccj = {k: list(map(int, v)) for k, v in cc.items() if not k.startswith("_")}
    del wdev
    torch.cuda.empty_cache()
    return dict(shape=shape_name, cost_constants=ccj, loads=loads, variants=V)


# prediction of a configuration outside the served menu: larger than any real one,
# so the device's argmin never takes it (finite, so the fp32 chain stays exact)
OFF_MENU_THETA0 = 1.0e30


def fit(data: dict, menu_size: int | None = None) -> dict:
    """theta per configuration from collected timings, with diagnostics.

    Every configuration's theta is fitted; the served menu (RaMP section 3.1) is
    then `menu_size` configurations picked by greedy_menu_served on the fit loads;
    the others get theta = (OFF_MENU_THETA0, 0, 0, 0), which the device's argmin
    never picks."""
    V = data["variants"]
    cc = data["cost_constants"]
    F = np.stack([features(ld["counts"], cc) for ld in data["loads"]])  # [n][V][4]
    t = np.array([ld["times_us"] for ld in data["loads"]], dtype=np.float64)  # [n][V]
    order = greedy_menu(t, V, relative=True)  # best-entry order, for the record
    theta_all = np.stack([fit_nnls(F[:, v, :], t[:, v]) for v in range(V)])
    pred_all = np.einsum("nvk,vk->nv", F, theta_all)
    menu = sorted(greedy_menu_served(pred_all, t, menu_size or V))
    theta = np.stack([theta_all[v] if v in menu else np.array([OFF_MENU_THETA0, 0.0, 0.0, 0.0])
                      for v in range(V)]).astype(np.float32)
    # diagnostics in float64 (the device's own fp32 choice is what the benchmark reports)
    pred = np.einsum("nvk,vk->nv", F, theta.astype(np.float64))
    pick = pred.argmin(axis=1)
    best = t.min(axis=1)
    gaps = t[np.arange(len(t)), pick] / best - 1.0
    rel_err = np.abs(pred[np.arange(len(t)), pick] / t[np.arange(len(t)), pick] - 1.0)
    return dict(
        theta=[[float(x) for x in row] for row in theta],
        fit_loads=len(t),
        fit_geomean_gap=float(np.exp(np.mean(np.log1p(gaps))) - 1.0),
        fit_worst_gap=float(gaps.max()),
        spearman_mean=float(np.mean([spearman(pred[i][menu], t[i][menu]) for i in range(len(t))])),
        picked_rel_err_median=float(np.median(rel_err)),
        greedy_menu=order,
        menu=menu,
        # cost of serving the menu instead of every compiled configuration, on
        # the fit loads: geomean of best-in-menu / best-overall - 1
        menu_geomean_loss=float(np.exp(np.mean(np.log(t[:, menu].min(axis=1) / best))) - 1.0),
    )


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--shapes", default="mixtral,qwen3,dsv3_share,kimi_share")
    ap.add_argument("--out", default=THETA_DIR, help="directory for <workload>.json")
    ap.add_argument("--reps", type=int, default=9, help="timed replays per configuration and load")
    ap.add_argument("--rep-loads", type=int, default=1, help="loads per (tokens, alpha)")
    ap.add_argument("--menu", type=int, default=6,
                    help="configurations in the served menu (greedy on the fit loads)")
    ap.add_argument("--refit", action="store_true",
                    help="no timing: refit theta and the menu from the loads stored in --out")
    args = ap.parse_args(argv)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    os.makedirs(args.out, exist_ok=True)
    for shp in [s for s in args.shapes.split(",") if s]:
        t0 = time.perf_counter()
        path = os.path.join(args.out, f"{shp}.json")
        if args.refit:  # the forced times already collected for this kernel build
            with open(path) as f:
                old = json.load(f)
            if old.get("kernel_source_sha") != kernel_source_hash():
                raise SystemExit(f"{path} was timed on another kernel build")
            data = dict(shape=shp, cost_constants=old["cost_constants"], loads=old["loads"],
                        variants=len(old["theta"]))
        else:
            data = collect(shp, args.reps, args.rep_loads,
                           log=lambda m: print(m, file=sys.stderr, flush=True))
        res = fit(data, args.menu)
        res.update(shape=shp, kernel_source_sha=kernel_source_hash(),
                   fit_alphas=FIT_ALPHAS, fit_tokens=FIT_TOKENS[shp], fit_rep0=FIT_REP0,
                   cost_constants=data["cost_constants"], loads=data["loads"],
                   wall_s=round(time.perf_counter() - t0, 1))
        with open(path, "w") as f:
            json.dump(res, f, indent=1)
        print(f"[tune] {shp}: menu {res['menu']} (greedy order {res['greedy_menu']}, menu loss "
              f"{res['menu_geomean_loss']:.4f}) fit gap {res['fit_geomean_gap']:.4f} "
              f"(worst {res['fit_worst_gap']:.4f}) spearman {res['spearman_mean']:.3f} -> {path}",
              flush=True)


if __name__ == "__main__":
    main()
