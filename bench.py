#!/usr/bin/env python3
"""Benchmark of the routing-aware fused-MoE layer on one MI355X.

Metric: fused-MoE layer microseconds, and the fraction of the HBM or bf16 MFMA
roofline, over token counts x Dirichlet(alpha) routing skew.

One step = one pass of the whole layer over one synthetic batch:
- route/top-k + histogram;
- on-GPU configuration choice;
- align/sort;
- grouped gate/up + SwiGLU;
- grouped down;
- combine.

It is replayed from a HIP graph with the inputs resident in HBM and the caches
cold. Before every timed replay a 1 GiB scratch write evicts L2 and the Infinity
Cache; the write is outside the timed events.

The headline point is the largest single-GPU configuration the metric is quoted
on: the Mixtral-8x7B-shaped layer (H 4096, I 14336, 8 experts, top-2, bf16) at
2048 tokens, alpha = 1.  The last stdout line is one compact JSON record (the
headline, its roofline and CPU baseline, one summary per swept workload); the
full result with every sweep point goes to --out.

The same run sweeps the four full-size workloads over their token counts and
alphas:
- Mixtral-shaped;
- Qwen3-30B-A3B-shaped;
- the DeepSeek-V3 one-GPU expert share;
- the Kimi-K2 one-GPU expert share.

On every sweep point it times each compiled tile configuration (exhaustive
search) and reports the gap of the on-GPU choice, and next to it the gaps of the
simpler policies the pages compare with (routing_aware_grouped_amd.choosers),
fit on the same fit loads as the cost model.

Work accounting follows GC-MoE's conventions:
- FLOPs = 6 * routed slots * H * I;
- algorithmic bytes = the distinct active experts' weights (+ fp8 scales), counted
  once, plus the activation rows read and the outputs written.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5166e15  # flop/s, dense bf16 MFMA (256 CU x 2.4 GHz x 4096)
MFMA_FP8_PEAK = 2 * MFMA_BF16_PEAK  # flop/s, dense fp8 MFMA (the FP8 activation path's gate/up)
METRIC = "fused-MoE layer µs + % of HBM/MFMA roofline vs tokens × Dirichlet α skew"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

SWEEPS = {
    "mixtral": dict(tokens=[1, 16, 128, 512, 2048], alphas=[0.1, 1.0, 10.0, 100.0]),
    "qwen3": dict(tokens=[1, 16, 128, 512, 2048, 4096], alphas=[0.05, 0.3, 1.0, 10.0]),
    "dsv3_share": dict(tokens=[1, 16, 64, 256], alphas=[0.1, 1.0, 10.0]),  # per GPU; B = 8T
    "kimi_share": dict(tokens=[8, 64, 512, 2048, 4096], alphas=[0.05]),
    # the expert shares again with FP8 activations in the gate/up GEMM
    "dsv3_share_fp8a": dict(tokens=[1, 16, 64, 256], alphas=[0.1, 1.0, 10.0]),  # B = 8T
    "kimi_share_fp8a": dict(tokens=[8, 64, 512, 2048, 4096], alphas=[0.05]),
    # and with FP8 activations in both GEMMs
    "dsv3_share_fp8ah": dict(tokens=[1, 16, 64, 256], alphas=[0.1, 1.0, 10.0]),  # B = 8T
    "kimi_share_fp8ah": dict(tokens=[8, 64, 512, 2048, 4096], alphas=[0.05]),
    # the DeepSeek-V3 share with its shared expert fused into the same launches
    "dsv3_share_sh": dict(tokens=[1, 16, 64, 256], alphas=[0.1, 1.0, 10.0]),  # B = 8T
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ accounting --
def work(layer, ids_np):
    """Algorithmic FLOPs and bytes of one layer invocation on this load, and of its
    gate/up kernel alone (h and y_slots are intermediates, not counted)."""
    import numpy as np
    import synth
    sh = layer.shape
    H, I, k, El, e0 = sh.hidden, sh.inter, sh.top_k, sh.local_experts, layer.expert_begin
    B = layer.tokens
    loc = (ids_np >= e0) & (ids_np < e0 + El)
    cnt = np.bincount((ids_np[loc] - e0).ravel(), minlength=El)
    # shared experts: B more slots each, every token, one more active expert each
    nsh = getattr(sh, "shared", 0)
    S = int(loc.sum()) + nsh * B
    A = int((cnt > 0).sum()) + nsh
    U = B if nsh else int(loc.any(axis=1).sum())
    wb = 1 if sh.weight_dtype == synth.FP8 else (4 if sh.weight_dtype == synth.F32 else 2)
    ab = 4 if sh.act_dtype == synth.F32 else 2
    mat_scale = (H // 128) * (I // 128) * 4 if sh.weight_dtype == synth.FP8 else 0
    wbytes = A * (3 * H * I * wb + 3 * mat_scale)
    layer_bytes = wbytes + U * H * ab + B * H * ab + B * sh.num_experts * 4 + B * k * 8
    gate_up_bytes = A * (2 * H * I * wb + 2 * mat_scale) + U * H * ab
    # time the MFMA pipes need at peak: bf16 rate, except the GEMMs that the FP8
    # activation path runs at the fp8 rate (gate/up; with act_quant 2 down too)
    aq = getattr(sh, "act_quant", 0)
    gu_peak = MFMA_FP8_PEAK if aq >= 1 else MFMA_BF16_PEAK
    dn_peak = MFMA_FP8_PEAK if aq == 2 else MFMA_BF16_PEAK
    mfma_s = 4 * S * H * I / gu_peak + 2 * S * H * I / dn_peak
    return dict(S=S, A=A, U=U, flops=6 * S * H * I, layer_bytes=layer_bytes,
                gate_up_bytes=gate_up_bytes, gate_up_flops=4 * S * H * I, gate_up_peak=gu_peak,
                # the fused plan's one FFN launch: every weight byte and the gathered x rows
                ffn_bytes=wbytes + U * H * ab,
                mfma_s=mfma_s, eff_exp=synth.eff_exp(cnt),
                # the chooser's view: a shared expert is a local expert with B tokens
                counts=np.concatenate([cnt, np.full(nsh, B, dtype=cnt.dtype)]))


PACK = None  # layer.allocate's pack argument (--pack)
PLAN = "grouped"  # the headline point's plan (--plan)


def roof_us(w):
    return max(w["layer_bytes"] / HBM_PEAK, w["mfma_s"]) * 1e6


def kernel_source_hash():
    from routing_aware_grouped_amd.tune import kernel_source_hash as h
    return h()


def measured_traffic(workload_key):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != kernel_source_hash():
        return None
    ent = d.get("workloads", {}).get(workload_key)
    if not ent:
        return None
    return int(ent["fetch_kib"] * 1024 * d["fetch_factor"] + ent["write_kib"] * 1024 * d["write_factor"])


# ---------------------------------------------------------------------- timing --
class Timer:
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

    def time_graph(self, g, reps, warmup):
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
        return [a.elapsed_time(b) * 1e3 for a, b in evs]  # us


def stats(us):
    s = sorted(us)
    q = lambda f: s[min(len(s) - 1, int(f * (len(s) - 1) + 0.5))]  # noqa: E731
    return dict(median=statistics.median(s), p10=q(0.1), p90=q(0.9), mean=statistics.fmean(s))


# ---------------------------------------------------------------------- theta --
def load_theta(shape_name, V):
    """The fitted chooser coefficients of a workload (routing_aware_grouped_amd.tune),
    and a label saying where they came from and whether they were fit on the
    current kernel sources."""
    import torch
    path = os.path.join(ROOT, "routing_aware_grouped_amd", "theta", f"{shape_name}.json")
    if os.path.exists(path):
        with open(path) as f:
            d = json.load(f)
        th = torch.tensor(d["theta"], dtype=torch.float32)
        if th.shape == (V, 4):
            fresh = d.get("kernel_source_sha") == kernel_source_hash()
            return th, (os.path.relpath(path, ROOT) +
                        ("" if fresh else " (fit on an older kernel build)"))
    # no fitted table: predict time by waves alone (th1 = 1)
    th = torch.zeros(V, 4, dtype=torch.float32)
    th[:, 1] = 1.0
    return th, None


def fit_loads(shape_name):
    """The loads the workload's chooser was fit on, with the forced time of every
    configuration, or None."""
    path = os.path.join(ROOT, "routing_aware_grouped_amd", "theta", f"{shape_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        return json.load(f).get("loads")


# ----------------------------------------------------------------------- points --
def device_weights(wdev):
    return (wdev["w1"], wdev["w3"], wdev["w2"], wdev["s1"], wdev["s3"], wdev["s2"])


def run_point(torch, np, synth, L, T, shape, tokens, alpha, wdev, whost, theta, V, reps, warmup,
              exhaustive=True, rep=0, force=None, plan="grouped"):
    layer = synth.make_layer(shape, tokens, alpha, rep, weights=whost)
    b = L.from_layer(layer, theta=theta, weights=device_weights(wdev), pack=PACK, plan=plan)
    L.forward(b)
    torch.cuda.synchronize()
    ids = b.topk_ids.cpu().numpy()
    t_hat = b.t_hat.cpu().numpy().tolist()
    if force is not None:  # a given configuration instead of the device's choice
        b.variant.fill_(force)
        L.forward(b, forced_variant=True)
        torch.cuda.synchronize()
    chosen = int(b.variant.item())
    w = work(layer, ids)
    g_chosen = T.graph(lambda: L.forward(b, forced_variant=force is not None))
    t_chosen = stats(T.time_graph(g_chosen, reps, warmup))
    res = dict(tokens=tokens, alpha=alpha, expert_begin=layer.expert_begin, S=w["S"], A=w["A"],
               eff_exp=round(w["eff_exp"], 3),
               ddist_x=round(layer.shape.local_experts / w["eff_exp"], 2) if w["eff_exp"] > 0 else None,
               variant=chosen, us=round(t_chosen["median"], 3),
               us_p10=round(t_chosen["p10"], 3), us_p90=round(t_chosen["p90"], 3),
               roof_us=round(roof_us(w), 3),
               hbm_frac=round(w["layer_bytes"] / (t_chosen["median"] * 1e-6) / HBM_PEAK, 4),
               mfma_frac=round(w["mfma_s"] / (t_chosen["median"] * 1e-6), 4),
               counts=[int(c) for c in w["counts"]], t_hat=[round(x, 4) for x in t_hat])
    res["binding"] = "hbm" if w["layer_bytes"] / HBM_PEAK >= w["mfma_s"] else "mfma"
    res["roof_frac"] = round(res["roof_us"] / res["us"], 4)
    if force is None and plan == "grouped" and L.choose_plan(b.p, "auto") == "fused":
        # the fused small-batch plan on the same load (the chooser's labels below
        # stay on the grouped plan)
        L.use_plan(b, "fused")
        g_fused = T.graph(lambda: L.forward(b))
        res["fused_us"] = round(stats(T.time_graph(g_fused, reps, warmup))["median"], 3)
        L.use_plan(b, "grouped")
        del g_fused
    if exhaustive:
        g_forced = T.graph(lambda: L.forward(b, forced_variant=True))
        per_v = []
        for v in range(V):
            b.variant.fill_(v)
            torch.cuda.synchronize()
            per_v.append(stats(T.time_graph(g_forced, reps, warmup))["median"])
        best = int(np.argmin(per_v))
        res["us_per_variant"] = [round(x, 3) for x in per_v]
        res["best_variant"] = best
        res["gap_to_exhaustive"] = round(per_v[chosen] / per_v[best] - 1.0, 4)
        b.variant.fill_(chosen)
        del g_forced
    del g_chosen
    return res, layer, b, w


def kernel_segments(torch, L, b, T, reps, forced=False):
    """Per-call HIP-event timing, eager, each step cold.  Every call is launched on
    one dedicated stream and its events are recorded on that same stream, so each
    pair brackets exactly that call's kernels."""
    names = ["route_select_align", "grouped_gate_up", "grouped_down", "combine"]
    fns = [lambda b_, stream: L.route_select_align(b_, stream, forced_variant=forced), L.gate_up,
           L.down, L.combine]
    if b.plan == "fused":
        names = ["route_select_align", "grouped_ffn_fused", "combine_fused"]
        fns = [fns[0], L.ffn_fused, L.combine_fused]
    acc = {n: [] for n in names}
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(reps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(fns))]
        for i, f in enumerate(fns):
            T.flush()
            s.wait_stream(torch.cuda.current_stream())
            evs[2 * i].record(s)
            f(b, stream=s)
            evs[2 * i + 1].record(s)
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i, n in enumerate(names):
            acc[n].append(evs[2 * i].elapsed_time(evs[2 * i + 1]) * 1e3)
    return {n: statistics.fmean(v) for n, v in acc.items()}


def cpu_baseline(np, oracle, layer, sample_tokens, nthreads=None):
    """The CPU oracle as it stands, on a bounded token sample of the same load;
    reported as microseconds per layer scaled by B / sample."""
    n = min(layer.tokens, sample_tokens)
    toks = np.random.default_rng(1234).choice(layer.tokens, n, replace=False).astype(np.int32)
    nthreads = nthreads or oracle.max_threads()
    t0 = time.perf_counter()
    ids, w = oracle.route_topk(layer.logits, layer.shape.top_k)
    oracle.counts(ids, layer.expert_begin, layer.shape.local_experts)
    oracle.align(ids, layer.expert_begin, layer.shape.local_experts, 16)
    t_route = time.perf_counter() - t0
    t1 = time.perf_counter()
    oracle.layer_tokens(layer, ids, w, toks, nthreads)
    t_ffn = time.perf_counter() - t1
    us = (t_route + t_ffn * layer.tokens / n) * 1e6
    return dict(value=round(us, 1), unit="us/layer", cores=nthreads, kind="oracle",
                sample=f"{n} of {layer.tokens} tokens through the expert FFN and combine (scaled "
                       f"x{layer.tokens / n:.2f}); routing, counts and align on the full batch; "
                       f"measured {t_route + t_ffn:.1f} s")


def cpu_one_thread(np, oracle, synth):
    """The oracle on one thread for the tiny workload (whole layer, 64 tokens) and
    the Qwen3-30B-A3B-shaped one (B = 128, alpha = 1, 32-token sample scaled)."""
    out = {}
    for name, shape, B, alpha, sample in (("tiny_b64", "tiny", 64, None, 64),
                                          ("qwen3_b128_a1", "qwen3", 128, 1.0, 32)):
        layer = synth.make_layer(shape, B, alpha, 0)
        r = cpu_baseline(np, oracle, layer, sample, nthreads=1)
        out[name] = dict(us=r["value"], sample=f"{min(B, sample)} of {B} tokens")
    return out


# the scoring grid of the blueprint: every power-of-two token count of each
# workload's range and reps 0..7 (used with --density full)
DENSE = {
    "mixtral": dict(tokens=[1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048],
                    alphas=[0.1, 1.0, 10.0, 100.0]),
    "qwen3": dict(tokens=[1 << i for i in range(13)], alphas=[0.05, 0.3, 1.0, 10.0]),
    "dsv3_share": dict(tokens=[1 << i for i in range(9)], alphas=[0.1, 1.0, 10.0]),
    "kimi_share": dict(tokens=[8 << i for i in range(10)], alphas=[0.05]),
}


def ranks(xs):
    """Ranks 1..n with ties averaged."""
    order = sorted(range(len(xs)), key=lambda i: xs[i])
    r = [0.0] * len(xs)
    i = 0
    while i < len(order):
        j = i
        while j + 1 < len(order) and xs[order[j + 1]] == xs[order[i]]:
            j += 1
        for q in range(i, j + 1):
            r[order[q]] = (i + j) / 2 + 1
        i = j + 1
    return r


def spearman(a, b):
    """Spearman rank correlation (Pearson correlation of the tie-averaged ranks)."""
    ra, rb = ranks(a), ranks(b)
    ma, mb = statistics.fmean(ra), statistics.fmean(rb)
    num = sum((x - ma) * (y - mb) for x, y in zip(ra, rb))
    den = math.sqrt(sum((x - ma) ** 2 for x in ra) * sum((y - mb) ** 2 for y in rb))
    return num / den if den > 0 else None


# a served-menu prediction is below this; configurations outside the menu carry a
# prediction of 1e30 (the fitted theta's off-menu constant)
OFF_MENU = 1.0e29


def sweep_shape(torch, np, synth, L, T, shape, V, reps, density="grid"):
    base = shape.split("_fp8")[0].removesuffix("_sh")
    sw = DENSE[base] if density == "full" else SWEEPS[shape]
    rep_list = range(8) if density == "full" else range(1)
    wdev = synth.make_weights_device(shape)
    theta, theta_src = load_theta(shape, V)
    nowts = {"w1": None, "w3": None, "w2": None, "s1": None, "s3": None, "s2": None}
    out = []
    for tok in sw["tokens"]:
        for a in sw["alphas"]:
            for rep in rep_list:
                tb = 8 * tok if shape.startswith("dsv3_share") else tok
                r, *_ = run_point(torch, np, synth, L, T, shape, tb, a, wdev, nowts, theta, V, reps,
                                  3, exhaustive=True, rep=rep)
                r["rep"] = rep
                if shape.startswith("dsv3_share"):
                    r["tokens_per_gpu"] = tok
                log(f"[bench] {shape} B={tb} alpha={a} rep={rep}: {r['us']:.1f} us, "
                    f"v={r['variant']} best={r['best_variant']} "
                    f"gap={r['gap_to_exhaustive']:.3f} roof={r['roof_frac']:.3f} ({r['binding']}) "
                    f"per-variant {r['us_per_variant']}")
                out.append(r)
    del wdev
    torch.cuda.empty_cache()
    gaps = [max(r["gap_to_exhaustive"], 0.0) for r in out]
    # rank agreement of the model's predictions with the measured times (RaMP
    # section 3.1 reports it): per load over the compiled configurations, and pooled
    # over every (load, configuration) pair
    # served-menu configurations only: the others carry the off-menu prediction
    menu = [v for v in range(V) if out and out[0]["t_hat"][v] < OFF_MENU]
    per_load = [spearman([r["t_hat"][v] for v in menu], [r["us_per_variant"][v] for v in menu])
                for r in out]
    per_load = [x for x in per_load if x is not None]
    pooled = spearman([r["t_hat"][v] for r in out for v in menu],
                      [r["us_per_variant"][v] for r in out for v in menu])
    # gap to the best served-menu configuration: the chooser's own error, apart
    # from what the menu leaves out
    mgaps = [max(r["us_per_variant"][r["variant"]] / min(r["us_per_variant"][v] for v in menu) - 1.0, 0.0)
             for r in out]
    worst = max(out, key=lambda r: r["gap_to_exhaustive"])
    chooser = dict(geomean_gap=round(math.exp(statistics.fmean([math.log1p(x) for x in gaps])) - 1, 4),
                   worst_gap=round(max(gaps), 4),
                   worst_load=dict(tokens=worst["tokens"], alpha=worst["alpha"], rep=worst["rep"]),
                   within_5pct=round(sum(g_ <= 0.05 for g_ in gaps) / len(gaps), 3),
                   menu=menu,
                   geomean_gap_in_menu=round(math.exp(statistics.fmean([math.log1p(x) for x in mgaps])) - 1, 4),
                   spearman_rho=round(statistics.fmean(per_load), 4) if per_load else None,
                   spearman_rho_pooled=round(pooled, 4) if pooled is not None else None,
                   theta=theta_src or "untuned default (th1 = 1: fewest waves)")
    res = dict(points=out, chooser=chooser, density=density)
    loads = fit_loads(shape)
    if loads:
        # the pages' simpler policies, fit on the cost model's fit loads and scored
        # on the same exhaustive labels
        from routing_aware_grouped_amd import choosers
        import routing_aware_grouped_amd as moe
        block_m = [moe.moe_variant_info(v)[0] for v in range(V)]
        res["alternatives"] = choosers.compare(loads, out, block_m)
        for name, g in res["alternatives"].items():
            log(f"[bench] {shape} chooser {name}: gap {g['geomean_gap']:.4f} "
                f"worst {g['worst_gap']:.4f} (cost model {chooser['geomean_gap']:.4f})")
    return res


# ----------------------------------------------------------------------- main --
WORKLOAD_NAMES = {
    "mixtral": "Mixtral-8x7B-shaped fused MoE layer",
    "qwen3": "Qwen3-30B-A3B-shaped fused MoE layer",
    "dsv3_share": "DeepSeek-V3-shaped one-GPU expert share",
    "kimi_share": "Kimi-K2-shaped one-GPU expert share",
}


def geomean(xs):
    xs = [x for x in xs if x and x > 0]
    return round(math.exp(statistics.fmean([math.log(x) for x in xs])), 4) if xs else None


def sweep_summary(res):
    """One short record per workload: points, the binding-roofline fraction of the
    chosen configuration (geomean, min, max) and the chooser's gap to exhaustive."""
    pts = res["points"]
    fr = [p["roof_frac"] for p in pts]
    out = dict(n=len(pts), roof_geo=geomean(fr), roof_min=round(min(fr), 4),
               roof_max=round(max(fr), 4), gap_geo=res["chooser"]["geomean_gap"],
               gap_worst=res["chooser"]["worst_gap"], within5=res["chooser"]["within_5pct"])
    rho = res["chooser"].get("spearman_rho")
    if rho is not None:
        out["rho"] = rho
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--shape", default="mixtral", choices=sorted(SWEEPS))
    ap.add_argument("--tokens", type=int, default=2048)
    ap.add_argument("--alpha", type=float, default=1.0)
    ap.add_argument("--sweep", default="mixtral,qwen3,dsv3_share,kimi_share,dsv3_share_fp8a,"
                                       "kimi_share_fp8a,dsv3_share_fp8ah,kimi_share_fp8ah,"
                                       "dsv3_share_sh",
                    help="comma-separated workloads to sweep ('' for none)")
    ap.add_argument("--sweep-reps", type=int, default=15)
    ap.add_argument("--density", default="grid", choices=["grid", "full"],
                    help="grid: the token counts and alphas of SWEEPS, rep 0; full: every "
                         "power-of-two token count and reps 0..7")
    ap.add_argument("--cpu", type=int, default=1, help="1: time the CPU oracle baseline")
    ap.add_argument("--cpu-sample", type=int, default=256)
    ap.add_argument("--exhaustive", type=int, default=1,
                    help="1: also time every configuration at the headline point")
    ap.add_argument("--force-variant", type=int, default=None,
                    help="run the headline in this configuration instead of the device's choice "
                         "(for profiling one configuration)")
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "bench_full.json"),
                    help="file for the full result (every sweep point); '' for none")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the "
                         "known-size kernel that scales HBM byte counters) and exit")
    ap.add_argument("--pack", type=int, default=1,
                    help="1: bf16 layers give the wide configuration its packed weight copy "
                         "(moe_pack_wide, written once per weight set before timing); 0: row-major")
    ap.add_argument("--plan", default="grouped", choices=["grouped", "fused"],
                    help="the headline point's plan: the grouped FFN, or the fused small-batch "
                         "plan (one FFN launch; its roofline line is that launch's)")
    ap.add_argument("--calibrate-gemm", type=int, default=0, metavar="N",
                    help="only time a dense bf16 N x N x N torch.mm (the vendor GEMM library on the "
                         "same GPU: a practical reference for the MFMA-bound rate) and exit")
    args = ap.parse_args()
    global PACK, PLAN
    PACK = None if args.pack else False
    PLAN = args.plan

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the layer runs on one GPU "
              "(one GPU's expert share at its real size); no multi-GPU figure is produced.",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for i in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            dst.copy_(src)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            print(f"copy {args.calibrate_copy} MiB: read {n} B + write {n} B in {dt * 1e6:.1f} us "
                  f"({2 * n / dt / 1e9:.1f} GB/s wall)", flush=True)
        return

    if args.calibrate_gemm:
        import torch
        n = args.calibrate_gemm
        a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        c = torch.mm(a, b)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(4):
            torch.cuda.synchronize()
            e0.record()
            for _ in range(10):
                torch.mm(a, b, out=c)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / 10
            tf = 2.0 * n ** 3 / us / 1e6
            print(f"bf16 GEMM {n}^3: {us:.1f} us per call, {tf:.1f} TFLOP/s "
                  f"({tf / (MFMA_BF16_PEAK / 1e12):.3f} of the dense bf16 peak)", flush=True)
        return

    import numpy as np
    import torch

    import oracle
    import synth
    import routing_aware_grouped_amd as moe
    from routing_aware_grouped_amd import layer as L

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    V = moe.moe_num_variants()
    T = Timer(torch)
    log(f"[bench] generating {args.shape} weights on the GPU")
    wdev = synth.make_weights_device(args.shape)
    whost = synth.host_weights(wdev) if args.cpu else {k: None for k in wdev}
    theta, theta_src = load_theta(args.shape, V)

    # ---- headline point: K timed steps ------------------------------------------------
    log(f"[bench] headline {args.shape} B={args.tokens} alpha={args.alpha}")
    head, layer, b, w = run_point(torch, np, synth, L, T, args.shape, args.tokens, args.alpha, wdev,
                                  whost, theta, V, max(10, args.steps // 2), 3,
                                  exhaustive=bool(args.exhaustive), force=args.force_variant,
                                  plan=PLAN)
    g = T.graph(lambda: L.forward(b, forced_variant=args.force_variant is not None))
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    steps_us = T.time_graph(g, args.steps, args.warmup)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    st = stats(steps_us)
    seg = kernel_segments(torch, L, b, T, max(10, args.steps), forced=args.force_variant is not None)
    log(f"[bench] headline median {st['median']:.1f} us; segments " +
        ", ".join(f"{k} {v:.1f}" for k, v in seg.items()))

    # dominant kernel: the grouped gate/up launch (2/3 of the weight bytes and FLOPs)
    if PLAN == "fused":  # the fused plan's one FFN launch
        seg["grouped_gate_up"] = seg["grouped_ffn_fused"]
        w = dict(w, gate_up_bytes=w["ffn_bytes"], gate_up_flops=w["flops"],
                 gate_up_peak=MFMA_BF16_PEAK)
    t_gu = seg["grouped_gate_up"] * 1e-6
    gu_peak = w["gate_up_peak"]  # the gate/up GEMM's own dtype: bf16, or fp8 x fp8
    bound = "hbm" if w["gate_up_bytes"] / HBM_PEAK >= w["gate_up_flops"] / gu_peak else "mfma"
    if bound == "hbm":
        achieved, peak, unit = w["gate_up_bytes"] / t_gu / 1e9, HBM_PEAK / 1e9, "GB/s"
    else:
        achieved, peak, unit = w["gate_up_flops"] / t_gu / 1e12, gu_peak / 1e12, "TFLOP/s"
    wl_key = f"{args.shape}:B{args.tokens}:a{args.alpha:g}:v{head['variant']}"
    # the chosen configuration's class: one workgroup per CU runs in the wide kernel
    gu_kernel = "ffn_wide_kernel" if moe.moe_variant_info(head["variant"])[9] == 1 else "ffn_kernel"
    kname = (f"{gu_kernel}<1,*> (moe_grouped_gate_up)" if PLAN == "grouped"
             else "fused_ffn_kernel (moe_grouped_ffn_fused)")
    roofline = dict(bound=bound, achieved=round(achieved, 2), peak=round(peak, 1), unit=unit,
                    frac=round(achieved / peak, 4),
                    traffic=measured_traffic(wl_key) if PLAN == "grouped" else None,
                    kernel=kname,
                    alg_bytes=int(w["gate_up_bytes"]), alg_flops=int(w["gate_up_flops"]),
                    avg_launch_us=round(seg["grouped_gate_up"], 3))

    # ---- CPU oracle baseline ------------------------------------------------------------
    cpu = cpu1 = None
    if args.cpu:
        log(f"[bench] timing the CPU oracle on a {args.cpu_sample}-token sample")
        cpu = cpu_baseline(np, oracle, layer, args.cpu_sample)
        log(f"[bench] cpu_baseline {cpu}")
        cpu1 = cpu_one_thread(np, oracle, synth)
        log(f"[bench] oracle on one thread: {cpu1}")
    del whost

    # ---- sweeps -------------------------------------------------------------------------
    sweeps = {}
    shapes = [s for s in args.sweep.split(",") if s]
    if shapes:
        del b, g
        del wdev
        torch.cuda.empty_cache()
    for shp in shapes:
        log(f"[bench] sweep {shp}")
        sweeps[shp] = sweep_shape(torch, np, synth, L, T, shp, V, args.sweep_reps,
                                   args.density)

    sh = layer.shape
    head_layer = dict(variant=head["variant"], best_variant=head.get("best_variant"),
                      gap_to_exhaustive=head.get("gap_to_exhaustive"),
                      us_per_variant=head.get("us_per_variant"), roof_us=head["roof_us"],
                      roof_frac=round(head["roof_us"] / st["median"], 4), binding=head["binding"],
                      hbm_frac=round(w["layer_bytes"] / (st["median"] * 1e-6) / HBM_PEAK, 4),
                      mfma_frac=round(w["mfma_s"] / (st["median"] * 1e-6), 4),
                      segments_us={k: round(v, 1) for k, v in seg.items()},
                      p10=round(st["p10"], 1), p90=round(st["p90"], 1),
                      timed_wall_s=round(t_wall, 3))
    wname = WORKLOAD_NAMES.get(sh.name.split("_fp8")[0].removesuffix("_sh"), sh.name)
    out = {
        "metric": METRIC,
        "value": round(st["median"], 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(st["mean"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {synth.F32: "f32", synth.BF16: "bf16"}[sh.act_dtype],
        "data": "synthetic (Dirichlet-skewed Gumbel-top-k routing, N(0,0.02) activations/weights)",
        "config": {"workload": f"{wname}, B={args.tokens}, alpha={args.alpha:g}",
                   "tokens": args.tokens, "alpha": args.alpha, "hidden": sh.hidden,
                   "inter": sh.inter, "experts": sh.num_experts, "top_k": sh.top_k,
                   "weights": synth.DTYPE_NAMES[sh.weight_dtype], "parallelism": "single GPU",
                   "plan": PLAN,
                   "timing": "HIP graph replay, cold L2/Infinity Cache, hipEvent per step, median"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "layer": head_layer,
    }
    full = dict(out, cpu_one_thread=cpu1, theta=theta_src or "untuned default (th1 = 1)",
                sweeps=sweeps, roofline=dict(roofline, traffic_key=wl_key,
                                             kernel_source_sha=kernel_source_hash()))
    if args.out:
        os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
        with open(args.out, "w") as f:
            json.dump(full, f)
            f.write("\n")
        log(f"[bench] full result (every sweep point) written to {args.out}")
    # the last stdout line: compact (a few kB), one summary record per swept workload
    out["sweep_summary"] = {k: sweep_summary(v) for k, v in sweeps.items()}
    if cpu1:
        out["cpu_one_thread_us"] = {k: v["us"] for k, v in cpu1.items()}
    line = json.dumps(out, separators=(",", ":"))
    print(line, flush=True)


if __name__ == "__main__":
    main()
