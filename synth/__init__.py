"""Seeded synthetic inputs for the fused-MoE layer (shared by the tests, the oracle
runs and the benchmark).

This module only *creates inputs*: router logits, activations, expert weights and
their fp8 block quantisation.  It holds none of the layer's own arithmetic (no
top-k, no counting, no sorting, no GEMM), so that the oracle and the GPU path
can both consume it without sharing any step of the method.

Routing skew follows the symmetric Dirichlet model of "Decoding the Skew"
(arXiv 2607.23099, section II-D, Eq. 1): one share vector p ~ Dir(alpha * 1_E)
is drawn per batch and every token's logits are log(p_e) + Gumbel(0, 1), so the
k largest logits of a token are k distinct experts drawn without replacement in
proportion to p (the Gumbel-top-k construction).  alpha -> infinity gives
near-uniform routing and alpha -> 0 concentrates the batch on few experts.
Activations and weights are N(0, 0.02) as the tiny fp32 workload states; the
same distribution is used for the larger shapes, whose pages do not state one.
fp8 weights are OCP E4M3FN with one fp32 scale per 128x128 block of each
(out, in) weight matrix, w = q * s, quantised as s = amax(block)/448 and
q = round-to-nearest-even(W / s) (the block-scaled FP8 recipe that RaMP, section
3.3, attributes to DeepSeek-V3).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

F32, BF16, FP8 = 0, 1, 2  # dtype codes used throughout (match the C ABI enum)
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8: "fp8_e4m3"}


@dataclasses.dataclass(frozen=True)
class Shape:
    """One layer geometry: hidden H, expert intermediate I, E global experts,
    E_loc local experts starting at e0 (chosen per batch for EP shares), top-k."""
    name: str
    hidden: int
    inter: int
    num_experts: int
    local_experts: int
    top_k: int
    act_dtype: int
    weight_dtype: int
    out_dtype: int
    logits: str  # "normal" (tiny) or "dirichlet"
    act_quant: int = 0  # FP8 E4M3 activations: 1 in the gate/up GEMM, 2 in both GEMMs
    shared: int = 0     # shared experts, stored after the local experts' weights


SHAPES = {
    "tiny": Shape("tiny", 128, 256, 8, 8, 2, F32, F32, F32, "normal"),
    "mixtral": Shape("mixtral", 4096, 14336, 8, 8, 2, BF16, BF16, BF16, "dirichlet"),
    "qwen3": Shape("qwen3", 2048, 768, 128, 128, 8, BF16, BF16, BF16, "dirichlet"),
    "dsv3_share": Shape("dsv3_share", 7168, 2048, 256, 32, 8, BF16, FP8, BF16, "dirichlet"),
    "kimi_share": Shape("kimi_share", 7168, 2048, 384, 48, 8, BF16, FP8, BF16, "dirichlet"),
    # the same two expert shares with FP8 activations in the gate/up GEMM (same
    # seeds, so the loads are identical to the bf16-activation ones)
    "dsv3_share_fp8a": Shape("dsv3_share_fp8a", 7168, 2048, 256, 32, 8, BF16, FP8, BF16,
                             "dirichlet", 1),
    "kimi_share_fp8a": Shape("kimi_share_fp8a", 7168, 2048, 384, 48, 8, BF16, FP8, BF16,
                             "dirichlet", 1),
    # a small fp8 layer for parity at sizes the oracle runs in seconds: a ragged
    # number of 128-column groups, so that stages of 256 and 512 are partly empty
    "small_fp8a": Shape("small_fp8a", 384, 256, 8, 8, 2, BF16, FP8, BF16, "dirichlet", 1),
    # FP8 activations in both GEMMs (h quantized before the down projection)
    "dsv3_share_fp8ah": Shape("dsv3_share_fp8ah", 7168, 2048, 256, 32, 8, BF16, FP8, BF16,
                              "dirichlet", 2),
    "kimi_share_fp8ah": Shape("kimi_share_fp8ah", 7168, 2048, 384, 48, 8, BF16, FP8, BF16,
                              "dirichlet", 2),
    "small_fp8ah": Shape("small_fp8ah", 384, 256, 8, 8, 2, BF16, FP8, BF16, "dirichlet", 2),
    # with shared experts (DeepSeek-V3 and Kimi-K2 each have one, of the routed
    # experts' size); the small ones have two, and the tiny one fp32 arithmetic
    "dsv3_share_sh": Shape("dsv3_share_sh", 7168, 2048, 256, 32, 8, BF16, FP8, BF16, "dirichlet",
                           0, 1),
    "kimi_share_sh": Shape("kimi_share_sh", 7168, 2048, 384, 48, 8, BF16, FP8, BF16, "dirichlet",
                           0, 1),
    "small_sh": Shape("small_sh", 384, 256, 8, 8, 2, BF16, FP8, BF16, "dirichlet", 0, 2),
    "tiny_sh": Shape("tiny_sh", 128, 256, 8, 8, 2, F32, F32, F32, "normal", 0, 2),
    "small_sh_fp8ah": Shape("small_sh_fp8ah", 384, 256, 8, 8, 2, BF16, FP8, BF16, "dirichlet", 2,
                            2),
    # bf16 with the shortest reductions the API admits: H = 128 (a gate/up
    # reduction of four 32-deep stages) and I = 384
    "tiny_bf16": Shape("tiny_bf16", 128, 384, 8, 8, 2, BF16, BF16, BF16, "dirichlet"),
    # a small fp8-weight layer with bf16 activations (no activation quantization)
    "small_fp8": Shape("small_fp8", 384, 256, 8, 8, 2, BF16, FP8, BF16, "dirichlet"),
}

CFG_INDEX = {"tiny": 1, "mixtral": 2, "qwen3": 3, "dsv3_share": 4, "kimi_share": 5,
             "dsv3_share_fp8a": 4, "kimi_share_fp8a": 5, "small_fp8a": 6,
             "dsv3_share_fp8ah": 4, "kimi_share_fp8ah": 5, "small_fp8ah": 6,
             "dsv3_share_sh": 4, "kimi_share_sh": 5, "small_sh": 6, "tiny_sh": 1,
             "small_sh_fp8ah": 6, "tiny_bf16": 7, "small_fp8": 6}


def seed_seq(shape: str, tokens: int, alpha: float | None, rep: int) -> np.random.SeedSequence:
    """Deterministic seed of one load: (config, B, round(1000*alpha), rep)."""
    a = 0 if alpha is None else int(round(1000 * alpha))
    return np.random.SeedSequence([CFG_INDEX[shape], tokens, a, rep])


# ----------------------------------------------------------------------------------
# Dirichlet shares and routing logits
# ----------------------------------------------------------------------------------
def log_dirichlet(rng: np.random.Generator, alpha: float, n: int) -> np.ndarray:
    """log p for p ~ Dir(alpha, ..., alpha) over n outcomes, in float64.

    Gamma(alpha) variates are drawn in log space, log G = log G' + log(U)/alpha
    with G' ~ Gamma(alpha + 1), U ~ U(0,1), so that tiny alpha never underflows
    to a zero share (p_i = G_i / sum G)."""
    g1 = rng.standard_gamma(alpha + 1.0, n)
    u = rng.random(n)
    u = np.where(u <= 0.0, np.finfo(np.float64).tiny, u)
    logg = np.log(g1) + np.log(u) / alpha
    m = logg.max()
    return logg - (m + np.log(np.exp(logg - m).sum()))


def dirichlet_shares(rng: np.random.Generator, alpha: float, n: int) -> np.ndarray:
    return np.exp(log_dirichlet(rng, alpha, n))


def gumbel(rng: np.random.Generator, size) -> np.ndarray:
    u = rng.random(size)
    u = np.clip(u, 1e-300, 1.0 - 1e-16)
    return -np.log(-np.log(u))


def routing_logits(shape: Shape, tokens: int, alpha: float | None, rng: np.random.Generator):
    """Router logits f32 [B][E] and the share vector p (None for the tiny shape)."""
    E = shape.num_experts
    if shape.logits == "normal":
        return rng.standard_normal((tokens, E)).astype(np.float32), None
    logp = log_dirichlet(rng, alpha, E)
    lg = logp[None, :] + gumbel(rng, (tokens, E))
    return lg.astype(np.float32), np.exp(logp)


def most_loaded_block(p: np.ndarray | None, shape: Shape) -> int:
    """First expert e0 of the contiguous local block with the largest expected
    share sum(p) - the slowest GPU under expert parallelism sets the layer time.
    Chosen from the sampling distribution p, not from the realised routing."""
    if p is None or shape.local_experts == shape.num_experts:
        return 0
    nb = shape.num_experts // shape.local_experts
    sums = p.reshape(nb, shape.local_experts).sum(axis=1)
    return int(np.argmax(sums)) * shape.local_experts


def eff_exp(counts) -> float:
    """Effective Experts, (sum t_i)^2 / sum t_i^2 ("Decoding the Skew", III-A Eq. 2)."""
    t = np.asarray(counts, dtype=np.float64)
    s2 = float((t * t).sum())
    return float(t.sum() ** 2 / s2) if s2 > 0 else 0.0


def ddist_alpha(x: float, n: int, samples: int = 64, iters: int = 40, seed: int = 0) -> float:
    """ddist:X ("Decoding the Skew", section III-A): the concentration of a
    symmetric Dirichlet over n experts whose shares have mean effective experts
    n / x.  Effective experts grow with alpha, so the search bisects [1e-6, 1e6]
    with the arithmetic midpoint as the page gives it, each step averaging
    eff_exp over `samples` draws of the shares.  x = 1 asks for n, which no draw
    reaches, so the search runs to the top of the range (near-uniform routing)."""
    if not (1.0 <= x <= n):
        raise ValueError("ddist:X needs 1 <= X <= n")
    target = n / x
    rng = np.random.default_rng(seed)
    lo, hi = 1e-6, 1e6
    mid = 0.5 * (lo + hi)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        v = float(np.mean([eff_exp(dirichlet_shares(rng, mid, n)) for _ in range(samples)]))
        if v < target:
            lo = mid
        else:
            hi = mid
    return mid


# ----------------------------------------------------------------------------------
# Tensors and dtype encodings
# ----------------------------------------------------------------------------------
def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_fp8_blocks(w: np.ndarray):
    """w f32 [rows][cols] (both multiples of 128) -> (q uint8 E4M3FN codes, s f32
    [rows/128][cols/128]) with s = amax/448 and q = RNE(w/s) per 128x128 block."""
    rows, cols = w.shape
    assert rows % 128 == 0 and cols % 128 == 0
    t = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32))
    blk = t.reshape(rows // 128, 128, cols // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    scaled = (blk / s[:, None, :, None]).clamp_(-448.0, 448.0)
    q = scaled.reshape(rows, cols).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), s.numpy().astype(np.float32)


@dataclasses.dataclass
class Layer:
    """Host copies of one layer's inputs (numpy).  Dtype-encoded arrays:
    f32 -> float32, bf16 -> uint16 bit patterns, fp8 -> uint8 E4M3FN codes."""
    shape: Shape
    tokens: int
    alpha: float | None
    expert_begin: int
    logits: np.ndarray          # f32 [B][E]
    x: np.ndarray               # [B][H]
    w1: np.ndarray              # [E_loc][I][H]  gate
    w3: np.ndarray              # [E_loc][I][H]  up
    w2: np.ndarray              # [E_loc][H][I]  down
    s1: np.ndarray | None = None  # f32 [E_loc][I/128][H/128]
    s3: np.ndarray | None = None
    s2: np.ndarray | None = None  # f32 [E_loc][H/128][I/128]
    shares: np.ndarray | None = None


def _encode(a32: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return a32.astype(np.float32)
    if dtype == BF16:
        return to_bf16_bits(a32)
    raise ValueError(dtype)


def make_weights(shape: Shape, rng: np.random.Generator, std: float = 0.02):
    """Expert weights for all local experts, generated expert by expert."""
    El, H, I = shape.local_experts + shape.shared, shape.hidden, shape.inter
    wd = shape.weight_dtype
    out = {}
    for name, (r, c) in (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I))):
        if wd == FP8:
            q = np.empty((El, r, c), np.uint8)
            s = np.empty((El, r // 128, c // 128), np.float32)
        else:
            q = np.empty((El, r, c), np.float32 if wd == F32 else np.uint16)
            s = None
        for e in range(El):
            w = (rng.standard_normal((r, c), dtype=np.float32) * np.float32(std))
            if wd == FP8:
                q[e], s[e] = quantize_fp8_blocks(w)
            else:
                q[e] = _encode(w, wd)
        out[name] = q
        out["s" + name[1]] = s
    return out


def make_layer(shape_name: str, tokens: int, alpha: float | None = None, rep: int = 0,
               weights: dict | None = None, x_std: float = 0.02) -> Layer:
    """All inputs of one load.  Pass `weights` to reuse one weight set across loads
    (the weights of a layer do not change between batches)."""
    shape = SHAPES[shape_name]
    ss = seed_seq(shape_name, tokens, alpha, rep)
    r_route, r_x = (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(2))
    logits, p = routing_logits(shape, tokens, alpha, r_route)
    e0 = most_loaded_block(p, shape)
    x = _encode(r_x.standard_normal((tokens, shape.hidden), dtype=np.float32) * np.float32(x_std),
                shape.act_dtype)
    if weights is None:
        weights = make_weights(shape, np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([CFG_INDEX[shape_name], 7777]))))
    return Layer(shape, tokens, alpha, e0, logits, x, weights["w1"], weights["w3"],
                 weights["w2"], weights.get("s1"), weights.get("s3"), weights.get("s2"), p)


def layer_weights_for(shape_name: str) -> dict:
    shape = SHAPES[shape_name]
    return make_weights(shape, np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([CFG_INDEX[shape_name], 7777]))))


# ----------------------------------------------------------------------------------
# On-device weight generation for the full-size shapes (seeded torch generator).
# Same distribution and fp8 recipe as make_weights; a different stream of numbers.
# ----------------------------------------------------------------------------------
def make_weights_device(shape_name: str, device="cuda", std: float = 0.02, seed: int | None = None):
    """Dict w1, w3, w2 (+ s1, s3, s2 for fp8) of torch tensors on `device`, dtype-
    encoded (float32 / bfloat16 / float8_e4m3fn)."""
    shape = SHAPES[shape_name]
    El, H, I = shape.local_experts + shape.shared, shape.hidden, shape.inter
    wd = shape.weight_dtype
    g = torch.Generator(device=device)
    g.manual_seed(CFG_INDEX[shape_name] * 1_000_003 + 7777 if seed is None else seed)
    out = {}
    tdt = {F32: torch.float32, BF16: torch.bfloat16, FP8: torch.float8_e4m3fn}[wd]
    for name, (r, c) in (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I))):
        q = torch.empty((El, r, c), dtype=tdt, device=device)
        s = torch.empty((El, r // 128, c // 128), dtype=torch.float32, device=device) if wd == FP8 else None
        for e in range(El):
            w = torch.randn((r, c), generator=g, device=device, dtype=torch.float32) * std
            if wd == FP8:
                blk = w.reshape(r // 128, 128, c // 128, 128)
                amax = blk.abs().amax(dim=(1, 3))
                sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
                q[e] = (blk / sc[:, None, :, None]).clamp_(-448.0, 448.0).reshape(r, c).to(tdt)
                s[e] = sc
            else:
                q[e] = w.to(tdt)
        out[name] = q
        out["s" + name[1]] = s
    return out


def host_weights(wdev: dict) -> dict:
    """Device weights -> the numpy encodings make_weights returns."""
    out = {}
    for k, v in wdev.items():
        if v is None:
            out[k] = None
            continue
        t = v.detach().cpu()
        if t.dtype == torch.bfloat16:
            out[k] = t.view(torch.int16).numpy().view(np.uint16)
        elif t.dtype == torch.float8_e4m3fn:
            out[k] = t.view(torch.uint8).numpy()
        else:
            out[k] = t.numpy()
    return out
