"""CPU oracle of the routing-aware fused-MoE layer (numpy front end over a plain C
library, moe_oracle.c, built with gcc).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing here is imported by the GPU
library, and this package imports nothing from it.  Each function names the
step of the method it follows; the arithmetic itself lives in moe_oracle.c in
fp64 (fp32 for the cost model, whose argmin both sides must take in the same
precision).

Pins (see tests/test_oracle_pins.py): brute force over k-subsets for top-k,
numpy stable argsort and bincount, the worked 16-expert tile example of RaMP
section 2.3, a one-hot router reducing to a dense FFN, identical experts
reducing to a dense FFN, the fp8 decoder on all 256 codes against
torch.float8_e4m3fn, and exact-rational checks of the fp32 cost chain.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8 = 0, 1, 2
F64 = 3  # fp64 activations: the dequantized x of the FP8 activation path


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc (-O2, OpenMP, strict IEEE: no fast-math, no
    FMA contraction, so that every fp64 expression is evaluated as written and the
    fp32 cost chain uses exactly the fmaf calls it names)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        L.oracle_route_topk.argtypes = [i32, i32, i32, i32, P, P, P]
        L.oracle_counts.argtypes = [i32, i32, i32, i32, P, P]
        L.oracle_counts.restype = None
        L.oracle_select.argtypes = [i32, P, i32, P, P, P, P, P, P, P, P]
        L.oracle_align.argtypes = [i32, i32, i32, i32, P, i32, P, i64, P, P, P]
        L.oracle_align.restype = i64
        L.oracle_ffn_slots.argtypes = [i32, i32, P, i32, P, P, P, i32, P, P, P, i32, P, P, P, i32,
                                       i32]
        L.oracle_layer_tokens.argtypes = [i32, i32, i32, i32, i32, P, i32, P, P, P, i32, P, P, P,
                                          P, P, i32, P, P, i32, i32, i32]
        L.oracle_decode_fp8.argtypes = [P, i64, P]
        L.oracle_decode_fp8.restype = None
        L.oracle_decode_bf16.argtypes = [P, i64, P]
        L.oracle_decode_bf16.restype = None
        L.oracle_quant_act_e4m3.argtypes = [i32, i32, P, P, P]
        L.oracle_e4m3_round.argtypes = [P, i64, P]
        L.oracle_max_threads.argtypes = []
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def max_threads() -> int:
    return int(lib().oracle_max_threads())


# ------------------------------------------------------------------ O1 - O4 ----
def route_topk(logits: np.ndarray, k: int, renormalize: bool = True):
    """O1: ordered top-k expert ids (int32 [B][k]) and fp64 weights [B][k]."""
    lg = _c(logits, np.float32)
    B, E = lg.shape
    ids = np.empty((B, k), np.int32)
    w = np.empty((B, k), np.float64)
    rc = lib().oracle_route_topk(B, E, k, int(bool(renormalize)), _p(lg), _p(ids), _p(w))
    if rc != 0:
        raise ValueError(f"oracle_route_topk rc={rc}")
    return ids, w


def counts(ids: np.ndarray, e0: int, E_loc: int) -> np.ndarray:
    """O2: tokens per local expert, int32 [E_loc]."""
    ids = _c(ids, np.int32)
    B, k = ids.shape
    out = np.empty(E_loc, np.int32)
    lib().oracle_counts(B, k, e0, E_loc, _p(ids), _p(out))
    return out


def select(counts_: np.ndarray, b, q1, q2, S1, S2, theta: np.ndarray):
    """O3: (chosen index, t_hat f32 [V], features int32 [V][3] = W, T, A)."""
    cnt = _c(counts_, np.int32)
    V = len(b)
    arr = lambda v: _c(np.broadcast_to(np.asarray(v), (V,)), np.int32)  # noqa: E731
    b_, q1_, q2_, S1_, S2_ = arr(b), arr(q1), arr(q2), arr(S1), arr(S2)
    th = _c(theta, np.float32).reshape(V, 4)
    t_hat = np.empty(V, np.float32)
    feat = np.empty((V, 3), np.int32)
    v = lib().oracle_select(len(cnt), _p(cnt), V, _p(b_), _p(q1_), _p(q2_), _p(S1_), _p(S2_),
                            _p(th), _p(t_hat), _p(feat))
    if v < 0:
        raise ValueError("oracle_select: invalid input")
    return int(v), t_hat, feat


def align(ids: np.ndarray, e0: int, E_loc: int, b: int):
    """O4: (sorted_slots [R], block_expert [R/b], num_blocks, slot_pos [B*k])."""
    ids = _c(ids, np.int32)
    B, k = ids.shape
    cap = B * k + E_loc * (b - 1) + 1
    ss = np.empty(cap, np.int32)
    be = np.empty(cap // b + 1, np.int32)
    nb = np.zeros(1, np.int32)
    sp = np.empty(B * k, np.int32)
    R = lib().oracle_align(B, k, e0, E_loc, _p(ids), b, _p(ss), cap, _p(be), _p(nb), _p(sp))
    if R < 0:
        raise ValueError("oracle_align: capacity")
    return ss[:R].copy(), be[: nb[0]].copy(), int(nb[0]), sp


# ------------------------------------------------------------------------ Q ----
def quant_act_e4m3(x_bits: np.ndarray):
    """Q: bf16 activations (uint16 bits [B][H]) -> (E4M3FN codes uint8 [B][H],
    fp32 scales [B][H/128]), one scale per token and 128-column group."""
    x = _c(x_bits, np.uint16)
    B, H = x.shape
    q = np.empty((B, H), np.uint8)
    s = np.empty((B, H // 128), np.float32)
    if lib().oracle_quant_act_e4m3(B, H, _p(x), _p(q), _p(s)) != 0:
        raise ValueError("oracle_quant_act_e4m3: H must be a multiple of 128")
    return q, s


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """The rounding step of Q alone: nearest E4M3FN codes of fp32 values, |v| <= 448."""
    a = _c(v, np.float32).ravel()
    q = np.empty(a.size, np.uint8)
    if lib().oracle_e4m3_round(_p(a), a.size, _p(q)) != 0:
        raise ValueError("e4m3_round: |v| must be <= 448")
    return q.reshape(np.shape(v))


def dequant_act(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """x = q * s in fp64 (exact), per 128-column group."""
    B, H = q.shape
    return decode_fp8(q) * np.repeat(np.asarray(s, np.float64), 128, axis=1)[:, :H]


def _h_quant(layer) -> int:
    """1 when the layer also quantizes h before the down projection (act_quant 2)."""
    return int(getattr(layer.shape, "act_quant", 0) == 2)


def _act_args(layer, tokens: np.ndarray):
    """The activation rows the FFN uses for `tokens`: (buffer, dtype, token
    indices into it).  With the FP8 activation path these are the dequantized
    rows of Q, computed for the listed tokens only (Q is per token)."""
    xdt = layer.shape.act_dtype
    if getattr(layer.shape, "act_quant", 0):
        toks = np.asarray(tokens, np.int64)
        q, s = quant_act_e4m3(np.asarray(layer.x)[toks])
        return _c(dequant_act(q, s), np.float64), F64, np.arange(len(toks), dtype=np.int32)
    return _c(layer.x, np.float32 if xdt == F32 else np.uint16), xdt, _c(tokens, np.int32)


# ------------------------------------------------------------------ O5 - O6 ----
def _weights_args(layer):
    wd = layer.shape.weight_dtype
    conv = {F32: np.float32, BF16: np.uint16, FP8: np.uint8}[wd]
    w1, w3, w2 = (_c(a, conv) for a in (layer.w1, layer.w3, layer.w2))
    s1, s3, s2 = ((None if s is None else _c(s, np.float32)) for s in (layer.s1, layer.s3, layer.s2))
    return wd, w1, w3, w2, s1, s3, s2


def ffn_slots(layer, tok: np.ndarray, exp_local: np.ndarray, nthreads: int | None = None):
    """O5: fp64 expert outputs [n][H] for (token, local expert) pairs."""
    H, I = layer.shape.hidden, layer.shape.inter
    x, xdt, tok = _act_args(layer, tok)
    wd, w1, w3, w2, s1, s3, s2 = _weights_args(layer)
    el = _c(exp_local, np.int32)
    y = np.empty((len(tok), H), np.float64)
    rc = lib().oracle_ffn_slots(H, I, _p(x), xdt, _p(w1), _p(w3), _p(w2), wd, _p(s1), _p(s3),
                                _p(s2), len(tok), _p(tok), _p(el), _p(y),
                                nthreads or max_threads(), _h_quant(layer))
    if rc != 0:
        raise RuntimeError(f"oracle_ffn_slots rc={rc}")
    return y


def layer_tokens(layer, ids: np.ndarray, w: np.ndarray, tokens: np.ndarray,
                 nthreads: int | None = None):
    """O5 + O6 for the listed tokens: fp64 Y rows [len(tokens)][H] (with the shared
    experts' lanes when the shape has them)."""
    H, I, k = layer.shape.hidden, layer.shape.inter, layer.shape.top_k
    if getattr(layer.shape, "act_quant", 0):
        # the FFN sees the listed tokens' dequantized rows; ids/w follow them
        sel = np.asarray(tokens, np.int64)
        x, xdt, toks = _act_args(layer, sel)
        ids = _c(np.asarray(ids)[sel], np.int32)
        w = _c(np.asarray(w)[sel], np.float64)
    else:
        x, xdt, toks = _act_args(layer, tokens)
        ids = _c(ids, np.int32)
        w = _c(w, np.float64)
    wd, w1, w3, w2, s1, s3, s2 = _weights_args(layer)
    Y = np.empty((len(toks), H), np.float64)
    rc = lib().oracle_layer_tokens(H, I, k, layer.expert_begin, layer.shape.local_experts,
                                   _p(x), xdt, _p(w1), _p(w3), _p(w2), wd, _p(s1), _p(s3),
                                   _p(s2), _p(ids), _p(w), len(toks), _p(toks), _p(Y),
                                   nthreads or max_threads(), _h_quant(layer),
                                   int(getattr(layer.shape, "shared", 0)))
    if rc != 0:
        raise RuntimeError(f"oracle_layer_tokens rc={rc}")
    return Y


def decode_fp8(codes: np.ndarray) -> np.ndarray:
    c = _c(codes, np.uint8).ravel()
    out = np.empty(c.size, np.float64)
    lib().oracle_decode_fp8(_p(c), c.size, _p(out))
    return out.reshape(np.shape(codes))


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    c = _c(bits, np.uint16).ravel()
    out = np.empty(c.size, np.float64)
    lib().oracle_decode_bf16(_p(c), c.size, _p(out))
    return out.reshape(np.shape(bits))


def full_layer(layer, b: int, token_sample: np.ndarray | None = None,
               nthreads: int | None = None):
    """O1 - O6 in order for one load; the FFN/combine part on all tokens or on a
    sample.  Returns a dict of every intermediate the GPU path also produces."""
    sh = layer.shape
    ids, w = route_topk(layer.logits, sh.top_k)
    cnt = counts(ids, layer.expert_begin, sh.local_experts)
    ss, be, nb, sp = align(ids, layer.expert_begin, sh.local_experts, b)
    toks = np.arange(layer.tokens, dtype=np.int32) if token_sample is None else token_sample
    Y = layer_tokens(layer, ids, w, toks, nthreads)
    return dict(ids=ids, w=w, counts=cnt, sorted_slots=ss, block_expert=be, num_blocks=nb,
                slot_pos=sp, tokens=toks, Y=Y)
