"""Helpers of the GPU parity tests: run the five library calls on one synthetic
load and fetch every output to the host; compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
from routing_aware_grouped_amd import layer as L
from tests import spec

TOL = {synth.F32: 1e-5, synth.BF16: 1e-2, synth.FP8: 5e-2}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def num_cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def theta_forcing(v: int, V: int | None = None) -> torch.Tensor:
    """theta that makes configuration v the unique argmin (t_v = 0, others 1)."""
    V = V or len(spec.MENU)
    th = torch.zeros(V, 4, dtype=torch.float32)
    th[:, 0] = 1.0
    th[v, 0] = 0.0
    return th


def layer_with_weights(shape_name: str, tokens: int, alpha, rep: int = 0, wdev=None, whost=None,
                       x_std: float = 0.02):
    """A synthetic load; weights come from `whost` (numpy) or are generated."""
    if whost is None:
        return synth.make_layer(shape_name, tokens, alpha, rep, x_std=x_std)
    return synth.make_layer(shape_name, tokens, alpha, rep, weights=whost, x_std=x_std)


_WCACHE: dict = {}


def weights(shape_name: str):
    """(device weights, host copies) of a shape, generated once per process."""
    if shape_name not in _WCACHE:
        wdev = synth.make_weights_device(shape_name)
        _WCACHE[shape_name] = (wdev, synth.host_weights(wdev))
    return _WCACHE[shape_name]


def device_weights(layer, wdev=None):
    if wdev is not None:
        return (wdev["w1"], wdev["w3"], wdev["w2"], wdev["s1"], wdev["s3"], wdev["s2"])
    return tuple(None if t is None else t.cuda() for t in L.weight_tensors(layer))


def run(layer, variant: int | None = None, theta=None, wdev=None, renormalize: int = 1,
        pack=None, plan="grouped"):
    """Whole layer on the GPU.  variant=None: the select step chooses with theta;
    else configuration `variant` is forced.  pack: see layer.allocate (default:
    bf16 layers give the wide configuration its packed weight copy).  plan: the
    grouped or the fused plan (layer.choose_plan)."""
    b = L.from_layer(layer, theta=theta if theta is not None else theta_forcing(0),
                     weights=device_weights(layer, wdev), renormalize=renormalize, pack=pack,
                     plan=plan)
    if variant is not None:
        b.variant.fill_(variant)
    torch.cuda.synchronize()
    L.forward(b, forced_variant=variant is not None)
    torch.cuda.synchronize()
    return b


def fetch(b) -> dict:
    nb = int(b.num_blocks.item())
    v = int(b.variant.item())
    bm = spec.MENU[v][0] if 0 <= v < len(spec.MENU) else 1
    R = nb * bm
    y = b.y.float().cpu().numpy()
    return dict(ids=b.topk_ids.cpu().numpy(), w=b.topk_w.cpu().numpy(),
                counts=b.counts.cpu().numpy(), variant=v, num_blocks=nb,
                sorted_slots=b.sorted_slots[:R].cpu().numpy(),
                block_expert=b.block_expert[:nb].cpu().numpy(),
                slot_pos=b.slot_pos.cpu().numpy(), Y=y)


def check_routing(layer, out: dict, renormalize: int = 1):
    sh = layer.shape
    ids, w = oracle.route_topk(layer.logits, sh.top_k, bool(renormalize))
    np.testing.assert_array_equal(out["ids"], ids)
    assert np.abs(out["w"].astype(np.float64) - w).max() <= 1e-6
    cnt = oracle.counts(ids, layer.expert_begin, sh.local_experts)
    np.testing.assert_array_equal(out["counts"], cnt)
    return ids, w


def check_align(layer, out: dict, ids):
    sh = layer.shape
    b = spec.MENU[out["variant"]][0]
    ss, be, nb, sp = oracle.align(ids, layer.expert_begin, sh.local_experts, b)
    assert out["num_blocks"] == nb
    np.testing.assert_array_equal(out["sorted_slots"], ss)
    np.testing.assert_array_equal(out["block_expert"], be)
    np.testing.assert_array_equal(out["slot_pos"], sp)


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    m = float(np.abs(ref).max())
    d = float(np.abs(gpu.astype(np.float64) - ref).max())
    return d / m if m > 0 else d


def check_y(layer, out: dict, ids, w, tokens=None, ref=None):
    toks = np.arange(layer.tokens, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    if ref is None:
        ref = oracle.layer_tokens(layer, ids, w, toks)
    err = rel_err(out["Y"][toks], ref)
    tol = TOL[layer.shape.weight_dtype if layer.shape.weight_dtype == synth.FP8 else layer.shape.act_dtype]
    assert err <= tol, f"max|gpu-ref|/max|ref| = {err:.3g} > {tol}"
    return err, ref
