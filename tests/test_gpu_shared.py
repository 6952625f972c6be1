"""GPU parity with shared experts (GC-MoE section 4): every token goes through each
shared expert with weight 1, fused into the grouped FFN launches (row-blocks after
the routed ones) and added as extra lanes of the combine.  Routing, counts and the
routed permutation bit-exact; Y against the oracle within the dtype tolerance; the
configuration choice, whose features count the shared row-tiles, bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synth
from routing_aware_grouped_amd import layer as L  # noqa: F401  (buffers via gpu_helpers)
from routing_aware_grouped_amd import moe_cost_constants
from tests import gpu_helpers as G
from tests import spec

pytestmark = pytest.mark.gpu
V = len(spec.MENU)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _layer(shape, B, alpha, rep=0):
    if shape.startswith(("small_", "tiny_")):
        return None, synth.make_layer(shape, B, alpha, rep)
    wdev, whost = G.weights(shape)
    return wdev, synth.make_layer(shape, B, alpha, rep, weights=whost)


@pytest.mark.parametrize("shape,B,alpha,sample", [
    ("tiny_sh", 64, None, None), ("tiny_sh", 37, None, None),
    ("small_sh", 1, 1.0, None), ("small_sh", 37, 0.3, None), ("small_sh", 130, 1.0, None),
    ("small_sh_fp8ah", 37, 0.3, None),
    ("dsv3_share_sh", 8, 1.0, None), ("dsv3_share_sh", 96, 0.1, 16),
    ("kimi_share_sh", 1000, 0.05, 16)])
def test_shared_layer_every_variant(shape, B, alpha, sample):
    G.say(f"shared layer {shape} B={B} alpha={alpha}")
    wdev, layer = _layer(shape, B, alpha)
    ids, w = oracle.route_topk(layer.logits, layer.shape.top_k)
    toks = None if sample is None else \
        np.random.default_rng(B).choice(B, sample, replace=False).astype(np.int32)
    ref = None
    for v in range(V):
        out = G.fetch(G.run(layer, variant=v, wdev=wdev))
        G.check_routing(layer, out)
        G.check_align(layer, out, ids)
        if layer.shape.act_quant:  # the oracle of the same method, quantization included
            tk = np.arange(B, dtype=np.int32) if toks is None else toks
            if ref is None:
                ref = oracle.layer_tokens(layer, ids, w, tk)
            err = G.rel_err(out["Y"][tk], ref)
            assert err <= 1e-2, err
        else:
            err, ref = G.check_y(layer, out, ids, w, toks, ref)
        G.say(f"  variant {v}: rel err {err:.3g}")


def test_empty_rank_keeps_shared_lanes():
    """No routed token on this GPU: no routed tiles, and Y is the shared experts'."""
    wdev, layer = _layer("dsv3_share_sh", 16, 1.0)
    layer.logits[:, layer.expert_begin:layer.expert_begin + 32] = -50.0
    ids, w = oracle.route_topk(layer.logits, layer.shape.top_k)
    for v in range(V):
        out = G.fetch(G.run(layer, variant=v, wdev=wdev))
        assert out["num_blocks"] == 0 and np.all(out["counts"] == 0)
        err, _ = G.check_y(layer, out, ids, w)
        assert np.abs(out["Y"]).max() > 0


def test_select_counts_shared_row_tiles():
    """The chosen configuration and every prediction equal the oracle's cost model
    on the local counts plus one count of B per shared expert."""
    rng = np.random.default_rng(9)
    for trial in range(6):
        B = int(rng.choice([1, 7, 64, 300]))
        layer = synth.make_layer("small_sh", B, float(rng.choice([0.1, 1.0])), trial)
        th = (rng.random((V, 4)) * np.array([20, 5, 0.05, 0.5])).astype(np.float32)
        b = G.run(layer, theta=torch.from_numpy(th))
        out = G.fetch(b)
        # the oracle's own counts and the documented constants (never the library's)
        cc = spec.cost_constants(layer.shape.hidden, layer.shape.inter, G.num_cus())
        assert moe_cost_constants(b.p) == cc
        ids, _ = oracle.route_topk(layer.logits, layer.shape.top_k)
        cnt_ref = oracle.counts(ids, layer.expert_begin, layer.shape.local_experts)
        np.testing.assert_array_equal(out["counts"], cnt_ref)
        cnt = np.concatenate([cnt_ref, np.full(layer.shape.shared, B, np.int32)])
        ref_v, ref_t, _ = oracle.select(cnt, cc["b"], cc["q1"], cc["q2"], cc["S1"], cc["S2"], th)
        assert out["variant"] == ref_v
        np.testing.assert_array_equal(b.t_hat.cpu().numpy().view(np.uint32), ref_t.view(np.uint32))


def test_graph_replay_fp8_activations_and_shared():
    """The whole layer with FP8 activations in both GEMMs and shared experts (two
    quantization launches, shared row-blocks, shared combine lanes) captured in one
    HIP graph replays to the eager result, with eager work between replays."""
    layer = synth.make_layer("small_sh_fp8ah", 130, 1.0, 4)
    th = torch.tensor([[5.0, 0.0, 0.01, 0.1]] * V, dtype=torch.float32)
    th[:, 0] += torch.arange(V, dtype=torch.float32)
    b = L.from_layer(layer, theta=th, weights=G.device_weights(layer))
    L.forward(b)
    torch.cuda.synchronize()
    eager = b.y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        L.forward(b, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    b.y.zero_()
    with torch.cuda.graph(g):
        L.forward(b)
    for r in range(4):
        b.y.fill_(float(r + 1))
        b.workspace.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(b.y.view(torch.int16), eager.view(torch.int16)), r
